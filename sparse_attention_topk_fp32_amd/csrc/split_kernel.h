// split_kernel.h - few rows: a row split over several workgroups that agree on a
// sampled bound, the last one finishing it on chip.
// Part of the topk_select library: included once, in order, by topk_select.hip.

#pragma once

#include "common.h"

namespace tks {

// ----------------------------------------------------------------- split kernel (few rows)
//
// BLOCK threads per WG, ITEMS logits per thread per tile; RESIDENT: the
// slice is one tile (loaded once, up front); KEYS: the keys of the output
// are recorded (ordered output); SPT: chunks of the row's sample per thread.  G WGs per row; a row of L valid logits
// uses the first ceil(chunks / chunks_per_wg) of them, and the last of those
// finishes the row.

template <int BLOCK>
struct SplitSmem {
    alignas(16) uint32_t hist[kHistWords];  // 256-bin histograms, kCopies copies (or 4096 bins)
    alignas(16) uint64_t cand[kBufCap];       // candidates (finishing WG); the bound's second histogram before
    uint64_t small[kSmall];                   // the last few, ranked exactly
    uint32_t cnt[kMaxSplit];                  // the other WGs' candidate counts (finishing WG)
    uint32_t pre[kMaxSplit];                  // their exclusive prefix
    uint32_t prex[kMaxSplit];                 // exclusive prefix of the counts past the speculative reads
    uint32_t scan[BLOCK / 64];
    uint32_t scan2[2][BLOCK / 64];
    uint32_t sel[4];
    uint32_t tot[2];  // the others' candidates; those past the speculative reads
    uint32_t tag;
    uint32_t bad;
};

// The arguments that the first loads depend on come first, one by one: the
// dispatcher can then place them in scalar registers as the waves start
// (kernel-argument preloading), and the row's loads need not wait for the
// argument fetch.  P holds the rest (its copies of these are not read).
template <int BLOCK, int ITEMS, bool RESIDENT, bool KEYS, int SPT>
__global__ __launch_bounds__(BLOCK) void topk_split_kernel(const float* logits, const int32_t* lengths, int32_t rows,
                                                           int32_t n, int32_t k, int32_t G, int32_t xcds, int32_t cpw,
                                                           int32_t sample_chunks, const KParams P) {
    static_assert(ITEMS % 4 == 0, "ITEMS counts whole 16-byte chunks");
    static_assert(BLOCK % 64 == 0 && BLOCK >= 256, "whole waves, 256 histogram owners");
    static_assert(kCopies * kStride * 4 <= kBufCap * 8, "the bound's second histogram fits in the buffer");
    constexpr int CHUNKS = ITEMS / 4;            // chunks per thread per tile
    constexpr int TILE_CHUNKS = BLOCK * CHUNKS;  // chunks per tile
    // SPT: sample chunks per thread (the host keeps the sample within it)
    static_assert(SPT >= 1 && SPT * BLOCK <= kSampleMax, "sample fits the block");
    __shared__ SplitSmem<BLOCK> sm;

    const int tid = threadIdx.x;
    // Block b runs on XCD b mod X (the dispatcher deals blocks out in turn).
    // Grouped: row r's WG w is block (r mod X) + X (w + G floor(r / X)), so
    // a row's WGs share one XCD's L2 and meet sooner there; blocks past the
    // last row exit.  WG w of a row still comes after WGs 0..w-1 in block
    // order, and nothing else depends on where a WG runs.
    int row, w;
    if (xcds > 1) {
        const int X = xcds;
        const int x = (int)(blockIdx.x % (unsigned)X);
        const int s = (int)(blockIdx.x / (unsigned)X);
        const int rg = s / G;
        row = x + X * rg;
        w = s - rg * G;
        if (row >= rows) return;
    } else {
        row = blockIdx.x / G;
        w = blockIdx.x - row * G;
    }
    const float* __restrict__ prow = logits + (size_t)row * (size_t)n;
    int32_t* __restrict__ out = P.out + (size_t)row * (size_t)k;
    uint32_t* const okey = KEYS ? P.keys + (size_t)row * (size_t)k : nullptr;
    const int L = valid_length(lengths, row, n);
    // ordered output made by the finishing WG itself (k <= kOrdLds): from
    // the unordered indices and keys it records, read back after a barrier
    int32_t* const oout = KEYS && P.oout ? P.oout + (size_t)row * (size_t)k : nullptr;
    float* const ovals = KEYS && P.oout && P.ovals ? P.ovals + (size_t)row * (size_t)k : nullptr;
    if (L <= k) {  // everything valid is selected; pad with -1
        if (w == 0) {
            bool done = false;
            if constexpr (KEYS) {
                if (oout && L > 0) {
                    ordered_finish<BLOCK, kOrdLds, kBufCap, true>(out, okey, true, prow, (uint32_t)L, (uint32_t)L, k, oout,
                                                            ovals, sm.cand, sm.hist, sm.scan);
                    done = true;
                } else if (oout) {
                    for (int i = tid; i < k; i += BLOCK) {
                        oout[i] = -1;
                        if (ovals) ovals[i] = -__builtin_huge_valf();
                    }
                    done = true;
                }
            }
            if (!done)
                for (int i = tid; i < k; i += BLOCK) out[i] = i < L ? i : -1;
        }
        return;
    }
    const int off = (int)(((uintptr_t)prow >> 2) & 3);  // elements before the first 16-byte boundary
    const int nchunks = (off + L + 3) >> 2;
    const int Geff = (nchunks + cpw - 1) / cpw;  // WGs with a non-empty slice
    if (w >= Geff) return;
    const bool multi = Geff > 1;
    const bool fin = w == Geff - 1;  // the finishing WG: every WG it waits for was dispatched before it
    const char* const base = reinterpret_cast<const char*>(prow - off);  // 16-byte aligned
    const int c_begin = w * cpw;
    const int c_end = min(nchunks, c_begin + cpw);
    const int cf_lo = off ? 1 : 0;      // chunks whose four elements are all valid: [cf_lo, cf_hi)
    const int cf_hi = (L + off) >> 2;
    SplitRow* const rw = multi ? P.rws + row : nullptr;
    const size_t R = (size_t)P.region;

    // keys of chunk c from its 16 bytes (0 for slots outside the row)
    auto chunk_keys = [&](int c, const uint4& v, uint32_t* kk) {
        const uint32_t raw[4] = {v.x, v.y, v.z, v.w};
        if (c >= cf_lo && c < cf_hi) {
#pragma unroll
            for (int e = 0; e < 4; ++e) kk[e] = key_of(__uint_as_float(raw[e]));
        } else {
            const int e0 = 4 * c - off;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = (c >= 0) & (c < nchunks) & ((uint32_t)(e0 + e) < (uint32_t)L);
                kk[e] = ok ? key_of(__uint_as_float(raw[e])) : 0u;
            }
        }
    };
    uint32_t keys[ITEMS];
    uint4 traw[CHUNKS];
    // one tile: chunk c = c_tile + j * BLOCK + tid of the slice, loaded raw
    // (lanes past the slice re-read chunk 0), then turned into keys (those
    // lanes hold empty slots)
    auto load_tile = [&](int c_tile) {
#pragma unroll
        for (int j = 0; j < CHUNKS; ++j) {
            const int c = c_tile + j * BLOCK + tid;
            traw[j] = *reinterpret_cast<const uint4*>(base + (size_t)(c < c_end ? c : 0) * 16u);
        }
    };
    auto tile_keys = [&](int c_tile) {
#pragma unroll
        for (int j = 0; j < CHUNKS; ++j) {
            const int c = c_tile + j * BLOCK + tid;
            chunk_keys(c < c_end ? c : -1, traw[j], &keys[4 * j]);
        }
    };

    // ---- the bound.  A row that one resident WG holds whole uses its own
    // keys: the 16-bit prefix of its k-th largest.  Otherwise every WG of
    // the row reads the same sample, blocks of 16 chunks spread evenly from
    // the row's first chunk to its last (all of it when the row is no
    // longer), and takes the prefix of the sample's element of rank
    // r = m + 4 sqrt(m) + 6, m = k S / L the expected count of the row's k
    // largest among its S sampled logits: a rank that the sample's count
    // above the row's k-th largest exceeds with a probability below 1e-5
    // (binomial tail, for logits drawn alike along the row), so a miss, and
    // the slow path below, comes about once in 10^5 calls or less.
    // The bound is a lower bound on the k-th largest key when it holds; the
    // finishing WG checks that at least k candidates came out, else the row
    // is finished by passes over it.
    const bool own_sample = !multi && RESIDENT;
    const int Sc = own_sample ? 0 : min(nchunks, sample_chunks);
    const bool whole_sample = nchunks <= sample_chunks;
    uint4 sraw[SPT];
    int sc[SPT];  // the sampled chunks (-1: none)
    if (!own_sample) {
        // block i of nb starts at chunk floor(i * (nchunks - 16) / (nb - 1))
        // (16.16 fixed point; the last block ends at the last chunk)
        const int nb = Sc / 16;
        const uint64_t step = whole_sample ? 0ull : (((uint64_t)(nchunks - 16)) << 16) / (uint64_t)(nb - 1);
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int qq = u * BLOCK + tid;
            const int blk = qq >> 4;
            const int start = blk == nb - 1 ? nchunks - 16 : (int)(((uint64_t)blk * step) >> 16);
            sc[u] = qq < Sc ? (whole_sample ? qq : start + (qq & 15)) : -1;
            sraw[u] = sc[u] >= 0 ? *reinterpret_cast<const uint4*>(base + (size_t)sc[u] * 16u)
                                 : uint4{0u, 0u, 0u, 0u};
        }
    }
    if constexpr (RESIDENT) load_tile(c_begin);
    // the launch's epoch (tags the published counts), one load per WG,
    // issued after the logits so that waiting for them does not wait for it
    uint32_t epoch = 0;
    if (multi && tid == 0) epoch = ld_dev(&rw->epoch);
    // while the loads are in flight: the bound's histograms cleared
    uint32_t* const h2 = reinterpret_cast<uint32_t*>(sm.cand);
    clear_words(sm.hist, kCopies * kStride, tid, BLOCK);
    clear_words(h2, kCopies * kStride, tid, BLOCK);
    if (tid == 0) sm.bad = 0u;
    lds_sync();
    if constexpr (RESIDENT) tile_keys(c_begin);
    uint32_t lo;
    if (own_sample) {
        lo = bound_select<BLOCK, ITEMS>(keys, (uint32_t)k, sm.hist, h2, sm.sel);
    } else {
        uint32_t sk[4 * SPT];
#pragma unroll
        for (int u = 0; u < SPT; ++u) chunk_keys(sc[u], sraw[u], &sk[4 * u]);
        // valid sampled logits: every chunk holds four, save the first and
        // the last chunk of the row, which the sample always includes
        const uint32_t S = whole_sample ? (uint32_t)L : (uint32_t)(4 * Sc - 4 * nchunks + L);
        uint32_t r = (uint32_t)k;
        if (!whole_sample) {
            const float mexp = (float)k * (float)S / (float)L;
            const float rf = ceilf(mexp + 4.0f * sqrtf(mexp) + 6.0f);
            r = rf >= (float)S ? S : (uint32_t)rf;
        }
        lo = bound_select<BLOCK, 4 * SPT>(sk, r, sm.hist, h2, sm.sel);
    }
    const uint32_t tag = make_tag(epoch);  // thread 0's
    if (tid == 0) sm.tag = tag;

    // ---- candidates: the slice's composites at or above the bound, in a
    // fixed order (tile, thread, slot), staged in LDS.  A WG that does not
    // finish publishes their number and copies them to its region; the
    // finishing WG keeps its own in LDS.
    const bool to_region = multi && !fin;
    // long slices stage their candidates in LDS for line-sized region
    // stores; short ones (few candidates per thread) store directly
    constexpr bool kStaged = ITEMS >= 16 || !RESIDENT;
    uint64_t* const region = to_region ? P.stage + ((size_t)row * (size_t)G + (size_t)w) * R : nullptr;
    // the finishing WG counts its candidates into the first round's window
    // histogram as they are placed (sm.hist is zero after the bound)
    uint32_t* const hc = sm.hist + (tid % kCopies) * kStride;
    uint32_t total = 0;
    int par = 0;
    auto place_tile = [&](int c_tile, uint32_t first) {
        uint32_t p = first;
        if (to_region) {  // staged in LDS and copied to the region afterwards (long slices), or direct
#pragma unroll
            for (int j = 0; j < CHUNKS; ++j) {
                const int ib = 4 * (c_tile + j * BLOCK + tid) - off;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t key = keys[4 * j + e];
                    const bool t = key >= lo;
                    if constexpr (kStaged) {
                        if (t & (p < (uint32_t)kBufCap)) sm.cand[p] = composite(key, (uint32_t)(ib + e));
                    } else {
                        if (t & (p < R)) st_dev(&region[p], composite(key, (uint32_t)(ib + e)));
                    }
                    p += t ? 1u : 0u;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < CHUNKS; ++j) {
                const int ib = 4 * (c_tile + j * BLOCK + tid) - off;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t key = keys[4 * j + e];
                    const bool t = key >= lo;
                    if (t & (p < (uint32_t)kBufCap)) {
                        const uint64_t c = composite(key, (uint32_t)(ib + e));
                        sm.cand[p] = c;
                        atomicAdd(&hc[window_bin(c, lo)], 1u);
                    }
                    p += t ? 1u : 0u;
                }
            }
        }
    };
    auto count_tile = [&]() {
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) c += keys[i] >= lo;
        return c;
    };
    if constexpr (RESIDENT) {
        const uint32_t first = block_append<BLOCK>(count_tile(), &sm.scan2[0][0], par, total);
        // the count is published before the entries are written: the
        // finishing WG polls each entry until it is non-zero
        if (to_region && tid == 0) st_dev(&rw->cnt[w], ((uint64_t)tag << 32) | (uint64_t)total);
        place_tile(c_begin, first);
    } else {
        for (int ct = c_begin; ct < c_end; ct += TILE_CHUNKS) {
            load_tile(ct);
            tile_keys(ct);
            const uint32_t first = block_append<BLOCK>(count_tile(), &sm.scan2[0][0], par, total);
            place_tile(ct, first);
        }
        if (to_region && tid == 0) st_dev(&rw->cnt[w], ((uint64_t)tag << 32) | (uint64_t)total);
    }
    if (to_region) {
        if constexpr (!kStaged) return;
        // the staged candidates to the region in consecutive order: each
        // wave's stores cover whole lines
        lds_sync();
        const uint32_t nw = min(total, (uint32_t)(R < (size_t)kBufCap ? R : (size_t)kBufCap));
        for (uint32_t i = (uint32_t)tid; i < nw; i += BLOCK) st_dev(&region[i], sm.cand[i]);
        return;
    }

    // ---- the finishing WG: its own candidates are cand[0 .. total); the
    // other WGs' follow in WG order
    uint32_t C = total;
    bool ok;
    if (multi) {
        const int others = Geff - 1;
        const uint32_t tagv = uniform(sm.tag);
        const uint64_t lim = spin_limit();
        // TPR threads per region: thread (wr, sub) polls region wr's count
        // (sub 0) and reads its entries sub, sub + TPR, ... speculatively, in
        // the same round trip; entries not yet written read as 0 and are
        // polled again once the count says they exist
        const int TPR = BLOCK / others;
        const int wr = tid / TPR, sub = tid - wr * TPR;
        const bool mine = wr < others;
        uint64_t* const rb = P.stage + ((size_t)row * (size_t)G + (size_t)(mine ? wr : 0)) * R;
        constexpr int U = 8;
        const uint32_t E = (uint32_t)(TPR * U);  // entries read speculatively per region
        uint64_t cv = 0;
        if (mine && sub == 0) cv = lim ? ld_dev(&rw->cnt[wr]) : 0ull;
        uint64_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t j = (uint32_t)(sub + TPR * u);
            v[u] = (mine && j < R) ? ld_dev(&rb[j]) : 0ull;
        }
        if (mine && sub == 0) {
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while ((uint32_t)(cv >> 32) != tagv) {
                if (__builtin_amdgcn_s_memrealtime() - t0 >= lim) {
                    raise_flag(P.status, kFlagTimeout);
                    sm.bad = 1u;
                    cv = 0ull;
                    break;
                }
                cv = ld_dev(&rw->cnt[wr]);
            }
            sm.cnt[wr] = (uint32_t)cv;
        }
        lds_sync();
        // prefixes over the regions: of the counts, and of the counts past
        // the speculative reads.  Up to 64 regions every wave scans them
        // itself (no barrier; the arrays, which only the reads past the
        // speculative ones use, are written when there are such); more
        // regions: wave 0 writes the arrays, then a barrier.
        uint32_t c_others, X, pn;
        if (others <= 64) {
            const int l = tid & 63;
            const uint32_t c = l < others ? sm.cnt[l] : 0u;
            const uint32_t x = c > E ? c - E : 0u;
            const uint32_t ia = wave_inclusive_scan(c), ix = wave_inclusive_scan(x);
            c_others = (uint32_t)__builtin_amdgcn_readlane((int)ia, 63);
            X = (uint32_t)__builtin_amdgcn_readlane((int)ix, 63);
            pn = (uint32_t)__shfl((int)(ia - c), mine ? wr : 0);
            if (X != 0u) {
                if (tid < others) {
                    sm.pre[tid] = ia - c;
                    sm.prex[tid] = ix - x;
                }
                lds_sync();
            }
        } else {
            if (tid < 64) {
                const int npl = (others + 63) / 64;  // regions per lane
                uint32_t a = 0, x = 0;
                for (int i = 0; i < npl; ++i) {
                    const int r2 = tid * npl + i;
                    if (r2 < others) {
                        const uint32_t c = sm.cnt[r2];
                        a += c;
                        x += c > E ? c - E : 0u;
                    }
                }
                const uint32_t ia = wave_inclusive_scan(a), ix = wave_inclusive_scan(x);
                uint32_t pa = ia - a, px = ix - x;
                for (int i = 0; i < npl; ++i) {
                    const int r2 = tid * npl + i;
                    if (r2 < others) {
                        const uint32_t c = sm.cnt[r2];
                        sm.pre[r2] = pa;
                        sm.prex[r2] = px;
                        pa += c;
                        px += c > E ? c - E : 0u;
                    }
                }
                if (tid == 63) {
                    sm.tot[0] = ia;
                    sm.tot[1] = ix;
                }
            }
            lds_sync();
            c_others = uniform(sm.tot[0]);
            X = uniform(sm.tot[1]);
            pn = sm.pre[mine ? wr : 0];
        }
        C = total + c_others;
        ok = sm.bad == 0u && C >= (uint32_t)k && C <= (uint32_t)kBufCap;
        // every entry is read (when the row is finished otherwise, waited
        // for; all missing ones polled again together), moved to the buffer
        // and cleared for the next launch
        {
            const uint32_t cn = sm.cnt[mine ? wr : 0];
            const uint32_t cw = mine ? min(cn, (uint32_t)R) : 0u, pw = mine ? pn : 0u;
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            for (;;) {
                bool miss = false;
#pragma unroll
                for (int u = 0; u < U; ++u) miss |= ((uint32_t)(sub + TPR * u) < cw) & (v[u] == 0ull);
                if (!miss) break;
                if (__builtin_amdgcn_s_memrealtime() - t0 >= lim) {
                    raise_flag(P.status, kFlagTimeout);
                    sm.bad = 1u;
                    break;
                }
                for (int u = 0; u < U; ++u) {
                    const uint32_t j = (uint32_t)(sub + TPR * u);
                    if ((j < cw) & (v[u] == 0ull)) v[u] = ld_dev(&rb[j]);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t j = (uint32_t)(sub + TPR * u);
                if (j < cw) {
                    if (ok && v[u] != 0ull) {
                        sm.cand[total + pw + j] = v[u];
                        atomicAdd(&hc[window_bin(v[u], lo)], 1u);
                    }
                    st_dev(&rb[j], (uint64_t)0);
                }
            }
        }
        // entries past the speculative reads (regions holding more than E):
        // entry i of that remainder is entry E + i - prex[w'] of region w',
        // w' the last region whose prefix is at most i (binary search)
        constexpr int UP = 8;
        for (uint32_t i0 = 0; i0 < X; i0 += UP * BLOCK) {
            uint64_t* addr[UP];
            uint32_t dst[UP];
            uint64_t vv[UP];
#pragma unroll
            for (int u = 0; u < UP; ++u) {
                const uint32_t i = i0 + (uint32_t)(u * BLOCK + tid);
                addr[u] = nullptr;
                dst[u] = 0;
                if (i < X) {
                    int a = 0, b = others;  // prex[a] <= i < prex[b] (prex[others] taken as infinite)
                    while (b - a > 1) {
                        const int mid = (a + b) >> 1;
                        if (sm.prex[mid] <= i) a = mid;
                        else b = mid;
                    }
                    const uint32_t j = E + i - sm.prex[a];
                    dst[u] = total + sm.pre[a] + j;
                    if (j < R) addr[u] = P.stage + ((size_t)row * (size_t)G + (size_t)a) * R + j;
                }
                vv[u] = addr[u] ? ld_dev(addr[u]) : 1ull;
            }
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            for (;;) {
                bool miss = false;
#pragma unroll
                for (int u = 0; u < UP; ++u) miss |= vv[u] == 0ull;
                if (!miss) break;
                if (__builtin_amdgcn_s_memrealtime() - t0 >= lim) {
                    raise_flag(P.status, kFlagTimeout);
                    sm.bad = 1u;
                    break;
                }
#pragma unroll
                for (int u = 0; u < UP; ++u)
                    if (vv[u] == 0ull) vv[u] = ld_dev(addr[u]);
            }
#pragma unroll
            for (int u = 0; u < UP; ++u) {
                if (!addr[u]) continue;
                if (ok && vv[u] != 0ull) {
                    sm.cand[dst[u]] = vv[u];
                    atomicAdd(&hc[window_bin(vv[u], lo)], 1u);
                }
                st_dev(addr[u], (uint64_t)0);
            }
        }
        // the counts and the epoch for the next launch
        if (mine && sub == 0) st_dev(&rw->cnt[wr], (uint64_t)0);
        if (tid == 0) st_dev(&rw->epoch, epoch + 1u);
        lds_sync();
        ok = ok && sm.bad == 0u;
    } else {
        ok = C >= (uint32_t)k && C <= (uint32_t)kBufCap;
        lds_sync();
    }
    if (__builtin_expect(ok, 1)) {
        // passes unrolled 4 times for the short-slice variants, twice for
        // the long ones (measured: 512x4 -0.17 us, 1024x8 -0.40; 512x16 and
        // 1024x32 +0.09 and +0.41 with 4)
        select_buffer<BLOCK, (ITEMS <= 8 ? 4 : 2)>(sm.cand, C, (uint32_t)k, 0u, lo, true, sm.hist, sm.small, sm.scan,
                                                   sm.sel, out, okey, k, P.status);
    } else {
        lds_sync();
        select_by_passes<BLOCK, kBufCap>(base, off, L, nchunks, k, out, okey, sm.cand, sm.hist, sm.small, sm.scan,
                                         sm.sel, P.status);
    }
    if constexpr (KEYS) {
        if (oout) {
            __syncthreads();  // the recorded unordered form (global scratch) is complete and visible to the WG
            ordered_finish<BLOCK, kOrdLds, kBufCap, true>(out, okey, false, prow, (uint32_t)L, (uint32_t)k, k, oout, ovals,
                                                    sm.cand, sm.hist, sm.scan);
        }
    }
}

}  // namespace tks
