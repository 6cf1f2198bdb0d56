// rows_kernel.h - many rows: one workgroup per row, a running bound over a single read,
// and the ordered form made in the same workgroup.
// Part of the topk_select library: included once, in order, by topk_select.hip.

#pragma once

#include "common.h"

namespace tks {

// ----------------------------------------------------------------- one WG per row
//
// Batches of many rows: one WG owns a whole row and streams it in tiles of
// BLOCK x ITEMS logits, the next PD tiles' loads in flight while the
// current one is processed.  During that single read it keeps every element
// whose key is at or above a running lower bound in an LDS buffer (the
// bound estimated from the elements seen so far and raised as the buffer
// fills); when the buffer ends up holding at least k elements, the row's
// k largest are the buffer's and the on-chip selection finishes the row.
// Otherwise the row is finished by passes over it.  Buffer positions come
// from block scans, so the buffer's order, and with it the output order, is
// fixed by the row's values.

// candidate buffer of the one-WG-per-row kernel (entries): as large as two
// WGs per CU allow with some LDS to spare (78 KB per WG)
constexpr int kRowsCap = 5376;
constexpr uint32_t kRowsDenseBin = 512;  // a bound bin holding more buffered entries is refined

template <int BLOCK>
struct RowsSmem {
    union {
        uint32_t h12[2 * 4097];                  // first digit: 2 copies of 4096 bins (stride 4097)
        alignas(16) uint32_t h8[kHistWords];     // 256-bin rounds (4096 bins in a pass over the row)
    } h;
    alignas(16) uint64_t cand[kRowsCap];  // candidates at or above the running bound
    static_assert(kHistWords >= 2 * kOrdBins, "the ordered form's bins fit the histogram area");
    static_assert(kHistWords + 2 * kOrdLds <= 2 * 4097, "the selection's output fits above the histograms");
    uint64_t small[kSmall];               // the last few, ranked exactly
    uint32_t scan[BLOCK / 64];
    uint32_t scan2[2][BLOCK / 64];
    uint32_t sel[4];
};

// MODE 0: unordered output; 1: unordered output with its keys recorded to
// global scratch (ordered by a second launch); 2: the ordered output made
// here (k <= kOrdLds), the unordered form kept in LDS.
template <int BLOCK, int ITEMS, int PD, int MODE>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4))) void topk_rows_kernel(const KParams P) {
    static_assert(ITEMS % 4 == 0, "ITEMS counts whole 16-byte chunks");
    constexpr bool KEYS = MODE != 0;
    constexpr bool ORD = MODE == 2;
    constexpr int F = 12;
    constexpr int NB0 = 1 << F;
    constexpr int CHUNKS = ITEMS / 4;
    constexpr int TILE_CHUNKS = BLOCK * CHUNKS;
    __shared__ RowsSmem<BLOCK> sm;

    const int tid = threadIdx.x;
    const int row = blockIdx.x;
    const int n = P.n;
    const int k = P.k;
    const float* __restrict__ prow = P.logits + (size_t)row * (size_t)n;
    const int L = valid_length(P.lengths, row, n);
    // ordered form made here (ORD): the selection's unordered output and
    // keys go to the upper half of the histogram area, unused by the
    // selection's rounds (LDS addresses known at compile time: LDS
    // instructions); else to out_idx, or to global scratch with the keys
    int32_t* const oout = ORD ? P.oout + (size_t)row * (size_t)k : nullptr;
    float* const ovals = ORD && P.ovals ? P.ovals + (size_t)row * (size_t)k : nullptr;
    int32_t* __restrict__ out =
        ORD ? reinterpret_cast<int32_t*>(sm.h.h12 + kHistWords) : P.out + (size_t)row * (size_t)k;
    uint32_t* const okey =
        !KEYS ? nullptr : (ORD ? sm.h.h12 + kHistWords + kOrdLds : P.keys + (size_t)row * (size_t)k);
    if (L <= k) {  // everything valid is selected; pad with -1
        if constexpr (ORD) {
            if (L > 0)
                ordered_finish<BLOCK, kOrdLds, kRowsCap>(out, okey, true, prow, (uint32_t)L, (uint32_t)L, k, oout, ovals,
                                                sm.cand, sm.h.h8, sm.scan);
            else
                for (int i = tid; i < k; i += BLOCK) {
                    oout[i] = -1;
                    if (ovals) ovals[i] = -__builtin_huge_valf();
                }
            return;
        }
        for (int i = tid; i < k; i += BLOCK) out[i] = i < L ? i : -1;
        return;
    }
    const int off = (int)(((uintptr_t)prow >> 2) & 3);
    const int nchunks = (off + L + 3) >> 2;
    const int cf_lo = off ? 1 : 0;         // chunks whose four elements are all valid
    const int cf_hi = (L + off) >> 2;
    const char* const base = reinterpret_cast<const char*>(prow - off);

    // f(keys, c_tile) for every tile of the row; slot 4j+e of a thread is
    // element 4(c_tile + j*BLOCK + tid) - off + e, key 0 when empty.  The
    // next tile is loaded while f runs on the current one.
    auto stream = [&](auto&& f) {
        uint4 buf[PD][CHUNKS];  // PD tiles in flight
#pragma unroll
        for (int d = 0; d < PD; ++d) {
            if (d * TILE_CHUNKS < nchunks) {
#pragma unroll
                for (int j = 0; j < CHUNKS; ++j) {
                    const int c = d * TILE_CHUNKS + j * BLOCK + tid;
                    buf[d][j] = *reinterpret_cast<const uint4*>(base + (size_t)(c < nchunks ? c : 0) * 16u);
                }
            }
        }
        for (int ct0 = 0; ct0 < nchunks; ct0 += PD * TILE_CHUNKS) {
#pragma unroll
            for (int d = 0; d < PD; ++d) {
                const int ct = ct0 + d * TILE_CHUNKS;
                if (ct < nchunks) {
                    uint32_t keys[ITEMS];
#pragma unroll
                    for (int j = 0; j < CHUNKS; ++j) {
                        const int c = ct + j * BLOCK + tid;
                        const uint32_t v[4] = {buf[d][j].x, buf[d][j].y, buf[d][j].z, buf[d][j].w};
                        if (c >= cf_lo && c < cf_hi) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) keys[4 * j + e] = key_of(__uint_as_float(v[e]));
                        } else {
                            const int e0 = 4 * c - off;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const bool ok = (c < nchunks) & ((uint32_t)(e0 + e) < (uint32_t)L);
                                keys[4 * j + e] = ok ? key_of(__uint_as_float(v[e])) : 0u;
                            }
                        }
                    }
                    const int cn = ct + PD * TILE_CHUNKS;  // the tile PD ahead reuses this buffer
                    if (cn < nchunks) {
#pragma unroll
                        for (int j = 0; j < CHUNKS; ++j) {
                            const int c = cn + j * BLOCK + tid;
                            buf[d][j] =
                                *reinterpret_cast<const uint4*>(base + (size_t)(c < nchunks ? c : 0) * 16u);
                        }
                    }
                    f(keys, ct);
                }
            }
        }
    };

    // ---------------- the single read: every element whose key is at or
    // above a lower bound `lo_key` kept in LDS.  The bound is an estimate:
    // the first-digit bin (12 bits) of the element of rank 1.125 * k * seen /
    // L + 16 among the `seen` elements read so far, where the k-th largest of
    // the row is expected near rank k * seen / L (in a dense bin, also that
    // element's next 8 key bits).  It is taken from the first tile and
    // raised (with the buffer compacted) whenever the buffer fills up, from
    // histograms of the buffer.  The buffer then holds every element whose
    // key is at or above the bound; when it holds at least k entries, the
    // k-th largest of the buffer is the row's and everything selected is in
    // it.  Otherwise, or when the buffer overflowed twice on one tile, the
    // row is finished by passes over it.
    clear_words(sm.h.h12, 2 * 4097, tid, BLOCK);
    lds_sync();
    bool keep = true;   // candidates are being buffered
    uint32_t used = 0;  // buffered entries
    int par = 0;        // half of scan2 used by the next append
    // running lower bound on the keys kept: a first-digit bin, refined by
    // the next 8 key bits where that bin is dense (at least 1: empty slots
    // are never kept)
    uint32_t lo_key = 1u;
    // Walk the buffer in slices of RC * BLOCK entries: every thread reads its
    // RC entries, a block scan numbers the chosen ones, and f(entry, rank)
    // places them.  pred returns 0 (drop) or 1 (keep).  A kept entry may be
    // moved to the front of the buffer: its new index is never above its old
    // one, and each slice is read before any of it is written.
    constexpr int RC = 3;
    auto compact = [&](auto&& pred) {
        uint32_t n2 = 0;
        for (uint32_t i0 = 0; i0 < used; i0 += RC * BLOCK) {
            uint64_t e[RC];
            uint32_t keepm = 0, cnt = 0;
#pragma unroll
            for (int u = 0; u < RC; ++u) {
                const uint32_t i = i0 + (uint32_t)(u * BLOCK + tid);
                e[u] = sm.cand[i < used ? i : used - 1u];  // clamped: an unpredicated load
                const uint32_t kd = i < used ? pred(e[u]) : 0u;
                keepm |= kd << u;
                cnt += kd;
            }
            uint32_t tot;
            uint32_t p = n2 + block_scan_total<BLOCK>(cnt, sm.scan, tot);
#pragma unroll
            for (int u = 0; u < RC; ++u)
                if ((keepm >> u) & 1u) sm.cand[p++] = e[u];
            n2 += tot;
        }
        return n2;
    };
    // rank of the bound after `seen` valid elements
    auto bound_rank = [&](uint32_t seen) -> uint32_t {
        // the margin at the end of the row, k / 8, is several standard
        // deviations of the count above a fixed rank for values drawn alike
        // along the row; a looser bound buffers (and later selects) more
        const uint64_t est = ((uint64_t)k * seen * 9u) / (8u * (uint64_t)L) + 16u;
        return (uint32_t)(est < seen ? est : seen);
    };
    // the element of rank `rank` among the buffered entries (all in
    // first-digit bins at or above lo, the bound's bin), over a 256-bin
    // window of bins lo .. lo+254, the last bin taking everything above: its
    // window bin, the count above it and the count in it (0 when there are
    // fewer entries)
    auto window_select = [&](uint32_t rank, uint32_t& bw, uint32_t& ab, uint32_t& hbw) {
        const uint32_t lo = lo_key >> (32 - F);
        clear_words(sm.h.h8, kCopies * kStride, tid, BLOCK);
        lds_sync();
        {
            uint32_t* const hcw = sm.h.h8 + (tid % kCopies) * kStride;
            for (uint32_t i = (uint32_t)tid; i < used; i += BLOCK) {
                const uint32_t bin = (uint32_t)(sm.cand[i] >> (64 - F));
                atomicAdd(&hcw[min(bin - lo, 255u)], 1u);
            }
        }
        lds_sync();
        local_select<BLOCK, 256, kCopies, kStride, false>(sm.h.h8, rank, sm.scan, sm.sel, P.status, bw, ab, hbw);
    };
    // the element of rank `rank` among the buffered entries of first-digit
    // bin b: its next 8 key bits (sub-bin s8), the count above it in the bin
    // and the count in it (0 when there are fewer entries)
    auto sub_select = [&](uint32_t b, uint32_t rank, uint32_t& s8, uint32_t& a8, uint32_t& h8v) {
        clear_words(sm.h.h8, kCopies * kStride, tid, BLOCK);
        lds_sync();
        {
            uint32_t* const hcw = sm.h.h8 + (tid % kCopies) * kStride;
            for (uint32_t i = (uint32_t)tid; i < used; i += BLOCK) {
                const uint32_t key = (uint32_t)(sm.cand[i] >> 32);
                if ((key >> (32 - F)) == b) atomicAdd(&hcw[(key >> (32 - F - 8)) & 0xFFu], 1u);
            }
        }
        lds_sync();
        local_select<BLOCK, 256, kCopies, kStride, false>(sm.h.h8, rank, sm.scan, sm.sel, P.status, s8, a8, h8v);
    };
    stream([&](const uint32_t* keys, int ct) {
        if (!keep) return;  // overflowed: the row is finished by passes over it
        // valid elements read once this tile is done
        const uint32_t seen = (uint32_t)min(L, 4 * min(nchunks, ct + TILE_CHUNKS) - off);
        if (ct == 0) {
            // the first bound, from the first tile: the 12-bit bin of the
            // element of rank bound_rank(seen), in two steps — its top 8
            // bits (256-bin histogram, 16 copies), then its next 4 bits
            // among the elements of that 8-bit bin (16 bins).  The union
            // is all zero here.
            uint32_t* const h8c = sm.h.h8 + (tid % kCopies) * kStride;
#pragma unroll
            for (int i = 0; i < ITEMS; ++i)
                if (keys[i] != 0u) atomicAdd(&h8c[keys[i] >> 24], 1u);
            lds_sync();
            uint32_t b8, ab8, hb8;
            const uint32_t rk = bound_rank(seen);
            local_select<BLOCK, 256, kCopies, kStride, false>(sm.h.h8, rk, sm.scan, sm.sel, P.status, b8, ab8, hb8);
            if (hb8 > 0u) {
                uint32_t* const h4 = sm.h.h12 + kCopies * kStride + (tid % kCopies) * 17;  // past the 8-bit copies
#pragma unroll
                for (int i = 0; i < ITEMS; ++i)
                    if ((keys[i] != 0u) & ((keys[i] >> 24) == b8)) atomicAdd(&h4[(keys[i] >> 20) & 15u], 1u);
                lds_sync();
                if (tid < 64) {
                    // lane l: sub-bin 15 - l (descending), summed over the copies
                    uint32_t c = 0;
                    if (tid < 16) {
#pragma unroll
                        for (int q = 0; q < kCopies; ++q) c += sm.h.h12[kCopies * kStride + q * 17 + 15 - tid];
                    }
                    const uint32_t inc = wave_inclusive_scan(c);
                    const uint32_t need4 = rk - ab8;  // 1-based rank inside the 8-bit bin
                    if (tid < 16 && inc - c < need4 && need4 <= inc) sm.sel[3] = 15u - (uint32_t)tid;
                }
                lds_sync();
                const uint32_t b12 = (b8 << 4) | uniform(sm.sel[3]);
                lo_key = max(lo_key, b12 << (32 - F));
            }
        }
        // append: a block scan numbers this tile's candidates in thread
        // order.  A tile that overflows the buffer (its entries past the end
        // are lost) raises the bound from what is buffered, drops its own
        // entries and is appended once more from the registers; a second
        // overflow gives up (passes over the row finish it).
        for (int pass = 0;; ++pass) {
            uint32_t c = 0;
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) c += keys[i] >= lo_key;
            uint32_t pos = block_append<BLOCK>(c, &sm.scan2[0][0], par, used);
            {
                const int ibase = 4 * (ct + tid) - off;
#pragma unroll
                for (int j = 0; j < CHUNKS; ++j) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t key = keys[4 * j + e];
                        if (key >= lo_key) {
                            const uint64_t cc = composite(key, (uint32_t)(ibase + 4 * BLOCK * j + e));
                            if (pos < (uint32_t)kRowsCap) sm.cand[pos] = cc;
                            ++pos;
                        }
                    }
                }
            }
            const bool over = used > (uint32_t)kRowsCap;  // entries of this tile were lost
            if (over && pass > 0) {
                keep = false;
                return;
            }
            if (!over && !(used > (uint32_t)kRowsCap * 3u / 4u && ct + TILE_CHUNKS < nchunks)) break;
            if (over) used = (uint32_t)kRowsCap;
            lds_sync();  // the appended entries are read next
            // tighter bound from more data, and drop what fell below it
            // (and, after an overflow, this tile's entries): the bin of
            // the entry of rank bound_rank(seen), or the top of the
            // window when it lies above (still a lower bound)
            {
                const uint32_t rk = bound_rank(seen);
                uint32_t bw, ab, hbw;
                window_select(rk, bw, ab, hbw);
                if (hbw > 0u) {
                    const uint32_t b12 = min((lo_key >> (32 - F)) + bw, (uint32_t)NB0 - 1u);
                    uint32_t nk = b12 << (32 - F);
                    if (bw < 255u && hbw > kRowsDenseBin) {
                        // a dense bin: the entry's next 8 key bits too
                        uint32_t s8, a8, h8v;
                        sub_select(b12, rk - ab, s8, a8, h8v);
                        if (h8v > 0u) nk |= s8 << (32 - F - 8);
                    }
                    lo_key = max(lo_key, nk);
                }
            }
            const uint32_t lob = lo_key;
            // this tile's index range (empty when nothing was lost)
            const int xlo = over ? 4 * ct - off : 0, xhi = over ? 4 * (ct + TILE_CHUNKS) - off : 0;
            used = compact([&](uint64_t e) -> uint32_t {
                const int idx = (int)~(uint32_t)e;
                return ((uint32_t)(e >> 32) >= lob) & ((idx < xlo) | (idx >= xhi)) ? 1u : 0u;
            });
            lds_sync();  // the moved entries are read next
            if (!over) break;
        }
    });
    // the first tile of the row `ahead` rows on (the one that probably runs
    // next on this WG's XCD) is touched now: its loads then hit the caches
    uint32_t sink = 0;
    if (P.ahead > 0 && row + P.ahead < P.rows && tid * 16 < n)
        sink = *reinterpret_cast<const uint32_t*>(P.logits + (size_t)(row + P.ahead) * (size_t)n + tid * 16);
    lds_sync();
    if (keep && used >= (uint32_t)k) {
        // every buffered entry is at or above the bound (compactions drop
        // what falls below a raised bound; appends use the current one)
        clear_words(sm.h.h8, kCopies * kStride, tid, BLOCK);
        lds_sync();
        select_buffer<BLOCK>(sm.cand, used, (uint32_t)k, 0u, lo_key, false, sm.h.h8, sm.small, sm.scan, sm.sel, out,
                             okey, k, P.status);
    } else {
        select_by_passes<BLOCK, kRowsCap>(base, off, L, nchunks, k, out, okey, sm.cand, sm.h.h8, sm.small, sm.scan,
                                          sm.sel, P.status);
    }
    __asm__ volatile("" ::"v"(sink));
    if constexpr (ORD) {
        lds_sync();  // the unordered form is complete in LDS
        ordered_finish<BLOCK, kOrdLds, kRowsCap>(out, okey, false, prow, (uint32_t)L, (uint32_t)k, k, oout, ovals,
                                                 sm.cand, sm.h.h8, sm.scan);
    }
}

}  // namespace tks
