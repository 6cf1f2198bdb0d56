// topk_select.hip - index-only radix-select TopK for MI355X (gfx950, CDNA4).
//
// Method: the web article "How to Use FlagOS's New Triton-TLE Language to
// Build a TopK Selector Faster Than FlashInfer" (below: the TopK article).
//  * Section 01: per row, the indices of the k largest logits; no values and
//    no sort.
//  * Section 02: radix select.  Floats become order-preserving unsigned keys
//    (mapping), keys are cut into digits from the top (binning), each round
//    histograms one digit of the surviving elements (histogramming), keeps
//    the bin holding the k-th element (thresholding) and finally collects the
//    elements above the threshold, then ties at the threshold in index order
//    (collection).
//  * Section 03: two refinements - keep the surviving candidates on chip once
//    the bucket is small after the first screening, and stop the screening
//    over global memory once the bucket holds at most 4096 elements; wide
//    vector loads.
//  * Section 5: one row split over several blocks that merge their
//    histograms and continue together after a barrier; -1 for empty slots.
//
// MI355X design (not a translation of the article's Triton/CUDA kernels):
//  * Each row is cut into slices of 16-byte chunks; one workgroup (WG) owns
//    one slice.  "Resident" variants load their slice once with 16-byte
//    loads, fuse the key map into the load and keep the keys in VGPRs for
//    every later round; "streaming" variants re-read their slice each round
//    (only used when a row is too long to stay on chip).
//  * Ties are made unique by ranking the 64-bit composite
//    (key << 32 | ~index): larger composite = larger value, or equal value and
//    smaller index.  Rounds run over 8-bit digits of the key (4 rounds) and,
//    only when the threshold value is tied past capacity, of the index.  The
//    k largest composites are exactly the selection with lowest-index ties.
//  * A row spread over G > 1 WGs (the batch-1 case) merges its 256-bin LDS
//    histograms through device-scope atomics into a per-row global histogram
//    and waits at a bounded spin barrier; every WG then picks the same
//    threshold bin from the merged counts, so no broadcast round trip is
//    needed.  The host only uses G > 1 when all WGs of the launch fit on the
//    GPU at once (occupancy query), so the barrier always completes.
//  * Once the threshold bucket holds <= 4096 elements, its (key, index) pairs
//    go to a candidate buffer (LDS for G == 1, global for G > 1) and one WG
//    (the last to arrive, for G > 1) finishes the selection on chip: more
//    digit rounds in LDS while the bucket exceeds 256, then an exact rank of
//    the remaining composites.
//  * Elements above the threshold bucket are written straight to the output
//    by the WG that holds them.  The per-row workspace is left zeroed by the
//    finishing WG, so no clearing launch is needed between calls.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <mutex>
#include <utility>

#include "topk_select.h"

namespace tks {

constexpr int kBins = 256;       // 8-bit digits
constexpr int kCap = 4096;       // candidate buffer capacity (elements)
constexpr int kSmall = 256;      // bucket size ranked directly by the finisher
constexpr int kMaxPasses = 8;    // 4 key digits + up to 4 index digits
constexpr uint32_t kFlagTimeout = 1u;
constexpr uint32_t kFlagCapacity = 2u;
// Bound on a cross-workgroup wait, in ticks of the 100 MHz constant clock
// (s_memrealtime): 2 s, far beyond any legitimate wait.
constexpr uint64_t kSpinLimitTicks = 200000000ull;

// Per-row scratch for rows spread over several workgroups.  Every field is
// zero between calls (the finishing WG of each row clears what it used).
struct alignas(256) RowWorkspace {
    uint32_t hist[kMaxPasses][kBins];
    uint32_t arrive;      // barrier arrivals, G per round
    uint32_t done;        // WGs finished with the row
    uint32_t out_count;   // outputs reserved by WGs (elements above the bucket)
    uint32_t cand_count;  // candidates appended
    uint32_t pad[60];
    uint64_t cand[kCap];  // (key << 32) | ~index of the bucket's elements
};

struct KParams {
    const float* logits;
    const int32_t* lengths;
    int32_t* out;
    RowWorkspace* ws;
    uint32_t* status;
    int32_t rows, n, k;
    int32_t G;              // workgroups per row
    int32_t chunks_per_wg;  // 16-byte chunks in one WG's slice
    int32_t idx_digits;     // 8-bit index digits that follow the 4 key digits
};

// ----------------------------------------------------------------- device helpers

// Mapping step: float bits -> unsigned key, order-preserving for non-NaN
// values, with -0.0 folded onto +0.0 so they tie.  Valid keys are >= 1; key 0
// marks "no element" (out-of-range lanes).  Only the NaN pattern 0xFFFFFFFF
// would map to 0 and is moved to 1 (NaN is outside the contract).
__device__ __forceinline__ uint32_t key_of_bits(uint32_t u) {
    u = (u == 0x80000000u) ? 0u : u;
    const uint32_t flip = (uint32_t)((int32_t)u >> 31) | 0x80000000u;
    const uint32_t key = u ^ flip;
    return key == 0u ? 1u : key;
}

__device__ __forceinline__ int pass_shift(int pass, int idx_digits) {
    return pass < 4 ? 56 - 8 * pass : 8 * (idx_digits - 1 - (pass - 4));
}

__device__ __forceinline__ uint32_t lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ __forceinline__ void raise_flag(uint32_t* status, uint32_t f) {
    __hip_atomic_fetch_or(status, f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thresholding step, run by wave 0: find the bin b holding the element of
// rank `need` (1-based, counted from the top) in a 256-bin histogram.
// Writes b, the count of elements in bins above b, and the count in b.
__device__ void select_bin(const uint32_t* hist, uint32_t need, uint32_t* s_sel, uint32_t* status) {
    const uint32_t lane = lane_id();
    const uint32_t h0 = hist[4 * lane + 0], h1 = hist[4 * lane + 1];
    const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
    const uint32_t s = h0 + h1 + h2 + h3;
    uint32_t incl = s;  // sum over this lane's bins and all higher lanes' bins
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_down(incl, o);
        if (lane + o < 64) incl += t;
    }
    const uint32_t excl = incl - s;
    const bool hit = excl < need && need <= incl;
    const uint64_t any = __ballot(hit);
    if (hit) {
        uint32_t above = excl, b, hb;
        if (above + h3 >= need) {
            b = 4 * lane + 3; hb = h3;
        } else {
            above += h3;
            if (above + h2 >= need) {
                b = 4 * lane + 2; hb = h2;
            } else {
                above += h2;
                if (above + h1 >= need) {
                    b = 4 * lane + 1; hb = h1;
                } else {
                    above += h1; b = 4 * lane; hb = h0;
                }
            }
        }
        s_sel[0] = b; s_sel[1] = above; s_sel[2] = hb;
    }
    if (any == 0 && lane == 0) {  // fewer elements than `need`: cannot happen for valid input
        s_sel[0] = 0; s_sel[1] = 0; s_sel[2] = 0;
        raise_flag(status, kFlagCapacity);
    }
}

// Bounded wait until *ctr >= target (device scope), by one thread.
__device__ void spin_until(uint32_t* ctr, uint32_t target, uint32_t* status) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
        __builtin_amdgcn_s_sleep(1);
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimitTicks) {
            raise_flag(status, kFlagTimeout);
            break;
        }
    }
}

// ----------------------------------------------------------------- the kernel

// Block-wide exclusive scan of two counters at once.  Every thread of the
// block calls it; returns this thread's exclusive prefixes and the totals.
template <int BLOCK>
__device__ __forceinline__ void block_scan2(uint32_t a, uint32_t b, uint32_t* s_w /* [2 * BLOCK / 64] */,
                                            uint32_t& ea, uint32_t& eb, uint32_t& ta, uint32_t& tb) {
    constexpr int NW = BLOCK / 64;
    const uint32_t lane = lane_id();
    const uint32_t wid = threadIdx.x / 64;
    uint32_t ia = a, ib = b;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t xa = __shfl_up(ia, o), xb = __shfl_up(ib, o);
        if (lane >= (uint32_t)o) { ia += xa; ib += xb; }
    }
    if (lane == 63) { s_w[wid] = ia; s_w[NW + wid] = ib; }
    __syncthreads();
    uint32_t pa = 0, pb = 0;
    ta = 0; tb = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint32_t wa = s_w[i], wb = s_w[NW + i];
        if ((uint32_t)i < wid) { pa += wa; pb += wb; }
        ta += wa; tb += wb;
    }
    ea = pa + ia - a;
    eb = pb + ib - b;
    __syncthreads();  // s_w may be reused right after
}

template <int BLOCK, int ITEMS, bool RESIDENT>
__global__ __launch_bounds__(BLOCK) void topk_select_kernel(const KParams P) {
    static_assert(ITEMS % 4 == 0, "ITEMS counts whole 16-byte chunks");
    static_assert(BLOCK % 64 == 0 && BLOCK >= kBins, "one bin per thread in the merge");
    constexpr int CHUNKS = ITEMS / 4;              // chunks per thread per tile
    constexpr int TILE_CHUNKS = BLOCK * CHUNKS;    // chunks per tile

    __shared__ uint32_t s_hist[kBins];
    __shared__ uint64_t s_cand[kCap];
    __shared__ uint64_t s_small[kSmall];
    __shared__ uint32_t s_scan[2 * (BLOCK / 64)];
    __shared__ uint32_t s_sel[3];   // threshold bin, count above it, count in it
    __shared__ uint32_t s_bc[3];    // broadcast: global output base, candidate base, last-WG flag

    const int tid = threadIdx.x;
    const int G = P.G;
    const int row = blockIdx.x / G;
    const int w = blockIdx.x - row * G;
    const int n = P.n;
    const int k = P.k;
    const float* __restrict__ p = P.logits + (size_t)row * (size_t)n;
    int32_t* __restrict__ out = P.out + (size_t)row * (size_t)k;
    int L = n;
    if (P.lengths) {
        L = P.lengths[row];
        L = L < 0 ? 0 : (L > n ? n : L);
    }

    if (L <= k) {  // everything valid is selected; pad with -1
        if (w == 0)
            for (int i = tid; i < k; i += BLOCK) out[i] = i < L ? i : -1;
        return;
    }

    RowWorkspace* ws = P.ws ? P.ws + row : nullptr;
    const int off = (int)(((uintptr_t)p >> 2) & 3);  // elements before the first 16-byte boundary
    const int nchunks = (off + L + 3) >> 2;
    const int c_begin = w * P.chunks_per_wg;
    const int c_end = min(nchunks, c_begin + P.chunks_per_wg);

    uint32_t keys[ITEMS];

    // Load one tile of the slice.  Chunk c of the row is the 16-byte aligned
    // block holding elements [4c - off, 4c - off + 4).  A chunk with at least
    // one valid element lies inside the allocation's page, so it is always
    // read whole; lanes past the slice re-read chunk 0 (valid: L > k >= 1).
    // All loads are issued before any is used; elements outside [0, L) get
    // key 0 ("no element").
    const float* __restrict__ pa = p - off;
    auto load_tile = [&](int c_tile) {
        float4 v[CHUNKS];
#pragma unroll
        for (int j = 0; j < CHUNKS; ++j) {
            const int c = c_tile + j * BLOCK + tid;
            v[j] = *reinterpret_cast<const float4*>(pa + 4 * (c < c_end ? c : 0));
        }
#pragma unroll
        for (int j = 0; j < CHUNKS; ++j) {
            const int c = c_tile + j * BLOCK + tid;
            const int e0 = 4 * c - off;
            const uint32_t u[4] = {__float_as_uint(v[j].x), __float_as_uint(v[j].y),
                                   __float_as_uint(v[j].z), __float_as_uint(v[j].w)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {  // bitwise tests: no branches
                const bool ok = (c < c_end) & ((uint32_t)(e0 + e) < (uint32_t)L);
                keys[4 * j + e] = ok ? key_of_bits(u[e]) : 0u;
            }
        }
    };
    // f(key, index) for every element of one tile; index of element e of
    // chunk j is ibase + 4 * BLOCK * j + e.
    auto visit_tile = [&](int c_tile, auto&& f) {
        const int ibase = 4 * (c_tile + tid) - off;
#pragma unroll
        for (int j = 0; j < CHUNKS; ++j) {
#pragma unroll
            for (int e = 0; e < 4; ++e) f(keys[4 * j + e], ibase + 4 * BLOCK * j + e);
        }
    };
    // Visit every element of the slice (uniform trip count across the WG).
    auto visit = [&](auto&& f) {
        if constexpr (RESIDENT) {
            visit_tile(c_begin, f);
        } else {
            for (int ct = c_begin; ct < c_end; ct += TILE_CHUNKS) {
                load_tile(ct);
                visit_tile(ct, f);
            }
        }
    };

    if constexpr (RESIDENT) load_tile(c_begin);

    // ---------------- screening rounds over the whole row
    // Resolved prefix of the composite (key, ~index): kpfx/kmask over the key,
    // ipfx/imask over ~index (only non-zero after all four key digits).
    const int npasses = 4 + P.idx_digits;
    uint32_t kpfx = 0, kmask = 0, ipfx = 0, imask = 0;
    uint32_t need = (uint32_t)k;
    int pass = 0;
    bool all_sel = false;
    for (;;) {
        if constexpr (RESIDENT) {
            // Opaque to the optimiser: stops it from hoisting per-element
            // values (one lane mask or VGPR per element) out of the rounds.
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) __asm__ volatile("" : "+v"(keys[i]));
        }
        for (int i = tid; i < kBins; i += BLOCK) s_hist[i] = 0;
        __syncthreads();
        if (pass < 4) {
            const int sh = 24 - 8 * pass;
            visit([&](uint32_t key, int) {
                if ((key != 0u) & ((key & kmask) == kpfx)) atomicAdd(&s_hist[(key >> sh) & 0xFFu], 1u);
            });
        } else {
            const int sh = 8 * (P.idx_digits - 1 - (pass - 4));
            visit([&](uint32_t key, int idx) {
                const uint32_t ni = ~(uint32_t)idx;
                if ((key != 0u) & (key == kpfx) & ((ni & imask) == ipfx)) atomicAdd(&s_hist[(ni >> sh) & 0xFFu], 1u);
            });
        }
        __syncthreads();
        if (G > 1) {
            // merge into the row's global histogram, then wait for all G WGs
            if (tid < kBins) {
                const uint32_t v = s_hist[tid];
                if (v) __hip_atomic_fetch_add(&ws->hist[pass][tid], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __syncthreads();
            if (tid == 0) {
                __hip_atomic_fetch_add(&ws->arrive, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                spin_until(&ws->arrive, (uint32_t)(pass + 1) * (uint32_t)G, P.status);
            }
            __syncthreads();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            if (tid < kBins)
                s_hist[tid] = __hip_atomic_load(&ws->hist[pass][tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
        }
        if (tid < 64) select_bin(s_hist, need, s_sel, P.status);
        __syncthreads();
        const uint32_t b = s_sel[0], above = s_sel[1], hb = s_sel[2];
        need -= above;
        if (pass < 4) {
            kpfx |= b << (24 - 8 * pass);
            kmask |= 0xFFu << (24 - 8 * pass);
        } else {
            const int sh = 8 * (P.idx_digits - 1 - (pass - 4));
            ipfx |= b << sh;
            imask |= 0xFFu << sh;
        }
        ++pass;
        if (hb == need) { all_sel = true; break; }
        if (hb <= (uint32_t)kCap || pass >= npasses) break;
    }

    // ---------------- collection over the row
    // Composite prefix above the bucket -> output now ("win"); in the bucket
    // -> candidate for the on-chip finish, unless the whole bucket is taken.
    auto classify = [&](uint32_t key, int idx, bool& win, bool& cand) {
        const uint32_t pk = key & kmask;
        const uint32_t pi = ~(uint32_t)idx & imask;
        const bool eq = (pk == kpfx) & (pi == ipfx);
        const bool gt = (pk > kpfx) | ((pk == kpfx) & (pi > ipfx));
        win = (key != 0u) & (gt | (all_sel & eq));
        cand = (key != 0u) & (!all_sel) & eq;
    };
    // Resident slices record the classification as two per-thread bit masks
    // (bit 4j+e = element e of chunk j), so the write pass below touches only
    // selected elements; streaming slices classify again tile by tile.
    uint32_t nw = 0, nc = 0;
    uint64_t wmask = 0, cmask = 0;
    if constexpr (RESIDENT) {
        static_assert(ITEMS <= 64, "one 64-bit mask per thread");
        visit_tile(c_begin, [&](uint32_t key, int idx) {
            bool win, cand;
            classify(key, idx, win, cand);
            wmask = (wmask >> 1) | ((uint64_t)win << 63);
            cmask = (cmask >> 1) | ((uint64_t)cand << 63);
        });
        wmask >>= 64 - ITEMS;
        cmask >>= 64 - ITEMS;
        nw = (uint32_t)__popcll(wmask);
        nc = (uint32_t)__popcll(cmask);
    } else {
        visit([&](uint32_t key, int idx) {
            bool win, cand;
            classify(key, idx, win, cand);
            nw += win;
            nc += cand;
        });
    }
    uint32_t ow, oc, tw, tc;
    block_scan2<BLOCK>(nw, nc, s_scan, ow, oc, tw, tc);
    if (G > 1) {
        if (tid == 0) {
            s_bc[0] = tw ? __hip_atomic_fetch_add(&ws->out_count, tw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
            s_bc[1] = tc ? __hip_atomic_fetch_add(&ws->cand_count, tc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
        }
        __syncthreads();
        ow += s_bc[0];
        oc += s_bc[1];
    }
    const uint32_t nwin_total = (uint32_t)k - (all_sel ? 0u : need);
    uint64_t* cand_dst = G > 1 ? ws->cand : s_cand;
    auto emit_win = [&](int idx) {
        if (ow < nwin_total) out[ow] = idx;
        else raise_flag(P.status, kFlagCapacity);
        ++ow;
    };
    auto emit_cand = [&](uint32_t key, int idx) {
        if (oc < (uint32_t)kCap) cand_dst[oc] = ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)idx);
        else raise_flag(P.status, kFlagCapacity);
        ++oc;
    };
    // per-thread loops: no barrier or wave operation inside
    if constexpr (RESIDENT) {
        const int ibase = 4 * (c_begin + tid) - off;
        while (wmask) {
            const int i = __builtin_ctzll(wmask);
            wmask &= wmask - 1;
            emit_win(ibase + 4 * BLOCK * (i >> 2) + (i & 3));
        }
        while (cmask) {
            const int i = __builtin_ctzll(cmask);
            cmask &= cmask - 1;
            const int idx = ibase + 4 * BLOCK * (i >> 2) + (i & 3);
            emit_cand(key_of_bits(__float_as_uint(p[idx])), idx);  // re-read: candidates are few
        }
    } else if (nw | nc) {
        visit([&](uint32_t key, int idx) {
            bool win, cand;
            classify(key, idx, win, cand);
            if (win) emit_win(idx);
            if (cand) emit_cand(key, idx);
        });
    }
    __syncthreads();

    uint32_t m = 0;
    if (G > 1) {
        // the last WG of the row to get here finishes it and clears the workspace
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = __hip_atomic_fetch_add(&ws->done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            s_bc[2] = (old == (uint32_t)G - 1u) ? 1u : 0u;
        }
        __syncthreads();
        if (s_bc[2] == 0u) return;
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (!all_sel) {
            m = __hip_atomic_load(&ws->cand_count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            m = m > (uint32_t)kCap ? (uint32_t)kCap : m;
            for (uint32_t i = tid; i < m; i += BLOCK)
                s_cand[i] = __hip_atomic_load(&ws->cand[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    } else {
        m = tc > (uint32_t)kCap ? (uint32_t)kCap : tc;
    }
    __syncthreads();

    // ---------------- on-chip finish over the candidate buffer
    if (!all_sel) {
        uint64_t pfx = ((uint64_t)kpfx << 32) | ipfx;
        uint64_t pmask = ((uint64_t)kmask << 32) | imask;
        int32_t* __restrict__ fout = out + nwin_total;  // `need` slots remain
        const uint32_t need0 = need;
        bool fin_all = false;
        uint32_t mb = m;
        while (mb > (uint32_t)kSmall && pass < npasses) {
            const int sh = pass_shift(pass, P.idx_digits);
            for (int i = tid; i < kBins; i += BLOCK) s_hist[i] = 0;
            __syncthreads();
            for (uint32_t i = tid; i < m; i += BLOCK) {
                const uint64_t ck = s_cand[i];
                if ((ck & pmask) == pfx) atomicAdd(&s_hist[(uint32_t)(ck >> sh) & 0xFFu], 1u);
            }
            __syncthreads();
            if (tid < 64) select_bin(s_hist, need, s_sel, P.status);
            __syncthreads();
            const uint32_t b = s_sel[0], above = s_sel[1], hb = s_sel[2];
            __syncthreads();
            need -= above;
            pfx |= (uint64_t)b << sh;
            pmask |= (uint64_t)0xFFu << sh;
            ++pass;
            mb = hb;
            if (hb == need) { fin_all = true; break; }
        }
        // winners among the candidates, and the small bucket to rank exactly;
        // positions come from a block scan, so the order is reproducible
        uint32_t fw = 0, fb = 0;
        for (uint32_t i = tid; i < m; i += BLOCK) {
            const uint64_t pm = s_cand[i] & pmask;
            fw += (pm > pfx) | (fin_all & (pm == pfx));
            fb += (!fin_all) & (pm == pfx);
        }
        uint32_t ofw, ofb, tfw, tfb;
        block_scan2<BLOCK>(fw, fb, s_scan, ofw, ofb, tfw, tfb);
        for (uint32_t i = tid; i < m; i += BLOCK) {
            const uint64_t ck = s_cand[i];
            const uint64_t pm = ck & pmask;
            if ((pm > pfx) | (fin_all & (pm == pfx))) {
                if (ofw < need0) fout[ofw] = (int32_t)~(uint32_t)ck;
                else raise_flag(P.status, kFlagCapacity);
                ++ofw;
            } else if ((!fin_all) & (pm == pfx)) {
                if (ofb < (uint32_t)kSmall) s_small[ofb] = ck;
                else raise_flag(P.status, kFlagCapacity);
                ++ofb;
            }
        }
        __syncthreads();
        if (!fin_all) {
            const uint32_t ms = tfb > (uint32_t)kSmall ? (uint32_t)kSmall : tfb;
            const uint32_t base = tfw;
            for (uint32_t i = tid; i < ms; i += BLOCK) {
                const uint64_t c = s_small[i];
                uint32_t rank = 0;
                for (uint32_t j = 0; j < ms; ++j) rank += s_small[j] > c;
                if (rank < need) {
                    const uint32_t pos = base + rank;
                    if (pos < need0) fout[pos] = (int32_t)~(uint32_t)c;
                    else raise_flag(P.status, kFlagCapacity);
                }
            }
        }
    }

    if (G > 1) {
        // leave the row's workspace zeroed for the next call
        for (int i = tid; i < pass * kBins; i += BLOCK) ws->hist[i / kBins][i % kBins] = 0u;
        if (tid == 0) {
            ws->arrive = 0u;
            ws->done = 0u;
            ws->out_count = 0u;
            ws->cand_count = 0u;
        }
    }
}

// ----------------------------------------------------------------- host side

using LaunchFn = void (*)(dim3, dim3, hipStream_t, const KParams&);
using OccFn = int (*)(int*, int);

template <int B, int I, bool R>
void launch_variant(dim3 grid, dim3 block, hipStream_t s, const KParams& p) {
    hipLaunchKernelGGL((topk_select_kernel<B, I, R>), grid, block, 0, s, p);
}

template <int B, int I, bool R>
int occupancy_variant(int* nb, int block) {
    return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(nb, topk_select_kernel<B, I, R>, block, 0);
}

struct Variant {
    int block, items, resident;
    LaunchFn launch;
    OccFn occupancy;
};

#define TKS_VARIANT(B, I, R) {B, I, R ? 1 : 0, &launch_variant<B, I, R>, &occupancy_variant<B, I, R>}
const Variant kVariants[] = {
    TKS_VARIANT(256, 4, true),    // 0: 1024 logits per WG
    TKS_VARIANT(256, 8, true),    // 1: 2048
    TKS_VARIANT(256, 16, true),   // 2: 4096
    TKS_VARIANT(512, 32, true),   // 3: 16384
    TKS_VARIANT(512, 64, true),   // 4: 32768
    TKS_VARIANT(1024, 64, true),  // 5: 65536
    TKS_VARIANT(256, 16, false),  // 6: streaming, 4096 per tile
    TKS_VARIANT(1024, 16, false), // 7: streaming, 16384 per tile
};
#undef TKS_VARIANT
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));
constexpr int kFirstStreaming = 6;

struct DeviceInfo {
    int cus = 0;
    int capacity[kNumVariants] = {};  // co-resident WGs per variant on the whole device
};

struct Workspace {
    void* base = nullptr;
    size_t bytes = 0;
};

std::mutex g_mu;
std::map<int, DeviceInfo> g_dev;
std::map<std::pair<int, uintptr_t>, Workspace> g_ws;

constexpr size_t kStatusBytes = 256;

int device_info(int dev, DeviceInfo** out) {
    auto it = g_dev.find(dev);
    if (it == g_dev.end()) {
        DeviceInfo d;
        if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || d.cus <= 0)
            return TOPK_SELECT_ERROR_NO_DEVICE;
        for (int v = 0; v < kNumVariants; ++v) {
            int nb = 0;
            if (kVariants[v].occupancy(&nb, kVariants[v].block) != (int)hipSuccess) return TOPK_SELECT_ERROR_LAUNCH;
            d.capacity[v] = nb * d.cus;
        }
        it = g_dev.emplace(dev, d).first;
    }
    *out = &it->second;
    return TOPK_SELECT_SUCCESS;
}

// Largest number of 16-byte chunks any row can span (rows start on 4-byte
// boundaries; a row that starts mid-chunk spans one chunk more).
int64_t max_row_chunks(const float* logits, int32_t n) {
    if (n % 4 == 0) {
        const int off = (int)(((uintptr_t)logits >> 2) & 3);
        return (off + (int64_t)n + 3) / 4;
    }
    return (3 + (int64_t)n + 3) / 4;
}

int idx_digits_for(int32_t n) {
    uint32_t top = (uint32_t)(n - 1);
    int bits = 0;
    while (top) { ++bits; top >>= 1; }
    return (bits + 7) / 8;
}

struct Launch {
    int variant;
    int G;
    int chunks_per_wg;
};

// Check an explicit shape: resident variants must cover the row in G slices;
// G > 1 needs every WG of the launch co-resident.
int check_shape(const DeviceInfo& d, int64_t rows, int64_t maxc, int v, int G, Launch* L) {
    if (v < 0 || v >= kNumVariants || G < 1) return TOPK_SELECT_ERROR_INVALID_VALUE;
    const Variant& var = kVariants[v];
    const int64_t tile_chunks = (int64_t)var.block * (var.items / 4);
    int64_t cpw = (maxc + G - 1) / G;
    if (var.resident) {
        if (cpw > tile_chunks) return TOPK_SELECT_ERROR_INVALID_VALUE;
        cpw = tile_chunks;
    }
    if (cpw < 1) cpw = 1;
    if (G > 1 && rows * (int64_t)G > (int64_t)d.capacity[v]) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (rows * (int64_t)G > 0x7FFFFFFFll) return TOPK_SELECT_ERROR_INVALID_VALUE;
    L->variant = v;
    L->G = G;
    L->chunks_per_wg = (int)cpw;
    return TOPK_SELECT_SUCCESS;
}

// Default shape: the smallest resident tile whose grid stays within one WG
// per CU (batch-1 rows spread over many WGs, long batches one WG per row);
// otherwise the largest resident tile that fits; otherwise streaming.
int choose_shape(const DeviceInfo& d, int64_t rows, int64_t maxc, Launch* L) {
    const int target = d.cus;
    int best = -1, bestG = 0;
    for (int v = 0; v < kFirstStreaming; ++v) {
        const int64_t tile_chunks = (int64_t)kVariants[v].block * (kVariants[v].items / 4);
        const int64_t G = (maxc + tile_chunks - 1) / tile_chunks;
        const bool fits = G == 1 || rows * G <= (int64_t)d.capacity[v];
        if (!fits) continue;
        if (rows * G <= target) return check_shape(d, rows, maxc, v, (int)G, L);
        best = v;
        bestG = (int)G;
    }
    if (best >= 0) return check_shape(d, rows, maxc, best, bestG, L);
    // streaming: as many WGs per row as can be co-resident, at least one
    const int v = (maxc >= 16384) ? 7 : 6;
    int64_t G = d.capacity[v] / (rows > 0 ? rows : 1);
    const int64_t tile_chunks = (int64_t)kVariants[v].block * (kVariants[v].items / 4);
    const int64_t gmax = (maxc + tile_chunks - 1) / tile_chunks;
    if (G > gmax) G = gmax;
    if (G < 1) G = 1;
    return check_shape(d, rows, maxc, v, (int)G, L);
}

int validate(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k, const int32_t* out) {
    if (rows < 0 || n < 1 || k < 1 || k > n) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (rows == 0) return TOPK_SELECT_SUCCESS;
    if (!logits || !out) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (((uintptr_t)logits & 3) || ((uintptr_t)out & 3) || ((uintptr_t)lengths & 3))
        return TOPK_SELECT_ERROR_INVALID_VALUE;
    const uintptr_t lo_a = (uintptr_t)logits, hi_a = lo_a + (uintptr_t)rows * (uintptr_t)n * 4u;
    const uintptr_t lo_o = (uintptr_t)out, hi_o = lo_o + (uintptr_t)rows * (uintptr_t)k * 4u;
    if (lo_o < hi_a && lo_a < hi_o) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (lengths) {
        const uintptr_t lo_l = (uintptr_t)lengths, hi_l = lo_l + (uintptr_t)rows * 4u;
        if (lo_o < hi_l && lo_l < hi_o) return TOPK_SELECT_ERROR_INVALID_VALUE;
    }
    return TOPK_SELECT_SUCCESS;
}

int get_workspace(int dev, hipStream_t stream, size_t need, Workspace** out) {
    Workspace& w = g_ws[{dev, (uintptr_t)stream}];
    if (w.bytes < need) {
        if (w.base) {
            if (hipStreamSynchronize(stream) != hipSuccess) return TOPK_SELECT_ERROR_LAUNCH;
            (void)hipFree(w.base);
            w.base = nullptr;
            w.bytes = 0;
        }
        void* p = nullptr;
        if (hipMalloc(&p, need) != hipSuccess) {
            (void)hipGetLastError();
            return TOPK_SELECT_ERROR_OUT_OF_MEMORY;
        }
        if (hipMemsetAsync(p, 0, need, stream) != hipSuccess) {
            (void)hipFree(p);
            return TOPK_SELECT_ERROR_LAUNCH;
        }
        w.base = p;
        w.bytes = need;
    }
    *out = &w;
    return TOPK_SELECT_SUCCESS;
}

int run(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k, int32_t* out,
        hipStream_t stream, const topk_select_plan_t* forced) {
    int rc = validate(logits, rows, n, lengths, k, out);
    if (rc != TOPK_SELECT_SUCCESS || rows == 0) return rc;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TOPK_SELECT_ERROR_NO_DEVICE;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceInfo* d = nullptr;
    rc = device_info(dev, &d);
    if (rc != TOPK_SELECT_SUCCESS) return rc;
    const int64_t maxc = max_row_chunks(logits, n);
    Launch L;
    rc = forced ? check_shape(*d, rows, maxc, forced->variant, forced->wgs_per_row, &L)
                : choose_shape(*d, rows, maxc, &L);
    if (rc != TOPK_SELECT_SUCCESS) return rc;
    const size_t ws_bytes = kStatusBytes + (L.G > 1 ? (size_t)rows * sizeof(RowWorkspace) : 0);
    Workspace* w = nullptr;
    rc = get_workspace(dev, stream, ws_bytes, &w);
    if (rc != TOPK_SELECT_SUCCESS) return rc;
    KParams P;
    P.logits = logits;
    P.lengths = lengths;
    P.out = out;
    P.status = reinterpret_cast<uint32_t*>(w->base);
    P.ws = L.G > 1 ? reinterpret_cast<RowWorkspace*>(reinterpret_cast<char*>(w->base) + kStatusBytes) : nullptr;
    P.rows = rows;
    P.n = n;
    P.k = k;
    P.G = L.G;
    P.chunks_per_wg = L.chunks_per_wg;
    P.idx_digits = idx_digits_for(n);
    const Variant& var = kVariants[L.variant];
    (void)hipGetLastError();
    var.launch(dim3((unsigned)(rows * L.G)), dim3((unsigned)var.block), stream, P);
    if (hipGetLastError() != hipSuccess) return TOPK_SELECT_ERROR_LAUNCH;
    return TOPK_SELECT_SUCCESS;
}

}  // namespace tks

extern "C" {

int topk_select(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k,
                int32_t* out_idx, topk_select_stream_t stream) {
    try {
        return tks::run(logits, rows, n, lengths, k, out_idx, (hipStream_t)stream, nullptr);
    } catch (...) {
        return TOPK_SELECT_ERROR_LAUNCH;
    }
}

int topk_select_ex(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k,
                   int32_t* out_idx, topk_select_stream_t stream, const topk_select_plan_t* plan) {
    if (!plan) return TOPK_SELECT_ERROR_INVALID_VALUE;
    try {
        return tks::run(logits, rows, n, lengths, k, out_idx, (hipStream_t)stream, plan);
    } catch (...) {
        return TOPK_SELECT_ERROR_LAUNCH;
    }
}

int topk_select_plan(int32_t rows, int32_t n, int32_t k, topk_select_plan_t* plan) {
    if (!plan || rows < 0 || n < 1 || k < 1 || k > n) return TOPK_SELECT_ERROR_INVALID_VALUE;
    try {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return TOPK_SELECT_ERROR_NO_DEVICE;
        std::lock_guard<std::mutex> lock(tks::g_mu);
        tks::DeviceInfo* d = nullptr;
        int rc = tks::device_info(dev, &d);
        if (rc != TOPK_SELECT_SUCCESS) return rc;
        tks::Launch L;
        // plan for 16-byte aligned logits
        rc = tks::choose_shape(*d, rows > 0 ? rows : 1, tks::max_row_chunks(nullptr, n), &L);
        if (rc != TOPK_SELECT_SUCCESS) return rc;
        plan->variant = L.variant;
        plan->wgs_per_row = L.G;
        plan->block = tks::kVariants[L.variant].block;
        plan->items = tks::kVariants[L.variant].items;
        plan->resident = tks::kVariants[L.variant].resident;
        return TOPK_SELECT_SUCCESS;
    } catch (...) {
        return TOPK_SELECT_ERROR_LAUNCH;
    }
}

int topk_select_num_variants(void) { return tks::kNumVariants; }

int topk_select_variant_info(int32_t v, topk_select_plan_t* plan) {
    if (!plan || v < 0 || v >= tks::kNumVariants) return TOPK_SELECT_ERROR_INVALID_VALUE;
    plan->variant = v;
    plan->wgs_per_row = 1;
    plan->block = tks::kVariants[v].block;
    plan->items = tks::kVariants[v].items;
    plan->resident = tks::kVariants[v].resident;
    return TOPK_SELECT_SUCCESS;
}

int topk_select_device_status(topk_select_stream_t stream, int32_t* flags) {
    if (!flags) return TOPK_SELECT_ERROR_INVALID_VALUE;
    *flags = 0;
    try {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return TOPK_SELECT_ERROR_NO_DEVICE;
        if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return TOPK_SELECT_ERROR_LAUNCH;
        std::lock_guard<std::mutex> lock(tks::g_mu);
        auto it = tks::g_ws.find({dev, (uintptr_t)stream});
        if (it == tks::g_ws.end() || !it->second.base) return TOPK_SELECT_SUCCESS;
        uint32_t v = 0;
        if (hipMemcpy(&v, it->second.base, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess)
            return TOPK_SELECT_ERROR_LAUNCH;
        if (v) {
            const uint32_t zero = 0;
            if (hipMemcpy(it->second.base, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
                return TOPK_SELECT_ERROR_LAUNCH;
        }
        *flags = (int32_t)v;
        return v ? TOPK_SELECT_ERROR_DEVICE_FLAG : TOPK_SELECT_SUCCESS;
    } catch (...) {
        return TOPK_SELECT_ERROR_LAUNCH;
    }
}

int topk_select_release_workspace(void) {
    try {
        std::lock_guard<std::mutex> lock(tks::g_mu);
        int rc = TOPK_SELECT_SUCCESS;
        for (auto& kv : tks::g_ws) {
            if (kv.second.base) {
                int cur = 0;
                (void)hipGetDevice(&cur);
                (void)hipSetDevice(kv.first.first);
                if (hipDeviceSynchronize() != hipSuccess) rc = TOPK_SELECT_ERROR_LAUNCH;
                if (hipFree(kv.second.base) != hipSuccess) rc = TOPK_SELECT_ERROR_LAUNCH;
                (void)hipSetDevice(cur);
            }
        }
        tks::g_ws.clear();
        return rc;
    } catch (...) {
        return TOPK_SELECT_ERROR_LAUNCH;
    }
}

const char* topk_select_error_string(int status) {
    switch (status) {
        case TOPK_SELECT_SUCCESS: return "success";
        case TOPK_SELECT_ERROR_INVALID_VALUE: return "invalid argument (nothing was enqueued)";
        case TOPK_SELECT_ERROR_OUT_OF_MEMORY: return "workspace allocation failed (nothing was enqueued)";
        case TOPK_SELECT_ERROR_LAUNCH: return "HIP call or kernel launch failed";
        case TOPK_SELECT_ERROR_NO_DEVICE: return "no usable HIP device is current";
        case TOPK_SELECT_ERROR_DEVICE_FLAG: return "a kernel raised a device-side error flag";
        default: return "unknown status";
    }
}

int topk_select_version(void) { return TOPK_SELECT_VERSION; }

}  // extern "C"
