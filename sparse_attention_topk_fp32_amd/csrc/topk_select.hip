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

constexpr int kCap = 4096;          // candidate buffer capacity (elements)
constexpr int kSmall = 256;         // bucket size ranked directly by the finisher
constexpr int kMaxPasses = 8;       // rounds after the first digit (8-bit digits)
constexpr int kStageLds = 8192;     // staged (key, index) entries a one-WG row may keep in LDS
constexpr int kFinCopies = 8;       // LDS histogram copies for the finisher's rounds
constexpr int kMergeCopies = 8;     // global copies of a row's 256-bin histogram (WG w adds into copy w mod 8)
constexpr int kLineWords = 32;      // one 128-byte line
constexpr uint32_t kFlagTimeout = 1u;
constexpr uint32_t kFlagCapacity = 2u;
// Bound on a cross-workgroup wait, in ticks of the 100 MHz constant clock
// (s_memrealtime): 2 s, far beyond any legitimate wait.
constexpr uint64_t kSpinLimitTicks = 200000000ull;

// Per-row scratch for rows spread over several workgroups.  Every field is
// zero between calls (the finishing WG of each row clears what it used).
// All cross-workgroup traffic goes through device-scope atomic operations
// (read-modify-writes, loads and stores), which are performed at the
// device's coherence point; their order within a wave is enforced with
// s_waitcnt vmcnt(0).  No L2 write-back or invalidate fence is needed.
struct alignas(256) RowWorkspace {
    uint32_t hist0[4096];                            // first-digit counts (4096 bins, or 8 copies of 256)
    uint32_t hist[kMaxPasses][kMergeCopies][256];    // later rounds (8-bit digits)
    uint32_t arrive[kMergeCopies * kLineWords];      // barrier arrivals, one counter per line
    uint32_t done;                                   // WGs finished with the row
    uint32_t reserve;                                // staged entries reserved in the row's stage
    uint32_t pad[62];
};

struct KParams {
    const float* logits;
    const int32_t* lengths;
    int32_t* out;
    RowWorkspace* ws;       // per row, when G > 1
    uint64_t* stage;        // per row, stage_cap entries: (key << 32) | ~index, or null
    uint32_t* status;
    int32_t rows, n, k;
    int32_t G;              // workgroups per row
    int32_t chunks_per_wg;  // 16-byte chunks in one WG's slice
    int32_t idx_bits;       // bits of the index that vary (multiple of 8, <= 32)
    int32_t stage_cap;      // entries per row in `stage`
};

// ----------------------------------------------------------------- device helpers

// Mapping step: float -> unsigned key with key(a) < key(b) iff a < b for
// non-NaN values.  Adding +0.0 turns -0.0 into +0.0 (IEEE round to nearest)
// and leaves every other value, subnormals included, unchanged, so -0.0 and
// +0.0 get the same key and tie.  Negative values have all bits flipped,
// non-negative ones only the sign bit.  Key 0 marks "no element": only the
// NaN pattern 0xFFFFFFFF also maps there (NaN is outside the contract).
__device__ __forceinline__ uint32_t key_of(float x) {
    const uint32_t u = __float_as_uint(x + 0.0f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ uint32_t lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// A value every lane holds identically (read from LDS after a barrier):
// make it scalar so the loop state and its branches stay in SGPRs.
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ void raise_flag(uint32_t* status, uint32_t f) {
    __hip_atomic_fetch_or(status, f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device-scope atomic accessors (relaxed): performed at the coherence point.
template <typename T>
__device__ __forceinline__ T ld_dev(T* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T add_dev(T* p, T v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_memory() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier that orders LDS only.  __syncthreads() also makes the
// compiler wait for this wave's outstanding global stores (vmcnt), which
// puts a memory round trip after every phase that writes output; here the
// global data crossing a barrier is published explicitly with wait_memory()
// and read with device-scope loads, so LDS ordering is all a barrier needs.
__device__ __forceinline__ void lds_sync() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Bounded wait until *ctr >= target (device scope), by one thread.
__device__ void spin_until(uint32_t* ctr, uint32_t target, uint32_t* status) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (ld_dev(ctr) < target) {
        __builtin_amdgcn_s_sleep(1);
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimitTicks) {
            raise_flag(status, kFlagTimeout);
            break;
        }
    }
}

// Row barrier for the G WGs of a row: WG w counts on line w mod 8, and
// threads 0..7 each wait for their line to reach its round's total.  The
// caller has made its own preceding device-scope operations complete.
__device__ void row_barrier(RowWorkspace* ws, int G, int w, int round, uint32_t* status) {
    if (threadIdx.x == 0) add_dev(&ws->arrive[(w % kMergeCopies) * kLineWords], 1u);
    const int t = threadIdx.x;
    if (t < kMergeCopies && t < G) {
        const uint32_t per_line = (uint32_t)((G - t + kMergeCopies - 1) / kMergeCopies);
        spin_until(&ws->arrive[t * kLineWords], per_line * (uint32_t)(round + 1), status);
    }
    lds_sync();
}

// Inclusive scan across the 64 lanes of a wave with DPP lane moves (no LDS
// round trip): shifts by 1, 2, 4, 8 inside each row of 16 lanes, then the
// last lane of a row is broadcast into the rows above it.  Lanes with no
// source lane read 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Block-wide exclusive scan of two counters at once.  Every thread of the
// block calls it; returns this thread's exclusive prefixes and the totals.
template <int BLOCK>
__device__ __forceinline__ void block_scan2(uint32_t a, uint32_t b, uint32_t* s_w /* [2 * BLOCK / 64] */,
                                            uint32_t& ea, uint32_t& eb, uint32_t& ta, uint32_t& tb) {
    constexpr int NW = BLOCK / 64;
    const uint32_t lane = lane_id();
    const uint32_t wid = threadIdx.x / 64;
    const uint32_t ia = wave_inclusive_scan(a), ib = wave_inclusive_scan(b);
    if (lane == 63) { s_w[wid] = ia; s_w[NW + wid] = ib; }
    lds_sync();
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
    ta = uniform(ta);
    tb = uniform(tb);
    lds_sync();  // s_w may be reused right after
}

// Digit schedule over the 64-bit composite (key << 32) | ~index, by the
// number r of top bits already resolved: the key's 32 bits in digits of up
// to 8 bits (the first digit may be wider), then the index bits that vary.
// ~index has its top (32 - idx_bits) bits set for every valid index, so they
// are skipped.
__device__ __forceinline__ int digit_width(int r) { return r < 32 ? min(8, 32 - r) : min(8, 64 - r); }

struct Prefix {
    uint32_t kpfx, kmask;  // resolved key bits
    uint32_t ipfx, imask;  // resolved ~index bits
    int r;                 // resolved bits of the composite
    // Value selects only (no branch that picks a field to update), so the
    // struct stays in registers.
    __device__ void add_digit(uint32_t b, int width, int idx_bits) {
        const int sh = 64 - r - width;
        const bool in_key = sh >= 32;
        const int s = in_key ? sh - 32 : sh;
        const uint32_t bb = b << s, mm = ((1u << width) - 1u) << s;  // width <= 12
        kpfx |= in_key ? bb : 0u;
        kmask |= in_key ? mm : 0u;
        ipfx |= in_key ? 0u : bb;
        imask |= in_key ? 0u : mm;
        r += width;
        // past the key: the top (32 - idx_bits) bits of ~index are constant ones
        const bool jump = r == 32;
        const uint32_t ones = idx_bits < 32 ? ~((1u << idx_bits) - 1u) : 0u;
        ipfx |= jump ? ones : 0u;
        imask |= jump ? ones : 0u;
        r = jump ? 64 - idx_bits : r;
    }
    __device__ uint64_t pfx64() const { return ((uint64_t)kpfx << 32) | ipfx; }
    __device__ uint64_t mask64() const { return ((uint64_t)kmask << 32) | imask; }
};

// Thresholding step over an NB-bin histogram held as NC LDS copies (stride
// NB + 1 words).  Finds the bin b holding the element of rank `need`
// (1-based, from the top): the caller gets b, the count above b and the
// count in b through s_sel.  Each owning thread sums the copies of its bins,
// optionally merges them across the row's WGs (G > 1: add into a global
// histogram, barrier, read back the sums), then one block scan over the
// owners' sums, taken from the top bin down, locates b.
template <int BLOCK, int NB, int NC>
__device__ void select_bin(const uint32_t* h, uint32_t bin0_sub, uint32_t need, int G, RowWorkspace* ws,
                           uint32_t* gm, int gcopies, int w, int round, uint32_t* s_sel, uint32_t* s_scan,
                           uint32_t* status) {
    constexpr int OWN = (NB + BLOCK - 1) / BLOCK;      // bins per owning thread
    constexpr int OWNERS = (NB + OWN - 1) / OWN;       // the last group may be partial
    const int t = threadIdx.x;
    const bool owner = t < OWNERS;
    const int g = OWNERS - 1 - t;  // thread 0 owns the top bins
    uint32_t tot[OWN];
#pragma unroll
    for (int i = 0; i < OWN; ++i) tot[i] = 0;
    if (owner) {
        // copy by copy, with a few LDS reads in flight at a time (the
        // caller's resident keys are live here)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int i = 0; i < OWN; ++i) {
                const int bin = g * OWN + i;
                if (bin < NB) tot[i] += h[c * (NB + 1) + bin];
            }
            if (OWN * (c + 1) % 8 == 0) __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < OWN; ++i)
            if (g * OWN + i == 0) tot[i] -= bin0_sub;
    }
    if (G > 1) {
        if (owner) {
            uint32_t* dst = gm + (gcopies > 1 ? (w % gcopies) * NB : 0);
#pragma unroll
            for (int i = 0; i < OWN; ++i)
                if (tot[i]) add_dev(&dst[g * OWN + i], tot[i]);
        }
        wait_memory();
        lds_sync();
        row_barrier(ws, G, w, round, status);
        if (owner) {
            const int nc = G < gcopies ? G : gcopies;
#pragma unroll
            for (int i = 0; i < OWN; ++i) {
                const int bin = g * OWN + i;
                uint32_t v = 0;
                if (bin < NB)
                    for (int c = 0; c < nc; ++c) v += ld_dev(&gm[c * NB + bin]);
                tot[i] = v;
            }
        }
    }
    uint32_t gsum = 0;
#pragma unroll
    for (int i = 0; i < OWN; ++i) gsum += tot[i];
    if (t == 0) s_sel[2] = 0xFFFFFFFFu;  // "not found" until an owner writes
    uint32_t excl, unused, total, unused2;
    block_scan2<BLOCK>(gsum, 0u, s_scan, excl, unused, total, unused2);
    if (owner && excl < need && need <= excl + gsum) {
        uint32_t above = excl;
#pragma unroll
        for (int i = OWN - 1; i >= 0; --i) {
            if (above + tot[i] >= need) {
                s_sel[0] = (uint32_t)(g * OWN + i);
                s_sel[1] = above;
                s_sel[2] = tot[i];
                break;
            }
            above += tot[i];
        }
    }
    lds_sync();
    if (uniform(s_sel[2]) == 0xFFFFFFFFu) {  // fewer elements than `need`: cannot happen for valid input
        lds_sync();
        if (t == 0) {
            s_sel[0] = 0; s_sel[1] = 0; s_sel[2] = 0;
            raise_flag(status, kFlagCapacity);
        }
        lds_sync();
    }
}

// ----------------------------------------------------------------- the kernel
//
// BLOCK threads per WG; ITEMS logits per thread per tile; FIRST_BITS = width
// of the first digit (8: 256 bins in 32 LDS copies; 12: 4096 bins in 4
// copies); RESIDENT: the slice is one tile kept in VGPRs across rounds;
// MULTI: rows may be spread over several WGs (G > 1).  Variants without
// MULTI carry none of the cross-workgroup code, which keeps their register
// budget for the resident keys.

template <int BLOCK, int ITEMS, int FIRST_BITS, bool RESIDENT, bool MULTI>
__global__ __launch_bounds__(BLOCK) void topk_select_kernel(const KParams P) {
    static_assert(ITEMS % 4 == 0, "ITEMS counts whole 16-byte chunks");
    static_assert(BLOCK % 64 == 0 && BLOCK >= 256, "one bin per thread in the 256-bin rounds");
    static_assert(FIRST_BITS == 8 || FIRST_BITS == 12, "first digit of 8 or 12 bits");
    constexpr int CHUNKS = ITEMS / 4;              // chunks per thread per tile
    constexpr int TILE_CHUNKS = BLOCK * CHUNKS;    // chunks per tile
    constexpr int NB0 = 1 << FIRST_BITS;           // first-digit bins
    constexpr int NC0 = FIRST_BITS == 8 ? 32 : 4;  // LDS copies of the first-digit histogram
    constexpr int NC8 = 32;                        // LDS copies in the later 8-bit rounds
    // LDS stage: a one-WG row stages at most its own tile; the finisher of
    // a split row pulls the row's whole staging area (up to kStageLds).
    constexpr int STAGE = (RESIDENT && !MULTI && BLOCK * ITEMS < kStageLds) ? BLOCK * ITEMS : kStageLds;
    constexpr int H0_WORDS = NC0 * (NB0 + 1);
    constexpr int H8_WORDS = NC8 * 257;

    // The rounds' histograms and the staged selection are never live at the
    // same time, so they share LDS.
    union BigLds {
        uint32_t h0[H0_WORDS];
        uint32_t h8[H8_WORDS];
        uint64_t stage[STAGE];
    };
    __shared__ BigLds s_big;
    __shared__ uint64_t s_cand[kCap];
    __shared__ uint32_t s_fin_hist[kFinCopies * 257];
    __shared__ uint64_t s_small[kSmall];
    __shared__ uint32_t s_scan[2 * (BLOCK / 64)];
    __shared__ uint32_t s_sel[3];   // threshold bin, count above it, count in it
    __shared__ uint32_t s_bc[2];    // broadcast: stage base, last-WG flag

    const int tid = threadIdx.x;
    const int G = MULTI ? P.G : 1;
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

    RowWorkspace* ws = (MULTI && P.ws) ? P.ws + row : nullptr;
    const int off = (int)(((uintptr_t)p >> 2) & 3);  // elements before the first 16-byte boundary
    const int nchunks = (off + L + 3) >> 2;
    const int c_begin = w * P.chunks_per_wg;
    const int c_end = min(nchunks, c_begin + P.chunks_per_wg);
    // chunks whose four elements are all valid
    const int cf_lo = max(c_begin, off ? 1 : 0);
    const int cf_hi = min(c_end, (L + off) >> 2);
    // slots of the slice's chunks that hold no element (key 0): at most the
    // three before element 0 and the three past L; the first-digit
    // histogram counts them in bin 0 and subtracts them after
    const int valid = c_end > c_begin ? max(0, min(L, 4 * c_end - off) - max(0, 4 * c_begin - off)) : 0;
    const uint32_t n_empty = c_end > c_begin ? (uint32_t)(4 * (c_end - c_begin) - valid) : 0u;

    uint32_t keys[ITEMS];
    const float* __restrict__ pa = p - off;  // 16-byte aligned

    // Load one tile: chunk c of the row is the aligned 16-byte block holding
    // elements [4c - off, 4c - off + 4).  A chunk with at least one valid
    // element lies in the page of that element, so it is read whole; lanes
    // past the slice re-read chunk 0 (valid: L > k >= 1).  All loads are
    // issued before any is used.
    auto load_tile = [&](int c_tile) {
        const char* const base = reinterpret_cast<const char*>(pa);  // uniform base, 32-bit offsets
#pragma unroll
        for (int j = 0; j < CHUNKS; ++j) {  // raw bits straight into the key registers
            const int c = c_tile + j * BLOCK + tid;
            const uint32_t byte_off = (uint32_t)(c < c_end ? c : 0) * 16u;
            const uint4 v = *reinterpret_cast<const uint4*>(base + byte_off);
            keys[4 * j + 0] = v.x;
            keys[4 * j + 1] = v.y;
            keys[4 * j + 2] = v.z;
            keys[4 * j + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < CHUNKS; ++j) {  // then mapped in place
            const int c = c_tile + j * BLOCK + tid;
            if (c >= cf_lo && c < cf_hi) {
#pragma unroll
                for (int e = 0; e < 4; ++e) keys[4 * j + e] = key_of(__uint_as_float(keys[4 * j + e]));
            } else {
                const int e0 = 4 * c - off;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = (c < c_end) & ((uint32_t)(e0 + e) < (uint32_t)L);
                    keys[4 * j + e] = ok ? key_of(__uint_as_float(keys[4 * j + e])) : 0u;
                }
            }
        }
    };
    // f(key, index) for every element of one tile; element e of chunk j has
    // index ibase + 4 * BLOCK * j + e.
    auto visit_tile = [&](int c_tile, auto&& f) {
        int ibase = 4 * (c_tile + tid) - off;
        __asm__ volatile("" : "+v"(ibase));  // indices are recomputed per visit, never kept live
#pragma unroll
        for (int j = 0; j < CHUNKS; ++j) {
#pragma unroll
            for (int e = 0; e < 4; ++e) f(keys[4 * j + e], ibase + 4 * BLOCK * j + e);
            // keep each chunk's temporaries local: without this the scheduler
            // hoists every element's address ahead of the LDS operations
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Visit every slot of the slice (uniform trip count across the WG).
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

    // f(key) for every slot of the chunks in [c_begin, c_end): chunks past
    // the slice are skipped (one test per chunk, not per element)
    auto visit_chunks = [&](auto&& f) {
        auto tile = [&](int c_tile) {
#pragma unroll
            for (int j = 0; j < CHUNKS; ++j) {
                if (c_tile + j * BLOCK + tid < c_end) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) f(keys[4 * j + e]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        if constexpr (RESIDENT) {
            tile(c_begin);
        } else {
            for (int ct = c_begin; ct < c_end; ct += TILE_CHUNKS) {
                load_tile(ct);
                tile(ct);
            }
        }
    };

    if constexpr (RESIDENT) load_tile(c_begin);

    // ---------------- screening rounds over the whole row
    Prefix pf{0u, 0u, 0u, 0u, 0};
    uint32_t need = (uint32_t)k;
    int round = 0;
    bool all_sel = false;
    for (;;) {
        if constexpr (RESIDENT) {
            // Opaque to the optimiser: stops it from hoisting per-element
            // values (one lane mask or VGPR per element) out of the rounds.
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) __asm__ volatile("" : "+v"(keys[i]));
        }
        int width;
        if (pf.r == 0) {
            // first digit: every slot adds into bin (key >> (32 - FIRST_BITS));
            // empty slots (key 0) land in bin 0 and are subtracted after
            width = FIRST_BITS;
            for (int i = tid; i < H0_WORDS / 4; i += BLOCK) reinterpret_cast<uint4*>(s_big.h0)[i] = uint4{0u, 0u, 0u, 0u};
            for (int i = H0_WORDS / 4 * 4 + tid; i < H0_WORDS; i += BLOCK) s_big.h0[i] = 0u;
            lds_sync();
            uint32_t* const hc = s_big.h0 + (tid % NC0) * (NB0 + 1);
            visit_chunks([&](uint32_t key) { atomicAdd(&hc[key >> (32 - FIRST_BITS)], 1u); });
            lds_sync();
            select_bin<BLOCK, NB0, NC0>(s_big.h0, n_empty, need, G, ws, ws ? ws->hist0 : nullptr,
                                        FIRST_BITS == 8 ? kMergeCopies : 1, w, round, s_sel, s_scan, P.status);
        } else {
            width = digit_width(pf.r);
            const int sh = 64 - pf.r - width;
            const uint32_t dmask = (1u << width) - 1u;
            for (int i = tid; i < H8_WORDS / 4; i += BLOCK) reinterpret_cast<uint4*>(s_big.h8)[i] = uint4{0u, 0u, 0u, 0u};
            for (int i = H8_WORDS / 4 * 4 + tid; i < H8_WORDS; i += BLOCK) s_big.h8[i] = 0u;
            lds_sync();
            uint32_t* const hc = s_big.h8 + (tid % NC8) * 257;
            if (sh >= 32) {
                const int ks = sh - 32;
                const uint32_t km = pf.kmask, kp = pf.kpfx;
                visit([&](uint32_t key, int) {
                    if ((key != 0u) & ((key & km) == kp)) atomicAdd(&hc[(key >> ks) & dmask], 1u);
                });
            } else {
                const uint32_t kp = pf.kpfx, im = pf.imask, ip = pf.ipfx;
                visit([&](uint32_t key, int idx) {
                    const uint32_t ni = ~(uint32_t)idx;
                    if ((key != 0u) & (key == kp) & ((ni & im) == ip)) atomicAdd(&hc[(ni >> sh) & dmask], 1u);
                });
            }
            lds_sync();
            select_bin<BLOCK, 256, NC8>(s_big.h8, 0u, need, G, ws, ws ? &ws->hist[round - 1][0][0] : nullptr,
                                        kMergeCopies, w, round, s_sel, s_scan, P.status);
        }
        const uint32_t b = uniform(s_sel[0]), above = uniform(s_sel[1]), hb = uniform(s_sel[2]);
        lds_sync();
        need -= above;
        pf.add_digit(b, width, P.idx_bits);
        ++round;
        if (hb == need) { all_sel = true; break; }
        if (hb <= (uint32_t)kCap || pf.r >= 64 || round > kMaxPasses) break;
    }

    // ---------------- collection over the row
    // Selected = composite prefix at or above the threshold prefix: every
    // element above the bucket plus the bucket itself.  They are staged as
    // (key << 32) | ~index; the finisher splits them.
    const bool key_only = pf.imask == 0u;
    const uint32_t lo = pf.kpfx > 1u ? pf.kpfx : 1u;
    auto selected = [&](uint32_t key, int idx) -> bool {
        if (key_only) return key >= lo;
        return (key != 0u) & ((key > pf.kpfx) | ((key == pf.kpfx) & ((~(uint32_t)idx & pf.imask) >= pf.ipfx)));
    };
    uint32_t nsel = 0;
    if constexpr (RESIDENT) {
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) __asm__ volatile("" : "+v"(keys[i]));
    }
    if (key_only) visit([&](uint32_t key, int) { nsel += key >= lo; });
    else visit([&](uint32_t key, int idx) { nsel += selected(key, idx); });
    uint32_t off_sel, unused, tot_sel, unused2;
    block_scan2<BLOCK>(nsel, 0u, s_scan, off_sel, unused, tot_sel, unused2);
    bool in_lds = (G == 1) && tot_sel <= (uint32_t)STAGE;
    uint64_t* const gstage = P.stage ? P.stage + (size_t)row * (size_t)P.stage_cap : nullptr;
    uint32_t cap = in_lds ? (uint32_t)STAGE : (uint32_t)P.stage_cap;
    if (!in_lds && !gstage) cap = 0;
    if (G > 1) {
        if (tid == 0) s_bc[0] = tot_sel ? add_dev(&ws->reserve, tot_sel) : 0u;
        lds_sync();
        off_sel += uniform(s_bc[0]);
    }
    // Capacity holds by construction (the rounds end with the bucket at most
    // kCap, so at most k + kCap entries); checked once, never per element.
    const bool fits = tot_sel <= cap;
    if (!fits && tid == 0) raise_flag(P.status, kFlagCapacity);
    if constexpr (RESIDENT) {  // no per-element result of the count pass stays live
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) __asm__ volatile("" : "+v"(keys[i]));
    }
    // one write loop per destination; per-thread loops: no barrier or wave
    // operation inside.  The key is copied before it is paired with the
    // index, so resident keys are not pinned to the high half of a register
    // pair (one extra VGPR per key).
    auto entry = [](uint32_t key, int idx) -> uint64_t {
        uint32_t kc = key;
        __asm__ volatile("" : "+v"(kc));
        return ((uint64_t)kc << 32) | (uint64_t)(~(uint32_t)idx);
    };
    if (fits && nsel) {
        if (!key_only) {
            visit([&](uint32_t key, int idx) {
                if (selected(key, idx)) {
                    const uint64_t ck = entry(key, idx);
                    if (in_lds) s_big.stage[off_sel] = ck;
                    else st_dev(&gstage[off_sel], ck);
                    ++off_sel;
                }
            });
        } else if (in_lds) {
            visit([&](uint32_t key, int idx) {
                if (key >= lo) s_big.stage[off_sel++] = entry(key, idx);
            });
        } else if (G > 1) {  // read by another WG: device-scope stores
            visit([&](uint32_t key, int idx) {
                if (key >= lo) st_dev(&gstage[off_sel++], entry(key, idx));
            });
        } else {
            visit([&](uint32_t key, int idx) {
                if (key >= lo) st_dev(&gstage[off_sel++], entry(key, idx));
            });
        }
    }

    if (!in_lds) wait_memory();  // the staging area is read by other threads (or WGs) next
    uint32_t m_sel = tot_sel;  // staged entries of the row
    if (G > 1) {
        // the last WG of the row to get here finishes it and clears the workspace
        wait_memory();
        lds_sync();
        if (tid == 0) s_bc[1] = (add_dev(&ws->done, 1u) == (uint32_t)G - 1u) ? 1u : 0u;
        lds_sync();
        if (uniform(s_bc[1]) == 0u) return;
        m_sel = uniform(ld_dev(&ws->reserve));
        if (m_sel > cap) m_sel = cap;
        if (m_sel <= (uint32_t)STAGE) {
            // the whole staging area on chip: eight independent loads in
            // flight per thread per step instead of one dependent chain
            for (uint32_t i0 = 0; i0 < m_sel; i0 += 8u * BLOCK) {
                uint64_t v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t i = i0 + u * BLOCK + tid;
                    v[u] = i < m_sel ? ld_dev(&gstage[i]) : 0ull;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t i = i0 + u * BLOCK + tid;
                    if (i < m_sel) s_big.stage[i] = v[u];
                }
            }
            in_lds = true;
        }
    }
    lds_sync();
    if (m_sel > cap) m_sel = cap;

    // ---------------- on-chip finish
    // Two-way partition of n entries (get(i) supplies entry i): cls(v) is 1
    // (-> putA), 2 (-> putB) or 0 (dropped).  Positions follow entry order
    // through a block scan, so the order is reproducible.  Loads are taken
    // eight per thread at a time before any store, so they overlap instead
    // of waiting behind the previous entry's LDS store.  When a total would
    // exceed its bound, a flag is raised and nothing is written.
    constexpr int U = 8;
    auto partition = [&](uint32_t n, auto&& get, auto&& cls, auto&& putA, auto&& putB, uint32_t capA,
                         uint32_t capB, uint32_t& tA, uint32_t& tB) {
        uint32_t ca = 0, cb = 0;
        for (uint32_t i0 = 0; i0 < n; i0 += U * BLOCK) {
            uint64_t v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = i0 + u * BLOCK + tid;
                v[u] = i < n ? get(i) : 0ull;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t c = (i0 + u * BLOCK + tid < n) ? cls(v[u]) : 0u;
                ca += c == 1u;
                cb += c == 2u;
            }
        }
        uint32_t oa, ob;
        block_scan2<BLOCK>(ca, cb, s_scan, oa, ob, tA, tB);
        const bool ok = tA <= capA && tB <= capB;
        if (!ok && tid == 0) raise_flag(P.status, kFlagCapacity);
        if (ok && (ca | cb)) {
            for (uint32_t i0 = 0; i0 < n; i0 += U * BLOCK) {
                uint64_t v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t i = i0 + u * BLOCK + tid;
                    v[u] = i < n ? get(i) : 0ull;
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t c = (i0 + u * BLOCK + tid < n) ? cls(v[u]) : 0u;
                    if (c == 1u) putA(oa++, v[u]);
                    else if (c == 2u) putB(ob++, v[u]);
                }
            }
        }
        lds_sync();
    };

    // Split the staged entries: above the threshold prefix (or the whole
    // bucket when it is taken entirely) -> output; in the bucket -> LDS
    // candidates.
    const uint64_t pfx0 = pf.pfx64(), pmask0 = pf.mask64();
    const uint32_t nwin_total = (uint32_t)k - (all_sel ? 0u : need);
    uint32_t tw = 0, tb = 0;
    auto put_out = [&](uint32_t pos, uint64_t v) { out[pos] = (int32_t)~(uint32_t)v; };
    auto put_cand = [&](uint32_t pos, uint64_t v) { s_cand[pos] = v; };
    auto cls0 = [&](uint64_t v) -> uint32_t {
        const uint64_t pm = v & pmask0;
        if ((pm > pfx0) | (all_sel & (pm == pfx0))) return 1u;
        return ((!all_sel) & (pm == pfx0)) ? 2u : 0u;
    };
    if (in_lds) {
        partition(m_sel, [&](uint32_t i) { return s_big.stage[i]; }, cls0, put_out, put_cand, nwin_total,
                  (uint32_t)kCap, tw, tb);
    } else {
        partition(m_sel, [&](uint32_t i) { return ld_dev(&gstage[i]); }, cls0, put_out, put_cand, nwin_total,
                  (uint32_t)kCap, tw, tb);
    }
    if (tw != nwin_total && tid == 0) raise_flag(P.status, kFlagCapacity);

    if (!all_sel && tb <= (uint32_t)kCap) {
        const uint32_t m = tb;
        int32_t* __restrict__ fout = out + nwin_total;  // `need` slots remain
        const uint32_t need0 = need;
        uint64_t pfx = pfx0, pmask = pmask0;
        bool fin_all = false;
        uint32_t mb = m;
        int fround = 0;
        while (mb > (uint32_t)kSmall && pf.r < 64) {
            const int width = digit_width(pf.r);
            const int sh = 64 - pf.r - width;
            const uint32_t dmask = (1u << width) - 1u;
            for (int i = tid; i < kFinCopies * 257; i += BLOCK) s_fin_hist[i] = 0u;
            lds_sync();
            uint32_t* const fc = s_fin_hist + (tid % kFinCopies) * 257;
            for (uint32_t i0 = 0; i0 < m; i0 += U * BLOCK) {
                uint64_t v[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t i = i0 + u * BLOCK + tid;
                    v[u] = i < m ? s_cand[i] : 0ull;
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if ((i0 + u * BLOCK + tid < m) & ((v[u] & pmask) == pfx))
                        atomicAdd(&fc[(uint32_t)(v[u] >> sh) & dmask], 1u);
                }
            }
            lds_sync();
            select_bin<BLOCK, 256, kFinCopies>(s_fin_hist, 0u, need, 1, nullptr, nullptr, 1, 0, fround,
                                               s_sel, s_scan, P.status);
            const uint32_t b = uniform(s_sel[0]), above = uniform(s_sel[1]), hb = uniform(s_sel[2]);
            lds_sync();
            need -= above;
            pf.add_digit(b, width, P.idx_bits);
            pfx = pf.pfx64();
            pmask = pf.mask64();
            ++fround;
            mb = hb;
            if (hb == need) { fin_all = true; break; }
        }
        // winners among the candidates, and the small bucket to rank exactly
        uint32_t tfw = 0, tfb = 0;
        partition(
            m, [&](uint32_t i) { return s_cand[i]; },
            [&](uint64_t v) -> uint32_t {
                const uint64_t pm = v & pmask;
                if ((pm > pfx) | (fin_all & (pm == pfx))) return 1u;
                return ((!fin_all) & (pm == pfx)) ? 2u : 0u;
            },
            [&](uint32_t pos, uint64_t v) { fout[pos] = (int32_t)~(uint32_t)v; },
            [&](uint32_t pos, uint64_t v) { s_small[pos] = v; }, need0, (uint32_t)kSmall, tfw, tfb);
        if (!fin_all && tfb <= (uint32_t)kSmall) {
            const uint32_t ms = tfb;
            const uint32_t base = tfw;
            for (uint32_t i = tid; i < ms; i += BLOCK) {
                const uint64_t c = s_small[i];
                uint32_t rank = 0;
#pragma unroll 8
                for (uint32_t j = 0; j < ms; ++j) rank += s_small[j] > c;
                const uint32_t pos = base + rank;
                if ((rank < need) & (pos < need0)) fout[pos] = (int32_t)~(uint32_t)c;
            }
        }
    }

    if (G > 1) {
        // leave the row's workspace zeroed for the next call
        for (int i = tid; i < 4096; i += BLOCK) st_dev(&ws->hist0[i], 0u);
        const int ncopy = G < kMergeCopies ? G : kMergeCopies;
        for (int i = tid; i < (round - 1) * kMergeCopies * 256; i += BLOCK) {
            const int c = (i / 256) % kMergeCopies;
            if (c < ncopy) st_dev(&ws->hist[i / (kMergeCopies * 256)][c][i % 256], 0u);
        }
        if (tid < kMergeCopies) st_dev(&ws->arrive[tid * kLineWords], 0u);
        if (tid == 0) {
            st_dev(&ws->done, 0u);
            st_dev(&ws->reserve, 0u);
        }
    }
}

// ----------------------------------------------------------------- host side

using LaunchFn = void (*)(dim3, dim3, hipStream_t, const KParams&);
using OccFn = int (*)(int*, int);

template <int B, int I, int F, bool R, bool M>
void launch_variant(dim3 grid, dim3 block, hipStream_t s, const KParams& p) {
    hipLaunchKernelGGL((topk_select_kernel<B, I, F, R, M>), grid, block, 0, s, p);
}

template <int B, int I, int F, bool R, bool M>
int occupancy_variant(int* nb, int block) {
    return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(nb, topk_select_kernel<B, I, F, R, M>, block, 0);
}

struct Variant {
    int block, items, first_bits, resident, multi;
    int stage_lds;  // staged entries a one-WG row keeps in LDS
    LaunchFn launch;
    OccFn occupancy;
};

constexpr int stage_lds_of(int b, int i, bool r) { return (r && b * i < kStageLds) ? b * i : kStageLds; }

#define TKS_VARIANT(B, I, F, R, M)                                                               \
    {B, I, F, R ? 1 : 0, M ? 1 : 0, stage_lds_of(B, I, R), &launch_variant<B, I, F, R, M>, \
     &occupancy_variant<B, I, F, R, M>}
const Variant kVariants[] = {
    TKS_VARIANT(256, 4, 8, true, true),      // 0: 1024 logits per WG, 8-bit first digit (many WGs per row)
    TKS_VARIANT(256, 8, 8, true, true),      // 1: 2048
    TKS_VARIANT(256, 16, 8, true, true),     // 2: 4096
    TKS_VARIANT(512, 32, 8, true, true),     // 3: 16384
    TKS_VARIANT(512, 64, 8, true, true),     // 4: 32768
    TKS_VARIANT(256, 16, 12, true, false),   // 5: 4096, 12-bit first digit, one WG per row
    TKS_VARIANT(512, 32, 12, true, false),   // 6: 16384
    TKS_VARIANT(512, 64, 12, true, true),    // 7: 32768 (also several WGs per row)
    TKS_VARIANT(1024, 32, 12, true, false),  // 8: 32768
    TKS_VARIANT(1024, 16, 12, false, true),  // 9: streaming, 16384 per tile
    TKS_VARIANT(256, 16, 8, false, true),    // 10: streaming, 4096 per tile
};
#undef TKS_VARIANT
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

struct DeviceInfo {
    int cus = 0;
    int capacity[kNumVariants] = {};  // co-resident WGs per variant on the whole device
};

// Scratch of one (device, stream).  `base` holds the status word and the
// per-row workspaces at fixed offsets (row r always at the same address,
// whatever the row count of a call); it is zeroed when allocated and left
// zeroed by every kernel.  `stage` holds staged entries; it needs no
// initial value and lives in its own allocation so that it never overlaps
// a row workspace of a later call.
struct Workspace {
    void* base = nullptr;
    size_t bytes = 0;
    void* stage = nullptr;
    size_t stage_bytes = 0;
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

int idx_bits_for(int32_t n) {
    uint32_t top = (uint32_t)(n - 1);
    int bits = 0;
    while (top) { ++bits; top >>= 1; }
    return (bits + 7) / 8 * 8;
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
    if (G > 1 && !var.multi) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (G > 1 && rows * (int64_t)G > (int64_t)d.capacity[v]) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (rows * (int64_t)G > 0x7FFFFFFFll) return TOPK_SELECT_ERROR_INVALID_VALUE;
    L->variant = v;
    L->G = G;
    L->chunks_per_wg = (int)cpw;
    return TOPK_SELECT_SUCCESS;
}

// Default shape (measured on MI355X: a cross-workgroup round costs a few
// microseconds whatever the split, so few rows use few, large workgroups).
// Many rows: one WG per row with the 12-bit first digit when the row fits
// one resident tile, else several 12-bit WGs per row when they can all be
// resident, else streaming.  Few rows: 512-thread WGs holding 16K (then
// 32K, then smaller) logits each, as many per row as the row needs.
int choose_shape(const DeviceInfo& d, int64_t rows, int64_t maxc, Launch* L) {
    const int target = d.cus;
    auto tile_chunks = [](int v) { return (int64_t)kVariants[v].block * (kVariants[v].items / 4); };
    if (rows >= target / 2) {
        const int one_wg[] = {5, 6, 8};
        for (int v : one_wg)
            if (maxc <= tile_chunks(v)) return check_shape(d, rows, maxc, v, 1, L);
        const int split[] = {7};
        for (int v : split) {
            const int64_t G = (maxc + tile_chunks(v) - 1) / tile_chunks(v);
            if (rows * G <= (int64_t)d.capacity[v]) return check_shape(d, rows, maxc, v, (int)G, L);
        }
    } else {
        const int few[] = {3, 4, 2, 1, 0};
        for (int v : few) {
            const int64_t G = (maxc + tile_chunks(v) - 1) / tile_chunks(v);
            if (G == 1 || rows * G <= (int64_t)d.capacity[v]) return check_shape(d, rows, maxc, v, (int)G, L);
        }
    }
    // streaming: as many WGs per row as can be co-resident, at least one
    const int v = (maxc >= 16384) ? 9 : 10;
    int64_t G = d.capacity[v] / (rows > 0 ? rows : 1);
    const int64_t gmax = (maxc + tile_chunks(v) - 1) / tile_chunks(v);
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

int grow(void** ptr, size_t* have, size_t need, bool zero, hipStream_t stream) {
    if (*have >= need) return TOPK_SELECT_SUCCESS;
    if (*ptr) {
        if (hipStreamSynchronize(stream) != hipSuccess) return TOPK_SELECT_ERROR_LAUNCH;
        (void)hipFree(*ptr);
        *ptr = nullptr;
        *have = 0;
    }
    void* p = nullptr;
    if (hipMalloc(&p, need) != hipSuccess) {
        (void)hipGetLastError();
        return TOPK_SELECT_ERROR_OUT_OF_MEMORY;
    }
    if (zero && hipMemsetAsync(p, 0, need, stream) != hipSuccess) {
        (void)hipFree(p);
        return TOPK_SELECT_ERROR_LAUNCH;
    }
    *ptr = p;
    *have = need;
    return TOPK_SELECT_SUCCESS;
}

int get_workspace(int dev, hipStream_t stream, size_t need, size_t stage_need, Workspace** out) {
    Workspace& w = g_ws[{dev, (uintptr_t)stream}];
    int rc = grow(&w.base, &w.bytes, need, true, stream);
    if (rc == TOPK_SELECT_SUCCESS && stage_need) rc = grow(&w.stage, &w.stage_bytes, stage_need, false, stream);
    if (rc != TOPK_SELECT_SUCCESS) return rc;
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
    const Variant& var0 = kVariants[L.variant];
    const bool need_stage = L.G > 1 || (int64_t)k + kCap > (int64_t)var0.stage_lds;
    const int64_t stage_cap = need_stage ? (int64_t)k + kCap : 0;
    const size_t rows_bytes = L.G > 1 ? (size_t)rows * sizeof(RowWorkspace) : 0;
    const size_t stage_bytes = (size_t)rows * (size_t)stage_cap * sizeof(uint64_t);
    const size_t ws_bytes = kStatusBytes + rows_bytes;
    Workspace* w = nullptr;
    rc = get_workspace(dev, stream, ws_bytes, stage_bytes, &w);
    if (rc != TOPK_SELECT_SUCCESS) return rc;
    char* base = reinterpret_cast<char*>(w->base);
    KParams P;
    P.logits = logits;
    P.lengths = lengths;
    P.out = out;
    P.status = reinterpret_cast<uint32_t*>(base);
    P.ws = L.G > 1 ? reinterpret_cast<RowWorkspace*>(base + kStatusBytes) : nullptr;
    P.stage = need_stage ? reinterpret_cast<uint64_t*>(w->stage) : nullptr;
    P.rows = rows;
    P.n = n;
    P.k = k;
    P.G = L.G;
    P.chunks_per_wg = L.chunks_per_wg;
    P.idx_bits = idx_bits_for(n);
    P.stage_cap = (int32_t)stage_cap;
    const Variant& var = var0;
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
        plan->first_bits = tks::kVariants[L.variant].first_bits;
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
    plan->first_bits = tks::kVariants[v].first_bits;
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
            if (kv.second.base || kv.second.stage) {
                int cur = 0;
                (void)hipGetDevice(&cur);
                (void)hipSetDevice(kv.first.first);
                if (hipDeviceSynchronize() != hipSuccess) rc = TOPK_SELECT_ERROR_LAUNCH;
                if (kv.second.base && hipFree(kv.second.base) != hipSuccess) rc = TOPK_SELECT_ERROR_LAUNCH;
                if (kv.second.stage && hipFree(kv.second.stage) != hipSuccess) rc = TOPK_SELECT_ERROR_LAUNCH;
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
