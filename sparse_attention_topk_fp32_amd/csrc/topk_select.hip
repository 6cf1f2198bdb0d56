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
//  * Section 03: keep the surviving candidates on chip once the bucket is
//    small, and stop the screening over global memory once the bucket holds
//    at most 4096 elements; wide vector loads.
//  * Section 5: one row split over several blocks that merge their
//    histograms and continue together; -1 for empty output slots.
//
// MI355X design (not a translation of the article's Triton/CUDA kernels):
//  * A row is cut into slices of 16-byte chunks, one workgroup (WG) per
//    slice, G WGs per row.  Resident variants load their slice once, fuse the
//    key map into the load and keep the keys in VGPRs for every later pass;
//    streaming variants re-read their slice in each pass (rows too long to
//    keep on chip).
//  * Ties are made unique by ranking the 64-bit composite
//    (key << 32 | ~index): larger composite = larger value, or equal value and
//    smaller index.  Rounds run over 8-bit digits of the key and, only when a
//    value is tied past capacity, of the index.
//  * Merge of a round across the G WGs of a row: each WG adds
//    (1 << 32 | count) for each of the 256 bins into the row's global
//    histogram with one 64-bit device-scope atomic per bin, and polls the bin
//    until its arrival field reaches G; no separate barrier, no cache fence.
//    The value the atomic returns is the count of the WGs that added before
//    this one, which gives every WG a private, disjoint range of output
//    positions inside each bin.  Every WG selects the threshold bin itself
//    from the merged counts.
//  * Elements above the threshold bin are written straight to the output by
//    the WG holding them, at (start of their bin) + (the WG's range) + (rank
//    inside the WG, from a wave-aggregated LDS counter).  Once the threshold
//    bucket holds at most 4096 elements, its (key, index) composites go to a
//    candidate buffer (LDS for G == 1, the row's global stage for G > 1) and
//    one WG finishes on chip: more digit rounds in LDS while more than 256
//    remain, then an exact rank.
//  * The per-row workspace is double-buffered by launch parity: a launch
//    uses one half, and its finishing WG clears the half the previous launch
//    used, so no clearing launch or end-of-kernel barrier is needed.
//  * Batches of many rows take one WG per row instead, reading the row once
//    and keeping only the elements above a running bound on chip (below).

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "topk_select.h"

namespace tks {

constexpr int kCap = 4096;        // final bucket size handed to one WG (entries)
constexpr int kSmall = 256;       // bucket ranked exactly by comparisons
constexpr int kRounds = 9;        // merge rounds: a window round, then up to 4 key + 4 index digits
constexpr int kCopies = 16;       // LDS copies of the 256-bin histogram (against atomic conflicts)
constexpr int kWinLength = 524288;  // rows at least this long take the sampled window round
constexpr int kMergeCopies = 4;   // global copies of a row's histogram per round (WG w -> copy w mod C)
constexpr uint32_t kFlagTimeout = 1u;
constexpr uint32_t kFlagCapacity = 2u;
// Bound on a cross-workgroup wait, in ticks of the 100 MHz constant clock
// (s_memrealtime): 2 s, far beyond any legitimate wait.
constexpr uint64_t kSpinLimitTicks = 200000000ull;

// Per-row scratch for rows spread over several workgroups, in two halves
// selected by the parity of the launch.  All cross-workgroup traffic uses
// device-scope atomic operations, performed at the device's coherence point.
struct alignas(256) RowWorkspace {
    uint64_t hist[2][kRounds][kMergeCopies][256];  // (arrivals << 32) | count
    uint64_t stage[2][kCap];                       // final-bucket composites; 0 = not written yet
    uint32_t parity;                               // half used by the next launch
    uint32_t used[2];  // what each half holds, cleared by the next launch: rounds | copies << 4 | stage entries << 8
    uint32_t pad[57];
};

struct KParams {
    const float* logits;
    const int32_t* lengths;
    int32_t* out;
    RowWorkspace* ws;       // per row, when G > 1
    uint32_t* status;
    int32_t rows, n, k;
    int32_t G;              // workgroups per row
    int32_t chunks_per_wg;  // 16-byte chunks in one WG's slice
    int32_t idx_bits;       // bits of the index that vary (multiple of 8, 8..32)
    int32_t mcopies;        // global histogram copies used (1..kMergeCopies)
    uint32_t* keys;         // [rows, k]: key of the element at each output slot (ordered output), or null
    int32_t ahead;          // one WG per row: rows from a row to the one whose first tile it touches (0: none)
};

// ----------------------------------------------------------------- device helpers

// 16 bytes as a native vector (register arrays of the uint4 struct can be
// placed in scratch memory when they are passed around)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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

// A value every lane holds identically: make it scalar.
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

// Workgroup barrier that orders LDS only (global data crossing WGs goes
// through device-scope atomics, global data inside a WG is never re-read).
__device__ __forceinline__ void lds_sync() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Inclusive scan across the 64 lanes of a wave with DPP lane moves: shifts
// by 1, 2, 4, 8 inside each row of 16 lanes, then the last lane of a row is
// broadcast into the rows above it.  Lanes with no source lane read 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Block-wide exclusive scan (thread order) of one counter over the first NT
// threads (NT a multiple of 64, <= BLOCK); every thread of the block calls
// it.  Returns this thread's exclusive prefix.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t a, uint32_t* s_w /* [NT / 64] */) {
    constexpr int NW = NT / 64;
    const uint32_t wid = threadIdx.x / 64;
    const uint32_t ia = wave_inclusive_scan(a);
    if (wid < NW && lane_id() == 63) s_w[wid] = ia;
    lds_sync();
    uint32_t pa = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i)
        if ((uint32_t)i < wid) pa += s_w[i];
    lds_sync();  // s_w may be reused right after
    return pa + ia - a;
}

// Block-wide exclusive scan over all BLOCK threads that also returns the
// total (uniform).
template <int BLOCK>
__device__ __forceinline__ uint32_t block_scan_total(uint32_t a, uint32_t* s_w /* [BLOCK / 64] */, uint32_t& total) {
    constexpr int NW = BLOCK / 64;
    const uint32_t wid = threadIdx.x / 64;
    const uint32_t ia = wave_inclusive_scan(a);
    if (lane_id() == 63) s_w[wid] = ia;
    lds_sync();
    uint32_t pa = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint32_t v = s_w[i];
        if ((uint32_t)i < wid) pa += v;
        tot += v;
    }
    lds_sync();
    total = uniform(tot);
    return pa + ia - a;
}

// Digit schedule: rounds 0..3 cut the key from the top, the first digit
// F bits wide (8 or 12) and the others 8 bits (the last key digit keeps what
// is left); later rounds cut the varying low idx_bits of ~index (its top
// 32 - idx_bits bits are ones for every valid index).  shift: bit position
// of round r's digit inside its 32-bit word; width: its bits.
__device__ __forceinline__ int digit_shift(int F, int r, int idx_bits) {
    if (r < 4) {
        const int s = 32 - F - 8 * r;
        return s < 0 ? 0 : s;
    }
    return idx_bits - 8 - 8 * (r - 4);
}
__device__ __forceinline__ int digit_width(int F, int r) {
    if (r == 0) return F;
    if (r < 4) return min(8, 32 - F - 8 * (r - 1));
    return 8;
}
__device__ __forceinline__ uint32_t digit_mask(int F, int r) { return (1u << digit_width(F, r)) - 1u; }
__device__ __forceinline__ int num_rounds(int idx_bits) { return 4 + idx_bits / 8; }

// The composite prefix resolved so far: key bits (kpfx under kmask) and
// ~index bits (ipfx under imask).
struct Prefix {
    uint32_t kpfx, kmask, ipfx, imask;
    // value selects only (a branch that picks the field to update would
    // put the struct in scratch memory)
    __device__ void add(int F, int r, uint32_t b, int idx_bits) {
        const int s = digit_shift(F, r, idx_bits);
        const bool in_key = r < 4;
        const uint32_t bb = b << s, mm = digit_mask(F, r) << s;
        kpfx |= in_key ? bb : 0u;
        kmask |= in_key ? mm : 0u;
        ipfx |= in_key ? 0u : bb;
        imask |= in_key ? 0u : mm;
    }
    // Does the element (key, ~index) match the prefix?
    __device__ __forceinline__ bool match(uint32_t key, uint32_t ni) const {
        return (key != 0u) & ((key & kmask) == kpfx) & ((ni & imask) == ipfx);
    }
    // Is the element above the prefix (a winner of some round done)?
    __device__ __forceinline__ bool above(uint32_t key, uint32_t ni) const {
        const uint32_t s = key & kmask;
        return (s > kpfx) | ((s == kpfx) & ((ni & imask) > ipfx));
    }
};

// Where the first round's digit comes from: the top F bits of the key, or
// (win) the 12-bit first digit seen through a window of 256 bins starting
// at bin LO (bins above the window fold into its top bin).
struct FirstDigit {
    int F;
    bool win;
    uint32_t LO;
    __device__ __forceinline__ uint32_t of(uint32_t key) const {
        return win ? min((key >> 20) - LO, 255u) : key >> (32 - F);
    }
};

// Position-counter slot (256 * round + digit) of a winner whose key differs
// from the prefix, x = the differing key bits (non-zero): the round is the
// one whose digit holds the top differing bit.
__device__ __forceinline__ uint32_t key_slot(uint32_t key, uint32_t x, const FirstDigit& fd, int idx_bits) {
    const int p = 31 - __builtin_clz(x);
    if (p >= 32 - fd.F) return fd.of(key);
    const int r = 1 + (31 - fd.F - p) / 8;
    return 256u * (uint32_t)r + ((key >> digit_shift(fd.F, r, idx_bits)) & digit_mask(fd.F, r));
}

// Relation of an element to the prefix after the rounds done: returns 1 when
// it is above it (a winner; *slot = its position-counter slot), 2 when it
// matches it (in the bucket), 0 otherwise.  Composites compare as
// (key, ~index) pairs.
__device__ __forceinline__ uint32_t classify(uint32_t key, uint32_t ni, const Prefix& pf, const FirstDigit& fd,
                                             int idx_bits, uint32_t* slot) {
    if (key == 0u) return 0u;
    const uint32_t s = key & pf.kmask;
    if (s != pf.kpfx) {
        if (s < pf.kpfx) return 0u;
        *slot = key_slot(key, s ^ pf.kpfx, fd, idx_bits);
        return 1u;
    }
    const uint32_t t = ni & pf.imask;
    if (t == pf.ipfx) return 2u;
    if (t < pf.ipfx) return 0u;
    const int lead = __builtin_clz(t ^ pf.ipfx) - (32 - idx_bits);  // leading bit inside the index digits
    const int r = 4 + lead / 8;
    *slot = (uint32_t)r * 256u + ((ni >> digit_shift(fd.F, r, idx_bits)) & 0xFFu);
    return 1u;
}

// Shared state of one WG.
template <int BLOCK>
struct Smem {
    alignas(16) uint32_t hist[kCopies * 257];  // histogram copies (stride 257 words)
    uint32_t pos[kRounds * 256];        // output / stage position counters per (round, bin)
    uint64_t cand[kCap];                // final bucket, on chip
    uint64_t small[kSmall];             // last few candidates, ranked exactly
    uint32_t scan[BLOCK / 64];
    uint32_t sel[4];                    // threshold bin, count above it, count in it
    uint32_t ctr[2];                    // finisher position counters
};

// Thresholding step on one WG's own histogram: NB bins held as NC LDS
// copies of stride STRIDE words.  Owner threads take NB / OWNERS bins each,
// in descending bin order across threads, so one block scan over the
// owners' sums locates the bin b that holds the element of rank `need`
// (1-based, from the top).  Returns b, the count above b and the count in b.
template <int BLOCK, int NB, int NC, int STRIDE, bool STRICT = true>
__device__ __forceinline__ void local_select(const uint32_t* h, uint32_t bin0_sub, uint32_t need, uint32_t* scan,
                                             uint32_t* sel, uint32_t* status, uint32_t& b_out, uint32_t& above_out,
                                             uint32_t& hb_out) {
    constexpr int OWNERS = NB < BLOCK ? NB : BLOCK;
    constexpr int OWN = NB / OWNERS;
    static_assert(OWNERS % 64 == 0, "whole waves of owners");
    const int t = threadIdx.x;
    const bool owner = t < OWNERS;
    uint32_t cnt[OWN];
    uint32_t tot = 0;
#pragma unroll
    for (int i = 0; i < OWN; ++i) {
        const int bin = NB - 1 - (t * OWN + i);
        uint32_t c = 0;
        if (owner) {
#pragma unroll
            for (int q = 0; q < NC; ++q) c += h[q * STRIDE + bin];
            if (bin == 0) c -= bin0_sub;
        }
        cnt[i] = c;
        tot += c;
    }
    if (t == 0) sel[2] = 0xFFFFFFFFu;  // "not found" until an owner writes
    uint32_t above = block_exclusive_scan<OWNERS>(tot, scan);
    if (owner && above < need && need <= above + tot) {
#pragma unroll
        for (int i = 0; i < OWN; ++i) {
            if (above < need && need <= above + cnt[i]) {
                sel[0] = (uint32_t)(NB - 1 - (t * OWN + i));
                sel[1] = above;
                sel[2] = cnt[i];
            }
            above += cnt[i];
        }
    }
    lds_sync();
    uint32_t b = uniform(sel[0]), ab = uniform(sel[1]), hb = uniform(sel[2]);
    lds_sync();
    if (hb == 0xFFFFFFFFu) {  // fewer elements than `need` (an error unless !STRICT)
        if (STRICT && t == 0) raise_flag(status, kFlagCapacity);
        b = 0; ab = 0; hb = 0;
    }
    b_out = b;
    above_out = ab;
    hb_out = hb;
}

// On-chip finish of the final bucket: the m composites in cand all match
// the prefix pf (rounds done: < r0); `need` of them remain to be selected,
// at output positions W..W+need-1.  More digit rounds in LDS while more
// than kSmall match, then an exact rank of the rest.  Uses the scratch
// `hist` (kCopies x 257 words), `small`, `scan`, `sel` and the counter
// `ctr`.  Every thread of the WG calls it.
template <int BLOCK>
__device__ __forceinline__ void finish_bucket(const uint64_t* cand, uint32_t m, uint32_t need, uint32_t W, Prefix pf, int r0,
                              int F, int idx_bits, bool cleared, uint32_t* hist, uint64_t* small, uint32_t* scan,
                              uint32_t* sel, uint32_t* ctr, int32_t* out, uint32_t* okey, int k,
                              uint32_t* status) {
    const int tid = threadIdx.x;
    const int nrounds = num_rounds(idx_bits);
    auto c_match = [&](uint64_t c) { return pf.match((uint32_t)(c >> 32), (uint32_t)c); };
    auto c_digit = [&](uint64_t c, int r) -> uint32_t {
        const int s = digit_shift(F, r, idx_bits);
        return ((r < 4 ? (uint32_t)(c >> 32) : (uint32_t)c) >> s) & digit_mask(F, r);
    };
    // f(entry) for every candidate, four LDS loads in flight per thread
    // (entries past m read as 0, which matches no prefix)
    auto for_each_cand = [&](auto&& f) {
        for (uint32_t i0 = 0; i0 < m; i0 += 4u * BLOCK) {
            uint64_t c[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t i = i0 + (uint32_t)(u * BLOCK + tid);
                c[u] = i < m ? cand[i] : 0ull;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) f(c[u]);
        }
    };
    int r = r0;
    uint32_t mb = m;        // entries still matching the prefix
    bool in_small = false;  // they are already gathered in small[0 .. ctr[1])
    while (mb > (uint32_t)kSmall && r < nrounds) {
        if (!cleared) {
            uint4* const h4 = reinterpret_cast<uint4*>(hist);
            for (int i = tid; i < kCopies * 257 / 4; i += BLOCK) h4[i] = uint4{0u, 0u, 0u, 0u};
            if (tid < 2) ctr[tid] = 0u;
            lds_sync();
        }
        cleared = false;
        uint32_t* const hc = hist + (tid % kCopies) * 257;
        for_each_cand([&](uint64_t c) {
            if (c_match(c)) atomicAdd(&hc[c_digit(c, r)], 1u);
        });
        lds_sync();
        uint32_t b, above, nb;
        local_select<BLOCK, 256, kCopies, 257>(hist, 0u, need, scan, sel, status, b, above, nb);
        const uint32_t need2 = need - above;
        const bool all = nb == need2;
        const bool gather = !all && nb <= (uint32_t)kSmall;
        // winners of this round (digit above b), and the bin itself when
        // taken whole; a small enough bin is gathered for the exact rank
        for_each_cand([&](uint64_t c) {
            const uint32_t d = c_digit(c, r);
            if (!c_match(c)) return;
            if (d > b || (all && d == b)) {
                const uint32_t pos = W + atomicAdd(&ctr[0], 1u);
                if (pos < (uint32_t)k) {
                    out[pos] = (int32_t)~(uint32_t)c;
                    if (okey) okey[pos] = (uint32_t)(c >> 32);
                } else {
                    raise_flag(status, kFlagCapacity);
                }
            } else if (gather && d == b) {
                const uint32_t pos = atomicAdd(&ctr[1], 1u);
                if (pos < (uint32_t)kSmall) small[pos] = c;
            }
        });
        need = need2;
        W += above;
        pf.add(F, r, b, idx_bits);
        mb = nb;
        ++r;
        lds_sync();
        if (all) return;
        in_small = gather;
    }
    if (!in_small) {
        // the few candidates still matching, gathered
        if (tid == 1) ctr[1] = 0u;
        lds_sync();
        for_each_cand([&](uint64_t c) {
            if (c_match(c)) {
                const uint32_t pos = atomicAdd(&ctr[1], 1u);
                if (pos < (uint32_t)kSmall) small[pos] = c;
            }
        });
        lds_sync();
    }
    uint32_t ms = uniform(ctr[1]);
    if (ms > (uint32_t)kSmall) {
        if (tid == 0) raise_flag(status, kFlagCapacity);
        ms = kSmall;
    }
    // exact rank by comparison, P lanes per candidate (each compares a
    // strided share, then the lanes add up their counts)
    uint32_t P = 1;
    while (P < 64u && 2u * P * ms <= (uint32_t)BLOCK) P *= 2u;
    const uint32_t i = (uint32_t)tid / P, q = (uint32_t)tid % P;
    const uint64_t c = i < ms ? small[i] : 0ull;
    uint32_t rank = 0;
    if (i < ms) {
        for (uint32_t j = q; j < ms; j += P) rank += small[j] > c;
    }
    for (uint32_t sft = 32u; sft >= 1u; sft >>= 1) {
        if (sft < P) rank += (uint32_t)__shfl_xor((int)rank, (int)sft);
    }
    if (i < ms && q == 0u && rank < need && W + rank < (uint32_t)k) {
        out[W + rank] = (int32_t)~(uint32_t)c;
        if (okey) okey[W + rank] = (uint32_t)(c >> 32);
    }
}

// Thresholding step for round r from the LDS histogram copies (the first
// 256 threads own one bin each, thread t the bin 255 - t, so thread order is
// descending bin order).  With G > 1 the counts are merged across the row's
// WGs first.  Finds the bin b holding the element of rank `need` (1-based,
// from the top) and sets the position counters of the bins at and above b:
// winners of bin j > b go to W + (count above j) + (this WG's range in j);
// the bucket bin b goes to the output the same way when it is taken whole
// (`need` == count in b after the elements above), else to positions
// (this WG's range in b) of the candidate buffer.
template <int BLOCK>
__device__ __forceinline__ void threshold(Smem<BLOCK>& sm, int r, int mslot, bool strict, uint32_t bin0_sub,
                                          uint32_t need, uint32_t W, RowWorkspace* ws, int p, int C, int w, int G,
                                          uint32_t* status, uint32_t& b_out, uint32_t& above_out, uint32_t& hb_out) {
    const int t = threadIdx.x;
    const bool owner = t < 256;
    const int j = 255 - t;
    uint32_t tot = 0, pre = 0;
    if (owner) {
        uint32_t cnt = 0;
#pragma unroll
        for (int c = 0; c < kCopies; ++c) cnt += sm.hist[c * 257 + j];
        if (j == 0) cnt -= bin0_sub;
        if (G > 1) {
            uint64_t* h = &ws->hist[p][mslot][0][0];
            const int mc = w % C;
            const uint64_t old = add_dev(&h[mc * 256 + j], (uint64_t)((1ull << 32) | cnt));
            // poll the copies (all loads in flight together) until every
            // WG of the row has added
            uint64_t v0, v1, v2, v3;
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            for (;;) {
                v0 = ld_dev(&h[j]);
                v1 = C > 1 ? ld_dev(&h[256 + j]) : 0ull;
                v2 = C > 2 ? ld_dev(&h[512 + j]) : 0ull;
                v3 = C > 3 ? ld_dev(&h[768 + j]) : 0ull;
                const uint32_t arr = (uint32_t)(v0 >> 32) + (uint32_t)(v1 >> 32) + (uint32_t)(v2 >> 32) +
                                     (uint32_t)(v3 >> 32);
                if (arr >= (uint32_t)G) break;
                if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimitTicks) {
                    raise_flag(status, kFlagTimeout);
                    break;
                }
                // many WGs: back off between polls, which otherwise crowd
                // the channel that holds the counts (measured)
                if (G > 64) __builtin_amdgcn_s_sleep(2);
            }
            tot = (uint32_t)v0 + (uint32_t)v1 + (uint32_t)v2 + (uint32_t)v3;
            pre = (uint32_t)old + (mc > 0 ? (uint32_t)v0 : 0u) + (mc > 1 ? (uint32_t)v1 : 0u) +
                  (mc > 2 ? (uint32_t)v2 : 0u);
        } else {
            tot = cnt;
        }
    }
    if (t == 0) sm.sel[2] = 0xFFFFFFFFu;  // "not found" until an owner writes
    const uint32_t excl = block_exclusive_scan<256>(owner ? tot : 0u, sm.scan);
    if (owner && excl < need && need <= excl + tot) {
        sm.sel[0] = (uint32_t)j;
        sm.sel[1] = excl;
        sm.sel[2] = tot;
    }
    lds_sync();
    uint32_t b = uniform(sm.sel[0]), above = uniform(sm.sel[1]), hb = uniform(sm.sel[2]);
    if (hb == 0xFFFFFFFFu) {  // fewer elements than `need`: an error unless !strict
        if (strict && t == 0) raise_flag(status, kFlagCapacity);
        b_out = 0;
        above_out = 0;
        hb_out = strict ? 0u : 0xFFFFFFFFu;
        lds_sync();
        return;
    }
    if (owner && (uint32_t)j >= b) {
        const bool whole = (uint32_t)j > b || hb == need - above;
        sm.pos[r * 256 + j] = whole ? W + excl + pre : pre;
    }
    lds_sync();
    b_out = b;
    above_out = above;
    hb_out = hb;
}

// ----------------------------------------------------------------- the kernel
//
// BLOCK threads per WG; ITEMS logits per thread per tile; RESIDENT: the
// slice is one tile kept in VGPRs across passes (else re-read every pass);
// KEYS: the keys of the output are recorded (ordered output); WIN: rows of
// kWinLength or more take the sampled window round.

template <int BLOCK, int ITEMS, bool RESIDENT, bool KEYS, bool WIN>
__global__ __launch_bounds__(BLOCK) void topk_select_kernel(const KParams P) {
    static_assert(ITEMS % 4 == 0, "ITEMS counts whole 16-byte chunks");
    static_assert(BLOCK % 64 == 0 && BLOCK >= 256, "one bin per thread in the 256-bin rounds");
    constexpr int CHUNKS = ITEMS / 4;            // chunks per thread per tile
    constexpr int TILE_CHUNKS = BLOCK * CHUNKS;  // chunks per tile
    __shared__ Smem<BLOCK> sm;

    const int tid = threadIdx.x;
    const int G = P.G;
    const int row = blockIdx.x / G;
    const int w = blockIdx.x - row * G;
    const int n = P.n;
    const int k = P.k;
    const float* __restrict__ prow = P.logits + (size_t)row * (size_t)n;
    int32_t* __restrict__ out = P.out + (size_t)row * (size_t)k;
    uint32_t* const okey = KEYS ? P.keys + (size_t)row * (size_t)k : nullptr;  // recorded keys (ordered output)
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

    const int off = (int)(((uintptr_t)prow >> 2) & 3);  // elements before the first 16-byte boundary
    const int nchunks = (off + L + 3) >> 2;
    const int Geff = min(G, (nchunks + P.chunks_per_wg - 1) / P.chunks_per_wg);  // WGs with a non-empty slice
    if (w >= Geff) return;
    const bool multi = Geff > 1;
    RowWorkspace* const ws = multi ? P.ws + row : nullptr;
    const int p = multi ? (int)(ld_dev(&ws->parity) & 1u) : 0;
    // what the previous launch left to clear (read by the finishing WG now,
    // off the critical path at the end)
    const uint32_t used0 = (multi && w == 0) ? ld_dev(&ws->used[0]) : 0u;
    const uint32_t used1 = (multi && w == 0) ? ld_dev(&ws->used[1]) : 0u;
    const int C = P.mcopies;
    const int idx_bits = P.idx_bits;
    const int nrounds = num_rounds(idx_bits);

    const int c_begin = w * P.chunks_per_wg;
    const int c_end = min(nchunks, c_begin + P.chunks_per_wg);
    // chunks whose four elements are all valid
    const int cf_lo = max(c_begin, off ? 1 : 0);
    const int cf_hi = min(c_end, (L + off) >> 2);
    // slots of the slice that hold no element (key 0): the first-round
    // histogram counts them in bin 0 and subtracts them after
    const int valid = max(0, min(L, 4 * c_end - off) - max(0, 4 * c_begin - off));
    const uint32_t n_empty = (uint32_t)(4 * (c_end - c_begin) - valid);

    uint32_t keys[ITEMS];
    const char* const base = reinterpret_cast<const char*>(prow - off);  // 16-byte aligned

    // Load one tile: chunk c of the row is the aligned 16-byte block holding
    // elements [4c - off, 4c - off + 4).  A chunk with at least one valid
    // element is read whole; lanes past the slice re-read chunk 0 (valid:
    // L > k >= 1) and hold empty slots.  All loads are issued before any is
    // used.
    auto load_tile = [&](int c_tile) {
#pragma unroll
        for (int j = 0; j < CHUNKS; ++j) {
            const int c = c_tile + j * BLOCK + tid;
            const uint32_t byte_off = (uint32_t)(c < c_end ? c : 0) * 16u;
            const uint4 v = *reinterpret_cast<const uint4*>(base + byte_off);
            keys[4 * j + 0] = v.x;
            keys[4 * j + 1] = v.y;
            keys[4 * j + 2] = v.z;
            keys[4 * j + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < CHUNKS; ++j) {
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
    // f(key, ~index) for every slot of the slice, tile by tile; element e of
    // chunk j of a tile has index ibase + 4 * BLOCK * j + e.
    auto visit = [&](auto&& f) {
        auto tile = [&](int c_tile) {
            int ibase = 4 * (c_tile + tid) - off;
            __asm__ volatile("" : "+v"(ibase));  // indices are recomputed per visit, never kept live
#pragma unroll
            for (int j = 0; j < CHUNKS; ++j) {
#pragma unroll
                for (int e = 0; e < 4; ++e) f(keys[4 * j + e], ~(uint32_t)(ibase + 4 * BLOCK * j + e));
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
    // f(key) for every slot of the chunks in [c_begin, c_end)
    auto visit_chunks = [&](auto&& f) {
        auto tile = [&](int c_tile) {
#pragma unroll
            for (int j = 0; j < CHUNKS; ++j) {
                if (c_tile + j * BLOCK + tid < c_end) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) f(keys[4 * j + e]);
                }
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
    // f(key, ~index) for every slot of the slice, re-read from global
    // memory in a rolled loop: the rare index-digit rounds use it, so that
    // their code stays small (at these sizes the code a launch runs costs
    // instruction fetches)
    auto visit_global = [&](auto&& f) {
#pragma unroll 1
        for (int c = c_begin + tid; c < c_end; c += BLOCK) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(base + (uint32_t)c * 16u);
            const int e0 = 4 * c - off;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = (uint32_t)(e0 + e) < (uint32_t)L;
                f(ok ? key_of(__uint_as_float(v[e])) : 0u, ~(uint32_t)(e0 + e));
            }
        }
    };
    auto opaque_keys = [&]() {
        if constexpr (RESIDENT) {
            // stops the optimiser from hoisting per-element values out of
            // the passes (one VGPR per element and pass)
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) __asm__ volatile("" : "+v"(keys[i]));
        }
    };

    auto clear_hist = [&]() {  // 16-byte LDS stores
        uint4* const h4 = reinterpret_cast<uint4*>(sm.hist);
        for (int i = tid; i < kCopies * 257 / 4; i += BLOCK) h4[i] = uint4{0u, 0u, 0u, 0u};
        if (tid < (kCopies * 257) % 4) sm.hist[kCopies * 257 / 4 * 4 + tid] = 0u;
    };

    // the window round's sample (the row's first chunks, one per thread) is
    // loaded together with the slice.  Only long rows (split over many WGs,
    // where a second merge round is expensive) take the window round: for
    // shorter rows its extra steps cost more than they save (measured).
    const bool try_win = WIN && L >= kWinLength;
    const int nsc = min(nchunks, BLOCK);
    uint4 sraw = uint4{0u, 0u, 0u, 0u};
    if (try_win && tid < nsc) sraw = *reinterpret_cast<const uint4*>(base + (uint32_t)tid * 16u);
    if constexpr (RESIDENT) load_tile(c_begin);

    // ---------------- screening rounds over the row
    Prefix pf{0u, 0u, 0u, 0u};
    uint32_t need = (uint32_t)k;  // rank still to place, counted inside the current bucket
    uint32_t W = 0;               // winners placed so far (output positions [0, W))
    uint32_t hb = 0;              // size of the current bucket
    int R = 0;                    // last round done
    bool whole = false;           // the last bucket is taken whole
    FirstDigit fd{8, false, 0u};  // first-round digit (set by the window round when it succeeds)
    uint32_t bwin = 0;            // the window round's threshold bin
    int slot_base = 0;            // merge slot of round 0 of the 8-bit schedule

    // -- window round.  A sample (the row's first chunks, one per thread)
    // estimates the threshold: the first-digit bin b8 (8 bits) of its
    // element of rank 1.25 * k * S / L + 64 (the k-th largest of the row is
    // expected near rank k * S / L).  Then every WG histograms the 12-bit
    // first digit of its elements at or above LO = b8 << 4 only, in a window
    // of 256 bins from LO (the top bin also takes all bins above the
    // window), merged like any round.  When the threshold falls inside the
    // window below its top bin, the counts it needs are exact and the first
    // round is done at 12-bit resolution; otherwise the row starts over with
    // the 8-bit schedule.
    if (try_win) {
        uint32_t sk[4];
        {
            const uint32_t raw[4] = {sraw.x, sraw.y, sraw.z, sraw.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ix = 4 * tid - off + e;
                sk[e] = (tid < nsc && ix >= 0 && ix < L) ? key_of(__uint_as_float(raw[e])) : 0u;
            }
        }
        const uint32_t s_valid = (uint32_t)min(L, 4 * nsc - off);
        const uint64_t est64 = ((uint64_t)k * s_valid * 5u) / (4u * (uint64_t)L) + 64u;
        const uint32_t est = (uint32_t)(est64 < s_valid ? est64 : s_valid);
        uint32_t* const hc = sm.hist + (tid % kCopies) * 257;
        clear_hist();
        lds_sync();
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (sk[e] != 0u) atomicAdd(&hc[sk[e] >> 24], 1u);
        lds_sync();
        uint32_t b8, ab8, hb8;
        local_select<BLOCK, 256, kCopies, 257, false>(sm.hist, 0u, est, sm.scan, sm.sel, P.status, b8, ab8, hb8);
        const uint32_t LO = hb8 ? b8 << 4 : 0u;
        opaque_keys();
        clear_hist();
        lds_sync();
        visit_chunks([&](uint32_t key) {
            const uint32_t b12 = key >> 20;
            if (b12 >= LO) atomicAdd(&hc[min(b12 - LO, 255u)], 1u);
        });
        lds_sync();
        uint32_t b, above, hw;
        threshold<BLOCK>(sm, 0, 0, false, LO == 0u ? n_empty : 0u, need, W, ws, p, C, w, Geff, P.status, b, above,
                         hw);
        if (hw != 0xFFFFFFFFu && b < 255u) {
            fd = FirstDigit{12, true, LO};
            bwin = b;
            hb = hw;
            need -= above;
            W += above;
            pf.kpfx = (LO + b) << 20;
            pf.kmask = 0xFFFu << 20;
            whole = hb == need;
        } else {
            slot_base = 1;
        }
    }
    const int F = fd.F;
    if (!fd.win || (!whole && hb > (uint32_t)kCap)) {
        for (int r = fd.win ? 1 : 0;; ++r) {
            opaque_keys();
            clear_hist();
            lds_sync();
            uint32_t* const hc = sm.hist + (tid % kCopies) * 257;
            if (r == 0) {
                // every slot of the slice's chunks adds into its top byte's
                // bin; the few empty ones (key 0) land in bin 0 and are
                // subtracted after.  Chunks past the slice are skipped.
                visit_chunks([&](uint32_t key) { atomicAdd(&hc[key >> 24], 1u); });
            } else if (r < 4) {
                const int sh = digit_shift(F, r, idx_bits);
                const uint32_t dm = digit_mask(F, r);
                visit([&](uint32_t key, uint32_t) {
                    if ((key != 0u) & ((key & pf.kmask) == pf.kpfx)) atomicAdd(&hc[(key >> sh) & dm], 1u);
                });
            } else {
                const int sh = digit_shift(F, r, idx_bits);
                visit_global([&](uint32_t key, uint32_t ni) {
                    if (pf.match(key, ni)) atomicAdd(&hc[(ni >> sh) & 0xFFu], 1u);
                });
            }
            lds_sync();
            uint32_t b, above;
            threshold<BLOCK>(sm, r, r + slot_base, true, r == 0 ? n_empty : 0u, need, W, ws, p, C, w, Geff, P.status,
                             b, above, hb);
            need -= above;
            W += above;
            pf.add(F, r, b, idx_bits);
            R = r;
            if (hb == need) { whole = true; break; }
            if (hb <= (uint32_t)kCap || r + 1 >= nrounds) break;
        }
    }
    const int last_slot = R + (fd.win ? 0 : slot_base);  // merge slots used: 0 .. last_slot

    // ---------------- collection over the row
    // Winners go to the output; the bucket goes to the output when taken
    // whole, else to the candidate buffer (LDS) or the row's stage (G > 1).
    const bool idx_rounds = R >= 4;
    uint32_t bslot;  // position counter of the bucket: its bin in round R
    if (R == 0) {
        bslot = fd.win ? bwin : pf.kpfx >> 24;
    } else {
        const int sft = digit_shift(F, R, idx_bits);
        bslot = (uint32_t)R * 256u + (((R < 4 ? pf.kpfx : pf.ipfx) >> sft) & digit_mask(F, R));
    }
    uint64_t* const gstage = multi ? &ws->stage[p][0] : nullptr;
    bool overflow = false;
    opaque_keys();
    // With many elements per thread, three steps, so that the per-element
    // work stays a compare: count the
    // selected elements (winners and bucket) per thread; copy them, in rank
    // order from a block scan, into a compact LDS list (the histogram
    // space, in chunks); place the list's entries with all lanes busy.
    const uint32_t kp = pf.kpfx, km = pf.kmask;
    // the key prefix has no bits outside its mask, so (key & km) >= kp
    // is key >= kp; the lower bound 1 also drops empty slots (key 0)
    const uint32_t kp1 = kp > 1u ? kp : 1u;
    // place one selected element (a winner or a bucket element); IDX: the
    // rounds went into the index digits
    auto place = [&](uint32_t key, uint32_t ni, auto idx) {
        uint32_t slot = bslot;
        bool ab;
        if constexpr (!decltype(idx)::value) {
            const uint32_t s = key & km;
            ab = s > kp;
            if (ab) slot = key_slot(key, s ^ kp, fd, idx_bits);
        } else {
            ab = classify(key, ni, pf, fd, idx_bits, &slot) == 1u;
        }
        const uint32_t pos = atomicAdd(&sm.pos[slot], 1u);
        if (ab || whole) {
            if (pos < (uint32_t)k) {
                out[pos] = (int32_t)~ni;
                if (okey) okey[pos] = key;
            } else {
                overflow = true;
            }
        } else if (pos < (uint32_t)kCap) {
            const uint64_t e = ((uint64_t)key << 32) | (uint64_t)ni;
            if (multi) st_dev(&gstage[pos], e);
            else sm.cand[pos] = e;
        } else {
            overflow = true;
        }
    };
    // the key-digit case (index-digit rounds are collected below)
    auto collect = [&](auto&& selected) {
    if constexpr (ITEMS <= 8) {
        // few elements per thread: place them directly
        visit([&](uint32_t key, uint32_t ni) {
            if (selected(key, ni)) place(key, ni, std::false_type{});
        });
    } else {
    uint32_t nsel = 0;
    visit([&](uint32_t key, uint32_t ni) { nsel += selected(key, ni); });
    uint32_t tot_sel;
    const uint32_t my_first = block_scan_total<BLOCK>(nsel, sm.scan, tot_sel);
    uint64_t* const list = reinterpret_cast<uint64_t*>(sm.hist);
    constexpr uint32_t LISTN = kCopies * 257 / 2;
    for (uint32_t c0 = 0; c0 < tot_sel; c0 += LISTN) {
        uint32_t rk = my_first - c0;  // wraps for ranks before the chunk: never < LISTN then
        opaque_keys();
        visit([&](uint32_t key, uint32_t ni) {
            if (selected(key, ni)) {
                if (rk < LISTN) list[rk] = ((uint64_t)key << 32) | (uint64_t)ni;
                ++rk;
            }
        });
        lds_sync();
        const uint32_t nl = min(LISTN, tot_sel - c0);
        for (uint32_t i = tid; i < nl; i += BLOCK) {
            const uint64_t e = list[i];
            place((uint32_t)(e >> 32), (uint32_t)e, std::false_type{});
        }
        lds_sync();
    }
    }
    };
    if (!idx_rounds) {
        collect([&](uint32_t key, uint32_t) -> bool { return key >= kp1; });
    } else {
        // ties beyond the key digits (rare): the slice is re-read
        visit_global([&](uint32_t key, uint32_t ni) {
            uint32_t slot;
            if (classify(key, ni, pf, fd, idx_bits, &slot) != 0u) place(key, ni, std::true_type{});
        });
    }
    if (overflow) raise_flag(P.status, kFlagCapacity);

    if (multi && w != 0) return;  // WG 0 finishes the row

    // ---------------- on-chip finish of the last bucket
    if (!whole) {
        uint32_t m = hb > (uint32_t)kCap ? (uint32_t)kCap : hb;
        // the finisher's first histogram is cleared while the pull's loads
        // are in flight
        clear_hist();
        if (tid < 2) sm.ctr[tid] = 0u;
        if (multi) {
            // pull the staged bucket: every entry is non-zero once written.
            // Eight loads in flight per thread; entries not written yet are
            // re-polled together (bounded wait).
            for (uint32_t i0 = 0; i0 < m; i0 += 8u * BLOCK) {
                uint64_t v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t i = i0 + (uint32_t)(u * BLOCK + tid);
                    v[u] = i < m ? ld_dev(&gstage[i]) : 1ull;
                }
                const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                for (;;) {
                    bool miss = false;
#pragma unroll
                    for (int u = 0; u < 8; ++u) miss |= v[u] == 0ull;
                    if (!miss) break;
                    if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimitTicks) {
                        raise_flag(P.status, kFlagTimeout);
                        break;
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (v[u] == 0ull) v[u] = ld_dev(&gstage[i0 + (uint32_t)(u * BLOCK + tid)]);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t i = i0 + (uint32_t)(u * BLOCK + tid);
                    if (i < m) sm.cand[i] = v[u];
                }
            }
        }
        lds_sync();
        finish_bucket<BLOCK>(sm.cand, m, need, W, pf, R + 1, F, idx_bits, true, sm.hist, sm.small, sm.scan, sm.sel,
                                sm.ctr, out, okey, k, P.status);
    }

    if (multi) {
        // clear the half the previous launch used, record this launch's use
        // and hand the other half to the next launch
        const int op = p ^ 1;
        const uint32_t prev = op ? used1 : used0;
        const uint32_t ur = min(prev & 15u, (uint32_t)kRounds);
        const uint32_t uc = min((prev >> 4) & 15u, (uint32_t)kMergeCopies);
        const uint32_t us = min(prev >> 8, (uint32_t)kCap);
        uint64_t* const h = &ws->hist[op][0][0][0];
        for (uint32_t i = tid; i < ur * kMergeCopies * 256u; i += BLOCK)
            if ((i / 256u) % kMergeCopies < uc) st_dev(&h[i], (uint64_t)0);
        for (uint32_t i = tid; i < us; i += BLOCK) st_dev(&ws->stage[op][i], (uint64_t)0);
        if (tid == 0) {
            const uint32_t stage = whole ? 0u : (hb > (uint32_t)kCap ? (uint32_t)kCap : hb);
            st_dev(&ws->used[p], (uint32_t)(last_slot + 1) | ((uint32_t)C << 4) | (stage << 8));
            st_dev(&ws->parity, (uint32_t)op);
        }
    }
}

// ----------------------------------------------------------------- one WG per row
//
// Batches of many rows: one WG owns a whole row and streams it in tiles of
// BLOCK x ITEMS logits, the next PD tiles' loads in flight while the
// current one is processed.  During that single read it keeps every element
// whose key is at or above a running lower bound in an LDS buffer (the
// bound estimated from the elements seen so far and raised as the buffer
// fills); when the buffer ends up holding at least k elements, the row's
// k-th largest is the buffer's and the row is finished from LDS: a 12-bit
// first digit (4096 bins), winners out, the threshold bin to the on-chip
// finish.  Otherwise the row is finished with re-reads (a full 12-bit
// histogram, more rounds while the bucket is large, a collection pass whose
// positions come from two wave-aggregated LDS counters).

// candidate buffer of the one-WG-per-row kernel (entries): as large as two
// WGs per CU allow with some LDS to spare (78 KB per WG)
constexpr int kRowsCap = 5376;
constexpr uint32_t kRowsDenseBin = 512;  // a bound bin holding more buffered entries is refined

template <int BLOCK>
struct RowsSmem {
    union {
        uint32_t h12[2 * 4097];                  // first digit: 2 copies of 4096 bins (stride 4097)
        alignas(16) uint32_t h8[kCopies * 257];  // later 8-bit rounds and the finisher
    } h;
    uint64_t cand[kRowsCap];  // candidates at or above the running bound; later the final bucket
    uint64_t small[kSmall];
    uint32_t scan[BLOCK / 64];
    uint32_t sel[4];
    uint32_t ctr[5];  // winners, bucket, finisher (2), buffered entries
};

template <int BLOCK, int ITEMS, int PD, bool KEYS>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4))) void topk_rows_kernel(const KParams P) {
    static_assert(ITEMS % 4 == 0, "ITEMS counts whole 16-byte chunks");
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
    int32_t* __restrict__ out = P.out + (size_t)row * (size_t)k;
    uint32_t* const okey = KEYS ? P.keys + (size_t)row * (size_t)k : nullptr;  // recorded keys (ordered output)
    int L = n;
    if (P.lengths) {
        L = P.lengths[row];
        L = L < 0 ? 0 : (L > n ? n : L);
    }
    if (L <= k) {  // everything valid is selected; pad with -1
        for (int i = tid; i < k; i += BLOCK) out[i] = i < L ? i : -1;
        return;
    }
    const int off = (int)(((uintptr_t)prow >> 2) & 3);
    const int nchunks = (off + L + 3) >> 2;
    const int cf_lo = off ? 1 : 0;         // chunks whose four elements are all valid
    const int cf_hi = (L + off) >> 2;
    const int idx_bits = P.idx_bits;
    const int nrounds = num_rounds(idx_bits);
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
                    buf[d][j] = *reinterpret_cast<const uint4*>(base + (uint32_t)(c < nchunks ? c : 0) * 16u);
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
                            buf[d][j] = *reinterpret_cast<const uint4*>(base + (uint32_t)(c < nchunks ? c : 0) * 16u);
                        }
                    }
                    f(keys, ct);
                }
            }
        }
    };

    // ---------------- first pass: every element whose key is at or above a
    // lower bound `lo_key` kept in LDS.  The bound is an estimate: the
    // first-digit bin (12 bits) of the element of rank 1.125 * k * seen / L
    // + 16 among the `seen` elements read so far, where the k-th largest of
    // the row is expected near rank k * seen / L (in a dense bin, also that
    // element's next 8 key bits).  It is taken from the first tile and
    // raised (with the buffer compacted) whenever the buffer fills up, from
    // histograms of the buffer.  The buffer then holds every element whose
    // key is at or above the bound; when it holds at least k entries, the
    // k-th largest of the buffer is the row's and everything selected is in
    // it.  Otherwise, or when the buffer overflowed twice on one tile, the
    // row is finished with re-reads.
    {
        uint4* const h4 = reinterpret_cast<uint4*>(sm.h.h12);
        for (int i = tid; i < 2 * 4097 / 4; i += BLOCK) h4[i] = uint4{0u, 0u, 0u, 0u};
        if (tid < (2 * 4097) % 4) sm.h.h12[2 * 4097 / 4 * 4 + tid] = 0u;
        if (tid < 5) sm.ctr[tid] = 0u;
    }
    lds_sync();
    bool keep = true;   // candidates are being buffered
    uint32_t used = 0;  // buffered entries
    // running lower bound on the keys kept: a first-digit bin, refined by
    // the next 8 key bits where that bin is dense (at least 1: empty slots
    // are never kept)
    uint32_t lo_key = 1u;
    // Walk the buffer in slices of RC * BLOCK entries: every thread reads its
    // RC entries, a block scan numbers the chosen ones, and f(entry, kind,
    // rank) places them.  Kinds: pred returns 0 (drop), 1 or 2, counted
    // separately (ranks are per kind, across slices).  A chosen entry of
    // kind 2 may be moved to the front of the buffer: its new index is never
    // above its old one, and each slice is read before any of it is written.
    constexpr int RC = 3;
    auto walk = [&](auto&& pred, auto&& f, uint32_t& n1, uint32_t& n2) {
        n1 = 0;
        n2 = 0;
        for (uint32_t i0 = 0; i0 < used; i0 += RC * BLOCK) {
            uint64_t e[RC];
            uint32_t kinds = 0, cnt = 0;
#pragma unroll
            for (int u = 0; u < RC; ++u) {
                const uint32_t i = i0 + (uint32_t)(u * BLOCK + tid);
                e[u] = i < used ? sm.cand[i] : 0ull;
                const uint32_t kd = i < used ? pred(e[u]) : 0u;
                kinds |= kd << (2 * u);
                cnt += kd == 1u ? (1u << 16) : (kd == 2u ? 1u : 0u);
            }
            uint32_t tot;
            const uint32_t pos = block_scan_total<BLOCK>(cnt, sm.scan, tot);
            uint32_t p1 = n1 + (pos >> 16), p2 = n2 + (pos & 0xFFFFu);
#pragma unroll
            for (int u = 0; u < RC; ++u) {
                const uint32_t kd = (kinds >> (2 * u)) & 3u;
                if (kd == 1u) f(e[u], 1u, p1++);
                else if (kd == 2u) f(e[u], 2u, p2++);
            }
            n1 += tot >> 16;
            n2 += tot & 0xFFFFu;
        }
    };
    // rank of the bound after `seen` valid elements
    auto bound_rank = [&](uint32_t seen) -> uint32_t {
        // the margin at the end of the row, k / 8, is several standard
        // deviations of the count above a fixed rank for values drawn alike
        // along the row; a looser bound buffers (and later partitions) more
        const uint64_t est = ((uint64_t)k * seen * 9u) / (8u * (uint64_t)L) + 16u;
        return (uint32_t)(est < seen ? est : seen);
    };
    // the first-digit histogram of the buffered entries
    auto hist_from_buffer = [&]() {
        uint4* const h4 = reinterpret_cast<uint4*>(sm.h.h12);
        for (int i = tid; i < 2 * 4097 / 4; i += BLOCK) h4[i] = uint4{0u, 0u, 0u, 0u};
        if (tid < (2 * 4097) % 4) sm.h.h12[2 * 4097 / 4 * 4 + tid] = 0u;
        lds_sync();
        uint32_t* const hcb = sm.h.h12 + (tid & 1) * 4097;
        for (uint32_t i = (uint32_t)tid; i < used; i += BLOCK) atomicAdd(&hcb[(uint32_t)(sm.cand[i] >> (64 - F))], 1u);
        lds_sync();
    };
    // the element of rank `rank` among the buffered entries (all in
    // first-digit bins at or above lo, the bound's bin), over a 256-bin
    // window of bins lo .. lo+254, the last bin taking everything above: its
    // window bin, the count above it and the count in it (0 when there are
    // fewer entries)
    auto window_select = [&](uint32_t rank, uint32_t& bw, uint32_t& ab, uint32_t& hbw) {
        const uint32_t lo = lo_key >> (32 - F);
        {
            uint4* const h4 = reinterpret_cast<uint4*>(sm.h.h8);
            for (int i = tid; i < kCopies * 257 / 4; i += BLOCK) h4[i] = uint4{0u, 0u, 0u, 0u};
        }
        lds_sync();
        {
            uint32_t* const hcw = sm.h.h8 + (tid % kCopies) * 257;
            for (uint32_t i = (uint32_t)tid; i < used; i += BLOCK) {
                const uint32_t bin = (uint32_t)(sm.cand[i] >> (64 - F));
                atomicAdd(&hcw[min(bin - lo, 255u)], 1u);
            }
        }
        lds_sync();
        local_select<BLOCK, 256, kCopies, 257, false>(sm.h.h8, 0u, rank, sm.scan, sm.sel, P.status, bw, ab, hbw);
    };
    // the element of rank `rank` among the buffered entries of first-digit
    // bin b: its next 8 key bits (sub-bin s8), the count above it in the bin
    // and the count in it (0 when there are fewer entries)
    auto sub_select = [&](uint32_t b, uint32_t rank, uint32_t& s8, uint32_t& a8, uint32_t& h8v) {
        {
            uint4* const h4 = reinterpret_cast<uint4*>(sm.h.h8);
            for (int i = tid; i < kCopies * 257 / 4; i += BLOCK) h4[i] = uint4{0u, 0u, 0u, 0u};
        }
        lds_sync();
        {
            uint32_t* const hcw = sm.h.h8 + (tid % kCopies) * 257;
            for (uint32_t i = (uint32_t)tid; i < used; i += BLOCK) {
                const uint32_t key = (uint32_t)(sm.cand[i] >> 32);
                if ((key >> (32 - F)) == b) atomicAdd(&hcw[(key >> (32 - F - 8)) & 0xFFu], 1u);
            }
        }
        lds_sync();
        local_select<BLOCK, 256, kCopies, 257, false>(sm.h.h8, 0u, rank, sm.scan, sm.sel, P.status, s8, a8, h8v);
    };
    {
        const uint32_t lane = lane_id();
        stream([&](const uint32_t* keys, int ct) {
            if (!keep) return;  // overflowed: the fallback re-reads the row
            // valid elements read once this tile is done
            const uint32_t seen = (uint32_t)min(L, 4 * min(nchunks, ct + TILE_CHUNKS) - off);
            if (ct == 0) {
                // the first bound, from the first tile: the 12-bit bin of the
                // element of rank bound_rank(seen), in two steps — its top 8
                // bits (256-bin histogram, 16 copies), then its next 4 bits
                // among the elements of that 8-bit bin (16 bins).  The union
                // is all zero here.
                uint32_t* const h8c = sm.h.h8 + (tid % kCopies) * 257;
#pragma unroll
                for (int i = 0; i < ITEMS; ++i)
                    if (keys[i] != 0u) atomicAdd(&h8c[keys[i] >> 24], 1u);
                lds_sync();
                uint32_t b8, ab8, hb8;
                const uint32_t rk = bound_rank(seen);
                local_select<BLOCK, 256, kCopies, 257, false>(sm.h.h8, 0u, rk, sm.scan, sm.sel, P.status, b8, ab8,
                                                              hb8);
                if (hb8 > 0u) {
                    uint32_t* const h4 = sm.h.h12 + kCopies * 257 + (tid % kCopies) * 17;  // past the 8-bit copies
#pragma unroll
                    for (int i = 0; i < ITEMS; ++i)
                        if ((keys[i] != 0u) & ((keys[i] >> 24) == b8)) atomicAdd(&h4[(keys[i] >> 20) & 15u], 1u);
                    lds_sync();
                    if (tid < 64) {
                        // lane l: sub-bin 15 - l (descending), summed over the copies
                        uint32_t c = 0;
                        if (tid < 16) {
#pragma unroll
                            for (int q = 0; q < kCopies; ++q) c += sm.h.h12[kCopies * 257 + q * 17 + 15 - tid];
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
            // append: lanes count their candidates, a wave prefix ranks
            // them, one LDS atomic per wave reserves the wave's range.  A
            // tile that overflows the buffer (its entries past the end are
            // lost) raises the bound from what is buffered, drops its own
            // entries and is appended once more from the registers; a
            // second overflow gives up (the re-reading path below).
            for (int pass = 0;; ++pass) {
                uint32_t c = 0;
#pragma unroll
                for (int i = 0; i < ITEMS; ++i) c += keys[i] >= lo_key;
                const uint32_t ic = wave_inclusive_scan(c);
                const uint32_t tw = (uint32_t)__builtin_amdgcn_readlane((int)ic, 63);
                if (tw) {
                    uint32_t wb = 0;
                    if (lane == 0) wb = atomicAdd(&sm.ctr[4], tw);
                    uint32_t pos = (uint32_t)__builtin_amdgcn_readlane((int)wb, 0) + ic - c;
                    const int ibase = 4 * (ct + tid) - off;
#pragma unroll
                    for (int j = 0; j < CHUNKS; ++j) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t key = keys[4 * j + e];
                            if (key >= lo_key) {
                                if (pos < (uint32_t)kRowsCap)
                                    sm.cand[pos] = ((uint64_t)key << 32) |
                                                   (uint64_t)~(uint32_t)(ibase + 4 * BLOCK * j + e);
                                ++pos;
                            }
                        }
                    }
                }
                lds_sync();
                used = uniform(sm.ctr[4]);
                const bool over = used > (uint32_t)kRowsCap;  // entries of this tile were lost
                if (over && pass > 0) {
                    keep = false;
                    return;
                }
                if (!over && !(used > (uint32_t)kRowsCap * 3u / 4u && ct + TILE_CHUNKS < nchunks)) break;
                if (over) used = (uint32_t)kRowsCap;
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
                uint32_t n1, n2;
                walk([&](uint64_t e) {
                         const int idx = (int)~(uint32_t)e;
                         return ((uint32_t)(e >> 32) >= lob) & ((idx < xlo) | (idx >= xhi)) ? 2u : 0u;
                     },
                     [&](uint64_t e, uint32_t, uint32_t r) { sm.cand[r] = e; }, n1, n2);
                used = n2;
                if (tid == 0) sm.ctr[4] = n2;
                lds_sync();
                if (!over) break;
            }
        });
    }
    // the first tile of the row `ahead` rows on (the one that probably runs
    // next on this WG's XCD) is touched now: its loads then hit the caches
    uint32_t sink = 0;
    if (P.ahead > 0 && row + P.ahead < P.rows && tid * 16 < n)
        sink = *reinterpret_cast<const uint32_t*>(P.logits + (size_t)(row + P.ahead) * (size_t)n + tid * 16);
    auto done = [&]() { __asm__ volatile("" ::"v"(sink)); };
    lds_sync();
    Prefix pf{0u, 0u, 0u, 0u};
    uint32_t need = (uint32_t)k, W = 0, hb = 0;
    int R = 0;
    bool whole = false;
    uint32_t b0 = 0, above = 0;
    if (keep) {
        // the threshold bin, from the buffer: first over the 256-bin window
        // from the bound's bin, which normally holds it; else over all 4096
        // bins
        uint32_t bw;
        window_select(need, bw, above, hb);
        if (hb > 0u && bw < 255u) {
            b0 = (lo_key >> (32 - F)) + bw;
        } else {
            hist_from_buffer();
            local_select<BLOCK, NB0, 2, 4097, false>(sm.h.h12, 0u, need, sm.scan, sm.sel, P.status, b0, above, hb);
        }
    }
    // one finisher call for both paths (its code inlined once)
    uint32_t fin_m = 0;
    int fin_r0 = 1;
    if (keep && hb > 0u && b0 >= (lo_key >> (32 - F))) {
        need -= above;
        W += above;
        pf.add(F, 0, b0, idx_bits);
        whole = hb == need;
        // every element at or above bin b0 is buffered: winners (above b0)
        // to the output, the bucket (bin b0) to the front of the buffer, or
        // to the output when it is taken whole
        uint32_t nw, nbk;
        const uint32_t bsel = b0;
        const bool wh = whole;
        const uint32_t Wv = W;
        walk([&](uint64_t e) {
                 const uint32_t bin = (uint32_t)(e >> (64 - F));
                 return bin > bsel ? 1u : (bin == bsel ? 2u : 0u);
             },
             [&](uint64_t e, uint32_t kind, uint32_t r) {
                 if (kind == 1u) {
                     if (r < Wv) {
                         out[r] = (int32_t)~(uint32_t)e;
                         if (okey) okey[r] = (uint32_t)(e >> 32);
                     }
                 } else if (wh) {
                     if (Wv + r < (uint32_t)k) {
                         out[Wv + r] = (int32_t)~(uint32_t)e;
                         if (okey) okey[Wv + r] = (uint32_t)(e >> 32);
                     }
                 } else {
                     sm.cand[r] = e;
                 }
             },
             nw, nbk);
        const bool bad = nw != W || nbk != hb;
        if (bad && tid == 0) raise_flag(P.status, kFlagCapacity);
        if (whole) {
            done();
            return;
        }
        fin_m = hb;
        fin_r0 = 1;
    } else {
        // ---------------- fallback: the full first-digit histogram by a second
        // read, then rounds and collection by further reads.  Rare (the
        // estimated bound failed), so its passes are rolled loops of U chunks
        // per lane: small code and few registers beside the streaming pass
        // above (measured: the fallback written like the first pass, unrolled
        // over whole tiles, costs that pass 14 % on the causal batch).
        constexpr int U = 2;
        auto reread = [&](auto&& f) {
    #pragma unroll 1
            for (int c0 = 0; c0 < nchunks; c0 += U * BLOCK) {
                u32x4_t v[U];
    #pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + u * BLOCK + tid;
                    v[u] = *reinterpret_cast<const u32x4_t*>(base + (uint32_t)(c < nchunks ? c : 0) * 16u);
                }
                uint32_t kk[4 * U], nn[4 * U];  // keys (0: empty slot) and ~indices
    #pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + u * BLOCK + tid;
                    const int e0 = 4 * c - off;
    #pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool ok = (c < nchunks) & ((uint32_t)(e0 + e) < (uint32_t)L);
                        kk[4 * u + e] = ok ? key_of(__uint_as_float(v[u][e])) : 0u;
                        nn[4 * u + e] = ~(uint32_t)(e0 + e);
                    }
                }
                f(kk, nn);
            }
        };
        {
            {
                uint4* const h4 = reinterpret_cast<uint4*>(sm.h.h12);
                for (int i = tid; i < 2 * 4097 / 4; i += BLOCK) h4[i] = uint4{0u, 0u, 0u, 0u};
                if (tid < (2 * 4097) % 4) sm.h.h12[2 * 4097 / 4 * 4 + tid] = 0u;
            }
            lds_sync();
            uint32_t* const hc = sm.h.h12 + (tid & 1) * 4097;
            reread([&](const uint32_t* kk, const uint32_t*) {
    #pragma unroll
                for (int i = 0; i < 4 * U; ++i)
                    if (kk[i] != 0u) atomicAdd(&hc[kk[i] >> (32 - F)], 1u);
            });
            lds_sync();
        }
        local_select<BLOCK, NB0, 2, 4097>(sm.h.h12, 0u, need, sm.scan, sm.sel, P.status, b0, above, hb);
        need -= above;
        W += above;
        pf.add(F, 0, b0, idx_bits);
        whole = hb == need;
        // ---------------- further rounds (only when the bucket is still large)
        for (int r = 1; !whole && hb > (uint32_t)kCap && r < nrounds; ++r) {
            {
                uint4* const h4 = reinterpret_cast<uint4*>(sm.h.h8);
                for (int i = tid; i < kCopies * 257 / 4; i += BLOCK) h4[i] = uint4{0u, 0u, 0u, 0u};
            }
            lds_sync();
            uint32_t* const hc = sm.h.h8 + (tid % kCopies) * 257;
            const int sh = digit_shift(F, r, idx_bits);
            const uint32_t dm = digit_mask(F, r);
            reread([&](const uint32_t* kk, const uint32_t* nn) {
    #pragma unroll
                for (int i = 0; i < 4 * U; ++i)
                    if (pf.match(kk[i], nn[i])) atomicAdd(&hc[((r < 4 ? kk[i] : nn[i]) >> sh) & dm], 1u);
            });
            lds_sync();
            uint32_t b, above;
            local_select<BLOCK, 256, kCopies, 257>(sm.h.h8, 0u, need, sm.scan, sm.sel, P.status, b, above, hb);
            need -= above;
            W += above;
            pf.add(F, r, b, idx_bits);
            R = r;
            whole = hb == need;
        }
        // ---------------- collection: winners to the output, the bucket to LDS
        // (or to the output when it is taken whole).  Positions per step: each
        // lane counts its winners and bucket elements, a wave prefix (DPP) ranks
        // the lanes, and one LDS atomic per wave and kind reserves the wave's
        // range.
        bool overflow = false;
        const uint32_t lane = lane_id();
        reread([&](const uint32_t* kk, const uint32_t* nn) {
            uint32_t mw = 0, mbk = 0;  // this lane's winners / bucket elements, one bit per slot
    #pragma unroll
            for (int i = 0; i < 4 * U; ++i) {
                mw |= (uint32_t)((kk[i] != 0u) & pf.above(kk[i], nn[i])) << i;
                mbk |= (uint32_t)pf.match(kk[i], nn[i]) << i;
            }
            const uint32_t nw = (uint32_t)__builtin_popcount(mw), nb = (uint32_t)__builtin_popcount(mbk);
            const uint32_t iw = wave_inclusive_scan(nw), ib = wave_inclusive_scan(nb);
            const uint32_t tw = (uint32_t)__builtin_amdgcn_readlane((int)iw, 63);
            const uint32_t tb = (uint32_t)__builtin_amdgcn_readlane((int)ib, 63);
            if (tw | tb) {
                uint32_t bw = 0, bb = 0;
                if (lane == 0) {
                    if (tw) bw = atomicAdd(&sm.ctr[0], tw);
                    if (tb) bb = atomicAdd(&sm.ctr[1], tb);
                }
                uint32_t pw = (uint32_t)__builtin_amdgcn_readlane((int)bw, 0) + iw - nw;
                uint32_t pb = (uint32_t)__builtin_amdgcn_readlane((int)bb, 0) + ib - nb;
    #pragma unroll
                for (int i = 0; i < 4 * U; ++i) {
                    const uint32_t key = kk[i], ni = nn[i];
                    if ((mw >> i) & 1u) {
                        if (pw < W) {
                            out[pw] = (int32_t)~ni;
                            if (okey) okey[pw] = key;
                        } else {
                            overflow = true;
                        }
                        ++pw;
                    } else if ((mbk >> i) & 1u) {
                        if (whole) {
                            if (W + pb < (uint32_t)k) {
                                out[W + pb] = (int32_t)~ni;
                                if (okey) okey[W + pb] = key;
                            } else {
                                overflow = true;
                            }
                        } else if (pb < (uint32_t)kCap) {
                            sm.cand[pb] = ((uint64_t)key << 32) | (uint64_t)ni;
                        } else {
                            overflow = true;
                        }
                        ++pb;
                    }
                }
            }
        });
        if (overflow) raise_flag(P.status, kFlagCapacity);
        if (whole) {
            done();
            return;
        }
        fin_m = hb > (uint32_t)kCap ? (uint32_t)kCap : hb;
        fin_r0 = R + 1;
    }
    lds_sync();
    finish_bucket<BLOCK>(sm.cand, fin_m, need, W, pf, fin_r0, F, idx_bits, false, sm.h.h8, sm.small, sm.scan, sm.sel,
                            &sm.ctr[2], out, okey, k, P.status);
    done();
}

// ----------------------------------------------------------------- ordered output
// The ordered form of the selection: section 02 of the TopK article gives
// radix_topk a need_sorted option that sorts the collected output in
// descending order; equal values are ordered by index ascending, the same
// rule that decides which of them are selected.  The selection kernels
// record, beside each output index, the key of its element; then one WG
// per row sorts the row's composites (key << 32 | ~index) in descending
// order with a bitonic network.  Rows longer than kSortRun are cut into
// runs of kSortRun that are sorted on chip, then merged pairwise in global
// memory (merge path: each thread finds where its outputs start on both
// runs by a binary search, then merges a few entries).

constexpr int kSortRun = 8192;  // composites one WG sorts on chip
constexpr int kMergeBlock = 256, kMergeItems = 8;

struct SortParams {
    const float* logits;
    const int32_t* lengths;
    int32_t* out;
    float* vals;            // [rows, k] or null
    const int32_t* idx;     // [rows, k]: the selection's output (unordered)
    const uint32_t* keys;   // [rows, k]: the key at each slot of idx
    const uint64_t* src;    // merge input, [rows, kp]
    uint64_t* dst;          // sorted runs / merge output, [rows, kp] (null: to out/vals)
    int32_t rows, n, k;
    int32_t kp;             // padded row length of the runs (multiple of kSortRun)
    int32_t nruns;          // runs per row (rank kernel: WGs per row)
    int32_t width;          // merge: length of the runs being merged
};

// The composite of slot g of a row's unordered selection: from the
// recorded key and index, or, when the whole valid row is selected (L <= k:
// the selection then writes 0..L-1 and records no keys), from the logits.
__device__ __forceinline__ uint64_t sort_input(const SortParams& P, int row, int L, uint32_t g) {
    uint32_t idx, key;
    if (L <= P.k) {
        idx = g;
        key = key_of(P.logits[(size_t)row * (size_t)P.n + g]);
    } else {
        const size_t at = (size_t)row * (size_t)P.k + g;
        idx = (uint32_t)P.idx[at];
        key = P.keys[at];
    }
    return ((uint64_t)key << 32) | (uint64_t)~idx;
}

// The logit a key came from; -0.0 and +0.0 share a key, so a zero key reads
// the logit itself to return its sign.
__device__ __forceinline__ float value_of(uint32_t key, const float* prow, uint32_t L, uint32_t idx) {
    if (key == 0x80000000u) return idx < L ? prow[idx] : 0.0f;
    return __uint_as_float(key & 0x80000000u ? key ^ 0x80000000u : ~key);
}

// Write output slot j of a row from a composite (0 = no element: -1, -inf).
__device__ __forceinline__ void put_sorted(uint64_t c, int32_t* orow, float* vrow, const float* prow, uint32_t L,
                                           uint32_t j) {
    const uint32_t idx = ~(uint32_t)c;
    const bool has = c != 0ull;
    orow[j] = has ? (int32_t)idx : -1;
    if (vrow) vrow[j] = has ? value_of((uint32_t)(c >> 32), prow, L, idx) : -__builtin_huge_valf();
}

__device__ __forceinline__ int valid_length(const int32_t* lengths, int row, int n) {
    if (!lengths) return n;
    const int L = lengths[row];
    return L < 0 ? 0 : (L > n ? n : L);
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a > b ? b : a; }

// Keep the larger of (mine, other) when keep_max, else the smaller: one
// 64-bit compare and two selects.
__device__ __forceinline__ uint64_t bitonic_pick(uint64_t mine, uint64_t other, bool keep_max) {
    return ((mine > other) == keep_max) ? mine : other;
}

// One bitonic step whose partner lanes are a DPP quad permutation away
// (QP 0xB1: lane ^ 1, 0x4E: lane ^ 2).
template <int E, int QP>
__device__ __forceinline__ void dpp_step(uint64_t (&c)[E], bool keep_max) {
#pragma unroll
    for (int u = 0; u < E; ++u) {
        const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)c[u], QP, 0xF, 0xF, false);
        const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(c[u] >> 32), QP, 0xF, 0xF, false);
        c[u] = bitonic_pick(c[u], ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo, keep_max);
    }
}

// Bitonic sort, descending, of the first Sp (a power of two, 2 <= Sp <=
// BLOCK*E) of the WG's BLOCK*E composites; entry e = tid*E + u is c[u] of
// thread tid.  At merge level p, entry e belongs to a descending block when
// (e & p) == 0; of the pair (e, e ^ j) the lower entry of a descending block
// keeps the larger value.  For j >= E (partner in another thread) both
// tests depend on the thread only, so each step costs one compare and two
// selects per entry.  buf: 2*BLOCK*E composites of LDS (double buffer, so
// one barrier per cross-wave step).  Every thread of the WG calls it.
template <int BLOCK, int E>
__device__ __forceinline__ void bitonic_desc(uint64_t (&c)[E], uint32_t Sp, uint64_t* buf) {
    const uint32_t e0 = threadIdx.x * (uint32_t)E;
    int par = 0;
    for (uint32_t p = 2; p <= Sp; p <<= 1) {
        const bool desc = (e0 & p) == 0u || p < (uint32_t)E;  // p < E: decided per entry below
        uint32_t j = p >> 1;
        for (; j >= 64u * E; j >>= 1) {  // partner in another wave
            uint64_t* const b = buf + par * (BLOCK * E);
            par ^= 1;
#pragma unroll
            for (int u = 0; u < E; ++u) b[e0 + u] = c[u];
            __syncthreads();
            const bool keep_max = ((e0 & j) == 0u) == desc;
            uint64_t o[E];
#pragma unroll
            for (int u = 0; u < E; ++u) o[u] = b[(e0 + (uint32_t)u) ^ j];
#pragma unroll
            for (int u = 0; u < E; ++u) c[u] = bitonic_pick(c[u], o[u], keep_max);
        }
        for (; j >= 4u * E; j >>= 1) {  // partner in another lane of the wave
            // every partner value of the step is fetched before any is used,
            // so the lane exchanges overlap
            const int lj = (int)(j / (uint32_t)E);
            const bool keep_max = ((e0 & j) == 0u) == desc;
            uint64_t o[E];
#pragma unroll
            for (int u = 0; u < E; ++u) o[u] = (uint64_t)__shfl_xor((unsigned long long)c[u], lj);
#pragma unroll
            for (int u = 0; u < E; ++u) c[u] = bitonic_pick(c[u], o[u], keep_max);
        }
        // partners 2 and 1 lanes away: DPP quad permutations, no LDS trip
        if (j == 2u * E) {
            dpp_step<E, 0x4E>(c, ((e0 & j) == 0u) == desc);
            j >>= 1;
        }
        if (j == (uint32_t)E) dpp_step<E, 0xB1>(c, ((e0 & j) == 0u) == desc);
#pragma unroll
        for (int jj = E / 2; jj >= 1; jj >>= 1) {  // partner in this thread
            if ((uint32_t)jj < p) {
#pragma unroll
                for (int u = 0; u < E; ++u) {
                    if ((u & jj) == 0) {
                        const bool d = p < (uint32_t)E ? (((uint32_t)u & p) == 0u) : desc;
                        const uint64_t a = c[u], b2 = c[u | jj];
                        const bool sw = (a < b2) == d;
                        c[u] = sw ? b2 : a;
                        c[u | jj] = sw ? a : b2;
                    }
                }
            }
        }
    }
}

// One WG per (row, run): load the run's composites (from the recorded keys,
// or from the logits when the whole valid row is selected), sort them, and
// write them to the output (one run per row) or to dst.
template <int BLOCK, int E>
__global__ void __launch_bounds__(BLOCK) topk_sort_kernel(SortParams P) {
    __shared__ uint64_t buf[2 * BLOCK * E];
    const int row = blockIdx.x / P.nruns;
    const int run = blockIdx.x - row * P.nruns;
    const int n = P.n, k = P.k;
    const int L = valid_length(P.lengths, row, n);
    const uint32_t take = (uint32_t)(L < k ? L : k);
    const float* const prow = P.logits + (size_t)row * (size_t)n;
    int32_t* const orow = P.out + (size_t)row * (size_t)k;
    float* const vrow = P.vals ? P.vals + (size_t)row * (size_t)k : nullptr;
    const uint32_t r0 = (uint32_t)run * (uint32_t)kSortRun;
    const uint32_t cnt = take > r0 ? min(take - r0, (uint32_t)(BLOCK * E)) : 0u;
    const uint32_t e0 = threadIdx.x * (uint32_t)E;
    uint64_t c[E];
#pragma unroll
    for (int u = 0; u < E; ++u) {
        const uint32_t e = e0 + (uint32_t)u;
        c[u] = e < cnt ? sort_input(P, row, L, r0 + e) : 0ull;
    }
    uint32_t Sp = 2;
    while (Sp < cnt) Sp <<= 1;
    bitonic_desc<BLOCK, E>(c, Sp, buf);
    if (P.dst) {
        uint64_t* const drow = P.dst + (size_t)row * (size_t)P.kp + r0;
#pragma unroll
        for (int u = 0; u < E; ++u) drow[e0 + u] = c[u];
        return;
    }
#pragma unroll
    for (int u = 0; u < E; ++u) {
        const uint32_t e = e0 + (uint32_t)u;
        if (e < take) put_sorted(c[u], orow, vrow, prow, (uint32_t)L, e);
    }
    for (uint32_t j = take + threadIdx.x; j < (uint32_t)k; j += BLOCK) put_sorted(0ull, orow, vrow, prow, 0u, j);
}

// One merge pass: runs of P.width entries, pairwise, descending.  Each
// thread writes kMergeItems consecutive entries of the merged pair: to dst,
// or (last pass) to the output.  Equal composites (only the zero padding)
// come from the first run first.
__global__ void __launch_bounds__(kMergeBlock) topk_merge_kernel(SortParams P) {
    const uint32_t per_row = (uint32_t)P.kp / (kMergeBlock * kMergeItems);
    const uint32_t row = blockIdx.x / per_row;
    const uint32_t o = ((blockIdx.x - row * per_row) * kMergeBlock + threadIdx.x) * kMergeItems;
    const uint32_t w = (uint32_t)P.width, kp = (uint32_t)P.kp;
    const uint32_t base = o / (2u * w) * (2u * w);
    const uint32_t lenA = min(w, kp - base);
    const uint32_t lenB = kp - base > w ? min(w, kp - base - w) : 0u;
    const uint64_t* const A = P.src + (size_t)row * kp + base;
    const uint64_t* const B = A + w;
    const uint32_t d = o - base;
    // co-rank: how many of the first d merged entries come from A
    uint32_t lo = d > lenB ? d - lenB : 0u, hi = min(d, lenA);
    while (lo < hi) {
        const uint32_t mid = (lo + hi) >> 1;
        if (A[mid] >= B[d - mid - 1u]) lo = mid + 1u;
        else hi = mid;
    }
    uint32_t i = lo, j = d - lo;
    const int k = P.k;
    int32_t* const orow = P.out + (size_t)row * (size_t)k;
    float* const vrow = P.vals ? P.vals + (size_t)row * (size_t)k : nullptr;
    const float* const prow = P.logits + (size_t)row * (size_t)P.n;
    const uint32_t L = P.dst ? 0u : (uint32_t)valid_length(P.lengths, (int)row, P.n);
#pragma unroll
    for (int t = 0; t < kMergeItems; ++t) {
        const uint64_t a = i < lenA ? A[i] : 0ull;
        const uint64_t b = j < lenB ? B[j] : 0ull;
        const bool fromA = j >= lenB || (i < lenA && a >= b);
        const uint64_t v = fromA ? a : b;
        i += fromA;
        j += !fromA;
        const uint32_t pos = o + (uint32_t)t;
        if (P.dst) P.dst[(size_t)row * kp + pos] = v;
        else if (pos < (uint32_t)k) put_sorted(v, orow, vrow, prow, L, pos);
    }
}

// Few rows: each row's order is spread over RG = P.nruns WGs.  Every WG
// holds the row's take composites in LDS and places a share of them: the
// output position of a composite is the number of larger ones, counted by
// Q lanes per composite over strided parts of the row (then added by lane
// shuffles).  Rows of at most kRankMax selected entries.
constexpr int kRankMax = 4096;
constexpr int kRankBlock = 256;

__global__ void __launch_bounds__(kRankBlock) topk_rank_kernel(SortParams P) {
    __shared__ uint64_t all[kRankMax];
    const int RG = P.nruns;
    const int row = blockIdx.x / RG;
    const int w = blockIdx.x - row * RG;
    const int tid = threadIdx.x;
    const int n = P.n, k = P.k;
    const int L = valid_length(P.lengths, row, n);
    const uint32_t take = (uint32_t)(L < k ? L : k);
    for (uint32_t g = tid; g < take; g += kRankBlock) all[g] = sort_input(P, row, L, g);
    __syncthreads();
    const float* const prow = P.logits + (size_t)row * (size_t)n;
    int32_t* const orow = P.out + (size_t)row * (size_t)k;
    float* const vrow = P.vals ? P.vals + (size_t)row * (size_t)k : nullptr;
    if (w == 0)
        for (uint32_t j = take + tid; j < (uint32_t)k; j += kRankBlock) put_sorted(0ull, orow, vrow, prow, 0u, j);
    const uint32_t chunk = (take + RG - 1) / RG;
    const uint32_t first = (uint32_t)w * chunk;
    if (chunk == 0u || first >= take) return;
    const uint32_t cnt = min(chunk, take - first);
    uint32_t Q = 1;
    while (Q < 64u && 2u * Q * cnt <= (uint32_t)kRankBlock) Q *= 2u;
    const uint32_t i = (uint32_t)tid / Q, q = (uint32_t)tid % Q;
    const uint64_t me = i < cnt ? all[first + i] : ~0ull;
    uint32_t above = 0;
    uint32_t j = q;
    for (; j + 3u * Q < take; j += 4u * Q) {
        const uint64_t a = all[j], b = all[j + Q], c = all[j + 2u * Q], d = all[j + 3u * Q];
        above += (uint32_t)(a > me) + (uint32_t)(b > me) + (uint32_t)(c > me) + (uint32_t)(d > me);
    }
    for (; j < take; j += Q) above += (uint32_t)(all[j] > me);
    for (uint32_t sft = 1u; sft < Q; sft <<= 1) above += (uint32_t)__shfl_xor((int)above, (int)sft);
    if (i < cnt && q == 0u) put_sorted(me, orow, vrow, prow, (uint32_t)L, above);
}

// ----------------------------------------------------------------- indexer logits
// The logits the selector is fed (the TopK article, section 01, step 1 of
// DSA: the current query against every historical token).  The article
// gives no formula; the one computed here is the plainest that its
// workloads support: H indexer heads share one key per token and
//     logits[r][t] = sum_h w[r][h] * max(0, q[r][h] . K[r][t]),
// q and K in bf16, products and sums in fp32.  It is a dense contraction,
// so it runs on the matrix cores: v_mfma_f32_16x16x32_bf16 with A = 16 heads
// x 32 dims of the query, B = 32 dims x 16 tokens of the keys.  Operand
// layout (64 lanes): A lane l holds head l%16, dims 8(l/16)..+7; B lane l
// holds token l%16, dims 8(l/16)..+7 — 16 contiguous bytes of one key, one
// 16-byte load; C lane l holds heads 4(l/16)..+3 of token l%16.  A lane
// weights and clamps its four heads, two lane exchanges add the four head
// groups, and each wave stores 64 consecutive logits.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

struct LogitParams {
    const uint16_t* q;      // [rows, H, D] bf16
    const uint16_t* kc;     // keys of row r at kc + r * kstride: [n, D] bf16
    const float* w;         // [rows, H]
    const int32_t* lengths; // [rows] or null
    float* logits;          // [rows, n]; -inf at positions >= the valid length
    int64_t kstride;        // elements between the keys of consecutive rows (0: shared)
    int32_t rows, n, H;
    int32_t gpw;            // groups of 64 tokens per wave
    int32_t tiles;          // WGs per row
};

constexpr int kLogitBlock = 256;  // 4 waves

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    return __builtin_bit_cast(bf16x8_t, v);
}

// The keys of the group (64 tokens of D bf16) at K + 2 D tw bytes, read
// contiguously: load i of a lane is bytes 1024 i + 16 lane of the group.
// Tokens past `last` (the last valid one, relative to tw) read that one
// instead (their values are zeroed when staged keys are used).
template <int D, int NL>
__device__ __forceinline__ void logits_load(u32x4_t (&r)[NL], const char* K, int tw, int last, int lane) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int off = 1024 * i + 16 * lane;
        const int tok = min(off / (2 * D), last);
        r[i] = *reinterpret_cast<const u32x4_t*>(K + ((size_t)(tw + tok) * D) * 2 + (off % (2 * D)));
    }
}

// Store the loaded group in the wave's LDS region: chunk c of token r in
// slot c ^ (r % CPR) of the token's row.
template <int D, int NL>
__device__ __forceinline__ void logits_stage(u32x4_t* st, const u32x4_t (&r)[NL], int lane) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int off = 1024 * i + 16 * lane;
        const int tok = off / (2 * D), c = (off % (2 * D)) / 16;
        st[tok * CPR + (c ^ (tok % CPR))] = r[i];
    }
}

template <int D, int HB>
__global__ void __launch_bounds__(kLogitBlock) topk_logits_kernel(LogitParams P) {
    constexpr int KB = D / 32;
    constexpr int CPR = D / 8;         // 16-byte chunks per key
    constexpr int GB = 64 * D * 2;     // bytes of one group's keys (64 tokens)
    constexpr int NL = GB / 1024;      // 16-byte loads per lane per group
    // each wave stages its current group of keys in its own LDS region;
    // chunk c of token r sits in slot c ^ (r % CPR) of the token's row, so
    // the MFMA-layout reads (16 tokens, one chunk each) hit distinct banks
    __shared__ u32x4_t stage[kLogitBlock / 64][GB / 16];
    // the row's queries, shared by the WG's waves: chunk c of head h in slot
    // c ^ (h % CPR) of the head's row
    __shared__ u32x4_t qs[HB * 16 * CPR];
    const int row = blockIdx.x / P.tiles;
    const int tile = blockIdx.x - row * P.tiles;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int n = P.n, H = P.H;
    const int L = valid_length(P.lengths, row, n);
    // this wave's tokens: gpw consecutive groups of 64
    const int t0 = (tile * (kLogitBlock / 64) + wave) * P.gpw * 64;
    const int t1 = min(t0 + P.gpw * 64, n);
    const int tv = min(t1, L);  // valid tokens end here
    const char* const K = reinterpret_cast<const char*>(P.kc + (size_t)row * (size_t)P.kstride);
    // a wave that streams several groups has its first group's keys in
    // flight while the queries are staged (measured: for one group per
    // wave the keys are better issued after the queries)
    u32x4_t r[NL];
    const bool early = P.gpw > 1 && t0 < tv;
    if (early) logits_load<D, NL>(r, K, t0, L - 1 - t0, lane);
    {
        const u32x4_t* const qrow = reinterpret_cast<const u32x4_t*>(P.q + (size_t)row * H * D);
        for (int i = threadIdx.x; i < H * CPR; i += kLogitBlock) {
            const int h = i / CPR, c = i % CPR;
            qs[h * CPR + (c ^ (h % CPR))] = qrow[i];
        }
    }
    __syncthreads();  // before any wave leaves
    if (t0 >= n) return;
    float* const lrow = P.logits + (size_t)row * (size_t)n;
    const float ninf = -__builtin_huge_valf();
    for (int t = max(t0, tv) + lane; t < t1; t += 64) lrow[t] = ninf;
    if (t0 >= tv) return;
    const int ng = (tv - t0 + 63) / 64;  // groups holding valid tokens
    // queries (A operands, from LDS) and the weights of this lane's four
    // heads per block, once for all of the wave's groups; padding heads are
    // zero
    bf16x8_t a[HB][KB];
    float wt[HB][4];
    const bf16x8_t zero = {};
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        const int h = hb * 16 + m;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int c = kb * 4 + g;
            const bf16x8_t x = __builtin_bit_cast(bf16x8_t, qs[h * CPR + (c ^ (h % CPR))]);
            a[hb][kb] = h < H ? x : zero;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hh = hb * 16 + 4 * g + i;
            const float x = P.w[(size_t)row * H + min(hh, H - 1)];
            wt[hb][i] = hh < H ? x : 0.0f;
        }
    }
    u32x4_t* const st = stage[wave];
    auto compute_store = [&](int tw) __attribute__((always_inline)) {
        float v[4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const int tok = blk * 16 + m;
            const bool ok = tw + tok < L;
            bf16x8_t b[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int c = kb * 4 + g;  // dims 32 kb + 8 g .. +7
                const bf16x8_t x = __builtin_bit_cast(bf16x8_t, st[tok * CPR + (c ^ (tok % CPR))]);
                b[kb] = ok ? x : zero;
            }
            float part = 0.0f;
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) {
                floatx4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[hb][kb], b[kb], acc, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) part += wt[hb][i] * fmaxf(acc[i], 0.0f);
            }
            part += __shfl_xor(part, 16);
            part += __shfl_xor(part, 32);
            v[blk] = part;
        }
        // lane l stores token tw + l: block l/16, token l%16 of it
        const float mine = g == 0 ? v[0] : (g == 1 ? v[1] : (g == 2 ? v[2] : v[3]));
        const int t = tw + lane;
        if (t < t1) lrow[t] = t < L ? mine : ninf;
    };
    // the next group's loads are in flight while the current one is
    // computed from LDS; the wave's region is its own, so no barrier
    if (!early) logits_load<D, NL>(r, K, t0, L - 1 - t0, lane);
    for (int gi = 0; gi < ng; ++gi) {
        const int tw = t0 + gi * 64;
        logits_stage<D, NL>(st, r, lane);
        if (gi + 1 < ng) logits_load<D, NL>(r, K, tw + 64, L - 1 - (tw + 64), lane);
        compute_store(tw);
    }
}

// ----------------------------------------------------------------- attention over the selected positions
// The step after the selection (the TopK article, section 01, step 3 of
// DSA: attention computed only on the keys and values of the k selected
// positions).  The article gives no formula; computed here is plain scaled
// dot-product attention of each query head over the selected positions,
// keys and values shared by the heads:
//     out[r][h] = sum_j softmax_j(scale * q[r][h] . K[idx_j]) V[idx_j],
// over the slots holding a position (-1, or a value outside [0, n), holds
// none).  Split over the slots: a WG takes 64 slots of one row, computes
// the scores on the matrix cores (A = 16 heads x 32 dims of the queries,
// B = 32 dims x 16 gathered keys), a softmax over its slots (maximum m,
// sum l) and P.V on the matrix cores (A = 16 heads x 32 slots of P in bf16,
// B = 32 slots x 16 dims of the gathered values, held transposed in LDS so
// that a lane's 8 slots of one dim are 16 contiguous bytes), and writes
// (m, l, partial output); a second kernel combines a row's chunks.

constexpr int kAttnBlock = 256;  // 4 waves, 16 slots each
constexpr int kAttnSlots = 64;   // slots per WG

struct AttnParams {
    const uint16_t* q;     // [rows, H, D] bf16
    const uint16_t* kc;    // keys of row r at kc + r * kvstride: [n, D] bf16
    const uint16_t* vc;    // values, same layout
    const int32_t* idx;    // [rows, k]
    float* out;            // [rows, H, D]
    float* part;           // [rows, S, H, D + 2]: partial output, then m and l
    int64_t kvstride;
    int32_t rows, n, H, k, S;
    float scale;
};

template <int D, int HB>
__global__ void __launch_bounds__(kAttnBlock) topk_attn_partial_kernel(AttnParams P) {
    constexpr int KB = D / 32;     // 32-dim steps of a score
    constexpr int CPR = D / 8;     // 16-byte chunks per key / value row
    constexpr int NH = HB * 16;    // padded heads
    __shared__ u32x4_t qs[NH * CPR];          // queries, chunk c of head h in slot c ^ (h % CPR)
    __shared__ u32x4_t ks[kAttnSlots * CPR];  // gathered keys, same swizzle by slot
    __shared__ u32x4_t vt[D * 8];             // values transposed: dim row of 64 slots, chunk c in c ^ vsw(dim)
    __shared__ u32x4_t ps[NH * 8];            // P in bf16: head row of 64 slots, chunk c in c ^ (head % 8)
    __shared__ float red[2][kAttnBlock / 64][NH];
    const int row = blockIdx.x / P.S;
    const int sp = blockIdx.x - row * P.S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int n = P.n, H = P.H, k = P.k;
    const int s0 = sp * kAttnSlots;
    const int32_t* const irow = P.idx + (size_t)row * (size_t)k;
    const char* const K = reinterpret_cast<const char*>(P.kc + (size_t)row * (size_t)P.kvstride);
    const char* const V = reinterpret_cast<const char*>(P.vc + (size_t)row * (size_t)P.kvstride);
    // queries (contiguous loads)
    {
        const u32x4_t* const qrow = reinterpret_cast<const u32x4_t*>(P.q + (size_t)row * H * D);
        const u32x4_t zero4 = {0u, 0u, 0u, 0u};
        for (int i = tid; i < NH * CPR; i += kAttnBlock) {
            const int h = i / CPR, c = i % CPR;
            qs[h * CPR + (c ^ (h % CPR))] = h < H ? qrow[i] : zero4;
        }
    }
    // gathered keys and values: 16-byte pieces, a row of D bf16 per slot;
    // empty slots read row 0 (their scores are discarded).  All positions
    // are read first, then all rows, then the LDS writes, so that the
    // dependent loads overlap.  Transposed value chunks are swizzled by
    // (dim ^ dim/8) mod 8: the MFMA-layout reads (16 dims, one chunk) and
    // the writes (16 dims c*8+e of one slot) both spread over the banks.
    auto vsw = [](int dim) { return (dim ^ (dim >> 3)) & 7; };
    constexpr int PIECES = kAttnSlots * CPR / kAttnBlock;
    int toks[PIECES];
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
        const int sl = s0 + (tid + u * kAttnBlock) / CPR;
        const int t = sl < k ? irow[sl] : -1;
        toks[u] = (t >= 0 && t < n) ? t : 0;
    }
    u32x4_t kr[PIECES], vr[PIECES];
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
        const int c = (tid + u * kAttnBlock) % CPR;
        const size_t off = (size_t)toks[u] * D * 2 + (size_t)c * 16;
        kr[u] = *reinterpret_cast<const u32x4_t*>(K + off);
        vr[u] = *reinterpret_cast<const u32x4_t*>(V + off);
    }
    uint16_t* const vt16 = reinterpret_cast<uint16_t*>(vt);
#pragma unroll
    for (int u = 0; u < PIECES; ++u) {
        const int i = tid + u * kAttnBlock;
        const int j = i / CPR, c = i % CPR;
        ks[j * CPR + (c ^ (j % CPR))] = kr[u];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int dim = c * 8 + e;
            const uint32_t w = vr[u][e >> 1];
            vt16[(dim * 8 + ((j >> 3) ^ vsw(dim))) * 8 + (j & 7)] = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
        }
    }
    __syncthreads();
    // scores of this wave's 16 slots: lane holds heads 4g+i (+16 hb) of slot 16 wave + m
    const int j = wave * 16 + m;
    const int sl = s0 + j;
    const int tj = sl < k ? irow[sl] : -1;
    const bool valid = tj >= 0 && tj < n;
    float sc[HB][4];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
        floatx4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int c = kb * 4 + g;
            const int h = hb * 16 + m;
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, qs[h * CPR + (c ^ (h % CPR))]);
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, ks[j * CPR + (c ^ (j % CPR))]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[hb][i] = valid ? acc[i] * P.scale : -__builtin_huge_valf();
    }
    // softmax over the WG's 64 slots, per head: the maximum and the sum,
    // over the 16 lanes of a head group, then over the 4 waves
    float mx[HB][4];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x = sc[hb][i];
#pragma unroll
            for (int sft = 1; sft < 16; sft <<= 1) x = fmaxf(x, __shfl_xor(x, sft));
            mx[hb][i] = x;
            if (m == 0) red[0][wave][hb * 16 + 4 * g + i] = x;
        }
    __syncthreads();
    float sum[HB][4];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = hb * 16 + 4 * g + i;
            float M = red[0][0][h];
#pragma unroll
            for (int w = 1; w < kAttnBlock / 64; ++w) M = fmaxf(M, red[0][w][h]);
            mx[hb][i] = M;
            const float p = valid ? __expf(sc[hb][i] - M) : 0.0f;  // M is finite when a slot is valid
            sc[hb][i] = p;
            float x = p;
#pragma unroll
            for (int sft = 1; sft < 16; sft <<= 1) x += __shfl_xor(x, sft);
            sum[hb][i] = x;
            if (m == 0) red[1][wave][h] = x;
            // P in bf16 (round to nearest even), head row h, slot j
            const uint32_t u = __float_as_uint(p);
            const uint16_t pb = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
            reinterpret_cast<uint16_t*>(ps)[(h * 8 + ((j >> 3) ^ (h % 8))) * 8 + (j & 7)] = pb;
        }
    __syncthreads();
    float* const prow = P.part + ((size_t)row * P.S + sp) * (size_t)H * (D + 2);
    if (wave == 0) {
        // m and l of each head of this chunk
        for (int h = lane; h < H; h += 64) {
            float M = red[0][0][h], Lsum = red[1][0][h];
#pragma unroll
            for (int w = 1; w < kAttnBlock / 64; ++w) {
                M = fmaxf(M, red[0][w][h]);
                Lsum += red[1][w][h];
            }
            prow[(size_t)h * (D + 2) + D] = M;
            prow[(size_t)h * (D + 2) + D + 1] = Lsum;
        }
    }
    // P.V: output tiles of 16 heads x 16 dims, HB * D/16 of them over the
    // four waves; two 32-slot steps each
    for (int tile = wave; tile < HB * (D / 16); tile += kAttnBlock / 64) {
        const int hb = tile / (D / 16), db = tile % (D / 16);
        floatx4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ts = 0; ts < kAttnSlots / 32; ++ts) {
            const int c = ts * 4 + g;  // slots 8c .. 8c+7
            const int h = hb * 16 + m, dim = db * 16 + m;
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ps[h * 8 + (c ^ (h % 8))]);
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, vt[dim * 8 + (c ^ vsw(dim))]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
        }
        // lane holds heads 4g+i of dim db*16 + m
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = hb * 16 + 4 * g + i;
            if (h < H) prow[(size_t)h * (D + 2) + db * 16 + m] = acc[i];
        }
    }
}

// Combine a row's chunks: out = sum_s e^(m_s - M) O_s / sum_s e^(m_s - M) l_s
// with M the largest m_s over the chunks holding a position; zeros when no
// slot of the row holds one.  One WG of D threads per (row, head): the
// chunks' (m, l) are read in parallel and their factors kept in LDS, then
// each thread adds up its dim with eight loads in flight.
constexpr int kAttnCombineMax = 1024;  // chunks per pass of the factor table
template <int D>
__global__ void __launch_bounds__(D) topk_attn_combine_kernel(AttnParams P) {
    __shared__ float fac[kAttnCombineMax];
    __shared__ float red[D / 64 > 0 ? D / 64 : 1];
    __shared__ float bcast[2];
    const int rh = blockIdx.x;  // row * H + head
    const int row = rh / P.H, h = rh - row * P.H;
    const int c = threadIdx.x;
    const float* const base = P.part + (size_t)row * P.S * (size_t)P.H * (D + 2) + (size_t)h * (D + 2);
    const size_t stride = (size_t)P.H * (D + 2);
    const float ninf = -__builtin_huge_valf();
    // the largest m over chunks with l > 0
    float M = ninf;
    for (int s = c; s < P.S; s += D) {
        const float l = base[s * stride + D + 1];
        if (l > 0.0f) M = fmaxf(M, base[s * stride + D]);
    }
    constexpr int SFT0 = D >= 64 ? 32 : D / 2;  // lanes of the (partial) wave
    for (int sft = SFT0; sft >= 1; sft >>= 1) M = fmaxf(M, __shfl_xor(M, sft));
    if (D > 64) {
        if ((c & 63) == 0) red[c >> 6] = M;
        __syncthreads();
        if (c == 0) {
            float x = red[0];
            for (int w = 1; w < D / 64; ++w) x = fmaxf(x, red[w]);
            bcast[0] = x;
        }
        __syncthreads();
        M = bcast[0];
    }
    float num = 0.0f, den = 0.0f;
    for (int s0 = 0; s0 < P.S; s0 += kAttnCombineMax) {
        const int cnt = min(P.S - s0, kAttnCombineMax);
        __syncthreads();  // the previous pass's factors are used up
        float dpart = 0.0f;
        for (int s = c; s < cnt; s += D) {
            const float l = base[(s0 + s) * stride + D + 1];
            const float f = l > 0.0f ? __expf(base[(s0 + s) * stride + D] - M) : 0.0f;
            fac[s] = f;
            dpart += f * l;
        }
        den += dpart;
        __syncthreads();
        int s = 0;
        for (; s + 8 <= cnt; s += 8) {
            float o[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) o[u] = base[(s0 + s + u) * stride + c];
#pragma unroll
            for (int u = 0; u < 8; ++u) num += fac[s + u] * o[u];
        }
        for (; s < cnt; ++s) num += fac[s] * base[(s0 + s) * stride + c];
    }
    // the denominator: each thread added a share of the chunks
    for (int sft = SFT0; sft >= 1; sft >>= 1) den += __shfl_xor(den, sft);
    if (D > 64) {
        __syncthreads();
        if ((c & 63) == 0) red[c >> 6] = den;
        __syncthreads();
        if (c == 0) {
            float x = 0.0f;
            for (int w = 0; w < D / 64; ++w) x += red[w];
            bcast[1] = x;
        }
        __syncthreads();
        den = bcast[1];
    }
    P.out[(size_t)rh * D + c] = den > 0.0f ? num / den : 0.0f;
}

// ----------------------------------------------------------------- host side

using LaunchFn = void (*)(dim3, dim3, hipStream_t, const KParams&);
using OccFn = int (*)(int*, int);

// The window round's code is compiled only into the instances that can
// meet a row that long (measured: the unused code alone costs C2 0.45 µs).
template <int B, int I, bool R>
void launch_variant(dim3 grid, dim3 block, hipStream_t s, const KParams& p) {
    const bool win = p.n >= kWinLength;
    if (p.keys) {
        if (win) hipLaunchKernelGGL((topk_select_kernel<B, I, R, true, true>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((topk_select_kernel<B, I, R, true, false>), grid, block, 0, s, p);
    } else {
        if (win) hipLaunchKernelGGL((topk_select_kernel<B, I, R, false, true>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((topk_select_kernel<B, I, R, false, false>), grid, block, 0, s, p);
    }
}

// co-resident WGs per CU: the smallest figure of the instantiations
template <int B, int I, bool R>
int occupancy_variant(int* nb, int block) {
    int c[4] = {0, 0, 0, 0};
    int r[4];
    r[0] = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&c[0], topk_select_kernel<B, I, R, false, false>, block, 0);
    r[1] = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&c[1], topk_select_kernel<B, I, R, true, false>, block, 0);
    r[2] = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&c[2], topk_select_kernel<B, I, R, false, true>, block, 0);
    r[3] = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&c[3], topk_select_kernel<B, I, R, true, true>, block, 0);
    int m = c[0];
    for (int i = 1; i < 4; ++i) m = c[i] < m ? c[i] : m;
    *nb = m;
    for (int i = 0; i < 4; ++i)
        if (r[i] != 0) return r[i];
    return 0;
}

template <int B, int I, int D>
void launch_rows(dim3 grid, dim3 block, hipStream_t s, const KParams& p) {
    if (p.keys) hipLaunchKernelGGL((topk_rows_kernel<B, I, D, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((topk_rows_kernel<B, I, D, false>), grid, block, 0, s, p);
}

template <int B, int I, int D>
int occupancy_rows(int* nb, int block) {
    int a = 0, b = 0;
    const int r1 = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, topk_rows_kernel<B, I, D, false>, block, 0);
    const int r2 = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, topk_rows_kernel<B, I, D, true>, block, 0);
    *nb = a < b ? a : b;
    return r1 != 0 ? r1 : r2;
}

struct Variant {
    int block, items, resident;
    int rows_kernel;  // 1: one WG per row, 12-bit first digit (wgs_per_row must be 1)
    LaunchFn launch;
    OccFn occupancy;
};

#define TKS_VARIANT(B, I, R) {B, I, R ? 1 : 0, 0, &launch_variant<B, I, R>, &occupancy_variant<B, I, R>}
#define TKS_ROWS(B, I, D) {B, I, 0, 1, &launch_rows<B, I, D>, &occupancy_rows<B, I, D>}
const Variant kVariants[] = {
    TKS_VARIANT(512, 4, true),     // 0: 2048 logits per WG
    TKS_VARIANT(512, 8, true),     // 1: 4096
    TKS_VARIANT(1024, 4, true),    // 2: 4096
    TKS_VARIANT(1024, 8, true),    // 3: 8192
    TKS_VARIANT(512, 16, true),    // 4: 8192
    TKS_VARIANT(1024, 16, true),   // 5: 16384
    TKS_VARIANT(512, 32, true),    // 6: 16384
    TKS_VARIANT(1024, 32, true),   // 7: 32768
    TKS_VARIANT(1024, 16, false),  // 8: streaming, 16384 per tile
    TKS_VARIANT(256, 16, false),   // 9: streaming, 4096 per tile
    TKS_ROWS(512, 16, 1),          // 10: one WG per row, 8192 per tile
    TKS_ROWS(1024, 16, 1),         // 11: one WG per row, 16384 per tile
};
#undef TKS_VARIANT
#undef TKS_ROWS
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

struct DeviceInfo {
    int cus = 0;
    int capacity[kNumVariants] = {};  // co-resident WGs per variant on the whole device
};

// Scratch of one (device, stream): the status word, then one RowWorkspace
// per row (row r always at the same address, whatever the row count of a
// call).  Zeroed when allocated; kernels keep it consistent across calls.
struct Workspace {
    void* base = nullptr;
    size_t bytes = 0;
    void* aux = nullptr;  // ordered output: recorded keys, merge buffers (no clearing needed)
    size_t aux_bytes = 0;
    void* lg = nullptr;   // indexer selection without a logits output: the logits
    size_t lg_bytes = 0;
    void* at = nullptr;   // attention over the selected positions: per-chunk partials
    size_t at_bytes = 0;
};

std::recursive_mutex g_mu;  // recursive: the indexer entry point holds it across its launches
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
            // WGs that are certainly co-resident: what the occupancy query
            // allows, but at most two per CU, and one for 1024-thread WGs
            // (measured with a bounded-wait probe on MI355X)
            const int cap = kVariants[v].block >= 1024 ? 1 : 2;
            d.capacity[v] = (nb < cap ? nb : cap) * d.cus;
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
    bits = (bits + 7) / 8 * 8;
    return bits < 8 ? 8 : bits;
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
    if (var.resident && cpw > tile_chunks) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (var.rows_kernel && G != 1) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (cpw < 1) cpw = 1;
    if (G > 1 && rows * (int64_t)G > (int64_t)d.capacity[v]) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (rows * (int64_t)G > 0x7FFFFFFFll) return TOPK_SELECT_ERROR_INVALID_VALUE;
    L->variant = v;
    L->G = G;
    L->chunks_per_wg = (int)cpw;
    return TOPK_SELECT_SUCCESS;
}

// Default shape (measured on MI355X).  A cross-workgroup merge round costs
// about the same for any split, while the per-pass time falls with the
// slice, so few rows are spread over many WGs of about 2K-8K logits each
// (1024 threads once a row uses more than 16 WGs).  Many rows: the fewest
// resident WGs per row that can all be co-resident, else streaming WGs.
int choose_shape(const DeviceInfo& d, int64_t rows, int64_t maxc, Launch* L) {
    auto tile_chunks = [](int v) { return (int64_t)kVariants[v].block * (kVariants[v].items / 4); };
    if (rows * 8 <= d.cus) {
        int64_t G = (maxc + 511) / 512;  // about 2K logits per WG
        if (G > 128) G = 128;
        if (G > d.cus / rows) G = d.cus / rows;
        if (G < 1) G = 1;
        const int64_t per = (maxc + G - 1) / G;
        const int v512[] = {0, 1, 4, 6, 7}, v1024[] = {2, 3, 5, 7};
        if (G <= 16) {
            for (int v : v512)
                if (per <= tile_chunks(v)) return check_shape(d, rows, maxc, v, (int)G, L);
        } else {
            for (int v : v1024)
                if (per <= tile_chunks(v)) return check_shape(d, rows, maxc, v, (int)G, L);
        }
    }
    const int order_many[] = {7, 5, 3, 1, 0};
    for (int v : order_many) {
        const int64_t G = (maxc + tile_chunks(v) - 1) / tile_chunks(v);
        if (G == 1 || rows * G <= (int64_t)d.capacity[v]) return check_shape(d, rows, maxc, v, (int)G, L);
    }
    // many rows: one streaming WG per row
    if (rows >= d.cus) return check_shape(d, rows, maxc, 10, 1, L);
    // few long rows: as many streaming WGs per row as can be co-resident
    const int v = (maxc >= 16384) ? 8 : 9;
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

int get_workspace(int dev, hipStream_t stream, size_t need, Workspace** out) {
    Workspace& w = g_ws[{dev, (uintptr_t)stream}];
    if (w.bytes < need) {
        if (w.base) {
            // the old workspace may still be in use by enqueued work
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

// Grow-only scratch that needs no clearing (the old one is freed once the
// stream has finished with it).
int grow_scratch(hipStream_t stream, void** ptr, size_t* bytes, size_t need) {
    if (*bytes < need) {
        if (*ptr) {
            if (hipStreamSynchronize(stream) != hipSuccess) return TOPK_SELECT_ERROR_LAUNCH;
            (void)hipFree(*ptr);
            *ptr = nullptr;
            *bytes = 0;
        }
        void* p = nullptr;
        if (hipMalloc(&p, need) != hipSuccess) {
            (void)hipGetLastError();
            return TOPK_SELECT_ERROR_OUT_OF_MEMORY;
        }
        *ptr = p;
        *bytes = need;
    }
    return TOPK_SELECT_SUCCESS;
}

int get_aux(hipStream_t stream, Workspace* w, size_t need) { return grow_scratch(stream, &w->aux, &w->aux_bytes, need); }

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a && b && a0 < b0 + bbytes && b0 < a0 + abytes;
}

// Launches of the ordered output: for a few rows with k <= kRankMax the
// rank kernel (up to 128 WGs per row); else one sorting WG per row when k
// fits one on-chip sort, or runs of kSortRun and merge passes.
struct SortShape {
    bool rank;
    int rank_wgs;      // rank kernel: WGs per row
    int block, items;  // sort kernel variant
    int nruns;
    int64_t kp;        // padded row length of the runs
};

SortShape sort_shape(int32_t rows, int32_t k) {
    SortShape s;
    s.rank = k <= kRankMax && (int64_t)rows * (int64_t)k * (int64_t)k <= (int64_t)1 << 25;
    s.rank_wgs = k / 16 < 1 ? 1 : (k / 16 > 128 ? 128 : k / 16);
    if (rows <= 128) {
        // few rows (fewer WGs than CUs): the most threads per row
        s.block = 1024;
        s.items = k <= 1024 ? 1 : (k <= 2048 ? 2 : (k <= 4096 ? 4 : 8));
    } else if (k <= 1024) { s.block = 256; s.items = 4; }
    else if (k <= 2048) { s.block = 512; s.items = 4; }
    else if (k <= 4096) { s.block = 1024; s.items = 4; }
    else { s.block = 1024; s.items = 8; }
    s.nruns = (int)((k + kSortRun - 1) / kSortRun);
    s.kp = (int64_t)s.nruns * kSortRun;
    return s;
}

void launch_sort(const SortShape& sh, int32_t rows, hipStream_t stream, const SortParams& p) {
    const dim3 grid((unsigned)((int64_t)rows * sh.nruns));
    if (sh.block == 256) topk_sort_kernel<256, 4><<<grid, 256, 0, stream>>>(p);
    else if (sh.block == 512) topk_sort_kernel<512, 4><<<grid, 512, 0, stream>>>(p);
    else if (sh.items == 1) topk_sort_kernel<1024, 1><<<grid, 1024, 0, stream>>>(p);
    else if (sh.items == 2) topk_sort_kernel<1024, 2><<<grid, 1024, 0, stream>>>(p);
    else if (sh.items == 4) topk_sort_kernel<1024, 4><<<grid, 1024, 0, stream>>>(p);
    else topk_sort_kernel<1024, 8><<<grid, 1024, 0, stream>>>(p);
}

int run(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k, int32_t* out,
        bool ordered, float* vals, hipStream_t stream, const topk_select_plan_t* forced) {
    int rc = validate(logits, rows, n, lengths, k, out);
    if (rc != TOPK_SELECT_SUCCESS || rows == 0) return rc;
    if (ordered && vals) {
        const size_t vb = (size_t)rows * (size_t)k * 4u;
        if (((uintptr_t)vals & 3) || overlaps(vals, vb, logits, (size_t)rows * (size_t)n * 4u) ||
            overlaps(vals, vb, out, vb) || overlaps(vals, vb, lengths, (size_t)rows * 4u))
            return TOPK_SELECT_ERROR_INVALID_VALUE;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TOPK_SELECT_ERROR_NO_DEVICE;
    std::lock_guard<std::recursive_mutex> lock(g_mu);
    DeviceInfo* d = nullptr;
    rc = device_info(dev, &d);
    if (rc != TOPK_SELECT_SUCCESS) return rc;
    const int64_t maxc = max_row_chunks(logits, n);
    Launch L;
    rc = forced ? check_shape(*d, rows, maxc, forced->variant, forced->wgs_per_row, &L)
                : choose_shape(*d, rows, maxc, &L);
    if (rc != TOPK_SELECT_SUCCESS) return rc;
    const Variant& var = kVariants[L.variant];
    const size_t rows_bytes = L.G > 1 ? (size_t)rows * sizeof(RowWorkspace) : 0;
    Workspace* w = nullptr;
    rc = get_workspace(dev, stream, kStatusBytes + rows_bytes, &w);
    if (rc != TOPK_SELECT_SUCCESS) return rc;
    SortShape sh{};
    size_t keys_bytes = 0;
    if (ordered) {
        sh = sort_shape(rows, k);
        keys_bytes = ((size_t)rows * (size_t)k * 4u + 255u) / 256u * 256u;
        const size_t run_bytes = (!sh.rank && sh.nruns > 1) ? 2u * (size_t)rows * (size_t)sh.kp * 8u : 0u;
        if ((int64_t)rows * sh.nruns > 0x7FFFFFFFll || (int64_t)rows * sh.rank_wgs > 0x7FFFFFFFll ||
            (int64_t)rows * (sh.kp / (kMergeBlock * kMergeItems)) > 0x7FFFFFFFll)
            return TOPK_SELECT_ERROR_INVALID_VALUE;
        rc = get_aux(stream, w, 2u * keys_bytes + run_bytes);
        if (rc != TOPK_SELECT_SUCCESS) return rc;
    }
    char* base = reinterpret_cast<char*>(w->base);
    KParams P;
    P.logits = logits;
    P.lengths = lengths;
    // ordered output: the selection writes its indices and their keys to
    // scratch, the sort writes out_idx
    char* const aux = reinterpret_cast<char*>(w->aux);
    P.out = ordered ? reinterpret_cast<int32_t*>(aux + keys_bytes) : out;
    P.keys = ordered ? reinterpret_cast<uint32_t*>(aux) : nullptr;
    P.status = reinterpret_cast<uint32_t*>(base);
    P.ws = L.G > 1 ? reinterpret_cast<RowWorkspace*>(base + kStatusBytes) : nullptr;
    P.rows = rows;
    P.n = n;
    P.k = k;
    P.G = L.G;
    P.chunks_per_wg = L.chunks_per_wg;
    P.idx_bits = idx_bits_for(n);
    P.mcopies = L.G <= 16 ? 1 : (L.G <= 32 ? 2 : kMergeCopies);
    P.ahead = var.rows_kernel ? d->capacity[L.variant] : 0;
    (void)hipGetLastError();
    var.launch(dim3((unsigned)(rows * L.G)), dim3((unsigned)var.block), stream, P);
    if (hipGetLastError() != hipSuccess) return TOPK_SELECT_ERROR_LAUNCH;
    if (!ordered) return TOPK_SELECT_SUCCESS;

    SortParams S;
    S.logits = logits;
    S.lengths = lengths;
    S.out = out;
    S.vals = vals;
    S.idx = P.out;
    S.keys = P.keys;
    S.rows = rows;
    S.n = n;
    S.k = k;
    S.kp = (int32_t)sh.kp;
    S.nruns = sh.nruns;
    S.width = 0;
    if (sh.rank) {
        S.nruns = sh.rank_wgs;
        topk_rank_kernel<<<dim3((unsigned)((int64_t)rows * sh.rank_wgs)), kRankBlock, 0, stream>>>(S);
        return hipGetLastError() == hipSuccess ? TOPK_SELECT_SUCCESS : TOPK_SELECT_ERROR_LAUNCH;
    }
    uint64_t* const run0 = reinterpret_cast<uint64_t*>(aux + 2u * keys_bytes);
    uint64_t* const run1 = run0 + (size_t)rows * (size_t)sh.kp;
    S.src = nullptr;
    S.dst = sh.nruns > 1 ? run0 : nullptr;
    launch_sort(sh, rows, stream, S);
    if (hipGetLastError() != hipSuccess) return TOPK_SELECT_ERROR_LAUNCH;
    uint64_t* bufs[2] = {run0, run1};
    int cur = 0;
    for (int64_t width = kSortRun; width < sh.kp; width *= 2) {
        S.width = (int32_t)width;
        S.src = bufs[cur];
        S.dst = 2 * width >= sh.kp ? nullptr : bufs[cur ^ 1];
        const int64_t wgs = (int64_t)rows * (sh.kp / (kMergeBlock * kMergeItems));
        topk_merge_kernel<<<dim3((unsigned)wgs), kMergeBlock, 0, stream>>>(S);
        if (hipGetLastError() != hipSuccess) return TOPK_SELECT_ERROR_LAUNCH;
        cur ^= 1;
    }
    return TOPK_SELECT_SUCCESS;
}

// ---- indexer logits and the selection on them

int validate_indexer(const uint16_t* q, const uint16_t* kc, const float* w, int32_t rows, int32_t n, int32_t heads,
                     int32_t dim, int64_t kstride, const int32_t* lengths, const float* logits) {
    if (rows < 0 || n < 1 || heads < 1 || heads > 64 || kstride < 0) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (dim != 32 && dim != 64 && dim != 128) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (rows == 0) return TOPK_SELECT_SUCCESS;
    if (!q || !kc || !w) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (((uintptr_t)q & 15) || ((uintptr_t)kc & 15) || ((uintptr_t)w & 3) || ((uintptr_t)lengths & 3) ||
        (kstride % 8) != 0)
        return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (kstride != 0 && kstride < (int64_t)n * dim) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (logits) {
        if ((uintptr_t)logits & 3) return TOPK_SELECT_ERROR_INVALID_VALUE;
        const size_t lb = (size_t)rows * (size_t)n * 4u;
        const size_t kb = ((kstride ? (size_t)(rows - 1) * (size_t)kstride : 0u) + (size_t)n * dim) * 2u;
        if (overlaps(logits, lb, q, (size_t)rows * heads * dim * 2u) || overlaps(logits, lb, kc, kb) ||
            overlaps(logits, lb, w, (size_t)rows * heads * 4u) || overlaps(logits, lb, lengths, (size_t)rows * 4u))
            return TOPK_SELECT_ERROR_INVALID_VALUE;
    }
    return TOPK_SELECT_SUCCESS;
}

template <int D, int HB>
void launch_logits_t(unsigned grid, hipStream_t stream, const LogitParams& p) {
    topk_logits_kernel<D, HB><<<grid, kLogitBlock, 0, stream>>>(p);
}

int launch_logits(const uint16_t* q, const uint16_t* kc, const float* w, int32_t rows, int32_t n, int32_t heads,
                  int32_t dim, int64_t kstride, const int32_t* lengths, float* logits, hipStream_t stream) {
    LogitParams p;
    p.q = q;
    p.kc = kc;
    p.w = w;
    p.lengths = lengths;
    p.logits = logits;
    p.kstride = kstride;
    p.rows = rows;
    p.n = n;
    p.H = heads;
    // groups of 64 tokens per wave: one when the grid is small (every
    // group its own wave), more for long or many rows, so that each wave
    // streams several groups with the next one's keys in flight (about two
    // WGs per CU resident, the grid about that many: fewer WG starts)
    int cus = 256;
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t groups = (int64_t)rows * ((n + 63) / 64);
    const int64_t resident_waves = (int64_t)cus * 2 * (kLogitBlock / 64);
    int64_t gpw = (groups + resident_waves - 1) / resident_waves;
    p.gpw = (int32_t)(gpw < 1 ? 1 : (gpw > 8 ? 8 : gpw));
    const int64_t tok_wg = (int64_t)p.gpw * kLogitBlock;
    p.tiles = (int32_t)((n + tok_wg - 1) / tok_wg);
    const int64_t grid = (int64_t)rows * p.tiles;
    if (grid > 0x7FFFFFFFll) return TOPK_SELECT_ERROR_INVALID_VALUE;
    const int hb = heads <= 16 ? 1 : (heads <= 32 ? 2 : 4);
    (void)hipGetLastError();
    const unsigned g = (unsigned)grid;
    if (dim == 32) {
        if (hb == 1) launch_logits_t<32, 1>(g, stream, p);
        else if (hb == 2) launch_logits_t<32, 2>(g, stream, p);
        else launch_logits_t<32, 4>(g, stream, p);
    } else if (dim == 64) {
        if (hb == 1) launch_logits_t<64, 1>(g, stream, p);
        else if (hb == 2) launch_logits_t<64, 2>(g, stream, p);
        else launch_logits_t<64, 4>(g, stream, p);
    } else {
        if (hb == 1) launch_logits_t<128, 1>(g, stream, p);
        else if (hb == 2) launch_logits_t<128, 2>(g, stream, p);
        else launch_logits_t<128, 4>(g, stream, p);
    }
    return hipGetLastError() == hipSuccess ? TOPK_SELECT_SUCCESS : TOPK_SELECT_ERROR_LAUNCH;
}

int run_indexer(const uint16_t* q, const uint16_t* kc, const float* w, int32_t rows, int32_t n, int32_t heads,
                int32_t dim, int64_t kstride, const int32_t* lengths, int32_t k, int32_t* out_idx, float* logits,
                hipStream_t stream) {
    int rc = validate_indexer(q, kc, w, rows, n, heads, dim, kstride, lengths, logits);
    if (rc != TOPK_SELECT_SUCCESS) return rc;
    if (k < 1 || k > n) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (rows == 0) return TOPK_SELECT_SUCCESS;
    if (!out_idx || ((uintptr_t)out_idx & 3)) return TOPK_SELECT_ERROR_INVALID_VALUE;
    const size_t ob = (size_t)rows * (size_t)k * 4u;
    if (overlaps(out_idx, ob, q, (size_t)rows * heads * dim * 2u) || overlaps(out_idx, ob, w, (size_t)rows * heads * 4u) ||
        overlaps(out_idx, ob, kc, ((kstride ? (size_t)(rows - 1) * (size_t)kstride : 0u) + (size_t)n * dim) * 2u))
        return TOPK_SELECT_ERROR_INVALID_VALUE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TOPK_SELECT_ERROR_NO_DEVICE;
    std::lock_guard<std::recursive_mutex> lock(g_mu);  // held across both launches (scratch stays put)
    float* lg = logits;
    if (!lg) {
        Workspace& ws = g_ws[{dev, (uintptr_t)stream}];
        rc = grow_scratch(stream, &ws.lg, &ws.lg_bytes, (size_t)rows * (size_t)n * 4u);
        if (rc != TOPK_SELECT_SUCCESS) return rc;
        lg = reinterpret_cast<float*>(ws.lg);
    }
    rc = launch_logits(q, kc, w, rows, n, heads, dim, kstride, lengths, lg, stream);
    if (rc != TOPK_SELECT_SUCCESS) return rc;
    return run(lg, rows, n, lengths, k, out_idx, false, nullptr, stream, nullptr);
}

// ---- attention over the selected positions

int run_attention(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const int32_t* idx, int32_t rows,
                  int32_t n, int32_t heads, int32_t dim, int64_t kvstride, int32_t k, float scale, float* out,
                  hipStream_t stream) {
    if (rows < 0 || n < 1 || heads < 1 || heads > 64 || k < 1 || kvstride < 0 || (kvstride % 8) != 0)
        return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (dim != 32 && dim != 64 && dim != 128) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (kvstride != 0 && kvstride < (int64_t)n * dim) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (!(scale == scale) || scale == __builtin_huge_valf() || scale == -__builtin_huge_valf())
        return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (rows == 0) return TOPK_SELECT_SUCCESS;
    if (!q || !kc || !vc || !idx || !out) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (((uintptr_t)q & 15) || ((uintptr_t)kc & 15) || ((uintptr_t)vc & 15) || ((uintptr_t)idx & 3) ||
        ((uintptr_t)out & 3))
        return TOPK_SELECT_ERROR_INVALID_VALUE;
    const size_t ob = (size_t)rows * heads * dim * 4u;
    const size_t kvb = ((kvstride ? (size_t)(rows - 1) * (size_t)kvstride : 0u) + (size_t)n * dim) * 2u;
    if (overlaps(out, ob, q, (size_t)rows * heads * dim * 2u) || overlaps(out, ob, kc, kvb) ||
        overlaps(out, ob, vc, kvb) || overlaps(out, ob, idx, (size_t)rows * k * 4u))
        return TOPK_SELECT_ERROR_INVALID_VALUE;
    const int64_t S = (k + kAttnSlots - 1) / kAttnSlots;
    if ((int64_t)rows * S > 0x7FFFFFFFll || (int64_t)rows * heads > 0x7FFFFFFFll) return TOPK_SELECT_ERROR_INVALID_VALUE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TOPK_SELECT_ERROR_NO_DEVICE;
    std::lock_guard<std::recursive_mutex> lock(g_mu);
    Workspace& ws = g_ws[{dev, (uintptr_t)stream}];
    int rc = grow_scratch(stream, &ws.at, &ws.at_bytes, (size_t)rows * (size_t)S * heads * (dim + 2) * 4u);
    if (rc != TOPK_SELECT_SUCCESS) return rc;
    AttnParams p;
    p.q = q;
    p.kc = kc;
    p.vc = vc;
    p.idx = idx;
    p.out = out;
    p.part = reinterpret_cast<float*>(ws.at);
    p.kvstride = kvstride;
    p.rows = rows;
    p.n = n;
    p.H = heads;
    p.k = k;
    p.S = (int32_t)S;
    p.scale = scale;
    const int hb = heads <= 16 ? 1 : (heads <= 32 ? 2 : 4);
    const dim3 g1((unsigned)((int64_t)rows * S)), g2((unsigned)((int64_t)rows * heads));
    (void)hipGetLastError();
#define TKS_ATTN(D_, HB_) topk_attn_partial_kernel<D_, HB_><<<g1, kAttnBlock, 0, stream>>>(p)
    if (dim == 32) {
        if (hb == 1) TKS_ATTN(32, 1); else if (hb == 2) TKS_ATTN(32, 2); else TKS_ATTN(32, 4);
        topk_attn_combine_kernel<32><<<g2, 32, 0, stream>>>(p);
    } else if (dim == 64) {
        if (hb == 1) TKS_ATTN(64, 1); else if (hb == 2) TKS_ATTN(64, 2); else TKS_ATTN(64, 4);
        topk_attn_combine_kernel<64><<<g2, 64, 0, stream>>>(p);
    } else {
        if (hb == 1) TKS_ATTN(128, 1); else if (hb == 2) TKS_ATTN(128, 2); else TKS_ATTN(128, 4);
        topk_attn_combine_kernel<128><<<g2, 128, 0, stream>>>(p);
    }
#undef TKS_ATTN
    return hipGetLastError() == hipSuccess ? TOPK_SELECT_SUCCESS : TOPK_SELECT_ERROR_LAUNCH;
}

}  // namespace tks

extern "C" {

int topk_sparse_attention(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const int32_t* idx,
                          int32_t rows, int32_t n, int32_t heads, int32_t dim, int64_t kvstride, int32_t k,
                          float scale, float* out, topk_select_stream_t stream) {
    try {
        return tks::run_attention(q, kc, vc, idx, rows, n, heads, dim, kvstride, k, scale, out, (hipStream_t)stream);
    } catch (...) {
        return TOPK_SELECT_ERROR_LAUNCH;
    }
}


int topk_indexer_logits(const uint16_t* q, const uint16_t* kc, const float* w, int32_t rows, int32_t n,
                        int32_t heads, int32_t dim, int64_t kstride, const int32_t* lengths, float* logits,
                        topk_select_stream_t stream) {
    try {
        int rc = tks::validate_indexer(q, kc, w, rows, n, heads, dim, kstride, lengths, logits);
        if (rc != TOPK_SELECT_SUCCESS || rows == 0) return rc;
        if (!logits) return TOPK_SELECT_ERROR_INVALID_VALUE;
        return tks::launch_logits(q, kc, w, rows, n, heads, dim, kstride, lengths, logits, (hipStream_t)stream);
    } catch (...) {
        return TOPK_SELECT_ERROR_LAUNCH;
    }
}

int topk_indexer_select(const uint16_t* q, const uint16_t* kc, const float* w, int32_t rows, int32_t n,
                        int32_t heads, int32_t dim, int64_t kstride, const int32_t* lengths, int32_t k,
                        int32_t* out_idx, float* out_logits, topk_select_stream_t stream) {
    try {
        return tks::run_indexer(q, kc, w, rows, n, heads, dim, kstride, lengths, k, out_idx, out_logits,
                                (hipStream_t)stream);
    } catch (...) {
        return TOPK_SELECT_ERROR_LAUNCH;
    }
}


int topk_select(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k,
                int32_t* out_idx, topk_select_stream_t stream) {
    try {
        return tks::run(logits, rows, n, lengths, k, out_idx, false, nullptr, (hipStream_t)stream, nullptr);
    } catch (...) {
        return TOPK_SELECT_ERROR_LAUNCH;
    }
}

int topk_select_ex(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k,
                   int32_t* out_idx, topk_select_stream_t stream, const topk_select_plan_t* plan) {
    if (!plan) return TOPK_SELECT_ERROR_INVALID_VALUE;
    try {
        return tks::run(logits, rows, n, lengths, k, out_idx, false, nullptr, (hipStream_t)stream, plan);
    } catch (...) {
        return TOPK_SELECT_ERROR_LAUNCH;
    }
}

int topk_select_sorted(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k,
                       int32_t* out_idx, float* out_val, topk_select_stream_t stream) {
    try {
        return tks::run(logits, rows, n, lengths, k, out_idx, true, out_val, (hipStream_t)stream, nullptr);
    } catch (...) {
        return TOPK_SELECT_ERROR_LAUNCH;
    }
}

int topk_select_sorted_ex(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k,
                          int32_t* out_idx, float* out_val, topk_select_stream_t stream,
                          const topk_select_plan_t* plan) {
    if (!plan) return TOPK_SELECT_ERROR_INVALID_VALUE;
    try {
        return tks::run(logits, rows, n, lengths, k, out_idx, true, out_val, (hipStream_t)stream, plan);
    } catch (...) {
        return TOPK_SELECT_ERROR_LAUNCH;
    }
}

int topk_select_plan(int32_t rows, int32_t n, int32_t k, topk_select_plan_t* plan) {
    if (!plan || rows < 0 || n < 1 || k < 1 || k > n) return TOPK_SELECT_ERROR_INVALID_VALUE;
    try {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return TOPK_SELECT_ERROR_NO_DEVICE;
        std::lock_guard<std::recursive_mutex> lock(tks::g_mu);
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
        plan->first_bits = tks::kVariants[L.variant].rows_kernel ? 12 : 8;
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
    plan->first_bits = tks::kVariants[v].rows_kernel ? 12 : 8;
    return TOPK_SELECT_SUCCESS;
}

int topk_select_device_status(topk_select_stream_t stream, int32_t* flags) {
    if (!flags) return TOPK_SELECT_ERROR_INVALID_VALUE;
    *flags = 0;
    try {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return TOPK_SELECT_ERROR_NO_DEVICE;
        if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return TOPK_SELECT_ERROR_LAUNCH;
        std::lock_guard<std::recursive_mutex> lock(tks::g_mu);
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
        std::lock_guard<std::recursive_mutex> lock(tks::g_mu);
        int rc = TOPK_SELECT_SUCCESS;
        for (auto& kv : tks::g_ws) {
            if (kv.second.base || kv.second.aux || kv.second.lg || kv.second.at) {
                int cur = 0;
                (void)hipGetDevice(&cur);
                (void)hipSetDevice(kv.first.first);
                if (hipDeviceSynchronize() != hipSuccess) rc = TOPK_SELECT_ERROR_LAUNCH;
                for (void* p : {kv.second.base, kv.second.aux, kv.second.lg, kv.second.at})
                    if (p && hipFree(p) != hipSuccess) rc = TOPK_SELECT_ERROR_LAUNCH;
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
