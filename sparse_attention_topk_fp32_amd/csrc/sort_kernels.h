// sort_kernels.h - ordered output in a second launch: the rank, sort and merge kernels.
// Part of the topk_select library: included once, in order, by topk_select.hip.

#pragma once

#include "common.h"

namespace tks {

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


// Write output slot j of a row from a composite (0 = no element: -1, -inf).
__device__ __forceinline__ void put_sorted(uint64_t c, int32_t* orow, float* vrow, const float* prow, uint32_t L,
                                           uint32_t j) {
    const uint32_t idx = ~(uint32_t)c;
    const bool has = c != 0ull;
    orow[j] = has ? (int32_t)idx : -1;
    if (vrow) vrow[j] = has ? value_of((uint32_t)(c >> 32), prow, L, idx) : -__builtin_huge_valf();
}

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
// The arguments that the first loads depend on come first, one by one (the
// dispatcher places them in scalar registers as the waves start: kernel-
// argument preloading); they stand in for the parameter block's copies.
__global__ void __launch_bounds__(BLOCK) topk_sort_kernel(const int32_t* idx_, const uint32_t* keys_, const int32_t* lengths_,
                                                           const float* logits_, int32_t n_, int32_t k_, int32_t nruns_,
                                                           const SortParams P0) {
    SortParams P = P0;
    P.idx = idx_, P.keys = keys_, P.lengths = lengths_, P.logits = logits_, P.n = n_, P.k = k_, P.nruns = nruns_;
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

// The arguments that the first loads depend on come first, one by one (the
// dispatcher places them in scalar registers as the waves start: kernel-
// argument preloading); they stand in for the parameter block's copies.
__global__ void __launch_bounds__(kRankBlock) topk_rank_kernel(const int32_t* idx_, const uint32_t* keys_,
                                                              const int32_t* lengths_, const float* logits_, int32_t n_,
                                                              int32_t k_, int32_t nruns_, const SortParams P0) {
    SortParams P = P0;
    P.idx = idx_, P.keys = keys_, P.lengths = lengths_, P.logits = logits_, P.n = n_, P.k = k_, P.nruns = nruns_;
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

}  // namespace tks
