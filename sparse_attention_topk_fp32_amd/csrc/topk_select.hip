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
//  * Section 5: one row split over several blocks that cooperate; -1 for
//    empty output slots.
//
// MI355X design (not a translation of the article's Triton/CUDA kernels):
//  * Ties are made unique by ranking the 64-bit composite
//    (key << 32 | ~index): larger composite = larger value, or equal value and
//    smaller index.  Every selection below is an exact selection of the k
//    largest composites, so the result is the article's (ties at the
//    threshold to the lowest index).
//  * Few rows (batch-1 decode): a row is cut into slices of 16-byte chunks,
//    one workgroup (WG) per slice.  Every WG of the row reads the same
//    sample of the row (blocks of chunks spread along it) and takes from it a
//    lower bound on the row's k-th largest key; it then writes the
//    composites of its slice at or above the bound to a region of its own
//    and publishes how many it wrote.  Only the row's last WG waits: it
//    gathers the regions in WG order into LDS and selects exactly on chip
//    (range-adaptive 256-bin rounds, then an exact rank).  No WG waits for a
//    later one, so no co-residency is required, and every position comes
//    from a block scan, so the output order is the same on every call.
//  * Many rows: one WG per row streams the row once, keeping the elements at
//    or above a running bound in LDS, then the same on-chip selection.
//  * When a bound overshoots or the candidates do not fit on chip, one WG
//    finishes the row exactly by passes over it in global memory.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "topk_select.h"
#include "key_map.h"

namespace tks {

constexpr int kSmall = 256;       // bucket ranked exactly by comparisons
constexpr int kCopies = 8;        // LDS copies of a 256-bin histogram (against atomic conflicts)
constexpr int kStride = 260;      // words per copy: 256 bins, a spare slot, 16-byte aligned
// a histogram area: kCopies 256-bin copies, or one 4096-bin copy (the first
// pass over a row in global memory)
constexpr int kHistWords = kCopies * kStride > 4096 ? kCopies * kStride : 4096;
constexpr int kBufCap = 7168;     // candidate buffer of the split kernel's finishing WG (entries)
constexpr int kMaxSplit = 256;    // WGs per row of the split kernel
constexpr int kSampleMax = 4096;  // chunks in a row's sample (split kernel)
constexpr uint32_t kFlagTimeout = 1u;
constexpr uint32_t kFlagCapacity = 2u;
// Bound on a wait for another workgroup, in ticks of the 100 MHz constant
// clock (s_memrealtime): 2 s, far beyond any legitimate wait.
constexpr uint64_t kSpinLimitTicks = 200000000ull;

#ifdef TKS_TEST_HOOKS
// Test builds only: the wait bound can be set from the host (0: give up
// before the first poll), so that the give-up path can be exercised with
// every kernel still ending normally.
__device__ uint64_t g_spin_limit = kSpinLimitTicks;
__device__ __forceinline__ uint64_t spin_limit() { return g_spin_limit; }
#else
__device__ __forceinline__ constexpr uint64_t spin_limit() { return kSpinLimitTicks; }
#endif

// Per-row coordination of the split kernel: the candidate count of each WG,
// tagged with the launch's epoch, and the epoch itself (advanced by the
// row's last WG at the end of every launch).
struct alignas(64) SplitRow {
    uint64_t cnt[kMaxSplit];  // (tag << 32) | candidates written by WG w; 0 = not published
    uint32_t epoch;
    uint32_t pad[15];
};

struct KParams {
    const float* logits;
    const int32_t* lengths;
    int32_t* out;
    uint32_t* keys;         // [rows, k]: key of the element at each output slot (ordered output), or null
    uint32_t* status;
    SplitRow* rws;          // split kernel, several WGs per row: per-row counts and epoch
    uint64_t* stage;        // split kernel: [rows][G][region] candidate composites, 0 where unused
    int32_t rows, n, k;
    int32_t G;              // workgroups per row
    int32_t chunks_per_wg;  // 16-byte chunks in one WG's slice
    int32_t region;         // entries of one WG's region in the stage
    int32_t sample_chunks;  // split kernel: chunks in a row's sample (a multiple of 16)
    int32_t ahead;          // one WG per row: rows from a row to the one whose first tile it touches (0: none)
    int32_t* oout;          // one WG per row, keys recorded: the ordered output's indices [rows, k] (null: none)
    float* ovals;           // and its values (null: none)
};

__device__ __forceinline__ uint32_t make_tag(uint32_t epoch) { return 0x80000000u | (epoch & 0x7FFFFFFFu); }

// ----------------------------------------------------------------- device helpers

// 16 bytes as a native vector (register arrays of the uint4 struct can be
// placed in scratch memory when they are passed around)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Mapping step (key_map.h, checked on the host over every bit pattern).
__device__ __forceinline__ uint32_t key_of(float x) { return tks_key_of(x); }

// The logit a key came from; -0.0 and +0.0 share a key, so a zero key reads
// the logit itself to return its sign.
__device__ __forceinline__ float value_of(uint32_t key, const float* prow, uint32_t L, uint32_t idx) {
    if (key == 0x80000000u) return idx < L ? prow[idx] : 0.0f;
    return __uint_as_float(key & 0x80000000u ? key ^ 0x80000000u : ~key);
}

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t idx) {
    return ((uint64_t)key << 32) | (uint64_t)~idx;
}

__device__ __forceinline__ uint32_t lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// A value every lane holds identically: make it scalar.
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
    return ((uint64_t)uniform((uint32_t)(v >> 32)) << 32) | (uint64_t)uniform((uint32_t)v);
}

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

// Workgroup barrier that orders LDS only (global data crossing WGs goes
// through device-scope atomics, global data inside a WG is never re-read).
__device__ __forceinline__ void lds_sync() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ int valid_length(const int32_t* lengths, int row, int n) {
    if (!lengths) return n;
    const int L = lengths[row];
    return L < 0 ? 0 : (L > n ? n : L);
}

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

// Block-wide exclusive scan over all BLOCK threads that also returns the
// total (uniform).  Two barriers; s_w may be reused right after.
template <int BLOCK>
__device__ __forceinline__ uint32_t block_scan_total(uint32_t a, uint32_t* s_w /* [BLOCK / 64] */, uint32_t& total) {
    constexpr int NW = BLOCK / 64;
    const uint32_t wid = threadIdx.x / 64;
    const uint32_t ia = wave_inclusive_scan(a);
    if (lane_id() == 63) s_w[wid] = ia;
    lds_sync();
    uint32_t pa = 0, tot = 0;
#pragma unroll 4
    for (int i = 0; i < NW; ++i) {
        const uint32_t v = s_w[i];
        if ((uint32_t)i < wid) pa += v;
        tot += v;
    }
    lds_sync();
    total = uniform(tot);
    return pa + ia - a;
}

// Positions in thread order for a running list: each thread appends `cnt`
// entries; returns the thread's first position and advances `total` by the
// block's sum (uniform).  One barrier: the two halves of s2 are used in turn
// (`par` flips), so a half is written again only after every wave has passed
// the next call's barrier, i.e. after it was read.
template <int BLOCK>
__device__ __forceinline__ uint32_t block_append(uint32_t cnt, uint32_t* s2 /* [2][BLOCK / 64] */, int& par,
                                                 uint32_t& total) {
    constexpr int NW = BLOCK / 64;
    const uint32_t wid = threadIdx.x / 64;
    uint32_t* const s = s2 + par * NW;
    par ^= 1;
    const uint32_t inc = wave_inclusive_scan(cnt);
    if (lane_id() == 63) s[wid] = inc;
    lds_sync();
    uint32_t pre = 0, tot = 0;
#pragma unroll 4
    for (int i = 0; i < NW; ++i) {
        const uint32_t v = s[i];
        if ((uint32_t)i < wid) pre += v;
        tot += v;
    }
    const uint32_t first = total + pre + inc - cnt;
    total += uniform(tot);
    return first;
}

// Thresholding step on one WG's own histogram: NB bins held as NC LDS
// copies of stride STRIDE words.  Owner threads take NB / OWNERS bins each,
// in descending bin order across threads, so one block scan over the
// owners' sums locates the bin b that holds the element of rank `need`
// (1-based, from the top).  Returns b, the count above b and the count in b
// (0, 0, 0 when there are fewer elements: an error unless !STRICT).
template <int BLOCK, int NB, int NC, int STRIDE, bool STRICT = true>
__device__ __forceinline__ void local_select(const uint32_t* h, uint32_t need, uint32_t* scan, uint32_t* sel,
                                             uint32_t* status, uint32_t& b_out, uint32_t& above_out,
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
#pragma unroll 4
            for (int q = 0; q < NC; ++q) c += h[q * STRIDE + bin];
        }
        cnt[i] = c;
        tot += c;
    }
    if (t == 0) sel[2] = 0xFFFFFFFFu;  // "not found" until an owner writes
    uint32_t tot_all;
    uint32_t above = block_scan_total<BLOCK>(owner ? tot : 0u, scan, tot_all);
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
    if (hb == 0xFFFFFFFFu) {
        if (STRICT && t == 0) raise_flag(status, kFlagCapacity);
        b = 0; ab = 0; hb = 0;
    }
    b_out = b;
    above_out = ab;
    hb_out = hb;
}

// Wave 0 locates, in an NC-copy 256-bin histogram (copy stride kStride
// words, 16-byte aligned), the bin b holding the element of rank `need`
// (1-based, from the top bin down) and writes b, the count above b and the
// count in b to sel[0..2] (0, 0, 0 when the histogram holds fewer
// elements).  Lane l owns bins 255 - 4l .. 252 - 4l (descending across
// lanes), four consecutive words that it reads from every copy with one
// 16-byte load (eight copies' loads in flight together); one wave scan over
// the lanes' sums.  Only wave 0 calls it; the caller syncs before sel is read.
template <int NC>
__device__ __forceinline__ void wave_select256(const uint32_t* h, uint32_t need, uint32_t* sel) {
    const uint32_t l = lane_id();
    const uint32_t top = 255u - 4u * l;
    uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 0;  // bins top, top-1, top-2, top-3
    constexpr int QB = NC < 8 ? NC : 8;        // copies read per batch (registers)
#pragma unroll
    for (int q0 = 0; q0 < NC; q0 += QB) {
        uint4 v[QB];
#pragma unroll
        for (int q = 0; q < QB; ++q) v[q] = *reinterpret_cast<const uint4*>(h + (q0 + q) * kStride + (top - 3u));
#pragma unroll
        for (int q = 0; q < QB; ++q) {
            c0 += v[q].w;
            c1 += v[q].z;
            c2 += v[q].y;
            c3 += v[q].x;
        }
    }
    const uint32_t t = c0 + c1 + c2 + c3;
    const uint32_t inc = wave_inclusive_scan(t);
    const uint32_t all = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    uint32_t ex = inc - t;
    if (ex < need && need <= inc) {
        uint32_t b = top, c = c0;
        if (need > ex + c0) {
            ex += c0;
            b = top - 1u;
            c = c1;
            if (need > ex + c1) {
                ex += c1;
                b = top - 2u;
                c = c2;
                if (need > ex + c2) {
                    ex += c2;
                    b = top - 3u;
                    c = c3;
                }
            }
        }
        sel[0] = b;
        sel[1] = ex;
        sel[2] = c;
    }
    if (all < need && l == 0) {
        sel[0] = 0u;
        sel[1] = 0u;
        sel[2] = 0u;
    }
}

__device__ __forceinline__ void clear_words(uint32_t* p, int nwords, int tid, int nthreads) {
    uint4* const p4 = reinterpret_cast<uint4*>(p);
    for (int i = tid; i < nwords / 4; i += nthreads) p4[i] = uint4{0u, 0u, 0u, 0u};
    if (tid < nwords % 4) p[nwords / 4 * 4 + tid] = 0u;
}

// Write output slot `pos` of a row from composite c (and its key when the
// keys are recorded for the ordered output).
// (positions past k are dropped: the selection checks its counts instead)
__device__ __forceinline__ void put_out(int32_t* out, uint32_t* okey, uint32_t pos, uint64_t c, int k,
                                        uint32_t*) {
    if (pos < (uint32_t)k) {
        out[pos] = (int32_t)~(uint32_t)c;
        if (okey) okey[pos] = (uint32_t)(c >> 32);
    }
}

// ----------------------------------------------------------------- on-chip selection
//
// Bin of a candidate in the first round of select_buffer: a window of 256
// bins of 2^16 keys each from the bound lo (every candidate's key is at
// least lo); the top bin also takes every key above the window.
__device__ __forceinline__ uint32_t window_bin(uint64_t c, uint32_t lo) {
    const uint32_t d = ((uint32_t)(c >> 32) - lo) >> 16;
    return d < 255u ? d : 255u;
}

// The `need` largest of the m distinct composites cand[0 .. m), whose keys
// are all at least lo, go to out[W .. W + need) (the thresholding and
// collection steps of section 02, on chip).  The entries stay where they
// are; each round narrows the range [mn, mx] of composites still undecided.
// The first round bins the keys in a window from lo (window_bin; its
// histogram may have been built while the buffer was filled: `prebuilt`),
// later rounds split the range into 256 bins of (c - mn) >> s.  Each round
// locates the bin b holding rank `need` (wave 0), then the entries above b
// go to the output at their rank among them in buffer order (count, one
// block scan, place).  Once b holds at most kSmall entries they are
// gathered (in any order) and ranked exactly.  Every position follows from
// the buffer's order and the values alone, so the output order is
// determined by them.  The loops are mostly rolled (UNR iterations per
// body): the cost of a pass is the instructions its waves issue, so it
// scales with the entries, and the code stays short (it runs once per
// launch, often from a cold instruction cache).  Uses hist
// (kCopies x kStride words; zero on entry unless prebuilt), small (kSmall
// entries), scan and sel.  Every thread of the WG calls it, after a barrier
// that follows the buffer's (and the histogram's) last write.
template <int BLOCK, int UNR = 2>
__device__ __forceinline__ void select_buffer(const uint64_t* cand, uint32_t m, uint32_t need, uint32_t W,
                                              uint32_t lo, bool prebuilt, uint32_t* hist, uint64_t* small,
                                              uint32_t* scan, uint32_t* sel, int32_t* out, uint32_t* okey, int k,
                                              uint32_t* status) {
    const int tid = threadIdx.x;
    uint32_t ms = 0;  // entries gathered in small
    uint64_t mn = (uint64_t)lo << 32, mx = ~0ull;
    for (int round = 0;; ++round) {
        const uint64_t range = mx - mn;
        const int q = range ? 64 - __builtin_clzll(range) : 0;
        const int s = q > 8 ? q - 8 : 0;
        if (round > 0 || !prebuilt) {
            if (round > 0) {
                clear_words(hist, kCopies * kStride, tid, BLOCK);
                lds_sync();
            }
            uint32_t* const hc = hist + (tid % kCopies) * kStride;
#pragma unroll UNR
            for (uint32_t i = (uint32_t)tid; i < m; i += BLOCK) {
                const uint64_t c = cand[i];
                uint32_t bin;
                if (round == 0) {
                    bin = window_bin(c, lo);
                } else {
                    const uint64_t d = c - mn;  // wraps above the range when c < mn
                    bin = d <= range ? (uint32_t)(d >> s) : 256u;  // 256: spare slot
                }
                atomicAdd(&hc[bin], 1u);
            }
        }
        lds_sync();
        if (tid < 64) wave_select256<kCopies>(hist, need, sel);
        lds_sync();
        const uint32_t b = uniform(sel[0]), above = uniform(sel[1]), hb = uniform(sel[2]);
        if (hb == 0u) {
            if (tid == 0) raise_flag(status, kFlagCapacity);
            return;
        }
        uint64_t blo, bhi;  // composites of bin b
        if (round == 0) {
            blo = ((uint64_t)lo + ((uint64_t)b << 16)) << 32;
            bhi = b < 255u ? blo + ((1ull << 48) - 1u) : ~0ull;
        } else {
            blo = mn + ((uint64_t)b << s);
            const uint64_t width = ((uint64_t)1 << s) - 1u;
            bhi = mx - blo > width ? blo + width : mx;
        }
        const bool all = hb == need - above;        // the bin is taken whole
        const bool last = all || hb <= (uint32_t)kSmall;
        const bool gath = last & !all;              // the bin is gathered for the exact rank
        // winners of this round: in (bhi, mx] (none when bhi == mx, and then
        // bhi + 1 wraps); with `all` also the bin
        const uint64_t wlo = all ? blo : bhi + 1u;
        const bool any = all || bhi < mx;
        // count winners (high half) and gathered entries (low half), one
        // block scan numbers both in buffer order, then place them
        uint32_t cnt = 0;
        const uint32_t bk = lo + (b << 16);
        const uint64_t wk64 = all ? (uint64_t)bk : (b < 255u ? (uint64_t)bk + 0x10000u : (1ull << 32));
        const bool anyk = wk64 <= 0xFFFFFFFFull;
        const uint32_t wk = (uint32_t)wk64;
        if (round == 0) {
            const uint32_t* const ch = reinterpret_cast<const uint32_t*>(cand) + 1;  // keys: high words
#pragma unroll UNR
            for (uint32_t i = (uint32_t)tid; i < m; i += BLOCK) {
                const uint32_t key = ch[2u * i];
                const bool w = anyk & (key >= wk);
                cnt += (w ? (1u << 16) : 0u) + ((gath & (key >= bk) & !w) ? 1u : 0u);
            }
        } else if (any | gath) {
#pragma unroll UNR
            for (uint32_t i = (uint32_t)tid; i < m; i += BLOCK) {
                const uint64_t c = cand[i];
                cnt += ((any & (c >= wlo) & (c <= mx)) ? (1u << 16) : 0u) + ((gath & (c >= blo) & (c <= bhi)) ? 1u : 0u);
            }
        }
        uint32_t tot;
        const uint32_t pos = block_scan_total<BLOCK>(cnt, scan, tot);
        uint32_t p = W + (pos >> 16), g = pos & 0xFFFFu;
        if (round == 0) {
#pragma unroll UNR
            for (uint32_t i = (uint32_t)tid; i < m; i += BLOCK) {
                const uint64_t c = cand[i];
                const uint32_t key = (uint32_t)(c >> 32);
                const bool w = anyk & (key >= wk);
                if (w) {
                    put_out(out, okey, p++, c, k, status);
                } else if (gath & (key >= bk)) {
                    if (g < (uint32_t)kSmall) small[g] = c;
                    ++g;
                }
            }
        } else if (any | gath) {
#pragma unroll UNR
            for (uint32_t i = (uint32_t)tid; i < m; i += BLOCK) {
                const uint64_t c = cand[i];
                if (any & (c >= wlo) & (c <= mx)) {
                    put_out(out, okey, p++, c, k, status);
                } else if (gath & (c >= blo) & (c <= bhi)) {
                    if (g < (uint32_t)kSmall) small[g] = c;
                    ++g;
                }
            }
        }
        tot >>= 16;
        if (tot != (all ? need : above)) {
            if (tid == 0) raise_flag(status, kFlagCapacity);
            return;
        }
        if (all) return;
        W += above;
        need -= above;
        mn = blo;
        mx = bhi;
        if (last) {
            ms = hb;
            break;
        }
        lds_sync();  // the histogram is cleared next
    }
    // exact rank of the gathered few: P consecutive lanes per candidate (P a
    // power of two up to 16 with P * ms within the block: one pass), each
    // comparing a strided share four at a time; the counts of a group are
    // summed into its first lane by DPP row shifts (a group never crosses a
    // row of 16 lanes)
    lds_sync();
    uint32_t P = 1;
    while (P < 16u && 2u * P * ms <= (uint32_t)BLOCK) P *= 2u;
    for (uint32_t i0 = 0; i0 < ms; i0 += (uint32_t)BLOCK / P) {
        const uint32_t i = i0 + (uint32_t)tid / P, qq = (uint32_t)tid % P;
        if (i0 + (uint32_t)(tid & ~63) / P >= ms) break;  // whole waves past the end
        const uint64_t c = i < ms ? small[i] : ~0ull;
        uint32_t rank = 0;
        uint32_t j = qq;
        for (; j + 3u * P < ms; j += 4u * P)
            rank += (uint32_t)(small[j] > c) + (uint32_t)(small[j + P] > c) + (uint32_t)(small[j + 2u * P] > c) +
                    (uint32_t)(small[j + 3u * P] > c);
        for (; j < ms; j += P) rank += small[j] > c;
        if (P > 1u) rank += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)rank, 0x101, 0xF, 0xF, false);  // row_shl:1
        if (P > 2u) rank += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)rank, 0x102, 0xF, 0xF, false);  // row_shl:2
        if (P > 4u) rank += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)rank, 0x104, 0xF, 0xF, false);  // row_shl:4
        if (P > 8u) rank += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)rank, 0x108, 0xF, 0xF, false);  // row_shl:8
        if (i < ms && qq == 0u && rank < need) put_out(out, okey, W + rank, c, k, status);
    }
}

// Exact selection of a row by passes over it in global memory (one WG): the
// rare case where the candidates of a bound do not fit on chip or the bound
// overshot.  Each pass histograms the composites inside the current range
// (4096 bins the first time, 256 later) and keeps the bin holding the k-th
// largest, until it holds at most `cap`; a last pass sends the composites
// above the range to the output and the range's to the buffer, in a fixed
// order (block scans), and select_buffer finishes.  Passes are rolled loops
// of U chunks per lane (small code beside the hot paths).  hist holds
// kHistWords words.
template <int BLOCK, int CAP>
__device__ __forceinline__ void select_by_passes(const char* base, int off, int L, int nchunks, int k, int32_t* out,
                                                 uint32_t* okey, uint64_t* cand, uint32_t* hist, uint64_t* small,
                                                 uint32_t* scan, uint32_t* sel, uint32_t* status) {
    constexpr int cap = CAP;
    constexpr int U = 2;
    const int tid = threadIdx.x;
    auto reread = [&](auto&& f) {
#pragma unroll 1
        for (int c0 = 0; c0 < nchunks; c0 += U * BLOCK) {
            u32x4_t v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * BLOCK + tid;
                v[u] = *reinterpret_cast<const u32x4_t*>(base + (size_t)(c < nchunks ? c : 0) * 16u);
            }
            uint32_t kk[4 * U], ii[4 * U];  // keys (0: empty slot) and indices
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * BLOCK + tid;
                const int e0 = 4 * c - off;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = (c < nchunks) & ((uint32_t)(e0 + e) < (uint32_t)L);
                    kk[4 * u + e] = ok ? key_of(__uint_as_float(v[u][e])) : 0u;
                    ii[4 * u + e] = (uint32_t)(e0 + e);
                }
            }
            f(kk, ii);
        }
    };
    uint64_t mn = 0, mx = ~0ull;
    uint32_t need = (uint32_t)k, W = 0, hb = 0;
    for (int pass = 0;; ++pass) {
        // once the range holds one key, only the valid indices' part of it
        if ((mn >> 32) == (mx >> 32)) {
            const uint64_t lo_i = (mn & 0xFFFFFFFF00000000ull) | (uint64_t)(0u - (uint32_t)L);
            if (mn < lo_i) mn = lo_i;
        }
        const bool first = pass == 0;
        const int nbits = first ? 12 : 8;
        const uint64_t range = mx - mn;
        const int q = range ? 64 - __builtin_clzll(range) : 0;
        const int s = q > nbits ? q - nbits : 0;
        clear_words(hist, first ? 4096 : kCopies * kStride, tid, BLOCK);
        lds_sync();
        uint32_t* const hc = first ? hist : hist + (tid % kCopies) * kStride;
        const uint64_t lo = mn, hi = mx;
        reread([&](const uint32_t* kk, const uint32_t* ii) {
#pragma unroll
            for (int i = 0; i < 4 * U; ++i) {
                const uint64_t c = composite(kk[i], ii[i]);
                if ((kk[i] != 0u) & (c >= lo) & (c <= hi)) atomicAdd(&hc[(uint32_t)((c - lo) >> s)], 1u);
            }
        });
        lds_sync();
        uint32_t b, above, hbin;
        if (first) local_select<BLOCK, 4096, 1, 4096>(hist, need, scan, sel, status, b, above, hbin);
        else local_select<BLOCK, 256, kCopies, kStride>(hist, need, scan, sel, status, b, above, hbin);
        need -= above;
        W += above;
        hb = hbin;
        mn += (uint64_t)b << s;
        const uint64_t width = ((uint64_t)1 << s) - 1u;
        if (mx - mn > width) mx = mn + width;
        if (hb <= (uint32_t)cap || s == 0 || hb == 0u) break;
    }
    // collection: above the range to the output, the range to the buffer (or
    // to the output when it is taken whole)
    const bool all = hb == need;
    const uint64_t lo = mn, hi = mx;
    uint32_t n1 = 0, n2 = 0;
    reread([&](const uint32_t* kk, const uint32_t* ii) {
        uint32_t cnt = 0, kinds = 0;
#pragma unroll
        for (int i = 0; i < 4 * U; ++i) {
            const uint64_t c = composite(kk[i], ii[i]);
            const uint32_t kd = kk[i] == 0u ? 0u : (c > hi ? 1u : (c >= lo ? 2u : 0u));
            kinds |= kd << (2 * i);
            cnt += kd == 1u ? (1u << 16) : (kd == 2u ? 1u : 0u);
        }
        uint32_t tot;
        const uint32_t pos = block_scan_total<BLOCK>(cnt, scan, tot);
        uint32_t p1 = n1 + (pos >> 16), p2 = n2 + (pos & 0xFFFFu);
#pragma unroll
        for (int i = 0; i < 4 * U; ++i) {
            const uint32_t kd = (kinds >> (2 * i)) & 3u;
            if (kd == 0u) continue;
            const uint64_t c = composite(kk[i], ii[i]);
            if (kd == 1u) {
                if (p1 < W) put_out(out, okey, p1, c, k, status);
                else raise_flag(status, kFlagCapacity);
                ++p1;
            } else {
                if (all) put_out(out, okey, W + p2, c, k, status);
                else if (p2 < (uint32_t)cap) cand[p2] = c;
                else raise_flag(status, kFlagCapacity);
                ++p2;
            }
        }
        n1 += tot >> 16;
        n2 += tot & 0xFFFFu;
    });
    if (all || hb == 0u) return;
    clear_words(hist, kCopies * kStride, tid, BLOCK);
    lds_sync();
    // the bucket's keys all lie in [mn >> 32, mx >> 32]; its lowest key is the window's origin
    select_buffer<BLOCK>(cand, hb < (uint32_t)cap ? hb : (uint32_t)cap, need, W, (uint32_t)(mn >> 32), false, hist,
                         small, scan, sel, out, okey, k, status);
}

// The 16-bit key prefix of the element of rank r (1-based, from the top)
// among the keys the WG's threads hold (NK each, 0 = empty): its top byte
// from a 256-bin histogram, then its second byte from a histogram of the
// keys in that bin (h1 and h2: kCopies x kStride words each, zero on entry,
// behind a barrier; h1 is zero again on return).  At least 1, so that the
// bound never admits empty slots.
template <int BLOCK, int NK>
__device__ __forceinline__ uint32_t bound_select(const uint32_t (&ks)[NK], uint32_t r, uint32_t* h1, uint32_t* h2, uint32_t* sel) {
    const int tid = threadIdx.x;
    uint32_t* const hc1 = h1 + (tid % kCopies) * kStride;
#pragma unroll
    for (int i = 0; i < NK; ++i) atomicAdd(&hc1[ks[i] != 0u ? ks[i] >> 24 : 256u], 1u);  // 256: spare slot
    lds_sync();
    if (tid < 64) wave_select256<kCopies>(h1, r, sel);
    lds_sync();
    const uint32_t b1 = uniform(sel[0]), a1 = uniform(sel[1]), n1 = uniform(sel[2]);
    clear_words(h1, kCopies * kStride, tid, BLOCK);  // left zero for the caller (ordered by the next barrier)
    if (n1 == 0u) {
        lds_sync();
        return 1u;
    }
    uint32_t* const hc2 = h2 + (tid % kCopies) * kStride;
#pragma unroll
    for (int i = 0; i < NK; ++i)
        if ((ks[i] != 0u) & ((ks[i] >> 24) == b1)) atomicAdd(&hc2[(ks[i] >> 16) & 0xFFu], 1u);
    lds_sync();
    if (tid < 64) wave_select256<kCopies>(h2, r - a1, sel);
    lds_sync();
    const uint32_t b2 = uniform(sel[0]);
    const uint32_t lo = (b1 << 24) | (b2 << 16);
    return lo > 1u ? lo : 1u;
}

// The key of rank r (1-based, from the top) among the keys the WG's threads
// hold (NK each, 0 = empty), located to within 1/4096 of their range in one
// pass: the range [min, max] of the keys split into 4096 bins; returns the
// lower edge of the bin holding rank r (at least 1), a lower bound on that
// key.  Bins follow the keys' own range, so keys that share their top bits
// (logits of one magnitude) still spread over many bins (few LDS atomics
// on one word).  hist: 4096 words, zero on entry, behind a barrier; scan:
// BLOCK / 64 words; red: 2 BLOCK / 64 words; sel: 4 words.
template <int BLOCK, int NK>
__device__ __forceinline__ uint32_t bound_select_range(const uint32_t (&ks)[NK], uint32_t r, uint32_t* hist,
                                                       uint32_t* scan, uint32_t* sel, uint32_t* red,
                                                       uint32_t* status) {
    constexpr int NW = BLOCK / 64;
    const int tid = threadIdx.x;
    uint32_t mn = ~0u, mx = 0u;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        if (ks[i] != 0u) {
            mn = min(mn, ks[i]);
            mx = max(mx, ks[i]);
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    }
    if ((tid & 63) == 0) {
        red[2 * (tid >> 6)] = mn;
        red[2 * (tid >> 6) + 1] = mx;
    }
    lds_sync();
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        mn = min(mn, red[2 * i]);
        mx = max(mx, red[2 * i + 1]);
    }
    mn = uniform(mn);
    mx = uniform(mx);
    if (mx == 0u) return 1u;  // no keys
    const uint32_t range = mx - mn;
    const int q = range ? 32 - __builtin_clz(range) : 0;
    const int s = q > 12 ? q - 12 : 0;  // (key - mn) >> s < 4096
#pragma unroll
    for (int i = 0; i < NK; ++i)
        if (ks[i] != 0u) atomicAdd(&hist[(ks[i] - mn) >> s], 1u);
    lds_sync();
    uint32_t b, above, hb;
    local_select<BLOCK, 4096, 1, 4096, false>(hist, r, scan, sel, status, b, above, hb);
    if (hb == 0u) return 1u;
    const uint32_t lo = mn + (b << s);
    return lo > 1u ? lo : 1u;
}

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

template <int BLOCK, int ITEMS, bool RESIDENT, bool KEYS, int SPT>
__global__ __launch_bounds__(BLOCK) void topk_split_kernel(const KParams P) {
    static_assert(ITEMS % 4 == 0, "ITEMS counts whole 16-byte chunks");
    static_assert(BLOCK % 64 == 0 && BLOCK >= 256, "whole waves, 256 histogram owners");
    static_assert(kCopies * kStride * 4 <= kBufCap * 8, "the bound's second histogram fits in the buffer");
    constexpr int CHUNKS = ITEMS / 4;            // chunks per thread per tile
    constexpr int TILE_CHUNKS = BLOCK * CHUNKS;  // chunks per tile
    // SPT: sample chunks per thread (the host keeps the sample within it)
    static_assert(SPT >= 1 && SPT * BLOCK <= kSampleMax, "sample fits the block");
    __shared__ SplitSmem<BLOCK> sm;

    const int tid = threadIdx.x;
    const int G = P.G;
    const int row = blockIdx.x / G;
    const int w = blockIdx.x - row * G;
    const int n = P.n;
    const int k = P.k;
    const float* __restrict__ prow = P.logits + (size_t)row * (size_t)n;
    int32_t* __restrict__ out = P.out + (size_t)row * (size_t)k;
    uint32_t* const okey = KEYS ? P.keys + (size_t)row * (size_t)k : nullptr;
    const int L = valid_length(P.lengths, row, n);
    if (L <= k) {  // everything valid is selected; pad with -1
        if (w == 0)
            for (int i = tid; i < k; i += BLOCK) out[i] = i < L ? i : -1;
        return;
    }
    const int off = (int)(((uintptr_t)prow >> 2) & 3);  // elements before the first 16-byte boundary
    const int nchunks = (off + L + 3) >> 2;
    const int cpw = P.chunks_per_wg;
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
    const int Sc = own_sample ? 0 : min(nchunks, P.sample_chunks);
    const bool whole_sample = nchunks <= P.sample_chunks;
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
        // prefixes over the regions (wave 0): of the counts, and of the
        // counts past the speculative reads
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
        const uint32_t c_others = uniform(sm.tot[0]), X = uniform(sm.tot[1]);
        C = total + c_others;
        ok = sm.bad == 0u && C >= (uint32_t)k && C <= (uint32_t)kBufCap;
        // every entry is read (when the row is finished otherwise, waited
        // for; all missing ones polled again together), moved to the buffer
        // and cleared for the next launch
        {
            const uint32_t cn = sm.cnt[mine ? wr : 0], pn = sm.pre[mine ? wr : 0];
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
#pragma unroll
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
}

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

// The ordered form of one row, produced by the WG that selected it (the
// need_sorted option of section 02's radix_topk: descending order; equal
// values by index ascending, the rule that selects them).  The row's cnt
// selected composites (recorded keys and indices, or keys of the logits
// when the whole valid row is selected) are binned by key into at most
// kOrdBins bins over their key range, counted, scattered into T bin by bin
// (descending bins), and each is written at its exact rank: the entries of
// the bins above its own plus the larger ones of its own bin (bins hold a
// few entries, or equal keys).  Positions follow from the values alone;
// slots past cnt get -1 and -inf.  T: CAP composites of LDS (cnt <= MAXC
// <= CAP; the ranked entries are staged after them when 2 cnt <= CAP);
// hist: 2 * kOrdBins words; scan: BLOCK / 64 words.
constexpr int kOrdBins = 2048;
constexpr int kOrdLds = 2048;  // one WG per row: k up to this keeps the unordered output in LDS
template <int BLOCK, int MAXC, int CAP>
__device__ __forceinline__ void ordered_finish(const int32_t* sidx, const uint32_t* skey, bool from_logits,
                                               const float* prow, uint32_t L, uint32_t cnt, int k, int32_t* oout,
                                               float* ovals, uint64_t* T, uint32_t* hist, uint32_t* scan) {
    static_assert(MAXC <= CAP, "the entries fit T");
    constexpr int NU = (MAXC + BLOCK - 1) / BLOCK;  // cnt <= MAXC
    constexpr int NW = BLOCK / 64;
    constexpr int BPT = kOrdBins / BLOCK;  // bins per thread for the starts
    static_assert(kOrdBins % BLOCK == 0 && kOrdBins >= BLOCK, "whole bins per thread");
    constexpr uint32_t BITS = 11;          // log2(kOrdBins)
    static_assert((1 << BITS) == kOrdBins, "kOrdBins is 2^BITS");
    const int tid = threadIdx.x;
    const uint32_t wid = (uint32_t)tid / 64u;
    uint32_t* const cur = hist + kOrdBins;
    clear_words(hist, kOrdBins, tid, BLOCK);
    uint64_t e[NU];
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const uint32_t i = (uint32_t)(tid + u * BLOCK);
        e[u] = 0ull;
        if (i < cnt) {
            const uint32_t idx = from_logits ? i : (uint32_t)sidx[i];
            const uint32_t key = from_logits ? key_of(prow[i]) : skey[i];
            e[u] = composite(key, idx);
            kmin = min(kmin, key);
            kmax = max(kmax, key);
        }
    }
    for (int sft = 32; sft >= 1; sft >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, sft));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, sft));
    }
    uint32_t* const red = cur;  // the cursors are written only after this is read
    if (lane_id() == 0) {
        red[wid] = kmin;
        red[NW + wid] = kmax;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        kmin = min(kmin, red[w]);
        kmax = max(kmax, red[NW + w]);
    }
    const uint32_t range = kmax - kmin;  // cnt >= 1
    const uint32_t q = range ? 32u - (uint32_t)__builtin_clz(range) : 0u;
    const uint32_t sh = q > BITS ? q - BITS : 0u;
#pragma unroll
    for (int u = 0; u < NU; ++u)
        if ((uint32_t)(tid + u * BLOCK) < cnt) atomicAdd(&hist[((uint32_t)(e[u] >> 32) - kmin) >> sh], 1u);
    __syncthreads();
    // bin starts, bins descending: thread t owns bins top .. top - BPT + 1
    {
        const uint32_t top = (uint32_t)kOrdBins - 1u - (uint32_t)(tid * BPT);
        uint32_t c[BPT], t = 0;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            c[i] = hist[top - (uint32_t)i];
            t += c[i];
        }
        uint32_t tot;
        uint32_t ex = block_scan_total<BLOCK>(t, scan, tot);
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            cur[top - (uint32_t)i] = ex;
            ex += c[i];
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        if ((uint32_t)(tid + u * BLOCK) < cnt) {
            const uint32_t b = ((uint32_t)(e[u] >> 32) - kmin) >> sh;
            T[atomicAdd(&cur[b], 1u)] = e[u];
        }
    }
    __syncthreads();
    // cur[b] is now the end of bin b in T.  The ranked entries are staged in
    // LDS after T when they fit (then written in order), else stored at
    // their ranks directly
    const bool staged = 2u * cnt <= (uint32_t)CAP;
    uint2* const O = reinterpret_cast<uint2*>(T + cnt);
    for (uint32_t qi = (uint32_t)tid; qi < cnt; qi += BLOCK) {
        const uint64_t c = T[qi];
        const uint32_t key = (uint32_t)(c >> 32);
        const uint32_t b = (key - kmin) >> sh;
        const uint32_t end = cur[b], st = end - hist[b];
        uint32_t r = st;
        for (uint32_t j = st; j < end; j += 8u) {
            uint64_t t[8];  // clamped loads, the slots past the bin not counted
#pragma unroll
            for (int u = 0; u < 8; ++u) t[u] = T[min(j + (uint32_t)u, end - 1u)];
#pragma unroll
            for (int u = 0; u < 8; ++u) r += (uint32_t)((j + (uint32_t)u < end) & (t[u] > c));
        }
        const uint32_t idx = ~(uint32_t)c;
        const float v = value_of(key, prow, L, idx);
        if (staged) {
            O[r] = make_uint2(idx, __float_as_uint(v));
        } else {
            oout[r] = (int32_t)idx;
            if (ovals) ovals[r] = v;
        }
    }
    if (staged) {  // in order: coalesced stores, marked non-temporal (written once, not read here)
        __syncthreads();
        for (uint32_t j = (uint32_t)tid; j < cnt; j += BLOCK) {
            const uint2 o = O[j];
            __builtin_nontemporal_store((int32_t)o.x, oout + j);
            if (ovals) __builtin_nontemporal_store(__uint_as_float(o.y), ovals + j);
        }
    }
    for (uint32_t j = cnt + (uint32_t)tid; j < (uint32_t)k; j += BLOCK) {
        oout[j] = -1;
        if (ovals) ovals[j] = -__builtin_huge_valf();
    }
}

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

// The row's queries staged in LDS, shared by the WG's waves: chunk c of
// head h in slot c ^ (h % CPR) of the head's row.
template <int D>
__device__ __forceinline__ void logits_stage_queries(u32x4_t* qs, const uint16_t* q, int row, int H) {
    constexpr int CPR = D / 8;
    const u32x4_t* const qrow = reinterpret_cast<const u32x4_t*>(q + (size_t)row * H * D);
    for (int i = threadIdx.x; i < H * CPR; i += kLogitBlock) {
        const int h = i / CPR, c = i % CPR;
        qs[h * CPR + (c ^ (h % CPR))] = qrow[i];
    }
}

// The A operands (queries, from LDS) and the weights of this lane's four
// heads per block of 16, once for all of a wave's groups; padding heads are
// zero.
template <int D, int HB>
__device__ __forceinline__ void logits_operands(const u32x4_t* qs, const float* wrow, int H, int lane,
                                                bf16x8_t (&a)[HB][D / 32], float (&wt)[HB][4]) {
    constexpr int KB = D / 32, CPR = D / 8;
    const int m = lane & 15, g = lane >> 4;
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
            const float x = wrow[min(hh, H - 1)];
            wt[hb][i] = hh < H ? x : 0.0f;
        }
    }
}

// The logit of token tw + lane, from the group of 64 keys staged at st
// (tokens at or past L take zero keys; their result is not used).
template <int D, int HB>
__device__ __forceinline__ float logits_group(const u32x4_t* st, const bf16x8_t (&a)[HB][D / 32],
                                              const float (&wt)[HB][4], int tw, int L, int lane) {
    constexpr int KB = D / 32, CPR = D / 8;
    const int m = lane & 15, g = lane >> 4;
    const bf16x8_t zero = {};
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
    // lane l's token is tw + l: block l/16, token l%16 of it
    return g == 0 ? v[0] : (g == 1 ? v[1] : (g == 2 ? v[2] : v[3]));
}

template <int D, int HB>
__global__ void __launch_bounds__(kLogitBlock) topk_logits_kernel(LogitParams P) {
    constexpr int CPR = D / 8;         // 16-byte chunks per key
    constexpr int GB = 64 * D * 2;     // bytes of one group's keys (64 tokens)
    constexpr int NL = GB / 1024;      // 16-byte loads per lane per group
    // each wave stages its current group of keys in its own LDS region;
    // chunk c of token r sits in slot c ^ (r % CPR) of the token's row, so
    // the MFMA-layout reads (16 tokens, one chunk each) hit distinct banks
    __shared__ u32x4_t stage[kLogitBlock / 64][GB / 16];
    __shared__ u32x4_t qs[HB * 16 * CPR];
    const int row = blockIdx.x / P.tiles;
    const int tile = blockIdx.x - row * P.tiles;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
    logits_stage_queries<D>(qs, P.q, row, H);
    __syncthreads();  // before any wave leaves
    if (t0 >= n) return;
    float* const lrow = P.logits + (size_t)row * (size_t)n;
    const float ninf = -__builtin_huge_valf();
    for (int t = max(t0, tv) + lane; t < t1; t += 64) lrow[t] = ninf;
    if (t0 >= tv) return;
    const int ng = (tv - t0 + 63) / 64;  // groups holding valid tokens
    bf16x8_t a[HB][D / 32];
    float wt[HB][4];
    logits_operands<D, HB>(qs, P.w + (size_t)row * H, H, lane, a, wt);
    u32x4_t* const st = stage[wave];
    // the next group's loads are in flight while the current one is
    // computed from LDS; the wave's region is its own, so no barrier
    if (!early) logits_load<D, NL>(r, K, t0, L - 1 - t0, lane);
    for (int gi = 0; gi < ng; ++gi) {
        const int tw = t0 + gi * 64;
        logits_stage<D, NL>(st, r, lane);
        if (gi + 1 < ng) logits_load<D, NL>(r, K, tw + 64, L - 1 - (tw + 64), lane);
        const float mine = logits_group<D, HB>(st, a, wt, tw, L, lane);
        const int t = tw + lane;
        if (t < t1) lrow[t] = t < L ? mine : ninf;
    }
}

// ----------------------------------------------------------------- indexer with the selection's first pass
//
// Steps 1 and 2 of DSA-style decoding (the TopK article, section 01) where
// the logits kernel also does the selection's pass over the row, so that
// the selection afterwards reads candidates only, never the logits row.  A
// row's groups of 64 tokens are split between sample WGs, which take every
// F-th group (sample group j is group j F + F - 1), and tile WGs, which
// take the others in order.  Both write the logits (the output, or
// scratch) as the logits kernel does and keep their keys in registers.
//  * Sample WGs publish their keys, tagged with the row's epoch; the row's
//    last sample WG reads them all and publishes the bound, a lower bound on
//    the sample's element of rank r = m + 4 sqrt(m) + 6, m = k S / L for S
//    sampled valid tokens (the split selection's rule).
//  * Tile WGs wait for the bound, then write how many of their keys reach
//    it and those composites, in a fixed order, to their region.
// Then one WG per row (topk_indexer_finish_kernel) gathers the sample's keys
// at or above the bound and every region into LDS and selects the row's k
// largest there (select_buffer, which needs every key at or above the
// bound and at least k of them).  When fewer than k or more than its
// buffer holds came out (the sample misled) it selects by passes over the
// logits row instead.
// The only wait is a tile WG's for its row's bound, which WGs placed before
// it in the grid publish (dispatched before it, so it never waits on a WG
// without a slot); it is bounded (spin_limit; flag kFlagTimeout), and a WG
// that gives up marks its count so that the row is selected by passes.

constexpr int kFusedMaxT = 512;        // tile WGs per row
constexpr int kFusedSample = 4096;     // sampled tokens per row at most (64 groups)
constexpr int kFinBlock = 1024;        // threads of the finishing WG
constexpr uint32_t kFusedGaveUp = 0xFFFFFFFFu;  // a tile WG's count when its wait for the bound gave up

// Per-row state; the rows' sample keys follow the array of these
// (kFusedSample tagged entries per row, row r always at the same place, so
// that a stale entry only ever carries an older epoch of its own row).
struct alignas(64) FusedRow {
    uint64_t bound;            // (tag << 32) | the row's bound
    uint32_t epoch;            // advanced by the finishing WG
    uint32_t pad[13];
    uint64_t cnt[kFusedMaxT];  // (tag << 32) | candidates of tile WG t
};

struct FusedParams {
    const uint16_t* q;       // [rows, H, D] bf16
    const uint16_t* kc;      // keys of row r at kc + r * kstride: [n, D] bf16
    const float* w;          // [rows, H]
    const int32_t* lengths;  // [rows] or null
    float* logits;           // [rows, n]
    int32_t* out;            // [rows, k]
    uint32_t* status;
    FusedRow* frs;           // [rows]
    uint64_t* samp;          // [rows][kFusedSample] tagged sample keys
    uint64_t* stage;         // [rows][NT][256 gpw] candidate composites
    int64_t kstride;
    int32_t rows, n, H, k;
    int32_t gpw;             // groups of 64 tokens per wave
    int32_t F;               // sample stride in groups (>= 2)
    int32_t ns;              // sample groups per row (<= 64)
    int32_t NS, NT;          // sample and tile WGs per row
};

template <int D, int HB>
__global__ void __launch_bounds__(kLogitBlock) topk_indexer_cand_kernel(FusedParams P) {
    constexpr int BLOCK = kLogitBlock;
    constexpr int CPR = D / 8;
    constexpr int GB = 64 * D * 2;   // bytes of one group's keys
    constexpr int NL = GB / 1024;    // 16-byte loads per lane per group
    constexpr int kStageBytes = (BLOCK / 64) * GB;
    constexpr int kLds = kStageBytes + HB * 16 * CPR * 16;
    static_assert((4096 + 4 + 3 * BLOCK / 64) * 4 <= kLds, "the bound's histogram fits");
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
    const int per_row = P.NS + P.NT;
    const int row = (int)blockIdx.x / per_row;
    const int wi = (int)blockIdx.x - row * per_row;
    const bool sampler = wi < P.NS;
    const int widx = sampler ? wi : wi - P.NS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = P.n, H = P.H, k = P.k;
    const int L = valid_length(P.lengths, row, n);
    const int F = P.F, ns = P.ns, gpw = P.gpw;
    const int ng = (n + 63) >> 6;
    const int gbase = (widx * (BLOCK / 64) + wave) * gpw;  // the wave's first group number in its role
    const int cntw = max(0, min(gpw, (sampler ? ns : ng - ns) - gbase));
    auto group_of = [&](int i) -> int {
        const int u = gbase + i;
        return sampler ? u * F + F - 1 : u + min(u / (F - 1), ns);
    };
    int nvw = 0;  // the wave's groups holding valid tokens (a prefix: groups ascend)
    for (int i = 0; i < cntw; ++i)
        if (64 * group_of(i) < L) nvw = i + 1;
    u32x4_t* const st = reinterpret_cast<u32x4_t*>(smem) + wave * (GB / 16);
    u32x4_t* const qs = reinterpret_cast<u32x4_t*>(smem + kStageBytes);
    const char* const K = reinterpret_cast<const char*>(P.kc + (size_t)row * (size_t)P.kstride);
    u32x4_t r[NL];
    const bool early = gpw > 1 && nvw > 0;
    if (early) {
        const int tw = 64 * group_of(0);
        logits_load<D, NL>(r, K, tw, L - 1 - tw, lane);
    }
    logits_stage_queries<D>(qs, P.q, row, H);
    FusedRow* const fr = P.frs + row;
    // a sample WG's epoch (tags of its keys) is loaded now, before its key
    // loads, and is there when they are; tile WGs load it once their keys
    // are done (the many WGs of a row then do not load it all at once)
    uint32_t ep = 0;
    if (sampler && L > k) ep = ld_dev(&fr->epoch);
    __syncthreads();
    float* const lrow = P.logits + (size_t)row * (size_t)n;
    const float ninf = -__builtin_huge_valf();
    uint32_t kk[8];  // key of token 64 group_of(i) + lane (0: none)
#pragma unroll
    for (int i = 0; i < 8; ++i) kk[i] = 0u;
    if (nvw > 0) {
        bf16x8_t a[HB][D / 32];
        float wt[HB][4];
        logits_operands<D, HB>(qs, P.w + (size_t)row * H, H, lane, a, wt);
        if (!early) {
            const int tw = 64 * group_of(0);
            logits_load<D, NL>(r, K, tw, L - 1 - tw, lane);
        }
        for (int i = 0; i < nvw; ++i) {
            const int tw = 64 * group_of(i);
            logits_stage<D, NL>(st, r, lane);
            if (i + 1 < nvw) {
                const int tn = 64 * group_of(i + 1);
                logits_load<D, NL>(r, K, tn, L - 1 - tn, lane);
            }
            const float mine = logits_group<D, HB>(st, a, wt, tw, L, lane);
            const int t = tw + lane;
            const bool valid = t < L;
            if (t < n) lrow[t] = valid ? mine : ninf;
            const uint32_t key = valid ? key_of(mine) : 0u;
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2)
                if (s2 == i) kk[s2] = key;
        }
    }
    for (int i = nvw; i < cntw; ++i) {
        const int t = 64 * group_of(i) + lane;
        if (t < n) lrow[t] = ninf;
    }
    if (L <= k) return;  // every valid token is selected: nothing to publish
    const uint64_t lim = spin_limit();
    uint64_t* const sp = P.samp + (size_t)row * (size_t)kFusedSample;
    if (sampler) {
        const uint32_t tag = make_tag(uniform(ep));
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2)
            if (s2 < cntw) st_dev(&sp[(gbase + s2) * 64 + lane], ((uint64_t)tag << 32) | kk[s2]);
        if (widx != P.NS - 1) return;
        // the row's last sample WG: every sample key (waited for), then the bound
        __syncthreads();  // the key stage and the queries are done with
        uint32_t* const hist = reinterpret_cast<uint32_t*>(smem);
        uint32_t* const sel = hist + 4096;
        uint32_t* const scan = sel + 4;
        uint32_t* const red = scan + BLOCK / 64;
        clear_words(hist, 4096, tid, BLOCK);
        const int SN = ns * 64;
        uint64_t v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int j = tid + u * BLOCK;
            v[u] = j < SN ? ld_dev(&sp[j]) : ((uint64_t)tag << 32);
        }
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (;;) {
            bool miss = false;
#pragma unroll
            for (int u = 0; u < 16; ++u) miss |= (uint32_t)(v[u] >> 32) != tag;
            if (!miss) break;
            if (__builtin_amdgcn_s_memrealtime() - t0 >= lim) {
                raise_flag(P.status, kFlagTimeout);  // the bound then comes from the keys seen
                break;
            }
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int j = tid + u * BLOCK;
                if ((uint32_t)(v[u] >> 32) != tag) v[u] = ld_dev(&sp[j]);
            }
        }
        uint32_t ks[16], cnt = 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            ks[u] = (uint32_t)(v[u] >> 32) == tag ? (uint32_t)v[u] : 0u;
            cnt += ks[u] != 0u;
        }
        uint32_t S;
        (void)block_scan_total<BLOCK>(cnt, scan, S);
        uint32_t lo = 1u;
        if (S > 0u) {
            const float mexp = (float)k * (float)S / (float)L;
            const float rf = ceilf(mexp + 4.0f * sqrtf(mexp) + 6.0f);
            lo = bound_select_range<BLOCK, 16>(ks, rf >= (float)S ? S : (uint32_t)rf, hist, scan, sel, red, P.status);
        }
        if (tid == 0) st_dev(&fr->bound, ((uint64_t)tag << 32) | lo);
        return;
    }
    // a tile WG: wave 0 waits for the bound (published by a sample WG placed
    // before), polling with a pause so that a row's many waiting WGs load
    // the memory system little; the bound reaches the other waves through
    // LDS (wave 0's key stage, which it no longer uses)
    uint32_t* const scan = reinterpret_cast<uint32_t*>(smem);
    uint32_t* const lo_w = scan + BLOCK / 64;
    uint32_t tag = 0;  // wave 0's
    if (wave == 0) {
        tag = make_tag(uniform(ld_dev(&fr->epoch)));
        uint32_t v = 1u;
        if (ns > 0) {
            uint64_t bv = ld_dev(&fr->bound);
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while ((uint32_t)(bv >> 32) != tag) {
                if (__builtin_amdgcn_s_memrealtime() - t0 >= lim) {
                    bv = 0ull;  // gave up: 0, never a bound
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
                bv = ld_dev(&fr->bound);
            }
            v = (uint32_t)bv;
        }
        if (lane == 0) *lo_w = v;
    }
    lds_sync();  // every wave is past its key stage; the bound is in LDS
    const uint32_t lo = *lo_w;
    const bool g = lo == 0u;  // the wait gave up: the WG writes no candidates
    uint32_t c = 0;
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) c += (s2 < nvw) & (kk[s2] >= lo) & !g;
    uint32_t total;
    uint32_t p = block_scan_total<BLOCK>(c, scan, total);
    if (tid == 0) {
        if (g) raise_flag(P.status, kFlagTimeout);
        fr->cnt[widx] = ((uint64_t)tag << 32) | (g ? kFusedGaveUp : total);
    }
    uint64_t* const region = P.stage + ((size_t)row * (size_t)P.NT + (size_t)widx) * (size_t)(256 * gpw);
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2) {
        if ((s2 < nvw) & (kk[s2] >= lo) & !g) {
            const uint32_t t = (uint32_t)(64 * group_of(s2) + lane);
            region[p++] = composite(kk[s2], t);
        }
    }
}

struct FusedFinSmem {
    alignas(16) uint32_t hist[kHistWords];
    alignas(16) uint64_t cand[kBufCap];
    uint64_t small[kSmall];
    uint32_t cnt[kFusedMaxT];  // the tile WGs' counts
    uint32_t pre[kFusedMaxT];  // their exclusive prefix
    uint32_t scan[kFinBlock / 64];
    uint32_t sel[4];
    uint32_t bad;
};

// The finishing WG of a row: everything the candidate kernel wrote is
// complete (the kernel before it on the stream), so it reads its counts,
// sample keys and regions directly.
__global__ void __launch_bounds__(kFinBlock) topk_indexer_finish_kernel(FusedParams P) {
    constexpr int BLOCK = kFinBlock;
    static_assert(BLOCK >= kFusedMaxT, "one count per thread");
    static_assert(4 * BLOCK >= kFusedSample, "four sample entries per thread");
    __shared__ FusedFinSmem sm;
    const int row = (int)blockIdx.x;
    const int tid = threadIdx.x;
    const int n = P.n, k = P.k;
    const int L = valid_length(P.lengths, row, n);
    int32_t* const out = P.out + (size_t)row * (size_t)k;
    if (L <= k) {  // every valid token is selected; pad with -1
        for (int i = tid; i < k; i += BLOCK) out[i] = i < L ? i : -1;
        return;
    }
    FusedRow* const fr = P.frs + row;
    const uint32_t epoch = fr->epoch;
    const uint32_t tag = make_tag(epoch);
    const int NT = P.NT, F = P.F;
    const int SN = P.ns * 64;  // sample entries
    const uint32_t R = 256u * (uint32_t)P.gpw;
    const uint64_t* const sp = P.samp + (size_t)row * (size_t)kFusedSample;
    uint64_t sv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = tid + u * BLOCK;
        sv[u] = j < SN ? sp[j] : 0ull;
    }
    bool bad = false;
    uint32_t lo = 1u;
    if (SN > 0) {
        const uint64_t bv = fr->bound;
        bad = (uint32_t)(bv >> 32) != tag;
        lo = bad ? 1u : (uint32_t)bv;
    }
    clear_words(sm.hist, kCopies * kStride, tid, BLOCK);
    if (tid == 0) sm.bad = 0u;
    if (tid < NT) {
        const uint64_t cv = fr->cnt[tid];
        uint32_t c = (uint32_t)cv;
        if ((uint32_t)(cv >> 32) != tag || c > R) {  // the tile WG gave up waiting for the bound
            bad = true;
            c = 0u;
        }
        sm.cnt[tid] = c;
    }
    uint32_t cs = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = tid + u * BLOCK;
        if (j < SN && (uint32_t)(sv[u] >> 32) != tag) bad = true;
        cs += (j < SN) & ((uint32_t)sv[u] >= lo);
    }
    if (bad) sm.bad = 1u;
    lds_sync();  // counts, cleared histogram
    // the sample's candidates first, in (thread, entry) order, counted into
    // the first round's window histogram as they are placed
    uint32_t* const hc = sm.hist + (tid % kCopies) * kStride;
    uint32_t nsc;
    uint32_t ps = block_scan_total<BLOCK>(cs, sm.scan, nsc);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = tid + u * BLOCK;
        const uint32_t key = (uint32_t)sv[u];
        if ((j < SN) & (key >= lo)) {
            const uint32_t t = (uint32_t)(((j >> 6) * F + F - 1) * 64 + (j & 63));
            if (ps < (uint32_t)kBufCap) {
                const uint64_t c = composite(key, t);
                sm.cand[ps] = c;
                atomicAdd(&hc[window_bin(c, lo)], 1u);
            }
            ++ps;
        }
    }
    // then the regions in WG order
    const uint32_t cmine = tid < NT ? sm.cnt[tid] : 0u;
    uint32_t X;
    const uint32_t pr = block_scan_total<BLOCK>(cmine, sm.scan, X);
    if (tid < NT) sm.pre[tid] = pr;
    lds_sync();
    const uint32_t C = nsc + X;
    const bool ok = sm.bad == 0u && C >= (uint32_t)k && C <= (uint32_t)kBufCap;
    if (__builtin_expect(ok, 1)) {
        // thread t takes entries [t E, t E + E) of the regions' sequence,
        // locating the first by a binary search over the prefixes and
        // walking from there
        const uint32_t E = (X + BLOCK - 1) / BLOCK;
        const uint32_t ib = (uint32_t)tid * E, ie = min(X, ib + E);
        if (ib < ie) {
            int a = 0, b = NT;  // the last region whose prefix is at most ib (it holds entry ib)
            while (b - a > 1) {
                const int mid = (a + b) >> 1;
                if (sm.pre[mid] <= ib) a = mid;
                else b = mid;
            }
            uint32_t j = ib - sm.pre[a];
            // addresses of eight entries first, then their loads together
            for (uint32_t i0 = ib; i0 < ie; i0 += 8u) {
                const uint64_t* ad[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    ad[u] = nullptr;
                    if (i0 + (uint32_t)u < ie) {
                        while (j >= sm.cnt[a]) {  // past region a: the next non-empty one
                            ++a;
                            j = 0;
                        }
                        ad[u] = P.stage + ((size_t)row * (size_t)NT + (size_t)a) * (size_t)R + j;
                        ++j;
                    }
                }
                uint64_t v8[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v8[u] = ad[u] ? *ad[u] : 0ull;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (ad[u]) {
                        sm.cand[nsc + i0 + (uint32_t)u] = v8[u];
                        atomicAdd(&hc[window_bin(v8[u], lo)], 1u);
                    }
                }
            }
        }
    }
    if (tid == 0) fr->epoch = epoch + 1u;
    lds_sync();
    if (__builtin_expect(ok, 1)) {
        select_buffer<BLOCK>(sm.cand, C, (uint32_t)k, 0u, lo, true, sm.hist, sm.small, sm.scan, sm.sel, out, nullptr,
                             k, P.status);
    } else {
        const float* const prow = P.logits + (size_t)row * (size_t)n;
        const int off = (int)(((uintptr_t)prow >> 2) & 3);
        const int nchunks = (off + L + 3) >> 2;
        select_by_passes<BLOCK, kBufCap>(reinterpret_cast<const char*>(prow - off), off, L, nchunks, k, out, nullptr,
                                         sm.cand, sm.hist, sm.small, sm.scan, sm.sel, P.status);
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
// sum l) and P.V on the matrix cores (A = 16 heads x 32 slots of P, as the
// sum of two bf16 terms, one product each; B = 32 slots x 16 dims of the
// gathered values, held transposed in LDS so
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
    __shared__ u32x4_t ps[NH * 8];            // P's high bf16 term: head row of 64 slots, chunk c in c ^ (head % 8)
    __shared__ u32x4_t pl[NH * 8];            // P's low bf16 term (P - high), same layout
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
            // P as two bf16 terms (each rounded to nearest even): hi, and lo
            // for the remainder p - hi (exact in float), so hi + lo is within
            // 2^-16 p of p; head row h, slot j
            auto bf16_rne = [](float x) {
                const uint32_t u = __float_as_uint(x);
                return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
            };
            const uint16_t ph = bf16_rne(p);
            const uint16_t plo = bf16_rne(p - __uint_as_float((uint32_t)ph << 16));
            const int pidx = (h * 8 + ((j >> 3) ^ (h % 8))) * 8 + (j & 7);
            reinterpret_cast<uint16_t*>(ps)[pidx] = ph;
            reinterpret_cast<uint16_t*>(pl)[pidx] = plo;
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
    // four waves; two 32-slot steps each, each step a matrix-core product
    // for P's low term and one for its high term into the same float sums
    for (int tile = wave; tile < HB * (D / 16); tile += kAttnBlock / 64) {
        const int hb = tile / (D / 16), db = tile % (D / 16);
        floatx4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ts = 0; ts < kAttnSlots / 32; ++ts) {
            const int c = ts * 4 + g;  // slots 8c .. 8c+7
            const int h = hb * 16 + m, dim = db * 16 + m;
            const bf16x8_t al = __builtin_bit_cast(bf16x8_t, pl[h * 8 + (c ^ (h % 8))]);
            const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, ps[h * 8 + (c ^ (h % 8))]);
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, vt[dim * 8 + (c ^ vsw(dim))]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, acc, 0, 0, 0);
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

// The sample's chunks per thread are a template parameter: 1 for the usual
// 1024-chunk sample of 1024-thread WGs (code for unused sample slots still
// costs issue cycles), else what the sample needs.
constexpr int split_spt(int block, int sample_chunks) {
    return sample_chunks <= block ? 1 : (sample_chunks <= 2 * block ? 2 : 4);
}

template <int B, int I, bool R>
void launch_split(dim3 grid, dim3 block, hipStream_t s, const KParams& p) {
    const int spt = split_spt(B, p.sample_chunks);
    if (p.keys) {
        if (spt == 1) hipLaunchKernelGGL((topk_split_kernel<B, I, R, true, 1>), grid, block, 0, s, p);
        else if (spt == 2) hipLaunchKernelGGL((topk_split_kernel<B, I, R, true, 2>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((topk_split_kernel<B, I, R, true, 4>), grid, block, 0, s, p);
    } else {
        if (spt == 1) hipLaunchKernelGGL((topk_split_kernel<B, I, R, false, 1>), grid, block, 0, s, p);
        else if (spt == 2) hipLaunchKernelGGL((topk_split_kernel<B, I, R, false, 2>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((topk_split_kernel<B, I, R, false, 4>), grid, block, 0, s, p);
    }
}

template <int B, int I, bool R>
int occupancy_split(int* nb, int block) {
    int a = 0, b = 0;
    const int r1 = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, topk_split_kernel<B, I, R, false, 4>, block, 0);
    const int r2 = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, topk_split_kernel<B, I, R, true, 4>, block, 0);
    *nb = a < b ? a : b;
    return r1 != 0 ? r1 : r2;
}

template <int B, int I, int D>
void launch_rows(dim3 grid, dim3 block, hipStream_t s, const KParams& p) {
    if (p.oout) hipLaunchKernelGGL((topk_rows_kernel<B, I, D, 2>), grid, block, 0, s, p);
    else if (p.keys) hipLaunchKernelGGL((topk_rows_kernel<B, I, D, 1>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((topk_rows_kernel<B, I, D, 0>), grid, block, 0, s, p);
}

template <int B, int I, int D>
int occupancy_rows(int* nb, int block) {
    int a = 0, b = 0, c = 0;
    const int r1 = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, topk_rows_kernel<B, I, D, 0>, block, 0);
    const int r2 = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, topk_rows_kernel<B, I, D, 1>, block, 0);
    const int r3 = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&c, topk_rows_kernel<B, I, D, 2>, block, 0);
    *nb = min(a, min(b, c));
    return r1 != 0 ? r1 : (r2 != 0 ? r2 : r3);
}

struct Variant {
    int block, items, resident;
    int rows_kernel;  // 1: one WG per row, 12-bit first digit (wgs_per_row must be 1)
    LaunchFn launch;
    OccFn occupancy;
};

#define TKS_SPLIT(B, I, R) {B, I, R ? 1 : 0, 0, &launch_split<B, I, R>, &occupancy_split<B, I, R>}
#define TKS_ROWS(B, I, D) {B, I, 0, 1, &launch_rows<B, I, D>, &occupancy_rows<B, I, D>}
const Variant kVariants[] = {
    TKS_SPLIT(512, 4, true),     // 0: 2048 logits per WG
    TKS_SPLIT(512, 8, true),     // 1: 4096
    TKS_SPLIT(512, 16, true),    // 2: 8192
    TKS_SPLIT(1024, 4, true),    // 3: 4096
    TKS_SPLIT(1024, 8, true),    // 4: 8192
    TKS_SPLIT(1024, 16, true),   // 5: 16384
    TKS_SPLIT(1024, 32, true),   // 6: 32768
    TKS_SPLIT(1024, 16, false),  // 7: streaming, 16384 per tile
    TKS_SPLIT(512, 16, false),   // 8: streaming, 8192 per tile
    TKS_ROWS(512, 16, 1),        // 9: one WG per row, 8192 per tile
    TKS_ROWS(1024, 16, 1),       // 10: one WG per row, 16384 per tile
};
#undef TKS_SPLIT
#undef TKS_ROWS
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));

struct DeviceInfo {
    int cus = 0;
    int resident[kNumVariants] = {};  // co-resident WGs per variant on the whole device
};

// Scratch of one (device, stream): the status word, then, for split
// launches with several WGs per row, one SplitRow per row (row r always at
// the same address, whatever the row count of a call) and the stage of
// candidate regions.  Zeroed when allocated; the kernels leave it as they
// found it (every count and entry they set is cleared by the row's last WG).
// Buffers replaced by larger ones are kept until the workspace is released,
// since captured graphs may still refer to them.
struct Workspace {
    void* base = nullptr;     // status word + SplitRow per row
    size_t bytes = 0;
    void* stage = nullptr;    // candidate regions
    size_t stage_bytes = 0;
    void* aux = nullptr;      // ordered output: recorded keys, merge buffers (no clearing needed)
    size_t aux_bytes = 0;
    void* lg = nullptr;       // indexer selection without a logits output: the logits
    size_t lg_bytes = 0;
    void* at = nullptr;       // attention over the selected positions: per-chunk partials
    size_t at_bytes = 0;
    void* fu = nullptr;       // indexer with the selection's first pass: FusedRow per row, then the sample keys
    size_t fu_bytes = 0;
    void* fst = nullptr;      // indexer with the selection's first pass: candidate regions
    size_t fst_bytes = 0;
    std::vector<void*> retired;
};

std::recursive_mutex g_mu;  // recursive: the indexer entry point holds it across its launches
std::map<int, DeviceInfo> g_dev;
std::map<std::pair<int, uintptr_t>, Workspace> g_ws;

constexpr size_t kStatusBytes = 256;
constexpr int32_t kMaxN = 1 << 30;  // longest row accepted (element offsets stay far from 32-bit limits)

// Fixed scratch of topk_select_no_alloc: the status word, a SplitRow for
// each of up to kScratchRows rows (row r always at the same address), then
// the stage of candidate regions.  One copy per device, for the life of the
// process.  Host code never passes `scratch` itself (on the host the name is
// only a stand-in): the device address comes from hipGetSymbolAddress, once
// per device, and is kept in g_scratch.
constexpr size_t kScratchBytes = (size_t)TOPK_SELECT_NO_ALLOC_SCRATCH_BYTES;
constexpr int kScratchRows = 256;
constexpr size_t kScratchStage = (kStatusBytes + (size_t)kScratchRows * sizeof(SplitRow) + 255u) / 256u * 256u;
static_assert(kScratchStage < kScratchBytes, "scratch too small for its row table");
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::map<int, void*> g_scratch;  // device -> device address of `scratch`

int device_info(int dev, DeviceInfo** out) {
    auto it = g_dev.find(dev);
    if (it == g_dev.end()) {
        DeviceInfo d;
        if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || d.cus <= 0)
            return TOPK_SELECT_ERROR_NO_DEVICE;
        for (int v = 0; v < kNumVariants; ++v) {
            int nb = 0;
            if (kVariants[v].occupancy(&nb, kVariants[v].block) != (int)hipSuccess) return TOPK_SELECT_ERROR_LAUNCH;
            d.resident[v] = (nb > 0 ? nb : 1) * d.cus;
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

struct Launch {
    int variant;
    int G;
    int chunks_per_wg;
    int region;         // entries per WG region (split kernel)
    int sample_chunks;  // split kernel
};

// Sample of a row for the split kernel's bound (chunks, a multiple of 16):
// 1024 chunks, 4096 for rows of 512K logits or more (the candidate count
// above the bound grows with sqrt(k n / sample)); at most what the variant's
// registers hold.
int sample_chunks_for(int64_t maxc, int block, int items) {
    const int want = maxc >= 131072 ? 4096 : 1024;
    // at most four sampled chunks per thread, two beside 32 logits per
    // thread (registers)
    const int most = items >= 32 ? 2 : 4;
    const int spt = kSampleMax / block > most ? most : kSampleMax / block;
    const int cap = spt * block;
    return want < cap ? want : cap;
}

// Check an explicit shape: resident variants must cover the row in G
// slices, the one-WG-per-row kernel takes G == 1, the split kernel at most
// min(block, kMaxSplit) WGs per row.
int check_shape(int64_t rows, int64_t maxc, int v, int G, Launch* L) {
    if (v < 0 || v >= kNumVariants || G < 1) return TOPK_SELECT_ERROR_INVALID_VALUE;
    const Variant& var = kVariants[v];
    const int64_t tile_chunks = (int64_t)var.block * (var.items / 4);
    int64_t cpw = (maxc + G - 1) / G;
    if (cpw < 1) cpw = 1;
    if (var.resident && cpw > tile_chunks) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (var.rows_kernel && G != 1) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (!var.rows_kernel && (G > kMaxSplit || G > var.block)) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (rows * (int64_t)G > 0x7FFFFFFFll) return TOPK_SELECT_ERROR_INVALID_VALUE;
    L->variant = v;
    L->G = G;
    L->chunks_per_wg = (int)cpw;
    const int64_t slice = 4 * cpw;
    L->region = (int)(slice < kBufCap ? slice : kBufCap);
    L->sample_chunks = sample_chunks_for(maxc, var.block, var.items);
    return TOPK_SELECT_SUCCESS;
}

// Default shape (measured on MI355X).  Few rows are spread over many WGs of
// about 2K-8K logits each (1024 threads once a row uses more than 16 WGs);
// a moderate number of rows over WGs of about 32K (fewer regions for each
// row's finishing WG to gather: 64 ragged rows of 131,072 take 19.5 us with
// 4 WGs per row against 31.9 with 8); many rows take the one-WG-per-row
// kernel; rows too long for resident slices stream.
int choose_shape(const DeviceInfo& d, int64_t rows, int64_t maxc, Launch* L) {
    auto tile_chunks = [](int v) { return (int64_t)kVariants[v].block * (kVariants[v].items / 4); };
    if (rows >= d.cus) return check_shape(rows, maxc, 9, 1, L);
    // Few rows: slices of up to 2048 chunks (8192 logits), at least 8 WGs
    // per row while slices stay >= 512 chunks.  The finishing WG's gather
    // grows with the number of regions, so fewer, longer slices beat many
    // short ones once a row has 8 or more.  Many rows: long slices.
    const bool few = rows * 8 <= d.cus;
    int64_t G = few ? (maxc + 2047) / 2048 : (maxc + 8191) / 8192;
    if (few) {
        const int64_t g8 = (maxc + 511) / 512;
        if (G < 8) G = g8 < 8 ? g8 : 8;
        if (G > 128) G = 128;
    }
    if (G > kMaxSplit) G = kMaxSplit;
    if (G < 1) G = 1;
    const int64_t per = (maxc + G - 1) / G;
    const int v512[] = {0, 1, 2}, v1024[] = {3, 4, 5, 6};
    if (G <= 16) {
        for (int v : v512)
            if (per <= tile_chunks(v)) return check_shape(rows, maxc, v, (int)G, L);
    }
    for (int v : v1024)
        if (per <= tile_chunks(v)) return check_shape(rows, maxc, v, (int)G, L);
    // rows too long for resident slices: streaming WGs
    G = kMaxSplit;
    const int64_t gmin = (maxc + tile_chunks(7) - 1) / tile_chunks(7);
    if (gmin < G) G = gmin < 1 ? 1 : gmin;
    return check_shape(rows, maxc, 7, (int)G, L);
}

int validate(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k, const int32_t* out) {
    if (rows < 0 || n < 1 || n > kMaxN || k < 1 || k > n) return TOPK_SELECT_ERROR_INVALID_VALUE;
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

__global__ void __launch_bounds__(256) topk_clear_kernel(uint4* p, size_t n16) {
    const size_t stride = (size_t)gridDim.x * 256u;
    for (size_t i = (size_t)blockIdx.x * 256u + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Streaming read of n16 16-byte words: WG b reads the contiguous span
// [b * per, (b + 1) * per), eight loads in flight per thread, folded into
// one word per thread; a word is stored only when the fold hits a value no
// input of interest produces, so the loads stay live and the kernel writes
// (almost) nothing.  Many short spans (128 WGs per CU) keep every channel
// busy to the end.
__global__ void __launch_bounds__(256) topk_stream_read_kernel(const uint4* __restrict__ p, size_t n16, size_t per,
                                                               uint32_t* sink) {
    size_t i = (size_t)blockIdx.x * per + threadIdx.x;
    const size_t end = min(n16, (size_t)(blockIdx.x + 1) * per);
    uint32_t acc = 0;
    for (; i + 7u * 256u < end; i += 8u * 256u) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = p[i + (size_t)u * 256u];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < end; i += 256u) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

bool capturing(hipStream_t stream);

// Device address of `scratch` on `dev` (the current device).  The first
// call on a device looks it up, clears the array with a kernel on `stream`
// and waits for it, so every later call on any stream finds it zeroed.
int scratch_address(int dev, hipStream_t stream, char** out) {
    auto it = g_scratch.find(dev);
    if (it == g_scratch.end()) {
        if (capturing(stream)) return TOPK_SELECT_ERROR_CAPTURE;
        void* ptr = nullptr;
        if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return TOPK_SELECT_ERROR_LAUNCH;
        }
        topk_clear_kernel<<<dim3(1024), dim3(256), 0, stream>>>(reinterpret_cast<uint4*>(ptr), kScratchBytes / 16u);
        if (hipGetLastError() != hipSuccess || hipStreamSynchronize(stream) != hipSuccess) return TOPK_SELECT_ERROR_LAUNCH;
        it = g_scratch.emplace(dev, ptr).first;
    }
    *out = reinterpret_cast<char*>(it->second);
    return TOPK_SELECT_SUCCESS;
}

// Is work being captured into a graph on `stream`?  Allocations and clears
// must not happen then: they would not be replayed, or would break the
// capture.
bool capturing(hipStream_t stream) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess) return false;
    return st != hipStreamCaptureStatusNone;
}

// Grow-only scratch buffer of a workspace: a larger need allocates a new
// buffer (cleared when `zero`) and retires the old one (kept until the
// workspace is released: enqueued work and captured graphs may use it).
int grow(Workspace& w, hipStream_t stream, void** ptr, size_t* bytes, size_t need, bool zero) {
    if (*bytes >= need) return TOPK_SELECT_SUCCESS;
    if (capturing(stream)) return TOPK_SELECT_ERROR_CAPTURE;
    void* p = nullptr;
    if (hipMalloc(&p, need) != hipSuccess) {
        (void)hipGetLastError();
        return TOPK_SELECT_ERROR_OUT_OF_MEMORY;
    }
    if (zero && hipMemsetAsync(p, 0, need, stream) != hipSuccess) {
        (void)hipFree(p);
        return TOPK_SELECT_ERROR_LAUNCH;
    }
    if (*ptr) w.retired.push_back(*ptr);
    *ptr = p;
    *bytes = need;
    return TOPK_SELECT_SUCCESS;
}

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
        bool ordered, float* vals, hipStream_t stream, const topk_select_plan_t* forced, bool no_alloc = false) {
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
    rc = forced ? check_shape(rows, maxc, forced->variant, forced->wgs_per_row, &L)
                : choose_shape(*d, rows, maxc, &L);
    if (rc != TOPK_SELECT_SUCCESS) return rc;
    const Variant& var = kVariants[L.variant];
    const bool split = !var.rows_kernel && L.G > 1;
    const size_t stage_bytes = split ? (size_t)rows * (size_t)L.G * (size_t)L.region * 8u : 0;
    char* base = nullptr;
    void* stage = nullptr;
    if (no_alloc) {
        if (ordered) return TOPK_SELECT_ERROR_INVALID_VALUE;
        if (split && (rows > kScratchRows || stage_bytes > kScratchBytes - kScratchStage))
            return TOPK_SELECT_ERROR_SCRATCH_LIMIT;
        rc = scratch_address(dev, stream, &base);
        if (rc != TOPK_SELECT_SUCCESS) return rc;
        stage = base + kScratchStage;
    }
    Workspace& w = g_ws[{dev, (uintptr_t)stream}];
    if (!no_alloc) {
        const size_t rows_bytes = split ? (size_t)rows * sizeof(SplitRow) : 0;
        rc = grow(w, stream, &w.base, &w.bytes, kStatusBytes + rows_bytes, true);
        if (rc != TOPK_SELECT_SUCCESS) return rc;
        if (split) {
            rc = grow(w, stream, &w.stage, &w.stage_bytes, stage_bytes, true);
            if (rc != TOPK_SELECT_SUCCESS) return rc;
        }
        base = reinterpret_cast<char*>(w.base);
        stage = w.stage;
    }
    SortShape sh{};
    size_t keys_bytes = 0;
    if (ordered) {
        sh = sort_shape(rows, k);
        keys_bytes = ((size_t)rows * (size_t)k * 4u + 255u) / 256u * 256u;
        const size_t run_bytes = (!sh.rank && sh.nruns > 1) ? 2u * (size_t)rows * (size_t)sh.kp * 8u : 0u;
        if ((int64_t)rows * sh.nruns > 0x7FFFFFFFll || (int64_t)rows * sh.rank_wgs > 0x7FFFFFFFll ||
            (int64_t)rows * (sh.kp / (kMergeBlock * kMergeItems)) > 0x7FFFFFFFll)
            return TOPK_SELECT_ERROR_INVALID_VALUE;
        rc = grow(w, stream, &w.aux, &w.aux_bytes, 2u * keys_bytes + run_bytes, false);
        if (rc != TOPK_SELECT_SUCCESS) return rc;
    }
    KParams P;
    P.logits = logits;
    P.lengths = lengths;
    // ordered output: the selection writes its indices and their keys to
    // scratch, the sort writes out_idx
    char* const aux = reinterpret_cast<char*>(w.aux);
    P.out = ordered ? reinterpret_cast<int32_t*>(aux + keys_bytes) : out;
    P.keys = ordered ? reinterpret_cast<uint32_t*>(aux) : nullptr;
    P.status = reinterpret_cast<uint32_t*>(base);
    P.rws = split ? reinterpret_cast<SplitRow*>(base + kStatusBytes) : nullptr;
    P.stage = split ? reinterpret_cast<uint64_t*>(stage) : nullptr;
    P.rows = rows;
    P.n = n;
    P.k = k;
    P.G = L.G;
    P.chunks_per_wg = L.chunks_per_wg;
    P.region = L.region;
    P.sample_chunks = L.sample_chunks;
    P.ahead = var.rows_kernel ? d->resident[L.variant] : 0;
    // ordered output from the one-WG-per-row kernel for k <= kOrdLds: its
    // WGs order their rows themselves (no sort kernel)
    const bool ordered_in_rows = ordered && var.rows_kernel && k <= kOrdLds;
    P.oout = ordered_in_rows ? out : nullptr;
    P.ovals = ordered_in_rows ? vals : nullptr;
    (void)hipGetLastError();
    var.launch(dim3((unsigned)(rows * L.G)), dim3((unsigned)var.block), stream, P);
    if (hipGetLastError() != hipSuccess) return TOPK_SELECT_ERROR_LAUNCH;
    if (!ordered || ordered_in_rows) return TOPK_SELECT_SUCCESS;

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
    if (rows < 0 || n < 1 || n > kMaxN || heads < 1 || heads > 64 || kstride < 0)
        return TOPK_SELECT_ERROR_INVALID_VALUE;
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

// Shape of the indexer with the selection's first pass: groups per wave as
// for the logits kernel; the sample stride F the smallest power of two from
// 2 that keeps the sample within 64 groups.  Taken when the tile WGs of a
// row stay within kFusedMaxT and the candidates a bound lets through (about
// k + 4 sqrt(k F) + 6 F, see the sample rank) fit the finishing WG's buffer
// with room to spare; else the logits kernel and topk_select run.
struct FusedShape {
    int gpw, F, ns, NS, NT;
    int64_t grid;
};

bool fused_shape(int cus, int32_t rows, int32_t n, int32_t k, FusedShape* f) {
    const int64_t ng = ((int64_t)n + 63) / 64;
    const int64_t resident_waves = (int64_t)cus * 2 * (kLogitBlock / 64);
    int64_t gpw = ((int64_t)rows * ng + resident_waves - 1) / resident_waves;
    gpw = gpw < 1 ? 1 : (gpw > 8 ? 8 : gpw);
    int64_t F = 2;
    while (ng / F > kFusedSample / 64) F *= 2;
    const int64_t ns = ng / F, nr = ng - ns, gw = (kLogitBlock / 64) * gpw;
    const int64_t NS = (ns + gw - 1) / gw, NT = (nr + gw - 1) / gw;
    if (NT < 1 || NT > kFusedMaxT) return false;
    const double est = (double)k + 4.0 * __builtin_sqrt((double)k * (double)F) + 6.0 * (double)F + 256.0;
    if (est > (double)kBufCap) return false;
    const int64_t grid = (int64_t)rows * (NS + NT);
    if (grid > 0x7FFFFFFFll) return false;
    f->gpw = (int)gpw;
    f->F = (int)F;
    f->ns = (int)ns;
    f->NS = (int)NS;
    f->NT = (int)NT;
    f->grid = grid;
    return true;
}

template <int D, int HB>
void launch_fused_t(unsigned grid, hipStream_t stream, const FusedParams& p) {
    topk_indexer_cand_kernel<D, HB><<<grid, kLogitBlock, 0, stream>>>(p);
}

int run_indexer(const uint16_t* q, const uint16_t* kc, const float* w, int32_t rows, int32_t n, int32_t heads,
                int32_t dim, int64_t kstride, const int32_t* lengths, int32_t k, int32_t* out_idx, float* logits,
                hipStream_t stream, bool fused) {
    int rc = validate_indexer(q, kc, w, rows, n, heads, dim, kstride, lengths, logits);
    if (rc != TOPK_SELECT_SUCCESS) return rc;
    if (k < 1 || k > n) return TOPK_SELECT_ERROR_INVALID_VALUE;
    if (rows == 0) return TOPK_SELECT_SUCCESS;
    if (!out_idx || ((uintptr_t)out_idx & 3)) return TOPK_SELECT_ERROR_INVALID_VALUE;
    const size_t ob = (size_t)rows * (size_t)k * 4u;
    if (overlaps(out_idx, ob, q, (size_t)rows * heads * dim * 2u) || overlaps(out_idx, ob, w, (size_t)rows * heads * 4u) ||
        overlaps(out_idx, ob, kc, ((kstride ? (size_t)(rows - 1) * (size_t)kstride : 0u) + (size_t)n * dim) * 2u) ||
        overlaps(out_idx, ob, logits, (size_t)rows * (size_t)n * 4u) || overlaps(out_idx, ob, lengths, (size_t)rows * 4u))
        return TOPK_SELECT_ERROR_INVALID_VALUE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TOPK_SELECT_ERROR_NO_DEVICE;
    std::lock_guard<std::recursive_mutex> lock(g_mu);  // held across both launches (scratch stays put)
    float* lg = logits;
    if (!lg) {
        Workspace& ws = g_ws[{dev, (uintptr_t)stream}];
        rc = grow(ws, stream, &ws.lg, &ws.lg_bytes, (size_t)rows * (size_t)n * 4u, false);
        if (rc != TOPK_SELECT_SUCCESS) return rc;
        lg = reinterpret_cast<float*>(ws.lg);
    }
    DeviceInfo* d = nullptr;
    rc = device_info(dev, &d);
    if (rc != TOPK_SELECT_SUCCESS) return rc;
    FusedShape fs;
    if (fused && fused_shape(d->cus, rows, n, k, &fs)) {
        Workspace& ws = g_ws[{dev, (uintptr_t)stream}];
        rc = grow(ws, stream, &ws.base, &ws.bytes, kStatusBytes, true);
        if (rc != TOPK_SELECT_SUCCESS) return rc;
        const size_t row_bytes = sizeof(FusedRow) + (size_t)kFusedSample * 8u;
        rc = grow(ws, stream, &ws.fu, &ws.fu_bytes, (size_t)rows * row_bytes, true);
        if (rc != TOPK_SELECT_SUCCESS) return rc;
        // regions sized for the rows of this call (read only up to the counts written in the same call)
        const size_t stage_bytes = (size_t)rows * (size_t)fs.NT * (size_t)(256 * fs.gpw) * 8u;
        rc = grow(ws, stream, &ws.fst, &ws.fst_bytes, stage_bytes, true);
        if (rc != TOPK_SELECT_SUCCESS) return rc;
        // the row table and the sample keys keep one fixed layout per
        // buffer: sized for the buffer's capacity, not this call's rows
        const size_t cap_rows = ws.fu_bytes / row_bytes;
        FusedParams p;
        p.q = q;
        p.kc = kc;
        p.w = w;
        p.lengths = lengths;
        p.logits = lg;
        p.out = out_idx;
        p.status = reinterpret_cast<uint32_t*>(ws.base);
        p.frs = reinterpret_cast<FusedRow*>(ws.fu);
        p.samp = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws.fu) + cap_rows * sizeof(FusedRow));
        p.stage = reinterpret_cast<uint64_t*>(ws.fst);
        p.kstride = kstride;
        p.rows = rows;
        p.n = n;
        p.H = heads;
        p.k = k;
        p.gpw = fs.gpw;
        p.F = fs.F;
        p.ns = fs.ns;
        p.NS = fs.NS;
        p.NT = fs.NT;
        const int hb = heads <= 16 ? 1 : (heads <= 32 ? 2 : 4);
        const unsigned g = (unsigned)fs.grid;
        (void)hipGetLastError();
        if (dim == 32) {
            if (hb == 1) launch_fused_t<32, 1>(g, stream, p);
            else if (hb == 2) launch_fused_t<32, 2>(g, stream, p);
            else launch_fused_t<32, 4>(g, stream, p);
        } else if (dim == 64) {
            if (hb == 1) launch_fused_t<64, 1>(g, stream, p);
            else if (hb == 2) launch_fused_t<64, 2>(g, stream, p);
            else launch_fused_t<64, 4>(g, stream, p);
        } else {
            if (hb == 1) launch_fused_t<128, 1>(g, stream, p);
            else if (hb == 2) launch_fused_t<128, 2>(g, stream, p);
            else launch_fused_t<128, 4>(g, stream, p);
        }
        if (hipGetLastError() != hipSuccess) return TOPK_SELECT_ERROR_LAUNCH;
        topk_indexer_finish_kernel<<<dim3((unsigned)rows), kFinBlock, 0, stream>>>(p);
        return hipGetLastError() == hipSuccess ? TOPK_SELECT_SUCCESS : TOPK_SELECT_ERROR_LAUNCH;
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
    int rc = grow(ws, stream, &ws.at, &ws.at_bytes, (size_t)rows * (size_t)S * heads * (dim + 2) * 4u, false);
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
                                (hipStream_t)stream, false);
    } catch (...) {
        return TOPK_SELECT_ERROR_LAUNCH;
    }
}

int topk_indexer_select_fused(const uint16_t* q, const uint16_t* kc, const float* w, int32_t rows, int32_t n,
                              int32_t heads, int32_t dim, int64_t kstride, const int32_t* lengths, int32_t k,
                              int32_t* out_idx, float* out_logits, topk_select_stream_t stream) {
    try {
        return tks::run_indexer(q, kc, w, rows, n, heads, dim, kstride, lengths, k, out_idx, out_logits,
                                (hipStream_t)stream, true);
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

int topk_select_no_alloc(const float* logits, int32_t rows, int32_t n, const int32_t* lengths, int32_t k,
                         int32_t* out_idx, topk_select_stream_t stream) {
    try {
        return tks::run(logits, rows, n, lengths, k, out_idx, false, nullptr, (hipStream_t)stream, nullptr, true);
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
        // Reads the status word at the start of `base` and clears it; after
        // a timeout (a WG gave up waiting for another, so counts or
        // candidates it did not see may have been written after the row was
        // finished) the whole coordination state is cleared instead.
        auto take = [](void* base, size_t bytes, std::initializer_list<std::pair<void*, size_t>> more,
                       uint32_t* v) -> bool {
            if (hipMemcpy(v, base, sizeof(*v), hipMemcpyDeviceToHost) != hipSuccess) return false;
            if (*v & tks::kFlagTimeout) {
                if (hipMemset(base, 0, bytes) != hipSuccess) return false;
                for (const auto& m : more)
                    if (m.first && hipMemset(m.first, 0, m.second) != hipSuccess) return false;
            } else if (*v) {
                const uint32_t zero = 0;
                if (hipMemcpy(base, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return false;
            }
            return true;
        };
        uint32_t v = 0, u = 0;
        auto it = tks::g_ws.find({dev, (uintptr_t)stream});
        if (it != tks::g_ws.end() && it->second.base) {
            tks::Workspace& w = it->second;
            if (!take(w.base, w.bytes, {{w.stage, w.stage_bytes}, {w.fu, w.fu_bytes}, {w.fst, w.fst_bytes}}, &u))
                return TOPK_SELECT_ERROR_LAUNCH;
            v |= u;
        }
        auto sc = tks::g_scratch.find(dev);
        if (sc != tks::g_scratch.end()) {
            if (!take(sc->second, tks::kScratchBytes, {}, &u)) return TOPK_SELECT_ERROR_LAUNCH;
            v |= u;
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
        int cur = 0;
        (void)hipGetDevice(&cur);
        for (auto& kv : tks::g_ws) {
            tks::Workspace& w = kv.second;
            std::vector<void*> bufs = w.retired;
            for (void* p : {w.base, w.stage, w.aux, w.lg, w.at, w.fu, w.fst})
                if (p) bufs.push_back(p);
            if (bufs.empty()) continue;
            (void)hipSetDevice(kv.first.first);
            if (hipDeviceSynchronize() != hipSuccess) rc = TOPK_SELECT_ERROR_LAUNCH;
            for (void* p : bufs)
                if (hipFree(p) != hipSuccess) rc = TOPK_SELECT_ERROR_LAUNCH;
        }
        (void)hipSetDevice(cur);
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
        case TOPK_SELECT_ERROR_CAPTURE:
            return "scratch would have to be allocated during graph capture (call once on the stream first)";
        case TOPK_SELECT_ERROR_SCRATCH_LIMIT:
            return "the input needs more scratch than the fixed array of topk_select_no_alloc (nothing was enqueued)";
        default: return "unknown status";
    }
}

int topk_select_version(void) { return TOPK_SELECT_VERSION; }

#ifdef TKS_TEST_HOOKS
// Test builds only (not part of the ABI): the bound on a wait for another
// workgroup, in ticks of the 100 MHz constant clock, on the current device
// (0: every wait gives up before its first poll).
int topk_select_test_set_spin_limit(uint64_t ticks) {
    return hipMemcpyToSymbol(HIP_SYMBOL(tks::g_spin_limit), &ticks, sizeof(ticks), 0, hipMemcpyHostToDevice) ==
                   hipSuccess
               ? TOPK_SELECT_SUCCESS
               : TOPK_SELECT_ERROR_LAUNCH;
}
#endif

int topk_stream_read(const void* p, size_t bytes, uint32_t* sink, topk_select_stream_t stream) {
    if (!p || !sink || ((uintptr_t)p & 15u) || (bytes & 15u) || bytes == 0) return TOPK_SELECT_ERROR_INVALID_VALUE;
    try {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return TOPK_SELECT_ERROR_NO_DEVICE;
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return TOPK_SELECT_ERROR_NO_DEVICE;
        const size_t n16 = bytes / 16u;
        size_t grid = (size_t)cus * 128u;  // spans of at least 256 words
        if (grid > (n16 + 255u) / 256u) grid = (n16 + 255u) / 256u;
        const size_t per = (n16 + grid - 1u) / grid;
        (void)hipGetLastError();
        tks::topk_stream_read_kernel<<<dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream>>>(
            reinterpret_cast<const uint4*>(p), n16, per, sink);
        return hipGetLastError() == hipSuccess ? TOPK_SELECT_SUCCESS : TOPK_SELECT_ERROR_LAUNCH;
    } catch (...) {
        return TOPK_SELECT_ERROR_LAUNCH;
    }
}

}  // extern "C"
