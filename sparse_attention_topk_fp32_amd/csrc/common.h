// common.h - constants, launch parameters, device helpers (key map, scans, digit
// histograms and their selects) and the on-chip exact selection shared by
// every selection kernel.
// Part of the topk_select library: included once, in order, by topk_select.hip.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
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
    int32_t xcds;           // split kernel: > 1 groups each row's WGs on one XCD (block b runs on XCD b mod xcds)
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

// ----------------------------------------------------------------- ordered form

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
constexpr int kOrdLds = 2048;  // k up to this: the selecting WG orders its row itself
template <int BLOCK, int MAXC, int CAP, bool RUNS = false>
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
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, kor = 0u, kand = 0xFFFFFFFFu;
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
            if (RUNS) {
                kor |= key;
                kand &= key;
            }
        }
    }
    for (int sft = 32; sft >= 1; sft >>= 1) {
        kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, sft));
        kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, sft));
        if (RUNS) {
            kor |= (uint32_t)__shfl_xor((int)kor, sft);
            kand &= (uint32_t)__shfl_xor((int)kand, sft);
        }
    }
    uint32_t* const red = cur;  // the cursors are written only after this is read
    if (lane_id() == 0) {
        red[wid] = kmin;
        red[NW + wid] = kmax;
        if (RUNS) {
            red[2 * NW + wid] = kor;
            red[3 * NW + wid] = kand;
        }
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        kmin = min(kmin, red[w]);
        kmax = max(kmax, red[NW + w]);
        if (RUNS) {
            kor |= red[2 * NW + w];
            kand &= red[3 * NW + w];
        }
    }
    const uint32_t range = kmax - kmin;  // cnt >= 1
    const uint32_t q = range ? 32u - (uint32_t)__builtin_clz(range) : 0u;
    const uint32_t sh0 = q > BITS ? q - BITS : 0u;
    // RUNS: keys that all share their low tz bits (logits of a coarser type,
    // such as bfloat16 values) lie at least 2^tz apart, so each distinct key owns
    // a run of bins: then bins are one bit wider and a key's entries spread
    // over its run by index (lower index, higher bin), 2^lsb bins per key at
    // most; bin order stays the composites' order, and runs of equal keys no
    // longer crowd one bin.
    const uint32_t dif = kor ^ kand;
    const uint32_t tz = dif ? (uint32_t)__builtin_ctz(dif) : 32u;
    const bool runs = RUNS && tz > sh0 + 1u;
    const uint32_t sh = runs ? sh0 + 1u : sh0;
    const uint32_t lsb = runs ? min(tz - sh, 10u) : 0u;
    const uint32_t smax = (1u << lsb) - 1u;
    const uint32_t lb = L > 1u ? 32u - (uint32_t)__builtin_clz(L - 1u) : 0u;  // every index < 2^lb
    const uint32_t ish = lb > lsb ? lb - lsb : 0u;
    auto bin_of = [&](uint64_t c) -> uint32_t {
        return (((uint32_t)(c >> 32) - kmin) >> sh) + smax - min(smax, (~(uint32_t)c) >> ish);
    };
    uint32_t bv[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        bv[u] = bin_of(e[u]);
        if ((uint32_t)(tid + u * BLOCK) < cnt) atomicAdd(&hist[bv[u]], 1u);
    }
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
            T[atomicAdd(&cur[bv[u]], 1u)] = e[u];
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
        const uint32_t b = bin_of(c);
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

}  // namespace tks
