// indexer.h - the indexer that feeds the selector: logits on the matrix cores, and
// the form with the selection's first pass inside it.
// Part of the topk_select library: included once, in order, by topk_select.hip.

#pragma once

#include "common.h"

namespace tks {

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
// The arguments that the first loads depend on come first, one by one (the
// dispatcher places them in scalar registers as the waves start: kernel-
// argument preloading); they stand in for the parameter block's copies.
__global__ void __launch_bounds__(kLogitBlock) topk_logits_kernel(const uint16_t* q_, const uint16_t* kc_,
                                                                 const int32_t* lengths_, int64_t kstride_, int32_t n_,
                                                                 int32_t H_, int32_t gpw_, int32_t tiles_,
                                                                 const LogitParams P0) {
    LogitParams P = P0;
    P.q = q_, P.kc = kc_, P.lengths = lengths_, P.kstride = kstride_, P.n = n_, P.H = H_, P.gpw = gpw_, P.tiles = tiles_;
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

}  // namespace tks
