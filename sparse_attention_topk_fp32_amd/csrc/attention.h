// attention.h - attention over the selected positions on the matrix cores.
// Part of the topk_select library: included once, in order, by topk_select.hip.

#pragma once

#include "indexer.h"

namespace tks {

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
constexpr int kAttnSlots = 64;   // slots per sub-chunk (one or two per WG)
constexpr int kAttnWideMinWgs = 512;  // WGs of 2 (or 4) sub-chunks from which a launch takes them

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

template <int D, int HB, int SUB>
// The arguments that the first loads depend on come first, one by one (the
// dispatcher places them in scalar registers as the waves start: kernel-
// argument preloading); they stand in for the parameter block's copies.
// SUB sub-chunks of 64 slots per WG: all of their positions, keys and
// values are loaded at once; the scores of each sub-chunk are taken in turn
// from the one key tile in LDS, the softmax runs over all of the WG's slots,
// and P.V adds up the sub-chunks in turn into the same sums (no rescaling).
// SUB = 2 halves the partial outputs a row writes and the combine reads,
// SUB = 4 quarters them.
__global__ void __launch_bounds__(kAttnBlock) topk_attn_partial_kernel(const int32_t* idx_, const uint16_t* kc_,
                                                                       const uint16_t* vc_, const uint16_t* q_,
                                                                       int64_t kvstride_, int32_t S_, int32_t H_, int32_t k_,
                                                                       int32_t n_, const AttnParams P0) {
    AttnParams P = P0;
    P.idx = idx_, P.kc = kc_, P.vc = vc_, P.q = q_, P.kvstride = kvstride_, P.S = S_, P.H = H_, P.k = k_, P.n = n_;
    static_assert(SUB == 1 || SUB == 2 || SUB == 4, "sub-chunks per WG");
    constexpr int KB = D / 32;     // 32-dim steps of a score
    constexpr int CPR = D / 8;     // 16-byte chunks per key / value row
    constexpr int NH = HB * 16;    // padded heads
    constexpr int TILES = HB * (D / 16);                        // P.V output tiles of 16 heads x 16 dims
    constexpr int NT = (TILES + kAttnBlock / 64 - 1) / (kAttnBlock / 64);  // tiles per wave
    __shared__ u32x4_t qs[NH * CPR];          // queries, chunk c of head h in slot c ^ (h % CPR)
    __shared__ u32x4_t ks[kAttnSlots * CPR];  // gathered keys, same swizzle by slot
    __shared__ u32x4_t vt[D * 8];             // values transposed: dim row of 64 slots, chunk c in c ^ vsw(dim)
    __shared__ u32x4_t ps[SUB][NH * 8];       // P's high bf16 term: head row of 64 slots, chunk c in c ^ (head % 8)
    __shared__ u32x4_t pl[SUB][NH * 8];       // P's low bf16 term (P - high), same layout
    __shared__ float red[2][kAttnBlock / 64][NH];
    const int row = blockIdx.x / P.S;
    const int sp = blockIdx.x - row * P.S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int n = P.n, H = P.H, k = P.k;
    const int s0 = sp * (kAttnSlots * SUB);
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
    int toks[SUB][PIECES];
#pragma unroll
    for (int t = 0; t < SUB; ++t)
#pragma unroll
        for (int u = 0; u < PIECES; ++u) {
            const int sl = s0 + t * kAttnSlots + (tid + u * kAttnBlock) / CPR;
            const int tk = sl < k ? irow[sl] : -1;
            toks[t][u] = (tk >= 0 && tk < n) ? tk : 0;
        }
    u32x4_t kr[SUB][PIECES], vr[SUB][PIECES];
#pragma unroll
    for (int t = 0; t < SUB; ++t)
#pragma unroll
        for (int u = 0; u < PIECES; ++u) {
            const int c = (tid + u * kAttnBlock) % CPR;
            const size_t off = (size_t)toks[t][u] * D * 2 + (size_t)c * 16;
            kr[t][u] = *reinterpret_cast<const u32x4_t*>(K + off);
            vr[t][u] = *reinterpret_cast<const u32x4_t*>(V + off);
        }
    uint16_t* const vt16 = reinterpret_cast<uint16_t*>(vt);
    auto put_keys = [&](const u32x4_t (&r)[PIECES]) {
#pragma unroll
        for (int u = 0; u < PIECES; ++u) {
            const int i = tid + u * kAttnBlock;
            const int j = i / CPR, c = i % CPR;
            ks[j * CPR + (c ^ (j % CPR))] = r[u];
        }
    };
    auto put_values = [&](const u32x4_t (&r)[PIECES]) {
#pragma unroll
        for (int u = 0; u < PIECES; ++u) {
            const int i = tid + u * kAttnBlock;
            const int j = i / CPR, c = i % CPR;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int dim = c * 8 + e;
                const uint32_t w = r[u][e >> 1];
                vt16[(dim * 8 + ((j >> 3) ^ vsw(dim))) * 8 + (j & 7)] = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
            }
        }
    };
    put_values(vr[0]);
    // scores: lane holds heads 4g+i (+16 hb) of slot 16 wave + m of each sub-chunk
    const int j = wave * 16 + m;
    float sc[SUB][HB][4];
    bool valid[SUB];
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
        if (t > 0) __syncthreads();  // the previous sub-chunk's scores have read the key tile
        put_keys(kr[t]);
        __syncthreads();
        const int sl = s0 + t * kAttnSlots + j;
        const int tj = sl < k ? irow[sl] : -1;
        valid[t] = tj >= 0 && tj < n;
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
            for (int i = 0; i < 4; ++i) sc[t][hb][i] = valid[t] ? acc[i] * P.scale : -__builtin_huge_valf();
        }
    }
    // softmax over the WG's slots, per head: the maximum and the sum, over
    // the sub-chunks, the 16 lanes of a head group, then the 4 waves
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x = sc[0][hb][i];
#pragma unroll
            for (int t = 1; t < SUB; ++t) x = fmaxf(x, sc[t][hb][i]);
#pragma unroll
            for (int sft = 1; sft < 16; sft <<= 1) x = fmaxf(x, __shfl_xor(x, sft));
            if (m == 0) red[0][wave][hb * 16 + 4 * g + i] = x;
        }
    __syncthreads();
    // P as two bf16 terms (each rounded to nearest even): hi, and lo for the
    // remainder p - hi (exact in float), so hi + lo is within 2^-16 p of p
    auto bf16_rne = [](float x) {
        const uint32_t u = __float_as_uint(x);
        return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
    };
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = hb * 16 + 4 * g + i;
            float M = red[0][0][h];
#pragma unroll
            for (int w = 1; w < kAttnBlock / 64; ++w) M = fmaxf(M, red[0][w][h]);
            float x = 0.0f;
#pragma unroll
            for (int t = 0; t < SUB; ++t) {
                const float p = valid[t] ? __expf(sc[t][hb][i] - M) : 0.0f;  // M is finite when a slot is valid
                x += p;
                const uint16_t ph = bf16_rne(p);
                const uint16_t plo = bf16_rne(p - __uint_as_float((uint32_t)ph << 16));
                const int pidx = (h * 8 + ((j >> 3) ^ (h % 8))) * 8 + (j & 7);  // head row h, slot j
                reinterpret_cast<uint16_t*>(ps[t])[pidx] = ph;
                reinterpret_cast<uint16_t*>(pl[t])[pidx] = plo;
            }
#pragma unroll
            for (int sft = 1; sft < 16; sft <<= 1) x += __shfl_xor(x, sft);
            if (m == 0) red[1][wave][h] = x;
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
    // P.V: output tiles of 16 heads x 16 dims, TILES of them over the four
    // waves; per sub-chunk two 32-slot steps each, each step a matrix-core
    // product for P's low term and one for its high term into the same
    // float sums
    floatx4_t acc[NT];
#pragma unroll
    for (int it = 0; it < NT; ++it) acc[it] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
        if (t > 0) {
            __syncthreads();  // the previous sub-chunk's products have read the value tile
            put_values(vr[t]);
            __syncthreads();
        }
#pragma unroll
        for (int it = 0; it < NT; ++it) {
            const int tile = wave + it * (kAttnBlock / 64);
            if (TILES % (kAttnBlock / 64) != 0 && tile >= TILES) break;
            const int hb = tile / (D / 16), db = tile % (D / 16);
#pragma unroll
            for (int ts = 0; ts < kAttnSlots / 32; ++ts) {
                const int c = ts * 4 + g;  // slots 8c .. 8c+7
                const int h = hb * 16 + m, dim = db * 16 + m;
                const bf16x8_t al = __builtin_bit_cast(bf16x8_t, pl[t][h * 8 + (c ^ (h % 8))]);
                const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, ps[t][h * 8 + (c ^ (h % 8))]);
                const bf16x8_t b = __builtin_bit_cast(bf16x8_t, vt[dim * 8 + (c ^ vsw(dim))]);
                acc[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, acc[it], 0, 0, 0);
                acc[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, acc[it], 0, 0, 0);
            }
        }
    }
    // lane holds heads 4g+i of dim db*16 + m
#pragma unroll
    for (int it = 0; it < NT; ++it) {
        const int tile = wave + it * (kAttnBlock / 64);
        if (TILES % (kAttnBlock / 64) != 0 && tile >= TILES) break;
        const int hb = tile / (D / 16), db = tile % (D / 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = hb * 16 + 4 * g + i;
            if (h < H) prow[(size_t)h * (D + 2) + db * 16 + m] = acc[it][i];
        }
    }
}

// Combine a row's chunks: out = sum_s e^(m_s - M) O_s / sum_s e^(m_s - M) l_s
// with M the largest m_s over the chunks holding a position; zeros when no
// slot of the row holds one.  One WG of D threads per (row, head), thread c
// owning dim c.  The chunks go in batches of SB: a batch's SB partial
// outputs of dim c and, in lane s of every wave, chunk s's (m, l) are all
// loaded at once (one memory round trip per batch), M and the denominator
// are reduced within each wave by shuffles, and lane s's factor is read by
// every lane with a lane read, so no LDS or barrier is used.  Across
// batches the sums are rescaled to the running maximum.  SB chunks per
// batch: 32 (one batch for k <= 2048) when the grid is small and each WG's
// latency is the time; 16 for many (row, head) pairs, where the
// fewer loads in flight per thread measured faster.
constexpr int kAttnCombineFewMax = 256;  // (row, head) pairs up to which SB = 32
template <int D, int SB>
__global__ void __launch_bounds__(D) topk_attn_combine_kernel(float* part_, float* out_, int32_t S_, int32_t H_,
                                                              const AttnParams P0) {
    AttnParams P = P0;  // the leading arguments are preloaded, as for the partial kernel
    P.part = part_, P.out = out_, P.S = S_, P.H = H_;
    static_assert(SB == 16 || SB == 32, "chunks per batch");
    constexpr int RW = D < 64 ? D : 64;  // lanes of a wave in the reductions (lanes past the batch hold nothing)
    const int rh = blockIdx.x;  // row * H + head
    const int row = rh / P.H, h = rh - row * P.H;
    const int c = threadIdx.x, cs = c & 63;
    const float* const base = P.part + (size_t)row * P.S * (size_t)P.H * (D + 2) + (size_t)h * (D + 2);
    const size_t stride = (size_t)P.H * (D + 2);
    const float ninf = -__builtin_huge_valf();
    float Mrun = ninf, num = 0.0f, den = 0.0f;
    for (int s0 = 0; s0 < P.S; s0 += SB) {
        const int cnt = min(P.S - s0, SB);
        const float* const b0 = base + (size_t)s0 * stride;
        float o[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u) o[u] = u < cnt ? b0[u * stride + c] : 0.0f;
        float m = ninf, l = 0.0f;
        if (cs < cnt) {
            const float2 ml = *reinterpret_cast<const float2*>(b0 + cs * stride + D);
            m = ml.x, l = ml.y;
        }
        float mb = l > 0.0f ? m : ninf;
#pragma unroll
        for (int sft = RW / 2; sft >= 1; sft >>= 1) mb = fmaxf(mb, __shfl_xor(mb, sft));
        const float Mnew = fmaxf(Mrun, mb);
        const float f = l > 0.0f ? __expf(m - Mnew) : 0.0f;
        float dl = f * l;
#pragma unroll
        for (int sft = RW / 2; sft >= 1; sft >>= 1) dl += __shfl_xor(dl, sft);
        const float r = Mrun == ninf ? 0.0f : __expf(Mrun - Mnew);
        num *= r;
        den = den * r + dl;
#pragma unroll
        for (int u = 0; u < SB; ++u)
            num += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), u)) * o[u];
        Mrun = Mnew;
    }
    P.out[(size_t)rh * D + c] = den > 0.0f ? num / den : 0.0f;
}

}  // namespace tks
