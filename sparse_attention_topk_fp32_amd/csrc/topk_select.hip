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

// the kernels, in dependency order
#include "common.h"
#include "split_kernel.h"
#include "rows_kernel.h"
#include "sort_kernels.h"
#include "indexer.h"
#include "attention.h"

namespace tks {

// ----------------------------------------------------------------- host side

using LaunchFn = void (*)(dim3, dim3, hipStream_t, const KParams&);
using OccFn = int (*)(int*, int);

// The sample's chunks per thread are a template parameter: 1 for the usual
// 1024-chunk sample of 1024-thread WGs (code for unused sample slots still
// costs issue cycles), else what the sample needs.
constexpr int split_spt(int block, int sample_chunks) {
    return sample_chunks <= block ? 1 : (sample_chunks <= 2 * block ? 2 : 4);
}

// the split kernel's leading scalar arguments, from P
#define SPLIT_HEAD(p) (p).logits, (p).lengths, (p).rows, (p).n, (p).k, (p).G, (p).xcds, (p).chunks_per_wg, (p).sample_chunks

// (32 logits per thread hold at most two sampled chunks per thread: see
// sample_chunks_for; no variant with four is compiled for them)
template <int I>
constexpr int split_spt_max() { return I >= 32 ? 2 : 4; }

template <int B, int I, bool R>
void launch_split(dim3 grid, dim3 block, hipStream_t s, const KParams& p) {
    constexpr int SM = split_spt_max<I>();
    const int spt = split_spt(B, p.sample_chunks);
    if (p.keys) {
        if (spt == 1) hipLaunchKernelGGL((topk_split_kernel<B, I, R, true, 1>), grid, block, 0, s, SPLIT_HEAD(p), p);
        else if (spt == 2 || SM == 2) hipLaunchKernelGGL((topk_split_kernel<B, I, R, true, 2>), grid, block, 0, s, SPLIT_HEAD(p), p);
        else hipLaunchKernelGGL((topk_split_kernel<B, I, R, true, SM>), grid, block, 0, s, SPLIT_HEAD(p), p);
    } else {
        if (spt == 1) hipLaunchKernelGGL((topk_split_kernel<B, I, R, false, 1>), grid, block, 0, s, SPLIT_HEAD(p), p);
        else if (spt == 2 || SM == 2) hipLaunchKernelGGL((topk_split_kernel<B, I, R, false, 2>), grid, block, 0, s, SPLIT_HEAD(p), p);
        else hipLaunchKernelGGL((topk_split_kernel<B, I, R, false, SM>), grid, block, 0, s, SPLIT_HEAD(p), p);
    }
}

template <int B, int I, bool R>
int occupancy_split(int* nb, int block) {
    constexpr int SM = split_spt_max<I>();
    int a = 0, b = 0;
    const int r1 = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, topk_split_kernel<B, I, R, false, SM>, block, 0);
    const int r2 = (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, topk_split_kernel<B, I, R, true, SM>, block, 0);
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
    int xcds = 1;                     // XCDs (each with its own L2); blocks are dealt to them in turn
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
        if (hipDeviceGetAttribute(&d.xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || d.xcds < 1 ||
            d.cus % d.xcds != 0) {
            (void)hipGetLastError();
            d.xcds = 1;
        }
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
    // a row whose WGs share one XCD (at most one row per XCD, see run):
    // slices of 1024 chunks while that makes at most 32 WGs (131,072
    // logits: 512x8 with 32 WGs 10.19 us against 10.84 for 512x16 with 16)
    int g512 = 16;
    if (few && d.xcds > 1 && rows <= d.xcds) {
        const int64_t g1k = (maxc + 1023) / 1024;
        if (g1k > G && g1k <= 32) {
            G = g1k;
            g512 = 32;
        }
    }
    if (G > kMaxSplit) G = kMaxSplit;
    if (G < 1) G = 1;
    const int64_t per = (maxc + G - 1) / G;
    const int v512[] = {0, 1, 2}, v1024[] = {3, 4, 5, 6};
    if (G <= g512) {
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

// the sort and rank kernels' leading scalar arguments, from S
#define SORT_HEAD(S) (S).idx, (S).keys, (S).lengths, (S).logits, (S).n, (S).k, (S).nruns

void launch_sort(const SortShape& sh, int32_t rows, hipStream_t stream, const SortParams& p) {
    const dim3 grid((unsigned)((int64_t)rows * sh.nruns));
    if (sh.block == 256) topk_sort_kernel<256, 4><<<grid, 256, 0, stream>>>(SORT_HEAD(p), p);
    else if (sh.block == 512) topk_sort_kernel<512, 4><<<grid, 512, 0, stream>>>(SORT_HEAD(p), p);
    else if (sh.items == 1) topk_sort_kernel<1024, 1><<<grid, 1024, 0, stream>>>(SORT_HEAD(p), p);
    else if (sh.items == 2) topk_sort_kernel<1024, 2><<<grid, 1024, 0, stream>>>(SORT_HEAD(p), p);
    else if (sh.items == 4) topk_sort_kernel<1024, 4><<<grid, 1024, 0, stream>>>(SORT_HEAD(p), p);
    else topk_sort_kernel<1024, 8><<<grid, 1024, 0, stream>>>(SORT_HEAD(p), p);
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
    // at most one row per XCD: each row's WGs on an XCD of their own when
    // they fit its share of the resident WGs (measured: C1 -0.24 us, C2
    // -0.28; with 8 rows of 4 WGs per XCD, 64 ragged rows, +0.19)
    P.xcds = (split && d->xcds > 1 && rows <= d->xcds && L.G <= d->resident[L.variant] / d->xcds) ? d->xcds : 0;
    const int64_t blocks = P.xcds ? (int64_t)d->xcds * L.G : (int64_t)rows * L.G;
    if (blocks > 0x7FFFFFFFll) return TOPK_SELECT_ERROR_INVALID_VALUE;
    P.chunks_per_wg = L.chunks_per_wg;
    P.region = L.region;
    P.sample_chunks = L.sample_chunks;
    P.ahead = var.rows_kernel ? d->resident[L.variant] : 0;
    // ordered output for k <= kOrdLds: the WG that finishes a row orders it
    // itself (one-WG-per-row kernel: from LDS; split kernel: from the
    // recorded scratch), no second launch
    const bool ordered_in_rows = ordered && k <= kOrdLds;
    P.oout = ordered_in_rows ? out : nullptr;
    P.ovals = ordered_in_rows ? vals : nullptr;
    (void)hipGetLastError();
    var.launch(dim3((unsigned)blocks), dim3((unsigned)var.block), stream, P);
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
        topk_rank_kernel<<<dim3((unsigned)((int64_t)rows * sh.rank_wgs)), kRankBlock, 0, stream>>>(SORT_HEAD(S), S);
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
    topk_logits_kernel<D, HB><<<grid, kLogitBlock, 0, stream>>>(p.q, p.kc, p.lengths, p.kstride, p.n, p.H, p.gpw,
                                                                 p.tiles, p);
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
    // four (256 slots) or two (128 slots) sub-chunks per WG when that still
    // gives kAttnWideMinWgs WGs: a quarter or half of the partial outputs to
    // write and combine
    const int64_t S2 = (k + 2 * kAttnSlots - 1) / (2 * kAttnSlots);
    const int64_t S4 = (k + 4 * kAttnSlots - 1) / (4 * kAttnSlots);
    const int sub = (k > 3 * kAttnSlots && (int64_t)rows * S4 >= kAttnWideMinWgs)   ? 4
                    : (k > kAttnSlots && (int64_t)rows * S2 >= kAttnWideMinWgs) ? 2
                                                                                  : 1;
    const int64_t S = (k + sub * kAttnSlots - 1) / (sub * kAttnSlots);
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
    // the combine's chunks per batch: 32 for a small grid, 16 for a large one
    const bool few = (int64_t)rows * heads <= kAttnCombineFewMax;
#define TKS_COMBINE(D_)                                                                              \
    do {                                                                                           \
        if (few)                                                                                   \
            topk_attn_combine_kernel<D_, 32><<<g2, D_, 0, stream>>>(p.part, p.out, p.S, p.H, p);   \
        else                                                                                       \
            topk_attn_combine_kernel<D_, 16><<<g2, D_, 0, stream>>>(p.part, p.out, p.S, p.H, p);   \
    } while (0)
#define TKS_ATTN(D_, HB_)                                                                                  \
    do {                                                                                                   \
        if (sub == 4)                                                                                      \
            topk_attn_partial_kernel<D_, HB_, 4><<<g1, kAttnBlock, 0, stream>>>(p.idx, p.kc, p.vc, p.q, p.kvstride, \
                                                                                p.S, p.H, p.k, p.n, p);   \
        else if (sub == 2)                                                                                 \
            topk_attn_partial_kernel<D_, HB_, 2><<<g1, kAttnBlock, 0, stream>>>(p.idx, p.kc, p.vc, p.q, p.kvstride, \
                                                                                p.S, p.H, p.k, p.n, p);   \
        else                                                                                               \
            topk_attn_partial_kernel<D_, HB_, 1><<<g1, kAttnBlock, 0, stream>>>(p.idx, p.kc, p.vc, p.q, p.kvstride, \
                                                                                p.S, p.H, p.k, p.n, p);   \
    } while (0)
    if (dim == 32) {
        if (hb == 1) TKS_ATTN(32, 1); else if (hb == 2) TKS_ATTN(32, 2); else TKS_ATTN(32, 4);
        TKS_COMBINE(32);
    } else if (dim == 64) {
        if (hb == 1) TKS_ATTN(64, 1); else if (hb == 2) TKS_ATTN(64, 2); else TKS_ATTN(64, 4);
        TKS_COMBINE(64);
    } else {
        if (hb == 1) TKS_ATTN(128, 1); else if (hb == 2) TKS_ATTN(128, 2); else TKS_ATTN(128, 4);
        TKS_COMBINE(128);
    }
#undef TKS_ATTN
#undef TKS_COMBINE
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
