// layout.hip -- counts, offsets, token-order capacity drops and send rows.
//
// Method: aicassindra "gpu_moe_all_to_all", "Two collectives per layer"
// (per-destination counts ahead of the payload) and "Bucketing" (sort by
// destination, build the offset table, keep indices and counts on the
// device); "MoE All-to-All Dispatch and Ragged Routing", "Fixed Capacity vs.
// Ragged Routing" (per-sender-expert slots, overflow dropped); ai-from-
// scratch "19. All-to-all", "Why the router can ruin your day" (a dropped
// token skips that expert).
//
// The layout is a stable counting sort of the T*k assignments by expert id
// (experts sit on destinations in contiguous blocks, so this also groups by
// destination). Positions must be bit-exact, so every rank is derived in
// assignment order, never from the order in which atomics happen to land;
// LDS atomics only build counts, whose totals do not depend on order.
//
// The work is tiny in bytes and latency-bound (the pages make the same point
// about the counts exchange), so the design minimises kernel launches and
// block-wide round trips:
//  * T*k <= kSmallAssignments and E <= 512: one 1024-thread block does
//    everything. Each of its 16 waves owns a contiguous range of assignments and counts it
//    into its own LDS row (pass A); a prefix over the waves gives each
//    wave's first rank per expert, a block scan gives the offsets; then each
//    wave walks its range again in order (pass B), 64 assignments at a time:
//    lanes holding the same expert find each other with a bit-sliced match
//    (one ballot per bit of the id), the rank is the wave's running count
//    plus the popcount of matching lower lanes, and the lowest matching lane
//    advances the count.
//  * larger: layout_count_kernel writes one E-bin histogram per tile (at
//    most kMaxTiles tiles); layout_rank_kernel then gives every tile one
//    block that reads all the histograms from L2 (spread over its threads,
//    summed with LDS integer atomics), derives the totals, its tile's prefix
//    and the offsets itself, and ranks its tile with the same two passes
//    over 16 waves (8 when E > 512). Block 0 publishes counts and offsets.
#include "launch.hpp"
#include "layout_device.hpp"
#include "moe_ep.h"

#include <atomic>

namespace moe {

// Workspace of the allocation-free entry point: one E-wide int32 histogram
// per tile, for every legal size (at most kMaxTiles tiles of at most 1024
// experts, 512 KiB). Each GPU the library runs on holds its own copy until
// the process ends. In host code this name is only a handle: the array's
// device address comes from hipGetSymbolAddress, once per device.
constexpr int64_t kScratchInts = kMaxTiles * 1024;
static __device__ __align__(256) int32_t scratch[kScratchInts];
static_assert(sizeof(scratch) == MOE_LAYOUT_SCRATCH_BYTES, "the header states the array's size");

namespace {

constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / kWave;

__global__ __launch_bounds__(kSmallThreads) void layout_small_kernel(
    const int32_t *__restrict__ idx, int64_t TK, int32_t k, int32_t E, int32_t R,
    int32_t capacity, int nbits, int32_t *__restrict__ expert_demand,
    int32_t *__restrict__ expert_counts, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ dest_counts, int32_t *__restrict__ dest_offsets,
    int32_t *__restrict__ pos, int32_t *__restrict__ send_src)
{
    extern __shared__ int32_t sm[];
    layout_small_body<kSmallThreads>(idx, TK, k, E, R, capacity, nbits, expert_demand, expert_counts,
                                     expert_offsets, dest_counts, dest_offsets, pos, send_src, sm);
}

__global__ __launch_bounds__(kLayoutThreads) void layout_count_kernel(
    const int32_t *__restrict__ idx, int64_t TK, int64_t tile, int32_t E,
    int32_t *__restrict__ tile_hist)
{
    extern __shared__ int32_t hist[];
    for (int e = threadIdx.x; e < E; e += kLayoutThreads)
        hist[e] = 0;
    __syncthreads();
    const int64_t begin = (int64_t)blockIdx.x * tile;
    const int64_t end = min(TK, begin + tile);
    count_range(idx, begin, end, threadIdx.x, kLayoutThreads, E, hist);
    __syncthreads();
    int32_t *out = tile_hist + (int64_t)blockIdx.x * E;
    for (int e = threadIdx.x; e < E; e += kLayoutThreads)
        out[e] = hist[e];
}

template <int kRankThreads>
__global__ __launch_bounds__(kRankThreads) void layout_rank_kernel(
    const int32_t *__restrict__ idx, int64_t TK, int64_t tile, int32_t B, int32_t k, int32_t E,
    int32_t R, int32_t capacity, int nbits, const int32_t *__restrict__ tile_hist,
    int32_t *__restrict__ expert_demand, int32_t *__restrict__ expert_counts,
    int32_t *__restrict__ expert_offsets, int32_t *__restrict__ dest_counts,
    int32_t *__restrict__ dest_offsets, int32_t *__restrict__ pos,
    int32_t *__restrict__ send_src)
{
    constexpr int kRankWaves = kRankThreads / kWave;
    extern __shared__ int32_t sm[];
    int32_t *wh = sm;                    // [kRankWaves][E]
    int32_t *cnt = wh + kRankWaves * E;  // [E]
    int32_t *base = cnt + E;             // [E] first rank of each expert in this tile
    int32_t *eoff = base + E;            // [E + 1]
    __shared__ int32_t wave_total[kRankWaves];
    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int b = blockIdx.x;

    // totals and this tile's prefix, straight from the tile histograms.
    // Thread tid owns a column (one expert, or with E % 4 == 0 four
    // consecutive experts read as one 16-byte word) and tiles g, g + G,
    // g + 2G, ... (G = threads per column), with 16 loads in flight; at
    // fine_grained (E = 512, 128 tiles) that is every tile in one batch.
    // The G partial sums per expert meet in LDS through integer atomics.
    // Loads read a clamped tile and the sum drops what is past the last
    // one, so no load carries a condition.
    for (int e = tid; e < E; e += kRankThreads) {
        cnt[e] = 0;
        base[e] = 0;
    }
    for (int i = tid; i < kRankWaves * E; i += kRankThreads)
        wh[i] = 0;
    __syncthreads();
    constexpr int kHistBatch = 16;
    // threads per column: the fewest that still take every tile in one batch
    // (fewer threads adding into each LDS word), at most what the block holds
    const int per_batch = (B + kHistBatch - 1) / kHistBatch;
    if (E % 4 == 0) {
        typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
        const i32x4 *hist4 = reinterpret_cast<const i32x4 *>(tile_hist);
        const int EQ = E / 4;
        const int G = max(1, min(EQ <= kRankThreads ? kRankThreads / EQ : 1, per_batch));
        for (int col = tid; col < G * EQ; col += kRankThreads) {
            const int eq = col % EQ;
            const int g = col / EQ;
            i32x4 total = {0, 0, 0, 0}, before = {0, 0, 0, 0};
            for (int t0 = g; t0 < B; t0 += G * kHistBatch) {
                i32x4 h[kHistBatch];
#pragma unroll
                for (int q = 0; q < kHistBatch; ++q) {
                    const int t = t0 + q * G;
                    h[q] = hist4[(int64_t)(t < B ? t : B - 1) * EQ + eq];
                }
#pragma unroll
                for (int q = 0; q < kHistBatch; ++q) {
                    const int t = t0 + q * G;
                    const i32x4 v = t < B ? h[q] : i32x4{0, 0, 0, 0};
                    total += v;
                    before += t < b ? v : i32x4{0, 0, 0, 0};
                }
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                atomicAdd(&cnt[4 * eq + c], total[c]);
                atomicAdd(&base[4 * eq + c], before[c]);
            }
        }
    } else {
        const int G = max(1, min(E <= kRankThreads ? kRankThreads / E : 1, per_batch));
        for (int col = tid; col < G * E; col += kRankThreads) {
            const int e = col % E;
            const int g = col / E;
            int32_t total = 0, before = 0;
            for (int t0 = g; t0 < B; t0 += G * kHistBatch) {
                int32_t h[kHistBatch];
#pragma unroll
                for (int q = 0; q < kHistBatch; ++q) {
                    const int t = t0 + q * G;
                    h[q] = tile_hist[(int64_t)(t < B ? t : B - 1) * E + e];
                }
#pragma unroll
                for (int q = 0; q < kHistBatch; ++q) {
                    const int t = t0 + q * G;
                    total += t < B ? h[q] : 0;
                    before += t < b ? h[q] : 0;
                }
            }
            atomicAdd(&cnt[e], total);
            atomicAdd(&base[e], before);
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kRankThreads) {
        const int32_t total = cnt[e];
        const int32_t kept = (capacity < 0 || total < capacity) ? total : capacity;
        cnt[e] = kept;
        if (b == 0) {
            expert_demand[e] = total;
            expert_counts[e] = kept;
        }
    }
    __syncthreads();
    block_scan_counts<kRankThreads>(cnt, E, eoff, wave_total);
    const int64_t begin = (int64_t)b * tile;
    const int64_t end = min(TK, begin + tile);
    int64_t lo, hi;
    wave_span(begin, end, w, kRankWaves, lo, hi);
    count_range(idx, lo, hi, lane_id(), kWave, E, wh + w * E);  // pass A
    __syncthreads();
    if (b == 0)
        publish_offsets(eoff, E, R, expert_offsets, dest_counts, dest_offsets);
    for (int e = tid; e < E; e += kRankThreads) {
        int32_t run = base[e];
        for (int v = 0; v < kRankWaves; ++v) {
            const int32_t c = wh[v * E + e];
            wh[v * E + e] = run;
            run += c;
        }
    }
    __syncthreads();
    rank_range(idx, lo, hi, k, E, capacity, nbits, wh + w * E, eoff, pos, send_src);  // pass B
}

}  // namespace

LayoutPlan layout_plan(int64_t TK, int32_t E)
{
    LayoutPlan p;
    p.small = TK <= kSmallAssignments && E <= kSmallMaxExperts;
    if (p.small || TK == 0) {
        p.tile = 0;
        p.tiles = 0;
        return p;
    }
    int64_t tile = layout_min_tile(E);
    if ((TK + tile - 1) / tile > kMaxTiles) {
        const int64_t per = (TK + kMaxTiles - 1) / kMaxTiles;
        tile = (per + kLayoutThreads - 1) / kLayoutThreads * kLayoutThreads;
    }
    p.tile = tile;
    p.tiles = (TK + tile - 1) / tile;
    return p;
}

hipError_t launch_dispatch_layout(const int32_t *topk_idx, int64_t T, int32_t E, int32_t k,
                                  int32_t R, int32_t capacity, int32_t *expert_demand,
                                  int32_t *expert_counts, int32_t *expert_offsets,
                                  int32_t *dest_counts, int32_t *dest_offsets, int32_t *pos,
                                  int32_t *send_src, int32_t *tile_hist, hipStream_t stream)
{
    const int64_t TK = T * (int64_t)k;
    int nbits = 0;
    while ((1 << nbits) < E)
        ++nbits;
    const LayoutPlan plan = layout_plan(TK, E);
    if (plan.small) {
        const size_t lds = (size_t)(kSmallWaves * E + E + E + 1) * sizeof(int32_t);
        hipLaunchKernelGGL(layout_small_kernel, dim3(1), dim3(kSmallThreads), lds, stream,
                           topk_idx, TK, k, E, R, capacity, nbits, expert_demand, expert_counts,
                           expert_offsets, dest_counts, dest_offsets, pos, send_src);
        return hipGetLastError();
    }
    if (plan.tiles > 0) {
        hipLaunchKernelGGL(layout_count_kernel, dim3((unsigned)plan.tiles), dim3(kLayoutThreads),
                           E * sizeof(int32_t), stream, topk_idx, TK, plan.tile, E, tile_hist);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    // with no assignments a single block still writes the (zero) counts;
    // 16 waves per block when the LDS rows fit (E <= 512), else 8
    const dim3 grid((unsigned)(plan.tiles > 0 ? plan.tiles : 1));
    if (E <= kSmallMaxExperts) {
        constexpr int threads = 1024;
        const size_t lds = (size_t)((threads / kWave) * E + 3 * E + 1) * sizeof(int32_t);
        hipLaunchKernelGGL(layout_rank_kernel<threads>, grid, dim3(threads), lds, stream, topk_idx,
                           TK, plan.tile, (int32_t)plan.tiles, k, E, R, capacity, nbits, tile_hist,
                           expert_demand, expert_counts, expert_offsets, dest_counts, dest_offsets,
                           pos, send_src);
    } else {
        constexpr int threads = 512;
        const size_t lds = (size_t)((threads / kWave) * E + 3 * E + 1) * sizeof(int32_t);
        hipLaunchKernelGGL(layout_rank_kernel<threads>, grid, dim3(threads), lds, stream, topk_idx,
                           TK, plan.tile, (int32_t)plan.tiles, k, E, R, capacity, nbits, tile_hist,
                           expert_demand, expert_counts, expert_offsets, dest_counts, dest_offsets,
                           pos, send_src);
    }
    return hipGetLastError();
}

size_t layout_scratch_bytes() { return sizeof(scratch); }

hipError_t layout_scratch(int32_t **ptr)
{
    constexpr int kMaxDevices = 64;
    static std::atomic<int32_t *> by_device[kMaxDevices];
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return err;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    int32_t *p = by_device[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // first call on this device (with it current): two threads may both
        // ask, and both get the same address
        void *addr = nullptr;
        if ((err = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch))) != hipSuccess)
            return err;
        p = static_cast<int32_t *>(addr);
        by_device[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace moe
