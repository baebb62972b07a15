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
// token order, never from the order in which atomics happen to land:
//
//   1. layout_count_kernel: one block per tile of kLayoutTile assignments
//      builds an E-bin LDS histogram (integer atomics: the totals do not
//      depend on their order) and writes it to the workspace.
//   2. layout_scan_kernel: one block per 64 experts turns the per-tile
//      histograms into exclusive prefixes over tiles (in place) and writes
//      demand and kept counts.
//   3. layout_rank_kernel: each block rebuilds the expert offsets with an
//      LDS scan over E (block 0 publishes them with the destination counts),
//      then ranks its tile. Each wave owns 512 consecutive assignments and
//      walks them 64 at a time; lanes holding the same expert find each
//      other with a bit-sliced match (one ballot per bit of the id), so the
//      rank inside a step is a popcount of the lanes below, and the lowest
//      such lane bumps the wave's LDS counter. A per-expert prefix over the
//      4 waves plus the tile's prefix from step 2 gives the global rank.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kScanWaves = 16;
constexpr int kRankWaves = kLayoutThreads / kWave;
constexpr int kWaveSpan = kLayoutTile / kRankWaves;
constexpr int kSteps = kWaveSpan / kWave;

__global__ __launch_bounds__(kLayoutThreads) void layout_count_kernel(
    const int32_t *__restrict__ idx, int64_t TK, int32_t E, int32_t *__restrict__ tile_hist)
{
    extern __shared__ int32_t hist[];
    for (int e = threadIdx.x; e < E; e += kLayoutThreads)
        hist[e] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kLayoutTile;
#pragma unroll
    for (int i = 0; i < kLayoutPerThread; ++i) {
        const int64_t a = base + i * kLayoutThreads + threadIdx.x;
        if (a < TK) {
            const int32_t e = idx[a];
            if ((uint32_t)e < (uint32_t)E)
                atomicAdd(&hist[e], 1);
        }
    }
    __syncthreads();
    int32_t *out = tile_hist + (int64_t)blockIdx.x * E;
    for (int e = threadIdx.x; e < E; e += kLayoutThreads)
        out[e] = hist[e];
}

__global__ __launch_bounds__(kScanWaves *kWave) void layout_scan_kernel(
    int32_t *__restrict__ tile_hist, int64_t B, int32_t E, int32_t capacity,
    int32_t *__restrict__ demand, int32_t *__restrict__ counts)
{
    __shared__ int32_t part[kScanWaves][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int32_t e = blockIdx.x * kWave + lane;
    const bool ok = e < E;
    // wave w owns tiles [b0, b1); the last wave's range always ends at B
    const int64_t per = (B + kScanWaves - 1) / kScanWaves;
    const int64_t b0 = min(B, (int64_t)w * per);
    const int64_t b1 = min(B, b0 + per);
    int32_t s = 0;
    if (ok)
        for (int64_t b = b0; b < b1; ++b)
            s += tile_hist[b * E + e];
    part[w][lane] = s;
    __syncthreads();
    int32_t run = 0;
    for (int v = 0; v < w; ++v)
        run += part[v][lane];
    if (ok) {
        for (int64_t b = b0; b < b1; ++b) {
            const int32_t c = tile_hist[b * E + e];
            tile_hist[b * E + e] = run;
            run += c;
        }
        if (w == kScanWaves - 1) {
            demand[e] = run;
            counts[e] = (capacity < 0 || run < capacity) ? run : capacity;
        }
    }
}

__global__ __launch_bounds__(kLayoutThreads) void layout_rank_kernel(
    const int32_t *__restrict__ idx, int64_t TK, int64_t B, int32_t k, int32_t E, int32_t R,
    int32_t capacity, int nbits, const int32_t *__restrict__ tile_base,
    const int32_t *__restrict__ counts, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ dest_counts, int32_t *__restrict__ dest_offsets,
    int32_t *__restrict__ pos, int32_t *__restrict__ send_src)
{
    extern __shared__ int32_t sm[];
    int32_t *eoff = sm;            // [E + 1] expert offsets
    int32_t *base = eoff + E + 1;  // [E] first rank of each expert in this tile
    int32_t *wh = base + E;        // [kRankWaves][E] per-wave counts, then first ranks
    __shared__ int32_t wave_total[kRankWaves];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;

    // (1) exclusive scan of the kept counts over experts, 4 experts per thread
    int32_t c4[4];
    int32_t mine = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = tid * 4 + q;
        c4[q] = e < E ? counts[e] : 0;
        mine += c4[q];
    }
    const int32_t inc = wave_inclusive_sum(mine);
    if (lane == kWave - 1)
        wave_total[w] = inc;
    for (int e = tid; e < E; e += kLayoutThreads)
        base[e] = blockIdx.x < B ? tile_base[(int64_t)blockIdx.x * E + e] : 0;
    for (int i = tid; i < kRankWaves * E; i += kLayoutThreads)
        wh[i] = 0;
    __syncthreads();
    int32_t ex = inc - mine;
    int32_t total = 0;
#pragma unroll
    for (int v = 0; v < kRankWaves; ++v) {
        ex += v < w ? wave_total[v] : 0;
        total += wave_total[v];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = tid * 4 + q;
        if (e < E)
            eoff[e] = ex;
        ex += c4[q];
    }
    if (tid == 0)
        eoff[E] = total;
    __syncthreads();

    // (2) block 0 publishes the offset table and the destination counts
    if (blockIdx.x == 0) {
        for (int e = tid; e <= E; e += kLayoutThreads)
            expert_offsets[e] = eoff[e];
        const int32_t el = E / R;
        for (int r = tid; r < R; r += kLayoutThreads) {
            dest_offsets[r] = eoff[r * el];
            dest_counts[r] = eoff[(r + 1) * el] - eoff[r * el];
        }
        if (tid == 0)
            dest_offsets[R] = eoff[E];
    }

    // (3) stable ranks inside each wave's span, in assignment order
    const int64_t a0 = (int64_t)blockIdx.x * kLayoutTile + (int64_t)w * kWaveSpan;
    int32_t ev[kSteps];
    int32_t rk[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int64_t a = a0 + s * kWave + lane;
        ev[s] = a < TK ? idx[a] : -1;
    }
    int32_t *my_wh = wh + w * E;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int32_t e = ev[s];
        const bool valid = (uint32_t)e < (uint32_t)E;
        uint64_t same = ballot64(valid);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t ones = ballot64(bit);
            same &= bit ? ones : ~ones;
        }
        const int32_t below = (int32_t)count_below(same);
        const int32_t seen = valid ? my_wh[e] : 0;
        if (valid && below == 0)
            my_wh[e] = seen + (int32_t)__popcll(same);
        rk[s] = seen + below;
        ev[s] = valid ? e : -1;
    }
    __syncthreads();

    // (4) per expert: first rank of each wave = tile base + earlier waves
    for (int e = tid; e < E; e += kLayoutThreads) {
        int32_t run = base[e];
#pragma unroll
        for (int v = 0; v < kRankWaves; ++v) {
            const int32_t c = wh[v * E + e];
            wh[v * E + e] = run;
            run += c;
        }
    }
    __syncthreads();

    // (5) positions, drops and the inverse map
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int64_t a = a0 + s * kWave + lane;
        if (a < TK) {
            const int32_t e = ev[s];
            int32_t p = -1;
            if (e >= 0) {
                const int32_t r = my_wh[e] + rk[s];
                if (capacity < 0 || r < capacity)
                    p = eoff[e] + r;
            }
            pos[a] = p;
            if (p >= 0 && send_src)
                send_src[p] = (int32_t)((uint32_t)a / (uint32_t)k);
        }
    }
}

}  // namespace

hipError_t launch_dispatch_layout(const int32_t *topk_idx, int64_t T, int32_t E, int32_t k,
                                  int32_t R, int32_t capacity, int32_t *expert_demand,
                                  int32_t *expert_counts, int32_t *expert_offsets,
                                  int32_t *dest_counts, int32_t *dest_offsets, int32_t *pos,
                                  int32_t *send_src, int32_t *tile_hist, hipStream_t stream)
{
    const int64_t TK = T * (int64_t)k;
    const int64_t B = layout_tiles(TK);
    int nbits = 0;
    while ((1 << nbits) < E)
        ++nbits;
    if (B > 0) {
        hipLaunchKernelGGL(layout_count_kernel, dim3((unsigned)B), dim3(kLayoutThreads),
                           E * sizeof(int32_t), stream, topk_idx, TK, E, tile_hist);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    hipLaunchKernelGGL(layout_scan_kernel, dim3((unsigned)((E + kWave - 1) / kWave)),
                       dim3(kScanWaves * kWave), 0, stream, tile_hist, B, E, capacity,
                       expert_demand, expert_counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const size_t lds = (size_t)(E + 1 + E + kRankWaves * E) * sizeof(int32_t);
    hipLaunchKernelGGL(layout_rank_kernel, dim3((unsigned)(B > 0 ? B : 1)), dim3(kLayoutThreads),
                       lds, stream, topk_idx, TK, B, k, E, R, capacity, nbits, tile_hist,
                       expert_counts, expert_offsets, dest_counts, dest_offsets, pos, send_src);
    return hipGetLastError();
}

}  // namespace moe
