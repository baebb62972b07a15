// layout_device.hpp -- the counting, scanning and ranking steps of the
// dispatch layout, shared by the layout kernels (layout.hip) and the fused
// routing + layout kernel for small batches (route_layout.hip). The method
// is described at the top of layout.hip.
#pragma once

#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

// Assignments are read kBatch steps of 64 at a time, so that each wave has
// kBatch independent loads in flight instead of one load per step.
constexpr int kBatch = 8;

// Rank one step of 64 consecutive assignments a0 + lane (the lane's id e;
// lanes at or past a_end hold -1) in order. `run` is the wave's LDS row: its
// next rank per expert, advanced past the step. Writes pos and send_src.
__device__ __forceinline__ void rank_step(int32_t e, int64_t a0, int64_t a_end, int32_t k,
                                          int32_t E, int32_t capacity, int nbits, int32_t *run,
                                          const int32_t *eoff, int32_t *__restrict__ pos,
                                          int32_t *__restrict__ send_src)
{
    const int64_t a = a0 + lane_id();
    const bool valid = (uint32_t)e < (uint32_t)E;
    uint64_t same = ballot64(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t ones = ballot64(bit);
        same &= bit ? ones : ~ones;
    }
    const int32_t below = (int32_t)count_below(same);
    const int32_t seen = valid ? run[e] : 0;
    if (valid && below == 0)
        run[e] = seen + (int32_t)__popcll(same);
    if (a < a_end) {
        const int32_t r = seen + below;
        int32_t p = -1;
        if (valid && (capacity < 0 || r < capacity))
            p = eoff[e] + r;
        pos[a] = p;
        if (p >= 0 && send_src)
            send_src[p] = (int32_t)((uint32_t)a / (uint32_t)k);
    }
}

// Rank the assignments [a_begin, a_end) of one wave in order. `run` is the
// wave's LDS row: on entry its first rank per expert, on exit advanced past
// the range. Writes pos and send_src.
__device__ __forceinline__ void rank_range(const int32_t *__restrict__ idx, int64_t a_begin,
                                           int64_t a_end, int32_t k, int32_t E, int32_t capacity,
                                           int nbits, int32_t *run, const int32_t *eoff,
                                           int32_t *__restrict__ pos,
                                           int32_t *__restrict__ send_src)
{
    const int lane = lane_id();
    for (int64_t a0 = a_begin; a0 < a_end; a0 += kBatch * kWave) {
        int32_t ev[kBatch];
#pragma unroll
        for (int s = 0; s < kBatch; ++s) {
            const int64_t a = a0 + s * kWave + lane;
            ev[s] = a < a_end ? idx[a] : -1;
        }
#pragma unroll
        for (int s = 0; s < kBatch; ++s) {
            if (a0 + s * kWave >= a_end)
                break;  // uniform: the wave's range is exhausted
            rank_step(ev[s], a0 + s * kWave, a_end, k, E, capacity, nbits, run, eoff, pos,
                      send_src);
        }
    }
}

// Exclusive scan of cnt[0..E) into eoff[0..E] with all threads of the
// block (E <= 4 * blockDim.x). wave_total holds one int per wave.
template <int THREADS>
__device__ __forceinline__ void block_scan_counts(const int32_t *cnt, int32_t E, int32_t *eoff,
                                                  int32_t *wave_total)
{
    constexpr int WAVES = THREADS / kWave;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    constexpr int PER = (1024 + THREADS - 1) / THREADS;  // E <= 1024
    int32_t c[PER];
    int32_t mine = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid * PER + q;
        c[q] = e < E ? cnt[e] : 0;
        mine += c[q];
    }
    const int32_t inc = wave_inclusive_sum(mine);
    if (lane == kWave - 1)
        wave_total[w] = inc;
    __syncthreads();
    int32_t ex = inc - mine;
    int32_t total = 0;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) {
        ex += v < w ? wave_total[v] : 0;
        total += wave_total[v];
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid * PER + q;
        if (e < E)
            eoff[e] = ex;
        ex += c[q];
    }
    if (tid == 0)
        eoff[E] = total;
}

// Publish the offset table and the per-destination counts and offsets.
__device__ __forceinline__ void publish_offsets(const int32_t *eoff, int32_t E, int32_t R,
                                                int32_t *__restrict__ expert_offsets,
                                                int32_t *__restrict__ dest_counts,
                                                int32_t *__restrict__ dest_offsets)
{
    for (int e = threadIdx.x; e <= E; e += blockDim.x)
        expert_offsets[e] = eoff[e];
    const int32_t el = E / R;
    for (int r = threadIdx.x; r < R; r += blockDim.x) {
        dest_offsets[r] = eoff[r * el];
        dest_counts[r] = eoff[(r + 1) * el] - eoff[r * el];
    }
    if (threadIdx.x == 0)
        dest_offsets[R] = eoff[E];
}

// Count the valid ids of [a_begin, a_end) into row[] (order-free), with
// kBatch loads in flight per lane. `first` and `stride` spread the range
// over the lanes of one wave or over a whole block.
__device__ __forceinline__ void count_range(const int32_t *__restrict__ idx, int64_t a_begin,
                                            int64_t a_end, int64_t first, int64_t stride,
                                            int32_t E, int32_t *row)
{
    for (int64_t a0 = a_begin + first; a0 < a_end; a0 += kBatch * stride) {
        int32_t ev[kBatch];
#pragma unroll
        for (int s = 0; s < kBatch; ++s) {
            const int64_t a = a0 + s * stride;
            ev[s] = a < a_end ? idx[a] : -1;
        }
#pragma unroll
        for (int s = 0; s < kBatch; ++s)
            if ((uint32_t)ev[s] < (uint32_t)E)
                atomicAdd(&row[ev[s]], 1);
    }
}

// Range of wave w when [begin, end) is split into `parts` chunks of whole
// 64-assignment steps.
__device__ __forceinline__ void wave_span(int64_t begin, int64_t end, int w, int parts,
                                          int64_t &lo, int64_t &hi)
{
    const int64_t steps = (end - begin + kWave - 1) / kWave;
    const int64_t per = (steps + parts - 1) / parts;
    lo = min(end, begin + (int64_t)w * per * kWave);
    hi = min(end, lo + per * kWave);
}

// The whole layout of TK <= kSmallAssignments assignments (E <= 512) in one
// block of THREADS threads. Each wave loads its contiguous range of ids once
// (at most kBatch steps of 64) and keeps them in registers: it counts them
// into its own LDS row (pass A), a prefix over the waves and a block scan
// give the first ranks and the offsets, then it ranks the same ids in order
// (pass B). sm holds (THREADS / 64 + 2) * E + 1 ints.
template <int THREADS>
__device__ __forceinline__ void layout_small_body(
    const int32_t *__restrict__ idx, int64_t TK, int32_t k, int32_t E, int32_t R,
    int32_t capacity, int nbits, int32_t *__restrict__ expert_demand,
    int32_t *__restrict__ expert_counts, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ dest_counts, int32_t *__restrict__ dest_offsets,
    int32_t *__restrict__ pos, int32_t *__restrict__ send_src, int32_t *sm)
{
    constexpr int kSmallThreads = THREADS;
    constexpr int kSmallWaves = THREADS / kWave;
    static_assert((int64_t)kSmallWaves * kBatch * kWave >= kSmallAssignments,
                  "a wave's range must fit in its registers");
    int32_t *wh = sm;                           // [kSmallWaves][E]
    int32_t *cnt = wh + kSmallWaves * E;        // [E]
    int32_t *eoff = cnt + E;                    // [E + 1]
    __shared__ int32_t wave_total[kSmallWaves];
    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = lane_id();

    int64_t lo, hi;
    wave_span(0, TK, w, kSmallWaves, lo, hi);
    int32_t ev[kBatch];
#pragma unroll
    for (int s = 0; s < kBatch; ++s) {
        const int64_t a = lo + s * kWave + lane;
        ev[s] = a < hi ? idx[a] : -1;
    }
    for (int i = tid; i < kSmallWaves * E; i += kSmallThreads)
        wh[i] = 0;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kBatch; ++s)  // pass A
        if ((uint32_t)ev[s] < (uint32_t)E)
            atomicAdd(&wh[w * E + ev[s]], 1);
    __syncthreads();
    for (int e = tid; e < E; e += kSmallThreads) {
        int32_t run = 0;
        for (int v = 0; v < kSmallWaves; ++v) {
            const int32_t c = wh[v * E + e];
            wh[v * E + e] = run;
            run += c;
        }
        const int32_t kept = (capacity < 0 || run < capacity) ? run : capacity;
        cnt[e] = kept;
        expert_demand[e] = run;
        expert_counts[e] = kept;
    }
    __syncthreads();
    block_scan_counts<kSmallThreads>(cnt, E, eoff, wave_total);
    __syncthreads();
    publish_offsets(eoff, E, R, expert_offsets, dest_counts, dest_offsets);
#pragma unroll
    for (int s = 0; s < kBatch; ++s) {  // pass B
        if (lo + s * kWave >= hi)
            break;  // uniform: the wave's range is exhausted
        rank_step(ev[s], lo + s * kWave, hi, k, E, capacity, nbits, wh + w * E, eoff, pos,
                  send_src);
    }
}

}  // namespace
}  // namespace moe
