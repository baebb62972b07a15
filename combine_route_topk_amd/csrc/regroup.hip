// regroup.hip -- receive side: source-major segments to expert-major rows,
// and back for the return path.
//
// Method: aicassindra "gpu_moe_all_to_all", "Two collectives per layer"
// (per-destination counts arrive before the payload so that the receiver
// can size and place it; outputs return along the inverse permutation) and
// "Bucketing" (one contiguous message per peer); "MoE All-to-All Dispatch
// and Ragged Routing", "Why MoE Token Dispatch is All-to-All" (a GPU holds a
// few of the experts) and "Fixed Capacity vs. Ragged Routing" (the receiver
// pools its local experts).
//
// A destination's receive buffer is the concatenation, in source order, of
// one segment per source; each segment holds cnt[s][l] rows of local expert
// l, l ascending. The regroup moves each (source, expert) block -- a
// contiguous run of rows -- to its place in the expert-major layout. The row
// count N never leaves the device.
//
//  * regroup_table_kernel (one block, S <= 1024, E_l <= 1024, S*E_l <= 4096):
//    LDS scans of the S x E_l counts give
//    the per-expert and per-source offsets and, for every block b = s*E_l+l,
//    its first source-major row and its first expert-major row.
//  * regroup_pos_kernel: recv_pos[i] for every received row, by a binary
//    search over the block table held in LDS.
//  * regroup_rows_kernel: a 16-byte-per-lane row move in either direction,
//    one block per (row, 4 KiB column slab), like the dispatch permute; past
//    2^22 rows the blocks stride over them.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kTableThreads = 1024;
constexpr int kPosThreads = 1024;
constexpr int kPosRowsPerThread = 8;
constexpr int kRowThreads = 256;

// Exclusive scan of one value per thread over the block (1024 threads);
// returns the thread's prefix and leaves the grand total in *total.
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t *wave_total,
                                                        int32_t *total)
{
    constexpr int WAVES = kTableThreads / kWave;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const int32_t inc = wave_inclusive_sum(v);
    if (lane == kWave - 1)
        wave_total[w] = inc;
    __syncthreads();
    int32_t before = 0, all = 0;
#pragma unroll
    for (int u = 0; u < WAVES; ++u) {
        before += u < w ? wave_total[u] : 0;
        all += wave_total[u];
    }
    *total = all;
    return before + inc - v;
}

__global__ __launch_bounds__(kTableThreads) void regroup_table_kernel(
    const int32_t *__restrict__ cnt, int32_t S, int32_t El,
    int32_t *__restrict__ local_expert_offsets, int32_t *__restrict__ source_offsets,
    int32_t *__restrict__ blk_src, int32_t *__restrict__ blk_dst)
{
    extern __shared__ int32_t sm[];
    const int SE = S * El;
    int32_t *c = sm;          // [SE] counts
    int32_t *rel = c + SE;    // [SE] offset of a block inside its source segment
    int32_t *col = rel + SE;  // [SE] offset of a block inside its expert's rows
    __shared__ int32_t wave_total[kTableThreads / kWave];
    const int tid = threadIdx.x;
    for (int i = tid; i < SE; i += kTableThreads)
        c[i] = max(cnt[i], 0);  // counts are device data: negative ones count as 0
    __syncthreads();
    // per source s (thread s): running offsets along its segment
    int32_t src_rows = 0;
    if (tid < S)
        for (int l = 0; l < El; ++l) {
            rel[tid * El + l] = src_rows;
            src_rows += c[tid * El + l];
        }
    // per local expert l (thread l): running offsets over the sources
    int32_t exp_rows = 0;
    if (tid < El)
        for (int s2 = 0; s2 < S; ++s2) {
            col[s2 * El + tid] = exp_rows;
            exp_rows += c[s2 * El + tid];
        }
    int32_t n_rows;
    const int32_t src_start = block_exclusive_scan(tid < S ? src_rows : 0, wave_total, &n_rows);
    __syncthreads();
    int32_t n_rows2;
    const int32_t exp_start = block_exclusive_scan(tid < El ? exp_rows : 0, wave_total, &n_rows2);
    if (tid < S)
        source_offsets[tid] = src_start;
    if (tid < El)
        local_expert_offsets[tid] = exp_start;
    if (tid == 0) {
        source_offsets[S] = n_rows;
        local_expert_offsets[El] = n_rows;
        blk_src[SE] = n_rows;
    }
    // every block of source s gets its source start; of expert l, the expert start
    __syncthreads();
    if (tid < S)
        for (int l = 0; l < El; ++l)
            blk_src[tid * El + l] = src_start + rel[tid * El + l];
    if (tid < El)
        for (int s2 = 0; s2 < S; ++s2)
            blk_dst[s2 * El + tid] = exp_start + col[s2 * El + tid];
}

__global__ __launch_bounds__(kPosThreads) void regroup_pos_kernel(
    const int32_t *__restrict__ blk_src, const int32_t *__restrict__ blk_dst, int32_t SE,
    int64_t max_rows, int32_t *__restrict__ recv_pos)
{
    extern __shared__ int32_t sm[];
    int32_t *bs = sm;           // [SE + 1]
    int32_t *bd = bs + SE + 1;  // [SE]
    for (int i = threadIdx.x; i <= SE; i += kPosThreads)
        bs[i] = blk_src[i];
    for (int i = threadIdx.x; i < SE; i += kPosThreads)
        bd[i] = blk_dst[i];
    __syncthreads();
    const int64_t N = min((int64_t)bs[SE], max_rows);
    const int64_t first = (int64_t)blockIdx.x * kPosThreads * kPosRowsPerThread;
    for (int q = 0; q < kPosRowsPerThread; ++q) {
        const int64_t i = first + q * kPosThreads + threadIdx.x;
        if (i >= N)
            break;
        // largest b with bs[b] <= i: the block holding row i (empty blocks
        // share their start with the next one and are skipped over)
        int lo = 0, hi = SE - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (bs[mid] <= i)
                lo = mid;
            else
                hi = mid - 1;
        }
        recv_pos[i] = bd[lo] + (int32_t)(i - bs[lo]);
    }
}

// GATHER = false: dst[map[i]] = src[i]; true: dst[i] = src[map[i]]
template <bool GATHER>
__global__ __launch_bounds__(kRowThreads) void regroup_rows_kernel(
    const u32x4 *__restrict__ src, const int32_t *__restrict__ map,
    const int32_t *__restrict__ n_rows, int64_t max_rows, int32_t C16, u32x4 *__restrict__ dst)
{
    const int32_t c = blockIdx.y * kRowThreads + threadIdx.x;
    const int64_t N = min((int64_t)*n_rows, max_rows);
    if (c >= C16)
        return;
    // one row per block; the grid is capped, so blocks stride over the rows
    for (int64_t i = blockIdx.x; i < N; i += gridDim.x) {
        const int32_t p = map[i];
        if (p < 0 || p >= max_rows)
            continue;
        const int64_t from = GATHER ? p : i, to = GATHER ? i : p;
        store_stream(dst + to * C16 + c, src[from * C16 + c]);
    }
}

}  // namespace

size_t regroup_workspace_bytes(int32_t S, int32_t El)
{
    return (size_t)(2 * (int64_t)S * El + 1) * sizeof(int32_t);
}

hipError_t launch_recv_regroup_layout(const int32_t *recv_counts, int32_t S, int32_t El,
                                      int32_t *local_expert_offsets, int32_t *source_offsets,
                                      int32_t *recv_pos, int64_t max_rows, int32_t *workspace,
                                      hipStream_t stream)
{
    const int32_t SE = S * El;
    int32_t *blk_src = workspace;       // [SE + 1]
    int32_t *blk_dst = workspace + SE + 1;  // [SE]
    const size_t lds_table = (size_t)(3 * SE) * sizeof(int32_t);
    hipLaunchKernelGGL(regroup_table_kernel, dim3(1), dim3(kTableThreads), lds_table, stream,
                       recv_counts, S, El, local_expert_offsets, source_offsets, blk_src, blk_dst);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || max_rows == 0)
        return err;
    const int64_t per_block = (int64_t)kPosThreads * kPosRowsPerThread;
    const size_t lds_pos = (size_t)(2 * SE + 1) * sizeof(int32_t);
    hipLaunchKernelGGL(regroup_pos_kernel, dim3((unsigned)((max_rows + per_block - 1) / per_block)),
                       dim3(kPosThreads), lds_pos, stream, blk_src, blk_dst, SE, max_rows, recv_pos);
    return hipGetLastError();
}

hipError_t launch_regroup_rows(const uint16_t *src, const int32_t *map, const int32_t *n_rows,
                               int64_t max_rows, int32_t H, bool gather, uint16_t *dst,
                               hipStream_t stream)
{
    if (max_rows == 0)
        return hipSuccess;
    const int32_t C16 = H / 8;
    const dim3 grid((unsigned)(max_rows < kMaxRowBlocks ? max_rows : kMaxRowBlocks),
                    (unsigned)((C16 + kRowThreads - 1) / kRowThreads));
    const u32x4 *s = reinterpret_cast<const u32x4 *>(src);
    u32x4 *d = reinterpret_cast<u32x4 *>(dst);
    if (gather)
        hipLaunchKernelGGL(regroup_rows_kernel<true>, grid, dim3(kRowThreads), 0, stream, s, map,
                           n_rows, max_rows, C16, d);
    else
        hipLaunchKernelGGL(regroup_rows_kernel<false>, grid, dim3(kRowThreads), 0, stream, s, map,
                           n_rows, max_rows, C16, d);
    return hipGetLastError();
}

}  // namespace moe
