// floor.hip -- the synthetic floor: a plain streaming kernel that moves a
// given number of bytes in and out of HBM with the same 16-byte lane
// accesses as the path's row kernels, and nothing else.
//
// Method: aicassindra "gpu_moe_all_to_all", "How to tell whether the
// all-to-all is your bottleneck" (time a synthetic transfer of the same
// sizes; the gap between it and the real path is overhead owned in
// software). On one GPU the transfer is HBM traffic, so the floor is a
// kernel that reads `read_bytes` and writes `write_bytes` contiguously:
// the best the memory system does for that volume and read:write mix,
// with no gather, scatter, index or launch structure of the path.
//
// Block b takes 16 KiB tiles b, b + grid, ...: every lane issues its four
// 16-byte loads before its four stores, so each wave keeps 4 KiB of reads
// in flight. Chunk i is read if i < n_read and written if i < n_write; a
// chunk that is written but not read stores a constant, and the loaded
// values that are not stored feed one conditional store that never fires
// for real data (so the compiler keeps the loads).
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kFloorThreads = 256;
constexpr int kFloorUnroll = 4;
constexpr int64_t kFloorTile = (int64_t)kFloorThreads * kFloorUnroll;  // chunks of 16 B
constexpr int64_t kMaxFloorBlocks = 1 << 20;

template <bool NT_STORE>
__global__ __launch_bounds__(kFloorThreads) void floor_kernel(const u32x4 *__restrict__ src,
                                                              int64_t n_read,
                                                              u32x4 *__restrict__ dst,
                                                              int64_t n_write)
{
    const int64_t n = n_read > n_write ? n_read : n_write;
    uint32_t sink = 0;
    for (int64_t base = (int64_t)blockIdx.x * kFloorTile; base < n;
         base += (int64_t)gridDim.x * kFloorTile) {
        u32x4 v[kFloorUnroll];
#pragma unroll
        for (int u = 0; u < kFloorUnroll; ++u) {
            const int64_t i = base + u * kFloorThreads + threadIdx.x;
            v[u] = i < n_read ? src[i] : u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
        }
#pragma unroll
        for (int u = 0; u < kFloorUnroll; ++u) {
            const int64_t i = base + u * kFloorThreads + threadIdx.x;
            if (i < n_write) {
                if (NT_STORE)
                    store_stream(dst + i, v[u]);
                else
                    dst[i] = v[u];
            } else {
                sink ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
            }
        }
    }
    // read-only chunks: their values meet here, stored only in the unlikely
    // event that they fold to this pattern (and only where a write is due)
    if (sink == 0x9E3779B9u && n_write > 0)
        dst[0] = u32x4{sink, sink, sink, sink};
}

}  // namespace

hipError_t launch_hbm_floor(const void *src, int64_t read_bytes, void *dst, int64_t write_bytes,
                            bool nt_store, hipStream_t stream)
{
    const int64_t n_read = read_bytes / 16, n_write = write_bytes / 16;
    const int64_t n = n_read > n_write ? n_read : n_write;
    if (n == 0)
        return hipSuccess;
    int64_t blocks = (n + kFloorTile - 1) / kFloorTile;
    if (blocks > kMaxFloorBlocks)
        blocks = kMaxFloorBlocks;
    const u32x4 *s = static_cast<const u32x4 *>(src);
    u32x4 *d = static_cast<u32x4 *>(dst);
    if (nt_store)
        hipLaunchKernelGGL(floor_kernel<true>, dim3((unsigned)blocks), dim3(kFloorThreads), 0,
                           stream, s, n_read, d, n_write);
    else
        hipLaunchKernelGGL(floor_kernel<false>, dim3((unsigned)blocks), dim3(kFloorThreads), 0,
                           stream, s, n_read, d, n_write);
    return hipGetLastError();
}

}  // namespace moe
