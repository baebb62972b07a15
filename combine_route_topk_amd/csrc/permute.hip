// permute.hip -- pack each kept replica of a token into its send row.
//
// Method: aicassindra "gpu_moe_all_to_all", "Bucketing" (make each
// destination's rows contiguous, with the permutation fused into the kernel
// that stages the sends) and "Two collectives per layer" (each token leaves
// k times); thecoregrid "Mixture-of-experts acceleration through overlap",
// paragraph on the remote-owner-aligned layout.
//
// Token-major scatter: block (t, y) reads a 4 KiB column slab of x[t] once,
// 16 bytes per lane, and writes it to each of the token's kept send rows.
// Row reads and writes are contiguous 16-byte-per-lane streams, so a wave
// moves 1 KiB per instruction. Tokens whose replicas were all dropped
// skip the read. The send rows are written with the non-temporal hint
// (streamed out, not kept in cache); x is read with an ordinary load. On
// MI355X that pairing measured fastest: 5.7 TB/s for k = 10 against 4.8 TB/s
// with the hint on both streams.
//
// A block stores only after its x load returns, so with x cold in HBM each
// block's life is one HBM round trip plus its k stores. For k >= 4 each
// block therefore also loads the same slab of token t + kPrefetchTokens (if
// that token keeps a replica) and discards it, so that the block which
// reads that slab later finds it in a cache. The distance is twice the
// blocks resident at once (256 CUs x 8 blocks), so the prefetch runs ahead
// of the blocks in flight, and a multiple of 8, so both blocks run on the
// same XCD (blocks are dealt to the 8 XCDs by linear block id mod 8, which
// a probe of the XCC_ID register confirmed on MI355X). The L2 does not keep
// the row that long (the stores that pass through it in between are
// several times its size): L2 fetches rise by the size of x, and the later
// load is served by the 256 MB Infinity Cache instead of HBM. On MI355X,
// with x evicted before the call, it took T = 32768, H = 2048 from 303.4 to
// 289.0 us at k = 10 and from 122.0 to 114.2 us at T = 16384, k = 8; at
// k = 2 it cost 2-3.5% (few stores wait on each load), so it is off there.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kRowThreads = 256;
constexpr int64_t kPrefetchTokens = 4096;
constexpr int32_t kPrefetchMinK = 4;
static_assert(kPrefetchTokens % 8 == 0, "the prefetching block and the reader share an XCD");

// n_ahead: tokens past this launch's last one whose rows may be prefetched
// (the launch covers tokens [0, T) of its pointers, and x and pos extend
// n_ahead tokens further); pf_dist: the prefetch distance in tokens, 0 for
// none
__global__ __launch_bounds__(kRowThreads) void permute_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ pos, int64_t T, int64_t n_ahead,
    int64_t pf_dist, int32_t C16, int32_t k, u32x4 *__restrict__ send, int64_t send_rows)
{
    const int64_t t = blockIdx.x;
    const int32_t c = blockIdx.y * kRowThreads + threadIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    // prefetch: token t + pf_dist's slab, if that token keeps a replica
    const int64_t tf = t + pf_dist;
    const bool ahead = pf_dist > 0 && tf < T + n_ahead;  // uniform across the block
    const int32_t pf = ahead && lane < k ? pos[tf * k + lane] : -1;
    // the token's k positions in one vector load (lane j < k holds entry j),
    // broadcast with readlane, instead of k scalar loads that wait in turn
    const int32_t pl = lane < k ? pos[t * k + lane] : -1;
    u32x4 warm = {0u, 0u, 0u, 0u};
    if (ahead && ballot64(pf >= 0 && pf < send_rows) != 0 && c < C16)
        warm = x[tf * C16 + c];
    const bool kept = pl >= 0 && pl < send_rows;
    if (ballot64(kept) != 0 && c < C16) {  // not every replica dropped (uniform)
        const u32x4 v = x[t * C16 + c];
        for (int j = 0; j < k; ++j) {
            const int32_t p = (int32_t)readlane_u32((uint32_t)pl, j);
            if (p >= 0 && p < send_rows)
                store_stream(send + (int64_t)p * C16 + c, v);
        }
    }
    // the prefetched value is not needed; this keeps its load
    asm volatile("" ::"v"(warm[0]), "v"(warm[1]), "v"(warm[2]), "v"(warm[3]));
}

}  // namespace

hipError_t launch_dispatch_permute(const uint16_t *x, const int32_t *pos, int64_t T, int32_t H,
                                   int32_t k, uint16_t *send, int64_t send_rows,
                                   hipStream_t stream)
{
    const int32_t C16 = H / 8;
    const int64_t pf_dist = k >= kPrefetchMinK ? kPrefetchTokens : 0;
    // one block per token; past kMaxRowBlocks tokens, one launch per chunk
    for (int64_t t0 = 0; t0 < T; t0 += kMaxRowBlocks) {
        const int64_t n = T - t0 < kMaxRowBlocks ? T - t0 : kMaxRowBlocks;
        const dim3 grid((unsigned)n, (unsigned)((C16 + kRowThreads - 1) / kRowThreads));
        hipLaunchKernelGGL(permute_kernel, grid, dim3(kRowThreads), 0, stream,
                           reinterpret_cast<const u32x4 *>(x) + t0 * C16, pos + t0 * k, n,
                           T - t0 - n, pf_dist, C16, k, reinterpret_cast<u32x4 *>(send), send_rows);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    return hipSuccess;
}

}  // namespace moe
