// launch.hpp -- internal launchers, one per kernel family. Each enqueues on
// `stream` and returns the hipError_t of the launch. Arguments have already
// been validated by the C ABI layer (api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_route_topk(const float *logits, const float *bias, int64_t T, int32_t E,
                             int32_t k, bool normalize, int32_t *topk_idx, float *topk_w,
                             hipStream_t stream);

// Assignments (t, j) are handled in tiles of kLayoutTile; the workspace holds
// one E-wide histogram per tile.
constexpr int kLayoutThreads = 256;
constexpr int kLayoutPerThread = 8;
constexpr int kLayoutTile = kLayoutThreads * kLayoutPerThread;

inline int64_t layout_tiles(int64_t TK) { return (TK + kLayoutTile - 1) / kLayoutTile; }
inline size_t layout_workspace_bytes(int64_t TK, int32_t E)
{
    return (size_t)layout_tiles(TK) * (size_t)E * sizeof(int32_t);
}

hipError_t launch_dispatch_layout(const int32_t *topk_idx, int64_t T, int32_t E, int32_t k,
                                  int32_t R, int32_t capacity, int32_t *expert_demand,
                                  int32_t *expert_counts, int32_t *expert_offsets,
                                  int32_t *dest_counts, int32_t *dest_offsets, int32_t *pos,
                                  int32_t *send_src, int32_t *tile_hist, hipStream_t stream);

hipError_t launch_dispatch_permute(const uint16_t *x, const int32_t *pos, int64_t T, int32_t H,
                                   int32_t k, uint16_t *send, int64_t send_rows,
                                   hipStream_t stream);

hipError_t launch_combine_reduce(const uint16_t *y, int64_t y_rows, const int32_t *pos,
                                 const float *topk_w, const uint16_t *shared,
                                 const uint16_t *residual, int64_t T, int32_t H, int32_t k,
                                 bool out_fp32, void *out, hipStream_t stream);

}  // namespace moe
