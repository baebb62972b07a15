// launch.hpp -- internal launchers, one per kernel family. Each enqueues on
// `stream` and returns the hipError_t of the launch. Arguments have already
// been validated by the C ABI layer (api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// n_groups == 0: plain top-k; otherwise at most topk_groups of n_groups
// contiguous expert groups per token (n_groups <= 64).
hipError_t launch_route_topk(const float *logits, const float *bias, int64_t T, int32_t E,
                             int32_t k, int32_t n_groups, int32_t topk_groups, bool normalize,
                             int32_t *topk_idx, float *topk_w, hipStream_t stream);

// Layout plan. Up to kSmallAssignments assignments (and E <= 512) one block
// does the whole layout. Above that, assignments are split into at most
// kMaxTiles tiles of at least layout_min_tile(E); the workspace holds one
// E-wide int32 histogram per tile.
constexpr int kLayoutThreads = 256;
// Smaller tiles put more blocks on the rank pass, whose time is latency;
// each rank block also reads every tile's histogram, which is cheap while E
// is small. On MI355X with 32768 assignments: E = 64 took 9.3 / 8.4 / 8.0 us
// with tiles of 2048 / 1024 / 512, E = 384 took 9.9 / 9.2 / 9.4 us.
constexpr int64_t layout_min_tile(int32_t E) { return E <= 128 ? 512 : 1024; }
constexpr int64_t kMaxTiles = 128;
constexpr int64_t kSmallAssignments = 4096;
constexpr int32_t kSmallMaxExperts = 512;

struct LayoutPlan {
    bool small;
    int64_t tile;   // assignments per tile (large path)
    int64_t tiles;  // number of tiles (large path), 0 otherwise
};

LayoutPlan layout_plan(int64_t TK, int32_t E);

inline size_t layout_workspace_bytes(int64_t TK, int32_t E)
{
    return (size_t)layout_plan(TK, E).tiles * (size_t)E * sizeof(int32_t);
}

// The allocation-free layout's device array (layout.hip): its size, and its
// address on the current device (looked up once per device).
size_t layout_scratch_bytes();
hipError_t layout_scratch(int32_t **ptr);

hipError_t launch_dispatch_layout(const int32_t *topk_idx, int64_t T, int32_t E, int32_t k,
                                  int32_t R, int32_t capacity, int32_t *expert_demand,
                                  int32_t *expert_counts, int32_t *expert_offsets,
                                  int32_t *dest_counts, int32_t *dest_offsets, int32_t *pos,
                                  int32_t *send_src, int32_t *tile_hist, hipStream_t stream);

// Routing and layout in one call (route_layout.hip): one launch for small
// batches, else the two kernels. The workspace starts with the fused
// kernel's ticket word; the tiled layout's histograms follow.
constexpr size_t kRouteLayoutHeaderBytes = 16;
inline size_t route_layout_workspace_bytes(int64_t TK, int32_t E)
{
    return kRouteLayoutHeaderBytes + layout_workspace_bytes(TK, E);
}
bool route_layout_fuses(int64_t T, int32_t E, int32_t k, const float *logits, const float *bias);
hipError_t launch_route_layout(const float *logits, const float *bias, int64_t T, int32_t E,
                               int32_t k, bool normalize, int32_t R, int32_t capacity,
                               int32_t *topk_idx, float *topk_w, int32_t *expert_demand,
                               int32_t *expert_counts, int32_t *expert_offsets,
                               int32_t *dest_counts, int32_t *dest_offsets, int32_t *pos,
                               int32_t *send_src, void *workspace, hipStream_t stream);

hipError_t launch_dispatch_permute(const uint16_t *x, const int32_t *pos, int64_t T, int32_t H,
                                   int32_t k, uint16_t *send, int64_t send_rows,
                                   hipStream_t stream);

hipError_t launch_combine_reduce(const uint16_t *y, int64_t y_rows, const int32_t *pos,
                                 const float *topk_w, const uint16_t *shared,
                                 const uint16_t *residual, int64_t T, int32_t H, int32_t k,
                                 bool out_fp32, void *out, hipStream_t stream);

// FP8 dispatch payload (fp8.hip).
int64_t fp8_row_bytes(int32_t H);
hipError_t launch_dispatch_permute_fp8(const uint16_t *x, const int32_t *pos, int64_t T,
                                       int32_t H, int32_t k, uint8_t *send, int64_t send_rows,
                                       hipStream_t stream);
hipError_t launch_fp8_dequant(const uint8_t *rows, const int32_t *n_rows, int64_t max_rows,
                              int32_t H, uint16_t *out, hipStream_t stream);

// Tile-signalled return with a stand-in expert GEMM (expert.hip).
size_t expert_linear_workspace_bytes(int32_t S, int32_t El, int64_t max_rows);
hipError_t expert_return_slots(int *slots);
hipError_t launch_expert_linear(const uint16_t *recv, const int32_t *cnt, int32_t S, int32_t El,
                                int32_t H, int32_t H_out, const uint16_t *W, int64_t max_rows,
                                uint16_t *y, int32_t *workspace, hipStream_t stream);
hipError_t launch_expert_return(const uint16_t *recv, const int32_t *cnt, int32_t S, int32_t El,
                                int32_t H, int32_t H_out, const uint16_t *W, int64_t max_rows,
                                int32_t self_rank, int32_t consumers, int32_t band_group,
                                uint16_t *y, uint16_t *ret, int32_t *workspace,
                                hipStream_t stream, int32_t *grid_used);

// Receive-side regroup (regroup.hip).
size_t regroup_workspace_bytes(int32_t S, int32_t El);
hipError_t launch_recv_regroup_layout(const int32_t *recv_counts, int32_t S, int32_t El,
                                      int32_t *local_expert_offsets, int32_t *source_offsets,
                                      int32_t *recv_pos, int64_t max_rows, int32_t *workspace,
                                      hipStream_t stream);
hipError_t launch_regroup_rows(const uint16_t *src, const int32_t *map, const int32_t *n_rows,
                               int64_t max_rows, int32_t H, bool gather, uint16_t *dst,
                               hipStream_t stream);

// Synthetic floor: a contiguous streaming read and write (floor.hip).
hipError_t launch_hbm_floor(const void *src, int64_t read_bytes, void *dst, int64_t write_bytes,
                            bool nt_store, hipStream_t stream);

}  // namespace moe
