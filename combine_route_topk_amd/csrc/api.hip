// api.hip -- the C ABI declared in include/moe_ep.h: argument validation on
// the host, then one launcher call on the caller's stream. Nothing here
// touches the GPU before every check has passed.
#include "moe_ep.h"

#include "launch.hpp"

namespace {

constexpr int32_t kMaxE = 1024;
constexpr int32_t kMaxK = 32;
constexpr int32_t kMaxH = 65536;
constexpr int32_t kMaxGroups = 64;
constexpr int32_t kMaxRegroupSide = 1024;
constexpr int32_t kMaxRegroupBlocks = 4096;
constexpr int64_t kMaxAssignments = (int64_t)1 << 31;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// k and the token count: shared by every entry point.
moe_status_t check_tokens(int64_t T, int32_t k)
{
    if (T < 0)
        return MOE_ERR_INVALID_ARG;
    if (k < 1 || k > kMaxK)
        return MOE_ERR_UNSUPPORTED;
    if (T * (int64_t)k >= kMaxAssignments)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status_t check_experts(int32_t E, int32_t k)
{
    if (E < 1 || E > kMaxE || k > E)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status_t check_hidden(int32_t H)
{
    if (H <= 0 || H % 8 != 0 || H > kMaxH)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status_t check_layout_sizes(int64_t T, int32_t E, int32_t k, int32_t R)
{
    moe_status_t s = check_tokens(T, k);
    if (s != MOE_OK)
        return s;
    if ((s = check_experts(E, k)) != MOE_OK)
        return s;
    if (R < 1 || E % R != 0)
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status_t from_hip(hipError_t err) { return err == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

// The permutes' sizes: the send buffer must hold every row the layout can
// keep, T * k when dropless, else min(T * k, E * capacity).
moe_status_t check_permute(int64_t T, int32_t H, int32_t k, int32_t E, int32_t capacity,
                           int64_t send_rows)
{
    moe_status_t s = check_tokens(T, k);
    if (s != MOE_OK)
        return s;
    if ((s = check_experts(E, k)) != MOE_OK)
        return s;
    if ((s = check_hidden(H)) != MOE_OK)
        return s;
    int64_t bound = T * (int64_t)k;
    if (capacity >= 0 && (int64_t)E * capacity < bound)
        bound = (int64_t)E * capacity;
    if (send_rows < bound)
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

moe_status_t check_regroup_sizes(int32_t S, int32_t El)
{
    if (S < 1 || El < 1)
        return MOE_ERR_INVALID_ARG;
    if (S > kMaxRegroupSide || El > kMaxRegroupSide || (int64_t)S * El > kMaxRegroupBlocks)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status_t regroup_rows(const uint16_t *src, const int32_t *map, const int32_t *n_rows,
                          int64_t max_rows, int32_t H, bool gather, uint16_t *dst, void *stream)
{
    if (max_rows < 0 || max_rows >= kMaxAssignments)
        return max_rows < 0 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED;
    moe_status_t s = check_hidden(H);
    if (s != MOE_OK)
        return s;
    if (max_rows == 0)
        return MOE_OK;
    if (!src || !map || !n_rows || !dst)
        return MOE_ERR_INVALID_ARG;
    if (!aligned(src, 16) || !aligned(dst, 16) || !aligned(map, 4) || !aligned(n_rows, 4))
        return MOE_ERR_INVALID_ARG;
    return from_hip(moe::launch_regroup_rows(src, map, n_rows, max_rows, H, gather, dst,
                                             static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

moe_status_t moe_route_topk(const float *logits, const float *bias, int64_t T, int32_t E,
                            int32_t k, uint32_t flags, int32_t *topk_idx, float *topk_w,
                            void *stream)
{
    moe_status_t s = check_tokens(T, k);
    if (s != MOE_OK)
        return s;
    if ((s = check_experts(E, k)) != MOE_OK)
        return s;
    if (flags & ~MOE_ROUTE_NORMALIZE)
        return MOE_ERR_INVALID_ARG;
    if (T == 0)
        return MOE_OK;
    if (!logits || !topk_idx || !topk_w)
        return MOE_ERR_INVALID_ARG;
    if (!aligned(logits, 4) || !aligned(bias, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4))
        return MOE_ERR_INVALID_ARG;
    return from_hip(moe::launch_route_topk(logits, bias, T, E, k, 0, 0,
                                           (flags & MOE_ROUTE_NORMALIZE) != 0, topk_idx, topk_w,
                                           static_cast<hipStream_t>(stream)));
}

moe_status_t moe_route_topk_grouped(const float *logits, const float *bias, int64_t T, int32_t E,
                                    int32_t k, int32_t n_groups, int32_t topk_groups,
                                    uint32_t flags, int32_t *topk_idx, float *topk_w,
                                    void *stream)
{
    moe_status_t s = check_tokens(T, k);
    if (s != MOE_OK)
        return s;
    if ((s = check_experts(E, k)) != MOE_OK)
        return s;
    if (flags & ~MOE_ROUTE_NORMALIZE)
        return MOE_ERR_INVALID_ARG;
    if (n_groups < 1 || E % n_groups != 0 || topk_groups < 1 || topk_groups > n_groups ||
        (int64_t)k > (int64_t)topk_groups * (E / n_groups))
        return MOE_ERR_INVALID_ARG;
    if (n_groups > kMaxGroups)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_OK;
    if (!logits || !topk_idx || !topk_w)
        return MOE_ERR_INVALID_ARG;
    if (!aligned(logits, 4) || !aligned(bias, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4))
        return MOE_ERR_INVALID_ARG;
    // every group allowed: plain routing
    const int32_t groups = topk_groups == n_groups ? 0 : n_groups;
    return from_hip(moe::launch_route_topk(logits, bias, T, E, k, groups, topk_groups,
                                           (flags & MOE_ROUTE_NORMALIZE) != 0, topk_idx, topk_w,
                                           static_cast<hipStream_t>(stream)));
}

moe_status_t moe_layout_workspace_size(int64_t T, int32_t E, int32_t k, int32_t R, size_t *bytes)
{
    if (!bytes)
        return MOE_ERR_INVALID_ARG;
    moe_status_t s = check_layout_sizes(T, E, k, R);
    if (s != MOE_OK)
        return s;
    *bytes = moe::layout_workspace_bytes(T * (int64_t)k, E);
    return MOE_OK;
}

moe_status_t moe_dispatch_layout(const int32_t *topk_idx, int64_t T, int32_t E, int32_t k,
                                 int32_t R, int32_t capacity, int32_t *expert_demand,
                                 int32_t *expert_counts, int32_t *expert_offsets,
                                 int32_t *dest_counts, int32_t *dest_offsets, int32_t *pos,
                                 int32_t *send_src, void *workspace, size_t workspace_bytes,
                                 void *stream)
{
    moe_status_t s = check_layout_sizes(T, E, k, R);
    if (s != MOE_OK)
        return s;
    if ((T > 0 && (!topk_idx || !pos)) || !expert_demand || !expert_counts || !expert_offsets ||
        !dest_counts || !dest_offsets)
        return MOE_ERR_INVALID_ARG;
    const void *ptrs[] = {topk_idx,     expert_demand, expert_counts, expert_offsets,
                          dest_counts, dest_offsets,  pos,           send_src};
    for (const void *p : ptrs)
        if (!aligned(p, 4))
            return MOE_ERR_INVALID_ARG;
    const size_t need = moe::layout_workspace_bytes(T * (int64_t)k, E);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
        return MOE_ERR_WORKSPACE;
    return from_hip(moe::launch_dispatch_layout(
        topk_idx, T, E, k, R, capacity, expert_demand, expert_counts, expert_offsets, dest_counts,
        dest_offsets, pos, send_src, static_cast<int32_t *>(workspace),
        static_cast<hipStream_t>(stream)));
}

moe_status_t moe_route_dispatch_layout_workspace_size(int64_t T, int32_t E, int32_t k, int32_t R,
                                                      size_t *bytes)
{
    if (!bytes)
        return MOE_ERR_INVALID_ARG;
    moe_status_t s = check_layout_sizes(T, E, k, R);
    if (s != MOE_OK)
        return s;
    *bytes = moe::route_layout_workspace_bytes(T * (int64_t)k, E);
    return MOE_OK;
}

moe_status_t moe_route_dispatch_layout(const float *logits, const float *bias, int64_t T,
                                       int32_t E, int32_t k, uint32_t flags, int32_t R,
                                       int32_t capacity, int32_t *topk_idx, float *topk_w,
                                       int32_t *expert_demand, int32_t *expert_counts,
                                       int32_t *expert_offsets, int32_t *dest_counts,
                                       int32_t *dest_offsets, int32_t *pos, int32_t *send_src,
                                       void *workspace, size_t workspace_bytes, void *stream)
{
    moe_status_t s = check_layout_sizes(T, E, k, R);
    if (s != MOE_OK)
        return s;
    if (flags & ~MOE_ROUTE_NORMALIZE)
        return MOE_ERR_INVALID_ARG;
    if ((T > 0 && (!logits || !topk_idx || !topk_w || !pos)) || !expert_demand ||
        !expert_counts || !expert_offsets || !dest_counts || !dest_offsets)
        return MOE_ERR_INVALID_ARG;
    const void *ptrs[] = {logits,         bias,        topk_idx,     topk_w,
                          expert_demand,  expert_counts, expert_offsets, dest_counts,
                          dest_offsets,   pos,         send_src};
    for (const void *p : ptrs)
        if (!aligned(p, 4))
            return MOE_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, 16) ||
        workspace_bytes < moe::route_layout_workspace_bytes(T * (int64_t)k, E))
        return MOE_ERR_WORKSPACE;
    return from_hip(moe::launch_route_layout(
        logits, bias, T, E, k, (flags & MOE_ROUTE_NORMALIZE) != 0, R, capacity, topk_idx, topk_w,
        expert_demand, expert_counts, expert_offsets, dest_counts, dest_offsets, pos, send_src,
        workspace, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_dispatch_layout_noalloc(const int32_t *topk_idx, int64_t T, int32_t E, int32_t k,
                                         int32_t R, int32_t capacity, int32_t *expert_demand,
                                         int32_t *expert_counts, int32_t *expert_offsets,
                                         int32_t *dest_counts, int32_t *dest_offsets,
                                         int32_t *pos, int32_t *send_src, void *stream)
{
    moe_status_t s = check_layout_sizes(T, E, k, R);
    if (s != MOE_OK)
        return s;
    if ((T > 0 && (!topk_idx || !pos)) || !expert_demand || !expert_counts || !expert_offsets ||
        !dest_counts || !dest_offsets)
        return MOE_ERR_INVALID_ARG;
    const void *ptrs[] = {topk_idx,     expert_demand, expert_counts, expert_offsets,
                          dest_counts, dest_offsets,  pos,           send_src};
    for (const void *p : ptrs)
        if (!aligned(p, 4))
            return MOE_ERR_INVALID_ARG;
    const size_t need = moe::layout_workspace_bytes(T * (int64_t)k, E);
    if (need > moe::layout_scratch_bytes())
        return MOE_ERR_WORKSPACE;
    int32_t *scratch = nullptr;
    if (need > 0 && moe::layout_scratch(&scratch) != hipSuccess)
        return MOE_ERR_LAUNCH;
    return from_hip(moe::launch_dispatch_layout(
        topk_idx, T, E, k, R, capacity, expert_demand, expert_counts, expert_offsets, dest_counts,
        dest_offsets, pos, send_src, scratch, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_dispatch_permute(const uint16_t *x, const int32_t *pos, int64_t T, int32_t H,
                                  int32_t k, int32_t E, int32_t capacity, uint16_t *send,
                                  int64_t send_rows, void *stream)
{
    moe_status_t s = check_permute(T, H, k, E, capacity, send_rows);
    if (s != MOE_OK)
        return s;
    if (T == 0)
        return MOE_OK;
    if (!x || !pos || (!send && send_rows > 0))
        return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(send, 16) || !aligned(pos, 4))
        return MOE_ERR_INVALID_ARG;
    return from_hip(moe::launch_dispatch_permute(x, pos, T, H, k, send, send_rows,
                                                 static_cast<hipStream_t>(stream)));
}

moe_status_t moe_fp8_row_bytes(int32_t H, int64_t *bytes)
{
    if (!bytes)
        return MOE_ERR_INVALID_ARG;
    moe_status_t s = check_hidden(H);
    if (s != MOE_OK)
        return s;
    if (H % 32 != 0)
        return MOE_ERR_UNSUPPORTED;
    *bytes = moe::fp8_row_bytes(H);
    return MOE_OK;
}

moe_status_t moe_dispatch_permute_fp8(const uint16_t *x, const int32_t *pos, int64_t T,
                                      int32_t H, int32_t k, int32_t E, int32_t capacity,
                                      uint8_t *send, int64_t send_rows, void *stream)
{
    moe_status_t s = check_permute(T, H, k, E, capacity, send_rows);
    if (s != MOE_OK)
        return s;
    if (H % 32 != 0)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0)
        return MOE_OK;
    if (!x || !pos || (!send && send_rows > 0))
        return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(send, 16) || !aligned(pos, 4))
        return MOE_ERR_INVALID_ARG;
    return from_hip(moe::launch_dispatch_permute_fp8(x, pos, T, H, k, send, send_rows,
                                                     static_cast<hipStream_t>(stream)));
}

moe_status_t moe_fp8_dequant(const uint8_t *rows, const int32_t *n_rows, int64_t max_rows,
                             int32_t H, uint16_t *out, void *stream)
{
    if (max_rows < 0)
        return MOE_ERR_INVALID_ARG;
    if (max_rows >= kMaxAssignments)
        return MOE_ERR_UNSUPPORTED;
    moe_status_t s = check_hidden(H);
    if (s != MOE_OK)
        return s;
    if (H % 32 != 0)
        return MOE_ERR_UNSUPPORTED;
    if (max_rows == 0)
        return MOE_OK;
    if (!rows || !out)
        return MOE_ERR_INVALID_ARG;
    if (!aligned(rows, 16) || !aligned(out, 16) || !aligned(n_rows, 4))
        return MOE_ERR_INVALID_ARG;
    return from_hip(moe::launch_fp8_dequant(rows, n_rows, max_rows, H, out,
                                            static_cast<hipStream_t>(stream)));
}

moe_status_t moe_combine_reduce(const uint16_t *y, int64_t y_rows, const int32_t *pos,
                                const float *topk_w, const uint16_t *shared,
                                const uint16_t *residual, int64_t T, int32_t H, int32_t k,
                                uint32_t flags, void *out, void *stream)
{
    moe_status_t s = check_tokens(T, k);
    if (s != MOE_OK)
        return s;
    if ((s = check_hidden(H)) != MOE_OK)
        return s;
    if (y_rows < 0 || (flags & ~MOE_COMBINE_OUT_FP32))
        return MOE_ERR_INVALID_ARG;
    if (T == 0)
        return MOE_OK;
    if (!pos || !topk_w || !out || (!y && y_rows > 0))
        return MOE_ERR_INVALID_ARG;
    if (!aligned(y, 16) || !aligned(shared, 16) || !aligned(residual, 16) || !aligned(out, 16) ||
        !aligned(pos, 4) || !aligned(topk_w, 4))
        return MOE_ERR_INVALID_ARG;
    return from_hip(moe::launch_combine_reduce(y, y_rows, pos, topk_w, shared, residual, T, H, k,
                                               (flags & MOE_COMBINE_OUT_FP32) != 0, out,
                                               static_cast<hipStream_t>(stream)));
}

moe_status_t moe_recv_regroup_workspace_size(int32_t S, int32_t El, size_t *bytes)
{
    if (!bytes)
        return MOE_ERR_INVALID_ARG;
    moe_status_t s = check_regroup_sizes(S, El);
    if (s != MOE_OK)
        return s;
    *bytes = moe::regroup_workspace_bytes(S, El);
    return MOE_OK;
}

moe_status_t moe_recv_regroup_layout(const int32_t *recv_counts, int32_t S, int32_t El,
                                     int32_t *local_expert_offsets, int32_t *source_offsets,
                                     int32_t *recv_pos, int64_t max_rows, void *workspace,
                                     size_t workspace_bytes, void *stream)
{
    moe_status_t s = check_regroup_sizes(S, El);
    if (s != MOE_OK)
        return s;
    if (max_rows < 0)
        return MOE_ERR_INVALID_ARG;
    if (max_rows >= kMaxAssignments)
        return MOE_ERR_UNSUPPORTED;
    if (!recv_counts || !local_expert_offsets || !source_offsets || (max_rows > 0 && !recv_pos))
        return MOE_ERR_INVALID_ARG;
    const void *ptrs[] = {recv_counts, local_expert_offsets, source_offsets, recv_pos};
    for (const void *p : ptrs)
        if (!aligned(p, 4))
            return MOE_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < moe::regroup_workspace_bytes(S, El) ||
        !aligned(workspace, 16))
        return MOE_ERR_WORKSPACE;
    return from_hip(moe::launch_recv_regroup_layout(
        recv_counts, S, El, local_expert_offsets, source_offsets, recv_pos, max_rows,
        static_cast<int32_t *>(workspace), static_cast<hipStream_t>(stream)));
}

moe_status_t moe_recv_regroup(const uint16_t *recv, const int32_t *recv_pos,
                              const int32_t *n_rows, int64_t max_rows, int32_t H,
                              uint16_t *grouped, void *stream)
{
    return regroup_rows(recv, recv_pos, n_rows, max_rows, H, false, grouped, stream);
}

moe_status_t moe_recv_ungroup(const uint16_t *grouped, const int32_t *recv_pos,
                              const int32_t *n_rows, int64_t max_rows, int32_t H, uint16_t *out,
                              void *stream)
{
    return regroup_rows(grouped, recv_pos, n_rows, max_rows, H, true, out, stream);
}

namespace {

moe_status_t check_linear(const uint16_t *recv, const int32_t *cnt, int32_t S, int32_t El,
                          int32_t H, int32_t H_out, const uint16_t *W, int64_t max_rows,
                          const void *y, const void *workspace, size_t workspace_bytes)
{
    moe_status_t s = check_regroup_sizes(S, El);
    if (s != MOE_OK)
        return s;
    if (max_rows < 0)
        return MOE_ERR_INVALID_ARG;
    if (max_rows >= kMaxAssignments)
        return MOE_ERR_UNSUPPORTED;
    if (H <= 0 || H % 64 != 0 || H > kMaxH || H_out <= 0 || H_out % 128 != 0 || H_out > kMaxH)
        return MOE_ERR_UNSUPPORTED;
    if (!cnt || (max_rows > 0 && (!recv || !W || !y)))
        return MOE_ERR_INVALID_ARG;
    if (!aligned(cnt, 4) || !aligned(recv, 16) || !aligned(W, 16) || !aligned(y, 16))
        return MOE_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < moe::expert_linear_workspace_bytes(S, El, max_rows) ||
        !aligned(workspace, 16))
        return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

}  // namespace

moe_status_t moe_expert_linear_workspace_size(int32_t S, int32_t E_l, int64_t max_rows,
                                              size_t *bytes)
{
    if (!bytes || max_rows < 0)
        return MOE_ERR_INVALID_ARG;
    moe_status_t s = check_regroup_sizes(S, E_l);
    if (s != MOE_OK)
        return s;
    if (max_rows >= kMaxAssignments)
        return MOE_ERR_UNSUPPORTED;
    *bytes = moe::expert_linear_workspace_bytes(S, E_l, max_rows);
    return MOE_OK;
}

moe_status_t moe_expert_linear(const uint16_t *recv, const int32_t *recv_counts, int32_t S,
                               int32_t E_l, int32_t H, int32_t H_out, const uint16_t *W,
                               int64_t max_rows, uint16_t *y, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    moe_status_t s = check_linear(recv, recv_counts, S, E_l, H, H_out, W, max_rows, y, workspace,
                                  workspace_bytes);
    if (s != MOE_OK)
        return s;
    return from_hip(moe::launch_expert_linear(recv, recv_counts, S, E_l, H, H_out, W, max_rows, y,
                                              static_cast<int32_t *>(workspace),
                                              static_cast<hipStream_t>(stream)));
}

moe_status_t moe_expert_linear_return(const uint16_t *recv, const int32_t *recv_counts,
                                      int32_t S, int32_t E_l, int32_t H, int32_t H_out,
                                      const uint16_t *W, int64_t max_rows, int32_t self_rank,
                                      int32_t consumer_blocks, int32_t band_group, uint16_t *y,
                                      uint16_t *ret, void *workspace, size_t workspace_bytes,
                                      void *stream)
{
    moe_status_t s = check_linear(recv, recv_counts, S, E_l, H, H_out, W, max_rows, y, workspace,
                                  workspace_bytes);
    if (s != MOE_OK)
        return s;
    if (self_rank < 0 || self_rank >= S || consumer_blocks < 0 || band_group < 1)
        return MOE_ERR_INVALID_ARG;
    if (max_rows > 0 && (!ret || !aligned(ret, 16)))
        return MOE_ERR_INVALID_ARG;
    int slots = 0;
    if (moe::expert_return_slots(&slots) != hipSuccess)
        return MOE_ERR_LAUNCH;
    if (consumer_blocks >= slots)
        return MOE_ERR_UNSUPPORTED;
    int32_t grid = 0;
    return from_hip(moe::launch_expert_return(
        recv, recv_counts, S, E_l, H, H_out, W, max_rows, self_rank, consumer_blocks, band_group,
        y, ret, static_cast<int32_t *>(workspace), static_cast<hipStream_t>(stream), &grid));
}

moe_status_t moe_expert_return_slots(int32_t *slots)
{
    if (!slots)
        return MOE_ERR_INVALID_ARG;
    int n = 0;
    if (moe::expert_return_slots(&n) != hipSuccess)
        return MOE_ERR_LAUNCH;
    *slots = n;
    return MOE_OK;
}

moe_status_t moe_hbm_floor(const void *src, int64_t read_bytes, void *dst, int64_t write_bytes,
                           uint32_t flags, void *stream)
{
    if (read_bytes < 0 || write_bytes < 0 || read_bytes % 16 || write_bytes % 16 ||
        (flags & ~MOE_FLOOR_NT_STORE))
        return MOE_ERR_INVALID_ARG;
    if ((read_bytes > 0 && (!src || !aligned(src, 16))) ||
        (write_bytes > 0 && (!dst || !aligned(dst, 16))))
        return MOE_ERR_INVALID_ARG;
    return from_hip(moe::launch_hbm_floor(src, read_bytes, dst, write_bytes,
                                          (flags & MOE_FLOOR_NT_STORE) != 0,
                                          static_cast<hipStream_t>(stream)));
}

const char *moe_status_string(moe_status_t status)
{
    switch (status) {
    case MOE_OK:
        return "MOE_OK";
    case MOE_ERR_INVALID_ARG:
        return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED:
        return "MOE_ERR_UNSUPPORTED: size outside the supported limits";
    case MOE_ERR_WORKSPACE:
        return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_LAUNCH:
        return "MOE_ERR_LAUNCH: kernel launch failed";
    default:
        break;
    }
    return "unknown moe_status_t";
}

}  // extern "C"
