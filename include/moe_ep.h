/*
 * moe_ep.h -- C ABI of the MoE expert-parallel dispatch/combine core, one
 * rank's share, for AMD Instinct MI355X (gfx950).
 *
 * The library performs the data-parallel steps around the two all-to-all
 * exchanges of an expert-parallel MoE layer: routing, the per-destination
 * counts and offsets, packing each destination's rows contiguously, and
 * the gate-weighted reduction when the expert outputs return. The R
 * destinations are logical partitions of one device buffer; the library
 * performs no inter-GPU transfer.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller. The
 *    library never allocates, frees or keeps a pointer after returning.
 *  - Every call only enqueues work on `stream` (a hipStream_t passed as
 *    void*; NULL is the null stream). No call synchronises the device or
 *    reads device memory from the host, so routing results never make a
 *    round trip through the host.
 *  - bf16 tensors are passed as uint16_t bit patterns, row-major.
 *  - Every scalar, required pointer and alignment is validated on the host
 *    before anything is enqueued; on error nothing is enqueued, outputs are
 *    untouched and the status says why. After a launch, a HIP launch error
 *    is reported as MOE_ERR_LAUNCH. No exception crosses the ABI and there
 *    is no global error state.
 *  - T = 0 is legal: the call enqueues nothing, except moe_dispatch_layout,
 *    which still writes its (all-zero) counts and offsets.
 *  - Results are bitwise reproducible from run to run: no floating-point
 *    atomics, integer atomics only where their order cannot matter.
 *  - Limits: 1 <= k <= min(E, 32); 1 <= E <= 1024; E % R == 0; H % 8 == 0;
 *    0 < H <= 65536; T * k < 2^31.
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,  /* NULL/misaligned pointer, bad size or relation */
    MOE_ERR_UNSUPPORTED = 2,  /* outside the limits above */
    MOE_ERR_WORKSPACE = 3,    /* workspace missing or too small */
    MOE_ERR_LAUNCH = 4,       /* the HIP runtime rejected a kernel launch */
    /* not a status: gives the type the range of a 32-bit int, so that any
       int value passed as a moe_status_t (moe_status_string of an unknown
       code) is a valid value of the type in C++ as well as in C */
    MOE_STATUS_RANGE_MIN = -0x7FFFFFFF - 1,
    MOE_STATUS_RANGE_MAX = 0x7FFFFFFF
} moe_status_t;

/* moe_route_topk flags */
#define MOE_ROUTE_NORMALIZE 1u   /* weights renormalised over the k selected */

/* moe_combine_reduce flags */
#define MOE_COMBINE_OUT_FP32 1u  /* out is float[T][H] instead of bf16[T][H] */

/*
 * moe_route_topk -- pick k experts per token and their gate weights.
 *
 * Defined by: ai-from-scratch "19. All-to-all", intro (after attention every
 * token holds a list of expert ids; results are mixed on return) and "Why
 * the router can ruin your day" (a per-expert balancing bias takes part in
 * the top-k decision only, never in the mix weights); aicassindra
 * "gpu_moe_all_to_all", "Two collectives per layer, and what each one
 * moves" (outputs are scaled by the router's gate weights).
 *
 * For each token t:
 *   s[e] = logits[t][e] + bias[e]   (one float32 add; bias may be NULL)
 *   topk_idx[t][0..k-1] = the k experts with the largest s, in descending
 *     order; -0 equals +0; any NaN ranks below every number (including
 *     -inf); ties go to the smaller expert id.
 *   topk_w[t][j] from the UNBIASED logits l of the selected experts:
 *     flags & MOE_ROUTE_NORMALIZE: w_j = exp(l_j - m) / sum_i exp(l_i - m)
 *       over the k selected (m = their max); the weights sum to 1.
 *     otherwise: w_j = exp(l_j - M) / sum over all E of exp(l_e - M)
 *       (softmax over all experts, not renormalised).
 *   Weights are computed in float32; for NaN or infinite logits they are
 *   unspecified.
 *
 * Arguments:
 *   logits   [T][E] float32, 4-byte aligned.
 *   bias     [E] float32 or NULL (selection only).
 *   topk_idx [T][k] int32 out;  topk_w [T][k] float32 out.
 * Errors: MOE_ERR_INVALID_ARG for NULL/misaligned pointers or T < 0;
 *   MOE_ERR_UNSUPPORTED outside the limits.
 */
moe_status_t moe_route_topk(const float *logits, const float *bias,
                            int64_t T, int32_t E, int32_t k, uint32_t flags,
                            int32_t *topk_idx, float *topk_w, void *stream);

/*
 * moe_route_topk_grouped -- group-limited routing: each token may use at
 * most topk_groups of n_groups contiguous expert groups (destination groups
 * such as nodes), then picks its k experts inside them.
 *
 * Defined by: ai-from-scratch "19. All-to-all", "DeepSeek's numbers" (each
 * token limited to at most 4 nodes, so the slow hop stays bounded) and the
 * closing section (node-limited routing as an architectural constraint);
 * zenaique Q&A "moe-hide-alltoall-techniques" (node-limited routing caps
 * cross-node traffic). The pages do not define a group's score; this call
 * ranks groups by their best selection score s[e] (as moe_route_topk orders
 * experts, so ties go to the lower group), keeps the best topk_groups, and
 * selects the k best experts among them. Gate weights are computed exactly
 * as in moe_route_topk, from the selected experts' unbiased logits.
 *
 * Arguments: as moe_route_topk, plus
 *   n_groups    groups of E / n_groups experts each; E % n_groups == 0,
 *               1 <= n_groups <= 64.
 *   topk_groups 1 <= topk_groups <= n_groups and
 *               k <= topk_groups * (E / n_groups).
 *   topk_groups == n_groups is plain moe_route_topk.
 * Errors: MOE_ERR_INVALID_ARG for bad pointers or group sizes;
 *   MOE_ERR_UNSUPPORTED outside the limits (n_groups > 64 included).
 */
moe_status_t moe_route_topk_grouped(const float *logits, const float *bias,
                                    int64_t T, int32_t E, int32_t k,
                                    int32_t n_groups, int32_t topk_groups,
                                    uint32_t flags, int32_t *topk_idx,
                                    float *topk_w, void *stream);

/*
 * moe_layout_workspace_size -- bytes of device workspace that
 * moe_dispatch_layout needs for these sizes (written to *bytes). The
 * workspace needs no initialisation: the layout call clears what it uses,
 * on-stream.
 * Errors: as moe_dispatch_layout's size checks; *bytes untouched on error.
 */
moe_status_t moe_layout_workspace_size(int64_t T, int32_t E, int32_t k,
                                       int32_t R, size_t *bytes);

/*
 * moe_dispatch_layout -- per-expert and per-destination counts, the offset
 * table, capacity drops in token order, and every replica's send row.
 *
 * Defined by: aicassindra "gpu_moe_all_to_all", "Two collectives per layer"
 * (per-destination counts precede the payload so that receivers can size
 * their buffers) and "Bucketing: cut the message count, not the byte count"
 * (sort by destination and build an offset table so that each destination
 * is one contiguous segment; keep indices and counts on the device);
 * "MoE All-to-All Dispatch and Ragged Routing", "Fixed Capacity vs. Ragged
 * Routing" (per-sender-expert slots under a capacity factor, the excess
 * dropped; ragged routing is dropless); ai-from-scratch "19. All-to-all",
 * "Why the router can ruin your day" (a dropped token counts as having
 * skipped that expert).
 *
 * Expert e lives on destination e / (E / R). With a = t * k + j:
 *   expert_demand[e]  = #{a : topk_idx[a] == e}
 *   rank(a)           = #{a' < a : topk_idx[a'] == topk_idx[a]}
 *   kept(a)           = capacity < 0 || rank(a) < capacity
 *   expert_counts[e]  = kept replicas of e = min(demand, capacity)
 *   expert_offsets    = exclusive prefix sum of counts, E + 1 entries;
 *                       expert_offsets[E] = N, the kept total
 *   dest_counts[r]    = sum of counts of r's experts
 *   dest_offsets[r]   = expert_offsets[r * E / R]; dest_offsets[R] = N
 *   pos[a]            = expert_offsets[e] + rank(a) if kept, else -1
 *   send_src[pos[a]]  = t for every kept a (send_src may be NULL)
 * The send rows are thereby grouped by destination, then by expert, then
 * by token. N stays on the device (expert_offsets[E]).
 *
 * Arguments:
 *   topk_idx  [T][k] int32 expert ids. Precondition: every id in [0, E)
 *             and distinct within a row; ids outside [0, E) are ignored
 *             (not counted, pos = -1).
 *   capacity  < 0: dropless; >= 0: at most `capacity` rows per expert.
 *   outputs   int32 arrays of the sizes above; send_src, when given,
 *             holds at least N entries: T * k when dropless, else
 *             min(T * k, E * capacity) (entries >= N are not written).
 *   workspace device memory of at least moe_layout_workspace_size() bytes,
 *             16-byte aligned; its contents on entry do not matter.
 * Errors: MOE_ERR_INVALID_ARG for NULL/misaligned pointers, T < 0, R < 1 or
 *   E % R != 0; MOE_ERR_UNSUPPORTED outside the limits; MOE_ERR_WORKSPACE
 *   when the workspace is NULL or too small.
 */
moe_status_t moe_dispatch_layout(const int32_t *topk_idx, int64_t T,
                                 int32_t E, int32_t k, int32_t R,
                                 int32_t capacity, int32_t *expert_demand,
                                 int32_t *expert_counts,
                                 int32_t *expert_offsets, int32_t *dest_counts,
                                 int32_t *dest_offsets, int32_t *pos,
                                 int32_t *send_src, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * moe_route_dispatch_layout -- moe_route_topk followed by
 * moe_dispatch_layout (no group limit), in one call: the same outputs, bit
 * for bit, with fewer launches for small batches.
 *
 * Defined by: the two calls' passages above, and aicassindra
 * "gpu_moe_all_to_all", "Latency-bound at decode, bandwidth-bound at
 * prefill" (at decode sizes the exchange is bound by latency: cut the
 * independent steps and synchronisation points, not the bytes).
 *
 * When T * k <= 4096, E <= 512, E % 4 == 0 and logits and bias are 16-byte
 * aligned, one kernel launch does both: its blocks route their tokens, and
 * the last block to finish (an atomic ticket in the first 16 bytes of the
 * workspace; no block waits for another) builds the layout from the ids the
 * others wrote. Otherwise the call launches the routing and the layout
 * kernels as the two separate calls do.
 *
 * Arguments: those of moe_route_topk (logits, bias, flags, topk_idx,
 *   topk_w) and of moe_dispatch_layout (R, capacity and its outputs), plus
 *   workspace  device memory of at least
 *              moe_route_dispatch_layout_workspace_size() bytes (16 or
 *              more), 16-byte aligned. Its contents on entry do not
 *              matter, with one exception: a call on a workspace its
 *              predecessor did not leave ready counts arrivals with a
 *              slower, stamp-keyed protocol, and every call leaves it
 *              ready; the exception is a first 64-bit word whose upper
 *              half holds the ready pattern 0x6D6F6574 and whose lower
 *              half is not 0 (no call leaves it so), which the call would
 *              take as arrivals already counted. Calls that overlap in
 *              time must not share a workspace.
 * Errors: those of the two calls; MOE_ERR_WORKSPACE when the workspace is
 *   NULL, misaligned or too small.
 */
moe_status_t moe_route_dispatch_layout_workspace_size(int64_t T, int32_t E,
                                                      int32_t k, int32_t R,
                                                      size_t *bytes);
moe_status_t moe_route_dispatch_layout(const float *logits, const float *bias,
                                       int64_t T, int32_t E, int32_t k,
                                       uint32_t flags, int32_t R,
                                       int32_t capacity, int32_t *topk_idx,
                                       float *topk_w, int32_t *expert_demand,
                                       int32_t *expert_counts,
                                       int32_t *expert_offsets,
                                       int32_t *dest_counts,
                                       int32_t *dest_offsets, int32_t *pos,
                                       int32_t *send_src, void *workspace,
                                       size_t workspace_bytes, void *stream);

/*
 * moe_dispatch_layout_noalloc -- moe_dispatch_layout with no workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments (minus workspace), outputs and errors. The call allocates
 * nothing: the per-tile histograms live in a device array of
 * MOE_LAYOUT_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; every legal size fits (sizes whose
 * moe_layout_workspace_size() exceeds it would return MOE_ERR_WORKSPACE).
 * All calls on one GPU share that array, and every call rewrites what it
 * reads, so nothing carries over from the previous call; calls that overlap
 * on one GPU (different streams, host threads) race on it and must be
 * serialised by the caller. MOE_ERR_LAUNCH also covers a failure to look
 * up the array's device address (once per device, on the first call).
 */
#define MOE_LAYOUT_SCRATCH_BYTES (128u * 1024u * 4u)
moe_status_t moe_dispatch_layout_noalloc(const int32_t *topk_idx, int64_t T,
                                         int32_t E, int32_t k, int32_t R,
                                         int32_t capacity, int32_t *expert_demand,
                                         int32_t *expert_counts,
                                         int32_t *expert_offsets,
                                         int32_t *dest_counts,
                                         int32_t *dest_offsets, int32_t *pos,
                                         int32_t *send_src, void *stream);

/*
 * moe_dispatch_permute -- pack each kept replica of each token into its
 * send row: send[pos[t][j]][:] = x[t][:] (a bit copy of the bf16 row).
 *
 * Defined by: aicassindra "gpu_moe_all_to_all", "Bucketing" (permute so that
 * everything bound for one destination is contiguous, fused into the
 * staging kernel) and "Two collectives per layer" (each token goes out k
 * times); thecoregrid "Mixture-of-experts acceleration through overlap",
 * paragraph on the remote-owner-aligned layout (each block of rows belongs
 * to one destination, so it leaves as one contiguous write).
 *
 * Arguments:
 *   x         [T][H] bf16, 16-byte aligned.
 *   pos       [T][k] int32 from moe_dispatch_layout (-1 = dropped).
 *   E, capacity  the expert count and capacity given to moe_dispatch_layout;
 *             they fix the bound on the kept rows N: T * k when dropless
 *             (capacity < 0), min(T * k, E * capacity) otherwise.
 *   send      [send_rows][H] bf16 out, 16-byte aligned, send_rows >= that
 *             bound. Rows that no replica points at are not written.
 *             Positions >= send_rows (a broken precondition on pos) are
 *             skipped, never written out of bounds.
 * Errors: MOE_ERR_INVALID_ARG for NULL/misaligned pointers, T < 0, or
 *   send_rows below the bound; MOE_ERR_UNSUPPORTED outside the limits.
 */
moe_status_t moe_dispatch_permute(const uint16_t *x, const int32_t *pos,
                                  int64_t T, int32_t H, int32_t k, int32_t E,
                                  int32_t capacity, uint16_t *send,
                                  int64_t send_rows, void *stream);

/*
 * moe_combine_reduce -- bring each token's k expert outputs back along the
 * inverse permutation and reduce them at the origin:
 *   out[t][h] = round( sum_{j : pos[t][j] >= 0} topk_w[t][j] * y[pos[t][j]][h]
 *                      + shared[t][h] + residual[t][h] )
 * accumulated in float32 with one fused multiply-add per kept replica in
 * ascending j, then + shared, then + residual, and one final rounding to
 * bf16 (nearest, ties to even) unless MOE_COMBINE_OUT_FP32 is set. Dropped
 * replicas contribute nothing; the other weights are not renormalised.
 *
 * Defined by: aicassindra "gpu_moe_all_to_all", "Two collectives per layer"
 * (outputs return along the inverse permutation, k partial results per
 * token, scaled by the gate weights at the origin); "MoE All-to-All
 * Dispatch and Ragged Routing", "Returning Tokens to the Original GPU" (the
 * residual x + dx is formed at the origin); ai-from-scratch "19.
 * All-to-all", section on 512 experts (10 routed + 1 always-active shared
 * expert) and "Why the router can ruin your day" (drops).
 *
 * Arguments:
 *   y         [y_rows][H] bf16 expert outputs in send layout, 16-byte
 *             aligned (may alias the send buffer of moe_dispatch_permute).
 *   pos       [T][k] int32; positions >= y_rows are skipped (a broken
 *             precondition, never a read out of bounds).
 *   topk_w    [T][k] float32.
 *   shared    [T][H] bf16 shared-expert output or NULL (weight 1).
 *   residual  [T][H] bf16 or NULL.
 *   out       [T][H] bf16, or float32 with MOE_COMBINE_OUT_FP32; 16-byte
 *             aligned; must not alias any input.
 * Errors: MOE_ERR_INVALID_ARG for NULL/misaligned pointers, T < 0,
 *   y_rows < 0; MOE_ERR_UNSUPPORTED outside the limits.
 */
moe_status_t moe_combine_reduce(const uint16_t *y, int64_t y_rows,
                                const int32_t *pos, const float *topk_w,
                                const uint16_t *shared,
                                const uint16_t *residual, int64_t T,
                                int32_t H, int32_t k, uint32_t flags,
                                void *out, void *stream);

/*
 * FP8 dispatch payload: the permute quantises each row as it packs it, so
 * the send buffer holds about half the bytes of the bf16 one.
 *
 * Defined by: aicassindra "gpu_moe_all_to_all", "Latency-bound at decode,
 * bandwidth-bound at prefill" (send fewer bytes: a lower-precision dispatch
 * payload, because the expert matmul casts its input anyway) and
 * "Bucketing" (the permutation fused into the staging kernel); zenaique Q&A
 * "moe-hide-alltoall-techniques" (shrink the payload). The pages fix no
 * format; this library's reading:
 *   - codes: OCP FP8 E4M3 (bias 7, largest finite 448, no infinities);
 *   - scales: one power of two 2^e per 32 consecutive values of a row,
 *     stored as the byte e + 127 (E8M0); e is the smallest integer >= -127
 *     with max|x| <= 448 * 2^e, so no value saturates;
 *   - code = the E4M3 value nearest to x / 2^e, ties to even (x / 2^e is
 *     exact, so the code does not depend on arithmetic precision);
 *   - a send row: H code bytes, then one 128-byte line per 4096 values
 *     holding that slab's 128 scale bytes, zero-padded in the last slab:
 *     moe_fp8_row_bytes(H) = H + 128 * ceil(H / 4096). For H % 128 == 0
 *     rows start on 128-byte lines and are written in whole lines; a
 *     destination's segment is still one contiguous range of rows.
 * NaN or infinite inputs give unspecified codes and scales.
 */

/* Bytes of one FP8 send row (written to *bytes). Needs H % 32 == 0. */
moe_status_t moe_fp8_row_bytes(int32_t H, int64_t *bytes);

/*
 * moe_dispatch_permute_fp8 -- as moe_dispatch_permute, but row pos[t][j] of
 * send ([send_rows][moe_fp8_row_bytes(H)] bytes, 16-byte aligned) receives
 * the FP8 codes, scale bytes and zero padding of x[t]. Rows no kept
 * assignment points at are left as they were. send_rows must cover the
 * same bound as in moe_dispatch_permute.
 * Errors: as moe_dispatch_permute; MOE_ERR_UNSUPPORTED when H % 32 != 0.
 */
moe_status_t moe_dispatch_permute_fp8(const uint16_t *x, const int32_t *pos, int64_t T,
                                      int32_t H, int32_t k, int32_t E, int32_t capacity,
                                      uint8_t *send, int64_t send_rows, void *stream);

/*
 * moe_fp8_dequant -- decode FP8 rows to bf16 (for an expert that takes
 * bf16, or to check a payload):
 *   out[i][h] = bf16 nearest to value(code[i][h]) * 2^(scale[i][h/32] - 127)
 * (ties to even; exact unless below bf16's subnormal spacing) for
 * i < min(*n_rows, max_rows), or i < max_rows when n_rows is NULL (n_rows
 * is a device pointer, e.g. expert_offsets + E). rows: [max_rows]
 * [moe_fp8_row_bytes(H)] bytes; out: [max_rows][H] bf16; both 16-byte
 * aligned. NaN codes give unspecified values.
 * Errors: MOE_ERR_INVALID_ARG (pointers, alignment, max_rows < 0),
 *   MOE_ERR_UNSUPPORTED (H limits, H % 32 != 0, max_rows >= 2^31).
 */
moe_status_t moe_fp8_dequant(const uint8_t *rows, const int32_t *n_rows, int64_t max_rows,
                             int32_t H, uint16_t *out, void *stream);

/*
 * Receive side: regroup a destination's receive buffer into expert-major
 * rows for the expert computation, and back for the return path.
 *
 * Defined by: aicassindra "gpu_moe_all_to_all", "Two collectives per layer"
 * (per-destination counts arrive before the payload so that the receiver
 * can size and place it; outputs return along the inverse permutation) and
 * "Bucketing" (one contiguous message per peer); "MoE All-to-All Dispatch
 * and Ragged Routing", "Why MoE Token Dispatch is All-to-All" (a GPU holds a
 * few of the experts) and "Fixed Capacity vs. Ragged Routing" (variable-
 * length exchange, the receiver pooling its local experts).
 *
 * The receive buffer is the concatenation, in source order, of one segment
 * per source s; each segment holds recv_counts[s][l] rows of local expert l
 * (l ascending), i.e. rows dest_offsets[r]..dest_offsets[r+1] of that
 * source's send buffer and expert_counts[r*E_l + l] of its counts. With
 * N = sum of recv_counts:
 *   local_expert_offsets[l] = rows of local experts < l     (E_l + 1 entries)
 *   source_offsets[s]       = rows of sources < s           (S + 1 entries)
 *   recv_pos[i]             = expert-major row of received row i: the block
 *                             (s, l) holding row i starts at
 *                             local_expert_offsets[l] + sum_{s' < s} recv_counts[s'][l]
 * so each local expert's rows are contiguous, sources in order within it.
 * N stays on the device: local_expert_offsets[E_l] == source_offsets[S].
 */

/* Workspace bytes for moe_recv_regroup_layout (written to *bytes). */
moe_status_t moe_recv_regroup_workspace_size(int32_t S, int32_t E_l, size_t *bytes);

/*
 * moe_recv_regroup_layout -- the offsets and recv_pos above.
 *   recv_counts [S][E_l] int32 (device; negative entries count as 0).
 *   recv_pos    [max_rows] int32; entries past N are not written, and rows
 *               past max_rows are not placed (a broken precondition when
 *               N > max_rows).
 *   workspace   moe_recv_regroup_workspace_size() bytes, 16-byte aligned;
 *               contents on entry do not matter.
 * Limits: 1 <= S, E_l <= 1024 and S * E_l <= 4096; max_rows < 2^31.
 * Device-side precondition: the counts total less than 2^31.
 * Errors: MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE.
 */
moe_status_t moe_recv_regroup_layout(const int32_t *recv_counts, int32_t S, int32_t E_l,
                                     int32_t *local_expert_offsets,
                                     int32_t *source_offsets, int32_t *recv_pos,
                                     int64_t max_rows, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * moe_recv_regroup -- grouped[recv_pos[i]][:] = recv[i][:] for i < N (bit
 * copies of bf16 rows). n_rows points at N on the device (for example
 * source_offsets + S); max_rows bounds the grid and both buffers' rows.
 * recv and grouped are [max_rows][H] bf16, 16-byte aligned, not aliased.
 * moe_recv_ungroup -- the inverse for the return path:
 *   out[i][:] = grouped[recv_pos[i]][:] for i < N,
 * after which out is in receive order again and segment s goes back to
 * source s, landing in exactly the rows that source's combine reads.
 * Positions outside [0, max_rows) are skipped, never accessed.
 * Errors: MOE_ERR_INVALID_ARG (pointers, alignment, max_rows < 0),
 *   MOE_ERR_UNSUPPORTED (H limits, max_rows >= 2^31).
 */
moe_status_t moe_recv_regroup(const uint16_t *recv, const int32_t *recv_pos,
                              const int32_t *n_rows, int64_t max_rows, int32_t H,
                              uint16_t *grouped, void *stream);
moe_status_t moe_recv_ungroup(const uint16_t *grouped, const int32_t *recv_pos,
                              const int32_t *n_rows, int64_t max_rows, int32_t H,
                              uint16_t *out, void *stream);

/*
 * Tile-signalled return: a stand-in expert computation on a destination's
 * receive buffer whose output tiles are returned to their sources as soon
 * as they are ready.
 *
 * Defined by: thecoregrid "Mixture-of-experts acceleration through
 * overlap" (a producer GEMM and a consumer synchronised per tile: the GEMM
 * epilogue publishes a readiness flag per tile, and the consumer starts a
 * transfer once enough row bands are ready, several bands per transfer;
 * each tile belongs to one destination, the remote-owner-aligned layout,
 * and remote tiles are computed first; compute units are split between the
 * roles); aicassindra "gpu_moe_all_to_all", "Overlapping dispatch with
 * expert compute" (dispatch, compute and combine form a strict chain).
 *
 * The receive buffer recv [max_rows][H] bf16 is laid out as in
 * moe_recv_regroup_layout: S source segments in order, each holding
 * recv_counts[s][l] rows of local expert l, l ascending. The stand-in
 * expert is one linear map per local expert, W [E_l][H_out][H] bf16
 * (output-major, as a linear layer's weight):
 *   y[i][o] = bf16( sum_h recv[i][h] * W[l][o][h] )
 * accumulated in fp32 (MFMA) and rounded once, to nearest even, for every
 * row i < N = sum of the counts (rows past N are not written). Tiles are
 * 128 rows of one (source, expert) block by 512 output columns (the last
 * narrower when H_out % 512 != 0), so every tile goes back to exactly one
 * source.
 *
 * Limits: as moe_recv_regroup_layout for S and E_l; H % 64 == 0,
 * H_out % 128 == 0, both <= 65536; max_rows < 2^31. Buffers 16-byte
 * aligned; recv, W, y and ret do not overlap. Device-side precondition:
 * N <= max_rows. If it fails, nothing is computed and the status word
 * (below) reads 2.
 *
 * Workspace: moe_expert_linear_workspace_size() bytes, 16-byte aligned.
 * Its first int32 is a status word, which the caller may read after the
 * call completes: 0 = done; 1 = a consumer wait exceeded its bound and
 * some rows of ret were not returned; 2 = counts total more than max_rows.
 */
moe_status_t moe_expert_linear_workspace_size(int32_t S, int32_t E_l, int64_t max_rows,
                                              size_t *bytes);

/* moe_expert_linear -- y only, as one grouped GEMM launch (the schedule
 * without overlap: the return starts after it completes). */
moe_status_t moe_expert_linear(const uint16_t *recv, const int32_t *recv_counts, int32_t S,
                               int32_t E_l, int32_t H, int32_t H_out, const uint16_t *W,
                               int64_t max_rows, uint16_t *y, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * moe_expert_linear_return -- y as above, and ret [max_rows][H_out] bf16
 * with ret[i] = y[i] for i < N: the rows returned to their sources (on one
 * device the sources' return buffers are partitions of ret, in the same
 * row positions, so moe_combine_reduce reads ret unchanged).
 *
 * One cooperative launch of moe_expert_return_slots() blocks, all resident.
 *   - Work units (a band -- the 128-row tile of one (source, expert) block --
 *     by one 512-column tile) go in remote-first order: sources
 *     self_rank+1, self_rank+2, ... (mod S), self_rank last.
 *   - After each unit a producer release-adds one to the band's count of
 *     column tiles.
 *   - A task is up to band_group consecutive bands of one source: one
 *     contiguous copy of rows from y to ret.
 * consumer_blocks > 0: that many blocks only return rows. Each takes tasks
 *   in order, waits until every band of the task has all its column tiles,
 *   and copies it. Every wait is bounded; on expiry the status word reads 1
 *   and that task is skipped, so no call hangs.
 * consumer_blocks == 0: every block computes. The unit that completes a
 *   band counts it toward its task, and the block that completes a task's
 *   last band copies the task itself. Nothing waits.
 * Errors: as moe_expert_linear; MOE_ERR_INVALID_ARG for self_rank outside
 *   [0, S), consumer_blocks < 0 or band_group < 1; MOE_ERR_UNSUPPORTED when
 *   consumer_blocks >= moe_expert_return_slots().
 */
moe_status_t moe_expert_linear_return(const uint16_t *recv, const int32_t *recv_counts,
                                      int32_t S, int32_t E_l, int32_t H, int32_t H_out,
                                      const uint16_t *W, int64_t max_rows, int32_t self_rank,
                                      int32_t consumer_blocks, int32_t band_group, uint16_t *y,
                                      uint16_t *ret, void *workspace, size_t workspace_bytes,
                                      void *stream);

/* Blocks of one moe_expert_linear_return launch on the current device
 * (resident blocks per compute unit x compute units). */
moe_status_t moe_expert_return_slots(int32_t *slots);

/* moe_hbm_floor flags */
#define MOE_FLOOR_NT_STORE 1u  /* stores carry the non-temporal hint */

/*
 * moe_hbm_floor -- the synthetic floor: read read_bytes from src and write
 * write_bytes to dst, both contiguous, with the 16-byte lane accesses of
 * the row kernels and nothing else (no gather, scatter or index). Timed
 * beside a call of the path with that call's read and write volumes, it is
 * the rate the memory system reaches for the same bytes; the gap is
 * overhead the path owns.
 *
 * Defined by: aicassindra "gpu_moe_all_to_all", "How to tell whether the
 * all-to-all is your bottleneck" (time a synthetic transfer of the same
 * sizes and compare).
 *
 * Arguments: src [read_bytes], dst [write_bytes], 16-byte aligned, not
 *   overlapping; sizes multiples of 16. dst receives the first write_bytes
 *   of src (a constant pattern past read_bytes); the contents are not part
 *   of the contract.
 * Errors: MOE_ERR_INVALID_ARG for negative or unaligned sizes, NULL or
 *   misaligned pointers with a non-zero size, or unknown flags.
 */
moe_status_t moe_hbm_floor(const void *src, int64_t read_bytes, void *dst,
                           int64_t write_bytes, uint32_t flags, void *stream);

/* moe_status_string -- a static, human-readable name for a status. */
const char *moe_status_string(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EP_H */
