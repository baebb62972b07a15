// route_layout.hip -- routing and the dispatch layout of a small batch in
// one kernel launch.
//
// Method: aicassindra "gpu_moe_all_to_all", "Latency-bound at decode,
// bandwidth-bound at prefill" (at decode sizes the exchange is bound by
// latency, so cut the number of independent steps and synchronisation
// points rather than bytes) and "Two collectives per layer" (the counts are
// tiny in bytes and latency-critical). The results are those of
// moe_route_topk followed by moe_dispatch_layout; only the launch structure
// differs.
//
// At decode sizes each kernel of the path costs a few microseconds of
// launch, first-load and drain latency whatever its work, so routing and
// layout share one launch when the batch has at most kSmallAssignments
// assignments (E <= 512, 16-byte rows):
//  * every block routes its tokens exactly as route_topk_kernel does (one
//    wave per 1..16 tokens, all blocks in parallel);
//  * after a block barrier, thread 0 arrives at a ticket in the caller's
//    workspace with one device-scope read-modify-write in acquire-release
//    order: its release makes the block's ids and weights visible on the
//    device, and the block that arrives last (an atomic count, no waiting)
//    acquires every other block's through the same read-modify-write, then
//    builds the whole layout with the one-block layout's passes over its 8
//    waves. A separate fence before the arrival and another after it would
//    only repeat the L2 write-back and invalidate that the read-modify-write
//    already performs: with them the decode call took 7.6-7.8 us back to
//    back, without them 7.2-7.4 us.
// Nothing waits on another block, so there is no co-residency requirement
// and no spin. The ticket is two 64-bit words:
//  * word 0, the fast path: one atomic add per block. It is valid when its
//    upper half holds kTicketMagic (the lower half then counts arrivals
//    from zero); the last block writes it back to kTicketMagic << 32, so
//    every call leaves it ready and a captured HIP graph replays cleanly.
//  * word 1, the slow path, taken by every block when word 0 does not hold
//    the magic (a new or reused workspace): a compare-and-swap count keyed
//    by a per-call stamp in its upper half, so whatever the word held, the
//    first block of the call starts the count afresh. Its last block also
//    writes word 0 ready. A compare-and-swap count costs one serialised
//    round trip per block (at 32 blocks it took 27 us against 11 us for the
//    atomic add), which is why it is only the fallback.
#include "launch.hpp"
#include "layout_device.hpp"
#include "route_device.hpp"

#include <atomic>

namespace moe {
namespace {

// Eight waves per block: at the decode workload (128 tokens, 256 experts,
// top-8; one wave per token) 16 blocks route and the last runs the layout
// with 8 waves. On MI355X the call took 8.2 us with 8 waves per block,
// 9.5 us with 4 (32 blocks, a 4-wave layout); the two separate kernels
// take 8.4-9.4 us back to back. At the tiny workload (256 tokens, 16
// experts, top-2) the one launch takes 6.0-6.6 us against 8.9-9.5.
constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = kFusedWaves * kWave;
constexpr unsigned long long kTicketMagic = 0x6D6F6574ull;  // word 0 ready: upper half

// Arrival of one block; true for the block that arrives last. Word 0 is read
// by the atomic add itself, so every block of a call takes the same path:
// the adds change only its lower half (a ready word counts up from zero and
// cannot carry; a garbage word could carry only from within a grid's width
// of 2^32 with an upper half one below the magic), and the last block
// rewrites it only after every block has added.
__device__ __forceinline__ bool arrive_last(unsigned long long *ticket, uint32_t stamp,
                                            uint32_t blocks)
{
    const unsigned long long ready = kTicketMagic << 32;
    const unsigned long long old =
        __hip_atomic_fetch_add(ticket, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if ((old >> 32) == kTicketMagic) {
        if ((uint32_t)old + 1 != blocks)
            return false;
        __hip_atomic_store(ticket, ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return true;
    }
    // slow path: a compare-and-swap count keyed by the call's stamp; one
    // success per block, so a block retries at most once per other block
    unsigned long long *word = ticket + 1;
    unsigned long long cur = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned long long want;
    do {
        want = (uint32_t)(cur >> 32) == stamp ? cur + 1 : (((unsigned long long)stamp << 32) | 1ull);
    } while (!__hip_atomic_compare_exchange_strong(word, &cur, want, __ATOMIC_ACQ_REL,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if ((uint32_t)want != blocks)
        return false;
    __hip_atomic_store(ticket, ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

template <int NSLOT, bool NORMALIZE, int TPW, int NC, bool BIAS>
__global__ __launch_bounds__(kFusedThreads) void route_layout_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int64_t T, int32_t E,
    int32_t k, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, int32_t R,
    int32_t capacity, int nbits, int32_t *__restrict__ expert_demand,
    int32_t *__restrict__ expert_counts, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ dest_counts, int32_t *__restrict__ dest_offsets,
    int32_t *__restrict__ pos, int32_t *__restrict__ send_src, unsigned long long *ticket,
    uint32_t stamp)
{
    extern __shared__ int32_t sm[];
    __shared__ int32_t last;
    const int64_t t0 = ((int64_t)blockIdx.x * kFusedWaves + threadIdx.x / kWave) * TPW;
    if (t0 < T)  // uniform across the wave; no barrier inside
        route_wave<NSLOT, 4, NORMALIZE, TPW, NC, BIAS>(logits, bias, T, E, k, 0, 0, topk_idx,
                                                       topk_w, t0);
    __syncthreads();  // the block's ids and weights are written
    if (threadIdx.x == 0)
        last = arrive_last(ticket, stamp, gridDim.x);  // release ours, acquire the others'
    __syncthreads();
    if (!last)
        return;
    layout_small_body<kFusedThreads>(topk_idx, T * k, k, E, R, capacity, nbits, expert_demand,
                                     expert_counts, expert_offsets, dest_counts, dest_offsets,
                                     pos, send_src, sm);
}

struct FusedArgs {
    const float *logits, *bias;
    int64_t T;
    int32_t E, k, R, capacity;
    int32_t *topk_idx;
    float *topk_w;
    int32_t *expert_demand, *expert_counts, *expert_offsets, *dest_counts, *dest_offsets, *pos,
        *send_src;
    unsigned long long *ticket;
};

template <int NSLOT, int TPW, int NC>
hipError_t launch_fused(const FusedArgs &a, bool normalize, hipStream_t stream)
{
    static std::atomic<uint32_t> calls{0};
    const uint32_t stamp = calls.fetch_add(1, std::memory_order_relaxed) % 0xFFFFFFFFu + 1u;
    int nbits = 0;
    while ((1 << nbits) < a.E)
        ++nbits;
    const int64_t per_block = (int64_t)kFusedWaves * TPW;
    const dim3 grid((unsigned)((a.T + per_block - 1) / per_block));
    const size_t lds = (size_t)((kFusedWaves + 2) * a.E + 1) * sizeof(int32_t);
#define MOE_FUSED_LAUNCH(N, B)                                                                    \
    hipLaunchKernelGGL((route_layout_kernel<NSLOT, N, TPW, NC, B>), grid, dim3(kFusedThreads), lds, \
                       stream, a.logits, a.bias, a.T, a.E, a.k, a.topk_idx, a.topk_w, a.R,          \
                       a.capacity, nbits, a.expert_demand, a.expert_counts, a.expert_offsets,      \
                       a.dest_counts, a.dest_offsets, a.pos, a.send_src, a.ticket, stamp)
    if (normalize) {
        if (a.bias)
            MOE_FUSED_LAUNCH(true, true);
        else
            MOE_FUSED_LAUNCH(true, false);
    } else {
        if (a.bias)
            MOE_FUSED_LAUNCH(false, true);
        else
            MOE_FUSED_LAUNCH(false, false);
    }
#undef MOE_FUSED_LAUNCH
    return hipGetLastError();
}

}  // namespace

bool route_layout_fuses(int64_t T, int32_t E, int32_t k, const float *logits, const float *bias)
{
    // 16-byte rows (as the routing kernel's fast path) and the one-block
    // layout's limits
    return T > 0 && T * (int64_t)k <= kSmallAssignments && E <= kSmallMaxExperts && E % 4 == 0 &&
           (uintptr_t)logits % 16 == 0 && (uintptr_t)bias % 16 == 0;
}

hipError_t launch_route_layout(const float *logits, const float *bias, int64_t T, int32_t E,
                               int32_t k, bool normalize, int32_t R, int32_t capacity,
                               int32_t *topk_idx, float *topk_w, int32_t *expert_demand,
                               int32_t *expert_counts, int32_t *expert_offsets,
                               int32_t *dest_counts, int32_t *dest_offsets, int32_t *pos,
                               int32_t *send_src, void *workspace, hipStream_t stream)
{
    int32_t *tile_hist = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) +
                                                     kRouteLayoutHeaderBytes);
    if (!route_layout_fuses(T, E, k, logits, bias)) {
        // two launches, as the separate calls make them
        hipError_t err = hipSuccess;
        if (T > 0 && (err = launch_route_topk(logits, bias, T, E, k, 0, 0, normalize, topk_idx,
                                              topk_w, stream)) != hipSuccess)
            return err;
        return launch_dispatch_layout(topk_idx, T, E, k, R, capacity, expert_demand, expert_counts,
                                      expert_offsets, dest_counts, dest_offsets, pos, send_src,
                                      tile_hist, stream);
    }
    const FusedArgs a{logits,        bias,          T,           E,           k,
                      R,             capacity,      topk_idx,    topk_w,      expert_demand,
                      expert_counts, expert_offsets, dest_counts, dest_offsets, pos,
                      send_src,      static_cast<unsigned long long *>(workspace)};
    // the tokens-per-wave shape the routing kernel picks for these sizes
    // (16-byte loads, no groups)
    int seg = 4;
    while (seg < (E + 3) / 4 || seg < k)
        seg *= 2;
    if (seg <= 16) {
        switch (seg) {
        case 4: return launch_fused<4, 16, 2>(a, normalize, stream);
        case 8: return launch_fused<4, 8, 2>(a, normalize, stream);
        default: return launch_fused<4, 4, 2>(a, normalize, stream);
        }
    }
    if (E <= 128)
        return launch_fused<4, 2, 2>(a, normalize, stream);
    if (E <= 256)
        return launch_fused<4, 1, 2>(a, normalize, stream);
    if (k >= 3)
        return launch_fused<8, 1, 3>(a, normalize, stream);
    return launch_fused<8, 1, 2>(a, normalize, stream);
}

}  // namespace moe
