// route_topk.hip -- top-k expert selection and gate weights, one wavefront
// per token.
//
// Method: ai-from-scratch "19. All-to-all", intro (each token gets a list of
// expert ids) and "Why the router can ruin your day" (the balancing bias
// moves the top-k decision only; the mix weights come from the unbiased
// router scores); aicassindra "gpu_moe_all_to_all", "Two collectives per
// layer" (gate weights scale the returning outputs).
//
// Group-limited routing (n_groups > 0): ai-from-scratch "19. All-to-all",
// "DeepSeek's numbers" (each token limited to a few nodes) and the closing
// section (node-limited routing as an architectural constraint). Groups are
// ranked by their best biased score, the plainest reading of a group score.
//
// Layout on gfx950. When E % 4 == 0 and the rows are 16-byte aligned, lane
// l of the wave owns experts 4l..4l+3, 256 + 4l.., ... and reads them with
// 16-byte non-temporal loads (one instruction covers 1 KiB of the row);
// otherwise lane l owns experts l, l + 64, ... with 4-byte loads. On MI355X
// the 16-byte form reads the logits at ~6.9 TB/s against ~2 TB/s for the
// 4-byte form, which made the load phase the bottleneck of this kernel.
// Either way a lane's slots are in ascending expert order. Small rows share
// a wave: with 16-byte loads and E <= 64 a token takes one DPP row or less
// (4, 8 or 16 tokens per wave), its reductions are butterfly steps inside the
// row, and a round's owner is the lane holding the smallest id among those
// with the best key; for E <= 128 each 32-lane half routes its own token
// with half-wave reductions. Scores become
// order-preserving 32-bit keys and each lane keeps its two or three best
// remaining (key, id) candidates, built without branches. A selection round
// is a wave-wide 32-bit maximum by DPP (six fused max steps, one readlane),
// a ballot of the lanes holding that key and -- only when two lanes hold an
// equal key -- a DPP minimum of their ids, so ties go to the smaller id.
// The winning lane pops its candidate; it rescans its registers only once
// every candidate is used. With 16-byte loads a lane holds runs of four
// consecutive experts, so a skewed router that favours low ids makes one
// lane win often: at E = 512, k = 10 with a Zipf-like skew a token needed
// 1.5 rescans on average with two candidates and 0.3 with three, which is
// why lanes with 8 or more slots (E > 256 with 16-byte loads) keep three
// when k >= 3.
// Lane j keeps round j's id; at the end lanes 0..k-1 gather their unbiased
// logits from the row (still in cache), take the softmax and write one
// coalesced row of ids and weights.
#include "launch.hpp"
#include "route_device.hpp"

namespace moe {
namespace {

// One wave per TPW tokens: whole waves past T leave at once.
template <int NSLOT, int VEC, bool NORMALIZE, int TPW, int NC, bool BIAS>
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int64_t T, int32_t E,
    int32_t k, int32_t n_groups, int32_t topk_groups, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w)
{
    const int64_t t0 = ((int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave) * TPW;
    if (t0 >= T)
        return;  // uniform across the wave: whole waves leave together
    route_wave<NSLOT, VEC, NORMALIZE, TPW, NC, BIAS>(logits, bias, T, E, k, n_groups, topk_groups,
                                                     topk_idx, topk_w, t0);
}

template <int NSLOT, int VEC, int TPW, int NC>
void launch_cand(const float *logits, const float *bias, int64_t T, int32_t E, int32_t k,
                 int32_t n_groups, int32_t topk_groups, bool normalize, int32_t *topk_idx,
                 float *topk_w, hipStream_t stream)
{
    const int64_t per_block = (int64_t)kWavesPerBlock * TPW;
    // one wave per TPW tokens; past kMaxRowBlocks blocks, one launch per chunk
    // of tokens (a loop inside the kernel cost it 20-30 VGPRs)
    const int64_t chunk = kMaxRowBlocks * per_block;
    for (int64_t t0 = 0; t0 < T; t0 += chunk) {
        const int64_t n = T - t0 < chunk ? T - t0 : chunk;
        const dim3 grid((unsigned)((n + per_block - 1) / per_block));
        const float *lg = logits + t0 * E;
        int32_t *ti = topk_idx + t0 * k;
        float *tw = topk_w + t0 * k;
#define MOE_ROUTE_LAUNCH(N, B)                                                                      \
    hipLaunchKernelGGL((route_topk_kernel<NSLOT, VEC, N, TPW, NC, B>), grid, dim3(kRouteThreads), 0, \
                       stream, lg, bias, n, E, k, n_groups, topk_groups, ti, tw)
        if (normalize) {
            if (bias)
                MOE_ROUTE_LAUNCH(true, true);
            else
                MOE_ROUTE_LAUNCH(true, false);
        } else {
            if (bias)
                MOE_ROUTE_LAUNCH(false, true);
            else
                MOE_ROUTE_LAUNCH(false, false);
        }
#undef MOE_ROUTE_LAUNCH
        if (hipPeekAtLastError() != hipSuccess)
            return;
    }
}

template <int NSLOT, int VEC, int TPW>
hipError_t launch_slots(const float *logits, const float *bias, int64_t T, int32_t E, int32_t k,
                        int32_t n_groups, int32_t topk_groups, bool normalize, int32_t *topk_idx,
                        float *topk_w, hipStream_t stream)
{
    // A third candidate costs every token a few instructions per slot and
    // saves the lanes that win three times a rescan of all their slots. On
    // MI355X it paid with 8 or more slots per lane and k >= 3 (E = 512,
    // k = 10: 28.2 against 30.8 us for 32768 tokens) and lost with 4 slots
    // (E = 256, k = 8: 18.5 against 18.0 us).
    if constexpr (NSLOT >= 8) {
        if (k >= 3) {
            launch_cand<NSLOT, VEC, TPW, 3>(logits, bias, T, E, k, n_groups, topk_groups, normalize,
                                            topk_idx, topk_w, stream);
            return hipGetLastError();
        }
    }
    launch_cand<NSLOT, VEC, TPW, 2>(logits, bias, T, E, k, n_groups, topk_groups, normalize,
                                    topk_idx, topk_w, stream);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route_topk(const float *logits, const float *bias, int64_t T, int32_t E,
                             int32_t k, int32_t n_groups, int32_t topk_groups, bool normalize,
                             int32_t *topk_idx, float *topk_w, hipStream_t stream)
{
    const bool vec4 = E % 4 == 0 && (uintptr_t)logits % 16 == 0 && (uintptr_t)bias % 16 == 0;
    // Two tokens per wave halve the selection rounds per token but double
    // each lane's slots once the row needs more than one pass of the half
    // wave. On MI355X two tokens per wave won at E = 64 (8.3 against 10.4 us,
    // 16384 tokens) and lost at E = 256 and 512 (46 against 36 us, 32768
    // tokens), so they are used only while the slots per lane stay the same:
    // E <= 128 with 16-byte loads, E <= 32 otherwise; and lane g of a half
    // must hold group g (<= 32 groups).
    const bool two = (vec4 ? E <= 4 * 32 : E <= 32) && n_groups <= 32;
    // With 16-byte loads and E <= 64, a token fits one DPP row (16 lanes of 4
    // experts) or less, so 4, 8 or 16 tokens share a wave: each reduction is
    // 2-4 butterfly steps inside the row and needs no readlane. The row must
    // also hold the k ids and one lane per group.
    int seg = 4;
    while (seg < (E + 3) / 4 || seg < k || seg < n_groups)
        seg *= 2;
#define MOE_ROUTE_ARGS logits, bias, T, E, k, n_groups, topk_groups, normalize, topk_idx, topk_w, stream
    if (vec4 && seg <= 16) {
        switch (seg) {
        case 4: return launch_slots<4, 4, 16>(MOE_ROUTE_ARGS);
        case 8: return launch_slots<4, 4, 8>(MOE_ROUTE_ARGS);
        default: return launch_slots<4, 4, 4>(MOE_ROUTE_ARGS);
        }
    }
    if (vec4 && two) {
        return launch_slots<4, 4, 2>(MOE_ROUTE_ARGS);
    }
    if (vec4) {
        switch ((E + 4 * kWave - 1) / (4 * kWave)) {
        case 1: return launch_slots<4, 4, 1>(MOE_ROUTE_ARGS);
        case 2: return launch_slots<8, 4, 1>(MOE_ROUTE_ARGS);
        case 3: return launch_slots<12, 4, 1>(MOE_ROUTE_ARGS);
        case 4: return launch_slots<16, 4, 1>(MOE_ROUTE_ARGS);
        default: return hipErrorInvalidValue;
        }
    }
    if (two)
        return launch_slots<1, 1, 2>(MOE_ROUTE_ARGS);
    switch ((E + kWave - 1) / kWave) {
#define MOE_ROUTE_CASE(n) \
    case n:               \
        return launch_slots<n, 1, 1>(MOE_ROUTE_ARGS);
        MOE_ROUTE_CASE(1) MOE_ROUTE_CASE(2) MOE_ROUTE_CASE(3) MOE_ROUTE_CASE(4)
        MOE_ROUTE_CASE(5) MOE_ROUTE_CASE(6) MOE_ROUTE_CASE(7) MOE_ROUTE_CASE(8)
        MOE_ROUTE_CASE(9) MOE_ROUTE_CASE(10) MOE_ROUTE_CASE(11) MOE_ROUTE_CASE(12)
        MOE_ROUTE_CASE(13) MOE_ROUTE_CASE(14) MOE_ROUTE_CASE(15) MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
    default:
        return hipErrorInvalidValue;
    }
#undef MOE_ROUTE_ARGS
}

}  // namespace moe
