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
// Either way a lane's slots are in ascending expert order. Scores become
// order-preserving 32-bit keys and each lane keeps its two best remaining
// (key, id) candidates, built without branches. A selection round is a
// wave-wide 32-bit maximum by DPP (six fused max steps, one readlane), a
// ballot of the lanes holding that key and -- only when two lanes hold an
// equal key -- a DPP minimum of their ids, so ties go to the smaller id.
// The winning lane pops its candidate; it rescans its registers only once
// both candidates are used (rare: a lane must win three of the k rounds).
// Lane j keeps round j's id; at the end lanes 0..k-1 gather their unbiased
// logits from the row (still in cache), take the softmax and write one
// coalesced row of ids and weights.
#include "device.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kTokensPerBlock = kRouteThreads / kWave;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Order-preserving map of a float score onto uint32: larger key = higher
// rank. The caller adds +0.0f first, which turns -0 into +0 and leaves
// every other value unchanged, so equal reals get equal keys. Every NaN
// maps to 1, below -inf (0x007FFFFF); 0 marks padding and used entries.
__device__ __forceinline__ uint32_t score_key(float s)
{
    const uint32_t u = __float_as_uint(s);
    const uint32_t k = u ^ (uint32_t)(((int32_t)u >> 31) | (int32_t)0x80000000);
    return s != s ? 1u : k;
}

// Expert id held in slot i of lane `lane`, and the lane that holds expert e.
template <int VEC>
__device__ __forceinline__ uint32_t slot_id(int i, int lane)
{
    return VEC == 4 ? (uint32_t)((i / 4) * 4 * kWave + 4 * lane + (i % 4))
                    : (uint32_t)(i * kWave + lane);
}
template <int VEC>
__device__ __forceinline__ int owner_lane(uint32_t e)
{
    return VEC == 4 ? (int)((e >> 2) & (kWave - 1)) : (int)(e & (kWave - 1));
}

// NSLOT keys per lane; VEC = 4 (16-byte loads) or 1 (4-byte loads)
template <int NSLOT, int VEC, bool NORMALIZE>
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int64_t T, int32_t E,
    int32_t k, int32_t n_groups, int32_t topk_groups, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kTokensPerBlock + (threadIdx.x / kWave);
    if (t >= T)
        return;  // t is uniform across the wave: whole waves leave together
    const float *row = logits + t * E;

    uint32_t key[NSLOT];
    if (VEC == 4) {
        const f32x4 *row4 = reinterpret_cast<const f32x4 *>(row);
        const f32x4 *bias4 = reinterpret_cast<const f32x4 *>(bias);
#pragma unroll
        for (int g = 0; g < NSLOT / 4; ++g) {
            if (g * 4 * kWave + 4 * lane < E) {
                const f32x4 v = __builtin_nontemporal_load(row4 + g * kWave + lane);
                const f32x4 b = bias ? bias4[g * kWave + lane] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    key[4 * g + c] = score_key((bias ? v[c] + b[c] : v[c]) + 0.0f);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    key[4 * g + c] = 0u;  // padding ranks below everything
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < NSLOT; ++i) {
            const int e = i * kWave + lane;
            if (e < E) {
                const float v = row[e];
                key[i] = score_key((bias ? v + bias[e] : v) + 0.0f);
            } else {
                key[i] = 0u;  // padding ranks below everything, NaN included
            }
        }
    }

    if (n_groups > 0) {
        // group-limited routing: rank the n_groups contiguous expert groups
        // by their best key (lane g holds group g's), keep the best
        // topk_groups -- ties to the lower group, i.e. the lower lane -- and
        // drop every expert outside them
        const int32_t gsize = E / n_groups;
        int gid[NSLOT];
#pragma unroll
        for (int i = 0; i < NSLOT; ++i)
            gid[i] = (int)(slot_id<VEC>(i, lane) / (uint32_t)gsize);
        uint32_t my_gkey = 0u;
        for (int g = 0; g < n_groups; ++g) {
            uint32_t v = 0u;
#pragma unroll
            for (int i = 0; i < NSLOT; ++i)
                v = gid[i] == g ? max(v, key[i]) : v;
            const uint32_t best = wave_max_u32(v);
            my_gkey = lane == g ? best : my_gkey;
        }
        uint64_t chosen = 0;
        for (int m = 0; m < topk_groups; ++m) {
            const uint32_t best = wave_max_u32(my_gkey);
            const uint64_t holders = ballot64(my_gkey == best && lane < n_groups);
            const int g = __ffsll((unsigned long long)holders) - 1;
            chosen |= 1ull << g;
            my_gkey = lane == g ? 0u : my_gkey;
        }
#pragma unroll
        for (int i = 0; i < NSLOT; ++i)
            key[i] = ((chosen >> gid[i]) & 1ull) ? key[i] : 0u;
    }

    // the lane's two best entries; ascending i is ascending id, so strict
    // comparisons keep the smaller id first among equal keys
    uint32_t c1k = key[0], c1i = slot_id<VEC>(0, lane), c2k = 0u, c2i = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 1; i < NSLOT; ++i) {
        const uint32_t kk = key[i], id = slot_id<VEC>(i, lane);
        const bool gt1 = kk > c1k, gt2 = kk > c2k;
        c2k = gt1 ? c1k : (gt2 ? kk : c2k);
        c2i = gt1 ? c1i : (gt2 ? id : c2i);
        c1k = gt1 ? kk : c1k;
        c1i = gt1 ? id : c1i;
    }

    uint32_t my_e = 0;
    for (int j = 0; j < k; ++j) {
        const uint32_t best = wave_max_u32(c1k);
        const uint64_t holders = ballot64(c1k == best);
        int owner;
        uint32_t ew;
        if (__popcll(holders) == 1) {
            owner = __ffsll((unsigned long long)holders) - 1;
            ew = readlane_u32(c1i, owner);
        } else {  // several lanes hold an equal key: the smallest id wins
            ew = wave_min_u32(c1k == best ? c1i : 0xFFFFFFFFu);
            owner = owner_lane<VEC>(ew);
        }
        my_e = lane == j ? ew : my_e;
        const bool own = lane == owner;
        const uint32_t gone_k = c1k, gone_i = c1i;
        c1k = own ? c2k : c1k;
        c1i = own ? c2i : c1i;
        c2k = own ? 0u : c2k;
        if (own && c1k == 0u) {
            // both candidates used: rescan the entries ranked below the last
            // one taken from this lane
            c2i = 0xFFFFFFFFu;
#pragma unroll
            for (int i = 0; i < NSLOT; ++i) {
                const uint32_t id = slot_id<VEC>(i, lane);
                const uint32_t kk =
                    (key[i] < gone_k || (key[i] == gone_k && id > gone_i)) ? key[i] : 0u;
                const bool gt1 = kk > c1k, gt2 = kk > c2k;
                c2k = gt1 ? c1k : (gt2 ? kk : c2k);
                c2i = gt1 ? c1i : (gt2 ? id : c2i);
                c1k = gt1 ? kk : c1k;
                c1i = gt1 ? id : c1i;
            }
        }
    }

    // unbiased logits of the selected experts, straight from the row
    const bool mine = lane < k;
    const float my_l = mine ? row[my_e] : -INFINITY;
    float w;
    if (NORMALIZE) {
        const float m = wave_max_f32_dpp(my_l);
        const float u = mine ? expf(my_l - m) : 0.f;
        w = u / wave_sum_f32_dpp(u);
    } else {
        float lm = -INFINITY;
        for (int e = lane; e < E; e += kWave)
            lm = fmaxf(lm, row[e]);
        const float M = wave_max_f32_dpp(lm);
        float part = 0.f;
        for (int e = lane; e < E; e += kWave)
            part += expf(row[e] - M);
        w = (mine ? expf(my_l - M) : 0.f) / wave_sum_f32_dpp(part);
    }
    if (mine) {
        topk_idx[t * k + lane] = (int32_t)my_e;
        topk_w[t * k + lane] = w;
    }
}

template <int NSLOT, int VEC>
hipError_t launch_slots(const float *logits, const float *bias, int64_t T, int32_t E, int32_t k,
                        int32_t n_groups, int32_t topk_groups, bool normalize, int32_t *topk_idx,
                        float *topk_w, hipStream_t stream)
{
    const dim3 grid((unsigned)((T + kTokensPerBlock - 1) / kTokensPerBlock));
    if (normalize)
        hipLaunchKernelGGL((route_topk_kernel<NSLOT, VEC, true>), grid, dim3(kRouteThreads), 0,
                           stream, logits, bias, T, E, k, n_groups, topk_groups, topk_idx, topk_w);
    else
        hipLaunchKernelGGL((route_topk_kernel<NSLOT, VEC, false>), grid, dim3(kRouteThreads), 0,
                           stream, logits, bias, T, E, k, n_groups, topk_groups, topk_idx, topk_w);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route_topk(const float *logits, const float *bias, int64_t T, int32_t E,
                             int32_t k, int32_t n_groups, int32_t topk_groups, bool normalize,
                             int32_t *topk_idx, float *topk_w, hipStream_t stream)
{
    const bool vec4 = E % 4 == 0 && (uintptr_t)logits % 16 == 0 && (uintptr_t)bias % 16 == 0;
    if (vec4) {
        switch ((E + 4 * kWave - 1) / (4 * kWave)) {
        case 1:
            return launch_slots<4, 4>(logits, bias, T, E, k, n_groups, topk_groups, normalize, topk_idx, topk_w, stream);
        case 2:
            return launch_slots<8, 4>(logits, bias, T, E, k, n_groups, topk_groups, normalize, topk_idx, topk_w, stream);
        case 3:
            return launch_slots<12, 4>(logits, bias, T, E, k, n_groups, topk_groups, normalize, topk_idx, topk_w, stream);
        case 4:
            return launch_slots<16, 4>(logits, bias, T, E, k, n_groups, topk_groups, normalize, topk_idx, topk_w, stream);
        default:
            return hipErrorInvalidValue;
        }
    }
    switch ((E + kWave - 1) / kWave) {
#define MOE_ROUTE_CASE(n) \
    case n:               \
        return launch_slots<n, 1>(logits, bias, T, E, k, n_groups, topk_groups, normalize, topk_idx, topk_w, stream);
        MOE_ROUTE_CASE(1)
        MOE_ROUTE_CASE(2)
        MOE_ROUTE_CASE(3)
        MOE_ROUTE_CASE(4)
        MOE_ROUTE_CASE(5)
        MOE_ROUTE_CASE(6)
        MOE_ROUTE_CASE(7)
        MOE_ROUTE_CASE(8)
        MOE_ROUTE_CASE(9)
        MOE_ROUTE_CASE(10)
        MOE_ROUTE_CASE(11)
        MOE_ROUTE_CASE(12)
        MOE_ROUTE_CASE(13)
        MOE_ROUTE_CASE(14)
        MOE_ROUTE_CASE(15)
        MOE_ROUTE_CASE(16)
#undef MOE_ROUTE_CASE
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace moe
