// route_device.hpp -- the per-wave top-k selection and gate weights shared
// by the routing kernel (route_topk.hip) and the fused routing + layout
// kernel for small batches (route_layout.hip). The method and the gfx950
// design are described at the top of route_topk.hip.
#pragma once

#include "device.hpp"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kWavesPerBlock = kRouteThreads / kWave;

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

// Insert (kk, id) into a lane's NC (2 or 3) best (key, id) candidates,
// kept in rank order; with NC = 2 the third stays empty (key 0). Callers
// present ids in ascending order, so the strict comparisons keep the
// smaller id ahead of an equal key; key 0 (padding or already taken) never
// enters.
template <int NC>
__device__ __forceinline__ void insert_cand(uint32_t kk, uint32_t id, uint32_t &c1k, uint32_t &c1i,
                                            uint32_t &c2k, uint32_t &c2i, uint32_t &c3k, uint32_t &c3i)
{
    const bool gt1 = kk > c1k, gt2 = kk > c2k;
    if (NC == 3) {
        const bool gt3 = kk > c3k;
        c3k = gt2 ? c2k : (gt3 ? kk : c3k);
        c3i = gt2 ? c2i : (gt3 ? id : c3i);
    }
    c2k = gt1 ? c1k : (gt2 ? kk : c2k);
    c2i = gt1 ? c1i : (gt2 ? id : c2i);
    c1k = gt1 ? kk : c1k;
    c1i = gt1 ? id : c1i;
}

// TPW tokens per wave: token h of the wave lives on lanes [h*HW, (h+1)*HW),
// HW = 64 / TPW lanes per token.
template <int TPW>
struct Group {
    static constexpr int HW = kWave / TPW;
    // reduce within each token's lanes; every lane gets its own token's result
    template <class Op>
    __device__ __forceinline__ static uint32_t reduce(uint32_t v, uint32_t identity, Op op)
    {
        v = op(v, dpp::mov<dpp::kQuadSwap1>(v, identity));
        v = op(v, dpp::mov<dpp::kQuadSwap2>(v, identity));
        if (HW >= 8)
            v = op(v, dpp::mov<dpp::kRowHalfMirror>(v, identity));
        if (HW >= 16)
            v = op(v, dpp::mov<dpp::kRowMirror>(v, identity));
        if (HW <= 16)
            return v;  // butterfly steps inside a row: every lane holds its token's result
        v = op(v, dpp::mov<dpp::kRowBcast15, 0xA>(v, identity));
        if (TPW == 1) {
            v = op(v, dpp::mov<dpp::kRowBcast31, 0xC>(v, identity));
            return readlane_u32(v, kWave - 1);
        }
        // lane 31 holds rows 0-1 (the first token), lane 63 rows 2-3
        const uint32_t lo = readlane_u32(v, 31), hi = readlane_u32(v, 63);
        return (threadIdx.x & (kWave - 1)) < 32 ? lo : hi;
    }
    __device__ __forceinline__ static uint32_t max_u32(uint32_t v)
    {
        return reduce(v, 0u, [](uint32_t a, uint32_t b) { return max(a, b); });
    }
    __device__ __forceinline__ static uint32_t min_u32(uint32_t v)
    {
        return reduce(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return min(a, b); });
    }
    __device__ __forceinline__ static float max_f32(float v)
    {
        return __uint_as_float(reduce(__float_as_uint(v), __float_as_uint(-INFINITY),
                                      [](uint32_t a, uint32_t b) {
                                          return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
                                      }));
    }
    __device__ __forceinline__ static float sum_f32(float v)
    {
        return __uint_as_float(reduce(__float_as_uint(v), 0u, [](uint32_t a, uint32_t b) {
            return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
        }));
    }
};

// Expert id held in slot i of in-token lane `gl`, and the in-token lane that
// holds expert e (HW lanes per token).
template <int VEC, int HW>
__device__ __forceinline__ uint32_t slot_id(int i, int gl)
{
    return VEC == 4 ? (uint32_t)((i / 4) * 4 * HW + 4 * gl + (i % 4)) : (uint32_t)(i * HW + gl);
}
template <int VEC, int HW>
__device__ __forceinline__ int owner_lane(uint32_t e)
{
    return VEC == 4 ? (int)((e >> 2) & (HW - 1)) : (int)(e & (HW - 1));
}

// NSLOT keys per lane; VEC = 4 (16-byte loads) or 1 (4-byte loads); TPW
// tokens per wave (2: each 32-lane half routes its own token, halving the
// cost of the selection rounds per token); NC candidates per lane (2 or 3);
// BIAS: a selection bias is given (without it, each slot's score costs two
// fewer instructions than a select between the biased and unbiased value)
// The wave routes tokens t0 .. t0 + TPW - 1 (t0 < T; tokens past T are
// skipped). Wave-level only: no block barrier, so callers may run it on a
// subset of their waves.
template <int NSLOT, int VEC, bool NORMALIZE, int TPW, int NC, bool BIAS>
__device__ __forceinline__ void route_wave(
    const float *__restrict__ logits, const float *__restrict__ bias, int64_t T, int32_t E,
    int32_t k, int32_t n_groups, int32_t topk_groups, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, int64_t t0)
{
    using G = Group<TPW>;
    constexpr int HW = G::HW;
    const int lane = threadIdx.x & (kWave - 1);
    const int gl = lane & (HW - 1);       // lane within its token
    const int gbase = lane - gl;          // first lane of its token
    const int64_t t = t0 + lane / HW;
    const bool valid = t < T;             // the second token of the last wave may not exist
    const float *row = logits + (valid ? t : t0) * E;

    uint32_t key[NSLOT];
    if (VEC == 4) {
        const f32x4 *row4 = reinterpret_cast<const f32x4 *>(row);
        const f32x4 *bias4 = reinterpret_cast<const f32x4 *>(bias);
#pragma unroll
        for (int g = 0; g < NSLOT / 4; ++g) {
            if (valid && g * 4 * HW + 4 * gl < E) {
                const f32x4 v = __builtin_nontemporal_load(row4 + g * HW + gl);
                const f32x4 b = BIAS ? bias4[g * HW + gl] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    key[4 * g + c] = score_key((BIAS ? v[c] + b[c] : v[c]) + 0.0f);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    key[4 * g + c] = 0u;  // padding ranks below everything
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < NSLOT; ++i) {
            const int e = i * HW + gl;
            if (valid && e < E) {
                const float v = row[e];
                key[i] = score_key((BIAS ? v + bias[e] : v) + 0.0f);
            } else {
                key[i] = 0u;  // padding ranks below everything, NaN included
            }
        }
    }

    if (n_groups > 0) {
        // group-limited routing: rank the n_groups contiguous expert groups
        // by their best key (in-token lane g holds group g's), keep the best
        // topk_groups -- ties to the lower group, i.e. the lower lane -- and
        // drop every expert outside them
        const int32_t gsize = E / n_groups;
        int gid[NSLOT];
        uint32_t my_gkey = 0u;
        if (VEC == 4 && TPW == 1 && (gsize == 16 || gsize == 32 || gsize == 64)) {
            // Slot quad q of lane l holds experts 256q + 4l .. +3 and a group
            // of 16, 32 or 64 divides 256, so the quad's group is
            // q * (256 / gsize) + l / (gsize / 4), and group g's best key is
            // the max over a segment of gsize / 4 consecutive lanes of one
            // quad (padding keys past E are 0 and fall in groups >=
            // n_groups). DPP steps inside 16-lane rows leave every lane of a
            // segment with its segment's max, and one bpermute per quad
            // hands group g's max to lane g: the values of the general loop
            // below, with no division and no wave-wide reduction per group.
            const int shift = gsize == 16 ? 2 : (gsize == 32 ? 3 : 4);  // log2 of lanes per group
            const int seg = 1 << shift;
            const int per_quad = kWave >> shift;  // groups in one quad
#pragma unroll
            for (int q = 0; q < NSLOT / 4; ++q) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    gid[4 * q + c] = q * per_quad + (gl >> shift);
                auto mx = [](uint32_t a, uint32_t b) { return max(a, b); };
                uint32_t v = mx(mx(key[4 * q], key[4 * q + 1]), mx(key[4 * q + 2], key[4 * q + 3]));
                v = mx(v, dpp::mov<dpp::kQuadSwap1>(v, 0u));
                v = mx(v, dpp::mov<dpp::kQuadSwap2>(v, 0u));
                if (seg >= 8)
                    v = mx(v, dpp::mov<dpp::kRowHalfMirror>(v, 0u));
                if (seg >= 16)
                    v = mx(v, dpp::mov<dpp::kRowMirror>(v, 0u));
                // lane g of this quad's groups reads the first lane of its segment
                const int gq = lane - q * per_quad;
                const bool here = gq >= 0 && gq < per_quad;
                const uint32_t got =
                    (uint32_t)__builtin_amdgcn_ds_bpermute((here ? gq << shift : 0) << 2, (int)v);
                my_gkey = here ? got : my_gkey;
            }
        } else {
#pragma unroll
            for (int i = 0; i < NSLOT; ++i)
                gid[i] = (int)(slot_id<VEC, HW>(i, gl) / (uint32_t)gsize);
            for (int g = 0; g < n_groups; ++g) {
                uint32_t v = 0u;
#pragma unroll
                for (int i = 0; i < NSLOT; ++i)
                    v = gid[i] == g ? max(v, key[i]) : v;
                const uint32_t best = G::max_u32(v);
                my_gkey = gl == g ? best : my_gkey;
            }
        }
        uint64_t chosen = 0;
        // with one token per wave and at most 16 groups every group key
        // lies in the first 16-lane row, so a row max suffices
        const bool row0 = TPW == 1 && n_groups <= 16;
        for (int m = 0; m < topk_groups; ++m) {
            uint32_t best;
            if (row0) {
                uint32_t v = my_gkey;
                v = max(v, dpp::mov<dpp::kQuadSwap1>(v, 0u));
                v = max(v, dpp::mov<dpp::kQuadSwap2>(v, 0u));
                v = max(v, dpp::mov<dpp::kRowHalfMirror>(v, 0u));
                v = max(v, dpp::mov<dpp::kRowMirror>(v, 0u));
                best = readlane_u32(v, 0);
            } else {
                best = G::max_u32(my_gkey);
            }
            int g;
            if (TPW >= 4) {
                // the lowest group of the token holding the best key, by a
                // minimum inside the token's row segment
                g = (int)G::min_u32(((my_gkey == best) & (gl < n_groups)) ? (uint32_t)gl : 0xFFFFFFFFu);
            } else {
                const uint64_t holders = ballot64(my_gkey == best && gl < n_groups);
                // the lowest holding lane of each token's lanes
                const uint64_t mine = TPW == 1 ? holders
                                               : (gbase == 0 ? holders & 0xFFFFFFFFull : holders >> 32);
                g = __ffsll((unsigned long long)mine) - 1;
            }
            chosen |= 1ull << g;
            my_gkey = gl == g ? 0u : my_gkey;
        }
#pragma unroll
        for (int i = 0; i < NSLOT; ++i)
            key[i] = ((chosen >> gid[i]) & 1ull) ? key[i] : 0u;
    }

    // the lane's NC best entries
    uint32_t c1k = key[0], c1i = slot_id<VEC, HW>(0, gl);
    uint32_t c2k = 0u, c2i = 0xFFFFFFFFu, c3k = 0u, c3i = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 1; i < NSLOT; ++i)
        insert_cand<NC>(key[i], slot_id<VEC, HW>(i, gl), c1k, c1i, c2k, c2i, c3k, c3i);

    uint32_t my_e = 0;
    for (int j = 0; j < k; ++j) {
        const uint32_t best = G::max_u32(c1k);
        uint32_t ew;
        bool own;
        if (TPW >= 4) {
            // a token per row segment: the smallest id among the lanes holding
            // the best key, by a minimum inside the segment; its lane owns it
            ew = G::min_u32(c1k == best ? c1i : 0xFFFFFFFFu);
            own = (c1k == best) & (c1i == ew);
        } else {
            const uint64_t holders = ballot64(c1k == best);
            int owner;
            bool unique;
            if (TPW == 1)
                unique = __popcll(holders) == 1;
            else
                unique = __popcll(holders & 0xFFFFFFFFull) == 1 && __popcll(holders >> 32) == 1;
            if (unique) {
                if (TPW == 1) {
                    owner = __ffsll((unsigned long long)holders) - 1;
                    ew = readlane_u32(c1i, owner);
                } else {
                    const int o0 = __ffsll((unsigned long long)(holders & 0xFFFFFFFFull)) - 1;
                    const int o1 = 32 + __ffsll((unsigned long long)(holders >> 32)) - 1;
                    const uint32_t e0 = readlane_u32(c1i, o0), e1 = readlane_u32(c1i, o1);
                    owner = gbase == 0 ? o0 : o1;
                    ew = gbase == 0 ? e0 : e1;
                }
            } else {  // several lanes of a token hold an equal key: the smallest id wins
                ew = G::min_u32(c1k == best ? c1i : 0xFFFFFFFFu);
                owner = gbase + owner_lane<VEC, HW>(ew);
            }
            own = lane == owner;
        }
        // lane j keeps round j's id: one writelane of the uniform id with one
        // token per wave, a select per token otherwise
        my_e = TPW == 1 ? writelane_u32(ew, j, my_e) : (gl == j ? ew : my_e);
        // in the owner lane the candidate taken is (best, ew): the round's
        // uniform key and id, so the pop below can overwrite c1 in place
        const uint32_t gone_k = best, gone_i = ew;
        c1k = own ? c2k : c1k;
        c1i = own ? c2i : c1i;
        if (NC == 3) {
            c2k = own ? c3k : c2k;
            c2i = own ? c3i : c2i;
            c3k = own ? 0u : c3k;
        } else {
            c2k = own ? 0u : c2k;  // an empty slot's id is never read
        }
        if (own && c1k == 0u) {
            // every candidate used: rescan the entries ranked below the last
            // one taken from this lane
            c1i = c2i = c3i = 0xFFFFFFFFu;
#pragma unroll
            for (int i = 0; i < NSLOT; ++i) {
                const uint32_t id = slot_id<VEC, HW>(i, gl);
                // bitwise, not short-circuit: a select per slot, no branches
                const bool below = (key[i] < gone_k) | ((key[i] == gone_k) & (id > gone_i));
                insert_cand<NC>(below ? key[i] : 0u, id, c1k, c1i, c2k, c2i, c3k, c3i);
            }
        }
    }

    // unbiased logits of the selected experts, straight from the row
    const bool mine = valid && gl < k;
    const float my_l = mine ? row[my_e] : -INFINITY;
    float w;
    if (NORMALIZE) {
        const float m = G::max_f32(my_l);
        const float u = mine ? expf(my_l - m) : 0.f;
        w = u / G::sum_f32(u);
    } else {
        float lm = -INFINITY;
        if (valid)
            for (int e = gl; e < E; e += HW)
                lm = fmaxf(lm, row[e]);
        const float M = G::max_f32(lm);
        float part = 0.f;
        if (valid)
            for (int e = gl; e < E; e += HW)
                part += expf(row[e] - M);
        w = (mine ? expf(my_l - M) : 0.f) / G::sum_f32(part);
    }
    if (mine) {
        topk_idx[t * k + gl] = (int32_t)my_e;
        topk_w[t * k + gl] = w;
    }
}

}  // namespace
}  // namespace moe
