/*
 * oracle.c -- plain, slow CPU oracle for the MoE dispatch/combine path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The product path
 * (the HIP library and its Python binding) never calls it, and the two share
 * no code: not a header, helper, table or constant.
 *
 * Every function is single-threaded, loops over tokens in order and writes
 * the definition out directly. Values (gate weights, combined rows) are
 * computed in double precision; the selection score is the single-precision
 * sum logit + bias, because that float decides the integer result (which
 * experts are picked) and both sides must take that decision in the same
 * precision.
 *
 * Sources (pages are cited by title and section):
 *  - ai-from-scratch "19. All-to-all", intro: every token carries a list of
 *    expert IDs, is shipped to those experts, and the results are mixed.
 *  - same page, "Why the router can ruin your day": a per-expert bias enters
 *    only the top-k decision, never the mix weights; an expert over capacity
 *    drops tokens, which then count as having skipped that expert.
 *  - aicassindra "gpu_moe_all_to_all", "Two collectives per layer, and what
 *    each one moves": k replicas out, k partial results back along the
 *    inverse permutation, scaled by the gate weights at the origin; counts
 *    per destination precede the payload.
 *  - same page, "Bucketing: cut the message count, not the byte count":
 *    sort by destination and build the offset table so that each
 *    destination's rows are contiguous.
 *  - "MoE All-to-All Dispatch and Ragged Routing", "Returning Tokens to the
 *    Original GPU": the residual x + dx is formed at the origin; "Fixed
 *    Capacity vs. Ragged Routing": per-sender-expert slots under a capacity
 *    factor, excess dropped; ragged routing is dropless.
 *  - ai-from-scratch "19. All-to-all", section on 512 experts (10 routed +
 *    1 shared): the shared expert is always active.
 *  - aicassindra "gpu_moe_all_to_all", "Latency-bound at decode,
 *    bandwidth-bound at prefill": a lower-precision dispatch payload (the
 *    FP8 section below states the reading taken for its format).
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -shared -fPIC.
 * Parity pins for every function live in the CPU test suite; none of the
 * functions here is unpinned.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if !defined(FLT_EVAL_METHOD) || FLT_EVAL_METHOD != 0
#error "the oracle needs float arithmetic evaluated in float (FLT_EVAL_METHOD == 0)"
#endif

/* ------------------------------------------------------------------ */
/* bf16 <-> real                                                       */
/* ------------------------------------------------------------------ */

/* A bf16 value is the upper half of an IEEE binary32 pattern. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round a real number to the nearest bf16 value, ties to even, straight from
 * the format's definition: 8 significant bits, exponent range of binary32,
 * subnormal spacing 2^-133, overflow to infinity. NaN becomes a quiet NaN
 * with the input's sign.
 */
uint16_t oracle_bf16_round(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    if (isinf(v))
        return (uint16_t)(sign | 0x7F80u);
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    int e = ilogb(a);             /* 2^e <= a < 2^(e+1) */
    if (e < -126)
        e = -126;                 /* subnormal range: fixed spacing */
    double q = ldexp(1.0, e - 7); /* spacing of bf16 values near a */
    double r = nearbyint(a / q) * q;   /* default mode: nearest, ties even */
    const double max_bf16 = ldexp(255.0, 120);   /* (2 - 2^-7) * 2^127 */
    if (r > max_bf16)
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)r;           /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

void oracle_bf16_round_array(const double *in, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_round(in[i]);
}

/* ------------------------------------------------------------------ */
/* route: top-k selection and gate weights                             */
/* ------------------------------------------------------------------ */

/*
 * Is score a (expert ia) ranked strictly above score b (expert ib)?
 * Real-valued comparison (-0 equals +0); any NaN ranks below every number,
 * including -inf, and all NaNs tie; ties go to the smaller expert id.
 */
static int ranks_above(float a, int ia, float b, int ib)
{
    int na = isnan(a), nb = isnan(b);
    if (!na && nb)
        return 1;
    if (na && !nb)
        return 0;
    if (!na && !nb) {
        if (a > b)
            return 1;
        if (a < b)
            return 0;
    }
    return ia < ib;
}

/* Selection scores of one token: one float add per expert. */
static void biased_scores(const float *row, const float *bias, int32_t E, float *s)
{
    for (int32_t e = 0; e < E; ++e)
        s[e] = bias ? row[e] + bias[e] : row[e];
}

/*
 * Gate weights of one token from its UNBIASED logits `row` and the k
 * selected experts:
 *   normalize != 0: w_j = exp(l_j - m) / sum_i exp(l_i - m) over the k
 *                   selected (softmax renormalised over the selection);
 *   normalize == 0: w_j = exp(l_j - M) / sum over all E experts of
 *                   exp(l_e - M) (full softmax, not renormalised).
 */
static void gate_weights(const float *row, const int32_t *idx, int32_t E, int32_t k,
                         int32_t normalize, double *w)
{
    if (normalize) {
        double m = -INFINITY;
        for (int32_t j = 0; j < k; ++j)
            if ((double)row[idx[j]] > m)
                m = (double)row[idx[j]];
        double sum = 0.0;
        for (int32_t j = 0; j < k; ++j) {
            w[j] = exp((double)row[idx[j]] - m);
            sum += w[j];
        }
        for (int32_t j = 0; j < k; ++j)
            w[j] /= sum;
    } else {
        double m = -INFINITY;
        for (int32_t e = 0; e < E; ++e)
            if ((double)row[e] > m)
                m = (double)row[e];
        double sum = 0.0;
        for (int32_t e = 0; e < E; ++e)
            sum += exp((double)row[e] - m);
        for (int32_t j = 0; j < k; ++j)
            w[j] = exp((double)row[idx[j]] - m) / sum;
    }
}

/*
 * For each token t: score s_e = logit[t][e] + bias[e] in float; select the k
 * experts with the highest scores, in descending rank order; gate weights
 * come from the unbiased logits of the selected experts (gate_weights).
 * Returns 0, or -1 on bad sizes or allocation failure.
 */
int oracle_route_topk(const float *logits, const float *bias, int64_t T,
                      int32_t E, int32_t k, int32_t normalize,
                      int32_t *topk_idx, double *topk_w)
{
    if (T < 0 || E <= 0 || k <= 0 || k > E)
        return -1;
    float *s = (float *)malloc((size_t)E * sizeof(float));
    char *taken = (char *)malloc((size_t)E);
    if (!s || !taken) {
        free(s);
        free(taken);
        return -1;
    }
    for (int64_t t = 0; t < T; ++t) {
        const float *row = logits + t * (int64_t)E;
        biased_scores(row, bias, E, s);
        for (int32_t e = 0; e < E; ++e)
            taken[e] = 0;
        int32_t *idx = topk_idx + t * (int64_t)k;
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || ranks_above(s[e], e, s[best], best))
                    best = e;
            }
            taken[best] = 1;
            idx[j] = best;
        }
        gate_weights(row, idx, E, k, normalize, topk_w + t * (int64_t)k);
    }
    free(s);
    free(taken);
    return 0;
}

/*
 * Group-limited routing. Experts form n_groups contiguous groups of
 * E / n_groups (destination groups, e.g. nodes). Each token may use at most
 * topk_groups of them: rank every group by its best expert score (the same
 * order as the expert selection, so ties go to the lower group id), keep the
 * best topk_groups groups, then select the k best experts inside them and
 * compute the weights exactly as oracle_route_topk does.
 *
 * Source: ai-from-scratch "19. All-to-all", "DeepSeek's numbers" (each
 * token limited to at most 4 nodes) and the closing section (node-limited
 * routing as an architectural constraint); zenaique Q&A
 * "moe-hide-alltoall-techniques" (node-limited routing caps cross-node
 * traffic). The pages do not define the group score; the group's best
 * biased score is the plainest reading.
 * Returns 0, or -1 on bad sizes.
 */
int oracle_route_topk_grouped(const float *logits, const float *bias, int64_t T,
                              int32_t E, int32_t k, int32_t n_groups,
                              int32_t topk_groups, int32_t normalize,
                              int32_t *topk_idx, double *topk_w)
{
    if (T < 0 || E <= 0 || k <= 0 || n_groups <= 0 || E % n_groups != 0 ||
        topk_groups <= 0 || topk_groups > n_groups ||
        k > topk_groups * (E / n_groups))
        return -1;
    const int32_t gsize = E / n_groups;
    float *s = (float *)malloc((size_t)E * sizeof(float));
    char *taken = (char *)malloc((size_t)E);
    char *gsel = (char *)malloc((size_t)n_groups);
    int32_t *gbest = (int32_t *)malloc((size_t)n_groups * sizeof(int32_t));
    if (!s || !taken || !gsel || !gbest) {
        free(s);
        free(taken);
        free(gsel);
        free(gbest);
        return -1;
    }
    for (int64_t t = 0; t < T; ++t) {
        const float *row = logits + t * (int64_t)E;
        biased_scores(row, bias, E, s);
        /* best expert of each group */
        for (int32_t g = 0; g < n_groups; ++g) {
            int32_t best = g * gsize;
            for (int32_t e = g * gsize + 1; e < (g + 1) * gsize; ++e)
                if (ranks_above(s[e], e, s[best], best))
                    best = e;
            gbest[g] = best;
            gsel[g] = 0;
        }
        /* the topk_groups groups whose best experts rank highest; comparing
         * the best experts' (score, id) pairs orders groups by score with
         * ties to the lower group, since ids grow with the group */
        for (int32_t m = 0; m < topk_groups; ++m) {
            int32_t pick = -1;
            for (int32_t g = 0; g < n_groups; ++g) {
                if (gsel[g])
                    continue;
                if (pick < 0 || ranks_above(s[gbest[g]], gbest[g], s[gbest[pick]], gbest[pick]))
                    pick = g;
            }
            gsel[pick] = 1;
        }
        for (int32_t e = 0; e < E; ++e)
            taken[e] = !gsel[e / gsize];   /* experts outside the groups are out */
        int32_t *idx = topk_idx + t * (int64_t)k;
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || ranks_above(s[e], e, s[best], best))
                    best = e;
            }
            taken[best] = 1;
            idx[j] = best;
        }
        gate_weights(row, idx, E, k, normalize, topk_w + t * (int64_t)k);
    }
    free(s);
    free(taken);
    free(gsel);
    free(gbest);
    return 0;
}

/* ------------------------------------------------------------------ */
/* dispatch layout: counts, offsets, capacity drops, positions         */
/* ------------------------------------------------------------------ */

/*
 * Experts are placed on destinations in contiguous blocks of E/R.
 * demand[e]  = number of (t, j) with topk_idx[t][j] == e.
 * Walking t = 0..T-1 and j = 0..k-1 in order, the assignment (t, j) to
 * expert e is kept iff capacity < 0 (dropless) or fewer than `capacity`
 * earlier assignments to e were kept; its rank is that number.
 * counts[e]  = kept assignments of e = min(demand[e], capacity).
 * expert_offsets = exclusive running sum of counts (E + 1 entries).
 * dest_counts[r] = sum of counts over r's experts;
 * dest_offsets[r] = expert_offsets[r * E/R], dest_offsets[R] = N.
 * pos[t][j] = expert_offsets[e] + rank, or -1 when dropped;
 * send_src[pos] = t for every kept assignment (may be NULL).
 * The send rows are therefore grouped by destination, by expert inside a
 * destination and by token inside an expert.
 * Returns 0, or -1 on bad sizes or an expert id outside [0, E).
 */
int oracle_dispatch_layout(const int32_t *topk_idx, int64_t T, int32_t E,
                           int32_t k, int32_t R, int32_t capacity,
                           int32_t *demand, int32_t *counts,
                           int32_t *expert_offsets, int32_t *dest_counts,
                           int32_t *dest_offsets, int32_t *pos,
                           int32_t *send_src)
{
    if (T < 0 || E <= 0 || k <= 0 || R <= 0 || E % R != 0)
        return -1;
    int64_t n = T * (int64_t)k;
    for (int64_t a = 0; a < n; ++a)
        if (topk_idx[a] < 0 || topk_idx[a] >= E)
            return -1;

    for (int32_t e = 0; e < E; ++e)
        demand[e] = 0;
    for (int64_t a = 0; a < n; ++a)
        demand[topk_idx[a]] += 1;

    for (int32_t e = 0; e < E; ++e)
        counts[e] = (capacity < 0 || demand[e] < capacity) ? demand[e] : capacity;

    expert_offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e)
        expert_offsets[e + 1] = expert_offsets[e] + counts[e];

    int32_t el = E / R;
    for (int32_t r = 0; r < R; ++r) {
        dest_counts[r] = 0;
        for (int32_t e = r * el; e < (r + 1) * el; ++e)
            dest_counts[r] += counts[e];
        dest_offsets[r] = expert_offsets[r * el];
    }
    dest_offsets[R] = expert_offsets[E];

    int32_t *seen = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    if (!seen)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int64_t a = t * k + j;
            int32_t e = topk_idx[a];
            if (capacity >= 0 && seen[e] >= capacity) {
                pos[a] = -1;
                continue;
            }
            int32_t rank = seen[e]++;
            pos[a] = expert_offsets[e] + rank;
            if (send_src)
                send_src[pos[a]] = (int32_t)t;
        }
    }
    free(seen);
    return 0;
}

/* ------------------------------------------------------------------ */
/* receive side: regroup source-major segments into expert-major rows  */
/* ------------------------------------------------------------------ */

/*
 * A destination receives, from each of S sources in source order, one
 * contiguous segment holding that source's rows for the destination's E_l
 * local experts, grouped by local expert (cnt[s][l] rows of expert l from
 * source s; the counts exchange delivers cnt). The expert computation wants
 * each local expert's rows together, so the rows are regrouped expert-major,
 * sources in order inside each expert:
 *   local_expert_offsets[l] = rows of experts < l over all sources
 *   source_offsets[s]       = rows of sources < s over all experts
 *   received row i (source s, expert l, j-th of that block) goes to
 *   recv_pos[i] = local_expert_offsets[l] + sum_{s' < s} cnt[s'][l] + j.
 * N = source_offsets[S] = local_expert_offsets[E_l]. Returns 0, or -1 on
 * bad sizes or negative counts.
 *
 * Source: aicassindra "gpu_moe_all_to_all", "Two collectives per layer"
 * (counts precede the payload so that receivers can size buffers; outputs
 * return along the inverse permutation) and "Bucketing" (one contiguous
 * message per peer); "MoE All-to-All Dispatch and Ragged Routing", "Why MoE
 * Token Dispatch is All-to-All" (a GPU holds 6 of 384 experts) and "Fixed
 * Capacity vs. Ragged Routing" (variable-length exchange pooled over the
 * local experts).
 */
int oracle_recv_regroup_layout(const int32_t *cnt, int32_t S, int32_t E_l,
                               int32_t *local_expert_offsets,
                               int32_t *source_offsets, int32_t *recv_pos)
{
    if (S <= 0 || E_l <= 0)
        return -1;
    for (int32_t i = 0; i < S * E_l; ++i)
        if (cnt[i] < 0)
            return -1;
    local_expert_offsets[0] = 0;
    for (int32_t l = 0; l < E_l; ++l) {
        int32_t col = 0;
        for (int32_t src = 0; src < S; ++src)
            col += cnt[src * E_l + l];
        local_expert_offsets[l + 1] = local_expert_offsets[l] + col;
    }
    source_offsets[0] = 0;
    for (int32_t src = 0; src < S; ++src) {
        int32_t rowsum = 0;
        for (int32_t l = 0; l < E_l; ++l)
            rowsum += cnt[src * E_l + l];
        source_offsets[src + 1] = source_offsets[src] + rowsum;
    }
    int64_t i = 0;
    for (int32_t src = 0; src < S; ++src) {
        for (int32_t l = 0; l < E_l; ++l) {
            int32_t before = 0;   /* rows of expert l from earlier sources */
            for (int32_t s2 = 0; s2 < src; ++s2)
                before += cnt[s2 * E_l + l];
            for (int32_t j = 0; j < cnt[src * E_l + l]; ++j)
                recv_pos[i++] = local_expert_offsets[l] + before + j;
        }
    }
    return 0;
}

/*
 * Move rows by a map: dst[map[i]][:] = src[i][:] for i < n (bit copies).
 * The regroup applies recv_pos this way; the return path applies it the
 * other way round (oracle_gather_rows). Returns -1 when a target falls
 * outside [0, dst_rows).
 */
int oracle_scatter_rows(const uint16_t *src, const int32_t *map, int64_t n, int32_t H,
                        uint16_t *dst, int64_t dst_rows)
{
    for (int64_t i = 0; i < n; ++i) {
        if (map[i] < 0 || map[i] >= dst_rows)
            return -1;
        for (int32_t h = 0; h < H; ++h)
            dst[(int64_t)map[i] * H + h] = src[i * H + h];
    }
    return 0;
}

/* dst[i][:] = src[map[i]][:] for i < n; -1 when a source row is out of range. */
int oracle_gather_rows(const uint16_t *src, int64_t src_rows, const int32_t *map, int64_t n,
                       int32_t H, uint16_t *dst)
{
    for (int64_t i = 0; i < n; ++i) {
        if (map[i] < 0 || map[i] >= src_rows)
            return -1;
        for (int32_t h = 0; h < H; ++h)
            dst[i * H + h] = src[(int64_t)map[i] * H + h];
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* dispatch permute: pack each kept replica into its send row          */
/* ------------------------------------------------------------------ */

/*
 * send[pos[t][j]][:] = x[t][:] for every kept (t, j): a bit copy of the bf16
 * row. Rows no assignment points at are left as they were.
 * Returns 0, or -1 when a position falls outside [0, send_rows).
 */
int oracle_dispatch_permute(const uint16_t *x, const int32_t *pos, int64_t T,
                            int32_t H, int32_t k, uint16_t *send,
                            int64_t send_rows)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int32_t p = pos[t * k + j];
            if (p < 0)
                continue;
            if (p >= send_rows)
                return -1;
            for (int32_t h = 0; h < H; ++h)
                send[(int64_t)p * H + h] = x[t * (int64_t)H + h];
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* combine: inverse permutation, gate-weighted sum, shared, residual   */
/* ------------------------------------------------------------------ */

/*
 * For each listed token t (all tokens when `tokens` is NULL; row i of `out`
 * belongs to tokens[i]) and each h:
 *   out = sum over kept j of w[t][j] * y[pos[t][j]][h]
 *       + shared[t][h]      (when shared is given; weight 1)
 *       + residual[t][h]    (when residual is given)
 * in double precision. A dropped replica (pos < 0) contributes nothing and
 * the remaining weights are not renormalised.
 * Returns 0, or -1 when a position falls outside [0, y_rows).
 */
int oracle_combine_reduce(const uint16_t *y, int64_t y_rows, const int32_t *pos,
                          const double *w, const uint16_t *shared,
                          const uint16_t *residual, int64_t T, int32_t H,
                          int32_t k, const int64_t *tokens, int64_t n_tokens,
                          double *out)
{
    int64_t rows = tokens ? n_tokens : T;
    for (int64_t i = 0; i < rows; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        if (t < 0 || t >= T)
            return -1;
        for (int32_t j = 0; j < k; ++j) {
            int32_t p = pos[t * k + j];
            if (p >= y_rows)
                return -1;
        }
        for (int32_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int32_t j = 0; j < k; ++j) {
                int32_t p = pos[t * k + j];
                if (p < 0)
                    continue;
                acc += w[t * k + j] * bf16_value(y[(int64_t)p * H + h]);
            }
            if (shared)
                acc += bf16_value(shared[t * (int64_t)H + h]);
            if (residual)
                acc += bf16_value(residual[t * (int64_t)H + h]);
            out[i * (int64_t)H + h] = acc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* FP8 dispatch payload: E4M3 codes with one power-of-two scale per 32 */
/* ------------------------------------------------------------------ */

/*
 * The pages name a smaller dispatch payload as the first lever once the
 * exchange is bandwidth-bound, because the expert matmul casts its input to
 * a lower precision anyway (aicassindra "gpu_moe_all_to_all", "Latency-bound
 * at decode, bandwidth-bound at prefill"; zenaique Q&A
 * "moe-hide-alltoall-techniques", the third family of fixes: shrink the
 * payload). They fix neither the format nor the scaling, so this oracle
 * takes the reading stated next.
 *
 * Element format: OCP 8-bit floating point E4M3 (1 sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, subnormals, no infinities; S.1111.111 is
 * NaN), largest finite value 448. Scale: one power of two 2^e per block of
 * 32 consecutive values along H, stored as its biased exponent e + 127 in
 * one byte (the E8M0 encoding of the OCP microscaling formats). For a block
 * with largest magnitude a, e is the smallest integer >= -127 with
 * a <= 448 * 2^e, so no value of the block saturates. Each code is the
 * E4M3 value nearest to x / 2^e (ties to the even code); x / 2^e is exact
 * in any binary format wide enough, so the choice does not depend on the
 * precision it is computed in. Decoding multiplies the code's value by 2^e.
 */

/* Value of an E4M3 code (NaN for S.1111.111). */
double oracle_e4m3_value(uint8_t code)
{
    int s = code >> 7, E = (code >> 3) & 0xF, m = code & 7;
    if (E == 15 && m == 7)
        return NAN;
    double mag = E == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, E - 7);
    return s ? -mag : mag;
}

/*
 * Nearest E4M3 code to v, ties to the code with an even last bit, found by
 * comparing v with every finite non-negative code; the sign is kept (a
 * negative value that rounds to zero gives -0). Returns -1 when |v| > 448
 * or v is NaN.
 */
int oracle_e4m3_round(double v)
{
    if (isnan(v) || fabs(v) > 448.0)
        return -1;
    double a = fabs(v);
    int best = 0;
    double best_d = a;
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(a - oracle_e4m3_value((uint8_t)c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (signbit(v) ? 0x80 : 0) | best;
}

/* Smallest e >= -127 with amax <= 448 * 2^e (amax finite, >= 0). */
int oracle_fp8_block_exponent(double amax)
{
    int e = -127;
    while (amax > ldexp(448.0, e))
        ++e;
    return e;
}

static int is_finite_bf16(uint16_t bits) { return (bits & 0x7F80u) != 0x7F80u; }

/* Codes and scale bytes of one row of H bf16 values (H % 32 == 0). */
static int quantize_row(const uint16_t *x, int32_t H, uint8_t *codes, uint8_t *scales)
{
    for (int32_t b = 0; b < H / 32; ++b) {
        double amax = 0.0;
        for (int32_t i = 0; i < 32; ++i) {
            if (!is_finite_bf16(x[b * 32 + i]))
                return -1;
            double a = fabs(bf16_value(x[b * 32 + i]));
            if (a > amax)
                amax = a;
        }
        int e = oracle_fp8_block_exponent(amax);
        scales[b] = (uint8_t)(e + 127);
        for (int32_t i = 0; i < 32; ++i)
            codes[b * 32 + i] = (uint8_t)oracle_e4m3_round(ldexp(bf16_value(x[b * 32 + i]), -e));
    }
    return 0;
}

/*
 * codes[r][:] and scales[r][:] (H / 32 bytes) of rows r < n of x.
 * Returns -1 when H % 32 != 0 or a row holds a NaN or an infinity (the
 * reading above leaves those unspecified).
 */
int oracle_fp8_quantize_rows(const uint16_t *x, int64_t n, int32_t H, uint8_t *codes,
                             uint8_t *scales)
{
    if (H <= 0 || H % 32 != 0)
        return -1;
    for (int64_t r = 0; r < n; ++r)
        if (quantize_row(x + r * H, H, codes + r * H, scales + r * (H / 32)) != 0)
            return -1;
    return 0;
}

/*
 * out[r][h] = bf16 nearest to value(codes[r][h]) * 2^(scales[r][h / 32] - 127),
 * ties to even. Returns -1 when H % 32 != 0 or a code is NaN.
 */
int oracle_fp8_dequant_rows(const uint8_t *codes, const uint8_t *scales, int64_t n, int32_t H,
                            uint16_t *out)
{
    if (H <= 0 || H % 32 != 0)
        return -1;
    for (int64_t r = 0; r < n; ++r)
        for (int32_t h = 0; h < H; ++h) {
            double v = oracle_e4m3_value(codes[r * H + h]);
            if (isnan(v))
                return -1;
            int e = (int)scales[r * (H / 32) + h / 32] - 127;
            out[r * H + h] = oracle_bf16_round(ldexp(v, e));
        }
    return 0;
}

/*
 * FP8 dispatch permute: for every kept (t, j), send row pos[t][j] (row_bytes
 * bytes, row_bytes >= H + H / 32) holds the H codes of x[t], then its H / 32
 * scale bytes, then zero bytes up to row_bytes. Rows no assignment points at
 * are left as they were. Returns -1 on a position outside [0, send_rows), a
 * short row, H % 32 != 0 or a non-finite x value of a kept token.
 */
int oracle_dispatch_permute_fp8(const uint16_t *x, const int32_t *pos, int64_t T, int32_t H,
                                int32_t k, uint8_t *send, int64_t send_rows, int64_t row_bytes)
{
    if (H <= 0 || H % 32 != 0 || row_bytes < H + H / 32)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < k; ++j) {
            int32_t p = pos[t * k + j];
            if (p < 0)
                continue;
            if (p >= send_rows)
                return -1;
            uint8_t *row = send + (int64_t)p * row_bytes;
            if (quantize_row(x + t * (int64_t)H, H, row, row + H) != 0)
                return -1;
            for (int64_t b = H + H / 32; b < row_bytes; ++b)
                row[b] = 0;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* tile-signalled return: stand-in expert computation                  */
/* ------------------------------------------------------------------ */

/*
 * The overlap the pages describe needs an expert matmul whose output tiles
 * each belong to one return destination: a grouped GEMM over the
 * (source, local expert) blocks of the receive buffer, so every tile's rows
 * go back to one source as one contiguous write (thecoregrid
 * "Mixture-of-experts acceleration through overlap": a producer GEMM with
 * per-tile readiness flags, a consumer that starts each transfer when its
 * tiles are ready, the remote-owner-aligned layout; aicassindra
 * "gpu_moe_all_to_all", "Overlapping dispatch with expert compute": the
 * strict chain dispatch -> compute -> combine).
 *
 * The stand-in expert is one linear map per local expert, W[l] of shape
 * [H_out][H] (output-major). For every received row i, held in block
 * (s, l) of the source-major receive buffer (cnt[s][l] rows of local
 * expert l from source s, sources in order, experts in order inside each):
 *   y[i][o] = sum_h recv[i][h] * W[l][o][h]
 * in double precision, rounded once to bf16 (nearest, ties to even). The
 * return is a bit copy of y's rows to the same positions of the sources'
 * return buffers, which on one device is y itself.
 * Returns 0, or -1 on bad sizes or negative counts.
 */
int oracle_expert_linear(const uint16_t *recv, const int32_t *cnt, int32_t S, int32_t E_l,
                         int32_t H, int32_t H_out, const uint16_t *W, uint16_t *y)
{
    if (S <= 0 || E_l <= 0 || H <= 0 || H_out <= 0)
        return -1;
    for (int32_t i = 0; i < S * E_l; ++i)
        if (cnt[i] < 0)
            return -1;
    int64_t row = 0;
    for (int32_t s = 0; s < S; ++s)
        for (int32_t l = 0; l < E_l; ++l)
            for (int32_t r = 0; r < cnt[s * E_l + l]; ++r, ++row) {
                const uint16_t *xr = recv + row * H;
                const uint16_t *wl = W + (int64_t)l * H_out * H;
                for (int32_t o = 0; o < H_out; ++o) {
                    double acc = 0.0;
                    for (int32_t h = 0; h < H; ++h)
                        acc += bf16_value(xr[h]) * bf16_value(wl[(int64_t)o * H + h]);
                    y[row * H_out + o] = oracle_bf16_round(acc);
                }
            }
    return 0;
}
