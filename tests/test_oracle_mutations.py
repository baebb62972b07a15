"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of oracle.c (a flipped tie-break, a
dropped term, an off-by-one, a wrong index), builds it with gcc and runs the
oracle pin tests against it in a subprocess; every variant must fail them.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PIN_TESTS = ["tests/test_oracle_route.py", "tests/test_oracle_layout.py", "tests/test_oracle_combine.py",
             "tests/test_oracle_regroup.py", "tests/test_oracle_fp8.py", "tests/test_oracle_expert.py",
             "tests/test_oracle_properties.py"]

MUTATIONS = {
    "tie_break_to_higher_id": ("    return ia < ib;\n", "    return ia > ib;\n"),
    "nan_ranks_on_top": ("    if (!na && nb)\n        return 1;", "    if (!na && nb)\n        return 0;"),
    # the first call is the plain router's (the grouped router makes the second)
    "weights_from_biased_scores": ("gate_weights(row, idx, E, k, normalize,", "gate_weights(s, idx, E, k, normalize,", "first"),
    "grouped_weights_from_biased_scores": ("gate_weights(row, idx, E, k, normalize,", "gate_weights(s, idx, E, k, normalize,", "last"),
    "weights_not_normalised": ("            w[j] /= sum;", "            w[j] /= 1.0;"),
    "score_ignores_bias": ("s[e] = bias ? row[e] + bias[e] : row[e];", "s[e] = row[e];"),
    "capacity_off_by_one": ("if (capacity >= 0 && seen[e] >= capacity)", "if (capacity >= 0 && seen[e] > capacity)"),
    "offsets_from_demand": ("expert_offsets[e] + counts[e];", "expert_offsets[e] + demand[e];"),
    "dest_offset_wrong_index": ("dest_offsets[r] = expert_offsets[r * el];", "dest_offsets[r] = expert_offsets[r];"),
    "permute_reversed_row": ("send[(int64_t)p * H + h] = x[t * (int64_t)H + h];",
                             "send[(int64_t)p * H + h] = x[t * (int64_t)H + (H - 1 - h)];"),
    "combine_drops_residual": ("acc += bf16_value(residual[t * (int64_t)H + h]);",
                               "acc += 0.0 * bf16_value(residual[t * (int64_t)H + h]);"),
    "combine_half_shared": ("acc += bf16_value(shared[t * (int64_t)H + h]);",
                            "acc += 0.5 * bf16_value(shared[t * (int64_t)H + h]);"),
    "combine_weight_index_reversed": ("acc += w[t * k + j] *", "acc += w[t * k + (k - 1 - j)] *"),
    "combine_keeps_dropped_term": ("                if (p < 0)\n                    continue;\n                acc",
                                   "                if (p < 0)\n                    p = 0;\n                acc"),
    "group_score_from_worst_member": ("                if (ranks_above(s[e], e, s[best], best))\n                    best = e;\n            gbest[g] = best;",
                                      "                if (ranks_above(s[best], best, s[e], e))\n                    best = e;\n            gbest[g] = best;"),
    "group_mask_ignored": ("            taken[e] = !gsel[e / gsize];", "            taken[e] = 0;"),
    "regroup_counts_earlier_experts": ("                before += cnt[s2 * E_l + l];", "                before += cnt[src * E_l + s2 % E_l];"),
    "regroup_expert_base_off_by_one": ("                recv_pos[i++] = local_expert_offsets[l] + before + j;",
                                       "                recv_pos[i++] = local_expert_offsets[l] + before + j + (l > 0);"),
    "e4m3_ties_to_odd": ("(d == best_d && (c & 1) == 0)", "(d == best_d && (c & 1) == 1)"),
    "e4m3_subnormal_spacing": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "e4m3_exponent_bias": ("ldexp(1.0 + m / 8.0, E - 7)", "ldexp(1.0 + m / 8.0, E - 8)"),
    "fp8_scale_one_too_large_at_the_edge": ("while (amax > ldexp(448.0, e))", "while (amax >= ldexp(448.0, e))"),
    "fp8_scale_for_256": ("while (amax > ldexp(448.0, e))", "while (amax > ldexp(256.0, e))"),
    "fp8_dequant_scale_bias": ("int e = (int)scales[r * (H / 32) + h / 32] - 127;",
                               "int e = (int)scales[r * (H / 32) + h / 32] - 126;"),
    "fp8_amax_ignores_sign": ("double a = fabs(bf16_value(x[b * 32 + i]));", "double a = bf16_value(x[b * 32 + i]);"),
    "fp8_permute_padding_not_cleared": ("            for (int64_t b = H + H / 32; b < row_bytes; ++b)\n                row[b] = 0;",
                                        "            for (int64_t b = H + H / 32 + 1; b < row_bytes; ++b)\n                row[b] = 0;"),
    "fp8_permute_scales_misplaced": ("quantize_row(x + t * (int64_t)H, H, row, row + H)",
                                     "quantize_row(x + t * (int64_t)H, H, row, row + H + 1)"),
    "expert_weights_of_next_expert": ("const uint16_t *wl = W + (int64_t)l * H_out * H;",
                                      "const uint16_t *wl = W + (int64_t)((l + 1) % E_l) * H_out * H;"),
    "expert_weights_transposed": ("acc += bf16_value(xr[h]) * bf16_value(wl[(int64_t)o * H + h]);",
                                  "acc += bf16_value(xr[h]) * bf16_value(wl[(int64_t)h * H_out + o]);"),
    "expert_drops_last_term": ("                    for (int32_t h = 0; h < H; ++h)\n                        acc +=",
                               "                    for (int32_t h = 0; h < H - 1; ++h)\n                        acc +="),
    "bf16_ties_away_from_zero": ("double r = nearbyint(a / q) * q;", "double r = round(a / q) * q;"),
    "bf16_no_subnormal_spacing": ("if (e < -126)\n        e = -126;", "if (e < -140)\n        e = -140;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, tmp_path):
    old, new, *where = MUTATIONS[name]
    src = open(SRC).read()
    if not where:
        assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
        text = src.replace(old, new)
    else:
        i = src.find(old) if where[0] == "first" else src.rfind(old)
        assert i >= 0 and src.count(old) == 2, f"mutation anchor for {name} not found twice"
        text = src[:i] + new + src[i + len(old):]
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(text)
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-shared",
                    "-fPIC", str(mutated), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PIN_TESTS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutation {name} survived the pins:\n{r.stdout[-2000:]}"
