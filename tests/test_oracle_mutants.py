"""Each plausible mistake in the oracle must fail at least one pin.

A mutant is the oracle source with one textual edit (a sign slip, a dropped
term, a swapped operand, the other grid_sample convention ...), compiled on
the CPU into a temporary library. The pins run against it in a child process
(a mutant that reads out of bounds may crash; that also counts as caught).
CPU only; nothing here touches a GPU.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "p3d_oracle.c")

# (id, text in the oracle source, replacement)
MUTANTS = [
    ("std_without_mean_square", "double var = (raw[4 + h] - N * mean * mean) / N;",
     "double var = raw[4 + h] / N;"),
    ("std_sample_not_population", "double var = (raw[4 + h] - N * mean * mean) / N;",
     "double var = (raw[4 + h] - N * mean * mean) / (N - 1.0);"),
    ("mean_over_tokens_not_samples", "const double mean = raw[2 + h] / N;",
     "const double mean = raw[2 + h] / tokens;"),
    ("camera_looks_down_plus_z", "float depth = dist[b] - pz;", "float depth = dist[b] + pz;"),
    ("image_y_not_flipped", "float gy = -((f * py) / depth);", "float gy = ((f * py) / depth);"),
    ("x_y_swapped", "float gx = (f * px) / depth;", "float gx = (f * py) / depth;"),
    ("align_corners_true", "float ix = ((g + 1.0f) * (float)size - 1.0f) / 2.0f;",
     "float ix = (g + 1.0f) / 2.0f * (float)(size - 1);"),
    ("half_texel_dropped", "float ix = ((g + 1.0f) * (float)size - 1.0f) / 2.0f;",
     "float ix = ((g + 1.0f) * (float)size) / 2.0f;"),
    ("clamp_corners_not_index",
     "    ix = fminf(fmaxf(ix, 0.0f), (float)(size - 1));\n    float fl = floorf(ix);\n    *i0 = (int32_t)fl;\n    *t = ix - fl;\n    *i1 = (*i0 + 1 < size) ? *i0 + 1 : size - 1;",
     "    float fl = floorf(ix);\n    *t = ix - fl;\n    int32_t a = (int32_t)fmaxf(fminf(fl, (float)(size - 1)), 0.0f);\n    int32_t c = (int32_t)fmaxf(fminf(fl + 1.0f, (float)(size - 1)), 0.0f);\n    if (!(*t >= 0.0f && *t <= 1.0f)) *t = 0.0f;\n    *i0 = a;\n    *i1 = c;"),
    ("second_texel_dropped", "*i1 = (*i0 + 1 < size) ? *i0 + 1 : size - 1;", "*i1 = *i0;"),
    ("weights_swapped", "float w01 = tx * (1.0f - ty);", "float w01 = (1.0f - tx) * ty;"),
    ("corner_rows_swapped", "int64_t r10 = (base + y1) * W + x0, r11 = (base + y1) * W + x1;",
     "int64_t r10 = (base + y1) * W + x1, r11 = (base + y1) * W + x0;"),
    ("cell_node_not_centre", "return ((float)c + 0.5f) / (float)R - 0.5f;",
     "return (float)c / (float)R - 0.5f;"),
    ("fov_as_half_angle_focal", "*focal = (float)(1.0 / tan(fov_deg * pi / 360.0));",
     "*focal = (float)(1.0 / tan(fov_deg * pi / 180.0));"),
    ("distance_full_extent", "return 0.5 / tan(half_angle) * half_size / (half_size + (double)extend_px);",
     "return 1.0 / tan(half_angle) * half_size / (half_size + (double)extend_px);"),
    ("distance_extend_ignored", "return 0.5 / tan(half_angle) * half_size / (half_size + (double)extend_px);",
     "return 0.5 / tan(half_angle);"),
    ("mask_exclusive_border", "gx >= -1.0f && gx <= 1.0f &&", "gx > -1.0f && gx < 1.0f &&"),
    ("mask_ignores_depth", "uint8_t m = (uint8_t)(valid && depth > 0.0f &&", "uint8_t m = (uint8_t)(valid &&"),
    ("linear_weight_transposed", "acc += param_at(weight, is_bf16, (int64_t)d * C + c) * S[i * (int64_t)C + c];",
     "acc += param_at(weight, is_bf16, (int64_t)(c % D) * C + (d % C)) * S[i * (int64_t)C + c];"),
    ("linear_bias_dropped", "            if (bias) acc += param_at(bias, is_bf16, d);\n            Y[i",
     "            Y[i"),
    ("null_rows_zero", "y[d] = bias ? param_at(bias, is_bf16, d) : 0.0;", "y[d] = 0.0;"),
    ("bf16_truncates", "if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))",
     "if (0)"),
    ("bf16_ties_away", "if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))",
     "if (dropped >= 0x8000u)"),
    ("dense_order_zyx", "cell[3] = (int32_t)(n % r);", "cell[3] = (int32_t)((n / (r * r)) % r); cell[1] = (int32_t)(n % r); if (0)"),
    ("node_spacing_over_R", "return (float)c / (float)(R - 1) - 0.5f;",
     "return (float)c / (float)R - 0.5f;"),
    ("node_full_linspace_extent", "return (float)c / (float)(R - 1) - 0.5f;",
     "return 2.0f * (float)c / (float)(R - 1) - 1.0f;"),
    ("node_mode_ignored", "return points ? grid_node(c, R) : cell_centre(c, R);",
     "return cell_centre(c, R);"),
    ("requant_round_floors", "if (2 * rem > den || (2 * rem == den && (q & 1))) q += 1;",
     "if (0) q += 1;"),
    ("requant_ties_up", "if (2 * rem > den || (2 * rem == den && (q & 1))) q += 1;",
     "if (2 * rem >= den) q += 1;"),
    ("requant_no_half_cell", "int64_t num = (2 * (int64_t)c + 1) * (int64_t)(grid - 1);",
     "int64_t num = (2 * (int64_t)c) * (int64_t)(grid - 1);"),
    ("requant_floor_over_grid_minus_1",
     "if (mode == 1) return (int32_t)(((2 * (int64_t)c + 1) * grid) / den);",
     "if (mode == 1) return (int32_t)(((2 * (int64_t)c + 1) * (grid - 1)) / den);"),
    ("two_maps_share_first_size",
     "sample_one(feats[m], is_bf16, b, Hs[m], Ws[m], Cs[m], gx, gy, s + off);",
     "sample_one(feats[m], is_bf16, b, Hs[0], Ws[0], Cs[m], gx, gy, s + off);"),
    ("two_maps_order_reversed",
     "sample_one(feats[m], is_bf16, b, Hs[m], Ws[m], Cs[m], gx, gy, s + off);",
     "sample_one(feats[m], is_bf16, b, Hs[m], Ws[m], Cs[m], gx, gy, s + (C - off - Cs[m]));"),
    ("grouped_bias_of_block_0",
     "orc_linear(S, nrows, K, weights[g], biases ? biases[g] : NULL, is_bf16, D, y);",
     "orc_linear(S, nrows, K, weights[g], biases ? biases[0] : NULL, is_bf16, D, y);"),
    ("grouped_weight_of_block_0",
     "orc_linear(S, nrows, K, weights[g], biases ? biases[g] : NULL, is_bf16, D, y);",
     "orc_linear(S, nrows, K, weights[0], biases ? biases[g] : NULL, is_bf16, D, y);"),
    ("grouped_residual_dropped", "y[i] += res[g][i];", "y[i] += 0.0 * res[g][i];"),
    ("sample_rows_map1_offset_dropped",
     "                       S_out + k * (int64_t)C + off);",
     "                       S_out + k * (int64_t)C);"),
    ("stats_maps_share_first_size",
     "sample_one(feats[m], is_bf16, b, Hs[m], Ws[m], Cs[m], gx, gy, &s[off]);",
     "sample_one(feats[m], is_bf16, b, Hs[0], Ws[0], Cs[m], gx, gy, &s[off]);"),
    ("stats_sum_sq_not_squared", "out[4 + m] += s[off + c] * s[off + c];",
     "out[4 + m] += s[off + c];"),
    ("stats_cosine_unnormalised", "out[6] += dot / (sqrt(n0) * sqrt(n1));", "out[6] += dot;"),
    ("stats_cosine_same_half", "dot += s[c] * s[Cs[0] + c];", "dot += s[c] * s[c];"),
    ("stats_coverage_counts_all", "out[1] += (double)msk;", "out[1] += 1.0;"),
    ("stats_halves_swapped", "out[2 + m] += s[off + c];", "out[3 - m] += s[off + c];"),
    ("stats_unrounded_bf16",
     "        if (is_bf16)\n            for (int32_t c = 0; c < C; ++c) s[c] = (double)orc_bf16_to_f32(orc_f64_to_bf16(s[c]));\n        out[0] += 1.0;",
     "        out[0] += 1.0;"),
]

RUNNER = r"""
import json, sys, traceback
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + "/tests")
import oracle, oracle_pins
o = oracle.Oracle(sys.argv[2])
failed = []
for name, fn in sorted(oracle_pins.ALL_PINS.items()):
    try:
        fn(o)
    except Exception:
        failed.append(name)
print(json.dumps(failed))
"""


def _build(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor for %s not found exactly once" % name
    path = tmp_path / ("mut_%s.c" % name)
    path.write_text(src.replace(old, new))
    lib = tmp_path / ("libmut_%s.so" % name)
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    obuild.build(src=str(path), out=str(lib), extra=["-Wno-unused-variable",
                                                     "-Wno-unused-but-set-variable",
                                                     "-Wno-unused-parameter",
                                                     "-Wno-unused-function"])
    return str(lib)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    lib = _build(tmp_path, name, old, new)
    r = subprocess.run([sys.executable, "-c", RUNNER, ROOT, lib], capture_output=True,
                       text=True, timeout=300)
    if r.returncode != 0:
        return  # crashed: caught
    failed = json.loads(r.stdout.strip().splitlines()[-1])
    assert failed, "mutant %s passed every pin" % name
