"""Plant plausible mistakes in a copy of the CPU oracle and check that the pins
catch every one of them. Each mutant is a textual edit of oracle/moe_oracle.c,
compiled with gcc into a temporary library; the real oracle is untouched."""
import os
import subprocess

import pytest

import oracle
from test_oracle_pins import PINS

MUTANTS = {
    "gate_up_swapped": [("float g = y[j];", "float g = y[n_half + j];"),
                        ("h[j] = s * y[n_half + j];", "h[j] = s * y[j];")],
    "sigmoid_sign": [("float ng = -g;", "float ng = g;")],
    "dequant_drops_row_scale": [("y[i] = f * row_scale;", "y[i] = f;")],
    "dequant_drops_weight_scale": [("f = f * wscale[i];", "f = f;")],
    "quant_scale_not_div127": [("*scale = a * inv127;", "*scale = a;")],
    "quant_truncates": [("float r = rintf(t);", "float r = truncf(t);")],
    "quant_round_half_away": [("float r = rintf(t);", "float r = roundf(t);")],
    "eps_added_not_floored": [("if (a < eps) a = eps;", "a = a + eps;")],
    "gemm_weight_transposed": [("s += (int64_t)a[k] * (int64_t)b[k];",
                                "s += (int64_t)a[k] * (int64_t)B[(size_t)k * N + n];")],
    "bf16_truncates": [("u += 0x7FFFu + lsb;", "u += 0u * lsb;")],
    "combine_ignores_weight": [("if (!d->fuse_route_scale) m = m * s;", "")],
    "fused_scale_drops_weight": [("const float rs2 = fold ? hs * route_w : hs;", "const float rs2 = hs;")],
    "fused_combine_weights_again": [("if (!d->fuse_route_scale) m = m * s;", "m = m * s;")],
    "fused_weight_of_first_k": [("d->fuse_route_scale != 0, expert_scales[t * K + k]",
                                 "d->fuse_route_scale != 0, expert_scales[t * K]")],
    "combine_skips_first_k": [("if (row_of_pair[t * K + k] < 0) continue;\n            const float s",
                               "if (k == 0 || row_of_pair[t * K + k] < 0) continue;\n            const float s")],
    "route_unstable_order": [("int32_t row = cursor[e]++;", "int32_t row = offsets[e + 1] - 1 - (cursor[e]++ - offsets[e]);")],
    "mask_ignored_in_route": [("    for (int32_t t = 0; t < T; ++t) {\n        if (mask && !mask[t]) continue;\n        for (int32_t k = 0; k < K; ++k) {\n            int32_t g = expert_ids[t * K + k];\n            if (g < 0 || g >= d->E_g) { ++bad; continue; }",
                               "    for (int32_t t = 0; t < T; ++t) {\n        for (int32_t k = 0; k < K; ++k) {\n            int32_t g = expert_ids[t * K + k];\n            if (g < 0 || g >= d->E_g) { ++bad; continue; }"),
                              ("    for (int32_t t = 0; t < T; ++t) {\n        if (mask && !mask[t]) continue;\n        for (int32_t k = 0; k < K; ++k) {\n            int32_t g = expert_ids[t * K + k];\n            if (g < 0 || g >= d->E_g) continue;",
                               "    for (int32_t t = 0; t < T; ++t) {\n        for (int32_t k = 0; k < K; ++k) {\n            int32_t g = expert_ids[t * K + k];\n            if (g < 0 || g >= d->E_g) continue;")],
    "smooth_after_quant": [("if (ev->smooth) v = v * ev->smooth[i];", "")],
    "shared_uses_routed_smooth": [("expert_view ev = {sw1, sw1s, sw2, sw2s, share_smooth, Is, sw1b, sw2b};",
                                   "expert_view ev = {sw1, sw1s, sw2, sw2s, smooth, Is, sw1b, sw2b};")],
    "ep_rank_offset_ignored": [("const int32_t base = d->ep_rank * E;", "const int32_t base = 0;")],
    # the FP4-weight / FP8-activation variant
    "e4m3_truncates": [("float m = rintf(ldexpf(a, 3 - E));", "float m = truncf(ldexpf(a, 3 - E));")],
    "e4m3_subnormal_step": [("const float m = rintf(a * 512.0f);", "const float m = rintf(a * 256.0f);")],
    "e2m1_bias_off": [("ldexpf(1.0f + 0.5f * (float)m, e - 1)", "ldexpf(1.0f + 0.5f * (float)m, e)")],
    "mx_nibble_order_swapped": [("(k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15)",
                                 "(k & 1) ? (uint8_t)(byte & 15) : (uint8_t)(byte >> 4)")],
    "mx_block_scale_bias": [("(int)sc[blk] - 127 - 10", "(int)sc[blk] - 128 - 10")],
    "fp8_quant_uses_127": [("float t = v[i] * 448.0f;", "float t = v[i] * 127.0f;")],
    # group-wise activation scales
    "group_scale_of_next_group": [("p = p * a_scales[g];", "p = p * a_scales[(g + 1) % (Kd / G)];")],
    "group_partial_skips_weight_scale": [("p = p * wscale[n];", "p = p + 0.0f * wscale[n];")],
    "group_sum_skips_first_group": [("for (int32_t g = 0; g < Kd / G; ++g) {", "for (int32_t g = 1; g < Kd / G; ++g) {")],
    "group_quant_whole_row": [("moe_oracle_quant_row(v + (size_t)g * G, G, eps, q + (size_t)g * G, &scales[g]);",
                               "{ float t_; moe_oracle_quant_row(v, n, eps, q, &t_); scales[g] = t_; }")],
}


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    src = source
    for old, new in MUTANTS[name]:
        assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(src)
    so = str(tmp_path / "libmutant.so")
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-I", os.path.dirname(oracle.SRC), str(path), "-o", so, "-lm"])
    caught = []
    with oracle.using(so):
        for pin in PINS:
            try:
                pin()
            except (AssertionError, OverflowError, RuntimeError):
                caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
