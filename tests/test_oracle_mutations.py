"""Planted mistakes: each mutant of the oracle source must fail at least one oracle pin.

The mutants are built on the CPU from a textual copy of oracle/moe_oracle.c in a temporary folder; the
committed oracle is never changed. This shows the pins (worked examples, the dense-MLP special case,
brute force, library softmax/sigmoid, metamorphic relations) are strong enough to catch a dropped term,
a wrong sign or index, a swapped operand or a wrong rounding.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "nibble_order": ("int code = (kk & 1) ? (byte >> 4) : (byte & 0xF);",
                     "int code = (kk & 1) ? (byte & 0xF) : (byte >> 4);"),
    "e2m1_bias": ("mag = ldexp(1.0 + 0.5 * (double)mant, expo - 1);",
                  "mag = ldexp(1.0 + 0.5 * (double)mant, expo);"),
    "e8m0_bias": ("return ldexp(1.0, byte - 127);", "return ldexp(1.0, byte - 128);"),
    "scale_row_offset": ("s[n * (long)(K / 32) + kk / 32]", "s[kk / 32]"),
    "gate_up_swapped": ("g += xd[hh] * oracle_mxfp4_element(q13, s13, H, i, hh);\n"
                        "        u += xd[hh] * oracle_mxfp4_element(q13, s13, H, (long)I + i, hh);",
                        "g += xd[hh] * oracle_mxfp4_element(q13, s13, H, (long)I + i, hh);\n"
                        "        u += xd[hh] * oracle_mxfp4_element(q13, s13, H, i, hh);"),
    "silu_sign": ("hv[i] = g / (1.0 + exp(-g)) * u;", "hv[i] = g / (1.0 + exp(g)) * u;"),
    "clamp_gate_only": ("u = fmin(fmax(u, -clamp_limit), clamp_limit);", ";"),
    "w2_k_reversed": ("oracle_mxfp4_element(q2, s2, I, n, i)", "oracle_mxfp4_element(q2, s2, I, n, I - 1 - i)"),
    "combine_weight_index": ("acc += topk_w[t * k + j] * y[(t * k + j) * H + n];",
                             "acc += topk_w[t * k] * y[(t * k + j) * H + n];"),
    "tie_to_higher_index": ("if (best < 0 || l[e] > l[best]) best = e;",
                            "if (best < 0 || l[e] >= l[best]) best = e;"),
    "no_renorm": ("topk_w[(long)t * k + j] = renorm ? sc / sel : sc;", "topk_w[(long)t * k + j] = sc;"),
    "softmax_denominator": ("for (int e = 0; e < E; ++e) score[e] /= z;",
                            "for (int e = 0; e < E; ++e) score[e] /= (z + 1.0);"),
    "sigmoid_sign": ("score[e] = 1.0 / (1.0 + exp(-(double)l[e]));", "score[e] = 1.0 / (1.0 + exp((double)l[e]));"),
    "unstable_group": ("sorted_pair[r] = (int32_t)p;", "sorted_pair[r] = (int32_t)(P - 1 - p);"),
    "bf16_truncate": ("double r = ldexp(nearbyint(ldexp(a, -q)), q);", "double r = ldexp(floor(ldexp(a, -q)), q);"),
    "x_decode_shift": ("uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    "router_last_term_dropped": ("for (long h = 0; h < H; ++h) acc +=", "for (long h = 0; h < H - 1; ++h) acc +="),
    "router_k_reversed": ("oracle_bf16_to_double(wr[h]);", "oracle_bf16_to_double(wr[H - 1 - h]);"),
    "e4m3_bias": ("mag = ldexp(1.0 + (double)mant / 8.0, expo - 7);", "mag = ldexp(1.0 + (double)mant / 8.0, expo - 8);"),
    "e4m3_subnormal_exponent": ("mag = ldexp((double)mant / 8.0, -6);", "mag = ldexp((double)mant / 8.0, -7);"),
    "e4m3_min_normal": ("round_to_grid(fabs(v), 3, -6, 448.0)", "round_to_grid(fabs(v), 3, -7, 448.0)"),
    "round_ties_away": ("double r = nearbyint(a / ulp) * ulp;", "double r = round(a / ulp) * ulp;"),
    "e2m1_no_saturation": ("round_to_grid(fabs(v), 1, 0, 6.0)", "round_to_grid(fabs(v), 1, 0, 8.0)"),
    "mx_emax_fp8": ("(fmt == ORACLE_ACT_MXFP8 ? 8 : 2)", "(fmt == ORACLE_ACT_MXFP8 ? 7 : 2)"),
    "mx_emax_fp4": ("(fmt == ORACLE_ACT_MXFP8 ? 8 : 2)", "(fmt == ORACLE_ACT_MXFP8 ? 8 : 1)"),
    "mx_shared_exponent_ceil": ("int shared = (e - 1) - ", "int shared = e - "),
    "mx_no_low_clamp": ("if (shared < -127) shared = -127;", ";"),
    "mx_last_element_ignored": ("for (int i = 0; i < 32; ++i)\n    if (fabs(v[i]) > amax)",
                                "for (int i = 0; i < 31; ++i)\n    if (fabs(v[i]) > amax)"),
    "mx_block_offset": ("oracle_mx_quantize_block(v + 32 * b, fmt, codes)", "oracle_mx_quantize_block(v, fmt, codes)"),
    "x_not_quantised": ("if (act_fmt != ORACLE_ACT_NONE) mx_fake_quantize(xd, H / 32, act_fmt);", ";"),
    "h_not_quantised": ("      mx_fake_quantize(hv, I / 32, act_fmt);", ";"),
    "h_not_rounded_to_binary32": ("hv[i] = (double)(float)hv[i];", "hv[i] = hv[i];"),
}

PIN_MODULES = ["test_oracle_formats.py", "test_oracle_route.py", "test_oracle_group.py", "test_oracle_ffn.py",
               "test_oracle_router.py", "test_oracle_act_quant.py"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation site for {name} not found exactly once"
    mut_src = tmp_path / "moe_oracle.c"
    mut_src.write_text(src.replace(before, after))
    lib = str(tmp_path / "libmutant.so")
    oracle.compile_oracle(str(mut_src), lib)
    env = dict(os.environ, MOE_ORACLE_LIB_OVERRIDE=lib)
    tests_dir = os.path.join(ROOT, "tests")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *[os.path.join(tests_dir, m) for m in PIN_MODULES]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived every pin:\n{r.stdout[-2000:]}"
