"""The fp64 oracle against its pins, and every planted mistake against them.

The mutation test copies the oracle's C source into a temporary folder,
replaces one snippet with a plausible mistake (a dropped term, a wrong sign or
index, a transposed operand, a wrong tie rule ...), compiles the copy, and
requires at least one pin to fail on it.
"""
import os
import shutil

import pytest

from oracle import oracle
from tests import oracle_pins as P


@pytest.fixture(scope="module")
def real():
    oracle.build()
    return oracle.Oracle(oracle.LIB)


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin_holds(real, pin):
    pin(real)


def test_routing_bruteforce_tiny_workload_shape(real):
    P.pin_routing_bruteforce_tiny_workload(real)


MUTANTS = {
    "drop_residual": ("out_t[n] = xt[n] + acc;", "out_t[n] = acc;"),
    "residual_sign": ("out_t[n] = xt[n] + acc;", "out_t[n] = xt[n] - acc;"),
    "relu_not_squared": ("h[j] = a * a;", "h[j] = a;"),
    "relu_of_square": ("double a = acc > 0.0 ? acc : 0.0;", "double a = acc;"),
    "transposed_W_down": ("widen(Wd, dt, (size_t)j * d + i)", "widen(Wd, dt, (size_t)i * l + j)"),
    "transposed_W1": ("expert_w(D, W1, s1, (e * m + j) * l + i, e * m + j)",
                      "expert_w(D, W1, s1, e * m * l + (size_t)i * m + j, e * m + j)"),
    "transposed_W2": ("expert_w(D, W2, s2, (e * l + i) * m + j, e * l + i)",
                      "expert_w(D, W2, s2, e * l * m + (size_t)j * l + i, e * l + i)"),
    "transposed_W_up": ("widen(Wu, dt, (size_t)n * l + i)", "widen(Wu, dt, (size_t)i * d + n)"),
    "router_from_latent": ("acc += widen(Wr, dt, (size_t)e * d + i) * xt[i];",
                           "acc += widen(Wr, dt, (size_t)e * d + i) * (i < l ? z[i] : 0.0);"),
    "bias_ignored": ("if (bias) acc += (double)bias[e];", "(void)bias;"),
    "tie_to_higher_index": ("(logit[a] == logit[b] && a < b)", "(logit[a] == logit[b] && a > b)"),
    "smallest_k": ("return logit[a] > logit[b] ||", "return logit[a] < logit[b] ||"),
    "gates_not_renormalised": ("gates_t[k] = p[ids_t[k]] / kept;", "gates_t[k] = p[ids_t[k]];"),
    "gate_dropped": ("s[i] += gates_t[k] * acc;", "s[i] += acc;"),
    "gate_wrong_index": ("s[i] += gates_t[k] * acc;", "s[i] += gates_t[0] * acc;"),
    "kept_sum_drops_first": ("for (int k = 0; k < K; ++k) kept += p[ids_t[k]];",
                             "for (int k = 1; k < K; ++k) kept += p[ids_t[k]];"),
    "last_expert_dropped": ("for (int k = 0; k < K; ++k) {\n        const size_t e",
                            "for (int k = 0; k < K - 1; ++k) {\n        const size_t e"),
    "softmax_temperature": ("p[e] = exp(logits_t[e] - mx);", "p[e] = exp(2.0 * (logits_t[e] - mx));"),
    "gap_from_top": ("*gap_t = logits_t[ids_t[K - 1]] - logits_t[next];",
                     "*gap_t = logits_t[ids_t[0]] - logits_t[next];"),
    "standard_mode_projects": ("            acc = s[n];\n", "            acc = 0.5 * s[n];\n"),
    "shared_dropped": ("out_t[n] += acc;", "(void)acc;"),
    "shared_relu_not_squared": ("hs[j] = r * r;", "hs[j] = r;"),
    "shared_on_latent": ("acc += widen(Ws1, dt, (size_t)j * d + i) * xt[i];",
                         "acc += widen(Ws1, dt, (size_t)j * d + i) * (i < l ? z[i] : 0.0);"),
    "shared_transposed_Ws1": ("widen(Ws1, dt, (size_t)j * d + i)", "widen(Ws1, dt, (size_t)i * ms + j)"),
    "shared_transposed_Ws2": ("widen(Ws2, dt, (size_t)n * ms + j)", "widen(Ws2, dt, (size_t)j * d + n)"),
    "fp8_exponent_bias": ("v = ldexp(1.0 + man / 8.0, ex - 7);", "v = ldexp(1.0 + man / 8.0, ex - 8);"),
    "fp8_mantissa_width": ("v = ldexp(1.0 + man / 8.0, ex - 7);", "v = ldexp(1.0 + man / 16.0, ex - 7);"),
    "fp8_subnormals_flushed": ("v = ldexp((double)man, -9);", "v = 0.0;"),
    "fp8_sign_dropped": ("return sign ? -v : v;", "return v;"),
    "fp8_scale_dropped": ("e4m3(((const uint8_t*)W)[i]) * (double)((const float*)scale)[row]",
                          "e4m3(((const uint8_t*)W)[i])"),
    "fp8_scale_wrong_row": ("e4m3(((const uint8_t*)W)[i]) * (double)((const float*)scale)[row]",
                            "e4m3(((const uint8_t*)W)[i]) * (double)((const float*)scale)[row / 2]"),
    "mx_nibbles_swapped": ("e2m1((i & 1) ? byte >> 4 : byte & 15)", "e2m1((i & 1) ? byte & 15 : byte >> 4)"),
    "mx_block_of_16": ("e8m0(((const uint8_t*)scale)[i >> 5])", "e8m0(((const uint8_t*)scale)[(i >> 4) % 64])"),
    "mx_scale_per_row": ("e8m0(((const uint8_t*)scale)[i >> 5])", "e8m0(((const uint8_t*)scale)[row])"),
    "mx_fp4_bias_2": ("ldexp(1.0 + 0.5 * man, ex - 1)", "ldexp(1.0 + 0.5 * man, ex - 2)"),
    "mx_fp4_subnormal_dropped": ("ex == 0 ? 0.5 * man :", "ex == 0 ? 0.0 :"),
    "mx_fp4_sign_dropped": ("return (c & 8) ? -v : v;", "return v;"),
    "mx_e8m0_bias_128": ("ldexp(1.0, (int)b - 127)", "ldexp(1.0, (int)b - 128)"),
    "zc_not_selectable": ("        for (int e = 0; e < Nr; ++e)\n            if (!chosen[e] && (best < 0",
                          "        for (int e = 0; e < N; ++e)\n            if (!chosen[e] && (best < 0"),
    "zc_zero_acts_as_copy": ("if (q < D->n_zero) return;", "if (q < 0) return;"),
    "zc_copy_outputs_x": ("zero_computation_expert(D, ids_t[k] - N, z, zc, gates_t[k], s);",
                          "zero_computation_expert(D, ids_t[k] - N, xt, zc, gates_t[k], s);"),
    "zc_copy_gate_dropped": ("s[i] += g * z[i];", "s[i] += z[i];"),
    "zc_const_first_only": ("q -= D->n_copy; /* constant", "q = 0; /* constant"),
    "zc_const_gate_dropped": ("s[i] += g * widen(zc,", "s[i] += widen(zc,"),
    "forced_ids_ignored": ("if (forced) for (int k = 0; k < K; ++k) ids_t[k] = forced[k];", "(void)forced;"),
    "forced_ids_first_only": ("if (forced) for (int k = 0; k < K; ++k) ids_t[k] = forced[k];",
                              "if (forced) ids_t[0] = forced[0];"),
    "forced_gates_from_own_set": (
        "    if (forced) for (int k = 0; k < K; ++k) ids_t[k] = forced[k];\n\n"
        "    /* step 3c: renormalise the kept probabilities */\n"
        "    double kept = 0.0;\n"
        "    for (int k = 0; k < K; ++k) kept += p[ids_t[k]];\n"
        "    for (int k = 0; k < K; ++k) gates_t[k] = p[ids_t[k]] / kept;\n",
        "    double kept = 0.0;\n"
        "    for (int k = 0; k < K; ++k) kept += p[ids_t[k]];\n"
        "    for (int k = 0; k < K; ++k) gates_t[k] = p[ids_t[k]] / kept;\n"
        "    if (forced) for (int k = 0; k < K; ++k) ids_t[k] = forced[k];\n"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    src = open(oracle.SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"snippet for {name} must occur once in the oracle"
    mpath = os.path.join(tmp_path, "mutant.c")
    with open(mpath, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(src=mpath, out=os.path.join(tmp_path, "libmutant.so"))
    o = oracle.Oracle(lib)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
            break
    assert caught, f"no pin fails on the planted mistake {name}"
