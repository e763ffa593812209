"""The workload table against the pages' figures, and the seeded generator."""
import json
import os

import numpy as np
import torch

from sparse_moe_layer_gemm_amd.inputs import WORKLOADS, make_inputs, draw_x, as_numpy_bits

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_workloads.json")))


def test_workloads_match_pages():
    ns = GOLD["nemotron3_super"]
    for name in ("decode", "prefill"):
        w = WORKLOADS[name]
        assert (w.N, w.K, w.l) == (ns["experts"], ns["top_k"], ns["latent"])
        assert w.l == ns["latent_fraction_of_d"] * w.d
    t1s, t1l = GOLD["table1_standard_moe"], GOLD["table1_latent_moe"]
    for name in ("standard_decode", "standard_prefill"):
        w = WORKLOADS[name]
        assert (w.d, w.N, w.K) == (t1s["d"], t1s["experts"], t1s["top_k"])
        assert w.standard and w.l == w.d
    assert (WORKLOADS["prefill"].l, WORKLOADS["prefill"].N, WORKLOADS["prefill"].K) == \
        (t1l["latent"], t1l["experts"], t1l["top_k"])
    k3 = GOLD["kimi_k3"]
    w = WORKLOADS["skewed"]
    assert (w.N, w.K) == (k3["experts"], k3["top_k"]) and w.N // w.K == k3["sparsity_ratio"]
    assert w.bias


def test_structural_relations():
    lat, std = WORKLOADS["prefill"], WORKLOADS["standard_prefill"]
    # per-expert weights are d/l = 4 times smaller
    ratio = (std.l * std.m) / (lat.l * lat.m)
    assert ratio == GOLD["expert_read_reduction"]["factor"]
    # N' = N d / l holds exactly for Table 1; K' = K d / l would be 24, the pages use 22
    assert std.N * std.d // lat.l == lat.N
    assert std.K * std.d // lat.l == 24 and lat.K == 22
    # total expert parameters are equal (parameter parity of the comparison)
    assert lat.N * 2 * lat.l * lat.m == std.N * 2 * std.l * std.m == 805_306_368


def test_generator_is_seeded_and_shaped():
    w = WORKLOADS["tiny_f32"]
    a = make_inputs(w, seed=0)
    b = make_inputs(w, seed=0)
    c = make_inputs(w, seed=1)
    for k in ("x", "W_down", "W_router", "W1", "W2", "W_up"):
        assert torch.equal(a[k], b[k])
        assert not torch.equal(a[k], c[k])
    assert a["x"].shape == (w.T, w.d) and a["W_down"].shape == (w.l, w.d)
    assert a["W_router"].shape == (w.N, w.d) and a["W1"].shape == (w.N, w.m, w.l)
    assert a["W2"].shape == (w.N, w.l, w.m) and a["W_up"].shape == (w.d, w.l)
    assert a["bias"] is None and a["x"].dtype == torch.float32
    # weights ~ N(0, 1/fan_in)
    assert abs(a["W1"].float().std().item() * np.sqrt(w.l) - 1.0) < 0.05


def test_generator_bf16_and_standard():
    w = WORKLOADS["standard_decode"].replace(T=4, d=64, l=64, N=8, m=32)
    a = make_inputs(w, seed=3)
    assert a["W_down"] is None and a["W_up"] is None
    assert a["x"].dtype == torch.bfloat16
    bits = as_numpy_bits(a["x"])
    assert bits.dtype == np.uint16
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, a["x"].float().numpy())
    ws = WORKLOADS["skewed"].replace(T=4, d=64, l=16, N=8, m=32)
    s = make_inputs(ws, seed=0)
    assert s["bias"].dtype == torch.float32 and s["bias"].shape == (8,)
    x2 = draw_x(w, 99)
    assert x2.shape == (4, 64) and not torch.equal(x2, a["x"])
