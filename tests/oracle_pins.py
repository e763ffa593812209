"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each pin is a function taking an `oracle.Oracle` handle and raising
AssertionError when the oracle disagrees with the fact.  tests/
test_oracle_pins.py runs them against the real oracle (all must hold) and
against copies of the oracle with a planted mistake (at least one must fail
for every mistake).

What pins what:
  routing      brute-force enumeration of every K-subset (itertools), with
               logits from a numpy float64 matmul
  tie-break    constructed bit-equal logits (one-hot tokens)
  gates        sum to 1; g_i / g_j = exp(l_i - l_j); K = 1 gives 1; K = N
               gives the full softmax (scipy.special.softmax)
  whole layer  l = d with identity projections equals the standard MoE
               bit-exactly; N = K = 1 is a dense FFN evaluated with numpy
               float64 matmuls; a hand-worked integer example with equal
               gates
  superposition out - x = sum_k g_k (single-expert output_k - x)
  residual     W_up = 0 or W2 = 0 gives out == x exactly
  homogeneity  2 W2 -> 2x, 2 W1 -> 4x (ReLU^2 is degree 2), 2 W_up -> 2x
  symmetry     token permutation permutes outputs; relabelling experts keeps
               outputs
  shared       with the routed experts silenced (W2 = 0) the layer is x plus
  expert       a dense FFN on x evaluated with numpy float64 matmuls; with
               them on, adding the shared expert adds exactly that FFN;
               W_s2 = 0 gives the layer without it bit-exactly
  FP8 experts  every E4M3 code, decoded by torch.float8_e4m3fn, times a
               power-of-two row scale is exact in float32: the FP8 layer
               equals the float32 layer on those weights bit-exactly; with
               arbitrary row scales, N = K = 1 is a dense FFN in numpy
  MXFP4        E2M1 codes decoded by a table of the OCP MX element values,
  experts      E8M0 scales by numpy ldexp, blocks by numpy repeat: the MXFP4
               layer equals the float32 layer on those weights bit-exactly
               (every byte value appears, the scales differ per block); N = K
               = 1 is a dense FFN in numpy
  zero-        a dense-mask evaluation in numpy (every routed id's output
  computation  for every token, weighted by a [T, Nr] gate matrix that is
  experts      zero off the top K); K = 1 special cases with closed forms:
               a zero expert gives x exactly, a copy expert x + W_up W_down x
               (2x exactly in standard mode), a constant expert x + W_up c;
               zero-computation experts that never win leave the layer
               bit-exactly as without them
"""
from __future__ import annotations

import itertools

import numpy as np
from scipy.special import softmax


def _rng(seed):
    return np.random.default_rng(seed)


def rand_layer(seed, T, d, l, N, m, *, dtype="f32", standard=False, bias=False):
    """Small random layer in the oracle's storage layout (float32 values)."""
    r = _rng(seed)
    f = np.float32
    L = {
        "x": r.standard_normal((T, d)).astype(f),
        "W_down": None if standard else (r.standard_normal((l, d)) / np.sqrt(d)).astype(f),
        "W_router": (r.standard_normal((N, d)) / np.sqrt(d)).astype(f),
        "W1": (r.standard_normal((N, m, l)) / np.sqrt(l)).astype(f),
        "W2": (r.standard_normal((N, l, m)) / np.sqrt(m)).astype(f),
        "W_up": None if standard else (r.standard_normal((d, l)) / np.sqrt(l)).astype(f),
        "bias": r.standard_normal(N).astype(f) if bias else None,
    }
    if dtype == "bf16":
        for k in ("x", "W_down", "W_router", "W1", "W2", "W_up"):
            if L[k] is not None:
                L[k] = to_bf16_bits(L[k])
    return L


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def f64(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def run(o, L, K, **kw):
    return o.forward(L["x"], L["W_down"], L["W_router"], L["W1"], L["W2"], L["W_up"], K,
                     bias=L.get("bias"), standard=L["W_down"] is None,
                     W_s1=L.get("W_s1"), W_s2=L.get("W_s2"), **kw)


def add_shared(L, seed, ms):
    """A shared expert of width ms on the layer L (float32 values)."""
    r = _rng(seed)
    T, d = L["x"].shape
    L = dict(L)
    L["W_s1"] = (r.standard_normal((ms, d)) / np.sqrt(d)).astype(np.float32)
    L["W_s2"] = (r.standard_normal((d, ms)) / np.sqrt(ms)).astype(np.float32)
    return L


def np_shared(L):
    """x -> W_s2 relu(W_s1 x)^2 with numpy float64 matmuls."""
    h = f64(L["x"]) @ f64(L["W_s1"]).T
    return (np.maximum(h, 0.0) ** 2) @ f64(L["W_s2"]).T


def np_logits(L):
    lg = f64(L["x"]) @ f64(L["W_router"]).T
    if L.get("bias") is not None:
        lg = lg + L["bias"].astype(np.float64)
    return lg


# ---------------------------------------------------------------------------
# routing

def brute_force_topk(logits_row, K):
    """The unique K-subset S with: every e in S outranks every f outside S
    (larger logit, or equal logit and lower index).  Found by enumeration."""
    N = len(logits_row)
    found = []
    for S in itertools.combinations(range(N), K):
        Sset = set(S)
        ok = True
        for e in S:
            for f in range(N):
                if f in Sset:
                    continue
                if not (logits_row[e] > logits_row[f] or (logits_row[e] == logits_row[f] and e < f)):
                    ok = False
                    break
            if not ok:
                break
        if ok:
            found.append(S)
    assert len(found) == 1, f"expected exactly one dominating subset, found {len(found)}"
    return set(found[0])


def pin_routing_bruteforce(o):
    for seed, (T, d, l, N, K, m), bias in [(1, (8, 16, 8, 6, 2, 8), False),
                                            (2, (6, 24, 8, 9, 4, 8), True),
                                            (3, (4, 32, 16, 12, 5, 8), False)]:
        L = rand_layer(seed, T, d, l, N, m, bias=bias)
        r = run(o, L, K)
        ref = np_logits(L)
        assert np.allclose(r["logits"], ref, rtol=1e-12, atol=1e-12), "logits differ from x W_router^T (+b)"
        for t in range(T):
            S = brute_force_topk(r["logits"][t], K)
            assert set(r["ids"][t].tolist()) == S, f"token {t}: ids {r['ids'][t]} != brute force {sorted(S)}"
            # rank order: non-increasing logits, ties by index
            ids = r["ids"][t]
            for a, b in zip(ids[:-1], ids[1:]):
                la, lb = r["logits"][t][a], r["logits"][t][b]
                assert la > lb or (la == lb and a < b), "ids not in rank order"
            # the chosen subset has the largest logit sum of all K-subsets
            best = max(sum(r["logits"][t][list(c)]) for c in itertools.combinations(range(N), K))
            assert np.isclose(sum(r["logits"][t][ids]), best, rtol=0, atol=1e-12)
            # gap = K-th minus (K+1)-th largest logit
            srt = np.sort(r["logits"][t])[::-1]
            assert np.isclose(r["gap"][t], srt[K - 1] - srt[K], rtol=0, atol=1e-12)


def pin_routing_bruteforce_tiny_workload(o, T=12):
    """The tiny workload's routing shape (N = 32, K = 4): C(32,4) = 35,960
    subsets per token, checked by a sum criterion that is equivalent to
    dominance when the logits are distinct."""
    L = rand_layer(11, T, 256, 64, 32, 128)
    r = run(o, L, 4)
    for t in range(T):
        lg = r["logits"][t]
        assert len(set(lg.tolist())) == len(lg)
        best = max(itertools.combinations(range(32), 4), key=lambda c: sum(lg[list(c)]))
        assert set(r["ids"][t].tolist()) == set(best)


def pin_tie_break(o):
    # One-hot tokens make each logit exactly one weight value.
    N, K, d, l, m = 8, 3, 8, 4, 4
    L = rand_layer(5, 3, d, l, N, m)
    x = np.zeros((3, d), np.float32)
    x[:, 0] = 1.0
    L["x"] = x
    col = np.array([0.5, 2.0, 0.25, 1.0, -1.0, 0.125, 2.0, 1.0], np.float32)
    L["W_router"][:, 0] = col
    r = run(o, L, K)
    # 2.0 at experts 1 and 6 (1 first), then 1.0 at experts 3 and 7: 3 wins the last place
    for t in range(3):
        assert r["ids"][t].tolist() == [1, 6, 3], r["ids"][t]
        assert r["gap"][t] == 0.0
    # duplicated router rows give bit-equal logits; the lower index must win
    L2 = rand_layer(6, 5, 16, 8, 7, 8)
    L2["W_router"][5] = L2["W_router"][2].copy()
    r2 = run(o, L2, 7)
    for t in range(5):
        ids = r2["ids"][t].tolist()
        assert r2["logits"][t][2] == r2["logits"][t][5]
        assert ids.index(2) < ids.index(5)


# ---------------------------------------------------------------------------
# gates

def pin_gates(o):
    L = rand_layer(7, 10, 32, 16, 12, 8, bias=True)
    for K in (1, 3, 12):
        r = run(o, L, K)
        g, ids, lg = r["gates"], r["ids"], r["logits"]
        assert np.all(np.abs(g.sum(axis=1) - 1.0) <= 1e-15 * K + 1e-15)
        assert np.all(g > 0)
        if K == 1:
            assert np.all(g == 1.0)
        for t in range(10):
            for i in range(K):
                for j in range(K):
                    ratio = g[t, i] / g[t, j]
                    assert np.isclose(ratio, np.exp(lg[t, ids[t, i]] - lg[t, ids[t, j]]), rtol=1e-12)
        if K == 12:  # K = N: the full softmax of the logits, in id order
            full = softmax(np_logits(L), axis=1)
            for t in range(10):
                assert np.allclose(g[t], full[t][ids[t]], rtol=1e-12, atol=0)


# ---------------------------------------------------------------------------
# whole layer

def pin_identity_reduces_to_standard(o):
    for dtype in ("f32", "bf16"):
        T, d, N, K, m = 9, 32, 10, 3, 16
        Ls = rand_layer(8, T, d, d, N, m, dtype=dtype, standard=True, bias=True)
        eye = np.eye(d, dtype=np.float32)
        Ll = dict(Ls)
        Ll["W_down"] = eye if dtype == "f32" else to_bf16_bits(eye)
        Ll["W_up"] = Ll["W_down"].copy()
        rs = run(o, Ls, K)
        rl = run(o, Ll, K)
        assert np.array_equal(rs["ids"], rl["ids"])
        assert np.array_equal(rs["gates"], rl["gates"])
        assert np.array_equal(rs["out"], rl["out"]), "identity projections must give the standard MoE bit-exactly"


def pin_dense_ffn_special_case(o):
    """N = K = 1: out = x + W_up (W2 relu(W1 W_down x)^2), by numpy matmuls."""
    for dtype, (T, d, l, m) in [("f32", (7, 48, 16, 24)), ("bf16", (5, 64, 32, 40))]:
        L = rand_layer(9, T, d, l, 1, m, dtype=dtype)
        r = run(o, L, 1)
        X = f64(L["x"])
        Z = X @ f64(L["W_down"]).T
        H = Z @ f64(L["W1"][0]).T
        A = np.maximum(H, 0.0) ** 2
        Y = A @ f64(L["W2"][0]).T
        ref = X + Y @ f64(L["W_up"]).T
        assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
        assert np.all(r["ids"] == 0) and np.all(r["gates"] == 1.0)


def pin_hand_worked_example(o):
    """A hand-computable case with integer weights and equal selected logits.

    d = 2, l = 2, N = 3, K = 2, m = 2, one token x = (1, 2).
    W_down = [[1, 0], [1, 1]]  -> z = (1, 3)
    W_router rows (1, 0), (1, 0), (0, 0) -> logits (1, 1, 0): experts 0 and 1
    tie at the top, each gets gate 1/2 exactly.
    Expert 0: W1 = [[1, 0], [0, -1]] -> h = (1, -3) -> a = (1, 0);
              W2 = [[2, 0], [0, 1]]  -> y0 = (2, 0)
    Expert 1: W1 = [[1, 1], [-1, 1]] -> h = (4, 2) -> a = (16, 4);
              W2 = [[1, 0], [1, 1]]  -> y1 = (16, 20)
    s = (2 + 16) / 2, (0 + 20) / 2 = (9, 10)
    W_up = [[1, 0], [0, 2]] -> W_up s = (9, 20); out = x + (9, 20) = (10, 22).
    """
    f = np.float32
    L = {
        "x": np.array([[1, 2]], f),
        "W_down": np.array([[1, 0], [1, 1]], f),
        "W_router": np.array([[1, 0], [1, 0], [0, 0]], f),
        "W1": np.array([[[1, 0], [0, -1]], [[1, 1], [-1, 1]], [[5, 5], [5, 5]]], f),
        "W2": np.array([[[2, 0], [0, 1]], [[1, 0], [1, 1]], [[5, 5], [5, 5]]], f),
        "W_up": np.array([[1, 0], [0, 2]], f),
        "bias": None,
    }
    r = run(o, L, 2)
    assert r["ids"].tolist() == [[0, 1]]
    assert r["gates"].tolist() == [[0.5, 0.5]]
    assert r["out"].tolist() == [[10.0, 22.0]], r["out"]


def pin_superposition(o):
    """out - x = sum_k g_k (out_k - x), where out_k is the layer with expert
    e_k alone (N = K = 1, gate 1).  Checks how the K expert outputs and the
    gates are combined."""
    T, d, l, N, K, m = 6, 24, 8, 7, 3, 8
    L = rand_layer(12, T, d, l, N, m)
    r = run(o, L, K)
    for t in range(T):
        acc = np.zeros(d)
        for k in range(K):
            e = r["ids"][t, k]
            Le = dict(L)
            Le["W_router"] = L["W_router"][e:e + 1]
            Le["W1"] = L["W1"][e:e + 1]
            Le["W2"] = L["W2"][e:e + 1]
            re = run(o, Le, 1, sel=[t])
            acc += r["gates"][t, k] * (re["out"][0] - f64(L["x"][t]))
        assert np.allclose(r["out"][t] - f64(L["x"][t]), acc, rtol=1e-12, atol=1e-13)


def pin_zero_weights_give_residual(o):
    for dtype in ("f32", "bf16"):
        L = rand_layer(13, 5, 32, 8, 6, 8, dtype=dtype, bias=True)
        for key in ("W2", "W_up"):
            Lz = dict(L)
            Lz[key] = np.zeros_like(L[key])
            r = run(o, Lz, 2)
            assert np.array_equal(r["out"], f64(L["x"])), f"{key} = 0 must give out == x"


def pin_homogeneity(o):
    L = rand_layer(14, 6, 32, 16, 8, 8)
    r = run(o, L, 3)
    base = r["out"] - f64(L["x"])
    for key, factor in (("W2", 2.0), ("W1", 4.0), ("W_up", 2.0)):
        Ls = dict(L)
        Ls[key] = (L[key] * np.float32(2.0)).astype(np.float32)
        rs = run(o, Ls, 3)
        assert np.array_equal(rs["ids"], r["ids"])
        part = rs["out"] - f64(L["x"])
        # exact up to the rounding of the residual add in double precision
        assert np.allclose(part, factor * base, rtol=0, atol=1e-14 * np.abs(part).max()), f"scaling {key} by 2"


def pin_symmetries(o):
    T, d, l, N, K, m = 10, 32, 8, 9, 3, 8
    L = rand_layer(15, T, d, l, N, m)
    r = run(o, L, K)
    perm = _rng(1).permutation(T)
    Lp = dict(L)
    Lp["x"] = L["x"][perm]
    rp = run(o, Lp, K)
    assert np.array_equal(rp["out"], r["out"][perm])
    relabel = _rng(2).permutation(N)
    Le = dict(L)
    Le["W_router"] = L["W_router"][relabel]
    Le["W1"] = L["W1"][relabel]
    Le["W2"] = L["W2"][relabel]
    re = run(o, Le, K)
    assert np.array_equal(relabel[re["ids"]], r["ids"])
    # equal up to the order of the softmax denominator's sum
    assert np.allclose(re["out"], r["out"], rtol=0, atol=1e-14 * np.abs(r["out"]).max())


def pin_selection_and_forced_ids(o):
    """Evaluating a subset of tokens gives the same rows; forcing a token's own
    ids changes nothing."""
    L = rand_layer(16, 9, 32, 8, 6, 8, bias=True)
    r = run(o, L, 2)
    sel = [7, 0, 4]
    rs = run(o, L, 2, sel=sel)
    assert np.array_equal(rs["out"], r["out"][sel])
    rf = run(o, L, 2, sel=sel, forced_ids=r["ids"][sel])
    assert np.array_equal(rf["out"], r["out"][sel])


def pin_forced_ids_reroute(o):
    """Forcing other ids routes the token to them: the gates are the
    softmax of the token's own logits renormalised over the forced set, in
    the forced order, and the output uses the forced experts; compared with
    a numpy float64 evaluation of the forced routing."""
    T, d, l, N, K, m = 6, 32, 8, 9, 3, 8
    L = rand_layer(17, T, d, l, N, m, bias=True)
    r = run(o, L, K)
    rng = _rng(18)
    forced = np.empty((T, K), np.int32)
    for t in range(T):
        own = set(r["ids"][t].tolist())
        # K distinct ids, at least one the token would not pick, in a
        # scrambled order
        outside = int(rng.choice([e for e in range(N) if e not in own]))
        rest = rng.choice([e for e in range(N) if e != outside], size=K - 1, replace=False)
        forced[t] = rng.permutation(np.concatenate([[outside], rest])).astype(np.int32)
        assert set(forced[t].tolist()) != own
    sel = np.arange(T, dtype=np.int32)
    rf = run(o, L, K, sel=sel, forced_ids=forced)
    assert np.array_equal(rf["ids"], forced), "the forced ids are the ones reported"
    x = f64(L["x"])
    z = x @ f64(L["W_down"]).T
    lg = np_logits(L)
    for t in range(T):
        S = forced[t]
        g = softmax(lg[t, S])
        assert np.allclose(rf["gates"][t], g, rtol=1e-12, atol=0), "gates: softmax over the forced set"
        s = np.zeros(l)
        for k in range(K):
            e = S[k]
            y = (np.maximum(z[t] @ f64(L["W1"][e]).T, 0.0) ** 2) @ f64(L["W2"][e]).T
            s += g[k] * y
        want = x[t] + s @ f64(L["W_up"]).T
        assert np.allclose(rf["out"][t], want, rtol=1e-12, atol=1e-13), "output with the forced experts"
        # the gap still describes the token's own selection
        assert rf["gap"][t] == r["gap"][t]


def pin_shared_expert(o):
    """The shared expert at full d: a dense FFN on x added to the layer."""
    for standard in (False, True):
        d = 24
        l = d if standard else 8
        L = add_shared(rand_layer(31, T=7, d=d, l=l, N=6, m=10, standard=standard), 32, ms=12)
        K = 3
        # routed experts silenced: out = x + shared(x), nothing else
        L0 = dict(L)
        L0["W2"] = np.zeros_like(L["W2"])
        r0 = run(o, L0, K)
        assert np.allclose(r0["out"], f64(L["x"]) + np_shared(L), rtol=1e-12, atol=1e-12), \
            "layer with silenced experts != x + W_s2 relu(W_s1 x)^2"
        # routed experts on: the shared expert adds exactly its FFN
        with_s = run(o, L, K)["out"]
        Ln = dict(L)
        Ln["W_s1"] = Ln["W_s2"] = None
        without = run(o, Ln, K)["out"]
        assert np.allclose(with_s - without, np_shared(L), rtol=1e-10, atol=1e-12), \
            "the shared expert does not add its own FFN output"
        # W_s2 = 0: the layer without a shared expert, bit-exactly
        Lz = dict(L)
        Lz["W_s2"] = np.zeros_like(L["W_s2"])
        assert np.array_equal(run(o, Lz, K)["out"], without), "W_s2 = 0 changed the output"


def fp8_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 codes -> float64 through torch's float8_e4m3fn (not the oracle's decoder)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def fp8_layer(seed, T, d, l, N, m, pow2_scales):
    """A float32 layer whose expert weights are E4M3 codes with row scales.
    Codes cycle through every non-NaN code."""
    r = _rng(seed)
    L = rand_layer(seed, T, d, l, N, m)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    L["W1"] = np.resize(r.permutation(codes), N * m * l).reshape(N, m, l)
    L["W2"] = np.resize(r.permutation(codes), N * l * m).reshape(N, l, m)
    if pow2_scales:
        L["W1_scale"] = np.ldexp(1.0, r.integers(-12, -6, N * m)).astype(np.float32)
        L["W2_scale"] = np.ldexp(1.0, r.integers(-12, -6, N * l)).astype(np.float32)
    else:
        L["W1_scale"] = (r.random(N * m) * 1e-3 + 1e-4).astype(np.float32)
        L["W2_scale"] = (r.random(N * l) * 1e-3 + 1e-4).astype(np.float32)
    return L


def run_fp8(o, L, K, **kw):
    return o.forward(L["x"], L["W_down"], L["W_router"], L["W1"], L["W2"], L["W_up"], K,
                     bias=L.get("bias"), W1_scale=L["W1_scale"], W2_scale=L["W2_scale"], **kw)


def pin_fp8_experts(o):
    """FP8 expert weights: decoded by an independent decoder, scaled per row."""
    # power-of-two scales: code * scale is exact in float32, so the FP8 layer
    # is the float32 layer on the decoded weights, bit for bit
    T, d, l, N, m, K = 6, 16, 8, 4, 64, 2
    L = fp8_layer(41, T, d, l, N, m, pow2_scales=True)
    ref = dict(L)
    ref["W1"] = (fp8_decode(L["W1"]) * L["W1_scale"].astype(np.float64).reshape(N, m, 1)).astype(np.float32)
    ref["W2"] = (fp8_decode(L["W2"]) * L["W2_scale"].astype(np.float64).reshape(N, l, 1)).astype(np.float32)
    assert np.array_equal(ref["W1"].astype(np.float64), fp8_decode(L["W1"]) * L["W1_scale"].reshape(N, m, 1))
    a = run_fp8(o, L, K)
    b = run(o, ref, K)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["ids"], b["ids"]), \
        "FP8 layer != float32 layer on the decoded weights"
    # arbitrary row scales, one expert: a dense FFN evaluated with numpy
    L = fp8_layer(42, T, d, l, 1, m, pow2_scales=False)
    w1 = fp8_decode(L["W1"])[0] * L["W1_scale"].astype(np.float64)[:, None]
    w2 = fp8_decode(L["W2"])[0] * L["W2_scale"].astype(np.float64)[:, None]
    x = f64(L["x"])
    z = x @ f64(L["W_down"]).T
    s = (np.maximum(z @ w1.T, 0.0) ** 2) @ w2.T
    want = x + s @ f64(L["W_up"]).T
    got = run_fp8(o, L, 1)["out"]
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12), "FP8 dense special case differs from numpy"


# the eight E2M1 magnitudes of the OCP Microscaling spec, by code & 7
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def mx_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 -> float64: codes [..., rows, cols/2] (even element in the low
    nibble), scales [..., rows, cols/32] E8M0 bytes."""
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(*codes.shape[:-1], 2 * codes.shape[-1])
    val = np.where(nib & 8, -1.0, 1.0) * E2M1_VALUES[nib & 7]
    return val * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)


def mx_layer(seed, T, d, l, N, m):
    """A float32 layer whose expert weights are MXFP4: every byte value as
    codes, block scales 2^-11 .. 2^-4 varying per block."""
    r = _rng(seed)
    L = rand_layer(seed, T, d, l, N, m)
    L["W1"] = np.resize(r.permutation(256).astype(np.uint8), N * m * l // 2).reshape(N, m, l // 2)
    L["W2"] = np.resize(r.permutation(256).astype(np.uint8), N * l * m // 2).reshape(N, l, m // 2)
    L["W1_scale"] = r.integers(116, 124, (N, m, l // 32)).astype(np.uint8)
    L["W2_scale"] = r.integers(116, 124, (N, l, m // 32)).astype(np.uint8)
    return L


def pin_mxfp4_experts(o):
    """MXFP4 expert weights, decoded independently."""
    T, d, l, N, m, K = 6, 16, 64, 4, 64, 2
    L = mx_layer(61, T, d, l, N, m)
    ref = dict(L)
    ref["W1"] = mx_decode(L["W1"], L["W1_scale"]).astype(np.float32)
    ref["W2"] = mx_decode(L["W2"], L["W2_scale"]).astype(np.float32)
    assert np.array_equal(ref["W1"].astype(np.float64), mx_decode(L["W1"], L["W1_scale"]))
    a = run_fp8(o, L, K)
    b = run(o, ref, K)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["ids"], b["ids"]), \
        "MXFP4 layer != float32 layer on the decoded weights"
    L = mx_layer(62, T, d, l, 1, m)
    w1 = mx_decode(L["W1"], L["W1_scale"])[0]
    w2 = mx_decode(L["W2"], L["W2_scale"])[0]
    x = f64(L["x"])
    s = (np.maximum((x @ f64(L["W_down"]).T) @ w1.T, 0.0) ** 2) @ w2.T
    want = x + s @ f64(L["W_up"]).T
    assert np.allclose(run_fp8(o, L, 1)["out"], want, rtol=1e-12, atol=1e-12), "MXFP4 dense case differs from numpy"


def zc_layer(seed, T, d, l, N, m, nz, nc, nk, *, standard=False):
    """A float32 layer with N FFN experts followed by nz zero, nc copy and nk
    constant experts (router rows for all of them)."""
    Nr = N + nz + nc + nk
    L = rand_layer(seed, T, d, l, Nr, m, standard=standard)
    L["W1"] = np.ascontiguousarray(L["W1"][:N])
    L["W2"] = np.ascontiguousarray(L["W2"][:N])
    L["zc_const"] = _rng(seed + 1000).standard_normal((nk, l)).astype(np.float32) if nk else None
    L["n_zero"], L["n_copy"] = nz, nc
    return L


def run_zc(o, L, K, **kw):
    return run(o, L, K, n_zero=L["n_zero"], n_copy=L["n_copy"], zc_const=L["zc_const"], **kw)


def np_dense_mask(L, K):
    """The layer with zero-computation experts, evaluated densely in numpy."""
    x = f64(L["x"])
    N, nz, nc = L["W1"].shape[0], L["n_zero"], L["n_copy"]
    standard = L["W_down"] is None
    z = x if standard else x @ f64(L["W_down"]).T
    lg = np_logits(L)
    T, Nr = lg.shape
    G = np.zeros((T, Nr))
    for t in range(T):
        top = sorted(range(Nr), key=lambda e: (-lg[t, e], e))[:K]
        p = softmax(lg[t])
        G[t, top] = p[top] / p[top].sum()
    Y = np.zeros((T, Nr, z.shape[1]))
    for e in range(N):
        Y[:, e] = (np.maximum(z @ f64(L["W1"][e]).T, 0.0) ** 2) @ f64(L["W2"][e]).T
    for q in range(nc):
        Y[:, N + nz + q] = z
    if L["zc_const"] is not None:
        for q in range(L["zc_const"].shape[0]):
            Y[:, N + nz + nc + q] = f64(L["zc_const"][q])
    s = np.einsum("te,tel->tl", G, Y)
    return x + (s if standard else s @ f64(L["W_up"]).T), G


def pin_zero_computation_experts(o):
    """Zero, copy and constant experts among the routed ids."""
    # dense mask, latent and standard mode, every kind present
    for standard in (False, True):
        L = zc_layer(51, T=9, d=16, l=16 if standard else 8, N=5, m=12, nz=2, nc=2, nk=3, standard=standard)
        for K in (3, 6):
            got = run_zc(o, L, K)
            want, G = np_dense_mask(L, K)
            for t in range(L["x"].shape[0]):
                assert set(got["ids"][t].tolist()) == set(np.nonzero(G[t])[0].tolist()), "selection"
            assert np.allclose(got["out"], want, rtol=1e-11, atol=1e-12), "dense-mask evaluation differs"
    # K = 1 with one routed id made to win by its bias: closed forms
    T, d, l, N, m = 7, 16, 8, 4, 12

    def winner(L, e):
        Nr = L["W_router"].shape[0]
        L["bias"] = np.full(Nr, -40.0, np.float32)
        L["bias"][e] = 40.0
        return L

    L = winner(zc_layer(52, T, d, l, N, m, 1, 1, 2), N)              # the zero expert
    got = run_zc(o, L, 1)
    x64 = f64(L["x"])
    assert np.array_equal(got["ids"][:, 0], np.full(T, N)) and np.array_equal(got["out"], x64), "zero expert"
    L = winner(zc_layer(52, T, d, l, N, m, 1, 1, 2), N + 1)          # the copy expert
    want = x64 + (x64 @ f64(L["W_down"]).T) @ f64(L["W_up"]).T
    assert np.allclose(run_zc(o, L, 1)["out"], want, rtol=1e-12, atol=1e-13), "copy expert"
    L = winner(zc_layer(52, T, d, l, N, m, 1, 1, 2), N + 3)          # the second constant expert
    want = x64 + np.outer(np.ones(T), f64(L["zc_const"][1]) @ f64(L["W_up"]).T)
    assert np.allclose(run_zc(o, L, 1)["out"], want, rtol=1e-12, atol=1e-13), "constant expert"
    L = winner(zc_layer(53, T, d, d, N, m, 1, 1, 0, standard=True), N + 1)   # copy, standard mode
    assert np.array_equal(run_zc(o, L, 1)["out"], 2.0 * f64(L["x"])), "standard-mode copy expert"
    # zero-computation experts that never win change nothing
    L = zc_layer(54, T, d, l, N, m, 2, 1, 1)
    L["bias"] = np.zeros(N + 4, np.float32)
    L["bias"][N:] = -1e30
    plain = dict(L, W_router=np.ascontiguousarray(L["W_router"][:N]), bias=L["bias"][:N].copy())
    a, b = run_zc(o, L, 3), run(o, plain, 3)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["ids"], b["ids"]), "losing experts changed out"


ALL_PINS = [
    pin_routing_bruteforce,
    pin_tie_break,
    pin_gates,
    pin_identity_reduces_to_standard,
    pin_dense_ffn_special_case,
    pin_hand_worked_example,
    pin_superposition,
    pin_zero_weights_give_residual,
    pin_homogeneity,
    pin_symmetries,
    pin_selection_and_forced_ids,
    pin_forced_ids_reroute,
    pin_shared_expert,
    pin_fp8_experts,
    pin_zero_computation_experts,
    pin_mxfp4_experts,
]
