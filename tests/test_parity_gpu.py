"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Every named workload at full size, every token: tiny float32, decode and
standard-MoE decode in one oracle call each; the prefill, standard-MoE
prefill and skewed workloads run once on the GPU in the launch configuration
the benchmark times and are compared chunk by chunk.  The extension
workloads at prefill size (shared expert, FP8, MXFP4, zero-computation
experts) are compared on sampled tokens plus the ragged tail.  Smaller
shapes cover several tiles, ragged tails and the edge cases.
"""
import numpy as np
import pytest
import torch

from sparse_moe_layer_gemm_amd import binding as B
from sparse_moe_layer_gemm_amd.inputs import WORKLOADS, Workload, make_inputs
from tests import parity as P

pytestmark = pytest.mark.gpu

S, TL = B.LMOE_PATH_STREAM, B.LMOE_PATH_TILED


def sample_tokens(T, n, seed=0):
    rng = np.random.default_rng(seed)
    picks = rng.choice(T, size=min(n, T), replace=False)
    tail = np.arange(max(0, T - 5), T)
    return np.unique(np.concatenate([picks, tail, [0]])).astype(np.int32)


# --- full-size workloads -------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_f32(seed):
    w = WORKLOADS["tiny_f32"]
    P.compare(w, P.gen(w, seed), w.K)


@pytest.fixture(scope="module")
def decode_inputs():
    w = WORKLOADS["decode"]
    return w, P.gen(w, 0)


@pytest.mark.parametrize("path", [B.LMOE_PATH_AUTO, TL])
def test_decode(decode_inputs, path):
    w, inp = decode_inputs
    P.compare(w, inp, w.K, path=path)


def test_decode_seed1():
    w = WORKLOADS["decode"]
    P.compare(w, P.gen(w, 1), w.K)


@pytest.mark.parametrize("path", [B.LMOE_PATH_AUTO, TL])
def test_standard_decode(path):
    w = WORKLOADS["standard_decode"]
    P.compare(w, P.gen(w, 0), w.K, path=path)


# Every token of the full-size prefill-shaped workloads: one GPU forward per
# workload, in the launch configuration the benchmark times, then the oracle
# on all T tokens in chunks, one test per chunk (each well under a minute on
# the host's cores).  The dispatch arrays are checked in full once.
FULL_CHUNKS = {"prefill": 8, "standard_prefill": 8, "skewed": 4}


@pytest.fixture(scope="module")
def full_run():
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()   # one workload at a time: its weights take GBs of host memory
            w = WORKLOADS[name]
            inp = P.gen(w, 0)
            g = P.GpuRun(w, inp, w.K)
            g.check_dispatch()
            cache[name] = (w, inp, P.oracle_arrays(inp), g)
        return cache[name]

    return get


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,chunk", [(n, c) for n, k in FULL_CHUNKS.items() for c in range(k)])
def test_full_size_every_token(full_run, name, chunk):
    w, inp, arr, g = full_run(name)
    n = FULL_CHUNKS[name]
    sel = np.arange(chunk * w.T // n, (chunk + 1) * w.T // n, dtype=np.int32)
    P.check_tokens(g, inp, sel, arr=arr, tag=f"{name}[{chunk + 1}/{n}]")
    if name == "skewed" and chunk == 0:
        counts = np.bincount(g.ids.reshape(-1), minlength=w.N)
        P.log(f"[skew] max rows/expert {counts.max()}, empty experts {(counts == 0).sum()}")
        assert counts.max() > 10 * w.T * w.K / w.N and (counts == 0).sum() > 0


# --- batch sweep: the decode-shaped layers at T = 1 ... 256 tokens ------------
# (x = the first T rows of one draw; the path and kernels change with T: the
# split skinny projection up to 64 tokens, the tiled projection above)

SWEEP_T = [1, 2, 4, 8, 16, 64, 128, 192, 256]


@pytest.fixture(scope="module")
def sweep_decode():
    w = WORKLOADS["decode"].replace(T=max(SWEEP_T))
    return w, make_inputs(w, 7)


@pytest.mark.parametrize("T", SWEEP_T)
def test_decode_batch_sweep(sweep_decode, T):
    w0, inp = sweep_decode
    w = w0.replace(name=f"decode_T{T}", T=T)
    P.compare(w, {**inp, "x": inp["x"][:T]}, w.K, tag=f"decode_T{T}")


@pytest.mark.parametrize("T", [1, 8, 64, 256])
def test_standard_decode_batch_sweep(T):
    w = WORKLOADS["standard_decode"].replace(name=f"standard_decode_T{T}", T=T)
    P.compare(w, make_inputs(w, 8), w.K, tag=f"standard_decode_T{T}")


# FP8 and MXFP4 experts across the batch sizes where the decode FFN's m-slice
# changes: 256 wide at T = 8 (the workgroups fill one round of the GPU), 128
# wide at T = 16, 256 wide at T = 64 and 128 (one draw per format, x = its
# first T rows)
@pytest.fixture(scope="module", params=["fp8", "mxfp4"])
def sweep_low_precision(request):
    w = WORKLOADS[f"decode_{request.param}"].replace(T=128)
    return w, make_inputs(w, 9)


@pytest.mark.parametrize("T", [8, 16, 64, 128])
def test_low_precision_decode_batch_sweep(sweep_low_precision, T):
    w0, inp = sweep_low_precision
    w = w0.replace(name=f"{w0.name}_T{T}", T=T)
    P.compare(w, {**inp, "x": inp["x"][:T]}, w.K, tag=f"{w0.name}_T{T}")


# 256-wide m-slices on shapes the named workloads do not reach: one slice per
# expert (m = 256) in every weight format, and two slices of MXFP4 experts
# (m = 512: the slice pairing across XCDs).  1280 experts, top-32 of 160
# tokens: ~1257 active experts expected, ~4 rows each.
WIDE = [Workload(f"wide_one_{e}", T=160, d=256, l=256, N=1280, K=32, m=256, dtype="bf16", experts=e)
        for e in ("dense", "fp8", "mxfp4")]
WIDE.append(Workload("wide_paired_mxfp4", T=160, d=256, l=256, N=1280, K=32, m=512, dtype="bf16", experts="mxfp4"))


@pytest.mark.parametrize("w", WIDE, ids=lambda w: w.name)
def test_wide_slice_shapes(w):
    P.compare(w, make_inputs(w, 12), w.K, tag=w.name)


# Seeded random shapes across the options (sizes, formats, shared expert,
# zero-computation experts, bias, standard mode, both paths), drawn once
# at import, to reach combinations the named cases do not.
def _random_shapes(n, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        standard = rng.random() < 0.25
        d = int(rng.choice([128, 192, 256, 384, 512]))
        l = d if standard else int(rng.choice([x for x in (64, 128, 192, 256) if x <= d]))
        m = int(rng.choice([64, 128, 192, 256, 320, 512]))
        experts = str(rng.choice(["dense", "dense", "fp8", "mxfp4"]))
        dtype = "bf16" if experts != "dense" or rng.random() < 0.8 else "f32"
        N = int(rng.integers(4, 600))
        nz = [int(x) for x in rng.integers(0, 3, size=3)] if rng.random() < 0.3 else [0, 0, 0]
        K = int(rng.integers(1, min(32, N + sum(nz)) + 1))
        T = int(rng.choice([1, 3, 17, 64, 129, 300, 777]))
        m_s = int(rng.choice([0, 0, 64, 128]))
        bias = bool(rng.random() < 0.3)
        out.append(Workload(f"rand{seed}_{i}", T=T, d=d, l=l, N=N, K=K, m=m, dtype=dtype, standard=standard,
                            bias=bias, m_shared=m_s, experts=experts, n_zero=nz[0], n_copy=nz[1], n_const=nz[2]))
    return out


RANDOM_SHAPES = _random_shapes(12) + _random_shapes(12, seed=7)


@pytest.mark.parametrize("w", RANDOM_SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("path", [B.LMOE_PATH_AUTO, S, TL])
def test_random_shapes(w, path):
    if w.dtype == "f32" and path == S:
        pytest.skip("the streaming FFN is bf16 only")
    P.log(f"[rand] {w}")
    P.compare(w, make_inputs(w, 13), w.K, path=path, tag=f"{w.name}/path{path}")


# --- the shared expert at full d ---------------------------------------------

@pytest.mark.parametrize("path", [B.LMOE_PATH_AUTO, TL])
def test_decode_shared(path):
    w = WORKLOADS["decode_shared"]
    P.compare(w, P.gen(w, 0), w.K, path=path, tag=f"decode_shared/path{path}")


def test_prefill_shared_sampled():
    w = WORKLOADS["prefill_shared"]
    P.compare(w, P.gen(w, 0), w.K, sample=sample_tokens(w.T, 96))


@pytest.mark.parametrize("w", [
    Workload("shared_latent", T=300, d=256, l=64, N=16, K=4, m=128, dtype="bf16", m_shared=192),
    Workload("shared_latent_f32", T=70, d=128, l=64, N=8, K=2, m=64, dtype="f32", m_shared=64),
    Workload("shared_standard", T=90, d=256, l=256, N=12, K=2, m=128, dtype="bf16", standard=True, m_shared=128),
    Workload("shared_standard_f32", T=45, d=128, l=128, N=9, K=3, m=64, dtype="f32", standard=True,
             m_shared=128),
    Workload("shared_one_token", T=1, d=256, l=64, N=16, K=3, m=128, dtype="bf16", m_shared=64),
], ids=lambda w: w.name)
@pytest.mark.parametrize("path", [B.LMOE_PATH_AUTO, S, TL])
def test_shared_expert_shapes(w, path):
    if w.dtype == "f32" and path == S:
        pytest.skip("the streaming FFN is bf16 only")
    P.compare(w, make_inputs(w, 9), w.K, path=path, tag=f"{w.name}/path{path}")


@pytest.mark.parametrize("path", [S, TL])
def test_shared_expert_with_zero_w2_is_the_plain_layer(path):
    """W_s2 = 0: bit-identical to the layer without a shared expert."""
    w = Workload("shared_zero", T=100, d=256, l=64, N=16, K=4, m=128, dtype="bf16", m_shared=128)
    inp = P.to_device(make_inputs(w, 10))
    plain = {k: v for k, v in inp.items() if k not in ("W_s1", "W_s2")}
    inp["W_s2"] = torch.zeros_like(inp["W_s2"])
    a = B.forward(inp, w.K, path=path)
    b = B.forward(plain, w.K, path=path)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# --- FP8 E4M3 routed-expert weights with per-row scales -----------------------

@pytest.mark.parametrize("path", [B.LMOE_PATH_AUTO, TL])
def test_decode_fp8(path):
    w = WORKLOADS["decode_fp8"]
    P.compare(w, P.gen(w, 0), w.K, path=path, tag=f"decode_fp8/path{path}")


def test_prefill_fp8_sampled():
    w = WORKLOADS["prefill_fp8"]
    P.compare(w, P.gen(w, 0), w.K, sample=sample_tokens(w.T, 96))


FP8_SHAPES = [
    Workload("fp8_latent", T=300, d=256, l=64, N=16, K=4, m=128, dtype="bf16", experts="fp8"),
    Workload("fp8_m192", T=37, d=512, l=256, N=64, K=8, m=192, dtype="bf16", experts="fp8"),
    Workload("fp8_large_tiles", T=2048, d=256, l=128, N=16, K=4, m=320, dtype="bf16", experts="fp8"),
    Workload("fp8_standard", T=90, d=256, l=256, N=12, K=2, m=128, dtype="bf16", standard=True, experts="fp8"),
    Workload("fp8_shared", T=100, d=256, l=64, N=16, K=4, m=128, dtype="bf16", m_shared=128, experts="fp8"),
    Workload("fp8_one_token", T=1, d=256, l=64, N=16, K=3, m=128, dtype="bf16", experts="fp8"),
]


@pytest.mark.parametrize("w", FP8_SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("path", [B.LMOE_PATH_AUTO, S, TL])
def test_fp8_shapes(w, path):
    P.compare(w, make_inputs(w, 11), w.K, path=path, tag=f"{w.name}/path{path}")


def every_code_inputs(w: Workload, seed: int):
    """FP8 inputs whose codes run through every non-NaN E4M3 code (so every
    decode the kernels do is exercised) with power-of-two row scales."""
    inp = make_inputs(w, seed)
    g = torch.Generator().manual_seed(seed + 1)
    codes = torch.tensor([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=torch.uint8)
    for name, rows in (("W1", w.m), ("W2", w.l)):
        n = inp[name].numel()
        perm = codes[torch.randperm(codes.numel(), generator=g)]
        inp[name] = perm.repeat(n // perm.numel() + 1)[:n].reshape(inp[name].shape).contiguous()
        # codes reach 448: scales 2^-14 .. 2^-10 keep the weights below 0.5
        inp[name + "_scale"] = torch.ldexp(torch.ones(w.N, rows),
                                           torch.randint(-14, -9, (w.N, rows), generator=g).float())
    return inp


@pytest.mark.parametrize("path", [S, TL])
def test_fp8_every_code(path):
    w = Workload("fp8_every_code", T=120, d=256, l=128, N=16, K=4, m=128, dtype="bf16", experts="fp8")
    P.compare(w, every_code_inputs(w, 12), w.K, path=path, tag=f"fp8_every_code/path{path}")


@pytest.mark.parametrize("path", [S, TL])
def test_fp8_layer_is_the_bf16_layer_on_decoded_weights(path):
    """With power-of-two row scales every decoded weight code * scale is a
    bfloat16 value and scaling a float32 dot product by the scale is exact,
    so the FP8 layer equals, bit for bit, the bf16 layer on those weights
    (with as many active experts as here both take the same m-slices on the
    streaming path, whose per-slice partials are rounded to fp16)."""
    w = Workload("fp8_pow2", T=120, d=256, l=128, N=128, K=4, m=256, dtype="bf16", experts="fp8")
    inp = every_code_inputs(w, 13)
    dense = dict(inp)
    for name in ("W1", "W2"):
        dec = inp[name].view(torch.float8_e4m3fn).float() * dense.pop(name + "_scale").unsqueeze(-1)
        dense[name] = dec.to(torch.bfloat16)
        assert torch.equal(dense[name].float(), dec)
    a = B.forward(P.to_device(inp), w.K, path=path)
    b = B.forward(P.to_device(dense), w.K, path=path)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# --- MXFP4 routed-expert weights (E2M1 codes, E8M0 scales per 32) -------------

@pytest.mark.parametrize("path", [B.LMOE_PATH_AUTO, TL])
def test_decode_mxfp4(path):
    w = WORKLOADS["decode_mxfp4"]
    P.compare(w, P.gen(w, 0), w.K, path=path, tag=f"decode_mxfp4/path{path}")


def test_prefill_mxfp4_sampled():
    w = WORKLOADS["prefill_mxfp4"]
    P.compare(w, P.gen(w, 0), w.K, sample=sample_tokens(w.T, 96))


@pytest.mark.parametrize("w", [x.replace(name=x.name.replace("fp8", "mxfp4"), experts="mxfp4") for x in FP8_SHAPES],
                         ids=lambda w: w.name)
@pytest.mark.parametrize("path", [B.LMOE_PATH_AUTO, S, TL])
def test_mxfp4_shapes(w, path):
    P.compare(w, make_inputs(w, 18), w.K, path=path, tag=f"{w.name}/path{path}")


def every_byte_mxfp4(w: Workload, seed: int):
    """MXFP4 inputs whose code bytes run through all 256 values, with block
    scales 2^-11 .. 2^-4 that differ from block to block."""
    inp = make_inputs(w, seed)
    g = torch.Generator().manual_seed(seed + 1)
    for name in ("W1", "W2"):
        n = inp[name].numel()
        perm = torch.randperm(256, generator=g).to(torch.uint8)
        inp[name] = perm.repeat(n // 256 + 1)[:n].reshape(inp[name].shape).contiguous()
        sc = inp[name + "_scale"]
        inp[name + "_scale"] = torch.randint(116, 124, sc.shape, generator=g).to(torch.uint8)
    return inp


# l = 128: the streaming FFN shared with bf16 and FP8 (8-byte code loads, a
# scale byte per block); l = 256, m = 256: the MXFP4 streaming kernel with
# 16-byte code loads.  At l = 128, 160 experts keep enough of them active that
# a bf16 layer of this shape also streams 128-wide m-slices, so both store the
# same fp16 partial planes.
MX_POW2 = [Workload("mxfp4_l128", T=120, d=256, l=128, N=160, K=4, m=128, dtype="bf16", experts="mxfp4"),
           Workload("mxfp4_l256", T=60, d=256, l=256, N=16, K=4, m=256, dtype="bf16", experts="mxfp4")]


@pytest.mark.parametrize("w", MX_POW2, ids=lambda w: w.name)
@pytest.mark.parametrize("path", [S, TL])
def test_mxfp4_every_byte(w, path):
    P.compare(w, every_byte_mxfp4(w, 19), w.K, path=path, tag=f"{w.name}_every_byte/path{path}")


@pytest.mark.parametrize("w", MX_POW2, ids=lambda w: w.name)
@pytest.mark.parametrize("path", [S, TL])
def test_mxfp4_scale_byte_zero(w, path):
    """E8M0 scale byte 0 (2^-127): the kernels decode such a block to 0, the
    oracle to its exact value; each product term differs by at most
    6 * 2^-127, far below anything the fp32 sums keep, so the two agree
    within the usual bar.  A quarter of the blocks, and every block of
    expert 0's W1, get byte 0."""
    inp = make_inputs(w, 21)
    g = torch.Generator().manual_seed(22)
    for name in ("W1_scale", "W2_scale"):
        sc = inp[name].clone()
        sc[torch.rand(sc.shape, generator=g) < 0.25] = 0
        inp[name] = sc.contiguous()
    inp["W1_scale"][0] = 0
    P.compare(w, inp, w.K, path=path, tag=f"{w.name}_scale_byte_zero/path{path}")


@pytest.mark.parametrize("w", MX_POW2, ids=lambda w: w.name)
@pytest.mark.parametrize("path", [S, TL])
def test_mxfp4_layer_is_the_bf16_layer_on_decoded_weights(w, path):
    """Every E2M1 value times a power-of-two block scale is a bfloat16 value,
    so where the MXFP4 kernels group the dot products' terms as the bf16
    ones do (the tiled FFN, and the streaming FFN shared with bf16), the
    MXFP4 layer equals the bf16 layer on the decoded weights bit for bit.
    The MXFP4 streaming kernel with 16-byte code loads groups them its own
    way: there the two agree to fp32 rounding (and both match the oracle)."""
    from sparse_moe_layer_gemm_amd.inputs import decode_mxfp4

    inp = every_byte_mxfp4(w, 20)
    dense = dict(inp)
    for name in ("W1", "W2"):
        dec = decode_mxfp4(inp[name], dense.pop(name + "_scale"))
        dense[name] = dec.to(torch.bfloat16).contiguous()
        assert torch.equal(dense[name].float(), dec)
    a = B.forward(P.to_device(inp), w.K, path=path)
    b = B.forward(P.to_device(dense), w.K, path=path)
    torch.cuda.synchronize()
    if path == S and w.l % 256 == 0:
        moe = (b.float() - P.to_device(inp)["x"].float())
        err = (a.float() - b.float()).abs().max().item()
        assert err <= 1e-2 * moe.pow(2).mean().sqrt().item() + 2 ** -7 * b.float().abs().max().item(), err
    else:
        assert torch.equal(a, b)


# --- zero-computation experts (zero, copy, constant) --------------------------

def zc_forward(w, inp, path, **kw):
    return B.forward(inp, w.K, path=path, n_zero=w.n_zero, n_copy=w.n_copy, **kw)


@pytest.mark.parametrize("path", [B.LMOE_PATH_AUTO, TL])
def test_decode_zc(path):
    w = WORKLOADS["decode_zc"]
    P.compare(w, P.gen(w, 0), w.K, path=path, tag=f"decode_zc/path{path}")


def test_prefill_zc_sampled():
    w = WORKLOADS["prefill_zc"]
    P.compare(w, P.gen(w, 0), w.K, sample=sample_tokens(w.T, 96))


ZC_SHAPES = [
    Workload("zc_latent", T=300, d=256, l=64, N=16, K=4, m=128, dtype="bf16", n_zero=4, n_copy=2, n_const=2),
    Workload("zc_standard", T=90, d=256, l=256, N=12, K=3, m=128, dtype="bf16", standard=True,
             n_zero=2, n_copy=2, n_const=2),
    Workload("zc_f32", T=70, d=128, l=64, N=8, K=3, m=64, dtype="f32", n_zero=1, n_copy=1, n_const=1),
    Workload("zc_every_id", T=20, d=256, l=64, N=6, K=10, m=64, dtype="bf16", n_zero=2, n_copy=1, n_const=1),
    Workload("zc_zero_only", T=200, d=256, l=64, N=16, K=6, m=128, dtype="bf16", n_zero=16),
    Workload("zc_one_token", T=1, d=256, l=64, N=16, K=5, m=128, dtype="bf16", n_zero=2, n_copy=2, n_const=2),
    Workload("zc_fp8_shared_bias", T=150, d=256, l=64, N=16, K=4, m=128, dtype="bf16", bias=True, m_shared=64,
             experts="fp8", n_zero=3, n_copy=3, n_const=3),
]


@pytest.mark.parametrize("w", ZC_SHAPES, ids=lambda w: w.name)
@pytest.mark.parametrize("path", [B.LMOE_PATH_AUTO, S, TL])
def test_zc_shapes(w, path):
    if w.dtype == "f32" and path == S:
        pytest.skip("the streaming FFN is bf16 only")
    P.compare(w, make_inputs(w, 14), w.K, path=path, tag=f"{w.name}/path{path}")


def one_winner(w, e, seed):
    """Inputs of w (K = 1) whose router bias makes routed id e win for every token."""
    inp = make_inputs(w.replace(bias=True), seed)
    bias = torch.full_like(inp["bias"], -40.0)
    bias[e] = 40.0
    inp["bias"] = bias
    return P.to_device(inp)


@pytest.mark.parametrize("path", [S, TL])
@pytest.mark.parametrize("standard", [False, True])
def test_zero_expert_gives_x(path, standard):
    w = Workload("zc_k1", T=80, d=256, l=256 if standard else 64, N=16, K=1, m=128, dtype="bf16",
                 standard=standard, n_zero=2, n_copy=2, n_const=2)
    inp = one_winner(w, w.N + 1, 15)
    out, ids, gates, _ = zc_forward(w, inp, path, routing=True)
    torch.cuda.synchronize()
    assert torch.all(ids == w.N + 1) and torch.all(gates == 1.0)
    assert torch.equal(out, inp["x"])


@pytest.mark.parametrize("path", [S, TL])
def test_standard_copy_and_constant_experts(path):
    """Standard mode, K = 1: a copy expert gives 2x, constant expert q gives
    x + c_q, each rounded once."""
    w = Workload("zc_k1_std", T=80, d=256, l=256, N=16, K=1, m=128, dtype="bf16", standard=True,
                 n_zero=1, n_copy=1, n_const=3)
    inp = one_winner(w, w.N + 1, 16)
    out = zc_forward(w, inp, path)
    torch.cuda.synchronize()
    assert torch.equal(out, (2.0 * inp["x"].float()).to(torch.bfloat16))
    inp = one_winner(w, w.N + 3, 16)
    out = zc_forward(w, inp, path)
    torch.cuda.synchronize()
    want = (inp["x"].float() + inp["zc_const"][1].float()).to(torch.bfloat16)
    assert torch.equal(out, want)


def test_losing_zc_experts_change_nothing():
    """Zero-computation experts whose logits never win: bit-identical to the
    layer without them (gates depend only on the kept logits)."""
    w = Workload("zc_lose", T=200, d=256, l=64, N=16, K=4, m=128, dtype="bf16", bias=True,
                 n_zero=2, n_copy=2, n_const=2)
    inp = make_inputs(w, 17)
    inp["bias"][w.N:] = -1e30
    plain = {k: v for k, v in inp.items() if k != "zc_const"}
    plain["W_router"] = inp["W_router"][:w.N].contiguous()
    plain["bias"] = inp["bias"][:w.N].contiguous()
    a = zc_forward(w, P.to_device(inp), TL)
    b = B.forward(P.to_device(plain), w.K, path=TL)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# --- smaller shapes: several tiles, ragged tails, both FFN paths --------------

SMALL_PREFILL = Workload("small_prefill", T=1000, d=512, l=128, N=64, K=6, m=256, dtype="bf16")
SMALL_DECODE = Workload("small_decode_m192", T=37, d=512, l=256, N=64, K=8, m=192, dtype="bf16")


@pytest.mark.parametrize("path", [B.LMOE_PATH_AUTO, S])
def test_small_prefill(path):
    P.compare(SMALL_PREFILL, make_inputs(SMALL_PREFILL, 3), SMALL_PREFILL.K, path=path)


@pytest.mark.parametrize("path", [B.LMOE_PATH_AUTO, TL])
def test_small_decode_m192(path):
    P.compare(SMALL_DECODE, make_inputs(SMALL_DECODE, 4), SMALL_DECODE.K, path=path)


@pytest.mark.parametrize("w", [
    Workload("one_token", T=1, d=256, l=64, N=16, K=3, m=128, dtype="bf16"),
    Workload("k_is_1", T=50, d=256, l=128, N=16, K=1, m=128, dtype="bf16"),
    Workload("k_is_n", T=20, d=256, l=64, N=8, K=8, m=64, dtype="bf16"),
    Workload("n_37", T=70, d=192, l=64, N=37, K=5, m=128, dtype="bf16"),
    Workload("multi_block_dispatch", T=700, d=256, l=64, N=300, K=7, m=64, dtype="bf16"),
    Workload("many_experts", T=40, d=256, l=64, N=2048, K=64, m=64, dtype="bf16"),
    Workload("f32_ragged", T=333, d=192, l=128, N=20, K=3, m=192, dtype="f32"),
    Workload("f32_one_token", T=1, d=64, l=64, N=4, K=2, m=64, dtype="f32"),
    Workload("standard_small", T=90, d=256, l=256, N=12, K=2, m=128, dtype="bf16", standard=True),
    Workload("standard_f32", T=45, d=128, l=128, N=9, K=3, m=64, dtype="f32", standard=True),
    Workload("biased", T=300, d=256, l=64, N=40, K=4, m=128, dtype="bf16", bias=True),
    # >= 512 rows per expert on average: the FFN runs on 256 x 256 tiles, here
    # with ragged rows (~750 per expert), ragged FFN columns (m = 320, l = 192)
    # and a ragged up-projection (T = 1500, d = 320)
    Workload("large_tile_ragged", T=1500, d=320, l=192, N=4, K=2, m=320, dtype="bf16"),
], ids=lambda w: w.name)
@pytest.mark.parametrize("path", [B.LMOE_PATH_AUTO, S, TL])
def test_edge_shapes(w, path):
    if w.dtype == "f32" and path == S:
        pytest.skip("the streaming FFN is bf16 only")
    P.compare(w, make_inputs(w, 5), w.K, path=path, tag=f"{w.name}/path{path}")


def test_all_tokens_on_few_experts():
    """A huge bias on experts 3 and 7 sends every token there: two experts of
    T rows each, all others empty (more than 256 rows for one expert)."""
    w = Workload("concentrated", T=400, d=256, l=128, N=32, K=2, m=128, dtype="bf16", bias=True)
    inp = make_inputs(w, 6)
    inp["bias"] = torch.full((w.N,), -50.0)
    inp["bias"][3] = 50.0
    inp["bias"][7] = 50.0
    for path in (S, TL):
        rep = P.compare(w, inp, w.K, path=path, tag=f"concentrated/path{path}")
        assert set(np.unique(rep["ids"])) == {3, 7}


def test_heavy_and_light_experts_tiled():
    """Two experts that nearly every token names (a bias of +3) beside 62
    light ones, on the 128-row FFN tiles: the two heavy experts (over 500
    rows each: two full 256-row tiles and a ragged one) run on the large GEMM
    tile from their own tile list, the light ones (at most 128 rows) on
    128-row tiles."""
    w = Workload("heavy_light", T=600, d=256, l=128, N=64, K=4, m=128, dtype="bf16", bias=True)
    inp = make_inputs(w, 8)
    inp["bias"] = torch.zeros(w.N)
    inp["bias"][5] = 3.0
    inp["bias"][40] = 3.0
    rep = P.compare(w, inp, w.K, path=TL, tag="heavy_light/path2")
    counts = np.bincount(np.asarray(rep["ids"]).ravel(), minlength=w.N)
    assert counts[5] > 512 and counts[40] > 512
    assert np.sort(counts)[-3] <= 128


# --- exact properties ----------------------------------------------------------

@pytest.mark.parametrize("path", [S, TL])
@pytest.mark.parametrize("N,K", [(16, 3), (200, 9), (512, 22), (640, 22), (1100, 16)])
def test_exact_ties_take_the_lower_index(path, N, K):
    """Small-integer x and router rows make every logit an exact integer in
    fp32 and fp64 alike, with router rows duplicated in pairs on top, so
    ties straddle the top-K boundary on most tokens: the ids, in rank order,
    must be exactly the oracle's (larger logit first, then lower index), on
    both top-K kernels and across the logits-per-lane tiers."""
    w = Workload(f"ties_{N}_{K}", T=96, d=256, l=64, N=N, K=K, m=64, dtype="bf16")
    inp = make_inputs(w, 22)
    g = torch.Generator().manual_seed(23)
    inp["x"] = torch.randint(-3, 4, inp["x"].shape, generator=g).to(torch.bfloat16)
    wr = torch.randint(-2, 3, inp["W_router"].shape, generator=g).to(torch.bfloat16)
    wr[1::2] = wr[0::2][: N // 2]
    inp["W_router"] = wr.contiguous()
    d = P.to_device(inp)
    _, ids, gates, _ = B.forward(d, w.K, path=path, routing=True)
    torch.cuda.synchronize()
    ref = P.run_oracle(P.oracle_arrays(inp), w.K)
    ids_g = ids.cpu().numpy()
    assert np.array_equal(ids_g, ref["ids"]), (
        f"{int((ids_g != ref['ids']).any(axis=1).sum())} tokens differ from the oracle's tie order")
    assert np.abs(gates.cpu().numpy() - ref["gates"]).max() <= 1e-5



@pytest.mark.parametrize("path", [S, TL])
def test_zero_weights_give_x_exactly(path):
    w = Workload("zeros", T=77, d=256, l=128, N=16, K=4, m=128, dtype="bf16")
    inp = make_inputs(w, 7)
    for key in ("W2", "W_up"):
        z = dict(inp)
        z[key] = torch.zeros_like(inp[key])
        d = P.to_device(z)
        out = B.forward(d, w.K, path=path)
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), inp["x"]), key


def test_identity_projection_matches_standard():
    """l = d with identity W_down and W_up runs the latent kernels and must
    agree with the standard MoE: bit-exactly in float32 (every identity
    product is exact); in bf16 both match the oracle (the latent path rounds
    s to bf16 once more, so they may differ by an output ulp)."""
    for dtype, path in (("f32", TL), ("bf16", S), ("bf16", TL)):
        w = Workload(f"identity_{dtype}", T=64, d=128, l=128, N=8, K=2, m=64, dtype=dtype, standard=True)
        inp = make_inputs(w, 8)
        lat = dict(inp)
        eye = torch.eye(w.d, dtype=w.torch_dtype)
        lat["W_down"], lat["W_up"] = eye, eye.clone()
        r_std = P.compare(w, inp, w.K, path=path, tag=f"identity/standard/{dtype}/path{path}")
        r_lat = P.compare(w.replace(standard=False), lat, w.K, path=path, tag=f"identity/latent/{dtype}/path{path}")
        assert np.array_equal(r_std["ids"], r_lat["ids"])
        if dtype == "f32":
            assert torch.equal(r_std["out"], r_lat["out"])


@pytest.mark.parametrize("path", [S, TL])
def test_deterministic(path):
    w = Workload("det", T=200, d=512, l=128, N=64, K=6, m=128, dtype="bf16")
    d = P.to_device(make_inputs(w, 9))
    a = B.forward(d, w.K, path=path)
    b = B.forward(d, w.K, path=path)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_routing_buffers_optional_and_stream_argument():
    w = Workload("opt", T=48, d=256, l=64, N=16, K=3, m=64, dtype="bf16")
    d = P.to_device(make_inputs(w, 10))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o1 = B.forward(d, w.K)
    o2, ids, gates, _ = B.forward(d, w.K, routing=True, stream=s)
    s.synchronize()
    assert torch.equal(o1, o2)
    assert ids.shape == (48, 3) and torch.allclose(gates.sum(1), torch.ones(48, device="cuda"))
