"""Seeded synthetic inputs for the LatentMoE layer forward.

This module is shared by the HIP path's tests and benchmark and by the
oracle's tests.  It only draws random numbers and casts them; it holds none
of the layer's arithmetic.

Shapes follow the pages' workloads:
  * Nemotron 3 Super: 512 experts, top-22, latent width l = 1024 = d/4
    (zhichai.net "LatentMoE: How MoE Made a Key Paradigm Leap in 2026",
    section 4 "Two Teams, Two Practices").
  * The Table-1 comparison: a standard MoE with d = 4096, 128 experts, top-6
    against a LatentMoE with l = 1024, 512 experts, top-22 (10100.com article,
    section 2.3 "评估", Table 1).
  * Kimi K3: 896 experts, top-16 (same zhichai.net page, section 4).
The expert width m and, for the Kimi-like shape, l are not on the pages; the
values below are choices of this library's workload set.

Storage layout (chosen for MFMA: the reduction index is contiguous for both
operands of every product):
  x        [T, d]
  W_down   [l, d]        z_j   = sum_i W_down[j, i] x_i
  W_router [N, d]        logit_e = sum_i W_router[e, i] x_i (+ bias_e)
  W1       [N, m, l]     h_j   = sum_i W1[e, j, i] z_i
  W2       [N, l, m]     y_i   = sum_j W2[e, i, j] a_j
  W_up     [d, l]        out_n = x_n + sum_i W_up[n, i] s_i
  bias     [N] float32 (skewed workload only)
  W_s1     [m_s, d], W_s2 [d, m_s]   shared expert (the *_shared workloads)
  FP8 experts (the *_fp8 workloads): W1, W2 as uint8 E4M3 codes in the same
  layout, W1_scale [N, m] and W2_scale [N, l] float32 row scales
  MXFP4 experts (the *_mxfp4 workloads): W1 [N, m, l/2], W2 [N, l, m/2]
  uint8 (two E2M1 codes per byte, even element in the low nibble),
  W1_scale [N, m, l/32] and W2_scale [N, l, m/32] uint8 E8M0 block scales
  zero-computation experts (the *_zc workloads): W_router (and bias) get
  n_zero + n_copy + n_const more rows; zc_const [n_const, l]

Recipe: one CPU torch.Generator seeded with `seed`; draws in the order x,
W_down, W_router, W1 (one draw of [m, l] per expert, expert 0 first), W2 (one
[l, m] draw per expert), W_up, bias, W_s1, W_s2 (the last two only for a
shared expert, so the other arrays are the same with or without one), then
for zero-computation experts their router rows, their bias entries and the
constant vectors (zc_const ~ N(0, 1), the scale of z), appended so that the
rest of the layer is the same with or without them.
Every draw is float32 N(0, 1); weights
are multiplied by 1/sqrt(fan_in) in float32; for bf16 workloads every array
except the bias is then rounded to bfloat16 (round-to-nearest-even).
FP8 experts stand for a checkpoint stored that way: each expert's float32
draw (the same draw as above) is cut into rows, each row gets the scale
max|row| / 448 (1 for an all-zero row) and its codes are the row divided by
that scale, rounded to E4M3 by torch's float8_e4m3fn conversion.  MXFP4
experts likewise: each block of 32 elements of a row gets the shared
exponent floor(log2 max|block|) - 2 (so the block's largest element lands
in [4, 8) and E2M1's largest value, 6, is reached), and each element is
rounded to the nearest E2M1 value (ties down, saturating at 6).
x ~ N(0, 1) throughout, so routing is near uniform except where the fixed
logit bias ~ N(0, 1) skews the expert loads.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    l: int
    N: int
    K: int
    m: int
    dtype: str            # "f32" or "bf16"
    standard: bool = False  # no projections: l == d, z = x, out = x + s
    bias: bool = False      # fixed per-expert logit bias ~ N(0, 1)
    m_shared: int = 0       # shared expert width (0: none)
    experts: str = "dense"  # routed expert weights: "dense" (the layer's dtype), "fp8" (E4M3 + row scales)
    #                         or "mxfp4" (E2M1 + E8M0 block scales)
    n_zero: int = 0         # zero-computation experts (ids N ...): zero,
    n_copy: int = 0         # copy
    n_const: int = 0        # and constant experts

    @property
    def n_zc(self) -> int:
        return self.n_zero + self.n_copy + self.n_const

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


# The five workloads (the standard-MoE one at two token counts), and the
# decode / prefill layers with a shared expert.
WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", T=64, d=256, l=64, N=32, K=4, m=128, dtype="f32"),
    "decode": Workload("decode", T=32, d=4096, l=1024, N=512, K=22, m=768, dtype="bf16"),
    "prefill": Workload("prefill", T=16384, d=4096, l=1024, N=512, K=22, m=768, dtype="bf16"),
    "standard_decode": Workload("standard_decode", T=32, d=4096, l=4096, N=128, K=6, m=768,
                                dtype="bf16", standard=True),
    "standard_prefill": Workload("standard_prefill", T=16384, d=4096, l=4096, N=128, K=6, m=768,
                                 dtype="bf16", standard=True),
    "skewed": Workload("skewed", T=8192, d=7168, l=1792, N=896, K=16, m=512, dtype="bf16",
                       bias=True),
    # The decode and prefill layers with a shared expert at the full width d
    # (the pages keep it at d but give no width: m_shared = m is a choice).
    "decode_shared": Workload("decode_shared", T=32, d=4096, l=1024, N=512, K=22, m=768, dtype="bf16",
                              m_shared=768),
    "prefill_shared": Workload("prefill_shared", T=16384, d=4096, l=1024, N=512, K=22, m=768, dtype="bf16",
                               m_shared=768),
    # The decode and prefill layers with FP8 E4M3 routed-expert weights.
    "decode_fp8": Workload("decode_fp8", T=32, d=4096, l=1024, N=512, K=22, m=768, dtype="bf16",
                           experts="fp8"),
    "prefill_fp8": Workload("prefill_fp8", T=16384, d=4096, l=1024, N=512, K=22, m=768, dtype="bf16",
                            experts="fp8"),
    # The decode and prefill layers with MXFP4 routed-expert weights.
    "decode_mxfp4": Workload("decode_mxfp4", T=32, d=4096, l=1024, N=512, K=22, m=768, dtype="bf16",
                             experts="mxfp4"),
    "prefill_mxfp4": Workload("prefill_mxfp4", T=16384, d=4096, l=1024, N=512, K=22, m=768, dtype="bf16",
                              experts="mxfp4"),
    # The decode and prefill layers with 64 zero-computation experts besides
    # the 512 FFN experts (32 zero, 16 copy, 16 constant): about 11 % of the
    # top-22 picks skip the FFN (the pages report LongCat's average activated
    # parameters ~10 % below the maximum; the split is a choice).
    "decode_zc": Workload("decode_zc", T=32, d=4096, l=1024, N=512, K=22, m=768, dtype="bf16",
                          n_zero=32, n_copy=16, n_const=16),
    "prefill_zc": Workload("prefill_zc", T=16384, d=4096, l=1024, N=512, K=22, m=768, dtype="bf16",
                           n_zero=32, n_copy=16, n_const=16),
}


E4M3_MAX = 448.0


# E2M1 magnitudes by code (OCP Microscaling spec) and the rounding
# boundaries between neighbours
_E2M1 = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1_MID = (_E2M1[1:] + _E2M1[:-1]) / 2


def quantize_mxfp4(w: torch.Tensor):
    """float32 [rows, cols] -> (uint8 codes [rows, cols/2], uint8 E8M0 scales [rows, cols/32])."""
    rows, cols = w.shape
    b = w.reshape(rows, cols // 32, 32)
    amax = b.abs().amax(dim=-1)
    ex = (torch.floor(torch.log2(amax.clamp_min(2.0 ** -120))) - 2).clamp(-126, 127)
    q = b / torch.exp2(ex).unsqueeze(-1)
    idx = torch.bucketize(q.abs(), _E2M1_MID)
    code = (idx | ((q < 0).to(idx.dtype) << 3)).reshape(rows, cols).to(torch.uint8)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return packed.contiguous(), (ex + 127).to(torch.uint8).contiguous()


def decode_mxfp4(codes: torch.Tensor, scales: torch.Tensor) -> torch.Tensor:
    """uint8 codes [..., cols/2], scales [..., cols/32] -> float32 [..., cols]."""
    nib = torch.stack([codes & 15, codes >> 4], dim=-1).reshape(*codes.shape[:-1], 2 * codes.shape[-1]).long()
    val = _E2M1[nib & 7] * torch.where((nib & 8) != 0, -1.0, 1.0)
    return val * torch.exp2(scales.float() - 127).repeat_interleave(32, dim=-1)


def quantize_rows_e4m3(w: torch.Tensor):
    """float32 [..., rows, cols] -> (uint8 E4M3 codes, float32 scales [..., rows])."""
    amax = w.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    codes = (w / scale.unsqueeze(-1)).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


def _draw(gen: torch.Generator, shape, scale: Optional[float]) -> torch.Tensor:
    t = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if scale is not None:
        t.mul_(scale)
    return t


def make_inputs(w: Workload, seed: int = 0, *, x_only_seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Draw the inputs of workload `w` on the CPU.

    Returns a dict with keys x, W_down, W_router, W1, W2, W_up, bias (None
    where the workload has no such array), W_s1, W_s2 for a shared expert,
    W1_scale, W2_scale for FP8 experts and zc_const for zero-computation
    experts.  Arrays are contiguous CPU tensors
    in the workload's storage dtype; bias stays float32.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    dt = w.torch_dtype
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = _draw(gen, (w.T, w.d), None).to(dt)
    if w.standard:
        out["W_down"] = None
    else:
        out["W_down"] = _draw(gen, (w.l, w.d), 1.0 / math.sqrt(w.d)).to(dt)
    out["W_router"] = _draw(gen, (w.N, w.d), 1.0 / math.sqrt(w.d)).to(dt)
    fp8, mx = w.experts == "fp8", w.experts == "mxfp4"
    if w.experts not in ("dense", "fp8", "mxfp4") or ((fp8 or mx) and w.dtype != "bf16"):
        raise ValueError(f"experts={w.experts!r} with dtype={w.dtype!r}")
    for name, rows, cols in (("W1", w.m, w.l), ("W2", w.l, w.m)):
        if mx:
            W = torch.empty((w.N, rows, cols // 2), dtype=torch.uint8)
            S = torch.empty((w.N, rows, cols // 32), dtype=torch.uint8)
        else:
            W = torch.empty((w.N, rows, cols), dtype=torch.uint8 if fp8 else dt)
            S = torch.empty((w.N, rows), dtype=torch.float32) if fp8 else None
        for e in range(w.N):
            we = _draw(gen, (rows, cols), 1.0 / math.sqrt(cols))
            if mx:
                W[e], S[e] = quantize_mxfp4(we)
            elif fp8:
                W[e], S[e] = quantize_rows_e4m3(we)
            else:
                W[e] = we.to(dt)
        out[name] = W
        if S is not None:
            out[name + "_scale"] = S
    if w.standard:
        out["W_up"] = None
    else:
        out["W_up"] = _draw(gen, (w.d, w.l), 1.0 / math.sqrt(w.l)).to(dt)
    out["bias"] = _draw(gen, (w.N,), None) if w.bias else None
    if w.m_shared > 0:
        out["W_s1"] = _draw(gen, (w.m_shared, w.d), 1.0 / math.sqrt(w.d)).to(dt)
        out["W_s2"] = _draw(gen, (w.d, w.m_shared), 1.0 / math.sqrt(w.m_shared)).to(dt)
    if w.n_zc > 0:
        zr = _draw(gen, (w.n_zc, w.d), 1.0 / math.sqrt(w.d)).to(dt)
        out["W_router"] = torch.cat([out["W_router"], zr]).contiguous()
        if w.bias:
            out["bias"] = torch.cat([out["bias"], _draw(gen, (w.n_zc,), None)]).contiguous()
        out["zc_const"] = _draw(gen, (w.n_const, w.l), None).to(dt) if w.n_const > 0 else None
    if x_only_seed is not None:
        g2 = torch.Generator(device="cpu")
        g2.manual_seed(x_only_seed)
        out["x"] = _draw(g2, (w.T, w.d), None).to(dt)
    return out


def draw_x(w: Workload, seed: int) -> torch.Tensor:
    """A fresh batch of tokens x ~ N(0, 1) for workload `w` from its own seed."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    return _draw(gen, (w.T, w.d), None).to(w.torch_dtype)


def as_numpy_bits(t: Optional[torch.Tensor]):
    """CPU tensor -> numpy array holding the same bits (bf16 as uint16)."""
    if t is None:
        return None
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
