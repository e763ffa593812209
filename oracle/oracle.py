"""Python access to the fp64 CPU oracle of the LatentMoE layer forward.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  Nothing here imports the
HIP library or its package, and the HIP library never calls this.

`build()` compiles latentmoe_oracle.c with gcc (OpenMP, no fast-math, no FP
contraction, so every sum is the plain double-precision sum in index order).
`forward()` runs it on numpy arrays holding the exact values the GPU gets
(float32, or bfloat16 bit patterns as uint16).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "latentmoe_oracle.c")
LIB = os.path.join(HERE, "liblatentmoe_oracle.so")

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11"]


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32)
                for n in ("T", "d", "l", "N", "K", "m", "dtype", "standard", "m_shared", "expert_format",
                          "n_zero", "n_copy", "n_const")]


def build(src: str = SRC, out: str = LIB, extra: Sequence[str] = ()) -> str:
    """Compile the oracle (or a variant source) into a shared library."""
    tmp = f"{out}.tmp{os.getpid()}"   # one per process: parallel test workers may build at once
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """Handle on one compiled oracle library."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            build(out=path) if path == LIB else None
        self.lib = ctypes.CDLL(path)
        f = self.lib.oracle_forward
        f.restype = ctypes.c_int
        P = ctypes.c_void_p
        f.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int32, P, P, P, P, P, P]
        self.lib.oracle_threads.restype = ctypes.c_int
        self.lib.oracle_set_threads.argtypes = [ctypes.c_int]

    def threads(self) -> int:
        return int(self.lib.oracle_threads())

    def set_threads(self, n: int) -> None:
        self.lib.oracle_set_threads(int(n))

    def forward(self, x, W_down, W_router, W1, W2, W_up, K: int, *, bias=None,
                standard: bool = False, sel: Optional[Sequence[int]] = None,
                forced_ids=None, W_s1=None, W_s2=None, W1_scale=None, W2_scale=None,
                n_zero: int = 0, n_copy: int = 0, zc_const=None):
        """Evaluate the layer for the tokens in `sel` (all tokens if None).

        Arrays: numpy float32, or uint16 holding bfloat16 bits, in the
        storage layout x [T,d], W_down [l,d], W_router [N,d], W1 [N,m,l],
        W2 [N,l,m], W_up [d,l]; bias float32 [N] or None; the shared expert
        W_s1 [m_s,d] and W_s2 [d,m_s], or None for none.  FP8 experts: W1 and
        W2 as uint8 E4M3 codes with float32 row scales W1_scale [N,m] and
        W2_scale [N,l].  MXFP4 experts: W1 [N,m,l/2] and W2 [N,l,m/2] uint8
        (two E2M1 codes per byte, even element in the low nibble) with uint8
        E8M0 block scales W1_scale [N,m,l/32] and W2_scale [N,l,m/32].  Zero-computation experts: n_zero zero and n_copy copy
        experts and zc_const [n_const, l] (same dtype as x) constant experts
        take the routed ids N, N+1, ... in that order; W_router (and bias)
        then have N + n_zero + n_copy + n_const rows (Nr).
        Returns dict(out [n,d] f64, ids [n,K] i32, gates [n,K] f64,
        logits [n,Nr] f64, gap [n] f64).
        """
        x = np.ascontiguousarray(x)
        dtype = 0 if x.dtype == np.float32 else 1
        if dtype == 1 and x.dtype != np.uint16:
            raise TypeError("x must be float32 or uint16 (bf16 bits)")
        T, d = x.shape
        fp8 = W1_scale is not None
        if fp8 != (W2_scale is not None):
            raise ValueError("W1_scale and W2_scale come together")
        mx = fp8 and np.asarray(W1_scale).dtype == np.uint8   # MXFP4: byte scales
        N = W1.shape[0]
        m = W1.shape[1]
        l = W1.shape[2] * (2 if mx else 1)
        n_const = 0 if zc_const is None else int(zc_const.shape[0])
        Nr = N + n_zero + n_copy + n_const
        if W_router.shape[0] != Nr:
            raise ValueError(f"W_router has {W_router.shape[0]} rows, expected N + zero-computation = {Nr}")
        if (W_s1 is None) != (W_s2 is None):
            raise ValueError("W_s1 and W_s2 come together")
        ms = 0 if W_s1 is None else int(W_s1.shape[0])
        if fp8 and (W1.dtype != np.uint8 or W2.dtype != np.uint8):
            raise TypeError("FP8 expert weights are uint8 E4M3 codes")
        arrs = [x, W_down, W_router, W1, W2, W_up, W_s1, W_s2, zc_const]
        for a in arrs:
            if a is not None and a.dtype != x.dtype and not (fp8 and (a is W1 or a is W2)):
                raise TypeError("all of x and the weights must share one dtype")
        arrs = [None if a is None else np.ascontiguousarray(a) for a in arrs]
        x, W_down, W_router, W1, W2, W_up, W_s1, W_s2, zc_const = arrs
        if zc_const is not None:
            assert zc_const.shape == (n_const, l)
        if bias is not None:
            bias = np.ascontiguousarray(bias, dtype=np.float32)
        if sel is None:
            sel_arr = None
            n = T
        else:
            sel_arr = np.ascontiguousarray(np.asarray(sel, dtype=np.int32))
            n = int(sel_arr.shape[0])
        if forced_ids is not None:
            forced_ids = np.ascontiguousarray(np.asarray(forced_ids, dtype=np.int32))
            assert forced_ids.shape == (n, K)
        if mx:
            W1_scale = np.ascontiguousarray(W1_scale)
            W2_scale = np.ascontiguousarray(W2_scale, dtype=np.uint8)
            assert W1.shape == (N, m, l // 2) and W2.shape == (N, l, m // 2)
            assert W1_scale.size == N * m * l // 32 and W2_scale.size == N * l * m // 32
        elif fp8:
            W1_scale = np.ascontiguousarray(W1_scale, dtype=np.float32)
            W2_scale = np.ascontiguousarray(W2_scale, dtype=np.float32)
            assert W1_scale.size == N * m and W2_scale.size == N * l
        D = _Dims(T, d, l, N, K, m, dtype, 1 if standard else 0, ms, 2 if mx else (1 if fp8 else 0),
                  n_zero, n_copy, n_const)
        out = np.empty((n, d), np.float64)
        ids = np.empty((n, K), np.int32)
        gates = np.empty((n, K), np.float64)
        logits = np.empty((n, Nr), np.float64)
        gap = np.empty((n,), np.float64)

        def p(a):
            return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

        rc = self.lib.oracle_forward(ctypes.byref(D), p(x), p(W_down), p(W_router), p(W1), p(W2),
                                     p(W_up), p(W_s1), p(W_s2), p(W1_scale), p(W2_scale), p(zc_const), p(bias),
                                     p(sel_arr),
                                     n, p(forced_ids),
                                     p(out), p(ids), p(gates), p(logits), p(gap))
        if rc != 0:
            raise ValueError("oracle_forward rejected its arguments")
        return {"out": out, "ids": ids, "gates": gates, "logits": logits, "gap": gap}


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIB):
            build()
        _default = Oracle(LIB)
    return _default


def forward(*args, **kw):
    return default().forward(*args, **kw)


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) or float32 to float64, exactly."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)
