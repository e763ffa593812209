"""ctypes binding of liblatentmoe.so: the C ABI of include/latentmoe.h.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind `latentmoe_forward`.  torch supplies device memory and the stream.
There is no other implementation here: if the library is missing the
functions raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblatentmoe.so")

LMOE_OK, LMOE_EINVAL, LMOE_EUNSUPPORTED, LMOE_EWORKSPACE, LMOE_EHIP = 0, -1, -2, -3, -4
LMOE_F32, LMOE_BF16 = 0, 1
LMOE_PATH_AUTO, LMOE_PATH_STREAM, LMOE_PATH_TILED = 0, 1, 2
LMOE_EXPERTS_DENSE, LMOE_EXPERTS_FP8_E4M3, LMOE_EXPERTS_MXFP4 = 0, 1, 2
LMOE_N_STAGE_EVENTS = 8
STAGES = ("proj_router", "topk", "dispatch", "ffn1", "ffn2", "combine", "up")

EXPORTED = (
    "latentmoe_workspace_bytes",
    "latentmoe_forward",
    "latentmoe_forward_shared",
    "latentmoe_forward_timed",
    "latentmoe_forward_ex",
    "latentmoe_forward_noalloc",
    "latentmoe_status_string",
    "latentmoe_last_error",
    "latentmoe_resolved_path",
    "latentmoe_workspace_layout",
)


class lmoe_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32)
                for n in ("T", "d", "l", "N", "m", "dtype", "path", "m_shared", "expert_format",
                          "n_zero", "n_copy", "n_const")]


class lmoe_args(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "W_down", "W_router", "W1", "W2", "W_up", "W_shared1", "W_shared2", "W1_scale", "W2_scale",
        "zc_const", "router_bias", "out", "topk_ids", "topk_gates", "workspace")] + [
        ("workspace_bytes", ctypes.c_size_t), ("stream", ctypes.c_void_p), ("events", ctypes.c_void_p)]


class lmoe_ws_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("counts", "offsets", "perm", "slot_of", "n_active", "written")]


class LatentMoEError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"latentmoe status {status}: {detail}")
        self.status = status


_lib = None


def lib():
    """Load liblatentmoe.so (built by __graft_entry__.build()); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.latentmoe_workspace_bytes.restype = ctypes.c_size_t
        L.latentmoe_workspace_bytes.argtypes = [ctypes.POINTER(lmoe_dims), ctypes.c_int32]
        L.latentmoe_forward.restype = ctypes.c_int
        L.latentmoe_forward.argtypes = [P, P, P, P, P, P, ctypes.c_int32, P, ctypes.POINTER(lmoe_dims),
                                        P, P, P, P, ctypes.c_size_t, P]
        L.latentmoe_forward_shared.restype = ctypes.c_int
        L.latentmoe_forward_shared.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int32, P,
                                               ctypes.POINTER(lmoe_dims), P, P, P, P, ctypes.c_size_t, P]
        L.latentmoe_forward_timed.restype = ctypes.c_int
        L.latentmoe_forward_timed.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_int32, P,
                                              ctypes.POINTER(lmoe_dims), P, P, P, P, ctypes.c_size_t, P, P]
        L.latentmoe_forward_ex.restype = ctypes.c_int
        L.latentmoe_forward_ex.argtypes = [ctypes.POINTER(lmoe_args), ctypes.c_int32, ctypes.POINTER(lmoe_dims)]
        L.latentmoe_forward_noalloc.restype = ctypes.c_int
        L.latentmoe_forward_noalloc.argtypes = [P, P, P, P, P, P, ctypes.c_int32, P, ctypes.POINTER(lmoe_dims),
                                                P, P, P, P]
        L.latentmoe_status_string.restype = ctypes.c_char_p
        L.latentmoe_status_string.argtypes = [ctypes.c_int]
        L.latentmoe_last_error.restype = ctypes.c_char_p
        L.latentmoe_last_error.argtypes = []
        L.latentmoe_resolved_path.restype = ctypes.c_int
        L.latentmoe_resolved_path.argtypes = [ctypes.POINTER(lmoe_dims), ctypes.c_int32]
        L.latentmoe_workspace_layout.restype = ctypes.c_int
        L.latentmoe_workspace_layout.argtypes = [ctypes.POINTER(lmoe_dims), ctypes.c_int32,
                                                 ctypes.POINTER(lmoe_ws_layout)]
        _lib = L
    return _lib


def make_dims(T, d, l, N, m, dtype, path=LMOE_PATH_AUTO, m_shared=0,
              expert_format=LMOE_EXPERTS_DENSE, n_zero=0, n_copy=0, n_const=0) -> lmoe_dims:
    if isinstance(dtype, torch.dtype):
        dtype = LMOE_F32 if dtype == torch.float32 else LMOE_BF16
    elif isinstance(dtype, str):
        dtype = LMOE_F32 if dtype == "f32" else LMOE_BF16
    return lmoe_dims(T, d, l, N, m, dtype, path, m_shared, expert_format, n_zero, n_copy, n_const)


def latentmoe_workspace_bytes(dims: lmoe_dims, K: int) -> int:
    return int(lib().latentmoe_workspace_bytes(ctypes.byref(dims), K))


def latentmoe_resolved_path(dims: lmoe_dims, K: int) -> int:
    return int(lib().latentmoe_resolved_path(ctypes.byref(dims), K))


def latentmoe_workspace_layout(dims: lmoe_dims, K: int) -> lmoe_ws_layout:
    lay = lmoe_ws_layout()
    rc = lib().latentmoe_workspace_layout(ctypes.byref(dims), K, ctypes.byref(lay))
    _check(rc)
    return lay


def latentmoe_status_string(status: int) -> str:
    return lib().latentmoe_status_string(status).decode()


def latentmoe_last_error() -> str:
    return lib().latentmoe_last_error().decode()


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check(rc: int) -> None:
    if rc != LMOE_OK:
        raise LatentMoEError(rc, f"{latentmoe_status_string(rc)}: {latentmoe_last_error()}")


def latentmoe_forward(x, W_down, W_router, W1, W2, W_up, K: int, out, dims: lmoe_dims,
                      router_bias=None, topk_ids=None, topk_gates=None, workspace=None,
                      workspace_bytes: Optional[int] = None, stream=None, check: bool = True,
                      events=None, W_shared1=None, W_shared2=None, W1_scale=None, W2_scale=None,
                      zc_const=None) -> int:
    """Call the C entry point with raw device pointers taken from tensors.

    `stream`: a torch.cuda.Stream, a raw hipStream_t int, or None for torch's
    current stream.  `events`: None, or a ctypes array of
    LMOE_N_STAGE_EVENTS hipEvent_t handles (calls latentmoe_forward_timed).
    W_shared1 / W_shared2 (with dims.m_shared > 0): calls
    latentmoe_forward_shared.  FP8 experts (W1_scale / W2_scale) or
    zero-computation experts (dims.n_zero / n_copy / n_const, zc_const):
    calls latentmoe_forward_ex.  Returns the status (raises on failure when
    check=True).
    """
    if stream is None:
        stream_ptr = torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    elif isinstance(stream, int):
        stream_ptr = stream
    else:
        stream_ptr = stream.cuda_stream
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ex = (W1_scale is not None or W2_scale is not None or zc_const is not None
          or dims.expert_format != LMOE_EXPERTS_DENSE or (dims.n_zero | dims.n_copy | dims.n_const) != 0)
    if ex:
        args = lmoe_args(_ptr(x), _ptr(W_down), _ptr(W_router), _ptr(W1), _ptr(W2), _ptr(W_up),
                         _ptr(W_shared1), _ptr(W_shared2), _ptr(W1_scale), _ptr(W2_scale), _ptr(zc_const),
                         _ptr(router_bias),
                         _ptr(out), _ptr(topk_ids), _ptr(topk_gates), _ptr(workspace), workspace_bytes,
                         stream_ptr, None if events is None else ctypes.cast(events, ctypes.c_void_p).value)
        rc = lib().latentmoe_forward_ex(ctypes.byref(args), int(K), ctypes.byref(dims))
        if check:
            _check(rc)
        return rc
    head = (_ptr(x), _ptr(W_down), _ptr(W_router), _ptr(W1), _ptr(W2), _ptr(W_up))
    shared = (_ptr(W_shared1), _ptr(W_shared2))
    tail = (int(K), _ptr(out), ctypes.byref(dims), _ptr(router_bias), _ptr(topk_ids), _ptr(topk_gates),
            _ptr(workspace), ctypes.c_size_t(workspace_bytes), stream_ptr)
    if events is not None:
        rc = lib().latentmoe_forward_timed(*head, *shared, *tail, ctypes.cast(events, ctypes.c_void_p))
    elif W_shared1 is not None or W_shared2 is not None:
        rc = lib().latentmoe_forward_shared(*head, *shared, *tail)
    else:
        rc = lib().latentmoe_forward(*head, *tail)
    if check:
        _check(rc)
    return rc


NOALLOC_SCRATCH_BYTES = 64 << 20


def latentmoe_forward_noalloc(x, W_down, W_router, W1, W2, W_up, K: int, out, dims: lmoe_dims,
                              router_bias=None, topk_ids=None, topk_gates=None, stream=None,
                              check: bool = True) -> int:
    """The no-workspace entry point (the library's own static scratch).
    `stream` as in latentmoe_forward.  Returns the status (raises on failure
    when check=True)."""
    if stream is None:
        stream_ptr = torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    elif isinstance(stream, int):
        stream_ptr = stream
    else:
        stream_ptr = stream.cuda_stream
    rc = lib().latentmoe_forward_noalloc(_ptr(x), _ptr(W_down), _ptr(W_router), _ptr(W1), _ptr(W2), _ptr(W_up),
                                         int(K), _ptr(out), ctypes.byref(dims), _ptr(router_bias), _ptr(topk_ids),
                                         _ptr(topk_gates), stream_ptr)
    if check:
        _check(rc)
    return rc


def dims_for(inputs: dict, K: int, path: int = LMOE_PATH_AUTO, n_zero: int = 0, n_copy: int = 0) -> lmoe_dims:
    """dims of the layer held in `inputs`.  The split of the zero-computation
    experts into kinds is not in the arrays: n_zero and n_copy give it (the
    constant experts are the rows of inputs["zc_const"])."""
    x, W1 = inputs["x"], inputs["W1"]
    T, d = x.shape
    N, m, l = W1.shape
    s1 = inputs.get("W1_scale")
    if s1 is None:
        fmt = LMOE_EXPERTS_DENSE
    elif s1.dtype == torch.uint8:   # E8M0 block scales: two E2M1 codes per byte
        fmt, l = LMOE_EXPERTS_MXFP4, 2 * l
    else:
        fmt = LMOE_EXPERTS_FP8_E4M3
    ws1 = inputs.get("W_s1")
    zc = inputs.get("zc_const")
    n_const = 0 if zc is None else zc.shape[0]
    if inputs["W_router"].shape[0] != N + n_zero + n_copy + n_const:
        raise ValueError(f"W_router has {inputs['W_router'].shape[0]} rows for N={N} + {n_zero} zero + "
                         f"{n_copy} copy + {n_const} constant experts")
    return make_dims(T, d, l, N, m, x.dtype, path, 0 if ws1 is None else ws1.shape[0], fmt, n_zero, n_copy, n_const)


def alloc_workspace(dims: lmoe_dims, K: int, device) -> torch.Tensor:
    nbytes = latentmoe_workspace_bytes(dims, K)
    if nbytes == 0:
        raise LatentMoEError(LMOE_EINVAL, latentmoe_last_error())
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def forward(inputs: dict, K: int, *, path: int = LMOE_PATH_AUTO, workspace: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, routing: bool = False, stream=None, n_zero: int = 0,
            n_copy: int = 0):
    """Run the layer on device tensors `inputs` (keys as in inputs.make_inputs;
    n_zero / n_copy: the zero-computation experts' split, as in dims_for).

    Allocates `out` (and the workspace, routing buffers) with torch when not
    given.  Returns out, or (out, ids, gates, workspace) when routing=True.
    """
    x = inputs["x"]
    dims = dims_for(inputs, K, path, n_zero, n_copy)
    if workspace is None:
        workspace = alloc_workspace(dims, K, x.device)
    if out is None:
        out = torch.empty_like(x)
    ids = gates = None
    if routing:
        ids = torch.empty((x.shape[0], K), dtype=torch.int32, device=x.device)
        gates = torch.empty((x.shape[0], K), dtype=torch.float32, device=x.device)
    latentmoe_forward(x, inputs.get("W_down"), inputs["W_router"], inputs["W1"], inputs["W2"],
                      inputs.get("W_up"), K, out, dims, router_bias=inputs.get("bias"),
                      topk_ids=ids, topk_gates=gates, workspace=workspace, stream=stream,
                      W_shared1=inputs.get("W_s1"), W_shared2=inputs.get("W_s2"),
                      W1_scale=inputs.get("W1_scale"), W2_scale=inputs.get("W2_scale"),
                      zc_const=inputs.get("zc_const"))
    if routing:
        return out, ids, gates, workspace
    return out
