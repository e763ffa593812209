"""The C-ABI library on the host: it loads, exports what the header declares,
sizes its workspace, and rejects bad arguments before touching a GPU.

No test here launches a kernel: every forward call below fails validation,
which happens before any HIP call.
"""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_moe_layer_gemm_amd import binding as B
from sparse_moe_layer_gemm_amd.inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "latentmoe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from sparse_moe_layer_gemm_amd import build
        build.build()
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(latentmoe_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    nm = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (latentmoe_\w+)", nm))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def dims_of(w, path=B.LMOE_PATH_AUTO):
    fmt = {"dense": B.LMOE_EXPERTS_DENSE, "fp8": B.LMOE_EXPERTS_FP8_E4M3, "mxfp4": B.LMOE_EXPERTS_MXFP4}[w.experts]
    return B.make_dims(w.T, w.d, w.l, w.N, w.m, w.dtype, path, w.m_shared, fmt, w.n_zero, w.n_copy, w.n_const)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workspace_sizes(lib, name):
    w = WORKLOADS[name]
    n = B.latentmoe_workspace_bytes(dims_of(w), w.K)
    assert n > 0 and n % 256 == 0
    lay = B.latentmoe_workspace_layout(dims_of(w), w.K)
    spans = [(lay.counts, 4 * w.N), (lay.offsets, 4 * (w.N + 1)), (lay.perm, 4 * w.T * w.K),
             (lay.slot_of, 4 * w.T * w.K), (lay.n_active, 4)]
    for off, size in spans:
        assert off % 256 == 0 and off + size <= n
    spans.sort()
    for (o1, s1), (o2, _) in zip(spans, spans[1:]):
        assert o1 + s1 <= o2


def test_resolved_paths(lib):
    S, Tl = B.LMOE_PATH_STREAM, B.LMOE_PATH_TILED
    assert B.latentmoe_resolved_path(dims_of(WORKLOADS["decode"]), 22) == S
    assert B.latentmoe_resolved_path(dims_of(WORKLOADS["standard_decode"]), 6) == S
    assert B.latentmoe_resolved_path(dims_of(WORKLOADS["prefill"]), 22) == Tl
    assert B.latentmoe_resolved_path(dims_of(WORKLOADS["skewed"]), 16) == Tl
    assert B.latentmoe_resolved_path(dims_of(WORKLOADS["tiny_f32"]), 4) == Tl
    assert B.latentmoe_resolved_path(dims_of(WORKLOADS["decode"], Tl), 22) == Tl
    assert B.latentmoe_resolved_path(dims_of(WORKLOADS["tiny_f32"], S), 4) == B.LMOE_EUNSUPPORTED


def test_dispatch_written_flag(lib):
    # the streaming path with T <= 256 routes inside the expert FFN and
    # writes no dispatch arrays; every other path does
    S, Tl = B.LMOE_PATH_STREAM, B.LMOE_PATH_TILED
    dec = WORKLOADS["decode"]
    assert B.latentmoe_workspace_layout(dims_of(dec), 22).written == 0
    assert B.latentmoe_workspace_layout(dims_of(dec, Tl), 22).written == 1
    assert B.latentmoe_workspace_layout(dims_of(WORKLOADS["prefill"]), 22).written == 1
    big = B.make_dims(300, dec.d, dec.l, dec.N, dec.m, dec.dtype, S)
    assert B.latentmoe_workspace_layout(big, 22).written == 1
    small = B.make_dims(256, dec.d, dec.l, dec.N, dec.m, dec.dtype, S)
    assert B.latentmoe_workspace_layout(small, 22).written == 0


@pytest.mark.parametrize("field,value,K", [
    ("T", 0, 4), ("d", 100, 4), ("l", 0, 4), ("m", 65, 4), ("N", 0, 4), ("N", 4096, 4),
    ("dtype", 7, 4), ("path", 9, 4), ("m_shared", 96, 4), ("m_shared", -64, 4), ("T", (1 << 24) + 1, 4),
    (None, None, 0), (None, None, 33), (None, None, 65),
])
def test_invalid_dims_rejected(lib, field, value, K):
    d = dims_of(WORKLOADS["tiny_f32"])
    if field:
        setattr(d, field, value)
    assert B.latentmoe_workspace_bytes(d, K) == 0
    assert B.latentmoe_resolved_path(d, K) < 0
    assert B.latentmoe_last_error() != ""


FAKE = 1 << 40  # 256-aligned, never dereferenced: every call below fails validation first


def call(dims, K, **over):
    args = dict(x=FAKE, W_down=FAKE + (1 << 30), W_router=FAKE + (2 << 30), W1=FAKE + (3 << 30),
                W2=FAKE + (4 << 30), W_up=FAKE + (5 << 30), out=FAKE + (6 << 30),
                workspace=FAKE + (7 << 30), workspace_bytes=B.latentmoe_workspace_bytes(dims, K) if K else 0)
    args.update(over)
    return B.latentmoe_forward(args["x"], args["W_down"], args["W_router"], args["W1"], args["W2"],
                               args["W_up"], K, args["out"], dims, router_bias=args.get("bias"),
                               topk_ids=args.get("ids"), topk_gates=args.get("gates"),
                               workspace=args["workspace"],
                               workspace_bytes=args["workspace_bytes"], stream=0, check=False)


def test_forward_argument_checks(lib):
    w = WORKLOADS["decode"]
    d = dims_of(w)
    need = B.latentmoe_workspace_bytes(d, w.K)
    assert call(d, 0) == B.LMOE_EINVAL
    assert call(d, w.K, x=None) == B.LMOE_EINVAL
    assert call(d, w.K, W1=None) == B.LMOE_EINVAL
    assert call(d, w.K, out=None) == B.LMOE_EINVAL
    assert call(d, w.K, W_down=None) == B.LMOE_EINVAL          # only one projection given
    assert call(d, w.K, W_down=None, W_up=None) == B.LMOE_EINVAL  # standard mode needs l == d
    assert call(d, w.K, workspace=None) == B.LMOE_EWORKSPACE
    assert call(d, w.K, workspace_bytes=need - 1) == B.LMOE_EWORKSPACE
    assert "needs" in B.latentmoe_last_error()
    assert call(d, w.K, out=FAKE) == B.LMOE_EINVAL               # out aliases x
    assert call(d, w.K, out=FAKE + 4096) == B.LMOE_EINVAL        # partial overlap
    assert call(d, w.K, workspace=FAKE + (7 << 30) + 8) == B.LMOE_EINVAL
    assert call(d, w.K, W2=FAKE + (4 << 30) + 2) == B.LMOE_EINVAL
    ws = B.make_dims(w.T, w.d, w.l, w.N, w.m, "f32", B.LMOE_PATH_STREAM)
    assert call(ws, w.K) == B.LMOE_EUNSUPPORTED


def test_written_buffers_alias_nothing(lib):
    """out, the routing buffers and the workspace may overlap neither one
    another nor any array the call reads (the header's promise)."""
    w = WORKLOADS["decode"]
    d = dims_of(w)
    GB = 1 << 30
    IDS, GATES = FAKE + (8 << 30), FAKE + (9 << 30)
    assert call(d, w.K, ids=IDS, gates=GATES, workspace_bytes=64) == B.LMOE_EWORKSPACE   # valid otherwise
    last_w1 = FAKE + 3 * GB + w.N * w.m * w.l * 2 - 16                   # W1's last 16 bytes
    cases = [
        (dict(out=FAKE + 3 * GB + 4096), "out must not alias W1"),
        (dict(out=last_w1), "out must not alias W1"),
        (dict(out=FAKE + 2 * GB), "out must not alias W_router"),
        (dict(out=FAKE + 5 * GB + 256), "out must not alias W_up"),
        (dict(out=FAKE + 1 * GB), "out must not alias W_down"),
        (dict(bias=FAKE + (6 << 30) + 64), "out must not alias router_bias"),
        (dict(ids=FAKE + (6 << 30), gates=GATES), "topk_ids must not alias out"),
        (dict(ids=IDS, gates=IDS + 64), "topk_gates must not alias topk_ids"),
        (dict(ids=FAKE + 4 * GB, gates=GATES), "topk_ids must not alias W2"),
        (dict(ids=IDS, gates=FAKE), "topk_gates must not alias x"),
        (dict(ids=IDS, gates=FAKE + (7 << 30) + 256), "the workspace must not alias topk_gates"),
        (dict(workspace=FAKE + 4 * GB), "the workspace must not alias W2"),
    ]
    for over, msg in cases:
        assert call(d, w.K, **over) == B.LMOE_EINVAL, over
        assert msg in B.latentmoe_last_error(), (over, B.latentmoe_last_error())
    # adjacent is fine: out right after W1's last byte (then the workspace size check fails)
    assert call(d, w.K, out=last_w1 + 16, workspace_bytes=64) == B.LMOE_EWORKSPACE


def call_shared(dims, K, **over):
    args = dict(x=FAKE, W_down=FAKE + (1 << 30), W_router=FAKE + (2 << 30), W1=FAKE + (3 << 30),
                W2=FAKE + (4 << 30), W_up=FAKE + (5 << 30), out=FAKE + (6 << 30),
                workspace=FAKE + (7 << 30), workspace_bytes=B.latentmoe_workspace_bytes(dims, K),
                W_shared1=FAKE + (8 << 30), W_shared2=FAKE + (9 << 30))
    args.update(over)
    P = ctypes.c_void_p
    return B.lib().latentmoe_forward_shared(
        P(args["x"]), P(args["W_down"]), P(args["W_router"]), P(args["W1"]), P(args["W2"]), P(args["W_up"]),
        None if args["W_shared1"] is None else P(args["W_shared1"]),
        None if args["W_shared2"] is None else P(args["W_shared2"]), K, P(args["out"]), ctypes.byref(dims),
        None, None, None, P(args["workspace"]), ctypes.c_size_t(args["workspace_bytes"]), None)


def test_shared_expert_argument_checks(lib):
    w = WORKLOADS["decode_shared"]
    d = dims_of(w)
    plain = dims_of(WORKLOADS["decode"])
    assert B.latentmoe_workspace_bytes(d, w.K) > B.latentmoe_workspace_bytes(plain, w.K)
    assert call(d, w.K) == B.LMOE_EINVAL                                  # m_shared > 0 needs the _shared call
    assert "latentmoe_forward_shared" in B.latentmoe_last_error()
    assert call_shared(plain, w.K) == B.LMOE_EINVAL                       # the _shared call needs m_shared > 0
    assert call_shared(d, w.K, W_shared2=None) == B.LMOE_EINVAL           # both shared weights or none
    assert call_shared(d, w.K, W_shared1=None, W_shared2=None) == B.LMOE_EINVAL
    assert call_shared(d, w.K, W_shared2=FAKE + (9 << 30) + 2) == B.LMOE_EINVAL   # misaligned
    assert call_shared(d, w.K, workspace_bytes=B.latentmoe_workspace_bytes(plain, w.K)) == B.LMOE_EWORKSPACE


def call_ex(dims, K, **over):
    args = dict(x=FAKE, W_down=FAKE + (1 << 30), W_router=FAKE + (2 << 30), W1=FAKE + (3 << 30),
                W2=FAKE + (4 << 30), W_up=FAKE + (5 << 30), out=FAKE + (6 << 30),
                workspace=FAKE + (7 << 30), workspace_bytes=B.latentmoe_workspace_bytes(dims, K),
                W1_scale=FAKE + (10 << 30), W2_scale=FAKE + (11 << 30))
    args.update(over)
    g = B.lmoe_args(**args)
    return B.lib().latentmoe_forward_ex(ctypes.byref(g), K, ctypes.byref(dims))


def test_fp8_expert_argument_checks(lib):
    w = WORKLOADS["decode_fp8"]
    d = dims_of(w)
    assert d.expert_format == B.LMOE_EXPERTS_FP8_E4M3
    # the FP8 weights change no workspace region (the same m-slices as bf16)
    for T in (16, 32):
        assert B.latentmoe_workspace_bytes(dims_of(w.replace(T=T)), w.K) == \
            B.latentmoe_workspace_bytes(dims_of(WORKLOADS["decode"].replace(T=T)), w.K)
    P = ctypes.c_void_p
    rc = B.lib().latentmoe_forward(P(FAKE), P(FAKE + (1 << 30)), P(FAKE + (2 << 30)), P(FAKE + (3 << 30)),
                                   P(FAKE + (4 << 30)), P(FAKE + (5 << 30)), w.K, P(FAKE + (6 << 30)),
                                   ctypes.byref(d), None, None, None, P(FAKE + (7 << 30)),
                                   ctypes.c_size_t(B.latentmoe_workspace_bytes(d, w.K)), None)
    assert rc == B.LMOE_EINVAL                                             # FP8 needs the _ex call
    assert "latentmoe_forward_ex" in B.latentmoe_last_error()
    assert call_shared(dims_of(w.replace(m_shared=64)), w.K) == B.LMOE_EINVAL
    assert call_ex(d, w.K, W2_scale=None) == B.LMOE_EINVAL                # both scales or none
    assert call_ex(d, w.K, W1_scale=None, W2_scale=None) == B.LMOE_EINVAL
    assert call_ex(d, w.K, W1_scale=FAKE + (10 << 30) + 4) == B.LMOE_EINVAL  # misaligned
    plain = dims_of(WORKLOADS["decode"])
    assert call_ex(plain, w.K) == B.LMOE_EINVAL                           # scales without FP8
    f32 = dims_of(WORKLOADS["tiny_f32"].replace(experts="fp8"))
    assert call_ex(f32, 4) == B.LMOE_EUNSUPPORTED                         # FP8 experts need bf16
    bad = dims_of(w)
    bad.expert_format = 3
    assert B.latentmoe_workspace_bytes(bad, w.K) == 0
    assert call_ex(bad, w.K) == B.LMOE_EINVAL
    assert B.lib().latentmoe_forward_ex(None, w.K, ctypes.byref(d)) == B.LMOE_EINVAL
    assert call_ex(d, w.K, workspace_bytes=100) == B.LMOE_EWORKSPACE


def test_mxfp4_expert_argument_checks(lib):
    w = WORKLOADS["decode_mxfp4"]
    d = dims_of(w)
    assert d.expert_format == B.LMOE_EXPERTS_MXFP4
    # the MXFP4 weights change no workspace region (the same m-slices as bf16)
    for T in (16, 32):
        assert B.latentmoe_workspace_bytes(dims_of(w.replace(T=T)), w.K) == \
            B.latentmoe_workspace_bytes(dims_of(WORKLOADS["decode"].replace(T=T)), w.K)
    assert call_ex(d, w.K, W1_scale=None, W2_scale=None) == B.LMOE_EINVAL   # scales required
    assert call_ex(d, w.K, W2_scale=None) == B.LMOE_EINVAL
    # the streaming kernel reads a row's scale bytes as 8-byte vectors
    assert call_ex(d, w.K, W1_scale=FAKE + (10 << 30) + 3) == B.LMOE_EINVAL
    assert call_ex(d, w.K, W2_scale=FAKE + (11 << 30) + 4) == B.LMOE_EINVAL
    assert "8-byte" in B.latentmoe_last_error()
    assert call_ex(d, w.K, W1_scale=FAKE + (10 << 30) + 8, workspace_bytes=64) == B.LMOE_EWORKSPACE
    f32 = dims_of(WORKLOADS["tiny_f32"].replace(experts="mxfp4"))
    assert call_ex(f32, 4) == B.LMOE_EUNSUPPORTED
    big = dims_of(w.replace(m=65536, l=65536))
    assert B.latentmoe_workspace_bytes(big, w.K) == 0                     # more than 2^31 code bytes
    assert "MXFP4" in B.latentmoe_last_error()


def test_zero_computation_argument_checks(lib):
    w = WORKLOADS["decode_zc"]
    d = dims_of(w)
    ZC = FAKE + (12 << 30)
    # the dispatch counts cover every routed id
    lay = B.latentmoe_workspace_layout(d, w.K)
    assert lay.offsets - lay.counts >= 4 * (w.N + w.n_zc)
    P = ctypes.c_void_p
    rc = B.lib().latentmoe_forward(P(FAKE), P(FAKE + (1 << 30)), P(FAKE + (2 << 30)), P(FAKE + (3 << 30)),
                                   P(FAKE + (4 << 30)), P(FAKE + (5 << 30)), w.K, P(FAKE + (6 << 30)),
                                   ctypes.byref(d), None, None, None, P(FAKE + (7 << 30)),
                                   ctypes.c_size_t(B.latentmoe_workspace_bytes(d, w.K)), None)
    assert rc == B.LMOE_EINVAL and "latentmoe_forward_ex" in B.latentmoe_last_error()
    nofp8 = dict(W1_scale=None, W2_scale=None)
    assert call_ex(d, w.K, **nofp8) == B.LMOE_EINVAL                       # constants need zc_const
    assert call_ex(d, w.K, zc_const=ZC + 8, **nofp8) == B.LMOE_EINVAL      # misaligned
    no_const = dims_of(w.replace(n_const=0))
    assert call_ex(no_const, w.K, zc_const=ZC, **nofp8) == B.LMOE_EINVAL   # zc_const without constants
    for bad in (dict(n_zero=-1), dict(n_copy=-2), dict(n_const=-1), dict(n_zero=2048 - 512)):
        bd = dims_of(w.replace(**bad))
        assert B.latentmoe_workspace_bytes(bd, w.K) == 0
    # K may exceed N (zero-computation ids count) but not N + n_zc
    small = w.replace(N=8, K=20, n_zero=6, n_copy=4, n_const=2)
    assert B.latentmoe_workspace_bytes(dims_of(small), 20) > 0
    assert B.latentmoe_workspace_bytes(dims_of(small), 21) == 0
    assert call_ex(d, w.K, zc_const=ZC, workspace_bytes=64, **nofp8) == B.LMOE_EWORKSPACE


def test_entry_point_option_checks(lib):
    """Each entry point other than latentmoe_forward_ex rejects the options it
    does not take before touching the device; the no-allocation entry point
    rejects dims whose workspace exceeds its static scratch."""
    P = ctypes.c_void_p
    w = WORKLOADS["decode"]
    ptrs = [P(FAKE + (i << 30)) for i in range(6)]
    out = P(FAKE + (6 << 30))

    def noalloc(d, K=w.K):
        return B.lib().latentmoe_forward_noalloc(*ptrs, K, out, ctypes.byref(d), None, None, None, None)

    big = dims_of(w.replace(T=1024))
    assert B.latentmoe_workspace_bytes(big, w.K) > B.NOALLOC_SCRATCH_BYTES
    assert noalloc(big) == B.LMOE_EUNSUPPORTED and "latentmoe_forward_noalloc" in B.latentmoe_last_error()
    assert noalloc(dims_of(w.replace(m_shared=64))) == B.LMOE_EINVAL
    assert "latentmoe_forward_shared" in B.latentmoe_last_error()
    assert noalloc(dims_of(WORKLOADS["decode_fp8"])) == B.LMOE_EINVAL
    assert noalloc(dims_of(WORKLOADS["decode_zc"])) == B.LMOE_EINVAL
    assert noalloc(dims_of(w), K=0) == B.LMOE_EINVAL
    assert call_shared(dims_of(w), w.K) == B.LMOE_EINVAL                  # m_shared = 0
    assert "m_shared > 0" in B.latentmoe_last_error()
    d = dims_of(w)
    rc = B.lib().latentmoe_forward_timed(*ptrs, None, None, w.K, out, ctypes.byref(d), None, None, None,
                                         P(FAKE + (7 << 30)), ctypes.c_size_t(B.latentmoe_workspace_bytes(d, w.K)),
                                         None, None)
    assert rc == B.LMOE_EINVAL and "events" in B.latentmoe_last_error()


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, 99):
        assert isinstance(B.latentmoe_status_string(code), str)
    assert B.latentmoe_status_string(0) == "ok"
