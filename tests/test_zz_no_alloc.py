"""The entry point that allocates nothing (latentmoe_forward_noalloc, the
library's static scratch) against latentmoe_forward with a caller workspace:
the same kernels, so the outputs, ids and gates must be equal bit for bit.
Two calls in a row share the scratch; the second has fewer tokens, so it
must not depend on anything the first left there."""
import pytest
import torch

from sparse_moe_layer_gemm_amd import binding as B
from sparse_moe_layer_gemm_amd.inputs import WORKLOADS, Workload, make_inputs
from tests import parity as P

pytestmark = pytest.mark.gpu


def noalloc(w, d, path=B.LMOE_PATH_AUTO):
    dims = B.dims_for(d, w.K, path)
    out = torch.empty_like(d["x"])
    ids = torch.empty((w.T, w.K), dtype=torch.int32, device=d["x"].device)
    gates = torch.empty((w.T, w.K), dtype=torch.float32, device=d["x"].device)
    B.latentmoe_forward_noalloc(d["x"], d.get("W_down"), d["W_router"], d["W1"], d["W2"], d.get("W_up"), w.K,
                                out, dims, router_bias=d.get("bias"), topk_ids=ids, topk_gates=gates)
    return out, ids, gates


def check_pair(w, inp, path=B.LMOE_PATH_AUTO):
    d = P.to_device(inp)
    a_out, a_ids, a_gates = noalloc(w, d, path)
    b_out, b_ids, b_gates, _ = B.forward(d, w.K, path=path, routing=True)
    torch.cuda.synchronize()
    P.log(f"[noalloc] {w.name}: T={w.T} path={path} max|diff|={(a_out.float() - b_out.float()).abs().max().item()}")
    assert torch.equal(a_ids, b_ids)
    assert torch.equal(a_gates, b_gates)
    assert torch.equal(a_out, b_out)


def fewer_tokens(w, inp, T, seed):
    """The same layer on T new tokens (x ~ N(0, 1), the workload's dtype)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, w.d, generator=g).to(w.torch_dtype)
    return w.replace(name=f"{w.name}_T{T}", T=T), {**inp, "x": x}


# (workload, tokens of the second, smaller call)
PAIRS = [
    (WORKLOADS["decode"], 5),
    (WORKLOADS["standard_decode"], 3),
    (Workload("tiled_noalloc", T=700, d=512, l=128, N=64, K=8, m=256, dtype="bf16", bias=True), 70),
    (WORKLOADS["tiny_f32"], 9),
]


@pytest.mark.parametrize("w,t_small", PAIRS, ids=lambda v: getattr(v, "name", str(v)))
def test_noalloc_equals_the_workspace_entry_point(w, t_small):
    inp = make_inputs(w, 31)
    check_pair(w, inp)
    check_pair(*fewer_tokens(w, inp, t_small, 32))


def test_noalloc_tiled_path_twice():
    w = WORKLOADS["decode"]
    inp = make_inputs(w, 33)
    check_pair(w, inp, path=B.LMOE_PATH_TILED)
    check_pair(*fewer_tokens(w, inp, 17, 34), path=B.LMOE_PATH_TILED)


def test_noalloc_rejects_dims_beyond_its_scratch():
    w = WORKLOADS["decode"].replace(T=1024)   # a workspace of ~107 MiB
    d = P.to_device(make_inputs(w.replace(T=1), 35))
    dims = B.dims_for(d, w.K)
    dims.T = w.T
    assert B.latentmoe_workspace_bytes(dims, w.K) > B.NOALLOC_SCRATCH_BYTES
    out = torch.empty((w.T, w.d), dtype=torch.bfloat16, device="cuda")
    rc = B.latentmoe_forward_noalloc(d["x"], d["W_down"], d["W_router"], d["W1"], d["W2"], d["W_up"], w.K, out,
                                     dims, check=False)
    assert rc == B.LMOE_EUNSUPPORTED and "latentmoe_forward_noalloc" in B.latentmoe_last_error()
