"""The forward captured into a HIP graph (torch.cuda.CUDAGraph on ROCm).

The C entry point only enqueues kernels on the caller's stream (no host
synchronisation, no allocation, no memset), so it can be captured.  Each
test captures one forward, then replays it several times with new tokens
written into x in between (eager work and synchronisations between the
replays) and requires every replay to equal, bit for bit, an eager forward
on the same inputs.
"""
import pytest
import torch

from sparse_moe_layer_gemm_amd import binding as B
from sparse_moe_layer_gemm_amd.inputs import WORKLOADS, Workload, draw_x, make_inputs
from tests import parity as P

pytestmark = pytest.mark.gpu

CASES = [
    (WORKLOADS["decode"], B.LMOE_PATH_AUTO),                      # split projection, streaming FFN
    (Workload("graph_tiled", T=700, d=512, l=128, N=64, K=6, m=256, dtype="bf16"), B.LMOE_PATH_AUTO),
    (Workload("graph_options", T=64, d=256, l=64, N=16, K=4, m=128, dtype="bf16", bias=True, m_shared=64,
              experts="mxfp4", n_zero=2, n_copy=1, n_const=1), B.LMOE_PATH_STREAM),
    (Workload("graph_options_tiled", T=300, d=256, l=64, N=16, K=4, m=128, dtype="bf16", m_shared=64,
              experts="fp8", n_zero=1, n_copy=1, n_const=1), B.LMOE_PATH_TILED),
    (Workload("graph_f32", T=64, d=256, l=64, N=32, K=4, m=128, dtype="f32"), B.LMOE_PATH_AUTO),
]


@pytest.mark.parametrize("w,path", CASES, ids=lambda c: c.name if isinstance(c, Workload) else str(c))
def test_graph_replays_match_eager(w, path):
    P.log(f"[graph] {w.name} path={path}")
    zc = dict(n_zero=w.n_zero, n_copy=w.n_copy)
    inp = P.to_device(make_inputs(w, 21))
    dims = B.dims_for(inp, w.K, path, **zc)
    ws = B.alloc_workspace(dims, w.K, "cuda")
    out = torch.empty_like(inp["x"])
    ids = torch.empty((w.T, w.K), dtype=torch.int32, device="cuda")
    gates = torch.empty((w.T, w.K), dtype=torch.float32, device="cuda")

    def call(out_t, ws_t, ids_t, gates_t):
        B.latentmoe_forward(inp["x"], inp["W_down"], inp["W_router"], inp["W1"], inp["W2"], inp["W_up"], w.K,
                            out_t, dims, router_bias=inp["bias"], topk_ids=ids_t, topk_gates=gates_t,
                            workspace=ws_t, W_shared1=inp.get("W_s1"), W_shared2=inp.get("W_s2"),
                            W1_scale=inp.get("W1_scale"), W2_scale=inp.get("W2_scale"),
                            zc_const=inp.get("zc_const"))

    call(out, ws, ids, gates)   # warm-up before capture (one-time set-up happens here)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, ws, ids, gates)
    torch.cuda.synchronize()

    ws_e = B.alloc_workspace(dims, w.K, "cuda")
    out_e = torch.empty_like(out)
    ids_e = torch.empty_like(ids)
    gates_e = torch.empty_like(gates)
    for r in range(4):
        inp["x"].copy_(draw_x(w, 100 + r).to("cuda"))   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(out_e, ws_e, ids_e, gates_e)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_e), f"replay {r}: ids"
        assert torch.equal(gates, gates_e), f"replay {r}: gates"
        assert torch.equal(out, out_e), f"replay {r}: out"
    del g
