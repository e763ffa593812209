"""The timed forward: the same output as the untimed call, and stage events
that bracket the stages in order.

latentmoe_forward_timed records caller-created hipEvents at the stage
boundaries; on the streaming path the expert FFN's two events are the FFN
kernel's own start and end (attached to its launch).  The computation must
not change, and the recorded times must be ordered and non-negative.
"""
import ctypes

import pytest
import torch

from sparse_moe_layer_gemm_amd import binding as B
from sparse_moe_layer_gemm_amd.inputs import WORKLOADS, Workload, make_inputs
from tests import parity as P

pytestmark = pytest.mark.gpu


class _Events:
    """hipEventCreate / ElapsedTime / Destroy through ctypes."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
            self.arr[i] = ev.value

    def ms(self, i, j):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.arr[i], self.arr[j]) == 0
        return out.value

    def close(self):
        for ev in self.arr:
            self.hip.hipEventDestroy(ev)


CASES = [
    (WORKLOADS["decode"], B.LMOE_PATH_AUTO),     # streaming FFN: kernel-attached FFN events
    (Workload("timed_tiled", T=700, d=512, l=128, N=64, K=6, m=256, dtype="bf16"), B.LMOE_PATH_AUTO),
    (WORKLOADS["decode_mxfp4"], B.LMOE_PATH_AUTO),
]


@pytest.mark.parametrize("w,path", CASES, ids=lambda c: c.name if isinstance(c, Workload) else str(c))
def test_timed_forward_equals_untimed_and_orders_its_events(w, path):
    P.log(f"[timed] {w.name} path={path}")
    inp = P.to_device(make_inputs(w, 31))
    dims = B.dims_for(inp, w.K, path)
    ws = B.alloc_workspace(dims, w.K, torch.device("cuda"))
    stream = torch.cuda.current_stream()

    def run(events):
        out = torch.empty_like(inp["x"])
        B.latentmoe_forward(inp["x"], inp["W_down"], inp["W_router"], inp["W1"], inp["W2"], inp["W_up"], w.K, out,
                            dims, router_bias=inp.get("bias"), workspace=ws, stream=stream, events=events,
                            W1_scale=inp.get("W1_scale"), W2_scale=inp.get("W2_scale"))
        return out

    plain = run(None)
    ev = _Events(B.LMOE_N_STAGE_EVENTS)
    try:
        timed = run(ev.arr)
        torch.cuda.synchronize()
        assert torch.equal(plain, timed)
        stages = [ev.ms(i, i + 1) for i in range(B.LMOE_N_STAGE_EVENTS - 1)]
        assert all(t >= 0.0 for t in stages), stages
        total = ev.ms(0, B.LMOE_N_STAGE_EVENTS - 1)
        assert total > 0.0 and abs(total - sum(stages)) <= 1e-3 * max(1.0, total) + 1e-3, (total, stages)
        assert stages[3] > 0.0   # the expert FFN ran between its events
    finally:
        ev.close()
