"""Host-side checks of bench.py (no GPU): the one-GPU refusal, the
algorithmic byte counts against the sizes of the arrays the layer reads and
writes, and the guard that drops a committed traffic record once the
kernel's sources differ from those it was measured on."""
import hashlib
import json
import os
import shutil
import subprocess
import sys
from glob import glob

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_moe_layer_gemm_amd.inputs import WORKLOADS, Workload, make_inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in rec["error"] and rec["n_gpus_requested"] == 2


SHAPES = [
    Workload("dense", T=5, d=64, l=32, N=6, K=2, m=64, dtype="bf16"),
    Workload("f32", T=5, d=64, l=32, N=6, K=2, m=64, dtype="f32"),
    Workload("fp8", T=5, d=64, l=32, N=6, K=2, m=64, dtype="bf16", experts="fp8"),
    Workload("mxfp4", T=5, d=128, l=64, N=6, K=2, m=96, dtype="bf16", experts="mxfp4"),
    Workload("standard", T=5, d=64, l=64, N=6, K=2, m=32, dtype="bf16", standard=True),
    Workload("options", T=7, d=64, l=32, N=6, K=3, m=64, dtype="bf16", m_shared=32, bias=True,
             n_zero=1, n_copy=1, n_const=2),
]


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


@pytest.mark.parametrize("w", SHAPES, ids=lambda w: w.name)
def test_algorithmic_bytes_are_the_arrays_read_and_written(w):
    """Bytes: every weight array read once (the experts' only for the A
    experts that got rows), x read and out (x's shape) written.  Flops: two
    per multiply-add of each product."""
    inp = make_inputs(w, 0)
    A, R = 3, 11
    per_expert = sum(_nbytes(inp[k][0]) for k in ("W1", "W2", "W1_scale", "W2_scale") if inp.get(k) is not None)
    assert bench.expert_bytes(w, A) == A * per_expert
    once = [inp[k] for k in ("W_down", "W_router", "W_up", "W_s1", "W_s2", "zc_const", "bias")
            if inp.get(k) is not None]
    want_bytes = 2 * _nbytes(inp["x"]) + sum(_nbytes(t) for t in once) + A * per_expert
    nb, nf = bench.algorithmic(w, A, R)
    assert nb == want_bytes
    # multiply-adds: z = W_down x and out = W_up s (T*l*d each, latent only),
    # the logits (T * routed ids * d), two expert products per routed row,
    # the shared expert's two products
    n_ids = inp["W_router"].shape[0]
    macs = w.T * n_ids * w.d + R * 2 * w.l * w.m + 2 * w.T * w.d * w.m_shared
    if not w.standard:
        macs += 2 * w.T * w.l * w.d
    assert nf == 2 * macs


def _mirror(rec_path: str, dst_root) -> dict:
    rec = json.load(open(rec_path))
    for rel in rec["sources"] + [os.path.relpath(rec_path, ROOT)]:
        dst = dst_root / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    return rec


def test_traffic_record_dropped_when_sources_change(tmp_path, monkeypatch):
    recs = sorted(glob(os.path.join(ROOT, "profiles", "*_traffic.json")))
    assert recs, "no committed traffic records"
    rec = _mirror(recs[0], tmp_path)
    rel = os.path.relpath(recs[0], ROOT)
    # stamp the mirrored record with the mirrored sources' hash, so that the
    # check below holds whether or not the committed record is current
    h = hashlib.sha256(b"".join((tmp_path / p).read_bytes() for p in rec["sources"])).hexdigest()
    rec["sources_sha256"] = h
    (tmp_path / rel).write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    w = WORKLOADS[rec["workload"]]
    assert bench.measured_traffic(w, rec["kernel"]) == rec["traffic_bytes_per_launch"]
    # another kernel's name, or a workload without a record: nothing
    assert bench.measured_traffic(w, "gemm2_kernel<Ffn1>+<Ffn2>" if rec["kernel"].startswith("ffn_stream")
                                  else "ffn_stream_kernel") is None
    assert bench.measured_traffic(WORKLOADS["tiny_f32"], rec["kernel"]) is None
    # one byte more in one source: the record no longer applies
    src = tmp_path / rec["sources"][-1]
    src.write_bytes(src.read_bytes() + b"\n")
    assert bench.measured_traffic(w, rec["kernel"]) is None


def test_traffic_records_name_their_workload_and_commands():
    for path in sorted(glob(os.path.join(ROOT, "profiles", "*_traffic.json"))):
        rec = json.load(open(path))
        assert rec["workload"] in WORKLOADS, path
        tag = "ffn_stream" if rec["kernel"].startswith("ffn_stream") else "gemm2_ffn"
        assert os.path.basename(path) == f"{tag}_{rec['workload']}_traffic.json"
        assert all(os.path.exists(os.path.join(ROOT, p)) for p in rec["sources"]), path
        assert any("--pmc FETCH_SIZE" in c for c in rec["commands"]) and \
            any("--pmc WRITE_SIZE" in c for c in rec["commands"]), path
        assert rec["traffic_bytes_per_launch"] == pytest.approx(rec["fetch_bytes"] + rec["write_bytes"])
