"""Benchmark of the LatentMoE layer forward on one MI355X.

Default workload: the decode-shaped layer (T=32 tokens, d=4096, l=1024,
512 experts, top-22, m=768, bf16 with fp32 accumulation).  One step is one
full forward through the C ABI: projection + router, top-K, dispatch, expert
FFN, combine, projection back with the residual.  Inputs are resident in HBM
before timing starts.  Two independent weight sets (seeds 0 and 1) alternate
between steps so that the 256 MB Infinity Cache cannot serve one step's
expert weights to the next.

Prints ONE JSON line.  `roofline` is for the dominant kernel (the expert FFN):
its algorithmic bytes (weights of the experts that received rows, read once)
or flops per launch over its mean duration measured with HIP events on the
launch stream in every timed step (on the streaming path the FFN kernel's
own start and end, attached to its launch; around the two tiled GEMMs
otherwise).  `cpu_baseline`
times the fp64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LatentMoE fwd tokens/s (d4096 ℓ1024 E512 top22); % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_VECTOR_PEAK_TFLOPS = 157.3   # the float32 path runs on the vector ALUs


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode")
    ap.add_argument("--path", type=int, default=0, help="0 auto, 1 streaming FFN, 2 tiled FFN")
    ap.add_argument("--weight-sets", type=int, default=2)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget; 0 skips it")
    ap.add_argument("--no-events", action="store_true", help="time without stage events")
    ap.add_argument("--extra", default=None,
                    help="comma-separated workloads also measured in the same run and reported under "
                         "extra_workloads (default: prefill,skewed with the decode workload, none otherwise)")
    ap.add_argument("--sweep", default="",
                    help="comma-separated token counts: one JSON line per count, the workload's shape with "
                         "T tokens (x = the first T rows of one draw), no CPU baseline")
    a = ap.parse_args()
    if a.extra is None:
        a.extra = "prefill,skewed" if a.config == "decode" and not a.sweep else ""
    return a


class Hip:
    """The few HIP runtime calls the stage timing needs (events)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed: {rc}")
        return ev.value

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)


def expert_bytes(w, A: float) -> float:
    """W1 and W2 of A experts, read once: elements at the layer's width; FP8:
    one byte each plus a float32 scale per row; MXFP4: half a byte each plus
    a scale byte per 32."""
    if w.experts == "fp8":
        return A * (2 * w.l * w.m + 4 * (w.l + w.m))
    if w.experts == "mxfp4":   # half a byte per code, a scale byte per 32 elements
        return A * 2 * w.l * w.m * (0.5 + 1.0 / 32)
    return A * 2 * w.l * w.m * w.elem_bytes


def algorithmic(w, A: float, R: float):
    """Whole-layer algorithmic bytes and flops (A = FFN experts that got rows,
    R = (token, rank) pairs routed to FFN experts: T*K without
    zero-computation experts)."""
    B = w.elem_bytes
    lat = 0 if w.standard else 1
    Nr = w.N + w.n_zc
    nbytes = B * (2 * w.T * w.d + lat * 2 * w.d * w.l + w.d * Nr + 2 * w.d * w.m_shared + w.n_const * w.l) \
        + expert_bytes(w, A) + (4 * Nr if w.bias else 0)
    flops = lat * 4 * w.T * w.d * w.l + 2 * w.T * w.d * Nr + 4 * R * w.l * w.m + 4 * w.T * w.d * w.m_shared
    return nbytes, flops


ARGS = None


def main():
    global ARGS
    args = ARGS = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the layer is not sharded "
                                   "across GPUs",
                          "n_gpus_requested": max(args.gpus, world)}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_moe_layer_gemm_amd import binding as B
    from sparse_moe_layer_gemm_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.lib()

    def draw_sets(wk, n=None):
        sets = []
        for s in range(max(1, args.weight_sets if n is None else n)):
            inp = make_inputs(wk, seed=s)
            sets.append((inp, {k: (None if v is None else v.to(dev)) for k, v in inp.items()}))
        return sets

    if args.sweep:
        counts = [int(t) for t in args.sweep.split(",") if t.strip()]
        base = draw_sets(w.replace(T=max(counts)))
        for T in counts:
            wt = w.replace(name=f"{w.name}_T{T}", T=T)
            sets = [({**c, "x": c["x"][:T]}, {**g, "x": g["x"][:T].contiguous()}) for c, g in base]
            print(json.dumps(measure(wt, sets, 0.0)), flush=True)
        return
    line = measure(w, draw_sets(w), args.cpu_seconds)
    # The MFMA-bound workloads, measured in the same run (shorter: one weight
    # set, no oracle, no yardsticks), so that one JSON line carries their step
    # time, tokens/s and roofline fractions too.
    extra = [e.strip() for e in args.extra.split(",") if e.strip()]
    if extra:
        line["extra_workloads"] = {}
    for name in extra:
        we = WORKLOADS[name]
        rec = measure(we, draw_sets(we, 1), 0.0, steps=min(args.steps, 10), warmup=min(args.warmup, 3),
                      references=False)
        line["extra_workloads"][name] = {
            "tokens_per_s": rec["value"], "ms_per_step": rec["ms_per_step"], "steps": rec["steps"],
            "ffn_path": rec["config"]["ffn_path"],
            "roofline": {k: rec["roofline"][k] for k in ("kernel", "bound", "achieved", "peak", "unit", "frac",
                                                          "kernel_us", "traffic", "layer_frac")},
            "stage_us": rec["layer"]["stage_us"], "active_experts": rec["layer"]["active_experts"]}
        torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)


def measure(w, sets, cpu_seconds: float, steps=None, warmup=None, references: bool = True) -> dict:
    """One JSON record: w's forward timed over `sets` (CPU and device copies
    of the inputs, alternating between steps); `steps` / `warmup` default to
    the command line's.  references: also time the in-run HBM and MFMA
    yardsticks (device copy, streaming read, library GEMM)."""
    import numpy as np
    import torch

    from sparse_moe_layer_gemm_amd import binding as B

    args = ARGS
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    dev = torch.device("cuda:0")
    dims = B.dims_for(sets[0][1], w.K, args.path, w.n_zero, w.n_copy)
    path = B.latentmoe_resolved_path(dims, w.K)
    ws = B.alloc_workspace(dims, w.K, dev)
    out = torch.empty_like(sets[0][1]["x"])
    stream = torch.cuda.current_stream()
    hip = Hip()
    nst = B.LMOE_N_STAGE_EVENTS

    def step(i, events=None):
        d = sets[i % len(sets)][1]
        B.latentmoe_forward(d["x"], d["W_down"], d["W_router"], d["W1"], d["W2"], d["W_up"], w.K, out, dims,
                            router_bias=d["bias"], workspace=ws, stream=stream, events=events,
                            W_shared1=d.get("W_s1"), W_shared2=d.get("W_s2"),
                            W1_scale=d.get("W1_scale"), W2_scale=d.get("W2_scale"), zc_const=d.get("zc_const"))

    # active FFN experts and FFN rows per weight set (for the algorithmic
    # counts), from the routed ids
    active, rows = [], []
    ids_t = torch.empty(w.T, w.K, dtype=torch.int32, device=out.device)
    for i in range(len(sets)):
        d = sets[i][1]
        B.latentmoe_forward(d["x"], d["W_down"], d["W_router"], d["W1"], d["W2"], d["W_up"], w.K, out, dims,
                            router_bias=d["bias"], topk_ids=ids_t, workspace=ws, stream=stream,
                            W_shared1=d.get("W_s1"), W_shared2=d.get("W_s2"),
                            W1_scale=d.get("W1_scale"), W2_scale=d.get("W2_scale"), zc_const=d.get("zc_const"))
        torch.cuda.synchronize()
        ffn_ids = ids_t.cpu().numpy().ravel()
        ffn_ids = ffn_ids[ffn_ids < w.N]   # FFN experts (zero-computation ids come after)
        active.append(int(np.unique(ffn_ids).size))
        rows.append(int(ffn_ids.size))
    A = float(np.mean(active))
    R = float(np.mean(rows))

    for i in range(warmup):
        step(i)
    # Timed region: the whole forward, with HIP events recorded on the launch
    # stream only around the expert FFN (the dominant kernel).
    # the FFN: stage 3 on the streaming path (its events are then the
    # kernel's own start and end), stages 3 and 4 (two kernels) otherwise
    ffn_end = 4 if path == B.LMOE_PATH_STREAM else 5
    ev_ffn = None
    if not args.no_events:
        ev_ffn = []
        for _ in range(steps):
            arr = (ctypes.c_void_p * nst)()
            arr[3], arr[ffn_end] = hip.event(), hip.event()
            ev_ffn.append(arr)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i, ev_ffn[i] if ev_ffn else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    tok_s = w.T / (ms * 1e-3)
    ffn_us = float("nan")
    if ev_ffn:
        ffn_us = float(np.mean([hip.elapsed_ms(ev[3], ev[ffn_end]) for ev in ev_ffn])) * 1e3

    # Stage breakdown (a separate pass with an event at every stage boundary).
    stages = {}
    if not args.no_events:
        ev_all = [(ctypes.c_void_p * nst)(*[hip.event() for _ in range(nst)]) for _ in range(steps)]
        for i in range(steps):
            step(i, ev_all[i])
        torch.cuda.synchronize()
        for si, name in enumerate(B.STAGES):
            stages[name] = float(np.mean([hip.elapsed_ms(ev[si], ev[si + 1]) for ev in ev_all])) * 1e3
    copy_gbs = copy_bandwidth(torch, dev) if references else None
    read_gbs = read_bandwidth(torch, dev) if references else None
    mm_tflops = matmul_rate(torch, dev) if references and w.dtype == "bf16" else None
    lay_bytes, lay_flops = algorithmic(w, A, R)

    # dominant kernel: the expert FFN
    if path == B.LMOE_PATH_STREAM:
        ffn_bytes = expert_bytes(w, A)
        # MXFP4 with 128-wide slices (m % 128 == 0), l % 256 == 0: its own kernel
        mx16 = w.experts == "mxfp4" and w.m % 128 == 0 and w.l % 256 == 0
        roof = {"kernel": "ffn_stream_mx_kernel" if mx16 else "ffn_stream_kernel", "bound": "hbm", "achieved": ffn_bytes / (ffn_us * 1e-6) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": None}
    elif w.dtype == "f32":
        ffn_flops = 4.0 * R * w.l * w.m
        roof = {"kernel": "gemm_simt_kernel<Ffn1>+<Ffn2>", "bound": "alu",
                "achieved": ffn_flops / (ffn_us * 1e-6) / 1e12, "peak": FP32_VECTOR_PEAK_TFLOPS,
                "unit": "TFLOP/s", "traffic": None}
    else:
        # FP8 / MXFP4 weights are decoded to bf16 on the way into LDS: the
        # products run on the bf16 MFMAs, so the bf16 peak is the compute
        # bound.  The FFN's bound is the one its arithmetic intensity (flops
        # over the active experts' weight bytes, read once) puts it under.
        ffn_flops = 4.0 * R * w.l * w.m
        ffn_bytes = expert_bytes(w, A)
        q = {"dense": "", "fp8": "Q", "mxfp4": "X"}[w.experts]
        kern = f"gemm2_kernel<Ffn1{q}>+<Ffn2{q}>"
        if ffn_flops / ffn_bytes >= MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
            roof = {"kernel": kern, "bound": "mfma", "achieved": ffn_flops / (ffn_us * 1e-6) / 1e12,
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "traffic": None}
        else:
            roof = {"kernel": kern, "bound": "hbm", "achieved": ffn_bytes / (ffn_us * 1e-6) / 1e9,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": None}
        roof["arithmetic_intensity"] = ffn_flops / ffn_bytes
    roof["traffic"] = measured_traffic(w, roof["kernel"])
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel_us"] = ffn_us
    roof["copy_GBps_measured"] = copy_gbs
    roof["read_GBps_measured"] = read_gbs
    roof["matmul_TFLOPs_measured"] = mm_tflops
    flop_peak = FP32_VECTOR_PEAK_TFLOPS if w.dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
    layer_frac = max(lay_bytes / (HBM_PEAK_GBS * 1e9), lay_flops / (flop_peak * 1e12)) / (ms * 1e-3)
    roof["layer_frac"] = layer_frac

    cpu = None
    if cpu_seconds > 0:
        cpu = cpu_baseline(w, sets[0][0], cpu_seconds)

    line = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "l": w.l, "N": w.N, "K": w.K, "m": w.m,
                   "m_shared": w.m_shared, "experts": w.experts, "n_zero": w.n_zero, "n_copy": w.n_copy,
                   "n_const": w.n_const, "standard": w.standard, "bias": w.bias, "weight_sets": len(sets),
                   "ffn_path": "stream" if path == B.LMOE_PATH_STREAM else "tiled",
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "layer": {"algorithmic_bytes": lay_bytes, "algorithmic_flops": lay_flops, "active_experts": A,
                  "ffn_rows": R,
                  "roofline_frac": layer_frac, "stage_us": stages},
    }
    return line


def measured_traffic(w, kernel: str):
    """HBM bytes per launch of `kernel` (the FFN: one streaming kernel, or the
    two tiled GEMMs together) from the committed rocprofv3 counter summary
    profiles/<kernel>_<workload>_traffic.json (FETCH_SIZE + WRITE_SIZE, each
    scaled by the same counter on a copy of known size), or None when there
    is none for this workload or the kernel's sources changed since the
    counters were taken."""
    import hashlib

    tag = "ffn_stream" if kernel.startswith("ffn_stream") else "gemm2_ffn"
    path = os.path.join(ROOT, "profiles", f"{tag}_{w.name}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel") != kernel or rec.get("workload") != w.name:
        return None
    h = hashlib.sha256(b"".join(open(os.path.join(ROOT, p), "rb").read() for p in rec["sources"])).hexdigest()
    return rec["traffic_bytes_per_launch"] if h == rec["sources_sha256"] else None


def matmul_rate(torch, dev, n: int = 8192, reps: int = 10) -> float:
    """In-run MFMA reference: a large bf16 library GEMM (torch.matmul, n^3),
    flops / s in TFLOP/s.  A yardstick for the tiled kernels, not part of the
    layer."""
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    c = torch.matmul(a, b)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        c = torch.matmul(a, b)
    t1.record()
    torch.cuda.synchronize()
    rate = 2.0 * n ** 3 * reps / (t0.elapsed_time(t1) * 1e-3) / 1e12
    del a, b, c
    return rate


def copy_bandwidth(torch, dev, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """In-run HBM reference: a device-to-device copy, (read + write) bytes / s."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    return gbs


def read_bandwidth(torch, dev, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """In-run HBM reference: the streaming-read kernel of libhbmread.so over
    1 GiB (every byte read once, each workgroup a contiguous share with eight
    16-byte loads in flight per thread, nothing written), the best of a few
    grid sizes, bytes read / s."""
    from sparse_moe_layer_gemm_amd import build as hipbuild

    lib = ctypes.CDLL(hipbuild.PROBE_LIB)
    lib.hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    best = 0.0
    for per_cu in (2, 4, 8):
        def run():
            rc = lib.hbm_read(src.data_ptr(), nbytes, sink.data_ptr(), cus * per_cu, stream)
            if rc != 0:
                raise RuntimeError(f"hbm_read failed: {rc}")
        run()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            run()
        b.record()
        torch.cuda.synchronize()
        best = max(best, nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src, sink
    return best


def cpu_baseline(w, inp, budget_s: float):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload."""
    import numpy as np

    from oracle import oracle as O
    from sparse_moe_layer_gemm_amd.inputs import as_numpy_bits

    arr = {k: (None if v is None else (v.numpy() if k == "bias" else as_numpy_bits(v))) for k, v in inp.items()}
    orc = O.default()
    n = 0
    t0 = time.perf_counter()
    chunk = min(w.T, 64)
    passes = 0
    while True:
        sel = np.arange(n % w.T, n % w.T + chunk, dtype=np.int32) % w.T
        orc.forward(arr["x"], arr["W_down"], arr["W_router"], arr["W1"], arr["W2"], arr["W_up"], w.K,
                    bias=arr["bias"], standard=w.standard, sel=sel, W_s1=arr.get("W_s1"), W_s2=arr.get("W_s2"),
                    W1_scale=arr.get("W1_scale"), W2_scale=arr.get("W2_scale"),
                    n_zero=w.n_zero, n_copy=w.n_copy, zc_const=arr.get("zc_const"))
        n += chunk
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": n / el, "unit": "tokens/s", "cores": orc.threads(), "kind": "oracle",
            "sample": f"{n} tokens ({passes} calls of {chunk} tokens) of the {w.name} workload, weight set 0, "
                      f"{el:.1f} s"}


if __name__ == "__main__":
    main()
