"""Benchmark of the exact-attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one fa_fwd call over one batch of the named workload (inputs already
resident in HBM). The timed region is K back-to-back calls between two HIP
events recorded on the stream the kernel is launched on, bracketed by device
synchronisation. Before it come W untimed warmup calls and then further untimed
calls until --settle-ms have passed, so the GPU clock has settled. One JSON
line is printed. The default workload is the batched
80x80-map YOLO attention (B=16, H=4, N=6400, d=32, fp16, non-causal); the
metric also names microseconds per call at N=400, which is measured on the
20x20-map workload in the same run.

Beside the headline workload, the line carries a record for every named
workload (time, TFLOP/s and fraction of the matrix peak, algorithmic and
measured HBM bytes), the FP8 forward on the two long workloads, the standard
(unfused) attention against the fused forward on the 2048-token workload, and
the vector-unit rates of exp2 and FMA with the vector-unit bound they set on
the d = 32 workload. The FP8 records cover the three workloads of 2048 tokens
and more. The backward pass is timed on the headline workload (`backward`) and
on the other two long workloads (`backward_workloads`); the matrix-rate,
co-execution and co-issue probes report what the matrix and vector units reach
on their own and together.

The CPU baseline times the fp64 oracle, unmodified, on the host's cores: one
worker process per core (at most 16), BLAS at one thread each, over whole
heads of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % MFMA peak; µs/call at N=400 and N=6400"
# MI355X dense fp16/bf16 matrix peak: 256 CUs x 4096 FLOP/clk x 2.4 GHz.
PEAK_MFMA_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
# MI355X dense fp8 matrix peak (twice the fp16 rate)
PEAK_MFMA_FP8_TFLOPS = 5033.2
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_23_amd", "csrc", f)
                  for f in ("fa_device.hpp", "fa_fwd16.hpp", "fa_fwd_kernel.hpp", "fa_fwd_short.hpp",
                            "fa_api.hip", "fa_host.hpp")]
BWD_KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_23_amd", "csrc", f)
                      for f in ("fa_device.hpp", "fa_bwd_kernel.hpp", "fa_bwd.hip", "fa_host.hpp")]
FP8_KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_23_amd", "csrc", f)
                      for f in ("fa_device.hpp", "fa_fwd_kernel.hpp", "fa_fwd_fp8.hpp", "fa_fp8.hip",
                                "fa_host.hpp")]
STD_KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_23_amd", "csrc", f)
                      for f in ("fa_device.hpp", "fa_std_kernel.hpp", "fa_std.hip")]
STD_KERNELS = ("fa_std_scores_kernel", "fa_std_softmax_kernel", "fa_std_pv_kernel")
# backward kernels as rocprofv3 names them, and the FA_BWD_* bit of each
BWD_KERNELS = (("pre", "fa_bwd_pre_kernel", 1), ("dkdv", "fa_bwd_dkdv_kernel", 2),
               ("dq", "fa_bwd_dq_kernel", 4))


def _code_only(text: str) -> str:
    """Source text without comments and blank lines, so that an edit of the
    comments alone does not mark the profiled kernel as changed."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    out = []
    for line in text.splitlines():
        line = re.sub(r"//.*$", "", line).rstrip()
        if line.strip():
            out.append(line)
    return "\n".join(out)


def kernel_source_hash(sources=None) -> str:
    """Hash of the code (comments stripped) of a kernel's source files."""
    h = hashlib.sha256()
    for p in (sources or KERNEL_SOURCES):
        with open(p, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(key: str, sources=None):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE runs,
    or None when absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get("workloads", {}).get(key)
    if not ent or ent.get("kernel_source_sha") != kernel_source_hash(sources):
        return None
    return ent.get("hbm_bytes_per_launch")


def layout_inputs(w, layout: str, dev):
    """q, k, v of w on the device as [B, H, N, d] tensors in a memory layout:
    "bhnd" contiguous, "bnhd" sequence-major views, "qkv" views of one fused
    [B, N, 3, H, d] buffer (Nq == Nk); plus an output of the matching layout."""
    import torch

    from workloads import make_inputs

    q, k, v = make_inputs(w)
    if layout == "bhnd":
        q, k, v = (t.to(dev) for t in (q, k, v))
        return q, k, v, torch.empty_like(q)
    if layout == "bnhd":
        q, k, v = (t.transpose(1, 2).contiguous().to(dev).transpose(1, 2) for t in (q, k, v))
    elif layout == "qkv":
        qkv = torch.stack([t.transpose(1, 2) for t in (q, k, v)], dim=2).contiguous().to(dev)
        q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    else:
        raise ValueError(layout)
    o = torch.empty((w.B, w.Nq, w.H, w.d), dtype=q.dtype, device=dev).transpose(1, 2)
    return q, k, v, o


def time_gpu(w, steps: int, warmup: int, settle_ms: float = 300.0, layout: str = "bhnd"):
    import torch

    import exact_attention_23_amd as fa

    dev = torch.device("cuda:0")
    q, k, v, o = layout_inputs(w, layout, dev)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        fa.attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    # The GPU clock takes a few hundred ms of load to settle: keep issuing
    # untimed calls until settle_ms have passed (the first calls of a cold GPU
    # run about 15% slower).
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(8):
            fa.attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)  # the stream fa_fwd launches on
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        fa.attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    if not torch.isfinite(o.float()).all():
        raise RuntimeError("non-finite output in the timed run")
    return ms


def time_fp8(w, steps: int, warmup: int, settle_ms: float = 300.0):
    """ms per FP8 forward call on w's inputs quantised to e4m3 (bf16 output)."""
    import torch

    import exact_attention_23_amd as fa
    from workloads import make_inputs_fp8

    dev = torch.device("cuda:0")
    q8, k8, v8, sq, sk, sv = make_inputs_fp8(w)
    q8, k8, v8 = (t.to(dev) for t in (q8, k8, v8))
    o = torch.empty((w.B, w.H, w.Nq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)

    def call():
        fa.attention_fp8(q8, k8, v8, sq, sk, sv, causal=w.causal, scale=w.scale, out=o, lse=lse)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(8):
            call()
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        call()
    ev1.record()
    torch.cuda.synchronize()
    if not torch.isfinite(o.float()).all():
        raise RuntimeError("non-finite output in the timed run")
    return ev0.elapsed_time(ev1) / steps


def launch_floor_us(calls: int = 100, replays: int = 20) -> float:
    """Device time per call of a trivial kernel (one-element add) from a
    replayed HIP graph of `calls` launches: the launch floor that the short
    sequences' device times sit on."""
    import torch

    x = torch.zeros(1, device="cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        x.add_(1.0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            x.add_(1.0)
    graph.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(replays):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) * 1e3 / (replays * calls)


def clock_under_load(w, seconds_cap: float = 15.0):
    """The engine clocks (MHz, mean/min/max over the XCDs) that `amd-smi
    metric --clock` reports while w's forward runs back to back, or None when
    the tool is unavailable. The reading is a snapshot taken once the load has
    run for a moment."""
    import shutil
    import subprocess
    import threading

    import torch

    import exact_attention_23_amd as fa

    tool = shutil.which("amd-smi")
    if tool is None:
        return None
    result = {}

    def sample():
        time.sleep(0.5)
        try:
            r = subprocess.run([tool, "metric", "--clock", "--json"], capture_output=True, text=True,
                               timeout=seconds_cap)
            data = json.loads(r.stdout)
            gpu = data["gpu_data"][0] if isinstance(data, dict) else data[0]
            clk = [v["clk"]["value"] for k, v in gpu["clock"].items() if k.startswith("gfx_")]
            result["mhz"] = [float(x) for x in clk if isinstance(x, (int, float))]
        except Exception as e:  # noqa: BLE001 - report the clock as unknown
            result["error"] = str(e)

    dev = torch.device("cuda:0")
    q, k, v, o = layout_inputs(w, "bhnd", dev)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    th = threading.Thread(target=sample, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while th.is_alive() and time.perf_counter() - t0 < seconds_cap:
        for _ in range(8):
            fa.attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
        torch.cuda.synchronize()
    th.join(timeout=1.0)
    mhz = result.get("mhz")
    if not mhz:
        return None
    return {"mean": round(sum(mhz) / len(mhz), 1), "min": min(mhz), "max": max(mhz),
            "xcds": len(mhz), "tool": "amd-smi metric --clock (snapshot under load)"}


def time_graph(w, calls: int = 100, replays: int = 20):
    """Device time per call (µs) with the host's launch cost taken out: `calls`
    back-to-back calls captured in one HIP graph, replayed `replays` times
    between two events. The result of the last replay is checked bit for bit
    against an eager call (the kernel is deterministic)."""
    import torch

    import exact_attention_23_amd as fa
    from workloads import make_inputs

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fa.attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            fa.attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(replays):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / (replays * calls)
    o_ref, lse_ref = fa.attention(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    if not (torch.equal(o, o_ref) and torch.equal(lse, lse_ref)):
        raise RuntimeError("graph replay disagrees with an eager call")
    return us


class _Bwd:
    """Device buffers and the raw fa_bwd_ex call for one workload: inputs, the
    forward's O and LSE, an upstream gradient, gradients and workspace."""

    def __init__(self, w):
        import torch

        import exact_attention_23_amd as fa
        from workloads import make_grad, make_inputs

        dev = torch.device("cuda:0")
        self.w = w
        self.q, self.k, self.v = (t.to(dev) for t in make_inputs(w))
        self.do = make_grad(w).to(dev)
        self.o, self.lse = fa.attention(self.q, self.k, self.v, causal=w.causal, scale=w.scale)
        self.dq, self.dk, self.dv = (torch.empty_like(t) for t in (self.q, self.k, self.v))
        self.lib = fa._lib.load()
        nbytes = self.lib.fa_bwd_workspace_bytes(w.B, w.H, w.Nq)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.args = (self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.o.data_ptr(),
                     self.do.data_ptr(), self.lse.data_ptr(), self.dq.data_ptr(),
                     self.dk.data_ptr(), self.dv.data_ptr(), self.ws.data_ptr(), nbytes,
                     w.B, w.H, w.Nq, w.Nk, w.d, float(w.scale), 1 if w.causal else 0,
                     fa._dtype_code(self.q))
        self.stream = fa._current_stream(0)
        self.fa = fa

    def __call__(self, mask: int = 7):
        st = self.lib.fa_bwd_ex(*self.args, mask, self.stream)
        if st != 0:
            raise RuntimeError(f"fa_bwd_ex failed: {self.fa.status_str(st)}")


def time_bwd(w, steps: int, warmup: int, settle_ms: float = 300.0):
    """Backward pass of w: ms per whole call (three kernels) and the average
    duration of each kernel alone (HIP events around `steps` launches of that
    kernel only, on the stream the library launches on)."""
    import torch

    b = _Bwd(w)
    for _ in range(warmup):
        b()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(4):
            b()
        torch.cuda.synchronize()

    def timed(mask):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(steps):
            b(mask)
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps

    ms = timed(7)
    per = {name: timed(bit) for name, _, bit in BWD_KERNELS}
    for t in (b.dq, b.dk, b.dv):
        if not torch.isfinite(t.float()).all():
            raise RuntimeError("non-finite gradient in the timed run")
    return ms, per


def bwd_record(w, ms: float, per: dict):
    """Backward figures of w: whole-pass TFLOP/s over the five products of
    the gradient definition (10*B*H*Nq*Nk*d, halved when causal) and the
    roofline of the dominant kernel."""
    flops_total = 2.5 * w.flops()
    # products each kernel computes: dK/dV forms S, dP, dV, dK; dQ forms S
    # and dP again and dQ (only dQ is new work); the D/LSE pass is bytes
    dom = max(("dkdv", "dq"), key=lambda n: per[n])
    dom_flops = {"dkdv": 2.0 * w.flops(), "dq": 1.5 * w.flops()}[dom]
    achieved = dom_flops / (per[dom] * 1e-3) / 1e12
    kname = dict((n, k) for n, k, _ in BWD_KERNELS)[dom]
    tflops = flops_total / (ms * 1e-3) / 1e12
    return {
        "value": round(tflops, 3), "unit": "TFLOP/s", "ms_per_step": round(ms, 6),
        "mfma_peak_frac": round(tflops / PEAK_MFMA_TFLOPS, 4),
        "kernels_us": {n: round(per[n] * 1e3, 3) for n in per},
        "roofline": {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 3),
                     "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_MFMA_TFLOPS, 4),
                     "traffic": measured_traffic(f"bwd:{w.name}", BWD_KERNEL_SOURCES)},
        "kernel_source_sha": kernel_source_hash(BWD_KERNEL_SOURCES),
    }


def short_stats(w, calls: int = 200):
    """Latency-bound sizes: device time per call (HIP graph of 100 calls),
    the eager rate, and the algorithmic HBM rate against the 8 TB/s peak.
    The launch_plus_event_* figures come from individually event-timed eager
    calls: they measure the launch and the event pair around each call, not
    the kernel (its device time is us_per_call_device)."""
    import statistics

    import torch

    import exact_attention_23_amd as fa

    dev_us = time_graph(w)
    eager_us = time_gpu(w, 100, 10, 100.0) * 1e3
    dev = torch.device("cuda:0")
    q, k, v, o = layout_inputs(w, "bhnd", dev)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(calls)]
    for e0, e1 in evs:
        e0.record()
        fa.attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)
        e1.record()
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    gbs = w.algorithmic_bytes() / (dev_us * 1e-6) / 1e9
    return {"us_per_call_device": round(dev_us, 3), "us_per_call_eager": round(eager_us, 3),
            "launch_plus_event_p50_us": round(t[len(t) // 2], 3),
            "launch_plus_event_p95_us": round(t[int(len(t) * 0.95)], 3),
            "launch_plus_event_std_over_mean": round(statistics.pstdev(t) / statistics.fmean(t), 4),
            "algorithmic_hbm_gbs": round(gbs, 1),
            "hbm_peak_frac": round(gbs / PEAK_HBM_GBS, 5),
            "tflops": round(w.flops() / (dev_us * 1e-6) / 1e12, 3)}


def cpu_baseline_bwd(w, budget_s: float = 12.0):
    """The gradient oracle on whole heads of w until ~budget_s of CPU time."""
    import numpy as np

    import oracle
    from workloads import make_grad, make_inputs

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    q, k, v = make_inputs(w)
    do = make_grad(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    order = [heads[i] for i in np.random.default_rng(0).permutation(len(heads))]
    done = 0
    t0 = time.perf_counter()
    for (b, h) in order:
        oracle.attention_backward_head(q[b, h], k[b, h], v[b, h], do[b, h], w.scale, w.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 2.5 * w.flops() * done / len(heads)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {len(heads)} heads (whole heads) of {w.name}, backward; "
                      f"{dt:.1f} s wall; numpy float64"}


def cpu_baseline(w, budget_s: float = 20.0):
    """The oracle, unmodified, on whole heads of w: one worker process per host
    core (at most 16), BLAS at one thread each, heads taken 16 at a time until
    all are done or budget_s has passed. The pool is started and warmed before
    the clock starts."""
    import numpy as np

    from oracle import pool
    from workloads import make_inputs

    q, k, v = make_inputs(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    order = [heads[i] for i in np.random.default_rng(0).permutation(len(heads))]
    with pool.make_executor() as ex:
        workers = ex._max_workers  # noqa: SLF001
        pool.warm(ex)
        done = 0
        t0 = time.perf_counter()
        while done < len(order) and time.perf_counter() - t0 < budget_s:
            chunk = order[done:done + workers]
            pool.attention_heads(q, k, v, chunk, scale=w.scale, causal=w.causal, executor=ex)
            done += len(chunk)
        dt = time.perf_counter() - t0
    flops = w.flops() * done / len(heads)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(workers), "kind": "oracle",
            "cpu_model": pool.cpu_model(), "host_cores_available": pool.host_cores(),
            "sample": f"{done} of {len(heads)} heads (whole heads, all {w.Nq} query rows) of "
                      f"{w.name}; {dt:.1f} s wall; numpy float64, {workers} worker processes, "
                      f"BLAS at one thread each"}


def workload_record(w, steps: int, warmup: int, settle_ms: float):
    """One named workload's forward: device time per call (events over `steps`
    back-to-back calls; a replayed HIP graph for the latency-bound sizes),
    TFLOP/s and fraction of the matrix peak, algorithmic and counter-measured
    HBM bytes, the latter only when taken on the current kernel source."""
    latency_bound = w.B * w.H * w.Nq * w.Nk < 10_000_000
    us = time_graph(w) if latency_bound else time_gpu(w, steps, warmup, settle_ms) * 1e3
    tflops = w.flops() / (us * 1e-6) / 1e12
    gbs = w.algorithmic_bytes() / (us * 1e-6) / 1e9
    traffic = measured_traffic(w.name)
    rec = {"B": w.B, "H": w.H, "N": w.Nq, "d": w.d, "dtype": w.dtype, "causal": w.causal,
           "us_per_call": round(us, 3),
           "timing": "device time per call of a replayed HIP graph" if latency_bound
           else f"HIP events over {steps} back-to-back calls",
           "tflops": round(tflops, 3), "mfma_peak_frac": round(tflops / PEAK_MFMA_TFLOPS, 4),
           "algorithmic_bytes": w.algorithmic_bytes(), "algorithmic_gbs": round(gbs, 1),
           "hbm_peak_frac": round(gbs / PEAK_HBM_GBS, 5),
           "traffic_bytes": traffic,
           "traffic_over_algorithmic": None if traffic is None else round(traffic / w.algorithmic_bytes(), 3)}
    return rec


def fp8_record(w, steps: int, warmup: int, settle_ms: float):
    ms = time_fp8(w, steps, warmup, settle_ms)
    tflops = w.flops() / (ms * 1e-3) / 1e12
    return {"us_per_call": round(ms * 1e3, 3), "tflops": round(tflops, 3),
            "fp8_mfma_peak_frac": round(tflops / PEAK_MFMA_FP8_TFLOPS, 4),
            "traffic_bytes": measured_traffic(f"fp8:{w.name}", FP8_KERNEL_SOURCES),
            "kernel_source_sha": kernel_source_hash(FP8_KERNEL_SOURCES)}


def std_vs_fused(w, steps: int = 10, warmup: int = 3):
    """The standard (unfused) attention against the fused forward on w: ms per
    call of each, their ratio, and the HBM bytes of each path, algorithmic
    (the fused forward reads Q, K, V and writes O and LSE once; the standard
    path also writes and reads S in fp32 and P in the input type) and, when
    taken on the current sources, measured by the counters."""
    import torch

    import exact_attention_23_amd as fa
    from workloads import make_inputs

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_inputs(w))
    lib = fa._lib.load()
    nkp = lib.fa_std_row_stride(w.Nk)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    sbuf = torch.empty((w.B, w.H, w.Nq, nkp), dtype=torch.float32, device=dev)
    pbuf = torch.empty((w.B, w.H, w.Nq, nkp), dtype=q.dtype, device=dev)
    stream = fa._current_stream(0)
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), sbuf.data_ptr(),
            pbuf.data_ptr(), w.B, w.H, w.Nq, w.Nk, w.d, float(w.scale), 1 if w.causal else 0,
            fa._dtype_code(q))

    def std_call():
        st = lib.fa_std_fwd(*args, stream)
        if st != 0:
            raise RuntimeError(fa.status_str(st))

    for _ in range(warmup):
        std_call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        std_call()
    ev1.record()
    torch.cuda.synchronize()
    std_ms = ev0.elapsed_time(ev1) / steps
    o_std = o.clone()
    fused_ms = time_gpu(w, 4 * steps, warmup, 200.0)
    o_f, _ = fa.attention(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    diff = float((o_f.float() - o_std.float()).abs().max())
    del sbuf, pbuf
    es = 2
    s_bytes = w.B * w.H * w.Nq * nkp * 4
    p_bytes = w.B * w.H * w.Nq * nkp * es
    std_alg = w.algorithmic_bytes() + 2 * s_bytes + 2 * p_bytes
    return {"workload": w.name, "fused_us": round(fused_ms * 1e3, 3), "standard_us": round(std_ms * 1e3, 3),
            "standard_over_fused": round(std_ms / fused_ms, 3),
            "max_abs_diff_of_outputs": diff,
            "algorithmic_bytes": {"fused": w.algorithmic_bytes(), "standard": std_alg},
            "standard_passes_over_nq_nk": "S written (fp32), S read, P written (input type), P read",
            "measured_bytes": {"fused": measured_traffic(w.name),
                               "standard": measured_traffic(f"std:{w.name}", STD_KERNEL_SOURCES)},
            "standard_kernel_source_sha": kernel_source_hash(STD_KERNEL_SOURCES)}


def vector_rates(iters: int = 4096, blocks: int = 256 * 16):
    """Chip-wide rates of v_exp_f32, v_fma_f32 and FMA-then-exp2 pairs (the
    softmax's work per score) from libfa_probe.so: instructions per second
    and lanes per clock per compute unit at the published 2.4 GHz."""
    import ctypes

    import torch

    import exact_attention_23_amd as fa
    from exact_attention_23_amd import build

    lib = ctypes.CDLL(build.PROBE_LIB_PATH)
    lib.fa_probe_vector_rate.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_probe_vector_rate.restype = ctypes.c_int
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    stream = fa._current_stream(0)
    res = {}
    for name, op in (("exp2", 0), ("fma", 1), ("fma_exp2_pair", 2)):
        for _ in range(2):  # warm up the clock
            assert lib.fa_probe_vector_rate(op, blocks, iters, 8, out.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        reps = 3
        for _ in range(reps):
            assert lib.fa_probe_vector_rate(op, blocks, iters, 8, out.data_ptr(), stream) == 0
        ev1.record()
        torch.cuda.synchronize()
        sec = ev0.elapsed_time(ev1) * 1e-3 / reps
        instr = blocks * 4 * iters * 8  # wave64 instructions (4 waves per workgroup)
        res[name] = {"wave_instr_per_s": instr / sec,
                     "lanes_per_clk_per_cu_at_2p4ghz": round(instr * 64 / sec / (256 * 2.4e9), 2)}
    if not torch.isfinite(out).all():
        raise RuntimeError("probe produced non-finite values")
    return res


def _probe_lib():
    import ctypes

    from exact_attention_23_amd import build

    lib = ctypes.CDLL(build.PROBE_LIB_PATH)
    lib.fa_probe_matrix_rate.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_probe_matrix_rate.restype = ctypes.c_int
    lib.fa_probe_coexec.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_probe_coexec.restype = ctypes.c_int
    lib.fa_probe_coissue.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_probe_coissue.restype = ctypes.c_int
    return lib


def _time_launches(launch, reps: int = 3) -> float:
    """Seconds per call of launch() (two warm-up calls, then `reps` timed)."""
    import torch

    for _ in range(2):
        launch()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        launch()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) * 1e-3 / reps


def matrix_rate(iters: int = 4096, blocks: int = 256 * 2):
    """The rate of the matrix instructions alone (independent accumulator
    chains, two waves per SIMD) from libfa_probe.so, for the 32x32x16 shape
    and the 16x16x32 shape the tiled forward uses: what an attention kernel
    built on them can reach on this chip, against the published dense fp16
    peak."""
    import torch

    import exact_attention_23_amd as fa

    lib = _probe_lib()
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    stream = fa._current_stream(0)
    res = {}
    for name, shape in (("v_mfma_f32_32x32x16_f16", 0), ("v_mfma_f32_16x16x32_f16", 1)):
        def launch(shape=shape):
            assert lib.fa_probe_matrix_rate(shape, blocks, iters, out.data_ptr(), stream) == 0

        sec = _time_launches(launch)
        if not torch.isfinite(out).all():
            raise RuntimeError("matrix probe produced non-finite values")
        tflops = blocks * 4 * iters * 131072 / sec / 1e12
        res[name] = {"tflops": round(tflops, 1), "frac_of_published_peak": round(tflops / PEAK_MFMA_TFLOPS, 4)}
    return res


def coexec(matrix_iters: int = 2048, vector_iters: int = 2048, blocks: int = 256):
    """Whether the SIMDs overlap matrix and vector work of different waves
    (libfa_probe.so's fa_probe_coexec): one wave per SIMD runs matrix chains,
    another the softmax's vector steps; timed alone and together. both/sum
    near 1 means the two kinds of work take turns, both/max near 1 that they
    overlap."""
    import torch

    import exact_attention_23_amd as fa

    lib = _probe_lib()
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda:0")
    stream = fa._current_stream(0)
    us = {}
    for name, roles in (("matrix_only", 1), ("vector_only", 2), ("both", 3)):
        def launch(roles=roles):
            assert lib.fa_probe_coexec(roles, blocks, matrix_iters, vector_iters, out.data_ptr(), stream) == 0

        us[name] = round(_time_launches(launch) * 1e6, 1)
        if not torch.isfinite(out).all():
            raise RuntimeError("co-execution probe produced non-finite values")
    m, v, b = us["matrix_only"], us["vector_only"], us["both"]
    return {"us": us, "both_over_sum": round(b / (m + v), 3), "both_over_max": round(b / max(m, v), 3)}


def coissue(iters: int = 2000, cus: int = 256):
    """How far one wave's own matrix and vector instructions overlap
    (libfa_probe.so's fa_probe_coissue), at one, two and four waves per SIMD:
    per step 16 16x16x32 matrix instructions and the softmax's vector work on
    32 values, timed alone, together in the compiler's order, and together
    interleaved one matrix instruction to five vector instructions. Per
    waves-per-SIMD setting: microseconds per launch, and `*_over_max`, the
    combined time over the larger of the two alone (1 = complete overlap)."""
    import torch

    import exact_attention_23_amd as fa

    lib = _probe_lib()
    out = torch.empty(4 * cus * 256, dtype=torch.float32, device="cuda:0")
    stream = fa._current_stream(0)
    res = {}
    for wps in (1, 2, 4):
        blocks = cus * wps
        us = {}
        for name, mode in (("matrix_only", 1), ("vector_only", 2), ("both_compiler_order", 3),
                           ("both_interleaved", 4)):
            def launch(mode=mode, blocks=blocks):
                assert lib.fa_probe_coissue(mode, blocks, iters, out.data_ptr(), stream) == 0

            us[name] = round(_time_launches(launch) * 1e6, 1)
            if not torch.isfinite(out[:blocks * 256]).all():
                raise RuntimeError("co-issue probe produced non-finite values")
        mx = max(us["matrix_only"], us["vector_only"])
        res[f"{wps}_waves_per_simd"] = {
            "us": us,
            "compiler_order_over_max": round(us["both_compiler_order"] / mx, 3),
            "interleaved_over_max": round(us["both_interleaved"] / mx, 3),
        }
    return res


def vector_roofline(w, us: float, rates):
    """The vector-unit bound of the forward on w: per score the softmax needs
    one FMA and one exp2 (the pair the probe times), so the pairs of all
    scores at the probed pair rate take `floor_us`; the measured time is
    reported as a fraction of that bound (1 = at the bound). Conversions,
    row sums and masking are left out, so the bound is optimistic."""
    scores = w.B * w.H * w.Nq * w.Nk / (2 if w.causal else 1)
    pair_lanes_per_s = rates["fma_exp2_pair"]["wave_instr_per_s"] * 64
    floor_us = scores / pair_lanes_per_s * 1e6
    return {"bound": "valu (exp2 + fma per score)", "floor_us": round(floor_us, 2),
            "achieved_us": round(us, 3), "frac": round(floor_us / us, 4)}


def copy_calibration(mib: int, reps: int = 5):
    """Run a plain device-to-device copy of `mib` MiB `reps` times, so the HBM
    byte counters can be scaled against a kernel of known traffic."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "reps": reps}),
          flush=True)


def _counter_rows(csv_dir: str, counter: str):
    """(kernel name, value) rows of one rocprofv3 --pmc CSV output directory."""
    import csv
    import glob

    rows = []
    for f in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def write_traffic(workload: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str,
                  copy_write_dir: str, copy_mib: int, command: str, bwd: bool = False,
                  fp8: bool = False, std: bool = False):
    """Record HBM bytes per launch of the attention kernel (the forward, or
    with bwd the dK/dV kernel of the backward, keyed "bwd:<workload>"; with
    std the three kernels of the standard attention summed per call, keyed
    "std:<workload>") from rocprofv3 FETCH_SIZE / WRITE_SIZE runs (KiB per
    dispatch), each scaled by what the same counter reads for a plain copy of
    copy_mib MiB (known bytes)."""
    import statistics

    known = copy_mib * (1 << 20)
    cf = [v for k, v in _counter_rows(copy_fetch_dir, "FETCH_SIZE") if "copyBuffer" in k or "copy" in k.lower()]
    cw = [v for k, v in _counter_rows(copy_write_dir, "WRITE_SIZE") if "copyBuffer" in k or "copy" in k.lower()]
    f_scale = known / (statistics.median(cf) * 1024) if cf else None
    w_scale = known / (statistics.median(cw) * 1024) if cw else None
    if std:
        kname = "+".join(STD_KERNELS)
        fetch = write = 0.0
        for kn in STD_KERNELS:
            kf = [v for k, v in _counter_rows(fetch_dir, "FETCH_SIZE") if kn in k]
            kw = [v for k, v in _counter_rows(write_dir, "WRITE_SIZE") if kn in k]
            if not (cf and cw and kf and kw):
                raise RuntimeError(f"missing counter rows for {kn}")
            fetch += statistics.median(kf) * 1024 * f_scale
            write += statistics.median(kw) * 1024 * w_scale
    else:
        kname = "fa_bwd_dkdv_kernel" if bwd else ("fa_fwd_fp8_kernel" if fp8 else "fa_fwd16_kernel")
        kf = [v for k, v in _counter_rows(fetch_dir, "FETCH_SIZE") if kname in k]
        if not kf and not (bwd or fp8):  # a latency-bound size runs the short-range kernel
            kname = "fa_fwd_short_kernel"
            kf = [v for k, v in _counter_rows(fetch_dir, "FETCH_SIZE") if kname in k]
        kw = [v for k, v in _counter_rows(write_dir, "WRITE_SIZE") if kname in k]
        if not (cf and cw and kf and kw):
            raise RuntimeError("missing counter rows")
        fetch = statistics.median(kf) * 1024 * f_scale
        write = statistics.median(kw) * 1024 * w_scale
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        rec = {}
    rec["about"] = ("HBM bytes per launch of fa_fwd16_kernel (key: workload), of "
                    "fa_bwd_dkdv_kernel (key: bwd:workload), of fa_fwd_fp8_kernel (key: "
                    "fp8:workload) and per call of the three standard-attention kernels (key: "
                    "std:workload) from rocprofv3 FETCH_SIZE and "
                    "WRITE_SIZE (KiB per dispatch), scaled by the same counters on a plain "
                    "device copy of known size. Written by bench.py --write-traffic.")
    key = f"bwd:{workload}" if bwd else (f"fp8:{workload}" if fp8 else
                                         (f"std:{workload}" if std else workload))
    rec.setdefault("workloads", {})[key] = {
        "kernel": kname,
        "kernel_source_sha": kernel_source_hash(BWD_KERNEL_SOURCES if bwd else
                                                (FP8_KERNEL_SOURCES if fp8 else
                                                 (STD_KERNEL_SOURCES if std else None))),
        "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
        "hbm_bytes_per_launch": round(fetch + write),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "copy_calibration_mib": copy_mib, "command": command,
    }
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w", encoding="utf-8") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    return rec["workloads"][key]


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed calls after the warmup steps until this much time has passed")
    ap.add_argument("--workload", default="yolo80b16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-n400", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain copy kernel of this many MiB (counter scaling)")
    ap.add_argument("--write-traffic", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                         "COPY_WRITE_DIR", "COPY_MIB"),
                    help="record HBM traffic of --workload from rocprofv3 --pmc CSV directories")
    ap.add_argument("--command", default="", help="profiling command recorded with --write-traffic")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="fwd (default): the forward line, with the backward of the same "
                         "workload attached; bwd: a line for the backward pass alone")
    ap.add_argument("--no-bwd", action="store_true", help="leave the backward out of the fwd line")
    ap.add_argument("--no-clock", action="store_true",
                    help="do not sample the engine clock (amd-smi) under the workload's load")
    ap.add_argument("--fp8", action="store_true",
                    help="forward on the workload's inputs quantised to e4m3 (fa_fwd_fp8), "
                         "against the fp8 matrix peak")
    ap.add_argument("--std", action="store_true",
                    help="a line for the standard (unfused) attention against the fused forward "
                         "on --workload only")
    ap.add_argument("--no-extras", action="store_true",
                    help="leave out the per-workload, FP8, standard-attention and vector-rate "
                         "sections of the forward line")
    ap.add_argument("--layout", choices=("bhnd", "bnhd", "qkv"), default="bhnd",
                    help="memory layout of q, k, v, o for the forward: contiguous [B,H,N,d] "
                         "(default), sequence-major [B,N,H,d], or views of a fused [B,N,3,H,d] "
                         "buffer (the latter two through fa_fwd_strided)")
    args = ap.parse_args(argv)
    if args.write_traffic:
        fd, wd, cfd, cwd, mib = args.write_traffic
        print(json.dumps(write_traffic(args.workload, fd, wd, cfd, cwd, int(mib), args.command,
                                       bwd=args.which == "bwd", fp8=args.fp8, std=args.std)))
        return 0
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return 0
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only; --gpus {args.gpus} is not supported. "
              "The path shards over (batch, head) with no exchange, so per-GPU work is the "
              "single-GPU kernel at a fraction of the heads.", file=sys.stderr)
        return 2

    from workloads import WORKLOAD_ORDER, WORKLOADS

    w = WORKLOADS[args.workload]
    if args.std:
        rec = std_vs_fused(w, max(args.steps // 5, 2), max(args.warmup // 3, 1))
        line = {"metric": "standard (unfused) attention against the fused forward, us per call",
                "value": rec["standard_us"], "unit": "us", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": rec["standard_us"] * 1e-3,
                "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
                "dtype": w.dtype, "data": "synthetic", "config": {"workload": w.name},
                "standard_vs_fused": rec}
        print(json.dumps(line), flush=True)
        return 0
    if args.which == "bwd":
        ms, per = time_bwd(w, args.steps, args.warmup, args.settle_ms)
        rec = bwd_record(w, ms, per)
        line = {
            "metric": "attention bwd TFLOP/s (dQ, dK, dV; 10*B*H*Nq*Nk*d FLOP, halved when "
                      "causal) and % MFMA peak",
            "value": rec["value"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": rec["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
            "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                       "causal": w.causal, "input_dtype": w.dtype, "accumulate": "fp32",
                       "parallelism": "single GPU; grids over (batch, head, key block) and "
                                      "(batch, head, query block)"},
            "mfma_peak_frac": rec["mfma_peak_frac"], "kernels_us": rec["kernels_us"],
            "roofline": rec["roofline"], "kernel_source_sha": rec["kernel_source_sha"],
        }
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_bwd(w)
        print(json.dumps(line), flush=True)
        return 0
    if args.fp8:
        ms = time_fp8(w, args.steps, args.warmup, args.settle_ms)
        tflops = w.flops() / (ms * 1e-3) / 1e12
        line = {
            "metric": "attention fwd TFLOP/s on FP8 (e4m3) inputs and % fp8 MFMA peak",
            "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
            "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                       "causal": w.causal, "input_dtype": "fp8_e4m3 (per-tensor amax scaling)",
                       "output_dtype": "bf16", "accumulate": "fp32",
                       "parallelism": "single GPU; grid over (batch, head, query block)"},
            "us_per_call": round(ms * 1e3, 3),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_MFMA_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_FP8_TFLOPS, 4),
                         "traffic": measured_traffic(f"fp8:{w.name}", FP8_KERNEL_SOURCES)},
            "kernel_source_sha": kernel_source_hash(FP8_KERNEL_SOURCES),
        }
        print(json.dumps(line), flush=True)
        return 0
    ms = time_gpu(w, args.steps, args.warmup, args.settle_ms, args.layout)
    tflops = w.flops() / (ms * 1e-3) / 1e12
    n400_us = n400_eager_us = None
    if not args.no_n400 and args.workload != "yolo20":
        n400_us = time_graph(WORKLOADS["yolo20"])
        n400_eager_us = time_gpu(WORKLOADS["yolo20"], max(args.steps, 50), args.warmup,
                                 args.settle_ms) * 1e3
    short = None
    floor_us = None
    if not args.no_n400 and args.workload != "yolo20":
        # the two latency-bound sizes (20x20 and 19x19 maps): HBM rate and latency spread
        short = {n: short_stats(WORKLOADS[n]) for n in ("yolo20", "tail361")}
        floor_us = launch_floor_us()
    clock = None if args.no_clock or args.layout != "bhnd" else clock_under_load(w)
    traffic = measured_traffic(w.name)
    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "input_dtype": w.dtype, "accumulate": "fp32",
                   "layout": args.layout,
                   "parallelism": "single GPU; grid over (batch, head, query block)"},
        "us_per_call": round(ms * 1e3, 3),
        # N=400 (20x20 map): device time per call from a replayed HIP graph of
        # 100 calls, and the eager rate of Python calls (host launch cost
        # included), which is what a caller without graphs sees
        "us_per_call_n400": None if n400_us is None else round(n400_us, 3),
        "us_per_call_n400_eager": None if n400_eager_us is None else round(n400_eager_us, 3),
        "short_sequences": short,
        "launch_floor_us": None if floor_us is None else round(floor_us, 3),
        "clock_mhz_under_load": clock,
        "mfma_peak_frac": round(tflops / PEAK_MFMA_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_MFMA_TFLOPS, 4),
                     "traffic": traffic},
        "algorithmic_hbm_gbs": round(w.algorithmic_bytes() / (ms * 1e-3) / 1e9, 1),
        "kernel_source_sha": kernel_source_hash(),
    }
    if not args.no_extras:
        # every named workload (the headline above is one of them), the FP8
        # forward of the two long ones, the standard attention against the
        # fused forward, and the vector-unit bound of the headline workload
        line["workloads"] = {n: workload_record(WORKLOADS[n], args.steps, args.warmup, args.settle_ms)
                             for n in WORKLOAD_ORDER}
        if not args.no_clock:
            line["workloads"]["long16k"]["clock_mhz_under_load"] = clock_under_load(WORKLOADS["long16k"])
            line["workloads"]["seq2048"]["clock_mhz_under_load"] = clock_under_load(WORKLOADS["seq2048"])
        line["fp8"] = {n: fp8_record(WORKLOADS[n], args.steps, args.warmup, args.settle_ms)
                       for n in ("yolo80b16", "seq2048", "long16k")}
        line["standard_vs_fused"] = std_vs_fused(WORKLOADS["seq2048"])
        rates = vector_rates()
        line["vector_rates"] = rates
        line["vector_roofline"] = vector_roofline(w, ms * 1e3, rates)
        line["matrix_rate"] = matrix_rate()
        line["coexec"] = coexec()
        line["coissue"] = coissue()
    if not args.no_bwd:
        # the backward pass of the same workload (a separate figure: the
        # headline value above is the forward's)
        bms, bper = time_bwd(w, max(args.steps // 2, 5), max(args.warmup // 2, 2), args.settle_ms)
        line["backward"] = bwd_record(w, bms, bper)
        if not args.no_extras:
            # the backward of the other long workloads, each on its own
            # inputs, so every head width's backward is measured in this run
            line["backward_workloads"] = {}
            for n in ("seq2048", "long16k"):
                if n == w.name:
                    continue
                bw = WORKLOADS[n]
                bms2, bper2 = time_bwd(bw, max(args.steps // 2, 5), max(args.warmup // 2, 2), args.settle_ms)
                line["backward_workloads"][n] = bwd_record(bw, bms2, bper2)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
