#!/usr/bin/env python3
"""Throughput of one tensor-parallel rank's Transformer-layer shard on one MI355X.

Headline workload: one rank (rank 0 of N = 8) of a bf16 layer with hidden 8192, 64 heads of
d = 128, ffn 32768, batch 1 x seq 4096, causal. One step is the rank's whole forward path:

    attention shard  (QKV column-parallel GEMM, causal attention, W_O row-parallel GEMM)
    sum of the N attention partials -> H (bf16)       [the all-reduce's sum, on device]
    MLP column-parallel GEMM + bias + GeLU on H
    MLP row-parallel GEMM -> fp32 partial
    sum of the N MLP partials -> Z (fp32)

The other seven ranks' partials are computed once before timing (they stand for what the
peers would contribute) and stay resident in HBM. Inputs are seeded synthetic tensors
(``synth``), already on the device when timing starts.

value = algorithmic FLOPs of the rank's shard (859.0 GFLOP, causal attention counted as the
s(s+1)/2 triangle) / wall time per step, in TFLOP/s. Per-stage times come from HIP events
recorded on the launch stream after each stage in as many instrumented steps before the timed
ones. The timed steps carry only the two events around the dominant kernel (the slower MLP
GEMM), whose rate is reported against the bf16 MFMA peak.

``configs`` times every measured workload on its own unit (an fp32 MLP block of two shards
and their sum, a bf16 MLP shard, a bf16 attention shard with each of its three steps, the
layer step above, and all N shards of a large MLP block for N = 1, 2, 4, 8), each with its
dominant kernel against its roofline. The fp64 CPU oracle is timed on the host cores on the
same units (bounded row samples where a unit is large) and its results are compared with the
GPU's outputs of the timed runs: a relative Frobenius error above the tolerance exits
non-zero.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "per-rank TP shard TFLOP/s (MLP + attention) and % of MI355X bf16 MFMA peak"
WORKLOAD = "layer_shard_bf16_b1_s4096_h8192_H64_f32768_n8"
W_MLP_F32 = "mlp_f32_t32_h1024_f4096_n2"
W_MLP_BF16 = "mlp_shard_bf16_t8192_h3072_f12288_n8"
W_ATTN = "attn_shard_bf16_b4_s2048_h4096_H32_n8"
W_BLOCK = "mlp_block_bf16_t2048_h12288_f49152"
# MI355X bf16 dense MFMA peak: 256 CUs x 4096 FLOP/clk/CU x 2.4 GHz (the published 2.5 PFLOP/s).
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP32_TFLOPS = 157.3     # fp32 matrix (MFMA) peak
PEAK_HBM_GBS = 8000.0
TOL = {"f32": 1e-4, "bf16": 1e-2}


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "tensor_transformer_layers_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stage_flops(w):
    """Algorithmic FLOPs of each stage of rank 0's layer shard."""
    T, h, F, N = w.tokens, w.hidden, w.ffn, w.n_shards
    d = h // w.heads
    hl = w.heads // N
    wl = hl * d
    keys = w.seq * (w.seq + 1) // 2 if w.causal else w.seq * w.seq
    return {
        "qkv_projection": 2.0 * T * h * 3 * wl,
        "attention": 4.0 * d * keys * hl * w.batch,
        "out_projection": 2.0 * T * wl * h,
        "mlp_column": 2.0 * T * h * (F // N),
        "mlp_row": 2.0 * T * (F // N) * h,
    }


def traffic_for(kernel: str, stage: str):
    """HBM bytes per launch of ``kernel`` in ``stage`` from the committed counter summary
    (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE scaled by a plain-copy calibration),
    or None when the summary was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != kernel_source_sha():
        return None
    for name, k in rec.get("kernels", {}).items():
        if name.split(" [")[0] == kernel and k.get("stage") == stage:
            return k.get("hbm_bytes_per_launch")
    return None


def gemm_kernel_name(M: int, N: int, K: int, epi: int, n_parts: int = 0) -> str:
    """The bf16 GEMM launched for an M x N x K product, named as the profiler names it:
    gemm_bf16_kernel<tile_m, tile_n, waves_m, waves_n, epilogue>. The Q/K/V scatter (2) always
    runs eight waves; the fused sums (6 fp32, 7 bf16 output, over ``n_parts`` partials) take
    the launch the library reports for them."""
    from tensor_transformer_layers_amd import binding
    if epi in (6, 7):
        _, tbm, tbn, nw, _form = binding.tp_row_parallel_sum_tile_info(
            M, N, K, n_parts, binding.TP_F32 if epi == 6 else binding.TP_BF16)
    else:
        _, tbm, tbn, nw = binding.tp_gemm_tile_info(M, N, K)
    if epi == 2:
        nw = 8
    wgrid = {(256, 256, 8): (2, 4), (256, 192, 8): (4, 2), (256, 128, 8): (4, 2),
             (128, 128, 8): (2, 4)}.get((tbm, tbn, nw), (2, 2))
    return "gemm_bf16_kernel<%d, %d, %d, %d, (tps::Epi)%d>" % (tbm, tbn, wgrid[0], wgrid[1], epi)


# ---- shader clock during the timed steps ----------------------------------------------------
class ClockSampler:
    """Samples the GPU's shader clock from sysfs every ~10 ms in a background thread: the
    hwmon ``freq1_input`` (current sclk, Hz) where the driver provides it, else the active
    level of ``pp_dpm_sclk``. Reports what it could read, or why it could not."""

    def __init__(self, period_s: float = 0.01):
        self.period = period_s
        self.samples = []
        self.source = None
        self._stop = threading.Event()
        self._thread = None
        cands = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/freq1_input"))
        if cands:
            self.source = ("hwmon", cands[0])
        else:
            cands = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
            if cands:
                self.source = ("dpm", cands[0])

    def _read(self):
        kind, path = self.source
        with open(path) as f:
            text = f.read()
        if kind == "hwmon":
            return int(text.strip()) / 1e6
        for line in text.splitlines():
            if line.strip().endswith("*"):
                return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                if v:
                    self.samples.append(v)
            except (OSError, ValueError, IndexError):
                pass
            time.sleep(self.period)

    def __enter__(self):
        if self.source:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread:
            self._thread.join()

    def summary(self):
        if not self.source:
            return {"mhz_mean": None, "note": "no sclk file under /sys/class/drm on this host"}
        s = self.samples
        if not s:
            return {"mhz_mean": None, "source": self.source[1], "note": "no readable sample"}
        return {"mhz_mean": sum(s) / len(s), "mhz_min": min(s), "mhz_max": max(s),
                "samples": len(s), "source": self.source[1]}


# ---- timing helpers -------------------------------------------------------------------------
def _time_events(fn, reps: int, warmup: int, stream, rounds: int = 3,
                 warm_ms: float = 60.0) -> float:
    """Microseconds per call of fn(): HIP events on ``stream`` around ``rounds`` rounds of
    ``reps`` calls each, the median round's average. The warm-up runs at least ``warmup``
    calls and at least ``warm_ms`` of wall time in batches of calls: the shader clock settles
    over the first tens of milliseconds of MFMA work, and a workload of a few hundred
    microseconds per call would otherwise be timed on a clock still rising."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < warm_ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    per = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / reps)
    return float(sorted(per)[len(per) // 2])


def _roof_mfma(name: str, flops: float, us: float, peak: float) -> dict:
    a = flops / us / 1e6
    return {"bound": "mfma", "kernel": name, "us": us, "achieved": a, "peak": peak,
            "unit": "TFLOP/s", "frac": a / peak}


def _roof_hbm(name: str, nbytes: float, us: float) -> dict:
    a = nbytes / us / 1e3
    return {"bound": "hbm", "kernel": name, "us": us, "achieved": a, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": a / PEAK_HBM_GBS, "algorithmic_bytes": nbytes}


def _up(x, dtype):
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dtype).cuda()


def _host(t):
    import numpy as np
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def _host32(t):
    """fp32 host copy (bf16 values are exact in fp32; half the memory of fp64)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


# ---- the layer step ---------------------------------------------------------------------------
def layer_stage_cost(w, stage: str):
    """Algorithmic (FLOPs, HBM bytes) of one stage of rank 0's layer step, or None for a stage
    of several kernels. Bytes count every operand once and every output once."""
    T, h, N = w.tokens, w.hidden, w.n_shards
    d = h // w.heads
    wl = (w.heads // N) * d
    Fl = w.ffn // N
    fl = stage_flops(w)
    peers = 4.0 * T * h * (N - 1)          # the other ranks' fp32 partials
    return {
        "qkv_projection": (fl["qkv_projection"], 2.0 * (T * h + 3 * wl * h + 3 * T * wl)),
        "out_projection_sum": (fl["out_projection"], 2.0 * (T * wl + h * wl) + peers + 2.0 * T * h),
        "mlp_column": (fl["mlp_column"], 2.0 * (T * h + Fl * h + Fl + T * Fl)),
        "mlp_row": (fl["mlp_row"], 2.0 * (T * Fl + h * Fl) + 4.0 * T * h),
        "mlp_row_sum": (fl["mlp_row"], 2.0 * (T * Fl + h * Fl) + peers + 4.0 * T * h),
        "sum_attention": (0.0, 4.0 * T * h * N + 2.0 * T * h),
        "sum_mlp": (0.0, 4.0 * T * h * N + 4.0 * T * h),
    }.get(stage)


def layer_stage_kernel(w, stage: str) -> str:
    """The kernel of a one-kernel stage, named as the profiler names it."""
    T, h, N = w.tokens, w.hidden, w.n_shards
    wl = (w.heads // N) * (h // w.heads)
    Fl = w.ffn // N
    return {"qkv_projection": lambda: gemm_kernel_name(T, 3 * wl, h, 2),
            "out_projection_sum": lambda: gemm_kernel_name(T, h, wl, 7, n_parts=N),
            "mlp_column": lambda: gemm_kernel_name(T, Fl, h, 0),
            "mlp_row": lambda: gemm_kernel_name(T, h, Fl, 1),
            "mlp_row_sum": lambda: gemm_kernel_name(T, h, Fl, 6, n_parts=N),
            "sum_attention": lambda: "sum_kernel<%d, 4, true>" % N,
            "sum_mlp": lambda: "sum_kernel<%d, 4, false>" % N}[stage]()


def stage_roofline(w, stage: str, us: float, traffic=None) -> dict:
    """The stage's kernel against the roofline that bounds it: HBM when its algorithmic bytes
    take longer at 8 TB/s than its FLOPs at the bf16 MFMA peak, else MFMA."""
    flops, nbytes = layer_stage_cost(w, stage)
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    name = layer_stage_kernel(w, stage)
    if t_hbm > t_mfma:
        r = _roof_hbm(name, nbytes, us)
        if flops:
            r["mfma_frac"] = flops / us / 1e6 / PEAK_BF16_TFLOPS
    else:
        r = _roof_mfma(name, flops, us, PEAK_BF16_TFLOPS)
        r["algorithmic_bytes"] = nbytes
    r["stage"] = stage
    r["traffic"] = traffic_for(name, stage) if traffic is None else traffic
    return r


def time_layer_step(drv, step, w, fl, steps: int, warmup: int, stream) -> dict:
    """Warm-up, then ``steps`` instrumented steps (an event after each stage) for the per-stage
    medians, then ``steps`` timed steps carrying only the two events around the dominant
    kernel (the longest one-kernel stage), bracketed by device synchronizations."""
    import numpy as np
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stages = drv.STAGES
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        marks = iter(ev[i][1:])
        step(on_stage=lambda name, m=marks: next(m).record(stream))
    torch.cuda.synchronize()
    # the median over the steps of each stage (one host stall between two launches would
    # otherwise lengthen the stage it falls into, in the mean)
    stage_us = {s: float(np.median([ev[i][j].elapsed_time(ev[i][j + 1]) * 1e3
                                    for i in range(steps)]))
                for j, s in enumerate(stages)}
    single = [s for s in stages if layer_stage_cost(w, s) is not None]
    dom = max(single, key=lambda s: stage_us[s])
    before = stages[stages.index(dom) - 1] if stages.index(dom) > 0 else None
    dev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]

    def mark_dominant(name, pair):
        if name == before:
            pair[0].record(stream)
        elif name == dom:
            pair[1].record(stream)

    torch.cuda.synchronize()
    with ClockSampler() as clock:
        t_start = time.perf_counter()
        for i in range(steps):
            if before is None:
                dev[i][0].record(stream)
            step(on_stage=lambda name, pair=dev[i]: mark_dominant(name, pair))
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
    dom_us = sum(a.elapsed_time(b) for a, b in dev) * 1e3 / steps
    breakdown = {}
    for s in stages:
        c = layer_stage_cost(w, s)
        e = {"us": stage_us[s]}
        if s == "attention_shard":
            f = fl["qkv_projection"] + fl["attention"] + fl["out_projection"]
            e["tflops"] = f / stage_us[s] / 1e6
        elif s == "attention":
            e["tflops"] = fl["attention"] / stage_us[s] / 1e6
        elif c is not None:
            if c[0]:
                e["tflops"] = c[0] / stage_us[s] / 1e6
            e["gbs"] = c[1] / stage_us[s] / 1e3
        breakdown[s] = e
    return {"ms_per_step": elapsed / steps * 1e3, "event_ms": sum(stage_us.values()) / 1e3,
            "stage_us": stage_us, "breakdown": breakdown,
            "roofline": stage_roofline(w, dom, dom_us), "clock": clock.summary()}


# ---- the measured workloads other than the layer step -----------------------------------------
def _time_graph(fn, reps: int, warmup: int = 3):
    """Microseconds per fn() when ``reps`` calls are captured once in a HIP graph and the graph
    is replayed (launch-bound work: the host's per-call overhead is left out); the median of
    three timed rounds after 60 ms of replays. Returns (us, graph)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()          # replays for 60 ms first, as _time_events warms up
    while (time.perf_counter() - t0) * 1e3 < 60.0:
        g.replay()
        torch.cuda.synchronize()
    n, per = 5, []
    for _ in range(3):                # the median of three rounds of n replays
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / (n * reps))
    return float(sorted(per)[1]), g


def measure_mlp_f32(reps: int = 200, warmup: int = 20):
    """fp32 MLP block GeLU(XA + a)B: both shards of N = 2 and their on-device sum. Each call
    is a few microseconds of GPU work, less than the host needs to issue it, so the block and
    its kernels are timed as replays of a captured HIP graph (the eager rate is reported too);
    every replay's output is checked bitwise against the eager result."""
    import torch
    from synth import WORKLOADS, mlp_inputs
    from tensor_transformer_layers_amd import layout, shard
    w = WORKLOADS[W_MLP_F32]
    T, h, F, N = w.tokens, w.hidden, w.ffn, w.n_shards
    d = mlp_inputs(w, seed=0)
    X = _up(d["X"], torch.float32)
    W = [dict(A=_up(layout.column_shard(d["A"], N, r), torch.float32),
              a=_up(layout.bias_shard(d["a"], N, r), torch.float32),
              B=_up(layout.row_shard(d["B"], N, r), torch.float32)) for r in range(N)]
    Zs = [torch.empty(T, h, device="cuda") for _ in range(N)]
    ws = [shard.mlp_workspace(T, h, F, N, torch.float32) for _ in range(N)]
    Z = torch.empty(T, h, device="cuda")
    stream = torch.cuda.current_stream()

    def block():
        for r in range(N):
            shard.mlp_shard(X, W[r]["A"], W[r]["a"], W[r]["B"], N, r, Z=Zs[r], workspace=ws[r])
        shard.sum_partials(Zs, out=Z)

    eager_us = _time_events(block, reps, warmup, stream)
    block()
    torch.cuda.synchronize()
    Z_eager = Z.clone()
    us, gblock = _time_graph(block, 20)
    for _ in range(3):           # every replay reproduces the eager bits
        Z.zero_()
        torch.cuda.synchronize()
        gblock.replay()
        torch.cuda.synchronize()
        if not torch.equal(Z, Z_eager):
            raise RuntimeError("graph replay of the fp32 block differs from the eager result")
    fl = F // N
    Y = shard.mlp_hidden_view(ws[0], T, fl, torch.float32)
    col_us, _ = _time_graph(lambda: shard.column_parallel(X, W[0]["A"], W[0]["a"], N, 0,
                                                          gelu=True, Y=Y), 50)
    row_us, _ = _time_graph(lambda: shard.row_parallel(Y, W[0]["B"], N, 0, Z=Zs[0]), 50)
    sum_us, _ = _time_graph(lambda: shard.sum_partials(Zs, out=Z), 50)
    block()
    torch.cuda.synchronize()
    flops = 2 * 2.0 * T * h * F
    # both GEMMs of a shard stream their fp32 weight shard (1024 x 2048 x 4 bytes = 8.4 MB)
    # plus a 32-row activation: bound by memory and latency, not by the matrix cores
    col_bytes = 4.0 * (T * h + fl * h + fl + T * fl)
    row_bytes = 4.0 * (T * fl + h * fl + T * h)
    dom, dom_us, dom_b = ("column", col_us, col_bytes) if col_us >= row_us else ("row", row_us, row_bytes)
    # the library's row blocks per workgroup (16-column blocks, rows split while the grid
    # stays within 256 workgroups), for the kernel's name
    cols = -(-(fl if dom == "column" else h) // 16)
    rblocks = -(-T // 16)
    groups = max(1, min(rblocks, 256 // cols))
    need = -(-rblocks // groups)
    mb = 1 if need <= 1 else (2 if need <= 2 else 4)
    kname = "gemm_f32_skinny_kernel<%d, (tps::Epi)%d>" % (mb, 0 if dom == "column" else 1)
    out = {"workload": w.name, "unit": "block: %d shards + on-device sum" % N, "dtype": "f32",
           "us": us, "timing": "HIP graph replay of 20 blocks",
           "eager_us": eager_us, "tflops": flops / us / 1e6, "peak": PEAK_FP32_TFLOPS,
           "frac_peak": flops / us / 1e6 / PEAK_FP32_TFLOPS,
           "per_shard_kernels_us": {"column": col_us, "row": row_us}, "sum_us": sum_us,
           "roofline": dict(_roof_hbm(kname, dom_b, dom_us),
                            mfma_frac=2.0 * T * h * fl / dom_us / 1e6 / PEAK_FP32_TFLOPS)}
    return out, {"d": d, "Z": _host(Z)}


def measure_mlp_bf16(reps: int = 30, warmup: int = 10):
    """One rank's bf16 MLP shard (rank 0 of N = 8): column GEMM + GeLU, row GEMM."""
    import torch
    from synth import WORKLOADS, mlp_inputs
    from tensor_transformer_layers_amd import layout, shard
    w = WORKLOADS[W_MLP_BF16]
    T, h, F, N = w.tokens, w.hidden, w.ffn, w.n_shards
    fl = F // N
    d = mlp_inputs(w, seed=0)
    X = _up(d["X"], torch.bfloat16)
    A = _up(layout.column_shard(d["A"], N, 0), torch.bfloat16)
    a = _up(layout.bias_shard(d["a"], N, 0), torch.bfloat16)
    Bm = _up(layout.row_shard(d["B"], N, 0), torch.bfloat16)
    Z = torch.empty(T, h, device="cuda")
    ws = shard.mlp_workspace(T, h, F, N, torch.bfloat16)
    stream = torch.cuda.current_stream()
    us = _time_events(lambda: shard.mlp_shard(X, A, a, Bm, N, 0, Z=Z, workspace=ws), reps, warmup,
                      stream)
    Y = shard.mlp_hidden_view(ws, T, fl, torch.bfloat16)
    col_us = _time_events(lambda: shard.column_parallel(X, A, a, N, 0, gelu=True, Y=Y), reps,
                          warmup, stream)
    row_us = _time_events(lambda: shard.row_parallel(Y, Bm, N, 0, Z=Z), reps, warmup, stream)
    shard.mlp_shard(X, A, a, Bm, N, 0, Z=Z, workspace=ws)
    torch.cuda.synchronize()
    flops = 4.0 * T * h * fl
    if col_us >= row_us:
        roof = _roof_mfma(gemm_kernel_name(T, fl, h, 0), flops / 2, col_us, PEAK_BF16_TFLOPS)
    else:
        roof = _roof_mfma(gemm_kernel_name(T, h, fl, 1), flops / 2, row_us, PEAK_BF16_TFLOPS)
    out = {"workload": w.name, "unit": "one rank's shard (rank 0 of %d)" % N, "dtype": "bf16",
           "us": us, "tflops": flops / us / 1e6, "peak": PEAK_BF16_TFLOPS,
           "frac_peak": flops / us / 1e6 / PEAK_BF16_TFLOPS,
           "kernels_us": {"column_gemm_gelu": col_us, "row_gemm": row_us}, "roofline": roof}
    return out, {"d": d, "Z": _host(Z)}


def measure_attn(reps: int = 30, warmup: int = 10):
    """One rank's bf16 causal attention shard (rank 0 of N = 8), the whole call and each of
    its three steps on their own (the same kernels: tp_qkv_projection_fwd,
    tp_head_attention_fwd, tp_row_parallel_fwd on the workspace's O)."""
    import torch
    from synth import WORKLOADS, attn_inputs
    from tensor_transformer_layers_amd import layout, shard
    w = WORKLOADS[W_ATTN]
    b, s, h, H, N = w.batch, w.seq, w.hidden, w.heads, w.n_shards
    T, d_h, hl = b * s, h // H, H // N
    wl = hl * d_h
    d = attn_inputs(w, seed=0)
    X = _up(d["X"], torch.bfloat16)
    Wqkv = _up(layout.qkv_shard(d["Wq"], d["Wk"], d["Wv"], N, 0), torch.bfloat16)
    bqkv = _up(layout.qkv_bias_shard(d["bq"], d["bk"], d["bv"], N, 0), torch.bfloat16)
    Wo = _up(layout.row_shard(d["Wo"], N, 0), torch.bfloat16)
    Z = torch.empty(T, h, device="cuda")
    ws = shard.attn_workspace(b, s, h, H, N)
    stream = torch.cuda.current_stream()
    us = _time_events(lambda: shard.attn_shard(X, Wqkv, bqkv, Wo, b, s, H, N, 0, True, Z=Z,
                                               workspace=ws), reps, warmup, stream)
    O = shard.attn_views(ws, b, s, h, H, N)["o"]
    q_us = _time_events(lambda: shard.qkv_projection(X, Wqkv, bqkv, b, s, H, H, N, 0, ws), reps,
                        warmup, stream)
    a_us = _time_events(lambda: shard.head_attention(b, s, h, H, H, N, 0, True, ws), reps,
                        warmup, stream)
    o_us = _time_events(lambda: shard.row_parallel(O, Wo, N, 0, Z=Z), reps, warmup, stream)
    shard.attn_shard(X, Wqkv, bqkv, Wo, b, s, H, N, 0, True, Z=Z, workspace=ws)
    torch.cuda.synchronize()
    fq = 2.0 * T * h * 3 * wl
    fa = 4.0 * d_h * (s * (s + 1) // 2) * hl * b
    fo = 2.0 * T * wl * h
    flops = fq + fa + fo
    # W_O: bf16 O_i [T, Hl d] and W_O,i [h, Hl d] in, fp32 Z_i [T, h] out
    wo_bytes = 2.0 * T * wl + 2.0 * h * wl + 4.0 * T * h
    out = {"workload": w.name, "unit": "one rank's shard (rank 0 of %d)" % N, "dtype": "bf16",
           "us": us, "tflops": flops / us / 1e6, "peak": PEAK_BF16_TFLOPS,
           "frac_peak": flops / us / 1e6 / PEAK_BF16_TFLOPS,
           "steps": {
               "qkv_projection": _roof_mfma(gemm_kernel_name(T, 3 * wl, h, 2), fq, q_us,
                                            PEAK_BF16_TFLOPS),
               "attention": _roof_mfma("attn_fwd_kernel (with its key-range merge, if any)",
                                       fa, a_us, PEAK_BF16_TFLOPS),
               "out_projection": dict(_roof_hbm(gemm_kernel_name(T, h, wl, 1), wo_bytes, o_us),
                                      mfma_frac=fo / o_us / 1e6 / PEAK_BF16_TFLOPS),
           }}
    dom = max(out["steps"], key=lambda k: out["steps"][k]["us"])
    out["roofline"] = dict(out["steps"][dom], step=dom)
    return out, {"d": d, "Z": _host(Z)}


def measure_block_sweep(reps: int = 20, warmup: int = 10):
    """All N shards of one bf16 MLP block (T 2048, h 12288, F 49152) plus the on-device sum,
    N in {1, 2, 4, 8}: how the shard's GEMM shape moves the MFMA utilisation. One set of full
    weights (seeded, on the device) is sliced into N shards for every N."""
    import torch
    from synth import WORKLOADS
    from tensor_transformer_layers_amd import binding, shard
    w = WORKLOADS[W_BLOCK]
    T, h, F = w.tokens, w.hidden, w.ffn
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    stream = torch.cuda.current_stream()

    def rnd(*shape, std=1.0):
        return (torch.randn(*shape, device="cuda", generator=g) * std).to(torch.bfloat16)

    X = rnd(T, h)
    At = rnd(F, h, std=0.02)       # [F, h]: column shards are row blocks
    a = rnd(F, std=0.02)
    Bt = rnd(h, F, std=0.02)       # [h, F]: row shards are column blocks
    sweep, keep = {}, {}
    for N in (1, 2, 4, 8):
        fl = F // N
        A_s = [At[r * fl:(r + 1) * fl] for r in range(N)]
        a_s = [a[r * fl:(r + 1) * fl] for r in range(N)]
        B_s = [Bt[:, r * fl:(r + 1) * fl].contiguous() for r in range(N)]
        Zs = [torch.empty(T, h, device="cuda") for _ in range(N)]
        Zsum = torch.empty(T, h, device="cuda")
        ws = shard.mlp_workspace(T, h, F, N, torch.bfloat16)
        shard_us = _time_events(lambda: shard.mlp_shard(X, A_s[0], a_s[0], B_s[0], N, 0, Z=Zs[0],
                                                        workspace=ws), reps, warmup, stream)

        def block():
            for r in range(N):
                shard.mlp_shard(X, A_s[r], a_s[r], B_s[r], N, r, Z=Zs[r], workspace=ws)
            shard.sum_partials(Zs, out=Zsum)

        block_us = _time_events(block, max(4, reps // N), 2, stream)
        sum_us = _time_events(lambda: shard.sum_partials(Zs, out=Zsum), reps, warmup, stream)
        block()
        torch.cuda.synchronize()
        fl_shard = 4.0 * T * h * fl
        sum_bytes = (N + 1) * T * h * 4
        _, cbm, cbn, cw = binding.tp_gemm_tile_info(T, fl, h)
        _, rbm, rbn, rw = binding.tp_gemm_tile_info(T, h, fl)
        sweep["N=%d" % N] = {
            "shard_us": shard_us, "shard_tflops": fl_shard / shard_us / 1e6,
            "shard_frac_bf16_peak": fl_shard / shard_us / 1e6 / PEAK_BF16_TFLOPS,
            "column_gemm": "%dx%dx%d, tile %dx%d, %d waves" % (T, fl, h, cbm, cbn, cw),
            "row_gemm": "%dx%dx%d, tile %dx%d, %d waves" % (T, h, fl, rbm, rbn, rw),
            "block_us": block_us, "block_tflops": N * fl_shard / block_us / 1e6,
            "sum_us": sum_us, "sum_gbs": sum_bytes / sum_us / 1e3}
        keep[N] = {"shard0": Zs[0], "block": Zsum}
        del A_s, a_s, B_s, Zs, ws
    out = {"workload": w.name, "unit": "all N shards + on-device sum (block); rank 0 (shard)",
           "dtype": "bf16", "per_n": sweep}
    best = max(sweep, key=lambda k: sweep[k]["block_tflops"])
    out["tflops"] = sweep[best]["block_tflops"]
    out["frac_peak"] = out["tflops"] / PEAK_BF16_TFLOPS
    out["best_n"] = best
    return out, {"X": X, "At": At, "a": a, "Bt": Bt, "keep": keep}


def measure_next_rows(reps: int = 20, warmup: int = 10) -> dict:
    """Throughput of the paths next to the core shard, each on its named workload.

    Inputs are drawn on the device from a seeded generator with the workload's shapes and
    distributions (activations N(0, 1), weights N(0, 0.02), bf16): only the rank's own shard
    is drawn, the full weights are never needed for timing.
    """
    import torch
    from synth import WORKLOADS
    from tensor_transformer_layers_amd import shard
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    stream = torch.cuda.current_stream()

    def rnd(*shape, std=1.0, dtype=torch.bfloat16):
        return (torch.randn(*shape, device="cuda", generator=g) * std).to(dtype)

    out = {}
    # gated MLP shard
    w = WORKLOADS["swiglu_shard_bf16_t4096_h8192_f28672_n8"]
    T, h, fl = w.tokens, w.hidden, w.ffn // w.n_shards
    X, Wg, Wu, Wd = rnd(T, h), rnd(fl, h, std=0.02), rnd(fl, h, std=0.02), rnd(h, fl, std=0.02)
    Z = torch.empty(T, h, device="cuda")
    ws = shard.swiglu_workspace(T, h, w.ffn, w.n_shards)
    us = _time_events(lambda: shard.swiglu_shard(X, Wg, Wu, Wd, w.n_shards, 0, Z=Z, workspace=ws),
                      reps, warmup, stream)
    fl_ = 2.0 * T * h * 2 * fl + 2.0 * T * fl * h
    out["swiglu_shard"] = {"workload": w.name, "us": us, "tflops": fl_ / us / 1e6,
                           "frac_bf16_peak": fl_ / us / 1e6 / PEAK_BF16_TFLOPS}
    del X, Wg, Wu, Wd, Z, ws
    # grouped-query attention shards
    for name in ("gqa_shard_bf16_b1_s4096_h8192_H64_kv8_n8", "gqa_shard_bf16_b1_s4096_h8192_H64_kv4_n8"):
        w = WORKLOADS[name]
        b, sq, h, H, Hkv, N = w.batch, w.seq, w.hidden, w.heads, w.kv_heads, w.n_shards
        d = h // H
        hl, kvl = H // N, (Hkv // N if Hkv % N == 0 else 1)
        T = b * sq
        X = rnd(T, h)
        Wqkv, bqkv = rnd((hl + 2 * kvl) * d, h, std=0.02), rnd((hl + 2 * kvl) * d, std=0.02)
        Wo = rnd(h, hl * d, std=0.02)
        Z = torch.empty(T, h, device="cuda")
        ws = shard.gqa_attn_workspace(b, sq, h, H, Hkv, N)
        us = _time_events(lambda: shard.gqa_attn_shard(X, Wqkv, bqkv, Wo, b, sq, H, Hkv, N, 0,
                                                       True, Z=Z, workspace=ws),
                          reps, warmup, stream)
        fl_ = (2.0 * T * h * (hl + 2 * kvl) * d + 4.0 * d * (sq * (sq + 1) // 2) * hl * b
               + 2.0 * T * hl * d * h)
        out[name.split("_bf16")[0] + "_kv%d" % Hkv] = {
            "workload": name, "us": us, "tflops": fl_ / us / 1e6,
            "frac_bf16_peak": fl_ / us / 1e6 / PEAK_BF16_TFLOPS}
        del X, Wqkv, bqkv, Wo, Z, ws
    # sequence-parallel boundary (reduce-scatter + residual + LayerNorm) and all-gather
    w = WORKLOADS["sp_boundary_bf16_b1_s4096_h8192_n8"]
    b, sq, h, N = w.batch, w.seq, w.hidden, w.n_shards
    T, rows = b * sq, b * sq // N
    parts = [torch.randn(T, h, device="cuda", generator=g) for _ in range(N)]
    resid = rnd(rows, h)
    gamma = 1.0 + 0.1 * torch.randn(h, device="cuda", generator=g)
    beta = 0.1 * torch.randn(h, device="cuda", generator=g)
    H_, Y_ = torch.empty(rows, h, device="cuda", dtype=torch.bfloat16), torch.empty_like(resid)
    us = _time_events(lambda: shard.sp_residual_layernorm(parts, resid, gamma, beta, b, sq, 0,
                                                          H=H_, Y=Y_), reps, warmup, stream)
    nbytes = N * rows * h * 4 + rows * h * 2 * 3 + 2 * h * 4
    out["sp_residual_layernorm"] = {"workload": w.name, "us": us, "gbs": nbytes / us / 1e3,
                                    "frac_hbm_peak": nbytes / us / 1e3 / PEAK_HBM_GBS}
    slices = [rnd(rows, h) for _ in range(N)]
    full = torch.empty(T, h, device="cuda", dtype=torch.bfloat16)
    us = _time_events(lambda: shard.all_gather_rows(slices, b, sq, out=full), reps, warmup, stream)
    nbytes = 2 * T * h * 2
    out["all_gather_rows"] = {"workload": w.name, "us": us, "gbs": nbytes / us / 1e3,
                              "frac_hbm_peak": nbytes / us / 1e3 / PEAK_HBM_GBS}
    del parts, resid, H_, Y_, slices, full
    # backward pass of the MLP shard
    w = WORKLOADS["mlp_bwd_bf16_t4096_h8192_f32768_n8"]
    T, h, fl, N = w.tokens, w.hidden, w.ffn // w.n_shards, w.n_shards
    X, A_i, a_i, B_i, dZ = rnd(T, h), rnd(fl, h, std=0.02), rnd(fl, std=0.02), rnd(h, fl, std=0.02), rnd(T, h)
    grads = {"dX": torch.empty(T, h, device="cuda"), "dA": torch.empty(fl, h, device="cuda"),
             "da": torch.empty(fl, device="cuda"), "dB": torch.empty(h, fl, device="cuda")}
    ws = shard.mlp_bwd_workspace(T, h, w.ffn, N)
    us = _time_events(lambda: shard.mlp_shard_backward(X, A_i, a_i, B_i, dZ, N, 0, out=grads,
                                                       workspace=ws), reps, warmup, stream)
    fl_ = 4 * 2.0 * T * h * fl   # dY, dX, dA, dB (the recomputed P is not counted)
    out["mlp_shard_backward"] = {"workload": w.name, "us": us, "tflops": fl_ / us / 1e6,
                                 "frac_bf16_peak": fl_ / us / 1e6 / PEAK_BF16_TFLOPS,
                                 "note": "algorithmic FLOPs of the four gradient products; the "
                                         "call also recomputes P (one more GEMM) and transposes "
                                         "six operands"}
    # the same backward on the P kept by the forward (tp_mlp_shard_fwd_save, outside the
    # timed region): the four gradient products and the transposes, no recomputation
    _, P, fws = shard.mlp_shard_save(X, A_i, a_i, B_i, N, 0)
    us_s = _time_events(lambda: shard.mlp_shard_backward(X, A_i, a_i, B_i, dZ, N, 0, out=grads,
                                                         workspace=ws, P=P), reps, warmup, stream)
    out["mlp_shard_backward_saved_p"] = {
        "workload": w.name, "us": us_s, "tflops": fl_ / us_s / 1e6,
        "frac_bf16_peak": fl_ / us_s / 1e6 / PEAK_BF16_TFLOPS,
        "note": "tp_mlp_shard_bwd_saved on the forward's P (same bits as the recomputing call)"}
    fz = torch.empty(T, h, device="cuda")
    us_f = _time_events(lambda: shard.mlp_shard(X, A_i, a_i, B_i, N, 0, Z=fz, workspace=fws),
                        reps, warmup, stream)
    us_fs = _time_events(lambda: shard.mlp_shard_save(X, A_i, a_i, B_i, N, 0, Z=fz, P=P,
                                                      workspace=fws), reps, warmup, stream)
    out["mlp_shard_forward_keeping_p"] = {
        "workload": w.name, "us_plain": us_f, "us_keeping_p": us_fs,
        "note": "tp_mlp_shard_fwd against tp_mlp_shard_fwd_save, which also stores P (bf16)"}
    del X, A_i, a_i, B_i, dZ, grads, ws, P, fws, fz
    torch.cuda.synchronize()
    return out


# ---- the CPU oracle: timings on the same units, and parity of the timed outputs ---------------
def _threads_used() -> int:
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the OpenMP count only
        blas = 1
    return int(max(oracle.threads(), blas))


def _timed(fn):
    t0 = time.perf_counter()
    r = fn()
    return r, time.perf_counter() - t0


def cpu_leg(layer, ctx) -> dict:
    """Time the fp64 oracle on each workload's unit (or a stated row sample of it) and compare
    its results with the GPU's outputs of the timed runs. Returns {"layer": cpu_baseline,
    workload: cpu_baseline, ..., "parity": {...}}."""
    import numpy as np
    import oracle
    from synth import WORKLOADS, sample_rows
    oracle._load()
    cores = _threads_used()
    res, parity = {}, {}

    def base(flops, dt, sample, unit="TFLOP/s", extra=None):
        b = {"value": flops / dt / 1e12, "unit": unit, "cores": cores, "kind": "oracle",
             "sample": sample + "; %.2f GFLOP in %.3f s" % (flops / 1e9, dt)}
        if extra:
            b.update(extra)
        return b

    # layer step, rank 0: attention partial on X and MLP partial on the GPU's own H, all rows
    w, d, g = layer["w"], layer["d"], layer["gpu"]
    T, h, N, H = w.tokens, w.hidden, w.n_shards, w.heads
    fl = stage_flops(w)
    Za, ta = _timed(lambda: oracle.attn_shard(d["X"], d["Wq"], d["Wk"], d["Wv"], d["bq"], d["bk"],
                                              d["bv"], d["Wo"], w.batch, w.seq, H, N, 0, w.causal))
    Zm, tm = _timed(lambda: oracle.mlp_shard(g["H"], d["A"], d["a"], d["B"], N, 0))
    rows = sample_rows(T, 32, seed=5, must=[0, 127, 128, 4095])
    Zz = oracle.mlp_shard(g["H"][rows], d["A"], d["a"], d["B"], 1, 0)
    parity[w.name] = {"attention_partial": oracle.rel_frobenius(g["Z_attn"], Za),
                      "mlp_partial_on_gpu_H": oracle.rel_frobenius(g["Z_mlp"], Zm),
                      "layer_output_sampled_rows": oracle.rel_frobenius(g["out"][rows], Zz),
                      "tol": TOL["bf16"]}
    res[w.name] = base(sum(fl.values()), ta + tm,
                       "rank 0 of the layer shard on all %d token rows: fp64 attention partial "
                       "and fp64 MLP partial (on the GPU's bf16 H)" % T)

    # fp32 MLP block: both shards and the sum, all threads (median of 3) and one thread
    c = ctx[W_MLP_F32]
    d1 = c["d"]
    w1 = WORKLOADS[W_MLP_F32]
    f1 = 2 * 2.0 * w1.tokens * w1.hidden * w1.ffn

    def blk():
        return oracle.sum_partials(np.stack([oracle.mlp_shard(d1["X"], d1["A"], d1["a"], d1["B"],
                                                              w1.n_shards, r).astype(np.float32)
                                             for r in range(w1.n_shards)]))
    times = []
    for _ in range(3):
        Zb, t = _timed(blk)
        times.append(t)
    t_all = sorted(times)[1]
    one = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            _, t1 = _timed(blk)
        one = {"value": f1 / t1 / 1e12, "unit": "TFLOP/s", "cores": 1, "seconds": t1}
    except Exception as e:  # threadpoolctl missing or unable to limit the pools
        one = {"value": None, "note": "single-thread run unavailable: %s" % e}
    Zu = oracle.mlp_shard(d1["X"], d1["A"], d1["a"], d1["B"], 1, 0)
    parity[w1.name] = {"block": oracle.rel_frobenius(c["Z"], Zu), "tol": TOL["f32"]}
    res[w1.name] = base(f1, t_all, "the whole block (%d shards and their sum), median of 3"
                        % w1.n_shards, extra={"single_thread": one})

    # bf16 MLP shard, rank 0, all rows
    c = ctx[W_MLP_BF16]
    w2 = WORKLOADS[W_MLP_BF16]
    Z2, t2 = _timed(lambda: oracle.mlp_shard(c["d"]["X"], c["d"]["A"], c["d"]["a"], c["d"]["B"],
                                             w2.n_shards, 0))
    parity[w2.name] = {"shard": oracle.rel_frobenius(c["Z"], Z2), "tol": TOL["bf16"]}
    res[w2.name] = base(4.0 * w2.tokens * w2.hidden * (w2.ffn // w2.n_shards), t2,
                        "rank 0's whole shard (all %d token rows)" % w2.tokens)

    # bf16 attention shard, rank 0, all rows
    c = ctx[W_ATTN]
    w3 = WORKLOADS[W_ATTN]
    d3 = c["d"]
    Z3, t3 = _timed(lambda: oracle.attn_shard(d3["X"], d3["Wq"], d3["Wk"], d3["Wv"], d3["bq"],
                                              d3["bk"], d3["bv"], d3["Wo"], w3.batch, w3.seq,
                                              w3.heads, w3.n_shards, 0, True))
    parity[w3.name] = {"shard": oracle.rel_frobenius(c["Z"], Z3), "tol": TOL["bf16"]}
    dh = w3.hidden // w3.heads
    wl = w3.hidden // w3.n_shards
    T3 = w3.batch * w3.seq
    f3 = (2.0 * T3 * w3.hidden * 3 * wl + 4.0 * dh * (w3.seq * (w3.seq + 1) // 2)
          * (w3.heads // w3.n_shards) * w3.batch + 2.0 * T3 * wl * w3.hidden)
    res[w3.name] = base(f3, t3, "rank 0's whole shard (all %d token rows)" % T3)

    # large MLP block, N = 1 .. 8: a 64-row sample, the block (= the N = 1 shard) and rank 0's
    # shard at N = 8; parity of every N's block sum and of the N = 8 shard on those rows
    c = ctx[W_BLOCK]
    w5 = WORKLOADS[W_BLOCK]
    rows5 = sample_rows(w5.tokens, 64, seed=6, must=[0, 255, 256, 2047])
    X5 = _host(c["X"][rows5])
    A5, a5, B5 = _host32(c["At"]).T, _host32(c["a"]), _host32(c["Bt"]).T
    Zb5, tb5 = _timed(lambda: oracle.mlp_shard(X5, A5, a5, B5, 1, 0))
    Zs5, ts5 = _timed(lambda: oracle.mlp_shard(X5, A5, a5, B5, 8, 0))
    par5 = {"tol": TOL["bf16"]}
    for N5, k in c["keep"].items():
        par5["block_N=%d" % N5] = oracle.rel_frobenius(_host(k["block"])[rows5], Zb5)
    par5["shard0_N=8"] = oracle.rel_frobenius(_host(c["keep"][8]["shard0"])[rows5], Zs5)
    parity[w5.name] = par5
    f5 = 4.0 * len(rows5) * w5.hidden * w5.ffn
    res[w5.name] = base(f5, tb5, "the block on %d sampled token rows (N = 1: the block is one "
                        "shard)" % len(rows5),
                        extra={"per_shard_n8": base(f5 / 8, ts5, "rank 0's shard at N = 8 on "
                                                    "the same %d rows" % len(rows5))})
    res["parity"] = parity
    return res


def parity_failures(parity: dict) -> list:
    bad = []
    for name, p in parity.items():
        tol = p["tol"]
        for k, v in p.items():
            if k != "tol" and not (v <= tol):
                bad.append("%s %s: %.3e > %.0e" % (name, k, v, tol))
    return bad


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The shader clock settles over the first tens of milliseconds of sustained MFMA work
    # (the chip is power-limited under these GEMMs), so the default warm-up is long.
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU-oracle timings and the parity check of the timed outputs")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the other measured workloads and the timings of the gated MLP, "
                         "GQA, sequence-parallel and backward paths")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy 5 times (the reference transfer "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.ones(64 << 20, device="cuda", dtype=torch.float32)   # 256 MiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied 5 x 256 MiB")
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: every tensor-parallel shard runs on a single device "
              "(the all-reduce is an on-device sum), so --gpus must be 1.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from synth import WORKLOADS, attn_inputs
    from tensor_transformer_layers_amd import shard
    from tensor_transformer_layers_amd import binding

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    binding.lib()   # fails loudly if the HIP library is not built
    torch.cuda.set_device(0)
    w = WORKLOADS[WORKLOAD]
    T, h, H, F, N = w.tokens, w.hidden, w.heads, w.ffn, w.n_shards
    wl, Fl = h // N, F // N

    t0 = time.perf_counter()
    log("drawing synthetic inputs for %s" % WORKLOAD)
    d = attn_inputs(w, seed=0)
    log("inputs drawn in %.1f s; uploading" % (time.perf_counter() - t0))

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()

    X = up(d["X"])
    # Full weights in the pages' [in, out] layout, transposed on the device to [out, in];
    # rank r's shards are then row blocks (column-parallel) or column blocks (row-parallel).
    WqT, WkT, WvT, WoT = (up(d[k]).t().contiguous() for k in ("Wq", "Wk", "Wv", "Wo"))
    AT, BT = up(d["A"]).t().contiguous(), up(d["B"]).t().contiguous()
    bq, bk, bv, a = (up(d[k]) for k in ("bq", "bk", "bv", "a"))
    ranks = []
    for r in range(N):
        c, cf = slice(r * wl, (r + 1) * wl), slice(r * Fl, (r + 1) * Fl)
        ranks.append(dict(
            Wqkv=torch.cat([WqT[c], WkT[c], WvT[c]]).contiguous(),
            bqkv=torch.cat([bq[c], bk[c], bv[c]]).contiguous(),
            Wo=WoT[:, c].contiguous(), A=AT[cf].contiguous(), a=a[cf].contiguous(),
            B=BT[:, cf].contiguous()))
    del WqT, WkT, WvT, WoT, AT, BT
    torch.cuda.synchronize()
    log("weights of %d ranks resident; computing the other ranks' partials" % N)

    # Peers' partials: attention of ranks 1..N-1 on X, then the MLP of ranks 1..N-1 on H.
    za = [shard.attn_shard(X, ranks[r]["Wqkv"], ranks[r]["bqkv"], ranks[r]["Wo"], w.batch,
                           w.seq, H, N, r, w.causal)[0] for r in range(N)]
    Hs = shard.sum_partials(za, out_dtype=torch.bfloat16)
    zm = [shard.row_parallel(shard.column_parallel(Hs, ranks[r]["A"], ranks[r]["a"], N, r,
                                                   gelu=True), ranks[r]["B"], N, r)
          for r in range(N)]
    za_other, zm_other = za[1:], zm[1:]
    del za[0], zm[0], Hs
    R0 = ranks[0]
    stream = torch.cuda.current_stream()
    fl = stage_flops(w)
    flop_step = sum(fl.values())
    # Two forms of the same step, the same bits of H and of the output: the unfused one writes
    # the rank's fp32 partials and sums them with tp_sum_partials; the fused one adds the
    # peers' partials in the row-parallel products' epilogues (tp_row_parallel_sum_fwd).
    variants = {}
    for fused in (False, True):
        name = "fused_sums" if fused else "separate_sums"
        log("%s: warmup (%d steps), instrumented and timed steps (%d each)"
            % (name, args.warmup, args.steps))
        drv = shard.LayerShard(w.batch, w.seq, h, H, F, N, rank=0, causal=w.causal, fused=fused)
        variants[name] = time_layer_step(drv, lambda drv=drv, on_stage=None: drv.forward(
            X, R0["Wqkv"], R0["bqkv"], R0["Wo"], R0["A"], R0["a"], R0["B"], za_other, zm_other,
            stream=stream, on_stage=on_stage), w, fl, args.steps, args.warmup, stream)
        variants[name]["drv"] = drv
    a_, b_ = variants["separate_sums"]["drv"], variants["fused_sums"]["drv"]
    if not (torch.equal(a_.out, b_.out) and torch.equal(a_.H, b_.H)):
        log("the fused and unfused steps differ")
        return 1
    if not bool(torch.isfinite(a_.out).all()):
        log("non-finite output")
        return 1
    best = min(variants, key=lambda k: variants[k]["ms_per_step"])
    v = variants[best]
    ms_per_step = v["ms_per_step"]
    value = flop_step / (ms_per_step * 1e-3) / 1e12
    unf = variants["separate_sums"]
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": w.batch, "seq": w.seq, "hidden": h,
                   "heads": H, "head_dim": h // H, "ffn": F, "n_shards": N, "rank": 0,
                   "causal": w.causal, "flop_per_step": flop_step,
                   "step": "attention shard, sum of %d partials, MLP shard, sum of %d partials"
                           % (N, N),
                   "step_form": best},
        "pct_of_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        # the shard kernels alone (the separate-sums form, whose sums are kernels of their own)
        "shard_tflops": (flop_step / ((unf["stage_us"]["attention_shard"]
                                       + unf["stage_us"]["mlp_column"]
                                       + unf["stage_us"]["mlp_row"]) * 1e-6) / 1e12),
        "event_ms_per_step": v["event_ms"],
        "breakdown": v["breakdown"],
        "roofline": v["roofline"],
        "clock": v["clock"],
        "step_forms": {k: {"ms_per_step": x["ms_per_step"],
                           "tflops": flop_step / (x["ms_per_step"] * 1e-3) / 1e12,
                           "breakdown": x["breakdown"], "roofline": x["roofline"],
                           "clock": x["clock"]} for k, x in variants.items()},
        "cpu_baseline": None,
    }
    layer = {"w": w, "d": d, "gpu": {"H": _host(a_.H), "Z_attn": _host(a_.Z_attn),
                                     "Z_mlp": _host(a_.Z_mlp), "out": _host(a_.out)}}
    configs = {WORKLOAD: {"workload": WORKLOAD, "unit": "one rank's layer step (rank 0 of %d)" % N,
                          "dtype": "bf16", "us": ms_per_step * 1e3, "tflops": value,
                          "peak": PEAK_BF16_TFLOPS, "frac_peak": value / PEAK_BF16_TFLOPS,
                          "step_form": best, "roofline": v["roofline"]}}
    del variants, a_, b_, v
    del ranks, za_other, zm_other, X
    torch.cuda.empty_cache()
    ctx = {}
    if not args.no_next_rows:
        for name, fn in ((W_MLP_F32, measure_mlp_f32), (W_MLP_BF16, measure_mlp_bf16),
                         (W_ATTN, measure_attn), (W_BLOCK, measure_block_sweep)):
            log("timing %s" % name)
            with ClockSampler() as ck:
                configs[name], ctx[name] = fn()
            configs[name]["clock"] = ck.summary()
            torch.cuda.empty_cache()
        log("timing the paths next to the core shard")
        line["next_rows"] = measure_next_rows()
    line["configs"] = configs
    if not args.no_cpu_baseline:
        log("timing the CPU oracle and checking the timed outputs")
        cb = cpu_leg(layer, ctx) if ctx else cpu_leg_layer_only(layer)
        line["cpu_baseline"] = cb.pop(WORKLOAD)
        line["parity"] = cb.pop("parity")
        for name, b in cb.items():
            configs[name]["cpu_baseline"] = b
        bad = parity_failures(line["parity"])
        if bad:
            print(json.dumps(line), flush=True)
            log("parity failure: " + "; ".join(bad))
            return 1
    print(json.dumps(line), flush=True)
    return 0


def cpu_leg_layer_only(layer) -> dict:
    """The layer step's oracle timing and parity alone (when the other workloads are skipped)."""
    import oracle
    from synth import sample_rows
    oracle._load()
    w, d, g = layer["w"], layer["d"], layer["gpu"]
    fl = stage_flops(w)
    Za, ta = _timed(lambda: oracle.attn_shard(d["X"], d["Wq"], d["Wk"], d["Wv"], d["bq"], d["bk"],
                                              d["bv"], d["Wo"], w.batch, w.seq, w.heads,
                                              w.n_shards, 0, w.causal))
    Zm, tm = _timed(lambda: oracle.mlp_shard(g["H"], d["A"], d["a"], d["B"], w.n_shards, 0))
    rows = sample_rows(w.tokens, 32, seed=5, must=[0, 127, 128, 4095])
    Zz = oracle.mlp_shard(g["H"][rows], d["A"], d["a"], d["B"], 1, 0)
    f = sum(fl.values())
    return {w.name: {"value": f / (ta + tm) / 1e12, "unit": "TFLOP/s", "cores": _threads_used(),
                     "kind": "oracle",
                     "sample": "rank 0 of the layer shard on all %d token rows: fp64 attention "
                               "partial and fp64 MLP partial (on the GPU's bf16 H); %.2f GFLOP "
                               "in %.3f s" % (w.tokens, f / 1e9, ta + tm)},
            "parity": {w.name: {"attention_partial": oracle.rel_frobenius(g["Z_attn"], Za),
                                "mlp_partial_on_gpu_H": oracle.rel_frobenius(g["Z_mlp"], Zm),
                                "layer_output_sampled_rows": oracle.rel_frobenius(g["out"][rows], Zz),
                                "tol": TOL["bf16"]}}}


if __name__ == "__main__":
    sys.exit(main())
