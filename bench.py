#!/usr/bin/env python3
"""Throughput of one tensor-parallel rank's Transformer-layer shard on one MI355X.

Workload (default): one rank (rank 0 of N = 8) of a bf16 layer with hidden 8192, 64 heads of
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
GEMM), whose rate is reported against the bf16 MFMA peak. The fp64 CPU oracle is timed on a bounded sample of the same
workload on the host cores (rank 0, N = 1 only).
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "per-rank TP shard TFLOP/s (MLP + attention) and % of MI355X bf16 MFMA peak"
WORKLOAD = "layer_shard_bf16_b1_s4096_h8192_H64_f32768_n8"
# MI355X bf16 dense MFMA peak: 256 CUs x 4096 FLOP/clk/CU x 2.4 GHz (the published 2.5 PFLOP/s).
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0


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


def cpu_baseline(w, d, rows_n: int):
    """Time the fp64 oracle on the last ``rows_n`` token rows of rank 0's layer shard."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the OpenMP count only
        blas = 1
    T, h, N, H = w.tokens, w.hidden, w.n_shards, w.heads
    rows = np.arange(T - rows_n, T, dtype=np.int64)
    hl, dd = H // N, h // H
    wl = hl * dd
    Fl = w.ffn // N
    # FLOPs the oracle performs for these rows: K and V over every position they see
    # (causal, one sequence), Q, attention, W_O, and the MLP shard on as many rows.
    need = int(rows.max() % w.seq) + 1
    flops = (2 * 2.0 * need * h * wl + 2.0 * rows_n * h * wl
             + sum(4.0 * dd * (int(t % w.seq) + 1) * hl for t in rows)
             + 2.0 * rows_n * wl * h + 2 * 2.0 * rows_n * h * Fl)
    oracle._load()
    t0 = time.perf_counter()
    oracle.attn_shard(d["X"], d["Wq"], d["Wk"], d["Wv"], d["bq"], d["bk"], d["bv"], d["Wo"],
                      w.batch, w.seq, H, N, 0, w.causal, rows=rows)
    oracle.mlp_shard(d["X"][rows], d["A"], d["a"], d["B"], N, 0)
    dt = time.perf_counter() - t0
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(max(oracle.threads(), blas)),
        "kind": "oracle",
        "sample": ("rank 0 of the same layer shard on the last %d token rows: fp64 attention "
                   "partial (K/V projected over all %d positions they see) and fp64 MLP partial "
                   "on those rows; %.1f GFLOP in %.2f s" % (rows_n, need, flops / 1e9, dt)),
    }


def _time_events(fn, reps: int, warmup: int, stream) -> float:
    """Average microseconds per call of fn(), HIP events on ``stream`` around ``reps`` calls."""
    import torch
    for _ in range(warmup):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def measure_next_rows(reps: int = 20, warmup: int = 10) -> dict:
    """Throughput of the paths next to the core shard, each on its named workload.

    Inputs are drawn on the device from a seeded generator with the workload's shapes and
    distributions (activations N(0, 1), weights N(0, 0.02), bf16): only the rank's own shard
    is drawn, the full weights are never needed for timing.
    """
    import torch
    from synth import WORKLOADS
    from tensor_transformer_layers_amd import binding, shard
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
    del X, A_i, a_i, B_i, dZ, grads, ws
    # all N shards of one MLP block, N in {1, 2, 4, 8}: how the shard's GEMM shape moves the
    # MFMA utilisation (column GEMM T x F/N x h, row GEMM T x h x F/N), the whole block (every
    # shard in turn, then the on-device sum) and the sum alone
    w = WORKLOADS["mlp_block_bf16_t2048_h12288_f49152"]
    T, h, F = w.tokens, w.hidden, w.ffn
    X = rnd(T, h)
    sweep = {}
    for N in (1, 2, 4, 8):
        fl = F // N
        A_s = [rnd(fl, h, std=0.02) for _ in range(N)]
        a_s = [rnd(fl, std=0.02) for _ in range(N)]
        B_s = [rnd(h, fl, std=0.02) for _ in range(N)]
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
        del A_s, a_s, B_s, Zs, Zsum, ws
    out["mlp_block_sweep"] = {"workload": w.name, "per_n": sweep}
    del X
    torch.cuda.synchronize()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The shader clock settles over the first tens of milliseconds of sustained MFMA work
    # (the chip is power-limited under these GEMMs), so the default warm-up is long.
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="token rows in the CPU-oracle sample (default: the whole shard)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the timings of the gated MLP, GQA, sequence-parallel and "
                         "backward paths")
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
    from tensor_transformer_layers_amd import binding, shard

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
    drv = shard.LayerShard(w.batch, w.seq, h, H, F, N, rank=0, causal=w.causal)
    R0 = ranks[0]
    stream = torch.cuda.current_stream()

    def step(on_stage=None):
        return drv.forward(X, R0["Wqkv"], R0["bqkv"], R0["Wo"], R0["A"], R0["a"], R0["B"],
                           za_other, zm_other, stream=stream, on_stage=on_stage)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done (%d steps); timing %d steps" % (args.warmup, args.steps))

    stages = shard.LayerShard.STAGES
    # Per-stage breakdown from as many instrumented steps, run before the timed ones: an event
    # after each stage's launches. Each event record leaves the stream idle for a few
    # microseconds, so the timed steps carry only the two events around the dominant kernel.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev[i][0].record(stream)
        marks = iter(ev[i][1:])
        step(on_stage=lambda name, m=marks: next(m).record(stream))
    torch.cuda.synchronize()
    stage_us = {s: 0.0 for s in stages}
    for i in range(args.steps):
        for j, s in enumerate(stages):
            stage_us[s] += ev[i][j].elapsed_time(ev[i][j + 1]) * 1e3 / args.steps
    event_ms = sum(stage_us.values()) / 1e3
    # Dominant kernel: the slower of the two MLP GEMMs (each stage is one kernel launch).
    dom = max(("mlp_column", "mlp_row"), key=lambda s: stage_us[s])
    before = stages[stages.index(dom) - 1]

    dev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]

    def mark_dominant(name, pair):
        if name == before:
            pair[0].record(stream)
        elif name == dom:
            pair[1].record(stream)

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(on_stage=lambda name, pair=dev[i]: mark_dominant(name, pair))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    out = drv.out
    if not bool(torch.isfinite(out).all()):
        log("non-finite output")
        return 1
    ms_per_step = elapsed / args.steps * 1e3
    dom_us = sum(a.elapsed_time(b) for a, b in dev) * 1e3 / args.steps

    fl = stage_flops(w)
    flop_step = sum(fl.values())
    value = flop_step / (ms_per_step * 1e-3) / 1e12
    sum_bytes = {"sum_attention": (N * 4 + 2) * T * h, "sum_mlp": (N * 4 + 4) * T * h}
    attn_flops = fl["qkv_projection"] + fl["attention"] + fl["out_projection"]
    breakdown = {
        "attention_shard": {"us": stage_us["attention_shard"],
                            "tflops": attn_flops / stage_us["attention_shard"] / 1e6},
        "mlp_column": {"us": stage_us["mlp_column"],
                       "tflops": fl["mlp_column"] / stage_us["mlp_column"] / 1e6},
        "mlp_row": {"us": stage_us["mlp_row"], "tflops": fl["mlp_row"] / stage_us["mlp_row"] / 1e6},
        "sum_attention": {"us": stage_us["sum_attention"],
                          "gbs": sum_bytes["sum_attention"] / stage_us["sum_attention"] / 1e3},
        "sum_mlp": {"us": stage_us["sum_mlp"], "gbs": sum_bytes["sum_mlp"] / stage_us["sum_mlp"] / 1e3},
    }
    # The dominant kernel named as the profiler names it:
    # gemm_bf16_kernel<tile_m, tile_n, waves_m, waves_n, epilogue>; its rate from the timed steps.
    M, Nn, K = (T, Fl, h) if dom == "mlp_column" else (T, h, Fl)
    _, tbm, tbn, nw = binding.tp_gemm_tile_info(M, Nn, K)
    wgrid = {(256, 256, 8): (2, 4), (256, 192, 8): (4, 2), (256, 128, 8): (4, 2),
             (128, 128, 8): (2, 4)}.get((tbm, tbn, nw), (2, 2))
    kname = "gemm_bf16_kernel<%d, %d, %d, %d, (tps::Epi)%d>" % (
        tbm, tbn, wgrid[0], wgrid[1], 0 if dom == "mlp_column" else 1)
    achieved = fl[dom] / (dom_us * 1e-6) / 1e12
    roofline = {"bound": "mfma", "kernel": kname, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": traffic_for(kname, dom)}

    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": w.batch, "seq": w.seq, "hidden": h,
                   "heads": H, "head_dim": h // H, "ffn": F, "n_shards": N, "rank": 0,
                   "causal": w.causal, "flop_per_step": flop_step,
                   "step": "attention shard, sum of %d partials, MLP shard, sum of %d partials"
                           % (N, N)},
        "pct_of_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "shard_tflops": (flop_step / ((stage_us["attention_shard"] + stage_us["mlp_column"]
                                       + stage_us["mlp_row"]) * 1e-6) / 1e12),
        "event_ms_per_step": event_ms,
        "breakdown": breakdown,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    del ranks, za_other, zm_other, drv
    torch.cuda.empty_cache()
    if not args.no_next_rows:
        log("timing the paths next to the core shard")
        line["next_rows"] = measure_next_rows()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a %d-row sample" % args.cpu_rows)
        line["cpu_baseline"] = cpu_baseline(w, d, args.cpu_rows)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
