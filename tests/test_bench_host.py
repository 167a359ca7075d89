"""Host-side checks of the benchmark's bookkeeping (no GPU): the algorithmic FLOP count of the
layer step, the counter-summary lookup and its source-hash guard, and the single-GPU refusal."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import WORKLOADS  # noqa: E402

LAYER = "layer_shard_bf16_b1_s4096_h8192_H64_f32768_n8"


def test_layer_step_flops():
    # rank 0 of N = 8 at hidden 8192, 64 heads of 128, ffn 32768, one causal sequence of 4096:
    # 8 local heads (1024 columns), ffn shard 4096; attention counts the s(s+1)/2 triangle.
    fl = bench.stage_flops(WORKLOADS[LAYER])
    assert fl["qkv_projection"] == 206_158_430_208        # 2 x 4096 x 8192 x 3072
    assert fl["out_projection"] == 68_719_476_736         # 2 x 4096 x 1024 x 8192
    assert fl["mlp_column"] == 274_877_906_944            # 2 x 4096 x 8192 x 4096
    assert fl["mlp_row"] == 274_877_906_944
    assert fl["attention"] == 34_368_126_976              # 4 x 128 x 8390656 x 8
    assert sum(fl.values()) == 859_001_847_808


def test_traffic_lookup_and_hash_guard(monkeypatch):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        pytest.skip("no committed counter summary")
    rec = json.load(open(path))
    name, k = next((n, k) for n, k in rec["kernels"].items() if k["stage"] == "mlp_column")
    kernel = name.split(" [")[0]
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: rec["source_sha"])
    assert bench.traffic_for(kernel, "mlp_column") == k["hbm_bytes_per_launch"]
    assert bench.traffic_for(kernel, "mlp_row") is None       # the column kernel, other stage
    assert bench.traffic_for("no_such_kernel<1>", "mlp_column") is None
    # other kernel sources: the figures no longer describe the library, so none is reported
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0" * 16)
    assert bench.traffic_for(kernel, "mlp_column") is None


def test_source_hash_covers_the_kernel_sources():
    h = bench.kernel_source_sha()
    assert len(h) == 16 and int(h, 16) >= 0
    assert h == bench.kernel_source_sha()


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "8"})])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, env=e,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr
    assert r.stdout == ""


def test_parity_failures_flag_errors_above_tolerance_and_nan():
    good = {"w": {"a": 1e-3, "b": 9.9e-3, "tol": 1e-2}}
    assert bench.parity_failures(good) == []
    bad = {"w": {"a": 1e-3, "b": 2e-2, "tol": 1e-2}, "f32": {"block": float("nan"), "tol": 1e-4}}
    msgs = bench.parity_failures(bad)
    assert len(msgs) == 2 and any("w b" in m for m in msgs) and any("f32 block" in m for m in msgs)


def test_clock_sampler_reports_what_it_can_read(tmp_path):
    s = bench.ClockSampler()
    with s:
        pass
    out = s.summary()
    assert "mhz_mean" in out
    # a dpm table with the active level starred, as the driver prints it
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1800Mhz *\n2: 2400Mhz\n")
    s.source = ("dpm", str(f))
    assert s._read() == 1800.0
    f2 = tmp_path / "freq1_input"
    f2.write_text("2100000000\n")
    s.source = ("hwmon", str(f2))
    assert s._read() == 2100.0


def test_layer_stage_costs_and_bounds():
    """Algorithmic FLOPs and bytes of the layer step's one-kernel stages, and the roofline each
    is rated against: the MFMA GEMMs against the bf16 peak, the sums (and the products with
    the sum fused in, whose 7 x 134 MB of peer partials take longer at 8 TB/s than their
    FLOPs at 2.5 PFLOP/s) against HBM."""
    w = WORKLOADS[LAYER]
    f, b = bench.layer_stage_cost(w, "mlp_column")
    assert f == 274_877_906_944 and b == 2 * (4096 * 8192 + 4096 * 8192 + 4096 + 4096 * 4096)
    f, b = bench.layer_stage_cost(w, "mlp_row_sum")
    assert b == 2 * (4096 * 4096 + 8192 * 4096) + 7 * 4 * 4096 * 8192 + 4 * 4096 * 8192
    assert bench.layer_stage_cost(w, "attention_shard") is None
    assert bench.layer_stage_cost(w, "sum_mlp") == (0.0, (8 * 4 + 4) * 4096 * 8192)
    for s, want in (("mlp_column", "mfma"), ("mlp_row", "mfma"), ("qkv_projection", "mfma"),
                    ("mlp_row_sum", "hbm"), ("out_projection_sum", "hbm"), ("sum_mlp", "hbm")):
        f, b = bench.layer_stage_cost(w, s)
        got = "hbm" if b / (bench.PEAK_HBM_GBS * 1e9) > f / (bench.PEAK_BF16_TFLOPS * 1e12) else "mfma"
        assert got == want, s
