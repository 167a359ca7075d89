"""GPU parity of tp_swiglu_shard_fwd (the gated MLP shard) against the fp64 oracle.

Gated half: A_i = SiLU(X W_gate,i) * (X W_up,i) read from the workspace; down half: the fp32
partial Z_i = A_i W_down,i. bf16 throughout with fp32 accumulation: tolerance 1e-2 relative
Frobenius error, the oracle fed the same bf16-rounded inputs.
"""
import numpy as np
import pytest

import oracle
from gpu_util import Canary, canary_tensor, dev, host, torch_cuda
from synth import WORKLOADS, Workload, sample_rows, swiglu_inputs
from tensor_transformer_layers_amd import layout

pytestmark = pytest.mark.gpu
TOL = 1e-2


def run_shard(d, N, r):
    """Rank r's gated shard on the GPU; returns (A_i, Z_i) on the host in fp64."""
    torch = torch_cuda()
    from tensor_transformer_layers_amd import binding as B
    from tensor_transformer_layers_amd import shard
    X = dev(d["X"], "bf16")
    Wg = dev(layout.column_shard(d["Wg"], N, r), "bf16")
    Wu = dev(layout.column_shard(d["Wu"], N, r), "bf16")
    Wd = dev(layout.row_shard(d["Wd"], N, r), "bf16")
    T, h = d["X"].shape
    F = d["Wg"].shape[1]
    Zc = canary_tensor((T, h), torch.float32)
    ws = Canary(B.tp_swiglu_workspace_bytes(T, h, F, N, B.TP_BF16), torch.uint8, None)
    shard.swiglu_shard(X, Wg, Wu, Wd, N, r, Z=Zc.tensor, workspace=ws.body)
    torch.cuda.synchronize()
    assert Zc.intact() and ws.intact(), "write outside an output buffer"
    A = host(shard.mlp_hidden_view(ws.body, T, F // N, torch.bfloat16))
    return A, host(Zc.tensor)


RAGGED = [(1, 64, 128, 1), (37, 200, 480, 2), (300, 264, 1040, 2), (513, 520, 2048, 4),
          (129, 1024, 1088, 8)]


@pytest.mark.parametrize("tile", [None, "256x256", "256x128", "128x128w4", "256x256w4",
                                  "256x128w4", "128x128",
                                  "256x192"])   # 256x192 cannot pair blocks: falls back
@pytest.mark.parametrize("shape", RAGGED)
def test_swiglu_ragged_tiles(shape, tile, overrides):
    if tile:
        overrides("gemm_tile=" + tile)
    T, h, F, N = shape
    w = Workload(name="t", kind="swiglu", dtype="bf16", tokens=T, hidden=h, ffn=F, n_shards=N)
    d = swiglu_inputs(w, seed=T + h)
    r = N - 1
    A, Z = run_shard(d, N, r)
    ea = oracle.rel_frobenius(A, oracle.swiglu_column(d["X"], d["Wg"], d["Wu"], N, r))
    ez = oracle.rel_frobenius(Z, oracle.swiglu_shard(d["X"], d["Wg"], d["Wu"], d["Wd"], N, r))
    print("%s tile %s: A err %.2e, Z err %.2e" % (shape, tile, ea, ez))
    assert ea < TOL and ez < TOL


def test_swiglu_shards_sum_to_block():
    """sum over the ranks' partials (on-device sum) = the unsharded gated MLP block."""
    torch = torch_cuda()
    from tensor_transformer_layers_amd import shard
    w = Workload(name="t", kind="swiglu", dtype="bf16", tokens=200, hidden=512, ffn=4096,
                 n_shards=4)
    d = swiglu_inputs(w, seed=5)
    ref = oracle.swiglu_shard(d["X"], d["Wg"], d["Wu"], d["Wd"], 1, 0)
    for N in (1, 2, 4, 8):
        Zs = [dev(run_shard(d, N, r)[1].astype(np.float32), "f32") for r in range(N)]
        tot = host(shard.sum_partials(Zs))
        e = oracle.rel_frobenius(tot, ref)
        print("N=%d block err %.2e" % (N, e))
        assert e < TOL
    torch.cuda.synchronize()


@pytest.mark.parametrize("rank", [0, 7])
def test_swiglu_full_size_shard_sampled_rows(rank):
    """One rank's gated shard at T 4096, h 8192, F 28672, N 8, on 96 sampled rows."""
    w = WORKLOADS["swiglu_shard_bf16_t4096_h8192_f28672_n8"]
    d = swiglu_inputs(w)
    N = w.n_shards
    A, Z = run_shard(d, N, rank)
    rows = sample_rows(w.tokens, 96, seed=rank, must=[255, 256, 4095 - 64])
    Xr = d["X"][rows]
    ea = oracle.rel_frobenius(A[rows], oracle.swiglu_column(Xr, d["Wg"], d["Wu"], N, rank))
    ez = oracle.rel_frobenius(Z[rows], oracle.swiglu_shard(Xr, d["Wg"], d["Wu"], d["Wd"], N, rank))
    print("full-size rank %d: A err %.2e, Z err %.2e" % (rank, ea, ez))
    assert ea < TOL and ez < TOL
    assert np.isfinite(Z).all()
    if rank == 0:
        _, Z2 = run_shard(d, N, rank)
        assert np.array_equal(Z, Z2), "results must be bitwise repeatable"
