"""GPU parity of tp_mlp_shard_bwd (backward pass of the MLP shard) against the fp64 oracle,
and of the pair that keeps P from the forward (tp_mlp_shard_fwd_save, tp_mlp_shard_bwd_saved)
against the recomputing calls, bitwise.

The oracle's gradients (themselves pinned against finite differences of the forward oracle)
are dX (rank's partial), dA [h, F/N], da and dB [F/N, h]; the library returns dA and dB in
the stored weight layouts, i.e. transposed. bf16 inputs with fp32 accumulation; P, dP and
GeLU(P) pass through bf16: tolerance 1e-2 relative Frobenius error.
"""
import numpy as np
import pytest

import oracle
from gpu_util import Canary, canary_tensor, dev, host, torch_cuda
from synth import WORKLOADS, Workload, bf16_round, mlp_inputs
from tensor_transformer_layers_amd import layout

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _dz(T, h, seed):
    rng = np.random.default_rng(seed + 9973)
    return bf16_round(rng.standard_normal((T, h)).astype(np.float32))


def run_bwd(d, dZ, N, r, bias=True, P=None):
    torch = torch_cuda()
    from tensor_transformer_layers_amd import binding as B
    from tensor_transformer_layers_amd import shard
    T, h = d["X"].shape
    F = d["A"].shape[1]
    fl = F // N
    X = dev(d["X"], "bf16")
    A_i = dev(layout.column_shard(d["A"], N, r), "bf16")
    a_i = dev(layout.bias_shard(d["a"], N, r), "bf16") if bias else None
    B_i = dev(layout.row_shard(d["B"], N, r), "bf16")
    out = {"dX": canary_tensor((T, h), torch.float32), "dA": canary_tensor((fl, h), torch.float32),
           "da": canary_tensor((fl,), torch.float32), "dB": canary_tensor((h, fl), torch.float32)}
    ws = Canary(B.tp_mlp_bwd_workspace_bytes(T, h, F, N, B.TP_BF16), torch.uint8, None)
    shard.mlp_shard_backward(X, A_i, a_i, B_i, dev(dZ, "bf16"), N, r,
                             out={k: c.tensor for k, c in out.items()}, workspace=ws.body, P=P)
    torch.cuda.synchronize()
    assert all(c.intact() for c in out.values()) and ws.intact(), "write outside a buffer"
    return {k: host(c.tensor) for k, c in out.items()}


def _compare(got, ref, what):
    e = {"dX": oracle.rel_frobenius(got["dX"], ref["dX"]),
         "dA": oracle.rel_frobenius(got["dA"], ref["dA"].T),
         "da": oracle.rel_frobenius(got["da"], ref["da"]),
         "dB": oracle.rel_frobenius(got["dB"], ref["dB"].T)}
    print(what, " ".join("%s %.2e" % kv for kv in e.items()))
    assert all(v < TOL for v in e.values()), e


@pytest.mark.parametrize("T,h,F,N", [(1, 64, 128, 1), (37, 200, 480, 2), (300, 264, 1040, 2),
                                     (129, 512, 2048, 4), (64, 1024, 4096, 8)])
def test_mlp_backward_small(T, h, F, N):
    w = Workload(name="b", kind="mlp_bwd", dtype="bf16", tokens=T, hidden=h, ffn=F, n_shards=N)
    d = mlp_inputs(w, seed=T + F)
    dZ = _dz(T, h, T)
    for r in sorted({0, N - 1}):
        got = run_bwd(d, dZ, N, r)
        ref = oracle.mlp_shard_backward(d["X"], d["A"], d["a"], d["B"], dZ, N, r)
        _compare(got, ref, "T=%d h=%d F=%d N=%d r=%d:" % (T, h, F, N, r))


@pytest.mark.parametrize("tile", ["256x256w4", "128x128w4", "256x192", "256x192w4"])
@pytest.mark.parametrize("T,h,F,N", [(37, 200, 480, 2), (300, 264, 1040, 2)])
def test_mlp_backward_small_forced_tiles(T, h, F, N, tile, overrides):
    """The same gradients with every GEMM of the call forced onto one tile layout (the
    GeLU' epilogue and the fp32 products in the 4-wave layouts, on ragged shapes)."""
    overrides("gemm_tile=" + tile)
    test_mlp_backward_small(T, h, F, N)


def test_mlp_backward_input_gradient_all_reduce():
    """The ranks' dX partials summed on the device = the unsharded block's dX."""
    torch = torch_cuda()
    from tensor_transformer_layers_amd import shard
    T, h, F = 96, 256, 1024
    w = Workload(name="b", kind="mlp_bwd", dtype="bf16", tokens=T, hidden=h, ffn=F, n_shards=4)
    d = mlp_inputs(w, seed=2)
    dZ = _dz(T, h, 2)
    ref = oracle.mlp_shard_backward(d["X"], d["A"], d["a"], d["B"], dZ, 1, 0)["dX"]
    for N in (2, 4):
        parts = [dev(run_bwd(d, dZ, N, r)["dX"].astype(np.float32), "f32") for r in range(N)]
        e = oracle.rel_frobenius(host(shard.sum_partials(parts)), ref)
        print("N=%d dX after the sum: %.2e" % (N, e))
        assert e < TOL
    torch.cuda.synchronize()


def test_mlp_backward_full_size():
    """One rank's backward at T 4096, h 8192, F 32768, N 8 (the layer's MLP shard)."""
    w = WORKLOADS["mlp_bwd_bf16_t4096_h8192_f32768_n8"]
    d = mlp_inputs(w)
    N, r = w.n_shards, 5
    dZ = _dz(w.tokens, w.hidden, 0)
    got = run_bwd(d, dZ, N, r)
    ref = oracle.mlp_shard_backward(d["X"], d["A"], d["a"], d["B"], dZ, N, r)
    _compare(got, ref, "full size r=%d:" % r)
    assert all(np.isfinite(v).all() for v in got.values())


def run_save(d, N, r, bias=True):
    """tp_mlp_shard_fwd_save: (Z_i, P_i on the device, P_i on the host), with guard bands
    around both outputs and the workspace."""
    torch = torch_cuda()
    from tensor_transformer_layers_amd import binding as B
    from tensor_transformer_layers_amd import shard
    T, h = d["X"].shape
    F = d["A"].shape[1]
    fl = F // N
    X = dev(d["X"], "bf16")
    A_i = dev(layout.column_shard(d["A"], N, r), "bf16")
    a_i = dev(layout.bias_shard(d["a"], N, r), "bf16") if bias else None
    B_i = dev(layout.row_shard(d["B"], N, r), "bf16")
    Z = canary_tensor((T, h), torch.float32)
    P = canary_tensor((T, fl), torch.bfloat16)
    ws = Canary(B.tp_mlp_workspace_bytes(T, h, F, N, B.TP_BF16), torch.uint8, None)
    shard.mlp_shard_save(X, A_i, a_i, B_i, N, r, Z=Z.tensor, P=P.tensor, workspace=ws.body)
    torch.cuda.synchronize()
    assert Z.intact() and P.intact() and ws.intact(), "write outside a buffer"
    return host(Z.tensor), P.tensor, host(P.tensor)


SAVE_SHAPES = [(1, 64, 128, 1), (37, 200, 480, 2), (300, 264, 1040, 2), (129, 512, 2048, 4)]


@pytest.mark.parametrize("T,h,F,N", SAVE_SHAPES)
@pytest.mark.parametrize("bias", [True, False])
def test_mlp_fwd_save_and_bwd_saved_bitwise(T, h, F, N, bias):
    """The forward that keeps P gives tp_mlp_shard_fwd's Z bits and the P that the column
    primitive without activation computes (the same accumulators, rounded once after the
    bias); the backward that takes it gives tp_mlp_shard_bwd's bits for every gradient."""
    from tensor_transformer_layers_amd import shard
    w = Workload(name="s", kind="mlp_bwd", dtype="bf16", tokens=T, hidden=h, ffn=F, n_shards=N)
    d = mlp_inputs(w, seed=3 * T + F)
    dZ = _dz(T, h, T + 1)
    for r in sorted({0, N - 1}):
        Zs, P_dev, P = run_save(d, N, r, bias)
        X = dev(d["X"], "bf16")
        A_i = dev(layout.column_shard(d["A"], N, r), "bf16")
        a_i = dev(layout.bias_shard(d["a"], N, r), "bf16") if bias else None
        B_i = dev(layout.row_shard(d["B"], N, r), "bf16")
        Z, _ = shard.mlp_shard(X, A_i, a_i, B_i, N, r)
        P_ref = host(shard.column_parallel(X, A_i, a_i, N, r, gelu=False))
        # (host() widens to fp64 exactly, so equal arrays are equal bits up to the sign of 0)
        assert np.array_equal(Zs, host(Z)), "Z differs from tp_mlp_shard_fwd"
        assert np.array_equal(P, P_ref), "P differs from the column primitive's"
        cols = slice(r * (F // N), (r + 1) * (F // N))
        P_or = oracle.linear(d["X"], d["A"][:, cols], d["a"][cols] if bias else None)
        assert oracle.rel_frobenius(P, P_or) < TOL
        got = run_bwd(d, dZ, N, r, bias=bias, P=P_dev)
        rec = run_bwd(d, dZ, N, r, bias=bias)
        for k in ("dX", "dA", "da", "dB"):
            assert np.array_equal(got[k], rec[k]), k
        a = d["a"] if bias else np.zeros_like(d["a"])
        ref = oracle.mlp_shard_backward(d["X"], d["A"], a, d["B"], dZ, N, r)
        _compare(got, ref, "saved P, bias %s, T=%d h=%d F=%d N=%d r=%d:" % (bias, T, h, F, N, r))


@pytest.mark.parametrize("tile", ["256x256w4", "128x128w4", "256x192"])
def test_mlp_fwd_save_and_bwd_saved_forced_tiles(tile, overrides):
    """The same bitwise checks with every GEMM forced onto one tile layout (the P store in
    the 8- and 4-wave epilogues), on ragged shapes."""
    overrides("gemm_tile=" + tile)
    for T, h, F, N in SAVE_SHAPES[1:3]:
        test_mlp_fwd_save_and_bwd_saved_bitwise(T, h, F, N, True)


def test_mlp_bwd_saved_full_size():
    """At the layer's MLP shard (T 4096, h 8192, F 32768, N 8, rank 5): the saved-P backward
    equals the recomputing one bitwise, and the oracle within the tolerance."""
    w = WORKLOADS["mlp_bwd_bf16_t4096_h8192_f32768_n8"]
    d = mlp_inputs(w)
    N, r = w.n_shards, 5
    dZ = _dz(w.tokens, w.hidden, 0)
    _, P_dev, _ = run_save(d, N, r)
    got = run_bwd(d, dZ, N, r, P=P_dev)
    rec = run_bwd(d, dZ, N, r)
    for k in ("dX", "dA", "da", "dB"):
        assert np.array_equal(got[k], rec[k]), k
    ref = oracle.mlp_shard_backward(d["X"], d["A"], d["a"], d["B"], dZ, N, r)
    _compare(got, ref, "full size, saved P, r=%d:" % r)
