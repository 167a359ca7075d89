"""GPU parity of the composed paths: a tensor-parallel layer (attention block, sum, MLP block,
sum) and the all-shards MLP block with its on-device sum across shard counts N."""
import numpy as np
import pytest

import oracle
from gpu_util import dev, host, torch_cuda
from synth import WORKLOADS, Workload, attn_inputs, bf16_round, normal_matrix, sample_rows
from tensor_transformer_layers_amd import layout

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _rank_weights(d, N, r):
    return dict(
        Wqkv=dev(layout.qkv_shard(d["Wq"], d["Wk"], d["Wv"], N, r), "bf16"),
        bqkv=dev(layout.qkv_bias_shard(d["bq"], d["bk"], d["bv"], N, r), "bf16"),
        Wo=dev(layout.row_shard(d["Wo"], N, r), "bf16"),
        A=dev(layout.column_shard(d["A"], N, r), "bf16"),
        a=dev(layout.bias_shard(d["a"], N, r), "bf16"),
        B=dev(layout.row_shard(d["B"], N, r), "bf16"),
    )


def test_layer_all_ranks_end_to_end_small():
    """Z = MLP(Attn(X)) with both blocks split over N = 2 ranks, one on-device sum per block,
    against the oracle's unsharded layer (fp64 throughout)."""
    torch = torch_cuda()
    from tensor_transformer_layers_amd import shard
    batch, seq, h, H, F, N = 2, 96, 512, 4, 1024, 2
    w = Workload(name="layer", kind="layer", dtype="bf16", tokens=batch * seq, batch=batch,
                 seq=seq, hidden=h, heads=H, ffn=F, n_shards=N)
    d = attn_inputs(w, seed=21)
    X = dev(d["X"], "bf16")
    W = [_rank_weights(d, N, r) for r in range(N)]
    za = [shard.attn_shard(X, W[r]["Wqkv"], W[r]["bqkv"], W[r]["Wo"], batch, seq, H, N, r)[0]
          for r in range(N)]
    Hs = shard.sum_partials(za, out_dtype=torch.bfloat16)
    zm = [shard.mlp_shard(Hs, W[r]["A"], W[r]["a"], W[r]["B"], N, r)[0] for r in range(N)]
    Z = shard.sum_partials(zm)
    # the rank-1 driver, fed the other rank's partials, reproduces the same bits
    drv = shard.LayerShard(batch, seq, h, H, F, N, 1)
    Zd = drv.forward(X, W[1]["Wqkv"], W[1]["bqkv"], W[1]["Wo"], W[1]["A"], W[1]["a"], W[1]["B"],
                     [za[0]], [zm[0]])
    torch.cuda.synchronize()
    assert torch.equal(Zd, Z)
    Ho = oracle.attn_shard(d["X"], d["Wq"], d["Wk"], d["Wv"], d["bq"], d["bk"], d["bv"], d["Wo"],
                           batch, seq, H, 1, 0, True)
    Zo = oracle.mlp_shard(Ho, d["A"], d["a"], d["B"], 1, 0)
    eh, ez = oracle.rel_frobenius(host(Hs), Ho), oracle.rel_frobenius(host(Z), Zo)
    print("layer: H err %.2e, Z err %.2e" % (eh, ez))
    assert eh < TOL and ez < TOL


def test_layer_full_size_rank0_blocks_sampled():
    """One rank of the layer at b 1, s 4096, h 8192, 64 heads, F 32768, N 8: the attention
    shard on sampled rows, and the MLP shard on a seeded stand-in for the attention output."""
    torch = torch_cuda()
    from tensor_transformer_layers_amd import shard
    w = WORKLOADS["layer_shard_bf16_b1_s4096_h8192_H64_f32768_n8"]
    d = attn_inputs(w)
    N, r, T = w.n_shards, 0, w.tokens
    W = _rank_weights(d, N, r)
    X = dev(d["X"], "bf16")
    Za, _ = shard.attn_shard(X, W["Wqkv"], W["bqkv"], W["Wo"], w.batch, w.seq, w.heads, N, r)
    rows = sample_rows(T, 16, seed=3, must=[127, 128, 2047])
    Zo = oracle.attn_shard(d["X"], d["Wq"], d["Wk"], d["Wv"], d["bq"], d["bk"], d["bv"],
                           d["Wo"], w.batch, w.seq, w.heads, N, r, True, rows=rows)
    ea = oracle.rel_frobenius(host(Za)[rows], Zo)
    # MLP input: a seeded bf16 matrix of the attention output's shape and scale
    Hin = bf16_round(normal_matrix(np.random.default_rng(99), (T, w.hidden), 1.0))
    Zm, _ = shard.mlp_shard(dev(Hin, "bf16"), W["A"], W["a"], W["B"], N, r)
    Zmo = oracle.mlp_shard(Hin[rows], d["A"], d["a"], d["B"], N, r)
    em = oracle.rel_frobenius(host(Zm)[rows], Zmo)
    print("layer shard full size: attention err %.2e, MLP err %.2e" % (ea, em))
    assert ea < TOL and em < TOL


def test_mlp_block_all_shards_sweep_n():
    """All N shards of the MLP block (T 2048, h 12288, F 49152) plus the on-device sum, for
    N in {1, 2, 4, 8}, against the oracle's unsharded block on sampled rows."""
    torch = torch_cuda()
    from tensor_transformer_layers_amd import shard
    w = WORKLOADS["mlp_block_bf16_t2048_h12288_f49152"]
    from synth import mlp_inputs
    d = mlp_inputs(w)
    rows = sample_rows(w.tokens, 8, seed=1, must=[1023])
    ref = oracle.mlp_shard(d["X"][rows], d["A"], d["a"], d["B"], 1, 0)
    X = dev(d["X"], "bf16")
    At = dev(d["A"].T, "bf16")        # [F, h]: column shards are contiguous row blocks
    Bt = dev(d["B"].T, "bf16")        # [h, F]: row shards are column blocks
    a = dev(d["a"], "bf16")
    F = w.ffn
    results = {}
    for N in (1, 2, 4, 8):
        fl = F // N
        parts = []
        for r in range(N):
            Z, _ = shard.mlp_shard(X, At[r * fl:(r + 1) * fl], a[r * fl:(r + 1) * fl],
                                   Bt[:, r * fl:(r + 1) * fl].contiguous(), N, r)
            parts.append(Z)
        total = host(shard.sum_partials(parts))
        del parts
        e = oracle.rel_frobenius(total[rows], ref)
        results[N] = e
        assert np.isfinite(total).all()
    print("MLP block by N: " + ", ".join("N=%d err %.2e" % kv for kv in results.items()))
    assert max(results.values()) < TOL
