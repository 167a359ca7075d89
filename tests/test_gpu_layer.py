"""GPU parity of the composed paths: a tensor-parallel layer (attention block, sum, MLP block,
sum) and the all-shards MLP block with its on-device sum across shard counts N."""
import numpy as np
import pytest

import oracle
from gpu_util import dev, host, torch_cuda
from synth import WORKLOADS, Workload, attn_inputs, sample_rows
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
    fz = shard.LayerShard(batch, seq, h, H, F, N, 1, fused=True)
    Zf = fz.forward(X, W[1]["Wqkv"], W[1]["bqkv"], W[1]["Wo"], W[1]["A"], W[1]["a"], W[1]["B"],
                    [za[0]], [zm[0]])
    torch.cuda.synchronize()
    assert torch.equal(Zd, Z)
    assert torch.equal(Zf, Z) and torch.equal(fz.H, Hs)
    Ho = oracle.attn_shard(d["X"], d["Wq"], d["Wk"], d["Wv"], d["bq"], d["bk"], d["bv"], d["Wo"],
                           batch, seq, H, 1, 0, True)
    Zo = oracle.mlp_shard(Ho, d["A"], d["a"], d["B"], 1, 0)
    eh, ez = oracle.rel_frobenius(host(Hs), Ho), oracle.rel_frobenius(host(Z), Zo)
    print("layer: H err %.2e, Z err %.2e" % (eh, ez))
    assert eh < TOL and ez < TOL


def test_layer_full_size_composed_step():
    """The layer at b 1, s 4096, h 8192, 64 heads, F 32768, N 8, composed as the benchmark
    composes it: the 8 attention partials, tp_sum_partials into a bf16 H, the 8 MLP partials
    on that H, tp_sum_partials into Z (one sum per block: ai360xpert.com "How It Works";
    llms.blog "Communication Budget and Scaling Limits"). On 40 sampled rows (query-tile and
    sequence edges included) it checks:
      * H against the oracle's unsharded attention block;
      * every rank's MLP partial, and Z, against the oracle fed the GPU's own bf16 H (the
        "same bf16-rounded inputs" rule);
      * Z end to end against the oracle's layer (fp64 throughout).
    Rank 0's LayerShard driver, fed the peers' partials, reproduces Z bitwise."""
    torch = torch_cuda()
    from tensor_transformer_layers_amd import shard
    w = WORKLOADS["layer_shard_bf16_b1_s4096_h8192_H64_f32768_n8"]
    d = attn_inputs(w)
    N, T = w.n_shards, w.tokens
    X = dev(d["X"], "bf16")
    za, zm, W0 = [], [], None
    for r in range(N):
        W = _rank_weights(d, N, r)
        za.append(shard.attn_shard(X, W["Wqkv"], W["bqkv"], W["Wo"], w.batch, w.seq, w.heads,
                                   N, r)[0])
        if r == 0:
            W0 = W
        del W
    Hs = shard.sum_partials(za, out_dtype=torch.bfloat16)
    mlp_w = []
    for r in range(N):
        A = dev(layout.column_shard(d["A"], N, r), "bf16")
        a = dev(layout.bias_shard(d["a"], N, r), "bf16")
        Bm = dev(layout.row_shard(d["B"], N, r), "bf16")
        zm.append(shard.mlp_shard(Hs, A, a, Bm, N, r)[0])
        if r == 0:
            mlp_w = (A, a, Bm)
        del A, a, Bm
    Z = shard.sum_partials(zm)
    drv = shard.LayerShard(w.batch, w.seq, w.hidden, w.heads, w.ffn, N, 0)
    Zd = drv.forward(X, W0["Wqkv"], W0["bqkv"], W0["Wo"], mlp_w[0], mlp_w[1], mlp_w[2],
                     za[1:], zm[1:])
    torch.cuda.synchronize()
    assert torch.equal(Zd, Z), "the rank-0 driver must reproduce the composed step bitwise"
    assert torch.equal(drv.H, Hs)
    # the fused step (each block's partial sum in its row-parallel product's epilogue)
    fz = shard.LayerShard(w.batch, w.seq, w.hidden, w.heads, w.ffn, N, 0, fused=True)
    Zf = fz.forward(X, W0["Wqkv"], W0["bqkv"], W0["Wo"], mlp_w[0], mlp_w[1], mlp_w[2],
                    za[1:], zm[1:])
    torch.cuda.synchronize()
    assert torch.equal(fz.H, Hs) and torch.equal(Zf, Z), "the fused step must give the same bits"
    del fz, Zf

    rows = sample_rows(T, 40, seed=4, must=[0, 1, 127, 128, 255, 2047, 2048, 4095])
    Hg = host(Hs)[rows]
    Zg = host(Z)[rows]
    assert np.isfinite(Zg).all()
    # attention block: the sum of the 8 rank partials is the unsharded block (N = 1)
    Ho = oracle.attn_shard(d["X"], d["Wq"], d["Wk"], d["Wv"], d["bq"], d["bk"], d["bv"],
                           d["Wo"], w.batch, w.seq, w.heads, 1, 0, True, rows=rows)
    eh = oracle.rel_frobenius(Hg, Ho)
    # MLP block on the GPU's own H: each rank's partial, then the sum
    ems = [oracle.rel_frobenius(host(zm[r])[rows], oracle.mlp_shard(Hg, d["A"], d["a"], d["B"], N, r))
           for r in range(N)]
    ez = oracle.rel_frobenius(Zg, oracle.mlp_shard(Hg, d["A"], d["a"], d["B"], 1, 0))
    e2e = oracle.rel_frobenius(Zg, oracle.mlp_shard(Ho, d["A"], d["a"], d["B"], 1, 0))
    print("composed layer step: H err %.2e; MLP partial errs %s; Z err %.2e; end-to-end %.2e"
          % (eh, " ".join("%.2e" % e for e in ems), ez, e2e))
    assert eh < TOL and max(ems) < TOL and ez < TOL and e2e < TOL


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
