"""GPU parity of tp_attn_shard_fwd against the fp64 oracle (bf16, fp32 accumulation).

Checked per step: the column-parallel Q/K/V projection (read from the workspace), the
head-local attention output O_i (heads concatenated locally) and the row-parallel partial
Z_i. Tolerance: relative Frobenius error 1e-2, oracle fed the same bf16-rounded inputs.
"""
import numpy as np
import pytest

import oracle
from gpu_util import Canary, canary_tensor, dev, host, torch_cuda
from synth import WORKLOADS, Workload, attn_inputs, sample_rows
from tensor_transformer_layers_amd import layout

pytestmark = pytest.mark.gpu
TOL = 1e-2


def run_attn(d, batch, seq, H, N, r, causal, bias=True):
    """Rank r's attention shard on the GPU; returns host fp64 (Z, O, Q, K, V) with Q/K/V
    as [T, Hl*d] (the oracle's layout)."""
    torch = torch_cuda()
    from tensor_transformer_layers_amd import binding as B
    from tensor_transformer_layers_amd import shard
    h = d["X"].shape[1]
    X = dev(d["X"], "bf16")
    Wqkv = dev(layout.qkv_shard(d["Wq"], d["Wk"], d["Wv"], N, r), "bf16")
    bqkv = dev(layout.qkv_bias_shard(d["bq"], d["bk"], d["bv"], N, r), "bf16") if bias else None
    Wo = dev(layout.row_shard(d["Wo"], N, r), "bf16")
    T = batch * seq
    Zc = canary_tensor((T, h), torch.float32)
    ws = Canary(B.tp_attn_workspace_bytes(batch, seq, h, H, N, B.TP_BF16), torch.uint8, None)
    shard.attn_shard(X, Wqkv, bqkv, Wo, batch, seq, H, N, r, causal, Z=Zc.tensor,
                     workspace=ws.body)
    torch.cuda.synchronize()
    assert Zc.intact() and ws.intact(), "write outside an output buffer"
    v = shard.attn_views(ws.body, batch, seq, h, H, N)
    hl, dd = H // N, h // H
    # [b, Hl, s, d] -> [b*s, Hl*d]
    # the workspace holds Q times the softmax's log2(e) / sqrt(d)
    q = host(v["q"].permute(0, 2, 1, 3).reshape(T, hl * dd)) / (np.log2(np.e) / np.sqrt(dd))
    k = host(v["k"].permute(0, 2, 1, 3).reshape(T, hl * dd))
    vv = host(v["vt"][..., :seq].permute(0, 3, 1, 2).reshape(T, hl * dd))
    return host(Zc.tensor), host(v["o"]), q, k, vv


def _bias(d, bias):
    return (d["bq"], d["bk"], d["bv"]) if bias else (None, None, None)


SMALL = [
    # batch, seq, hidden, heads, N, causal, bias
    (2, 200, 512, 4, 2, True, True),
    (2, 200, 512, 4, 2, False, True),
    (1, 130, 512, 4, 1, True, False),
    (3, 7, 256, 2, 2, True, True),
    (2, 1, 256, 2, 1, True, True),
    (2, 65, 256, 4, 2, True, True),     # d = 64
    (1, 257, 256, 4, 4, False, False),  # d = 64, one head per rank
]


@pytest.mark.parametrize("case", SMALL)
def test_attn_small_every_step(case):
    batch, seq, h, H, N, causal, bias = case
    w = Workload(name="a", kind="attn", dtype="bf16", tokens=batch * seq, batch=batch, seq=seq,
                 hidden=h, heads=H, n_shards=N)
    d = attn_inputs(w, seed=seq + h, with_bias=bias)
    bq, bk, bv = _bias(d, bias)
    for r in sorted({0, N - 1}):
        Z, O, q, k, v = run_attn(d, batch, seq, H, N, r, causal, bias)
        Qo, Ko, Vo = oracle.qkv_shard(d["X"], d["Wq"], d["Wk"], d["Wv"], bq, bk, bv, H, N, r)
        Zo, Oo = oracle.attn_shard(d["X"], d["Wq"], d["Wk"], d["Wv"], bq, bk, bv, d["Wo"],
                                   batch, seq, H, N, r, causal, want_heads=True)
        errs = [oracle.rel_frobenius(a, b) for a, b in ((q, Qo), (k, Ko), (v, Vo), (O, Oo),
                                                         (Z, Zo))]
        print("%s rank %d: Q %.1e K %.1e V %.1e O %.1e Z %.1e" % (case, r, *errs))
        assert max(errs) < TOL


@pytest.mark.parametrize("case", SMALL)
def test_attn_forced_key_range_split(case, overrides):
    """The same shards with each query tile's keys halved between two workgroups and the
    halves merged by a second kernel (the path long causal sequences take by default; the
    knob forces it on these small grids): ragged tails, single-tile sequences, halves that
    hold no visible key for some queries, d = 64, and the unmasked case."""
    overrides("attn_split=2")
    test_attn_small_every_step(case)


@pytest.mark.parametrize("case", SMALL)
def test_attn_qkv_k_split(case, overrides):
    """The multi-head shards with the Q/K/V projection forced through the K-split path."""
    overrides("qkv_split=3")
    test_attn_small_every_step(case)


@pytest.mark.parametrize("spec", ["attn_split=2,attn_sets=2", "attn_split=1,attn_sets=1",
                                  "attn_pair=1"])
@pytest.mark.parametrize("case", [SMALL[0], SMALL[1], SMALL[3], SMALL[5]])
def test_attn_other_set_counts(case, spec, overrides):
    """The combinations the default does not take: the key-range split with two sets of
    waves per workgroup (merged through LDS, then across the halves), one set without the
    split (no merge at all), and causal query tiles of 128 without the pairing."""
    overrides(spec)
    test_attn_small_every_step(case)


PAIRED = [
    # batch, seq, hidden, heads, N, causal, bias: causal shapes for the paired layout (a
    # workgroup owns 64-query tiles i and n64 - 1 - i); odd tile counts leave the middle
    # tile alone, ragged ends cut the last tile
    (1, 960, 512, 4, 2, True, True),     # 15 tiles
    (2, 1088, 512, 4, 2, True, True),    # 17 tiles
    (1, 1023, 256, 2, 1, True, False),   # 16 tiles, ragged
    (3, 191, 256, 4, 2, True, True),     # 3 tiles, ragged, d = 64
]


@pytest.mark.parametrize("case", PAIRED)
def test_attn_paired_layout(case):
    """The paired causal layout (the default for causal attention) on odd and ragged tile
    counts, against the oracle."""
    test_attn_small_every_step(case)


@pytest.mark.parametrize("case", PAIRED[:2])
def test_attn_paired_agrees_with_unpaired(case, overrides):
    """Paired and unpaired layouts compute the same softmax: agreement to bf16 rounding."""
    batch, seq, h, H, N, causal, _ = case
    w = Workload(name="a", kind="attn", dtype="bf16", tokens=batch * seq, batch=batch, seq=seq,
                 hidden=h, heads=H, n_shards=N)
    d = attn_inputs(w, seed=5)
    _, O_pair, *_ = run_attn(d, batch, seq, H, N, N - 1, causal)
    overrides("attn_pair=1")
    _, O_one, *_ = run_attn(d, batch, seq, H, N, N - 1, causal)
    e = oracle.rel_frobenius(O_pair, O_one)
    print("paired vs unpaired O: %.2e" % e)
    assert e < 5e-3


@pytest.mark.parametrize("causal", [True, False])
def test_attn_split_and_unsplit_agree(causal, overrides):
    """Both paths compute the same softmax: agreement to bf16 rounding of O."""
    batch, seq, h, H, N = 2, 300, 512, 4, 2
    w = Workload(name="a", kind="attn", dtype="bf16", tokens=batch * seq, batch=batch, seq=seq,
                 hidden=h, heads=H, n_shards=N)
    d = attn_inputs(w, seed=17)
    overrides("attn_split=2")
    _, O_split, *_ = run_attn(d, batch, seq, H, N, 1, causal)
    overrides("attn_split=1")
    _, O_one, *_ = run_attn(d, batch, seq, H, N, 1, causal)
    e = oracle.rel_frobenius(O_split, O_one)
    print("split vs unsplit O: %.2e" % e)
    assert e < 5e-3


def test_attn_causal_first_row_is_projected_value():
    """Causal row 0 of every sequence attends only to itself: O[b, 0] = V[b, 0] (to bf16)."""
    batch, seq, h, H, N = 3, 33, 256, 2, 1
    w = Workload(name="a", kind="attn", dtype="bf16", tokens=batch * seq, batch=batch, seq=seq,
                 hidden=h, heads=H, n_shards=N)
    d = attn_inputs(w, seed=2)
    _, O, _, _, v = run_attn(d, batch, seq, H, N, 0, True)
    for b in range(batch):
        np.testing.assert_allclose(O[b * seq], v[b * seq], rtol=1e-2, atol=1e-2)


@pytest.mark.parametrize("rank,spec", [(0, None), (5, None), (5, "attn_split=2"),
                                       (5, "attn_pair=1")])
def test_attn_full_size_shard_sampled_rows(rank, spec, overrides):
    """One rank's shard at b 4, s 2048, h 4096, 32 heads, N 8 (causal), 48 sampled rows: the
    default takes the paired layout (256 workgroups, each two 64-query tiles of one head);
    also with the key-range split forced, and with neither (one two-set workgroup per
    128-query tile)."""
    if spec:
        overrides(spec)
    w = WORKLOADS["attn_shard_bf16_b4_s2048_h4096_H32_n8"]
    d = attn_inputs(w)
    Z, O, *_ = run_attn(d, w.batch, w.seq, w.heads, w.n_shards, rank, True)
    s = w.seq
    # rows of sequences 0 and 3, with each sequence's first and last positions
    rows = np.unique(np.concatenate([
        sample_rows(s, 24, seed=rank, must=[127, 128, 1000]),
        3 * s + sample_rows(s, 24, seed=rank + 1, must=[64, 1919]),
    ]))
    Zo, Oo = oracle.attn_shard(d["X"], d["Wq"], d["Wk"], d["Wv"], d["bq"], d["bk"], d["bv"],
                               d["Wo"], w.batch, s, w.heads, w.n_shards, rank, True, rows=rows,
                               want_heads=True)
    eo, ez = oracle.rel_frobenius(O[rows], Oo), oracle.rel_frobenius(Z[rows], Zo)
    print("full-size attention rank %d: O err %.2e, Z err %.2e" % (rank, eo, ez))
    assert eo < TOL and ez < TOL
    assert np.isfinite(Z).all()
    if rank == 0:
        Z2, *_ = run_attn(d, w.batch, w.seq, w.heads, w.n_shards, rank, True)
        assert np.array_equal(Z, Z2), "results must be bitwise repeatable"


def test_attn_head_locality_on_gpu():
    """Each rank evaluates attention for its own heads with no cross-head exchange (llms.blog,
    "Partitioning Multi-Head and Grouped-Query Attention", step 2), checked on the GPU:
      * perturbing the W_Q, W_K, W_V columns and W_O rows of every head outside rank r leaves
        the GPU's Z_r bitwise unchanged;
      * inside the rank, perturbing local head j's query, key or value columns changes head
        j's output columns of O_r and leaves the other local head's bits unchanged;
      * perturbing W_O rows changes Z_r but not O_r."""
    batch, seq, h, H, N, r = 2, 200, 512, 4, 2, 1      # d = 128, local heads 2 and 3
    w = Workload(name="a", kind="attn", dtype="bf16", tokens=batch * seq, batch=batch, seq=seq,
                 hidden=h, heads=H, n_shards=N)
    d = attn_inputs(w, seed=31)
    dd, hl = h // H, H // N
    Z0, O0, *_ = run_attn(d, batch, seq, H, N, r, True)
    # other ranks' heads: columns [0, r h/N) of W_Q/W_K/W_V and the same rows of W_O
    e = {k: v.copy() for k, v in d.items()}
    other = slice(0, r * h // N)
    for k in ("Wq", "Wk", "Wv"):
        e[k][:, other] += 0.5
    e["Wo"][other, :] -= 0.5
    Z1, O1, *_ = run_attn(e, batch, seq, H, N, r, True)
    assert np.array_equal(Z1, Z0) and np.array_equal(O1, O0)
    # local head 0 of the rank (global head r * hl): its columns only
    g0 = slice((r * hl) * dd, (r * hl + 1) * dd)
    for k in ("Wq", "Wk", "Wv"):
        e = {kk: v.copy() for kk, v in d.items()}
        e[k][:, g0] = np.flip(e[k][:, g0], axis=0).copy()
        _, O2, *_ = run_attn(e, batch, seq, H, N, r, True)
        assert np.array_equal(O2[:, dd:], O0[:, dd:]), k       # local head 1 untouched
        assert not np.array_equal(O2[:, :dd], O0[:, :dd]), k   # local head 0 changed
    e = {kk: v.copy() for kk, v in d.items()}
    e["Wo"][g0, :] *= -1.0
    Z3, O3, *_ = run_attn(e, batch, seq, H, N, r, True)
    assert np.array_equal(O3, O0) and not np.array_equal(Z3, Z0)


@pytest.mark.parametrize("case", [SMALL[0], SMALL[3], SMALL[5]])
def test_attn_steps_one_by_one_equal_the_shard_call(case):
    """The projection, head-local attention and output projection called one by one give
    the shard call's bits (Z and every workspace region the steps write)."""
    torch = torch_cuda()
    from tensor_transformer_layers_amd import binding as B
    from tensor_transformer_layers_amd import shard
    batch, seq, h, H, N, causal, bias = case
    w = Workload(name="a", kind="attn", dtype="bf16", tokens=batch * seq, batch=batch, seq=seq,
                 hidden=h, heads=H, n_shards=N)
    d = attn_inputs(w, seed=seq + 3, with_bias=bias)
    r = N - 1
    X = dev(d["X"], "bf16")
    Wqkv = dev(layout.qkv_shard(d["Wq"], d["Wk"], d["Wv"], N, r), "bf16")
    bqkv = dev(layout.qkv_bias_shard(d["bq"], d["bk"], d["bv"], N, r), "bf16") if bias else None
    Wo = dev(layout.row_shard(d["Wo"], N, r), "bf16")
    Z1, ws1 = shard.attn_shard(X, Wqkv, bqkv, Wo, batch, seq, H, N, r, causal)
    ws2 = torch.zeros_like(ws1)
    shard.qkv_projection(X, Wqkv, bqkv, batch, seq, H, H, N, r, ws2)
    shard.head_attention(batch, seq, h, H, H, N, r, causal, ws2)
    O2 = shard.attn_views(ws2, batch, seq, h, H, N)["o"]
    Z2 = shard.row_parallel(O2, Wo, N, r)
    torch.cuda.synchronize()
    assert torch.equal(Z1, Z2)
    v1, v2 = shard.attn_views(ws1, batch, seq, h, H, N), shard.attn_views(ws2, batch, seq, h, H, N)
    for k in ("q", "k", "o"):
        assert torch.equal(v1[k], v2[k]), k
    assert torch.equal(v1["vt"][..., :seq], v2["vt"][..., :seq])
