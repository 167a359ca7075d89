"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test states what it pins and which plausible mistake it would catch. None of them
retypes the oracle's own formula: the checks are textbook constants, closed forms,
brute force with explicit loops on tiny inputs, the algebraic invariants of tensor
parallelism stated on the pages, and independent numpy/scipy routines.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import ndtr

import oracle
from synth import WORKLOADS, attn_inputs, mlp_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
pytestmark = pytest.mark.usefixtures("oracle_lib")


def _phi_table():
    rows = []
    with open(os.path.join(GOLDEN, "normal_cdf.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                x, p = line.split()
                rows.append((float(x), float(p)))
    return rows


# --------------------------------------------------------------------------------------
# GeLU: exact erf form (the pages name GeLU without a formula)
# --------------------------------------------------------------------------------------
def test_gelu_textbook_values():
    """GeLU(x) = x Phi(x) at tabulated Phi; catches a missing 1/2, a wrong sqrt(2) or tanh form."""
    for x, phi in _phi_table():
        for sx, sphi in ((x, phi), (-x, 1.0 - phi)):
            got = float(oracle.gelu([sx])[0])
            want = sx * sphi
            assert abs(got - want) <= 1e-15 * max(1.0, abs(want)), (sx, got, want)


def test_gelu_identities_and_limits():
    xs = np.linspace(-8, 8, 4001)
    g = oracle.gelu(xs)
    gm = oracle.gelu(-xs)
    # Phi(x) + Phi(-x) = 1  =>  GeLU(x) - GeLU(-x) = x
    np.testing.assert_allclose(g - gm, xs, rtol=0, atol=4e-15)
    assert oracle.gelu([0.0])[0] == 0.0
    assert oracle.gelu([40.0])[0] == 40.0          # Phi(40) = 1 in fp64
    assert abs(oracle.gelu([-40.0])[0]) < 1e-300   # x Phi(x) -> 0
    # independent implementation of Phi (scipy's ndtr), whole sweep; 1 + erf cancels for
    # x << 0, so the absolute error there is a few ulps of 1e-16
    np.testing.assert_allclose(g, xs * ndtr(xs), rtol=2e-15, atol=5e-16)


def test_gelu_is_not_tanh_approximation():
    """At x = 1 the tanh form differs from x Phi(x) by ~1.6e-4; the oracle must be exact."""
    x = 1.0
    tanh_form = 0.5 * x * (1 + math.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))
    exact = 0.8413447460685429
    assert abs(oracle.gelu([x])[0] - exact) < 1e-15
    assert abs(tanh_form - exact) > 1e-4


# --------------------------------------------------------------------------------------
# Linear layer Y = X W + b (llms.blog, "The Core Primitives")
# --------------------------------------------------------------------------------------
def _int_matrix(rng, shape):
    return rng.integers(-2, 3, size=shape).astype(np.float32)


def test_linear_brute_force_nonsquare():
    """Explicit triple loop on a 3x5 @ 5x4 + bias; catches a transposed W or dropped bias."""
    rng = np.random.default_rng(1)
    X = _int_matrix(rng, (3, 5))
    W = _int_matrix(rng, (5, 4))
    b = _int_matrix(rng, (4,))
    Y = oracle.linear(X, W, b)
    for t in range(3):
        for o in range(4):
            acc = float(b[o])
            for k in range(5):
                acc += float(X[t, k]) * float(W[k, o])
            assert Y[t, o] == acc
    Y0 = oracle.linear(X, W, None)
    assert np.array_equal(Y0, Y - b.astype(np.float64))


def test_linear_matches_numpy():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((37, 129)).astype(np.float32)
    W = rng.standard_normal((129, 71)).astype(np.float32)
    b = rng.standard_normal(71).astype(np.float32)
    ref = X.astype(np.float64) @ W.astype(np.float64) + b
    np.testing.assert_allclose(oracle.linear(X, W, b), ref, rtol=1e-13, atol=1e-12)


# --------------------------------------------------------------------------------------
# MLP block and its column/row split (ai360xpert.com "How It Works"; llms.blog MLP block)
# --------------------------------------------------------------------------------------
def _brute_mlp_shard(X, A, a, B, N, r):
    """Explicit loops: rank r takes columns [r F/N, (r+1) F/N) of A and a, same rows of B."""
    T, h = X.shape
    F = A.shape[1]
    w = F // N
    cols = range(r * w, (r + 1) * w)
    Y = [[0.0] * w for _ in range(T)]
    for t in range(T):
        for j, c in enumerate(cols):
            s = float(a[c])
            for k in range(h):
                s += float(X[t, k]) * float(A[k, c])
            Y[t][j] = s * float(ndtr(s))
    Z = np.zeros((T, h))
    for t in range(T):
        for o in range(h):
            s = 0.0
            for j, c in enumerate(cols):
                s += Y[t][j] * float(B[c, o])
            Z[t, o] = s
    return np.array(Y), Z


@pytest.mark.parametrize("N", [1, 2, 4])
def test_mlp_shard_brute_force_tiny(N):
    rng = np.random.default_rng(3)
    T, h, F = 3, 8, 16
    X, A, a, B = (_int_matrix(rng, s) for s in ((T, h), (h, F), (F,), (F, h)))
    for r in range(N):
        Yb, Zb = _brute_mlp_shard(X, A, a, B, N, r)
        np.testing.assert_allclose(oracle.mlp_column(X, A, a, N, r), Yb, rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(oracle.mlp_shard(X, A, a, B, N, r), Zb, rtol=1e-13, atol=1e-13)


def test_column_concat_equals_unsharded():
    """[Y_0 | ... | Y_{N-1}] = GeLU(X A + a): disjoint columns pass GeLU independently."""
    w = WORKLOADS["mlp_f32_t32_h1024_f4096_n2"]
    d = mlp_inputs(w)
    full = oracle.mlp_column(d["X"], d["A"], d["a"], 1, 0)
    for N in (2, 4, 8):
        parts = [oracle.mlp_column(d["X"], d["A"], d["a"], N, r) for r in range(N)]
        # same dot products; only the matmul's blocking may differ between shapes
        np.testing.assert_allclose(np.concatenate(parts, axis=1), full, rtol=1e-13, atol=1e-15)


def test_row_partials_sum_to_unsharded():
    """sum_r Y_r B_r = Y B (llms.blog, Row-Parallel Linear Layer)."""
    rng = np.random.default_rng(4)
    T, F, h = 9, 48, 20
    Y = rng.standard_normal((T, F))
    B = rng.standard_normal((F, h)).astype(np.float32)
    full = Y @ B.astype(np.float64)
    for N in (1, 2, 3, 4, 6):
        s = sum(oracle.mlp_row(Y[:, r * F // N:(r + 1) * F // N], B, N, r) for r in range(N))
        np.testing.assert_allclose(s, full, rtol=1e-12, atol=1e-12)


def test_tp_mlp_equals_unsharded_block_cfg1():
    """sum_r GeLU(X A_r + a_r) B_r = GeLU(X A + a) B at the fp32 worked-example shapes."""
    w = WORKLOADS["mlp_f32_t32_h1024_f4096_n2"]
    d = mlp_inputs(w)
    full = oracle.mlp_shard(d["X"], d["A"], d["a"], d["B"], 1, 0)
    # independent numpy / scipy float64 reference of the unsharded block
    P = d["X"].astype(np.float64) @ d["A"].astype(np.float64) + d["a"]
    ref = (P * ndtr(P)) @ d["B"].astype(np.float64)
    assert oracle.rel_frobenius(full, ref) < 1e-13
    for N in (2, 4, 8):
        s = sum(oracle.mlp_shard(d["X"], d["A"], d["a"], d["B"], N, r) for r in range(N))
        assert oracle.rel_frobenius(s, full) < 1e-13


def test_naive_row_split_must_synchronize_before_gelu():
    """GeLU of summed row-split partials differs from the sum of GeLUs (fanout.sh digest).

    X is split by columns and A by rows; sum_r GeLU(X_r A^(r)) is far from GeLU(X A).
    """
    # scalar closed form: GeLU(0.5) + GeLU(0.5) = Phi(0.5) != GeLU(1) = Phi(1)
    g = oracle.gelu([0.5, 1.0])
    assert abs(2 * g[0] - 0.6914624612740131) < 1e-15
    assert abs(g[1] - 0.8413447460685429) < 1e-15
    w = WORKLOADS["mlp_f32_t32_h1024_f4096_n2"]
    d = mlp_inputs(w)
    X, A = d["X"], d["A"]
    h = X.shape[1]
    good = oracle.gelu(oracle.linear(X, A))
    for N in (2, 4, 8):
        k = h // N
        naive = sum(oracle.gelu(oracle.linear(X[:, r * k:(r + 1) * k], A[r * k:(r + 1) * k]))
                    for r in range(N))
        synced = oracle.gelu(sum(oracle.linear(X[:, r * k:(r + 1) * k], A[r * k:(r + 1) * k])
                                 for r in range(N)))
        assert oracle.rel_frobenius(synced, good) < 1e-13
        assert oracle.rel_frobenius(naive, good) > 0.1


def test_column_parallel_listing_shapes():
    """The apxml.com listing: 32x1024 through a 1024->4096 layer split over 2 GPUs."""
    with open(os.path.join(GOLDEN, "column_parallel_listing.json")) as f:
        g = json.load(f)
    rng = np.random.default_rng(5)
    X = rng.standard_normal((g["batch"], g["in_features"])).astype(np.float32)
    A = rng.standard_normal((g["in_features"], g["out_features"])).astype(np.float32)
    N = g["tensor_model_parallel_size"]
    parts = [oracle.mlp_column(X, A, None, N, r) for r in range(N)]
    assert all(list(p.shape) == g["per_rank_output"] for p in parts)
    assert list(np.concatenate(parts, axis=1).shape) == g["gathered_output"]


def test_mlp_rejects_uneven_split():
    rng = np.random.default_rng(6)
    X, A, a, B = (_int_matrix(rng, s) for s in ((2, 4), (4, 10), (10,), (10, 4)))
    with pytest.raises(oracle.OracleError):
        oracle.mlp_shard(X, A, a, B, 4, 0)
    with pytest.raises(oracle.OracleError):
        oracle.mlp_shard(X, A, a, B, 2, 2)


# --------------------------------------------------------------------------------------
# Attention (llms.blog, "Partitioning Multi-Head and Grouped-Query Attention")
# --------------------------------------------------------------------------------------
def _brute_attention(Q, K, V, batch, seq, n_heads, causal):
    T, w = Q.shape
    d = w // n_heads
    O = np.zeros((T, w))
    for b in range(batch):
        for j in range(n_heads):
            cs = slice(j * d, (j + 1) * d)
            for i in range(seq):
                keys = range(i + 1) if causal else range(seq)
                sc = [sum(Q[b * seq + i, cs] * K[b * seq + k, cs]) / math.sqrt(d) for k in keys]
                m = max(sc)
                p = [math.exp(s - m) for s in sc]
                z = sum(p)
                for k, pk in zip(keys, p):
                    O[b * seq + i, cs] += (pk / z) * V[b * seq + k, cs]
    return O


@pytest.mark.parametrize("causal", [True, False])
def test_attention_brute_force_small(causal):
    rng = np.random.default_rng(7)
    batch, seq, H, d = 2, 5, 2, 8
    Q, K, V = (rng.standard_normal((batch * seq, H * d)) for _ in range(3))
    got = oracle.attention(Q, K, V, batch, seq, H, causal)
    np.testing.assert_allclose(got, _brute_attention(Q, K, V, batch, seq, H, causal),
                               rtol=1e-13, atol=1e-14)


def test_attention_closed_forms():
    rng = np.random.default_rng(8)
    batch, seq, H, d = 3, 7, 2, 4
    T = batch * seq
    Q, K, V = (rng.standard_normal((T, H * d)) for _ in range(3))
    O = oracle.attention(Q, K, V, batch, seq, H, True)
    # causal row 0 of every sequence is V at that row (catches an off-by-one mask k < i)
    for b in range(batch):
        assert np.array_equal(O[b * seq], V[b * seq])
    # K = 0: all scores equal -> prefix mean (causal) / full mean (non-causal)
    Oz = oracle.attention(Q, np.zeros_like(K), V, batch, seq, H, True)
    Oz_nc = oracle.attention(Q, np.zeros_like(K), V, batch, seq, H, False)
    for b in range(batch):
        for i in range(seq):
            blk = V[b * seq:b * seq + i + 1]
            np.testing.assert_allclose(Oz[b * seq + i], blk.mean(axis=0), rtol=1e-14, atol=1e-15)
            np.testing.assert_allclose(Oz_nc[b * seq + i], V[b * seq:(b + 1) * seq].mean(axis=0),
                                       rtol=1e-14, atol=1e-15)
    # constant V = c gives c everywhere (softmax weights sum to 1)
    Oc = oracle.attention(Q, K, np.full_like(V, 2.5), batch, seq, H, True)
    np.testing.assert_allclose(Oc, 2.5, rtol=1e-15, atol=0)
    # seq = 1 returns V
    O1 = oracle.attention(Q[:4], K[:4], V[:4], 4, 1, H, True)
    assert np.array_equal(O1, V[:4])


def test_attention_logit_gap_ln3_and_scale():
    """Two visible keys whose scaled logits differ by ln 3 get weights 1/4 and 3/4.

    d = 4 so the 1/sqrt(d) scale matters: <q, k1> = 2 ln 3 gives a logit gap of ln 3 only
    with the 1/sqrt(d_k) scale of the pages' attention formula (1/d would give ln 3 / 2).
    """
    d = 4
    Q = np.zeros((2, d)); K = np.zeros((2, d)); V = np.zeros((2, d))
    Q[1, 0] = 1.0
    K[1, 0] = 2.0 * math.log(3.0)
    V[0] = [4.0, 0.0, 1.0, -1.0]
    V[1] = [8.0, 4.0, 1.0, 3.0]
    O = oracle.attention(Q, K, V, 1, 2, 1, True)
    np.testing.assert_allclose(O[1], 0.25 * V[0] + 0.75 * V[1], rtol=1e-15, atol=1e-15)


def test_attention_row_selection_and_head_locality():
    rng = np.random.default_rng(9)
    batch, seq, H, d = 2, 9, 3, 4
    Q, K, V = (rng.standard_normal((batch * seq, H * d)) for _ in range(3))
    full = oracle.attention(Q, K, V, batch, seq, H, True)
    rows = np.array([0, 4, 8, 9, 17])
    assert np.array_equal(oracle.attention(Q, K, V, batch, seq, H, True, rows=rows), full[rows])
    # perturbing head 2's keys/values leaves heads 0 and 1 bitwise unchanged
    K2, V2 = K.copy(), V.copy()
    K2[:, 2 * d:] += 1.0
    V2[:, 2 * d:] -= 3.0
    pert = oracle.attention(Q, K2, V2, batch, seq, H, True)
    assert np.array_equal(pert[:, :2 * d], full[:, :2 * d])
    assert not np.array_equal(pert[:, 2 * d:], full[:, 2 * d:])


def _numpy_attn_block(X, Wq, Wk, Wv, bq, bk, bv, Wo, batch, seq, H, causal):
    """Independent vectorized float64 reference of the unsharded attention block."""
    X = X.astype(np.float64)
    Q = X @ Wq + bq
    K = X @ Wk + bk
    V = X @ Wv + bv
    h = X.shape[1]
    d = h // H
    O = np.zeros_like(Q)
    mask = np.tril(np.ones((seq, seq), dtype=bool)) if causal else np.ones((seq, seq), bool)
    for b in range(batch):
        sl = slice(b * seq, (b + 1) * seq)
        for j in range(H):
            cs = slice(j * d, (j + 1) * d)
            S = Q[sl, cs] @ K[sl, cs].T / np.sqrt(d)
            S = np.where(mask, S, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            O[sl, cs] = P @ V[sl, cs]
    return O @ Wo


def _small_attn_inputs(seed=10, batch=2, seq=6, h=16, bias=True):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32) * np.float32(0.3)
    X = rng.standard_normal((batch * seq, h)).astype(np.float32)
    d = dict(X=X, Wq=f(h, h), Wk=f(h, h), Wv=f(h, h), bq=f(h), bk=f(h), bv=f(h), Wo=f(h, h))
    if not bias:
        for k in ("bq", "bk", "bv"):
            d[k] = None
    return d


@pytest.mark.parametrize("causal", [True, False])
def test_attn_block_matches_numpy_and_shards_sum(causal):
    batch, seq, h, H = 2, 6, 16, 4
    d = _small_attn_inputs()
    args = (d["X"], d["Wq"], d["Wk"], d["Wv"], d["bq"], d["bk"], d["bv"], d["Wo"])
    full = oracle.attn_shard(*args, batch, seq, H, 1, 0, causal)
    ref = _numpy_attn_block(*args, batch, seq, H, causal)
    assert oracle.rel_frobenius(full, ref) < 1e-13
    for N in (2, 4):
        s = sum(oracle.attn_shard(*args, batch, seq, H, N, r, causal) for r in range(N))
        assert oracle.rel_frobenius(s, full) < 1e-13


def test_attn_identity_projections():
    """W_Q = W_K = W_V = W_O = I, no bias: the block output is attention(X, X, X)."""
    batch, seq, h, H = 2, 5, 8, 2
    rng = np.random.default_rng(11)
    X = rng.standard_normal((batch * seq, h)).astype(np.float32)
    I = np.eye(h, dtype=np.float32)
    Z = oracle.attn_shard(X, I, I, I, None, None, None, I, batch, seq, H, 1, 0, True)
    Xd = X.astype(np.float64)
    np.testing.assert_allclose(Z, _brute_attention(Xd, Xd, Xd, batch, seq, H, True),
                               rtol=1e-13, atol=1e-14)


def test_attn_shard_head_locality():
    """Z_r depends only on W_Q/W_K/W_V columns and W_O rows of rank r's heads."""
    batch, seq, h, H, N, r = 2, 6, 16, 4, 2, 1
    d = _small_attn_inputs()
    args = [d["X"], d["Wq"], d["Wk"], d["Wv"], d["bq"], d["bk"], d["bv"], d["Wo"]]
    base = oracle.attn_shard(*args, batch, seq, H, N, r, True)
    w = h // N
    other = slice(0, w)          # rank 0's columns
    mine = slice(w, 2 * w)
    pert = [a.copy() if a is not None else None for a in args]
    for i in (1, 2, 3):
        pert[i][:, other] += 5.0
    for i in (4, 5, 6):
        pert[i][other] -= 2.0
    pert[7][other, :] *= -3.0
    assert np.array_equal(oracle.attn_shard(*pert, batch, seq, H, N, r, True), base)
    pert[2][:, mine] += 1.0
    assert not np.array_equal(oracle.attn_shard(*pert, batch, seq, H, N, r, True), base)


def test_attn_shard_sampled_rows_equal_full():
    batch, seq, h, H, N = 2, 6, 16, 4, 2
    d = _small_attn_inputs()
    args = (d["X"], d["Wq"], d["Wk"], d["Wv"], d["bq"], d["bk"], d["bv"], d["Wo"])
    full, Ofull = oracle.attn_shard(*args, batch, seq, H, N, 0, True, want_heads=True)
    rows = np.array([1, 5, 6, 11])
    Z, O = oracle.attn_shard(*args, batch, seq, H, N, 0, True, rows=rows, want_heads=True)
    np.testing.assert_allclose(Z, full[rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(O, Ofull[rows], rtol=1e-13, atol=1e-14)
    # the head outputs are the attention of the projected Q, K, V of rank 0's heads
    Q, K, V = oracle.qkv_shard(d["X"], d["Wq"], d["Wk"], d["Wv"], d["bq"], d["bk"], d["bv"],
                               H, N, 0)
    np.testing.assert_allclose(oracle.attention(Q, K, V, batch, seq, H // N, True), Ofull,
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(oracle.out_proj_shard(Ofull, d["Wo"], H, N, 0), full,
                               rtol=1e-13, atol=1e-14)


def test_attn_rejects_bad_head_split():
    d = _small_attn_inputs()
    args = (d["X"], d["Wq"], d["Wk"], d["Wv"], d["bq"], d["bk"], d["bv"], d["Wo"])
    with pytest.raises(oracle.OracleError):
        oracle.attn_shard(*args, 2, 6, 4, 3, 0, True)     # 4 heads over 3 ranks
    with pytest.raises(oracle.OracleError):
        oracle.attn_shard(*args, 2, 6, 3, 1, 0, True)     # 16 not divisible by 3 heads


# --------------------------------------------------------------------------------------
# Partial sum (what the all-reduce computes)
# --------------------------------------------------------------------------------------
def test_sum_partials_exact_and_fsum():
    rng = np.random.default_rng(12)
    P = rng.integers(-1000, 1001, size=(8, 1000)).astype(np.float32)
    assert np.array_equal(oracle.sum_partials(P), P.astype(np.int64).sum(axis=0).astype(float))
    Pf = rng.standard_normal((5, 300)).astype(np.float32)
    S = oracle.sum_partials(Pf)
    for i in range(0, 300, 37):
        assert abs(S[i] - math.fsum(float(v) for v in Pf[:, i])) < 1e-15


# --------------------------------------------------------------------------------------
# Workload generator sanity (shapes and the bf16-exactness of bf16 workloads)
# --------------------------------------------------------------------------------------
def test_bf16_workload_inputs_are_bf16_exact():
    from synth import bf16_round
    w = WORKLOADS["attn_shard_bf16_b4_s2048_h4096_H32_n8"]
    d = attn_inputs(w, batch=1, seq=8)
    for k, v in d.items():
        assert np.array_equal(bf16_round(v), v), k
    # RNE: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -1 - 2.0 ** -8], dtype=np.float32)
    assert list(bf16_round(x)) == [1.0, 1 + 2.0 ** -6, -1.0]


# --------------------------------------------------------------------------------------
# The parity metric: relative Frobenius error ||got - ref||_F / ||ref||_F over the whole
# tensor (the acceptance test every GPU parity assertion goes through)
# --------------------------------------------------------------------------------------
def test_rel_frobenius_hand_computed_values():
    # ref (3, 4) has norm 5; got differs by (0, 1/2): 0.5 / 5 = 0.1 exactly. The squared
    # ratio would give 0.01, and ||got|| in the denominator 0.5 / sqrt(29.25) = 0.0925.
    assert oracle.rel_frobenius([3.0, 4.5], [3.0, 4.0]) == pytest.approx(0.1, rel=1e-15, abs=0)
    assert abs(oracle.rel_frobenius([3.0, 4.5], [3.0, 4.0]) - 0.1) < 1e-16
    # The denominator is the reference's norm, not the result's: the error of an all-zero
    # result is exactly 1, and swapping the arguments changes the value.
    assert oracle.rel_frobenius([0.0, 0.0], [3.0, 4.0]) == 1.0
    assert oracle.rel_frobenius([6.0, 8.0], [3.0, 4.0]) == 1.0
    assert oracle.rel_frobenius([3.0, 4.0], [6.0, 8.0]) == 0.5
    # Negated result: ||2 ref|| / ||ref|| = 2 (a sum instead of a difference gives 0).
    assert oracle.rel_frobenius([-3.0, -4.0], [3.0, 4.0]) == 2.0


def test_rel_frobenius_is_over_the_whole_tensor():
    # ref [[1, 2], [2, 4]] has Frobenius norm 5; got differs in one element by 3: 3 / 5.
    # Row-wise variants differ: the worst row gives 3 / sqrt(20) = 0.671, the mean of the
    # rows' errors 0.335, the largest element error over the largest element 0.75.
    ref = np.array([[1.0, 2.0], [2.0, 4.0]])
    got = np.array([[1.0, 2.0], [2.0, 1.0]])
    assert abs(oracle.rel_frobenius(got, ref) - 0.6) < 1e-15
    # shape-agnostic: the same 4 numbers flattened or transposed give the same value
    assert oracle.rel_frobenius(got.ravel(), ref.ravel()) == oracle.rel_frobenius(got, ref)
    assert oracle.rel_frobenius(got.T, ref.T) == oracle.rel_frobenius(got, ref)


def test_rel_frobenius_is_computed_in_fp64():
    # A 1e-9 relative difference on 2^20 fp32-exact elements: in fp64 the metric returns it
    # to 1e-6 relative; an fp32 computation of the difference would round it away (each
    # element's difference is below half an fp32 ulp of the values).
    n = 1 << 20
    ref = np.full(n, 1.0, dtype=np.float64)
    got = ref + 1e-9
    assert abs(oracle.rel_frobenius(got, ref) - 1e-9) < 1e-15
    assert oracle.rel_frobenius(got.astype(np.float32), ref.astype(np.float32)) == 0.0
