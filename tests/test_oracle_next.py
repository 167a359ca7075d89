"""Pins of the oracle's functions for the paths next to the core shard (CPU only).

SwiGLU gate, LayerNorm and the sequence-parallel reduce-scatter / all-gather, grouped-query
attention and the backward pass of the MLP shard. As for the core oracle, every check is
something the pages or the mathematics fix independently of the oracle's code: closed
forms and textbook values, worked examples computed by hand, explicit loops on tiny
inputs, finite differences of the forward functions, and the algebraic identities of
tensor and sequence parallelism stated on the pages.
"""
import math

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.usefixtures("oracle_lib")


def _int_matrix(rng, shape):
    return rng.integers(-2, 3, size=shape).astype(np.float64)


# --------------------------------------------------------------------------------------
# SiLU and the SwiGLU shard (llms.blog, "Partitioning the MLP Block", steps 2-3)
# --------------------------------------------------------------------------------------
def test_silu_closed_forms():
    """sigmoid(ln 3) = 3/4 and sigmoid(0) = 1/2: catches exp(x) for exp(-x) or a missing x."""
    assert oracle.silu([0.0])[0] == 0.0
    # within a few ulps (exp(-ln 3) = 1/3 is itself rounded)
    assert abs(oracle.silu([math.log(3.0)])[0] - 0.75 * math.log(3.0)) < 4e-16
    assert abs(oracle.silu([-math.log(3.0)])[0] + 0.25 * math.log(3.0)) < 4e-16
    assert abs(oracle.silu([1.0])[0] - 0.7310585786300049) < 1e-16   # 1 / (1 + e^-1)
    assert oracle.silu([40.0])[0] == 40.0
    assert -1e-15 < oracle.silu([-40.0])[0] < 0.0


def test_silu_odd_part_identity():
    """sigmoid(x) + sigmoid(-x) = 1, so SiLU(x) - SiLU(-x) = x."""
    xs = np.linspace(-30, 30, 6001)
    np.testing.assert_allclose(oracle.silu(xs) - oracle.silu(-xs), xs, rtol=0, atol=1e-14)


def _brute_swiglu(X, Wg, Wu, Wd, N, r):
    T, h = X.shape
    w = Wg.shape[1] // N
    cols = range(r * w, (r + 1) * w)
    Aact = np.zeros((T, w))
    for t in range(T):
        for j, c in enumerate(cols):
            g = sum(float(X[t, k]) * float(Wg[k, c]) for k in range(h))
            u = sum(float(X[t, k]) * float(Wu[k, c]) for k in range(h))
            Aact[t, j] = g / (1.0 + math.exp(-g)) * u
    Z = np.zeros((T, Wd.shape[1]))
    for t in range(T):
        for o in range(Wd.shape[1]):
            Z[t, o] = sum(Aact[t, j] * float(Wd[c, o]) for j, c in enumerate(cols))
    return Aact, Z


@pytest.mark.parametrize("N", [1, 2, 4])
def test_swiglu_shard_brute_force_tiny(N):
    rng = np.random.default_rng(21)
    T, h, F = 3, 8, 16
    X, Wg, Wu, Wd = (_int_matrix(rng, s) for s in ((T, h), (h, F), (h, F), (F, h)))
    for r in range(N):
        Ab, Zb = _brute_swiglu(X, Wg, Wu, Wd, N, r)
        np.testing.assert_allclose(oracle.swiglu_column(X, Wg, Wu, N, r), Ab, rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(oracle.swiglu_shard(X, Wg, Wu, Wd, N, r), Zb, rtol=1e-13,
                                   atol=1e-13)


def test_swiglu_tp_equals_unsharded_and_gate_is_local():
    """sum_r A_r Wd_r = SwiGLU block (the gate product is element-wise, so column shards need
    no exchange); the gate applied to the full product equals the concatenated shards."""
    rng = np.random.default_rng(22)
    T, h, F = 6, 32, 64
    X = rng.standard_normal((T, h))
    Wg, Wu = rng.standard_normal((h, F)) / 6, rng.standard_normal((h, F)) / 6
    Wd = rng.standard_normal((F, h)) / 8
    full = oracle.swiglu_shard(X, Wg, Wu, Wd, 1, 0)
    for N in (2, 4, 8):
        tot = sum(oracle.swiglu_shard(X, Wg, Wu, Wd, N, r) for r in range(N))
        assert oracle.rel_frobenius(tot, full) < 1e-13
        cat = np.concatenate([oracle.swiglu_column(X, Wg, Wu, N, r) for r in range(N)], axis=1)
        np.testing.assert_allclose(cat, oracle.swiglu_column(X, Wg, Wu, 1, 0), rtol=1e-14,
                                   atol=1e-15)
    # the gate is not linear: gating the sum of row-split partials differs (why the split
    # must be by columns)
    Xa, Xb = X[:, : h // 2], X[:, h // 2:]
    naive = oracle.silu(Xa @ Wg[: h // 2]) + oracle.silu(Xb @ Wg[h // 2:])
    assert oracle.rel_frobenius(naive, oracle.silu(X @ Wg)) > 0.1


def test_swiglu_rejects_uneven_split():
    X = np.zeros((2, 4))
    with pytest.raises(oracle.OracleError):
        oracle.swiglu_shard(X, np.zeros((4, 6)), np.zeros((4, 6)), np.zeros((6, 4)), 4, 0)


# --------------------------------------------------------------------------------------
# LayerNorm and sequence parallelism (llms.blog, "Sequence Parallelism")
# --------------------------------------------------------------------------------------
def test_layernorm_worked_example():
    """x = [1, 2, 3, 4]: mean 5/2, variance 5/4, so (x - mean)/sqrt(5/4) = [-3, -1, 1, 3]/sqrt 5."""
    y = oracle.layernorm(np.array([[1.0, 2.0, 3.0, 4.0]]), np.ones(4), np.zeros(4), 0.0)
    want = np.array([-3.0, -1.0, 1.0, 3.0]) / math.sqrt(5.0)
    np.testing.assert_allclose(y[0], want, rtol=0, atol=2e-16)
    # gamma and beta act per column after the normalisation
    y2 = oracle.layernorm(np.array([[1.0, 2.0, 3.0, 4.0]]), np.array([2.0, 1.0, 1.0, 0.5]),
                          np.array([0.0, 1.0, -1.0, 0.0]), 0.0)
    np.testing.assert_allclose(y2[0], want * [2.0, 1.0, 1.0, 0.5] + [0.0, 1.0, -1.0, 0.0],
                               rtol=0, atol=4e-16)
    # eps enters under the root: x = [-1, 1] has variance 1, so eps = 3 halves the output
    y3 = oracle.layernorm(np.array([[-1.0, 1.0]]), np.ones(2), np.zeros(2), 3.0)
    np.testing.assert_allclose(y3[0], [-0.5, 0.5], rtol=0, atol=1e-16)


def test_layernorm_moments_and_invariances():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((7, 96)) * 3 + 1.5
    y = oracle.layernorm(x, np.ones(96), np.zeros(96), 0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose(y.var(axis=1), 1.0, atol=1e-13)   # biased variance, eps = 0
    # shift and positive-scale invariance (eps = 0)
    np.testing.assert_allclose(oracle.layernorm(2.5 * x - 7.0, np.ones(96), np.zeros(96), 0.0), y,
                               rtol=0, atol=1e-13)


def test_sp_slices_partition_the_tokens():
    batch, seq, N = 3, 8, 4
    allrows = np.concatenate([oracle.sp_rows(batch, seq, N, r) for r in range(N)])
    assert sorted(allrows.tolist()) == list(range(batch * seq))
    # rank 1's slice: positions 2, 3 of each of the 3 sequences
    assert oracle.sp_rows(batch, seq, N, 1).tolist() == [2, 3, 10, 11, 18, 19]
    with pytest.raises(oracle.OracleError):
        oracle.sp_rows(batch, 6, 4, 0)


def test_reduce_scatter_then_all_gather_is_all_reduce():
    """The page: an all-reduce is a reduce-scatter followed by an all-gather."""
    rng = np.random.default_rng(24)
    batch, seq, h, N = 2, 12, 16, 4
    parts = rng.standard_normal((N, batch * seq, h)).astype(np.float32)
    rs = [oracle.reduce_scatter(parts, batch, seq, N, r) for r in range(N)]
    ag = oracle.all_gather(rs, batch, seq)
    assert np.array_equal(ag, oracle.sum_partials(parts))
    # exact on integer-valued partials, against Python's exact sum
    ip = rng.integers(-50, 50, size=(N, batch * seq, h)).astype(np.float32)
    r1 = oracle.reduce_scatter(ip, batch, seq, N, 1)
    rows = oracle.sp_rows(batch, seq, N, 1)
    want = np.array([[math.fsum(float(ip[q, t, c]) for q in range(N)) for c in range(h)] for t in rows])
    assert np.array_equal(r1, want)


def test_sp_boundary_matches_replicated_block():
    """Sharded residual + LayerNorm on the slices equals the replicated computation's rows."""
    rng = np.random.default_rng(25)
    batch, seq, h, N = 2, 8, 24, 4
    parts = rng.standard_normal((N, batch * seq, h)).astype(np.float32)
    resid = rng.standard_normal((batch * seq, h))
    gamma, beta = rng.standard_normal(h), rng.standard_normal(h)
    Hfull = oracle.sum_partials(parts) + resid
    Yfull = oracle.layernorm(Hfull, gamma, beta, 1e-5)
    for r in range(N):
        rows = oracle.sp_rows(batch, seq, N, r)
        Hr, Yr = oracle.sp_boundary(parts, resid[rows], gamma, beta, batch, seq, N, r, 1e-5)
        np.testing.assert_array_equal(Hr, Hfull[rows])
        np.testing.assert_array_equal(Yr, Yfull[rows])


# --------------------------------------------------------------------------------------
# Grouped-query attention (llms.blog, "Grouped-Query Attention (GQA) Constraints")
# --------------------------------------------------------------------------------------
def _gqa_inputs(rng, batch, seq, h, H, H_kv):
    d = h // H
    X = rng.standard_normal((batch * seq, h))
    Wq = rng.standard_normal((h, H * d)) / math.sqrt(h)
    Wk = rng.standard_normal((h, H_kv * d)) / math.sqrt(h)
    Wv = rng.standard_normal((h, H_kv * d)) / math.sqrt(h)
    bq, bk, bv = (rng.standard_normal(n) * 0.1 for n in (H * d, H_kv * d, H_kv * d))
    Wo = rng.standard_normal((H * d, h)) / math.sqrt(h)
    return X, Wq, Wk, Wv, bq, bk, bv, Wo


def _expand_kv(W, H, H_kv, d):
    """Repeat each key/value head's columns for the H / H_kv query heads that read it."""
    g = H // H_kv
    return np.concatenate([W[..., (j // g) * d:(j // g + 1) * d] for j in range(H)], axis=-1)


@pytest.mark.parametrize("H_kv", [1, 2, 4])
def test_gqa_equals_mha_with_repeated_kv_heads(H_kv):
    """GQA = multi-head attention whose key/value heads are copies shared by a group."""
    rng = np.random.default_rng(26)
    batch, seq, h, H = 2, 6, 32, 8
    d = h // H
    X, Wq, Wk, Wv, bq, bk, bv, Wo = _gqa_inputs(rng, batch, seq, h, H, H_kv)
    got = oracle.attn_shard_gqa(X, Wq, Wk, Wv, bq, bk, bv, Wo, batch, seq, H, H_kv)
    want = oracle.attn_shard(X, Wq, _expand_kv(Wk, H, H_kv, d), _expand_kv(Wv, H, H_kv, d), bq,
                             _expand_kv(bk, H, H_kv, d), _expand_kv(bv, H, H_kv, d), Wo, batch,
                             seq, H)
    # the projections are matrix products of different widths (the library may block them
    # differently), so agreement is to rounding, not bitwise
    assert oracle.rel_frobenius(got, want) < 1e-13


def test_gqa_with_all_kv_heads_is_mha():
    rng = np.random.default_rng(27)
    batch, seq, h, H = 1, 9, 16, 4
    X, Wq, Wk, Wv, bq, bk, bv, Wo = _gqa_inputs(rng, batch, seq, h, H, H)
    for N in (1, 2, 4):
        for r in range(N):
            np.testing.assert_array_equal(
                oracle.attn_shard_gqa(X, Wq, Wk, Wv, bq, bk, bv, Wo, batch, seq, H, H, N, r),
                oracle.attn_shard(X, Wq, Wk, Wv, bq, bk, bv, Wo, batch, seq, H, N, r))


@pytest.mark.parametrize("H_kv,N", [(4, 2), (4, 4), (2, 4), (1, 4), (2, 8), (4, 8)])
def test_gqa_shards_sum_to_block(H_kv, N):
    """N | H_kv splits the key/value heads; N > H_kv duplicates them (the page's TP = 8 with
    4 key/value heads): either way the ranks' partials sum to the unsharded block."""
    rng = np.random.default_rng(28)
    batch, seq, h, H = 2, 5, 64, 8
    X, Wq, Wk, Wv, bq, bk, bv, Wo = _gqa_inputs(rng, batch, seq, h, H, H_kv)
    full = oracle.attn_shard_gqa(X, Wq, Wk, Wv, bq, bk, bv, Wo, batch, seq, H, H_kv)
    tot = sum(oracle.attn_shard_gqa(X, Wq, Wk, Wv, bq, bk, bv, Wo, batch, seq, H, H_kv, N, r)
              for r in range(N))
    assert oracle.rel_frobenius(tot, full) < 1e-13


def test_gqa_head_assignment_and_constraints():
    # N divides H_kv: contiguous key/value heads
    assert list(oracle.kv_heads_of_rank(32, 8, 4, 2)) == [4, 5]
    # N = 8 > H_kv = 4: ranks 2q and 2q+1 share (duplicate) head q
    assert [list(oracle.kv_heads_of_rank(32, 4, 8, r)) for r in range(8)] == [[q // 2] for q in range(8)]
    # neither divides: the page's divisibility constraint
    with pytest.raises(oracle.OracleError):
        oracle.kv_heads_of_rank(24, 6, 4, 0)
    with pytest.raises(oracle.OracleError):
        oracle.kv_heads_of_rank(30, 4, 2, 0)   # 30 query heads are not a multiple of 4


# --------------------------------------------------------------------------------------
# Backward pass of the MLP shard (llms.blog, "Partitioning the MLP Block", last paragraph)
# --------------------------------------------------------------------------------------
def test_gelu_grad_closed_forms_and_finite_differences():
    assert oracle.gelu_grad([0.0])[0] == 0.5
    # GeLU'(1) = Phi(1) + phi(1), textbook values of the standard normal
    assert abs(oracle.gelu_grad([1.0])[0] - (0.8413447460685429 + 0.24197072451914337)) < 1e-15
    xs = np.linspace(-6, 6, 1201)
    np.testing.assert_allclose(oracle.gelu_grad(xs) + oracle.gelu_grad(-xs), 1.0, atol=1e-15)
    hstep = 1e-5
    fd = (oracle.gelu(xs + hstep) - oracle.gelu(xs - hstep)) / (2 * hstep)
    np.testing.assert_allclose(oracle.gelu_grad(xs), fd, rtol=0, atol=1e-9)


def _loss(X, A, a, B, dZ, N, r):
    """L = <dZ, Z_r>: its gradient with respect to each input is what the backward returns."""
    return float(np.sum(oracle.mlp_shard(X, A, a, B, N, r) * dZ))


@pytest.mark.parametrize("N,r", [(1, 0), (2, 1), (4, 2)])
def test_mlp_backward_matches_finite_differences(N, r):
    rng = np.random.default_rng(29)
    T, h, F = 4, 8, 16
    X = rng.standard_normal((T, h))
    A = rng.standard_normal((h, F)) / 3
    a = rng.standard_normal(F) / 3
    B = rng.standard_normal((F, h)) / 4
    dZ = rng.standard_normal((T, h))
    g = oracle.mlp_shard_backward(X, A, a, B, dZ, N, r)
    cols = slice(r * F // N, (r + 1) * F // N)
    eps = 1e-6
    for name, arr, grad, sl in (("X", X, g["dX"], None), ("A", A, g["dA"], (slice(None), cols)),
                                ("a", a, g["da"], cols), ("B", B, g["dB"], (cols, slice(None)))):
        D = rng.standard_normal(arr.shape)
        if sl is not None:   # only the rank's slice moves its partial
            mask = np.zeros_like(D)
            mask[sl] = 1.0
            D *= mask
        args = {"X": X, "A": A, "a": a, "B": B}
        plus = dict(args, **{name: arr + eps * D})
        minus = dict(args, **{name: arr - eps * D})
        fd = (_loss(plus["X"], plus["A"], plus["a"], plus["B"], dZ, N, r)
              - _loss(minus["X"], minus["A"], minus["a"], minus["B"], dZ, N, r)) / (2 * eps)
        an = float(np.sum(grad * (D if sl is None else D[sl])))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_mlp_backward_tp_sums():
    """Column/row shards: dX partials sum to the block's dX (the backward all-reduce); dA, da
    and dB of the ranks are disjoint slices of the block's."""
    rng = np.random.default_rng(30)
    T, h, F = 5, 16, 32
    X = rng.standard_normal((T, h))
    A = rng.standard_normal((h, F)) / 4
    a = rng.standard_normal(F) / 4
    B = rng.standard_normal((F, h)) / 5
    dZ = rng.standard_normal((T, h))
    full = oracle.mlp_shard_backward(X, A, a, B, dZ, 1, 0)
    for N in (2, 4):
        parts = [oracle.mlp_shard_backward(X, A, a, B, dZ, N, r) for r in range(N)]
        assert oracle.rel_frobenius(sum(p["dX"] for p in parts), full["dX"]) < 1e-13
        np.testing.assert_allclose(np.concatenate([p["dA"] for p in parts], axis=1), full["dA"],
                                   rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(np.concatenate([p["da"] for p in parts]), full["da"],
                                   rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(np.concatenate([p["dB"] for p in parts], axis=0), full["dB"],
                                   rtol=1e-13, atol=1e-14)
