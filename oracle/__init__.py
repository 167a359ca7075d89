"""fp64 CPU oracle for one tensor-parallel rank's Transformer-block shard.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package. It shares no code with the HIP library
(``tensor_transformer_layers_amd``) and imports nothing from it.

The oracle follows the pages' notation and layout: activations X [rows, H_in], weights
W in R^{H_in x H_out} (llms.blog, "The Core Primitives"), token row t = b * seq + s.
Every step is fp64. The linear layers are fp64 matrix products (numpy's matmul serves as
the library primitive; inputs are exact fp32/bf16 values widened to fp64); GeLU, the
softmax attention (query by query) and the partial sum are plain loops in ``oracle.c``.

* ``gelu``                      exact-erf GeLU x Phi(x) (the pages name GeLU without a
                                formula; the exact form is the reading taken).
* ``linear``                    Y = X W + b (llms.blog, "The Core Primitives").
* ``mlp_column``/``mlp_row``    rank r's column-parallel GeLU(X A_r + a_r) and row-parallel
                                Y_r B_r, A_r = A[:, r F/N:(r+1) F/N], B_r = B[r F/N:(r+1) F/N, :]
                                (ai360xpert.com, "How It Works", steps 1-2; llms.blog,
                                "Partitioning the Multi-Layer Perceptron (MLP) Block").
* ``mlp_shard``                 rank r's partial; N = 1 is the unsharded block GeLU(XA + a)B.
* ``qkv_shard``/``attention``/``out_proj_shard``/``attn_shard``
                                head-partitioned attention: rank r owns heads r H/N ... of
                                width d = h/H, i.e. columns [r h/N, (r+1) h/N) of W_Q, W_K,
                                W_V and the same rows of W_O (llms.blog, "Partitioning
                                Multi-Head and Grouped-Query Attention", steps 1-3).
* ``sum_partials``              the all-reduce's sum (llms.blog, "Row-Parallel Linear Layer").
* ``silu``/``swiglu_column``/``swiglu_shard``
                                gated MLP shard SiLU(X W_gate,r) * (X W_up,r) W_down,r with the
                                gate and up projections split by columns and W_down by rows
                                (llms.blog, "Partitioning the MLP Block", steps 2-3).
* ``layernorm``/``sp_rows``/``reduce_scatter``/``all_gather``/``sp_boundary``
                                sequence parallelism: the row-parallel partials are summed onto
                                rank r's s/N slice of every sequence (reduce-scatter), the
                                residual is added and LayerNorm runs on the slice; an
                                all-gather restores the full sequence (llms.blog, "Sequence
                                Parallelism"; reduce-scatter then all-gather is the all-reduce).
* ``kv_heads_of_rank``/``attn_shard_gqa``
                                grouped-query attention: H_kv key/value heads, each shared by
                                H / H_kv query heads; a rank holds H_kv / N of them, or one
                                duplicated head when N > H_kv (llms.blog, "Grouped-Query
                                Attention (GQA) Constraints").
* ``gelu_grad``/``mlp_shard_backward``
                                rank r's gradients of the MLP shard: dY = dZ B_r^T, dP = dY *
                                GeLU'(P), dA_r = X^T dP, da_r = column sums of dP,
                                dB_r = Y_r^T dZ and the input-gradient partial dX_r = dP A_r^T,
                                whose sum over ranks is the backward all-reduce (llms.blog,
                                "Partitioning the MLP Block", closing paragraph).

Unequal splits raise ``OracleError``: the pages only use exact shards. Every function is
pinned in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_d = ctypes.POINTER(ctypes.c_double)
_f = ctypes.POINTER(ctypes.c_float)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64
_int = ctypes.c_int

# Column chunk of a weight widened to fp64 at a time (bounds memory; each output element's
# dot product is still computed whole by the matmul).
_CHUNK_ELEMS = 1 << 26


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, IEEE fp64, no fast-math)."""
    global _lib
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.oracle_gelu.restype = ctypes.c_double
    lib.oracle_gelu.argtypes = [ctypes.c_double]
    lib.oracle_gelu_array.argtypes = [_d, _d, _i64]
    lib.oracle_attention.argtypes = [_d, _d, _d, _d, _i64, _i64, _int, _i64, _int, _i64p, _i64]
    lib.oracle_attention.restype = _int
    lib.oracle_gelu_grad.restype = ctypes.c_double
    lib.oracle_gelu_grad.argtypes = [ctypes.c_double]
    lib.oracle_gelu_grad_array.argtypes = [_d, _d, _i64]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_silu_array.argtypes = [_d, _d, _i64]
    lib.oracle_layernorm.argtypes = [_d, _d, _d, ctypes.c_double, _i64, _i64, _d]
    lib.oracle_layernorm.restype = _int
    lib.oracle_attention_gqa.argtypes = [_d, _d, _d, _d, _i64, _i64, _int, _int, _i64, _int,
                                         _i64p, _i64]
    lib.oracle_attention_gqa.restype = _int
    lib.oracle_sum_partials.argtypes = [_f, _int, _i64, _d]
    lib.oracle_sum_partials.restype = _int
    lib.oracle_max_threads.restype = _int
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _dp(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_d)


def _as_d(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError("%s failed (rc=%d): invalid shape, rank or split" % (what, rc))


def _split(n: int, N: int, r: int, what: str) -> slice:
    """Rank r's contiguous 1/N of a dimension of size n (exact splits only)."""
    if N < 1 or r < 0 or r >= N or n % N != 0:
        raise OracleError("cannot split %s=%d over N=%d for rank %d" % (what, n, N, r))
    w = n // N
    return slice(r * w, (r + 1) * w)


def threads() -> int:
    return int(_load().oracle_max_threads())


# ---- element-wise -------------------------------------------------------------------------
def gelu(x):
    x = _as_d(x)
    y = np.empty_like(x)
    _load().oracle_gelu_array(_dp(x), _dp(y), x.size)
    return y


def gelu_grad(x):
    """GeLU'(x) = Phi(x) + x phi(x)."""
    x = _as_d(x)
    y = np.empty_like(x)
    _load().oracle_gelu_grad_array(_dp(x), _dp(y), x.size)
    return y


def silu(x):
    """SiLU(x) = x sigmoid(x)."""
    x = _as_d(x)
    y = np.empty_like(x)
    _load().oracle_silu_array(_dp(x), _dp(y), x.size)
    return y


def layernorm(x, gamma, beta, eps: float = 1e-5):
    """Row-wise (x - mean) / sqrt(var + eps) * gamma + beta over the last dimension."""
    x = _as_d(x)
    cols = x.shape[-1]
    g, b = _as_d(gamma), _as_d(beta)
    if g.shape != (cols,) or b.shape != (cols,):
        raise OracleError("layernorm: gamma/beta must have %d entries" % cols)
    y = np.empty_like(x)
    _check(_load().oracle_layernorm(_dp(x), _dp(g), _dp(b), float(eps), x.size // cols, cols,
                                    _dp(y)), "layernorm")
    return y


# ---- linear layer -------------------------------------------------------------------------
def linear(X, W, b=None) -> np.ndarray:
    """Y = X W (+ b): X [rows, H_in], W [H_in, H_out] (pages' layout), b [H_out], all fp64."""
    X = _as_d(X)
    W = np.asarray(W)
    rows, k = X.shape
    k2, n = W.shape
    if k != k2:
        raise OracleError("linear: X has %d columns, W has %d rows" % (k, k2))
    Y = np.empty((rows, n), dtype=np.float64)
    step = max(1, _CHUNK_ELEMS // max(1, k))
    for c0 in range(0, n, step):
        c1 = min(n, c0 + step)
        np.matmul(X, W[:, c0:c1].astype(np.float64), out=Y[:, c0:c1])
    if b is not None:
        Y += np.asarray(b, dtype=np.float64)
    return Y


# ---- MLP block ----------------------------------------------------------------------------
def mlp_column(X, A, a, N: int, r: int) -> np.ndarray:
    """Y_r = GeLU(X A_r + a_r) with A_r = A[:, r F/N:(r+1) F/N] and a_r the same slice of a."""
    cols = _split(np.shape(A)[1], N, r, "F")
    return gelu(linear(X, A[:, cols], None if a is None else a[cols]))


def mlp_row(Y_r, B, N: int, r: int) -> np.ndarray:
    """Z_r = Y_r B_r with B_r = B[r F/N:(r+1) F/N, :]."""
    rows = _split(np.shape(B)[0], N, r, "F")
    return linear(Y_r, B[rows, :])


def mlp_shard(X, A, a, B, N: int = 1, r: int = 0) -> np.ndarray:
    """Rank r's partial GeLU(X A_r + a_r) B_r; N = 1 gives the unsharded MLP block."""
    return mlp_row(mlp_column(X, A, a, N, r), B, N, r)


# ---- attention block ---------------------------------------------------------------------
def _head_cols(h: int, H: int, N: int, r: int) -> slice:
    if H < 1 or h % H != 0:
        raise OracleError("hidden %d is not divisible by %d heads" % (h, H))
    if H % N != 0:
        raise OracleError("%d heads are not divisible over N=%d" % (H, N))
    return _split(h, N, r, "hidden")


def qkv_shard(X, Wq, Wk, Wv, bq=None, bk=None, bv=None, H: int = 1, N: int = 1, r: int = 0):
    """Q_r = X W_Q[:, C_r] + b_Q[C_r] and alike for K and V, each [T, h/N]."""
    h = np.shape(X)[1]
    c = _head_cols(h, H, N, r)
    sl = lambda b: None if b is None else b[c]
    return (linear(X, Wq[:, c], sl(bq)), linear(X, Wk[:, c], sl(bk)), linear(X, Wv[:, c], sl(bv)))


def attention(Q, K, V, batch: int, seq: int, n_heads: int, causal: bool = True,
              rows=None, n_kv_heads: Optional[int] = None) -> np.ndarray:
    """softmax(Q_j K_g^T / sqrt(d) + mask) V_g per query head j, heads concatenated, on query
    rows; g = j / (n_heads / n_kv_heads) is the key/value head (g = j when n_kv_heads is None)."""
    Q, K, V = _as_d(Q), _as_d(K), _as_d(V)
    T, w = Q.shape
    d = w // n_heads
    hkv = n_heads if n_kv_heads is None else int(n_kv_heads)
    if K.shape != (T, hkv * d) or V.shape != (T, hkv * d):
        raise OracleError("attention: K and V must be [%d, %d]" % (T, hkv * d))
    rws = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nq = T if rws is None else rws.size
    O = np.empty((nq, w), dtype=np.float64)
    _check(_load().oracle_attention_gqa(_dp(Q), _dp(K), _dp(V), _dp(O), batch, seq, n_heads,
                                        hkv, d, int(bool(causal)),
                                        None if rws is None else rws.ctypes.data_as(_i64p), nq),
           "attention")
    return O


def out_proj_shard(O_r, Wo, H: int, N: int, r: int) -> np.ndarray:
    """Z_r = O_r W_O[C_r, :]: the locally concatenated heads times the row slice of W_O."""
    h = np.shape(Wo)[0]
    c = _head_cols(h, H, N, r)
    return linear(O_r, Wo[c, :])


def attn_shard(X, Wq, Wk, Wv, bq, bk, bv, Wo, batch: int, seq: int, H: int, N: int = 1,
               r: int = 0, causal: bool = True, rows=None, want_heads: bool = False):
    """Rank r's attention partial on the requested token rows (all rows if None).

    Only the key positions a requested query can see are projected (causal: positions up to
    the latest requested one in its sequence). Returns Z_r [n_rows, h] (fp64), or
    (Z_r, O_r) with O_r [n_rows, h/N] the locally concatenated head outputs.
    """
    X = np.asarray(X)
    T, h = X.shape
    if T != batch * seq:
        raise OracleError("X has %d rows, batch*seq = %d" % (T, batch * seq))
    c = _head_cols(h, H, N, r)
    Hl = H // N
    w = h // N
    rws = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    if rws.size and (rws.min() < 0 or rws.max() >= T):
        raise OracleError("row index out of range")
    sl = lambda b: None if b is None else b[c]
    Q = np.zeros((T, w))
    K = np.zeros((T, w))
    V = np.zeros((T, w))
    for b in np.unique(rws // seq):
        pos = rws[rws // seq == b] % seq
        need = int(pos.max()) + 1 if causal else seq
        blk = slice(b * seq, b * seq + need)
        K[blk] = linear(X[blk], Wk[:, c], sl(bk))
        V[blk] = linear(X[blk], Wv[:, c], sl(bv))
    Q[rws] = linear(X[rws], Wq[:, c], sl(bq))
    O = attention(Q, K, V, batch, seq, Hl, causal, rows=rws)
    Z = out_proj_shard(O, Wo, H, N, r)
    return (Z, O) if want_heads else Z


# ---- grouped-query attention ------------------------------------------------------------------
def kv_heads_of_rank(H: int, H_kv: int, N: int, r: int) -> range:
    """Global key/value heads rank r holds: H_kv / N contiguous heads when N divides H_kv,
    else (N a multiple of H_kv: the heads are duplicated) the one head its query heads read."""
    if H_kv < 1 or H % H_kv != 0:
        raise OracleError("%d query heads are not a multiple of %d key/value heads" % (H, H_kv))
    if H % N != 0 or N < 1 or r < 0 or r >= N:
        raise OracleError("%d query heads cannot be split over N=%d for rank %d" % (H, N, r))
    if H_kv % N == 0:
        n = H_kv // N
        return range(r * n, (r + 1) * n)
    if N % H_kv == 0:
        g = (r * (H // N)) // (H // H_kv)
        return range(g, g + 1)
    raise OracleError("%d key/value heads neither divide nor are divided by N=%d" % (H_kv, N))


def attn_shard_gqa(X, Wq, Wk, Wv, bq, bk, bv, Wo, batch: int, seq: int, H: int, H_kv: int,
                   N: int = 1, r: int = 0, causal: bool = True, rows=None,
                   want_heads: bool = False):
    """Rank r's grouped-query attention partial on the requested token rows.

    Wq [h, H d] and Wo [H d, h] as in ``attn_shard``; Wk, Wv [h, H_kv d]. Rank r owns query
    heads r H/N .. and the key/value heads of ``kv_heads_of_rank``; local query head j reads
    local key/value head (global j) / (H / H_kv) - (first local key/value head).
    """
    X = np.asarray(X)
    T, h = X.shape
    if T != batch * seq:
        raise OracleError("X has %d rows, batch*seq = %d" % (T, batch * seq))
    if h % H != 0:
        raise OracleError("hidden %d is not divisible by %d heads" % (h, H))
    d = h // H
    kvr = kv_heads_of_rank(H, H_kv, N, r)
    Hl = H // N
    qc = slice(r * Hl * d, (r + 1) * Hl * d)
    kc = slice(kvr.start * d, kvr.stop * d)
    rws = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    if rws.size and (rws.min() < 0 or rws.max() >= T):
        raise OracleError("row index out of range")
    sl = lambda b, c: None if b is None else b[c]
    nkv = len(kvr)
    Q = np.zeros((T, Hl * d))
    K = np.zeros((T, nkv * d))
    V = np.zeros((T, nkv * d))
    for b in np.unique(rws // seq):
        pos = rws[rws // seq == b] % seq
        need = int(pos.max()) + 1 if causal else seq
        blk = slice(b * seq, b * seq + need)
        K[blk] = linear(X[blk], Wk[:, kc], sl(bk, kc))
        V[blk] = linear(X[blk], Wv[:, kc], sl(bv, kc))
    Q[rws] = linear(X[rws], Wq[:, qc], sl(bq, qc))
    # The global map (query head -> key/value head = head / (H / H_kv)) restricted to this
    # rank is local query head j -> local key/value head j / (Hl / nkv), which is what
    # ``attention`` applies with nkv key/value heads.
    group = H // H_kv
    loc = [(r * Hl + j) // group - kvr.start for j in range(Hl)]
    if Hl % nkv != 0 or loc != [j // (Hl // nkv) for j in range(Hl)]:
        raise OracleError("rank %d's query heads read key/value heads it does not hold" % r)
    O = attention(Q, K, V, batch, seq, Hl, causal, rows=rws, n_kv_heads=nkv)
    Z = linear(O, Wo[qc, :])
    return (Z, O) if want_heads else Z


# ---- sequence parallelism --------------------------------------------------------------------
def sp_rows(batch: int, seq: int, N: int, r: int) -> np.ndarray:
    """Token rows (t = b seq + s) of rank r's sequence slice s in [r seq/N, (r+1) seq/N)."""
    sl = _split(seq, N, r, "seq")
    return (np.arange(batch, dtype=np.int64)[:, None] * seq
            + np.arange(sl.start, sl.stop, dtype=np.int64)[None, :]).ravel()


def reduce_scatter(parts, batch: int, seq: int, N: int, r: int) -> np.ndarray:
    """sum_q parts[q] on rank r's rows only: [batch seq/N, h] (fp64)."""
    P = np.asarray(parts, dtype=np.float32)
    rows = sp_rows(batch, seq, N, r)
    return sum_partials(np.ascontiguousarray(P[:, rows, :]))


def all_gather(slices, batch: int, seq: int) -> np.ndarray:
    """Concatenate the N ranks' sequence slices back into [batch seq, h]."""
    N = len(slices)
    h = np.shape(slices[0])[-1]
    out = np.empty((batch * seq, h), dtype=np.asarray(slices[0]).dtype)
    for r, s in enumerate(slices):
        out[sp_rows(batch, seq, N, r)] = s
    return out


def sp_boundary(parts, residual_r, gamma, beta, batch: int, seq: int, N: int, r: int,
                eps: float = 1e-5):
    """Rank r's block boundary: H_r = reduce_scatter(parts) + residual_r, Y_r = LayerNorm(H_r)."""
    Hr = reduce_scatter(parts, batch, seq, N, r) + _as_d(residual_r)
    return Hr, layernorm(Hr, gamma, beta, eps)


# ---- SwiGLU MLP shard --------------------------------------------------------------------------
def swiglu_column(X, Wg, Wu, N: int, r: int) -> np.ndarray:
    """A_r = SiLU(X Wg_r) * (X Wu_r) with Wg_r, Wu_r the r-th column slices."""
    cols = _split(np.shape(Wg)[1], N, r, "F")
    if np.shape(Wu) != np.shape(Wg):
        raise OracleError("gate and up projections differ in shape")
    return silu(linear(X, Wg[:, cols])) * linear(X, Wu[:, cols])


def swiglu_shard(X, Wg, Wu, Wd, N: int = 1, r: int = 0) -> np.ndarray:
    """Rank r's partial A_r Wd_r with Wd_r = Wd[r F/N:(r+1) F/N, :]; N = 1 is the whole block."""
    rows = _split(np.shape(Wd)[0], N, r, "F")
    return linear(swiglu_column(X, Wg, Wu, N, r), Wd[rows, :])


# ---- backward pass of the MLP shard ------------------------------------------------------------
def mlp_shard_backward(X, A, a, B, dZ, N: int = 1, r: int = 0) -> dict:
    """Gradients of rank r's MLP partial Z_r = GeLU(X A_r + a_r) B_r for an upstream dZ.

    The loss sees Z = sum_r Z_r, so every rank receives the same dZ; dX is the sum over ranks
    of the returned dX partials. Returns dX [T, h] (rank r's partial), dA [h, F/N], da [F/N]
    and dB [F/N, h].
    """
    cols = _split(np.shape(A)[1], N, r, "F")
    X = _as_d(X)
    dZ = _as_d(dZ)
    Ar = _as_d(A[:, cols])
    Br = _as_d(B[cols, :])
    P = linear(X, Ar, None if a is None else a[cols])
    Y = gelu(P)
    dY = dZ @ Br.T
    dP = dY * gelu_grad(P)
    return {"dX": dP @ Ar.T, "dA": X.T @ dP, "da": dP.sum(axis=0), "dB": Y.T @ dZ}


# ---- partial sum ----------------------------------------------------------------------------
def sum_partials(parts) -> np.ndarray:
    """Z = sum_r parts[r] in fp64; parts is [n_parts, numel] float32."""
    P = np.ascontiguousarray(parts, dtype=np.float32)
    n = P.shape[0]
    numel = int(np.prod(P.shape[1:]))
    Z = np.empty(numel, dtype=np.float64)
    _check(_load().oracle_sum_partials(P.ctypes.data_as(_f), n, numel, _dp(Z)), "sum_partials")
    return Z.reshape(P.shape[1:])


def rel_frobenius(got, ref) -> float:
    """||got - ref||_F / ||ref||_F in fp64 (the parity metric)."""
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(o.ravel()))
    num = float(np.linalg.norm((g - o).ravel()))
    return num / den if den > 0 else num
