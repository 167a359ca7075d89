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
              rows=None) -> np.ndarray:
    """softmax(Q_j K_j^T / sqrt(d) + mask) V_j per head j, heads concatenated, on query rows."""
    Q, K, V = _as_d(Q), _as_d(K), _as_d(V)
    T, w = Q.shape
    d = w // n_heads
    rws = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nq = T if rws is None else rws.size
    O = np.empty((nq, w), dtype=np.float64)
    _check(_load().oracle_attention(_dp(Q), _dp(K), _dp(V), _dp(O), batch, seq, n_heads, d,
                                    int(bool(causal)),
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
