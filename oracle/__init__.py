"""fp64 CPU oracle for one tensor-parallel rank's Transformer-block shard.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package. It shares no code with the HIP library
(``tensor_transformer_layers_amd``) and imports nothing from it.

The arithmetic lives in ``oracle.c`` (plain loops, fp64, OpenMP over rows); this module
only builds it with gcc and marshals numpy arrays through ctypes. Every function follows
the passages cited in ``oracle.c``:

* ``gelu``                      exact-erf GeLU (the pages name GeLU without a formula).
* ``linear``                    Y = X W + b (llms.blog, "The Core Primitives").
* ``mlp_column``/``mlp_row``    rank r's column-parallel GeLU(X A_r + a_r) and row-parallel
                                Y_r B_r (ai360xpert.com, "How It Works"; llms.blog, MLP block).
* ``mlp_shard``                 rank r's partial; N = 1 is the unsharded block.
* ``qkv_shard``/``attention``/``out_proj_shard``/``attn_shard``
                                head-partitioned attention (llms.blog, "Partitioning
                                Multi-Head and Grouped-Query Attention").
* ``sum_partials``              the all-reduce's sum (llms.blog, "Row-Parallel Linear Layer").

Parity pins live in ``tests/test_oracle.py``; every function above is pinned there.
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
    lib.oracle_linear.argtypes = [_d, _f, _f, _d, _i64, _i64, _i64]
    lib.oracle_mlp_column.argtypes = [_d, _f, _f, _d, _i64, _i64, _i64, _int, _int]
    lib.oracle_mlp_row.argtypes = [_d, _f, _d, _i64, _i64, _i64, _int, _int]
    lib.oracle_mlp_shard.argtypes = [_d, _f, _f, _f, _d, _i64, _i64, _i64, _int, _int]
    lib.oracle_qkv_shard.argtypes = [_d, _f, _f, _f, _f, _f, _f, _d, _d, _d,
                                     _i64, _i64, _int, _int, _int]
    lib.oracle_attention.argtypes = [_d, _d, _d, _d, _i64, _i64, _int, _i64, _int, _i64p, _i64]
    lib.oracle_out_proj_shard.argtypes = [_d, _f, _d, _i64, _i64, _int, _int, _int]
    lib.oracle_attn_shard.argtypes = [_d, _f, _f, _f, _f, _f, _f, _f, _d, _d,
                                      _i64, _i64, _i64, _int, _int, _int, _int, _i64p, _i64]
    lib.oracle_sum_partials.argtypes = [_f, _int, _i64, _d]
    lib.oracle_matmul_dd.argtypes = [_d, _d, _d, _i64, _i64, _i64]
    lib.oracle_max_threads.restype = _int
    for name in ("oracle_mlp_column", "oracle_mlp_row", "oracle_mlp_shard", "oracle_qkv_shard",
                 "oracle_attention", "oracle_out_proj_shard", "oracle_attn_shard",
                 "oracle_sum_partials"):
        getattr(lib, name).restype = _int
    _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _dp(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_d)


def _fp(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_f)


def _as_d(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _as_f(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError("oracle weights must be float32 arrays (got %s)" % a.dtype)
    return a


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError("%s failed (rc=%d): invalid shape, rank or split" % (what, rc))


def threads() -> int:
    return int(_load().oracle_max_threads())


def gelu(x):
    x = _as_d(x)
    y = np.empty_like(x)
    _load().oracle_gelu_array(_dp(x), _dp(y), x.size)
    return y


def linear(X, W, b=None) -> np.ndarray:
    """Y = X W (+ b); X [rows, in] (fp64 copy), W [in, out] float32 (pages' layout)."""
    X = _as_d(X)
    W = _as_f(W)
    b = _as_f(b)
    rows, k = X.shape
    k2, n = W.shape
    assert k == k2
    Y = np.empty((rows, n), dtype=np.float64)
    _load().oracle_linear(_dp(X), _fp(W), _fp(b), _dp(Y), rows, k, n)
    return Y


def mlp_column(X, A, a, N: int, r: int) -> np.ndarray:
    X = _as_d(X)
    A = _as_f(A)
    a = _as_f(a)
    T, h = X.shape
    F = A.shape[1]
    Y = np.empty((T, F // max(N, 1)), dtype=np.float64)
    _check(_load().oracle_mlp_column(_dp(X), _fp(A), _fp(a), _dp(Y), T, h, F, N, r),
           "mlp_column")
    return Y


def mlp_row(Y_r, B, N: int, r: int) -> np.ndarray:
    Y_r = _as_d(Y_r)
    B = _as_f(B)
    F, h = B.shape
    T = Y_r.shape[0]
    Z = np.empty((T, h), dtype=np.float64)
    _check(_load().oracle_mlp_row(_dp(Y_r), _fp(B), _dp(Z), T, h, F, N, r), "mlp_row")
    return Z


def mlp_shard(X, A, a, B, N: int = 1, r: int = 0) -> np.ndarray:
    """Rank r's partial GeLU(X A_r + a_r) B_r; N = 1 gives the unsharded MLP block."""
    X = _as_d(X)
    A, a, B = _as_f(A), _as_f(a), _as_f(B)
    T, h = X.shape
    F = A.shape[1]
    Z = np.empty((T, h), dtype=np.float64)
    _check(_load().oracle_mlp_shard(_dp(X), _fp(A), _fp(a), _fp(B), _dp(Z), T, h, F, N, r),
           "mlp_shard")
    return Z


def qkv_shard(X, Wq, Wk, Wv, bq=None, bk=None, bv=None, H: int = 1, N: int = 1, r: int = 0):
    X = _as_d(X)
    Wq, Wk, Wv = _as_f(Wq), _as_f(Wk), _as_f(Wv)
    bq, bk, bv = _as_f(bq), _as_f(bk), _as_f(bv)
    T, h = X.shape
    w = h // N
    Q = np.empty((T, w)); K = np.empty((T, w)); V = np.empty((T, w))
    _check(_load().oracle_qkv_shard(_dp(X), _fp(Wq), _fp(Wk), _fp(Wv), _fp(bq), _fp(bk),
                                    _fp(bv), _dp(Q), _dp(K), _dp(V), T, h, H, N, r),
           "qkv_shard")
    return Q, K, V


def attention(Q, K, V, batch: int, seq: int, n_heads: int, causal: bool = True,
              rows=None) -> np.ndarray:
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
    O_r = _as_d(O_r)
    Wo = _as_f(Wo)
    n, _ = O_r.shape
    h = Wo.shape[1]
    Z = np.empty((n, h), dtype=np.float64)
    _check(_load().oracle_out_proj_shard(_dp(O_r), _fp(Wo), _dp(Z), n, h, H, N, r),
           "out_proj_shard")
    return Z


def attn_shard(X, Wq, Wk, Wv, bq, bk, bv, Wo, batch: int, seq: int, H: int, N: int = 1,
               r: int = 0, causal: bool = True, rows=None, want_heads: bool = False):
    """Rank r's attention partial on the requested token rows (all rows if None).

    Returns Z_r [n_rows, h] (fp64) or (Z_r, O_r) with O_r [n_rows, h/N], the locally
    concatenated head outputs, when ``want_heads``.
    """
    X = _as_d(X)
    Wq, Wk, Wv, Wo = _as_f(Wq), _as_f(Wk), _as_f(Wv), _as_f(Wo)
    bq, bk, bv = _as_f(bq), _as_f(bk), _as_f(bv)
    T, h = X.shape
    assert T == batch * seq
    rws = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nq = T if rws is None else rws.size
    Z = np.empty((nq, h), dtype=np.float64)
    O = np.empty((nq, h // N), dtype=np.float64) if want_heads else None
    _check(_load().oracle_attn_shard(_dp(X), _fp(Wq), _fp(Wk), _fp(Wv), _fp(bq), _fp(bk),
                                     _fp(bv), _fp(Wo), _dp(Z), _dp(O), batch, seq, h, H, N, r,
                                     int(bool(causal)),
                                     None if rws is None else rws.ctypes.data_as(_i64p), nq),
           "attn_shard")
    return (Z, O) if want_heads else Z


def sum_partials(parts) -> np.ndarray:
    """Z = sum_r parts[r] in fp64; parts is [n_parts, numel] float32."""
    P = np.ascontiguousarray(parts, dtype=np.float32)
    n = P.shape[0]
    numel = int(np.prod(P.shape[1:]))
    Z = np.empty(numel, dtype=np.float64)
    _check(_load().oracle_sum_partials(_fp(P), n, numel, _dp(Z)), "sum_partials")
    return Z.reshape(P.shape[1:])


def matmul_dd(X, W) -> np.ndarray:
    X, W = _as_d(X), _as_d(W)
    Y = np.empty((X.shape[0], W.shape[1]))
    _load().oracle_matmul_dd(_dp(X), _dp(W), _dp(Y), X.shape[0], X.shape[1], W.shape[1])
    return Y


def rel_frobenius(got, ref) -> float:
    """||got - ref||_F / ||ref||_F in fp64 (the parity metric)."""
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(o.ravel()))
    num = float(np.linalg.norm((g - o).ravel()))
    return num / den if den > 0 else num
