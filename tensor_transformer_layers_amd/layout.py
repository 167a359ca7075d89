"""Shard extraction: from full weights in the pages' layout to one rank's arrays in the ABI's.

The pages write a linear layer as Y = X W with W in R^{H_in x H_out} (llms.blog, "The Core
Primitives"). The library stores a weight as a linear layer does, [out_features,
in_features], so that both GEMM operands are contiguous along the reduced dimension.
These helpers only slice and transpose (pure indexing, no arithmetic):

* ``column_shard(W, N, r)``  W = [W_1 ... W_N] split on the output dimension
                             (ColumnParallelLinear): rank r's W_r^T, [H_out/N, H_in].
* ``row_shard(W, N, r)``     W = [W_1; ...; W_N] split on the input dimension
                             (RowParallelLinear): rank r's W_r^T, [H_out, H_in/N].
* ``bias_shard(b, N, r)``    the column bias slice that goes with ``column_shard``.
* ``qkv_shard(...)``         [W_Q | W_K | W_V] restricted to rank r's heads, [3 h/N, h]
                             (attention step 1: Q, K, V sliced column-wise by head).
* ``gqa_kv_heads(...)``, ``gqa_qkv_shard(...)``, ``gqa_qkv_bias_shard(...)``
                             grouped-query attention: rank r's query heads r H/N ... and its
                             key/value heads (H_kv / N of them, or the one duplicated head its
                             query heads read when N > H_kv), [(H/N + 2 KVl) d, h].
"""
from __future__ import annotations

import numpy as np


def _split(n: int, N: int, what: str) -> int:
    if N < 1 or n % N != 0:
        raise ValueError("%s=%d is not divisible by N=%d" % (what, n, N))
    return n // N


def column_shard(W: np.ndarray, N: int, r: int) -> np.ndarray:
    w = _split(W.shape[1], N, "H_out")
    return np.ascontiguousarray(W[:, r * w:(r + 1) * w].T)


def row_shard(W: np.ndarray, N: int, r: int) -> np.ndarray:
    w = _split(W.shape[0], N, "H_in")
    return np.ascontiguousarray(W[r * w:(r + 1) * w, :].T)


def bias_shard(b, N: int, r: int):
    if b is None:
        return None
    w = _split(b.shape[0], N, "bias")
    return np.ascontiguousarray(b[r * w:(r + 1) * w])


def qkv_shard(Wq: np.ndarray, Wk: np.ndarray, Wv: np.ndarray, N: int, r: int) -> np.ndarray:
    return np.concatenate([column_shard(W, N, r) for W in (Wq, Wk, Wv)], axis=0)


def qkv_bias_shard(bq, bk, bv, N: int, r: int):
    if bq is None:
        return None
    return np.concatenate([bias_shard(b, N, r) for b in (bq, bk, bv)])


def gqa_kv_heads(H: int, H_kv: int, N: int, r: int) -> range:
    """Global key/value heads held by rank r (H_kv / N contiguous heads, or one duplicated)."""
    if H % H_kv != 0 or H % N != 0:
        raise ValueError("heads %d / key-value heads %d / N %d do not split" % (H, H_kv, N))
    if H_kv % N == 0:
        n = H_kv // N
        return range(r * n, (r + 1) * n)
    if N % H_kv == 0:
        g = (r * (H // N)) // (H // H_kv)
        return range(g, g + 1)
    raise ValueError("%d key/value heads do not split over N=%d" % (H_kv, N))


def gqa_qkv_shard(Wq, Wk, Wv, H: int, H_kv: int, N: int, r: int) -> np.ndarray:
    """Rows [W_Q[:, C_r]^T ; W_K[:, K_r]^T ; W_V[:, K_r]^T] of rank r (d = W_Q width / H)."""
    d = Wq.shape[1] // H
    kv = gqa_kv_heads(H, H_kv, N, r)
    kc = slice(kv.start * d, kv.stop * d)
    return np.concatenate([column_shard(Wq, N, r), np.ascontiguousarray(Wk[:, kc].T),
                           np.ascontiguousarray(Wv[:, kc].T)], axis=0)


def gqa_qkv_bias_shard(bq, bk, bv, H: int, H_kv: int, N: int, r: int):
    if bq is None:
        return None
    d = bq.shape[0] // H
    kv = gqa_kv_heads(H, H_kv, N, r)
    kc = slice(kv.start * d, kv.stop * d)
    return np.concatenate([bias_shard(bq, N, r), bk[kc], bv[kc]])
