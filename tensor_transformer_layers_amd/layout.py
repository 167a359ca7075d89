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
