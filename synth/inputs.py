"""Seeded synthetic workloads for one tensor-parallel rank's Transformer-block shard.

Everything here is input preparation: random draws, bfloat16 rounding of those draws
(round-to-nearest-even) and the choice of sampled rows. No step of the method itself
(projection, activation, attention, reduction) is computed in this module.

Weights are drawn in the pages' layout ``W in R^{H_in x H_out}`` (llms.blog, "The Core
Primitives"); the HIP library's storage layout is produced from these arrays by pure
indexing in ``tensor_transformer_layers_amd.layout``.

Draw recipe (one ``numpy.random.default_rng(seed)`` stream per workload, seed 0 unless a
caller says otherwise): full, unsharded tensors are drawn one after another in a fixed
order with ``standard_normal(shape, dtype=float32)`` times a float32 standard deviation,
then rounded to bfloat16 for the bf16 workloads. Shards are later sliced out of the
full tensors, so every shard count N sees the same weights.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np


# ---------------------------------------------------------------------------------------
# bfloat16 rounding (round to nearest, ties to even) of float32 inputs
# ---------------------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Return the bfloat16 bit patterns (uint16) nearest to float32 ``x`` (ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite inputs: |bits| <= 0xFF7FFFFF, so adding at most 0x8000 cannot wrap in uint32
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16))
    r = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 array holding the bfloat16 values nearest to ``x`` (exactly representable)."""
    b = bf16_bits(x).astype(np.uint32) << 16
    return b.view(np.float32)


def normal_matrix(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


# ---------------------------------------------------------------------------------------
# Workload table: the five layer shapes measured and parity-tested
# ---------------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "mlp", "attn" or "layer"
    dtype: str                # "f32" or "bf16"
    tokens: int               # T = batch * seq
    hidden: int               # h
    ffn: int = 0              # F (MLP width)
    heads: int = 0            # H (attention heads); head dim d = h / H
    kv_heads: int = 0         # H_kv (grouped-query attention; 0 = H)
    batch: int = 1
    seq: int = 0
    n_shards: int = 1         # TP degree N
    causal: bool = True
    x_std: float = 1.0
    w_std: float = 0.02       # weights and biases
    fan_in_scaled: bool = False   # True: each weight/bias scaled by 1/sqrt(fan_in)
    description: str = ""


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(
            name="mlp_f32_t32_h1024_f4096_n2", kind="mlp", dtype="f32",
            tokens=32, hidden=1024, ffn=4096, n_shards=2, fan_in_scaled=True,
            description="fp32 MLP block GeLU(XA+a)B, X 32x1024, A 1024x4096, B 4096x1024, "
                        "N=2 shards on one device plus on-device sum (worked example shapes "
                        "of the apxml.com page's ColumnParallelLinear listing)"),
        Workload(
            name="mlp_shard_bf16_t8192_h3072_f12288_n8", kind="mlp", dtype="bf16",
            tokens=8192, batch=8, seq=1024, hidden=3072, ffn=12288, n_shards=8,
            description="one rank's bf16 MLP shard: A_i 3072x1536, B_i 1536x3072, fp32 partial"),
        Workload(
            name="attn_shard_bf16_b4_s2048_h4096_H32_n8", kind="attn", dtype="bf16",
            tokens=8192, batch=4, seq=2048, hidden=4096, heads=32, n_shards=8,
            description="one rank's bf16 causal attention shard: 4 local heads of d=128, "
                        "W_qkv,i 4096x1536, W_o,i 512x4096"),
        Workload(
            name="layer_shard_bf16_b1_s4096_h8192_H64_f32768_n8", kind="layer", dtype="bf16",
            tokens=4096, batch=1, seq=4096, hidden=8192, heads=64, ffn=32768, n_shards=8,
            description="one rank's bf16 Transformer-layer shard: attention (8 local heads) "
                        "then MLP (ffn shard 4096)"),
        Workload(
            name="mlp_block_bf16_t2048_h12288_f49152", kind="mlp", dtype="bf16",
            tokens=2048, hidden=12288, ffn=49152, n_shards=8,
            description="all N shards of one bf16 MLP block plus on-device sum, N in {1,2,4,8}"),
        # Paths next to the core shard (none of these is among the measured configurations
        # above; the shapes follow the model family the pages name for each feature).
        Workload(
            name="swiglu_shard_bf16_t4096_h8192_f28672_n8", kind="swiglu", dtype="bf16",
            tokens=4096, batch=1, seq=4096, hidden=8192, ffn=28672, n_shards=8,
            description="one rank's gated (SwiGLU) MLP shard of a LLaMA-style layer: W_gate,i and "
                        "W_up,i 8192x3584, W_down,i 3584x8192, fp32 partial"),
        Workload(
            name="gqa_shard_bf16_b1_s4096_h8192_H64_kv8_n8", kind="gqa", dtype="bf16",
            tokens=4096, batch=1, seq=4096, hidden=8192, heads=64, kv_heads=8, n_shards=8,
            description="one rank's grouped-query attention shard: 8 local query heads sharing "
                        "one local key/value head (64 query and 8 key/value heads, d=128)"),
        Workload(
            name="gqa_shard_bf16_b1_s4096_h8192_H64_kv4_n8", kind="gqa", dtype="bf16",
            tokens=4096, batch=1, seq=4096, hidden=8192, heads=64, kv_heads=4, n_shards=8,
            description="the same with 4 key/value heads on N=8 ranks: each key/value head is "
                        "duplicated on 2 ranks"),
        Workload(
            name="sp_boundary_bf16_b1_s4096_h8192_n8", kind="sp", dtype="bf16",
            tokens=4096, batch=1, seq=4096, hidden=8192, n_shards=8,
            description="sequence-parallel block boundary of one rank: reduce-scatter of 8 fp32 "
                        "partials onto its 512-token slice, residual add, LayerNorm"),
        Workload(
            name="mlp_bwd_bf16_t4096_h8192_f32768_n8", kind="mlp_bwd", dtype="bf16",
            tokens=4096, batch=1, seq=4096, hidden=8192, ffn=32768, n_shards=8,
            description="backward pass of one rank's bf16 MLP shard (the layer's ffn shard 4096)"),
    ]
}


def _std(w: Workload, fan_in: int) -> float:
    if w.fan_in_scaled:
        return 1.0 / math.sqrt(fan_in)
    return w.w_std


def mlp_inputs(w: Workload, seed: int = 0, tokens: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Full, unsharded MLP tensors in the pages' layout, drawn in the order X, A, a, B.

    X [T, h], A [h, F], a [F], B [F, h]; float32 (bf16-exact for bf16 workloads).
    ``tokens`` overrides T (the first rows of the same stream are not reused: the
    whole draw uses the overridden shape).
    """
    T = w.tokens if tokens is None else tokens
    h, F = w.hidden, w.ffn
    rng = np.random.default_rng(seed)
    X = normal_matrix(rng, (T, h), w.x_std)
    A = normal_matrix(rng, (h, F), _std(w, h))
    a = normal_matrix(rng, (F,), _std(w, h))
    B = normal_matrix(rng, (F, h), _std(w, F))
    out = dict(X=X, A=A, a=a, B=B)
    if w.dtype == "bf16":
        out = {k: bf16_round(v) for k, v in out.items()}
    return out


def attn_inputs(w: Workload, seed: int = 0, with_bias: bool = True,
                batch: Optional[int] = None, seq: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Full attention-block tensors in the pages' layout.

    Draw order X, W_Q, W_K, W_V, b_Q, b_K, b_V, W_O; for a layer workload the MLP
    tensors A, a, B follow in the same stream. X [batch*seq, h] with row t = b*seq + s,
    W_Q/W_K/W_V/W_O [h, h], biases [h].
    """
    b = w.batch if batch is None else batch
    s = w.seq if seq is None else seq
    h = w.hidden
    rng = np.random.default_rng(seed)
    out = {}
    out["X"] = normal_matrix(rng, (b * s, h), w.x_std)
    for k in ("Wq", "Wk", "Wv"):
        out[k] = normal_matrix(rng, (h, h), _std(w, h))
    for k in ("bq", "bk", "bv"):
        out[k] = normal_matrix(rng, (h,), _std(w, h))
    out["Wo"] = normal_matrix(rng, (h, h), _std(w, h))
    if w.kind == "layer":
        F = w.ffn
        out["A"] = normal_matrix(rng, (h, F), _std(w, h))
        out["a"] = normal_matrix(rng, (F,), _std(w, h))
        out["B"] = normal_matrix(rng, (F, h), _std(w, F))
    if not with_bias:
        for k in ("bq", "bk", "bv"):
            out[k] = np.zeros_like(out[k])
    if w.dtype == "bf16":
        out = {k: bf16_round(v) for k, v in out.items()}
    return out


def swiglu_inputs(w: Workload, seed: int = 0, tokens: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Full gated-MLP tensors in the pages' layout, drawn in the order X, W_gate, W_up, W_down:
    X [T, h], Wg and Wu [h, F], Wd [F, h]; float32, bf16-exact for bf16 workloads."""
    T = w.tokens if tokens is None else tokens
    h, F = w.hidden, w.ffn
    rng = np.random.default_rng(seed)
    out = dict(X=normal_matrix(rng, (T, h), w.x_std))
    out["Wg"] = normal_matrix(rng, (h, F), _std(w, h))
    out["Wu"] = normal_matrix(rng, (h, F), _std(w, h))
    out["Wd"] = normal_matrix(rng, (F, h), _std(w, F))
    if w.dtype == "bf16":
        out = {k: bf16_round(v) for k, v in out.items()}
    return out


def gqa_inputs(w: Workload, seed: int = 0, batch: Optional[int] = None,
               seq: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Grouped-query attention tensors, drawn in the order X, W_Q, W_K, W_V, b_Q, b_K, b_V,
    W_O: W_Q [h, H d], W_K and W_V [h, H_kv d], W_O [H d, h] (d = h / H)."""
    b = w.batch if batch is None else batch
    s = w.seq if seq is None else seq
    h, H = w.hidden, w.heads
    hkv = w.kv_heads or H
    d = h // H
    rng = np.random.default_rng(seed)
    out = dict(X=normal_matrix(rng, (b * s, h), w.x_std))
    out["Wq"] = normal_matrix(rng, (h, H * d), _std(w, h))
    out["Wk"] = normal_matrix(rng, (h, hkv * d), _std(w, h))
    out["Wv"] = normal_matrix(rng, (h, hkv * d), _std(w, h))
    out["bq"] = normal_matrix(rng, (H * d,), _std(w, h))
    out["bk"] = normal_matrix(rng, (hkv * d,), _std(w, h))
    out["bv"] = normal_matrix(rng, (hkv * d,), _std(w, h))
    out["Wo"] = normal_matrix(rng, (H * d, h), _std(w, h))
    if w.dtype == "bf16":
        out = {k: bf16_round(v) for k, v in out.items()}
    return out


def layernorm_params(h: int, seed: int = 0) -> Dict[str, np.ndarray]:
    """LayerNorm gain and shift of width h: gamma ~ 1 + N(0, 0.1), beta ~ N(0, 0.1), fp32."""
    rng = np.random.default_rng(seed + 104729)
    return dict(gamma=(1.0 + 0.1 * rng.standard_normal(h)).astype(np.float32),
                beta=(0.1 * rng.standard_normal(h)).astype(np.float32))


def partials_inputs(n_parts: int, numel: int, seed: int = 0, integer: bool = False) -> np.ndarray:
    """``n_parts`` fp32 partials of ``numel`` elements, [n_parts, numel].

    ``integer=True`` draws integers in [-1000, 1000] (sums exact in fp32 for any order).
    """
    rng = np.random.default_rng(seed)
    if integer:
        return rng.integers(-1000, 1001, size=(n_parts, numel)).astype(np.float32)
    return rng.standard_normal((n_parts, numel), dtype=np.float32)


def sample_rows(n_rows: int, n_sample: int, seed: int = 0,
                must: Sequence[int] = ()) -> np.ndarray:
    """Sorted distinct row indices: the first and last rows, ``must``, and seeded picks."""
    if n_sample >= n_rows:
        return np.arange(n_rows, dtype=np.int64)
    rng = np.random.default_rng(seed + 7919)
    picks = set([0, n_rows - 1]) | {int(m) for m in must if 0 <= m < n_rows}
    while len(picks) < n_sample:
        picks.add(int(rng.integers(0, n_rows)))
    return np.array(sorted(picks), dtype=np.int64)
