"""Host-side checks of the C ABI (no GPU): the library loads, exports every declared symbol,
and its validation rejects bad arguments with the documented status before any HIP call.

The pointers passed here are fake non-NULL values: every call is expected to fail
validation, so none of them is ever dereferenced and no kernel is launched.
"""
import os
import re
import subprocess

import pytest

from tensor_transformer_layers_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_shard.h")
P = 0x10000          # a fake, 16-byte aligned, non-NULL address (never dereferenced)
BIG = 1 << 40        # "large enough" workspace size
BF16, F32 = B.TP_BF16, B.TP_F32


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(B.LIB_PATH):
        from tensor_transformer_layers_amd import build
        build.build()
    B.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    declared = _declared_functions()
    assert set(declared) == set(B.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (tp_[a-z0-9_]+)$", out, flags=re.M))
    missing = [f for f in declared if f not in exported]
    assert not missing, missing
    for f in declared:
        assert hasattr(B.lib(), f)


def test_abi_version_matches_header():
    text = open(HEADER).read()
    v = int(re.search(r"#define TP_SHARD_ABI_VERSION (\d+)", text).group(1))
    assert B.tp_abi_version() == v


def _mlp(**kw):
    a = dict(X=P, A_i=P, a_i=P, B_i=P, Z_i=P, tokens=32, hidden=1024, ffn=4096, n_shards=2,
             rank=0, dt=F32, workspace=P, workspace_bytes=BIG)
    a.update(kw)
    return B.tp_mlp_shard_fwd(**a)


def _swiglu(**kw):
    a = dict(X=P, Wgate_i=P, Wup_i=P, Wdown_i=P, Z_i=P, tokens=4096, hidden=8192, ffn=28672,
             n_shards=8, rank=0, dt=BF16, workspace=P, workspace_bytes=BIG)
    a.update(kw)
    return B.tp_swiglu_shard_fwd(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), 1), (dict(Wgate_i=None), 1), (dict(Wup_i=None), 1), (dict(Wdown_i=None), 1),
    (dict(Z_i=None), 1),
    (dict(n_shards=3), 3),                 # 28672 % 3 != 0
    (dict(tokens=0), 2), (dict(rank=8), 4),
    (dict(dt=F32), 5),                     # bf16 only
    (dict(Wup_i=P + 8), 6), (dict(hidden=8196), 6),
    (dict(workspace=None), 7), (dict(workspace_bytes=4096 * 3584 * 2 - 1), 7),
    (dict(hidden=(1 << 22) + 8), 2),
])
def test_swiglu_validation(kw, status):
    assert _swiglu(**kw) == status
    assert B.tp_last_error() != ""


def test_sp_validation():
    parts = [P] * 8
    # reduce-scatter: seq not divisible into N slices, bad rank, missing rank, dtype
    assert B.tp_reduce_scatter_partials(parts, 8, 1, 4095, 8192, 0, P, F32) == 3
    assert B.tp_reduce_scatter_partials(parts, 8, 1, 4096, 8192, 8, P, F32) == 4
    assert B.tp_reduce_scatter_partials([P, None] + [P] * 6, 8, 1, 4096, 8192, 0, P, F32) == 1
    assert B.tp_reduce_scatter_partials(parts, 8, 1, 4096, 8192, 0, P, 3) == 5
    assert B.tp_reduce_scatter_partials(parts, 8, 1, 4096, 8196, 0, P, F32) == 6
    assert B.tp_reduce_scatter_partials(parts, 0, 1, 4096, 8192, 0, P, F32) == 2
    # residual + LayerNorm: hidden above the per-row LDS limit, NULL gamma, bad eps
    lnargs = dict(Z_parts=parts, n_parts=8, residual_r=None, gamma=P, beta=P, eps=1e-5, H_r=P,
                  Y_r=P, batch=1, seq=4096, hidden=8192, rank=0, dt=BF16)
    assert B.tp_sp_residual_layernorm_fwd(**dict(lnargs, hidden=16392)) == 2
    assert B.tp_sp_residual_layernorm_fwd(**dict(lnargs, gamma=None)) == 1
    assert B.tp_sp_residual_layernorm_fwd(**dict(lnargs, eps=-1.0)) == 2
    assert B.tp_sp_residual_layernorm_fwd(**dict(lnargs, residual_r=P + 4)) == 6
    assert B.tp_sp_residual_layernorm_fwd(**dict(lnargs, seq=100)) == 3
    # all-gather
    assert B.tp_all_gather_rows(parts, 8, 1, 4095, 8192, P, BF16) == 3
    assert B.tp_all_gather_rows(parts, 8, 1, 4096, 8192, None, BF16) == 1
    assert B.tp_last_error() != ""


def _attn(**kw):
    a = dict(X=P, Wqkv_i=P, bqkv_i=None, Wo_i=P, Z_i=P, batch=4, seq=2048, hidden=4096,
             n_heads=32, causal=1, n_shards=8, rank=0, dt=BF16, workspace=P,
             workspace_bytes=BIG)
    a.update(kw)
    return B.tp_attn_shard_fwd(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), 1), (dict(A_i=None), 1), (dict(B_i=None), 1), (dict(Z_i=None), 1),
    (dict(n_shards=3), 3),                 # 4096 % 3 != 0 (pages only use exact shards)
    (dict(n_shards=0), 2), (dict(tokens=0), 2), (dict(hidden=-1), 2),
    (dict(rank=2), 4), (dict(rank=-1), 4),
    (dict(dt=7), 5),
    (dict(X=P + 8), 6), (dict(a_i=P + 4), 6), (dict(hidden=1020), 6),
    (dict(ffn=4096 + 2 * 4), 6),           # ffn/N = 2052 is not a multiple of 8
    (dict(workspace=None), 7), (dict(workspace_bytes=100), 7),
    (dict(hidden=(1 << 22) + 8), 2),       # reduced dimension above 2^22 (32-bit tile offsets)
])
def test_mlp_validation(kw, status):
    assert _mlp(**kw) == status
    assert B.tp_last_error() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), 1), (dict(Wqkv_i=None), 1), (dict(Wo_i=None), 1), (dict(Z_i=None), 1),
    (dict(n_heads=30), 3),                 # 4096 % 30 != 0
    (dict(n_shards=3), 3),                 # 32 heads over 3 ranks
    (dict(n_heads=16), 2),                 # d = 256: unsupported head width
    (dict(rank=8), 4),
    (dict(dt=F32), 5),
    (dict(bqkv_i=P + 2), 6),
    (dict(workspace_bytes=1), 7),
    (dict(seq=0), 2),
    (dict(hidden=(1 << 22) + 4096), 2),   # reduced dimension of the QKV projection above 2^22
    (dict(batch=1, seq=(1 << 22) + 1), 2),  # a head's keys past 32-bit offsets
])
def test_attn_validation(kw, status):
    assert _attn(**kw) == status
    assert B.tp_last_error() != ""


def test_mlp_bwd_validation_and_workspace():
    args = dict(X=P, A_i=P, a_i=None, B_i=P, dZ=P, dX_i=P, dA_i=P, da_i=None, dB_i=P, tokens=4096,
                hidden=8192, ffn=32768, n_shards=8, rank=0, dt=BF16, workspace=P, workspace_bytes=BIG)
    g = lambda **kw: B.tp_mlp_shard_bwd(**dict(args, **kw))
    assert g(dZ=None) == 1 and g(dB_i=None) == 1
    assert g(dt=F32) == 5
    assert g(n_shards=3) == 3
    assert g(rank=9) == 4
    assert g(da_i=P + 4) == 6
    assert g(workspace_bytes=1024) == 7
    assert g(tokens=(1 << 22) + 1) == 2        # dA and dB reduce over the tokens
    assert B.tp_mlp_bwd_workspace_bytes((1 << 22) + 1, 8192, 32768, 8, BF16) == 0
    # P, dP [T, F/N]; B^T [F/N, h]; A^T [h, F/N]; dP^T, GeLU(P)^T [F/N, T8]; X^T, dZ^T [h, T8]
    T, h, fl = 4096, 8192, 4096
    want = 2 * (2 * T * fl + 2 * fl * h + 2 * fl * T + 2 * h * T)
    assert B.tp_mlp_bwd_workspace_bytes(T, h, 32768, 8, BF16) == want
    # tokens are padded to a multiple of 8 in the transposed buffers
    assert B.tp_mlp_bwd_workspace_bytes(5, 8, 16, 1, BF16) > 0
    assert B.tp_mlp_bwd_workspace_bytes(5, 8, 16, 1, F32) == 0


def test_gqa_validation_and_layout():
    args = dict(X=P, Wqkv_i=P, bqkv_i=None, Wo_i=P, Z_i=P, batch=1, seq=4096, hidden=8192,
                n_heads=64, n_kv_heads=8, causal=1, n_shards=8, rank=0, dt=BF16, workspace=P,
                workspace_bytes=BIG)
    g = lambda **kw: B.tp_gqa_attn_shard_fwd(**dict(args, **kw))
    assert g(n_kv_heads=6) == 3        # 64 query heads are not a multiple of 6
    assert g(n_kv_heads=12, n_heads=48, hidden=6144) == 3  # 12 % 8 != 0 and 8 % 12 != 0
    assert g(n_kv_heads=3, n_heads=48, hidden=6144) == 3   # 3 neither divides nor is divided by 8
    assert g(rank=8) == 4
    assert g(dt=F32) == 5
    assert g(workspace_bytes=1) == 7
    # layout: Q for 8 local query heads, K and V^T for one local key/value head (64 / 8 / 8)
    st, off = B.tp_gqa_attn_workspace_layout(1, 4096, 8192, 64, 8, 8, BF16)
    q = 4096 * 8 * 128 * 2
    kv = 4096 * 1 * 128 * 2
    assert st == 0 and off == dict(q=0, k=q, vt=q + kv, o=q + 2 * kv)
    # 4 key/value heads on 8 ranks: duplicated, still one per rank
    st, off4 = B.tp_gqa_attn_workspace_layout(1, 4096, 8192, 64, 4, 8, BF16)
    assert st == 0 and off4 == off
    # H_kv = H is the multi-head layout
    assert (B.tp_gqa_attn_workspace_bytes(4, 2048, 4096, 32, 32, 8, BF16)
            == B.tp_attn_workspace_bytes(4, 2048, 4096, 32, 8, BF16))


def test_gqa_workspace_holds_the_split_projection(overrides):
    """4096 x 1280 x 8192 (8 query heads and one key/value head per rank) gives 80 tiles of
    256 x 256: the projection is split three ways along K, and its fp32 partials
    [3][4096][1280] take the space from O on (past the attention's own partials)."""
    q, kv = 4096 * 8 * 128 * 2, 4096 * 1 * 128 * 2
    o = q + 2 * kv
    assert B.tp_gqa_attn_workspace_bytes(1, 4096, 8192, 64, 8, 8, BF16) == o + 3 * 4096 * 1280 * 4
    # without the split: O, then the key-range halves' outputs and (max, denominator)
    overrides("qkv_split=1")
    unsplit = o + 4096 * 1024 * 2 + 256 * 2 * 128 * 128 * 4 + 256 * 2 * 128 * 2 * 4
    assert B.tp_gqa_attn_workspace_bytes(1, 4096, 8192, 64, 8, 8, BF16) == unsplit
    # the multi-head layer shape (4096 x 3072 x 8192: 192 tiles) is not split
    overrides(None)
    st, off = B.tp_attn_workspace_layout(1, 4096, 8192, 64, 8, BF16)
    assert st == 0
    assert B.tp_attn_workspace_bytes(1, 4096, 8192, 64, 8, BF16) == (
        off["o"] + 4096 * 1024 * 2 + 256 * 2 * 128 * 130 * 4)


def test_sum_validation():
    assert B.tp_sum_partials([P, P], 0, 10, P, F32) == 2
    assert B.tp_sum_partials([P] * 65, 65, 10, P, F32) == 2
    assert B.tp_sum_partials([P, P], 2, 0, P, F32) == 2
    assert B.tp_sum_partials([P, None, P], 3, 10, P, F32) == 1   # a missing rank
    assert "partial 1" in B.tp_last_error()
    assert B.tp_sum_partials([P, P + 4], 2, 10, P, F32) == 6
    assert B.tp_sum_partials([P, P], 2, 10, P, 3) == 5
    assert B.tp_sum_partials([P, P], 2, 10, None, F32) == 1


def test_sum_and_exchange_aliasing():
    """An fp32 sum may be written over one of its partials (same pointer); a bf16 output
    over a partial, or any partial overlap, is TP_ERR_ALIAS. (Calls that pass validation
    stop at the device check on a host without a GPU: status 8, never 10.)"""
    Q = P + (1 << 20)
    assert B.tp_sum_partials([P, Q], 2, 1000, Q, F32) != 10
    assert B.tp_sum_partials([P, Q], 2, 1000, P, BF16) == 10
    assert "partial 0" in B.tp_last_error()
    assert B.tp_sum_partials([P, Q], 2, 1000, Q + 16, F32) == 10
    assert B.tp_sum_partials([P, Q], 2, 1000, P - 16, F32) == 10
    assert B.tp_sum_partials([P, Q], 2, 1000, P + 4000, F32) != 10     # just past partial 0
    # reduce-scatter / boundary / all-gather outputs must not touch an input
    parts = [P + i * (1 << 26) for i in range(8)]
    far = P + (1 << 30)
    assert B.tp_reduce_scatter_partials(parts, 8, 1, 4096, 8192, 0, parts[3], BF16) == 10
    assert B.tp_reduce_scatter_partials(parts, 8, 1, 4096, 8192, 0, far, BF16) != 10
    ln = dict(Z_parts=parts, n_parts=8, residual_r=None, gamma=P, beta=P, eps=1e-5, H_r=far,
              Y_r=far + (1 << 24), batch=1, seq=4096, hidden=8192, rank=0, dt=BF16)
    assert B.tp_sp_residual_layernorm_fwd(**ln) != 10
    assert B.tp_sp_residual_layernorm_fwd(**dict(ln, Y_r=far)) == 10            # Y over H
    assert B.tp_sp_residual_layernorm_fwd(**dict(ln, H_r=parts[7] + 256)) == 10
    assert B.tp_sp_residual_layernorm_fwd(**dict(ln, residual_r=far)) != 10     # H is the residual
    assert B.tp_sp_residual_layernorm_fwd(**dict(ln, residual_r=far + 16)) == 10
    assert B.tp_all_gather_rows(parts, 8, 1, 4096, 8192, parts[0] + 1024, BF16) == 10


def test_reduced_dimension_limit_is_below_2_22():
    """256 bf16 rows of K = 2^22 elements span 2^31 bytes, past a buffer descriptor's range:
    K = 2^22 is rejected, K = 2^22 - 8 passes validation."""
    big, ok = 1 << 22, (1 << 22) - 8
    assert B.tp_column_parallel_fwd(P, P, None, P, 8, big, 8, 1, 0, 0, BF16) == 2
    assert B.tp_column_parallel_fwd(P, P, None, P, 8, ok, 8, 1, 0, 0, BF16) != 2
    assert B.tp_row_parallel_fwd(P, P, P, 8, big, 8, 1, 0, BF16) == 2
    assert B.tp_mlp_workspace_bytes(8, big, 8, 1, BF16) == 0
    assert B.tp_mlp_workspace_bytes(8, 8, big, 1, BF16) == 0
    assert B.tp_mlp_workspace_bytes(8, ok, ok, 1, BF16) > 0
    assert B.tp_mlp_bwd_workspace_bytes(big, 8, 8, 1, BF16) == 0
    assert B.tp_mlp_bwd_workspace_bytes(ok, 8, 8, 1, BF16) > 0


def test_test_overrides_parsing():
    assert B.tp_set_test_overrides(None) == 0
    assert B.tp_set_test_overrides("") == 0
    for good in ("gemm_tile=256x192", "gemm_tile=128x128w4,qkv_split=3", "attn_sets=1",
                 "attn_split=2,sum_grid=7,sum_unroll=2", "sum_defer=0", "sum_defer=1",
                 "attn_pair=1", "attn_pair=2", "sum_ring=1", "sum_ring=2"):
        assert B.tp_set_test_overrides(good) == 0, good
    for bad in ("gemm_tile=100x100", "gemm_tile=256x256w8", "qkv_split=9", "attn_sets=3",
                "sum_unroll=3", "nope=1", "qkv_split", "qkv_split=2,", "sum_grid=-1",
                "sum_defer=2", "attn_pair=0", "attn_pair=3", "sum_ring=0", "sum_ring=3"):
        assert B.tp_set_test_overrides(bad) == 2, bad
    B.tp_set_test_overrides(None)
    # a rejected spec leaves the previous setting in place
    assert B.tp_set_test_overrides("gemm_tile=128x128") == 0
    assert B.tp_set_test_overrides("gemm_tile=1x1") == 2
    assert B.tp_gemm_tile_info(4096, 8192, 4096)[1:] == (128, 128, 8)
    B.tp_set_test_overrides(None)
    assert B.tp_gemm_tile_info(4096, 8192, 4096)[1:] == (256, 256, 4)


def test_workspace_sizes():
    # MLP: Y_i [tokens, ffn/N] of the element type, rounded up to 256 bytes
    assert B.tp_mlp_workspace_bytes(32, 1024, 4096, 2, F32) == 32 * 2048 * 4
    assert B.tp_mlp_workspace_bytes(8192, 3072, 12288, 8, BF16) == 8192 * 1536 * 2
    assert B.tp_mlp_workspace_bytes(3, 8, 16, 2, BF16) == 256
    assert B.tp_mlp_workspace_bytes(32, 1024, 4096, 3, F32) == 0
    # SwiGLU: the gated activation A_i [tokens, ffn/N] bf16
    assert B.tp_swiglu_workspace_bytes(4096, 8192, 28672, 8, BF16) == 4096 * 3584 * 2
    assert B.tp_swiglu_workspace_bytes(4096, 8192, 28672, 8, F32) == 0
    # attention: Q, K, V^T (seq padded to 8), O, each 256-byte aligned
    st, off = B.tp_attn_workspace_layout(4, 2048, 4096, 32, 8, BF16)
    assert st == 0
    e = 4 * 4 * 2048 * 128 * 2
    assert off == dict(q=0, k=e, vt=2 * e, o=3 * e)
    # 16 x 16 = 256 query tiles (< 2 per compute unit): two key-range halves per tile keep
    # fp32 partials after O: outputs [512][128][128], then (max, denominator) [512][128][2]
    part_o, part_ml = 512 * 128 * 128 * 4, 512 * 128 * 2 * 4
    assert B.tp_attn_workspace_bytes(4, 2048, 4096, 32, 8, BF16) == 4 * e + part_o + part_ml
    # 8 sequences x 16 heads x 16 tiles = 2048 query tiles: no split, no partials
    e8 = 8 * 16 * 2048 * 128 * 2
    assert B.tp_attn_workspace_bytes(8, 2048, 8192, 64, 4, BF16) == 4 * e8
    st, off = B.tp_attn_workspace_layout(1, 5, 256, 2, 1, BF16)
    # 2 heads of d = 128, seq 5: Q and K are 2560 bytes; V^T rows are padded to 8 keys
    assert st == 0 and off == dict(q=0, k=2560, vt=5120, o=5120 + 2 * 128 * 8 * 2)
    assert B.tp_attn_workspace_bytes(1, 5, 256, 2, 1, F32) == 0


def test_gemm_tile_info(overrides):
    overrides(None)
    st, bm, bn, w = B.tp_gemm_tile_info(4096, 4096, 8192)
    assert st == 0 and (bm, bn, w) == (256, 256, 8)      # one tile per CU: eight waves
    st, bm, bn, w = B.tp_gemm_tile_info(4096, 3072, 8192)
    assert st == 0 and (bm, bn) == (256, 192)
    # 256 x 256 with two or more tiles per CU and K >= 2048: four waves
    assert B.tp_gemm_tile_info(4096, 8192, 4096)[1:] == (256, 256, 4)
    assert B.tp_gemm_tile_info(8192, 8192, 8192)[1:] == (256, 256, 4)
    assert B.tp_gemm_tile_info(4096, 8192, 1024)[1:] == (256, 256, 8)   # short K
    # 256 x 192 tiles likewise: the MLP block's row GEMM at N = 1 and 2 (512 tiles)
    assert B.tp_gemm_tile_info(2048, 12288, 49152)[1:] == (256, 192, 4)
    assert B.tp_gemm_tile_info(2048, 12288, 24576)[1:] == (256, 192, 4)
    assert B.tp_gemm_tile_info(4096, 3072, 8192)[1:] == (256, 192, 8)    # 256 tiles
    # the override names the layout
    overrides("gemm_tile=256x256")
    assert B.tp_gemm_tile_info(4096, 8192, 4096)[1:] == (256, 256, 8)
    overrides("gemm_tile=128x128w4")
    assert B.tp_gemm_tile_info(4096, 8192, 4096)[1:] == (128, 128, 4)
    assert B.tp_gemm_tile_info(0, 1, 1)[0] == 2


def test_noalloc_mlp_validation():
    """The allocation-free MLP shard validates like tp_mlp_shard_fwd and refuses a Y_i larger
    than its 64 MiB device scratch (TP_ERR_WORKSPACE) before touching the device."""
    a = dict(X=P, A_i=P, a_i=P, B_i=P, Z_i=P, tokens=32, hidden=1024, ffn=4096, n_shards=2,
             rank=0, dt=F32)
    assert B.tp_mlp_shard_fwd_noalloc(**dict(a, X=None)) == 1
    assert B.tp_mlp_shard_fwd_noalloc(**dict(a, n_shards=3)) == 3
    assert B.tp_mlp_shard_fwd_noalloc(**dict(a, rank=2)) == 4
    assert B.tp_mlp_shard_fwd_noalloc(**dict(a, dt=7)) == 5
    assert B.tp_mlp_shard_fwd_noalloc(**dict(a, Z_i=P + 4)) == 6
    # 8192 x 4096 bf16 = 64 MiB exactly fits; one more token row does not
    big = dict(a, tokens=8192, hidden=1024, ffn=8192, dt=BF16)
    assert B.tp_mlp_shard_fwd_noalloc(**big) not in (1, 2, 3, 4, 5, 6, 7)
    assert B.tp_mlp_shard_fwd_noalloc(**dict(big, tokens=8193)) == 7
    assert "scratch" in B.tp_last_error()


def test_row_parallel_sum_tile_info():
    """The fused-sum launch the library reports: the ring form for the layer's output
    projection (16-slab K loop, 2048 tiles of 128 x 128), the deferred form for its MLP row
    GEMM (fp32 output, K = 4096), the in-epilogue form for a bf16 output with a long K loop,
    and none of the ring where the override turns it off. No kernel runs."""
    F32, BF16 = B.TP_F32, B.TP_BF16
    B.tp_set_test_overrides(None)
    assert B.tp_row_parallel_sum_tile_info(4096, 8192, 1024, 8, BF16) == (0, 128, 128, 8, 2)
    assert B.tp_row_parallel_sum_tile_info(4096, 8192, 1024, 8, F32) == (0, 128, 128, 8, 2)
    assert B.tp_row_parallel_sum_tile_info(4096, 8192, 4096, 8, F32) == (0, 256, 256, 8, 1)
    assert B.tp_row_parallel_sum_tile_info(4096, 8192, 4096, 8, BF16) == (0, 256, 256, 8, 0)
    # ragged rows, columns and K still divide into rounds of 256 workgroups
    assert B.tp_row_parallel_sum_tile_info(4000, 8184, 1000, 3, BF16)[1:] == (128, 128, 8, 2)
    # no partials to add, or tiles that do not fill whole rounds: no ring
    assert B.tp_row_parallel_sum_tile_info(4096, 8192, 1024, 1, BF16)[4] != 2
    assert B.tp_row_parallel_sum_tile_info(4096, 8000, 1024, 8, BF16)[4] != 2
    # a K loop other than 16 slabs: no ring
    assert B.tp_row_parallel_sum_tile_info(4096, 8192, 2048, 8, BF16)[4] != 2
    assert B.tp_row_parallel_sum_tile_info(4096, 8192, 960, 8, BF16)[4] != 2
    assert B.tp_set_test_overrides("sum_ring=1") == 0
    assert B.tp_row_parallel_sum_tile_info(4096, 8192, 1024, 8, BF16) == (0, 256, 256, 8, 0)
    assert B.tp_set_test_overrides("sum_defer=0") == 0
    assert B.tp_row_parallel_sum_tile_info(4096, 8192, 4096, 8, F32) == (0, 256, 256, 8, 0)
    B.tp_set_test_overrides(None)
    assert B.tp_row_parallel_sum_tile_info(4096, 8192, 1024, 9, BF16)[0] == 2   # TP_ERR_SHAPE
    assert B.tp_row_parallel_sum_tile_info(0, 8192, 1024, 8, BF16)[0] == 2
    assert B.tp_row_parallel_sum_tile_info(4096, 8192, 1024, 8, 7)[0] != 0


def test_mlp_fwd_save_and_bwd_saved_validation():
    """The forward that keeps P_i and the backward that takes it validate like
    tp_mlp_shard_fwd / tp_mlp_shard_bwd, bf16 only, and refuse a P_i that overlaps a buffer
    written during the call (TP_ERR_ALIAS), all before touching the device."""
    T, h, ffn, N = 4096, 8192, 32768, 8
    fl = ffn // N
    ws = 1 << 32                                   # fake workspace address, far from the rest
    need = B.tp_mlp_workspace_bytes(T, h, ffn, N, BF16)
    f = dict(X=P, A_i=P, a_i=None, B_i=P, Z_i=P, P_i=1 << 36, tokens=T, hidden=h, ffn=ffn,
             n_shards=N, rank=0, dt=BF16, workspace=ws, workspace_bytes=need)
    g = lambda **kw: B.tp_mlp_shard_fwd_save(**dict(f, **kw))
    assert g(P_i=None) == 1 and g(Z_i=None) == 1
    assert g(dt=F32) == 5                          # bf16 only
    assert g(n_shards=3) == 3 and g(rank=8) == 4
    assert g(P_i=(1 << 36) + 8) == 6
    assert g(workspace_bytes=need - 256) == 7
    assert g(P_i=ws + need - 256) == 10            # P_i runs into Y_i
    assert g(P_i=ws - T * fl * 2 + 16) == 10       # ... from below
    assert g(Z_i=(1 << 36) + 4096) == 10           # Z_i inside P_i
    assert g(X=(1 << 36) + 4096) == 10             # ... or an input
    assert g(a_i=(1 << 36) + T * fl * 2 - 16) == 10
    # adjacent is fine: validation passes and the call reaches the device check (no GPU here)
    assert g(P_i=ws + need) not in (1, 2, 3, 4, 5, 6, 7, 10)
    assert "overlap" not in B.tp_last_error()
    wsb = B.tp_mlp_bwd_workspace_bytes(T, h, ffn, N, BF16)
    b = dict(X=P, A_i=P, B_i=P, P_i=1 << 36, dZ=P, dX_i=P, dA_i=P, da_i=None, dB_i=P, tokens=T,
             hidden=h, ffn=ffn, n_shards=N, rank=0, dt=BF16, workspace=ws, workspace_bytes=wsb)
    k = lambda **kw: B.tp_mlp_shard_bwd_saved(**dict(b, **kw))
    assert k(P_i=None) == 1 and k(dZ=None) == 1
    assert k(dt=F32) == 5
    assert k(n_shards=3) == 3 and k(rank=-1) == 4
    assert k(P_i=(1 << 36) + 4) == 6
    assert k(workspace_bytes=wsb - 1) == 7
    assert k(tokens=(1 << 22) + 1) == 2
    assert k(P_i=ws + wsb - 16) == 10              # the workspace is written while P_i is read
    assert k(dX_i=(1 << 36) + 64) == 10            # ... and so are the gradients
    assert k(da_i=(1 << 36) + T * fl * 2 - 16) == 10
    assert k(P_i=ws + wsb) not in (1, 2, 3, 4, 5, 6, 7, 10)
