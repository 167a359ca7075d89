"""ctypes binding of libtpshard (include/tp_shard.h), with the same entry-point names.

Argument marshalling only: tensors are passed as device pointers (``data_ptr()``), streams
as their ``hipStream_t`` handle. Every step of the computation runs in the library's HIP
kernels; there is no host or PyTorch fallback. If the library has not been built, loading
it raises ``TPShardNotBuilt``.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libtpshard.so")

TP_F32 = 0
TP_BF16 = 1
TP_ERR_SHAPE = 2
TP_ACT_NONE = 0
TP_ACT_GELU = 1

STATUS_NAMES = {
    0: "TP_OK", 1: "TP_ERR_NULL", 2: "TP_ERR_SHAPE", 3: "TP_ERR_NOT_DIVISIBLE", 4: "TP_ERR_RANK",
    5: "TP_ERR_DTYPE", 6: "TP_ERR_ALIGN", 7: "TP_ERR_WORKSPACE", 8: "TP_ERR_HIP",
    9: "TP_ERR_DEVICE", 10: "TP_ERR_ALIAS",
}

# Every symbol include/tp_shard.h declares.
EXPORTED = (
    "tp_column_parallel_fwd", "tp_row_parallel_fwd", "tp_row_parallel_sum_fwd",
    "tp_mlp_workspace_bytes", "tp_mlp_shard_fwd", "tp_mlp_shard_fwd_save",
    "tp_mlp_shard_fwd_noalloc",
    "tp_mlp_bwd_workspace_bytes", "tp_mlp_shard_bwd", "tp_mlp_shard_bwd_saved",
    "tp_swiglu_workspace_bytes", "tp_swiglu_shard_fwd", "tp_reduce_scatter_partials",
    "tp_sp_residual_layernorm_fwd", "tp_all_gather_rows", "tp_gqa_attn_workspace_bytes",
    "tp_gqa_attn_workspace_layout", "tp_gqa_attn_shard_fwd", "tp_attn_workspace_bytes",
    "tp_attn_workspace_layout", "tp_attn_shard_fwd", "tp_qkv_projection_fwd",
    "tp_head_attention_fwd", "tp_sum_partials", "tp_gemm_tile_info",
    "tp_row_parallel_sum_tile_info",
    "tp_set_test_overrides", "tp_last_error", "tp_abi_version",
)


class TPShardNotBuilt(RuntimeError):
    pass


class TPError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, str(status)), message))
        self.status = status


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise TPShardNotBuilt(
            "libtpshard.so is not built (%s); run `python -m tensor_transformer_layers_amd.build`"
            % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    L.tp_abi_version.restype = _int
    L.tp_last_error.restype = ctypes.c_char_p
    L.tp_column_parallel_fwd.restype = _int
    L.tp_column_parallel_fwd.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int,
                                         _int, _vp]
    L.tp_row_parallel_fwd.restype = _int
    L.tp_row_parallel_fwd.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _vp]
    L.tp_row_parallel_sum_fwd.restype = _int
    L.tp_row_parallel_sum_fwd.argtypes = [_vp, _vp, ctypes.POINTER(_vp), _vp, _int, _i64, _i64,
                                          _i64, _int, _int, _int, _vp]
    L.tp_mlp_workspace_bytes.restype = _sz
    L.tp_mlp_workspace_bytes.argtypes = [_i64, _i64, _i64, _int, _int]
    L.tp_mlp_shard_fwd.restype = _int
    L.tp_mlp_shard_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int,
                                   _vp, _sz, _vp]
    L.tp_mlp_shard_fwd_save.restype = _int
    L.tp_mlp_shard_fwd_save.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int,
                                        _int, _int, _vp, _sz, _vp]
    L.tp_mlp_shard_fwd_noalloc.restype = _int
    L.tp_mlp_shard_fwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int,
                                           _int, _vp]
    L.tp_mlp_bwd_workspace_bytes.restype = _sz
    L.tp_mlp_bwd_workspace_bytes.argtypes = [_i64, _i64, _i64, _int, _int]
    L.tp_mlp_shard_bwd.restype = _int
    L.tp_mlp_shard_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
                                   _i64, _int, _int, _int, _vp, _sz, _vp]
    L.tp_mlp_shard_bwd_saved.restype = _int
    L.tp_mlp_shard_bwd_saved.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
                                         _i64, _int, _int, _int, _vp, _sz, _vp]
    L.tp_swiglu_workspace_bytes.restype = _sz
    L.tp_swiglu_workspace_bytes.argtypes = [_i64, _i64, _i64, _int, _int]
    L.tp_swiglu_shard_fwd.restype = _int
    L.tp_swiglu_shard_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int,
                                      _int, _vp, _sz, _vp]
    L.tp_reduce_scatter_partials.restype = _int
    L.tp_reduce_scatter_partials.argtypes = [ctypes.POINTER(_vp), _int, _i64, _i64, _i64, _int,
                                             _vp, _int, _vp]
    L.tp_sp_residual_layernorm_fwd.restype = _int
    L.tp_sp_residual_layernorm_fwd.argtypes = [ctypes.POINTER(_vp), _int, _vp, _vp, _vp,
                                               ctypes.c_float, _vp, _vp, _i64, _i64, _i64, _int,
                                               _int, _vp]
    L.tp_all_gather_rows.restype = _int
    L.tp_all_gather_rows.argtypes = [ctypes.POINTER(_vp), _int, _i64, _i64, _i64, _vp, _int, _vp]
    L.tp_gqa_attn_workspace_bytes.restype = _sz
    L.tp_gqa_attn_workspace_bytes.argtypes = [_i64, _i64, _i64, _int, _int, _int, _int]
    L.tp_gqa_attn_workspace_layout.restype = _int
    L.tp_gqa_attn_workspace_layout.argtypes = [_i64, _i64, _i64, _int, _int, _int, _int,
                                               ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                               ctypes.POINTER(_sz), ctypes.POINTER(_sz)]
    L.tp_gqa_attn_shard_fwd.restype = _int
    L.tp_gqa_attn_shard_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int,
                                        _int, _int, _int, _int, _vp, _sz, _vp]
    L.tp_attn_workspace_bytes.restype = _sz
    L.tp_attn_workspace_bytes.argtypes = [_i64, _i64, _i64, _int, _int, _int]
    L.tp_attn_workspace_layout.restype = _int
    L.tp_attn_workspace_layout.argtypes = [_i64, _i64, _i64, _int, _int, _int,
                                           ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                           ctypes.POINTER(_sz), ctypes.POINTER(_sz)]
    L.tp_attn_shard_fwd.restype = _int
    L.tp_attn_shard_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int,
                                    _int, _int, _vp, _sz, _vp]
    L.tp_qkv_projection_fwd.restype = _int
    L.tp_qkv_projection_fwd.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _int,
                                        _int, _vp, _sz, _vp]
    L.tp_head_attention_fwd.restype = _int
    L.tp_head_attention_fwd.argtypes = [_i64, _i64, _i64, _int, _int, _int, _int, _int, _int,
                                        _vp, _sz, _vp]
    L.tp_gemm_tile_info.restype = _int
    L.tp_gemm_tile_info.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_int), ctypes.POINTER(_int),
                                    ctypes.POINTER(_int)]
    L.tp_row_parallel_sum_tile_info.restype = _int
    L.tp_row_parallel_sum_tile_info.argtypes = [_i64, _i64, _i64, _int, _int] + \
        [ctypes.POINTER(_int)] * 4
    L.tp_sum_partials.restype = _int
    L.tp_sum_partials.argtypes = [ctypes.POINTER(_vp), _int, _i64, _vp, _int, _vp]
    L.tp_set_test_overrides.restype = _int
    L.tp_set_test_overrides.argtypes = [ctypes.c_char_p]
    _lib = L
    return L


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (or an int / None passed through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def tp_last_error() -> str:
    return lib().tp_last_error().decode()


def tp_abi_version() -> int:
    return lib().tp_abi_version()


def tp_column_parallel_fwd(X, W_i, b_i, Y_i, rows, in_features, out_features, n_shards, rank,
                           act, dt, stream=None) -> int:
    return lib().tp_column_parallel_fwd(_ptr(X), _ptr(W_i), _ptr(b_i), _ptr(Y_i), rows,
                                        in_features, out_features, n_shards, rank, act, dt,
                                        _stream(stream))


def tp_row_parallel_fwd(X_i, W_i, Z_i, rows, in_features, out_features, n_shards, rank, dt,
                        stream=None) -> int:
    return lib().tp_row_parallel_fwd(_ptr(X_i), _ptr(W_i), _ptr(Z_i), rows, in_features,
                                     out_features, n_shards, rank, dt, _stream(stream))


def tp_row_parallel_sum_fwd(X_i, W_i, Z_parts, Z, out_dt, rows, in_features, out_features,
                            n_shards, rank, dt, stream=None) -> int:
    return lib().tp_row_parallel_sum_fwd(_ptr(X_i), _ptr(W_i), _ptr_array(Z_parts), _ptr(Z),
                                         out_dt, rows, in_features, out_features, n_shards, rank,
                                         dt, _stream(stream))


def tp_mlp_workspace_bytes(tokens, hidden, ffn, n_shards, dt) -> int:
    return lib().tp_mlp_workspace_bytes(tokens, hidden, ffn, n_shards, dt)


def tp_mlp_shard_fwd(X, A_i, a_i, B_i, Z_i, tokens, hidden, ffn, n_shards, rank, dt,
                     workspace, workspace_bytes, stream=None) -> int:
    return lib().tp_mlp_shard_fwd(_ptr(X), _ptr(A_i), _ptr(a_i), _ptr(B_i), _ptr(Z_i), tokens,
                                  hidden, ffn, n_shards, rank, dt, _ptr(workspace),
                                  workspace_bytes, _stream(stream))


def tp_mlp_shard_fwd_save(X, A_i, a_i, B_i, Z_i, P_i, tokens, hidden, ffn, n_shards, rank, dt,
                          workspace, workspace_bytes, stream=None) -> int:
    return lib().tp_mlp_shard_fwd_save(_ptr(X), _ptr(A_i), _ptr(a_i), _ptr(B_i), _ptr(Z_i),
                                       _ptr(P_i), tokens, hidden, ffn, n_shards, rank, dt,
                                       _ptr(workspace), workspace_bytes, _stream(stream))


def tp_mlp_shard_fwd_noalloc(X, A_i, a_i, B_i, Z_i, tokens, hidden, ffn, n_shards, rank, dt,
                             stream=None) -> int:
    return lib().tp_mlp_shard_fwd_noalloc(_ptr(X), _ptr(A_i), _ptr(a_i), _ptr(B_i), _ptr(Z_i),
                                          tokens, hidden, ffn, n_shards, rank, dt,
                                          _stream(stream))


def tp_mlp_bwd_workspace_bytes(tokens, hidden, ffn, n_shards, dt) -> int:
    return lib().tp_mlp_bwd_workspace_bytes(tokens, hidden, ffn, n_shards, dt)


def tp_mlp_shard_bwd(X, A_i, a_i, B_i, dZ, dX_i, dA_i, da_i, dB_i, tokens, hidden, ffn,
                     n_shards, rank, dt, workspace, workspace_bytes, stream=None) -> int:
    return lib().tp_mlp_shard_bwd(_ptr(X), _ptr(A_i), _ptr(a_i), _ptr(B_i), _ptr(dZ), _ptr(dX_i),
                                  _ptr(dA_i), _ptr(da_i), _ptr(dB_i), tokens, hidden, ffn,
                                  n_shards, rank, dt, _ptr(workspace), workspace_bytes,
                                  _stream(stream))


def tp_mlp_shard_bwd_saved(X, A_i, B_i, P_i, dZ, dX_i, dA_i, da_i, dB_i, tokens, hidden, ffn,
                           n_shards, rank, dt, workspace, workspace_bytes, stream=None) -> int:
    return lib().tp_mlp_shard_bwd_saved(_ptr(X), _ptr(A_i), _ptr(B_i), _ptr(P_i), _ptr(dZ),
                                        _ptr(dX_i), _ptr(dA_i), _ptr(da_i), _ptr(dB_i), tokens,
                                        hidden, ffn, n_shards, rank, dt, _ptr(workspace),
                                        workspace_bytes, _stream(stream))


def tp_swiglu_workspace_bytes(tokens, hidden, ffn, n_shards, dt) -> int:
    return lib().tp_swiglu_workspace_bytes(tokens, hidden, ffn, n_shards, dt)


def tp_swiglu_shard_fwd(X, Wgate_i, Wup_i, Wdown_i, Z_i, tokens, hidden, ffn, n_shards, rank,
                        dt, workspace, workspace_bytes, stream=None) -> int:
    return lib().tp_swiglu_shard_fwd(_ptr(X), _ptr(Wgate_i), _ptr(Wup_i), _ptr(Wdown_i),
                                     _ptr(Z_i), tokens, hidden, ffn, n_shards, rank, dt,
                                     _ptr(workspace), workspace_bytes, _stream(stream))


def _ptr_array(items):
    arr = (_vp * max(1, len(items)))()
    for i, t in enumerate(items):
        arr[i] = _ptr(t)
    return arr


def tp_reduce_scatter_partials(Z_parts, n_parts, batch, seq, hidden, rank, H_r, out_dt,
                               stream=None) -> int:
    return lib().tp_reduce_scatter_partials(_ptr_array(Z_parts), n_parts, batch, seq, hidden,
                                            rank, _ptr(H_r), out_dt, _stream(stream))


def tp_sp_residual_layernorm_fwd(Z_parts, n_parts, residual_r, gamma, beta, eps, H_r, Y_r,
                                 batch, seq, hidden, rank, dt, stream=None) -> int:
    return lib().tp_sp_residual_layernorm_fwd(_ptr_array(Z_parts), n_parts, _ptr(residual_r),
                                              _ptr(gamma), _ptr(beta), eps, _ptr(H_r),
                                              _ptr(Y_r), batch, seq, hidden, rank, dt,
                                              _stream(stream))


def tp_all_gather_rows(slices, n_parts, batch, seq, hidden, X, dt, stream=None) -> int:
    return lib().tp_all_gather_rows(_ptr_array(slices), n_parts, batch, seq, hidden, _ptr(X),
                                    dt, _stream(stream))


def tp_gqa_attn_workspace_bytes(batch, seq, hidden, n_heads, n_kv_heads, n_shards, dt) -> int:
    return lib().tp_gqa_attn_workspace_bytes(batch, seq, hidden, n_heads, n_kv_heads, n_shards, dt)


def tp_gqa_attn_workspace_layout(batch, seq, hidden, n_heads, n_kv_heads, n_shards, dt):
    """(status, {"q": off, "k": off, "vt": off, "o": off}) byte offsets in the workspace."""
    offs = [_sz(0) for _ in range(4)]
    st = lib().tp_gqa_attn_workspace_layout(batch, seq, hidden, n_heads, n_kv_heads, n_shards,
                                            dt, *[ctypes.byref(o) for o in offs])
    return st, dict(zip(("q", "k", "vt", "o"), (o.value for o in offs)))


def tp_gqa_attn_shard_fwd(X, Wqkv_i, bqkv_i, Wo_i, Z_i, batch, seq, hidden, n_heads,
                          n_kv_heads, causal, n_shards, rank, dt, workspace, workspace_bytes,
                          stream=None) -> int:
    return lib().tp_gqa_attn_shard_fwd(_ptr(X), _ptr(Wqkv_i), _ptr(bqkv_i), _ptr(Wo_i),
                                       _ptr(Z_i), batch, seq, hidden, n_heads, n_kv_heads,
                                       int(causal), n_shards, rank, dt, _ptr(workspace),
                                       workspace_bytes, _stream(stream))


def tp_attn_workspace_bytes(batch, seq, hidden, n_heads, n_shards, dt) -> int:
    return lib().tp_attn_workspace_bytes(batch, seq, hidden, n_heads, n_shards, dt)


def tp_attn_workspace_layout(batch, seq, hidden, n_heads, n_shards, dt):
    """(status, {"q": off, "k": off, "vt": off, "o": off}) byte offsets in the workspace."""
    offs = [_sz(0) for _ in range(4)]
    st = lib().tp_attn_workspace_layout(batch, seq, hidden, n_heads, n_shards, dt,
                                        *[ctypes.byref(o) for o in offs])
    return st, dict(zip(("q", "k", "vt", "o"), (o.value for o in offs)))


def tp_attn_shard_fwd(X, Wqkv_i, bqkv_i, Wo_i, Z_i, batch, seq, hidden, n_heads, causal,
                      n_shards, rank, dt, workspace, workspace_bytes, stream=None) -> int:
    return lib().tp_attn_shard_fwd(_ptr(X), _ptr(Wqkv_i), _ptr(bqkv_i), _ptr(Wo_i), _ptr(Z_i),
                                   batch, seq, hidden, n_heads, int(causal), n_shards, rank, dt,
                                   _ptr(workspace), workspace_bytes, _stream(stream))


def tp_qkv_projection_fwd(X, Wqkv_i, bqkv_i, batch, seq, hidden, n_heads, n_kv_heads, n_shards,
                          rank, dt, workspace, workspace_bytes, stream=None) -> int:
    return lib().tp_qkv_projection_fwd(_ptr(X), _ptr(Wqkv_i), _ptr(bqkv_i), batch, seq, hidden,
                                       n_heads, n_kv_heads, n_shards, rank, dt, _ptr(workspace),
                                       workspace_bytes, _stream(stream))


def tp_head_attention_fwd(batch, seq, hidden, n_heads, n_kv_heads, causal, n_shards, rank, dt,
                          workspace, workspace_bytes, stream=None) -> int:
    return lib().tp_head_attention_fwd(batch, seq, hidden, n_heads, n_kv_heads, int(causal),
                                       n_shards, rank, dt, _ptr(workspace), workspace_bytes,
                                       _stream(stream))


def tp_sum_partials(Z_parts: Sequence, n_parts, numel, Z, out_dt, stream=None) -> int:
    arr = (_vp * max(1, len(Z_parts)))(*[_ptr(z) for z in Z_parts])
    return lib().tp_sum_partials(arr, n_parts, numel, _ptr(Z), out_dt, _stream(stream))


def tp_gemm_tile_info(M, N, K):
    """(status, tile_m, tile_n, waves) of the bf16 GEMM launched for this shape."""
    a, b, c = _int(0), _int(0), _int(0)
    st = lib().tp_gemm_tile_info(M, N, K, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    return st, a.value, b.value, c.value


def tp_row_parallel_sum_tile_info(rows, out_features, k_local, n_parts, out_dt):
    """(status, tile_m, tile_n, waves, form) of tp_row_parallel_sum_fwd's launch."""
    v = [_int(0) for _ in range(4)]
    st = lib().tp_row_parallel_sum_tile_info(rows, out_features, k_local, n_parts, out_dt,
                                             *[ctypes.byref(x) for x in v])
    return (st,) + tuple(x.value for x in v)


def tp_set_test_overrides(spec: Optional[str]) -> int:
    return lib().tp_set_test_overrides(None if spec is None else spec.encode())


@contextlib.contextmanager
def forced_launch(spec: Optional[str]):
    """Launch choices forced by ``tp_set_test_overrides(spec)`` inside the block, the library's
    own choices again after it."""
    check(tp_set_test_overrides(spec))
    try:
        yield
    finally:
        tp_set_test_overrides(None)


def check(status: int) -> None:
    if status != 0:
        raise TPError(status, tp_last_error())
