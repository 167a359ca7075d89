"""PyTorch-facing calls of one tensor-parallel rank's shard.

PyTorch supplies device memory and streams only: these functions allocate outputs and
workspaces with torch and pass pointers to the C ABI (``binding``). Every arithmetic step
runs in libtpshard's HIP kernels.

* ``mlp_shard``       Z_i = GeLU(X A_i + a_i) B_i            (tp_mlp_shard_fwd)
* ``attn_shard``      Z_i = concat_j Head_j  W_O,i            (tp_attn_shard_fwd)
* ``sum_partials``    Z = sum_r Z_r, the all-reduce stand-in  (tp_sum_partials)
* ``column_parallel`` / ``row_parallel``  the two linear primitives on their own
* ``LayerShard``      one rank's layer: attention partial, sum over the N partials,
                      MLP partial on that sum, sum again -- one sum per block, as the
                      pages count one all-reduce per block in the forward pass.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Optional, Sequence

import torch

from . import binding as B

_DT = {torch.float32: B.TP_F32, torch.bfloat16: B.TP_BF16}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError("unsupported dtype %s" % t.dtype)
    return _DT[t.dtype]


def _require_cuda(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors are on different devices (%s and %s)" % (dev, t.device))


def _need(name: str, t: Optional[torch.Tensor], shape, dtype, optional: bool = False) -> None:
    """Exact shape and dtype of one argument (checked before any ABI call: a mismatched
    tensor would otherwise become an out-of-bounds access in a kernel)."""
    if t is None:
        if optional:
            return
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a tensor" % name)
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))


def _need_2d(name: str, t: torch.Tensor, dtype=None):
    """A 2-D tensor (of ``dtype`` if given); returns its shape."""
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError("%s must be a 2-D tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    return tuple(t.shape)


def _need_workspace(ws: torch.Tensor, nbytes: int) -> int:
    """A workspace of at least ``nbytes``; returns its size in bytes."""
    if not isinstance(ws, torch.Tensor):
        raise ValueError("workspace must be a tensor")
    have = ws.numel() * ws.element_size()
    if have < nbytes:
        raise ValueError("workspace holds %d bytes, %d needed" % (have, nbytes))
    return have


def _stream(stream):
    return torch.cuda.current_stream() if stream is None else stream


# ---- column / row-parallel linear layers ----------------------------------------------------
def column_parallel(X: torch.Tensor, W_i: torch.Tensor, b_i: Optional[torch.Tensor],
                    n_shards: int, rank: int, gelu: bool = False, Y: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Y_i = act(X W_i + b_i), W_i [out/N, in] (tp_column_parallel_fwd)."""
    _need_2d("X", X)
    rows, k = X.shape
    dt = X.dtype
    _dt(X)
    width = _need_2d("W_i", W_i)[0]
    _need("W_i", W_i, (width, k), dt)
    _need("b_i", b_i, (width,), dt, optional=True)
    if Y is None:
        Y = torch.empty(rows, width, dtype=X.dtype, device=X.device)
    _need("Y", Y, (rows, width), dt)
    _require_cuda(X, W_i, b_i, Y)
    st = B.tp_column_parallel_fwd(X, W_i, b_i, Y, rows, k, width * n_shards, n_shards, rank,
                                  B.TP_ACT_GELU if gelu else B.TP_ACT_NONE, _dt(X),
                                  _stream(stream))
    B.check(st)
    return Y


def row_parallel(X_i: torch.Tensor, W_i: torch.Tensor, n_shards: int, rank: int,
                 Z: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Z_i = X_i W_i (fp32 partial), W_i [out, in/N] (tp_row_parallel_fwd)."""
    _need_2d("X_i", X_i)
    rows, k = X_i.shape
    _dt(X_i)
    width = _need_2d("W_i", W_i)[0]
    _need("W_i", W_i, (width, k), X_i.dtype)
    if Z is None:
        Z = torch.empty(rows, width, dtype=torch.float32, device=X_i.device)
    _need("Z", Z, (rows, width), torch.float32)
    _require_cuda(X_i, W_i, Z)
    st = B.tp_row_parallel_fwd(X_i, W_i, Z, rows, k * n_shards, width, n_shards, rank, _dt(X_i),
                               _stream(stream))
    B.check(st)
    return Z


def row_parallel_sum(X_i: torch.Tensor, W_i: torch.Tensor,
                     partials: Sequence[Optional[torch.Tensor]], n_shards: int, rank: int,
                     out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """Z = sum over the N ranks of the row-parallel partials, this rank's X_i W_i computed and
    added in the same kernel (tp_row_parallel_sum_fwd). ``partials`` holds N entries: the
    other ranks' fp32 partials [rows, out], and None (or anything: it is not read) at
    ``rank``. The same bits as row_parallel followed by sum_partials."""
    _need_2d("X_i", X_i, torch.bfloat16)
    rows, k = X_i.shape
    width = _need_2d("W_i", W_i)[0]
    _need("W_i", W_i, (width, k), torch.bfloat16)
    if len(partials) != n_shards:
        raise ValueError("%d partials given for %d shards" % (len(partials), n_shards))
    peers = [None if q == rank else partials[q] for q in range(n_shards)]
    for q, t in enumerate(peers):
        _need("partial %d" % q, t, (rows, width), torch.float32, optional=q == rank)
    if out is None:
        out = torch.empty(rows, width, dtype=out_dtype, device=X_i.device)
    if out.dtype not in _DT:
        raise ValueError("out has dtype %s, expected float32 or bfloat16" % out.dtype)
    _need("out", out, (rows, width), out.dtype)
    _require_cuda(X_i, W_i, out, *[t for t in peers if t is not None])
    st = B.tp_row_parallel_sum_fwd(X_i, W_i, peers, out, _DT[out.dtype], rows, k * n_shards,
                                   width, n_shards, rank, B.TP_BF16, _stream(stream))
    B.check(st)
    return out


# ---- MLP ------------------------------------------------------------------------------------
def mlp_workspace(tokens: int, hidden: int, ffn: int, n_shards: int, dtype, device="cuda"):
    nbytes = B.tp_mlp_workspace_bytes(tokens, hidden, ffn, n_shards, _DT[dtype])
    if nbytes == 0:
        raise B.TPError(B.TP_ERR_SHAPE, B.tp_last_error())
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def mlp_hidden_view(workspace: torch.Tensor, tokens: int, ffn_local: int, dtype) -> torch.Tensor:
    """Y_i = GeLU(X A_i + a_i), [tokens, ffn/N], stored at offset 0 of the MLP workspace."""
    esz = torch.tensor([], dtype=dtype).element_size()
    return workspace[: tokens * ffn_local * esz].view(dtype).view(tokens, ffn_local)


def mlp_shard(X: torch.Tensor, A_i: torch.Tensor, a_i: Optional[torch.Tensor], B_i: torch.Tensor,
              n_shards: int, rank: int, Z: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, stream=None):
    """Rank ``rank``'s MLP partial. A_i [F/N, h], B_i [h, F/N] (see include/tp_shard.h).

    Returns (Z_i fp32 [tokens, hidden], workspace).
    """
    _need_2d("X", X)
    tokens, hidden = X.shape
    dt = _dt(X)
    fl = _need_2d("A_i", A_i)[0]
    ffn = fl * n_shards
    _need("A_i", A_i, (fl, hidden), X.dtype)
    _need("a_i", a_i, (fl,), X.dtype, optional=True)
    _need("B_i", B_i, (hidden, fl), X.dtype)
    if Z is None:
        Z = torch.empty(tokens, hidden, dtype=torch.float32, device=X.device)
    _need("Z", Z, (tokens, hidden), torch.float32)
    if workspace is None:
        workspace = mlp_workspace(tokens, hidden, ffn, n_shards, X.dtype, X.device)
    wsb = _need_workspace(workspace, B.tp_mlp_workspace_bytes(tokens, hidden, ffn, n_shards, dt))
    _require_cuda(X, A_i, a_i, B_i, Z, workspace)
    st = B.tp_mlp_shard_fwd(X, A_i, a_i, B_i, Z, tokens, hidden, ffn, n_shards, rank, dt,
                            workspace, wsb, _stream(stream))
    B.check(st)
    return Z, workspace


def mlp_shard_save(X: torch.Tensor, A_i: torch.Tensor, a_i: Optional[torch.Tensor],
                   B_i: torch.Tensor, n_shards: int, rank: int, Z: Optional[torch.Tensor] = None,
                   P: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   stream=None):
    """Rank ``rank``'s MLP partial (bf16), keeping the pre-activation P_i = X A_r + a_r for
    ``mlp_shard_backward(..., P=P_i)``. Returns (Z_i fp32 [tokens, hidden], P_i bf16
    [tokens, F/N], workspace)."""
    _need_2d("X", X, torch.bfloat16)
    tokens, hidden = X.shape
    fl = _need_2d("A_i", A_i)[0]
    ffn = fl * n_shards
    bf = torch.bfloat16
    _need("A_i", A_i, (fl, hidden), bf)
    _need("a_i", a_i, (fl,), bf, optional=True)
    _need("B_i", B_i, (hidden, fl), bf)
    if Z is None:
        Z = torch.empty(tokens, hidden, dtype=torch.float32, device=X.device)
    if P is None:
        P = torch.empty(tokens, fl, dtype=bf, device=X.device)
    _need("Z", Z, (tokens, hidden), torch.float32)
    _need("P", P, (tokens, fl), bf)
    if workspace is None:
        workspace = mlp_workspace(tokens, hidden, ffn, n_shards, X.dtype, X.device)
    wsb = _need_workspace(workspace, B.tp_mlp_workspace_bytes(tokens, hidden, ffn, n_shards,
                                                              B.TP_BF16))
    _require_cuda(X, A_i, a_i, B_i, Z, P, workspace)
    st = B.tp_mlp_shard_fwd_save(X, A_i, a_i, B_i, Z, P, tokens, hidden, ffn, n_shards, rank,
                                 B.TP_BF16, workspace, wsb, _stream(stream))
    B.check(st)
    return Z, P, workspace


def mlp_bwd_workspace(tokens: int, hidden: int, ffn: int, n_shards: int, device="cuda"):
    nbytes = B.tp_mlp_bwd_workspace_bytes(tokens, hidden, ffn, n_shards, B.TP_BF16)
    if nbytes == 0:
        raise B.TPError(B.TP_ERR_SHAPE, "invalid MLP backward sizes")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def mlp_shard_backward(X: torch.Tensor, A_i: torch.Tensor, a_i: Optional[torch.Tensor],
                       B_i: torch.Tensor, dZ: torch.Tensor, n_shards: int, rank: int,
                       out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None, P: Optional[torch.Tensor] = None):
    """Gradients of rank ``rank``'s MLP partial for the upstream dZ (bf16).

    Returns ({"dX": [T, h], "dA": [F/N, h], "da": [F/N], "dB": [h, F/N]} fp32, in the stored
    layouts of X, A_i, a_i, B_i; workspace). dX is the rank's input-gradient partial. With P
    (the pre-activation ``mlp_shard_save`` kept) the call takes it instead of recomputing it;
    a_i then only decides whether da is computed."""
    _need_2d("X", X, torch.bfloat16)
    tokens, hidden = X.shape
    fl = _need_2d("A_i", A_i)[0]
    ffn = fl * n_shards
    bf = torch.bfloat16
    _need("A_i", A_i, (fl, hidden), bf)
    _need("a_i", a_i, (fl,), bf, optional=True)
    _need("B_i", B_i, (hidden, fl), bf)
    _need("dZ", dZ, (tokens, hidden), bf)
    _need("P", P, (tokens, fl), bf, optional=True)
    f32 = dict(dtype=torch.float32, device=X.device)
    if out is None:
        out = {"dX": torch.empty(tokens, hidden, **f32), "dA": torch.empty(fl, hidden, **f32),
               "da": torch.empty(fl, **f32) if a_i is not None else None,
               "dB": torch.empty(hidden, fl, **f32)}
    _need("dX", out.get("dX"), (tokens, hidden), torch.float32)
    _need("dA", out.get("dA"), (fl, hidden), torch.float32)
    _need("da", out.get("da"), (fl,), torch.float32, optional=True)
    _need("dB", out.get("dB"), (hidden, fl), torch.float32)
    if workspace is None:
        workspace = mlp_bwd_workspace(tokens, hidden, ffn, n_shards, X.device)
    wsb = _need_workspace(workspace, B.tp_mlp_bwd_workspace_bytes(tokens, hidden, ffn, n_shards,
                                                                  B.TP_BF16))
    _require_cuda(X, A_i, a_i, B_i, dZ, P, out["dX"], out["dA"], out.get("da"), out["dB"],
                  workspace)
    if P is None:
        st = B.tp_mlp_shard_bwd(X, A_i, a_i, B_i, dZ, out["dX"], out["dA"], out.get("da"),
                                out["dB"], tokens, hidden, ffn, n_shards, rank, _dt(X), workspace,
                                wsb, _stream(stream))
    else:
        st = B.tp_mlp_shard_bwd_saved(X, A_i, B_i, P, dZ, out["dX"], out["dA"], out.get("da"),
                                      out["dB"], tokens, hidden, ffn, n_shards, rank, _dt(X),
                                      workspace, wsb, _stream(stream))
    B.check(st)
    return out, workspace


# ---- gated (SwiGLU) MLP ----------------------------------------------------------------------
def swiglu_workspace(tokens: int, hidden: int, ffn: int, n_shards: int, device="cuda"):
    nbytes = B.tp_swiglu_workspace_bytes(tokens, hidden, ffn, n_shards, B.TP_BF16)
    if nbytes == 0:
        raise B.TPError(B.TP_ERR_SHAPE, "invalid SwiGLU shard sizes")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def swiglu_shard(X: torch.Tensor, Wg_i: torch.Tensor, Wu_i: torch.Tensor, Wd_i: torch.Tensor,
                 n_shards: int, rank: int, Z: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None):
    """Rank ``rank``'s gated MLP partial (SiLU(X Wg_i^T) * (X Wu_i^T)) Wd_i^T.

    Wg_i, Wu_i [F/N, h], Wd_i [h, F/N], bf16 (see include/tp_shard.h). Returns (Z_i fp32
    [tokens, hidden], workspace); the gated activation A_i [tokens, F/N] bf16 sits at offset
    0 of the workspace (``mlp_hidden_view``).
    """
    _need_2d("X", X, torch.bfloat16)
    tokens, hidden = X.shape
    fl = _need_2d("Wg_i", Wg_i)[0]
    ffn = fl * n_shards
    _need("Wg_i", Wg_i, (fl, hidden), torch.bfloat16)
    _need("Wu_i", Wu_i, (fl, hidden), torch.bfloat16)
    _need("Wd_i", Wd_i, (hidden, fl), torch.bfloat16)
    if Z is None:
        Z = torch.empty(tokens, hidden, dtype=torch.float32, device=X.device)
    _need("Z", Z, (tokens, hidden), torch.float32)
    if workspace is None:
        workspace = swiglu_workspace(tokens, hidden, ffn, n_shards, X.device)
    wsb = _need_workspace(workspace, B.tp_swiglu_workspace_bytes(tokens, hidden, ffn, n_shards,
                                                                 B.TP_BF16))
    _require_cuda(X, Wg_i, Wu_i, Wd_i, Z, workspace)
    st = B.tp_swiglu_shard_fwd(X, Wg_i, Wu_i, Wd_i, Z, tokens, hidden, ffn, n_shards, rank,
                               _dt(X), workspace, wsb, _stream(stream))
    B.check(st)
    return Z, workspace


# ---- attention ---------------------------------------------------------------------------
def attn_workspace(batch: int, seq: int, hidden: int, n_heads: int, n_shards: int, device="cuda"):
    nbytes = B.tp_attn_workspace_bytes(batch, seq, hidden, n_heads, n_shards, B.TP_BF16)
    if nbytes == 0:
        st, _ = B.tp_attn_workspace_layout(batch, seq, hidden, n_heads, n_shards, B.TP_BF16)
        B.check(st)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def attn_views(workspace: torch.Tensor, batch: int, seq: int, hidden: int, n_heads: int,
               n_shards: int) -> Dict[str, torch.Tensor]:
    """Views of the attention workspace: q, k [b, Hl, s, d], vt [b, Hl, d, ld_vt], o [b*s, Hl*d].
    q holds the projected queries times log2(e) / sqrt(d) (the softmax's scale, folded in)."""
    st, off = B.tp_attn_workspace_layout(batch, seq, hidden, n_heads, n_shards, B.TP_BF16)
    B.check(st)
    hl = n_heads // n_shards
    d = hidden // n_heads
    ld_vt = (seq + 7) // 8 * 8

    def view(o, shape):
        n = 1
        for s in shape:
            n *= s
        return workspace[o:o + 2 * n].view(torch.bfloat16).view(*shape)

    return dict(q=view(off["q"], (batch, hl, seq, d)), k=view(off["k"], (batch, hl, seq, d)),
                vt=view(off["vt"], (batch, hl, d, ld_vt)), o=view(off["o"], (batch * seq, hl * d)))


def attn_shard(X: torch.Tensor, Wqkv_i: torch.Tensor, bqkv_i: Optional[torch.Tensor],
               Wo_i: torch.Tensor, batch: int, seq: int, n_heads: int, n_shards: int, rank: int,
               causal: bool = True, Z: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, stream=None):
    """Rank ``rank``'s attention partial. Returns (Z_i fp32 [batch*seq, hidden], workspace)."""
    return gqa_attn_shard(X, Wqkv_i, bqkv_i, Wo_i, batch, seq, n_heads, n_heads, n_shards, rank,
                          causal, Z=Z, workspace=workspace, stream=stream)
    B.check(st)
    return Z, workspace


def gqa_attn_workspace(batch: int, seq: int, hidden: int, n_heads: int, n_kv_heads: int,
                       n_shards: int, device="cuda"):
    nbytes = B.tp_gqa_attn_workspace_bytes(batch, seq, hidden, n_heads, n_kv_heads, n_shards,
                                           B.TP_BF16)
    if nbytes == 0:
        st, _ = B.tp_gqa_attn_workspace_layout(batch, seq, hidden, n_heads, n_kv_heads, n_shards,
                                               B.TP_BF16)
        B.check(st)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def gqa_attn_shard(X: torch.Tensor, Wqkv_i: torch.Tensor, bqkv_i: Optional[torch.Tensor],
                   Wo_i: torch.Tensor, batch: int, seq: int, n_heads: int, n_kv_heads: int,
                   n_shards: int, rank: int, causal: bool = True, Z: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    """Rank ``rank``'s grouped-query attention partial (see include/tp_shard.h).

    Returns (Z_i fp32 [batch*seq, hidden], workspace)."""
    hidden = _need_2d("X", X, torch.bfloat16)[1]
    _need("X", X, (batch * seq, hidden), torch.bfloat16)
    if n_heads < 1 or n_shards < 1 or n_kv_heads < 1 or hidden % n_heads or n_heads % n_shards:
        raise ValueError("hidden %d, %d heads, %d key/value heads and %d shards do not split "
                         "evenly" % (hidden, n_heads, n_kv_heads, n_shards))
    d = hidden // n_heads
    hl = n_heads // n_shards
    kvl = n_kv_heads // n_shards if n_kv_heads % n_shards == 0 else 1
    width = (hl + 2 * kvl) * d
    _need("Wqkv_i", Wqkv_i, (width, hidden), torch.bfloat16)
    _need("bqkv_i", bqkv_i, (width,), torch.bfloat16, optional=True)
    _need("Wo_i", Wo_i, (hidden, hl * d), torch.bfloat16)
    if Z is None:
        Z = torch.empty(batch * seq, hidden, dtype=torch.float32, device=X.device)
    _need("Z", Z, (batch * seq, hidden), torch.float32)
    if workspace is None:
        workspace = gqa_attn_workspace(batch, seq, hidden, n_heads, n_kv_heads, n_shards, X.device)
    wsb = _need_workspace(workspace, B.tp_gqa_attn_workspace_bytes(
        batch, seq, hidden, n_heads, n_kv_heads, n_shards, B.TP_BF16))
    _require_cuda(X, Wqkv_i, bqkv_i, Wo_i, Z, workspace)
    st = B.tp_gqa_attn_shard_fwd(X, Wqkv_i, bqkv_i, Wo_i, Z, batch, seq, hidden, n_heads,
                                 n_kv_heads, causal, n_shards, rank, _dt(X), workspace,
                                 wsb, _stream(stream))
    B.check(st)
    return Z, workspace


def qkv_projection(X: torch.Tensor, Wqkv_i: torch.Tensor, bqkv_i: Optional[torch.Tensor],
                   batch: int, seq: int, n_heads: int, n_kv_heads: int, n_shards: int, rank: int,
                   workspace: torch.Tensor, stream=None) -> torch.Tensor:
    """Step 1 of the attention shard alone: Q, K, V^T of the local heads into ``workspace``
    (tp_qkv_projection_fwd)."""
    hidden = _need_2d("X", X, torch.bfloat16)[1]
    _need("X", X, (batch * seq, hidden), torch.bfloat16)
    if n_heads < 1 or n_shards < 1 or n_kv_heads < 1 or hidden % n_heads or n_heads % n_shards:
        raise ValueError("hidden %d, %d heads, %d key/value heads and %d shards do not split "
                         "evenly" % (hidden, n_heads, n_kv_heads, n_shards))
    d = hidden // n_heads
    hl = n_heads // n_shards
    kvl = n_kv_heads // n_shards if n_kv_heads % n_shards == 0 else 1
    _need("Wqkv_i", Wqkv_i, ((hl + 2 * kvl) * d, hidden), torch.bfloat16)
    _need("bqkv_i", bqkv_i, ((hl + 2 * kvl) * d,), torch.bfloat16, optional=True)
    wsb = _need_workspace(workspace, B.tp_gqa_attn_workspace_bytes(
        batch, seq, hidden, n_heads, n_kv_heads, n_shards, B.TP_BF16))
    _require_cuda(X, Wqkv_i, bqkv_i, workspace)
    B.check(B.tp_qkv_projection_fwd(X, Wqkv_i, bqkv_i, batch, seq, hidden, n_heads, n_kv_heads,
                                    n_shards, rank, B.TP_BF16, workspace, wsb, _stream(stream)))
    return workspace


def head_attention(batch: int, seq: int, hidden: int, n_heads: int, n_kv_heads: int,
                   n_shards: int, rank: int, causal: bool, workspace: torch.Tensor,
                   stream=None) -> torch.Tensor:
    """Step 2 of the attention shard alone: every local head's attention from the workspace's
    Q, K, V^T into its O (tp_head_attention_fwd)."""
    wsb = _need_workspace(workspace, B.tp_gqa_attn_workspace_bytes(
        batch, seq, hidden, n_heads, n_kv_heads, n_shards, B.TP_BF16))
    _require_cuda(workspace)
    B.check(B.tp_head_attention_fwd(batch, seq, hidden, n_heads, n_kv_heads, causal, n_shards,
                                    rank, B.TP_BF16, workspace, wsb, _stream(stream)))
    return workspace


# ---- partial sum ------------------------------------------------------------------------------
def _need_parts(parts: Sequence[torch.Tensor]):
    if len(parts) < 1:
        raise ValueError("at least one partial is needed")
    shape = tuple(parts[0].shape)
    for q, t in enumerate(parts):
        _need("partial %d" % q, t, shape, torch.float32)
    return shape


def sum_partials(parts: Sequence[torch.Tensor], out_dtype=torch.float32,
                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    shape = _need_parts(parts)
    numel = parts[0].numel()
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=parts[0].device)
    if out.dtype not in _DT:
        raise ValueError("out has dtype %s, expected float32 or bfloat16" % out.dtype)
    _need("out", out, shape, out.dtype)
    _require_cuda(*parts, out)
    st = B.tp_sum_partials(list(parts), len(parts), numel, out, _DT[out.dtype], _stream(stream))
    B.check(st)
    return out


# ---- sequence parallelism ----------------------------------------------------------------------
def reduce_scatter(parts: Sequence[torch.Tensor], batch: int, seq: int, rank: int,
                   out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """Rank ``rank``'s slice [batch*seq/N, hidden] of sum(parts) (N = len(parts))."""
    N = len(parts)
    _need_parts(parts)
    hidden = parts[0].shape[-1]
    _need("partial 0", parts[0], (batch * seq, hidden), torch.float32)
    if out is None:
        out = torch.empty(batch * (seq // N), hidden, dtype=out_dtype, device=parts[0].device)
    if out.dtype not in _DT:
        raise ValueError("out has dtype %s, expected float32 or bfloat16" % out.dtype)
    _need("out", out, (batch * (seq // N), hidden), out.dtype)
    _require_cuda(*parts, out)
    st = B.tp_reduce_scatter_partials(list(parts), N, batch, seq, hidden, rank, out,
                                      _DT[out.dtype], _stream(stream))
    B.check(st)
    return out


def sp_residual_layernorm(parts: Sequence[torch.Tensor], residual: Optional[torch.Tensor],
                          gamma: torch.Tensor, beta: torch.Tensor, batch: int, seq: int,
                          rank: int, eps: float = 1e-5, dtype=torch.bfloat16,
                          H: Optional[torch.Tensor] = None, Y: Optional[torch.Tensor] = None,
                          stream=None):
    """(H_r, Y_r): the rank's slice of sum(parts) + residual, and its LayerNorm (fp32 gamma,
    beta), both [batch*seq/N, hidden] of ``dtype``."""
    N = len(parts)
    _need_parts(parts)
    hidden = parts[0].shape[-1]
    _need("partial 0", parts[0], (batch * seq, hidden), torch.float32)
    rows = batch * (seq // N)
    if dtype not in _DT:
        raise ValueError("dtype %s is not float32 or bfloat16" % dtype)
    _need("residual", residual, (rows, hidden), dtype, optional=True)
    _need("gamma", gamma, (hidden,), torch.float32)
    _need("beta", beta, (hidden,), torch.float32)
    if H is None:
        H = torch.empty(rows, hidden, dtype=dtype, device=parts[0].device)
    if Y is None:
        Y = torch.empty(rows, hidden, dtype=dtype, device=parts[0].device)
    _need("H", H, (rows, hidden), dtype)
    _need("Y", Y, (rows, hidden), dtype)
    _require_cuda(*parts, residual, gamma, beta, H, Y)
    st = B.tp_sp_residual_layernorm_fwd(list(parts), N, residual, gamma, beta, float(eps), H, Y,
                                        batch, seq, hidden, rank, _DT[dtype], _stream(stream))
    B.check(st)
    return H, Y


def all_gather_rows(slices: Sequence[torch.Tensor], batch: int, seq: int,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The full [batch*seq, hidden] tensor from the N ranks' sequence slices."""
    N = len(slices)
    if N < 1:
        raise ValueError("at least one slice is needed")
    hidden = slices[0].shape[-1]
    dt = slices[0].dtype
    if dt not in _DT:
        raise ValueError("slices have dtype %s, expected float32 or bfloat16" % dt)
    for q, t in enumerate(slices):
        _need("slice %d" % q, t, (batch * (seq // N), hidden), dt)
    if out is None:
        out = torch.empty(batch * seq, hidden, dtype=dt, device=slices[0].device)
    _need("out", out, (batch * seq, hidden), dt)
    _require_cuda(*slices, out)
    st = B.tp_all_gather_rows(list(slices), N, batch, seq, hidden, out, _DT[out.dtype],
                              _stream(stream))
    B.check(st)
    return out


# ---- one rank's Transformer layer ------------------------------------------------------------
class LayerShard:
    """Rank ``rank`` of an N-way tensor-parallel layer: attention block then MLP block.

    The other ranks' partials are supplied by the caller (on one device they are computed
    by running the other shards); each block ends in exactly one partial sum. Buffers are
    allocated once so that repeated calls allocate nothing.

    ``fused=True`` runs each block's row-parallel product with the partial sum in its
    epilogue (tp_row_parallel_sum_fwd): the rank's own partials are never written, and H and
    the output are the same bits as the unfused step's.
    """

    STAGES_UNFUSED = ("attention_shard", "sum_attention", "mlp_column", "mlp_row", "sum_mlp")
    STAGES_FUSED = ("qkv_projection", "attention", "out_projection_sum", "mlp_column",
                    "mlp_row_sum")
    STAGES = STAGES_UNFUSED

    def __init__(self, batch: int, seq: int, hidden: int, n_heads: int, ffn: int,
                 n_shards: int, rank: int, causal: bool = True, device="cuda",
                 fused: bool = False):
        self.batch, self.seq, self.hidden = batch, seq, hidden
        self.n_heads, self.ffn, self.n_shards, self.rank = n_heads, ffn, n_shards, rank
        self.causal, self.fused = causal, fused
        self.STAGES = self.STAGES_FUSED if fused else self.STAGES_UNFUSED
        T = batch * seq
        self.attn_ws = attn_workspace(batch, seq, hidden, n_heads, n_shards, device)
        self.mlp_ws = mlp_workspace(T, hidden, ffn, n_shards, torch.bfloat16, device)
        self.O = attn_views(self.attn_ws, batch, seq, hidden, n_heads, n_shards)["o"]
        self.Z_attn = None if fused else torch.empty(T, hidden, dtype=torch.float32, device=device)
        self.H = torch.empty(T, hidden, dtype=torch.bfloat16, device=device)
        self.Y = torch.empty(T, ffn // n_shards, dtype=torch.bfloat16, device=device)
        self.Z_mlp = None if fused else torch.empty(T, hidden, dtype=torch.float32, device=device)
        self.out = torch.empty(T, hidden, dtype=torch.float32, device=device)

    def forward(self, X, Wqkv_i, bqkv_i, Wo_i, A_i, a_i, B_i,
                attn_partials_other: List[torch.Tensor], mlp_partials_other: List[torch.Tensor],
                stream=None, on_stage: Optional[Callable[[str], None]] = None) -> torch.Tensor:
        """attn partial -> H = bf16(sum of N attention partials) -> MLP partial on H -> sum.

        ``on_stage(name)`` (optional) is called after each stage's launches are enqueued,
        with the names in ``self.STAGES`` (used to bracket stages with stream events).
        """
        mark = on_stage or (lambda name: None)
        r, N = self.rank, self.n_shards
        if self.fused:
            H_ = self.n_heads
            qkv_projection(X, Wqkv_i, bqkv_i, self.batch, self.seq, H_, H_, N, r, self.attn_ws,
                           stream=stream)
            mark("qkv_projection")
            head_attention(self.batch, self.seq, self.hidden, H_, H_, N, r, self.causal,
                           self.attn_ws, stream=stream)
            mark("attention")
            peers = list(attn_partials_other)
            peers.insert(r, None)
            row_parallel_sum(self.O, Wo_i, peers, N, r, out=self.H, stream=stream)
            mark("out_projection_sum")
            column_parallel(self.H, A_i, a_i, N, r, gelu=True, Y=self.Y, stream=stream)
            mark("mlp_column")
            peers = list(mlp_partials_other)
            peers.insert(r, None)
            row_parallel_sum(self.Y, B_i, peers, N, r, out=self.out, stream=stream)
            mark("mlp_row_sum")
            return self.out
        attn_shard(X, Wqkv_i, bqkv_i, Wo_i, self.batch, self.seq, self.n_heads, N, r,
                   self.causal, Z=self.Z_attn, workspace=self.attn_ws, stream=stream)
        mark("attention_shard")
        parts = list(attn_partials_other)
        parts.insert(r, self.Z_attn)
        sum_partials(parts, out=self.H, stream=stream)
        mark("sum_attention")
        column_parallel(self.H, A_i, a_i, N, r, gelu=True, Y=self.Y, stream=stream)
        mark("mlp_column")
        row_parallel(self.Y, B_i, N, r, Z=self.Z_mlp, stream=stream)
        mark("mlp_row")
        parts = list(mlp_partials_other)
        parts.insert(r, self.Z_mlp)
        sum_partials(parts, out=self.out, stream=stream)
        mark("sum_mlp")
        return self.out
