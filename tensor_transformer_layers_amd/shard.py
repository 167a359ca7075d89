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
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def _stream(stream):
    return torch.cuda.current_stream() if stream is None else stream


# ---- column / row-parallel linear layers ----------------------------------------------------
def column_parallel(X: torch.Tensor, W_i: torch.Tensor, b_i: Optional[torch.Tensor],
                    n_shards: int, rank: int, gelu: bool = False, Y: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Y_i = act(X W_i + b_i), W_i [out/N, in] (tp_column_parallel_fwd)."""
    _require_cuda(X, W_i, b_i)
    rows, k = X.shape
    width = W_i.shape[0]
    if Y is None:
        Y = torch.empty(rows, width, dtype=X.dtype, device=X.device)
    st = B.tp_column_parallel_fwd(X, W_i, b_i, Y, rows, k, width * n_shards, n_shards, rank,
                                  B.TP_ACT_GELU if gelu else B.TP_ACT_NONE, _dt(X),
                                  _stream(stream))
    B.check(st)
    return Y


def row_parallel(X_i: torch.Tensor, W_i: torch.Tensor, n_shards: int, rank: int,
                 Z: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Z_i = X_i W_i (fp32 partial), W_i [out, in/N] (tp_row_parallel_fwd)."""
    _require_cuda(X_i, W_i)
    rows, k = X_i.shape
    width = W_i.shape[0]
    if Z is None:
        Z = torch.empty(rows, width, dtype=torch.float32, device=X_i.device)
    st = B.tp_row_parallel_fwd(X_i, W_i, Z, rows, k * n_shards, width, n_shards, rank, _dt(X_i),
                               _stream(stream))
    B.check(st)
    return Z


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
    _require_cuda(X, A_i, a_i, B_i)
    tokens, hidden = X.shape
    fl = A_i.shape[0]
    ffn = fl * n_shards
    dt = _dt(X)
    if Z is None:
        Z = torch.empty(tokens, hidden, dtype=torch.float32, device=X.device)
    if workspace is None:
        workspace = mlp_workspace(tokens, hidden, ffn, n_shards, X.dtype, X.device)
    st = B.tp_mlp_shard_fwd(X, A_i, a_i, B_i, Z, tokens, hidden, ffn, n_shards, rank, dt,
                            workspace, workspace.numel(), _stream(stream))
    B.check(st)
    return Z, workspace


def mlp_bwd_workspace(tokens: int, hidden: int, ffn: int, n_shards: int, device="cuda"):
    nbytes = B.tp_mlp_bwd_workspace_bytes(tokens, hidden, ffn, n_shards, B.TP_BF16)
    if nbytes == 0:
        raise B.TPError(B.TP_ERR_SHAPE, "invalid MLP backward sizes")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def mlp_shard_backward(X: torch.Tensor, A_i: torch.Tensor, a_i: Optional[torch.Tensor],
                       B_i: torch.Tensor, dZ: torch.Tensor, n_shards: int, rank: int,
                       out: Optional[dict] = None, workspace: Optional[torch.Tensor] = None,
                       stream=None):
    """Gradients of rank ``rank``'s MLP partial for the upstream dZ (bf16).

    Returns ({"dX": [T, h], "dA": [F/N, h], "da": [F/N], "dB": [h, F/N]} fp32, in the stored
    layouts of X, A_i, a_i, B_i; workspace). dX is the rank's input-gradient partial."""
    _require_cuda(X, A_i, a_i, B_i, dZ)
    tokens, hidden = X.shape
    fl = A_i.shape[0]
    ffn = fl * n_shards
    f32 = dict(dtype=torch.float32, device=X.device)
    if out is None:
        out = {"dX": torch.empty(tokens, hidden, **f32), "dA": torch.empty(fl, hidden, **f32),
               "da": torch.empty(fl, **f32) if a_i is not None else None,
               "dB": torch.empty(hidden, fl, **f32)}
    if workspace is None:
        workspace = mlp_bwd_workspace(tokens, hidden, ffn, n_shards, X.device)
    st = B.tp_mlp_shard_bwd(X, A_i, a_i, B_i, dZ, out["dX"], out["dA"], out.get("da"), out["dB"],
                            tokens, hidden, ffn, n_shards, rank, _dt(X), workspace,
                            workspace.numel(), _stream(stream))
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
    _require_cuda(X, Wg_i, Wu_i, Wd_i)
    tokens, hidden = X.shape
    fl = Wg_i.shape[0]
    ffn = fl * n_shards
    if Z is None:
        Z = torch.empty(tokens, hidden, dtype=torch.float32, device=X.device)
    if workspace is None:
        workspace = swiglu_workspace(tokens, hidden, ffn, n_shards, X.device)
    st = B.tp_swiglu_shard_fwd(X, Wg_i, Wu_i, Wd_i, Z, tokens, hidden, ffn, n_shards, rank,
                               _dt(X), workspace, workspace.numel(), _stream(stream))
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
    _require_cuda(X, Wqkv_i, bqkv_i, Wo_i)
    hidden = X.shape[1]
    if Z is None:
        Z = torch.empty(batch * seq, hidden, dtype=torch.float32, device=X.device)
    if workspace is None:
        workspace = attn_workspace(batch, seq, hidden, n_heads, n_shards, X.device)
    st = B.tp_attn_shard_fwd(X, Wqkv_i, bqkv_i, Wo_i, Z, batch, seq, hidden, n_heads, causal,
                             n_shards, rank, _dt(X), workspace, workspace.numel(),
                             _stream(stream))
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
    _require_cuda(X, Wqkv_i, bqkv_i, Wo_i)
    hidden = X.shape[1]
    if Z is None:
        Z = torch.empty(batch * seq, hidden, dtype=torch.float32, device=X.device)
    if workspace is None:
        workspace = gqa_attn_workspace(batch, seq, hidden, n_heads, n_kv_heads, n_shards, X.device)
    st = B.tp_gqa_attn_shard_fwd(X, Wqkv_i, bqkv_i, Wo_i, Z, batch, seq, hidden, n_heads,
                                 n_kv_heads, causal, n_shards, rank, _dt(X), workspace,
                                 workspace.numel(), _stream(stream))
    B.check(st)
    return Z, workspace


# ---- partial sum ------------------------------------------------------------------------------
def sum_partials(parts: Sequence[torch.Tensor], out_dtype=torch.float32,
                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _require_cuda(*parts)
    numel = parts[0].numel()
    if out is None:
        out = torch.empty(parts[0].shape, dtype=out_dtype, device=parts[0].device)
    st = B.tp_sum_partials(list(parts), len(parts), numel, out, _DT[out.dtype], _stream(stream))
    B.check(st)
    return out


# ---- sequence parallelism ----------------------------------------------------------------------
def reduce_scatter(parts: Sequence[torch.Tensor], batch: int, seq: int, rank: int,
                   out_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """Rank ``rank``'s slice [batch*seq/N, hidden] of sum(parts) (N = len(parts))."""
    _require_cuda(*parts)
    N = len(parts)
    hidden = parts[0].shape[-1]
    if out is None:
        out = torch.empty(batch * (seq // N), hidden, dtype=out_dtype, device=parts[0].device)
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
    _require_cuda(*parts, residual, gamma, beta)
    N = len(parts)
    hidden = parts[0].shape[-1]
    rows = batch * (seq // N)
    if H is None:
        H = torch.empty(rows, hidden, dtype=dtype, device=parts[0].device)
    if Y is None:
        Y = torch.empty(rows, hidden, dtype=dtype, device=parts[0].device)
    st = B.tp_sp_residual_layernorm_fwd(list(parts), N, residual, gamma, beta, float(eps), H, Y,
                                        batch, seq, hidden, rank, _DT[dtype], _stream(stream))
    B.check(st)
    return H, Y


def all_gather_rows(slices: Sequence[torch.Tensor], batch: int, seq: int,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The full [batch*seq, hidden] tensor from the N ranks' sequence slices."""
    _require_cuda(*slices)
    N = len(slices)
    hidden = slices[0].shape[-1]
    if out is None:
        out = torch.empty(batch * seq, hidden, dtype=slices[0].dtype, device=slices[0].device)
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
    """

    def __init__(self, batch: int, seq: int, hidden: int, n_heads: int, ffn: int,
                 n_shards: int, rank: int, causal: bool = True, device="cuda"):
        self.batch, self.seq, self.hidden = batch, seq, hidden
        self.n_heads, self.ffn, self.n_shards, self.rank = n_heads, ffn, n_shards, rank
        self.causal = causal
        T = batch * seq
        self.attn_ws = attn_workspace(batch, seq, hidden, n_heads, n_shards, device)
        self.mlp_ws = mlp_workspace(T, hidden, ffn, n_shards, torch.bfloat16, device)
        self.Z_attn = torch.empty(T, hidden, dtype=torch.float32, device=device)
        self.H = torch.empty(T, hidden, dtype=torch.bfloat16, device=device)
        self.Y = torch.empty(T, ffn // n_shards, dtype=torch.bfloat16, device=device)
        self.Z_mlp = torch.empty(T, hidden, dtype=torch.float32, device=device)
        self.out = torch.empty(T, hidden, dtype=torch.float32, device=device)

    STAGES = ("attention_shard", "sum_attention", "mlp_column", "mlp_row", "sum_mlp")

    def forward(self, X, Wqkv_i, bqkv_i, Wo_i, A_i, a_i, B_i,
                attn_partials_other: List[torch.Tensor], mlp_partials_other: List[torch.Tensor],
                stream=None, on_stage: Optional[Callable[[str], None]] = None) -> torch.Tensor:
        """attn partial -> H = bf16(sum of N attention partials) -> MLP partial on H -> sum.

        ``on_stage(name)`` (optional) is called after each stage's launches are enqueued,
        with the names in ``STAGES`` (used to bracket stages with stream events).
        """
        mark = on_stage or (lambda name: None)
        r, N = self.rank, self.n_shards
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
