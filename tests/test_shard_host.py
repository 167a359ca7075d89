"""Host-side checks of the torch wrappers (no GPU, no kernel launch): every tensor argument,
outputs and workspaces included, is checked for shape, dtype, device and contiguity before any
call into the library, and a mismatch raises ValueError.

The tensors here are CPU tensors: a wrongly shaped one must be rejected for its shape, and a
correctly shaped one for not being on the device -- in both cases before the library sees it.
"""
import pytest
import torch

from tensor_transformer_layers_amd import shard

bf = torch.bfloat16
f32 = torch.float32


def _mlp(T=16, h=64, fl=32, dt=bf):
    return dict(X=torch.zeros(T, h, dtype=dt), A_i=torch.zeros(fl, h, dtype=dt),
                a_i=torch.zeros(fl, dtype=dt), B_i=torch.zeros(h, fl, dtype=dt))


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_mlp_shard_checks_every_argument():
    m = _mlp()
    # B_i in the pages' [in, out] layout has the right element count but the wrong shape
    _raises("B_i has shape", shard.mlp_shard, m["X"], m["A_i"], m["a_i"], m["B_i"].t().contiguous(), 2, 0)
    _raises("a_i has shape", shard.mlp_shard, m["X"], m["A_i"], torch.zeros(33, dtype=bf), m["B_i"], 2, 0)
    _raises("A_i has dtype", shard.mlp_shard, m["X"], m["A_i"].float(), m["a_i"], m["B_i"], 2, 0)
    _raises("Z has shape", shard.mlp_shard, m["X"], m["A_i"], m["a_i"], m["B_i"], 2, 0,
            Z=torch.zeros(16, 32, dtype=f32))
    _raises("Z has dtype", shard.mlp_shard, m["X"], m["A_i"], m["a_i"], m["B_i"], 2, 0,
            Z=torch.zeros(16, 64, dtype=bf))
    _raises("workspace holds", shard.mlp_shard, m["X"], m["A_i"], m["a_i"], m["B_i"], 2, 0,
            workspace=torch.zeros(16 * 32 * 2 - 1, dtype=torch.uint8))
    _raises("X must be a 2-D", shard.mlp_shard, m["X"].view(-1), m["A_i"], m["a_i"], m["B_i"], 2, 0)
    # correct shapes, but host memory: rejected for the device
    _raises("device tensors", shard.mlp_shard, m["X"], m["A_i"], m["a_i"], m["B_i"], 2, 0)


def test_linear_primitives_check_outputs():
    X, W = torch.zeros(16, 64, dtype=bf), torch.zeros(32, 64, dtype=bf)
    _raises("b_i has shape", shard.column_parallel, X, W, torch.zeros(64, dtype=bf), 2, 0)
    _raises("Y has shape", shard.column_parallel, X, W, None, 2, 0, Y=torch.zeros(16, 33, dtype=bf))
    _raises("W_i has shape", shard.column_parallel, X, torch.zeros(32, 63, dtype=bf), None, 2, 0)
    _raises("Z has dtype", shard.row_parallel, X, W.t().contiguous().t().contiguous()[:, :64], 2, 0,
            Z=torch.zeros(16, 32, dtype=bf))
    _raises("device tensors", shard.row_parallel, X, W, 2, 0)
    # a non-contiguous output is refused too
    Y = torch.zeros(32, 16, dtype=bf).t()
    _raises("device tensors", shard.column_parallel, X, W, None, 2, 0, Y=Y)


def test_attention_wrappers_check_weights():
    b, s, h, H, N = 1, 8, 256, 2, 2          # d = 128, one head per rank
    X = torch.zeros(b * s, h, dtype=bf)
    Wqkv, Wo = torch.zeros(3 * 128, h, dtype=bf), torch.zeros(h, 128, dtype=bf)
    _raises("Wo_i has shape", shard.attn_shard, X, Wqkv, None, Wo.t().contiguous(), b, s, H, N, 0)
    _raises("bqkv_i has shape", shard.attn_shard, X, Wqkv, torch.zeros(128, dtype=bf), Wo, b, s, H, N, 0)
    _raises("X has shape", shard.attn_shard, X[:7], Wqkv, None, Wo, b, s, H, N, 0)
    # 4 query heads of d = 128 with 2 key/value heads over N = 2: one key/value head per rank,
    # so a multi-head [Q | K | V] shard (6 heads) is the wrong width for the grouped layout (4)
    X4, Wqkv4, Wo4 = torch.zeros(b * s, 512, dtype=bf), torch.zeros(6 * 128, 512, dtype=bf), \
        torch.zeros(512, 256, dtype=bf)
    _raises("Wqkv_i has shape", shard.gqa_attn_shard, X4, Wqkv4, None, Wo4, b, s, 4, 2, N, 0)
    _raises("device tensors", shard.gqa_attn_shard, X4, Wqkv4[:512], None, Wo4, b, s, 4, 2, N, 0)
    _raises("do not split", shard.attn_shard, X, Wqkv, None, Wo, b, s, 3, N, 0)
    _raises("device tensors", shard.attn_shard, X, Wqkv, None, Wo, b, s, H, N, 0)


def test_exchange_wrappers_check_partials():
    p = [torch.zeros(8, 16, dtype=f32) for _ in range(3)]
    _raises("partial 2 has shape", shard.sum_partials, p[:2] + [torch.zeros(8, 8, dtype=f32)])
    _raises("partial 1 has dtype", shard.sum_partials, [p[0], p[1].to(bf)])
    _raises("out has shape", shard.sum_partials, p, out=torch.zeros(128, dtype=f32))
    _raises("out has dtype", shard.sum_partials, p, out=torch.zeros(8, 16, dtype=torch.float16))
    _raises("device tensors", shard.sum_partials, p)
    parts = [torch.zeros(8, 16, dtype=f32) for _ in range(2)]
    _raises("out has shape", shard.reduce_scatter, parts, 1, 8, 0, out=torch.zeros(8, 16))
    _raises("gamma has shape", shard.sp_residual_layernorm, parts, None, torch.zeros(8),
            torch.zeros(16), 1, 8, 0)
    _raises("slice 1 has shape", shard.all_gather_rows,
            [torch.zeros(4, 16, dtype=bf), torch.zeros(5, 16, dtype=bf)], 1, 8)


def test_backward_checks_gradients():
    m = _mlp()
    dZ = torch.zeros(16, 64, dtype=bf)
    out = {"dX": torch.zeros(16, 64), "dA": torch.zeros(64, 32), "da": torch.zeros(32),
           "dB": torch.zeros(64, 32)}
    _raises("dA has shape", shard.mlp_shard_backward, m["X"], m["A_i"], m["a_i"], m["B_i"], dZ, 2, 0,
            out=out)
    _raises("dZ has shape", shard.mlp_shard_backward, m["X"], m["A_i"], m["a_i"], m["B_i"], dZ[:8], 2, 0)


def test_forward_keeping_p_and_backward_taking_it_check_p():
    m = _mlp()
    dZ = torch.zeros(16, 64, dtype=bf)
    _raises("P has shape", shard.mlp_shard_save, m["X"], m["A_i"], m["a_i"], m["B_i"], 2, 0,
            P=torch.zeros(16, 64, dtype=bf))
    _raises("P has dtype", shard.mlp_shard_save, m["X"], m["A_i"], m["a_i"], m["B_i"], 2, 0,
            P=torch.zeros(16, 32, dtype=f32))
    _raises("X has dtype", shard.mlp_shard_save, m["X"].float(), m["A_i"], m["a_i"], m["B_i"], 2, 0)
    _raises("device tensors", shard.mlp_shard_save, m["X"], m["A_i"], m["a_i"], m["B_i"], 2, 0)
    _raises("P has shape", shard.mlp_shard_backward, m["X"], m["A_i"], m["a_i"], m["B_i"], dZ, 2, 0,
            P=torch.zeros(32, 16, dtype=bf))
    _raises("device tensors", shard.mlp_shard_backward, m["X"], m["A_i"], m["a_i"], m["B_i"], dZ,
            2, 0, P=torch.zeros(16, 32, dtype=bf))
