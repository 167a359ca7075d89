"""GPU parity of the row-parallel layer with the partial sum fused into its epilogue
(tp_row_parallel_sum_fwd): Z = sum_q Z_q with Z_rank = X_i W_i computed in the same kernel.

It must give exactly the bits of tp_row_parallel_fwd into Z_rank followed by tp_sum_partials
(the same fp32 adds in the same order q = 0 .. N-1), for fp32 and bf16 outputs, every tile
layout, ragged shapes and any rank; and match the fp64 oracle (sum of the partials plus the
product) within the bf16 tolerance.
"""
import numpy as np
import pytest

import oracle
from gpu_util import canary_tensor, host, torch_cuda

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _inputs(torch, T, k, width, N, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    X = torch.randn(T, k, device="cuda", generator=g).to(torch.bfloat16)
    W = (0.05 * torch.randn(width, k, device="cuda", generator=g)).to(torch.bfloat16)
    parts = [torch.randn(T, width, device="cuda", generator=g) for _ in range(N)]
    return X, W, parts


def _check(T, k, width, N, rank, out_dtype, seed=0):
    torch = torch_cuda()
    from tensor_transformer_layers_amd import shard
    X, W, parts = _inputs(torch, T, k, width, N, seed)
    own = shard.row_parallel(X, W, N, rank)
    ref_parts = list(parts)
    ref_parts[rank] = own
    Z_ref = shard.sum_partials(ref_parts, out_dtype=out_dtype)
    peers = list(parts)
    peers[rank] = None
    Zc = canary_tensor((T, width), out_dtype)
    Z = shard.row_parallel_sum(X, W, peers, N, rank, out=Zc.tensor)
    torch.cuda.synchronize()
    assert Zc.intact(), "write outside the output"
    assert torch.equal(Z, Z_ref), "fused sum differs from row GEMM + tp_sum_partials"
    # fp64: the peers' partials plus the product
    Pn = np.stack([host(p) for q, p in enumerate(parts) if q != rank] or [np.zeros((T, width))])
    ref = Pn.sum(axis=0) + oracle.linear(host(X), host(W).T)
    return oracle.rel_frobenius(host(Z), ref)


@pytest.mark.parametrize("case", [
    # T, k, width, N, rank
    (200, 520, 264, 2, 0), (200, 520, 264, 2, 1), (77, 64, 8, 3, 2), (513, 1024, 1000, 8, 5),
    (1, 256, 64, 1, 0), (300, 2048, 512, 8, 7), (256, 4096, 2048, 4, 0),
])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_fused_sum_bitwise_equal_ragged(case, out):
    torch = torch_cuda()
    e = _check(*case, torch.float32 if out == "f32" else torch.bfloat16)
    print("%s %s: err %.2e" % (case, out, e))
    assert e < TOL


@pytest.mark.parametrize("tile", ["256x256", "256x192", "256x128", "128x128", "256x256w4",
                                  "256x192w4", "256x128w4", "128x128w4"])
def test_fused_sum_every_tile_layout(tile, overrides):
    torch = torch_cuda()
    overrides("gemm_tile=" + tile)
    for out in (torch.float32, torch.bfloat16):
        e = _check(333, 2056, 776, 5, 3, out, seed=len(tile))
        assert e < TOL, (tile, out)


@pytest.mark.parametrize("rank", [0, 5])
def test_fused_sum_layer_shapes(rank):
    """The layer's two fused sums at full size: the output projection (4096 x 8192 x 1024,
    bf16 H) and the MLP row GEMM (4096 x 8192 x 4096, fp32 Z), N = 8."""
    torch = torch_cuda()
    e1 = _check(4096, 1024, 8192, 8, rank, torch.bfloat16, seed=rank)
    e2 = _check(4096, 4096, 8192, 8, rank, torch.float32, seed=rank + 1)
    print("rank %d: W_O + sum err %.2e, MLP row + sum err %.2e" % (rank, e1, e2))
    assert e1 < TOL and e2 < TOL


@pytest.mark.parametrize("case", [
    # T, k, width, N, rank, tile: shapes whose launch takes two tiles per workgroup and streams
    # the first tile's sum during the second one's K loop (ragged rows and K included)
    (4096, 4096, 8192, 8, 0, None), (4096, 4096, 8192, 8, 7, None),
    (3996, 4160, 8184, 3, 1, None), (4096, 3072, 6144, 2, 1, "256x192"),
    (4096, 2048, 4096, 8, 4, "256x128"), (2048, 1024, 4096, 5, 0, "128x128"),
])
def test_fused_sum_deferred_form_bitwise(case, overrides):
    """The deferred form gives the bits of the in-epilogue form and of row GEMM + sum."""
    torch = torch_cuda()
    from tensor_transformer_layers_amd import shard
    T, k, width, N, rank, tile = case
    if tile:
        overrides("gemm_tile=" + tile)
    X, W, parts = _inputs(torch, T, k, width, N, seed=T + N)
    peers = list(parts)
    peers[rank] = None
    Zc = canary_tensor((T, width), torch.float32)
    Z = shard.row_parallel_sum(X, W, peers, N, rank, out=Zc.tensor)
    torch.cuda.synchronize()
    assert Zc.intact(), "write outside the output"
    overrides(("gemm_tile=%s," % tile if tile else "") + "sum_defer=0")
    Z0 = shard.row_parallel_sum(X, W, peers, N, rank)
    ref_parts = list(parts)
    ref_parts[rank] = shard.row_parallel(X, W, N, rank)
    Z_ref = shard.sum_partials(ref_parts, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(Z, Z0), "deferred form differs from the in-epilogue form"
    assert torch.equal(Z, Z_ref), "deferred form differs from row GEMM + tp_sum_partials"


@pytest.mark.parametrize("case", [
    # T, k, width, N, rank, out: shapes that take the ring form (128 x 128 tiles in rounds of
    # 256 workgroups, a 16-slab K loop): the layer's output projection, ragged rows, columns
    # and K, two, three and five partials, the last rank
    (4096, 1024, 8192, 8, 0, "bf16"), (4096, 1024, 8192, 8, 5, "f32"),
    (4096, 1024, 8192, 8, 7, "bf16"), (4000, 1000, 8184, 3, 1, "bf16"),
    (4040, 1000, 8184, 3, 2, "f32"), (2048, 1024, 4096, 2, 1, "f32"),
    (2048, 984, 4096, 5, 4, "bf16"),
])
def test_fused_sum_ring_form_bitwise(case, overrides):
    """The ring form (each tile's own product kept in LDS, its sum streamed during the next
    tile's K loop) gives the bits of row GEMM + tp_sum_partials and of the other forms."""
    torch = torch_cuda()
    from tensor_transformer_layers_amd import shard
    T, k, width, N, rank, out = case
    odt = torch.float32 if out == "f32" else torch.bfloat16
    X, W, parts = _inputs(torch, T, k, width, N, seed=T + k + N)
    peers = list(parts)
    peers[rank] = None
    overrides("sum_ring=2")
    Zc = canary_tensor((T, width), odt)
    Z = shard.row_parallel_sum(X, W, peers, N, rank, out=Zc.tensor)
    torch.cuda.synchronize()
    assert Zc.intact(), "write outside the output"
    overrides("sum_ring=1")
    Z1 = shard.row_parallel_sum(X, W, peers, N, rank, out=torch.empty_like(Z))
    ref_parts = list(parts)
    ref_parts[rank] = shard.row_parallel(X, W, N, rank)
    Z_ref = shard.sum_partials(ref_parts, out_dtype=odt)
    torch.cuda.synchronize()
    assert torch.equal(Z, Z_ref), "ring form differs from row GEMM + tp_sum_partials"
    assert torch.equal(Z, Z1), "ring form differs from the other fused form"
