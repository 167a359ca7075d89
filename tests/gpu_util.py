"""Helpers of the GPU parity tests: device upload, guard-band canaries, shard preparation.

Inputs come from ``synth`` (seeded, in the pages' layout); ``layout`` slices them into each
rank's arrays by pure indexing; expected values come from ``oracle`` only.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GUARD = 256          # guard-band bytes on each side of a canary buffer
SENTINEL = 0xA5


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tensor_transformer_layers_amd import binding
    binding.lib()    # fails loudly if the HIP library was not built
    return torch


def dev(x: np.ndarray, dtype: str):
    """numpy float32 (bf16-exact when dtype is bf16) -> contiguous device tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)      # exact: the values are bf16-representable
    return t.cuda()


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


class Canary:
    """A device buffer of ``nbytes`` with sentinel-filled guard bands on both sides."""

    def __init__(self, nbytes: int, dtype, shape):
        import torch
        self.nbytes = nbytes
        self.raw = torch.full((nbytes + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
        self.body = self.raw[GUARD:GUARD + nbytes]
        self.tensor = self.body.view(dtype).view(*shape) if shape is not None else self.body

    def intact(self) -> bool:
        import torch
        torch.cuda.synchronize()
        lo = self.raw[:GUARD].cpu().numpy()
        hi = self.raw[GUARD + self.nbytes:].cpu().numpy()
        return bool((lo == SENTINEL).all() and (hi == SENTINEL).all())


def canary_tensor(shape, dtype) -> Canary:
    import torch
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    return Canary(n, dtype, shape)


def rel_err(got, ref) -> float:
    import oracle
    return oracle.rel_frobenius(got, ref)
