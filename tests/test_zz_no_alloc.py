"""strata_moe_decode_static, the decode entry point that allocates nothing (its scratch is a
fixed device array of the library), against strata_moe_decode on the same inputs: the same
kernels, so the outputs must be bit-identical, on two calls in a row with the second smaller."""
import ctypes

import numpy as np
import pytest
import torch

import bit_expert_ffn_fp32_amd as sm
import moe_inputs as mi
from gpu_helpers import Layer, dev

pytestmark = pytest.mark.gpu


def both(L, T, k, accumulate=False, seed_y=None):
    s = L.shape
    x, lg = L.x[:T].contiguous(), L.logits[:T].contiguous()
    y0 = torch.zeros((T, s.H), dtype=torch.float32, device=dev())
    if seed_y is not None:
        y0.copy_(seed_y[:T])
    y1 = y0.clone()
    ids0 = torch.empty((T, k), dtype=torch.int32, device=dev())
    ids1 = torch.empty_like(ids0)
    w0 = torch.empty((T, k), dtype=torch.float32, device=dev())
    w1 = torch.empty_like(w0)
    ws = sm.alloc_workspace(sm.workspace_bytes(T, s.E, k, s.H, s.I), dev())
    sm.strata_moe_decode(L.w, x, lg, k, y0, accumulate, ids0, w0, ws)
    sm.strata_moe_decode_static(L.w, x, lg, k, y1, accumulate, ids1, w1)
    torch.cuda.synchronize()
    return (y0, ids0, w0), (y1, ids1, w1)


@pytest.mark.parametrize("shape", [mi.DECODE, mi.Shape("q3", T=8, H=1024, E=64, k=6, I=256, fmt=3)],
                         ids=lambda s: s.name)
def test_decode_static_matches_decode(shape):
    L = Layer(shape, seed=3, T=8)
    seed_y = torch.randn((8, shape.H), dtype=torch.float32, device=dev())
    for T, acc in ((min(8, 4 if shape.name == "decode" else 8), False), (2, True), (1, False)):
        ref, got = both(L, T, shape.k, accumulate=acc, seed_y=seed_y if acc else None)
        for a, b in zip(ref, got):
            assert torch.equal(a, b), (shape.name, T)


def test_decode_static_limits():
    L = sm.lib()
    assert L.strata_moe_decode_static_max_bytes() == 128 * 1024
    A = 0x10000
    w = sm.CWeights(2, 512, 3072, 768, A, A, A, A, A, A, 0)
    assert L.strata_moe_decode_static(ctypes.byref(w), A, A, 9, 10, A, 0, None, None, None) == 2
    assert L.strata_moe_decode_static(ctypes.byref(w), A, A, 4, 10, None, 0, None, None, None) == 1
    assert L.strata_moe_decode_static(ctypes.byref(w), A, A, 0, 10, A, 0, None, None, None) == 0
    w_big = sm.CWeights(2, 512, 4096, 4096, A, A, A, A, A, A, 0)  # outside the decode limits
    assert L.strata_moe_decode_static(ctypes.byref(w_big), A, A, 8, 16, A, 0, None, None, None) == 2
