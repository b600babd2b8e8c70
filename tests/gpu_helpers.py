"""Shared helpers of the GPU tests and the benchmark: device copies of the seeded inputs and the
per-row relative L2 metric.  No layer arithmetic lives here."""
from __future__ import annotations

import numpy as np
import torch

import bit_expert_ffn_fp32_amd as sm
import moe_inputs as mi

TOL_REL_L2 = 5e-3  # per output row, against the fp64 oracle


def dev():
    return torch.device("cuda:0")


def to_dev_bf16(x_np: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).to(dev())


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def rel_l2_rows(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref, axis=1)
    assert np.all(den > 0), "a reference row is zero"
    return np.linalg.norm(got - ref, axis=1) / den


def bf16_tensor_to_f64(t: torch.Tensor) -> np.ndarray:
    return mi.bf16_bits_to_f32(t.cpu().numpy().view(np.uint16)).astype(np.float64)


class Layer:
    """A layer's inputs on the host (numpy) and the device (torch)."""

    def __init__(self, shape: mi.Shape, seed: int = 0, layer: int = 0, T: int | None = None):
        self.shape = shape
        self.T = shape.T if T is None else T
        self.w_np = mi.make_weights(shape, seed, layer)
        self.x_np = mi.make_x(shape, seed, layer, self.T)
        self.l_np = mi.make_logits(shape, seed, layer, self.T)
        self.w = sm.Weights.from_numpy(self.w_np, dev())
        self.x = to_dev_bf16(self.x_np)
        self.logits = to_dev(self.l_np)

    def workspace(self, T: int | None = None) -> torch.Tensor:
        s = self.shape
        T = self.T if T is None else T
        return sm.alloc_workspace(sm.workspace_bytes(T, s.E, s.k, s.H, s.I), dev())
