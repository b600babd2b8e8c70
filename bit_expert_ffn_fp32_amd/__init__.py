"""Python binding of libstrata_moe.so, the MI355X routed-MoE expert layer.

Argument marshalling only: every function below calls the C ABI entry point of the same name
(declared in include/strata_moe.h) with device pointers taken from torch tensors and torch's
current HIP stream.  All arithmetic runs in the library's gfx950 kernels.  There is no fallback:
if the library is missing or was not built, import-time use raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libstrata_moe.so")

STRATA_OK, STRATA_ERR_INVALID_ARGUMENT, STRATA_ERR_UNSUPPORTED = 0, 1, 2
STRATA_ERR_WORKSPACE_TOO_SMALL, STRATA_ERR_HIP = 3, 4
Q2, Q3 = 2, 3
CODE_BYTES = {Q2: 8, Q3: 12}

EXPORTS = ["strata_moe_route", "strata_moe_permute", "strata_moe_expert_ffn", "strata_moe_combine",
           "strata_moe_decode", "strata_moe_layer", "strata_moe_rmsnorm", "strata_moe_pack_matrix",
           "strata_moe_router_logits", "strata_moe_shared_expert",
           "strata_moe_usage_update", "strata_moe_usage_rank", "strata_moe_layer_residual",
           "strata_moe_weight_stats", "strata_moe_decode_static",
           "strata_moe_decode_static_max_bytes",
           "strata_moe_residual_workspace_bytes", "strata_moe_block", "strata_moe_block_workspace_bytes",
           "strata_moe_permute_workspace_bytes", "strata_moe_workspace_bytes",
           "strata_moe_shared_workspace_bytes", "strata_status_string"]


class StrataError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class CWeights(ctypes.Structure):
    """strata_moe_weights, field for field (include/strata_moe.h)."""
    _fields_ = [("fmt", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("gate_codes", ctypes.c_void_p), ("up_codes", ctypes.c_void_p),
                ("gate_scales", ctypes.c_void_p), ("up_scales", ctypes.c_void_p),
                ("down_codes", ctypes.c_void_p), ("down_scales", ctypes.c_void_p),
                ("stats", ctypes.c_void_p)]


class CExpertStats(ctypes.Structure):
    """strata_moe_expert_stats (16 bytes per expert)."""
    _fields_ = [("shift_gate", ctypes.c_int32), ("shift_up", ctypes.c_int32),
                ("shift_down", ctypes.c_int32), ("norm_gate_up", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        i32, vp, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
        W = ctypes.POINTER(CWeights)
        sig = {
            "strata_moe_route": [vp, i32, i32, i32, vp, vp, vp],
            "strata_moe_permute": [vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp],
            "strata_moe_expert_ffn": [W, vp, i32, i32, vp, vp, vp, vp, sz, vp],
            "strata_moe_combine": [vp, vp, i32, i32, i32, vp, i32, vp],
            "strata_moe_decode": [W, vp, vp, i32, i32, vp, i32, vp, vp, vp, sz, vp],
            "strata_moe_layer": [W, vp, vp, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp],
            "strata_moe_rmsnorm": [vp, i32, i32, ctypes.c_float, vp, vp],
            "strata_moe_pack_matrix": [i32, i32, i32, i32, vp, vp, vp, vp, vp],
            "strata_moe_router_logits": [vp, vp, i32, i32, i32, vp, vp],
            "strata_moe_shared_expert": [vp, vp, vp, vp, i32, i32, i32, vp, i32, vp, sz, vp],
            "strata_moe_usage_update": [vp, i32, i32, i32, vp, vp],
            "strata_moe_usage_rank": [vp, i32, vp, vp],
            "strata_moe_layer_residual": [W, vp, vp, i32, i32, ctypes.c_float, vp, sz, vp],
            "strata_moe_block": [W, vp, i32, i32, vp, vp, vp, vp, i32, vp, vp, i32, vp, sz, vp],
            "strata_moe_weight_stats": [W, vp, vp],
            "strata_moe_decode_static": [W, vp, vp, i32, i32, vp, i32, vp, vp, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.strata_moe_permute_workspace_bytes.argtypes = [i32, i32, i32]
        L.strata_moe_permute_workspace_bytes.restype = sz
        L.strata_moe_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.strata_moe_workspace_bytes.restype = sz
        L.strata_moe_block_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
        L.strata_moe_block_workspace_bytes.restype = sz
        L.strata_moe_residual_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.strata_moe_residual_workspace_bytes.restype = sz
        L.strata_moe_shared_workspace_bytes.argtypes = [i32, i32]
        L.strata_moe_shared_workspace_bytes.restype = sz
        L.strata_moe_decode_static_max_bytes.argtypes = []
        L.strata_moe_decode_static_max_bytes.restype = sz
        L.strata_status_string.argtypes = [ctypes.c_int]
        L.strata_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != STRATA_OK:
        raise StrataError(fn, status, lib().strata_status_string(status).decode())


def _p(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


@dataclass
class Weights:
    """One layer's packed expert weights as device tensors (see include/strata_moe.h)."""
    fmt: int
    E: int
    H: int
    I: int
    gate_codes: torch.Tensor
    up_codes: torch.Tensor
    down_codes: torch.Tensor
    gate_scales: torch.Tensor
    up_scales: torch.Tensor
    down_scales: torch.Tensor
    stats: torch.Tensor | None = None  # int32 [E][4] holding strata_moe_expert_stats

    def c_struct(self) -> CWeights:
        return CWeights(self.fmt, self.E, self.H, self.I, _p(self.gate_codes), _p(self.up_codes),
                        _p(self.gate_scales), _p(self.up_scales), _p(self.down_codes),
                        _p(self.down_scales), _p(self.stats))

    def compute_stats(self, stream=None) -> "Weights":
        """Fills self.stats with the range statistics of the tiled weights (strata_moe_weight_stats;
        the prefill path needs them)."""
        self.stats = torch.zeros((self.E, 4), dtype=torch.int32, device=self.gate_codes.device)
        strata_moe_weight_stats(self, self.stats, stream)
        return self

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.gate_codes, self.up_codes,
                                                          self.down_codes, self.gate_scales,
                                                          self.up_scales, self.down_scales))

    @staticmethod
    def from_numpy(w: dict, device="cuda") -> "Weights":
        """Uploads row-major arrays ([E][rows][K/32][cb] codes, [E][rows][K/32] fp16 scales) and
        repacks them on the device into the tiled layout the kernels read."""
        fmt, E, H, I = w["fmt"], w["E"], w["H"], w["I"]

        def packed(codes, scales, rows, K):
            c = torch.from_numpy(codes).to(device)
            s_ = torch.from_numpy(scales.view("int16")).to(device)
            tc, ts = torch.empty_like(c), torch.empty_like(s_)
            strata_moe_pack_matrix(fmt, E, rows, K, c, s_, tc, ts)
            return tc, ts

        gc, gs = packed(w["gate_codes"], w["gate_scales"], I, H)
        uc, us = packed(w["up_codes"], w["up_scales"], I, H)
        dc, ds = packed(w["down_codes"], w["down_scales"], H, I)
        return Weights(fmt, E, H, I, gc, uc, dc, gs, us, ds).compute_stats()


def permute_workspace_bytes(T: int, E: int, k: int) -> int:
    return lib().strata_moe_permute_workspace_bytes(T, E, k)


def workspace_bytes(T: int, E: int, k: int, H: int, I: int) -> int:
    return lib().strata_moe_workspace_bytes(T, E, k, H, I)


def block_workspace_bytes(T: int, E: int, k: int, H: int, I: int, Is: int) -> int:
    return lib().strata_moe_block_workspace_bytes(T, E, k, H, I, Is)


def residual_workspace_bytes(T: int, E: int, k: int, H: int, I: int) -> int:
    return lib().strata_moe_residual_workspace_bytes(T, E, k, H, I)


def shared_workspace_bytes(T: int, I: int) -> int:
    return lib().strata_moe_shared_workspace_bytes(T, I)


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def strata_moe_route(logits, k, topk_ids, topk_w, stream=None) -> None:
    T, E = logits.shape
    _check("strata_moe_route", lib().strata_moe_route(_p(logits), T, E, k, _p(topk_ids), _p(topk_w),
                                                      _stream(stream)))


def strata_moe_permute(topk_ids, E, counts, offsets, sorted_slot, slot_pos, workspace,
                       stream=None) -> None:
    T, k = topk_ids.shape
    _check("strata_moe_permute", lib().strata_moe_permute(
        _p(topk_ids), T, E, k, _p(counts), _p(offsets), _p(sorted_slot), _p(slot_pos),
        _p(workspace), workspace.numel() if workspace is not None else 0, _stream(stream)))


def strata_moe_expert_ffn(w: Weights, x, k, offsets, sorted_slot, expert_out, workspace,
                          stream=None) -> None:
    cw = w.c_struct()
    _check("strata_moe_expert_ffn", lib().strata_moe_expert_ffn(
        ctypes.byref(cw), _p(x), x.shape[0], k, _p(offsets), _p(sorted_slot), _p(expert_out),
        _p(workspace), workspace.numel(), _stream(stream)))


def strata_moe_combine(expert_out, topk_w, y, accumulate=False, stream=None) -> None:
    T, k = topk_w.shape
    _check("strata_moe_combine", lib().strata_moe_combine(
        _p(expert_out), _p(topk_w), T, k, y.shape[1], _p(y), int(accumulate), _stream(stream)))


def strata_moe_decode(w: Weights, x, logits, k, y, accumulate=False, topk_ids=None, topk_w=None,
                      workspace=None, stream=None) -> None:
    cw = w.c_struct()
    _check("strata_moe_decode", lib().strata_moe_decode(
        ctypes.byref(cw), _p(x), _p(logits), x.shape[0], k, _p(y), int(accumulate), _p(topk_ids),
        _p(topk_w), _p(workspace), workspace.numel() if workspace is not None else 0,
        _stream(stream)))


def strata_moe_decode_static(w: Weights, x, logits, k, y, accumulate=False, topk_ids=None,
                             topk_w=None, stream=None) -> None:
    """strata_moe_decode with the library's fixed scratch instead of a workspace (no allocation;
    calls that overlap on one GPU race)."""
    cw = w.c_struct()
    _check("strata_moe_decode_static", lib().strata_moe_decode_static(
        ctypes.byref(cw), _p(x), _p(logits), x.shape[0], k, _p(y), int(accumulate), _p(topk_ids),
        _p(topk_w), _stream(stream)))


def strata_moe_layer(w: Weights, x, logits, k, y, accumulate=False, topk_ids=None, topk_w=None,
                     counts=None, offsets=None, sorted_slot=None, workspace=None,
                     stream=None) -> None:
    cw = w.c_struct()
    _check("strata_moe_layer", lib().strata_moe_layer(
        ctypes.byref(cw), _p(x), _p(logits), x.shape[0], k, _p(y), int(accumulate), _p(topk_ids),
        _p(topk_w), _p(counts), _p(offsets), _p(sorted_slot), _p(workspace),
        workspace.numel() if workspace is not None else 0, _stream(stream)))


def strata_moe_pack_matrix(fmt, n_mat, rows, K, codes, scales, tiled_codes, tiled_scales,
                           stream=None) -> None:
    _check("strata_moe_pack_matrix", lib().strata_moe_pack_matrix(
        fmt, n_mat, rows, K, _p(codes), _p(scales), _p(tiled_codes), _p(tiled_scales),
        _stream(stream)))


def strata_moe_weight_stats(w: Weights, stats, stream=None) -> None:
    """stats (int32 [E][4] viewed as strata_moe_expert_stats) = range statistics of w."""
    cw = w.c_struct()
    _check("strata_moe_weight_stats", lib().strata_moe_weight_stats(ctypes.byref(cw), _p(stats),
                                                                    _stream(stream)))


def strata_moe_rmsnorm(h, x, eps=1e-6, stream=None) -> None:
    T, H = h.shape
    _check("strata_moe_rmsnorm", lib().strata_moe_rmsnorm(_p(h), T, H, eps, _p(x), _stream(stream)))


def strata_moe_router_logits(x, w_router, logits, stream=None) -> None:
    """logits fp32 [T][E] = x W_r^T (x bf16 [T][H], w_router bf16 [E][H]; bf16 tensors or their
    int16 bit patterns)."""
    T, H = x.shape
    E = w_router.shape[0]
    _check("strata_moe_router_logits", lib().strata_moe_router_logits(
        _p(x), _p(w_router), T, H, E, _p(logits), _stream(stream)))


def strata_moe_shared_expert(x, w_gate, w_up, w_down, y, workspace, accumulate=False,
                             stream=None) -> None:
    """y (=, or += with accumulate) SwiGLU shared expert of x (bf16 [T][H]); w_gate, w_up
    [I][H] and w_down [H][I] bf16; y fp32 [T][H]."""
    T, H = x.shape
    I = w_gate.shape[0]
    _check("strata_moe_shared_expert", lib().strata_moe_shared_expert(
        _p(x), _p(w_gate), _p(w_up), _p(w_down), T, H, I, _p(y), int(accumulate), _p(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream)))


def strata_moe_usage_update(topk_ids, E, usage, stream=None) -> None:
    """usage (int64 tensor [E], read as uint64) += per-expert slot counts of topk_ids [T][k]."""
    T, k = topk_ids.shape
    _check("strata_moe_usage_update", lib().strata_moe_usage_update(
        _p(topk_ids), T, k, E, _p(usage), _stream(stream)))


def strata_moe_usage_rank(usage, order, stream=None) -> None:
    """order (int32 [E]) = experts by usage, most used first, ties to the lower index."""
    E = usage.shape[0]
    _check("strata_moe_usage_rank", lib().strata_moe_usage_rank(_p(usage), E, _p(order),
                                                                _stream(stream)))


def strata_moe_layer_residual(w: Weights, h, logits, k, workspace, eps=1e-6, stream=None) -> None:
    """h (fp32 [T][H]) <- h + MoE(RMSNorm(h))."""
    cw = w.c_struct()
    _check("strata_moe_layer_residual", lib().strata_moe_layer_residual(
        ctypes.byref(cw), _p(h), _p(logits), h.shape[0], k, eps, _p(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream)))


def strata_moe_block(w: Weights, x, k, w_router, w_sgate, w_sup, w_sdown, logits, y,
                     accumulate=False, workspace=None, stream=None) -> None:
    """logits = x W_r^T; y (+)= routed layer(x, logits) + shared expert(x)."""
    cw = w.c_struct()
    _check("strata_moe_block", lib().strata_moe_block(
        ctypes.byref(cw), _p(x), x.shape[0], k, _p(w_router), _p(w_sgate), _p(w_sup), _p(w_sdown),
        w_sgate.shape[0], _p(logits), _p(y), int(bool(accumulate)), _p(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream)))
