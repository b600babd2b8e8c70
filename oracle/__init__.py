"""CPU oracle of the routed-MoE expert layer (TEST INFRASTRUCTURE ONLY).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The GPU library never imports, links or calls it, and the two share no code.

Thin numpy/ctypes marshalling around ``oracle.c`` (plain single-threaded C, fp64, sequential
sums); every function documents the definition it implements there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build_library(verbose: bool = False) -> str:
    """gcc -O2 -ffp-contract=off (no fast-math): every fp64 operation rounds as written."""
    src = os.path.join(_HERE, "oracle.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11",
           src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Weights(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("E", ctypes.c_int32), ("H", ctypes.c_int32),
                ("I", ctypes.c_int32),
                ("gate_codes", ctypes.c_void_p), ("gate_scales", ctypes.c_void_p),
                ("up_codes", ctypes.c_void_p), ("up_scales", ctypes.c_void_p),
                ("down_codes", ctypes.c_void_p), ("down_scales", ctypes.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        src = os.path.join(_HERE, "oracle.c")
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(src) > os.path.getmtime(_LIB_PATH):
            build_library()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = dbl
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = dbl
        L.oracle_code.argtypes = [i32, vp, i32]
        L.oracle_code.restype = i32
        L.oracle_dequant_block.argtypes = [i32, vp, ctypes.c_uint16, vp]
        L.oracle_dequant_block.restype = None
        L.oracle_dequant_matrix.argtypes = [i32, vp, vp, i64, i64, vp]
        L.oracle_dequant_matrix.restype = None
        L.oracle_route.argtypes = [vp, i32, i32, i32, vp, vp]
        L.oracle_route.restype = None
        L.oracle_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
        L.oracle_permute.restype = None
        L.oracle_expert_ffn.argtypes = [ctypes.POINTER(_Weights), i32, vp, vp, vp]
        L.oracle_expert_ffn.restype = None
        L.oracle_combine.argtypes = [vp, vp, i32, i32, i32, vp]
        L.oracle_combine.restype = None
        L.oracle_layer.argtypes = [ctypes.POINTER(_Weights), vp, vp, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_layer.restype = i32
        L.oracle_layer_rows.argtypes = [ctypes.POINTER(_Weights), vp, vp, i32, i32, vp, i32, vp]
        L.oracle_layer_rows.restype = i32
        L.oracle_rmsnorm.argtypes = [vp, i32, i32, dbl, vp]
        L.oracle_router_logits.argtypes = [vp, vp, i32, i32, i32, vp]
        L.oracle_shared_expert.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp]
        L.oracle_rmsnorm.restype = None
        L.oracle_router_logits.restype = None
        L.oracle_usage_update.argtypes = [vp, i32, i32, i32, vp]
        L.oracle_usage_update.restype = None
        L.oracle_usage_rank.argtypes = [vp, i32, vp]
        L.oracle_usage_rank.restype = None
        L.oracle_shared_expert.restype = None
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def _weights(w: dict):
    keep = []
    vals = {}
    for name in ("gate_codes", "up_codes", "down_codes"):
        a, p = _c(w[name], np.uint8)
        keep.append(a)
        vals[name] = p
    for name in ("gate_scales", "up_scales", "down_scales"):
        a, p = _c(w[name], np.uint16)
        keep.append(a)
        vals[name] = p
    s = _Weights(w["fmt"], w["E"], w["H"], w["I"], vals["gate_codes"], vals["gate_scales"],
                 vals["up_codes"], vals["up_scales"], vals["down_codes"], vals["down_scales"])
    return s, keep


def bf16_to_f64(bits: int) -> float:
    return lib().oracle_bf16_to_f64(bits)


def f16_to_f64(bits: int) -> float:
    return lib().oracle_f16_to_f64(bits)


def code(fmt: int, block: np.ndarray, i: int) -> int:
    b, p = _c(block, np.uint8)
    return lib().oracle_code(fmt, p, i)


def dequant_block(fmt: int, block: np.ndarray, scale_bits: int) -> np.ndarray:
    b, p = _c(block, np.uint8)
    out = np.zeros(32, dtype=np.float64)
    lib().oracle_dequant_block(fmt, p, int(scale_bits), out.ctypes.data)
    return out


def dequant_matrix(fmt: int, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes [R][K/32][cb], scales [R][K/32] -> fp64 [R][K]."""
    c, pc = _c(codes, np.uint8)
    s, ps = _c(scales, np.uint16)
    R, nb = s.shape[-2], s.shape[-1]
    out = np.empty((R, nb * 32), dtype=np.float64)
    lib().oracle_dequant_matrix(fmt, pc, ps, R, nb * 32, out.ctypes.data)
    return out


def route(logits: np.ndarray, k: int):
    l, p = _c(logits, np.float32)
    T, E = l.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    lib().oracle_route(p, T, E, k, ids.ctypes.data, w.ctypes.data)
    return ids, w


def permute(ids: np.ndarray, E: int):
    i, p = _c(ids, np.int32)
    T, k = i.shape
    S = T * k
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    sorted_slot = np.empty(S, dtype=np.int32)
    slot_pos = np.empty(S, dtype=np.int32)
    lib().oracle_permute(p, T, E, k, counts.ctypes.data, offsets.ctypes.data,
                         sorted_slot.ctypes.data, slot_pos.ctypes.data)
    return counts, offsets, sorted_slot, slot_pos


def expert_ffn(w: dict, e: int, x_row: np.ndarray):
    s, keep = _weights(w)
    x, px = _c(x_row, np.uint16)
    out = np.empty(w["H"], dtype=np.float64)
    a = np.empty(w["I"], dtype=np.float64)
    lib().oracle_expert_ffn(ctypes.byref(s), e, px, out.ctypes.data, a.ctypes.data)
    return out, a


def combine(expert_out: np.ndarray, weights: np.ndarray, k: int) -> np.ndarray:
    o, po = _c(expert_out, np.float64)
    wt, pw = _c(weights, np.float64)
    S, H = o.shape
    T = S // k
    y = np.empty((T, H), dtype=np.float64)
    lib().oracle_combine(po, pw, T, k, H, y.ctypes.data)
    return y


def layer(w: dict, x: np.ndarray, logits: np.ndarray, k: int, intermediates: bool = False):
    """y fp64 [T][H]; with intermediates also ids, weights, expert_out [T*k][H], a [T*k][I]."""
    s, keep = _weights(w)
    xx, px = _c(x, np.uint16)
    ll, pl = _c(logits, np.float32)
    T = xx.shape[0]
    y = np.empty((T, w["H"]), dtype=np.float64)
    ids = np.empty((T, k), dtype=np.int32)
    rw = np.empty((T, k), dtype=np.float64)
    out = np.empty((T * k, w["H"]), dtype=np.float64) if intermediates else None
    a = np.empty((T * k, w["I"]), dtype=np.float64) if intermediates else None
    rc = lib().oracle_layer(ctypes.byref(s), px, pl, T, k, y.ctypes.data, ids.ctypes.data,
                            rw.ctypes.data, out.ctypes.data if intermediates else None,
                            a.ctypes.data if intermediates else None)
    if rc != 0:
        raise MemoryError("oracle_layer: out of memory")
    if intermediates:
        return y, ids, rw, out, a
    return y


def layer_rows(w: dict, x: np.ndarray, logits: np.ndarray, k: int, rows) -> np.ndarray:
    """Layer output rows for the listed token indices only, fp64 [len(rows)][H]."""
    s, keep = _weights(w)
    xx, px = _c(x, np.uint16)
    ll, pl = _c(logits, np.float32)
    r, pr = _c(np.asarray(rows), np.int32)
    y = np.empty((r.size, w["H"]), dtype=np.float64)
    rc = lib().oracle_layer_rows(ctypes.byref(s), px, pl, xx.shape[0], k, pr, r.size, y.ctypes.data)
    if rc != 0:
        raise MemoryError("oracle_layer_rows: out of memory")
    return y


def rmsnorm(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    hh, ph = _c(h, np.float32)
    T, H = hh.shape
    x = np.empty((T, H), dtype=np.uint16)
    lib().oracle_rmsnorm(ph, T, H, eps, x.ctypes.data)
    return x


def router_logits(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    """logits fp64 [T][E] = x W_r^T (x bf16 bits [T][H], W_r bf16 bits [E][H])."""
    xx, px = _c(x, np.uint16)
    ww, pw = _c(wr, np.uint16)
    T, H = xx.shape
    E = ww.shape[0]
    out = np.empty((T, E), dtype=np.float64)
    lib().oracle_router_logits(px, pw, T, H, E, out.ctypes.data)
    return out


def shared_expert(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """Shared expert output fp64 [T][H] (all arguments bf16 bits: x [T][H], W_sg and W_su
    [Is][H], W_sd [H][Is])."""
    xx, px = _c(x, np.uint16)
    g, pg = _c(wg, np.uint16)
    u, pu = _c(wu, np.uint16)
    d, pd = _c(wd, np.uint16)
    T, H = xx.shape
    Is = g.shape[0]
    out = np.empty((T, H), dtype=np.float64)
    lib().oracle_shared_expert(px, pg, pu, pd, T, H, Is, out.ctypes.data)
    return out


def usage_update(ids: np.ndarray, E: int, usage: np.ndarray | None = None) -> np.ndarray:
    """usage uint64 [E] += number of slots of ids (int32 [T][k]) routed to each expert."""
    ii, pi = _c(ids, np.int32)
    T, k = ii.shape
    u = np.zeros(E, dtype=np.uint64) if usage is None else np.ascontiguousarray(usage, dtype=np.uint64).copy()
    lib().oracle_usage_update(pi, T, k, E, u.ctypes.data)
    return u


def usage_rank(usage: np.ndarray) -> np.ndarray:
    """Experts by usage, most used first, ties to the lower index (int32 [E])."""
    u, pu = _c(usage, np.uint64)
    order = np.empty(u.shape[0], dtype=np.int32)
    lib().oracle_usage_rank(pu, u.shape[0], order.ctypes.data)
    return order
