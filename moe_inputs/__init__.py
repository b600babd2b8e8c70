"""Seeded synthetic inputs for the routed-MoE expert layer.

The one input generator that both the CPU oracle's tests and the GPU path's tests and benchmark
use: a counter-based Philox4x32-10 stream per tensor (see ``gen.c``), so a tensor is the same
bytes no matter which side asks for it.  Nothing here computes any part of the layer.

Workload shapes (the pages fix 512 experts per layer, 10 active per token and 48 layers:
"Strata vs Llama.cpp vs vLLM", transcript at 08:23; "Local AI Is Now 6x Faster on Your PC", key
technological idea.  They describe multi-token-prediction verification of up to 3 drafted
tokens, "Strata - the details", How it works, and prefill chunks of up to 8,192 tokens,
"Strata vs Llama.cpp vs vLLM", transcript at 10:30):

* ``tiny``     T=16,   H=256,  E=64,  k=4,  I=128, Q2   (oracle-sized)
* ``decode``   T=4,    H=3072, E=512, k=10, I=768, Q2   (1 token + 3 drafts)
* ``prefill``  T=8192, H=3072, E=512, k=10, I=768, Q2   (one prefill chunk)
* ``skewed``   T=2048, H=3072, E=512, k=10, I=768, Q3, Zipf(1.1)-biased router logits
* ``stack``    48 layers of the prefill / decode shapes, h <- h + MoE(RMSNorm(h))

Distributions: x = bf16(N(0,1)); logits = fp32(N(0,1)) (+ 2 ln p_rank for ``skewed``, with
p_r proportional to r^-1.1 over a seeded ranking of the experts; the normalising constant of p
is dropped because adding one constant to a token's logits changes neither its top-k nor its
weights); codes uniform (uniform random bytes are uniform packed codes in both formats);
scales fp16(0.02 |N(0,1)|).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_inputs.so")
_lib = None

# tensor tags of the stream id: stream = (layer << 8) | tag
TAG_X, TAG_LOGITS, TAG_GATE_CODES, TAG_UP_CODES, TAG_DOWN_CODES = 1, 2, 3, 4, 5
TAG_GATE_SCALES, TAG_UP_SCALES, TAG_DOWN_SCALES, TAG_ZIPF_RANK = 6, 7, 8, 9
TAG_ROUTER_W, TAG_SHARED_GATE, TAG_SHARED_UP, TAG_SHARED_DOWN = 10, 11, 12, 13

Q2, Q3 = 2, 3
CODE_BYTES = {Q2: 8, Q3: 12}


def build_library(verbose: bool = False) -> str:
    """Compile gen.c into libmoe_inputs.so (host code, gcc, OpenMP)."""
    import subprocess

    src = os.path.join(_HERE, "gen.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_library()
        L = ctypes.CDLL(_LIB_PATH)
        u64, u32, i64, i32, vp, dbl = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_double)
        L.mi_philox4x32_10.argtypes = [vp, vp, vp]
        L.mi_fill_bytes.argtypes = [u64, u32, vp, u64]
        L.mi_fill_normal_f32.argtypes = [u64, u32, dbl, vp, i64, vp, u64]
        L.mi_fill_normal_bf16.argtypes = [u64, u32, vp, u64]
        L.mi_fill_abs_normal_f16.argtypes = [u64, u32, dbl, vp, u64]
        L.mi_permutation.argtypes = [u64, u32, vp, i32]
        L.mi_f32_to_bf16_array.argtypes = [vp, vp, u64]
        L.mi_f32_to_f16_array.argtypes = [vp, vp, u64]
        for f in (L.mi_philox4x32_10, L.mi_fill_bytes, L.mi_fill_normal_f32, L.mi_fill_normal_bf16,
                  L.mi_fill_abs_normal_f16, L.mi_permutation, L.mi_f32_to_bf16_array,
                  L.mi_f32_to_f16_array):
            f.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().mi_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def stream_id(layer: int, tag: int) -> int:
    return ((layer & 0xFFFFFF) << 8) | tag


def random_bytes(seed: int, stream: int, n: int, out: np.ndarray | None = None) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8) if out is None else out
    assert out.dtype == np.uint8 and out.size == n
    lib().mi_fill_bytes(seed, stream, _ptr(out), n)
    return out


def normal_f32(seed: int, stream: int, n: int, scale: float = 1.0,
               bias: np.ndarray | None = None) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if bias is not None:
        b = np.ascontiguousarray(bias, dtype=np.float64)
        lib().mi_fill_normal_f32(seed, stream, scale, _ptr(b), b.size, _ptr(out), n)
    else:
        lib().mi_fill_normal_f32(seed, stream, scale, None, 1, _ptr(out), n)
    return out


def normal_bf16(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().mi_fill_normal_bf16(seed, stream, _ptr(out), n)
    return out


def abs_normal_f16(seed: int, stream: int, n: int, mult: float) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().mi_fill_abs_normal_f16(seed, stream, mult, _ptr(out), n)
    return out


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    lib().mi_permutation(seed, stream, _ptr(out), n)
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().mi_f32_to_bf16_array(_ptr(a), _ptr(out), a.size)
    return out


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().mi_f32_to_f16_array(_ptr(a), _ptr(out), a.size)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Shape:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    fmt: int = Q2
    zipf: bool = False
    layers: int = 1

    @property
    def code_bytes(self) -> int:
        return CODE_BYTES[self.fmt]

    @property
    def expert_bytes(self) -> int:
        """Packed bytes of one expert (codes + scales of gate, up and down)."""
        per_block = self.code_bytes + 2
        return 3 * self.I * (self.H // 32) * per_block

    @property
    def layer_bytes(self) -> int:
        return self.E * self.expert_bytes


TINY = Shape("tiny", T=16, H=256, E=64, k=4, I=128)
DECODE = Shape("decode", T=4, H=3072, E=512, k=10, I=768)
PREFILL = Shape("prefill", T=8192, H=3072, E=512, k=10, I=768)
SKEWED = Shape("skewed", T=2048, H=3072, E=512, k=10, I=768, fmt=Q3, zipf=True)
STACK_PREFILL = replace(PREFILL, name="stack_prefill", layers=48)
STACK_DECODE = replace(DECODE, name="stack_decode", layers=48)
# the pruned coder variant keeps 256 of a layer's 512 experts
PRUNED_DECODE = replace(DECODE, name="pruned_decode", E=256)
PRUNED_PREFILL = replace(PREFILL, name="pruned_prefill", E=256)
# mid-size chunks at the full dims (prompt-lookup verify, short prefill chunks): ~5 and ~20 rows
# per expert
MID256 = replace(PREFILL, name="mid256", T=256)
MID1024 = replace(PREFILL, name="mid1024", T=1024)
SHAPES = {s.name: s for s in (TINY, DECODE, PREFILL, SKEWED, STACK_PREFILL, STACK_DECODE,
                              PRUNED_DECODE, PRUNED_PREFILL, MID256, MID1024)}


def zipf_bias(seed: int, layer: int, E: int, s: float = 1.1, strength: float = 2.0) -> np.ndarray:
    """strength * ln(r^-s) for each expert, r = its rank in a seeded permutation (1-based)."""
    perm = permutation(seed, stream_id(layer, TAG_ZIPF_RANK), E)  # perm[r-1] = expert of rank r
    rank = np.empty(E, dtype=np.float64)
    rank[perm] = np.arange(1, E + 1, dtype=np.float64)
    return strength * (-s) * np.log(rank)


def make_weights(shape: Shape, seed: int = 0, layer: int = 0) -> dict:
    """Packed expert weights of one layer as numpy arrays (SoA, expert-major)."""
    E, H, I, cb = shape.E, shape.H, shape.I, shape.code_bytes
    nb_h, nb_i = H // 32, I // 32
    w = {"fmt": shape.fmt, "E": E, "H": H, "I": I}
    for name, tag, rows, nb in (("gate", TAG_GATE_CODES, I, nb_h), ("up", TAG_UP_CODES, I, nb_h),
                                ("down", TAG_DOWN_CODES, H, nb_i)):
        n = E * rows * nb * cb
        w[name + "_codes"] = random_bytes(seed, stream_id(layer, tag), n).reshape(E, rows, nb, cb)
    for name, tag, rows, nb in (("gate", TAG_GATE_SCALES, I, nb_h), ("up", TAG_UP_SCALES, I, nb_h),
                                ("down", TAG_DOWN_SCALES, H, nb_i)):
        n = E * rows * nb
        w[name + "_scales"] = abs_normal_f16(seed, stream_id(layer, tag), n, 0.02).reshape(E, rows, nb)
    return w


def make_x(shape: Shape, seed: int = 0, layer: int = 0, T: int | None = None) -> np.ndarray:
    T = shape.T if T is None else T
    return normal_bf16(seed, stream_id(layer, TAG_X), T * shape.H).reshape(T, shape.H)


def make_logits(shape: Shape, seed: int = 0, layer: int = 0, T: int | None = None) -> np.ndarray:
    T = shape.T if T is None else T
    bias = zipf_bias(seed, layer, shape.E) if shape.zipf else None
    return normal_f32(seed, stream_id(layer, TAG_LOGITS), T * shape.E, bias=bias).reshape(T, shape.E)


def dense_bf16(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    """bf16 bits [rows][cols] of N(0, 1/cols): a dense layer that keeps unit-variance inputs at
    unit variance."""
    return f32_to_bf16_bits(normal_f32(seed, stream, rows * cols, scale=cols ** -0.5)).reshape(rows, cols)


def make_router(shape: Shape, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Router projection W_r, bf16 bits [E][H] (logits of unit-variance x are ~N(0,1))."""
    return dense_bf16(seed, stream_id(layer, TAG_ROUTER_W), shape.E, shape.H)


def make_shared(shape: Shape, seed: int = 0, layer: int = 0) -> dict:
    """Shared expert, bf16 bits: W_sg, W_su [I][H] and W_sd [H][I] (intermediate size I, the
    same as a routed expert's)."""
    H, I = shape.H, shape.I
    return {"H": H, "I": I,
            "gate": dense_bf16(seed, stream_id(layer, TAG_SHARED_GATE), I, H),
            "up": dense_bf16(seed, stream_id(layer, TAG_SHARED_UP), I, H),
            "down": dense_bf16(seed, stream_id(layer, TAG_SHARED_DOWN), H, I)}


def make_h0(shape: Shape, seed: int = 0, T: int | None = None) -> np.ndarray:
    """Initial residual stream of a layer stack: the layer-0 activations widened to fp32."""
    return bf16_bits_to_f32(make_x(shape, seed, 0, T))
