"""The C ABI on the host: the library loads, exports every entry point the header declares, and
rejects bad arguments with the documented status before touching the GPU (no compute call is
made here: every call below fails validation or is the T = 0 no-op)."""
import ctypes
import os
import re
import subprocess

import pytest

import bit_expert_ffn_fp32_amd as sm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "strata_moe.h")

OK, INVAL, UNSUP, WS = 0, 1, 2, 3
A = 0x10000      # a 16-byte aligned stand-in address (never dereferenced: validation fails first)
MIS = 0x10004    # misaligned stand-in


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sm.LIB_PATH):
        pytest.skip("libstrata_moe.so not built")
    return sm.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(strata_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert "strata_moe_layer" in names and len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert sorted(sm.EXPORTS) == names


def weights(fmt=2, E=512, H=3072, I=768, ptr=A, stats=A):
    return sm.CWeights(fmt, E, H, I, ptr, ptr, ptr, ptr, ptr, ptr, stats)


FIELDS = ["fmt", "num_experts", "hidden", "inter", "gate_codes", "up_codes", "gate_scales",
          "up_scales", "down_codes", "down_scales", "stats"]


def test_weights_struct_layout(tmp_path):
    """The header's struct, compiled by the host C compiler, has the documented field order and
    offsets, and the binding's ctypes mirror matches it field for field."""
    src = tmp_path / "offsets.c"
    body = ", ".join(f"offsetof(strata_moe_weights, {f})" for f in FIELDS)
    fmt = " ".join(["%zu"] * (len(FIELDS) + 2))
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "strata_moe.h"\n'
                   f'int main(void) {{ printf("{fmt}\\n", {body}, sizeof(strata_moe_weights), '
                   'sizeof(strata_moe_expert_stats)); return 0; }\n')
    exe = tmp_path / "offsets"
    subprocess.check_call(["gcc", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                           "-I" + os.path.join(ROOT, "include"), str(src), "-o", str(exe)])
    got = [int(v) for v in subprocess.check_output([str(exe)], text=True).split()]
    assert got[:len(FIELDS)] == [0, 4, 8, 12, 16, 24, 32, 40, 48, 56, 64]
    assert got[len(FIELDS):] == [72, 16]
    assert [getattr(sm.CWeights, f).offset for f in FIELDS] == got[:len(FIELDS)]
    assert ctypes.sizeof(sm.CWeights) == 72 and ctypes.sizeof(sm.CExpertStats) == 16


def test_status_strings(L):
    for st, text in [(0, b"ok"), (1, b"invalid argument"), (2, b"unsupported shape"),
                     (3, b"workspace too small"), (4, b"HIP launch error"), (99, b"unknown status")]:
        assert L.strata_status_string(st) == text


def test_route_validation(L):
    assert L.strata_moe_route(A, 4, 8, 9, A, A, None) == INVAL        # k > E
    assert L.strata_moe_route(A, 4, 512, 0, A, A, None) == INVAL      # k = 0
    assert L.strata_moe_route(A, -1, 512, 10, A, A, None) == INVAL    # T < 0
    assert L.strata_moe_route(A, 4, 2048, 10, A, A, None) == UNSUP    # E > 1024
    assert L.strata_moe_route(A, 4, 512, 17, A, A, None) == UNSUP     # k > 16
    assert L.strata_moe_route(None, 4, 512, 10, A, A, None) == INVAL  # null
    assert L.strata_moe_route(MIS, 4, 512, 10, A, A, None) == INVAL   # misaligned
    assert L.strata_moe_route(None, 0, 512, 10, None, None, None) == OK  # T = 0: no-op


def test_permute_validation(L):
    need = L.strata_moe_permute_workspace_bytes(8192, 512, 10)
    assert need >= 2 * 80 * 512 * 4
    assert L.strata_moe_permute(A, 8192, 512, 10, A, A, A, A, A, need - 1, None) == WS
    assert L.strata_moe_permute(A, 8192, 512, 10, A, A, None, A, A, need, None) == INVAL
    assert L.strata_moe_permute(A, 8192, 512, 10, A, MIS, A, A, A, need, None) == INVAL
    assert L.strata_moe_permute(A, 10, 4, 5, A, A, A, A, A, need, None) == INVAL


def test_weights_validation(L):
    ws = L.strata_moe_workspace_bytes(8192, 512, 10, 3072, 768)
    call = lambda w, T=8192, k=10, wsb=ws: L.strata_moe_layer(
        ctypes.byref(w), A, A, T, k, A, 0, None, None, None, None, None, A, wsb, None)
    assert call(weights(fmt=4)) == INVAL
    assert call(weights(H=3000)) == INVAL          # not a multiple of 32
    assert call(weights(H=3072 + 128)) == UNSUP    # multiple of 32 but not of 256
    assert call(weights(I=800)) == UNSUP           # not a multiple of 128
    assert call(weights(E=2000)) == UNSUP
    assert call(weights(ptr=MIS)) == INVAL
    assert call(weights(ptr=0)) == INVAL
    assert call(weights(), k=0) == INVAL
    assert call(weights(), wsb=ws - 1) == WS
    assert L.strata_moe_layer(None, A, A, 16, 4, A, 0, None, None, None, None, None, A, ws, None) == INVAL
    # the prefill path needs the weights' range statistics (aligned)
    assert call(weights(stats=0)) == INVAL
    assert call(weights(stats=MIS)) == INVAL
    assert L.strata_moe_expert_ffn(ctypes.byref(weights(stats=0)), A, 8192, 10, A, A, A, A, ws,
                                   None) == INVAL
    # the decode paths also produce the permutation on request: the workspace covers it
    w4 = L.strata_moe_workspace_bytes(4, 512, 10, 3072, 768)
    w48 = L.strata_moe_workspace_bytes(48, 512, 10, 3072, 768)
    assert w4 >= 3 * 40 * 4 + 2 * 512 * 4 and w48 >= 3 * 480 * 4 + 2 * 512 * 4
    assert L.strata_moe_layer(ctypes.byref(weights()), A, A, 4, 10, A, 0, None, None, A, None, None,
                              A, w4 - 1, None) == WS
    assert L.strata_moe_decode(ctypes.byref(weights()), A, A, 9, 10, A, 0, None, None, A, ws,
                               None) == UNSUP
    assert L.strata_moe_expert_ffn(ctypes.byref(weights()), A, 8192, 10, A, A, A, A, ws - 1,
                                   None) == WS


def test_layer_residual_validation(L):
    ws = L.strata_moe_residual_workspace_bytes(4, 512, 10, 3072, 768)
    assert ws >= L.strata_moe_workspace_bytes(4, 512, 10, 3072, 768) + 4 * 3072 * 2
    assert L.strata_moe_residual_workspace_bytes(-1, 512, 10, 3072, 768) == 0
    call = lambda w, h=A, T=4, k=10, eps=1e-6, wsb=ws: L.strata_moe_layer_residual(
        ctypes.byref(w), h, A, T, k, ctypes.c_float(eps), A, wsb, None)
    assert call(weights(), wsb=ws - 1) == WS
    assert call(weights(), eps=-1.0) == INVAL
    assert call(weights(), eps=float("nan")) == INVAL
    assert call(weights(), h=MIS) == INVAL
    assert call(weights(), h=None) == INVAL
    assert call(weights(E=8), k=9) == INVAL
    assert call(weights(fmt=4)) == INVAL
    assert call(weights(), T=0, h=None) == OK       # T = 0: no-op


def test_block_validation(L):
    ws = L.strata_moe_block_workspace_bytes(4, 512, 10, 3072, 768, 768)
    assert ws >= L.strata_moe_workspace_bytes(4, 512, 10, 3072, 768) + 4 * 768 * 2
    assert L.strata_moe_block_workspace_bytes(4, 512, 10, 3072, 768, 0) == 0
    call = lambda w, x=A, T=4, k=10, Is=768, lg=A, wsb=ws: L.strata_moe_block(
        ctypes.byref(w), x, T, k, A, A, A, A, Is, lg, A, 0, A, wsb, None)
    assert call(weights(), wsb=ws - 1) == WS
    assert call(weights(), Is=0) == INVAL
    assert call(weights(), Is=96) == UNSUP          # not a multiple of 64
    assert call(weights(), x=MIS) == INVAL
    assert call(weights(), lg=None) == INVAL
    assert call(weights(fmt=4)) == INVAL
    assert call(weights(E=8), k=9) == INVAL
    assert call(weights(), T=0, x=None, lg=None) == OK   # T = 0: no-op


def test_combine_and_rmsnorm_validation(L):
    assert L.strata_moe_combine(A, A, 4, 10, 3072, None, 0, None) == INVAL
    assert L.strata_moe_combine(A, A, 4, 10, 3071, A, 0, None) == UNSUP
    assert L.strata_moe_combine(A, A, 0, 10, 3072, A, 0, None) == OK
    assert L.strata_moe_rmsnorm(A, 4, 3072, ctypes.c_float(-1.0), A, None) == INVAL
    assert L.strata_moe_rmsnorm(A, 4, 3071, ctypes.c_float(1e-6), A, None) == UNSUP
    assert L.strata_moe_rmsnorm(MIS, 4, 3072, ctypes.c_float(1e-6), A, None) == INVAL


def test_weight_stats_validation(L):
    assert L.strata_moe_weight_stats(ctypes.byref(weights()), None, None) == INVAL
    assert L.strata_moe_weight_stats(ctypes.byref(weights()), MIS, None) == INVAL
    assert L.strata_moe_weight_stats(ctypes.byref(weights(fmt=4)), A, None) == INVAL
    assert L.strata_moe_weight_stats(ctypes.byref(weights(I=800)), A, None) == UNSUP
    assert L.strata_moe_weight_stats(ctypes.byref(weights(ptr=MIS)), A, None) == INVAL
    assert L.strata_moe_weight_stats(None, A, None) == INVAL


def test_pack_matrix_validation(L):
    B = A + (1 << 30)  # a second fake buffer, far from A
    assert L.strata_moe_pack_matrix(4, 1, 64, 64, A, A + 4096, B, B + 4096, None) == INVAL
    assert L.strata_moe_pack_matrix(2, 1, 66, 64, A, A + 4096, B, B + 4096, None) == UNSUP
    assert L.strata_moe_pack_matrix(2, 1, 64, 96, A, A + 4096, B, B + 4096, None) == UNSUP
    assert L.strata_moe_pack_matrix(2, 0, 64, 64, A, A + 4096, B, B + 4096, None) == INVAL
    assert L.strata_moe_pack_matrix(2, 1, 64, 64, MIS, A + 4096, B, B + 4096, None) == INVAL
    assert L.strata_moe_pack_matrix(2, 1, 64, 64, A, A + 4096, None, B + 4096, None) == INVAL
    # 64 x 64 Q2 is 1 KB of codes and 256 B of scales: overlapping source and destination
    assert L.strata_moe_pack_matrix(2, 1, 64, 64, A, A + 4096, A + 512, B + 4096, None) == INVAL
    assert L.strata_moe_pack_matrix(2, 1, 64, 64, A, A + 4096, B, A + 4096 + 128, None) == INVAL
    assert L.strata_moe_pack_matrix(3, 1, 64, 64, A, A + 4096, A + 1024, B + 4096, None) == INVAL


def test_router_and_shared_validation(L):
    assert L.strata_moe_router_logits(A, A, -1, 3072, 512, A, None) == INVAL
    assert L.strata_moe_router_logits(A, A, 4, 3072, 0, A, None) == INVAL
    assert L.strata_moe_router_logits(A, A, 4, 3000, 512, A, None) == UNSUP    # H % 64
    assert L.strata_moe_router_logits(MIS, A, 4, 3072, 512, A, None) == INVAL
    assert L.strata_moe_router_logits(A, None, 4, 3072, 512, A, None) == INVAL
    assert L.strata_moe_router_logits(None, None, 0, 3072, 512, None, None) == OK  # T = 0
    ws = L.strata_moe_shared_workspace_bytes(8192, 768)
    assert ws >= 8192 * 768 * 2 and L.strata_moe_shared_workspace_bytes(-1, 768) == 0
    call = lambda T=8192, H=3072, I=768, y=A, wsb=ws, x=A: L.strata_moe_shared_expert(
        x, A, A, A, T, H, I, y, 0, A, wsb, None)
    assert call(H=3000) == UNSUP
    assert call(I=800) == UNSUP
    assert call(I=0) == INVAL
    assert call(y=None) == INVAL
    assert call(x=MIS) == INVAL
    assert call(wsb=ws - 1) == WS
    assert call(T=0, y=None, x=None) == OK


def test_usage_validation(L):
    assert L.strata_moe_usage_update(A, 4, 10, 0, A, None) == INVAL
    assert L.strata_moe_usage_update(A, 4, 0, 512, A, None) == INVAL
    assert L.strata_moe_usage_update(A, 4, 10, 2048, A, None) == UNSUP
    assert L.strata_moe_usage_update(None, 4, 10, 512, A, None) == INVAL
    assert L.strata_moe_usage_update(A, 4, 10, 512, MIS, None) == INVAL
    assert L.strata_moe_usage_update(None, 0, 10, 512, None, None) == OK
    assert L.strata_moe_usage_rank(A, 0, A, None) == INVAL
    assert L.strata_moe_usage_rank(A, 1025, A, None) == UNSUP
    assert L.strata_moe_usage_rank(None, 512, A, None) == INVAL
    assert L.strata_moe_usage_rank(A, 512, MIS, None) == INVAL


def test_workspace_sizes(L):
    assert L.strata_moe_workspace_bytes(-1, 512, 10, 3072, 768) == 0
    # shapes the compute calls reject get no size (E above 1024, k above 16 or E, T * k too big)
    assert L.strata_moe_workspace_bytes(4, 2048, 10, 3072, 768) == 0
    assert L.strata_moe_workspace_bytes(4, 2**31 - 1, 10, 3072, 768) == 0
    assert L.strata_moe_workspace_bytes(4, 512, 17, 3072, 768) == 0
    assert L.strata_moe_permute_workspace_bytes(4, 8, 9) == 0
    assert L.strata_moe_permute_workspace_bytes(2**28, 512, 16) == 0
    assert L.strata_moe_residual_workspace_bytes(4, 2048, 10, 3072, 768) == 0
    assert L.strata_moe_block_workspace_bytes(4, 2048, 10, 3072, 768, 768) == 0
    assert L.strata_moe_permute_workspace_bytes(4, 1024, 16) > 0
    small = L.strata_moe_workspace_bytes(16, 64, 4, 256, 128)
    big = L.strata_moe_workspace_bytes(8192, 512, 10, 3072, 768)
    assert 0 < small < big
    # prefill: intermediate a (S x I fp16) and expert outputs (S x H bf16) dominate
    S = 8192 * 10
    assert big >= S * 768 * 2 + S * 3072 * 2 + 8192 * 3072 * 2


def test_python_binding_raises():
    if not os.path.exists(sm.LIB_PATH):
        pytest.skip("libstrata_moe.so not built")
    with pytest.raises(sm.StrataError) as ei:
        sm._check("strata_moe_route", INVAL)
    assert ei.value.status == INVAL
