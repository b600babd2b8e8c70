"""GPU parity of the expert usage statistics and of the pruned (E = 256) layer variant.

Usage counts and the hotness order are integer results: bit-exact against the oracle, over
several accumulating calls, with ties, ignored out-of-range ids and 64-bit counts.  The pruned
variant (256 experts per layer, the pages' coder model) runs the same kernels at E = 256: full
decode rows and sampled prefill rows against the oracle, routing and permutation bit-exact.
"""
import numpy as np
import pytest
import torch

import bit_expert_ffn_fp32_amd as sm
import moe_inputs as mi
import oracle
from gpu_helpers import TOL_REL_L2, Layer, dev, rel_l2_rows, to_dev

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def gpu_usage_update(ids_np, E, usage):
    sm.strata_moe_usage_update(to_dev(ids_np.astype(np.int32)), E, usage)


@pytest.mark.parametrize("E,k,Ts", [(512, 10, (8192, 4, 2048)), (64, 4, (16, 1)), (1, 1, (5,)),
                                    (1024, 16, (333,))])
def test_usage_update_accumulates(E, k, Ts):
    log(f"usage E={E} k={k} T={Ts}")
    usage = torch.zeros(E, dtype=torch.int64, device=dev())
    ref = None
    for i, T in enumerate(Ts):
        logits = mi.normal_f32(i, 700 + E, T * E).reshape(T, E)
        ids, _ = oracle.route(logits, k)
        gpu_usage_update(ids, E, usage)
        ref = oracle.usage_update(ids, E, ref)
    torch.cuda.synchronize()
    got = usage.cpu().numpy().view(np.uint64)
    assert np.array_equal(got, ref)
    assert int(got.sum()) == sum(Ts) * k


def test_usage_ignores_out_of_range_ids():
    E = 8
    ids = np.array([[0, 7, -1], [8, 3, 3], [1 << 30, 7, 0]], dtype=np.int32)
    usage = torch.zeros(E, dtype=torch.int64, device=dev())
    gpu_usage_update(ids, E, usage)
    torch.cuda.synchronize()
    assert np.array_equal(usage.cpu().numpy().view(np.uint64), oracle.usage_update(ids, E))
    assert usage.cpu().tolist() == [2, 0, 0, 2, 0, 0, 0, 2]


@pytest.mark.parametrize("E,kind", [(1, "rand"), (7, "rand"), (256, "rand"), (512, "ties"),
                                    (1024, "rand"), (1024, "zeros"), (300, "big")])
def test_usage_rank(E, kind):
    rng = np.random.default_rng(E)
    if kind == "rand":
        u = rng.integers(0, 1 << 20, size=E).astype(np.uint64)
    elif kind == "ties":
        u = rng.integers(0, 4, size=E).astype(np.uint64)
    elif kind == "zeros":
        u = np.zeros(E, dtype=np.uint64)
    else:
        u = (np.uint64(1) << np.uint64(40)) + rng.integers(0, 3, size=E).astype(np.uint64)
    order = torch.full((E,), -1, dtype=torch.int32, device=dev())
    sm.strata_moe_usage_rank(to_dev(u.view(np.int64)), order)
    torch.cuda.synchronize()
    assert np.array_equal(order.cpu().numpy(), oracle.usage_rank(u))


def test_usage_of_a_prefill_layer_matches_its_permutation():
    """Counts accumulated from the layer's own top-k output equal its permutation counts."""
    s = mi.PRUNED_PREFILL
    log("usage from a pruned prefill layer")
    L = Layer(s)
    S = s.T * s.k
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device=dev())
    counts = torch.empty(s.E, dtype=torch.int32, device=dev())
    y = torch.empty((s.T, s.H), dtype=torch.float32, device=dev())
    sm.strata_moe_layer(L.w, L.x, L.logits, s.k, y, topk_ids=ids, counts=counts,
                        offsets=torch.empty(s.E + 1, dtype=torch.int32, device=dev()),
                        sorted_slot=torch.empty(S, dtype=torch.int32, device=dev()),
                        workspace=L.workspace())
    usage = torch.zeros(s.E, dtype=torch.int64, device=dev())
    sm.strata_moe_usage_update(ids, s.E, usage)
    order = torch.empty(s.E, dtype=torch.int32, device=dev())
    sm.strata_moe_usage_rank(usage, order)
    torch.cuda.synchronize()
    u = usage.cpu().numpy().view(np.uint64)
    assert np.array_equal(u.astype(np.int64), counts.cpu().numpy().astype(np.int64))
    ids_ref, _ = oracle.route(L.l_np, s.k)
    assert np.array_equal(u, oracle.usage_update(ids_ref, s.E))
    assert np.array_equal(order.cpu().numpy(), oracle.usage_rank(u))


def test_pruned_decode_full_size():
    s = mi.PRUNED_DECODE
    log("pruned decode full size")
    L = Layer(s)
    y = torch.empty((s.T, s.H), dtype=torch.float32, device=dev())
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device=dev())
    sm.strata_moe_layer(L.w, L.x, L.logits, s.k, y, topk_ids=ids, workspace=L.workspace())
    torch.cuda.synchronize()
    y_ref, ids_ref, *_ = oracle.layer(L.w_np, L.x_np, L.l_np, s.k, intermediates=True)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert rel_l2_rows(y.cpu().numpy(), y_ref).max() <= TOL_REL_L2


def test_pruned_prefill_sampled_rows():
    s = mi.PRUNED_PREFILL
    log("pruned prefill full size")
    L = Layer(s)
    y = torch.empty((s.T, s.H), dtype=torch.float32, device=dev())
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device=dev())
    sm.strata_moe_layer(L.w, L.x, L.logits, s.k, y, topk_ids=ids, workspace=L.workspace())
    torch.cuda.synchronize()
    ids_ref, _ = oracle.route(L.l_np, s.k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    rows = np.random.default_rng(256).choice(s.T, size=10, replace=False)
    y_ref = oracle.layer_rows(L.w_np, L.x_np, L.l_np, s.k, rows)
    assert rel_l2_rows(y.cpu().numpy()[rows], y_ref).max() <= TOL_REL_L2
