"""GPU parity: every stage of the HIP path against the CPU oracle, through the C ABI.

Bars: routing ids, counts, offsets and the permutation bit-exact; router weights within 1e-6
relative; expert outputs and layer outputs within 5e-3 per-row relative L2 against the fp64
oracle.  Inputs come from the seeded generator shared with the oracle's tests.
"""
import numpy as np
import pytest
import torch

import bit_expert_ffn_fp32_amd as sm
import moe_inputs as mi
import oracle
from gpu_helpers import TOL_REL_L2, Layer, bf16_tensor_to_f64, dev, rel_l2_rows, to_dev

pytestmark = pytest.mark.gpu


def shape(name="s", T=16, H=256, E=64, k=4, I=128, fmt=2, zipf=False):
    return mi.Shape(name, T=T, H=H, E=E, k=k, I=I, fmt=fmt, zipf=zipf)


def log(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------------------------------------
# Route


def gpu_route(logits_np, k):
    T, E = logits_np.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=dev())
    w = torch.empty((T, k), dtype=torch.float32, device=dev())
    sm.strata_moe_route(to_dev(logits_np), k, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("T,E,k,kind", [
    (16, 64, 4, "normal"), (4, 512, 10, "normal"), (8192, 512, 10, "normal"),
    (2048, 512, 10, "zipf"), (333, 1024, 16, "normal"), (50, 5, 5, "normal"), (7, 1, 1, "normal"),
    (257, 512, 10, "ties"), (64, 64, 8, "ties2"), (31, 200, 3, "signed_zero"),
    (9, 1024, 16, "crowded"), (12, 512, 10, "crowded")])
def test_route_bit_exact(T, E, k, kind):
    log(f"route T={T} E={E} k={k} {kind}")
    rng = np.random.default_rng(T * 7 + E)
    if kind == "normal":
        logits = mi.normal_f32(0, 900 + E, T * E).reshape(T, E)
    elif kind == "zipf":
        logits = mi.make_logits(mi.SKEWED, T=T)
    elif kind == "ties":
        logits = (rng.integers(0, 6, size=(T, E)) * 0.25).astype(np.float32)
    elif kind == "ties2":
        logits = np.zeros((T, E), dtype=np.float32)
        logits[::2, 5:] = 1.0
    elif kind == "crowded":
        # lanes 0..k-2 of the selecting wave (experts e with e % 64 < k - 1) hold only large
        # logits and lane k-1 one: more than 64 entries reach the k-th largest lane head, the case
        # the selection hands to its round-by-round arg-max
        logits = mi.normal_f32(0, 950 + E, T * E).reshape(T, E)
        lane = np.arange(E) % 64
        logits[:, lane < k - 1] += 100.0
        logits[:, k - 1] += 50.0
    else:
        logits = np.where(rng.random((T, E)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        logits[:, 17] = -1.0
    ids, w = gpu_route(logits, k)
    rids, rw = oracle.route(logits, k)
    assert np.array_equal(ids, rids)
    np.testing.assert_allclose(w, rw, rtol=1e-6, atol=0)
    assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1) < 1e-6)


# ---------------------------------------------------------------------------------------------
# Permute


def gpu_permute(ids_np, E):
    T, k = ids_np.shape
    S = T * k
    ids = to_dev(ids_np.astype(np.int32))
    counts = torch.empty(E, dtype=torch.int32, device=dev())
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev())
    ss = torch.empty(S, dtype=torch.int32, device=dev())
    sp = torch.empty(S, dtype=torch.int32, device=dev())
    ws = sm.alloc_workspace(sm.permute_workspace_bytes(T, E, k), dev())
    sm.strata_moe_permute(ids, E, counts, offsets, ss, sp, ws)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in (counts, offsets, ss, sp)]


@pytest.mark.parametrize("T,E,k,kind", [
    (16, 64, 4, "route"), (4, 512, 10, "route"), (8192, 512, 10, "route"), (2048, 512, 10, "zipf"),
    (103, 7, 7, "route"), (1, 1024, 16, "route"), (5000, 3, 2, "route"), (3000, 1024, 1, "one"),
    (4096, 512, 10, "hot")])
def test_permute_bit_exact(T, E, k, kind):
    log(f"permute T={T} E={E} k={k} {kind}")
    if kind == "zipf":
        ids, _ = oracle.route(mi.make_logits(mi.SKEWED, T=T), k)
    elif kind == "one":
        ids = np.full((T, 1), 77, dtype=np.int32)
    elif kind == "hot":  # every token picks experts 0..9: ten segments of T rows each
        ids = np.tile(np.arange(k, dtype=np.int32), (T, 1))
    else:
        ids, _ = oracle.route(mi.normal_f32(0, 77, T * E).reshape(T, E), k)
    got = gpu_permute(ids, E)
    want = oracle.permute(ids, E)
    for g, r, name in zip(got, want, ("counts", "offsets", "sorted_slot", "slot_pos")):
        assert np.array_equal(g, r), name


def test_permute_twice_identical():
    ids, _ = oracle.route(mi.normal_f32(0, 5, 8192 * 512).reshape(8192, 512), 10)
    a = gpu_permute(ids, 512)
    b = gpu_permute(ids, 512)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------------------------------------
# Expert FFN (staged prefill path) and combine


def staged(L: Layer, ids_np=None):
    """route -> permute -> expert_ffn -> combine through the staged entry points."""
    s, T = L.shape, L.T
    S = T * s.k
    ids = torch.empty((T, s.k), dtype=torch.int32, device=dev())
    rw = torch.empty((T, s.k), dtype=torch.float32, device=dev())
    sm.strata_moe_route(L.logits, s.k, ids, rw)
    counts = torch.empty(s.E, dtype=torch.int32, device=dev())
    offsets = torch.empty(s.E + 1, dtype=torch.int32, device=dev())
    ss = torch.empty(S, dtype=torch.int32, device=dev())
    sp = torch.empty(S, dtype=torch.int32, device=dev())
    ws = L.workspace()
    sm.strata_moe_permute(ids, s.E, counts, offsets, ss, sp, ws)
    out = torch.empty((S, s.H), dtype=torch.int16, device=dev())
    sm.strata_moe_expert_ffn(L.w, L.x, s.k, offsets, ss, out, ws)
    y = torch.empty((T, s.H), dtype=torch.float32, device=dev())
    sm.strata_moe_combine(out, rw, y)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), rw.cpu().numpy(), bf16_tensor_to_f64(out), y.cpu().numpy()


SMALL_SHAPES = [
    shape("tiny"),
    shape("tiny_q3", fmt=3),
    shape("ragged", T=77, H=512, E=16, k=3, I=256),          # chunks of ~14 rows, ragged fragments
    shape("hot", T=300, H=256, E=4, k=2, I=128),             # 150 rows per expert: 5 fragments
    shape("big_expert", T=700, H=256, E=2, k=1, I=128),      # 350 rows: 2 chunks
    shape("q3_zipf", T=200, H=512, E=64, k=6, I=256, fmt=3, zipf=True),
    shape("one_expert", T=9, H=256, E=1, k=1, I=128),
    # up to 24 rows per expert on average: the small-fragment GEMMs, chunks of at most 64 rows
    shape("small_split", T=96, H=256, E=8, k=2, I=128),     # ~24 rows per expert, some split
    shape("hot_q3", T=300, H=256, E=4, k=2, I=128, fmt=3),  # large-chunk GEMMs, 3-bit
    # ~20 rows per expert on the skinny GEMMs with I = 2048: the down projection's a rows exceed
    # the LDS, so it reduces in phases with one 64-row item a wave
    shape("skinny_phases", T=800, H=256, E=40, k=1, I=2048),
    shape("skinny_phases_q3", T=800, H=256, E=40, k=1, I=2048, fmt=3),
    # skinny GEMMs with I = 384 and H = 256: the second gate/up unit of a chunk and half the waves
    # of the down units hold items past the matrix (computed, not stored)
    shape("skinny_i384", T=900, H=256, E=200, k=2, I=384),
]


@pytest.mark.parametrize("s", SMALL_SHAPES, ids=lambda s: s.name)
def test_staged_prefill_path(s):
    log(f"staged {s}")
    L = Layer(s)
    y_ref, ids_ref, w_ref, out_ref, _ = oracle.layer(L.w_np, L.x_np, L.l_np, s.k, intermediates=True)
    ids, rw, out, y = staged(L)
    assert np.array_equal(ids, ids_ref)
    np.testing.assert_allclose(rw, w_ref, rtol=1e-6)
    e_out = rel_l2_rows(out, out_ref)
    e_y = rel_l2_rows(y, y_ref)
    log(f"  expert_out max rel-L2 {e_out.max():.3e}, y max rel-L2 {e_y.max():.3e}")
    assert e_out.max() <= TOL_REL_L2
    assert e_y.max() <= TOL_REL_L2


@pytest.mark.parametrize("T,k,H", [(37, 5, 512), (9, 1, 256), (5, 16, 64), (6, 20, 128)])
def test_combine_against_oracle(T, k, H):
    rng = np.random.default_rng(3 + k)
    out_bits = mi.f32_to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    w = rng.random((T, k)).astype(np.float32)
    y0 = rng.standard_normal((T, H)).astype(np.float32)
    ref = oracle.combine(mi.bf16_bits_to_f32(out_bits).astype(np.float64), w.astype(np.float64), k)
    out_d = torch.from_numpy(out_bits.view(np.int16)).to(dev())
    y = to_dev(y0.copy())
    sm.strata_moe_combine(out_d, to_dev(w), y, accumulate=False)
    torch.cuda.synchronize()
    np.testing.assert_allclose(y.cpu().numpy(), ref, rtol=1e-5, atol=1e-6)
    y = to_dev(y0.copy())
    sm.strata_moe_combine(out_d, to_dev(w), y, accumulate=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(y.cpu().numpy(), ref + y0, rtol=1e-5, atol=1e-5)


# ---------------------------------------------------------------------------------------------
# One-call layer: prefill and decode paths, determinism, accumulate


def gpu_layer(L: Layer, accumulate=False, y0=None, want_ids=False):
    s, T = L.shape, L.T
    y = to_dev(y0.copy()) if y0 is not None else torch.empty((T, s.H), dtype=torch.float32, device=dev())
    ids = torch.empty((T, s.k), dtype=torch.int32, device=dev())
    rw = torch.empty((T, s.k), dtype=torch.float32, device=dev())
    sm.strata_moe_layer(L.w, L.x, L.logits, s.k, y, accumulate=accumulate, topk_ids=ids, topk_w=rw,
                        workspace=L.workspace())
    torch.cuda.synchronize()
    return y.cpu().numpy(), ids.cpu().numpy(), rw.cpu().numpy()


@pytest.mark.parametrize("s", SMALL_SHAPES + [shape("t9", T=9), shape("t8", T=8), shape("t1", T=1),
                                              shape("t17", T=17), shape("t32", T=32), shape("t40", T=40),
                                              shape("t41", T=41), shape("t33_q3", T=33, fmt=3),
                                              shape("t5_q3", T=5, fmt=3), shape("t3_e1", T=3, E=1, k=1),
                                              shape("t4_q3_i768", T=4, H=512, I=768, fmt=3),
                                              shape("t3_i1024", T=3, I=1024),
                                              shape("t6_q3_i1024", T=6, I=1024, fmt=3)],
                         ids=lambda s: s.name)
def test_layer_against_oracle(s):
    log(f"layer {s}")
    L = Layer(s)
    y_ref, ids_ref, w_ref, _, _ = oracle.layer(L.w_np, L.x_np, L.l_np, s.k, intermediates=True)
    y, ids, rw = gpu_layer(L)
    assert np.array_equal(ids, ids_ref)
    err = rel_l2_rows(y, y_ref)
    path = "decode" if s.T <= 8 else "decode slices" if s.T <= 32 else "prefill"
    log(f"  y max rel-L2 {err.max():.3e} (T={s.T}, {path} path)")
    assert err.max() <= TOL_REL_L2
    y2, _, _ = gpu_layer(L)
    assert np.array_equal(y, y2), "second call differs"
    y0 = np.random.default_rng(1).standard_normal((s.T, s.H)).astype(np.float32)
    ya, _, _ = gpu_layer(L, accumulate=True, y0=y0)
    np.testing.assert_allclose(ya, y0 + y, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("n_small,fmt", [(70, 2), (70, 3), (161, 2), (60, 2)],
                         ids=["split", "split_q3", "small", "fallback"])
def test_chunk_list_boundaries(n_small, fmt):
    """Routing crafted so that experts hold exactly 1, 2, 31, 32, 33, 63 and 64 rows (the small part
    of the GEMM chunk list) and 65, 96, 97, 224, 225, 300 and 449 rows (the large part: 224 is one
    7-fragment chunk, 225 two, 449 three), plus untouched experts.  With I = 1024 the small part
    needs 64 such experts: 70 use it, with the 30 experts of 33-64 rows split into two skinny
    chunks each (all 70 on the skinny GEMMs); 161 use it with 69 such experts, more than are split,
    so those run on the small-fragment GEMMs; 60 fall back to the large part for every expert.
    Rows at both ends of every expert's segment and at its fragment boundaries, plus random rows,
    against the oracle."""
    small = [1, 2, 31, 32, 33, 63, 64]
    large = [65, 96, 97, 224, 225, 300, 449]
    counts = [small[i % len(small)] for i in range(n_small)] + large + [0] * 4
    E = len(counts)
    T = sum(counts)
    s = mi.Shape(f"chunks_{n_small}", T=T, H=256, E=E, k=1, I=1024, fmt=fmt)
    rng = np.random.default_rng(11 + n_small)
    target = rng.permutation(np.repeat(np.arange(E), counts))
    L = Layer(s)
    L.l_np = (rng.standard_normal((T, E)) * 0.01).astype(np.float32)
    L.l_np[np.arange(T), target] = 1.0
    L.logits = to_dev(L.l_np)
    log(f"chunk list boundaries: {n_small} small experts, T = {T}")
    y, ids, _ = gpu_layer(L)
    assert np.array_equal(ids[:, 0], target)
    rows = set(rng.choice(T, size=64, replace=False).tolist())
    for e in range(E):
        toks = np.nonzero(target == e)[0]  # slot order = token order (k = 1)
        for p in (0, 30, 31, 32, 33, 63, 64, 65, 223, 224, 225, len(toks) - 1):
            if 0 <= p < len(toks):
                rows.add(int(toks[p]))
    rows = np.array(sorted(rows))
    err = rel_l2_rows(y[rows], oracle.layer_rows(L.w_np, L.x_np, L.l_np, 1, rows))
    log(f"  {len(rows)} rows, max rel-L2 {err.max():.3e}")
    assert err.max() <= TOL_REL_L2
    y2, _, _ = gpu_layer(L)
    assert np.array_equal(y, y2), "second call differs"


@pytest.mark.parametrize("T", [1, 4, 8])
def test_decode_crowded_routing(T):
    """Routing inside the decode kernel where more than 64 entries reach the k-th largest lane
    head (its round-by-round arg-max) for some tokens, and the threshold path for the others."""
    s = shape("crowd", T=T, E=512, k=10)
    L = Layer(s)
    l = L.l_np.copy()
    lane = np.arange(s.E) % 64
    l[::2, lane < s.k - 1] += 100.0
    l[::2, s.k - 1] += 50.0
    L.l_np, L.logits = l, to_dev(l)
    y_ref, ids_ref, w_ref, _, _ = oracle.layer(L.w_np, L.x_np, l, s.k, intermediates=True)
    y, ids, rw = gpu_layer(L)
    assert np.array_equal(ids, ids_ref)
    np.testing.assert_allclose(rw, w_ref, rtol=1e-6, atol=0)
    assert rel_l2_rows(y, y_ref).max() <= TOL_REL_L2


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_decode_matches_prefill_path(T):
    s = shape("dp", T=T, H=512, E=32, k=4, I=256)
    L = Layer(s)
    y_dec, _, _ = gpu_layer(L)
    _, _, _, y_pre = staged(L)
    y_ref = oracle.layer(L.w_np, L.x_np, L.l_np, s.k)
    assert rel_l2_rows(y_dec, y_ref).max() <= TOL_REL_L2
    assert rel_l2_rows(y_pre, y_ref).max() <= TOL_REL_L2
    assert rel_l2_rows(y_dec, y_pre).max() <= 2 * TOL_REL_L2


def test_zero_tokens_is_noop():
    s = shape("t0", T=4)
    L = Layer(s)
    y = torch.full((1, s.H), 7.0, device=dev())
    empty_x = L.x[:0]
    sm.strata_moe_layer(L.w, empty_x, L.logits[:0], s.k, y, workspace=L.workspace())
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ---------------------------------------------------------------------------------------------
# Residual layer of a stack: h <- h + MoE(RMSNorm(h))


@pytest.mark.parametrize("s", [shape("r1", T=1), shape("r4", T=4, H=512, E=32, k=4, I=256),
                               shape("r8_q3", T=8, fmt=3), shape("r3_e1", T=3, E=1, k=1),
                               shape("r9", T=9), shape("r40", T=40, fmt=3), shape("r70", T=70)],
                         ids=lambda s: s.name)
def test_layer_residual_against_oracle(s):
    log(f"layer residual {s}")
    L = Layer(s)
    rng = np.random.default_rng(s.T + 31)
    h_np = (rng.standard_normal((s.T, s.H)) * 2.5).astype(np.float32)
    h = to_dev(h_np)
    ws = sm.alloc_workspace(sm.residual_workspace_bytes(s.T, s.E, s.k, s.H, s.I), dev())
    sm.strata_moe_layer_residual(L.w, h, L.logits, s.k, ws, eps=1e-6)
    torch.cuda.synchronize()
    got = h.cpu().numpy().astype(np.float64) - h_np.astype(np.float64)
    x_ref = oracle.rmsnorm(h_np, 1e-6)
    y_ref = oracle.layer(L.w_np, x_ref, L.l_np, s.k)
    err = rel_l2_rows(got, y_ref)
    path = "fused decode" if s.T <= 8 else "rmsnorm + layer"
    log(f"  max rel-L2 {err.max():.3e} ({path})")
    assert err.max() <= TOL_REL_L2
    # the same step with the normalisation as its own call, then the layer accumulating into h
    h2 = to_dev(h_np)
    x = torch.empty((s.T, s.H), dtype=torch.int16, device=dev())
    sm.strata_moe_rmsnorm(h2, x, 1e-6)
    sm.strata_moe_layer(L.w, x, L.logits, s.k, h2, accumulate=True, workspace=L.workspace())
    torch.cuda.synchronize()
    got2 = h2.cpu().numpy().astype(np.float64) - h_np.astype(np.float64)
    assert rel_l2_rows(got, got2).max() <= TOL_REL_L2
    h3 = to_dev(h_np)
    sm.strata_moe_layer_residual(L.w, h3, L.logits, s.k, ws, eps=1e-6)
    torch.cuda.synchronize()
    assert torch.equal(h, h3), "second call differs"


# ---------------------------------------------------------------------------------------------
# RMSNorm


def test_rmsnorm_against_oracle():
    rng = np.random.default_rng(9)
    h = (rng.standard_normal((64, 3072)) * 3).astype(np.float32)
    h[0] = 0.0
    h[1] = 1.0
    x = torch.empty((64, 3072), dtype=torch.int16, device=dev())
    sm.strata_moe_rmsnorm(to_dev(h), x, 1e-6)
    torch.cuda.synchronize()
    got = x.cpu().numpy().view(np.uint16).astype(np.int32)
    ref = oracle.rmsnorm(h, 1e-6).astype(np.int32)
    diff = np.abs(got - ref)
    assert diff.max() <= 1              # at most one bf16 ulp (rounding of a near-tie)
    assert np.mean(diff == 0) > 0.999


def test_rmsnorm_pinned_rows():
    """The rows that pin the oracle's RMSNorm (eps inside the root, ties to even, one rounding):
    the GPU rounds through fp32, so it may differ by one bf16 ulp where the quotient sits within
    half an fp32 ulp of a tie, and nowhere else."""
    rows = np.array([[257, 676, 35, 6, 1, 1, 0, 0], [259, 676, 15, 2, 1, 1, 0, 0],
                     [257, 676, 35, 6, 1, 1 - 2.0 ** -9, 0, 0]], dtype=np.float32)
    for h, eps in ((rows, 0.0), (np.full((2, 256), 1e-4, dtype=np.float32), 1e-6)):
        x = torch.empty(h.shape, dtype=torch.int16, device=dev())
        sm.strata_moe_rmsnorm(to_dev(h), x, eps)
        torch.cuda.synchronize()
        got = x.cpu().numpy().view(np.uint16).astype(np.int32)
        ref = oracle.rmsnorm(h, eps).astype(np.int32)
        assert np.abs(got - ref).max() <= 1
        if eps == 0.0:
            assert np.array_equal(got[:2], ref[:2])   # exact ties: the same even choice
            assert np.array_equal(got[2, 1:], ref[2, 1:])


@pytest.mark.parametrize("T", [1, 4, 8, 20, 32])
def test_layer_permutation_on_decode_paths(T):
    """strata_moe_layer's optional routing and permutation outputs on the decode paths (T <= 8
    and the sliced path up to 32): bit-exact against the oracle."""
    s = mi.DECODE
    log(f"layer permutation outputs T={T}")
    L = Layer(s, T=T)
    S = T * s.k
    ids = torch.empty((T, s.k), dtype=torch.int32, device=dev())
    wts = torch.empty((T, s.k), dtype=torch.float32, device=dev())
    counts = torch.empty(s.E, dtype=torch.int32, device=dev())
    offsets = torch.empty(s.E + 1, dtype=torch.int32, device=dev())
    sorted_slot = torch.empty(S, dtype=torch.int32, device=dev())
    y = torch.empty((T, s.H), dtype=torch.float32, device=dev())
    sm.strata_moe_layer(L.w, L.x, L.logits, s.k, y, topk_ids=ids, topk_w=wts, counts=counts,
                        offsets=offsets, sorted_slot=sorted_slot, workspace=L.workspace())
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.route(L.l_np, s.k)
    c_ref, o_ref, ss_ref, _ = oracle.permute(ids_ref, s.E)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(wts.cpu().numpy() - w_ref).max() <= 1e-6
    assert np.array_equal(counts.cpu().numpy(), c_ref)
    assert np.array_equal(offsets.cpu().numpy(), o_ref)
    assert np.array_equal(sorted_slot.cpu().numpy(), ss_ref)
    # the same layer output as without the optional outputs; only the permutation, no ids
    y2 = torch.empty_like(y)
    sm.strata_moe_layer(L.w, L.x, L.logits, s.k, y2, workspace=L.workspace())
    counts2 = torch.empty_like(counts)
    y3 = torch.empty_like(y)
    sm.strata_moe_layer(L.w, L.x, L.logits, s.k, y3, counts=counts2, workspace=L.workspace())
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(y, y3)
    assert np.array_equal(counts2.cpu().numpy(), c_ref)


# ---------------------------------------------------------------------------------------------
# Weight repack (row-major -> tiled): a pure byte permutation, so bit-exact against the index
# arithmetic written out with numpy.


@pytest.mark.parametrize("fmt,n_mat,rows,K", [(2, 3, 128, 256), (3, 2, 196, 128), (2, 1, 4, 64)])
def test_pack_matrix_bit_exact(fmt, n_mat, rows, K):
    cb = sm.CODE_BYTES[fmt]
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 256, size=(n_mat, rows, K // 32, cb), dtype=np.uint8)
    scales = rng.integers(0, 1 << 16, size=(n_mat, rows, K // 32), dtype=np.uint16)
    c = torch.from_numpy(codes).to(dev())
    s = torch.from_numpy(scales.view(np.int16)).to(dev())
    tc, ts = torch.empty_like(c), torch.empty_like(s)
    sm.strata_moe_pack_matrix(fmt, n_mat, rows, K, c, s, tc, ts)
    torch.cuda.synchronize()
    # block b of row r -> tile (r // 4, b // 2), tile row r % 4, slot b % 2
    want_c = codes.reshape(n_mat, rows // 4, 4, K // 64, 2, cb).transpose(0, 1, 3, 2, 4, 5)
    want_s = scales.reshape(n_mat, rows // 4, 4, K // 64, 2).transpose(0, 1, 3, 2, 4)
    assert np.array_equal(tc.cpu().numpy().reshape(-1), np.ascontiguousarray(want_c).reshape(-1))
    assert np.array_equal(ts.cpu().numpy().view(np.uint16).reshape(-1),
                          np.ascontiguousarray(want_s).reshape(-1))

