"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin is chosen so that a plausible mistake in the oracle fails it: a wrong code bit order
or offset (exhaustive closed-form dequantization), a wrong tie rule or slot order (brute-force
stable sort), a wrong weight formula (full softmax then renormalise, a different route to the
same numbers), a transposed or dropped FFN term (independent numpy/torch float64 layer), a
wrong combine (k = 1 and scale-doubling identities), and an order dependence between tokens
(permutation equivariance).
"""
import os

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# ---------------------------------------------------------------------------------------------
# Independent vectorised decoders of the formats, written from the format description (byte i/4
# at bits 2*(i%4) for 2-bit codes; an LSB-first 96-bit little-endian bitstream for 3-bit codes).


def codes_q2(blocks: np.ndarray) -> np.ndarray:
    b = blocks.astype(np.uint8)[..., :, None]                    # [..., 8, 1]
    q = (b >> (2 * np.arange(4, dtype=np.uint8))) & 3            # [..., 8, 4]: weight 4*byte + j
    return q.reshape(*blocks.shape[:-1], 32).astype(np.int64)


def codes_q3(blocks: np.ndarray) -> np.ndarray:
    bits = np.unpackbits(blocks.astype(np.uint8), axis=-1, bitorder="little")  # [..., 96]
    bits = bits.reshape(*blocks.shape[:-1], 32, 3).astype(np.int64)
    return bits[..., 0] + 2 * bits[..., 1] + 4 * bits[..., 2]


def f16_values(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequant_np(fmt, codes, scales):
    q = codes_q2(codes) if fmt == 2 else codes_q3(codes)         # [R, nb, 32]
    c0 = 1.5 if fmt == 2 else 3.5
    w = f16_values(scales)[..., None] * (q - c0)
    return w.reshape(*scales.shape[:-1], scales.shape[-1] * 32)


def encode_q2(q: np.ndarray) -> np.ndarray:
    """32 codes -> 8 bytes, byte i/4 holding weight i at bits 2*(i%4)."""
    out = np.zeros(8, dtype=np.uint8)
    for i, v in enumerate(q):
        out[i // 4] |= np.uint8(int(v) << (2 * (i % 4)))
    return out


def encode_q3(q: np.ndarray) -> np.ndarray:
    v = 0
    for i, c in enumerate(q):
        v |= int(c) << (3 * i)
    return np.frombuffer(v.to_bytes(12, "little"), dtype=np.uint8).copy()


SCALE_BITS = [0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x3555, 0x7BFF, 0xBC00, 0x8001]


# ---------------------------------------------------------------------------------------------
# Number formats


def test_f16_decode_all_patterns(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_bf16_decode_is_upper_half_of_f32(oracle_lib):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 65536, size=4000).astype(np.uint16)
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    ok = np.isfinite(ref)
    assert np.array_equal(got[ok], ref[ok])


# ---------------------------------------------------------------------------------------------
# Dequantization: closed form, exhaustively over codes x positions x scales


@pytest.mark.parametrize("fmt", [2, 3])
def test_dequant_closed_form_exhaustive(oracle_lib, fmt):
    nq = 4 if fmt == 2 else 8
    c0 = 1.5 if fmt == 2 else 3.5
    enc = encode_q2 if fmt == 2 else encode_q3
    for pos in range(32):
        for q in range(nq):
            codes = np.array([(pos + 3 * i + 1) % nq for i in range(32)], dtype=np.int64)
            codes[pos] = q
            blk = enc(codes)
            assert oracle.code(fmt, blk, pos) == q
            for sb in SCALE_BITS:
                d = float(np.uint16(sb).view(np.float16))
                got = oracle.dequant_block(fmt, blk, sb)
                want = np.array([d * (float(c) - c0) for c in codes])
                assert np.array_equal(got, want), (fmt, pos, q, hex(sb))


@pytest.mark.parametrize("fmt", [2, 3])
def test_dequant_matrix_matches_vectorised_decoder(oracle_lib, fmt):
    rng = np.random.default_rng(7)
    cb = 8 if fmt == 2 else 12
    codes = rng.integers(0, 256, size=(24, 8, cb)).astype(np.uint8)
    scales = mi.f32_to_f16_bits(rng.standard_normal((24, 8)).astype(np.float32) * 0.02)
    got = oracle.dequant_matrix(fmt, codes, scales)
    assert np.array_equal(got, dequant_np(fmt, codes, scales))


def test_q3_codes_straddling_byte_edges(oracle_lib):
    # weights whose 3 bits cross a byte boundary: bit 3i mod 8 > 5
    straddle = [i for i in range(32) if (3 * i) % 8 > 5]
    assert straddle == [2, 5, 10, 13, 18, 21, 26, 29]
    for i in straddle:
        for q in range(8):
            codes = np.zeros(32, dtype=np.int64)
            codes[i] = q
            assert oracle.code(3, encode_q3(codes), i) == q


# ---------------------------------------------------------------------------------------------
# Routing


def brute_route(logits: np.ndarray, k: int):
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))
        ids[t] = order[:k]
        # full softmax over all experts, then renormalise the k kept probabilities
        l = logits[t].astype(np.float64)
        p = np.exp(l - l.max())
        p /= p.sum()
        kept = p[ids[t]]
        w[t] = kept / kept.sum()
    return ids, w


@pytest.mark.parametrize("T,E,k,levels", [(16, 64, 4, None), (9, 17, 5, 4), (5, 512, 10, None),
                                          (7, 8, 8, 2), (3, 33, 1, 3)])
def test_route_brute_force(oracle_lib, T, E, k, levels):
    rng = np.random.default_rng(T * 1000 + E)
    if levels is None:
        logits = rng.standard_normal((T, E)).astype(np.float32)
    else:  # few distinct values: many ties
        logits = rng.integers(0, levels, size=(T, E)).astype(np.float32) * 0.5
    ids, w = oracle.route(logits, k)
    bids, bw = brute_route(logits, k)
    assert np.array_equal(ids, bids)
    np.testing.assert_allclose(w, bw, rtol=1e-13, atol=0)
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
        assert abs(w[t].sum() - 1.0) < 1e-14
        assert np.all(np.diff(w[t]) <= 0)


def test_route_all_equal_and_signed_zero(oracle_lib):
    logits = np.zeros((2, 12), dtype=np.float32)
    logits[1, :] = -0.0
    logits[1, 5] = 0.0  # +0 == -0: still a tie, lower index wins
    ids, w = oracle.route(logits, 4)
    assert ids.tolist() == [[0, 1, 2, 3], [0, 1, 2, 3]]
    assert np.all(w == 0.25)


# ---------------------------------------------------------------------------------------------
# Permutation


@pytest.mark.parametrize("T,E,k", [(16, 64, 4), (1, 5, 5), (37, 3, 2), (64, 512, 10)])
def test_permute_is_stable_sort(oracle_lib, T, E, k):
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, sorted_slot, slot_pos = oracle.permute(ids, E)
    flat = ids.reshape(-1)
    S = flat.size
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == S
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(sorted_slot, np.array(sorted(range(S), key=lambda s: flat[s])))
    assert np.array_equal(np.sort(sorted_slot), np.arange(S))
    assert np.array_equal(slot_pos[sorted_slot], np.arange(S))
    for e in range(E):
        seg = sorted_slot[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


# ---------------------------------------------------------------------------------------------
# Expert FFN and the whole layer against an independent float64 implementation


def independent_layer(w, x_bits, logits, k):
    """Vectorised numpy/torch float64 layer: stable argsort routing, full-softmax weights,
    SwiGLU via torch matmul, weighted sum."""
    E, H, I, fmt = w["E"], w["H"], w["I"], w["fmt"]
    x = torch.from_numpy(mi.bf16_bits_to_f32(x_bits).astype(np.float64))
    T = x.shape[0]
    ids = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k]
    l = logits.astype(np.float64)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    kept = np.take_along_axis(p, ids, axis=1)
    rw = kept / kept.sum(axis=1, keepdims=True)
    y = torch.zeros((T, H), dtype=torch.float64)
    outs = torch.zeros((T * k, H), dtype=torch.float64)
    for e in np.unique(ids):
        Wg = torch.from_numpy(dequant_np(fmt, w["gate_codes"][e], w["gate_scales"][e]))
        Wu = torch.from_numpy(dequant_np(fmt, w["up_codes"][e], w["up_scales"][e]))
        Wd = torch.from_numpy(dequant_np(fmt, w["down_codes"][e], w["down_scales"][e]))
        tok, slot = np.nonzero(ids == e)
        xe = x[torch.from_numpy(tok)]
        a = torch.nn.functional.silu(xe @ Wg.T) * (xe @ Wu.T)
        o = a @ Wd.T
        outs[torch.from_numpy(tok * k + slot)] = o
    for j in range(k):
        y += torch.from_numpy(rw[:, j:j + 1]) * outs[j::k]
    return y.numpy(), ids, rw, outs.numpy()


def small_shape(fmt=2, T=16, H=256, E=64, k=4, I=128, zipf=False):
    return mi.Shape("t", T=T, H=H, E=E, k=k, I=I, fmt=fmt, zipf=zipf)


@pytest.mark.parametrize("shape", [mi.TINY, small_shape(fmt=3, zipf=True, T=24),
                                   small_shape(T=5, H=128, E=7, k=3, I=128)])
def test_layer_matches_independent_float64(oracle_lib, shape):
    w = mi.make_weights(shape, seed=0)
    x = mi.make_x(shape)
    logits = mi.make_logits(shape)
    y, ids, rw, out, a = oracle.layer(w, x, logits, shape.k, intermediates=True)
    yi, idsi, rwi, outi = independent_layer(w, x, logits, shape.k)
    assert np.array_equal(ids, idsi)
    np.testing.assert_allclose(rw, rwi, rtol=1e-13)
    np.testing.assert_allclose(out, outi, rtol=1e-11, atol=1e-12 * np.abs(outi).max())
    np.testing.assert_allclose(y, yi, rtol=1e-11, atol=1e-12 * np.abs(yi).max())
    assert np.all(np.linalg.norm(y, axis=1) > 0)


def test_single_expert_top1_is_plain_swiglu(oracle_lib):
    shape = small_shape(T=6, H=256, E=1, k=1, I=128)
    w = mi.make_weights(shape, seed=3)
    x = mi.make_x(shape, seed=3)
    logits = mi.make_logits(shape, seed=3)
    y = oracle.layer(w, x, logits, 1)
    Wg = dequant_np(2, w["gate_codes"][0], w["gate_scales"][0])
    Wu = dequant_np(2, w["up_codes"][0], w["up_scales"][0])
    Wd = dequant_np(2, w["down_codes"][0], w["down_scales"][0])
    xf = torch.from_numpy(mi.bf16_bits_to_f32(x).astype(np.float64))
    ref = (torch.nn.functional.silu(xf @ torch.from_numpy(Wg).T) * (xf @ torch.from_numpy(Wu).T)) \
        @ torch.from_numpy(Wd).T
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_expert_ffn_matches_layer_slot(oracle_lib):
    shape = mi.TINY
    w = mi.make_weights(shape)
    x = mi.make_x(shape)
    logits = mi.make_logits(shape)
    y, ids, rw, out, a = oracle.layer(w, x, logits, shape.k, intermediates=True)
    for t, j in [(0, 0), (5, 3), (15, 2)]:
        o, aa = oracle.expert_ffn(w, int(ids[t, j]), x[t])
        assert np.array_equal(o, out[t * shape.k + j])
        assert np.array_equal(aa, a[t * shape.k + j])


def test_combine_identities(oracle_lib):
    shape = small_shape(T=8, E=16, k=1)
    w = mi.make_weights(shape)
    x = mi.make_x(shape)
    logits = mi.make_logits(shape)
    y, ids, rw, out, a = oracle.layer(w, x, logits, 1, intermediates=True)
    assert np.all(rw == 1.0)
    assert np.array_equal(y, out)
    # doubling every down-projection scale doubles the output exactly
    w2 = dict(w)
    w2["down_scales"] = (f16_values(w["down_scales"]) * 2).astype(np.float16).view(np.uint16)
    shape4 = small_shape(T=8, E=16, k=4)
    y4 = oracle.layer(w, x, mi.make_logits(shape4), 4)
    y4d = oracle.layer(w2, x, mi.make_logits(shape4), 4)
    assert np.array_equal(y4d, 2 * y4)


def test_token_permutation_equivariance(oracle_lib):
    shape = mi.TINY
    w = mi.make_weights(shape)
    x = mi.make_x(shape)
    logits = mi.make_logits(shape)
    y = oracle.layer(w, x, logits, shape.k)
    perm = np.random.default_rng(5).permutation(shape.T)
    yp = oracle.layer(w, x[perm], logits[perm], shape.k)
    assert np.array_equal(yp, y[perm])
    rows = [3, 0, 15, 3]
    assert np.array_equal(oracle.layer_rows(w, x, logits, shape.k, rows), y[rows])


def test_expert_relabelling_invariance(oracle_lib):
    shape = mi.TINY
    w = mi.make_weights(shape)
    x = mi.make_x(shape)
    logits = mi.make_logits(shape)
    y = oracle.layer(w, x, logits, shape.k)
    for t in range(shape.T):
        assert len(np.unique(logits[t])) == shape.E  # no ties, so relabelling keeps the order
    perm = np.random.default_rng(11).permutation(shape.E)  # new expert p holds old expert perm[p]
    w2 = dict(w)
    for name in ("gate_codes", "up_codes", "down_codes", "gate_scales", "up_scales", "down_scales"):
        w2[name] = np.ascontiguousarray(w[name][perm])
    y2 = oracle.layer(w2, x, np.ascontiguousarray(logits[:, perm]), shape.k)
    assert np.array_equal(y2, y)


# ---------------------------------------------------------------------------------------------
# RMSNorm


def test_rmsnorm_special_rows(oracle_lib):
    H = 256
    h = np.zeros((4, H), dtype=np.float32)
    h[0] = 1.0                                    # -> 1/sqrt(1 + eps) rounds to 1.0 in bf16
    h[1] = np.where(np.arange(H) % 2 == 0, 3.0, -3.0)  # -> +-1
    h[2, 0] = 16.0                                # one spike: mean = 1 -> 16/sqrt(1+eps) -> 16
    h[3] = 0.0                                    # all zero -> 0 / sqrt(eps) = 0
    x = mi.bf16_bits_to_f32(oracle.rmsnorm(h, 1e-6))
    assert np.all(x[0] == 1.0)
    assert np.array_equal(x[1], np.where(np.arange(H) % 2 == 0, 1.0, -1.0).astype(np.float32))
    assert x[2, 0] == 16.0 and np.all(x[2, 1:] == 0)
    assert np.all(x[3] == 0)


def test_rmsnorm_unit_rms_and_scale_invariance(oracle_lib):
    rng = np.random.default_rng(2)
    h = (rng.standard_normal((8, 3072)) * 7).astype(np.float32)
    x = mi.bf16_bits_to_f32(oracle.rmsnorm(h, 1e-6)).astype(np.float64)
    rms = np.sqrt((x ** 2).mean(axis=1))
    assert np.all(np.abs(rms - 1) < 4e-3)  # bf16 rounding of each element
    x2 = oracle.rmsnorm(h * np.float32(4.0), 1e-6)  # scaling by 4 is exact; eps effect < 1 ulp
    assert np.mean(x2 == oracle.rmsnorm(h, 1e-6)) > 0.999


def bf16_nearest_by_search(v: float) -> float:
    """bf16 value nearest to the fp64 value v, ties to the even bit pattern, found by comparing
    v with the candidate bit patterns around its binary32 rounding (exact fp64 distances; a
    different route from the oracle's frexp/rint)."""
    f = np.float32(v)
    c = int(f.view(np.uint32)) >> 16
    best, best_d = None, None
    for b in (c - 1, c, c + 1, c + 2):
        val = float(np.uint32((b & 0xFFFF) << 16).view(np.float32))
        d = abs(val - v)
        if best is None or d < best_d or (d == best_d and (b & 1) == 0):
            best, best_d = b & 0xFFFF, d
    return float(np.uint32(best << 16).view(np.float32))


def test_rmsnorm_eps_inside_the_square_root(oracle_lib):
    """mean(h^2) = 1e-8 is far below eps = 1e-6: x = h / sqrt(mean + eps) = 0.0995 differs from
    h / (sqrt(mean) + eps) = 0.990, from h / sqrt((sum + eps) / H) = 0.848 and from h / sqrt(mean)
    = 1, so a misplaced eps fails."""
    H, eps = 256, 1e-6
    h = np.full((2, H), 1e-4, dtype=np.float32)
    h[1, ::2] = -1e-4
    x = mi.bf16_bits_to_f32(oracle.rmsnorm(h, eps)).astype(np.float64)
    hv = float(np.float32(1e-4))
    want = bf16_nearest_by_search(hv / np.sqrt(hv * hv + eps))
    assert abs(want - 0.0995) < 1e-3
    assert np.all(x[0] == want)
    assert np.array_equal(x[1], np.where(np.arange(H) % 2 == 0, -want, want))
    for wrong in (hv / (hv + eps), hv / np.sqrt((H * hv * hv + eps) / H), 1.0):
        assert bf16_nearest_by_search(wrong) != want


def test_rmsnorm_ties_round_to_even(oracle_lib):
    """Rows whose mean square is exactly 256^2 (eps = 0), so each quotient is exact: 257/256 and
    259/256 lie half-way between neighbouring bf16 values and go to the even one (1 and 260/256),
    which truncation, half-up or half-down rounding each get wrong in one of the two rows."""
    rows = np.array([[257, 676, 35, 6, 1, 1, 0, 0], [259, 676, 15, 2, 1, 1, 0, 0]], dtype=np.float32)
    assert np.all((rows.astype(np.float64) ** 2).sum(axis=1) == 8 * 256.0 ** 2)
    x = mi.bf16_bits_to_f32(oracle.rmsnorm(rows, 0.0)).astype(np.float64)
    assert x[0, 0] == 1.0 and x[1, 0] == 260 / 256
    assert np.array_equal(x[0, 1:], rows[0, 1:] / 256.0)  # exactly representable
    assert np.array_equal(x[1, 1:], rows[1, 1:] / 256.0)


def test_rmsnorm_rounds_once(oracle_lib):
    """h[5] = 1 - 2^-9 makes the mean square 2^-30 below 256^2, so 257 / rms lies 2^-28 (relative)
    above the tie 257/256: rounded once it goes up to 258/256; rounded to binary32 first it
    would land on the tie and then go down to 1."""
    row = np.array([[257, 676, 35, 6, 1, 1 - 2.0 ** -9, 0, 0]], dtype=np.float32)
    q = 257.0 / np.sqrt((row.astype(np.float64) ** 2).sum() / 8)
    assert q > 257 / 256 and float(np.float32(q)) == 257 / 256
    x = mi.bf16_bits_to_f32(oracle.rmsnorm(row, 0.0)).astype(np.float64)
    assert x[0, 0] == 258 / 256


def test_rmsnorm_matches_numpy_fp64(oracle_lib):
    """Random rows over a wide range of scales against numpy in fp64 (exact sum of squares by
    math.fsum) rounded by the candidate search above."""
    import math

    rng = np.random.default_rng(12)
    H = 512
    scales = [1e-30, 1e-6, 3e-3, 1.0, 7.0, 4e5, 1e30]
    h = np.concatenate([(rng.standard_normal((2, H)) * s).astype(np.float32) for s in scales])
    eps = 1e-6
    x = mi.bf16_bits_to_f32(oracle.rmsnorm(h, eps)).astype(np.float64)
    for t in range(h.shape[0]):
        r = h[t].astype(np.float64)
        den = math.sqrt(math.fsum(r * r) / H + eps)
        want = np.array([bf16_nearest_by_search(v / den) for v in r])
        assert np.array_equal(x[t], want), t


# ---------------------------------------------------------------------------------------------
# ---------------------------------------------------------------------------------------------
# Router projection and shared expert (dense bf16 layers on either side of the routed experts)


def test_router_logits_one_hot_rows_pick_weight_columns(oracle_lib):
    """x = rows of the identity: logits[t][e] must be W_r[e][t] exactly (E != H, so a transposed
    weight index or a dropped term fails)."""
    H, E = 64, 24
    wr = mi.dense_bf16(5, 77, E, H)
    x = mi.f32_to_bf16_bits(np.eye(H, dtype=np.float32)[:10])
    l = oracle.router_logits(x, wr)
    assert l.shape == (10, E)
    assert np.array_equal(l, mi.bf16_bits_to_f32(wr).astype(np.float64)[:, :10].T)


def test_router_logits_matches_float64_matmul(oracle_lib):
    shape = small_shape(T=7, H=256, E=48)
    x = mi.make_x(shape, seed=2)
    wr = mi.make_router(shape, seed=2)
    ref = mi.bf16_bits_to_f32(x).astype(np.float64) @ mi.bf16_bits_to_f32(wr).astype(np.float64).T
    l = oracle.router_logits(x, wr)
    np.testing.assert_allclose(l, ref, rtol=1e-13, atol=1e-14 * np.abs(ref).max())
    # products of bf16 values are exact in fp64 and the sums of 256 of them lose at most a few
    # ulps: the unit-variance generator gives logits of about unit spread
    assert 0.7 < l.std() < 1.4


def shared_reference(x, wg, wu, wd):
    f = lambda b: torch.from_numpy(mi.bf16_bits_to_f32(b).astype(np.float64))
    xx = f(x)
    a = torch.nn.functional.silu(xx @ f(wg).T) * (xx @ f(wu).T)
    return (a @ f(wd).T).numpy()


def test_shared_expert_matches_torch_swiglu(oracle_lib):
    shape = small_shape(T=9, H=256, I=128)
    sh = mi.make_shared(shape, seed=4)
    x = mi.make_x(shape, seed=4)
    out = oracle.shared_expert(x, sh["gate"], sh["up"], sh["down"])
    ref = shared_reference(x, sh["gate"], sh["up"], sh["down"])
    assert out.shape == (9, 256)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13 * np.abs(ref).max())
    # gate and up are not interchangeable: SiLU acts on the gate projection only
    swapped = oracle.shared_expert(x, sh["up"], sh["gate"], sh["down"])
    assert np.abs(swapped - out).max() > 1e-3 * np.abs(out).max()


def test_shared_expert_equals_routed_expert_with_exact_weights(oracle_lib):
    """A shared expert whose bf16 weights equal a routed expert's dequantized weights computes
    the same SwiGLU FFN as that expert: with every block scale 2^-6 the weights d(q - 1.5) are
    exact in bf16, so the two oracle paths (quantized-block and dense) must agree to rounding."""
    shape = small_shape(T=4, H=128, E=2, k=1, I=64)
    w = mi.make_weights(shape, seed=6)
    for name in ("gate", "up", "down"):
        w[name + "_scales"] = np.full_like(w[name + "_scales"], 0x2400)   # fp16 2^-6
    e = 1
    dense = {}
    for name in ("gate", "up", "down"):
        m = dequant_np(2, w[name + "_codes"][e], w[name + "_scales"][e])
        bits = mi.f32_to_bf16_bits(m.astype(np.float32))
        assert np.array_equal(mi.bf16_bits_to_f32(bits).astype(np.float64), m)
        dense[name] = bits
    x = mi.make_x(shape, seed=6)
    out = oracle.shared_expert(x, dense["gate"], dense["up"], dense["down"])
    for t in range(shape.T):
        o, _ = oracle.expert_ffn(w, e, x[t])
        np.testing.assert_allclose(out[t], o, rtol=1e-12, atol=1e-14 * np.abs(o).max())


def test_shared_expert_zero_and_scaling(oracle_lib):
    shape = small_shape(T=3, H=128, I=64)
    sh = mi.make_shared(shape, seed=8)
    x = mi.make_x(shape, seed=8)
    out = oracle.shared_expert(x, sh["gate"], sh["up"], sh["down"])
    zero = np.zeros_like(sh["gate"])
    assert np.array_equal(oracle.shared_expert(x, zero, sh["up"], sh["down"]), np.zeros((3, 128)))
    assert np.array_equal(oracle.shared_expert(x, sh["gate"], zero, sh["down"]), np.zeros((3, 128)))
    # doubling W_sd (exact in bf16) doubles the output exactly; the output is linear in W_su
    d2 = mi.f32_to_bf16_bits(2 * mi.bf16_bits_to_f32(sh["down"]))
    assert np.array_equal(oracle.shared_expert(x, sh["gate"], sh["up"], d2), 2 * out)
    u2 = mi.f32_to_bf16_bits(-2 * mi.bf16_bits_to_f32(sh["up"]))
    np.testing.assert_allclose(oracle.shared_expert(x, sh["gate"], u2, sh["down"]), -2 * out,
                               rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------------------------
# Expert usage statistics and the hotness order


def test_usage_counts_brute_force_and_accumulate(oracle_lib):
    rng = np.random.default_rng(3)
    E, k = 37, 5
    u = None
    total = np.zeros(E, dtype=np.int64)
    for T in (1, 13, 64):
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        u = oracle.usage_update(ids, E, u)
        total += np.bincount(ids.reshape(-1), minlength=E)
        assert np.array_equal(u.astype(np.int64), total)
    assert int(u.sum()) == (1 + 13 + 64) * k


def test_usage_counts_from_routing(oracle_lib):
    """Counts of a routed layer equal the permutation's per-expert counts and sum to T*k."""
    shape = mi.TINY
    ids, _ = oracle.route(mi.make_logits(shape), shape.k)
    u = oracle.usage_update(ids, shape.E)
    counts, *_ = oracle.permute(ids, shape.E)
    assert np.array_equal(u.astype(np.int64), counts.astype(np.int64))
    assert int(u.sum()) == shape.T * shape.k


def test_usage_rank_hand_example_and_ties(oracle_lib):
    assert oracle.usage_rank(np.array([3, 5, 5, 0, 3], dtype=np.uint64)).tolist() == [1, 2, 0, 4, 3]
    assert oracle.usage_rank(np.zeros(6, dtype=np.uint64)).tolist() == list(range(6))
    assert oracle.usage_rank(np.array([1 << 40, 1, (1 << 40) + 1], dtype=np.uint64)).tolist() == [2, 0, 1]


def test_usage_rank_matches_library_sort(oracle_lib):
    rng = np.random.default_rng(9)
    for E in (1, 7, 512, 1024):
        u = rng.integers(0, 6, size=E).astype(np.uint64)  # many ties
        order = oracle.usage_rank(u)
        ref = np.lexsort((np.arange(E), -u.astype(np.int64)))
        assert np.array_equal(order, ref)
        assert sorted(order.tolist()) == list(range(E))
        assert np.all(np.diff(u[order].astype(np.int64)) <= 0)


# Golden regression values (written by tests/golden/make_golden.py from the oracle only)


def test_golden_tiny_layer(oracle_lib):
    path = os.path.join(GOLDEN, "tiny_layer.txt")
    rows = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, *vals = line.split()
            rows[key] = vals
    shape = mi.TINY
    y, ids, rw, out, a = oracle.layer(mi.make_weights(shape), mi.make_x(shape),
                                      mi.make_logits(shape), shape.k, intermediates=True)
    assert ids.reshape(-1).tolist() == [int(v) for v in rows["ids"]]
    np.testing.assert_allclose(y[:, :8].reshape(-1), [float.fromhex(v) for v in rows["y_head"]],
                               rtol=0, atol=0)
    np.testing.assert_allclose(y.sum(axis=1), [float.fromhex(v) for v in rows["y_rowsum"]],
                               rtol=1e-15)


def test_pages_shape_facts():
    facts = {}
    with open(os.path.join(GOLDEN, "pages_shapes.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                facts[k] = int(v)
    assert facts["experts_per_layer"] * facts["layers"] == facts["experts_total"]
    for s in (mi.DECODE, mi.PREFILL, mi.SKEWED):
        assert s.E == facts["experts_per_layer"] and s.k == facts["active_per_token"]
    assert mi.DECODE.T == 1 + facts["mtp_drafts"]
    assert mi.PREFILL.T == facts["max_prefill_chunk"]
    assert mi.STACK_PREFILL.layers == facts["layers"]
