"""The seeded input generator: Philox4x32-10 against its published known answers, the storage
roundings against numpy's, and the stream layout (distinct tensors draw distinct streams)."""
import os

import numpy as np

import moe_inputs as mi

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_philox_known_answers():
    n = 0
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            v = [int(t, 16) for t in line.split()]
            assert list(mi.philox4x32_10(v[0:4], v[4:6])) == v[6:10]
            n += 1
    assert n == 3


def test_f32_to_bf16_round_to_nearest_even():
    rng = np.random.default_rng(0)
    f = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0, -0.0,
                                  3.0e38, 1e-40], dtype=np.float32)])
    got = mi.f32_to_bf16_bits(f)
    # reference: exact rational rounding via float64 of the two candidates
    lo = (f.view(np.uint32) >> 16).astype(np.uint16)
    hi = lo + 1
    vlo = mi.bf16_bits_to_f32(lo).astype(np.float64)
    vhi = mi.bf16_bits_to_f32(hi).astype(np.float64)
    x = f.astype(np.float64)
    dlo, dhi = np.abs(x - vlo), np.abs(vhi - x)
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    assert np.array_equal(got, want)


def test_f32_to_f16_matches_numpy():
    rng = np.random.default_rng(1)
    f = np.concatenate([(rng.standard_normal(50000) * 0.02).astype(np.float32),
                        (rng.standard_normal(5000) * 1e-6).astype(np.float32),
                        np.float32([65504, 65519.99, 65520, 1e6, 2**-24, 2**-25, 3 * 2**-26, 0])])
    assert np.array_equal(mi.f32_to_f16_bits(f), f.astype(np.float16).view(np.uint16))


def test_streams_are_distinct_and_reproducible():
    a = mi.random_bytes(0, mi.stream_id(0, mi.TAG_GATE_CODES), 4096)
    b = mi.random_bytes(0, mi.stream_id(0, mi.TAG_UP_CODES), 4096)
    c = mi.random_bytes(0, mi.stream_id(1, mi.TAG_GATE_CODES), 4096)
    d = mi.random_bytes(1, mi.stream_id(0, mi.TAG_GATE_CODES), 4096)
    assert np.array_equal(a, mi.random_bytes(0, mi.stream_id(0, mi.TAG_GATE_CODES), 4096))
    for o in (b, c, d):
        assert np.mean(a == o) < 0.02
    # a prefix of a longer draw is the shorter draw (counter-based)
    assert np.array_equal(mi.random_bytes(0, 77, 100), mi.random_bytes(0, 77, 1000)[:100])


def test_distributions():
    z = mi.normal_f32(0, 123, 200000).astype(np.float64)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    s = mi.abs_normal_f16(0, 124, 200000, 0.02).view(np.float16).astype(np.float64)
    assert np.all(s >= 0) and abs(s.mean() - 0.02 * np.sqrt(2 / np.pi)) < 2e-4
    codes = mi.random_bytes(0, 125, 100000)
    q = (codes[:, None] >> (2 * np.arange(4))) & 3
    assert np.all(np.abs(np.bincount(q.reshape(-1), minlength=4) / q.size - 0.25) < 0.01)


def test_zipf_skew():
    s = mi.SKEWED
    logits = mi.make_logits(s, T=2048)
    top = np.argsort(-logits, axis=1, kind="stable")[:, :s.k]
    counts = np.bincount(top.reshape(-1), minlength=s.E)
    assert counts.max() >= 0.9 * 2048       # the hottest experts take (almost) every token
    assert (counts == 0).sum() > 300         # most experts get no token
    assert counts.sum() == 2048 * s.k


def test_layer_sizes():
    assert mi.DECODE.expert_bytes == 2211840
    assert mi.PREFILL.layer_bytes == 1132462080
    assert mi.SKEWED.layer_bytes == 1585446912
    assert mi.TINY.layer_bytes == 1966080
