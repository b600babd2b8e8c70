"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

* decode:  T=4,    H=3072, E=512, k=10, I=768, 2-bit: every output row against the oracle.
* prefill: T=8192, same dims: routing, counts, offsets and permutation bit-exact over all 81,920
           slots; layer output rows on a seeded sample of tokens (the oracle computes those rows
           one by one; tokens are independent in the layer).
* skewed:  T=2048, 3-bit, Zipf-biased routing: same checks.
* mid-size chunks at the full dims (T = 256 and 1024, 2-bit; T = 512, 3-bit): about 5, 20 and 10
           rows per expert, the skinny GEMMs with their activation rows staged in one or in
           several phases of the reduction; same checks.
* stack:   two layers of h <- h + MoE(RMSNorm(h)) at the prefill shape, each layer checked
           teacher-forced (the oracle gets the GPU's h and x of that layer).
"""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import replace

import numpy as np
import pytest
import torch

import bit_expert_ffn_fp32_amd as sm
import moe_inputs as mi
import oracle
from gpu_helpers import TOL_REL_L2, Layer, dev, rel_l2_rows, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def log(msg):
    print(msg, flush=True)


CHUNK_ROWS, FRAG = 224, 32  # rows of one grouped-GEMM work unit, rows of a matrix-core fragment
SMALL_CHUNK_ROWS = 64        # the most rows of an expert whose segment is one small-fragment unit


def oracle_rows(w_np, x_np, l_np, k, rows):
    """oracle.layer_rows over many tokens on the host's cores (the C call releases the GIL; the
    rows are independent)."""
    rows = np.asarray(rows)
    n = max(1, min(16, os.cpu_count() or 1))
    parts = [p for p in np.array_split(rows, n) if p.size]
    with ThreadPoolExecutor(len(parts)) as ex:
        out = list(ex.map(lambda r: oracle.layer_rows(w_np, x_np, l_np, k, r), parts))
    return np.concatenate(out)


def coverage_rows(counts, offsets, sorted_slot, k, rng, n_random):
    """Tokens whose rows reach every expert's first and last (ragged) fragment and both ends of
    every GEMM work unit (an expert's segment is one chunk of the small-fragment GEMMs when it has
    at most 64 rows and the slots average at most 128 rows per expert, else chunks of at most 224
    rows, split into balanced 32-row fragments), plus random tokens."""
    pos = []
    small_rows = SMALL_CHUNK_ROWS if len(sorted_slot) <= 128 * len(counts) else 0
    for e in np.nonzero(counts)[0]:
        cnt, row = int(counts[e]), int(offsets[e])
        nfrag = -(-cnt // FRAG)
        nch = 1 if cnt <= small_rows else -(-nfrag // (CHUNK_ROWS // FRAG))
        fb, extra = divmod(nfrag, nch)
        used = 0
        for c in range(nch):
            nf = fb + (1 if c < extra else 0)
            rows = min(nf * FRAG, cnt - used * FRAG)
            pos += [row, row + rows - 1, row + rows - 1 - (rows - 1) % FRAG]  # ends, last fragment
            row += rows
            used += nf
    tokens = set(int(sorted_slot[p]) // k for p in pos)
    tokens |= set(int(t) for t in rng.choice(len(sorted_slot) // k, size=n_random, replace=False))
    return np.array(sorted(tokens))


def run_layer(L: Layer, x=None, logits=None, y=None, accumulate=False, perm=None):
    s, T = L.shape, L.T
    S = T * s.k
    x = L.x if x is None else x
    logits = L.logits if logits is None else logits
    y = torch.empty((T, s.H), dtype=torch.float32, device=dev()) if y is None else y
    ids = torch.empty((T, s.k), dtype=torch.int32, device=dev())
    rw = torch.empty((T, s.k), dtype=torch.float32, device=dev())
    extra = {}
    if (T > 8) if perm is None else perm:
        extra = dict(counts=torch.empty(s.E, dtype=torch.int32, device=dev()),
                     offsets=torch.empty(s.E + 1, dtype=torch.int32, device=dev()),
                     sorted_slot=torch.empty(S, dtype=torch.int32, device=dev()))
    sm.strata_moe_layer(L.w, x, logits, s.k, y, accumulate=accumulate, topk_ids=ids, topk_w=rw,
                        workspace=L.workspace(), **extra)
    torch.cuda.synchronize()
    return y, ids, rw, extra


@pytest.mark.parametrize("T", [1, 4, 6, 8, 20])
def test_decode_full_size(T):
    """T = 4: MTP verify (1 + 3 drafts); T = 6: prompt-lookup verify (1 + 5 drafts); T = 20: the
    decode path on slices of at most 8 tokens."""
    log(f"decode full size T={T}: generating")
    L = Layer(mi.DECODE, T=T)
    y, ids, rw, _ = run_layer(L, perm=False)
    y_ref, ids_ref, w_ref, _, _ = oracle.layer(L.w_np, L.x_np, L.l_np, 10, intermediates=True)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    err = rel_l2_rows(y.cpu().numpy(), y_ref)
    log(f"decode full size max rel-L2 {err.max():.3e}")
    assert err.max() <= TOL_REL_L2


MID_SHAPES = {"mid512_q3": replace(mi.PREFILL, name="mid512_q3", T=512, fmt=mi.Q3)}


@pytest.mark.parametrize("name,n_rows", [("prefill", 256), ("skewed", 128), ("mid256", 64),
                                         ("mid1024", 64), ("mid512_q3", 64)])
def test_prefill_full_size(name, n_rows):
    s = MID_SHAPES[name] if name in MID_SHAPES else mi.SHAPES[name]
    log(f"{name} full size: generating")
    L = Layer(s)
    y, ids, rw, extra = run_layer(L)
    ids_ref, w_ref = oracle.route(L.l_np, s.k)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(rw.cpu().numpy(), w_ref, rtol=1e-6)
    counts, offsets, ss, _ = oracle.permute(ids_ref, s.E)
    assert np.array_equal(extra["counts"].cpu().numpy(), counts)
    assert np.array_equal(extra["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(extra["sorted_slot"].cpu().numpy(), ss)
    rows = coverage_rows(counts, offsets, ss, s.k, np.random.default_rng(2024), n_rows)
    y_ref = oracle_rows(L.w_np, L.x_np, L.l_np, s.k, rows)
    err = rel_l2_rows(y.cpu().numpy()[rows], y_ref)
    log(f"{name} full size: sampled rows {len(rows)}, max rel-L2 {err.max():.3e}")
    assert err.max() <= TOL_REL_L2
    y2, _, _, _ = run_layer(L)
    assert torch.equal(y, y2), "second call differs"


def test_stack_two_layers_teacher_forced():
    s = mi.PREFILL
    h = to_dev(mi.make_h0(s))
    x = torch.empty((s.T, s.H), dtype=torch.int16, device=dev())
    rows = np.random.default_rng(7).choice(s.T, size=64, replace=False)
    for layer in range(2):
        log(f"stack layer {layer}: generating")
        L = Layer(s, layer=layer)
        h_in = h.cpu().numpy()
        sm.strata_moe_rmsnorm(h, x, 1e-6)
        torch.cuda.synchronize()
        x_np = x.cpu().numpy().view(np.uint16)
        x_ref = oracle.rmsnorm(h_in, 1e-6)
        d = np.abs(x_np.astype(np.int32) - x_ref.astype(np.int32))
        assert d.max() <= 1 and np.mean(d == 0) > 0.999
        run_layer(L, x=x, y=h, accumulate=True)
        y_rows = h.cpu().numpy()[rows] - h_in[rows]
        y_ref = oracle_rows(L.w_np, x_np, L.l_np, s.k, rows)  # teacher-forced on the GPU's x
        err = rel_l2_rows(y_rows, y_ref)
        log(f"stack layer {layer}: max rel-L2 {err.max():.3e}")
        assert err.max() <= TOL_REL_L2
