#!/usr/bin/env python3
"""Benchmark of the MI355X routed-MoE expert layer (one GPU).

Headline (the default workload): one decode / multi-token-verify step of one MoE layer,
T = 4 tokens (1 + 3 drafts), H = 3072, E = 512 experts, top-10, I = 768, 2-bit block-quantized
experts.  A step is one call of the whole layer (route, group, gate/up + SiLU*mul, down,
weighted combine).  To keep the 256 MB Infinity Cache from serving the ~86 MB of touched
experts, the steps cycle over 16 resident layers (each with its own weights, activations and
logits): a layer's experts are re-read only after ~1.4 GB of other layers' traffic.

Secondary (same JSON line, key "prefill"): one prefill chunk of one layer, T = 8192, same
dimensions; a step is one whole-layer call.  Keys "block_decode" and "prefill.block": the dense
layers on either side of the routed experts (router projection x W_r^T, shared SwiGLU expert),
alone and as the whole block router -> routed layer -> + shared expert.  Key "pruned": the same
decode and prefill legs with 256 experts per layer (the pages' pruned coder variant).  Key
"sweep": the decode path at T = 1 .. 8, the prefill path at T = 1 .. 1024 (crossover) and the
one-call layer's own choice at T = 9 .. 80.

value = whole-job layer-tokens/s = T * steps / timed seconds, inputs resident in HBM.
roofline: HBM-bound decode (touched experts' packed bytes per layer call / call duration, peak
8 TB/s) and MFMA-bound prefill (6*T*k*H*I FLOP per expert-FFN call / call duration, dense fp16
peak 2.5 PFLOP/s), durations from HIP events on the stream the library launches on.
Every timed leg is preceded by ~0.3 s of untimed back-to-back calls (--preroll-s) so that it
measures the GPU's sustained clock rather than its ramp from idle, then by the warmup steps.

cpu_baseline: the CPU oracle (single-threaded C, fp64, one pinned core) on bounded samples: whole
decode layers (the headline workload), token samples of the prefill chunk and the skewed 3-bit
layer, and two layers of the 48-layer stack extrapolated to 48 (key "configs").
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
METRIC = "MoE-layer tokens/s (T=4 decode, T=8192 prefill) + % of HBM/MFMA roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def event_time_ms(fn, steps, stream):
    import torch

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end)


def source_sha256(name):
    import hashlib

    path = os.path.join(ROOT, "bit_expert_ffn_fp32_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def measured_traffic(summary, source):
    """HBM bytes per call from a committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE,
    scaled by a plain copy's counters), or None when the summary is missing or was taken on other
    kernel source."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    if fields.get("source_sha256") != source_sha256(source):
        return None
    try:
        return float(fields["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mb, stream):
    """A plain device-to-device copy of known size, for scaling the memory counters."""
    import torch

    n = mb * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        for _ in range(3):
            dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 copies of {n} bytes")


def preroll(fn, stream, seconds):
    """Runs fn back to back for about `seconds` before a leg's warmup and timed steps (not part of
    either): a GPU that was idle while the inputs were generated ramps its clock up over several
    milliseconds, and a timed region of a few milliseconds would otherwise measure the ramp, not
    the sustained rate (measured: 39.2 vs 37.2 us per decode layer, 1.72 vs 1.53 ms per prefill
    layer)."""
    import torch

    t0 = time.time()
    n = 0
    while time.time() - t0 < seconds:
        for _ in range(8):
            fn(n)
            n += 1
        torch.cuda.synchronize()
    return n


def bench_decode(args, stream, shape=None):
    import torch

    import bit_expert_ffn_fp32_amd as sm
    import moe_inputs as mi
    from gpu_helpers import Layer

    s = mi.DECODE if shape is None else shape
    n_layers = args.decode_layers
    t0 = time.time()
    layers = []
    for l in range(n_layers):
        layers.append(Layer(s, seed=args.seed, layer=l))
        del layers[-1].w_np  # host copy no longer needed
    log(f"decode: {n_layers} layers generated and uploaded in {time.time() - t0:.1f}s")
    ws = layers[0].workspace()
    y = torch.empty((s.T, s.H), dtype=torch.float32, device="cuda")
    touched = []
    for L in layers:
        ids = np.argsort(-L.l_np.astype(np.float64), axis=1, kind="stable")[:, :s.k]
        touched.append(len(np.unique(ids)))
    bytes_per_layer = [n * s.expert_bytes for n in touched]

    def step(i, strm):
        L = layers[i % n_layers]
        sm.strata_moe_layer(L.w, L.x, L.logits, s.k, y, workspace=ws, stream=strm)

    # Eager launches: each call costs ~20 us of host time (Python + ctypes + two kernel launches),
    # which is of the order of the GPU time, so the timed loop replays a HIP graph of one pass over
    # the resident layers instead; the eager rate is reported beside it.
    for i in range(args.warmup):
        step(i, stream)
    eager_ms = event_time_ms(lambda i: step(i, stream), args.steps, stream) / args.steps
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(n_layers):
            step(i, side)
    stream.wait_stream(side)
    torch.cuda.synchronize()

    def capture(first, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream()
            for i in range(first, first + count):
                step(i, cap)
        return g

    # exactly args.steps steps: full passes over the layers, then the remainder
    full, rem = divmod(args.steps, n_layers)
    graph = capture(0, n_layers)
    tail = capture(0, rem) if rem else None
    preroll(lambda i: graph.replay(), stream, args.preroll_s)
    for _ in range(2):
        graph.replay()
    steps = args.steps

    def timed(r):
        if r < full:
            graph.replay()
        else:
            tail.replay()

    ms = event_time_ms(timed, full + (1 if rem else 0), stream)
    ms_per_step = ms / steps
    algo_bytes = (full * sum(bytes_per_layer) + sum(bytes_per_layer[:rem])) / steps
    achieved_gbs = algo_bytes / (ms_per_step * 1e-3) / 1e9
    return {
        "ms_per_step": ms_per_step,
        "steps": steps,
        "eager_ms_per_step": eager_ms,
        "value": s.T / (ms_per_step * 1e-3),
        "touched_experts_mean": float(np.mean(touched)),
        "bytes_per_layer": algo_bytes,
        "preroll_s": args.preroll_s,
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic("decode_t4_traffic.txt", "decode.hip"),
                     "kernel": "strata_moe_decode (route, gate/up GEMV, down GEMV, combine)",
                     "unit_of_work": "touched experts' packed bytes (2,211,840 B each) per layer"},
        "layers": layers,
    }


def bench_block_decode(args, stream, layers):
    """The dense layers around the routed experts at T = 4: router projection (logits = x W_r^T,
    bf16 [E][H]) and the shared SwiGLU expert (bf16 W_sg, W_su [I][H], W_sd [H][I]), each layer
    with its own seeded weights so the 16 resident layers (~270 MB of dense weights) are not
    served from the Infinity Cache.  Graph replays of one pass over the layers: router alone,
    shared expert alone, and the whole block (router -> routed layer -> + shared expert)."""
    import torch

    import bit_expert_ffn_fp32_amd as sm
    import moe_inputs as mi
    from gpu_helpers import to_dev_bf16

    s = mi.DECODE
    n = len(layers)
    wr = [to_dev_bf16(mi.make_router(s, args.seed, l)) for l in range(n)]
    sh = []
    for l in range(n):
        d = mi.make_shared(s, args.seed, l)
        sh.append((to_dev_bf16(d["gate"]), to_dev_bf16(d["up"]), to_dev_bf16(d["down"])))
    logits = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    y = torch.empty((s.T, s.H), dtype=torch.float32, device="cuda")
    ws = layers[0].workspace()
    sws = sm.alloc_workspace(sm.shared_workspace_bytes(s.T, s.I), "cuda")

    def router(i, strm):
        sm.strata_moe_router_logits(layers[i].x, wr[i], logits, stream=strm)

    def shared(i, strm):
        sm.strata_moe_shared_expert(layers[i].x, *sh[i], y, sws, accumulate=True, stream=strm)

    def block(i, strm):
        router(i, strm)
        sm.strata_moe_layer(layers[i].w, layers[i].x, logits, s.k, y, workspace=ws, stream=strm)
        shared(i, strm)

    bws = sm.alloc_workspace(sm.block_workspace_bytes(s.T, s.E, s.k, s.H, s.I, s.I), "cuda")

    def block_fused(i, strm):  # one call: three launches
        sm.strata_moe_block(layers[i].w, layers[i].x, s.k, wr[i], *sh[i], logits, y,
                            workspace=bws, stream=strm)

    def graph_ms(fn):
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(n):
                fn(i, side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream()
            for i in range(n):
                fn(i, cap)
        g.replay()
        reps = max(1, args.steps // n)
        return event_time_ms(lambda r: g.replay(), reps, stream) / (reps * n)

    ms_r, ms_s, ms_b = graph_ms(router), graph_ms(shared), graph_ms(block)
    ms_f = graph_ms(block_fused)
    r_bytes = s.E * s.H * 2 + s.T * s.H * 2
    s_bytes = 3 * s.H * s.I * 2
    out = {
        "T": s.T, "layers_cycled": n,
        "router_us": ms_r * 1e3, "router_GBs": r_bytes / (ms_r * 1e-3) / 1e9,
        "shared_us": ms_s * 1e3, "shared_GBs": s_bytes / (ms_s * 1e-3) / 1e9,
        "block_us": ms_b * 1e3, "block_tokens_per_s": s.T / (ms_b * 1e-3),
        "block_one_call_us": ms_f * 1e3, "block_one_call_tokens_per_s": s.T / (ms_f * 1e-3),
        "unit_of_work": "router: E*H*2 + T*H*2 bytes; shared: 3*H*I*2 bytes of bf16 weights",
    }
    log(f"block decode: router {out['router_us']:.2f} us ({out['router_GBs']:.0f} GB/s), shared "
        f"{out['shared_us']:.2f} us ({out['shared_GBs']:.0f} GB/s), router+layer+shared "
        f"{out['block_us']:.2f} us, one call (strata_moe_block) {out['block_one_call_us']:.2f} us")
    return out


def block_prefill(args, stream, L, ws, y):
    """Router projection and shared expert at T = 8192 (matrix-core GEMMs), and the whole block."""
    import torch

    import bit_expert_ffn_fp32_amd as sm
    import moe_inputs as mi
    from gpu_helpers import to_dev_bf16

    s = L.shape
    wr = to_dev_bf16(mi.make_router(s, args.seed))
    d = mi.make_shared(s, args.seed)
    sh = (to_dev_bf16(d["gate"]), to_dev_bf16(d["up"]), to_dev_bf16(d["down"]))
    logits = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    sws = sm.alloc_workspace(sm.shared_workspace_bytes(s.T, s.I), "cuda")

    def router(i):
        sm.strata_moe_router_logits(L.x, wr, logits, stream=stream)

    def shared(i):
        sm.strata_moe_shared_expert(L.x, *sh, y, sws, accumulate=True, stream=stream)

    def block(i):
        router(i)
        sm.strata_moe_layer(L.w, L.x, logits, s.k, y, workspace=ws, stream=stream)
        shared(i)

    steps = max(3, args.prefill_steps)
    res = {}
    for name, fn in (("router", router), ("shared", shared), ("block", block)):
        fn(0)
        res[name] = event_time_ms(fn, steps, stream) / steps
    f_r = 2.0 * s.T * s.H * s.E
    f_s = 6.0 * s.T * s.H * s.I
    out = {
        "T": s.T,
        "router_us": res["router"] * 1e3, "router_TFLOPs": f_r / (res["router"] * 1e-3) / 1e12,
        "shared_us": res["shared"] * 1e3, "shared_TFLOPs": f_s / (res["shared"] * 1e-3) / 1e12,
        "block_ms": res["block"], "block_tokens_per_s": s.T / (res["block"] * 1e-3),
        "peak_TFLOPs": MFMA_F16_PEAK_TFLOPS,
        "unit_of_work": "router: 2*T*H*E FLOP; shared: 6*T*H*I FLOP (bf16 MFMA, fp32 accumulate)",
    }
    log(f"block prefill: router {out['router_us']:.1f} us ({out['router_TFLOPs']:.0f} TFLOP/s), "
        f"shared {out['shared_us']:.1f} us ({out['shared_TFLOPs']:.0f} TFLOP/s), block "
        f"{out['block_ms']:.3f} ms")
    return out


def bench_sweep(args, stream, layers):
    """Decode / verify T-sweep and the decode-prefill crossover.  For T = 1 .. 8 (MTP verify is
    T = 4, prompt-lookup verify up to T = 6) the layer runs on the decode path and, through the
    staged entry points (route, permute, expert FFN, combine), on the prefill path; the prefill
    path is also timed at T = 16 .. 256.  Each point is a graph replay of one call per resident
    layer (16 layers cycled, each with its own experts, activations and logits)."""
    import torch

    import bit_expert_ffn_fp32_amd as sm
    import moe_inputs as mi
    from gpu_helpers import to_dev, to_dev_bf16

    s = mi.DECODE
    n = len(layers)
    t_dec = list(range(1, 9))
    t_pre = t_dec + [16, 32, 40, 48, 64, 128, 256, 512, 1024]
    tmax = max(t_pre)
    xs = [to_dev_bf16(mi.make_x(s, args.seed, l, tmax)) for l in range(n)]
    lg_np = [mi.make_logits(s, args.seed, l, tmax) for l in range(n)]
    lgs = [to_dev(a) for a in lg_np]
    ws = sm.alloc_workspace(max(sm.workspace_bytes(T, s.E, s.k, s.H, s.I) for T in t_pre), "cuda")
    y = torch.empty((tmax, s.H), dtype=torch.float32, device="cuda")
    S = tmax * s.k
    ids = torch.empty((tmax, s.k), dtype=torch.int32, device="cuda")
    rw = torch.empty((tmax, s.k), dtype=torch.float32, device="cuda")
    counts = torch.empty(s.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(s.E + 1, dtype=torch.int32, device="cuda")
    ss = torch.empty(S, dtype=torch.int32, device="cuda")
    sp = torch.empty(S, dtype=torch.int32, device="cuda")
    out = torch.empty((S, s.H), dtype=torch.int16, device="cuda")

    def decode_path(T):
        def f(i, strm):
            L = layers[i]
            sm.strata_moe_layer(L.w, xs[i][:T], lgs[i][:T], s.k, y[:T], workspace=ws, stream=strm)
        return f

    def prefill_path(T):
        def f(i, strm):
            L = layers[i]
            sm.strata_moe_route(lgs[i][:T], s.k, ids[:T], rw[:T], stream=strm)
            sm.strata_moe_permute(ids[:T], s.E, counts, offsets, ss[:T * s.k], sp[:T * s.k], ws,
                                  stream=strm)
            sm.strata_moe_expert_ffn(L.w, xs[i][:T], s.k, offsets, ss[:T * s.k], out[:T * s.k], ws,
                                     stream=strm)
            sm.strata_moe_combine(out[:T * s.k], rw[:T], y[:T], stream=strm)
        return f

    def graph_us(fn):
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(n):
                fn(i, side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream()
            for i in range(n):
                fn(i, cap)
        g.replay()
        reps = 4
        return event_time_ms(lambda r: g.replay(), reps, stream) / (reps * n) * 1e3

    def touched_bytes(T):
        tot = 0
        for a in lg_np:
            top = np.argsort(-a[:T].astype(np.float64), axis=1, kind="stable")[:, :s.k]
            tot += len(np.unique(top))
        return tot / n * s.expert_bytes

    dec, pre, lay = [], [], []
    for T in (9, 12, 16, 24, 32, 40, 41, 48, 64, 80):  # the layer call's own choice
        us = graph_us(decode_path(T))
        lay.append({"T": T, "us": us, "tokens_per_s": T / (us * 1e-6)})
    for T in t_dec:
        us = graph_us(decode_path(T))
        b = touched_bytes(T)
        dec.append({"T": T, "us": us, "tokens_per_s": T / (us * 1e-6), "GBs": b / (us * 1e-6) / 1e9})
    for T in t_pre:
        us = graph_us(prefill_path(T))
        pre.append({"T": T, "us": us, "tokens_per_s": T / (us * 1e-6)})
    faster = [p["T"] for p, d in zip(pre, dec) if p["us"] < d["us"]]
    out_d = {"decode_path": dec, "prefill_path": pre, "layer_call": lay,
             "crossover_T": min(faster) if faster else None,
             "note": "strata_moe_layer runs the decode path for T <= 8, and on slices of at most "
                     "8 tokens for T <= 32; layer_call times that choice"}
    log("sweep: decode path " + ", ".join(f"T={d['T']} {d['us']:.1f}us" for d in dec))
    log("sweep: prefill path " + ", ".join(f"T={p['T']} {p['us']:.1f}us" for p in pre))
    log("sweep: layer call " + ", ".join(f"T={p['T']} {p['us']:.1f}us" for p in lay))
    del xs, lgs, ws, out
    return out_d


def bench_prefill(args, stream, name):
    import torch

    import bit_expert_ffn_fp32_amd as sm
    import moe_inputs as mi
    from gpu_helpers import Layer

    s = mi.SHAPES[name]
    t0 = time.time()
    L = Layer(s, seed=args.seed)
    del L.w_np
    log(f"{name}: layer generated and uploaded in {time.time() - t0:.1f}s")
    ids_host = np.argsort(-L.l_np.astype(np.float64), axis=1, kind="stable")[:, :s.k]
    touched = len(np.unique(ids_host))
    ws = L.workspace()
    y = torch.empty((s.T, s.H), dtype=torch.float32, device="cuda")
    S = s.T * s.k
    flops = 6.0 * S * s.H * s.I

    def step(i):
        sm.strata_moe_layer(L.w, L.x, L.logits, s.k, y, workspace=ws, stream=stream)

    preroll(step, stream, args.preroll_s)
    for i in range(max(2, args.warmup // 10)):
        step(i)
    steps = args.prefill_steps
    ms = event_time_ms(step, steps, stream)
    ms_per_step = ms / steps
    # the expert-FFN entry point alone (x conversion + up GEMM + down GEMM), on the same stream
    ids = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
    rw = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
    counts = torch.empty(s.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(s.E + 1, dtype=torch.int32, device="cuda")
    ss = torch.empty(S, dtype=torch.int32, device="cuda")
    sp = torch.empty(S, dtype=torch.int32, device="cuda")
    out = torch.empty((S, s.H), dtype=torch.int16, device="cuda")
    sm.strata_moe_route(L.logits, s.k, ids, rw, stream=stream)
    sm.strata_moe_permute(ids, s.E, counts, offsets, ss, sp, ws, stream=stream)

    def ffn(i):
        sm.strata_moe_expert_ffn(L.w, L.x, s.k, offsets, ss, out, ws, stream=stream)

    preroll(ffn, stream, args.preroll_s)
    ms_ffn = event_time_ms(ffn, steps, stream) / steps
    tflops_ffn = flops / (ms_ffn * 1e-3) / 1e12
    tflops_layer = flops / (ms_per_step * 1e-3) / 1e12
    traffic = measured_traffic("prefill_t8192_traffic.txt", "prefill.hip") if name == "prefill" else None
    block = block_prefill(args, stream, L, ws, y) if name == "prefill" and not args.no_block else None
    res = {
        "workload": f"{s.name} T={s.T} H={s.H} E={s.E} k={s.k} I={s.I} "
                    f"{'Q3' if s.fmt == 3 else 'Q2'}-block experts"
                    + (", Zipf(1.1)-skewed routing" if s.zipf else ""),
        "touched_experts": touched,
        "value": s.T / (ms_per_step * 1e-3),
        "unit": "layer-tokens/s",
        "ms_per_step": ms_per_step,
        "steps": steps,
        "layer_tflops": tflops_layer,
        "layer_frac": tflops_layer / MFMA_F16_PEAK_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": tflops_ffn, "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops_ffn / MFMA_F16_PEAK_TFLOPS,
                     "traffic": traffic,
                     "kernel": "strata_moe_expert_ffn (x to fp16, gate/up GEMM, down GEMM)",
                     "ms_per_call": ms_ffn, "unit_of_work": "6*T*k*H*I FLOP per call"},
        "dtype": "f16 MFMA, fp32 accumulate",
    }
    if block is not None:
        res["block"] = block
    return res


def bench_mid(args, stream):
    """Mid-size chunks at the full dims (T = 256 and 1024, 2-bit; about 5 and 20 rows per expert,
    all 512 experts touched): the layer call and the expert-FFN entry point, whose work is
    streaming the touched experts' packed weights (HBM-bound; the skinny GEMMs)."""
    import torch

    import bit_expert_ffn_fp32_amd as sm
    import moe_inputs as mi
    from gpu_helpers import Layer

    res = []
    for name in ("mid256", "mid1024"):
        s = mi.SHAPES[name]
        L = Layer(s, seed=args.seed)
        del L.w_np
        ids_host = np.argsort(-L.l_np.astype(np.float64), axis=1, kind="stable")[:, :s.k]
        touched = len(np.unique(ids_host))
        ws = L.workspace()
        y = torch.empty((s.T, s.H), dtype=torch.float32, device="cuda")
        S = s.T * s.k

        def step(i):
            sm.strata_moe_layer(L.w, L.x, L.logits, s.k, y, workspace=ws, stream=stream)

        preroll(step, stream, args.preroll_s)
        steps = args.prefill_steps
        ms = event_time_ms(step, steps, stream) / steps
        ids = torch.empty((s.T, s.k), dtype=torch.int32, device="cuda")
        rw = torch.empty((s.T, s.k), dtype=torch.float32, device="cuda")
        counts = torch.empty(s.E, dtype=torch.int32, device="cuda")
        offsets = torch.empty(s.E + 1, dtype=torch.int32, device="cuda")
        ss = torch.empty(S, dtype=torch.int32, device="cuda")
        sp = torch.empty(S, dtype=torch.int32, device="cuda")
        out = torch.empty((S, s.H), dtype=torch.int16, device="cuda")
        sm.strata_moe_route(L.logits, s.k, ids, rw, stream=stream)
        sm.strata_moe_permute(ids, s.E, counts, offsets, ss, sp, ws, stream=stream)

        def ffn(i):
            sm.strata_moe_expert_ffn(L.w, L.x, s.k, offsets, ss, out, ws, stream=stream)

        preroll(ffn, stream, args.preroll_s)
        ms_ffn = event_time_ms(ffn, steps, stream) / steps
        gbs = touched * s.expert_bytes / (ms_ffn * 1e-3) / 1e9
        res.append({"workload": f"{s.name} T={s.T} H={s.H} E={s.E} k={s.k} I={s.I} Q2-block experts",
                    "T": s.T, "touched_experts": touched, "ms_per_step": ms,
                    "value": s.T / (ms * 1e-3), "unit": "layer-tokens/s",
                    "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                                 "kernel": "strata_moe_expert_ffn (x to fp16, skinny gate/up and down GEMMs)",
                                 "ms_per_call": ms_ffn,
                                 "unit_of_work": "touched experts' packed bytes per call"}})
        log(f"{name}: layer {ms * 1e3:.1f} us, expert FFN {ms_ffn * 1e3:.1f} us = {gbs:.0f} GB/s "
            f"of the {touched} touched experts ({gbs / HBM_PEAK_GBS * 100:.1f}% of HBM peak)")
        del L, ws, out
        torch.cuda.empty_cache()
    return res


def bench_stack(args, stream):
    """48-layer expert stack, all experts resident: h <- h + MoE(RMSNorm(h)) per layer with fresh
    seeded logits, one T=4 decode step and one T=8192 prefill chunk through all layers."""
    import torch

    import bit_expert_ffn_fp32_amd as sm
    import moe_inputs as mi
    from gpu_helpers import to_dev

    sd, sp = mi.STACK_DECODE, mi.STACK_PREFILL
    n = args.stack_layers
    t0 = time.time()
    weights, lg_dec, lg_pre, touched = [], [], [], []
    for l in range(n):
        w_np = mi.make_weights(sp, args.seed, l)
        weights.append(sm.Weights.from_numpy(w_np, "cuda"))
        del w_np
        ld = mi.make_logits(sd, args.seed, l)
        ids = np.argsort(-ld.astype(np.float64), axis=1, kind="stable")[:, :sd.k]
        touched.append(len(np.unique(ids)))
        lg_dec.append(to_dev(ld))
        lg_pre.append(to_dev(mi.make_logits(sp, args.seed, l)))
    log(f"stack: {n} layers generated and uploaded in {time.time() - t0:.1f}s")
    out = {"layers": n}
    for s, lg, tag in ((sd, lg_dec, "decode"), (sp, lg_pre, "prefill")):
        h = to_dev(mi.make_h0(s, args.seed))
        ws = sm.alloc_workspace(sm.residual_workspace_bytes(s.T, s.E, s.k, s.H, s.I), "cuda")

        def step(strm):
            for l in range(n):
                sm.strata_moe_layer_residual(weights[l], h, lg[l], s.k, ws, eps=1e-6, stream=strm)

        step(stream)
        steps = args.stack_steps if tag == "decode" else max(1, args.stack_steps // 10)
        if tag == "decode":  # replay a graph of the 48-layer step (launch-bound otherwise)
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                step(side)
            stream.wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(torch.cuda.current_stream())
            preroll(lambda i: g.replay(), stream, args.preroll_s)
            ms = event_time_ms(lambda i: g.replay(), steps, stream) / steps
            gbs = sum(touched) * s.expert_bytes / (ms * 1e-3) / 1e9
            out[tag] = {"T": s.T, "ms_per_step": ms, "stack_tokens_per_s": s.T / (ms * 1e-3),
                        "steps": steps, "achieved_GBs": gbs, "frac_hbm": gbs / HBM_PEAK_GBS,
                        "touched_experts_total": sum(touched)}
        else:
            ms = event_time_ms(lambda i: step(stream), steps, stream) / steps
            tf = n * 6.0 * s.T * s.k * s.H * s.I / (ms * 1e-3) / 1e12
            out[tag] = {"T": s.T, "ms_per_step": ms, "stack_tokens_per_s": s.T / (ms * 1e-3),
                        "steps": steps, "achieved_TFLOPs": tf, "frac_mfma": tf / MFMA_F16_PEAK_TFLOPS}
        log(f"stack {tag}: {ms:.3f} ms per {n}-layer step, {s.T / (ms * 1e-3):.4g} stack-tokens/s")
        del h, ws
    return out


def cpu_baseline(args, layers):
    """The oracle (single-threaded C, fp64) on one pinned host core, on a bounded sample of each
    workload: the decode layers of the headline (full layers), token samples of the prefill chunk
    and of the skewed 3-bit layer (tokens are independent in the layer, so a sample's rate is the
    layer's), and two layers of the 48-layer stack (RMSNorm + layer + residual per sampled token,
    extrapolated to 48 layers).  Each entry states its sample."""
    import moe_inputs as mi
    import oracle

    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    affinity = os.sched_getaffinity(0)
    core = min(affinity)
    where = f"{model}; pinned to core {core} of {len(affinity)} available"
    budget = args.cpu_seconds
    out = {}

    def timed(fn):
        os.sched_setaffinity(0, {core})  # the single-threaded oracle on one pinned core
        try:
            t1 = time.perf_counter()
            r = fn()
            return r, time.perf_counter() - t1
        finally:
            os.sched_setaffinity(0, affinity)  # (inputs are generated on every core)

    try:
        # headline workload: whole decode layers (T = 4), as many as fit in a third of the budget
        s = mi.DECODE
        n, t_dec = 0, 0.0
        while n < len(layers) and t_dec < budget / 3:
            w_np = mi.make_weights(s, args.seed, n)
            L = layers[n]
            _, dt = timed(lambda: oracle.layer(w_np, L.x_np, L.l_np, s.k))
            t_dec += dt
            n += 1
        out["decode_t4"] = {"value": n * s.T / t_dec, "unit": "layer-tokens/s",
                            "sample": f"{n} whole decode layers (T=4 each), {t_dec:.1f}s"}
        # prefill chunk and skewed layer: token samples of the benchmark's own inputs
        for name, ntok in (("prefill", 16), ("skewed", 8)):
            sh = mi.SHAPES[name]
            w_np = mi.make_weights(sh, args.seed)
            x = mi.make_x(sh, args.seed)
            lg = mi.make_logits(sh, args.seed)
            rows = np.random.default_rng(17).choice(sh.T, size=ntok, replace=False)
            _, dt = timed(lambda: oracle.layer_rows(w_np, x, lg, sh.k, rows))
            out[name] = {"value": ntok / dt, "unit": "layer-tokens/s",
                         "sample": f"{ntok} of the T={sh.T} tokens, {dt:.1f}s"}
            del w_np, x, lg
        # 48-layer stack: two layers on a token sample, extrapolated to 48
        for tag, sh, ntok in (("stack_prefill", mi.STACK_PREFILL, 8), ("stack_decode", mi.STACK_DECODE, 4)):
            h = mi.make_h0(sh, args.seed)
            rows = np.arange(ntok) if sh.T == ntok else np.random.default_rng(19).choice(sh.T, size=ntok, replace=False)
            hs = h[rows].astype(np.float32)
            t_st = 0.0
            for l in range(2):
                w_np = mi.make_weights(sh, args.seed, l)
                lg = mi.make_logits(sh, args.seed, l)[rows]

                def one():
                    xr = oracle.rmsnorm(hs, 1e-6)
                    return oracle.layer(w_np, xr, lg, sh.k)

                y, dt = timed(one)
                hs = (hs.astype(np.float64) + y).astype(np.float32)
                t_st += dt
                del w_np
            per_step = t_st / 2 * sh.layers
            out[tag] = {"value": ntok / per_step, "unit": "stack-tokens/s",
                        "sample": f"{ntok} tokens through 2 of the {sh.layers} layers ({t_st:.1f}s), "
                                  f"extrapolated x{sh.layers // 2}"}
    finally:
        os.sched_setaffinity(0, affinity)
    head = out["decode_t4"]
    cpu = {"value": head["value"], "unit": "layer-tokens/s", "cores": 1, "kind": "oracle",
           "cpu": where, "sample": head["sample"], "configs": out}
    log("cpu oracle: " + ", ".join(f"{k} {v['value']:.3g} {v['unit']}" for k, v in out.items()))
    return cpu


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--decode-layers", type=int, default=16)
    p.add_argument("--prefill-steps", type=int, default=20)
    p.add_argument("--preroll-s", type=float, default=0.3,
                   help="seconds of untimed back-to-back calls before each leg's warmup")
    p.add_argument("--no-skewed", action="store_true")
    p.add_argument("--no-stack", action="store_true")
    p.add_argument("--stack-layers", type=int, default=48)
    p.add_argument("--stack-steps", type=int, default=20)
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-mid", action="store_true",
                   help="skip the mid-size chunks (T = 256 and 1024)")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the decode T-sweep and the decode-prefill crossover")
    p.add_argument("--no-pruned", action="store_true",
                   help="skip the 256-expert (pruned) variant")
    p.add_argument("--no-block", action="store_true",
                   help="skip the router projection / shared expert measurements")
    p.add_argument("--copy-calibration-mb", type=int, default=0,
                   help="also run a plain copy of this many MiB (for scaling memory counters)")
    args = p.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); every layer's "
              "experts fit in one MI355X's HBM and the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_expert_ffn_fp32_amd as sm
    import moe_inputs as mi
    import oracle

    sm.lib()  # fail loudly if the HIP library is missing
    torch.cuda.init()
    stream = torch.cuda.current_stream()
    dec = bench_decode(args, stream)
    log(f"decode: {dec['ms_per_step'] * 1e3:.2f} us/layer (graph replay; eager "
        f"{dec['eager_ms_per_step'] * 1e3:.2f} us), {dec['value']:.4g} layer-tokens/s, "
        f"{dec['roofline']['achieved']:.0f} GB/s ({dec['roofline']['frac'] * 100:.1f}% of HBM peak)")
    layers = dec.pop("layers")
    blk = None if args.no_block else bench_block_decode(args, stream, layers)
    torch.cuda.empty_cache()
    sweep = None if args.no_sweep else bench_sweep(args, stream, layers)
    torch.cuda.empty_cache()
    pruned = None
    if not args.no_pruned:  # the pages' pruned coder variant: 256 experts per layer
        for L in layers:
            del L.w
        torch.cuda.empty_cache()
        pd = bench_decode(args, stream, mi.PRUNED_DECODE)
        for L in pd.pop("layers"):
            del L.w
        torch.cuda.empty_cache()
        pruned = {"decode": {k: pd[k] for k in ("ms_per_step", "value", "touched_experts_mean")},
                  "decode_roofline": pd["roofline"]}
        pruned["decode"]["unit"] = "layer-tokens/s"
        pruned["decode_roofline"]["traffic"] = None
        log(f"pruned decode (E=256): {pd['ms_per_step'] * 1e3:.2f} us/layer, "
            f"{pd['roofline']['achieved']:.0f} GB/s")
        if not args.no_prefill:
            pp = bench_prefill(args, stream, "pruned_prefill")
            pruned["prefill"] = {k: pp[k] for k in ("workload", "value", "unit", "ms_per_step",
                                                    "layer_tflops", "roofline")}
            log(f"pruned prefill (E=256): {pp['ms_per_step']:.3f} ms/layer, expert FFN "
                f"{pp['roofline']['achieved']:.0f} TFLOP/s")
            torch.cuda.empty_cache()
    pre = skw = None
    if not args.no_prefill:
        for L in layers:
            if hasattr(L, "w"):
                del L.w
        torch.cuda.empty_cache()
        pre = bench_prefill(args, stream, "prefill")
        log(f"prefill: {pre['ms_per_step']:.3f} ms/layer, {pre['value']:.4g} tokens/s, layer "
            f"{pre['layer_tflops']:.0f} TFLOP/s; expert FFN {pre['roofline']['achieved']:.0f} TFLOP/s "
            f"({pre['roofline']['frac'] * 100:.1f}% of MFMA peak)")
        if not args.no_skewed:
            skw = bench_prefill(args, stream, "skewed")
            log(f"skewed: {skw['ms_per_step']:.3f} ms/layer, {skw['touched_experts']} experts touched, "
                f"expert FFN {skw['roofline']['achieved']:.0f} TFLOP/s")
            torch.cuda.empty_cache()
    mid = None
    if not args.no_mid:
        for L in layers:
            if hasattr(L, "w"):
                del L.w
        torch.cuda.empty_cache()
        mid = bench_mid(args, stream)
    stack = None
    if not args.no_stack:
        stack = bench_stack(args, stream)
        torch.cuda.empty_cache()
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb, stream)
    cpu = None if args.no_cpu else cpu_baseline(args, layers)
    s = mi.DECODE
    line = {
        "metric": METRIC,
        "value": dec["value"],
        "unit": "layer-tokens/s",
        "n_gpus": 1,
        "steps": dec["steps"],
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"],
        "eager_ms_per_step": dec["eager_ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Philox inputs, random-init 2-bit experts)",
        "config": {"workload": f"decode/verify step of one MoE layer: T={s.T} (1+3 drafts), "
                               f"H={s.H}, E={s.E}, top-{s.k}, I={s.I}, Q2-block experts; "
                               f"{args.decode_layers} resident layers cycled",
                   "T": s.T, "H": s.H, "E": s.E, "k": s.k, "I": s.I, "format": "Q2_B32",
                   "touched_experts_mean": dec["touched_experts_mean"],
                   "parallelism": "single GPU"},
        "roofline": dec["roofline"],
        "cpu_baseline": cpu,
    }
    if blk is not None:
        line["block_decode"] = blk
    if pruned is not None:
        line["pruned"] = pruned
    if sweep is not None:
        line["sweep"] = sweep
    if pre is not None:
        line["prefill"] = pre
    if skw is not None:
        line["skewed"] = skw
    if mid is not None:
        line["mid"] = mid
    if stack is not None:
        line["stack"] = stack
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
