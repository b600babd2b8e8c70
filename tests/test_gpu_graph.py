"""Graph capture of the layer entry point: a captured decode-path call and a captured prefill-path
call, each replayed several times with other GPU work and synchronizations in between, give
exactly the eager result on every replay (the benchmark times graph replays)."""
import pytest
import torch

import bit_expert_ffn_fp32_amd as sm
import moe_inputs as mi
from gpu_helpers import Layer, dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [4, 16])
def test_graph_replay_matches_eager(T):
    s = mi.TINY
    L = Layer(s, T=T)
    ws = L.workspace()
    y_eager = torch.empty((T, s.H), dtype=torch.float32, device=dev())
    sm.strata_moe_layer(L.w, L.x, L.logits, s.k, y_eager, workspace=ws)
    torch.cuda.synchronize()
    y = torch.zeros_like(y_eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sm.strata_moe_layer(L.w, L.x, L.logits, s.k, y, workspace=ws, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sm.strata_moe_layer(L.w, L.x, L.logits, s.k, y, workspace=ws,
                            stream=torch.cuda.current_stream())
    for rep in range(3):
        y.fill_(float("nan"))
        scratch = torch.randn(1 << 16, device=dev()).sum()  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {rep} differs from the eager result"
        del scratch


@pytest.mark.parametrize("T,one_call", [(4, False), (40, False), (4, True), (40, True)])
def test_graph_replay_of_the_block_matches_eager(T, one_call):
    """Router projection -> routed layer -> + shared expert captured in one graph, as three entry
    points or as strata_moe_block: every replay equals the eager result (the benchmark replays
    such graphs)."""
    import moe_inputs as mi
    from gpu_helpers import to_dev_bf16

    s = mi.TINY
    L = Layer(s, T=T)
    ws = L.workspace()
    wr = to_dev_bf16(mi.make_router(s))
    sh = mi.make_shared(s)
    g_, u_, d_ = (to_dev_bf16(sh[n]) for n in ("gate", "up", "down"))
    sws = sm.alloc_workspace(sm.shared_workspace_bytes(T, s.I), dev())
    logits = torch.empty((T, s.E), dtype=torch.float32, device=dev())

    bws = sm.alloc_workspace(sm.block_workspace_bytes(T, s.E, s.k, s.H, s.I, s.I), dev())

    def block(y, strm):
        if one_call:
            sm.strata_moe_block(L.w, L.x, s.k, wr, g_, u_, d_, logits, y, workspace=bws,
                                stream=strm)
            return
        sm.strata_moe_router_logits(L.x, wr, logits, stream=strm)
        sm.strata_moe_layer(L.w, L.x, logits, s.k, y, workspace=ws, stream=strm)
        sm.strata_moe_shared_expert(L.x, g_, u_, d_, y, sws, accumulate=True, stream=strm)

    y_eager = torch.empty((T, s.H), dtype=torch.float32, device=dev())
    block(y_eager, torch.cuda.current_stream())
    torch.cuda.synchronize()
    y = torch.zeros_like(y_eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        block(y, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        block(y, torch.cuda.current_stream())
    for rep in range(3):
        y.fill_(float("nan"))
        logits.fill_(float("nan"))
        scratch = torch.randn(1 << 16, device=dev()).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {rep} differs from the eager result"
        del scratch
