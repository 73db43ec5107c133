"""Prefill (every kernel family), segment checkpoints, OSDN phase 1, the
Memory-Caching read-out and the delta-mem pass inside captured HIP graphs.  The library allocates
nothing, clears nothing with memsets and launches only its own kernels, so a call
made on a capturing stream is recorded whole.  Each case captures one call, then
replays the graph three times with eager work between the replays, and every
replay must equal, bit for bit, the same call run eagerly (the kernels are
deterministic)."""
import numpy as np
import pytest

import gdr_inputs as gi
from tests.gpu_util import gpu, log, upload

pytestmark = pytest.mark.gpu


def _capture(torch, fn):
    """Capture fn() on a side stream; returns (graph, whatever fn returned)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            res = fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return graph, res


def _replay_and_compare(torch, graph, graph_out, eager, name):
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        ref = eager()
        torch.cuda.synchronize()
        same = [torch.equal(a, b) for a, b in zip(graph_out, ref)]
        log(f"[graph {name}] replay {rep}: outputs equal {same}")
        assert all(same)
        _ = sum(float(t.float().abs().sum().item()) for t in ref)  # eager work between replays


PREFILL_CASES = {
    "gdn_mfma_ragged": dict(base=gi.GDN_PREFILL, B=2, T=300, H=3, seed=120),
    "kda_fg2plus_general_gates": dict(base=gi.KDA_FG2PLUS_PREFILL, B=1, T=200, H=2, seed=121),
    "osdn_write_key_S0": dict(base=gi.OSDN_LONG_PREFILL, B=1, T=257, H=2, seed=122),
    "valu_f32_d64": dict(base=gi.GDN_PREFILL, B=1, T=130, H=2, dk=64, dv=64, io=gi.F32, seed=123),
    # few heads, 258 chunks walked in order
    "osdn_long_T16500": dict(base=gi.OSDN_LONG_PREFILL, B=1, T=16500, H=2, seed=127),
}


@pytest.mark.parametrize("case", list(PREFILL_CASES))
def test_prefill_graph_replays_equal_eager(case):
    torch, g = gpu()
    spec = dict(PREFILL_CASES[case])
    w = spec.pop("base").scaled(**spec)
    d = upload(gi.make_prefill(w), w)
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta_k"])
    kw = dict(k_w=d.get("k_w"), beta_v=d.get("beta_v"), S0=d.get("S0"))
    o_g = torch.empty(w.B, w.T, w.H, w.dv, dtype=d["q"].dtype, device="cuda")
    S_g = torch.empty(w.B, w.H, w.dk, w.dv, dtype=torch.float32, device="cuda")
    desc = g.make_desc(d["q"], d["v"], d["alpha"], d["beta_k"], d.get("beta_v"))
    need = g.gdr_chunk_fwd_workspace_size(desc)
    ws_g = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    graph, _ = _capture(torch, lambda: g.chunk_fwd(*args, **kw, out=o_g, final_state=S_g, workspace=ws_g))
    _replay_and_compare(torch, graph, (o_g, S_g), lambda: g.chunk_fwd(*args, **kw), case)


def test_prefill_with_context_graph_replays_equal_eager():
    """A long prefill with an execution context: the prep of each chunk block is forked
    onto the context's second stream and every state launch waits for its block's event,
    all recorded in the one graph."""
    torch, g = gpu()
    w = gi.OSDN_LONG_PREFILL.scaled(B=1, T=16500, H=2, seed=129)
    d = upload(gi.make_prefill(w), w)
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta_k"])
    kw = dict(k_w=d["k_w"], S0=d["S0"])
    ctx = g.Context()
    o_g = torch.empty(w.B, w.T, w.H, w.dv, dtype=d["q"].dtype, device="cuda")
    S_g = torch.empty(w.B, w.H, w.dk, w.dv, dtype=torch.float32, device="cuda")
    desc = g.make_desc(d["q"], d["v"], d["alpha"], d["beta_k"], None)
    ws_g = torch.empty(g.gdr_chunk_fwd_workspace_size(desc), dtype=torch.uint8, device="cuda")
    graph, _ = _capture(torch, lambda: g.chunk_fwd(*args, **kw, out=o_g, final_state=S_g, workspace=ws_g,
                                                   ctx=ctx))
    _replay_and_compare(torch, graph, (o_g, S_g), lambda: g.chunk_fwd(*args, **kw), "prefill context")


def test_checkpointed_prefill_graph_replays_equal_eager():
    torch, g = gpu()
    w = gi.GDN_PREFILL.scaled(B=1, T=520, H=2, seed=124)
    d = upload(gi.make_prefill(w), w)
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta_k"], 128)
    graph, res = _capture(torch, lambda: g.chunk_fwd_ckpt(*args))
    _replay_and_compare(torch, graph, res, lambda: g.chunk_fwd_ckpt(*args), "ckpt")


# T = 16,500 with an execution context: the chunks are cut into blocks, with the chunk
# solve and the emission forked onto the context's second stream and joined back
# through events
@pytest.mark.parametrize("T,use_ctx", [(700, False), (16500, False), (16500, True)])
def test_osdn_precond_graph_replays_equal_eager(T, use_ctx):
    torch, g = gpu()
    w = gi.OSDN_LONG_PREFILL.scaled(B=1, T=T, H=3, seed=125)
    x = gi.make_prefill(w)
    k = gi.to_torch(x["k"], w.io)
    beta = gi.to_torch(x["beta_k"], w.gate)
    r = gi.to_torch(gi.make_retention(w), w.gate)
    ctx = g.Context() if use_ctx else None
    graph, res = _capture(torch, lambda: g.osdn_precond(k, beta, 0.05, r=r, ctx=ctx))
    _replay_and_compare(torch, graph, res, lambda: g.osdn_precond(k, beta, 0.05, r=r, ctx=ctx),
                        f"osdn_precond T={T} context={use_ctx}")


def test_mc_readout_graph_replays_equal_eager():
    torch, g = gpu()
    w = gi.MC_LONG_GRM.scaled(B=1, T=600, H=2, seg=128, seed=126)
    x = gi.make_cache_readout(w)
    q = gi.to_torch(x["q"], gi.BF16)
    ckpt = gi.to_torch(x["ckpt"], gi.F32)
    gates = gi.to_torch(x["gates"], gi.F32)
    o_in = gi.to_torch(x["o_in"], gi.BF16)
    o_g = torch.empty_like(o_in)
    graph, _ = _capture(torch, lambda: g.mc_readout(q, ckpt, w.seg, gates=gates, o_in=o_in, out=o_g))
    _replay_and_compare(torch, graph, (o_g,), lambda: (g.mc_readout(q, ckpt, w.seg, gates=gates, o_in=o_in),),
                        "mc_readout")


@pytest.mark.parametrize("seg", [False, True], ids=["token_writes", "segment_writes"])
def test_dmem_pass_graph_replays_equal_eager(seg):
    """The delta-mem pass (memories updated in place) captured in a graph: before each
    replay the memories are reset from M0 outside the graph; every replay's reads and
    memories equal an eager call on a copy of M0, bit for bit."""
    import numpy as np

    torch, g = gpu()
    w = gi.DMEM_MSW.scaled(B=40, T=70, H=8, J=4, seg_mean=5.0 if seg else 0.0, seed=128)
    x = gi.make_dmem_seq(w)
    q, k, v = (gi.to_torch(x[n], w.io) for n in ("q", "k", "v"))
    lam, beta = gi.to_torch(x["lam"], w.gate), gi.to_torch(x["beta"], w.gate)
    se = torch.from_numpy(np.ascontiguousarray(x["seg_end"])).cuda() if seg else None
    M0 = gi.to_torch(x["M0"], gi.F32)
    M_g = M0.clone()
    out_g = torch.empty((w.B, w.T, w.H // w.J, w.r), dtype=q.dtype, device="cuda")
    graph, _ = _capture(torch, lambda: g.dmem_fwd(M_g, q, k, v, lam, beta, seg_end=se, J=w.J, out=out_g))
    for rep in range(3):
        M_g.copy_(M0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        M_e = M0.clone()
        out_e = g.dmem_fwd(M_e, q, k, v, lam, beta, seg_end=se, J=w.J)
        torch.cuda.synchronize()
        same = (torch.equal(out_g, out_e), torch.equal(M_g, M_e))
        log(f"[graph dmem seg={seg}] replay {rep}: reads, memories equal {same}")
        assert all(same)
