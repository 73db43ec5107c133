"""Sparse Delta Memory inside a captured HIP graph: a call of T >= 1024 given an
execution context forks its selection onto the context's second stream and joins
back through events, which a capture of the caller's stream takes in.  Each replay (with eager work between the
replays) must equal, bit for bit, the same call run eagerly on a copy of the table."""
import numpy as np
import pytest

import gdr_inputs as gi
from tests.gpu_util import gpu, log

pytestmark = pytest.mark.gpu


def test_sdm_graph_replays_equal_eager_calls():
    torch, g = gpu()
    w = gi.SDM_B4H16.scaled(B=1, T=1100, H=2, n=32, W=8, R=8, seed=110)
    x = gi.make_sparse_memory(w)
    ks, qs = gi.to_torch(x["ks"], gi.F32), gi.to_torch(x["qs"], gi.F32)
    v = gi.to_torch(x["v"], w.io)
    a, b = gi.to_torch(x["alpha"], w.gate), gi.to_torch(x["beta"], w.gate)
    M_graph = gi.to_torch(x["M0"], gi.F32)
    M_eager = M_graph.clone()
    desc = g.Desc(B=w.B, T=w.T, H=w.H, dk=128, dv=128, chunk=64, io_dtype=g.GDR_BF16, gate_dtype=g.GDR_F32,
                  alpha_mode=0, beta_mode=0, flags=0)
    need = g.gdr_sdm_workspace_size(desc, w.n, w.W, w.R)
    ws_graph = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws_eager = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_graph = torch.empty_like(v)
    o_eager = torch.empty_like(v)

    ctx = g.Context()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            rc = g.gdr_sdm_fwd(desc, w.n, w.W, w.R, ks, qs, v, a, b, M_graph, o_graph, None, None, ws_graph, need,
                               ctx=ctx, stream=side)
    assert rc == g.GDR_OK
    torch.cuda.synchronize()
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        rc = g.gdr_sdm_fwd(desc, w.n, w.W, w.R, ks, qs, v, a, b, M_eager, o_eager, None, None, ws_eager, need)
        assert rc == g.GDR_OK
        torch.cuda.synchronize()
        same_o = torch.equal(o_graph, o_eager)
        same_m = torch.equal(M_graph, M_eager)
        log(f"[sdm graph] replay {rep}: o equal {same_o}, table equal {same_m}")
        assert same_o and same_m
        _ = (v.float() * 2).sum().item()  # eager work between the replays
