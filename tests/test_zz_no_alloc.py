"""gdr_chunk_fwd_noalloc (the prefill entry point that allocates nothing, its per-chunk
record in the library's static scratch array) against gdr_chunk_fwd with a caller
workspace, through the C-ABI: two calls in a row on one device, the second smaller
than the first (the array keeps the first call's contents), then a general-gate call,
a call on the vector-ALU path (no scratch needed) and a capture in a HIP graph.  The
two entry points run the same kernels, so their outputs must be equal bit for bit;
each is also held to the oracle's tolerance."""
import pytest

import gdr_inputs as gi
import oracle
from tests.gpu_util import TOL, gpu, log, to_np, upload

pytestmark = pytest.mark.gpu


def _both(w, x):
    torch, g = gpu()
    d = upload(x, w)
    desc = g.make_desc(d["q"], d["v"], d["alpha"], d["beta_k"], d["beta_v"], chunk=w.chunk)
    args = (d["q"], d["k"], d["k_w"], d["v"], d["alpha"], d["beta_k"], d["beta_v"], d["S0"])
    o_n = torch.empty(w.B, w.T, w.H, w.dv, dtype=d["q"].dtype, device="cuda")
    S_n = torch.empty(w.B, w.H, w.dk, w.dv, dtype=torch.float32, device="cuda")
    rc = g.gdr_chunk_fwd_noalloc(desc, *args, o_n, S_n)
    assert rc == g.GDR_OK, g.gdr_status_string(rc)
    o_w, S_w = torch.empty_like(o_n), torch.empty_like(S_n)
    need = g.gdr_chunk_fwd_workspace_size(desc)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    rc = g.gdr_chunk_fwd(desc, *args, o_w, S_w, ws, need)
    assert rc == g.GDR_OK, g.gdr_status_string(rc)
    torch.cuda.synchronize()
    return desc, d, (o_n, S_n), (o_w, S_w)


def _check(w, x, name):
    torch, g = gpu()
    desc, _, (o_n, S_n), (o_w, S_w) = _both(w, x)
    same = torch.equal(o_n, o_w) and torch.equal(S_n, S_w)
    f = gi.prefill_f64(w, x)
    o_r, S_r = oracle.forward(f["q"], f["k"], f["v"], f["alpha"], f["beta_k"], k_w=f["k_w"], beta_v=f["beta_v"],
                              S0=f["S0"])
    eo, es = oracle.rel_l2(to_np(o_n), o_r), oracle.rel_l2(to_np(S_n), S_r)
    log(f"[noalloc] {name}: workspace {g.gdr_chunk_fwd_workspace_size(desc)} B; equal to gdr_chunk_fwd {same}; "
        f"rel-L2 o={eo:.3e} S={es:.3e}")
    assert same
    assert eo <= TOL[w.io] and es <= TOL[w.io]


def test_two_calls_in_a_row_second_smaller():
    big = gi.OSDN_LONG_PREFILL.scaled(name="noalloc_big", B=2, T=1000, H=4, seed=601)
    small = gi.GDN_PREFILL.scaled(name="noalloc_small", B=1, T=300, H=3, seed=602)
    _check(big, gi.make_prefill(big), "first call (larger)")
    _check(small, gi.make_prefill(small), "second call (smaller)")


def test_general_gates_and_vector_alu_path():
    kda = gi.KDA_FG2PLUS_PREFILL.scaled(name="noalloc_kda", B=1, T=260, H=2, seed=603)
    _check(kda, gi.make_prefill(kda), "general gates")
    valu = gi.GDN_PREFILL.scaled(name="noalloc_valu", B=1, T=100, H=2, chunk=32, seed=604)
    _check(valu, gi.make_prefill(valu), "vector-ALU path")


def test_captured_in_a_graph():
    """Callers under graph capture are the ones this entry point is for: a captured call
    replays equal to the eager one, with other work between the replays."""
    torch, g = gpu()
    w = gi.GDN_PREFILL.scaled(name="noalloc_graph", B=1, T=400, H=4, seed=605)
    x = gi.make_prefill(w)
    desc, d, (o_ref, S_ref), _ = _both(w, x)
    args = (d["q"], d["k"], d["k_w"], d["v"], d["alpha"], d["beta_k"], d["beta_v"], d["S0"])
    o_g, S_g = torch.empty_like(o_ref), torch.empty_like(S_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            rc = g.gdr_chunk_fwd_noalloc(desc, *args, o_g, S_g, side)
    assert rc == g.GDR_OK
    torch.cuda.synchronize()
    other = gi.GDN_PREFILL.scaled(name="noalloc_between", B=1, T=200, H=2, seed=606)
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(o_g, o_ref) and torch.equal(S_g, S_ref)
        log(f"[noalloc graph] replay {rep}: equal to the eager call {same}")
        assert same
        _both(other, gi.make_prefill(other))  # another call through the shared array in between
