"""GPU parity of gdr_decode_step against the fp64 oracle (through the C-ABI)."""
import numpy as np
import pytest

import gdr_inputs as gi
import oracle
from tests.gpu_util import TOL, gpu, log, to_np, upload

pytestmark = pytest.mark.gpu


def _oracle_steps(w, x, heads=None, nthreads=0):
    """Sequential fp64 decode over all steps (optionally on sampled (b, h) pairs)."""
    f = gi.decode_f64(w, x)
    S = f["S"]
    sel = (lambda a: a) if heads is None else (lambda a: a.reshape((-1,) + a.shape[2:])[heads][:, None])
    selS = (lambda a: a) if heads is None else (lambda a: a.reshape((-1,) + a.shape[2:])[heads][:, None])
    S = selS(S)
    outs = []
    for i in range(w.steps):
        step = {key: (None if f[key] is None else sel(f[key][i])) for key in
                ("q", "k", "k_w", "v", "alpha", "beta_k", "beta_v")}
        o, S = oracle.decode_step(S, step["q"], step["k"], step["v"], step["alpha"], step["beta_k"],
                                  k_w=step["k_w"], beta_v=step["beta_v"], nthreads=nthreads)
        outs.append(o)
    return np.stack(outs), S


def _gpu_steps(w, x, graph=False, flags=0):
    torch, g = gpu()
    d = upload(x, w)
    S = d["S"].clone()
    if graph:
        from gated_delta_rule_84_amd.graph import DecodeGraph

        dg = DecodeGraph(S, d["q"], d["k"], d["v"], d["alpha"], d["beta_k"], k_w=d["k_w"], beta_v=d["beta_v"],
                         flags=flags)
        out = dg.replay()
    else:
        outs = []
        for i in range(w.steps):
            sel = lambda key: None if d[key] is None else d[key][i]
            outs.append(g.decode_step(S, sel("q"), sel("k"), sel("v"), sel("alpha"), sel("beta_k"),
                                      k_w=sel("k_w"), beta_v=sel("beta_v"), flags=flags))
        out = torch.stack(outs)
    torch.cuda.synchronize()
    return to_np(out), to_np(S)


BASE = gi.DECODE_B512.scaled(name="dec_small", B=4, H=3, steps=6, seed=41)
CASES = [
    ("d128_scalar", BASE),
    ("d128_channel_alpha", BASE.scaled(alpha_mode=gi.GATE_CHANNEL)),
    ("d128_fg2_shared", BASE.scaled(beta_mode=gi.BETA_SHARED, gate=gi.F32)),
    ("d128_fg2plus", BASE.scaled(beta_mode=gi.BETA_KV, alpha_mode=gi.GATE_CHANNEL)),
    ("d64", BASE.scaled(dk=64, dv=64)),
    ("d32", BASE.scaled(dk=32, dv=32)),
    ("d16", BASE.scaled(dk=16, dv=16, B=9)),
    ("d8", BASE.scaled(dk=8, dv=8, B=37)),
    ("dk64_dv128_generic", BASE.scaled(dk=64, dv=128)),
    ("dk24_dv40_generic", BASE.scaled(dk=24, dv=40, beta_mode=gi.BETA_KV)),
    ("f32_io", BASE.scaled(io=gi.F32, gate=gi.F32)),
]


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_decode_parity_small(name, w):
    x = gi.make_decode(w)
    o, S = _gpu_steps(w, x)
    o_ref, S_ref = _oracle_steps(w, x)
    eo, es = oracle.rel_l2(o, o_ref), oracle.rel_l2(S, S_ref)
    log(f"[decode] {name}: rel-L2 o={eo:.3e} S={es:.3e}")
    tol_s = 1e-5  # the state stays fp32 end to end
    assert eo <= TOL[w.io] and es <= tol_s


def test_decode_write_key():
    w = BASE.scaled(seed=42)
    x = gi.make_decode(w)
    rng = np.random.default_rng(5)
    kf = gi.as_f64(x["k"], w.io)
    x["k_w"] = gi.store(kf * (1 + 0.1 * rng.standard_normal(kf.shape)), w.io)
    o, S = _gpu_steps(w, x)
    o_ref, S_ref = _oracle_steps(w, x)
    assert oracle.rel_l2(o, o_ref) <= 2e-3 and oracle.rel_l2(S, S_ref) <= 1e-5


def test_decode_graph_equals_eager():
    w = BASE.scaled(steps=16, seed=43)
    x = gi.make_decode(w)
    o1, S1 = _gpu_steps(w, x, graph=False)
    o2, S2 = _gpu_steps(w, x, graph=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_decode_full_b512_graph():
    """B=512 H=16 d=128, 256 steps replayed as one HIP graph (as timed); the oracle
    follows 48 sampled (b, h) pairs through all 256 steps."""
    w = gi.DECODE_B512
    x = gi.make_decode(w)
    o, S = _gpu_steps(w, x, graph=True)
    heads = sorted(np.random.default_rng(1).choice(w.B * w.H, 48, replace=False).tolist())
    o_ref, S_ref = _oracle_steps(w, x, heads=heads)
    og = o.reshape(w.steps, -1, w.dv)[:, heads]
    Sg = S.reshape(-1, w.dk, w.dv)[heads]
    eo, es = oracle.rel_l2(og, o_ref[:, :, 0]), oracle.rel_l2(Sg, S_ref[:, 0])
    log(f"[decode] full B512: rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= 2e-3 and es <= 1e-5


def test_decode_full_deltamem_graph():
    """B=8192 H=1 r=8, 256 steps, every head checked."""
    w = gi.DECODE_DMEM_R8
    x = gi.make_decode(w)
    o, S = _gpu_steps(w, x, graph=True)
    o_ref, S_ref = _oracle_steps(w, x)
    eo, es = oracle.rel_l2(o, o_ref), oracle.rel_l2(S, S_ref)
    log(f"[decode] full delta-mem r8: rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= 2e-3 and es <= 1e-5


# ---------------------------------------------------------------------------
# delta-mem options: read before the write, prediction from the undecayed state
# ---------------------------------------------------------------------------
def _dmem_steps(w, x):
    """The delta-mem recurrence in its own orientation (M = S^T), scalar lambda = alpha
    and write strength beta; returns per-step reads r_t = M_{t-1} q_t, the memories
    after every step (in S orientation) and the final state."""
    f = gi.decode_f64(w, x)
    M = np.ascontiguousarray(np.swapaxes(f["S"], -1, -2))
    rs, Ss = [], []
    for i in range(w.steps):
        r, M = oracle.dmem_step(M, f["q"][i], f["k"][i], f["v"][i], f["alpha"][i], f["beta_k"][i])
        rs.append(r)
        Ss.append(np.swapaxes(M, -1, -2))
    return np.stack(rs), np.stack(Ss)


DMEM_CASES = [
    ("d8", gi.DECODE_DMEM_R8.scaled(B=64, steps=8, seed=44)),
    ("d16", BASE.scaled(dk=16, dv=16, B=9, seed=45)),
    ("d128", BASE.scaled(seed=46)),
    ("dk24_dv40_generic", BASE.scaled(dk=24, dv=40, seed=47)),
]


@pytest.mark.parametrize("name,w", DMEM_CASES, ids=[c[0] for c in DMEM_CASES])
def test_dmem_read_before_write_undecayed(name, w):
    """Both options together are the delta-mem step exactly."""
    _, g = gpu()
    x = gi.make_decode(w)
    o, S = _gpu_steps(w, x, flags=g.GDR_FLAG_READ_BEFORE_WRITE | g.GDR_FLAG_UNDECAYED_PREDICTION)
    r_ref, S_ref = _dmem_steps(w, x)
    eo, es = oracle.rel_l2(o, r_ref), oracle.rel_l2(S, S_ref[-1])
    log(f"[decode] delta-mem {name}: rel-L2 r={eo:.3e} S={es:.3e}")
    assert eo <= TOL[w.io] and es <= 1e-5


def test_dmem_options_one_at_a_time():
    """Undecayed prediction alone: the delta-mem memories, read after the write.
    Read-before-write alone: the ordinary gated states, read before the write."""
    _, g = gpu()
    w = BASE.scaled(seed=48)
    x = gi.make_decode(w)
    f = gi.decode_f64(w, x)

    o, S = _gpu_steps(w, x, flags=g.GDR_FLAG_UNDECAYED_PREDICTION)
    _, S_all = _dmem_steps(w, x)
    o_ref = np.einsum("nbhkv,nbhk->nbhv", S_all, f["q"])
    assert oracle.rel_l2(o, o_ref) <= TOL[w.io] and oracle.rel_l2(S, S_all[-1]) <= 1e-5

    o, S = _gpu_steps(w, x, flags=g.GDR_FLAG_READ_BEFORE_WRITE)
    S_prev = f["S"]
    reads = []
    for i in range(w.steps):
        reads.append(np.einsum("bhkv,bhk->bhv", S_prev, f["q"][i]))
        _, S_prev = oracle.decode_step(S_prev, f["q"][i], f["k"][i], f["v"][i], f["alpha"][i], f["beta_k"][i])
    assert oracle.rel_l2(o, np.stack(reads)) <= TOL[w.io] and oracle.rel_l2(S, S_prev) <= 1e-5


def test_dmem_full_r8_graph():
    """B=8192 H=1 r=8, 256 steps of the delta-mem step replayed as one HIP graph."""
    _, g = gpu()
    w = gi.DECODE_DMEM_R8
    x = gi.make_decode(w)
    o, S = _gpu_steps(w, x, graph=True, flags=g.GDR_FLAG_READ_BEFORE_WRITE | g.GDR_FLAG_UNDECAYED_PREDICTION)
    r_ref, S_ref = _dmem_steps(w, x)
    eo, es = oracle.rel_l2(o, r_ref), oracle.rel_l2(S, S_ref[-1])
    log(f"[decode] full delta-mem r8 (read before write): rel-L2 r={eo:.3e} S={es:.3e}")
    assert eo <= 2e-3 and es <= 1e-5
