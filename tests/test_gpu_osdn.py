"""GPU parity of gdr_osdn_precond (OSDN phase 1, through the C-ABI) against the
fp64 oracle.  The scan is fp32 arithmetic on the stored inputs: the final
preconditioner and q_geo within 1e-5 (rel-L2 / relative); the write keys within
the io tolerance (2e-3 bf16, which is their rounding, 1e-5 fp32)."""
import numpy as np
import pytest

import gdr_inputs as gi
import oracle
from tests.gpu_util import TOL, gpu, log, to_np

pytestmark = pytest.mark.gpu


def _run(w, eta, *, apf, d0_std=0.0, zero_keys=(), ctx=None, with_plain=False):
    torch, g = gpu()
    x = gi.make_prefill(w)
    k = x["k"].copy()
    for (b, t, h) in zero_keys:
        k[b, t, h] = 0
    beta = x["beta_k"]
    r = gi.make_retention(w) if apf else None
    d0 = None
    if d0_std > 0:
        d0 = (1.0 + np.random.default_rng(w.seed).normal(0, d0_std, (w.B, w.H, w.dk))).astype(np.float32)
    args = (gi.to_torch(k, w.io), gi.to_torch(beta, w.gate), eta)
    kwargs = dict(r=None if r is None else gi.to_torch(r, w.gate), d0=None if d0 is None else gi.to_torch(d0, gi.F32))
    kw, dT, qg = g.osdn_precond(*args, **kwargs, ctx=ctx)
    torch.cuda.synchronize()
    if with_plain:
        # the same call without a context (every pass on the caller's stream): bit for bit equal
        plain = g.osdn_precond(*args, **kwargs)
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in zip((kw, dT, qg), plain))
        log(f"[osdn] blocked on the context's second stream equal to the single-stream call: {same}")
        assert same
    ref = oracle.osdn_precond(gi.as_f64(k, w.io), gi.as_f64(beta, w.gate), eta,
                              r=None if r is None else gi.as_f64(r, w.gate), d0=d0)
    return (to_np(kw), to_np(dT), to_np(qg)), ref


BASE = gi.OSDN_LONG_PREFILL.scaled(B=2, T=1000, H=3, seed=91)
CASES = [
    ("osdn_vanilla_ragged", BASE, 1.0, False, 0.0),
    ("osdn_apf_d0", BASE.scaled(seed=92), 1.0, True, 0.3),
    ("osdn_apf_strong_eta", BASE.scaled(T=640, seed=93), 4.0, True, 0.0),
    ("f32_io_dk24", BASE.scaled(T=300, dk=24, dv=24, io=gi.F32, seed=94), 1.0, True, 0.2),
    ("bf16_dk8_bf16_gates", BASE.scaled(T=200, dk=8, dv=8, gate=gi.BF16, seed=95), 0.5, True, 0.0),
    # with an execution context, 256 chunks and more are cut into blocks that the chain
    # walks in order while the parallel passes of other blocks run beside it on the
    # context's second stream (here 4 blocks, the last ragged)
    ("chunk_blocks_ragged", BASE.scaled(B=1, T=16500, H=2, seed=97), 1.0, True, 0.3),
    ("chunk_blocks_f32_dk24", BASE.scaled(B=2, T=16384, H=1, dk=24, dv=24, io=gi.F32, seed=98), 1.0, False, 0.0),
    ("chunk_blocks_bf16_gates", BASE.scaled(B=1, T=20000, H=1, gate=gi.BF16, seed=99), 0.7, True, 0.2),
]


@pytest.mark.parametrize("name,w,eta,apf,d0_std", CASES, ids=[c[0] for c in CASES])
def test_precond_parity(name, w, eta, apf, d0_std):
    torch, g = gpu()
    blocks = name.startswith("chunk_blocks")
    ctx = g.Context() if blocks else None
    (kw, dT, qg), (kw_r, dT_r, qg_r) = _run(w, eta, apf=apf, d0_std=d0_std, ctx=ctx, with_plain=blocks)
    ek, ed = oracle.rel_l2(kw, kw_r), oracle.rel_l2(dT, dT_r)
    eq = float(np.max(np.abs(qg - qg_r) / np.abs(qg_r)))
    log(f"[osdn] {name}: rel-L2 kw={ek:.3e} dT={ed:.3e} qgeo max rel={eq:.3e} (qgeo {qg_r.mean():.3f})")
    assert ek <= TOL[w.io] and ed <= 1e-5 and eq <= 1e-5


def test_zero_keys_and_empty_sequence():
    w = BASE.scaled(T=130, H=2, seed=96)
    (kw, dT, qg), (kw_r, dT_r, qg_r) = _run(w, 1.0, apf=True, zero_keys=[(0, 5, 1), (1, 64, 0), (1, 129, 1)])
    assert oracle.rel_l2(dT, dT_r) <= 1e-5 and oracle.rel_l2(kw, kw_r) <= TOL[w.io]
    torch, g = gpu()
    k0 = torch.zeros((2, 0, 3, 128), dtype=torch.bfloat16, device="cuda")
    b0 = torch.zeros((2, 0, 3), dtype=torch.float32, device="cuda")
    d0 = torch.rand((2, 3, 128), device="cuda") + 0.5
    _, dT0, qg0 = g.osdn_precond(k0, b0, 1.0, d0=d0)
    torch.cuda.synchronize()
    assert torch.equal(dT0, d0) and bool((qg0 == 1).all())


def test_precond_full_size_sampled():
    """B=1 H=32 T=65536 (the long-context shape), retention gates; the oracle runs
    4 of the 32 heads over all tokens."""
    torch, g = gpu()
    w = gi.OSDN_LONG_PREFILL
    x = gi.make_prefill(w)
    r = gi.make_retention(w)
    kw, dT, qg = g.osdn_precond(gi.to_torch(x["k"], w.io), gi.to_torch(x["beta_k"], w.gate), 1.0,
                                r=gi.to_torch(r, w.gate))
    torch.cuda.synchronize()
    heads = [0, 9, 22, 31]
    kh = np.ascontiguousarray(x["k"][:, :, heads])
    ref = oracle.osdn_precond(gi.as_f64(kh, w.io), gi.as_f64(x["beta_k"][:, :, heads], w.gate), 1.0,
                              r=gi.as_f64(r[:, :, heads], w.gate))
    ek = oracle.rel_l2(to_np(kw)[:, :, heads], ref[0])
    ed = oracle.rel_l2(to_np(dT)[:, heads], ref[1])
    eq = float(np.max(np.abs(to_np(qg)[:, heads] - ref[2]) / ref[2]))
    log(f"[osdn] full size sampled: rel-L2 kw={ek:.3e} dT={ed:.3e} qgeo rel={eq:.3e}")
    assert ek <= 2e-3 and ed <= 1e-5 and eq <= 1e-5


def test_phase_one_then_phase_two():
    """Phase 1 write keys feed the chunked pass (OSDN page, section 2.2, the two
    phases); against the oracle's phase 1 (rounded to bf16 like the GPU's) and its
    sequential recurrence."""
    torch, g = gpu()
    w = gi.OSDN_LONG_PREFILL.scaled(T=1024, H=2, seed=97)
    x = gi.make_prefill(w)
    r = gi.make_retention(w)
    kw, _, _ = g.osdn_precond(gi.to_torch(x["k"], w.io), gi.to_torch(x["beta_k"], w.gate), 1.0,
                              r=gi.to_torch(r, w.gate))
    d = {key: gi.to_torch(x[key], w.io if key in ("q", "k", "v") else (w.gate if key != "S0" else gi.F32))
         for key in ("q", "k", "v", "alpha", "beta_k", "S0")}
    o, ST = g.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta_k"], k_w=kw, S0=d["S0"])
    torch.cuda.synchronize()
    f = gi.prefill_f64(w, x)
    kw_r, _, _ = oracle.osdn_precond(f["k"], f["beta_k"], 1.0, r=gi.as_f64(r, w.gate))
    kw_r = gi.as_f64(gi.store(kw_r, w.io), w.io)
    o_r, S_r = oracle.forward(f["q"], f["k"], f["v"], f["alpha"], f["beta_k"], k_w=kw_r, S0=f["S0"])
    eo, es = oracle.rel_l2(to_np(o), o_r), oracle.rel_l2(to_np(ST), S_r)
    log(f"[osdn] phase 1 + phase 2: rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= 2e-3 and es <= 2e-3
