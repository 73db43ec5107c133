"""Shared helpers for the GPU parity tests (not collected: no test_ prefix)."""
import os
import sys
import time

import numpy as np

import gdr_inputs as gi
import oracle

TOL = {gi.BF16: 2e-3, gi.F32: 1e-5}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu():
    import torch

    import gated_delta_rule_84_amd as g

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch, g


def upload(x: dict, w) -> dict:
    io = {"q", "k", "k_w", "v"}
    out = {}
    for key, val in x.items():
        if key in io:
            out[key] = gi.to_torch(val, w.io)
        elif key in ("alpha", "beta_k", "beta_v"):
            out[key] = gi.to_torch(val, w.gate)
        else:
            out[key] = gi.to_torch(val, gi.F32)
    return out


def to_np(t):
    import torch

    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype != torch.float32 else \
        t.detach().cpu().numpy().astype(np.float64)


def run_prefill(w, x, *, heads=None, nthreads=0):
    """GPU chunk forward vs the fp64 oracle on (optionally sampled) heads.
    Returns dict of rel-L2 errors and the path used."""
    torch, g = gpu()
    d = upload(x, w)
    desc = g.make_desc(d["q"], d["v"], d["alpha"], d["beta_k"], d["beta_v"], chunk=w.chunk)
    path = g.gdr_chunk_fwd_path(desc)
    log(f"[prefill] {w.name} B={w.B} T={w.T} H={w.H} dk={w.dk} dv={w.dv} C={w.chunk} path={path}")
    o, ST = g.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta_k"], k_w=d["k_w"], beta_v=d["beta_v"],
                        S0=d["S0"], chunk=w.chunk)
    torch.cuda.synchronize()
    o_gpu, S_gpu = to_np(o), to_np(ST)
    f = gi.prefill_f64(w, x)
    t0 = time.time()
    o_ref, S_ref = oracle.forward(f["q"], f["k"], f["v"], f["alpha"], f["beta_k"], k_w=f["k_w"],
                                  beta_v=f["beta_v"], S0=f["S0"], heads=heads, nthreads=nthreads)
    t_or = time.time() - t0
    if heads is not None:
        hb = [(bh // w.H, bh % w.H) for bh in heads]
        sel_o = lambda a: np.stack([a[b, :, h] for b, h in hb])
        sel_s = lambda a: np.stack([a[b, h] for b, h in hb])
        o_gpu, o_ref, S_gpu, S_ref = sel_o(o_gpu), sel_o(o_ref), sel_s(S_gpu), sel_s(S_ref)
    res = dict(path=path, o=oracle.rel_l2(o_gpu, o_ref), S=oracle.rel_l2(S_gpu, S_ref),
               o_vs_rounded=oracle.rel_l2(o_gpu, gi.as_f64(gi.store(o_ref, w.io), w.io)),
               finite=bool(np.isfinite(o_gpu).all() and np.isfinite(S_gpu).all()), oracle_s=t_or)
    log(f"          rel-L2 o={res['o']:.3e} S={res['S']:.3e} o_vs_rounded_oracle={res['o_vs_rounded']:.3e} "
        f"oracle {t_or:.1f}s")
    # the stored output is as close to the oracle's own stored output as to the exact one
    # (rounding both to the storage type removes no more than the tolerance)
    assert res["o_vs_rounded"] <= TOL[w.io], res
    return res
