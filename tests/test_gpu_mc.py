"""GPU parity of the Memory-Caching entry points (gdr_chunk_fwd_ckpt, gdr_mc_readout)
through the C-ABI, against oracle/memcache.py.

Tolerances: segment states as the final state (rel-L2 <= 2e-3 bf16, <= 1e-5 fp32);
read-out rel-L2 <= 2e-3 (one bf16 rounding of the result).  The end-to-end case
(prefill with caches, then the read-out added to the prefill's bf16 output) rounds
twice -- o once in the prefill and the sum once more: against an oracle that stores
its own o as bf16 before the read-out it must meet 2e-3, and against the exact
oracle sqrt(2) * 2e-3 ~ 3e-3.
"""
import numpy as np
import pytest

import gdr_inputs as gi
import oracle
from oracle import memcache
from tests.gpu_util import TOL, gpu, log, to_np, upload

pytestmark = pytest.mark.gpu


def _ckpt_run(w, x, seg):
    torch, g = gpu()
    d = upload(x, w)
    kw = dict(k_w=d["k_w"], beta_v=d["beta_v"], S0=d["S0"], chunk=w.chunk)
    o, ST, ck = g.chunk_fwd_ckpt(d["q"], d["k"], d["v"], d["alpha"], d["beta_k"], seg, **kw)
    o2, ST2 = g.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta_k"], **kw)
    torch.cuda.synchronize()
    return o, ST, ck, o2, ST2


CKPT_CASES = [
    ("gdn_mfma_ragged", gi.GDN_PREFILL.scaled(B=2, T=1000, H=3, seed=61), 256),
    ("osdn_mfma_write_key_S0", gi.OSDN_LONG_PREFILL.scaled(T=768, H=2, seed=62), 128),
    ("kda_fg2plus_mfma", gi.KDA_FG2PLUS_PREFILL.scaled(B=1, T=640, H=2, seed=63), 192),
    ("valu_f32", gi.TINY_GDN_F32.scaled(B=2, T=200, H=2, dk=32, dv=24, chunk=16, seed=64), 48),
    ("valu_bf16_channel", gi.KDA_FG2PLUS_PREFILL.scaled(B=1, T=300, H=2, dk=64, dv=40, chunk=32, seed=65), 64),
]


@pytest.mark.parametrize("name,w,seg", CKPT_CASES, ids=[c[0] for c in CKPT_CASES])
def test_segment_states(name, w, seg):
    torch, g = gpu()
    x = gi.make_prefill(w)
    log(f"[mc] checkpoints {name}: B={w.B} T={w.T} H={w.H} dk={w.dk} dv={w.dv} C={w.chunk} seg={seg}")
    o, ST, ck, o2, ST2 = _ckpt_run(w, x, seg)
    # keeping the segment states changes nothing else, bit for bit
    assert torch.equal(o, o2) and torch.equal(ST, ST2)
    f = gi.prefill_f64(w, x)
    _, _, ck_ref = memcache.segment_states(f["q"], f["k"], f["v"], f["alpha"], f["beta_k"], seg, k_w=f["k_w"],
                                           beta_v=f["beta_v"], S0=f["S0"])
    ckg = to_np(ck)
    assert ckg.shape == ck_ref.shape == (w.B, w.H, w.T // seg, w.dk, w.dv)
    per = [oracle.rel_l2(ckg[:, :, s], ck_ref[:, :, s]) for s in range(ck_ref.shape[2])]
    log(f"          rel-L2 per segment state {[f'{e:.2e}' for e in per]}")
    assert max(per) <= TOL[w.io]


def _readout_gpu(w, x, in_place=False):
    torch, g = gpu()
    q = gi.to_torch(x["q"], gi.BF16)
    ck = gi.to_torch(x["ckpt"], gi.F32)
    gates = None if x["gates"] is None else gi.to_torch(x["gates"], gi.F32)
    o_in = None if x["o_in"] is None else gi.to_torch(x["o_in"], gi.BF16)
    if in_place:
        out = g.mc_readout(q, ck, w.seg, gates=gates, o_in=o_in, out=o_in)
    else:
        out = g.mc_readout(q, ck, w.seg, gates=gates, o_in=o_in)
    torch.cuda.synchronize()
    return out


def _readout_ref(w, x, heads=None, tokens=None):
    q = gi.as_f64(x["q"], gi.BF16)
    o_in = None if x["o_in"] is None else gi.as_f64(x["o_in"], gi.BF16)
    return memcache.readout(q, x["ckpt"], w.seg, gates=x["gates"], o_in=o_in, heads=heads, tokens=tokens)


RO_BASE = gi.MC_LONG_GRM.scaled(B=2, T=1000, H=3, seg=128, seed=71)
RO_CASES = [
    ("grm_dense_ragged", RO_BASE),
    ("residual_seg256", RO_BASE.scaled(T=1536, seg=256, gate_kind="residual", seed=72)),
    ("residual_seg64_several_per_block", RO_BASE.scaled(T=700, seg=64, gate_kind="residual", seed=73)),
    ("topk_router", RO_BASE.scaled(T=1024, gate_kind="topk", topk=2, seed=74)),
    ("grm_no_o_in", RO_BASE.scaled(T=512, with_o_in=False, seed=75)),
    ("grm_seg_not_block_multiple", RO_BASE.scaled(T=900, seg=320, seed=76)),
]


@pytest.mark.parametrize("name,w", RO_CASES, ids=[c[0] for c in RO_CASES])
def test_readout(name, w):
    x = gi.make_cache_readout(w)
    log(f"[mc] read-out {name}: B={w.B} T={w.T} H={w.H} seg={w.seg} N={w.N} gates={w.gate_kind}")
    out = to_np(_readout_gpu(w, x))
    ref = _readout_ref(w, x)
    e = oracle.rel_l2(out, ref)
    log(f"          rel-L2 {e:.3e}")
    assert np.isfinite(out).all() and e <= 2e-3


def test_readout_in_place_equals_out_of_place():
    torch, g = gpu()
    w = RO_BASE.scaled(seed=77)
    x = gi.make_cache_readout(w)
    a = _readout_gpu(w, x)
    b = _readout_gpu(w, x, in_place=True)
    assert torch.equal(a, b)


def test_readout_without_caches_copies_o_in():
    torch, g = gpu()
    w = RO_BASE.scaled(T=300, seg=512, seed=78)  # N = 0
    x = gi.make_cache_readout(w)
    out = _readout_gpu(w, x)
    assert w.N == 0 and torch.equal(out, gi.to_torch(x["o_in"], gi.BF16))


def test_readout_full_size_sampled():
    """B=1 H=32 T=65536, 16 cached segments, dense gates (the timed read-out); the
    oracle evaluates 4 heads at 96 tokens spread over every segment."""
    w = gi.MC_LONG_GRM
    x = gi.make_cache_readout(w)
    out = to_np(_readout_gpu(w, x))
    rng = np.random.default_rng(2)
    heads = sorted(rng.choice(w.B * w.H, 4, replace=False).tolist())
    tokens = np.sort(rng.choice(w.T, 96, replace=False))
    ref = _readout_ref(w, x, heads=heads, tokens=tokens)
    got = np.stack([out[bh // w.H, tokens, bh % w.H] for bh in heads])
    e = oracle.rel_l2(got, ref)
    log(f"[mc] full read-out sampled rel-L2 {e:.3e}")
    assert e <= 2e-3


def test_prefill_then_readout_end_to_end():
    """Prefill keeps its segment states, the read-out adds their gated read-outs to the
    prefill's output; against the oracle's exact states and output."""
    torch, g = gpu()
    w = gi.GDN_PREFILL.scaled(B=1, T=1024, H=2, seed=79)
    seg = 256
    x = gi.make_prefill(w)
    o, ST, ck, _, _ = _ckpt_run(w, x, seg)
    n = w.T // seg
    gates = np.random.default_rng(3).uniform(0, 1, (w.B, w.T, w.H, n)).astype(np.float32)
    out = g.mc_readout(gi.to_torch(x["q"], gi.BF16), ck, seg, gates=gi.to_torch(gates, gi.F32), o_in=o)
    torch.cuda.synchronize()
    f = gi.prefill_f64(w, x)
    o_ref, _, ck_ref = memcache.segment_states(f["q"], f["k"], f["v"], f["alpha"], f["beta_k"], seg)
    ref = memcache.readout(f["q"], ck_ref, seg, gates=gates, o_in=o_ref)
    # the read-out's own input is the prefill's stored (bf16) output: against the
    # oracle's output stored the same way, one rounding (the sum's) is left
    ref_stored = memcache.readout(f["q"], ck_ref, seg, gates=gates, o_in=gi.as_f64(gi.store(o_ref, w.io), w.io))
    out_np = to_np(out)
    e, e_stored = oracle.rel_l2(out_np, ref), oracle.rel_l2(out_np, ref_stored)
    log(f"[mc] prefill + read-out rel-L2 {e:.3e} (exact oracle), {e_stored:.3e} (oracle's o stored as bf16)")
    assert e_stored <= 2e-3
    assert e <= 3e-3
