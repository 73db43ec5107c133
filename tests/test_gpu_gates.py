"""Forget gates at the edges of their range, on the GPU against the fp64 oracle.

A gate of exactly 0 is a hard reset (the decay across it is 0): the FG2-GDN page,
section 1, allows any alpha_t in [0, 1] for the scalar (GDN) and channel-wise (KDA)
decay, and the SDM page's forget gate multiplies the slot by alpha.  Channel gates
whose decay inside one 64-token chunk falls far below e^{-80} (alpha ~ 0.27 held for
a chunk) must come out right too.  Every prefill kernel family is covered: the bf16
matrix-core kernels (dk = dv = 128, chunk 64; scalar and general-gate preps) and the
fp32 vector-ALU kernel (other chunks and shapes); also the decode step with zero
gates and OSDN phase 1 with zero retention."""
import numpy as np
import pytest

import gdr_inputs as gi
import oracle
from tests.gpu_util import TOL, gpu, log, run_prefill, to_np, upload
from tests.test_gpu_decode import _gpu_steps, _oracle_steps

pytestmark = pytest.mark.gpu

# tokens whose gate is set to 0: the first token, the middle and the last token of the
# first chunk, the first of the second chunk, and the last token of the sequence
ZERO_TOKENS = [0, 30, 63, 64, 127]


def _plant_zeros(w, x, tokens, channels=None):
    a = x["alpha"]
    for t in tokens:
        t = min(t, w.T - 1)
        if w.alpha_mode == gi.GATE_SCALAR:
            a[:, t, :] = 0
        else:
            a[:, t, :, channels if channels is not None else slice(None)] = 0
    a[:, w.T - 1] = 0
    return x


SCALAR_MFMA = gi.GDN_PREFILL.scaled(name="zero_gates_mfma", B=2, T=200, H=3, s0_std=0.02, seed=501)
CHANNEL_MFMA = gi.KDA_FG2PLUS_PREFILL.scaled(name="zero_gates_chan_mfma", B=1, T=200, H=2, s0_std=0.02,
                                             seed=502)
ZERO_CASES = [
    ("scalar_mfma", SCALAR_MFMA, None),
    ("scalar_mfma_bf16_gates", SCALAR_MFMA.scaled(gate=gi.BF16, seed=503), None),
    ("scalar_valu_C32", SCALAR_MFMA.scaled(chunk=32, seed=504), None),
    ("scalar_valu_f32", SCALAR_MFMA.scaled(io=gi.F32, dk=64, dv=64, seed=505), None),
    ("channel_mfma_some_channels", CHANNEL_MFMA, [3, 17, 64, 127]),
    ("channel_mfma_all_channels", CHANNEL_MFMA.scaled(seed=506), None),
    ("channel_valu_C32", CHANNEL_MFMA.scaled(chunk=32, seed=507), [0, 5, 100]),
    ("channel_valu_f32", CHANNEL_MFMA.scaled(io=gi.F32, dk=64, dv=48, beta_mode=gi.BETA_SCALAR, seed=508),
     [1, 2, 63]),
]


@pytest.mark.parametrize("name,w,channels", ZERO_CASES, ids=[c[0] for c in ZERO_CASES])
def test_zero_gates(name, w, channels):
    x = _plant_zeros(w, gi.make_prefill(w), ZERO_TOKENS, channels)
    r = run_prefill(w, x)
    assert r["finite"], r
    assert r["o"] <= TOL[w.io] and r["S"] <= TOL[w.io], r


def test_every_gate_zero():
    """alpha = 0 at every token: each token's state is its own write, S_t = w_t vh_t^T."""
    w = SCALAR_MFMA.scaled(T=130, seed=509)
    x = gi.make_prefill(w)
    x["alpha"][:] = 0
    r = run_prefill(w, x)
    assert r["finite"] and r["o"] <= TOL[w.io] and r["S"] <= TOL[w.io], r


# alpha = sigmoid(-N(1, 1)) per channel: the cumulative log decay of a 64-token chunk
# is about -90 on average, so most chunks leave the range of the factored decay
STRONG = gi.KDA_FG2PLUS_PREFILL.scaled(name="strong_channel_decay", B=1, T=300, H=2, alpha_mu=1.0,
                                       alpha_sd=1.0, s0_std=0.02, seed=511)
STRONG_CASES = [
    ("mfma_kv_beta", STRONG),
    ("mfma_scalar_beta_write_key", STRONG.scaled(beta_mode=gi.BETA_SCALAR, write_key=True, seed=512)),
    ("mfma_bf16_gates", STRONG.scaled(gate=gi.BF16, seed=513)),
    ("valu_C32", STRONG.scaled(chunk=32, alpha_mu=3.0, seed=514)),  # about -97 per 32-token chunk
    ("valu_f32_d64", STRONG.scaled(io=gi.F32, dk=64, dv=64, beta_mode=gi.BETA_SHARED, seed=515)),
]


@pytest.mark.parametrize("name,w", STRONG_CASES, ids=[c[0] for c in STRONG_CASES])
def test_strong_channel_decay(name, w):
    x = gi.make_prefill(w)
    a = gi.as_f64(x["alpha"], w.gate)
    n = w.T // w.chunk * w.chunk
    per_chunk = np.log(a[:, :n]).reshape(w.B, -1, w.chunk, w.H, w.dk).sum(axis=2)
    log(f"[gates] {name}: per-chunk cumulative log decay min {per_chunk.min():.1f} "
        f"median {np.median(per_chunk):.1f}")
    assert per_chunk.min() < -80
    r = run_prefill(w, x)
    assert r["finite"], r
    assert r["o"] <= TOL[w.io] and r["S"] <= TOL[w.io], r


def test_mixed_chunks_strong_and_mild():
    """One call whose chunks alternate between the factored and the exact form of the
    general-gate prep (mild gates in even chunks, strong ones in odd chunks, a zero
    gate in one)."""
    w = STRONG.scaled(T=320, seed=516)
    x = gi.make_prefill(w)
    mild = gi.make_prefill(w.scaled(alpha_mu=-4.0))["alpha"]
    for c in range(0, w.T // 64, 2):
        x["alpha"][:, 64 * c:64 * (c + 1)] = mild[:, 64 * c:64 * (c + 1)]
    x["alpha"][0, 200, 1, 40] = 0
    r = run_prefill(w, x)
    assert r["finite"] and r["o"] <= TOL[w.io] and r["S"] <= TOL[w.io], r


def test_tiny_nonzero_scalar_gates():
    """Scalar gates of 1e-30 (nonzero, far below any factored range) on the matrix-core
    path: the scalar decays are exact differences and stay correct."""
    w = SCALAR_MFMA.scaled(seed=517)
    x = gi.make_prefill(w)
    x["alpha"][:, [5, 70, 71, 150]] = 1e-30
    r = run_prefill(w, x)
    assert r["finite"] and r["o"] <= TOL[w.io] and r["S"] <= TOL[w.io], r


@pytest.mark.parametrize("alpha_mode", [gi.GATE_SCALAR, gi.GATE_CHANNEL], ids=["scalar", "channel"])
def test_decode_zero_gates(alpha_mode):
    """The decode step with some gates exactly 0 (a hard reset of that (b, h) or channel)."""
    w = gi.DECODE_B512.scaled(name="dec_zero", B=4, H=3, steps=5, alpha_mode=alpha_mode, seed=518)
    x = gi.make_decode(w)
    x["alpha"][1, 0, 1] = 0
    x["alpha"][3, 2] = 0
    o_g, S_g = _gpu_steps(w, x)
    o_r, S_r = _oracle_steps(w, x)
    eo, es = oracle.rel_l2(o_g, o_r), oracle.rel_l2(S_g, S_r)
    log(f"[gates] decode zero gates ({alpha_mode}): rel-L2 o={eo:.3e} S={es:.3e}")
    assert eo <= 2e-3 and es <= 1e-5


def test_osdn_precond_zero_retention():
    """OSDN phase 1 with the retention gate exactly 0 at some tokens: d restarts from
    that token's gradient step alone."""
    torch, g = gpu()
    w = gi.OSDN_LONG_PREFILL.scaled(B=2, T=300, H=2, seed=519)
    x = gi.make_prefill(w)
    r = gi.make_retention(w)
    r[:, [0, 63, 64, 200], :] = 0
    r[1, 100, 1] = 0
    kw, dT, qg = g.osdn_precond(gi.to_torch(x["k"], w.io), gi.to_torch(x["beta_k"], w.gate), 1.0,
                                r=gi.to_torch(r, w.gate))
    torch.cuda.synchronize()
    kw_r, dT_r, qg_r = oracle.osdn_precond(gi.as_f64(x["k"], w.io), gi.as_f64(x["beta_k"], w.gate), 1.0,
                                           r=gi.as_f64(r, w.gate))
    ek, ed = oracle.rel_l2(to_np(kw), kw_r), oracle.rel_l2(to_np(dT), dT_r)
    eq = float(np.max(np.abs(to_np(qg) - qg_r) / np.abs(qg_r)))
    log(f"[gates] OSDN zero retention: rel-L2 kw={ek:.3e} dT={ed:.3e} qgeo rel={eq:.3e}")
    assert ek <= TOL[w.io] and ed <= 1e-5 and eq <= 1e-5
