"""The sequential fp64 oracle equals an independent chunkwise (WY / UT-transform)
evaluation on tiny inputs, for every variant and chunk sizes from 1 to T
(C = 1 and C = T are the degenerate cases; T not a multiple of C exercises the
ragged last chunk)."""
import numpy as np
import pytest

import oracle
from oracle.chunked import forward_chunked


def _inputs(rng, B, T, H, dk, dv, channel, beta_mode, kw, s0):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    alpha = rng.uniform(0.7, 1.0, (B, T, H, dk) if channel else (B, T, H))
    beta_k = rng.uniform(0.0, 1.0, (B, T, H) if beta_mode == 0 else (B, T, H, dk))
    beta_v = rng.uniform(0.0, 1.0, (B, T, H, dv)) if beta_mode == 2 else None
    k_w = k * (1.0 + 0.1 * rng.standard_normal(k.shape)) if kw else None
    S0 = 0.5 * rng.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, alpha, beta_k, dict(k_w=k_w, beta_v=beta_v, S0=S0)


VARIANTS = {
    "gdn": dict(channel=False, beta_mode=0, kw=False),
    "kda": dict(channel=True, beta_mode=0, kw=False),
    "fg2": dict(channel=True, beta_mode=1, kw=False),
    "fg2plus": dict(channel=True, beta_mode=2, kw=False),
    "osdn": dict(channel=False, beta_mode=0, kw=True),
    "osdn_kda": dict(channel=True, beta_mode=0, kw=True),
}


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("chunk", [1, 2, 4, 16, 37])
def test_chunked_equals_sequential(variant, chunk):
    rng = np.random.default_rng(100 + chunk)
    B, T, H, d = 2, 37, 2, 8
    dv = d if VARIANTS[variant]["beta_mode"] == 1 else 6
    q, k, v, a, b, kw = _inputs(rng, B, T, H, d, dv, s0=True, **VARIANTS[variant])
    o_seq, S_seq = oracle.forward(q, k, v, a, b, **kw)
    o_chk, S_chk = forward_chunked(q, k, v, a, b, chunk=chunk, **kw)
    assert oracle.rel_l2(o_chk, o_seq) < 1e-12
    assert oracle.rel_l2(S_chk, S_seq) < 1e-12


def test_chunked_zero_state_and_chunk_larger_than_T():
    rng = np.random.default_rng(7)
    q, k, v, a, b, kw = _inputs(rng, 1, 5, 1, 4, 4, channel=False, beta_mode=0, kw=False, s0=False)
    o_seq, S_seq = oracle.forward(q, k, v, a, b, **kw)
    o_chk, S_chk = forward_chunked(q, k, v, a, b, chunk=64, **kw)
    assert oracle.rel_l2(o_chk, o_seq) < 1e-13
    assert oracle.rel_l2(S_chk, S_seq) < 1e-13
