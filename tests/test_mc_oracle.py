"""Pins of the Memory-Caching oracle (oracle/memcache.py) on the CPU.

Each pin fixes the oracle against something other than its own formula: the page's
statement that memory soup equals the gated residual read-out for a linear memory,
the prefix-sum form of the residual memory, one-hot queries (closed form by
indexing), the degenerate cases (no cache: the plain recurrent read-out), and the
segment states against one uninterrupted run of the sequential oracle.
"""
import numpy as np
import pytest

import gdr_inputs as gi
import oracle
from oracle import memcache

SMALL = gi.CacheReadout("mc_tiny", B=2, T=40, H=3, dk=6, dv=5, seg=8, gate_kind="dense", s_std=0.5, seed=3)


def _f64(x):
    w = SMALL
    q = gi.as_f64(x["q"], gi.BF16)
    ck = x["ckpt"].astype(np.float64)
    g = None if x["gates"] is None else x["gates"].astype(np.float64)
    oi = None if x["o_in"] is None else gi.as_f64(x["o_in"], gi.BF16)
    return q, ck, g, oi


def test_soup_equals_gated_residual():
    """Memory Caching: RNNs with Growing Memory, section 3: for a linear memory, mixing
    the cached memories with the gates first (memory soup) gives the gated residual
    read-out.  The soup is formed here per token, then applied once."""
    x = gi.make_cache_readout(SMALL)
    q, ck, g, oi = _f64(x)
    got = memcache.readout(q, ck, SMALL.seg, gates=g, o_in=oi)
    B, T, H, _ = q.shape
    N = ck.shape[2]
    want = oi.copy()
    for b in range(B):
        for h in range(H):
            for t in range(T):
                soup = np.zeros(ck.shape[-2:])
                for s in range(min(t // SMALL.seg, N)):
                    soup += g[b, t, h, s] * ck[b, h, s]
                want[b, t, h] += soup.T @ q[b, t, h]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_residual_is_prefix_sum():
    """Residual memory (all gates 1): each token reads the running sum of the caches
    of the segments before its own (cumulative sum, then one product)."""
    x = gi.make_cache_readout(SMALL.scaled(gate_kind="residual", seed=4))
    q, ck, _, oi = _f64(x)
    got = memcache.readout(q, ck, SMALL.seg, gates=None, o_in=oi)
    N = ck.shape[2]
    pref = np.concatenate([np.zeros_like(ck[:, :, :1]), np.cumsum(ck, axis=2)], axis=2)  # [B, H, N + 1, dk, dv]
    j = np.minimum(np.arange(q.shape[1]) // SMALL.seg, N)
    want = oi + np.einsum("bhtkv,bthk->bthv", pref[:, :, j], q)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_one_hot_query_reads_a_row():
    """q_t = e_i: the read-out of cache s is row i of M_s, weighted (closed form)."""
    w = SMALL.scaled(with_o_in=False, seed=5)
    x = gi.make_cache_readout(w)
    _, ck, g, _ = _f64(x)
    B, T, H, dk = x["q"].shape
    q = np.zeros((B, T, H, dk))
    idx = np.random.default_rng(0).integers(0, dk, (B, T, H))
    np.put_along_axis(q, idx[..., None], 1.0, axis=-1)
    got = memcache.readout(q, ck, w.seg, gates=g)
    N = ck.shape[2]
    for b in range(B):
        for h in range(H):
            for t in range(T):
                want = sum(g[b, t, h, s] * ck[b, h, s, idx[b, t, h], :] for s in range(min(t // w.seg, N)))
                np.testing.assert_allclose(got[b, t, h], want if np.ndim(want) else np.zeros(w.dv), atol=1e-14)


@pytest.mark.parametrize("case", ["no_cache", "segment_longer_than_T", "zero_gates"])
def test_degenerate_cases_are_the_online_read_out(case):
    """No cache to read (one segment: the plain recurrent read-out) or a router that
    keeps none: o_out == o_in exactly."""
    x = gi.make_cache_readout(SMALL.scaled(seed=6))
    q, ck, g, oi = _f64(x)
    seg = SMALL.seg
    if case == "no_cache":
        ck = ck[:, :, :0]
        g = g[..., :0]
    elif case == "segment_longer_than_T":
        seg = q.shape[1] + 1
    else:
        g = np.zeros_like(g)
    np.testing.assert_array_equal(memcache.readout(q, ck, seg, gates=g, o_in=oi), oi)


def test_sparse_router_is_gate_subset():
    """Sparse selective caching: the read-out with a top-k router equals the dense
    gated read-out with the gates of the unselected caches set to zero (linearity
    in the gates) and differs from the dense read-out when caches are dropped."""
    w = SMALL.scaled(gate_kind="topk", topk=2, seed=7)
    x = gi.make_cache_readout(w)
    q, ck, g, oi = _f64(x)
    dense = np.random.default_rng(1).uniform(0.5, 1.0, g.shape)
    got = memcache.readout(q, ck, w.seg, gates=g * dense, o_in=oi)
    a = memcache.readout(q, ck, w.seg, gates=dense * (g > 0), o_in=None)
    np.testing.assert_allclose(got, a + oi, rtol=1e-12, atol=1e-12)
    full = memcache.readout(q, ck, w.seg, gates=dense, o_in=oi)
    assert np.max(np.abs(full - got)) > 1e-3


def test_segment_states_match_uninterrupted_run():
    """The segment states are the states an uninterrupted run passes through: the last
    one (T a multiple of the segment) equals that run's final state, the read-outs are
    the run's, and an earlier one equals the final state of the run cut at its end."""
    w = gi.TINY_GDN_F32.scaled(B=2, T=48, H=2, dk=8, dv=8, chunk=16, s0_std=0.3, seed=21)
    x = gi.make_prefill(w)
    f = gi.prefill_f64(w, x)
    o, ST, ck = memcache.segment_states(f["q"], f["k"], f["v"], f["alpha"], f["beta_k"], 16, S0=f["S0"])
    o_full, ST_full = oracle.forward(f["q"], f["k"], f["v"], f["alpha"], f["beta_k"], S0=f["S0"])
    assert ck.shape == (2, 2, 3, 8, 8)
    np.testing.assert_allclose(o, o_full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ck[:, :, 2], ST_full, rtol=1e-12, atol=1e-13)
    cut = {k: (None if f[k] is None else f[k][:, :32]) for k in ("q", "k", "v", "alpha", "beta_k")}
    _, S32 = oracle.forward(cut["q"], cut["k"], cut["v"], cut["alpha"], cut["beta_k"], S0=f["S0"])
    np.testing.assert_allclose(ck[:, :, 1], S32, rtol=1e-12, atol=1e-13)
