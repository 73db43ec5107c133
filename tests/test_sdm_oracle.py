"""Pins of the Sparse Delta Memory oracle (oracle/sdm.py) on the CPU."""
import numpy as np
import pytest

import gdr_inputs as gi
import oracle
from oracle import sdm

TINY = gi.SDM_B4H16.scaled(name="sdm_tiny", B=2, T=12, H=2, n=6, dv=5, W=4, R=3, m0_std=0.5, seed=5)


@pytest.mark.parametrize("seed", range(6))
def test_product_key_identity(seed):
    """Resumo Técnico: Sparse Delta Memory, Mecanismo Central item 2: the top-k of the
    outer sum is the top-k of the outer sum of each half's top-k (computed here from
    the halves alone)."""
    rng = np.random.default_rng(seed)
    n, k = 9, 7
    s1 = rng.standard_normal(n).astype(np.float32)
    s2 = rng.standard_normal(n).astype(np.float32)
    slots, sc = sdm.select(s1, s2, k)
    a = np.argsort(-s1, kind="stable")[:k]
    b = np.argsort(-s2, kind="stable")[:k]
    cand = [(float(np.float32(s1[i] + s2[j])), i * n + j) for i in a for j in b]
    cand.sort(key=lambda x: (-x[0], x[1]))
    assert [c[1] for c in cand[:k]] == slots.tolist()
    np.testing.assert_array_equal(sc, np.array([c[0] for c in cand[:k]], dtype=np.float32))


def test_ties_take_the_lower_slot():
    s1 = np.array([1.0, 1.0, 0.0], dtype=np.float32)
    s2 = np.array([0.5, 0.5, 0.5], dtype=np.float32)
    slots, _ = sdm.select(s1, s2, 4)
    assert slots.tolist() == [0, 1, 2, 3]


def test_one_slot_is_the_dense_gated_delta_rule():
    """N = 1, W = R = 1: the only slot has weight 1 and is the dk = 1 state of the
    gated delta rule with k = q = 1 (the recurrence oracle, read after the write)."""
    w = TINY.scaled(n=1, W=1, R=1, seed=6)
    x = gi.make_sparse_memory(w)
    v = gi.as_f64(x["v"], w.io)
    o, MT, _, _ = sdm.forward(x["M0"], x["ks"], x["qs"], v, x["alpha"], x["beta"], 1, 1)
    ones = np.ones((w.B, w.T, w.H, 1))
    S0 = x["M0"].astype(np.float64)[:, :, :1, :]                  # [B, H, 1, dv]
    o_ref, S_ref = oracle.forward(ones, ones, v, x["alpha"].astype(np.float64), x["beta"].astype(np.float64),
                                  S0=S0)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(MT, S_ref, rtol=1e-12, atol=1e-14)


def test_no_write_reads_the_initial_table():
    """beta = 0, alpha = 1: the table is unchanged and o is the softmax-weighted
    read of M0 (closed form)."""
    w = TINY.scaled(seed=7)
    x = gi.make_sparse_memory(w)
    v = gi.as_f64(x["v"], w.io)
    ones, zeros = np.ones((w.B, w.T, w.H)), np.zeros((w.B, w.T, w.H))
    o, MT, _, rsl = sdm.forward(x["M0"], x["ks"], x["qs"], v, ones, zeros, w.W, w.R)
    np.testing.assert_array_equal(MT, x["M0"].astype(np.float64))
    b, t, h = 1, 7, 0
    s = (x["qs"][b, t, h, 0][:, None] + x["qs"][b, t, h, 1][None, :]).reshape(-1)
    sel = rsl[b, t, h]
    e = np.exp(s[sel].astype(np.float64) - s[sel].max())
    np.testing.assert_allclose(o[b, t, h], (e / e.sum()) @ x["M0"][b, h, sel].astype(np.float64), rtol=1e-12)


def test_untouched_slots_keep_their_values():
    w = TINY.scaled(seed=8)
    x = gi.make_sparse_memory(w)
    v = gi.as_f64(x["v"], w.io)
    _, MT, wsl, _ = sdm.forward(x["M0"], x["ks"], x["qs"], v, x["alpha"], x["beta"], w.W, w.R)
    for b in range(w.B):
        for h in range(w.H):
            touched = set(wsl[b, :, h].reshape(-1).tolist())
            for i in range(w.N):
                if i not in touched:
                    assert np.array_equal(MT[b, h, i], x["M0"][b, h, i].astype(np.float64))
    assert len(touched) < w.N


def test_single_full_write_stores_v():
    """alpha = beta = 1 and W = 1 (weight 1): the written slot becomes v_t exactly."""
    w = TINY.scaled(W=1, seed=9)
    x = gi.make_sparse_memory(w)
    v = gi.as_f64(x["v"], w.io)
    ones = np.ones((w.B, w.T, w.H))
    _, MT, wsl, _ = sdm.forward(x["M0"], x["ks"][:, :1], x["qs"][:, :1], v[:, :1], ones[:, :1], ones[:, :1], 1, w.R)
    for b in range(w.B):
        for h in range(w.H):
            np.testing.assert_array_equal(MT[b, h, wsl[b, 0, h, 0]], v[b, 0, h])
