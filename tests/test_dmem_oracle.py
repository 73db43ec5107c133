"""Pins of the delta-mem write-granularity oracle (oracle/dmem.py) on the CPU.

delta-mem: Efficient Online Memory for Large Language Models, sections 2.A (update),
2.C (read before the write) and 2.D (token-state, sequence-state and multi-state
writes).  The token-state case is pinned to the C oracle's delta-mem step (a separate
implementation, itself pinned by the reparametrisation identity); the segment and
sub-state cases by closed forms and by reductions to the token-state case."""
import numpy as np
import pytest

import gdr_inputs as gi
import oracle
from oracle import dmem

SMALL = gi.DmemSeq("dmem_tiny", B=3, T=23, H=4, J=1, r=8, lam_mu=-2.0, m_std=0.3, seed=41)


def _inputs(w):
    return gi.dmem_seq_f64(w, gi.make_dmem_seq(w))


def _c_steps(x):
    """Token-by-token delta-mem steps of the C oracle: reads [B, T, H, r] and M."""
    M = x["M0"].copy()
    B, T, H, r = x["q"].shape
    reads = np.zeros((B, T, H, r))
    for t in range(T):
        reads[:, t], M = oracle.dmem_step(M, x["q"][:, t], x["k"][:, t], x["v"][:, t], x["lam"][:, t],
                                          x["beta"][:, t])
    return reads, M


def test_token_writes_match_the_per_token_step():
    """TSW (no segment marks) is the page's per-token step, read before the write."""
    x = _inputs(SMALL)
    out, M = dmem.forward(x["M0"], x["q"], x["k"], x["v"], x["lam"], x["beta"])
    reads, Mc = _c_steps(x)
    np.testing.assert_allclose(out, reads, rtol=0, atol=1e-13)
    np.testing.assert_allclose(M, Mc, rtol=0, atol=1e-13)


def test_one_token_segments_are_token_writes():
    """SSW with every token marked as a segment end is TSW."""
    x = _inputs(SMALL)
    marks = np.ones(x["q"].shape[:2], dtype=np.uint8)
    a = dmem.forward(x["M0"], x["q"], x["k"], x["v"], x["lam"], x["beta"], seg_end=marks)
    b = dmem.forward(x["M0"], x["q"], x["k"], x["v"], x["lam"], x["beta"])
    for u, w in zip(a, b):
        np.testing.assert_array_equal(u, w)


@pytest.mark.parametrize("J", [2, 4])
def test_sub_state_reads_are_summed_over_independent_memories(J):
    """MSW: each sub-state evolves as its own token-state memory; the group's read is
    the sum of its sub-states' reads."""
    x = _inputs(SMALL)
    out, M = dmem.forward(x["M0"], x["q"], x["k"], x["v"], x["lam"], x["beta"], J=J)
    reads, Mc = _c_steps(x)
    B, T, H, r = reads.shape
    want = np.stack([reads[:, :, g * J:(g + 1) * J].sum(axis=2) for g in range(H // J)], axis=2)
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-13)
    np.testing.assert_allclose(M, Mc, rtol=0, atol=1e-13)


def test_one_sub_state_is_token_writes():
    x = _inputs(SMALL)
    a = dmem.forward(x["M0"], x["q"], x["k"], x["v"], x["lam"], x["beta"], J=1)
    reads, Mc = _c_steps(x)
    np.testing.assert_allclose(a[0], reads, rtol=0, atol=1e-13)


def test_disjoint_orthonormal_sub_states_retrieve_exactly():
    """MSW, J = 4 sub-states of an 8-wide memory, sub-state j writing only keys in
    span(e_2j, e_2j+1) with lambda = beta = 1 from M0 = 0: a query equal to any stored
    key (sent to every sub-state) reads back exactly its value -- the other sub-states
    hold nothing along it -- and a query outside every written key reads 0."""
    r, J, T = 8, 4, 9
    rng = np.random.default_rng(3)
    q = np.zeros((1, T, J, r))
    k = np.zeros((1, T, J, r))
    v = np.zeros((1, T, J, r))
    stored = []
    for j in range(J):
        for s in range(2):                      # tokens 0, 1: sub-state j writes e_2j, e_2j+1
            k[0, s, j, 2 * j + s] = 1.0
            v[0, s, j] = rng.standard_normal(r)
            stored.append((j, s))
    # tokens 2 .. 8 write nothing (beta = 0) and query
    queries = [(0, 0), (0, 1), (1, 0), (2, 1), (3, 0), (3, 1)]
    for t, (j, s) in enumerate(queries, start=2):
        q[0, t, :, 2 * j + s] = 1.0             # the same query to every sub-state
    q[0, T - 1, :] = 0.0
    lam = np.ones((1, T, J))
    beta = np.zeros((1, T, J))
    beta[0, :2] = 1.0
    out, _ = dmem.forward(np.zeros((1, J, r, r)), q, k, v, lam, beta, J=J)
    for t, (j, s) in enumerate(queries, start=2):
        np.testing.assert_allclose(out[0, t, 0], v[0, s, j], rtol=0, atol=1e-15)
    np.testing.assert_array_equal(out[0, T - 1, 0], np.zeros(r))


def test_segment_write_uses_the_mean_key_and_value():
    """Closed form: from M0 = 0 with lambda = beta = 1, a two-token segment with keys e1,
    e2 and values v1, v2 leaves M = vbar kbar^T (kbar = (e1 + e2) / 2,
    vbar = (v1 + v2) / 2), so the next token's query e1 reads (v1 + v2) / 4."""
    r = 8
    rng = np.random.default_rng(4)
    v1, v2 = rng.standard_normal(r), rng.standard_normal(r)
    q = np.zeros((1, 3, 1, r))
    k = np.zeros((1, 3, 1, r))
    v = np.zeros((1, 3, 1, r))
    k[0, 0, 0, 0] = 1.0
    k[0, 1, 0, 1] = 1.0
    v[0, 0, 0], v[0, 1, 0] = v1, v2
    q[0, 2, 0, 0] = 1.0
    lam = np.ones((1, 3, 1))
    beta = np.ones((1, 3, 1))
    beta[0, 2] = 0.0
    marks = np.array([[0, 1, 1]], dtype=np.uint8)
    out, M = dmem.forward(np.zeros((1, 1, r, r)), q, k, v, lam, beta, seg_end=marks)
    kbar = np.zeros(r)
    kbar[:2] = 0.5
    np.testing.assert_allclose(M[0, 0], np.outer((v1 + v2) / 2, kbar), rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 2, 0], (v1 + v2) / 4, rtol=0, atol=1e-15)


@pytest.mark.parametrize("n", [2, 5, 11])
def test_segment_of_one_repeated_token_is_one_token_write(n):
    """A segment of n copies of one token (k, v) is a single write of that token with
    the segment's closing gates, whatever n is (a mean, not a sum)."""
    r = 8
    rng = np.random.default_rng(5 + n)
    M0 = rng.standard_normal((1, 1, r, r)) * 0.3
    kk = rng.standard_normal(r)
    kk /= np.linalg.norm(kk)
    vv = rng.standard_normal(r)
    q = rng.standard_normal((1, n, 1, r))
    k = np.broadcast_to(kk, (1, n, 1, r)).copy()
    v = np.broadcast_to(vv, (1, n, 1, r)).copy()
    lam = rng.uniform(0.2, 0.9, (1, n, 1))
    beta = rng.uniform(0.2, 0.9, (1, n, 1))
    marks = np.zeros((1, n), dtype=np.uint8)
    marks[0, -1] = 1
    _, M = dmem.forward(M0, q, k, v, lam, beta, seg_end=marks)
    lt, bt = lam[0, -1, 0], beta[0, -1, 0]
    want = lt * M0[0, 0] + bt * np.outer(vv - M0[0, 0] @ kk, kk)
    np.testing.assert_allclose(M[0, 0], want, rtol=0, atol=1e-14)


def test_reads_inside_a_segment_see_the_memory_before_it():
    """Every token of a segment reads M_before q_t: from M0 the first segment's reads are
    M0 q_t exactly; the second segment's reads are the first write's memory times q_t."""
    w = SMALL.scaled(B=2, T=17, H=2, seg_mean=6.0, seed=42)
    x = _inputs(w)
    marks = np.zeros((2, 17), dtype=np.uint8)
    marks[:, 6] = 1
    marks[:, 16] = 1
    out, _ = dmem.forward(x["M0"], x["q"], x["k"], x["v"], x["lam"], x["beta"], seg_end=marks)
    for b in range(2):
        for h in range(2):
            M1 = dmem.write(x["M0"][b, h], x["k"][b, :7, h].mean(axis=0), x["v"][b, :7, h].mean(axis=0),
                            x["lam"][b, 6, h], x["beta"][b, 6, h])
            for t in range(17):
                Mt = x["M0"][b, h] if t <= 6 else M1
                np.testing.assert_allclose(out[b, t, h], Mt @ x["q"][b, t, h], rtol=0, atol=1e-14)


def test_only_the_closing_tokens_gates_matter():
    """The gates of a segment's other tokens are not used: changing them changes
    nothing; the last token of the sequence closes a segment even unmarked."""
    w = SMALL.scaled(seg_mean=5.0, seed=43)
    x = _inputs(w)
    marks = x["seg_end"].copy()
    a = dmem.forward(x["M0"], x["q"], x["k"], x["v"], x["lam"], x["beta"], seg_end=marks)
    lam2, beta2 = x["lam"].copy(), x["beta"].copy()
    open_ = marks == 0
    open_[:, -1] = False
    lam2[open_] = 0.123
    beta2[open_] = 0.987
    marks2 = marks.copy()
    marks2[:, -1] = 0                                # the last token closes anyway
    b = dmem.forward(x["M0"], x["q"], x["k"], x["v"], lam2, beta2, seg_end=marks2)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_no_write_only_decays():
    """beta = 0: every segment write only multiplies by its closing lambda, so
    M_T = (product of the closing lambdas) M0."""
    w = SMALL.scaled(seg_mean=4.0, seed=44)
    x = _inputs(w)
    beta = np.zeros_like(x["beta"])
    _, M = dmem.forward(x["M0"], x["q"], x["k"], x["v"], x["lam"], beta, seg_end=x["seg_end"])
    closes = x["seg_end"].astype(bool)
    for b in range(w.B):
        for h in range(w.H):
            f = np.prod(x["lam"][b, closes[b], h])
            np.testing.assert_allclose(M[b, h], f * x["M0"][b, h], rtol=1e-14, atol=1e-300)
