"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle (oracle/gdr_ref.c) against something other than
itself: hand-derived worked examples (tests/golden), closed forms, invariants
of the recurrence, and a textbook library routine (a first-order IIR filter).
No test here re-types the oracle's own formula.
"""
import glob
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def _rand_inputs(rng, B, T, H, dk, dv, *, channel=False, beta_mode=0, kw=False, s0=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    alpha = rng.uniform(0.6, 1.0, (B, T, H, dk) if channel else (B, T, H))
    beta_k = rng.uniform(0.05, 1.0, (B, T, H) if beta_mode == 0 else (B, T, H, dk))
    beta_v = rng.uniform(0.05, 1.0, (B, T, H, dv)) if beta_mode == 2 else None
    k_w = k * (1.0 + 0.1 * rng.standard_normal(k.shape)) if kw else None
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.3 if s0 else None
    return dict(q=q, k=k, v=v, alpha=alpha, beta_k=beta_k, beta_v=beta_v, k_w=k_w, S0=S0)


def _run(x, **kw):
    return oracle.forward(x["q"], x["k"], x["v"], x["alpha"], x["beta_k"], k_w=x["k_w"],
                          beta_v=x["beta_v"], S0=x["S0"], **kw)


# --------------------------------------------------------------------------
# hand-derived worked examples
# --------------------------------------------------------------------------

@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "*.json"))),
                         ids=lambda p: os.path.basename(p))
def test_golden_worked_examples(path):
    g = json.load(open(path))
    T = len(g["k"])
    k = np.array(g["k"], dtype=np.float64)
    v = np.array(g["v"], dtype=np.float64)
    q = np.array(g["q"], dtype=np.float64)
    dk, dv = k.shape[1], v.shape[1]
    shape = lambda a, d: np.asarray(a, dtype=np.float64).reshape(1, T, 1, d)
    kw = None
    if "lambda" in g:  # delta-mem: alpha = lambda, beta' = 1, write key (beta/lambda) k, value lambda v
        lam = np.array(g["lambda"])
        beta = np.array(g["beta"])
        alpha = lam.reshape(1, T, 1)
        beta_k = np.ones((1, T, 1))
        kw = shape((beta / lam)[:, None] * k, dk)
        v_in = shape(lam[:, None] * v, dv)
    else:
        a = np.array(g["alpha"])
        alpha = a.reshape(1, T, 1) if a.ndim == 1 else a.reshape(1, T, 1, dk)
        b = np.array(g["beta"])
        beta_k = b.reshape(1, T, 1) if b.ndim == 1 else b.reshape(1, T, 1, dk)
        v_in = shape(v, dv)
        if "d" in g:
            kw = shape(np.array(g["d"]) * k, dk)
    if g["orientation"] == "page":
        S0 = np.array(g["S0_page"]).T.reshape(1, 1, dk, dv)
        ST_expect = np.array(g["ST_page"]).T
    else:
        S0 = np.array(g["S0"]).reshape(1, 1, dk, dv)
        ST_expect = np.array(g["ST"])
    o, ST = oracle.forward(shape(q, dk), shape(k, dk), v_in, alpha, beta_k, k_w=kw, S0=S0)
    np.testing.assert_allclose(o.reshape(T, dv), np.array(g["o"]), rtol=0, atol=TOL)
    np.testing.assert_allclose(ST[0, 0], ST_expect, rtol=0, atol=TOL)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("channel", [False, True])
@pytest.mark.parametrize("beta_mode", [0, 1, 2])
def test_beta_zero_is_pure_decay(channel, beta_mode):
    """beta = 0: S_t = Diag(prod_{s<=t} alpha_s) S0 and o_t = S_t^T q_t."""
    rng = np.random.default_rng(1)
    B, T, H, d = 2, 19, 3, 6
    x = _rand_inputs(rng, B, T, H, d, d, channel=channel, beta_mode=beta_mode)
    x["beta_k"] = np.zeros_like(x["beta_k"])
    if x["beta_v"] is not None:
        x["beta_v"] = np.zeros_like(x["beta_v"])
    o, ST = _run(x)
    a = x["alpha"] if channel else np.repeat(x["alpha"][..., None], d, axis=-1)
    cum = np.cumprod(a, axis=1)  # [B, T, H, dk]
    for b in range(B):
        for h in range(H):
            for t in range(T):
                St = cum[b, t, h][:, None] * x["S0"][b, h]
                np.testing.assert_allclose(o[b, t, h], St.T @ x["q"][b, t, h], atol=TOL, rtol=0)
            np.testing.assert_allclose(ST[b, h], cum[b, -1, h][:, None] * x["S0"][b, h],
                                       atol=TOL, rtol=0)


@pytest.mark.parametrize("beta_mode", [0, 1])
def test_orthonormal_keys_retrieve_exactly(beta_mode):
    """alpha = 1, beta = 1, orthonormal keys, T <= dk: S_T^T k_s = v_s for every s,
    and a query equal to an earlier key reads back its value."""
    rng = np.random.default_rng(2)
    d, T = 8, 8
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Qm.T[rng.permutation(d)[:T]]  # orthonormal rows
    k = keys.reshape(1, T, 1, d)
    v = rng.standard_normal((1, T, 1, d))
    alpha = np.ones((1, T, 1))
    beta = np.ones((1, T, 1)) if beta_mode == 0 else np.ones((1, T, 1, d))
    sel = [int(rng.integers(0, t + 1)) for t in range(T)]  # s <= t
    q = np.stack([keys[s] for s in sel]).reshape(1, T, 1, d)
    o, ST = oracle.forward(q, k, v, alpha, beta)
    for s in range(T):
        np.testing.assert_allclose(ST[0, 0].T @ keys[s], v[0, s, 0], atol=1e-12, rtol=0)
    for t in range(T):
        np.testing.assert_allclose(o[0, t, 0], v[0, sel[t], 0], atol=1e-12, rtol=0)


def test_osdn_write_key_equals_right_preconditioned_gradient_step():
    """Scaling the write key by d equals right-preconditioning the gradient of
    f(S) = 1/2 |S k - v|^2 (page orientation); gradient taken by central finite
    differences of f, which are exact for a quadratic up to rounding."""
    rng = np.random.default_rng(3)
    dk, dv = 5, 4
    for _ in range(5):
        Sp = rng.standard_normal((dv, dk))  # page orientation
        k = rng.standard_normal(dk)
        v = rng.standard_normal(dv)
        d = 1.0 + 0.3 * rng.standard_normal(dk)
        beta = rng.uniform(0.1, 1.0)
        f = lambda M: 0.5 * np.sum((M @ k - v) ** 2)
        grad = np.zeros_like(Sp)
        h = 1e-3
        for i in range(dv):
            for j in range(dk):
                E = np.zeros_like(Sp)
                E[i, j] = h
                grad[i, j] = (f(Sp + E) - f(Sp - E)) / (2 * h)
        expect = Sp - beta * grad @ np.diag(d)
        o, ST = oracle.forward(np.zeros((1, 1, 1, dk)), k.reshape(1, 1, 1, dk), v.reshape(1, 1, 1, dv),
                               np.ones((1, 1, 1)), np.full((1, 1, 1), beta),
                               k_w=(d * k).reshape(1, 1, 1, dk), S0=Sp.T.reshape(1, 1, dk, dv).copy())
        np.testing.assert_allclose(ST[0, 0].T, expect, atol=1e-9, rtol=0)


def test_osdn_hypergradient_surrogate_closed_form():
    """For the ungated preconditioned step, (f(S_t) - f(S_{t-1})) / |grad f(S_{t-1})|_F^2
    equals ((1 - beta <d, k^2>)^2 - 1) / (2 |k|^2), independent of S and v."""
    rng = np.random.default_rng(4)
    dk, dv = 7, 5
    for _ in range(10):
        S = rng.standard_normal((dk, dv))
        k = rng.standard_normal(dk)
        v = rng.standard_normal(dv)
        d = np.abs(1.0 + 0.5 * rng.standard_normal(dk))
        beta = rng.uniform(0.05, 1.0)
        _, ST = oracle.forward(np.zeros((1, 1, 1, dk)), k.reshape(1, 1, 1, dk), v.reshape(1, 1, 1, dv),
                               np.ones((1, 1, 1)), np.full((1, 1, 1), beta),
                               k_w=(d * k).reshape(1, 1, 1, dk), S0=S.reshape(1, 1, dk, dv).copy())
        f = lambda M: 0.5 * np.sum((M.T @ k - v) ** 2)
        gnorm2 = np.sum((S.T @ k - v) ** 2) * np.sum(k * k)
        h_num = (f(ST[0, 0]) - f(S)) / gnorm2
        h_closed = ((1 - beta * np.dot(d, k * k)) ** 2 - 1) / (2 * np.dot(k, k))
        assert abs(h_num - h_closed) <= 1e-12 * max(1.0, abs(h_closed))


@pytest.mark.parametrize("beta_mode,kw", [(0, False), (0, True), (1, False), (2, False), (2, True)])
@pytest.mark.parametrize("channel", [False, True])
def test_residual_contracts_by_one_minus_u_dot_w(beta_mode, kw, channel):
    """After each step the residual on the erase key shrinks by (1 - u.w):
    vh - S_t^T u = (1 - u.w) (vh - (Diag(alpha) S_{t-1})^T u), with
    u = sqrt(beta^k) k, w = sqrt(beta^k) k_w, vh = sqrt(beta^v) v."""
    rng = np.random.default_rng(5)
    d = 6
    for _ in range(6):
        x = _rand_inputs(rng, 1, 1, 1, d, d, channel=channel, beta_mode=beta_mode, kw=kw)
        _, ST = _run(x)
        k = x["k"][0, 0, 0]
        kwv = k if x["k_w"] is None else x["k_w"][0, 0, 0]
        bk = x["beta_k"][0, 0, 0]
        bv = bk if beta_mode != 2 else x["beta_v"][0, 0, 0]
        u, w, vh = np.sqrt(bk) * k, np.sqrt(bk) * kwv, np.sqrt(bv) * x["v"][0, 0, 0]
        a = x["alpha"][0, 0, 0]
        Xd = (a[:, None] if channel else a) * x["S0"][0, 0]
        lhs = vh - ST[0, 0].T @ u
        rhs = (1.0 - u @ w) * (vh - Xd.T @ u)
        np.testing.assert_allclose(lhs, rhs, atol=1e-12, rtol=0)


def test_fg2_constant_beta_vector_is_scalar_gdn():
    """A beta vector c*1 through the absorbed (I - kk^T) form equals the scalar-beta gated
    delta rule with beta = c; separate beta^k = beta^v equals one shared vector."""
    rng = np.random.default_rng(6)
    B, T, H, d = 2, 23, 2, 8
    x = _rand_inputs(rng, B, T, H, d, d, channel=True, beta_mode=0)
    o0, S0 = _run(x)
    xv = dict(x)
    xv["beta_k"] = np.repeat(x["beta_k"][..., None], d, axis=-1)
    o1, S1 = _run(xv)
    np.testing.assert_allclose(o1, o0, atol=1e-12, rtol=0)
    np.testing.assert_allclose(S1, S0, atol=1e-12, rtol=0)
    xv["beta_v"] = xv["beta_k"].copy()
    o2, S2 = _run(xv)
    np.testing.assert_allclose(o2, o0, atol=1e-12, rtol=0)
    np.testing.assert_allclose(S2, S0, atol=1e-12, rtol=0)


def test_deltamem_reparametrisation():
    """The delta-mem update (prediction from the undecayed state, page orientation)
    equals the oracle's decayed-prediction step with alpha = lambda, beta' = 1,
    write key (beta/lambda) k and value lambda v, for lambda > 0 (r = 8 state)."""
    rng = np.random.default_rng(7)
    r, T = 8, 40
    lam = rng.uniform(0.5, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T)
    k = rng.standard_normal((T, r))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, r))
    q = rng.standard_normal((T, r))
    Sp = 0.1 * rng.standard_normal((r, r))
    Sp0 = Sp.copy()
    o_lit = np.zeros((T, r))
    for t in range(T):  # page formula, page orientation, read-out after the write
        Sp = lam[t] * Sp + beta[t] * np.outer(v[t] - Sp @ k[t], k[t])
        o_lit[t] = Sp @ q[t]
    o, ST = oracle.forward(q.reshape(1, T, 1, r), k.reshape(1, T, 1, r),
                           (lam[:, None] * v).reshape(1, T, 1, r), lam.reshape(1, T, 1),
                           np.ones((1, T, 1)), k_w=((beta / lam)[:, None] * k).reshape(1, T, 1, r),
                           S0=Sp0.T.reshape(1, 1, r, r).copy())
    np.testing.assert_allclose(o.reshape(T, r), o_lit, atol=1e-12, rtol=0)
    np.testing.assert_allclose(ST[0, 0].T, Sp, atol=1e-12, rtol=0)


def test_scalar_case_is_first_order_iir_filter():
    """dk = dv = 1 with constant alpha, beta, k: s_t = alpha (1 - beta k^2) s_{t-1} + beta k v_t,
    a first-order IIR filter (scipy.signal.lfilter), read out as o_t = q_t s_t."""
    from scipy import signal

    rng = np.random.default_rng(8)
    T = 300
    for alpha, beta, kk in [(0.97, 0.4, 0.8), (1.0, 1.0, 1.0), (0.5, 0.9, -1.2)]:
        v = rng.standard_normal(T)
        q = rng.standard_normal(T)
        s0 = 0.7
        a1 = alpha * (1.0 - beta * kk * kk)
        zi = signal.lfiltic([beta * kk], [1.0, -a1], y=[s0])
        s, _ = signal.lfilter([beta * kk], [1.0, -a1], v, zi=zi)
        o, ST = oracle.forward(q.reshape(1, T, 1, 1), np.full((1, T, 1, 1), kk), v.reshape(1, T, 1, 1),
                               np.full((1, T, 1), alpha), np.full((1, T, 1), beta),
                               S0=np.full((1, 1, 1, 1), s0))
        np.testing.assert_allclose(o.ravel(), q * s, atol=1e-11, rtol=1e-12)
        np.testing.assert_allclose(ST.ravel(), [s[-1]], atol=1e-11, rtol=1e-12)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("beta_mode", [0, 2])
def test_linear_in_values_and_initial_state(beta_mode):
    rng = np.random.default_rng(9)
    B, T, H, d = 1, 30, 2, 6
    x1 = _rand_inputs(rng, B, T, H, d, d, channel=True, beta_mode=beta_mode, kw=True)
    x2 = dict(x1)
    x2["v"] = rng.standard_normal(x1["v"].shape)
    x2["S0"] = rng.standard_normal(x1["S0"].shape)
    a, b = 0.7, -1.3
    x3 = dict(x1)
    x3["v"] = a * x1["v"] + b * x2["v"]
    x3["S0"] = a * x1["S0"] + b * x2["S0"]
    o1, S1 = _run(x1)
    o2, S2 = _run(x2)
    o3, S3 = _run(x3)
    np.testing.assert_allclose(o3, a * o1 + b * o2, atol=1e-11, rtol=0)
    np.testing.assert_allclose(S3, a * S1 + b * S2, atol=1e-11, rtol=0)


def test_segment_resume_equals_one_pass():
    rng = np.random.default_rng(10)
    B, T, H, d = 2, 50, 2, 8
    x = _rand_inputs(rng, B, T, H, d, d, channel=True, beta_mode=2, kw=True)
    o, ST = _run(x)
    t1 = 17
    cut = lambda a, s: None if a is None else a[:, s]
    xa = {key: cut(x[key], slice(0, t1)) for key in ("q", "k", "v", "alpha", "beta_k", "beta_v", "k_w")}
    xa["S0"] = x["S0"]
    oa, Sa = _run(xa)
    xb = {key: cut(x[key], slice(t1, T)) for key in ("q", "k", "v", "alpha", "beta_k", "beta_v", "k_w")}
    xb["S0"] = Sa
    ob, Sb = _run(xb)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(Sb, ST, atol=1e-12, rtol=0)


def test_decode_step_matches_forward_of_one_token():
    rng = np.random.default_rng(11)
    B, H, d = 3, 4, 8
    x = _rand_inputs(rng, B, 1, H, d, d, channel=True, beta_mode=2, kw=True)
    o, ST = _run(x)
    od, Sd = oracle.decode_step(x["S0"], x["q"][:, 0], x["k"][:, 0], x["v"][:, 0], x["alpha"][:, 0],
                                x["beta_k"][:, 0], k_w=x["k_w"][:, 0], beta_v=x["beta_v"][:, 0])
    np.testing.assert_array_equal(od, o[:, 0])
    np.testing.assert_array_equal(Sd, ST)


def test_head_subset_matches_full_run():
    rng = np.random.default_rng(12)
    x = _rand_inputs(rng, 2, 9, 3, 4, 4)
    o, ST = _run(x)
    os_, Ss = _run(x, heads=[4, 1])
    for bh in (4, 1):
        b, h = divmod(bh, 3)
        np.testing.assert_array_equal(os_[b, :, h], o[b, :, h])
        np.testing.assert_array_equal(Ss[b, h], ST[b, h])
    assert np.isnan(os_[0, :, 0]).all()


def test_rejects_bad_arguments():
    rng = np.random.default_rng(13)
    x = _rand_inputs(rng, 1, 4, 1, 4, 6, beta_mode=1)  # shared beta needs dk == dv
    with pytest.raises(ValueError):
        _run(x)


# ---------------------------------------------------------------------------
# delta-mem step in the page's own form (oracle.dmem_step) [delta-mem page,
# section 2.A update rule, section 2.C read]
# ---------------------------------------------------------------------------
def _unit_rows(n, d, seed):
    """n orthonormal rows in R^d (QR of a Gaussian), fp64."""
    q_, _ = np.linalg.qr(np.random.default_rng(seed).normal(size=(d, n)))
    return q_.T


def test_dmem_reads_before_the_write_and_retrieves_exactly():
    """lambda = beta = 1, orthonormal keys, zero memory: reading k_s after its write returns
    v_s; reading the key being written at the same step returns 0 (the read sees M_{t-1})."""
    d, T = 8, 5
    keys = _unit_rows(T, d, 3)
    vals = np.random.default_rng(4).normal(size=(T, d))
    M = np.zeros((1, 1, d, d))
    one = np.ones((1, 1))
    for t in range(T):
        # query the current key: nothing stored along it yet
        r, M_next = oracle.dmem_step(M, keys[t][None, None], keys[t][None, None], vals[t][None, None], one, one)
        assert np.allclose(r[0, 0], 0.0, atol=1e-12)
        M = M_next
        for s in range(t + 1):  # every earlier write is retrieved exactly
            r, _ = oracle.dmem_step(M, keys[s][None, None], keys[t][None, None], vals[t][None, None], one, 0 * one)
            assert np.allclose(r[0, 0], vals[s], atol=1e-12)


def test_dmem_zero_write_gate_is_pure_decay():
    """beta = 0: M_t = lambda_t M_{t-1}, r_t = (prod_{s<t} lambda_s) M_0 q (closed form)."""
    rng = np.random.default_rng(7)
    B, H, d = 2, 3, 6
    M0 = rng.normal(size=(B, H, d, d))
    M = M0.copy()
    prod = np.ones((B, H))
    for t in range(4):
        q = rng.normal(size=(B, H, d))
        lam = rng.uniform(0.5, 1.0, size=(B, H))
        r, M = oracle.dmem_step(M, q, rng.normal(size=(B, H, d)), rng.normal(size=(B, H, d)), lam, np.zeros((B, H)))
        assert np.allclose(r, np.einsum("bhac,bhc->bha", M0, q) * prod[..., None], atol=1e-12)
        prod *= lam


def test_dmem_one_shot_write():
    """lambda = 1 and beta = 1 / |k|^2: after the step the memory maps k_t to v_t exactly
    (the residual v - M k is fully corrected along k)."""
    rng = np.random.default_rng(9)
    d = 7
    M = rng.normal(size=(1, 1, d, d))
    k = rng.normal(size=(1, 1, d))
    v = rng.normal(size=(1, 1, d))
    beta = np.array([[1.0 / float(k[0, 0] @ k[0, 0])]])
    _, M1 = oracle.dmem_step(M, rng.normal(size=(1, 1, d)), k, v, np.ones((1, 1)), beta)
    assert np.allclose(M1[0, 0] @ k[0, 0], v[0, 0], atol=1e-12)


def test_dmem_equals_gated_step_reparametrised():
    """Against the independent gated delta-rule oracle (decayed prediction): with
    alpha = lambda, unit write strength, write key (beta / lambda) k and value lambda v,
    its state is the transposed delta-mem memory after the step."""
    rng = np.random.default_rng(11)
    B, H, dk, dv = 2, 2, 5, 4
    M = rng.normal(size=(B, H, dv, dk))
    q, k = rng.normal(size=(B, H, dk)), rng.normal(size=(B, H, dk))
    v = rng.normal(size=(B, H, dv))
    lam = rng.uniform(0.3, 1.0, size=(B, H))
    beta = rng.uniform(0.0, 1.0, size=(B, H))
    _, M1 = oracle.dmem_step(M, q, k, v, lam, beta)
    S = np.ascontiguousarray(np.swapaxes(M, -1, -2))
    _, S1 = oracle.decode_step(S, q, k, lam[..., None] * v, lam, np.ones((B, H)),
                               k_w=(beta / lam)[..., None] * k)
    assert np.allclose(np.swapaxes(S1, -1, -2), M1, atol=1e-12)
