"""Pins of the OSDN phase-1 oracle (oracle.osdn_precond) on the CPU.

The surrogate h_t is rebuilt here from its definition -- the change of the
per-token loss f_t(S) = 1/2 |S^T k - v|^2 over one step of the gated delta rule
(run by the independent recurrence oracle, write key d (.) k), divided by the
squared gradient norm [OSDN page, section 2.2] -- and the scan's update is checked
against a finite-difference gradient of it.  q_geo is checked against loss ratios
measured on the phase-2 recurrence itself.
"""
import numpy as np
import pytest

import oracle


def _loss(S, k, v):
    r = S.T @ k - v
    return 0.5 * float(r @ r)


def _h_from_definition(d, S, k, v, beta):
    """(f(S_t) - f(S_{t-1})) / |grad f(S_{t-1})|^2 with S_t one step of the delta rule
    (alpha = 1) whose write key is d (.) k."""
    dk, dv = S.shape
    _, S1 = oracle.decode_step(S[None, None], np.zeros((1, 1, dk)), k[None, None], v[None, None],
                               np.ones((1, 1)), np.full((1, 1), beta), k_w=(d * k)[None, None])
    g2 = float(k @ k) * float(np.sum((S.T @ k - v) ** 2))     # |k (S^T k - v)^T|_F^2
    return (_loss(S1[0, 0], k, v) - _loss(S, k, v)) / g2


def _one_token(seed, dk=6, dv=4):
    rng = np.random.default_rng(seed)
    S = rng.normal(size=(dk, dv))
    k = rng.normal(size=dk)
    v = rng.normal(size=dv)
    d = rng.uniform(0.5, 1.5, dk)
    beta = float(rng.uniform(0.2, 0.9))
    return S, k, v, d, beta


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_update_is_gradient_descent_on_the_surrogate(seed):
    S, k, v, d, beta = _one_token(seed)
    eta = 0.3
    _, d1, _ = oracle.osdn_precond(k[None, None, None], np.full((1, 1, 1), beta), eta, d0=d[None, None])
    step = (d - d1[0, 0]) / eta                                   # = grad h at d
    fd = np.empty_like(d)
    for i in range(d.size):
        e = np.zeros_like(d)
        e[i] = 1e-6
        fd[i] = (_h_from_definition(d + e, S, k, v, beta) - _h_from_definition(d - e, S, k, v, beta)) / 2e-6
    np.testing.assert_allclose(step, fd, rtol=1e-6, atol=1e-9)


def test_one_step_lowers_the_surrogate():
    S, k, v, d, beta = _one_token(5)
    _, d1, _ = oracle.osdn_precond(k[None, None, None], np.full((1, 1, 1), beta), 0.05, d0=d[None, None])
    assert _h_from_definition(d1[0, 0], S, k, v, beta) < _h_from_definition(d, S, k, v, beta)


def test_newton_condition_is_a_fixed_point():
    """beta <d, k^2> = 1 [OSDN page, section 3, gated Newton condition]: zero gradient
    (d only retained), and the step removes the residual: loss ratio 0."""
    rng = np.random.default_rng(7)
    k = rng.normal(size=8)
    beta = 0.5
    d = np.full(8, 1.0 / (beta * float(k @ k)))
    kw, d1, qg = oracle.osdn_precond(k[None, None, None], np.full((1, 1, 1), beta), 0.7,
                                     r=np.full((1, 1, 1), 0.9), d0=d[None, None])
    np.testing.assert_allclose(d1[0, 0], 0.9 * d, rtol=1e-14)
    assert qg[0, 0] == 0.0


def test_frozen_preconditioner():
    """eta = 0, r = 1: the write keys are d0 (.) k, d stays d0, and q_geo is the
    geometric mean of (1 - beta <d0, k^2>)^2 (closed form)."""
    rng = np.random.default_rng(9)
    B, T, H, dk = 2, 7, 3, 5
    k = rng.normal(size=(B, T, H, dk))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    d0 = rng.uniform(0.5, 1.5, (B, H, dk))
    kw, dT, qg = oracle.osdn_precond(k, beta, 0.0, d0=d0)
    np.testing.assert_array_equal(kw, d0[:, None] * k)
    np.testing.assert_array_equal(dT, d0)
    u = 1.0 - beta * np.einsum("bhi,bthi->bth", d0, k * k)
    np.testing.assert_allclose(qg, np.exp(np.mean(np.log(u * u), axis=1)), rtol=1e-12)


def test_full_forgetting():
    """r = 0: the preconditioner restarts from the last gradient step alone,
    d_{t+1} = eta beta_t (1 - beta_t <d_t, k_t^2>) k_t^2 / |k_t|^2 (closed form)."""
    rng = np.random.default_rng(11)
    k = rng.normal(size=(1, 2, 1, 4))
    beta = np.array([[[0.4], [0.6]]])
    d0 = np.array([[[1.0, 2.0, 0.5, 1.5]]])
    eta = 0.8
    kw, dT, _ = oracle.osdn_precond(k, beta, eta, r=np.zeros((1, 2, 1)), d0=d0)
    a0, a1 = k[0, 0, 0] ** 2, k[0, 1, 0] ** 2
    d1 = eta * 0.4 * (1 - 0.4 * d0[0, 0] @ a0) * a0 / a0.sum()
    np.testing.assert_allclose(kw[0, 1, 0], d1 * k[0, 1, 0], rtol=1e-13)
    d2 = eta * 0.6 * (1 - 0.6 * d1 @ a1) * a1 / a1.sum()
    np.testing.assert_allclose(dT[0, 0], d2, rtol=1e-13)


def test_qgeo_matches_the_phase_two_recurrence():
    """Run phase 2 (delta rule, alpha = 1, scalar beta) token by token with the
    phase-1 write keys and measure f_t(S_t) / f_t(S_{t-1}) on its states; q_geo is
    their geometric mean [OSDN page, section 4.2]."""
    rng = np.random.default_rng(13)
    B, T, H, dk, dv = 1, 12, 2, 6, 3
    k = rng.normal(size=(B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(B, T, H, dv))
    beta = rng.uniform(0.2, 0.8, (B, T, H))
    r = rng.uniform(0.8, 1.0, (B, T, H))
    kw, _, qg = oracle.osdn_precond(k, beta, 0.5, r=r)
    S = rng.normal(size=(B, H, dk, dv))
    logs = np.zeros((B, H))
    for t in range(T):
        before = np.array([[_loss(S[b, h], k[b, t, h], v[b, t, h]) for h in range(H)] for b in range(B)])
        _, S = oracle.decode_step(S, np.zeros((B, H, dk)), k[:, t], v[:, t], np.ones((B, H)), beta[:, t],
                                  k_w=kw[:, t])
        after = np.array([[_loss(S[b, h], k[b, t, h], v[b, t, h]) for h in range(H)] for b in range(B)])
        logs += np.log(after / before)
    np.testing.assert_allclose(qg, np.exp(logs / T), rtol=1e-9)
