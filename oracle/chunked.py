"""Chunkwise (WY / UT-transform) evaluation of the gated delta rule in NumPy fp64.

TEST INFRASTRUCTURE ONLY (part of the oracle package; never used by the GPU
library).  It is deliberately unoptimised and is meant for tiny inputs.

The pages name the chunk-parallel WY form (FG2-GDN page, sections 2.A and 3;
OSDN page, sections 1 and 2.1: only the storage key K is replaced by the
preconditioned key in the block Gram matrix and the intra-block scores) but do
not write it out.  The form below is derived from the per-token step

    X_t = Diag(a_t) S_{t-1},   S_t = X_t + w_t (vh_t - X_t^T u_t)^T,   o_t = S_t^T q_t

with erase key u = sqrt(beta^k) k, write key w = sqrt(beta^k) k_w and written
value vh = sqrt(beta^v) v (scalar beta broadcasts; k_w defaults to k).  For a
chunk of C tokens entering with state S, with g_t = sum_{s<=t} log a_s (a
vector over key channels) and Ub = e^g U, Wb = W e^{-g}, Qb = e^g Q row-wise:

    A   = strictly-lower(Ub Wb^T)                     block Gram matrix
    Tm  = (I + A)^{-1}                                unit lower-triangular
    W'  = Tm Ub,  U' = Tm Vh                          WY factors
    D   = U' - W' S                                   per-token residuals
    P   = lower-incl-diagonal(Qb Wb^T)                intra-chunk scores
    O   = Qb S + P D
    S  <- Diag(e^{g_C}) S + (Wb e^{g_C})^T D

Every step is a plain matrix product or inverse; no blocking, fusion or
reordering beyond these equations.
"""
from __future__ import annotations

import numpy as np


def _expand(x, n):
    """Scalar-per-token gate [..] -> per-channel [.., n] (broadcast)."""
    return np.repeat(x[..., None], n, axis=-1) if x.ndim == 3 else x


def forward_chunked(q, k, v, alpha, beta_k, *, chunk, k_w=None, beta_v=None, S0=None):
    """Same contract as ``oracle.forward`` (fp64 [B, T, H, D] arrays)."""
    q, k, v, alpha, beta_k = (np.asarray(a, dtype=np.float64) for a in (q, k, v, alpha, beta_k))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    kw = k if k_w is None else np.asarray(k_w, dtype=np.float64)
    a = _expand(alpha, dk)
    bk = _expand(beta_k, dk)
    if beta_v is not None:
        bv = np.asarray(beta_v, dtype=np.float64)
    elif beta_k.ndim == 3:
        bv = _expand(beta_k, dv)
    else:
        bv = bk  # one shared beta vector (needs dk == dv)
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            for c0 in range(0, T, chunk):
                c1 = min(T, c0 + chunk)
                n = c1 - c0
                U = np.sqrt(bk[b, c0:c1, h]) * k[b, c0:c1, h]
                W = np.sqrt(bk[b, c0:c1, h]) * kw[b, c0:c1, h]
                Vh = np.sqrt(bv[b, c0:c1, h]) * v[b, c0:c1, h]
                Q = q[b, c0:c1, h]
                g = np.cumsum(np.log(a[b, c0:c1, h]), axis=0)
                Ub, Wb, Qb = np.exp(g) * U, W * np.exp(-g), np.exp(g) * Q
                A = np.tril(Ub @ Wb.T, -1)
                Tm = np.linalg.inv(np.eye(n) + A)
                Wp, Up = Tm @ Ub, Tm @ Vh
                D = Up - Wp @ S
                P = np.tril(Qb @ Wb.T, 0)
                o[b, c0:c1, h] = Qb @ S + P @ D
                gC = np.exp(g[-1])
                S = gC[:, None] * S + (Wb * gC).T @ D
            ST[b, h] = S
    return o, ST
