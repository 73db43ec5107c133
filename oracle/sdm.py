"""Sparse Delta Memory in fp64 -- TEST INFRASTRUCTURE (same rules as the rest of oracle/).

Resumo Técnico: Sparse Delta Memory (SDM), Mecanismo Central items 1-4: the memory of
one (batch, head) is an explicit table M of N slots x dv.  At every token the
projected key and query are each split in two halves; the score of slot
i = a * n + b (N = n * n) is the sum of half-score a of the first half and
half-score b of the second.  The W best-scoring slots by the key are written with
the gated delta update
    M~[i] = alpha_t M[i],    M[i] = M~[i] + beta_t k_t^(i) (v_t - M~[i]),
the others stay as they are, and the read-out is the weighted sum of the R
best-scoring slots by the query.

Readings (the page leaves them open): the slot weights k_t^(i) and the read
weights are the softmax of the selected scores; the read comes after the write
(as for the dense gated delta rule); scores are formed and ranked in fp32 (the
selection is an integer decision, taken in the GPU's precision), highest first,
equal scores by lower slot index.  Everything else is fp64.

This oracle ranks all N slot scores directly (no product-key shortcut); the GPU
path uses topk(s1 (+) s2) = topk(topk(s1) (+) topk(s2)) [same page, item 2].
"""
from __future__ import annotations

import numpy as np


def select(s1, s2, k: int):
    """Top-k slots of the outer sum of two half-score vectors (fp32 sums), by the
    full ranking of all n * n slots.  Returns (slot indices, fp32 scores), best first."""
    s1 = np.asarray(s1, dtype=np.float32)
    s2 = np.asarray(s2, dtype=np.float32)
    n = s1.size
    full = (s1[:, None] + s2[None, :]).reshape(-1)          # fp32 sums, slot i = a * n + b
    order = np.lexsort((np.arange(n * n), -full.astype(np.float64)))
    top = order[:k]
    return top, full[top]


def softmax(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def forward(M, ks, qs, v, alpha, beta, W: int, R: int):
    """Sequential fp64 SDM over T tokens for every (b, h).

    M  [B, H, N, dv] initial tables (the learned M_0), not modified
    ks, qs [B, T, H, 2, n] half scores of the key and the query
    v [B, T, H, dv]; alpha, beta [B, T, H]
    Returns (o [B, T, H, dv], M_T [B, H, N, dv], write slots [B, T, H, W], read slots [B, T, H, R]).
    """
    M = np.array(M, dtype=np.float64, copy=True)
    ks, qs = np.asarray(ks), np.asarray(qs)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, _, n = ks.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    wsl = np.zeros((B, T, H, W), dtype=np.int64)
    rsl = np.zeros((B, T, H, R), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            Mh = M[b, h]
            for t in range(T):
                slots, sc = select(ks[b, t, h, 0], ks[b, t, h, 1], W)
                wk = softmax(sc)
                a, be = float(alpha[b, t, h]), float(beta[b, t, h])
                for i, w in zip(slots, wk):
                    mt = a * Mh[i]                                  # forget gate on the slot
                    Mh[i] = mt + be * w * (v[b, t, h] - mt)         # delta update toward v
                rs, rsc = select(qs[b, t, h, 0], qs[b, t, h, 1], R)
                o[b, t, h] = softmax(rsc) @ Mh[rs]
                wsl[b, t, h] = slots
                rsl[b, t, h] = rs
    return o, M, wsl, rsl
