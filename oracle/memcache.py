"""Memory Caching in fp64 -- TEST INFRASTRUCTURE (same rules as the rest of oracle/).

Memory Caching: RNNs with Growing Memory, section 2: the sequence is cut into
segments, the memory is updated online inside each segment, and the memory state
at the end of every segment is stored in a cache.  A token of a later segment
retrieves from the cached states as well as from the online state.  Section 3
names the aggregations: residual memory (the cached read-outs are added), gated
residual memory (each cached read-out is weighted by a context-dependent gate),
memory soup (the cached memories are mixed with the same weights first -- for a
linear memory this is the same number, which one of the pins checks), and sparse
selective caching (a router keeps only a few caches per token, i.e. the other
gates are zero).

Everything here is plain: segment states come from the sequential oracle run one
segment at a time, each starting from the state the previous one ended with (the
recurrence itself does not change at a segment end); the read-out is the sum over
the earlier segments' states of gate * M^T q, one matrix product per (segment,
cache) pair.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import forward


def segment_states(q, k, v, alpha, beta_k, seg_len: int, *, k_w=None, beta_v=None, S0=None,
                   nthreads: int = 0):
    """Sequential fp64 prefill that also returns the state after every complete segment.

    Returns (o [B, T, H, dv], ST [B, H, dk, dv], ckpt [B, H, N, dk, dv]) with
    N = T // seg_len and ckpt[:, :, s] the state after token (s + 1) * seg_len - 1.
    """
    q = np.asarray(q)
    B, T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    n = T // seg_len
    S = None if S0 is None else np.asarray(S0, dtype=np.float64)
    o = np.empty((B, T, H, dv))
    ckpt = np.empty((B, H, n, dk, dv))
    sl = lambda a, t0, t1: None if a is None else np.asarray(a)[:, t0:t1]
    bounds = [(s * seg_len, (s + 1) * seg_len) for s in range(n)]
    if n * seg_len < T:
        bounds.append((n * seg_len, T))
    if not bounds:
        bounds = [(0, T)]
    for i, (t0, t1) in enumerate(bounds):
        o_s, S = forward(sl(q, t0, t1), sl(k, t0, t1), sl(v, t0, t1), sl(alpha, t0, t1), sl(beta_k, t0, t1),
                         k_w=sl(k_w, t0, t1), beta_v=sl(beta_v, t0, t1), S0=S, nthreads=nthreads)
        o[:, t0:t1] = o_s
        if i < n:
            ckpt[:, :, i] = S
    return o, S, ckpt


def readout(q, ckpt, seg_len: int, gates=None, o_in=None, heads=None, tokens=None):
    """o_out[t] = o_in[t] + sum_{s < min(t // seg_len, N)} g[t, s] * M_s^T q[t], in fp64.

    q [B, T, H, dk]; ckpt [B, H, N, dk, dv]; gates [B, T, H, N] or None (all ones:
    residual memory); o_in [B, T, H, dv] or None.  ``heads`` (list of b * H + h) and
    ``tokens`` (list of t) restrict the evaluation to those entries; the result then
    has shape [len(heads), len(tokens), dv].
    """
    q = np.asarray(q, dtype=np.float64)
    ckpt = np.asarray(ckpt, dtype=np.float64)
    B, T, H, dk = q.shape
    N, dv = ckpt.shape[2], ckpt.shape[-1]
    g = None if gates is None else np.asarray(gates, dtype=np.float64)
    oi = None if o_in is None else np.asarray(o_in, dtype=np.float64)
    hl = list(range(B * H)) if heads is None else list(heads)
    tl = np.arange(T) if tokens is None else np.asarray(tokens)
    out = np.zeros((len(hl), len(tl), dv))
    for a, bh in enumerate(hl):
        b, h = divmod(bh, H)
        for s in range(N):
            # tokens whose own segment starts after cache s ends
            sel = np.nonzero(np.minimum(tl // seg_len, N) > s)[0]
            if sel.size == 0:
                continue
            r = q[b, tl[sel], h] @ ckpt[b, h, s]          # [n, dv] = (M_s^T q_t)^T
            w = np.ones(sel.size) if g is None else g[b, tl[sel], h, s]
            out[a, sel] += w[:, None] * r
        if oi is not None:
            out[a] += oi[b, tl, h]
    if heads is None and tokens is None:
        return out.reshape(B, H, T, dv).transpose(0, 2, 1, 3).copy()
    return out
