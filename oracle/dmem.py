"""delta-mem write granularities in fp64 -- TEST INFRASTRUCTURE (same rules as the rest of oracle/).

delta-mem: Efficient Online Memory for Large Language Models, section 2.A (update
rule) and section 2.C (read): the online memory M (r x r) of one head predicts a
value from a key as M k.  Per write with key k, value v, forget gate lambda and
write gate beta,
    M <- lambda M + beta (v - M k) k^T          (the prediction uses M before the gate)
and the read of token t is M q_t, taken from the memory before token t's write.
Section 2.D names three write granularities:
  * token-state write (TSW): one write per token;
  * sequence-state write (SSW): the hidden states of a message / segment are
    averaged before the memory is updated -- here one write per segment whose key
    and value are the means of the segment's keys and values;
  * multi-state write (MSW): several parallel sub-states, each written on its own,
    whose reads are aggregated -- here J consecutive heads form a group and the
    group's read is the sum of its J sub-state reads.

Readings (the page leaves them open):
  * the segment mean is taken over the keys and values as given (already projected;
    the mean is not renormalised), which is the projection of the mean hidden state
    for a linear projection;
  * a segment's write uses the gates stored at the segment's last token (the gates of
    the segment's other tokens are not used);
  * every token of a segment reads the memory as it was before the segment's write
    (with one-token segments this is the page's read-before-write, M_{t-1} q_t);
  * the last token of the sequence always closes a segment;
  * the reads of a group's sub-states are summed (not averaged).

Shapes: M0 [B, H, r, r] (row a predicts value component a); q, k, v [B, T, H, r];
lam, beta [B, T, H]; seg_end [B, T] (true where a segment ends; None: every token
ends one, TSW); H = G J.  Returns (out [B, T, G, r], M [B, H, r, r]).
"""
from __future__ import annotations

import numpy as np


def write(M, k, v, lam, beta):
    """One delta-mem write (section 2.A): lambda M + beta (v - M k) k^T."""
    return lam * M + beta * np.outer(v - M @ k, k)


def forward(M0, q, k, v, lam, beta, seg_end=None, J: int = 1):
    M0, q, k, v, lam, beta = (np.asarray(a, dtype=np.float64) for a in (M0, q, k, v, lam, beta))
    B, T, H, r = q.shape
    if H % J:
        raise ValueError("H must be a multiple of J")
    M = M0.copy()
    reads = np.zeros((B, T, H, r))
    for b in range(B):
        for h in range(H):
            Mh = M[b, h]
            ks = np.zeros(r)
            vs = np.zeros(r)
            n = 0
            for t in range(T):
                reads[b, t, h] = Mh @ q[b, t, h]          # before this token's segment is written
                ks += k[b, t, h]
                vs += v[b, t, h]
                n += 1
                closes = seg_end is None or bool(seg_end[b][t]) or t == T - 1
                if closes:
                    kb = ks / n
                    vb = vs / n
                    Mh = write(Mh, kb, vb, lam[b, t, h], beta[b, t, h])
                    ks = np.zeros(r)
                    vs = np.zeros(r)
                    n = 0
            M[b, h] = Mh
    out = reads.reshape(B, T, H // J, J, r).sum(axis=3)
    return out, M
