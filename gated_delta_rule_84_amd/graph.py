"""Replay of many decode steps as one HIP graph.

A decode step is one short kernel launch; a long run of them is bound by launch
overhead unless the launches are captured once and replayed.  ``DecodeGraph``
captures ``steps`` consecutive ``gdr_decode_step`` calls (each reading its own
slice of the per-step inputs and updating the resident state in place) on a
side stream and replays them with a single graph launch.
"""
from __future__ import annotations

import torch

from . import GDR_OK, GdrError, gdr_decode_step, make_desc


class DecodeGraph:
    """Per-step tensors carry a leading step axis: q, k [steps, B, H, dk], ..."""

    def __init__(self, S, q, k, v, alpha, beta_k, *, k_w=None, beta_v=None, out=None, flags=0):
        self.steps = q.shape[0]
        self.S = S
        self.out = out if out is not None else torch.empty(
            (self.steps,) + q.shape[1:-1] + (v.shape[-1],), dtype=q.dtype, device=q.device)
        desc = make_desc(q[0], v[0], alpha[0], beta_k[0], None if beta_v is None else beta_v[0], decode=True,
                         flags=flags)
        self.graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        sel = lambda t, i: None if t is None else t[i]
        with torch.cuda.stream(side):
            with torch.cuda.graph(self.graph, stream=side):
                for i in range(self.steps):
                    rc = gdr_decode_step(desc, q[i], k[i], sel(k_w, i), v[i], alpha[i], beta_k[i],
                                         sel(beta_v, i), S, self.out[i], torch.cuda.current_stream())
                    if rc != GDR_OK:
                        raise GdrError(rc, "gdr_decode_step (graph capture)")
        torch.cuda.current_stream().wait_stream(side)

    def replay(self):
        self.graph.replay()
        return self.out
