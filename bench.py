#!/usr/bin/env python3
"""Throughput of the gated delta-rule hot path on one MI355X.

One step = one gdr_chunk_fwd over the batch B=4, H=16, T=4096, dk=dv=128,
chunk 64 (bf16 q/k/v, fp32 scalar gates, zero initial state, o and the final
state written), inputs resident in HBM.  The same run times every other
configuration the library is specified on, each with its own roofline, under
"configs": the tiny fp32 GDN batch, the KDA / FG2-GDN+ batch (channel decay,
key and value beta vectors), the long-context OSDN batch (B=1, H=32, T=65536,
write key, nonzero S0), and the decode step (B=512, H=16, d=128, 256 steps
replayed as one HIP graph, and the r=8 delta-mem case).  Also reported: the
delta-mem context pass (segment and multi-state writes), the Memory-Caching
read-out, OSDN phase 1 and Sparse Delta Memory.

Prints ONE JSON line.  `value` is prefill tokens/s (B*T per step) of the headline
batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 matrix peak
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["gdr_api.hip", "chunk_mfma.hip", "chunk_valu.hip", "decode.hip", "mc_readout.hip", "osdn_precond.hip",
                  "sdm.hip", "dmem.hip", "gdr_ut.hpp", "gdr_device.hpp", "gdr_internal.hpp", "gdr_mfma.hpp"]


def prefill_flops_per_token_head(C, dk, dv):
    """Algorithmic flops of the chunked WY / UT form per token per head:
    Gram C*dk, UT inverse C^2/3, W' C*dk, U' C*dv, intra scores C*dk, P.Delta C*dv
    (triangular products at their nonzero half, 2 flops per MAC) plus the three
    dk x dv state products (W'S, QS, W^T Delta) at 2*dk*dv each."""
    return 3 * C * dk + 2 * C * dv + C * C / 3.0 + 6 * dk * dv


def prefill_bytes(w):
    """Every input read once, every output written once."""
    io = 2 if w.io == "bf16" else 4
    g = 2 if w.gate == "bf16" else 4
    ntok = w.B * w.T * w.H
    n = ntok * (2 * w.dk + w.dv) * io                    # q, k, v
    n += ntok * (w.dk if w.write_key else 0) * io        # k_w
    n += ntok * (w.dk if w.alpha_mode else 1) * g        # alpha
    n += ntok * (w.dk if w.beta_mode else 1) * g         # beta_k
    n += ntok * (w.dv if w.beta_mode == 2 else 0) * g    # beta_v
    n += ntok * w.dv * io                                # o
    st = w.B * w.H * w.dk * w.dv * 4
    n += st * (2 if w.s0_std > 0 else 1)                 # S0 (if any), ST
    return n


def decode_bytes_per_step(w):
    io = 2 if w.io == "bf16" else 4
    g = 2 if w.gate == "bf16" else 4
    nbh = w.B * w.H
    return nbh * (2 * w.dk * w.dv * 4 + (2 * w.dk + 2 * w.dv) * io + 2 * g)


def mc_readout_flops(w):
    """Algorithmic flops of the cache read-out: every token reads the caches of the
    segments before its own, 2 * dk * dv per (token, cache) (the split-precision
    second product is not counted)."""
    import numpy as np

    caches = np.minimum(np.arange(w.T) // w.seg, w.N).sum()
    return float(w.B * w.H * caches * 2 * w.dk * w.dv)


def kernel_source_digest():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_delta_rule_84_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(name, digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources."""
    path = os.path.join(PROFILE_DIR, f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_digest") != digest:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, x, budget_heads):
    """The fp64 oracle as it stands, on a bounded sample of the same batch:
    `budget_heads` (b, h) pairs over the full T."""
    import numpy as np

    import gdr_inputs as gi
    import oracle

    oracle.build(force=False)
    f = gi.prefill_f64(w, x)
    heads = list(range(min(budget_heads, w.B * w.H)))
    threads = min(len(heads), os.cpu_count() or 1, 16)
    t0 = time.perf_counter()
    oracle.forward(f["q"], f["k"], f["v"], f["alpha"], f["beta_k"], k_w=f["k_w"], beta_v=f["beta_v"], S0=f["S0"],
                   heads=heads, nthreads=threads)
    dt = time.perf_counter() - t0
    tokens = w.T * len(heads) / w.H  # tokens carry all H heads in the GPU metric
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(heads)} of {w.B * w.H} (batch, head) pairs x {w.T} tokens, fp64 sequential "
                      f"recurrence, OpenMP over pairs, {dt:.2f} s wall"}


def cpu_baseline_detail(gi):
    """The fp64 oracle on bounded samples of the other configurations (a few seconds
    each), and single-threaded on the headline batch: wall time and tokens/s."""
    import numpy as np

    import oracle

    oracle.build(force=False)
    cores = min(os.cpu_count() or 1, 16)
    out = {"cores_available": os.cpu_count(), "threads_cap": 16}

    def prefill(w, heads, threads, label):
        x = gi.make_prefill(w)
        f = gi.prefill_f64(w, x)
        hs = list(range(min(heads, w.B * w.H)))
        t0 = time.perf_counter()
        oracle.forward(f["q"], f["k"], f["v"], f["alpha"], f["beta_k"], k_w=f["k_w"], beta_v=f["beta_v"],
                       S0=f["S0"], heads=hs, nthreads=threads)
        dt = time.perf_counter() - t0
        return {"tokens_per_s": w.T * len(hs) / w.H / dt, "head_tokens_per_s": w.T * len(hs) / dt, "wall_s": dt,
                "threads": threads, "sample": f"{label}: {len(hs)} (batch, head) pairs x {w.T} tokens"}

    out[gi.TINY_GDN_F32.name] = prefill(gi.TINY_GDN_F32, 1, 1, "the whole workload")
    w2 = gi.GDN_PREFILL
    out[w2.name + "_single_thread"] = prefill(w2, 4, 1, "4 of 64 pairs, one thread")
    out[gi.KDA_FG2PLUS_PREFILL.name] = prefill(gi.KDA_FG2PLUS_PREFILL, 16, min(16, cores), "16 of 64 pairs")
    w4 = gi.OSDN_LONG_PREFILL.scaled(H=4)
    out[gi.OSDN_LONG_PREFILL.name] = prefill(w4, 4, min(4, cores), "4 of 32 heads (drawn as an H=4 batch)")
    for wd, label in ((gi.DECODE_B512.scaled(B=16), "16 of 512 batch rows x 16 heads"),
                      (gi.DECODE_DMEM_R8, "the whole workload")):
        x = gi.make_decode(wd)
        f = gi.decode_f64(wd, x)
        S = f["S"]
        t0 = time.perf_counter()
        for t in range(wd.steps):
            _, S = oracle.decode_step(S, f["q"][t], f["k"][t], f["v"][t], f["alpha"][t], f["beta_k"][t],
                                      nthreads=cores)
        dt = time.perf_counter() - t0
        name = gi.DECODE_B512.name if wd.B == 16 else wd.name
        out[name] = {"tokens_per_s": wd.B * wd.steps / dt, "us_per_step": dt / wd.steps * 1e6, "wall_s": dt,
                     "threads": cores, "sample": f"{label}, {wd.steps} steps"}
    return out


def copy_bandwidth(reps=5):
    """Attainable HBM bandwidth for context: a plain 1 GiB device-to-device copy,
    bytes read + written / time (median of `reps`)."""
    import torch

    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = sorted(ts)[len(ts) // 2]
    del a, b
    return {"bytes_per_copy": 2 << 30, "ms": ms, "GBps": (2 << 30) / (ms * 1e-3) / 1e9}


def bench_mc_readout(g, gi, stream, reps, digest=None):
    """The cache read-out of the long-context batch, inputs resident, events on the
    launch stream around each call (the small cache-preparation launch included)."""
    import torch

    w = gi.MC_LONG_GRM
    x = gi.make_cache_readout(w)
    q = gi.to_torch(x["q"], gi.BF16)
    ck = gi.to_torch(x["ckpt"], gi.F32)
    gates = gi.to_torch(x["gates"], gi.F32)
    o_in = gi.to_torch(x["o_in"], gi.BF16)
    out = torch.empty_like(o_in)
    desc = g.Desc(B=w.B, T=w.T, H=w.H, dk=w.dk, dv=w.dv, chunk=64, io_dtype=g.GDR_BF16, gate_dtype=g.GDR_F32,
                  alpha_mode=0, beta_mode=0, flags=0)
    need = g.gdr_mc_readout_workspace_size(desc, w.N)
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)

    def call():
        rc = g.gdr_mc_readout(desc, q, ck, w.N, w.seg, gates, o_in, out, ws, need, stream)
        if rc != g.GDR_OK:
            raise g.GdrError(rc, "gdr_mc_readout")

    call()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = sorted(times)[len(times) // 2]
    fl = mc_readout_flops(w)
    tf = fl / (ms * 1e-3) / 1e12
    return {"workload": w.name, "ms_per_call": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3),
            "algorithmic_flops": fl, "caches": w.N, "gates": w.gate_kind,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tf / BF16_MFMA_PEAK_TFLOPS, "traffic": load_traffic(w.name, digest)}}


def bench_osdn_precond(g, gi, stream, reps, digest=None, x=None):
    """OSDN phase 1 over the long-context batch's keys (B=1, H=32, T=65536, retention
    gates), inputs resident; events on the launch stream around each call (chunk
    solve + scan).  Algorithmic bytes: k read and k_w written (bf16), beta and r
    read (fp32), the preconditioner in and out."""
    import torch

    w = gi.OSDN_LONG_PREFILL
    if x is None:
        x = gi.make_prefill(w)
    k = gi.to_torch(x["k"], w.io)
    beta = gi.to_torch(x["beta_k"], w.gate)
    r = gi.to_torch(gi.make_retention(w), w.gate)
    desc = g.Desc(B=w.B, T=w.T, H=w.H, dk=w.dk, dv=w.dk, chunk=64, io_dtype=g.GDR_BF16, gate_dtype=g.GDR_F32,
                  alpha_mode=0, beta_mode=0, flags=0)
    need = g.gdr_osdn_precond_workspace_size(desc)
    ws = torch.empty(need, dtype=torch.uint8, device=k.device)
    kw = torch.empty_like(k)
    ctx = g.Context()  # the chunk solve and emission of later blocks overlap the scan on its stream
    dT = torch.empty((w.B, w.H, w.dk), dtype=torch.float32, device=k.device)
    qg = torch.empty((w.B, w.H), dtype=torch.float32, device=k.device)

    def call():
        rc = g.gdr_osdn_precond(desc, k, beta, r, 1.0, None, kw, dT, qg, ws, need, ctx, stream)
        if rc != g.GDR_OK:
            raise g.GdrError(rc, "gdr_osdn_precond")

    call()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = sorted(times)[len(times) // 2]
    ntok = w.B * w.T * w.H
    nbytes = ntok * (2 * w.dk * 2 + 2 * 4) + 2 * w.B * w.H * w.dk * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    name = "osdn_precond_bf16_B1H32T65536d128_retention"
    return {"workload": name, "ms_per_call": ms,
            "tokens_per_s": w.B * w.T / (ms * 1e-3), "algorithmic_bytes": nbytes, "qgeo_mean": float(qg.mean()),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": load_traffic(name, digest)}}


def sdm_bytes(w, gi):
    """Algorithmic HBM bytes of one Sparse Delta Memory call: per (token, head) the two
    half-score vectors of the key and of the query read (fp32), the selected slots and
    weights written then read back, W rows gathered and scattered and R rows gathered
    (fp32, dv values each), v read and o written, alpha and beta read."""
    es = 2 if w.io == gi.BF16 else 4
    per = (2 * 2 * w.n * 4 + 2 * (w.W + w.R) * 8 + (2 * w.W + w.R) * w.dv * 4 + 2 * w.dv * es + 2 * 4)
    return w.B * w.T * w.H * per


def bench_sdm(g, gi, stream, reps, digest=None):
    """Sparse Delta Memory at B=4 H=16 T=4096, 65,536 slots x 128 per head, W = R = 128,
    inputs and the 2 GiB of tables resident; events on the launch stream around each call
    (selection + table pass; the table evolves from call to call, the work does not)."""
    import torch

    w = gi.SDM_B4H16
    x = gi.make_sparse_memory(w)
    ks, qs = gi.to_torch(x["ks"], gi.F32), gi.to_torch(x["qs"], gi.F32)
    v = gi.to_torch(x["v"], w.io)
    alpha, beta = gi.to_torch(x["alpha"], w.gate), gi.to_torch(x["beta"], w.gate)
    M = gi.to_torch(x["M0"], gi.F32)
    del x
    o = torch.empty_like(v)
    desc = g.Desc(B=w.B, T=w.T, H=w.H, dk=w.dv, dv=w.dv, chunk=64, io_dtype=g.GDR_BF16, gate_dtype=g.GDR_F32,
                  alpha_mode=0, beta_mode=0, flags=0)
    need = g.gdr_sdm_workspace_size(desc, w.n, w.W, w.R)
    ws = torch.empty(need, dtype=torch.uint8, device=v.device)
    ctx = g.Context()  # the selection of later token blocks overlaps the table pass on its stream

    def call():
        rc = g.gdr_sdm_fwd(desc, w.n, w.W, w.R, ks, qs, v, alpha, beta, M, o, None, None, ws, need, ctx, stream)
        if rc != g.GDR_OK:
            raise g.GdrError(rc, "gdr_sdm_fwd")

    call()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = sorted(times)[len(times) // 2]
    nbytes = sdm_bytes(w, gi)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": w.name, "ms_per_call": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3),
            "algorithmic_bytes": nbytes,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": load_traffic(w.name, digest)}}


def progress(msg):
    """A progress line on stderr (stdout carries only the JSON line)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def time_prefill(g, gi, w, x, steps, warmup, stream, digest, cold=False, use_ctx=True):
    """`steps` gdr_chunk_fwd_ctx calls (gdr_chunk_fwd without `use_ctx`) back to back between one pair of HIP events on the
    launch stream after `warmup` untimed calls (an event pair around every call would
    add its own few microseconds per call); with `cold`, also the median of 5 calls
    after flushing L2 and the Infinity Cache.  Returns times and the roofline."""
    import torch

    dev = torch.device("cuda:0")
    d = {k: gi.to_torch(x[k], w.io if k in ("q", "k", "k_w", "v") else (w.gate if k != "S0" else gi.F32))
         for k in x}
    desc = g.make_desc(d["q"], d["v"], d["alpha"], d["beta_k"], d["beta_v"], chunk=w.chunk)
    path = g.gdr_chunk_fwd_path(desc)
    o = torch.empty((w.B, w.T, w.H, w.dv), dtype=d["q"].dtype, device=dev)
    ST = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    wsz = g.gdr_chunk_fwd_workspace_size(desc)
    ws = torch.empty(max(wsz, 1), dtype=torch.uint8, device=dev)
    # with few (batch, head) pairs and a long sequence the prep of later chunk blocks runs
    # on the context's stream beside the state recurrence; other shapes ignore it
    ctx = g.Context() if use_ctx else None

    def step():
        if ctx is None:
            rc = g.gdr_chunk_fwd(desc, d["q"], d["k"], d["k_w"], d["v"], d["alpha"], d["beta_k"], d["beta_v"],
                                 d["S0"], o, ST, ws, wsz, stream)
        else:
            rc = g.gdr_chunk_fwd_ctx(desc, d["q"], d["k"], d["k_w"], d["v"], d["alpha"], d["beta_k"],
                                     d["beta_v"], d["S0"], o, ST, ws, wsz, ctx, stream)
        if rc != g.GDR_OK:
            raise g.GdrError(rc, "gdr_chunk_fwd" if ctx is None else "gdr_chunk_fwd_ctx")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_event = e0.elapsed_time(e1) / steps
    res = {}
    if cold:
        flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
        times = []
        for _ in range(5):
            flush.fill_(1.0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        del flush
        res["ms_cold_median"] = sorted(times)[len(times) // 2]
    del d, o, ST, ws
    tokens = w.B * w.T
    flops = prefill_flops_per_token_head(w.chunk, w.dk, w.dv) * tokens * w.H
    nbytes = prefill_bytes(w)
    gbs = nbytes / (ms_event * 1e-3) / 1e9
    res.update({
        "ms_per_call": ms_event, "ms_wall": wall * 1e3 / steps, "tokens_per_s": tokens / (ms_event * 1e-3),
        "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": load_traffic(w.name, digest)},
        "mfma_frac": flops / (ms_event * 1e-3) / (BF16_MFMA_PEAK_TFLOPS * 1e12),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv, "chunk": w.chunk,
                   "io": w.io,
                   "gates": (w.gate + " " + ("channel" if w.alpha_mode else "scalar") + " alpha, "
                             + ["scalar", "shared-vector", "key/value-vector"][w.beta_mode] + " beta"
                             + (", write key" if w.write_key else "")),
                   "S0": "nonzero" if w.s0_std > 0 else "zero",
                   "kernel_path": {1: "bf16-mfma", 2: "fp32-valu"}[path]},
    })
    return res


def dmem_bytes(w):
    """Algorithmic HBM bytes of one delta-mem context pass: q, k, v and the two gates
    read per (token, head), the segment marks per token, the memories read and
    written, the group reads written."""
    es = 2 if w.io == "bf16" else 4
    gs = 2 if w.gate == "bf16" else 4
    ntok = w.B * w.T * w.H
    n = ntok * (3 * w.r * es + 2 * gs) + (w.B * w.T if w.seg_mean > 0 else 0)
    n += 2 * w.B * w.H * w.r * w.r * 4 + ntok // w.J * w.r * es
    return n


def bench_dmem(g, gi, stream, reps, digest=None):
    """The delta-mem context passes (8192 memories of 8 x 8, 256 tokens): segment writes
    (SSW) and four sub-states per group (MSW), inputs resident; events on the launch
    stream around each call (the memories evolve from call to call, the work does not)."""
    import numpy as np
    import torch

    res = {}
    for w in (gi.DMEM_SSW, gi.DMEM_MSW):
        x = gi.make_dmem_seq(w)
        q, k, v = (gi.to_torch(x[n], w.io) for n in ("q", "k", "v"))
        lam, beta = gi.to_torch(x["lam"], w.gate), gi.to_torch(x["beta"], w.gate)
        se = torch.from_numpy(np.ascontiguousarray(x["seg_end"])).cuda() if x["seg_end"] is not None else None
        M = gi.to_torch(x["M0"], gi.F32)
        o = torch.empty((w.B, w.T, w.H // w.J, w.r), dtype=q.dtype, device=q.device)
        desc = g.Desc(B=w.B, T=w.T, H=w.H, dk=w.r, dv=w.r, chunk=64, io_dtype=g._dtype_code(q),
                      gate_dtype=g._dtype_code(lam), alpha_mode=0, beta_mode=0, flags=0)

        def call():
            rc = g.gdr_dmem_fwd(desc, w.J, q, k, v, lam, beta, se, M, o, stream)
            if rc != g.GDR_OK:
                raise g.GdrError(rc, "gdr_dmem_fwd")

        call()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            call()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        ms = sorted(times)[len(times) // 2]
        nbytes = dmem_bytes(w)
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[w.name] = {"ms_per_call": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3), "algorithmic_bytes": nbytes,
                       "writes": "segment (SSW)" if w.seg_mean > 0 else f"token, {w.J} sub-states (MSW)",
                       "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": gbs / HBM_PEAK_GBS, "traffic": load_traffic(w.name, digest)}}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the card's clocks settle only after a few tens of calls (≈ 245 µs per headline call
    # right after a handful, ≈ 215 µs once settled), so the default warms up for 50
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--decode-reps", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-heads", type=int, default=64)
    ap.add_argument("--only-prefill", action="store_true")
    ap.add_argument("--mc-reps", type=int, default=5, help="timed Memory-Caching read-out calls")
    ap.add_argument("--workload", choices=["gdn", "kda_fg2plus", "osdn_long"], default="gdn",
                    help="prefill workload (default: the B4 H16 T4096 GDN batch the metric is quoted on)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy 3 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(sequences shard over (batch, head) with no communication).", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_84_amd as g
    import gdr_inputs as gi
    from gated_delta_rule_84_amd.graph import DecodeGraph

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = 1 << 28  # 2^28 fp32 = 1 GiB read + 1 GiB written per copy
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 3}))
        return
    wl = {"gdn": gi.GDN_PREFILL, "kda_fg2plus": gi.KDA_FG2PLUS_PREFILL, "osdn_long": gi.OSDN_LONG_PREFILL}
    w = wl[args.workload]
    digest = kernel_source_digest()
    stream = torch.cuda.current_stream()
    inputs = {w.name: gi.make_prefill(w)}
    x = inputs[w.name]
    head = time_prefill(g, gi, w, x, args.steps, args.warmup, stream, digest, cold=True)
    progress(f"prefill {w.name}: {head['ms_per_call']:.4f} ms per call")
    ms_step = head["ms_wall"]
    tokens = w.B * w.T
    out = {
        "metric": "tokens/s gated-delta chunk fwd (H=16,d=128,T=4096); % MFMA peak; decode GB/s",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": dict(head["config"], global_batch=w.B, seq_len=w.T, parallelism="single GPU"),
        "roofline": head["roofline"],
        "mfma_frac": head["mfma_frac"],
        "prefill_detail": {"ms_event_mean": head["ms_per_call"], "ms_cold_median": head["ms_cold_median"],
                           "algorithmic_bytes": head["algorithmic_bytes"], "algorithmic_flops": head["algorithmic_flops"],
                           "gbs_cold": head["algorithmic_bytes"] / (head["ms_cold_median"] * 1e-3) / 1e9,
                           "kernel_source_digest": digest},
    }
    if not args.only_prefill:
        # every other prefill configuration, timed the same way (fewer calls)
        cfgs = {}
        for wc, steps in ((gi.TINY_GDN_F32, 200), (gi.GDN_PREFILL, 20), (gi.KDA_FG2PLUS_PREFILL, 20),
                          (gi.OSDN_LONG_PREFILL, 5)):
            if wc.name == w.name:
                cfgs[wc.name] = {k: head[k] for k in ("ms_per_call", "tokens_per_s", "roofline", "mfma_frac",
                                                      "config")}
                continue
            if wc.name not in inputs:
                inputs[wc.name] = gi.make_prefill(wc)
            r = time_prefill(g, gi, wc, inputs[wc.name], steps, max(steps // 2, 3), stream, digest)
            progress(f"prefill {wc.name}: {r['ms_per_call']:.4f} ms per call")
            cfgs[wc.name] = {k: r[k] for k in ("ms_per_call", "tokens_per_s", "roofline", "mfma_frac", "config")}
        out["configs"] = cfgs

    if not args.only_prefill:
        dec = {}
        for wd in (gi.DECODE_B512.scaled(steps=args.decode_steps), gi.DECODE_DMEM_R8.scaled(steps=args.decode_steps)):
            xd = gi.make_decode(wd)
            dd = {k: gi.to_torch(xd[k], wd.io if k in ("q", "k", "k_w", "v") else (wd.gate if k != "S" else gi.F32))
                  for k in xd}
            S = dd["S"].clone()
            # the delta-mem workload runs delta-mem's own step (read before the write,
            # prediction from the undecayed state)
            fl = (g.GDR_FLAG_READ_BEFORE_WRITE | g.GDR_FLAG_UNDECAYED_PREDICTION) if wd.dk == 8 else 0
            graph = DecodeGraph(S, dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta_k"], k_w=dd["k_w"],
                                beta_v=dd["beta_v"], flags=fl)
            graph.replay()
            torch.cuda.synchronize()
            times = []
            for _ in range(args.decode_reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                graph.replay()
                b.record(stream)
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b))
            ms = sorted(times)[len(times) // 2]
            us_step = ms * 1e3 / wd.steps
            bps = decode_bytes_per_step(wd)
            gbs = bps / (us_step * 1e-6) / 1e9
            dec[wd.name] = {"us_per_step": us_step, "flags": fl, "tokens_per_s": wd.B / (us_step * 1e-6),
                            "GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS, "steps_per_graph": wd.steps,
                            "bytes_per_step": bps,
                            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                         "frac": gbs / HBM_PEAK_GBS, "traffic": load_traffic(wd.name, digest)}}
            del graph, dd, S
        out["decode"] = dec
        out["configs"].update(dec)  # the decode configuration (and its delta-mem case) in the same table
        progress("decode done")
        out["mc_readout"] = bench_mc_readout(g, gi, stream, args.mc_reps, digest)
        progress("mc_readout done")
        out["dmem_pass"] = bench_dmem(g, gi, stream, args.mc_reps, digest)
        progress("delta-mem passes done")
        out["osdn_precond"] = bench_osdn_precond(g, gi, stream, args.mc_reps, digest,
                                                 inputs.get(gi.OSDN_LONG_PREFILL.name))
        progress("osdn_precond done")
        out["sdm"] = bench_sdm(g, gi, stream, args.mc_reps, digest)
        progress("sdm done")
        out["copy_bandwidth"] = copy_bandwidth()
        progress("copy_bandwidth done")

    if not args.no_cpu:
        progress("CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(w, x, args.cpu_heads)
        if not args.only_prefill:
            out["cpu_baseline_detail"] = cpu_baseline_detail(gi)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
