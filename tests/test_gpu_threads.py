"""Calls from several host threads at once.  The library holds no shared state: the
calls that overlap work on a second stream (long OSDN phase 1, long Sparse Delta
Memory) take it from a caller-owned execution context, one per thread here, and the
prefill forks nothing.  Threads each issue their own call on their own stream, at
the same time and several times over; every result must equal, bit for bit, the
same call made alone."""
import threading

import pytest

import gdr_inputs as gi
from tests.gpu_util import gpu, log, upload

pytestmark = pytest.mark.gpu


def _run_threads(torch, calls, reps=3):
    """calls: list of functions f(stream) -> tuple of tensors.  Runs each in its own
    host thread and stream, all started together, `reps` times."""
    streams = [torch.cuda.Stream() for _ in calls]
    outs = [None] * len(calls)
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(reps):
                    outs[i] = calls[i](streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported in the main thread
            errors.append(e)

    torch.cuda.synchronize()
    th = [threading.Thread(target=worker, args=(i,)) for i in range(len(calls))]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    return outs


def test_concurrent_side_stream_calls_equal_solo_calls():
    torch, g = gpu()
    wo = gi.OSDN_LONG_PREFILL.scaled(B=1, T=16500, H=2, seed=131)
    xo = gi.make_prefill(wo)
    k, beta = gi.to_torch(xo["k"], wo.io), gi.to_torch(xo["beta_k"], wo.gate)
    r = gi.to_torch(gi.make_retention(wo), wo.gate)
    wp = gi.OSDN_LONG_PREFILL.scaled(B=1, T=16500, H=2, seed=132)
    dp = upload(gi.make_prefill(wp), wp)
    ws = gi.SDM_B4H16.scaled(B=1, T=1100, H=2, n=32, W=8, R=8, seed=133)
    xs = gi.make_sparse_memory(ws)
    ks, qs = gi.to_torch(xs["ks"], gi.F32), gi.to_torch(xs["qs"], gi.F32)
    v, a, b = gi.to_torch(xs["v"], ws.io), gi.to_torch(xs["alpha"], ws.gate), gi.to_torch(xs["beta"], ws.gate)
    M0 = gi.to_torch(xs["M0"], gi.F32)

    def osdn(stream, ctx=None):
        return g.osdn_precond(k, beta, 0.5, r=r, ctx=ctx, stream=stream)

    def prefill(stream, ctx=None):
        return g.chunk_fwd(dp["q"], dp["k"], dp["v"], dp["alpha"], dp["beta_k"], k_w=dp["k_w"], S0=dp["S0"],
                           stream=stream)

    def sdm(stream, ctx=None):
        M = M0.clone()  # on the calling thread's stream
        o = g.sdm_fwd(M, ks, qs, v, a, b, ws.W, ws.R, ctx=ctx, stream=stream)
        return (o, M)

    wd = gi.DMEM_SSW.scaled(B=512, T=200, H=1, seed=134)
    xd = gi.make_dmem_seq(wd)
    dq, dkk, dv = (gi.to_torch(xd[n], wd.io) for n in ("q", "k", "v"))
    dl, db = gi.to_torch(xd["lam"], wd.gate), gi.to_torch(xd["beta"], wd.gate)
    dse = torch.from_numpy(xd["seg_end"]).cuda()
    dM0 = gi.to_torch(xd["M0"], gi.F32)

    def dmem(stream, ctx=None):
        M = dM0.clone()
        o = g.dmem_fwd(M, dq, dkk, dv, dl, db, seg_end=dse, stream=stream)
        return (o, M)

    solo = [osdn(None), prefill(None), sdm(None), dmem(None)]
    torch.cuda.synchronize()
    for name, pair in (("osdn + prefill", [osdn, prefill]), ("osdn + osdn", [osdn, osdn]),
                       ("sdm + prefill", [sdm, prefill]), ("all three", [osdn, prefill, sdm]),
                       ("dmem + prefill + sdm", [dmem, prefill, sdm])):
        ctxs = [g.Context() for _ in pair]
        outs = _run_threads(torch, [lambda st, f=f, c=c: f(st, c) for f, c in zip(pair, ctxs)])
        for c in ctxs:
            c.close()
        ref = {osdn: solo[0], prefill: solo[1], sdm: solo[2], dmem: solo[3]}
        same = [all(torch.equal(x, y) for x, y in zip(out, ref[f])) for f, out in zip(pair, outs)]
        log(f"[threads] {name}: equal to the solo calls {same}")
        assert all(same)
