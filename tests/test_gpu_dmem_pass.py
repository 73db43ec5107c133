"""delta-mem context pass on the GPU (gdr_dmem_fwd) against the fp64 oracle
(oracle/dmem.py): token-state, sequence-state and multi-state writes [delta-mem page,
sections 2.A, 2.C, 2.D].  Reads are compared element by element to rel-L2 <= 2e-3
(bf16 I/O) or <= 1e-5 (fp32 I/O); the final memories to 1e-5 (fp32 arithmetic on
exact inputs).  Small cases run whole; the full 8192-memory batches are checked on
sampled batch rows."""
import numpy as np
import pytest

import gdr_inputs as gi
import oracle
from oracle import dmem
from tests.gpu_util import TOL, gpu, log, to_np

pytestmark = pytest.mark.gpu


def _run_gpu(w, x, seg=True):
    torch, g = gpu()
    q, k, v = (gi.to_torch(x[n], w.io) for n in ("q", "k", "v"))
    lam, beta = gi.to_torch(x["lam"], w.gate), gi.to_torch(x["beta"], w.gate)
    se = None
    if seg and x["seg_end"] is not None:
        se = torch.from_numpy(np.ascontiguousarray(x["seg_end"])).cuda()
    M = gi.to_torch(x["M0"], gi.F32)
    out = g.dmem_fwd(M, q, k, v, lam, beta, seg_end=se, J=w.J)
    torch.cuda.synchronize()
    return to_np(out), to_np(M)


def _check(w, x, rows=None, seg=True):
    out_g, M_g = _run_gpu(w, x, seg)
    f = gi.dmem_seq_f64(w, x)
    sel = slice(None) if rows is None else rows
    se = f["seg_end"][sel] if (seg and f["seg_end"] is not None) else None
    out_r, M_r = dmem.forward(f["M0"][sel], f["q"][sel], f["k"][sel], f["v"][sel], f["lam"][sel], f["beta"][sel],
                              seg_end=se, J=w.J)
    eo, em = oracle.rel_l2(out_g[sel], out_r), oracle.rel_l2(M_g[sel], M_r)
    log(f"[dmem] {w.name} B={w.B} T={w.T} H={w.H} J={w.J} r={w.r} seg={se is not None} "
        f"rows={'all' if rows is None else len(rows)}: rel-L2 out={eo:.3e} M={em:.3e}")
    assert np.isfinite(out_g).all() and np.isfinite(M_g).all()
    assert eo <= TOL[w.io] and em <= 1e-5, (eo, em)
    return out_g, M_g


BASE = gi.DMEM_SSW.scaled(name="dmem_small", B=13, T=45, H=1, seg_mean=6.0, m_std=0.3, lam_mu=-2.0, seed=601)
CASES = [
    ("tsw_bf16", BASE.scaled(seg_mean=0.0)),
    ("ssw_bf16", BASE),
    ("ssw_bf16_long_segments", BASE.scaled(seg_mean=40.0, seed=602)),
    ("ssw_f32", BASE.scaled(io=gi.F32, gate=gi.F32, seed=603)),
    ("tsw_f32_gates_bf16", BASE.scaled(io=gi.F32, seg_mean=0.0, seed=604)),
    ("msw_J2", BASE.scaled(H=4, J=2, seg_mean=0.0, seed=605)),
    ("msw_J4_ssw", BASE.scaled(H=8, J=4, seed=606)),
    ("msw_J8", BASE.scaled(B=5, H=8, J=8, seg_mean=0.0, seed=607)),
    ("msw_J8_f32", BASE.scaled(B=5, H=16, J=8, io=gi.F32, gate=gi.F32, seg_mean=3.0, seed=608)),
    ("r16_tsw", BASE.scaled(r=16, seg_mean=0.0, seed=609)),
    ("r16_msw_J4_ssw", BASE.scaled(r=16, H=8, J=4, seed=610)),
    ("r16_f32_J2", BASE.scaled(r=16, H=2, J=2, io=gi.F32, gate=gi.F32, seed=611)),
    ("one_token", BASE.scaled(T=1, seed=612)),
    ("ragged_block_T6", BASE.scaled(B=3, T=6, H=2, seed=613)),
    # tensors under 4 bytes (one bf16 gate, three segment marks) and a gate tensor
    # whose size is not a multiple of 4 bytes (its last element in a half word)
    ("one_memory_one_token", BASE.scaled(B=1, T=1, H=1, seed=614)),
    ("one_memory_three_tokens", BASE.scaled(B=1, T=3, H=1, seed=615)),
    ("odd_gate_count_r16", BASE.scaled(B=7, T=33, H=1, r=16, seed=616)),
]


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_dmem_pass_parity(name, w):
    x = gi.make_dmem_seq(w)
    _check(w, x)


def test_every_token_marked_equals_token_writes():
    """SSW with every token marked is TSW, bit for bit (a mean over one token is the
    token itself)."""
    w = BASE.scaled(seg_mean=0.0, seed=620)
    x = gi.make_dmem_seq(w)
    a = _run_gpu(w, x)
    x2 = dict(x, seg_end=np.ones((w.B, w.T), dtype=np.uint8))
    b = _run_gpu(w, x2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_unmarked_sequence_is_one_segment():
    """No marks at all: one segment closed by the last token, so every read is M0 q_t."""
    w = BASE.scaled(seed=621)
    x = gi.make_dmem_seq(w)
    x["seg_end"] = np.zeros((w.B, w.T), dtype=np.uint8)
    out, _ = _check(w, x)
    f = gi.dmem_seq_f64(w, x)
    want = np.einsum("bhac,bthc->btha", f["M0"], f["q"])
    assert oracle.rel_l2(out, want) <= TOL[w.io]


@pytest.mark.parametrize("w", [gi.DMEM_SSW, gi.DMEM_MSW], ids=["ssw_B8192", "msw_B2048_J4"])
def test_full_batch_sampled_rows(w):
    x = gi.make_dmem_seq(w)
    rows = np.unique(np.concatenate([np.arange(4), np.linspace(0, w.B - 1, 20).astype(int), [w.B - 1]]))
    _check(w, x, rows=rows)
