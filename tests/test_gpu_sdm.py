"""GPU parity of the Sparse Delta Memory entry point (gdr_sdm_fwd) through the C-ABI,
against oracle/sdm.py (full fp32 ranking of all n * n slot scores, fp64 table).

The selected slots are integer results decided in fp32 on both sides: they must
match bit for bit, best first.  The table is fp32 on the GPU: the final table
within 1e-5 rel-L2 of the fp64 oracle; the read-out within the io precision's
bound (2e-3 bf16: one rounding of the result; 1e-5 fp32).
"""
import dataclasses

import numpy as np
import pytest

import gdr_inputs as gi
from oracle import rel_l2, sdm
from tests.gpu_util import TOL, gpu, log, to_np

pytestmark = pytest.mark.gpu


def _upload(w, x):
    return dict(ks=gi.to_torch(x["ks"], gi.F32), qs=gi.to_torch(x["qs"], gi.F32), v=gi.to_torch(x["v"], w.io),
                alpha=gi.to_torch(x["alpha"], w.gate), beta=gi.to_torch(x["beta"], w.gate),
                M=gi.to_torch(x["M0"], gi.F32))


def _run(w, x, ctx=None):
    torch, g = gpu()
    d = _upload(w, x)
    o, wsl, rsl = g.sdm_fwd(d["M"], d["ks"], d["qs"], d["v"], d["alpha"], d["beta"], w.W, w.R, want_slots=True,
                            ctx=ctx)
    torch.cuda.synchronize()
    return o, d["M"], wsl, rsl


def _ref(w, x, b=slice(None), t=slice(None), h=slice(None)):
    v = gi.as_f64(x["v"], w.io)
    a = gi.as_f64(x["alpha"], w.gate)
    be = gi.as_f64(x["beta"], w.gate)
    return sdm.forward(x["M0"][b, h], x["ks"][b, t, h], x["qs"][b, t, h], v[b, t, h], a[b, t, h], be[b, t, h],
                       w.W, w.R)


BASE = gi.SDM_B4H16.scaled(B=2, T=24, H=3, n=16, W=8, R=5, seed=91)
CASES = [
    ("small_bf16", BASE),
    ("small_f32", BASE.scaled(io=gi.F32, seed=92)),
    ("bf16_gates", BASE.scaled(gate=gi.BF16, seed=93)),
    ("write_all_slots", BASE.scaled(n=4, W=16, R=16, T=12, seed=94)),
    ("one_slot", BASE.scaled(n=1, W=1, R=1, T=9, seed=95)),
    ("n_not_multiple_of_64", BASE.scaled(n=100, W=37, R=64, T=16, H=2, seed=96)),
    ("headline_widths_n256", BASE.scaled(B=1, H=2, T=20, n=256, W=128, R=128, seed=97)),
    ("n1024_np16", BASE.scaled(B=1, H=1, T=6, n=1024, W=128, R=100, seed=98)),
    ("widths_over_64", BASE.scaled(B=1, H=2, T=10, n=128, W=65, R=127, seed=99)),
    # T >= 1024 with an execution context: selection and table pass in eight token
    # blocks on two streams
    ("token_blocks_T1100", BASE.scaled(B=2, H=2, T=1100, n=16, W=6, R=5, seed=100)),
]


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_sdm_parity(name, w):
    x = gi.make_sparse_memory(w)
    log(f"[sdm] {name}: B={w.B} T={w.T} H={w.H} n={w.n} W={w.W} R={w.R} io={w.io} gate={w.gate}")
    torch, g = gpu()
    blocks = name.startswith("token_blocks")
    o, M, wsl, rsl = _run(w, x, ctx=g.Context() if blocks else None)
    if blocks:
        o1, M1, wsl1, rsl1 = _run(w, x)
        same = torch.equal(o, o1) and torch.equal(M, M1) and torch.equal(wsl, wsl1) and torch.equal(rsl, rsl1)
        log(f"          two streams equal to one stream: {same}")
        assert same
    o_ref, M_ref, wsl_ref, rsl_ref = _ref(w, x)
    assert np.array_equal(wsl.cpu().numpy(), wsl_ref), "write slots differ"
    assert np.array_equal(rsl.cpu().numpy(), rsl_ref), "read slots differ"
    eo, em = rel_l2(to_np(o), o_ref), rel_l2(to_np(M), M_ref)
    log(f"          rel-L2 o={eo:.3e} M_T={em:.3e}")
    assert eo <= TOL[w.io] and em <= 1e-5


def _tie_case(seed, n, W, R, T=8, B=1, H=2, kind="int"):
    """Scores with many exact ties: small integers (exact fp32 sums), or values whose
    fp32 sums collide by rounding."""
    w = BASE.scaled(B=B, T=T, H=H, n=n, W=W, R=R, seed=seed)
    x = gi.make_sparse_memory(w)
    rng = np.random.default_rng(seed + 1)
    shape = x["ks"].shape
    if kind == "int":
        x["ks"] = rng.integers(-2, 3, shape).astype(np.float32)
        x["qs"] = rng.integers(-1, 2, shape).astype(np.float32)
    elif kind == "rounding":
        # first half 1 + j 2^-23, second half 3 + {0, 1, 2}: the 2^-23 steps vanish in the sums
        for key in ("ks", "qs"):
            s = np.empty(shape, np.float32)
            s[..., 0, :] = 1.0 + rng.integers(0, 4, shape[:-2] + (n,)) * 2.0 ** -23
            s[..., 1, :] = 3.0 + rng.integers(0, 3, shape[:-2] + (n,))
            x[key] = s
    elif kind == "zeros":
        x["ks"] = np.zeros(shape, np.float32)
        x["qs"] = np.where(rng.random(shape) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    return w, x


TIE_CASES = [
    ("int_scores", dict(seed=101, n=16, W=7, R=11)),
    ("int_scores_n100", dict(seed=102, n=100, W=64, R=128)),
    ("rounding_collisions", dict(seed=103, n=12, W=9, R=30, kind="rounding")),
    ("all_equal_and_signed_zeros", dict(seed=104, n=20, W=13, R=50, kind="zeros")),
]


@pytest.mark.parametrize("name,kw", TIE_CASES, ids=[c[0] for c in TIE_CASES])
def test_sdm_ties(name, kw):
    w, x = _tie_case(**kw)
    log(f"[sdm] ties {name}: n={w.n} W={w.W} R={w.R}")
    o, M, wsl, rsl = _run(w, x)
    o_ref, M_ref, wsl_ref, rsl_ref = _ref(w, x)
    assert np.array_equal(wsl.cpu().numpy(), wsl_ref) and np.array_equal(rsl.cpu().numpy(), rsl_ref)
    assert rel_l2(to_np(o), o_ref) <= TOL[w.io] and rel_l2(to_np(M), M_ref) <= 1e-5


def test_sdm_empty_sequence_leaves_table():
    torch, g = gpu()
    w = BASE.scaled(T=0, seed=105)
    x = gi.make_sparse_memory(w)
    o, M, _, _ = _run(w, x)
    assert o.numel() == 0 and np.array_equal(M.cpu().numpy(), x["M0"])


def test_sdm_unselected_slots_untouched():
    """Slots that no token writes keep their initial rows bit for bit."""
    w = BASE.scaled(B=1, H=2, T=30, n=32, W=6, R=6, seed=106)
    x = gi.make_sparse_memory(w)
    _, M, _, _ = _run(w, x)
    _, _, wsl_ref, _ = _ref(w, x)
    Mg = M.cpu().numpy()
    for h in range(w.H):
        untouched = np.setdiff1d(np.arange(w.N), wsl_ref[0, :, h].reshape(-1))
        assert untouched.size > 0 and np.array_equal(Mg[0, h, untouched], x["M0"][0, h, untouched])


def test_sdm_full_size_sampled():
    """B=4 T=4096 H=16, 65,536 slots x 128 per head, W = R = 128 (the timed call): the
    selections of 48 sampled (token, head) pairs spread over the sequence, and the
    read-outs of the first 192 tokens of two heads, against the oracle."""
    w = gi.SDM_B4H16
    x = gi.make_sparse_memory(w)
    o, M, wsl, rsl = _run(w, x)
    del M
    o, wsl, rsl = to_np(o), wsl.cpu().numpy(), rsl.cpu().numpy()
    rng = np.random.default_rng(5)
    for _ in range(48):
        b, t, h = int(rng.integers(w.B)), int(rng.integers(w.T)), int(rng.integers(w.H))
        ws_, _ = sdm.select(x["ks"][b, t, h, 0], x["ks"][b, t, h, 1], w.W)
        rs_, _ = sdm.select(x["qs"][b, t, h, 0], x["qs"][b, t, h, 1], w.R)
        assert np.array_equal(wsl[b, t, h], ws_) and np.array_equal(rsl[b, t, h], rs_), (b, t, h)
    for b, h in ((1, 5), (3, 14)):
        o_ref, _, _, _ = _ref(w, x, b=slice(b, b + 1), t=slice(0, 192), h=slice(h, h + 1))
        e = rel_l2(o[b, :192, h], o_ref[0, :, 0])
        log(f"[sdm] full size, head ({b}, {h}), first 192 tokens: rel-L2 o={e:.3e}")
        assert e <= TOL[w.io]
