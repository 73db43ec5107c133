"""GPU parity of gdr_chunk_fwd against the fp64 oracle (through the C-ABI).

Tolerances: rel-L2 <= 2e-3 for bf16 inputs, <= 1e-5 for fp32 inputs, on o and
on the final state, against the unrounded fp64 oracle."""
import numpy as np
import pytest

import gdr_inputs as gi
from tests.gpu_util import TOL, gpu, log, run_prefill, to_np, upload

pytestmark = pytest.mark.gpu

SMALL = gi.GDN_PREFILL.scaled(name="gdn_small", B=2, T=200, H=3, seed=11)

CASES = [
    # name, workload (several chunks, ragged last chunk unless noted)
    ("gdn_bf16_d128_C64", SMALL),
    ("gdn_bf16_d128_C16", SMALL.scaled(chunk=16, T=77)),
    ("gdn_bf16_d128_C32", SMALL.scaled(chunk=32, T=130)),
    ("kda_fg2plus_bf16", gi.KDA_FG2PLUS_PREFILL.scaled(B=2, T=150, H=2, seed=12)),
    ("fg2_shared_beta", gi.KDA_FG2PLUS_PREFILL.scaled(B=1, T=100, H=2, beta_mode=gi.BETA_SHARED, seed=13)),
    ("kda_scalar_beta", gi.KDA_FG2PLUS_PREFILL.scaled(B=1, T=129, H=2, beta_mode=gi.BETA_SCALAR, seed=14)),
    ("osdn_kw_S0", gi.OSDN_LONG_PREFILL.scaled(B=2, T=256, H=2, seed=15)),
    ("gdn_dk64_dv128", SMALL.scaled(dk=64, dv=128, T=90, seed=16)),
    ("gdn_dk128_dv48", SMALL.scaled(dk=128, dv=48, T=70, seed=17)),
    ("gdn_d8_C16", SMALL.scaled(dk=8, dv=8, T=45, chunk=16, s0_std=0.1, seed=18)),
    ("gdn_T1", SMALL.scaled(T=1, seed=19)),
    ("gdn_T_lt_C", SMALL.scaled(T=37, s0_std=0.02, seed=20)),
    ("gdn_T_multiple_of_C", SMALL.scaled(T=128, seed=21)),
    ("bf16_gates", SMALL.scaled(gate=gi.BF16, T=100, seed=22)),
    ("f32_io_d64", SMALL.scaled(io=gi.F32, dk=64, dv=64, T=150, seed=23)),
    # bf16 shapes the matrix-core kernels do not take run the vector-ALU kernel
    ("valu_kda_fg2plus_C32", gi.KDA_FG2PLUS_PREFILL.scaled(B=2, T=150, H=2, chunk=32, seed=24)),
    ("valu_osdn_kw_S0_C32", gi.OSDN_LONG_PREFILL.scaled(B=2, T=130, H=2, chunk=32, seed=25)),
    ("valu_fg2_shared_d64", gi.KDA_FG2PLUS_PREFILL.scaled(B=1, T=100, H=2, dk=64, dv=64,
                                                          beta_mode=gi.BETA_SHARED, seed=26)),
]


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_prefill_parity_small(name, w):
    r = run_prefill(w, gi.make_prefill(w))
    assert r["finite"]
    assert r["o"] <= TOL[w.io], r
    assert r["S"] <= TOL[w.io], r


def test_tiny_fp32_workload():
    """The tiny fp32 workload at full size: B=1 H=1 T=64 d=16 C=16."""
    w = gi.TINY_GDN_F32
    r = run_prefill(w, gi.make_prefill(w))
    assert r["o"] <= 1e-5 and r["S"] <= 1e-5, r


@pytest.mark.parametrize("w", [gi.GDN_PREFILL, gi.KDA_FG2PLUS_PREFILL], ids=lambda w: w.name)
def test_full_size_prefill(w):
    """Full-size batches; the oracle runs on a sample of 12 (batch, head) pairs."""
    rng = np.random.default_rng(0)
    heads = sorted(rng.choice(w.B * w.H, size=12, replace=False).tolist())
    r = run_prefill(w, gi.make_prefill(w), heads=heads)
    assert r["o"] <= TOL[w.io] and r["S"] <= TOL[w.io], r


# Long sequences with few heads (hundreds of chunks walked in order): against the
# oracle, and the read-out bit for bit equal whether or not the final state is asked for.
LONG = [
    ("gdn_T16500_ragged", gi.GDN_PREFILL.scaled(B=1, T=16500, H=2, seed=41)),
    ("osdn_kw_S0_T16384", gi.OSDN_LONG_PREFILL.scaled(B=2, T=16384, H=1, seed=42)),
    ("gdn_bf16_gates_T16400", gi.GDN_PREFILL.scaled(B=1, T=16400, H=1, gate=gi.BF16, seed=44)),
]


@pytest.mark.parametrize("name,w", LONG, ids=[c[0] for c in LONG])
def test_long_sequence(name, w):
    x = gi.make_prefill(w)
    r = run_prefill(w, x)
    assert r["o"] <= TOL[w.io] and r["S"] <= TOL[w.io], r
    torch, g = gpu()
    d = upload(x, w)
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta_k"])
    o_st, _ = g.chunk_fwd(*args, k_w=d["k_w"], S0=d["S0"])
    o_one, none = g.chunk_fwd(*args, k_w=d["k_w"], S0=d["S0"], want_state=False)
    torch.cuda.synchronize()
    assert none is None
    log(f"[prefill long] {name}: o equal with and without the final state: {torch.equal(o_st, o_one)}")
    assert torch.equal(o_st, o_one)


# With an execution context, a long sequence of few heads runs the prep of chunk blocks on
# the context's second stream beside the state recurrence (one state launch per block):
# bit for bit the call without a context, in place too.
CTX_LONG = [
    ("gdn_T16500_two_blocks", gi.GDN_PREFILL.scaled(B=1, T=16500, H=2, seed=45)),
    ("osdn_kw_S0_T65536_eight_blocks", gi.OSDN_LONG_PREFILL.scaled(B=1, T=65536, H=1, seed=46)),
    ("bf16_gates_T40000_ragged", gi.GDN_PREFILL.scaled(B=2, T=40000, H=1, gate=gi.BF16, seed=47)),
]


@pytest.mark.parametrize("name,w", CTX_LONG, ids=[c[0] for c in CTX_LONG])
def test_long_sequence_with_context(name, w):
    torch, g = gpu()
    x = gi.make_prefill(w)
    d = upload(x, w)
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta_k"])
    ctx = g.Context()
    o_ref, S_ref = g.chunk_fwd(*args, k_w=d["k_w"], S0=d["S0"])
    o_c, S_c = g.chunk_fwd(*args, k_w=d["k_w"], S0=d["S0"], ctx=ctx)
    S_io = (d["S0"] if d["S0"] is not None else torch.zeros_like(S_ref)).clone()
    o_io, _ = g.chunk_fwd(*args, k_w=d["k_w"], S0=S_io, final_state=S_io, ctx=ctx)
    torch.cuda.synchronize()
    same = torch.equal(o_c, o_ref) and torch.equal(S_c, S_ref)
    if d["S0"] is not None:
        same_io = torch.equal(o_io, o_ref) and torch.equal(S_io, S_ref)
    else:
        same_io = True  # S0 = zeros differs from S0 = NULL only in how the zero is read
    log(f"[prefill ctx] {name}: equal to the call without a context {same}; in place {same_io}")
    assert same and same_io
    # and against the oracle on one (batch, head)
    r = run_prefill(w, x, heads=[0])
    assert r["o"] <= TOL[w.io] and r["S"] <= TOL[w.io], r


def test_long_in_place_and_checkpoints():
    """A long sequence with S0 and S_T in one buffer (in-place resume), and with segment
    states kept: both bit for bit against the plain call."""
    torch, g = gpu()
    w = gi.OSDN_LONG_PREFILL.scaled(B=1, T=16500, H=2, seed=43)
    d = upload(gi.make_prefill(w), w)
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta_k"])
    o_ref, S_ref = g.chunk_fwd(*args, k_w=d["k_w"], S0=d["S0"])
    S_io = d["S0"].clone()
    o_io, S_out = g.chunk_fwd(*args, k_w=d["k_w"], S0=S_io, final_state=S_io)
    torch.cuda.synchronize()
    assert S_out.data_ptr() == S_io.data_ptr()
    same_io = torch.equal(o_io, o_ref) and torch.equal(S_io, S_ref)
    o_c, S_c, ck = g.chunk_fwd_ckpt(*args, 4096, k_w=d["k_w"], S0=d["S0"])
    o_c1, none, ck1 = g.chunk_fwd_ckpt(*args, 4096, k_w=d["k_w"], S0=d["S0"], want_state=False)
    torch.cuda.synchronize()
    assert none is None and ck.shape[2] == 4
    same_ck = torch.equal(o_c, o_ref) and torch.equal(S_c, S_ref) and torch.equal(o_c1, o_ref) and torch.equal(ck, ck1)
    log(f"[prefill long] in place equal {same_io}; checkpoints equal {same_ck}")
    assert same_io and same_ck


def test_full_size_long_context():
    """B=1 H=32 T=65536 with write key and nonzero S0; oracle on 4 sampled heads."""
    w = gi.OSDN_LONG_PREFILL
    r = run_prefill(w, gi.make_prefill(w), heads=[0, 9, 22, 31])
    assert r["o"] <= TOL[w.io] and r["S"] <= TOL[w.io], r


def test_T0_copies_initial_state():
    torch, g = gpu()
    w = SMALL.scaled(T=0, s0_std=0.05, seed=30)
    x = gi.make_prefill(w)
    d = upload(x, w)
    o, ST = g.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta_k"], S0=d["S0"], chunk=64)
    torch.cuda.synchronize()
    assert o.numel() == 0
    np.testing.assert_array_equal(to_np(ST), x["S0"].astype(np.float64))
    w0 = SMALL.scaled(T=0, seed=31)
    d0 = upload(gi.make_prefill(w0), w0)
    _, ST0 = g.chunk_fwd(d0["q"], d0["k"], d0["v"], d0["alpha"], d0["beta_k"], chunk=64)
    torch.cuda.synchronize()
    assert float(ST0.abs().max()) == 0.0


def test_in_place_resume_and_segments():
    """One call over T equals two calls chained through the state (S0 == ST in place)."""
    torch, g = gpu()
    w = SMALL.scaled(T=192, s0_std=0.02, seed=32)
    x = gi.make_prefill(w)
    d = upload(x, w)
    o_full, S_full = g.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta_k"], S0=d["S0"])
    cut = lambda t, a, b: t[:, a:b].contiguous()
    S = d["S0"].clone()
    o1, _ = g.chunk_fwd(cut(d["q"], 0, 64), cut(d["k"], 0, 64), cut(d["v"], 0, 64), cut(d["alpha"], 0, 64),
                        cut(d["beta_k"], 0, 64), S0=S, final_state=S)
    o2, _ = g.chunk_fwd(cut(d["q"], 64, 192), cut(d["k"], 64, 192), cut(d["v"], 64, 192),
                        cut(d["alpha"], 64, 192), cut(d["beta_k"], 64, 192), S0=S, final_state=S)
    torch.cuda.synchronize()
    # chunk boundaries coincide, so the two runs perform the same arithmetic
    np.testing.assert_array_equal(to_np(torch.cat([o1, o2], dim=1)), to_np(o_full))
    np.testing.assert_array_equal(to_np(S), to_np(S_full))


def test_deterministic():
    torch, g = gpu()
    w = SMALL.scaled(seed=33)
    d = upload(gi.make_prefill(w), w)
    a = g.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta_k"])
    b = g.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta_k"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_beta_zero_pure_decay_on_gpu():
    """beta = 0: the state only decays (closed form), checked on the GPU path."""
    torch, g = gpu()
    w = SMALL.scaled(T=130, s0_std=0.05, seed=34)
    x = gi.make_prefill(w)
    x["beta_k"] = np.zeros_like(x["beta_k"])
    d = upload(x, w)
    _, ST = g.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta_k"], S0=d["S0"])
    torch.cuda.synchronize()
    a = gi.as_f64(x["alpha"], w.gate)  # [B, T, H]
    decay = np.prod(a, axis=1)          # [B, H]
    expect = decay[:, :, None, None] * x["S0"].astype(np.float64)
    from oracle import rel_l2
    assert rel_l2(to_np(ST), expect) < 1e-5


def test_orthonormal_keys_exact_retrieval_on_gpu():
    """alpha = beta = 1 with permuted standard-basis keys (exact in bf16): every stored value
    is read back by its key."""
    torch, g = gpu()
    d, T = 128, 96
    rng = np.random.default_rng(35)
    perm = rng.permutation(d)[:T]
    k = np.zeros((1, T, 1, d), np.float32)
    k[0, np.arange(T), 0, perm] = 1.0
    v = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    sel = np.array([rng.integers(0, t + 1) for t in range(T)])
    q = k[:, sel]
    bf = lambda a: gi.to_torch(gi.f32_to_bf16_bits(a), gi.BF16)
    alpha = torch.ones((1, T, 1), device="cuda")
    beta = torch.ones((1, T, 1), device="cuda")
    o, ST = g.chunk_fwd(bf(q), bf(k), bf(v), alpha, beta)
    torch.cuda.synchronize()
    vb = gi.bf16_bits_to_f32(gi.f32_to_bf16_bits(v)).astype(np.float64)
    from oracle import rel_l2
    assert rel_l2(to_np(o)[0, :, 0], vb[0, sel, 0]) < 4e-3  # o stored in bf16
    St = to_np(ST)[0, 0]
    assert rel_l2(St[perm].reshape(T, d), vb[0, :, 0]) < 1e-5
