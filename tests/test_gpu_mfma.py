"""The bf16 matrix-core prefill path: its per-chunk workspace record (UT transform,
intra-chunk scores, decay factors) against NumPy fp64 built from the same stored
inputs, and the path selection.  The end-to-end parity of this path against the
oracle is in test_gpu_prefill.py (every bf16 d=128 chunk-64 scalar-gate case
selects it)."""
import numpy as np
import pytest

import gdr_inputs as gi
from tests.gpu_util import TOL, gpu, log, run_prefill, upload

pytestmark = pytest.mark.gpu

REC_BYTES = 25728  # per-chunk record: T bf16[64][64] | P hi bf16[64][64] | P lo (columns permuted, below)
#                    | gam f32[64] | fac f32[64]
#                    | gC (128-byte slot) | g f32[64] | beta f32[64]


def _bf16(u16):
    return gi.bf16_bits_to_f32(u16).astype(np.float64)


# Tm and P keep their token columns in the order the state kernels' fragments read them:
# column s = 32 kk + 16 h + 4 q + i is stored at 32 kk + 8 q + 4 h + i.
_STORED_COL = np.array([(s & 32) | ((s & 12) << 1) | ((s & 16) >> 2) | (s & 3) for s in range(64)])
assert sorted(_STORED_COL.tolist()) == list(range(64))


@pytest.mark.parametrize("T,write_key", [(200, False), (128, True)])
def test_prep_record_matches_numpy(T, write_key):
    torch, g = gpu()
    w = gi.GDN_PREFILL.scaled(B=1, T=T, H=2, write_key=write_key, seed=51)
    x = gi.make_prefill(w)
    d = upload(x, w)
    desc = g.make_desc(d["q"], d["v"], d["alpha"], d["beta_k"], None, chunk=64)
    assert g.gdr_chunk_fwd_path(desc) == g.PATH_MFMA
    nbytes = g.gdr_chunk_fwd_workspace_size(desc)
    NT = (T + 63) // 64
    assert nbytes == w.B * w.H * NT * REC_BYTES
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    g.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta_k"], k_w=d["k_w"], workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    f = gi.prefill_f64(w, x)
    kw = f["k"] if f["k_w"] is None else f["k_w"]
    worst = {"T": 0.0, "P": 0.0, "gam": 0.0, "fac": 0.0}
    for bh in range(w.B * w.H):
        b, h = divmod(bh, w.H)
        for c in range(NT):
            rec = raw[(bh * NT + c) * REC_BYTES:(bh * NT + c + 1) * REC_BYTES]
            Tg = _bf16(rec[0:8192].view(np.uint16).reshape(64, 64))[:, _STORED_COL]
            Pg = (_bf16(rec[8192:16384].view(np.uint16).reshape(64, 64)) +
                  _bf16(rec[16384:24576].view(np.uint16).reshape(64, 64)))[:, _STORED_COL]
            gam = rec[24576:24832].view(np.float32).astype(np.float64)
            fac = rec[24832:25088].view(np.float32).astype(np.float64)
            gC = float(rec[25088:25092].view(np.float32)[0])
            glog = rec[25216:25472].view(np.float32).astype(np.float64)
            beta = rec[25472:25728].view(np.float32).astype(np.float64)
            t0, n = 64 * c, min(64, T - 64 * c)
            K = np.zeros((64, 128)); KW = np.zeros((64, 128)); Q = np.zeros((64, 128))
            K[:n] = f["k"][b, t0:t0 + n, h]
            KW[:n] = kw[b, t0:t0 + n, h]
            Q[:n] = f["q"][b, t0:t0 + n, h]
            be = np.zeros(64); be[:n] = f["beta_k"][b, t0:t0 + n, h]
            la = np.zeros(64); la[:n] = np.log(f["alpha"][b, t0:t0 + n, h])
            gcum = np.cumsum(la)
            W = be[None, :] * np.exp(gcum[:, None] - gcum[None, :])
            A = np.tril((K @ KW.T) * W, -1)
            Tr = np.linalg.inv(np.eye(64) + A)
            Pr = np.tril((Q @ KW.T) * W, 0)
            worst["T"] = max(worst["T"], np.abs(Tg - Tr).max() / np.abs(Tr).max())
            worst["P"] = max(worst["P"], np.abs(Pg - Pr).max() / max(np.abs(Pr).max(), 1e-30))
            worst["gam"] = max(worst["gam"], np.abs(gam - np.exp(gcum)).max())
            worst["g"] = max(worst.get("g", 0.0), np.abs(glog - gcum).max())
            worst["beta"] = max(worst.get("beta", 0.0), np.abs(beta - be).max())
            fr = be * np.exp(gcum[n - 1] - gcum)
            fr[n:] = 0
            worst["fac"] = max(worst["fac"], np.abs(fac - fr).max())
            assert abs(gC - np.exp(gcum[n - 1])) < 1e-5
    log(f"[prep record] worst {worst}")
    assert worst["T"] < 8e-3      # stored in bf16
    assert worst["P"] < 1e-5      # two bf16 terms
    assert worst["gam"] < 1e-5 and worst["fac"] < 1e-5
    assert worst["g"] < 1e-4 and worst["beta"] < 1e-6


def test_matrix_core_and_vector_alu_kernels_agree():
    """The same bf16 inputs through chunk 64 (matrix-core kernels) and chunk 32 (the
    fp32 vector-ALU kernel): both are exact forms of the one recurrence."""
    torch, g = gpu()
    w = gi.OSDN_LONG_PREFILL.scaled(B=2, T=333, H=3, seed=52)
    d = upload(gi.make_prefill(w), w)
    a = g.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta_k"], k_w=d["k_w"], S0=d["S0"], chunk=64)
    b = g.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta_k"], k_w=d["k_w"], S0=d["S0"], chunk=32)
    torch.cuda.synchronize()
    from oracle import rel_l2
    eo = rel_l2(a[0].float().cpu().numpy(), b[0].float().cpu().numpy())
    es = rel_l2(a[1].cpu().numpy(), b[1].cpu().numpy())
    log(f"[chunk 64 mfma vs chunk 32 valu] o {eo:.3e} S {es:.3e}")
    assert eo < 2e-3 and es < 2e-3


def test_path_selection_on_device():
    torch, g = gpu()
    w = gi.GDN_PREFILL.scaled(B=1, T=64, H=1)
    d = upload(gi.make_prefill(w), w)
    desc = g.make_desc(d["q"], d["v"], d["alpha"], d["beta_k"], None, chunk=64)
    assert g.gdr_chunk_fwd_path(desc) == g.PATH_MFMA
    desc32 = g.make_desc(d["q"], d["v"], d["alpha"], d["beta_k"], None, chunk=32)
    assert g.gdr_chunk_fwd_path(desc32) == g.PATH_VALU


STATE_CASES = [
    # several chunks with a ragged tail; B * H not a multiple of 8 (idle workgroups)
    ("gdn_ragged", gi.GDN_PREFILL.scaled(B=3, T=333, H=3, seed=61)),
    ("osdn_kw_S0", gi.OSDN_LONG_PREFILL.scaled(B=1, T=300, H=5, seed=62)),
    ("gdn_T_lt_C", gi.GDN_PREFILL.scaled(B=2, T=41, H=2, s0_std=0.02, seed=63)),
    ("gdn_T_one_chunk", gi.GDN_PREFILL.scaled(B=1, T=64, H=9, seed=64)),
    # 64 (batch, head) pairs: the wave-specialised kernel takes two column tiles per workgroup
    ("gdn_64heads_ragged", gi.GDN_PREFILL.scaled(B=4, T=130, H=16, seed=65)),
    ("osdn_64heads_S0", gi.OSDN_LONG_PREFILL.scaled(B=2, T=100, H=32, seed=66)),
]


@pytest.mark.parametrize("name,w", STATE_CASES, ids=[c[0] for c in STATE_CASES])
def test_state_kernel_cases(name, w):
    """The matrix-core state kernel on ragged, short, one-chunk and many-head shapes."""
    torch, g = gpu()
    r = run_prefill(w, gi.make_prefill(w))
    assert r["path"] == g.PATH_MFMA
    assert r["finite"]
    assert r["o"] <= TOL[w.io] and r["S"] <= TOL[w.io], r


GENERAL_CASES = [
    # channel forget gate and / or beta vectors on the matrix-core path
    ("kda_kv_beta_bf16_gates", gi.KDA_FG2PLUS_PREFILL.scaled(B=2, T=200, H=3, gate=gi.BF16, seed=67)),
    ("kda_write_key_S0", gi.KDA_FG2PLUS_PREFILL.scaled(B=1, T=150, H=4, write_key=True, s0_std=0.02, seed=68)),
    ("fg2_shared_beta_bf16_gates", gi.KDA_FG2PLUS_PREFILL.scaled(B=1, T=90, H=3, beta_mode=gi.BETA_SHARED,
                                                                  gate=gi.BF16, seed=69)),
    ("scalar_alpha_kv_beta", gi.KDA_FG2PLUS_PREFILL.scaled(B=2, T=128, H=2, alpha_mode=gi.GATE_SCALAR, seed=70)),
    ("kda_scalar_beta_T_lt_C", gi.KDA_FG2PLUS_PREFILL.scaled(B=3, T=37, H=2, beta_mode=gi.BETA_SCALAR, seed=71)),
    ("kda_64heads", gi.KDA_FG2PLUS_PREFILL.scaled(B=4, T=70, H=16, seed=72)),
]


@pytest.mark.parametrize("name,w", GENERAL_CASES, ids=[c[0] for c in GENERAL_CASES])
def test_general_gate_path(name, w):
    """The general-gate record and kernels (channel decay, beta vectors) against the oracle."""
    torch, g = gpu()
    r = run_prefill(w, gi.make_prefill(w))
    assert r["path"] == g.PATH_MFMA
    assert r["finite"]
    assert r["o"] <= TOL[w.io] and r["S"] <= TOL[w.io], r
