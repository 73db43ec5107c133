"""The C-ABI library loads, exports every symbol include/gdr.h declares, and
rejects bad arguments on the host with the documented status before anything
is launched (these calls never reach the GPU, so they run anywhere)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")


@pytest.fixture(scope="module")
def g():
    import gated_delta_rule_84_amd as g

    return g


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(g):
    declared = _declared_functions()
    assert {"gdr_chunk_fwd", "gdr_decode_step", "gdr_chunk_fwd_workspace_size"} <= set(declared)
    out = subprocess.run(["nm", "-D", "--defined-only", g.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (gdr_[a-z0-9_]+)", out))
    missing = [f for f in declared if f not in exported]
    assert not missing, f"declared but not exported: {missing}"
    assert set(g.EXPORTED) == set(declared)


def test_header_compiles_as_c():
    src = '#include "gdr.h"\nint main(void){gdr_desc d={0};(void)d;return (int)sizeof(gdr_desc);}\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-x", "c", "-",
                        "-fsyntax-only"], input=src, text=True, capture_output=True)
    assert r.returncode == 0, r.stderr


def test_version_and_status_strings(g):
    assert g.gdr_version() >> 16 == 2  # 2.0: execution contexts, testing flags removed
    for s in (g.GDR_OK, g.GDR_EINVAL, g.GDR_EUNSUPPORTED, g.GDR_EWORKSPACE, g.GDR_EHIP):
        assert g.gdr_status_string(s).startswith("GDR_")
    assert "unknown" in g.gdr_status_string(12345)


def _desc(g, **kw):
    base = dict(B=2, T=100, H=3, dk=128, dv=128, chunk=64, io_dtype=g.GDR_BF16, gate_dtype=g.GDR_F32,
                alpha_mode=g.GDR_ALPHA_SCALAR, beta_mode=g.GDR_BETA_SCALAR, flags=0)
    base.update(kw)
    return g.Desc(**base)


class FakePtr:
    """A stand-in tensor: only data_ptr() is used by the binding and the
    library never dereferences it on a rejected call."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def _ptrs(start=0x10000000, n=10, step=0x1000000):
    return [FakePtr(start + i * step) for i in range(n)]


@pytest.mark.parametrize("field,value,status", [
    ("B", -1, -1), ("T", -1, -1), ("H", -1, -1),
    ("dk", 0, -2), ("dk", 12, -2), ("dk", 136, -2), ("dv", 4, -2), ("dv", 256, -2),
    ("chunk", 8, -2), ("chunk", 128, -2), ("chunk", 48, -2),
    ("io_dtype", 7, -1), ("gate_dtype", -3, -1), ("alpha_mode", 2, -1), ("beta_mode", 3, -1),
    ("flags", 0x40, -1), ("flags", 0x1, -1), ("flags", 0x2, -1), ("flags", 0x8, -1),
    ("flags", 0x10, -2), ("flags", 0x20, -2),  # decode-only options
])
def test_descriptor_validation(g, field, value, status):
    d = _desc(g, **{field: value})
    q, k, v, a, b, o, st = _ptrs(n=7)
    assert g.gdr_chunk_fwd(d, q, k, None, v, a, b, None, None, o, st, None, 0, 0) == status
    assert g.gdr_chunk_fwd_ctx(d, q, k, None, v, a, b, None, None, o, st, None, 0, None, 0) == status
    assert g.gdr_chunk_fwd_path(d) == status
    assert g.gdr_chunk_fwd_workspace_size(d) == 0


def test_shared_beta_needs_square(g):
    d = _desc(g, dk=64, dv=128, beta_mode=g.GDR_BETA_SHARED)
    q, k, v, a, b, o, st = _ptrs(n=7)
    assert g.gdr_chunk_fwd(d, q, k, None, v, a, b, None, None, o, st, None, 0, 0) == g.GDR_EINVAL


def test_null_and_misaligned_pointers(g):
    d = _desc(g)
    q, k, v, a, b, o, st = _ptrs(n=7)
    assert g.gdr_chunk_fwd(d, None, k, None, v, a, b, None, None, o, st, None, 0, 0) == g.GDR_EINVAL
    assert g.gdr_chunk_fwd(d, q, k, None, v, a, b, None, None, None, st, None, 0, 0) == g.GDR_EINVAL
    assert g.gdr_chunk_fwd(d, FakePtr(q.addr + 8), k, None, v, a, b, None, None, o, st, None, 0, 0) \
        == g.GDR_EINVAL
    # beta_v given without the KV layout, and missing with it
    assert g.gdr_chunk_fwd(d, q, k, None, v, a, b, FakePtr(0x20000000), None, o, st, None, 0, 0) \
        == g.GDR_EINVAL
    dkv = _desc(g, beta_mode=g.GDR_BETA_KV)
    assert g.gdr_chunk_fwd(dkv, q, k, None, v, a, b, None, None, o, st, None, 0, 0) == g.GDR_EINVAL
    # the context-taking prefill checks the same arguments before it looks at the context
    assert g.gdr_chunk_fwd_ctx(d, None, k, None, v, a, b, None, None, o, st, None, 0, None, 0) == g.GDR_EINVAL
    assert g.gdr_chunk_fwd_ctx(d, q, k, None, v, a, b, None, None, q, st, None, 0, None, 0) == g.GDR_EINVAL


def test_output_may_not_alias_inputs(g):
    d = _desc(g)
    q, k, v, a, b, o, st = _ptrs(n=7)
    assert g.gdr_chunk_fwd(d, q, k, None, v, a, b, None, None, q, st, None, 0, 0) == g.GDR_EINVAL
    assert g.gdr_chunk_fwd(d, q, k, None, v, a, b, None, None, FakePtr(v.addr + 64), st, None, 0, 0) \
        == g.GDR_EINVAL
    # partial overlap of S0 and ST is rejected
    s0 = FakePtr(0x50000000)
    assert g.gdr_chunk_fwd(d, q, k, None, v, a, b, None, s0, o, FakePtr(s0.addr + 256), None, 0, 0) \
        == g.GDR_EINVAL


def test_decode_validation(g):
    d = _desc(g, T=1)
    q, k, v, a, b, S, o = _ptrs(n=7)
    assert g.gdr_decode_step(_desc(g, dk=20), q, k, None, v, a, b, None, S, o, 0) == g.GDR_EUNSUPPORTED
    assert g.gdr_decode_step(d, q, k, None, v, a, None, None, S, o, 0) == g.GDR_EINVAL
    assert g.gdr_decode_step(d, q, k, None, v, a, b, None, S, S, 0) == g.GDR_EINVAL
    assert g.gdr_decode_step(d, q, k, None, v, a, b, None, FakePtr(S.addr + 4), o, 0) == g.GDR_EINVAL
    # empty batch is a no-op even with NULL pointers
    assert g.gdr_decode_step(_desc(g, B=0), None, None, None, None, None, None, None, None, None, 0) == g.GDR_OK


def test_empty_batch_is_noop(g):
    d = _desc(g, B=0)
    assert g.gdr_chunk_fwd(d, None, None, None, None, None, None, None, None, None, None, None, 0, 0) == g.GDR_OK


def test_path_selection(g):
    assert g.gdr_chunk_fwd_path(_desc(g)) == g.PATH_MFMA
    # channel decay and beta vectors take the matrix-core path too (general-gate record)
    assert g.gdr_chunk_fwd_path(_desc(g, alpha_mode=g.GDR_ALPHA_CHANNEL, beta_mode=g.GDR_BETA_KV)) == g.PATH_MFMA
    assert g.gdr_chunk_fwd_path(_desc(g, beta_mode=g.GDR_BETA_SHARED)) == g.PATH_MFMA
    assert g.gdr_chunk_fwd_path(_desc(g, chunk=32)) == g.PATH_VALU
    assert g.gdr_chunk_fwd_path(_desc(g, io_dtype=g.GDR_F32)) == g.PATH_VALU


def test_workspace_sizes(g):
    """One record per (batch, head, chunk): 25728 bytes for scalar gates, 123392 for the
    general-gate record (Tm, P, and U, Q, W as two bf16 terms each, e^{g_C})."""
    nrec = 2 * 3 * 2  # B=2, H=3, T=100 -> 2 chunks of 64
    assert g.gdr_chunk_fwd_workspace_size(_desc(g)) == nrec * 25728
    assert g.gdr_chunk_fwd_workspace_size(_desc(g, alpha_mode=g.GDR_ALPHA_CHANNEL)) == nrec * 123392
    assert g.gdr_chunk_fwd_workspace_size(_desc(g, beta_mode=g.GDR_BETA_SHARED)) == nrec * 123392
    assert g.gdr_chunk_fwd_path(_desc(g, dk=64, dv=64)) == g.PATH_VALU


def test_binding_fails_loudly_without_library(tmp_path):
    """Importing the binding with no built library raises; nothing falls back."""
    import shutil
    import sys

    pkg = tmp_path / "gated_delta_rule_84_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "gated_delta_rule_84_amd", "__init__.py"), pkg / "__init__.py")
    code = "import gated_delta_rule_84_amd"
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode != 0 and "ImportError" in r.stderr


# ---------------------------------------------------------------------------
# Memory-Caching entry points: host-side validation (nothing is launched)
# ---------------------------------------------------------------------------
def test_chunk_fwd_ckpt_validation(g):
    d = _desc(g, T=512)
    q, k, v, a, b, o, st, ck, ws = _ptrs(n=9)
    call = lambda desc, seg, ckpt, out=o: g.gdr_chunk_fwd_ckpt(desc, q, k, None, v, a, b, None, None, out, st,
                                                               seg, ckpt, ws, 1 << 30, 0)
    assert call(d, 0, ck) == g.GDR_EINVAL            # segment length must be positive
    assert call(d, 96, ck) == g.GDR_EINVAL           # and a multiple of the chunk
    assert call(d, 128, None) == g.GDR_EINVAL        # 4 segment states need a buffer
    assert call(d, 128, FakePtr(ck.addr + 4)) == g.GDR_EINVAL  # misaligned
    assert call(d, 128, o) == g.GDR_EINVAL           # overlaps the output
    assert call(_desc(g, T=512, chunk=48), 128, ck) == g.GDR_EUNSUPPORTED


def test_mc_readout_validation(g):
    d = _desc(g, T=1024)
    q, ck, gt, oi, oo, ws = _ptrs(n=6, step=0x10000000)
    need = g.gdr_mc_readout_workspace_size(d, 4)
    assert need == 2 * 3 * 4 * 128 * 128 * 4
    call = lambda desc, **kw: g.gdr_mc_readout(desc, kw.get("q", q), kw.get("ck", ck), kw.get("n", 4),
                                               kw.get("seg", 256), kw.get("gt", gt), kw.get("oi", oi),
                                               kw.get("oo", oo), kw.get("ws", ws), kw.get("wb", need), 0)
    assert call(_desc(g, T=1024, io_dtype=g.GDR_F32)) == g.GDR_EUNSUPPORTED
    assert call(_desc(g, T=1024, dk=64, dv=64)) == g.GDR_EUNSUPPORTED
    assert call(d, seg=0) == g.GDR_EINVAL
    assert call(d, n=-1) == g.GDR_EINVAL
    assert call(d, ck=None) == g.GDR_EINVAL
    assert call(d, q=None) == g.GDR_EINVAL
    assert call(d, oo=FakePtr(oo.addr + 8)) == g.GDR_EINVAL
    assert call(d, wb=need - 1) == g.GDR_EWORKSPACE
    assert call(d, ws=None) == g.GDR_EWORKSPACE
    assert call(d, oo=FakePtr(q.addr + 256)) == g.GDR_EINVAL           # output overlaps q
    assert call(d, oi=FakePtr(oo.addr + 256)) == g.GDR_EINVAL          # partial overlap of o_in and o_out
    assert call(d, ws=FakePtr(ck.addr)) == g.GDR_EINVAL                # workspace overlaps the caches
    assert call(_desc(g, B=0)) == g.GDR_OK                             # empty batch: nothing to do


def test_osdn_precond_validation(g):
    d = _desc(g, T=256)
    k, b, r, kw, dT, qg, ws = _ptrs(n=7, step=0x10000000)
    need = g.gdr_osdn_precond_workspace_size(d)
    assert need == 2 * 3 * 4 * 19200
    call = lambda desc, **kw_: g.gdr_osdn_precond(desc, kw_.get("k", k), kw_.get("b", b), kw_.get("r", r), 1.0,
                                                 None, kw_.get("kw", kw), kw_.get("dT", dT), kw_.get("qg", qg),
                                                 kw_.get("ws", ws), kw_.get("wb", need), None, 0)
    assert call(_desc(g, T=256, beta_mode=g.GDR_BETA_SHARED)) == g.GDR_EINVAL  # scalar write strength only
    assert call(_desc(g, T=256, dk=136)) == g.GDR_EUNSUPPORTED
    assert call(d, k=None) == g.GDR_EINVAL
    assert call(d, kw=FakePtr(k.addr + 512)) == g.GDR_EINVAL            # output overlaps the keys
    assert call(d, ws=None) == g.GDR_EWORKSPACE
    assert call(d, wb=need - 16) == g.GDR_EWORKSPACE
    assert call(d, ws=FakePtr(b.addr)) == g.GDR_EINVAL                  # workspace overlaps an input
    assert call(_desc(g, B=0)) == g.GDR_OK


def test_sdm_validation(g):
    d = _desc(g, T=50)
    ks, qs, v, a, b, M, o, ws_, rs_, ws = _ptrs(n=10, step=0x10000000)
    need = g.gdr_sdm_workspace_size(d, 256, 128, 64)
    assert need == 2 * 50 * 3 * (128 + 64) * 8
    call = lambda desc, n=256, W=128, R=64, **kw_: g.gdr_sdm_fwd(
        desc, n, W, R, kw_.get("ks", ks), kw_.get("qs", qs), v, a, b, kw_.get("M", M), kw_.get("o", o),
        kw_.get("wsl", ws_), rs_, kw_.get("ws", ws), kw_.get("wb", need), None, 0)
    assert call(_desc(g, T=50, dv=64)) == g.GDR_EUNSUPPORTED             # rows of 128 values only
    assert call(d, n=1025) == g.GDR_EUNSUPPORTED
    assert call(d, W=129) == g.GDR_EUNSUPPORTED
    assert call(d, n=8, R=65) == g.GDR_EUNSUPPORTED                      # more slots than the table holds
    assert call(d, W=0) == g.GDR_EINVAL
    assert call(d, ks=None) == g.GDR_EINVAL
    assert call(d, M=FakePtr(M.addr + 2)) == g.GDR_EINVAL                # table must be 16-byte aligned
    assert call(d, o=FakePtr(v.addr + 256)) == g.GDR_EINVAL              # output overlaps v
    assert call(d, wsl=FakePtr(M.addr + 64)) == g.GDR_EINVAL             # slot output inside the table
    assert call(d, ws=None) == g.GDR_EWORKSPACE
    assert call(d, wb=need - 8) == g.GDR_EWORKSPACE
    assert call(_desc(g, B=0)) == g.GDR_OK                               # nothing to do
    assert call(_desc(g, T=50, io_dtype=5)) == g.GDR_EINVAL


def test_binding_refuses_host_and_strided_tensors(g):
    """The binding passes raw addresses: a host tensor or a non-contiguous view is
    refused before any call reaches the library."""
    import torch

    d = _desc(g, B=1, T=4, H=1, dk=8, dv=8, io_dtype=g.GDR_F32)
    host, gate, state = torch.zeros((1, 1, 8)), torch.zeros((1, 1)), torch.zeros((1, 1, 8, 8))
    with pytest.raises(ValueError, match="device tensor"):
        g.gdr_decode_step(d, host, host, None, host, gate, gate, None, state, host, 0)
    with pytest.raises(ValueError, match="elements"):
        g.gdr_decode_step(d, host, host, None, host, host, host, None, host, host, 0)
    with pytest.raises(ValueError, match="contiguous"):
        g._ptr(torch.zeros((4, 4)).t())
    assert g._ptr(None) is None


# ---- the binding checks every tensor against the descriptor before the call ----

def _prefill_tensors(g, B=1, T=5, H=2, dk=16, dv=16, io=None, gate=None):
    import torch

    io = io or torch.bfloat16
    gate = gate or torch.float32
    return dict(q=torch.zeros(B, T, H, dk, dtype=io), k=torch.zeros(B, T, H, dk, dtype=io),
                v=torch.zeros(B, T, H, dv, dtype=io), alpha=torch.zeros(B, T, H, dtype=gate),
                beta_k=torch.zeros(B, T, H, dtype=gate), o=torch.zeros(B, T, H, dv, dtype=io),
                ST=torch.zeros(B, H, dk, dv, dtype=torch.float32))


@pytest.mark.parametrize("bad", ["S0_bf16", "k_other_dk", "k_w_fp32", "beta_k_bf16", "beta_v_shape", "ST_short",
                                 "o_fp32", "alpha_channel_missing"])
def test_binding_rejects_mismatched_tensors(g, bad):
    import torch

    t = _prefill_tensors(g)
    d = _desc(g, B=1, T=5, H=2, dk=16, dv=16)
    kw = dict(k_w=None, beta_v=None, S0=None)
    if bad == "S0_bf16":
        kw["S0"] = torch.zeros(1, 2, 16, 16, dtype=torch.bfloat16)
    elif bad == "k_other_dk":
        t["k"] = torch.zeros(1, 5, 2, 8, dtype=torch.bfloat16)
    elif bad == "k_w_fp32":
        kw["k_w"] = torch.zeros(1, 5, 2, 16, dtype=torch.float32)
    elif bad == "beta_k_bf16":
        t["beta_k"] = torch.zeros(1, 5, 2, dtype=torch.bfloat16)
    elif bad == "beta_v_shape":
        d = _desc(g, B=1, T=5, H=2, dk=16, dv=16, beta_mode=g.GDR_BETA_KV)
        t["beta_k"] = torch.zeros(1, 5, 2, 16)
        kw["beta_v"] = torch.zeros(1, 5, 2, 8)
    elif bad == "ST_short":
        t["ST"] = torch.zeros(1, 2, 16, 8)
    elif bad == "o_fp32":
        t["o"] = torch.zeros(1, 5, 2, 16, dtype=torch.float32)
    elif bad == "alpha_channel_missing":
        d = _desc(g, B=1, T=5, H=2, dk=16, dv=16, alpha_mode=g.GDR_ALPHA_CHANNEL)
    with pytest.raises(ValueError):
        g.gdr_chunk_fwd(d, t["q"], t["k"], kw["k_w"], t["v"], t["alpha"], t["beta_k"], kw["beta_v"], kw["S0"],
                        t["o"], t["ST"], None, 0, 0)


def test_binding_rejects_host_tensors_of_the_right_shape(g):
    t = _prefill_tensors(g)
    d = _desc(g, B=1, T=5, H=2, dk=16, dv=16)
    with pytest.raises(ValueError, match="device tensor"):
        g.gdr_chunk_fwd(d, t["q"], t["k"], None, t["v"], t["alpha"], t["beta_k"], None, None, t["o"], t["ST"],
                        None, 0, 0)


def test_binding_rejects_oversized_workspace_claim(g):
    import torch

    d = _desc(g, B=1, T=5, H=2, dk=16, dv=16)
    ws = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="workspace"):
        g.gdr_chunk_fwd(d, None, None, None, None, None, None, None, None, None, None, ws, 65, 0)


def test_dmem_validation(g):
    d = _desc(g, T=40, H=4, dk=8, dv=8)
    q, k, v, lam, beta, seg, M, out = _ptrs(n=8, step=0x10000000)
    call = lambda desc, J=1, **kw_: g.gdr_dmem_fwd(
        desc, J, kw_.get("q", q), k, v, lam, beta, kw_.get("seg", seg), kw_.get("M", M), kw_.get("out", out), 0)
    assert call(_desc(g, T=40, H=4, dk=4, dv=4)) == g.GDR_EUNSUPPORTED   # r = 8 or 16
    assert call(_desc(g, T=40, H=4, dk=16, dv=16), J=8) == g.GDR_EUNSUPPORTED  # 16-wide: at most 4 sub-states
    assert call(d, J=3) == g.GDR_EUNSUPPORTED
    assert call(_desc(g, T=40, H=6, dk=8, dv=8), J=4) == g.GDR_EINVAL   # H a multiple of J
    assert call(_desc(g, T=40, H=4, dk=8, dv=16)) == g.GDR_EINVAL       # square memory
    assert call(d, J=0) == g.GDR_EINVAL
    assert call(_desc(g, T=40, H=4, dk=8, dv=8, alpha_mode=1)) == g.GDR_EINVAL
    assert call(_desc(g, T=40, H=4, dk=8, dv=8, flags=0x10)) == g.GDR_EINVAL
    assert call(d, q=None) == g.GDR_EINVAL
    assert call(d, q=FakePtr(q.addr + 8)) == g.GDR_EINVAL               # rows are read 16 bytes at a time
    assert call(d, out=FakePtr(k.addr + 64)) == g.GDR_EINVAL            # output overlaps k
    assert call(d, M=FakePtr(out.addr)) == g.GDR_EINVAL                 # memory overlaps the output
    assert call(_desc(g, T=0, H=4, dk=8, dv=8)) == g.GDR_OK             # nothing to do
    assert call(_desc(g, B=0, H=4, dk=8, dv=8), q=None) == g.GDR_OK


def test_binding_checks_the_other_entry_points(g):
    import torch

    bf, f32 = torch.bfloat16, torch.float32
    dd = _desc(g, B=2, H=3, dk=16, dv=16, gate_dtype=g.GDR_BF16)
    with pytest.raises(ValueError, match="S"):          # state given in bf16
        g.gdr_decode_step(dd, torch.zeros(2, 3, 16, dtype=bf), torch.zeros(2, 3, 16, dtype=bf), None,
                          torch.zeros(2, 3, 16, dtype=bf), torch.zeros(2, 3, dtype=bf), torch.zeros(2, 3, dtype=bf),
                          None, torch.zeros(2, 3, 16, 16, dtype=bf), torch.zeros(2, 3, 16, dtype=bf))
    do = _desc(g, B=1, T=4, H=2, dk=16, dv=16)
    with pytest.raises(ValueError, match="k_w"):        # write key of another size
        g.gdr_osdn_precond(do, torch.zeros(1, 4, 2, 16, dtype=bf), torch.zeros(1, 4, 2), None, 1.0, None,
                           torch.zeros(1, 4, 2, 8, dtype=bf), None, None, None, 0, None, 0)
    dm = _desc(g, B=1, T=4, H=2, dk=128, dv=128)
    with pytest.raises(ValueError, match="gates"):      # gates for another number of caches
        g.gdr_mc_readout(dm, torch.zeros(1, 4, 2, 128, dtype=bf), torch.zeros(1, 2, 3, 128, 128), 3, 64,
                         torch.zeros(1, 4, 2, 2), None, torch.zeros(1, 4, 2, 128, dtype=bf), None, 0, 0)
    dd = _desc(g, B=1, T=4, H=4, dk=8, dv=8, gate_dtype=g.GDR_BF16)
    with pytest.raises(ValueError, match="out"):        # reads of every head where groups of 2 were asked for
        g.gdr_dmem_fwd(dd, 2, torch.zeros(1, 4, 4, 8, dtype=bf), torch.zeros(1, 4, 4, 8, dtype=bf),
                       torch.zeros(1, 4, 4, 8, dtype=bf), torch.zeros(1, 4, 4, dtype=bf), torch.zeros(1, 4, 4, dtype=bf),
                       None, torch.zeros(1, 4, 8, 8), torch.zeros(1, 4, 4, 8, dtype=bf))
    with pytest.raises(ValueError, match="seg_end"):    # segment marks as booleans
        g.gdr_dmem_fwd(dd, 1, torch.zeros(1, 4, 4, 8, dtype=bf), torch.zeros(1, 4, 4, 8, dtype=bf),
                       torch.zeros(1, 4, 4, 8, dtype=bf), torch.zeros(1, 4, 4, dtype=bf), torch.zeros(1, 4, 4, dtype=bf),
                       torch.zeros(1, 4, dtype=torch.bool), torch.zeros(1, 4, 8, 8), torch.zeros(1, 4, 4, 8, dtype=bf))
    ds = _desc(g, B=1, T=4, H=2, dk=128, dv=128)
    with pytest.raises(ValueError, match="w_slots"):    # slot list of the wrong integer type
        g.gdr_sdm_fwd(ds, 4, 2, 2, torch.zeros(1, 4, 2, 2, 4), torch.zeros(1, 4, 2, 2, 4),
                      torch.zeros(1, 4, 2, 128, dtype=bf), torch.zeros(1, 4, 2), torch.zeros(1, 4, 2),
                      torch.zeros(1, 2, 16, 128), torch.zeros(1, 4, 2, 128, dtype=bf),
                      torch.zeros(1, 4, 2, 2, dtype=torch.int64), None, None, 0, None, 0)


def test_context_create_and_destroy_arguments(g):
    """gdr_context_create refuses a NULL out-pointer; destroying NULL is a no-op."""
    assert g._lib.gdr_context_create(None) == g.GDR_EINVAL
    assert g.gdr_context_destroy(None) == g.GDR_OK


def test_noalloc_rejects_calls_beyond_its_scratch(g):
    """gdr_chunk_fwd_noalloc refuses, before touching any device, a call whose record
    would not fit its static scratch (GDR_ETOOLARGE); a descriptor error comes first."""
    q, k, v, a, b, o, st = _ptrs(n=7, step=0x40000000)
    big = _desc(g, B=4, H=16, T=8192)            # 8,192 chunks x 25,728 B > 128 MiB
    assert g.gdr_chunk_fwd_workspace_size(big) > g.GDR_NOALLOC_SCRATCH_BYTES
    assert g.gdr_chunk_fwd_noalloc(big, q, k, None, v, a, b, None, None, o, st, 0) == g.GDR_ETOOLARGE
    chan = _desc(g, B=1, H=1, T=64 * 1088, alpha_mode=g.GDR_ALPHA_CHANNEL)
    assert g.gdr_chunk_fwd_noalloc(chan, q, k, None, v, a, b, None, None, o, st, 0) == g.GDR_ETOOLARGE
    assert g.gdr_chunk_fwd_noalloc(_desc(g, dk=12), q, k, None, v, a, b, None, None, o, st, 0) == g.GDR_EUNSUPPORTED
    fits = _desc(g, B=4, H=16, T=4096)           # the headline batch: 105 MB of records
    assert g.gdr_chunk_fwd_workspace_size(fits) <= g.GDR_NOALLOC_SCRATCH_BYTES
    assert "scratch" in g.gdr_status_string(g.GDR_ETOOLARGE)
