"""The oracle's mirrors of the library's entry points (gdr_ref_chunk_fwd,
gdr_ref_decode_step: the library's argument lists, host pointers, stored dtypes in,
fp64 inside) equal the fp64 oracle entry points they wrap, with o rounded the way
the input generator stores values (fp64 -> fp32 -> bf16, nearest-even) and the
states in fp32."""
import ctypes

import numpy as np
import pytest

import gdr_inputs as gi
import oracle

DT = {gi.BF16: 0, gi.F32: 1}


class RefDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "H", "dk", "dv", "chunk", "io_dtype", "gate_dtype", "alpha_mode", "beta_mode", "flags")]


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _lib():
    return oracle._load()


CASES = [
    gi.GDN_PREFILL.scaled(name="mirror_gdn", B=2, T=37, H=3, dk=16, dv=24, chunk=16, s0_std=0.1, seed=71),
    gi.KDA_FG2PLUS_PREFILL.scaled(name="mirror_kda", B=1, T=20, H=2, dk=16, dv=16, chunk=16, seed=72),
    gi.OSDN_LONG_PREFILL.scaled(name="mirror_osdn", B=1, T=21, H=2, dk=8, dv=8, chunk=16, io=gi.F32,
                                gate=gi.BF16, seed=73),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_chunk_fwd_mirror_equals_the_fp64_oracle(w):
    x = gi.make_prefill(w)
    d = RefDesc(B=w.B, T=w.T, H=w.H, dk=w.dk, dv=w.dv, chunk=w.chunk, io_dtype=DT[w.io], gate_dtype=DT[w.gate],
                alpha_mode=w.alpha_mode, beta_mode=w.beta_mode, flags=0)
    es = np.uint16 if w.io == gi.BF16 else np.float32
    o = np.zeros((w.B, w.T, w.H, w.dv), dtype=es)
    ST = np.zeros((w.B, w.H, w.dk, w.dv), dtype=np.float32)
    rc = _lib().gdr_ref_chunk_fwd(ctypes.byref(d), _p(x["q"]), _p(x["k"]), _p(x["k_w"]), _p(x["v"]), _p(x["alpha"]),
                                  _p(x["beta_k"]), _p(x["beta_v"]), _p(x["S0"]), _p(o), _p(ST), None, 0, None)
    assert rc == 0
    f = gi.prefill_f64(w, x)
    o64, S64 = oracle.forward(f["q"], f["k"], f["v"], f["alpha"], f["beta_k"], k_w=f["k_w"], beta_v=f["beta_v"],
                              S0=f["S0"])
    np.testing.assert_array_equal(o, gi.store(o64, w.io))
    np.testing.assert_array_equal(ST, S64.astype(np.float32))


def test_chunk_fwd_mirror_without_tokens_copies_the_state():
    w = CASES[0].scaled(T=0)
    S0 = np.random.default_rng(5).standard_normal((w.B, w.H, w.dk, w.dv)).astype(np.float32)
    ST = np.zeros_like(S0)
    d = RefDesc(B=w.B, T=0, H=w.H, dk=w.dk, dv=w.dv, chunk=16, io_dtype=0, gate_dtype=1, alpha_mode=0,
                beta_mode=0, flags=0)
    assert _lib().gdr_ref_chunk_fwd(ctypes.byref(d), None, None, None, None, None, None, None, _p(S0), None,
                                    _p(ST), None, 0, None) == 0
    np.testing.assert_array_equal(ST, S0)


def test_decode_mirror_equals_the_fp64_step():
    w = gi.DECODE_B512.scaled(name="mirror_dec", B=3, H=2, dk=16, dv=8, steps=4, seed=74)
    x = gi.make_decode(w)
    f = gi.decode_f64(w, x)
    S = x["S"].copy()
    S64 = f["S"].copy()
    d = RefDesc(B=w.B, T=0, H=w.H, dk=w.dk, dv=w.dv, chunk=64, io_dtype=0, gate_dtype=0, alpha_mode=0, beta_mode=0,
                flags=0)
    for t in range(w.steps):
        o = np.zeros((w.B, w.H, w.dv), dtype=np.uint16)
        assert _lib().gdr_ref_decode_step(ctypes.byref(d), _p(np.ascontiguousarray(x["q"][t])),
                                          _p(np.ascontiguousarray(x["k"][t])), None,
                                          _p(np.ascontiguousarray(x["v"][t])),
                                          _p(np.ascontiguousarray(x["alpha"][t])),
                                          _p(np.ascontiguousarray(x["beta_k"][t])), None, _p(S), _p(o), None) == 0
        o64, S64 = oracle.decode_step(S64, f["q"][t], f["k"][t], f["v"][t], f["alpha"][t], f["beta_k"][t])
        np.testing.assert_array_equal(o, gi.store(o64, gi.BF16))
        # the mirror keeps its state in fp32 between calls, as the library does
        S64 = S.astype(np.float64)


@pytest.mark.parametrize("field,value", [("flags", 0x10), ("io_dtype", 3), ("beta_mode", 5), ("dk", 0), ("B", -1)])
def test_mirrors_reject_bad_descriptors(field, value):
    kw = dict(B=1, T=4, H=1, dk=8, dv=8, chunk=16, io_dtype=1, gate_dtype=1, alpha_mode=0, beta_mode=0, flags=0)
    kw[field] = value
    d = RefDesc(**kw)
    a = np.zeros(64, dtype=np.float32)
    assert _lib().gdr_ref_chunk_fwd(ctypes.byref(d), *[_p(a)] * 7, None, _p(a), _p(a), None, 0, None) == -1
    assert _lib().gdr_ref_decode_step(ctypes.byref(d), *[_p(a)] * 7, _p(a), _p(a), None) == -1
