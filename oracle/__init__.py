"""fp64 CPU oracle for the gated delta-rule recurrence -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and it shares no code with the GPU library.

Contents:
  * ``forward`` / ``decode_step``: ctypes front-end of ``gdr_ref.c``, the plain
    sequential recurrence in double precision (see that file's header for the
    per-variant formulas and their sources).
  * ``chunked``: an independent NumPy evaluation of the same recurrence in the
    chunkwise WY / UT-transform form, used on tiny inputs to pin the sequential
    oracle (and the chunked algebra) against each other.
  * ``osdn_precond``: OSDN phase 1, the preconditioner scan over the key stream
    (write keys, final preconditioner, geometric-mean loss ratio q_geo).
  * ``sdm``: Sparse Delta Memory -- product-key slot selection (all slot scores
    ranked directly), per-slot gated delta writes and the weighted sparse read.
  * ``dmem``: delta-mem write granularities -- one write per token (TSW) or per
    segment with the segment's mean key and value (SSW), and J sub-states per group
    of heads with summed reads (MSW), reads taken before the write, plain fp64.
  * ``memcache``: Memory Caching -- the state after every segment (the sequential
    run, one segment at a time) and the residual / gated read-out over those
    cached states, plain fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_ref.c")
_LIB = os.path.join(_HERE, "libgdr_ref.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gdr_ref.c with gcc into oracle/libgdr_ref.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.gdr_ref_forward.argtypes = [ctypes.c_int] * 7 + [dp] * 10 + [ip, ctypes.c_int, ctypes.c_int]
    lib.gdr_ref_forward.restype = ctypes.c_int
    lib.gdr_ref_decode_step_f64.argtypes = [ctypes.c_int] * 6 + [dp] * 9 + [ctypes.c_int]
    lib.gdr_ref_decode_step_f64.restype = ctypes.c_int
    vp = ctypes.c_void_p
    lib.gdr_ref_chunk_fwd.argtypes = [vp] * 12 + [ctypes.c_size_t, vp]
    lib.gdr_ref_chunk_fwd.restype = ctypes.c_int
    lib.gdr_ref_decode_step.argtypes = [vp] * 11
    lib.gdr_ref_decode_step.restype = ctypes.c_int
    lib.gdr_ref_dmem_step.argtypes = [ctypes.c_int] * 4 + [dp] * 7 + [ctypes.c_int]
    lib.gdr_ref_dmem_step.restype = ctypes.c_int
    lib.gdr_ref_osdn_precond.argtypes = [ctypes.c_int] * 4 + [dp] * 3 + [ctypes.c_double] + [dp] * 4 + [ctypes.c_int]
    lib.gdr_ref_osdn_precond.restype = ctypes.c_int
    lib.gdr_ref_max_threads.argtypes = []
    lib.gdr_ref_max_threads.restype = ctypes.c_int
    return lib


def build_variant(src_text: str, path: str) -> str:
    """Compile an edited copy of the oracle source to ``path`` (used by the
    mutation tests, which plant mistakes in a temporary copy)."""
    csrc = path + ".c"
    with open(csrc, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", csrc, "-o", path, "-lm"],
                   check=True)
    return path


class use_library:
    """Context manager: route this module's calls to another compiled oracle."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        _load()
        self._saved = _lib
        _lib = _bind(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def source() -> str:
    with open(_SRC) as f:
        return f.read()


def _dp(x: Optional[np.ndarray]):
    if x is None:
        return None
    assert x.dtype == np.float64 and x.flags["C_CONTIGUOUS"]
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _c64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def max_threads() -> int:
    return int(_load().gdr_ref_max_threads())


def forward(q, k, v, alpha, beta_k, *, k_w=None, beta_v=None, S0=None, alpha_mode=None,
            beta_mode=None, heads: Optional[Sequence[int]] = None, nthreads: int = 0):
    """Sequential fp64 forward.  Arrays use the [B, T, H, D] prefill layout.

    Returns (o [B, T, H, dv], ST [B, H, dk, dv]) as float64.  When ``heads``
    lists (b*H + h) indices, only those pairs are computed; the other entries
    of o and ST are NaN.
    """
    q, k, v, alpha, beta_k = map(_c64, (q, k, v, alpha, beta_k))
    k_w, beta_v, S0 = map(_c64, (k_w, beta_v, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if alpha_mode is None:
        alpha_mode = 1 if alpha.ndim == 4 else 0
    if beta_mode is None:
        beta_mode = 0 if beta_k.ndim == 3 else (2 if beta_v is not None else 1)
    o = np.full((B, T, H, dv), np.nan)
    ST = np.full((B, H, dk, dv), np.nan)
    hp, nh = None, 0
    if heads is not None:
        harr = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
        hp, nh = harr.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), int(harr.size)
    rc = _load().gdr_ref_forward(B, T, H, dk, dv, alpha_mode, beta_mode, _dp(q), _dp(k), _dp(k_w),
                                 _dp(v), _dp(alpha), _dp(beta_k), _dp(beta_v), _dp(S0), _dp(o),
                                 _dp(ST), hp, nh, nthreads)
    if rc != 0:
        raise ValueError(f"gdr_ref_forward rejected its arguments (status {rc})")
    return o, ST


def decode_step(S, q, k, v, alpha, beta_k, *, k_w=None, beta_v=None, alpha_mode=None,
                beta_mode=None, nthreads: int = 0):
    """One fp64 step on state S [B, H, dk, dv]; returns (o [B, H, dv], S_new)."""
    S = np.array(S, dtype=np.float64, order="C", copy=True)
    q, k, v, alpha, beta_k = map(_c64, (q, k, v, alpha, beta_k))
    k_w, beta_v = map(_c64, (k_w, beta_v))
    B, H, dk = q.shape
    dv = v.shape[-1]
    if alpha_mode is None:
        alpha_mode = 1 if alpha.ndim == 3 else 0
    if beta_mode is None:
        beta_mode = 0 if beta_k.ndim == 2 else (2 if beta_v is not None else 1)
    o = np.empty((B, H, dv))
    rc = _load().gdr_ref_decode_step_f64(B, H, dk, dv, alpha_mode, beta_mode, _dp(q), _dp(k), _dp(k_w),
                                     _dp(v), _dp(alpha), _dp(beta_k), _dp(beta_v), _dp(S), _dp(o),
                                     nthreads)
    if rc != 0:
        raise ValueError(f"gdr_ref_decode_step_f64 rejected its arguments (status {rc})")
    return o, S


def dmem_step(M, q, k, v, lam, beta, nthreads: int = 0):
    """One delta-mem step in the page's orientation: M [B, H, dv, dk] (predicts M k),
    lam, beta [B, H]; returns (r [B, H, dv] read before the write, M_new)."""
    M = np.array(M, dtype=np.float64, order="C", copy=True)
    q, k, v, lam, beta = map(_c64, (q, k, v, lam, beta))
    B, H, dk = q.shape
    dv = v.shape[-1]
    r = np.empty((B, H, dv))
    rc = _load().gdr_ref_dmem_step(B, H, dk, dv, _dp(q), _dp(k), _dp(v), _dp(lam), _dp(beta), _dp(M), _dp(r),
                                   nthreads)
    if rc != 0:
        raise ValueError(f"gdr_ref_dmem_step rejected its arguments (status {rc})")
    return r, M


def osdn_precond(k, beta, eta: float, *, r=None, d0=None, nthreads: int = 0):
    """OSDN phase 1 in fp64: k [B, T, H, dk], beta [B, T, H], r [B, T, H] or None
    (retention 1), d0 [B, H, dk] or None (ones).  Returns (kw [B, T, H, dk],
    dT [B, H, dk], qgeo [B, H])."""
    k, beta, r, d0 = map(_c64, (k, beta, r, d0))
    B, T, H, dk = k.shape
    kw = np.empty((B, T, H, dk))
    dT = np.empty((B, H, dk))
    qg = np.empty((B, H))
    rc = _load().gdr_ref_osdn_precond(B, T, H, dk, _dp(k), _dp(beta), _dp(r), float(eta), _dp(d0), _dp(kw),
                                      _dp(dT), _dp(qg), nthreads)
    if rc != 0:
        raise ValueError(f"gdr_ref_osdn_precond rejected its arguments (status {rc})")
    return kw, dT, qg


def rel_l2(x, ref) -> float:
    """||x - ref||_2 / ||ref||_2 over the whole array, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.sqrt(np.sum(ref * ref)))
    num = float(np.sqrt(np.sum((x - ref) ** 2)))
    return num / den if den > 0 else num
