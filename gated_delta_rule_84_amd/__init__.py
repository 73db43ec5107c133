"""Python binding of the gated delta-rule HIP library (libgdr.so, include/gdr.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C-ABI.  PyTorch supplies device memory and the current
stream.  The functions with the C names (``gdr_chunk_fwd``, ``gdr_decode_step``,
``gdr_chunk_fwd_workspace_size``, ``gdr_chunk_fwd_path``, ``gdr_status_string``)
take a ``Desc`` and tensors (or None) and return the C status code;
``chunk_fwd`` and ``decode_step`` allocate outputs and raise on a non-OK
status.

The library must have been built (``python gated_delta_rule_84_amd/build.py``);
importing this package without it raises ImportError.  There is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # loads the HIP runtime the library binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdr.so")

GDR_OK, GDR_EINVAL, GDR_EUNSUPPORTED, GDR_EWORKSPACE, GDR_EHIP, GDR_ETOOLARGE = 0, -1, -2, -3, -4, -5
GDR_NOALLOC_SCRATCH_BYTES = 128 << 20
GDR_BF16, GDR_F32 = 0, 1
GDR_ALPHA_SCALAR, GDR_ALPHA_CHANNEL = 0, 1
GDR_BETA_SCALAR, GDR_BETA_SHARED, GDR_BETA_KV = 0, 1, 2
GDR_FLAG_READ_BEFORE_WRITE = 0x10
GDR_FLAG_UNDECAYED_PREDICTION = 0x20
PATH_MFMA, PATH_VALU = 1, 2


class Desc(ctypes.Structure):
    """Mirror of ``gdr_desc``."""

    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "T", "H", "dk", "dv", "chunk", "io_dtype", "gate_dtype", "alpha_mode",
                 "beta_mode", "flags")]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python gated_delta_rule_84_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)
_vp = ctypes.c_void_p
_dp = ctypes.POINTER(Desc)
_lib.gdr_chunk_fwd_workspace_size.argtypes = [_dp]
_lib.gdr_chunk_fwd_workspace_size.restype = ctypes.c_size_t
_lib.gdr_chunk_fwd.argtypes = [_dp] + [_vp] * 10 + [_vp, ctypes.c_size_t, _vp]
_lib.gdr_chunk_fwd.restype = ctypes.c_int
_lib.gdr_chunk_fwd_ctx.argtypes = [_dp] + [_vp] * 10 + [_vp, ctypes.c_size_t, _vp, _vp]
_lib.gdr_chunk_fwd_ctx.restype = ctypes.c_int
_lib.gdr_chunk_fwd_noalloc.argtypes = [_dp] + [_vp] * 10 + [_vp]
_lib.gdr_chunk_fwd_noalloc.restype = ctypes.c_int
_lib.gdr_decode_step.argtypes = [_dp] + [_vp] * 9 + [_vp]
_lib.gdr_decode_step.restype = ctypes.c_int
_lib.gdr_chunk_fwd_path.argtypes = [_dp]
_lib.gdr_chunk_fwd_path.restype = ctypes.c_int
_lib.gdr_status_string.argtypes = [ctypes.c_int]
_lib.gdr_status_string.restype = ctypes.c_char_p
_lib.gdr_version.argtypes = []
_lib.gdr_version.restype = ctypes.c_int
_lib.gdr_chunk_fwd_ckpt.argtypes = [_dp] + [_vp] * 10 + [ctypes.c_int32, _vp, _vp, ctypes.c_size_t, _vp]
_lib.gdr_chunk_fwd_ckpt.restype = ctypes.c_int
_lib.gdr_mc_readout_workspace_size.argtypes = [_dp, ctypes.c_int32]
_lib.gdr_mc_readout_workspace_size.restype = ctypes.c_size_t
_lib.gdr_mc_readout.argtypes = [_dp, _vp, _vp, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp, _vp,
                                ctypes.c_size_t, _vp]
_lib.gdr_mc_readout.restype = ctypes.c_int
_lib.gdr_osdn_precond_workspace_size.argtypes = [_dp]
_lib.gdr_osdn_precond_workspace_size.restype = ctypes.c_size_t
_lib.gdr_osdn_precond.argtypes = [_dp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp,
                                  _vp]
_lib.gdr_osdn_precond.restype = ctypes.c_int
_lib.gdr_sdm_workspace_size.argtypes = [_dp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
_lib.gdr_sdm_workspace_size.restype = ctypes.c_size_t
_lib.gdr_sdm_fwd.argtypes = [_dp] + [ctypes.c_int32] * 3 + [_vp] * 10 + [ctypes.c_size_t, _vp, _vp]
_lib.gdr_sdm_fwd.restype = ctypes.c_int
_lib.gdr_dmem_fwd.argtypes = [_dp, ctypes.c_int32] + [_vp] * 8 + [_vp]
_lib.gdr_dmem_fwd.restype = ctypes.c_int
_lib.gdr_context_create.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
_lib.gdr_context_create.restype = ctypes.c_int
_lib.gdr_context_destroy.argtypes = [_vp]
_lib.gdr_context_destroy.restype = ctypes.c_int

EXPORTED = ("gdr_chunk_fwd_workspace_size", "gdr_chunk_fwd", "gdr_decode_step", "gdr_chunk_fwd_path",
            "gdr_status_string", "gdr_version", "gdr_chunk_fwd_ckpt", "gdr_mc_readout_workspace_size",
            "gdr_mc_readout", "gdr_osdn_precond_workspace_size", "gdr_osdn_precond",
            "gdr_sdm_workspace_size", "gdr_sdm_fwd", "gdr_context_create", "gdr_context_destroy",
            "gdr_chunk_fwd_noalloc", "gdr_dmem_fwd", "gdr_chunk_fwd_ctx")


class GdrError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {gdr_status_string(status)} ({status})")
        self.status = status


def _ptr(t: Optional[torch.Tensor]):
    """Device address of a tensor for the library, which reads every tensor as dense
    row-major device memory: a view with other strides or a host tensor is refused
    here (ValueError) instead of being read wrongly or faulting on the device."""
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        if not t.is_contiguous():
            raise ValueError("expected a contiguous (dense row-major) tensor")
        if t.device.type != "cuda":
            raise ValueError(f"expected a device tensor, got one on {t.device}")
    return ctypes.c_void_p(t.data_ptr())


_TORCH_DTYPE = {GDR_BF16: torch.bfloat16, GDR_F32: torch.float32}


def _check_all(specs) -> None:
    """The library trusts the descriptor: every tensor handed to it must hold exactly
    the element count and dtype the descriptor implies, on the current device, else
    ValueError before the call (a short or mistyped buffer would be read or written
    past its end on the device).  `specs` is a list of (name, tensor or None, count,
    dtype); sizes and dtypes are checked for all before devices.  An object that is not
    a tensor but has data_ptr() is a raw device address: it is passed as it is, and
    the caller answers for its size."""
    specs = [s for s in specs if isinstance(s[1], torch.Tensor)]
    for name, t, count, dtype in specs:
        if t.dtype != dtype:
            raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
        if t.numel() != count:
            raise ValueError(f"{name}: expected {count} elements for this descriptor, got {t.numel()} "
                             f"(shape {tuple(t.shape)})")
    for name, t, _, _ in specs:
        if t.device.type != "cuda":
            raise ValueError(f"{name}: expected a device tensor, got one on {t.device}")
        if t.device.index is not None and t.device.index != torch.cuda.current_device():
            raise ValueError(f"{name}: tensor on {t.device}, current device is cuda:{torch.cuda.current_device()}")


def _check_workspace(workspace, workspace_bytes: int) -> None:
    if workspace is None or not isinstance(workspace, torch.Tensor):
        return
    have = workspace.numel() * workspace.element_size()
    if int(workspace_bytes) > have:
        raise ValueError(f"workspace_bytes = {int(workspace_bytes)} exceeds the workspace tensor ({have} bytes)")


def _io(desc: Desc):
    if desc.io_dtype not in _TORCH_DTYPE or desc.gate_dtype not in _TORCH_DTYPE:
        return None, None
    return _TORCH_DTYPE[desc.io_dtype], _TORCH_DTYPE[desc.gate_dtype]


def _prefill_specs(desc: Desc, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST) -> list:
    io, gt = _io(desc)
    if io is None or min(desc.B, desc.T, desc.H, desc.dk, desc.dv) < 0:
        return []  # the library rejects the descriptor itself
    n = desc.B * desc.T * desc.H
    st = desc.B * desc.H * desc.dk * desc.dv
    return [("q", q, n * desc.dk, io), ("k", k, n * desc.dk, io), ("k_w", k_w, n * desc.dk, io),
            ("v", v, n * desc.dv, io), ("o", o, n * desc.dv, io),
            ("alpha", alpha, n * (desc.dk if desc.alpha_mode == GDR_ALPHA_CHANNEL else 1), gt),
            ("beta_k", beta_k, n * (desc.dk if desc.beta_mode in (GDR_BETA_SHARED, GDR_BETA_KV) else 1), gt),
            ("beta_v", beta_v, n * desc.dv, gt), ("S0", S0, st, torch.float32), ("ST", ST, st, torch.float32)]


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# ---------------------------------------------------------------------------
# the C entry points, one to one
# ---------------------------------------------------------------------------

def gdr_context_create() -> ctypes.c_void_p:
    """A caller-owned execution context (a second stream and events) on the current
    device; raises on failure.  Release it with gdr_context_destroy."""
    h = ctypes.c_void_p()
    rc = int(_lib.gdr_context_create(ctypes.byref(h)))
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_context_create")
    return h


def gdr_context_destroy(ctx) -> int:
    return int(_lib.gdr_context_destroy(ctx))


class Context:
    """Owns one gdr_context; usable as a context manager.  Pass it (or its `handle`)
    as `ctx` to osdn_precond / sdm_fwd to overlap their parallel passes on the
    context's second stream."""

    def __init__(self):
        self.handle = gdr_context_create()

    def close(self):
        if self.handle is not None:
            rc = gdr_context_destroy(self.handle)
            self.handle = None
            if rc != GDR_OK:
                raise GdrError(rc, "gdr_context_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _ctx(ctx):
    if ctx is None:
        return None
    return ctx.handle if isinstance(ctx, Context) else ctx


def gdr_version() -> int:
    return int(_lib.gdr_version())


def gdr_status_string(status: int) -> str:
    return _lib.gdr_status_string(int(status)).decode()


def gdr_chunk_fwd_workspace_size(desc: Desc) -> int:
    return int(_lib.gdr_chunk_fwd_workspace_size(ctypes.byref(desc)))


def gdr_chunk_fwd_path(desc: Desc) -> int:
    return int(_lib.gdr_chunk_fwd_path(ctypes.byref(desc)))


def gdr_chunk_fwd(desc: Desc, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST, workspace,
                  workspace_bytes: int, stream=None) -> int:
    _check_all(_prefill_specs(desc, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST))
    _check_workspace(workspace, workspace_bytes)
    return int(_lib.gdr_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(k_w), _ptr(v), _ptr(alpha),
                                  _ptr(beta_k), _ptr(beta_v), _ptr(S0), _ptr(o), _ptr(ST),
                                  _ptr(workspace), int(workspace_bytes), _stream(stream)))


def gdr_chunk_fwd_ctx(desc: Desc, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST, workspace,
                      workspace_bytes: int, ctx, stream=None) -> int:
    _check_all(_prefill_specs(desc, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST))
    _check_workspace(workspace, workspace_bytes)
    return int(_lib.gdr_chunk_fwd_ctx(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(k_w), _ptr(v), _ptr(alpha),
                                      _ptr(beta_k), _ptr(beta_v), _ptr(S0), _ptr(o), _ptr(ST),
                                      _ptr(workspace), int(workspace_bytes), _ctx(ctx), _stream(stream)))


def gdr_chunk_fwd_noalloc(desc: Desc, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST, stream=None) -> int:
    _check_all(_prefill_specs(desc, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST))
    return int(_lib.gdr_chunk_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(k_w), _ptr(v), _ptr(alpha),
                                          _ptr(beta_k), _ptr(beta_v), _ptr(S0), _ptr(o), _ptr(ST), _stream(stream)))


def gdr_chunk_fwd_ckpt(desc: Desc, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST, seg_len: int, ckpt,
                       workspace, workspace_bytes: int, stream=None) -> int:
    specs = _prefill_specs(desc, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST)
    if specs and int(seg_len) > 0:
        specs.append(("ckpt", ckpt, desc.B * desc.H * (desc.T // int(seg_len)) * desc.dk * desc.dv, torch.float32))
    _check_all(specs)
    _check_workspace(workspace, workspace_bytes)
    return int(_lib.gdr_chunk_fwd_ckpt(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(k_w), _ptr(v), _ptr(alpha),
                                       _ptr(beta_k), _ptr(beta_v), _ptr(S0), _ptr(o), _ptr(ST), int(seg_len),
                                       _ptr(ckpt), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def gdr_mc_readout_workspace_size(desc: Desc, n_ckpt: int) -> int:
    return int(_lib.gdr_mc_readout_workspace_size(ctypes.byref(desc), int(n_ckpt)))


def gdr_mc_readout(desc: Desc, q, ckpt, n_ckpt: int, seg_len: int, gates, o_in, o_out, workspace,
                   workspace_bytes: int, stream=None) -> int:
    io, _ = _io(desc)
    if io is not None and min(desc.B, desc.T, desc.H, desc.dk, desc.dv, int(n_ckpt)) >= 0:
        n = desc.B * desc.T * desc.H
        _check_all([("q", q, n * desc.dk, io),
                    ("ckpt", ckpt, desc.B * desc.H * int(n_ckpt) * desc.dk * desc.dv, torch.float32),
                    ("gates", gates, n * int(n_ckpt), torch.float32), ("o_in", o_in, n * desc.dv, io),
                    ("o_out", o_out, n * desc.dv, io)])
    _check_workspace(workspace, workspace_bytes)
    return int(_lib.gdr_mc_readout(ctypes.byref(desc), _ptr(q), _ptr(ckpt), int(n_ckpt), int(seg_len),
                                   _ptr(gates), _ptr(o_in), _ptr(o_out), _ptr(workspace), int(workspace_bytes),
                                   _stream(stream)))


def gdr_osdn_precond_workspace_size(desc: Desc) -> int:
    return int(_lib.gdr_osdn_precond_workspace_size(ctypes.byref(desc)))


def gdr_osdn_precond(desc: Desc, k, beta, r, eta: float, d0, k_w, dT, qgeo, workspace, workspace_bytes: int,
                     ctx=None, stream=None) -> int:
    io, gt = _io(desc)
    if io is not None and min(desc.B, desc.T, desc.H, desc.dk) >= 0:
        n = desc.B * desc.T * desc.H
        _check_all([("k", k, n * desc.dk, io), ("k_w", k_w, n * desc.dk, io), ("beta", beta, n, gt),
                    ("r", r, n, gt), ("d0", d0, desc.B * desc.H * desc.dk, torch.float32),
                    ("dT", dT, desc.B * desc.H * desc.dk, torch.float32),
                    ("qgeo", qgeo, desc.B * desc.H, torch.float32)])
    _check_workspace(workspace, workspace_bytes)
    return int(_lib.gdr_osdn_precond(ctypes.byref(desc), _ptr(k), _ptr(beta), _ptr(r), float(eta), _ptr(d0), _ptr(k_w),
                                     _ptr(dT), _ptr(qgeo), _ptr(workspace), int(workspace_bytes), _ctx(ctx),
                                     _stream(stream)))


def gdr_sdm_workspace_size(desc: Desc, n: int, W: int, R: int) -> int:
    return int(_lib.gdr_sdm_workspace_size(ctypes.byref(desc), int(n), int(W), int(R)))


def gdr_sdm_fwd(desc: Desc, n: int, W: int, R: int, ks, qs, v, alpha, beta, M, o, w_slots, r_slots, workspace,
                workspace_bytes: int, ctx=None, stream=None) -> int:
    io, gt = _io(desc)
    if io is not None and min(desc.B, desc.T, desc.H, desc.dv, int(n), int(W), int(R)) >= 0:
        nt = desc.B * desc.T * desc.H
        _check_all([("ks", ks, nt * 2 * int(n), torch.float32), ("qs", qs, nt * 2 * int(n), torch.float32),
                    ("v", v, nt * desc.dv, io), ("o", o, nt * desc.dv, io), ("alpha", alpha, nt, gt),
                    ("beta", beta, nt, gt), ("M", M, desc.B * desc.H * int(n) * int(n) * desc.dv, torch.float32),
                    ("w_slots", w_slots, nt * int(W), torch.int32), ("r_slots", r_slots, nt * int(R), torch.int32)])
    _check_workspace(workspace, workspace_bytes)
    return int(_lib.gdr_sdm_fwd(ctypes.byref(desc), int(n), int(W), int(R), _ptr(ks), _ptr(qs), _ptr(v), _ptr(alpha),
                                _ptr(beta), _ptr(M), _ptr(o), _ptr(w_slots), _ptr(r_slots), _ptr(workspace),
                                int(workspace_bytes), _ctx(ctx), _stream(stream)))


def gdr_dmem_fwd(desc: Desc, J: int, q, k, v, lam, beta, seg_end, M, out, stream=None) -> int:
    io, gt = _io(desc)
    if io is not None and min(desc.B, desc.T, desc.H, desc.dk) >= 0 and int(J) >= 1 and desc.H % int(J) == 0:
        nt = desc.B * desc.T * desc.H
        _check_all([("q", q, nt * desc.dk, io), ("k", k, nt * desc.dk, io), ("v", v, nt * desc.dk, io),
                    ("lam", lam, nt, gt), ("beta", beta, nt, gt), ("seg_end", seg_end, desc.B * desc.T, torch.uint8),
                    ("M", M, desc.B * desc.H * desc.dk * desc.dk, torch.float32),
                    ("out", out, nt // int(J) * desc.dk, io)])
    return int(_lib.gdr_dmem_fwd(ctypes.byref(desc), int(J), _ptr(q), _ptr(k), _ptr(v), _ptr(lam), _ptr(beta),
                                 _ptr(seg_end), _ptr(M), _ptr(out), _stream(stream)))


def gdr_decode_step(desc: Desc, q, k, k_w, v, alpha, beta_k, beta_v, S, o, stream=None) -> int:
    io, gt = _io(desc)
    if io is not None and min(desc.B, desc.H, desc.dk, desc.dv) >= 0:
        n = desc.B * desc.H
        _check_all([("q", q, n * desc.dk, io), ("k", k, n * desc.dk, io), ("k_w", k_w, n * desc.dk, io),
                    ("v", v, n * desc.dv, io), ("o", o, n * desc.dv, io),
                    ("alpha", alpha, n * (desc.dk if desc.alpha_mode == GDR_ALPHA_CHANNEL else 1), gt),
                    ("beta_k", beta_k, n * (desc.dk if desc.beta_mode in (GDR_BETA_SHARED, GDR_BETA_KV) else 1), gt),
                    ("beta_v", beta_v, n * desc.dv, gt), ("S", S, n * desc.dk * desc.dv, torch.float32)])
    return int(_lib.gdr_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(k_w), _ptr(v), _ptr(alpha),
                                    _ptr(beta_k), _ptr(beta_v), _ptr(S), _ptr(o), _stream(stream)))


# ---------------------------------------------------------------------------
# convenience wrappers (allocate outputs, raise on error)
# ---------------------------------------------------------------------------

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDR_BF16
    if t.dtype == torch.float32:
        return GDR_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def make_desc(q, v, alpha, beta_k, beta_v=None, *, chunk=64, decode=False, flags=0) -> Desc:
    """Descriptor from tensor shapes: prefill q [B, T, H, dk], decode q [B, H, dk]."""
    if decode:
        B, H, dk = q.shape
        T = 1
        alpha_ch = alpha.dim() == 3
        beta_vec = beta_k.dim() == 3
    else:
        B, T, H, dk = q.shape
        alpha_ch = alpha.dim() == 4
        beta_vec = beta_k.dim() == 4
    beta_mode = GDR_BETA_KV if beta_v is not None else (GDR_BETA_SHARED if beta_vec else GDR_BETA_SCALAR)
    return Desc(B=B, T=T, H=H, dk=dk, dv=v.shape[-1], chunk=chunk, io_dtype=_dtype_code(q),
                gate_dtype=_dtype_code(alpha), alpha_mode=GDR_ALPHA_CHANNEL if alpha_ch else GDR_ALPHA_SCALAR,
                beta_mode=beta_mode, flags=flags)


def chunk_fwd(q, k, v, alpha, beta_k, *, k_w=None, beta_v=None, S0=None, chunk=64, want_state=True,
              out=None, final_state=None, workspace=None, ctx=None, stream=None):
    """Prefill.  Returns (o [B, T, H, dv] in q's dtype, ST [B, H, dk, dv] fp32 or None).
    With an execution context `ctx` the call goes through gdr_chunk_fwd_ctx."""
    desc = make_desc(q, v, alpha, beta_k, beta_v, chunk=chunk)
    o = out if out is not None else torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=q.dtype, device=q.device)
    ST = final_state
    if ST is None and want_state:
        ST = torch.empty((desc.B, desc.H, desc.dk, desc.dv), dtype=torch.float32, device=q.device)
    need = gdr_chunk_fwd_workspace_size(desc)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if ctx is None:
        rc = gdr_chunk_fwd(desc, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST, workspace, wbytes, stream)
    else:
        rc = gdr_chunk_fwd_ctx(desc, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST, workspace, wbytes, ctx, stream)
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_chunk_fwd" if ctx is None else "gdr_chunk_fwd_ctx")
    return o, ST


def chunk_fwd_ckpt(q, k, v, alpha, beta_k, seg_len, *, k_w=None, beta_v=None, S0=None, chunk=64,
                   want_state=True, workspace=None, stream=None):
    """Prefill that also keeps the state after every complete segment of seg_len tokens.
    Returns (o, ST or None, ckpt [B, H, floor(T / seg_len), dk, dv] fp32)."""
    desc = make_desc(q, v, alpha, beta_k, beta_v, chunk=chunk)
    o = torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=q.dtype, device=q.device)
    ST = torch.empty((desc.B, desc.H, desc.dk, desc.dv), dtype=torch.float32, device=q.device) if want_state else None
    n = desc.T // int(seg_len) if seg_len > 0 else 0
    ckpt = torch.empty((desc.B, desc.H, n, desc.dk, desc.dv), dtype=torch.float32, device=q.device)
    need = gdr_chunk_fwd_workspace_size(desc)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = gdr_chunk_fwd_ckpt(desc, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST, seg_len,
                            ckpt if n > 0 else None, workspace, wbytes, stream)
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_chunk_fwd_ckpt")
    return o, ST, ckpt


def mc_readout(q, ckpt, seg_len, *, gates=None, o_in=None, out=None, workspace=None, stream=None):
    """o_out[t] = o_in[t] + sum_{s < min(t // seg_len, N)} g[t, s] M_s^T q[t] (g = 1 without gates).
    q [B, T, H, 128] bf16, ckpt [B, H, N, 128, 128] fp32, gates [B, T, H, N] fp32 or None."""
    B, T, H, dk = q.shape
    n = ckpt.shape[2]
    desc = Desc(B=B, T=T, H=H, dk=dk, dv=ckpt.shape[-1], chunk=64, io_dtype=_dtype_code(q), gate_dtype=GDR_F32,
                alpha_mode=0, beta_mode=0, flags=0)
    o = out if out is not None else torch.empty(q.shape[:-1] + (ckpt.shape[-1],), dtype=q.dtype, device=q.device)
    need = gdr_mc_readout_workspace_size(desc, n)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = gdr_mc_readout(desc, q, ckpt, n, seg_len, gates, o_in, o, workspace, wbytes, stream)
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_mc_readout")
    return o


def osdn_precond(k, beta, eta, *, r=None, d0=None, workspace=None, ctx=None, stream=None):
    """OSDN phase 1.  k [B, T, H, dk] (bf16 or fp32), beta and r [B, T, H].
    Returns (k_w like k, dT [B, H, dk] fp32, qgeo [B, H] fp32)."""
    B, T, H, dk = k.shape
    desc = Desc(B=B, T=T, H=H, dk=dk, dv=dk, chunk=64, io_dtype=_dtype_code(k), gate_dtype=_dtype_code(beta),
                alpha_mode=0, beta_mode=0, flags=0)
    kw = torch.empty_like(k)
    dT = torch.empty((B, H, dk), dtype=torch.float32, device=k.device)
    qg = torch.empty((B, H), dtype=torch.float32, device=k.device)
    need = gdr_osdn_precond_workspace_size(desc)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=k.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = gdr_osdn_precond(desc, k, beta, r, eta, d0, kw, dT, qg, workspace, wbytes, ctx, stream)
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_osdn_precond")
    return kw, dT, qg


def sdm_fwd(M, ks, qs, v, alpha, beta, W, R, *, want_slots=False, workspace=None, ctx=None, stream=None):
    """Sparse Delta Memory over T tokens.  M [B, H, n * n, dv] fp32 is updated in place;
    ks, qs [B, T, H, 2, n] fp32; v [B, T, H, dv].  Returns o (and the selected write /
    read slots when want_slots)."""
    B, T, H, _, n = ks.shape
    dv = v.shape[-1]
    desc = Desc(B=B, T=T, H=H, dk=dv, dv=dv, chunk=64, io_dtype=_dtype_code(v), gate_dtype=_dtype_code(alpha),
                alpha_mode=0, beta_mode=0, flags=0)
    o = torch.empty_like(v)
    ws_ = ((torch.empty((B, T, H, W), dtype=torch.int32, device=v.device),
            torch.empty((B, T, H, R), dtype=torch.int32, device=v.device)) if want_slots else (None, None))
    need = gdr_sdm_workspace_size(desc, n, W, R)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=v.device)
    rc = gdr_sdm_fwd(desc, n, W, R, ks, qs, v, alpha, beta, M, o, ws_[0], ws_[1], workspace,
                     workspace.numel() * workspace.element_size(), ctx, stream)
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_sdm_fwd")
    return (o, ws_[0], ws_[1]) if want_slots else o


def dmem_fwd(M, q, k, v, lam, beta, *, seg_end=None, J=1, out=None, stream=None):
    """delta-mem context pass: M [B, H, r, r] fp32 is updated in place; q, k, v
    [B, T, H, r]; lam, beta [B, T, H]; seg_end [B, T] uint8 or None (one write per
    token).  Returns the reads [B, T, H // J, r] (J sub-states per group, reads summed)."""
    B, T, H, r = q.shape
    desc = Desc(B=B, T=T, H=H, dk=r, dv=r, chunk=64, io_dtype=_dtype_code(q), gate_dtype=_dtype_code(lam),
                alpha_mode=0, beta_mode=0, flags=0)
    o = out if out is not None else torch.empty((B, T, H // J, r), dtype=q.dtype, device=q.device)
    rc = gdr_dmem_fwd(desc, J, q, k, v, lam, beta, seg_end, M, o, stream)
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_dmem_fwd")
    return o


def decode_step(S, q, k, v, alpha, beta_k, *, k_w=None, beta_v=None, out=None, flags=0, stream=None):
    """One token for every (b, h); S [B, H, dk, dv] fp32 is updated in place.  Returns o [B, H, dv].
    `flags`: GDR_FLAG_READ_BEFORE_WRITE and / or GDR_FLAG_UNDECAYED_PREDICTION."""
    desc = make_desc(q, v, alpha, beta_k, beta_v, decode=True, flags=flags)
    o = out if out is not None else torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=q.dtype, device=q.device)
    rc = gdr_decode_step(desc, q, k, k_w, v, alpha, beta_k, beta_v, S, o, stream)
    if rc != GDR_OK:
        raise GdrError(rc, "gdr_decode_step")
    return o


def loaded_library_path() -> str:
    return LIB_PATH
