"""Seeded synthetic inputs for the gated delta-rule recurrence.

This module is shared by the oracle-side tests and the GPU path (tests, smoke,
bench).  It draws random numbers, applies the input recipe of each workload
(L2-normalised q and k, sigmoid gates, bf16 storage) and nothing else: none of
the recurrence's arithmetic lives here.

Every tensor is returned as a NumPy array in its *stored* form:

* bf16 tensors as ``uint16`` bit patterns (round-to-nearest-even from fp32),
* fp32 tensors as ``float32``.

``as_f64`` turns a stored array into the exact fp64 values it represents, which
is what the oracle consumes; ``to_torch`` uploads a stored array with its
dtype.

Layouts (row-major):
  prefill  q, k, k_w: [B, T, H, dk]   v: [B, T, H, dv]
           alpha: [B, T, H] (scalar gate) or [B, T, H, dk] (channel gate)
           beta_k: [B, T, H] (scalar) or [B, T, H, dk] (vector)
           beta_v: [B, T, H, dv] (vector, separate write strength) or None
           S0: [B, H, dk, dv] fp32 or None
  decode   per-step tensors gain a leading step axis: q [steps, B, H, dk], ...
           S: [B, H, dk, dv] fp32
  sparse memory  ks, qs: [B, T, H, 2, n] fp32 half scores, v: [B, T, H, dv],
           alpha, beta: [B, T, H], M0: [B, H, n * n, dv] fp32
  delta-mem pass  q, k, v: [B, T, H, r], lam, beta: [B, T, H], seg_end: [B, T] uint8
           or None, M0: [B, H, r, r] fp32 (row a predicts value component a)
  cache read-out  q: [B, T, H, dk] bf16, ckpt: [B, H, N, dk, dv] fp32,
           gates: [B, T, H, N] fp32 or None, o_in: [B, T, H, dv] bf16 or None
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"

GATE_SCALAR = 0
GATE_CHANNEL = 1
BETA_SCALAR = 0
BETA_SHARED = 1
BETA_KV = 2


# ----------------------------------------------------------------------------
# storage conversions (no method arithmetic)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16, nearest-even, returned as uint16 bit patterns."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f64(x: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    """Exact fp64 value of a stored array (bf16 bits or fp32)."""
    if x is None:
        return None
    if dtype == BF16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def store(x64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 draw -> stored form (fp32 first, then bf16 RNE when asked)."""
    x32 = np.asarray(x64, dtype=np.float32)
    return f32_to_bf16_bits(x32) if dtype == BF16 else x32


def to_torch(x: Optional[np.ndarray], dtype: str, device="cuda"):
    """Upload a stored array to a torch tensor of the matching dtype."""
    import torch

    if x is None:
        return None
    if dtype == BF16:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    """Per-token L2 normalisation over the last axis, fp64, no epsilon."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


# ----------------------------------------------------------------------------
# workload descriptions
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Prefill:
    """A prefill (chunk forward) workload and its input recipe."""

    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    chunk: int
    io: str = BF16              # q, k, k_w, v, o
    gate: str = F32             # alpha, beta_k, beta_v
    alpha_mode: int = GATE_SCALAR
    beta_mode: int = BETA_SCALAR
    alpha_mu: float = -4.0      # alpha = sigmoid(-N(mu, sd)) == exp(-softplus(N(mu, sd)))
    alpha_sd: float = 1.0
    alpha_flip: bool = False    # alpha = sigmoid(+N(mu, sd)) instead
    write_key: bool = False     # k_w = bf16(d * k), d = 1 + 0.1 N(0, 1)
    s0_std: float = 0.0         # 0 -> S0 is None
    seed: int = 0

    def scaled(self, **kw) -> "Prefill":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Decode:
    """A batched one-token decode workload: `steps` consecutive steps."""

    name: str
    B: int
    H: int
    dk: int
    dv: int
    steps: int
    io: str = BF16
    gate: str = BF16
    alpha_mode: int = GATE_SCALAR
    beta_mode: int = BETA_SCALAR
    alpha_mu: float = -4.0
    alpha_sd: float = 1.0
    s_std: float = 0.02
    seed: int = 0

    def scaled(self, **kw) -> "Decode":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class CacheReadout:
    """A Memory-Caching read-out: cached segment states read by later tokens.

    gate_kind: "residual" (no gates), "dense" (every gate uniform in (0, 1)), or
    "topk" (a router keeps `topk` of the earlier segments per token, uniform
    weights on those, the rest 0)."""

    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    seg: int                    # tokens per segment
    gate_kind: str = "dense"
    topk: int = 2
    s_std: float = 0.02         # cached states ~ N(0, s_std)
    with_o_in: bool = True      # o_in ~ bf16(N(0, 1))
    seed: int = 0

    @property
    def N(self) -> int:
        return self.T // self.seg

    def scaled(self, **kw) -> "CacheReadout":
        return dataclasses.replace(self, **kw)


# The five workloads the library is specified against (named by content).
TINY_GDN_F32 = Prefill("tiny_gdn_f32_B1H1T64d16C16", B=1, T=64, H=1, dk=16, dv=16, chunk=16,
                       io=F32, gate=F32, alpha_mu=3.0, alpha_sd=0.5, alpha_flip=True, seed=8401)
GDN_PREFILL = Prefill("gdn_bf16_B4H16T4096d128C64", B=4, T=4096, H=16, dk=128, dv=128, chunk=64,
                      seed=8402)
KDA_FG2PLUS_PREFILL = Prefill("kda_fg2plus_bf16_B4H16T4096d128C64", B=4, T=4096, H=16, dk=128,
                              dv=128, chunk=64, alpha_mode=GATE_CHANNEL, beta_mode=BETA_KV,
                              seed=8403)
OSDN_LONG_PREFILL = Prefill("osdn_bf16_B1H32T65536d128C64", B=1, T=65536, H=32, dk=128, dv=128,
                            chunk=64, write_key=True, s0_std=0.02, seed=8404)
DECODE_B512 = Decode("decode_bf16_B512H16d128", B=512, H=16, dk=128, dv=128, steps=256, seed=8405)
DECODE_DMEM_R8 = Decode("decode_deltamem_bf16_B8192H1r8", B=8192, H=1, dk=8, dv=8, steps=256,
                        seed=8406)

@dataclasses.dataclass(frozen=True)
class SparseMemory:
    """A Sparse Delta Memory batch: per (b, h) a table of n * n slots x dv, W slots
    written and R read per token."""

    name: str
    B: int
    T: int
    H: int
    n: int                      # half-score length; N = n * n slots
    dv: int
    W: int
    R: int
    io: str = BF16              # v, o
    gate: str = F32             # alpha, beta
    alpha_mu: float = -4.0      # alpha = sigmoid(-N(mu, sd)), as the dense workloads
    alpha_sd: float = 1.0
    m0_std: float = 0.02        # M0 ~ N(0, m0_std) (the learned initial table)
    seed: int = 0

    @property
    def N(self) -> int:
        return self.n * self.n

    def scaled(self, **kw) -> "SparseMemory":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class DmemSeq:
    """A delta-mem context pass: per (b, h) an r x r memory written over T tokens, one
    write per token (TSW) or per segment (SSW, segments of a length mix), with J
    sub-states per group of heads whose reads are aggregated (MSW; H = G J)."""

    name: str
    B: int
    T: int
    H: int
    J: int
    r: int
    seg_mean: float = 0.0       # mean segment length (lengths 1 + geometric); 0: every token is one (TSW)
    io: str = BF16              # q, k, v, out
    gate: str = BF16            # lambda, beta
    lam_mu: float = -4.0        # lambda = sigmoid(-N(mu, sd)), as the decode workloads
    lam_sd: float = 1.0
    m_std: float = 0.02         # M0 ~ N(0, m_std) fp32
    seed: int = 0

    def scaled(self, **kw) -> "DmemSeq":
        return dataclasses.replace(self, **kw)


# Sparse Delta Memory at the headline batch's shape: 65,536 slots of 128 values per
# (b, h) (2 GiB of tables), W = R = 128 (the dense query width)
SDM_B4H16 = SparseMemory("sdm_bf16_B4H16T4096N65536dv128W128R128", B=4, T=4096, H=16, n=256, dv=128, W=128,
                         R=128, seed=8408)

# read-out of the long-context batch's segment caches: 16 segments of 4096 tokens
MC_LONG_GRM = CacheReadout("mc_grm_bf16_B1H32T65536d128seg4096", B=1, T=65536, H=32, dk=128, dv=128,
                           seg=4096, gate_kind="dense", seed=8407)

# delta-mem context passes at the small-state decode batch's shape (8192 memories of 8 x 8):
# segment writes over messages of ~16 tokens, and four sub-states per group of heads
DMEM_SSW = DmemSeq("deltamem_ssw_bf16_B8192T256H1r8", B=8192, T=256, H=1, J=1, r=8, seg_mean=16.0, seed=8409)
DMEM_MSW = DmemSeq("deltamem_msw_bf16_B2048T256H4J4r8", B=2048, T=256, H=4, J=4, r=8, seed=8410)

PREFILL_WORKLOADS = [TINY_GDN_F32, GDN_PREFILL, KDA_FG2PLUS_PREFILL, OSDN_LONG_PREFILL]
DECODE_WORKLOADS = [DECODE_B512, DECODE_DMEM_R8]


# ----------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------

def make_prefill(w: Prefill) -> dict:
    """Draw one prefill batch.  Draw order: q, k, v, alpha, beta_k, beta_v, d, S0."""
    rng = np.random.default_rng(w.seed)
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    q = store(_l2_normalise(rng.standard_normal((B, T, H, dk))), w.io)
    k64 = _l2_normalise(rng.standard_normal((B, T, H, dk)))
    k = store(k64, w.io)
    v = store(rng.standard_normal((B, T, H, dv)), w.io)
    ash = (B, T, H) if w.alpha_mode == GATE_SCALAR else (B, T, H, dk)
    x = rng.normal(w.alpha_mu, w.alpha_sd, ash)
    alpha = store(_sigmoid(x if w.alpha_flip else -x), w.gate)
    bsh = (B, T, H) if w.beta_mode == BETA_SCALAR else (B, T, H, dk)
    beta_k = store(_sigmoid(rng.standard_normal(bsh)), w.gate)
    beta_v = None
    if w.beta_mode == BETA_KV:
        beta_v = store(_sigmoid(rng.standard_normal((B, T, H, dv))), w.gate)
    k_w = None
    if w.write_key:
        d = 1.0 + 0.1 * rng.standard_normal((B, T, H, dk))
        # the write key is formed from the *stored* key, in fp32, then rounded
        k_w = store(d.astype(np.float32) * as_f64(k, w.io).astype(np.float32), w.io)
    S0 = None
    if w.s0_std > 0.0:
        S0 = rng.normal(0.0, w.s0_std, (B, H, dk, dv)).astype(np.float32)
    return dict(q=q, k=k, k_w=k_w, v=v, alpha=alpha, beta_k=beta_k, beta_v=beta_v, S0=S0)


def make_decode(w: Decode) -> dict:
    """Draw a decode run: per-step tensors [steps, B, H, .] and the initial state."""
    rng = np.random.default_rng(w.seed)
    n, B, H, dk, dv = w.steps, w.B, w.H, w.dk, w.dv
    q = store(_l2_normalise(rng.standard_normal((n, B, H, dk))), w.io)
    k = store(_l2_normalise(rng.standard_normal((n, B, H, dk))), w.io)
    v = store(rng.standard_normal((n, B, H, dv)), w.io)
    ash = (n, B, H) if w.alpha_mode == GATE_SCALAR else (n, B, H, dk)
    alpha = store(_sigmoid(-rng.normal(w.alpha_mu, w.alpha_sd, ash)), w.gate)
    bsh = (n, B, H) if w.beta_mode == BETA_SCALAR else (n, B, H, dk)
    beta_k = store(_sigmoid(rng.standard_normal(bsh)), w.gate)
    beta_v = None
    if w.beta_mode == BETA_KV:
        beta_v = store(_sigmoid(rng.standard_normal((n, B, H, dv))), w.gate)
    S = rng.normal(0.0, w.s_std, (B, H, dk, dv)).astype(np.float32)
    return dict(q=q, k=k, k_w=None, v=v, alpha=alpha, beta_k=beta_k, beta_v=beta_v, S=S)


def make_sparse_memory(w: SparseMemory) -> dict:
    """Draw an SDM batch.  Draw order: key half scores, query half scores, v, alpha,
    beta, M0.  Half scores ~ N(0, 1) fp32 (stand-ins for the projected key / query
    halves against their sub-key sets)."""
    rng = np.random.default_rng(w.seed)
    B, T, H, n, dv = w.B, w.T, w.H, w.n, w.dv
    ks = rng.standard_normal((B, T, H, 2, n)).astype(np.float32)
    qs = rng.standard_normal((B, T, H, 2, n)).astype(np.float32)
    v = store(rng.standard_normal((B, T, H, dv)), w.io)
    alpha = store(_sigmoid(-rng.normal(w.alpha_mu, w.alpha_sd, (B, T, H))), w.gate)
    beta = store(_sigmoid(rng.standard_normal((B, T, H))), w.gate)
    M0 = rng.normal(0.0, w.m0_std, (B, H, n * n, dv)).astype(np.float32)
    return dict(ks=ks, qs=qs, v=v, alpha=alpha, beta=beta, M0=M0)


def make_cache_readout(w: CacheReadout) -> dict:
    """Draw a cache read-out.  Draw order: q, ckpt, gates, o_in."""
    rng = np.random.default_rng(w.seed)
    B, T, H, dk, dv, N = w.B, w.T, w.H, w.dk, w.dv, w.N
    q = store(_l2_normalise(rng.standard_normal((B, T, H, dk))), BF16)
    ckpt = rng.normal(0.0, w.s_std, (B, H, N, dk, dv)).astype(np.float32)
    gates = None
    if w.gate_kind == "dense":
        gates = rng.uniform(0.0, 1.0, (B, T, H, N)).astype(np.float32)
    elif w.gate_kind == "topk":
        score = rng.standard_normal((B, T, H, N))
        seg_of = np.minimum(np.arange(T) // w.seg, N)
        allowed = np.arange(N)[None, :] < seg_of[:, None]            # [T, N]
        score = np.where(allowed[None, :, None, :], score, -np.inf)
        keep = np.argsort(-score, axis=-1)[..., :w.topk]
        gates = np.zeros((B, T, H, N), dtype=np.float32)
        np.put_along_axis(gates, keep, 1.0, axis=-1)
        gates = np.where(allowed[None, :, None, :], gates, 0.0).astype(np.float32)
    elif w.gate_kind != "residual":
        raise ValueError(w.gate_kind)
    o_in = store(rng.standard_normal((B, T, H, dv)), BF16) if w.with_o_in else None
    return dict(q=q, ckpt=ckpt, gates=gates, o_in=o_in)


def make_dmem_seq(w: DmemSeq) -> dict:
    """Draw a delta-mem context pass.  Draw order: q, k, v, lambda, beta, segment
    lengths, M0.  seg_end [B, T] uint8 marks each segment's last token (None for TSW);
    every row's last token closes its last segment."""
    rng = np.random.default_rng(w.seed)
    B, T, H, r = w.B, w.T, w.H, w.r
    q = store(_l2_normalise(rng.standard_normal((B, T, H, r))), w.io)
    k = store(_l2_normalise(rng.standard_normal((B, T, H, r))), w.io)
    v = store(rng.standard_normal((B, T, H, r)), w.io)
    lam = store(_sigmoid(-rng.normal(w.lam_mu, w.lam_sd, (B, T, H))), w.gate)
    beta = store(_sigmoid(rng.standard_normal((B, T, H))), w.gate)
    seg_end = None
    if w.seg_mean > 0.0:
        # lengths 1 + Geometric(1 / seg_mean) (mean seg_mean), enough of them to cover T
        n = int(2 * T / w.seg_mean) + 16
        lens = rng.geometric(1.0 / w.seg_mean, (B, n))
        ends = np.cumsum(lens, axis=1) - 1
        seg_end = np.zeros((B, T), dtype=np.uint8)
        rows = np.repeat(np.arange(B), n)
        e = ends.reshape(-1)
        keep = e < T
        seg_end[rows[keep], e[keep]] = 1
        seg_end[:, T - 1] = 1
    M0 = rng.normal(0.0, w.m_std, (B, H, r, r)).astype(np.float32)
    return dict(q=q, k=k, v=v, lam=lam, beta=beta, seg_end=seg_end, M0=M0)


def dmem_seq_f64(w: DmemSeq, x: dict) -> dict:
    out = {key: as_f64(x[key], w.io) for key in ("q", "k", "v")}
    out["lam"] = as_f64(x["lam"], w.gate)
    out["beta"] = as_f64(x["beta"], w.gate)
    out["M0"] = as_f64(x["M0"], F32)
    out["seg_end"] = x["seg_end"]
    return out


def make_retention(w: Prefill, mu: float = 4.0, sd: float = 1.0) -> np.ndarray:
    """Retention gate of the OSDN preconditioner (APF), r = sigmoid(N(mu, sd)) per
    (b, t, h), stored in the workload's gate dtype; drawn from its own stream."""
    rng = np.random.default_rng(w.seed + 100000)
    return store(_sigmoid(rng.normal(mu, sd, (w.B, w.T, w.H))), w.gate)


def prefill_f64(w: Prefill, x: dict) -> dict:
    """The exact fp64 values of a prefill batch (what the oracle reads)."""
    out = {}
    for key in ("q", "k", "k_w", "v"):
        out[key] = as_f64(x[key], w.io)
    for key in ("alpha", "beta_k", "beta_v"):
        out[key] = as_f64(x[key], w.gate)
    out["S0"] = as_f64(x["S0"], F32)
    return out


def decode_f64(w: Decode, x: dict) -> dict:
    out = {}
    for key in ("q", "k", "k_w", "v"):
        out[key] = as_f64(x[key], w.io)
    for key in ("alpha", "beta_k", "beta_v"):
        out[key] = as_f64(x[key], w.gate)
    out["S"] = as_f64(x["S"], F32)
    return out
