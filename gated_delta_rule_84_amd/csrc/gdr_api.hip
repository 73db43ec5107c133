// gdr_api.hip -- the C-ABI entry points declared in include/gdr.h: host-side
// validation, path selection and launches on the caller's stream.
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <new>

#include "gdr.h"
#include "gdr_internal.hpp"

namespace gdr {
size_t chunk_valu_lds_bytes(int dk, int C);

namespace {

__global__ void state_copy_kernel(const float *__restrict__ src, float *__restrict__ dst, long n) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.f;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Byte ranges [a, a + na) and [b, b + nb) intersect (both non-empty).
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

int check_desc(const gdr_desc *d, bool prefill) {
    if (!d) return GDR_EINVAL;
    if (d->B < 0 || d->H < 0 || (prefill && d->T < 0)) return GDR_EINVAL;
    if (d->io_dtype != GDR_BF16 && d->io_dtype != GDR_F32) return GDR_EINVAL;
    if (d->gate_dtype != GDR_BF16 && d->gate_dtype != GDR_F32) return GDR_EINVAL;
    if (d->alpha_mode != GDR_ALPHA_SCALAR && d->alpha_mode != GDR_ALPHA_CHANNEL) return GDR_EINVAL;
    if (d->beta_mode < GDR_BETA_SCALAR || d->beta_mode > GDR_BETA_KV) return GDR_EINVAL;
    if (d->flags & ~(GDR_FLAG_READ_BEFORE_WRITE | GDR_FLAG_UNDECAYED_PREDICTION)) return GDR_EINVAL;
    if (d->beta_mode == GDR_BETA_SHARED && d->dk != d->dv) return GDR_EINVAL;
    if (d->dk < 8 || d->dk > 128 || (d->dk & 7) || d->dv < 8 || d->dv > 128 || (d->dv & 7))
        return GDR_EUNSUPPORTED;
    if (prefill && d->chunk != 16 && d->chunk != 32 && d->chunk != 64) return GDR_EUNSUPPORTED;
    if (prefill && (d->flags & (GDR_FLAG_READ_BEFORE_WRITE | GDR_FLAG_UNDECAYED_PREDICTION))) return GDR_EUNSUPPORTED;
    const long long bh = (long long)d->B * d->H;
    if (bh > 0x7fffffffLL) return GDR_EUNSUPPORTED;
    return GDR_OK;
}

ChunkParams chunk_params(const gdr_desc *d) {
    ChunkParams p;
    memset(&p, 0, sizeof(p));
    p.B = d->B; p.T = d->T; p.H = d->H; p.dk = d->dk; p.dv = d->dv; p.C = d->chunk;
    p.io_bf16 = d->io_dtype == GDR_BF16;
    p.gate_bf16 = d->gate_dtype == GDR_BF16;
    p.alpha_ch = d->alpha_mode == GDR_ALPHA_CHANNEL;
    p.beta_mode = d->beta_mode;
    return p;
}

int select_path(const gdr_desc *, const ChunkParams &p) { return chunk_mfma_supported(p) ? 1 : 2; }

// A context passed to a call must belong to the current device.
bool context_ok(const gdr_context *ctx) {
    if (!ctx) return true;
    int dev = -1;
    return hipGetDevice(&dev) == hipSuccess && dev == ctx->device;
}

// Scratch of gdr_chunk_fwd_noalloc: one static array per device.  In host code its
// name is a host-side stand-in, so kernels and copies get the device address looked up
// once per device (kept in noalloc_ptr, guarded by noalloc_mu).
static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex noalloc_mu;
void *noalloc_ptr[kMaxDevices] = {};

hipError_t noalloc_scratch(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(noalloc_mu);
    if (!noalloc_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        noalloc_ptr[dev] = ptr;
    }
    *out = noalloc_ptr[dev];
    return hipSuccess;
}

int device_lds_limit() {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return -1;
    return v;
}

}  // namespace
}  // namespace gdr

using namespace gdr;

extern "C" {

int gdr_version(void) { return (2 << 16) | 0; }

int gdr_context_create(gdr_context **out) {
    if (!out) return GDR_EINVAL;
    *out = nullptr;
    gdr_context *c = new (std::nothrow) gdr_context;
    if (!c) return GDR_EHIP;
    memset(c, 0, sizeof(*c));
    hipError_t e = hipGetDevice(&c->device);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->stream, hipStreamNonBlocking);
    int made = 0;
    for (; e == hipSuccess && made < kCtxEvents; ++made)
        e = hipEventCreateWithFlags(&c->ev[made], hipEventDisableTiming);
    if (e != hipSuccess) {
        for (int j = 0; j < made; ++j)
            if (c->ev[j]) (void)hipEventDestroy(c->ev[j]);
        if (c->stream) (void)hipStreamDestroy(c->stream);
        delete c;
        return GDR_EHIP;
    }
    *out = c;
    return GDR_OK;
}

int gdr_context_destroy(gdr_context *c) {
    if (!c) return GDR_OK;
    hipError_t e = hipStreamSynchronize(c->stream);
    for (int j = 0; j < kCtxEvents; ++j) {
        const hipError_t f = hipEventDestroy(c->ev[j]);
        if (e == hipSuccess) e = f;
    }
    const hipError_t f = hipStreamDestroy(c->stream);
    if (e == hipSuccess) e = f;
    delete c;
    return e == hipSuccess ? GDR_OK : GDR_EHIP;
}

const char *gdr_status_string(int s) {
    switch (s) {
    case GDR_OK: return "GDR_OK: success";
    case GDR_EINVAL: return "GDR_EINVAL: invalid argument (NULL pointer, bad enum, negative size, "
                            "misaligned or overlapping buffer, beta layout not matching beta_mode)";
    case GDR_EUNSUPPORTED: return "GDR_EUNSUPPORTED: shape not implemented (dk, dv must be multiples "
                                  "of 8 in [8, 128]; chunk must be 16, 32 or 64)";
    case GDR_EWORKSPACE: return "GDR_EWORKSPACE: workspace missing or smaller than "
                                "gdr_chunk_fwd_workspace_size()";
    case GDR_EHIP: return "GDR_EHIP: the HIP runtime reported an error";
    case GDR_ETOOLARGE: return "GDR_ETOOLARGE: the call needs more scratch than the static scratch array of "
                               "gdr_chunk_fwd_noalloc holds (GDR_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown gdr status";
    }
}

int gdr_chunk_fwd_path(const gdr_desc *d) {
    const int rc = check_desc(d, true);
    if (rc) return rc;
    return select_path(d, chunk_params(d));
}

size_t gdr_chunk_fwd_workspace_size(const gdr_desc *d) {
    if (check_desc(d, true)) return 0;
    const ChunkParams p = chunk_params(d);
    return select_path(d, p) == 1 ? chunk_mfma_workspace(p) : 0;
}

// Prefill shared by gdr_chunk_fwd, gdr_chunk_fwd_ckpt and gdr_chunk_fwd_ctx.
static int chunk_fwd_impl(const gdr_desc *d, const void *q, const void *k, const void *k_w, const void *v,
                          const void *alpha, const void *beta_k, const void *beta_v, const float *S0,
                          void *o, float *ST, int32_t seg_len, float *ckpt, void *workspace,
                          size_t workspace_bytes, const gdr_context *ctx, void *stream) {
    int rc = check_desc(d, true);
    if (rc) return rc;
    if (!context_ok(ctx)) return GDR_EINVAL;
    ChunkParams p = chunk_params(d);
    if (seg_len <= 0 || seg_len % d->chunk) return GDR_EINVAL;
    const int nck = d->T / seg_len;
    const long long ntok = (long long)d->B * d->T * d->H;
    const size_t es = p.io_bf16 ? 2 : 4, gs = p.gate_bf16 ? 2 : 4;
    const size_t nq = ntok * d->dk * es, nv = ntok * d->dv * es;
    const size_t na = ntok * (p.alpha_ch ? d->dk : 1) * gs;
    const size_t nbk = ntok * (d->beta_mode ? d->dk : 1) * gs, nbv = ntok * d->dv * gs;
    const size_t ns = (size_t)d->B * d->H * d->dk * d->dv * sizeof(float);
    if ((d->beta_mode == GDR_BETA_KV) != (beta_v != nullptr)) return GDR_EINVAL;
    if (ntok > 0) {
        if (!q || !k || !v || !alpha || !beta_k || !o) return GDR_EINVAL;
        const void *vec[] = {q, k, k_w, v, o};
        for (const void *x : vec)
            if (x && !aligned16(x)) return GDR_EINVAL;
        const void *gates[] = {alpha, beta_k, beta_v};
        for (const void *x : gates)
            if (x && !aligned_to(x, gs)) return GDR_EINVAL;
        const void *ins[] = {q, k, k_w, v, alpha, beta_k, beta_v, S0};
        const size_t lens[] = {nq, nq, nq, nv, na, nbk, nbv, ns};
        for (int i = 0; i < 8; ++i)
            if (overlaps(o, nv, ins[i], lens[i])) return GDR_EINVAL;
        if (ST && overlaps(o, nv, ST, ns)) return GDR_EINVAL;
    }
    if ((S0 && !aligned16(S0)) || (ST && !aligned16(ST))) return GDR_EINVAL;
    if (nck > 0) {
        if (!ckpt || !aligned16(ckpt)) return GDR_EINVAL;
        const size_t nc = ns * (size_t)nck;
        const void *ins[] = {q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST};
        const size_t lens[] = {nq, nq, nq, nv, na, nbk, nbv, ns, nv, ns};
        for (int i = 0; i < 10; ++i)
            if (overlaps(ckpt, nc, ins[i], lens[i])) return GDR_EINVAL;
    }
    if (ST && S0 && ST != S0 && overlaps(ST, ns, S0, ns)) return GDR_EINVAL;
    if (ST && ntok > 0) {
        const void *ins[] = {q, k, k_w, v, alpha, beta_k, beta_v};
        const size_t lens[] = {nq, nq, nq, nv, na, nbk, nbv};
        for (int i = 0; i < 7; ++i)
            if (overlaps(ST, ns, ins[i], lens[i])) return GDR_EINVAL;
    }
    const int path = select_path(d, p);
    const size_t ws_need = path == 1 ? chunk_mfma_workspace(p) : 0;
    if (ws_need > 0 && (!workspace || workspace_bytes < ws_need || !aligned16(workspace)))
        return GDR_EWORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const long long nbh = (long long)d->B * d->H;
    if (nbh == 0) return GDR_OK;
    if (path == 2 && d->T > 0) {
        const int lim = device_lds_limit();
        if (lim < 0) return GDR_EHIP;
        if (chunk_valu_lds_bytes(d->dk, d->chunk) > (size_t)lim) return GDR_EUNSUPPORTED;
    }
    if (d->T == 0) {
        if (!ST || ST == S0) return GDR_OK;
        const long n = (long)(ns / sizeof(float));
        const float *src = S0;
        float *dst = ST;
        long nn = n;
        void *args[] = {&src, &dst, &nn};
        const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&state_copy_kernel),
                                             dim3((unsigned)((n + 255) / 256)), dim3(256), args, 0, st);
        return e == hipSuccess ? GDR_OK : GDR_EHIP;
    }
    p.q = q; p.k = k; p.kw = k_w ? k_w : k; p.v = v;
    p.alpha = alpha; p.beta_k = beta_k; p.beta_v = beta_v;
    p.S0 = S0; p.o = o; p.ST = ST; p.ws = workspace;
    if (nck > 0) {
        p.ckpt = ckpt;
        p.seg_chunks = seg_len / d->chunk;
        p.nck = nck;
    }
    const hipError_t e = path == 1 ? launch_chunk_mfma(p, ctx, st) : launch_chunk_valu(p, st);
    return e == hipSuccess ? GDR_OK : GDR_EHIP;
}

int gdr_chunk_fwd_ckpt(const gdr_desc *d, const void *q, const void *k, const void *k_w, const void *v,
                       const void *alpha, const void *beta_k, const void *beta_v, const float *S0,
                       void *o, float *ST, int32_t seg_len, float *ckpt, void *workspace,
                       size_t workspace_bytes, void *stream) {
    return chunk_fwd_impl(d, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST, seg_len, ckpt, workspace,
                          workspace_bytes, nullptr, stream);
}

int gdr_chunk_fwd_ctx(const gdr_desc *d, const void *q, const void *k, const void *k_w, const void *v,
                      const void *alpha, const void *beta_k, const void *beta_v, const float *S0, void *o,
                      float *ST, void *workspace, size_t workspace_bytes, const gdr_context *ctx, void *stream) {
    // no segment ends are kept: a segment longer than any T
    const int32_t seg = d && d->chunk > 0 ? (0x7fffffff / d->chunk) * d->chunk : 1;
    return chunk_fwd_impl(d, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST, seg, nullptr, workspace,
                          workspace_bytes, ctx, stream);
}

int gdr_chunk_fwd(const gdr_desc *d, const void *q, const void *k, const void *k_w, const void *v,
                  const void *alpha, const void *beta_k, const void *beta_v, const float *S0,
                  void *o, float *ST, void *workspace, size_t workspace_bytes, void *stream) {
    // no segment ends are kept: a segment longer than any T
    const int32_t seg = d && d->chunk > 0 ? (0x7fffffff / d->chunk) * d->chunk : 1;
    return gdr_chunk_fwd_ckpt(d, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST, seg, nullptr, workspace,
                              workspace_bytes, stream);
}

int gdr_chunk_fwd_noalloc(const gdr_desc *d, const void *q, const void *k, const void *k_w, const void *v,
                          const void *alpha, const void *beta_k, const void *beta_v, const float *S0,
                          void *o, float *ST, void *stream) {
    // everything that needs no device is checked first, the size against the array included
    const int rc = check_desc(d, true);
    if (rc) return rc;
    const size_t need = gdr_chunk_fwd_workspace_size(d);
    if (need > GDR_NOALLOC_SCRATCH_BYTES) return GDR_ETOOLARGE;
    void *ws = nullptr;
    if (need > 0) {
        const hipError_t e = noalloc_scratch(&ws);
        if (e != hipSuccess) return GDR_EHIP;
    }
    return gdr_chunk_fwd(d, q, k, k_w, v, alpha, beta_k, beta_v, S0, o, ST, ws, need > 0 ? GDR_NOALLOC_SCRATCH_BYTES : 0,
                         stream);
}

size_t gdr_mc_readout_workspace_size(const gdr_desc *d, int32_t n_ckpt) {
    if (!d || d->B < 0 || d->H < 0 || n_ckpt < 0) return 0;
    return mc_readout_workspace(d->B, d->H, n_ckpt);
}

int gdr_mc_readout(const gdr_desc *d, const void *q, const float *ckpt, int32_t n_ckpt, int32_t seg_len,
                   const float *gates, const void *o_in, void *o_out, void *workspace, size_t workspace_bytes,
                   void *stream) {
    if (!d || d->B < 0 || d->T < 0 || d->H < 0 || n_ckpt < 0 || seg_len <= 0) return GDR_EINVAL;
    if (d->io_dtype != GDR_BF16 && d->io_dtype != GDR_F32) return GDR_EINVAL;
    if (d->io_dtype != GDR_BF16 || d->dk != 128 || d->dv != 128) return GDR_EUNSUPPORTED;
    const long long nbh = (long long)d->B * d->H, ntok = nbh * d->T;
    if (nbh > 0x7fffffffLL) return GDR_EUNSUPPORTED;
    if (ntok == 0) return GDR_OK;
    if (!q || !o_out || !aligned16(q) || !aligned16(o_out)) return GDR_EINVAL;
    if (o_in && !aligned16(o_in)) return GDR_EINVAL;
    const size_t nq = ntok * 128 * 2, nc = (size_t)nbh * n_ckpt * 128 * 128 * sizeof(float);
    const size_t ng = (size_t)ntok * n_ckpt * sizeof(float);
    const size_t wneed = mc_readout_workspace(d->B, d->H, n_ckpt);
    if (n_ckpt > 0) {
        if (!ckpt || !aligned16(ckpt)) return GDR_EINVAL;
        if (gates && !aligned_to(gates, 4)) return GDR_EINVAL;
        if (!workspace || workspace_bytes < wneed || !aligned16(workspace)) return GDR_EWORKSPACE;
    }
    // o_out may be o_in itself but overlaps nothing else; the workspace overlaps nothing
    if (o_in && o_in != o_out && overlaps(o_out, nq, o_in, nq)) return GDR_EINVAL;
    {
        const void *ins[] = {q, n_ckpt ? ckpt : nullptr, n_ckpt ? gates : nullptr};
        const size_t lens[] = {nq, nc, ng};
        for (int i = 0; i < 3; ++i)
            if (overlaps(o_out, nq, ins[i], lens[i])) return GDR_EINVAL;
        if (n_ckpt > 0) {
            const void *all[] = {q, ckpt, gates, o_in, o_out};
            const size_t alens[] = {nq, nc, ng, nq, nq};
            for (int i = 0; i < 5; ++i)
                if (overlaps(workspace, wneed, all[i], alens[i])) return GDR_EINVAL;
        }
    }
    const hipError_t e = launch_mc_readout(d->B, d->T, d->H, n_ckpt, seg_len, q, ckpt, gates, o_in, o_out,
                                           workspace, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDR_OK : GDR_EHIP;
}

size_t gdr_osdn_precond_workspace_size(const gdr_desc *d) {
    if (!d || d->B < 0 || d->T < 0 || d->H < 0) return 0;
    return osdn_precond_workspace(d->B, d->T, d->H);
}

int gdr_osdn_precond(const gdr_desc *d, const void *k, const void *beta, const void *r, float eta, const float *d0,
                     void *k_w, float *dT, float *qgeo, void *workspace, size_t workspace_bytes, gdr_context *ctx,
                     void *stream) {
    if (!d || d->B < 0 || d->T < 0 || d->H < 0) return GDR_EINVAL;
    if (!context_ok(ctx)) return GDR_EINVAL;
    if (d->io_dtype != GDR_BF16 && d->io_dtype != GDR_F32) return GDR_EINVAL;
    if (d->gate_dtype != GDR_BF16 && d->gate_dtype != GDR_F32) return GDR_EINVAL;
    if (d->beta_mode != GDR_BETA_SCALAR) return GDR_EINVAL;
    if (!(eta == eta)) return GDR_EINVAL;  // NaN
    if (d->dk < 8 || d->dk > 128 || (d->dk & 7)) return GDR_EUNSUPPORTED;
    const long long nbh = (long long)d->B * d->H, ntok = nbh * d->T;
    if (nbh > 0x7fffffffLL) return GDR_EUNSUPPORTED;
    if (nbh == 0) return GDR_OK;
    const size_t es = d->io_dtype == GDR_BF16 ? 2 : 4, gs = d->gate_dtype == GDR_BF16 ? 2 : 4;
    const size_t nk = (size_t)ntok * d->dk * es, ng = (size_t)ntok * gs, nd = (size_t)nbh * d->dk * sizeof(float);
    if (ntok > 0) {
        if (!k || !beta || !k_w || !aligned16(k) || !aligned16(k_w)) return GDR_EINVAL;
        if (!aligned_to(beta, gs) || (r && !aligned_to(r, gs))) return GDR_EINVAL;
    }
    if ((d0 && !aligned16(d0)) || (dT && !aligned_to(dT, 4)) || (qgeo && !aligned_to(qgeo, 4))) return GDR_EINVAL;
    const size_t wneed = osdn_precond_workspace(d->B, d->T, d->H);
    if (wneed > 0 && (!workspace || workspace_bytes < wneed || !aligned16(workspace))) return GDR_EWORKSPACE;
    // outputs overlap no input and no other output; the workspace overlaps nothing
    {
        const void *outs[] = {ntok ? k_w : nullptr, dT, qgeo};
        const size_t olens[] = {nk, nd, (size_t)nbh * sizeof(float)};
        const void *ins[] = {k, beta, r, d0};
        const size_t ilens[] = {nk, ng, ng, nd};
        for (int i = 0; i < 3; ++i) {
            for (int j = 0; j < 4; ++j)
                if (overlaps(outs[i], olens[i], ins[j], ilens[j])) return GDR_EINVAL;
            for (int j = i + 1; j < 3; ++j)
                if (overlaps(outs[i], olens[i], outs[j], olens[j])) return GDR_EINVAL;
            if (overlaps(workspace, wneed, outs[i], olens[i])) return GDR_EINVAL;
        }
        for (int j = 0; j < 4; ++j)
            if (overlaps(workspace, wneed, ins[j], ilens[j])) return GDR_EINVAL;
    }
    const hipError_t e = launch_osdn_precond(d->B, d->T, d->H, d->dk, d->io_dtype == GDR_BF16, d->gate_dtype == GDR_BF16,
                                             eta, k, beta, r, d0, k_w, dT, qgeo, workspace, ctx,
                                             static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDR_OK : GDR_EHIP;
}

size_t gdr_sdm_workspace_size(const gdr_desc *d, int32_t n, int32_t W, int32_t R) {
    if (!d || d->B < 0 || d->T < 0 || d->H < 0 || W < 1 || R < 1 || n < 1) return 0;
    return sdm_workspace(d->B, d->T, d->H, W, R);
}

int gdr_sdm_fwd(const gdr_desc *d, int32_t n, int32_t W, int32_t R, const float *ks, const float *qs, const void *v,
                const void *alpha, const void *beta, float *M, void *o, int32_t *w_slots, int32_t *r_slots,
                void *workspace, size_t workspace_bytes, gdr_context *ctx, void *stream) {
    if (!d || d->B < 0 || d->T < 0 || d->H < 0) return GDR_EINVAL;
    if (!context_ok(ctx)) return GDR_EINVAL;
    if (d->io_dtype != GDR_BF16 && d->io_dtype != GDR_F32) return GDR_EINVAL;
    if (d->gate_dtype != GDR_BF16 && d->gate_dtype != GDR_F32) return GDR_EINVAL;
    if (n < 1 || W < 1 || R < 1) return GDR_EINVAL;
    if (d->dv != 128 || n > 1024 || W > 128 || R > 128 || W > n * n || R > n * n) return GDR_EUNSUPPORTED;
    const long long nbh = (long long)d->B * d->H, ntok = nbh * d->T;
    if (nbh > 0x7fffffffLL || ntok * 2 > 0x7fffffffLL) return GDR_EUNSUPPORTED;
    if (ntok == 0) return GDR_OK;
    const size_t es = d->io_dtype == GDR_BF16 ? 2 : 4, gs = d->gate_dtype == GDR_BF16 ? 2 : 4;
    const size_t nsc = (size_t)ntok * 2 * n * sizeof(float), nv = (size_t)ntok * 128 * es, ng = (size_t)ntok * gs;
    const size_t nm = (size_t)nbh * n * n * 128 * sizeof(float);
    if (!ks || !qs || !v || !alpha || !beta || !M || !o) return GDR_EINVAL;
    if (!aligned16(M) || !aligned_to(ks, 4) || !aligned_to(qs, 4) || !aligned_to(v, es) || !aligned_to(o, es))
        return GDR_EINVAL;
    if (!aligned_to(alpha, gs) || !aligned_to(beta, gs)) return GDR_EINVAL;
    if ((w_slots && !aligned_to(w_slots, 4)) || (r_slots && !aligned_to(r_slots, 4))) return GDR_EINVAL;
    const size_t wneed = sdm_workspace(d->B, d->T, d->H, W, R);
    if (!workspace || workspace_bytes < wneed || !aligned16(workspace)) return GDR_EWORKSPACE;
    {
        const void *ins[] = {ks, qs, v, alpha, beta};
        const size_t il[] = {nsc, nsc, nv, ng, ng};
        const void *outs[] = {M, o, w_slots, r_slots, workspace};
        const size_t ol[] = {nm, nv, (size_t)ntok * W * 4, (size_t)ntok * R * 4, wneed};
        for (int i = 0; i < 5; ++i) {
            for (int j = 0; j < 5; ++j)
                if (overlaps(outs[i], ol[i], ins[j], il[j])) return GDR_EINVAL;
            for (int j = i + 1; j < 5; ++j)
                if (overlaps(outs[i], ol[i], outs[j], ol[j])) return GDR_EINVAL;
        }
    }
    const hipError_t e = launch_sdm(d->B, d->T, d->H, n, W, R, d->io_dtype == GDR_BF16, d->gate_dtype == GDR_BF16,
                                    ks, qs, v, alpha, beta, M, o, w_slots, r_slots, workspace, ctx,
                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDR_OK : GDR_EHIP;
}

int gdr_dmem_fwd(const gdr_desc *d, int32_t J, const void *q, const void *k, const void *v, const void *lam,
                 const void *beta, const uint8_t *seg_end, float *M, void *out, void *stream) {
    if (!d || d->B < 0 || d->T < 0 || d->H < 0 || d->dk < 1 || d->dk != d->dv) return GDR_EINVAL;
    if (d->io_dtype != GDR_BF16 && d->io_dtype != GDR_F32) return GDR_EINVAL;
    if (d->gate_dtype != GDR_BF16 && d->gate_dtype != GDR_F32) return GDR_EINVAL;
    if (d->alpha_mode != GDR_ALPHA_SCALAR || d->beta_mode != GDR_BETA_SCALAR || d->flags != 0) return GDR_EINVAL;
    if (J < 1) return GDR_EINVAL;
    const int r = d->dk;
    if ((r != 8 && r != 16) || (J != 1 && J != 2 && J != 4 && J != 8) || J > 64 / r) return GDR_EUNSUPPORTED;
    if (d->H % J) return GDR_EINVAL;
    const long long nbh = (long long)d->B * d->H, ntok = nbh * d->T;
    // every tensor is addressed with 32-bit byte offsets
    if (nbh > 0x7fffffffLL || ntok * r * (d->io_dtype == GDR_BF16 ? 2 : 4) > 0x7fffffffLL ||
        (long long)d->B * d->T > 0x7fffffffLL)
        return GDR_EUNSUPPORTED;
    if (ntok == 0) return GDR_OK;
    if (!q || !k || !v || !lam || !beta || !M || !out) return GDR_EINVAL;
    const size_t es = d->io_dtype == GDR_BF16 ? 2 : 4, gs = d->gate_dtype == GDR_BF16 ? 2 : 4;
    if (!aligned16(q) || !aligned16(k) || !aligned_to(v, es) || !aligned_to(out, es) || !aligned_to(M, 4))
        return GDR_EINVAL;
    if (!aligned_to(lam, gs) || !aligned_to(beta, gs)) return GDR_EINVAL;
    {
        const size_t nrow = (size_t)ntok * r * es, ng = (size_t)ntok * gs;
        const void *ins[] = {q, k, v, lam, beta, seg_end};
        const size_t il[] = {nrow, nrow, nrow, ng, ng, (size_t)d->B * d->T};
        const size_t nm = (size_t)nbh * r * r * sizeof(float), no = (size_t)ntok / J * r * es;
        for (int i = 0; i < 6; ++i)
            if (overlaps(M, nm, ins[i], il[i]) || overlaps(out, no, ins[i], il[i])) return GDR_EINVAL;
        if (overlaps(M, nm, out, no)) return GDR_EINVAL;
    }
    DmemParams p{};
    p.B = d->B;
    p.T = d->T;
    p.H = d->H;
    p.R = r;
    p.J = J;
    p.io_bf16 = d->io_dtype == GDR_BF16;
    p.gate_bf16 = d->gate_dtype == GDR_BF16;
    p.q = q;
    p.k = k;
    p.v = v;
    p.lam = lam;
    p.beta = beta;
    p.seg = seg_end;
    p.M = M;
    p.out = out;
    return launch_dmem(p, static_cast<hipStream_t>(stream)) == hipSuccess ? GDR_OK : GDR_EHIP;
}

int gdr_decode_step(const gdr_desc *d, const void *q, const void *k, const void *k_w, const void *v,
                    const void *alpha, const void *beta_k, const void *beta_v, float *S, void *o,
                    void *stream) {
    int rc = check_desc(d, false);
    if (rc) return rc;
    if ((d->beta_mode == GDR_BETA_KV) != (beta_v != nullptr)) return GDR_EINVAL;
    const long long nbh = (long long)d->B * d->H;
    if (nbh == 0) return GDR_OK;
    if (!q || !k || !v || !alpha || !beta_k || !S || !o) return GDR_EINVAL;
    const size_t es = d->io_dtype == GDR_BF16 ? 2 : 4, gs = d->gate_dtype == GDR_BF16 ? 2 : 4;
    const void *vec[] = {q, k, k_w, v, S, o};
    for (const void *x : vec)
        if (x && !aligned16(x)) return GDR_EINVAL;
    const void *gates[] = {alpha, beta_k, beta_v};
    for (const void *x : gates)
        if (x && !aligned_to(x, gs)) return GDR_EINVAL;
    const size_t no = nbh * d->dv * es, ns = nbh * d->dk * d->dv * sizeof(float);
    const void *ins[] = {q, k, k_w, v, alpha, beta_k, beta_v};
    const size_t lens[] = {nbh * d->dk * es, nbh * d->dk * es, nbh * d->dk * es, no,
                           nbh * (d->alpha_mode ? d->dk : 1) * gs, nbh * (d->beta_mode ? d->dk : 1) * gs,
                           nbh * d->dv * gs};
    for (int i = 0; i < 7; ++i)
        if (overlaps(o, no, ins[i], lens[i]) || overlaps(S, ns, ins[i], lens[i])) return GDR_EINVAL;
    if (overlaps(o, no, S, ns)) return GDR_EINVAL;

    DecodeParams p;
    memset(&p, 0, sizeof(p));
    p.B = d->B; p.H = d->H; p.dk = d->dk; p.dv = d->dv;
    p.io_bf16 = d->io_dtype == GDR_BF16;
    p.gate_bf16 = d->gate_dtype == GDR_BF16;
    p.alpha_ch = d->alpha_mode == GDR_ALPHA_CHANNEL;
    p.beta_mode = d->beta_mode;
    p.read_before_write = (d->flags & GDR_FLAG_READ_BEFORE_WRITE) != 0;
    p.undecayed_prediction = (d->flags & GDR_FLAG_UNDECAYED_PREDICTION) != 0;
    p.q = q; p.k = k; p.kw = k_w ? k_w : k; p.v = v;
    p.alpha = alpha; p.beta_k = beta_k; p.beta_v = beta_v;
    p.S = S; p.o = o;
    const hipError_t e = launch_decode(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDR_OK : GDR_EHIP;
}

}  // extern "C"
