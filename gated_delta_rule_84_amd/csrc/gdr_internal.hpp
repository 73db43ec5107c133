// gdr_internal.hpp -- parameter blocks and launcher declarations shared by the
// host API (gdr_api.cpp) and the kernel translation units.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// A caller-owned execution context (include/gdr.h): a second stream on one device and
// the events that fork work onto it from the caller's stream and join it back.  The
// library keeps no copy of it; one context serves one call at a time.
constexpr int kCtxEvents = 66;
struct gdr_context {
    int device;
    hipStream_t stream;
    hipEvent_t ev[kCtxEvents];
};

namespace gdr {

// Parameters of one prefill call, already validated by the host API.
struct ChunkParams {
    int B, T, H, dk, dv, C;
    int io_bf16;    // q, k, k_w, v, o are bf16 (else fp32)
    int gate_bf16;  // alpha, beta_k, beta_v are bf16 (else fp32)
    int alpha_ch;   // alpha is per key channel
    int beta_mode;  // 0 scalar, 1 shared vector, 2 separate k / v vectors
    const void *q, *k, *kw, *v, *alpha, *beta_k, *beta_v;  // kw never NULL here (defaults to k)
    const float *S0;  // may be NULL (zero state)
    void *o;
    float *ST;        // may be NULL
    float *ckpt;      // may be NULL: states at segment ends, [B, H, nck, dk, dv]
    int seg_chunks;   // chunks per segment (ckpt only)
    int nck;          // segment ends stored per (batch, head): floor(T / segment length)
    void *ws;         // workspace (path dependent)
    int c0, c1;       // matrix-core prep and wave-specialised state kernels: the launch covers
                      // chunks c0 .. c1 - 1 (set by the launcher)
};

// True when chunk c (0-based) ends a segment whose state is kept; its slot is then
// (c + 1) / seg_chunks - 1.
__device__ __forceinline__ bool ckpt_after(const ChunkParams &p, int c) {
    return p.ckpt && (c + 1) % p.seg_chunks == 0 && (c + 1) / p.seg_chunks <= p.nck;
}

// Parameters of one decode step.
struct DecodeParams {
    int B, H, dk, dv;
    int io_bf16, gate_bf16, alpha_ch, beta_mode;
    int read_before_write;     // o = S_{t-1}^T q instead of S_t^T q
    int undecayed_prediction;  // residual against S_{t-1} instead of Diag(alpha) S_{t-1}
    const void *q, *k, *kw, *v, *alpha, *beta_k, *beta_v;
    float *S;
    void *o;
};

// Parameters of one delta-mem context pass (R x R memories, J sub-states per group).
struct DmemParams {
    int B, T, H, R, J;
    int io_bf16, gate_bf16;
    const void *q, *k, *v, *lam, *beta;
    const uint8_t *seg;  // NULL: every token closes its segment
    float *M;
    void *out;
};

// Launchers (defined next to their kernels).  They only enqueue work.
hipError_t launch_decode(const DecodeParams &p, hipStream_t s);
hipError_t launch_dmem(const DmemParams &p, hipStream_t s);
hipError_t launch_chunk_valu(const ChunkParams &p, hipStream_t s);
size_t chunk_mfma_workspace(const ChunkParams &p);
bool chunk_mfma_supported(const ChunkParams &p);
hipError_t launch_chunk_mfma(const ChunkParams &p, const gdr_context *ctx, hipStream_t s);
hipError_t launch_state_copy(const float *S0, float *ST, long n, hipStream_t s);
size_t mc_readout_workspace(int B, int H, int N);
size_t osdn_precond_workspace(int B, int T, int H);
size_t sdm_workspace(int B, int T, int H, int W, int R);
hipError_t launch_sdm(int B, int T, int H, int n, int W, int R, int io_bf16, int gate_bf16, const float *ks,
                      const float *qs, const void *v, const void *alpha, const void *beta, float *M, void *o,
                      int32_t *wslots, int32_t *rslots, void *ws, const gdr_context *ctx, hipStream_t s);
hipError_t launch_osdn_precond(int B, int T, int H, int dk, int io_bf16, int gate_bf16, float eta, const void *k,
                               const void *beta, const void *r, const float *d0, void *kw, float *dT, float *qgeo,
                               void *ws, const gdr_context *ctx, hipStream_t s);
hipError_t launch_mc_readout(int B, int T, int H, int N, int seg, const void *q, const float *ckpt,
                             const float *gates, const void *oin, void *oout, void *ws, hipStream_t s);

}  // namespace gdr
