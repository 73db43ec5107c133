/*
 * gdr.h -- C-ABI of the gated delta-rule library for AMD Instinct MI355X (gfx950).
 *
 * The library evaluates the gated delta-rule state recurrence.  For one
 * (batch b, head h) the state S is a dk x dv fp32 matrix (row i = key
 * channel, column j = value channel).  Each token t applies
 *
 *     X_t = Diag(alpha_t) S_{t-1}                                   (forget gate)
 *     S_t = X_t + w_t (vh_t - X_t^T u_t)^T                          (rank-1 delta write)
 *     o_t = S_t^T q_t                                               (read-out after the write)
 *
 * with erase key u = sqrt(beta^k) (.) k, write key w = sqrt(beta^k) (.) k_w and
 * written value vh = sqrt(beta^v) (.) v; a scalar beta broadcasts.  This one
 * step covers the variants on the source pages:
 *   - Gated DeltaNet: scalar alpha and beta, k_w = k
 *       [FG2-GDN page, section 1; SDM page, Mecanismo Central item 3];
 *   - Kimi Delta Attention: one alpha per key channel
 *       [FG2-GDN page, section 1];
 *   - FG2-GDN: one beta vector absorbed as sqrt(beta) into k and v (dk == dv)
 *       [FG2-GDN page, section 2.A, state-update equation];
 *   - FG2-GDN+: separate erase and write strengths beta^k, beta^v
 *       [FG2-GDN page, section 2.B];
 *   - OSDN: write key k_w = d (.) k, the diagonally right-preconditioned
 *       online-gradient step [OSDN page, section 2.1, both update equations].
 * Prefill runs the chunkwise-parallel WY / UT-transform form of the same
 * recurrence (the block Gram matrix of the write and erase keys, its
 * unit-lower-triangular inverse, and the intra-chunk scores: FG2-GDN page,
 * section 3; OSDN page, section 2.1); decode applies one step to a resident state
 * [OSDN page, section 1; delta-mem page, section 2.A].
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates no device memory, keeps no pointer after a call returns and has no
 *     global mutable state beyond the per-device address of gdr_chunk_fwd_noalloc's
 *     static scratch array (looked up once, under a lock), so calls from several
 *     host threads are safe (gdr_chunk_fwd_noalloc: see its own rule).  The calls
 *     that can overlap independent work on a second stream (gdr_chunk_fwd_ctx,
 *     gdr_osdn_precond, gdr_sdm_fwd) take it from a caller-owned gdr_context (below);
 *     with a NULL context they run everything on `stream`.
 *   - Every tensor is dense and row-major.  q, k, k_w, v, o and the fp32 states
 *     must be 16-byte aligned; alpha, beta_k, beta_v need only their element
 *     alignment (so per-step slices of a gate array are accepted).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  Nothing synchronises inside the library.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     non-OK status nothing has been launched and no output was touched.
 *   - NaN / Inf inputs propagate; they are not detected.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
typedef enum gdr_status {
    GDR_OK = 0,
    GDR_EINVAL = -1,       /* NULL required pointer, bad enum, negative size, misalignment,
                              aliasing output, beta layout inconsistent with beta_mode */
    GDR_EUNSUPPORTED = -2, /* shape outside what the kernels implement (see below) */
    GDR_EWORKSPACE = -3,   /* workspace missing or smaller than gdr_chunk_fwd_workspace_size */
    GDR_EHIP = -4,         /* the HIP runtime reported an error at launch */
    GDR_ETOOLARGE = -5     /* gdr_chunk_fwd_noalloc: the call needs more scratch than the
                              library's static scratch array holds */
} gdr_status;

/* Element types. */
typedef enum gdr_dtype {
    GDR_BF16 = 0,          /* bfloat16; the library rounds to nearest-even when it stores one */
    GDR_F32 = 1
} gdr_dtype;

/* Forget-gate layout.  SCALAR: alpha [.., H]   CHANNEL: alpha [.., H, dk]. */
typedef enum gdr_alpha_mode { GDR_ALPHA_SCALAR = 0, GDR_ALPHA_CHANNEL = 1 } gdr_alpha_mode;

/* Write-strength layout.
 *   SCALAR: beta_k [.., H], beta_v must be NULL           (GDN / KDA / OSDN)
 *   SHARED: beta_k [.., H, dk] used for k and v, dk == dv,
 *           beta_v must be NULL                           (FG2-GDN)
 *   KV:     beta_k [.., H, dk] and beta_v [.., H, dv]     (FG2-GDN+) */
typedef enum gdr_beta_mode { GDR_BETA_SCALAR = 0, GDR_BETA_SHARED = 1, GDR_BETA_KV = 2 } gdr_beta_mode;

/* Flags (gdr_desc.flags), decode only (gdr_chunk_fwd returns GDR_EUNSUPPORTED for them); together they give the
 * delta-mem step [delta-mem page, section 2.A update rule, section 2.C read]:
 *   READ_BEFORE_WRITE:      o = S_{t-1}^T q        (the state before the gate and the write)
 *   UNDECAYED_PREDICTION:   S_t = Diag(alpha) S_{t-1} + w (vh - S_{t-1}^T u)^T
 *                           (the residual is taken against the state before the gate) */
#define GDR_FLAG_READ_BEFORE_WRITE 0x10
#define GDR_FLAG_UNDECAYED_PREDICTION 0x20

/* Problem descriptor.
 *   B, H  >= 0; T >= 0 (prefill only; ignored by decode).
 *   dk, dv: multiples of 8 in [8, 128]                      (else GDR_EUNSUPPORTED)
 *   chunk:  prefill chunk length, 16, 32 or 64              (else GDR_EUNSUPPORTED)
 *   io_dtype:   element type of q, k, k_w, v and o
 *   gate_dtype: element type of alpha, beta_k, beta_v
 * The bf16 matrix-core kernels serve io_dtype == GDR_BF16, dk == dv == 128,
 * chunk == 64, for every gate and beta layout (a faster pair for scalar alpha
 * and scalar beta); every other accepted shape runs the fp32 vector-ALU kernel. */
typedef struct gdr_desc {
    int32_t B, T, H, dk, dv;
    int32_t chunk;
    int32_t io_dtype;
    int32_t gate_dtype;
    int32_t alpha_mode;
    int32_t beta_mode;
    int32_t flags;
} gdr_desc;

/*
 * Execution context: a second stream on one device (default priority, non-blocking)
 * and the events that fork work onto it from the caller's stream and join it back
 * before the call's last launch.  Created and destroyed by the caller; the library
 * holds no reference to it between calls.  A call given a context leaves all of its
 * work ordered on `stream` (and capturable into a HIP graph of `stream`: the fork
 * and join pull the second stream into the capture).  One context serves one call at
 * a time: the caller must not pass the same context to two calls that may run
 * concurrently, nor use it elsewhere while a graph capture that used it is open.
 *
 * gdr_context_create: on the current device; *ctx receives the handle.
 *   GDR_EINVAL for a NULL ctx, GDR_EHIP if the runtime cannot create the stream or
 *   events (nothing is left allocated then).
 * gdr_context_destroy: waits for the second stream to drain, then releases it;
 *   NULL is accepted and does nothing.
 */
typedef struct gdr_context gdr_context;
int gdr_context_create(gdr_context **ctx);
int gdr_context_destroy(gdr_context *ctx);

/* Bytes of device workspace gdr_chunk_fwd needs for `desc` (0 if none).
 * Returns 0 for a descriptor gdr_chunk_fwd would reject. */
size_t gdr_chunk_fwd_workspace_size(const gdr_desc *desc);

/*
 * Prefill: run T tokens for every (b, h) and write every read-out.
 *
 *   q, k      [B, T, H, dk]  io_dtype   (required)
 *   k_w       [B, T, H, dk]  io_dtype   write key; NULL means k_w = k
 *   v         [B, T, H, dv]  io_dtype   (required)
 *   alpha     [B, T, H] or [B, T, H, dk]            gate_dtype (required)
 *   beta_k    [B, T, H] or [B, T, H, dk]            gate_dtype (required)
 *   beta_v    [B, T, H, dv]  gate_dtype, GDR_BETA_KV only, else NULL
 *   S0        [B, H, dk, dv] fp32 initial state; NULL means zero
 *   o         [B, T, H, dv]  io_dtype   output (required; must not overlap any input)
 *   ST        [B, H, dk, dv] fp32 final state; NULL means not written.
 *             ST == S0 is allowed (in-place resume); partial overlap is not.
 *   workspace device scratch of at least gdr_chunk_fwd_workspace_size(desc) bytes
 *             (may be NULL when that size is 0); its contents on entry do not matter.
 *
 * A T that is not a multiple of chunk is handled inside the kernels (the last
 * chunk is shorter).  T == 0 writes ST = S0 (or zeros) and no o.  Results are
 * deterministic: the same inputs give bit-identical outputs.
 */
int gdr_chunk_fwd(const gdr_desc *desc, const void *q, const void *k, const void *k_w,
                  const void *v, const void *alpha, const void *beta_k, const void *beta_v,
                  const float *S0, void *o, float *ST, void *workspace, size_t workspace_bytes,
                  void *stream);

/*
 * Prefill given an execution context: the arguments, results (bit for bit) and
 * workspace of gdr_chunk_fwd, plus `ctx` (NULL: exactly gdr_chunk_fwd).  The chunked
 * pass of the same pages; what the context changes is only where the work runs.
 * With a context, a call on the scalar-gate matrix-core path (scalar alpha and beta)
 * with fewer than 64 (b, h) pairs, at least 256 chunks per sequence and ST != NULL is
 * cut into blocks of chunks: the per-chunk preparation of every block runs on the
 * context's second stream while the state recurrence, which then occupies fewer than
 * all compute units, walks the blocks in order on `stream`, each block entering with the
 * state the block before left in ST.  Any other call runs on `stream` alone.
 * GDR_EINVAL also for a context created on another device.
 */
int gdr_chunk_fwd_ctx(const gdr_desc *desc, const void *q, const void *k, const void *k_w,
                      const void *v, const void *alpha, const void *beta_k, const void *beta_v,
                      const float *S0, void *o, float *ST, void *workspace, size_t workspace_bytes,
                      const gdr_context *ctx, void *stream);

/*
 * Prefill with no workspace argument and no allocation, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments, results and kernels as
 * gdr_chunk_fwd, except that the scratch gdr_chunk_fwd takes as `workspace` is a
 * static device array inside the library, GDR_NOALLOC_SCRATCH_BYTES (128 MiB) per
 * device, held by every device the library runs on until the process ends.
 *
 *   - A call whose gdr_chunk_fwd_workspace_size(desc) exceeds the array returns
 *     GDR_ETOOLARGE before anything is enqueued (the scalar-gate matrix-core path
 *     takes up to 5,216 chunks of 64 tokens over all (b, h), e.g. B=4, H=16, T=4096;
 *     the general-gate path up to 1,087).
 *   - The first call on a device looks the array's address up (a runtime symbol
 *     query, no allocation) and keeps it for that device.
 *   - Every call on one device shares that device's array and nothing in it needs
 *     clearing (each call writes what it reads).  Calls that may overlap on one device
 *     (concurrent streams, or host threads issuing at the same time) race on it and
 *     must be serialised by the caller.
 */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int gdr_chunk_fwd_noalloc(const gdr_desc *desc, const void *q, const void *k, const void *k_w,
                          const void *v, const void *alpha, const void *beta_k, const void *beta_v,
                          const float *S0, void *o, float *ST, void *stream);

/*
 * Decode: one token for every (b, h), applied in place to a resident state
 * (desc->flags may add GDR_FLAG_READ_BEFORE_WRITE and / or GDR_FLAG_UNDECAYED_PREDICTION).
 *
 *   q, k, k_w [B, H, dk], v [B, H, dv]          io_dtype (k_w NULL means k)
 *   alpha     [B, H] or [B, H, dk]              gate_dtype
 *   beta_k    [B, H] or [B, H, dk]; beta_v [B, H, dv] (GDR_BETA_KV only)
 *   S         [B, H, dk, dv] fp32, read and overwritten with the new state
 *   o         [B, H, dv] io_dtype, o = S_new^T q (must not overlap any input)
 * desc->T and desc->chunk are ignored.
 */
int gdr_decode_step(const gdr_desc *desc, const void *q, const void *k, const void *k_w,
                    const void *v, const void *alpha, const void *beta_k, const void *beta_v,
                    float *S, void *o, void *stream);

/*
 * Prefill that also keeps the state at every segment end, for Memory Caching
 * [Memory Caching: RNNs with Growing Memory, section 2 (segmentation, cache of states)]:
 * the sequence is cut into segments of seg_len tokens and the state after the
 * last token of each complete segment is stored.
 *
 *   seg_len   tokens per segment, a positive multiple of desc->chunk (else GDR_EINVAL)
 *   ckpt      [B, H, N, dk, dv] fp32, N = floor(T / seg_len): slot s holds the state
 *             after token (s + 1) * seg_len - 1.  May be NULL when N == 0; must not
 *             overlap any input, o or ST.
 * Everything else is exactly gdr_chunk_fwd (same outputs, same workspace size).
 */
int gdr_chunk_fwd_ckpt(const gdr_desc *desc, const void *q, const void *k, const void *k_w,
                       const void *v, const void *alpha, const void *beta_k, const void *beta_v,
                       const float *S0, void *o, float *ST, int32_t seg_len, float *ckpt,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Memory-Caching read-out [Memory Caching: RNNs with Growing Memory, sections 2 (retrieval) and 3
 * (residual memory, gated residual memory; memory soup equals the gated form for
 * a linear memory; sparse selective caching is the gated form with most gates 0)]:
 *
 *   o_out[t] = o_in[t] + sum over s < min(floor(t / seg_len), n_ckpt) of
 *              g[t, s] * M_s^T q[t]
 *
 * for every (b, h), with M_s = ckpt[b, h, s] (a dk x dv state, M_s^T q reads it
 * like the online state) and g[t, s] = gates[b, t, h, s], or 1 for every s when
 * gates is NULL (residual memory).  Token t sees only the segments that end
 * before its own segment starts.
 *
 *   q         [B, T, H, dk] bf16 (required)
 *   ckpt      [B, H, n_ckpt, dk, dv] fp32 (required when n_ckpt > 0)
 *   gates     [B, T, H, n_ckpt] fp32 or NULL
 *   o_in      [B, T, H, dv] bf16, or NULL for zero; may equal o_out (in place)
 *   o_out     [B, T, H, dv] bf16 (required); the sum is formed in fp32 and rounded once
 *   workspace at least gdr_mc_readout_workspace_size() bytes
 * Supported: io_dtype bf16, dk == dv == 128 (else GDR_EUNSUPPORTED).  desc->chunk,
 * alpha_mode, beta_mode and gate_dtype are not used.  Gate rows that are zero for
 * a whole 64-token tile skip that cache's products.
 */
size_t gdr_mc_readout_workspace_size(const gdr_desc *desc, int32_t n_ckpt);
int gdr_mc_readout(const gdr_desc *desc, const void *q, const float *ckpt, int32_t n_ckpt,
                   int32_t seg_len, const float *gates, const void *o_in, void *o_out,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * OSDN phase 1: the preconditioner scan that produces the write keys of the
 * chunked pass [OSDN page, section 2.2 (hypergradient surrogate, two phases),
 * section 2.3 (retention gate of the preconditioner)].  For every (b, h), with
 * the diagonal preconditioner d (d0, or all ones when d0 is NULL) and per token t
 *
 *     k_w[t] = d_t (.) k[t]
 *     d_{t+1} = r[t] d_t + eta beta[t] (1 - beta[t] <d_t, k[t]^2>) k[t]^2 / |k[t]|^2
 *
 * (online gradient descent on the surrogate; r == 1 is plain OSDN; a zero key
 * leaves d scaled by r only).  q_geo[b, h] = exp(mean_t log (1 - beta[t] <d_t,
 * k[t]^2>)^2), the geometric mean of phase 2's per-token loss ratio.
 *
 *   k      [B, T, H, dk] io_dtype (required); k_w [B, T, H, dk] io_dtype output
 *   beta   [B, T, H] gate_dtype (required; desc->beta_mode must be GDR_BETA_SCALAR)
 *   r      [B, T, H] gate_dtype retention in [0, 1], or NULL for 1 (values below
 *          1e-30 act as 1e-30, which for d's update is indistinguishable from 0)
 *   d0     [B, H, dk] fp32 or NULL;  dT [B, H, dk] fp32 final preconditioner or NULL
 *   qgeo   [B, H] fp32 or NULL (1 when T == 0)
 *   workspace at least gdr_osdn_precond_workspace_size() bytes
 *   ctx    an execution context of the current device, or NULL
 * dk: multiple of 8 in [8, 128].  desc->dv, chunk and alpha_mode are not used.
 * With a context and T >= 16,384 (256 chunks of 64) the chunk solve and the
 * emission of the write keys run on the context's second stream beside the
 * sequential scan, block by block; the results are the same bit for bit.  A
 * context of another device gives GDR_EINVAL.
 */
size_t gdr_osdn_precond_workspace_size(const gdr_desc *desc);
int gdr_osdn_precond(const gdr_desc *desc, const void *k, const void *beta, const void *r, float eta,
                     const float *d0, void *k_w, float *dT, float *qgeo, void *workspace,
                     size_t workspace_bytes, gdr_context *ctx, void *stream);

/*
 * Sparse Delta Memory [Resumo Técnico: Sparse Delta Memory (SDM), Mecanismo Central
 * items 1-4]: per (b, h) an explicit table M of N = n * n slots x dv, read and
 * written sparsely.  For every token t in order, with the slot score of
 * i = a * n + b equal to s1[a] + s2[b] (fp32) from two half-score vectors:
 *   - the W best slots by the key scores ks[t] are written:
 *       M[i] <- alpha[t] M[i] + beta[t] w_i (v[t] - alpha[t] M[i]),  w = softmax of
 *     their scores; every other slot is left as it is;
 *   - o[t] = sum_r w'_r M[i_r] over the R best slots by the query scores qs[t]
 *     (softmax weights), read after the write.
 * Ranking: higher score first, equal scores by lower slot index.  Selection uses
 * topk(s1 (+) s2) = topk(topk(s1) (+) topk(s2)).
 *
 *   ks, qs    [B, T, H, 2, n] fp32 half scores (required)
 *   v         [B, T, H, dv] io_dtype; o [B, T, H, dv] io_dtype output
 *   alpha, beta [B, T, H] gate_dtype
 *   M         [B, H, n * n, dv] fp32, the initial table (e.g. a learned M_0) on entry,
 *             the final table on return (updated in place)
 *   w_slots, r_slots [B, T, H, W] / [B, T, H, R] int32 outputs (selected slots, best
 *             first) or NULL
 *   workspace at least gdr_sdm_workspace_size() bytes
 *   ctx       an execution context of the current device, or NULL
 * Supported: dv == 128, 1 <= n <= 1024, 1 <= W, R <= min(128, n * n) (else
 * GDR_EUNSUPPORTED).  desc->dk, chunk, alpha_mode and beta_mode are not used.
 * With a context and T >= 1024 the selection of later token blocks runs on the
 * context's second stream beside the table pass (the results are the same bit for
 * bit); a context of another device gives GDR_EINVAL.
 */
size_t gdr_sdm_workspace_size(const gdr_desc *desc, int32_t n, int32_t W, int32_t R);
int gdr_sdm_fwd(const gdr_desc *desc, int32_t n, int32_t W, int32_t R, const float *ks, const float *qs,
                const void *v, const void *alpha, const void *beta, float *M, void *o, int32_t *w_slots,
                int32_t *r_slots, void *workspace, size_t workspace_bytes, gdr_context *ctx, void *stream);

/*
 * delta-mem context pass [delta-mem: Efficient Online Memory for Large Language
 * Models, section 2.A (update rule), 2.C (read before the write), 2.D (write
 * granularities)].  Per (b, h) an r x r fp32 memory M, row a predicting value
 * component a as M k.  Tokens are grouped into segments; every token t of a segment
 * reads the memory as it was before the segment's write, and the segment is then
 * written once:
 *     read   r_t = M q_t
 *     write  M <- lam M + beta (vbar - M kbar) kbar^T
 * with kbar, vbar the means of the segment's keys and values and lam, beta the gates
 * stored at the segment's last token (the gates of its other tokens are not read).
 *   - token-state write (TSW): seg_end NULL, every token is its own segment (the
 *     page's per-token step with the read before the write);
 *   - sequence-state write (SSW): seg_end[b, t] != 0 marks the last token of a
 *     segment (a message); the last token of the sequence always closes one;
 *   - multi-state write (MSW): J sub-states per group of heads, heads h = g J + j
 *     (j < J) of one group each written as above from their own q, k, v and gates;
 *     the group's read is the sum of its J sub-state reads.
 *
 *   q, k, v   [B, T, H, r] io_dtype (16-byte aligned)
 *   lam, beta [B, T, H] gate_dtype
 *   seg_end   [B, T] uint8 or NULL
 *   M         [B, H, r, r] fp32, the memory before the pass on entry, after it on return
 *   out       [B, T, H / J, r] io_dtype (bf16 rounded to nearest even)
 * desc: B, T, H >= 0; dk == dv == r; alpha_mode, beta_mode scalar; flags 0; chunk
 * not used.  Supported: r = 8 (J = 1, 2, 4, 8) or r = 16 (J = 1, 2, 4), H a multiple
 * of J, each of q, k, v at most 2^31 - 1 bytes (else GDR_EUNSUPPORTED / GDR_EINVAL).
 * Outputs must not overlap the inputs.
 * Runs on `stream`; returns once the work is enqueued.
 */
int gdr_dmem_fwd(const gdr_desc *desc, int32_t J, const void *q, const void *k, const void *v, const void *lam,
                 const void *beta, const uint8_t *seg_end, float *M, void *out, void *stream);

/* Which prefill kernel `desc` selects: 1 = bf16 matrix-core kernel,
 * 2 = fp32 vector-ALU kernel, or a negative gdr_status if desc is rejected. */
int gdr_chunk_fwd_path(const gdr_desc *desc);

/* Static, NUL-terminated description of a status code. */
const char *gdr_status_string(int status);

/* ABI version: (major << 16) | minor. */
int gdr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
