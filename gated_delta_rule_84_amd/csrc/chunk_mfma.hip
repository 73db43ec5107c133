// chunk_mfma.hip -- chunkwise WY / UT-transform prefill on gfx950 bf16 matrix cores.
//
// Serves bf16 q / k / k_w / v, dk == dv == 128, chunk 64.  Per chunk of n <= 64
// tokens with g_t the cumulative log-decay inside the chunk, erase key u, write
// key w and written value vh (scalar beta: u = k, w = beta k_w, vh = v):
//     A  = strictly-lower( u_t . (e^{g_t - g_s} (.) w_s) )      block Gram matrix
//     Tm = (I + A)^{-1}                                          UT transform
//     P  = lower-incl-diag( q_t . (e^{g_t - g_s} (.) w_s) )      intra-chunk scores
//     R  = Vh - (e^{g_t} (.) U) S                                residual before the chunk
//     D  = Tm R                                                  per-token residuals
//     O  = (e^{g_t} (.) Q) S + P D
//     S <- Diag(e^{g_C}) S + sum_s (e^{g_C - g_s} (.) w_s) D_s^T
// (the WY factors of the pages' chunk-parallel form are Tm (e^g (.) U) and Tm Vh;
// the write key replaces the key in the Gram matrix and the scores exactly as the
// OSDN page, section 2.1 states; FG2-GDN page, section 3).  A scalar decay is a
// per-row / per-column factor applied in fp32 after the product; a decay per key
// channel is folded into the key-side operands before it.
//
// Kernels, two per call:
//  * prep (scalar alpha and beta) -- one 256-thread block per chunk, fully
//        parallel: the Gram and score products on MFMA from the raw bf16 keys,
//        exact-difference decay weights, the UT transform (diagonal blocks by
//        forward substitution, off-diagonal blocks on fp32 MFMA) and a per-chunk
//        record: Tm (bf16), P as two bf16 terms, e^{g_t}, beta_s e^{g_C - g_s},
//        e^{g_C}, g_t, beta_t.
//  * prep (general gates) -- the same for a decay per key channel and / or beta
//        vectors: it forms U = u (.) e^{g}, Q = q (.) e^{g}, W = w (.) e^{g_C - g}
//        as two bf16 terms each (the record carries them), takes the Gram and
//        score products on the factored decay, and the same UT transform.
//  * state -- one workgroup per (batch * head, 32 value columns), walking the
//        chunks in order: two chain waves carry Y, R, D and the state update for
//        16 value columns each, two side waves copy operands into LDS and form the
//        output (wave-specialised kernels, scalar and general-gate variants; a
//        four-wave kernel that splits every product over the waves is kept as an
//        alternative for testing).  Every product that touches the state or a
//        residual uses a two-term bf16 split of the fp32 operand (hi + lo), so the
//        state path keeps ~16 mantissa bits.
// For few heads and long sequences (the state kernel then leaves CUs free) the
// chunks are cut into blocks: the prep of every block runs on a side stream and the
// state kernel is launched once per block on the caller's stream, after its block's
// prep, carrying the state through S_T (launch_blocked below).
//
// MFMA operand layouts (v_mfma_f32_16x16x32_bf16, lane l, r = l % 16, q = l / 16):
//   A (16 x 32): lane holds A[r][8q .. 8q+7];  B (32 x 16): B[8q .. 8q+7][r];
//   C (16 x 16): lane holds C[4q .. 4q+3][r].
#include <stdlib.h>

#include "gdr_device.hpp"
#include "gdr_internal.hpp"
#include "gdr_mfma.hpp"
#include "gdr_ut.hpp"

namespace gdr {
namespace {


constexpr int kC = 64;
constexpr int kD = 128;
constexpr int kThreads = 256;

// per-chunk workspace record (bytes)
constexpr int kRecT = 0;        // bf16 [64][64]  Tm
constexpr int kRecPhi = 8192;   // bf16 [64][64]  P, leading term
constexpr int kRecPlo = 16384;  // bf16 [64][64]  P, remainder
constexpr int kRecGam = 24576;  // f32 [64]  e^{g_t}
constexpr int kRecFac = 24832;  // f32 [64]  beta_s e^{g_C - g_s}, 0 past the chunk end
constexpr int kRecGC = 25088;   // f32       e^{g_C}
constexpr int kRecGlog = 25216; // f32 [64]  g_t (cumulative log decay inside the chunk)
constexpr int kRecBeta = 25472; // f32 [64]  beta_t, 0 past the chunk end
constexpr int kRecBytes = 25728;

// per-chunk workspace record of the general-gate path (channel decay and/or beta
// vectors): every key-side operand already carries its decay and beta, as two bf16
// terms (hi + lo) each
constexpr int kRcT = 0;          // bf16 [64][64]   Tm
constexpr int kRcPh = 8192;      // bf16 [64][64]   P, leading term
constexpr int kRcPl = 16384;     // bf16 [64][64]   P, remainder
constexpr int kRcUh = 24576;     // bf16 [64][128]  U_t = u_t (.) e^{g_t}              (erase key)
constexpr int kRcUl = 40960;
constexpr int kRcQh = 57344;     // bf16 [64][128]  Q_t = q_t (.) e^{g_t}
constexpr int kRcQl = 73728;
constexpr int kRcWh = 90112;     // bf16 [64][128]  W_t = w_t (.) e^{g_C - g_t}        (write key)
constexpr int kRcWl = 106496;
constexpr int kRcGC = 122880;    // f32 [128]       e^{g_C} per key channel
constexpr int kRcBytes = 123392;


// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), both round-to-nearest-even.
__device__ __forceinline__ void split8(const float *x, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const __bf16 h = (__bf16)x[j];
        hi[j] = h;
        lo[j] = (__bf16)(x[j] - (float)h);
    }
}

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ float ld_gate(const void *p, long i, int bf16) { return ld_elem(p, i, bf16); }


// Workgroup barrier ordered for LDS only: the fences are restricted to the local
// address space, so the barrier waits for this wave's LDS traffic but not for its
// outstanding global loads into registers, which stay in flight across it.  Copies
// into LDS (global_load_lds) write LDS, so the compiler waits for those too.
// __syncthreads() would drain every outstanding global load at each barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// pieces shared by the two prep kernels (256 threads, four waves)
// ---------------------------------------------------------------------------
// The lower-triangular Tm (fp32 rows in Ts, unit diagonal implied) to the record as
// bf16 rows of 64, 16 bytes per store.
__device__ __forceinline__ void store_ut(char *dst, const float (*Ts)[kC + 8], const int tid) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {  // 512 pieces of 8 bf16
        const int pc = tid + 256 * m, row = pc >> 3, c0 = (pc & 7) * 8;
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ca = c0 + 2 * j, cb = ca + 1;
            const float va = ca < row ? Ts[row][ca] : (ca == row ? 1.f : 0.f);
            const float vb = cb < row ? Ts[row][cb] : (cb == row ? 1.f : 0.f);
            o[j] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)va) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)vb) << 16);
        }
        *reinterpret_cast<u32x4 *>(dst + (row * kC + c0) * 2) = o;
    }
}

// The two bf16 terms of P (rows of 64 in LDS, pitch kC + 8) to the record.
__device__ __forceinline__ void store_p(char *dh, char *dl, const uint16_t (*Ph)[kC + 8],
                                        const uint16_t (*Pl)[kC + 8], const int tid) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int pc = tid + 256 * m, row = pc >> 3, c0 = (pc & 7) * 8;
        *reinterpret_cast<u32x4 *>(dh + (row * kC + c0) * 2) = *reinterpret_cast<const u32x4 *>(&Ph[row][c0]);
        *reinterpret_cast<u32x4 *>(dl + (row * kC + c0) * 2) = *reinterpret_cast<const u32x4 *>(&Pl[row][c0]);
    }
}

// ---------------------------------------------------------------------------
// prep kernel
// ---------------------------------------------------------------------------
// GBF16: the gates are bf16 (compile time, so the gate loads carry no branch)
template <bool GBF16>
__global__ void __launch_bounds__(kThreads, 4) gdr_prep_kernel(ChunkParams p, int NT) {
    __shared__ float gl[kC], bl[kC];
    __shared__ __align__(16) float As[kC][kC + 4];  // Gram matrix, strictly lower part (first: the write keys)
    __shared__ __align__(16) float Ts[kC][kC + 8];  // UT transform; first holds the two P terms
    __shared__ __align__(16) float Xs[4][16][16];  // the four 16 x 16 blocks of A_2:4,0:2 T_0:2,0:2
    uint16_t(*Ph)[kC + 8] = reinterpret_cast<uint16_t(*)[kC + 8]>(&Ts[0][0]);
    uint16_t(*Pl)[kC + 8] = reinterpret_cast<uint16_t(*)[kC + 8]>(&Ts[kC / 2][0]);

    const int blk = blockIdx.x, nc = p.c1 - p.c0;  // chunks c0 .. c1 - 1 of every (batch, head)
    const int c = p.c0 + blk % nc, bh = blk / nc;
    const int b = bh / p.H, h = bh % p.H;
    const int t0 = c * kC, n = min(kC, p.T - t0);
    const int tid = threadIdx.x, l = tid & 63, r = l & 15, q = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    auto tok = [&](int t) -> long { return ((long)b * p.T + t0 + t) * p.H + h; };
    const uint16_t *K = static_cast<const uint16_t *>(p.k);
    const uint16_t *KW = static_cast<const uint16_t *>(p.kw);
    const uint16_t *Q = static_cast<const uint16_t *>(p.q);

    // gates first (rows past the chunk end read the last row, replaced below), so
    // that the gate math waits for them alone, not for the tiles issued after them
    const float a_raw = ld_gate(p.alpha, tok(min(l, n - 1)), GBF16);
    const float b_raw = ld_gate(p.beta_k, tok(min(l, n - 1)), GBF16);
    // Gram row-block I = w (tiles J <= w) and score row-block IP = 3 - w (tiles J <= IP)
    const int IG = w, IP = 3 - w;
    // rows past the end of a short chunk read the last valid row; their Gram and
    // score entries are masked below
    auto rowt = [&](int t) -> long { return tok(min(t, n - 1)) * kD; };
    u32x4 qa[4];
    {
        const int tp = 16 * IP + r;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qa[kk] = ld16(Q + rowt(tp) + kk * 32 + 8 * q);
    }
    // the write-key tile is copied once into LDS (the space As takes later; wave w copies
    // rows 16 w .. 16 w + 15, 16-byte pieces of row t stored at piece ^ (t & 15)) and
    // every wave reads its B fragments from there; the key tile, when it is a different
    // tensor, likewise into the space Ts takes later -- each tile is read from HBM once
    const bool sep = p.kw != p.k;
    uint16_t(*KWs)[kD] = reinterpret_cast<uint16_t(*)[kD]>(&As[0][0]);
    uint16_t(*Ks)[kD] = sep ? reinterpret_cast<uint16_t(*)[kD]>(&Ts[0][0]) : KWs;
#pragma unroll
    for (int u = 4 * w; u < 4 * w + 4; ++u) {
        const int t = 4 * u + (l >> 4), pc = (l & 15) ^ (t & 15);
        dma16(KW + rowt(t) + 8 * pc, &KWs[4 * u][0]);
        if (sep) dma16(K + rowt(t) + 8 * pc, &Ks[4 * u][0]);
    }
    __syncthreads();  // drains this block's copies and loads
    u32x4 ka[4];
    {
        const int tg = 16 * IG + r;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) ka[kk] = *reinterpret_cast<const u32x4 *>(&Ks[tg][8 * ((4 * kk + q) ^ (tg & 15))]);
    }
    f32x4 accG[4], accP[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        accG[J] = f32x4{0.f, 0.f, 0.f, 0.f};
        accP[J] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 kb = as_bf16x8(*reinterpret_cast<const u32x4 *>(&KWs[16 * J + r][8 * ((4 * kk + q) ^ r)]));
            if (J <= IG) accG[J] = mfma(as_bf16x8(ka[kk]), kb, accG[J]);
            if (J <= IP) accP[J] = mfma(as_bf16x8(qa[kk]), kb, accP[J]);
        }
    }
    // cumulative log decay and beta (wave 0)
    if (w == 0) {
        float la = l < n ? logf(a_raw) : 0.f;
        const float be = l < n ? b_raw : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(la, off);
            if (l >= off) la += y;
        }
        gl[l] = la;
        bl[l] = be;
    }

    __syncthreads();

    // decay / beta weights; Gram to LDS (fp32), scores to LDS as two bf16 terms.
    // Every LDS read is hoisted ahead of the stores so none waits behind them.
    float gG[4], gP[4], gS[4], bS[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        gG[i] = gl[16 * IG + 4 * q + i];
        gP[i] = gl[16 * IP + 4 * q + i];
        gS[i] = gl[16 * i + r];
        bS[i] = bl[16 * i + r];
    }
#pragma unroll
    for (int J = 0; J < 4; ++J) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = 16 * J + r;
            // computed for every lane and selected (no divergent branch); the exponent is
            // clamped at 0, which changes only entries the mask discards (g decreases in t)
            if (J <= IG) {
                const int t = 16 * IG + 4 * q + i;
                const float v = accG[J][i] * bS[J] * __expf(fminf(gG[i] - gS[J], 0.f));
                As[t][s] = (s < t && t < n) ? v : 0.f;
            }
            const int tp = 16 * IP + 4 * q + i;
            float pv = 0.f;
            if (J <= IP) {
                const float v = accP[J][i] * bS[J] * __expf(fminf(gP[i] - gS[J], 0.f));
                pv = (s <= tp && tp < n) ? v : 0.f;
            }
            const __bf16 hi = (__bf16)pv;
            const __bf16 lo = (__bf16)(pv - (float)hi);
            Ph[tp][s] = __builtin_bit_cast(uint16_t, hi);
            Pl[tp][s] = __builtin_bit_cast(uint16_t, lo);
        }
    }
    __syncthreads();
    char *rec = static_cast<char *>(p.ws) + ((long)bh * NT + c) * kRecBytes;
    store_p(rec + kRecPhi, rec + kRecPlo, Ph, Pl, tid);
    __syncthreads();

    ut_transform(As, Ts, Xs, w, l);

    // write the rest of the record
    store_ut(rec + kRecT, Ts, tid);
    if (tid < kC) {
        float *gam = reinterpret_cast<float *>(rec + kRecGam);
        float *fac = reinterpret_cast<float *>(rec + kRecFac);
        gam[tid] = __expf(gl[tid]);
        fac[tid] = tid < n ? bl[tid] * __expf(gl[n - 1] - gl[tid]) : 0.f;
        if (tid == 0) *reinterpret_cast<float *>(rec + kRecGC) = __expf(gl[n - 1]);
        reinterpret_cast<float *>(rec + kRecGlog)[tid] = gl[tid];
        reinterpret_cast<float *>(rec + kRecBeta)[tid] = bl[tid];
    }
}


// ---------------------------------------------------------------------------
// prep kernel, general gates
// ---------------------------------------------------------------------------
// One 256-thread block per chunk for a forget gate per key channel (ACH) and / or
// beta vectors (BVEC; u = sqrt(beta^k) (.) k, w = sqrt(beta^k) (.) k_w; a scalar beta
// gives u = k, w = beta k_w).  With g_t the per-channel cumulative log decay inside
// the chunk, the decay factor e^{g_t - g_s} of the Gram matrix and of the scores
// splits per channel into a row and a column factor, so both are plain products of
// rescaled operands:
//     A = strictly-lower( U What^T ),  P = lower-incl-diag( Q What^T ),
//     U = u (.) e^{g_t},  Q = q (.) e^{g_t},  What = w (.) e^{-g_t}
// (FG2-GDN page, section 3: the factored decay of the chunkwise form).  The factor
// e^{-g_t} bounds the decay one chunk may accumulate per channel (about e^{-80}).
// The record carries U, Q and W = w (.) e^{g_C - g_t} as two bf16 terms, Tm and P
// as for the scalar path, and e^{g_C} per channel.
template <bool GBF16, bool ACH, bool BVEC>
__global__ void __launch_bounds__(kThreads) gdr_prep_chan_kernel(ChunkParams p, int NT) {
    // the cumulative log decay g[t][i] is dead once the operands are formed; the
    // Gram and UT arrays take its place
    __shared__ __align__(16) float pool[kC * (kC + 4) + kC * (kC + 8)];
    __shared__ __align__(16) uint16_t Whs[kC][kD + 8], Wls[kC][kD + 8];  // What, two bf16 terms
    __shared__ __align__(16) float Xs[4][16][16];
    float(*gs)[kD + 4] = reinterpret_cast<float(*)[kD + 4]>(pool);
    float(*As)[kC + 4] = reinterpret_cast<float(*)[kC + 4]>(pool);
    float(*Ts)[kC + 8] = reinterpret_cast<float(*)[kC + 8]>(pool + kC * (kC + 4));
    uint16_t(*Ph)[kC + 8] = reinterpret_cast<uint16_t(*)[kC + 8]>(&Ts[0][0]);
    uint16_t(*Pl)[kC + 8] = reinterpret_cast<uint16_t(*)[kC + 8]>(&Ts[kC / 2][0]);
    static_assert(kC * (kD + 4) <= kC * (kC + 4) + kC * (kC + 8), "pool holds g");

    const int blk = blockIdx.x;
    const int c = blk % NT, bh = blk / NT;
    const int b = bh / p.H, h = bh % p.H;
    const int t0 = c * kC, n = min(kC, p.T - t0);
    const int tid = threadIdx.x, l = tid & 63, r = l & 15, q = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    auto tok = [&](int t) -> long { return ((long)b * p.T + t0 + min(t, n - 1)) * p.H + h; };
    const uint16_t *K = static_cast<const uint16_t *>(p.k);
    const uint16_t *KW = static_cast<const uint16_t *>(p.kw);
    const uint16_t *Q = static_cast<const uint16_t *>(p.q);
    char *rec = static_cast<char *>(p.ws) + ((long)bh * NT + c) * kRcBytes;

    // g[t][i]: thread (i, half) scans 32 tokens of channel i; the upper half then adds
    // the lower half's total.  Tokens past the chunk end decay by 1.
    {
        const int i = tid & (kD - 1), hf = tid >> 7;
        float a[32];
#pragma unroll
        for (int j = 0; j < 32; ++j)
            a[j] = ACH ? ld_gate(p.alpha, tok(32 * hf + j) * kD + i, GBF16) : ld_gate(p.alpha, tok(32 * hf + j), GBF16);
        float run = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            run += 32 * hf + j < n ? logf(a[j]) : 0.f;
            gs[32 * hf + j][i] = run;
        }
        __syncthreads();
        if (hf == 1) {
            const float off = gs[31][i];
#pragma unroll
            for (int j = 0; j < 32; ++j) gs[32 + j][i] += off;
        }
        __syncthreads();
        if (tid < kD) reinterpret_cast<float *>(rec + kRcGC)[tid] = __expf(gs[n - 1][tid]);
    }

    // operands: lane (r, q) of wave w forms keys 32 kk + 8 q .. + 7 of token t = 16 w + r
    // for U, W, What and of token tp = 16 (3 - w) + r for Q; U and Q stay in registers
    // as the A fragments of the Gram and score row blocks w and 3 - w
    const int t = 16 * w + r, tp = 16 * (3 - w) + r;
    const long rt = tok(t) * kD, rtp = tok(tp) * kD;
    u32x4 uh[4], ul[4], qh[4], ql[4];
    {
        const float bsc = BVEC ? 0.f : ld_gate(p.beta_k, tok(t), GBF16);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int k0 = 32 * kk + 8 * q;
            const u32x4 kr = ld16(K + rt + k0), kwr = ld16(KW + rt + k0), qr = ld16(Q + rtp + k0);
            float u8[8], q8[8], wh8[8], wt8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t kb = kr[j >> 1], kwb = kwr[j >> 1], qb = qr[j >> 1];
                const float kv = __uint_as_float((j & 1) ? (kb & 0xffff0000u) : (kb << 16));
                const float kwv = __uint_as_float((j & 1) ? (kwb & 0xffff0000u) : (kwb << 16));
                const float qv = __uint_as_float((j & 1) ? (qb & 0xffff0000u) : (qb << 16));
                float u = kv, wv = kwv;
                if (BVEC) {
                    const float sb = sqrtf(ld_gate(p.beta_k, rt + k0 + j, GBF16));
                    u *= sb;
                    wv *= sb;
                } else {
                    wv *= bsc;
                }
                const float g = gs[t][k0 + j], gq = gs[tp][k0 + j], gC = gs[n - 1][k0 + j];
                u8[j] = t < n ? u * __expf(g) : 0.f;
                wh8[j] = t < n ? wv * __expf(-g) : 0.f;
                wt8[j] = t < n ? wv * __expf(gC - g) : 0.f;
                q8[j] = tp < n ? qv * __expf(gq) : 0.f;
            }
            bf16x8 h8, l8;
            split8(u8, h8, l8);
            uh[kk] = __builtin_bit_cast(u32x4, h8);
            ul[kk] = __builtin_bit_cast(u32x4, l8);
            *reinterpret_cast<u32x4 *>(rec + kRcUh + (t * kD + k0) * 2) = uh[kk];
            *reinterpret_cast<u32x4 *>(rec + kRcUl + (t * kD + k0) * 2) = ul[kk];
            split8(q8, h8, l8);
            qh[kk] = __builtin_bit_cast(u32x4, h8);
            ql[kk] = __builtin_bit_cast(u32x4, l8);
            *reinterpret_cast<u32x4 *>(rec + kRcQh + (tp * kD + k0) * 2) = qh[kk];
            *reinterpret_cast<u32x4 *>(rec + kRcQl + (tp * kD + k0) * 2) = ql[kk];
            split8(wt8, h8, l8);
            *reinterpret_cast<u32x4 *>(rec + kRcWh + (t * kD + k0) * 2) = __builtin_bit_cast(u32x4, h8);
            *reinterpret_cast<u32x4 *>(rec + kRcWl + (t * kD + k0) * 2) = __builtin_bit_cast(u32x4, l8);
            split8(wh8, h8, l8);
            *reinterpret_cast<u32x4 *>(&Whs[t][k0]) = __builtin_bit_cast(u32x4, h8);
            *reinterpret_cast<u32x4 *>(&Wls[t][k0]) = __builtin_bit_cast(u32x4, l8);
        }
    }
    __syncthreads();

    // Gram row block IG = w and score row block IP = 3 - w against What (three bf16
    // products per term pair: hi.hi + hi.lo + lo.hi)
    const int IG = w, IP = 3 - w;
    f32x4 accG[4], accP[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        accG[J] = f32x4{0.f, 0.f, 0.f, 0.f};
        accP[J] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            const bf16x8 bh8 = as_bf16x8(*reinterpret_cast<const u32x4 *>(&Whs[16 * J + r][32 * kk + 8 * q]));
            const bf16x8 bl8 = as_bf16x8(*reinterpret_cast<const u32x4 *>(&Wls[16 * J + r][32 * kk + 8 * q]));
            if (J <= IG) {
                accG[J] = mfma(as_bf16x8(uh[kk]), bh8, accG[J]);
                accG[J] = mfma(as_bf16x8(uh[kk]), bl8, accG[J]);
                accG[J] = mfma(as_bf16x8(ul[kk]), bh8, accG[J]);
            }
            if (J <= IP) {
                accP[J] = mfma(as_bf16x8(qh[kk]), bh8, accP[J]);
                accP[J] = mfma(as_bf16x8(qh[kk]), bl8, accP[J]);
                accP[J] = mfma(as_bf16x8(ql[kk]), bh8, accP[J]);
            }
        }
    __syncthreads();  // g is dead: As and Ts take its place

#pragma unroll
    for (int J = 0; J < 4; ++J) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = 16 * J + r;
            if (J <= IG) {
                const int tg = 16 * IG + 4 * q + i;
                As[tg][s] = (s < tg && tg < n) ? accG[J][i] : 0.f;
            }
            const int tq = 16 * IP + 4 * q + i;
            const float pv = (J <= IP && s <= tq && tq < n) ? accP[J][i] : 0.f;
            const __bf16 hi = (__bf16)pv;
            const __bf16 lo = (__bf16)(pv - (float)hi);
            Ph[tq][s] = __builtin_bit_cast(uint16_t, hi);
            Pl[tq][s] = __builtin_bit_cast(uint16_t, lo);
        }
    }
    __syncthreads();
    store_p(rec + kRcPh, rec + kRcPl, Ph, Pl, tid);
    __syncthreads();
    ut_transform(As, Ts, Xs, w, l);
    store_ut(rec + kRcT, Ts, tid);
}

// ---------------------------------------------------------------------------
// state kernel
// ---------------------------------------------------------------------------
// Operand orientation: every product takes a token-major input (rows of K, Q,
// Tm, P, or of the transposed write key) as the A operand and a
// [value column][k] bf16 array in LDS as the B operand.  A C tile then holds,
// per lane, 4 consecutive tokens (or key channels) of one value column, which
// is stored with one 8-byte write per term into exactly the layout the next
// product reads with 16-byte loads.  The fp32 -> (hi, lo) split is done once,
// by the lane that produced the value; consumers read ready bf16 fragments.
template <int BV>
struct ChunkFrags {
    u32x4 k[4], q[4];          // A operands: K and Q rows of this wave's 16 tokens
    u32x4 kw[4];               // rows of a separate write key (same layout as k)
    u32x4 t[2], ph[2], pl[2];  // rows of Tm and of the two P terms (second half: waves 2, 3)
    u32x4 v;                   // 16 bytes of this wave's 16 rows of the V tile
    u32x4 gf;                  // wave 0: 16 bytes of the record's e^{g_t} | fac_t | e^{g_C}
};

// Per wave and chunk: K and Q rows of its 16 tokens, its rows of Tm and P (the
// upper half of a triangular row block is never read), its 16 rows of the V tile
// and, for wave 0, the chunk's decay factors.  Token rows past the end of a short
// last chunk read the last valid row (their contributions are cancelled where
// they are used), so every load is unconditional per lane and the whole chunk is
// in flight while the previous one computes.
template <int BV>
__device__ __forceinline__ void load_chunk(const ChunkParams &p, int NT, int bh, int b, int h, int j0, int c,
                                           int tid, bool sep_kw, ChunkFrags<BV> &f) {
    constexpr int P8 = BV / 8;  // 16-byte pieces per token row of the V tile
    const int w = tid >> 6, l = tid & 63, r = l & 15, q = l >> 4;
    const int t0 = c * kC, n = min(kC, p.T - t0);
    auto tok = [&](int t) -> long { return ((long)b * p.T + t0 + min(t, n - 1)) * p.H + h; };
    const uint16_t *K = static_cast<const uint16_t *>(p.k);
    const uint16_t *Q = static_cast<const uint16_t *>(p.q);
    const uint16_t *V = static_cast<const uint16_t *>(p.v);
    const char *rec = static_cast<const char *>(p.ws) + ((long)bh * NT + c) * kRecBytes;
    const long rowk = tok(16 * w + r) * kD + 8 * q;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        f.k[kk] = ld16(K + rowk + kk * 32);
        f.q[kk] = ld16(Q + rowk + kk * 32);
    }
    if (sep_kw) {
        const uint16_t *KW = static_cast<const uint16_t *>(p.kw);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) f.kw[kk] = ld16(KW + rowk + kk * 32);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        if (kk == 1 && w < 2) break;
        const int off = ((16 * w + r) * kC + kk * 32 + 8 * q) * 2;
        f.t[kk] = ld16(rec + kRecT + off);
        f.ph[kk] = ld16(rec + kRecPhi + off);
        f.pl[kk] = ld16(rec + kRecPlo + off);
    }
    const int lv = l % (16 * P8);
    f.v = ld16(V + tok(16 * w + lv / P8) * kD + j0 + 8 * (lv % P8));
    if (w == 0) f.gf = ld16(rec + kRecGam + 16 * min(l, 32));
}


// fp32 x = hi + lo, both bf16 round-to-nearest-even, packed four to a u32x2.
__device__ __forceinline__ void split4(f32x4 x, u32x2 &hi, u32x2 &lo) {
    const uint32_t h0 = pk_bf16(x[0], x[1]), h1 = pk_bf16(x[2], x[3]);
    hi = u32x2{h0, h1};
    lo = u32x2{pk_bf16(x[0] - __uint_as_float(h0 << 16), x[1] - __uint_as_float(h0 & 0xffff0000u)),
               pk_bf16(x[2] - __uint_as_float(h1 << 16), x[3] - __uint_as_float(h1 & 0xffff0000u))};
}

// SEPKW: a separate write key is streamed (compile time, so that with k_w = k the
// key fragments are used directly and no register copy of a load in flight exists)
template <int BV, bool SEPKW>
__global__ void __launch_bounds__(kThreads, BV == 16 ? 2 : 1) gdr_state_kernel(ChunkParams p, int NT, int nbh) {
    constexpr int NJ = BV / 16;    // value-column tiles
    constexpr int NVB = kD / BV;
    constexpr int LZ = kD + 8;     // bf16 row pitch of the state operand arrays
    constexpr int LT = kC + 8;     // bf16 row pitch of the residual operand arrays
    constexpr int P8 = BV / 8;
    // write keys, channel-major; the 8-token column blocks of row ch are XOR-swizzled
    // by (ch / 8) % 8 so the transposing stores spread over the LDS banks
    __shared__ __align__(16) uint16_t kwT[2][kD][kC + 8];
    __shared__ __align__(16) float gfs[2][2 * kC + 4];            // e^{g_t} | fac_t | e^{g_C}
    __shared__ __align__(16) uint16_t VO[4][16][BV + 8];          // per wave: its V rows, then its O rows
    __shared__ __align__(16) uint16_t Zh[BV][LZ], Zl[BV][LZ];     // S^T as two bf16 terms
    __shared__ __align__(16) uint16_t Rh[BV][LT], Rl[BV][LT];     // R^T
    __shared__ __align__(16) uint16_t Dh[BV][LT], Dl[BV][LT];     // D^T
    __shared__ __align__(16) uint16_t Eh[BV][LT], El[BV][LT];     // (fac D)^T

    // block -> (head, value block): the NVB blocks of one head share an XCD (its L2)
    const int x = blockIdx.x;
    const int xcd = x & 7, rr = x >> 3;
    const int vb = rr % NVB, grp = rr / NVB;
    const int bh = grp * 8 + xcd;
    if (bh >= nbh) return;
    const int b = bh / p.H, h = bh % p.H, j0 = vb * BV;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 15, q = l >> 4;
    constexpr bool sep_kw = SEPKW;

    // state, C layout: sacc[ct][nt][i] = S[16 (2 w + ct) + 4 q + i][j0 + 16 nt + r]
    f32x4 sacc[2][NJ];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int nt = 0; nt < NJ; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = 16 * (2 * w + ct) + 4 * q + i;
                sacc[ct][nt][i] = p.S0 ? p.S0[((long)bh * kD + ch) * kD + j0 + 16 * nt + r] : 0.f;
            }

    auto put_z = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int nt = 0; nt < NJ; ++nt) {
                u32x2 hi, lo;
                split4(sacc[ct][nt], hi, lo);
                *reinterpret_cast<u32x2 *>(&Zh[16 * nt + r][16 * (2 * w + ct) + 4 * q]) = hi;
                *reinterpret_cast<u32x2 *>(&Zl[16 * nt + r][16 * (2 * w + ct) + 4 * q]) = lo;
            }
    };
    // the transposed write key comes from the key rows the wave already holds
    auto put_inputs = [&](const ChunkFrags<BV> &f, int buf) __attribute__((always_inline)) {
        const int s = 16 * w + r;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const u32x4 src = sep_kw ? f.kw[kk] : f.k[kk];
            const int col = (((s >> 3) ^ ((4 * kk + q) & 7)) << 3) | (s & 7);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                kwT[buf][32 * kk + 8 * q + 2 * j][col] = (uint16_t)(src[j] & 0xffffu);
                kwT[buf][32 * kk + 8 * q + 2 * j + 1][col] = (uint16_t)(src[j] >> 16);
            }
        }
        const int lv = l % (16 * P8);
        *reinterpret_cast<u32x4 *>(&VO[w][lv / P8][8 * (lv % P8)]) = f.v;
        if (w == 0 && l <= 32) *reinterpret_cast<u32x4 *>(&gfs[buf][4 * l]) = f.gf;
    };

    uint16_t *O = static_cast<uint16_t *>(p.o);
    // one chunk: consumes `cur` (loaded one chunk earlier) and fills `nxt`; the loop
    // below alternates the two buffers so no fragment is ever copied
    auto chunk_step = [&](const int c, ChunkFrags<BV> &cur, ChunkFrags<BV> &nxt) __attribute__((always_inline)) {
        const int t0 = c * kC, n = min(kC, p.T - t0);
        const int buf = c & 1;
        load_chunk<BV>(p, NT, bh, b, h, j0, min(c + 1, NT - 1), tid, sep_kw, nxt);
        const f32x4 gam = *reinterpret_cast<const f32x4 *>(&gfs[buf][16 * w + 4 * q]);

        // Y = K S and O0 = Q S for this wave's 16 tokens (S as two bf16 terms)
        f32x4 accY[NJ], accO[NJ];
#pragma unroll
        for (int nt = 0; nt < NJ; ++nt) {
            accY[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            accO[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int nt = 0; nt < NJ; ++nt) {
                const bf16x8 zh = as_bf16x8(*reinterpret_cast<const u32x4 *>(&Zh[16 * nt + r][32 * kk + 8 * q]));
                const bf16x8 zl = as_bf16x8(*reinterpret_cast<const u32x4 *>(&Zl[16 * nt + r][32 * kk + 8 * q]));
                accY[nt] = mfma(as_bf16x8(cur.k[kk]), zh, accY[nt]);
                accY[nt] = mfma(as_bf16x8(cur.k[kk]), zl, accY[nt]);
                accO[nt] = mfma(as_bf16x8(cur.q[kk]), zh, accO[nt]);
                accO[nt] = mfma(as_bf16x8(cur.q[kk]), zl, accO[nt]);
            }
        }
        // R = V - e^{g_t} Y, zero past the end of the chunk
#pragma unroll
        for (int nt = 0; nt < NJ; ++nt) {
            // V is read unconditionally (a read inside the tail test becomes a branch
            // with its own LDS round trip per element); rows past the end are zeroed after
            f32x4 rv;
#pragma unroll
            for (int i = 0; i < 4; ++i) rv[i] = bf16_to_f32(VO[w][4 * q + i][16 * nt + r]) - gam[i] * accY[nt][i];
            if (n < kC) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * w + 4 * q + i >= n) rv[i] = 0.f;
            }
            u32x2 hi, lo;
            split4(rv, hi, lo);
            *reinterpret_cast<u32x2 *>(&Rh[16 * nt + r][16 * w + 4 * q]) = hi;
            *reinterpret_cast<u32x2 *>(&Rl[16 * nt + r][16 * w + 4 * q]) = lo;
        }
        lds_barrier();

        // D = Tm R (Tm unit lower triangular: waves 0, 1 need only the first 32 tokens)
        f32x4 accD[NJ];
#pragma unroll
        for (int nt = 0; nt < NJ; ++nt) accD[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk == 1 && w < 2) break;
#pragma unroll
            for (int nt = 0; nt < NJ; ++nt) {
                const bf16x8 rh = as_bf16x8(*reinterpret_cast<const u32x4 *>(&Rh[16 * nt + r][32 * kk + 8 * q]));
                const bf16x8 rl = as_bf16x8(*reinterpret_cast<const u32x4 *>(&Rl[16 * nt + r][32 * kk + 8 * q]));
                accD[nt] = mfma(as_bf16x8(cur.t[kk]), rh, accD[nt]);
                accD[nt] = mfma(as_bf16x8(cur.t[kk]), rl, accD[nt]);
            }
        }
        const f32x4 fac = *reinterpret_cast<const f32x4 *>(&gfs[buf][kC + 16 * w + 4 * q]);
#pragma unroll
        for (int nt = 0; nt < NJ; ++nt) {
            u32x2 hi, lo;
            split4(accD[nt], hi, lo);
            *reinterpret_cast<u32x2 *>(&Dh[16 * nt + r][16 * w + 4 * q]) = hi;
            *reinterpret_cast<u32x2 *>(&Dl[16 * nt + r][16 * w + 4 * q]) = lo;
            split4(accD[nt] * fac, hi, lo);
            *reinterpret_cast<u32x2 *>(&Eh[16 * nt + r][16 * w + 4 * q]) = hi;
            *reinterpret_cast<u32x2 *>(&El[16 * nt + r][16 * w + 4 * q]) = lo;
        }
        lds_barrier();

        // O = e^{g_t} O0 + P D, staged through this wave's rows of VO, stored 16 bytes per lane
#pragma unroll
        for (int nt = 0; nt < NJ; ++nt) accO[nt] *= gam;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk == 1 && w < 2) break;
#pragma unroll
            for (int nt = 0; nt < NJ; ++nt) {
                const bf16x8 dh = as_bf16x8(*reinterpret_cast<const u32x4 *>(&Dh[16 * nt + r][32 * kk + 8 * q]));
                const bf16x8 dl = as_bf16x8(*reinterpret_cast<const u32x4 *>(&Dl[16 * nt + r][32 * kk + 8 * q]));
                accO[nt] = mfma(as_bf16x8(cur.ph[kk]), dh, accO[nt]);
                accO[nt] = mfma(as_bf16x8(cur.ph[kk]), dl, accO[nt]);
                accO[nt] = mfma(as_bf16x8(cur.pl[kk]), dh, accO[nt]);
            }
        }
#pragma unroll
        for (int nt = 0; nt < NJ; ++nt)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const uint32_t o2 = pk_bf16(accO[nt][i], accO[nt][i + 1]);
                VO[w][4 * q + i][16 * nt + r] = (uint16_t)(o2 & 0xffffu);
                VO[w][4 * q + i + 1][16 * nt + r] = (uint16_t)(o2 >> 16);
            }
        {
            const int lv = l % (16 * P8);
            const int t = 16 * w + lv / P8;
            const u32x4 ov = *reinterpret_cast<const u32x4 *>(&VO[w][lv / P8][8 * (lv % P8)]);
            if (l < 16 * P8 && t < n)
                *reinterpret_cast<u32x4 *>(O + (((long)b * p.T + t0 + t) * p.H + h) * kD + j0 + 8 * (lv % P8)) = ov;
        }

        // S <- e^{g_C} S + K_w^T (fac D): channels 32 w .. 32 w + 31 of this wave
        const float gC = gfs[buf][2 * kC];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int nt = 0; nt < NJ; ++nt) sacc[ct][nt] *= gC;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 ka[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const int ch = 16 * (2 * w + ct) + r;
                const int col = ((4 * kk + q) ^ ((ch >> 3) & 7)) << 3;
                ka[ct] = as_bf16x8(*reinterpret_cast<const u32x4 *>(&kwT[buf][ch][col]));
            }
#pragma unroll
            for (int nt = 0; nt < NJ; ++nt) {
                const bf16x8 eh = as_bf16x8(*reinterpret_cast<const u32x4 *>(&Eh[16 * nt + r][32 * kk + 8 * q]));
                const bf16x8 el = as_bf16x8(*reinterpret_cast<const u32x4 *>(&El[16 * nt + r][32 * kk + 8 * q]));
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    sacc[ct][nt] = mfma(ka[ct], eh, sacc[ct][nt]);
                    sacc[ct][nt] = mfma(ka[ct], el, sacc[ct][nt]);
                }
            }
        }
        put_z();
        put_inputs(nxt, (c + 1) & 1);
        lds_barrier();
    };

    ChunkFrags<BV> fa, fb;
    load_chunk<BV>(p, NT, bh, b, h, j0, 0, tid, sep_kw, fa);
    put_inputs(fa, 0);
    put_z();
    __syncthreads();
    int c = 0;
    for (; c + 1 < NT; c += 2) {
        chunk_step(c, fa, fb);
        chunk_step(c + 1, fb, fa);
    }
    if (c < NT) chunk_step(c, fa, fb);

    if (p.ST) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int nt = 0; nt < NJ; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ch = 16 * (2 * w + ct) + 4 * q + i;
                    p.ST[((long)bh * kD + ch) * kD + j0 + 16 * nt + r] = sacc[ct][nt][i];
                }
    }
}

// ---------------------------------------------------------------------------
// state kernel, wave-specialised form
// ---------------------------------------------------------------------------
// Four waves per workgroup, one per SIMD, for value columns j0 .. j0 + 31 of one
// (batch, head).  Waves 0 and 1 ("chain" waves) own value columns
// j0 + 16 w .. j0 + 16 w + 15 for all 64 tokens and 128 key channels and carry
// only the sequential part of a chunk:
//     Y = K S,  R = V - Diag(e^g) Y,  D = Tm R,  S <- e^{g_C} S + K_w^T (fac D).
// The state, R, D and the weighted residuals never leave the wave: each product
// is a 16-column MFMA whose B operand is built in registers from the C tiles of
// the product before it.  A C tile holds rows 4q .. 4q+3 of its 16 rows in lane
// (r, q), so two vertically adjacent C tiles give lane (r, q) the eight rows
// {4q .. 4q+3, 16+4q .. 16+4q+3} of a 32-row block: the contraction index of
// every product runs in that order within each 32-block, and the A operands are
// read from LDS in the same order (two 8-byte reads per fragment).  The
// transposed write key comes from the row-major key tile with the gfx950
// transposing LDS read (ds_read_b64_tr_b16: lane j of each 16-lane group receives
// element j of the 4 rows addressed by its group).
// Waves 2 and 3 ("side" waves) take the rest for the same columns: they copy the
// next chunk's operands global -> LDS (global_load_lds; keys, queries, write keys,
// Tm and the decay factors into the other half of a double buffer at the chunk
// start, V and the two P terms into single buffers once the current ones have
// been read), form O0 = Q S from the state fragments the chain wave leaves in
// LDS, and after the chain wave has published D, form and store
// O = Diag(e^g) O0 + P D.  Two barriers per chunk.
// LDS rows are kept whole; 16-byte pieces are XOR-swizzled by row so that each
// read spreads over the LDS banks.
constexpr int kCW = 32;  // value columns per workgroup

struct WsBuf {
    uint16_t K[kC][kD];   // key rows; piece p of row t stored at piece p ^ (t & 15)
    uint16_t Q[kC][kD];   // query rows, same layout
    uint16_t KW[kC][kD];  // separate write-key rows, same layout
    uint16_t T[kC][kC];   // Tm rows; piece p of row t stored at p ^ ((t >> 1) & 7)
    float G[288];         // record tail: e^{g_t} | fac_t | e^{g_C} (+pad) | g_t | beta_t
};
constexpr int kGFac = 64, kGGC = 128, kGLog = 160, kGBeta = 224;
static_assert((kRecBytes - kRecGam) == 288 * 4, "gate block of the record");
static_assert(kRecFac - kRecGam == 4 * kGFac && kRecGC - kRecGam == 4 * kGGC, "gate block layout");
static_assert(kRecGlog - kRecGam == 4 * kGLog && kRecBeta - kRecGam == 4 * kGBeta, "gate block layout");
static_assert(4 * 64 * 16 >= kC * 24 * 2, "a chain wave's D slot holds a 64 x 16 bf16 output tile (pitch 24)");

struct WsLds {
    WsBuf buf[2];          // double buffered: copied one chunk ahead at the chunk start
    uint16_t V[kC][kCW];   // single buffered: the next chunk's copy is issued once the
    uint16_t Ph[kC][kC];   //   chain waves have read V and the side waves have read
    uint16_t Pl[kC][kC];   //   the P terms (first barrier of the chunk); layout as T
    u32x4 Sx[2][8][64];    // per chain wave: state fragments (hi, lo for 4 k steps) of the chunk start
    u32x4 Dx[2][4][64];    // per chain wave: D fragments (hi, lo for 2 k steps)
};

__device__ __forceinline__ u32x2 ld8(const uint16_t *p) { return *reinterpret_cast<const u32x2 *>(p); }

__device__ __forceinline__ u32x2 ld_tr(const uint16_t *p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t)(p)));
}

__device__ __forceinline__ u32x4 cat(u32x2 a, u32x2 b) { return u32x4{a.x, a.y, b.x, b.y}; }

// two C tiles (rows 4q..4q+3 of each) -> one B fragment as two bf16 terms
__device__ __forceinline__ void split_frag(f32x4 a, f32x4 b, u32x4 &hi, u32x4 &lo) {
    u32x2 ha, la, hb, lb;
    split4(a, ha, la);
    split4(b, hb, lb);
    hi = cat(ha, hb);
    lo = cat(la, lb);
}

// A fragment of rows t (lane row r) of a key-width tile, k step kk, in the
// contraction order {4q .. 4q+3, 16+4q .. 16+4q+3} of the 32-block
__device__ __forceinline__ u32x4 frag_wide(const uint16_t (*M)[kD], int t, int kk, int q) {
    const int p1 = 4 * kk + (q >> 1), p2 = p1 + 2, hf = 4 * (q & 1), sw = t & 15;
    return cat(ld8(&M[t][8 * (p1 ^ sw) + hf]), ld8(&M[t][8 * (p2 ^ sw) + hf]));
}

// B fragment (natural order: 8 consecutive keys) of a key-width tile row t
__device__ __forceinline__ u32x4 frag_row(const uint16_t (*M)[kD], int t, int kk, int q) {
    return *reinterpret_cast<const u32x4 *>(&M[t][8 * ((4 * kk + q) ^ (t & 15))]);
}

template <bool SEPKW>
__global__ void __launch_bounds__(256) gdr_state_ws_kernel(ChunkParams p, int NT, int nbh) {
    __shared__ WsLds sm;
    const int x = blockIdx.x;
    const int xcd = x & 7, rr = x >> 3;
    const int vb = rr % (kD / kCW), bh = rr / (kD / kCW) * 8 + xcd;  // the 4 blocks of a head share an XCD
    if (bh >= nbh) return;
    const int b = bh / p.H, h = bh % p.H, j0 = vb * kCW;
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int w = wv & 1;  // column tile of this wave
    const int l = threadIdx.x & 63, r = l & 15, q = l >> 4;
    const int cw = j0 + 16 * w;
    const bool chain = wv < 2;

    // copies of chunk c into buffer bb, by the two side waves.  For a full chunk every
    // copy is a uniform base plus one of a few per-lane offsets fixed for the whole
    // kernel: row l / 16 of a 4-row unit of a key-width tile (its stored piece depends
    // on the unit index mod 4), row l / 8 of an 8-row unit of Tm (unit index mod 2),
    // row l / 4 of a 16-row unit of the V tile.  A short last chunk clamps its rows.
    const unsigned rstr = (unsigned)p.H * kD;  // elements from one token to the next
    unsigned offW[4], offT[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = 4 * j + (l >> 4);
        offW[j] = (unsigned)(l >> 4) * rstr + 8u * (unsigned)((l & 15) ^ (t & 15));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int t = 8 * j + (l >> 3);
        offT[j] = (unsigned)((l >> 3) * kC + 8 * ((l & 7) ^ ((t >> 1) & 7)));
    }
    const unsigned offV = (unsigned)(l >> 2) * rstr + (unsigned)(j0 + 8 * (l & 3));
    auto issue = [&](int c, int bb) __attribute__((always_inline)) {
        WsBuf &B = sm.buf[bb];
        const int t0 = c * kC, n = min(kC, p.T - t0);
        const long base = (((long)b * p.T + t0) * p.H + h) * kD;
        const char *rec = static_cast<const char *>(p.ws) + ((long)bh * NT + c) * kRecBytes;
        auto wide = [&](const void *src, uint16_t(*dst)[kD]) __attribute__((always_inline)) {
            const uint16_t *s16 = static_cast<const uint16_t *>(src) + base;
            if (n == kC) {
#pragma unroll
                for (int u = 0; u < 16; ++u) dma16(s16 + (long)(4 * u) * rstr + offW[u & 3], &dst[4 * u][0]);
            } else {
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int t = 4 * u + (l >> 4), pc = (l & 15) ^ (t & 15);
                    dma16(s16 + (long)min(t, n - 1) * rstr + 8 * pc, &dst[4 * u][0]);
                }
            }
        };
        if (w == 0) {
            wide(p.k, B.K);
#pragma unroll
            for (int u = 0; u < 8; ++u) dma16(rec + kRecT + 2 * (512 * u + offT[u & 1]), &B.T[8 * u][0]);
        } else {
            wide(p.q, B.Q);
            if (SEPKW) wide(p.kw, B.KW);
            dma16(rec + kRecGam + 16 * l, &B.G[0]);
            if (l < 8) dma16(rec + kRecGam + 1024 + 16 * l, &B.G[256]);
        }
    };
    // the single-buffered tiles of chunk c: V (side wave 0) and the P terms
    auto issue_late = [&](int c) __attribute__((always_inline)) {
        const int t0 = c * kC, n = min(kC, p.T - t0);
        const char *rec = static_cast<const char *>(p.ws) + ((long)bh * NT + c) * kRecBytes;
        if (w == 0) {
            const uint16_t *Vg = static_cast<const uint16_t *>(p.v) + (((long)b * p.T + t0) * p.H + h) * kD;
            if (n == kC) {
#pragma unroll
                for (int u = 0; u < 4; ++u) dma16(Vg + (long)(16 * u) * rstr + offV, &sm.V[16 * u][0]);
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int t = 16 * u + (l >> 2);
                    dma16(Vg + (long)min(t, n - 1) * rstr + j0 + 8 * (l & 3), &sm.V[16 * u][0]);
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) dma16(rec + kRecPhi + 2 * (512 * u + offT[u & 1]), &sm.Ph[8 * u][0]);
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) dma16(rec + kRecPlo + 2 * (512 * u + offT[u & 1]), &sm.Pl[8 * u][0]);
        }
    };

    f32x4 S[8];  // chain waves: S[kt][i] = S[16 kt + 4 q + i][cw + r]
    auto publish_state = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u32x4 hi, lo;
            split_frag(S[2 * kk], S[2 * kk + 1], hi, lo);
            sm.Sx[w][2 * kk][l] = hi;
            sm.Sx[w][2 * kk + 1][l] = lo;
        }
    };
    if (chain) {
        if (p.S0) {
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[kt][i] = p.S0[((long)bh * kD + 16 * kt + 4 * q + i) * kD + cw + r];
        } else {
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) S[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        publish_state();
    } else {
        issue(p.c0, 0);
        issue_late(p.c0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    __syncthreads();

    // chunks c0 .. c1 - 1 (a later block of chunks starts from the state the launch for
    // the block before left in ST, passed as S0)
    for (int c = p.c0; c < p.c1; ++c) {
        const int bb = (c - p.c0) & 1;
        const WsBuf &B = sm.buf[bb];
        const int t0 = c * kC, n = min(kC, p.T - t0);
        if (chain) {
            // Y = K S (S as two bf16 terms)
            f32x4 Y[4];
            {
                u32x4 ka[4][4], sh[4], sl[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) ka[kk][tt] = frag_wide(B.K, 16 * tt + r, kk, q);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    sh[kk] = sm.Sx[w][2 * kk][l];
                    sl[kk] = sm.Sx[w][2 * kk + 1][l];
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) Y[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        Y[tt] = mfma(as_bf16x8(ka[kk][tt]), as_bf16x8(sh[kk]), Y[tt]);
                        Y[tt] = mfma(as_bf16x8(ka[kk][tt]), as_bf16x8(sl[kk]), Y[tt]);
                    }
            }
            // R = V - e^{g_t} Y (rows past the chunk end zeroed)
            u32x4 rh[2], rl[2];
            {
                f32x4 R[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const f32x4 gam = *reinterpret_cast<const f32x4 *>(&B.G[16 * tt + 4 * q]);
                    f32x4 vf;
#pragma unroll
                    for (int i = 0; i < 4; ++i) vf[i] = bf16_to_f32(sm.V[16 * tt + 4 * q + i][16 * w + r]);
                    R[tt] = vf - gam * Y[tt];
                }
                if (n < kC) {
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (16 * tt + 4 * q + i >= n) R[tt][i] = 0.f;
                }
                split_frag(R[0], R[1], rh[0], rl[0]);
                split_frag(R[2], R[3], rh[1], rl[1]);
            }
            // D = Tm R (Tm unit lower triangular: token tiles 0, 1 need k step 0 only)
            f32x4 D[4];
            {
                u32x4 ta[6];
#pragma unroll
                for (int tt = 0, f = 0; tt < 4; ++tt) {
                    const int t = 16 * tt + r, sw = (t >> 1) & 7;
#pragma unroll
                    for (int kk = 0; kk < (tt < 2 ? 1 : 2); ++kk, ++f) {
                        const int p1 = 4 * kk + (q >> 1), p2 = p1 + 2, hf = 4 * (q & 1);
                        ta[f] = cat(ld8(&B.T[t][8 * (p1 ^ sw) + hf]), ld8(&B.T[t][8 * (p2 ^ sw) + hf]));
                    }
                }
#pragma unroll
                for (int tt = 0, f = 0; tt < 4; ++tt) {
                    D[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < (tt < 2 ? 1 : 2); ++kk, ++f) {
                        D[tt] = mfma(as_bf16x8(ta[f]), as_bf16x8(rh[kk]), D[tt]);
                        D[tt] = mfma(as_bf16x8(ta[f]), as_bf16x8(rl[kk]), D[tt]);
                    }
                }
            }
            // publish D for the side wave; E = fac D stays here
            u32x4 eh[2], el[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                u32x4 dh, dl;
                split_frag(D[2 * kk], D[2 * kk + 1], dh, dl);
                sm.Dx[w][2 * kk][l] = dh;
                sm.Dx[w][2 * kk + 1][l] = dl;
                const f32x4 f0 = *reinterpret_cast<const f32x4 *>(&B.G[kGFac + 32 * kk + 4 * q]);
                const f32x4 f1 = *reinterpret_cast<const f32x4 *>(&B.G[kGFac + 32 * kk + 16 + 4 * q]);
                split_frag(D[2 * kk] * f0, D[2 * kk + 1] * f1, eh[kk], el[kk]);
            }
            lds_barrier();  // B1: D published; V and the P terms of this chunk consumed

            // S <- e^{g_C} S + K_w^T E; A fragments of K_w^T by the transposing read
            {
                const float gC = B.G[kGGC];
                const uint16_t(*KWs)[kD] = SEPKW ? B.KW : B.K;
                const int a = r & 3, m = r >> 2;
                u32x4 kw[8][2];
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const int t1 = 32 * kk + 4 * q + m, t2 = t1 + 16;
                        const int pc = 2 * kt + (a >> 1), hf = 4 * (a & 1);
                        kw[kt][kk] = cat(ld_tr(&KWs[t1][8 * (pc ^ (t1 & 15)) + hf]),
                                         ld_tr(&KWs[t2][8 * (pc ^ (t2 & 15)) + hf]));
                    }
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) S[kt] *= gC;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int kt = 0; kt < 8; ++kt) {
                        S[kt] = mfma(as_bf16x8(kw[kt][kk]), as_bf16x8(eh[kk]), S[kt]);
                        S[kt] = mfma(as_bf16x8(kw[kt][kk]), as_bf16x8(el[kk]), S[kt]);
                    }
            }
            publish_state();  // for the next chunk (the side wave read this chunk's before B1)
            if (ckpt_after(p, c)) {
                float *Ck = p.ckpt + ((long)bh * p.nck + (c + 1) / p.seg_chunks - 1) * kD * kD;
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) Ck[(long)(16 * kt + 4 * q + i) * kD + cw + r] = S[kt][i];
            }
        } else {
            if (c + 1 < p.c1) issue(c + 1, bb ^ 1);
            // O0 = Q S from the published state fragments
            f32x4 O[4];
            {
                u32x4 qa[4][4], sh[4], sl[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) qa[kk][tt] = frag_wide(B.Q, 16 * tt + r, kk, q);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    sh[kk] = sm.Sx[w][2 * kk][l];
                    sl[kk] = sm.Sx[w][2 * kk + 1][l];
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) O[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        O[tt] = mfma(as_bf16x8(qa[kk][tt]), as_bf16x8(sh[kk]), O[tt]);
                        O[tt] = mfma(as_bf16x8(qa[kk][tt]), as_bf16x8(sl[kk]), O[tt]);
                    }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) O[tt] *= *reinterpret_cast<const f32x4 *>(&B.G[16 * tt + 4 * q]);
            }
            // A fragments of the two P terms (record), read before the first barrier:
            // the next chunk's copy into the same tiles is issued right after it
            u32x4 ph[6], pl[6];
#pragma unroll
            for (int tt = 0, f = 0; tt < 4; ++tt) {
                const int t = 16 * tt + r, sw = (t >> 1) & 7;
#pragma unroll
                for (int kk = 0; kk < (tt < 2 ? 1 : 2); ++kk, ++f) {
                    const int p1 = 4 * kk + (q >> 1), p2 = p1 + 2, hf = 4 * (q & 1);
                    ph[f] = cat(ld8(&sm.Ph[t][8 * (p1 ^ sw) + hf]), ld8(&sm.Ph[t][8 * (p2 ^ sw) + hf]));
                    pl[f] = cat(ld8(&sm.Pl[t][8 * (p1 ^ sw) + hf]), ld8(&sm.Pl[t][8 * (p2 ^ sw) + hf]));
                }
            }
            lds_barrier();  // B1: D published; V and the P terms of this chunk consumed
            if (c + 1 < p.c1) issue_late(c + 1);

            // O += P D, then stored per lane (4 tokens of one value column per tile)
            {
                u32x4 dh[2], dl[2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    dh[kk] = sm.Dx[w][2 * kk][l];
                    dl[kk] = sm.Dx[w][2 * kk + 1][l];
                }
#pragma unroll
                for (int tt = 0, f = 0; tt < 4; ++tt)
#pragma unroll
                    for (int kk = 0; kk < (tt < 2 ? 1 : 2); ++kk, ++f) {
                        O[tt] = mfma(as_bf16x8(ph[f]), as_bf16x8(dh[kk]), O[tt]);
                        O[tt] = mfma(as_bf16x8(ph[f]), as_bf16x8(dl[kk]), O[tt]);
                        O[tt] = mfma(as_bf16x8(pl[f]), as_bf16x8(dh[kk]), O[tt]);
                    }
                // O goes out as rows: staged (bf16) in this wave's D slot, whose fragments are
                // already in registers, then 16 bytes per lane and store
                uint16_t(*Ost)[24] = reinterpret_cast<uint16_t(*)[24]>(&sm.Dx[w][0][0]);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; i += 2) {
                        const uint32_t o2 = pk_bf16(O[tt][i], O[tt][i + 1]);
                        Ost[16 * tt + 4 * q + i][r] = (uint16_t)(o2 & 0xffffu);
                        Ost[16 * tt + 4 * q + i + 1][r] = (uint16_t)(o2 >> 16);
                    }
                uint16_t *Og = static_cast<uint16_t *>(p.o) + (((long)b * p.T + t0) * p.H + h) * kD + cw;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int row = (l >> 1) + 32 * m, half = l & 1;
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(&Ost[row][8 * half]);
                    // plain stores: L2 joins the 32-byte row pieces of the column blocks into whole
                    // lines before they reach HBM (non-temporal ones went out as partial lines)
                    if (row < n) *reinterpret_cast<u32x4 *>(Og + (long)row * p.H * kD + 8 * half) = v;
                }
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next chunk's copies have landed
        }
        __syncthreads();  // B2: next buffer complete, next state published, this buffer free
    }

    if (chain && p.ST) {
#pragma unroll
        for (int kt = 0; kt < 8; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) p.ST[((long)bh * kD + 16 * kt + 4 * q + i) * kD + cw + r] = S[kt][i];
    }
}


// ---------------------------------------------------------------------------
// state kernel, general gates (wave-specialised, as above)
// ---------------------------------------------------------------------------
// The key-side operands come from the general-gate record with their decay and
// beta applied (U, Q, W as two bf16 terms each), so the products take three bf16
// terms (hi.hi + hi.lo + lo.hi):
//     Y = U S,  R = vh - Y,  D = Tm R,  O = Q S + P D,  S <- Diag(e^{g_C}) S + W^T D.
// vh = sqrt(beta) (.) v for a beta vector over the value channels (VSCALE).  The
// operand tiles do not fit twice in LDS, so everything is single buffered: after
// the first barrier of chunk c the side waves copy U, Q, Tm, P, V (and beta) of
// chunk c + 1 (all consumed before it); after the second, W and e^{g_C}, which the
// chain waves read between the two barriers.
struct ChanLds {
    uint16_t Uh[kC][kD], Ul[kC][kD];  // rows; piece p of row t stored at piece p ^ (t & 15)
    uint16_t Qh[kC][kD], Ql[kC][kD];
    uint16_t Wh[kC][kD], Wl[kC][kD];
    uint16_t T[kC][kC];               // rows; piece p of row t stored at p ^ ((t >> 1) & 7)
    uint16_t Ph[kC][kC], Pl[kC][kC];
    uint16_t V[kC][kCW];
    float Bv[kC][kCW];                // beta over the value channels (fp32 or bf16 bits)
    float GC[kD];                     // e^{g_C} per key channel
    u32x4 Sx[2][8][64];
    u32x4 Dx[2][4][64];
};

template <bool VSCALE, bool GBF16>
__global__ void __launch_bounds__(256) gdr_state_chan_kernel(ChunkParams p, int NT, int nbh) {
    __shared__ ChanLds sm;
    const int x = blockIdx.x;
    const int xcd = x & 7, rr = x >> 3;
    const int vb = rr % (kD / kCW), bh = rr / (kD / kCW) * 8 + xcd;
    if (bh >= nbh) return;
    const int b = bh / p.H, h = bh % p.H, j0 = vb * kCW;
    const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int w = wv & 1;
    const int l = threadIdx.x & 63, r = l & 15, q = l >> 4;
    const int cw = j0 + 16 * w;
    const bool chain = wv < 2;
    const unsigned rstr = (unsigned)p.H * kD;
    const void *bvsrc = p.beta_mode == 2 ? p.beta_v : p.beta_k;  // value-side beta (VSCALE)

    // per-lane parts of the copies (see the scalar kernel): key-width record rows
    // (4 rows per copy), chunk-width rows (8 per copy), the V tile (16 rows of 32)
    unsigned offR[4], offT[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = 4 * j + (l >> 4);
        offR[j] = (unsigned)((l >> 4) * kD + 8 * ((l & 15) ^ (t & 15)));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int t = 8 * j + (l >> 3);
        offT[j] = (unsigned)((l >> 3) * kC + 8 * ((l & 7) ^ ((t >> 1) & 7)));
    }
    auto rec = [&](int c) -> const char * { return static_cast<const char *>(p.ws) + ((long)bh * NT + c) * kRcBytes; };
    auto wide = [&](const char *src, uint16_t(*dst)[kD]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 16; ++u) dma16(src + 2 * (512 * u + offR[u & 3]), &dst[4 * u][0]);
    };
    auto narrow = [&](const char *src, uint16_t(*dst)[kC]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 8; ++u) dma16(src + 2 * (512 * u + offT[u & 1]), &dst[8 * u][0]);
    };
    // W and e^{g_C} of chunk c (read by the chain waves between the two barriers)
    auto issue_w = [&](int c) __attribute__((always_inline)) {
        const char *rc = rec(c);
        if (w == 0) {
            wide(rc + kRcWh, sm.Wh);
        } else {
            wide(rc + kRcWl, sm.Wl);
            if (l < 32) dma16(rc + kRcGC + 16 * l, &sm.GC[0]);
        }
    };
    // everything else of chunk c (read before the first barrier)
    auto issue_rest = [&](int c) __attribute__((always_inline)) {
        const char *rc = rec(c);
        const int t0 = c * kC, n = min(kC, p.T - t0);
        auto row = [&](int t) -> long { return ((long)b * p.T + t0 + min(t, n - 1)) * p.H + h; };
        if (w == 0) {
            wide(rc + kRcUh, sm.Uh);
            wide(rc + kRcQh, sm.Qh);
            narrow(rc + kRcT, sm.T);
            const uint16_t *V = static_cast<const uint16_t *>(p.v);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = 16 * u + (l >> 2);
                dma16(V + row(t) * kD + j0 + 8 * (l & 3), &sm.V[16 * u][0]);
            }
        } else {
            wide(rc + kRcUl, sm.Ul);
            wide(rc + kRcQl, sm.Ql);
            narrow(rc + kRcPh, sm.Ph);
            narrow(rc + kRcPl, sm.Pl);
            if (VSCALE) {
                if (GBF16) {  // 64 rows of 32 bf16
                    const uint16_t *Bsrc = static_cast<const uint16_t *>(bvsrc);
                    uint16_t *Bdst = reinterpret_cast<uint16_t *>(&sm.Bv[0][0]);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int t = 16 * u + (l >> 2);
                        dma16(Bsrc + row(t) * kD + j0 + 8 * (l & 3), Bdst + 16 * u * kCW);
                    }
                } else {      // 64 rows of 32 fp32
                    const float *Bsrc = static_cast<const float *>(bvsrc);
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int t = 8 * u + (l >> 3);
                        dma16(Bsrc + row(t) * kD + j0 + 4 * (l & 7), &sm.Bv[8 * u][0]);
                    }
                }
            }
        }
    };
    auto vbeta = [&](int t, int col) -> float {
        if (GBF16) return bf16_to_f32(reinterpret_cast<const uint16_t *>(&sm.Bv[0][0])[t * kCW + col]);
        return sm.Bv[t][col];
    };

    f32x4 S[8];
    auto publish_state = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u32x4 hi, lo;
            split_frag(S[2 * kk], S[2 * kk + 1], hi, lo);
            sm.Sx[w][2 * kk][l] = hi;
            sm.Sx[w][2 * kk + 1][l] = lo;
        }
    };
    if (chain) {
        if (p.S0) {
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[kt][i] = p.S0[((long)bh * kD + 16 * kt + 4 * q + i) * kD + cw + r];
        } else {
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) S[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        publish_state();
    } else {
        issue_w(0);
        issue_rest(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    __syncthreads();

    for (int c = 0; c < NT; ++c) {
        const int t0 = c * kC, n = min(kC, p.T - t0);
        if (chain) {
            // Y = U S
            f32x4 Y[4];
            {
                u32x4 sh[4], sl[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    sh[kk] = sm.Sx[w][2 * kk][l];
                    sl[kk] = sm.Sx[w][2 * kk + 1][l];
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) Y[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    u32x4 ah[4], al[4];
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        ah[tt] = frag_wide(sm.Uh, 16 * tt + r, kk, q);
                        al[tt] = frag_wide(sm.Ul, 16 * tt + r, kk, q);
                    }
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        Y[tt] = mfma(as_bf16x8(ah[tt]), as_bf16x8(sh[kk]), Y[tt]);
                        Y[tt] = mfma(as_bf16x8(ah[tt]), as_bf16x8(sl[kk]), Y[tt]);
                        Y[tt] = mfma(as_bf16x8(al[tt]), as_bf16x8(sh[kk]), Y[tt]);
                    }
                }
            }
            // R = vh - Y (rows past the chunk end zeroed)
            u32x4 rh[2], rl[2];
            {
                f32x4 R[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    f32x4 vf;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tk = 16 * tt + 4 * q + i;
                        vf[i] = bf16_to_f32(sm.V[tk][16 * w + r]);
                        if (VSCALE) vf[i] *= sqrtf(vbeta(tk, 16 * w + r));
                    }
                    R[tt] = vf - Y[tt];
                }
                if (n < kC) {
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (16 * tt + 4 * q + i >= n) R[tt][i] = 0.f;
                }
                split_frag(R[0], R[1], rh[0], rl[0]);
                split_frag(R[2], R[3], rh[1], rl[1]);
            }
            // D = Tm R
            f32x4 D[4];
            {
                u32x4 ta[6];
#pragma unroll
                for (int tt = 0, f = 0; tt < 4; ++tt) {
                    const int t = 16 * tt + r, sw = (t >> 1) & 7;
#pragma unroll
                    for (int kk = 0; kk < (tt < 2 ? 1 : 2); ++kk, ++f) {
                        const int p1 = 4 * kk + (q >> 1), p2 = p1 + 2, hf = 4 * (q & 1);
                        ta[f] = cat(ld8(&sm.T[t][8 * (p1 ^ sw) + hf]), ld8(&sm.T[t][8 * (p2 ^ sw) + hf]));
                    }
                }
#pragma unroll
                for (int tt = 0, f = 0; tt < 4; ++tt) {
                    D[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < (tt < 2 ? 1 : 2); ++kk, ++f) {
                        D[tt] = mfma(as_bf16x8(ta[f]), as_bf16x8(rh[kk]), D[tt]);
                        D[tt] = mfma(as_bf16x8(ta[f]), as_bf16x8(rl[kk]), D[tt]);
                    }
                }
            }
            // publish D; it is also the state update's right operand (its weights are in W)
            u32x4 dh[2], dl[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                split_frag(D[2 * kk], D[2 * kk + 1], dh[kk], dl[kk]);
                sm.Dx[w][2 * kk][l] = dh[kk];
                sm.Dx[w][2 * kk + 1][l] = dl[kk];
            }
            lds_barrier();  // B1: D published; U, Q, Tm, P, V of this chunk consumed; W landed

            // S <- Diag(e^{g_C}) S + W^T D; A fragments of W^T by the transposing read
            {
                const int a = r & 3, m = r >> 2;
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) S[kt] *= *reinterpret_cast<const f32x4 *>(&sm.GC[16 * kt + 4 * q]);
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const int t1 = 32 * kk + 4 * q + m, t2 = t1 + 16;
                        const int pc = 2 * kt + (a >> 1), hf = 4 * (a & 1);
                        const u32x4 wh = cat(ld_tr(&sm.Wh[t1][8 * (pc ^ (t1 & 15)) + hf]),
                                             ld_tr(&sm.Wh[t2][8 * (pc ^ (t2 & 15)) + hf]));
                        const u32x4 wl = cat(ld_tr(&sm.Wl[t1][8 * (pc ^ (t1 & 15)) + hf]),
                                             ld_tr(&sm.Wl[t2][8 * (pc ^ (t2 & 15)) + hf]));
                        S[kt] = mfma(as_bf16x8(wh), as_bf16x8(dh[kk]), S[kt]);
                        S[kt] = mfma(as_bf16x8(wh), as_bf16x8(dl[kk]), S[kt]);
                        S[kt] = mfma(as_bf16x8(wl), as_bf16x8(dh[kk]), S[kt]);
                    }
            }
            publish_state();
            if (ckpt_after(p, c)) {
                float *Ck = p.ckpt + ((long)bh * p.nck + (c + 1) / p.seg_chunks - 1) * kD * kD;
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) Ck[(long)(16 * kt + 4 * q + i) * kD + cw + r] = S[kt][i];
            }
        } else {
            if (c > 0) issue_w(c);
            // O0 = Q S
            f32x4 O[4];
            {
                u32x4 sh[4], sl[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    sh[kk] = sm.Sx[w][2 * kk][l];
                    sl[kk] = sm.Sx[w][2 * kk + 1][l];
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) O[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    u32x4 ah[4], al[4];
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        ah[tt] = frag_wide(sm.Qh, 16 * tt + r, kk, q);
                        al[tt] = frag_wide(sm.Ql, 16 * tt + r, kk, q);
                    }
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        O[tt] = mfma(as_bf16x8(ah[tt]), as_bf16x8(sh[kk]), O[tt]);
                        O[tt] = mfma(as_bf16x8(ah[tt]), as_bf16x8(sl[kk]), O[tt]);
                        O[tt] = mfma(as_bf16x8(al[tt]), as_bf16x8(sh[kk]), O[tt]);
                    }
                }
            }
            u32x4 ph[6], pl[6];
#pragma unroll
            for (int tt = 0, f = 0; tt < 4; ++tt) {
                const int t = 16 * tt + r, sw = (t >> 1) & 7;
#pragma unroll
                for (int kk = 0; kk < (tt < 2 ? 1 : 2); ++kk, ++f) {
                    const int p1 = 4 * kk + (q >> 1), p2 = p1 + 2, hf = 4 * (q & 1);
                    ph[f] = cat(ld8(&sm.Ph[t][8 * (p1 ^ sw) + hf]), ld8(&sm.Ph[t][8 * (p2 ^ sw) + hf]));
                    pl[f] = cat(ld8(&sm.Pl[t][8 * (p1 ^ sw) + hf]), ld8(&sm.Pl[t][8 * (p2 ^ sw) + hf]));
                }
            }
            lds_barrier();  // B1 (also: this wave's copies of W have landed)
            if (c + 1 < NT) issue_rest(c + 1);
            {
                u32x4 dh[2], dl[2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    dh[kk] = sm.Dx[w][2 * kk][l];
                    dl[kk] = sm.Dx[w][2 * kk + 1][l];
                }
#pragma unroll
                for (int tt = 0, f = 0; tt < 4; ++tt)
#pragma unroll
                    for (int kk = 0; kk < (tt < 2 ? 1 : 2); ++kk, ++f) {
                        O[tt] = mfma(as_bf16x8(ph[f]), as_bf16x8(dh[kk]), O[tt]);
                        O[tt] = mfma(as_bf16x8(ph[f]), as_bf16x8(dl[kk]), O[tt]);
                        O[tt] = mfma(as_bf16x8(pl[f]), as_bf16x8(dh[kk]), O[tt]);
                    }
                // O out as rows, staged in this wave's D slot (as in the scalar kernel)
                uint16_t(*Ost)[24] = reinterpret_cast<uint16_t(*)[24]>(&sm.Dx[w][0][0]);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; i += 2) {
                        const uint32_t o2 = pk_bf16(O[tt][i], O[tt][i + 1]);
                        Ost[16 * tt + 4 * q + i][r] = (uint16_t)(o2 & 0xffffu);
                        Ost[16 * tt + 4 * q + i + 1][r] = (uint16_t)(o2 >> 16);
                    }
                uint16_t *Og = static_cast<uint16_t *>(p.o) + (((long)b * p.T + t0) * p.H + h) * kD + cw;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int row = (l >> 1) + 32 * m, half = l & 1;
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(&Ost[row][8 * half]);
                    if (row < n) *reinterpret_cast<u32x4 *>(Og + (long)row * p.H * kD + 8 * half) = v;
                }
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next chunk's operands have landed
        }
        __syncthreads();  // B2
    }

    if (chain && p.ST) {
#pragma unroll
        for (int kt = 0; kt < 8; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) p.ST[((long)bh * kD + 16 * kt + 4 * q + i) * kD + cw + r] = S[kt][i];
    }
}

// State kernel: 1 = the wave-specialised kernel (default), 16 / 32 = the four-wave
// kernel with that many value columns per workgroup (selected by flags, for testing).
int state_variant(const ChunkParams &p) { return p.state_cols == 16 || p.state_cols == 32 ? p.state_cols : 1; }

}  // namespace

bool chunk_mfma_supported(const ChunkParams &p) { return p.io_bf16 && p.dk == kD && p.dv == kD && p.C == kC; }

// scalar forget gate and scalar beta: the scalar record and kernels; anything else
// takes the general-gate record and kernels
static bool general_gates(const ChunkParams &p) { return p.alpha_ch || p.beta_mode != 0; }

size_t chunk_mfma_workspace(const ChunkParams &p) {
    const long NT = (p.T + kC - 1) / kC;
    return (size_t)p.B * p.H * NT * (general_gates(p) ? kRcBytes : kRecBytes);
}

namespace {
constexpr int kPrefillBlocks = 8;   // most chunk blocks of a call (8 measured best: 16 and 4 both slower)
static_assert(1 + kPrefillBlocks <= kSideEvents, "events of one call");
SideStream g_prefill_side[kSideMaxDevices];

// Scalar gates, wave-specialised state kernel, chunks cut into nblk blocks: the prep of
// every block on the side stream, the state kernel block by block on the caller's
// stream, each launch after its block's prep; the launches after the first start from
// the state the one before left in ST.
hipError_t launch_blocked(const ChunkParams &p, int NT, int nblk, const void *ws_fn, unsigned ws_grid,
                          hipStream_t st) {
    SideStream *sd = nullptr;
    std::unique_lock<std::mutex> lock;
    hipError_t e = side_stream_acquire(g_prefill_side, sd, lock);
    if (e != hipSuccess) return e;
    hipEvent_t fork = sd->ev[0], *prepped = sd->ev + 1;
    const void *prep = p.gate_bf16 ? reinterpret_cast<const void *>(&gdr_prep_kernel<true>)
                                   : reinterpret_cast<const void *>(&gdr_prep_kernel<false>);
    const long nbh = (long)p.B * p.H;
    int nt = NT, nb = (int)nbh;
    auto bound = [&](int j) { return (int)((long)NT * j / nblk); };
    if ((e = hipEventRecord(fork, st)) != hipSuccess) return e;  // inputs ready on st
    if ((e = hipStreamWaitEvent(sd->stream, fork, 0)) != hipSuccess) return e;
    for (int j = 0; j < nblk; ++j) {
        ChunkParams a = p;
        a.c0 = bound(j);
        a.c1 = bound(j + 1);
        void *args[] = {&a, &nt};
        if ((e = hipLaunchKernel(prep, dim3((unsigned)(nbh * (a.c1 - a.c0))), dim3(kThreads), args, 0,
                                 sd->stream)) != hipSuccess)
            return e;
        if ((e = hipEventRecord(prepped[j], sd->stream)) != hipSuccess) return e;
    }
    for (int j = 0; j < nblk; ++j) {
        ChunkParams a = p;
        a.c0 = bound(j);
        a.c1 = bound(j + 1);
        if (j > 0) a.S0 = a.ST;  // in place: each workgroup reads and writes only its own columns
        void *args[] = {&a, &nt, &nb};
        if ((e = hipStreamWaitEvent(st, prepped[j], 0)) != hipSuccess) return e;
        if ((e = hipLaunchKernel(ws_fn, dim3(ws_grid), dim3(256), args, 0, st)) != hipSuccess) return e;
    }
    return hipSuccess;
}
}  // namespace

hipError_t launch_chunk_mfma(const ChunkParams &p, hipStream_t st) {
    const long nbh = (long)p.B * p.H;
    const int NT = (p.T + kC - 1) / kC;
    if (nbh == 0 || NT == 0) return hipSuccess;
    ChunkParams arg = p;
    arg.c0 = 0;
    arg.c1 = NT;
    int nt = NT;
    int nb = (int)nbh;
    const long groups = (nbh + 7) / 8;
    if (general_gates(p)) {
        const bool g16 = p.gate_bf16 != 0, ach = p.alpha_ch != 0, bvec = p.beta_mode != 0;
        // prep: <GBF16, ACH, BVEC>
        const void *preps[8] = {
            reinterpret_cast<const void *>(&gdr_prep_chan_kernel<false, false, false>),
            reinterpret_cast<const void *>(&gdr_prep_chan_kernel<false, false, true>),
            reinterpret_cast<const void *>(&gdr_prep_chan_kernel<false, true, false>),
            reinterpret_cast<const void *>(&gdr_prep_chan_kernel<false, true, true>),
            reinterpret_cast<const void *>(&gdr_prep_chan_kernel<true, false, false>),
            reinterpret_cast<const void *>(&gdr_prep_chan_kernel<true, false, true>),
            reinterpret_cast<const void *>(&gdr_prep_chan_kernel<true, true, false>),
            reinterpret_cast<const void *>(&gdr_prep_chan_kernel<true, true, true>)};
        void *pargs[] = {&arg, &nt};
        const hipError_t e = hipLaunchKernel(preps[(g16 ? 4 : 0) + (ach ? 2 : 0) + (bvec ? 1 : 0)],
                                             dim3((unsigned)(nbh * NT)), dim3(kThreads), pargs, 0, st);
        if (e != hipSuccess) return e;
        // state: <VSCALE, GBF16>
        const void *states[4] = {reinterpret_cast<const void *>(&gdr_state_chan_kernel<false, false>),
                                 reinterpret_cast<const void *>(&gdr_state_chan_kernel<false, true>),
                                 reinterpret_cast<const void *>(&gdr_state_chan_kernel<true, false>),
                                 reinterpret_cast<const void *>(&gdr_state_chan_kernel<true, true>)};
        void *sargs[] = {&arg, &nt, &nb};
        return hipLaunchKernel(states[(bvec ? 2 : 0) + (g16 ? 1 : 0)], dim3((unsigned)(groups * 8 * (kD / kCW))),
                               dim3(256), sargs, 0, st);
    }
    const int bv = state_variant(p);
    const bool sep = p.kw != p.k;
    const void *ws_fn = sep ? reinterpret_cast<const void *>(&gdr_state_ws_kernel<true>)
                            : reinterpret_cast<const void *>(&gdr_state_ws_kernel<false>);
    const unsigned ws_grid = (unsigned)(groups * 8 * (kD / kCW));
    // Few heads and many chunks: the state kernel holds one CU per workgroup (all of its
    // LDS) on at most three quarters of the CUs, so the prep of later blocks of chunks
    // runs beside it on a side stream; the state kernel walks the blocks in order, one
    // launch per block, carrying the state through ST.
    const int nblk = (bv == 1 && p.ST && NT >= 256 && ws_grid <= 192) ? min(kPrefillBlocks, NT / 64) : 1;
    if (nblk > 1) return launch_blocked(arg, NT, nblk, ws_fn, ws_grid, st);
    {
        void *args[] = {&arg, &nt};
        const void *prep = p.gate_bf16 ? reinterpret_cast<const void *>(&gdr_prep_kernel<true>)
                                       : reinterpret_cast<const void *>(&gdr_prep_kernel<false>);
        const hipError_t e = hipLaunchKernel(prep,
                                             dim3((unsigned)(nbh * NT)), dim3(kThreads), args, 0, st);
        if (e != hipSuccess) return e;
    }
    void *args[] = {&arg, &nt, &nb};
    if (bv == 1) return hipLaunchKernel(ws_fn, dim3(ws_grid), dim3(256), args, 0, st);
    const void *fn = bv == 32 ? (sep ? reinterpret_cast<const void *>(&gdr_state_kernel<32, true>)
                                     : reinterpret_cast<const void *>(&gdr_state_kernel<32, false>))
                              : (sep ? reinterpret_cast<const void *>(&gdr_state_kernel<16, true>)
                                     : reinterpret_cast<const void *>(&gdr_state_kernel<16, false>));
    return hipLaunchKernel(fn, dim3((unsigned)(groups * 8 * (kD / bv))), dim3(kThreads), args, 0, st);
}

}  // namespace gdr
