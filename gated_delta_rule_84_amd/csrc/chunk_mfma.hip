// chunk_mfma.hip -- chunkwise WY / UT-transform prefill on gfx950 bf16 matrix cores.
//
// Serves bf16 q / k / k_w / v, dk == dv == 128, chunk 64.  Per chunk of n <= 64
// tokens with d(s, t) the decay from token s to token t >= s inside the chunk
// (gamma_t = d(start, t)), erase key u, write key w and written value vh (scalar
// beta: u = k, w = beta k_w, vh = v):
//     A  = strictly-lower( u_t . (d(s, t) (.) w_s) )        block Gram matrix
//     Tm = (I + A)^{-1}                                     UT transform
//     P  = lower-incl-diag( q_t . (d(s, t) (.) w_s) )       intra-chunk scores
//     R  = Vh - (gamma_t (.) U) S                           residual before the chunk
//     D  = Tm R                                             per-token residuals
//     O  = (gamma_t (.) Q) S + P D
//     S <- Diag(gamma_end) S + sum_s (d(s, end) (.) w_s) D_s^T
// (the WY factors of the pages' chunk-parallel form are Tm (gamma (.) U) and Tm Vh;
// the write key replaces the key in the Gram matrix and the scores exactly as the
// OSDN page, section 2.1 states).  Decays are kept segmented at zero gates (a hard
// reset): with P the cumulative log decay in which a zero gate adds 0,
// d(s, t) = [no zero gate in (s, t]] e^{P_t - P_s}, so every factor is <= 1 and no
// infinity is subtracted from another.  A scalar decay is a per-row / per-column
// factor applied in fp32 after the product; a decay per key channel is folded into
// the key-side operands before it.
//
// Kernels, two per call:
//  * prep (scalar alpha and beta) -- one 256-thread block per chunk, fully
//        parallel: the Gram and score products on MFMA from the raw bf16 keys,
//        exact-difference decay weights, the UT transform (diagonal blocks by
//        forward substitution, off-diagonal blocks on fp32 MFMA) and a per-chunk
//        record: Tm (bf16), P as two bf16 terms, gamma_t, beta_s d(s, end),
//        gamma_end, P_t, beta_t.
//  * prep (general gates) -- the same for a decay per key channel and / or beta
//        vectors: it forms U = u (.) gamma, Q = q (.) gamma, W = w (.) d(., end)
//        as two bf16 terms each (the record carries them), takes the Gram and
//        score products as matrix-core products of rescaled operands when the
//        chunk's decays allow it and entry by entry otherwise, and the same UT
//        transform.
//  * state -- one workgroup per (batch * head, 32 value columns), walking the
//        chunks in order: two chain waves carry Y, R, D and the state update for
//        16 value columns each, two side waves copy operands into LDS and form the
//        output (wave-specialised kernels, scalar and general-gate variants).
//        Every product that touches the state or a residual uses a two-term bf16
//        split of the fp32 operand (hi + lo), so the state path keeps ~16 mantissa
//        bits.
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
constexpr int kRecGam = 24576;  // f32 [64]  gamma_t = d(start, t)
constexpr int kRecFac = 24832;  // f32 [64]  beta_s d(s, end), 0 past the chunk end
constexpr int kRecGC = 25088;   // f32       gamma_end
constexpr int kRecGlog = 25216; // f32 [64]  P_t (cumulative log decay inside the chunk, zero gates adding 0)
constexpr int kRecBeta = 25472; // f32 [64]  beta_t, 0 past the chunk end
constexpr int kRecBytes = 25728;

// per-chunk workspace record of the general-gate path (channel decay and/or beta
// vectors): every key-side operand already carries its decay and beta, as two bf16
// terms (hi + lo) each
constexpr int kRcT = 0;          // bf16 [64][64]   Tm
constexpr int kRcPh = 8192;      // bf16 [64][64]   P, leading term
constexpr int kRcPl = 16384;     // bf16 [64][64]   P, remainder
constexpr int kRcUh = 24576;     // bf16 [64][128]  U_t = u_t (.) gamma_t              (erase key)
constexpr int kRcUl = 40960;
constexpr int kRcQh = 57344;     // bf16 [64][128]  Q_t = q_t (.) gamma_t
constexpr int kRcQl = 73728;
constexpr int kRcWh = 90112;     // bf16 [64][128]  W_t = w_t (.) d(t, end)            (write key)
constexpr int kRcWl = 106496;
constexpr int kRcGC = 122880;    // f32 [128]       gamma_end per key channel
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

// Orders that let every matrix-core fragment come out of LDS as one 16-byte read.
// A B fragment built from two vertically adjacent C tiles holds, in lane (r, q), rows
// 4q .. 4q+3 of each tile, i.e. contraction slots 8q .. 8q+7 of a 32-block.
//  * Key order inside the state kernels: row 4q + i of state tile kt holds key
//    skey(kt, q, i), so the state fragment of k step kk covers the consecutive keys
//    32 kk + 8 q .. + 7 and the key / query fragments are plain 16-byte row pieces.
//  * Token columns of Tm and P in the record: column s = 32 kk + 16 h + 4 q + i sits at
//    pcol(s) = 32 kk + 8 q + 4 h + i, the order of the residual fragments built from
//    C tiles of token rows.
__device__ __forceinline__ int skey(int kt, int q, int i) { return 32 * (kt >> 1) + 8 * q + 4 * (kt & 1) + i; }
__device__ __forceinline__ int pcol(int s) { return (s & 32) | ((s & 12) << 1) | ((s & 16) >> 2) | (s & 3); }
__device__ __forceinline__ int pcol_inv(int c) { return (c & 32) | ((c & 4) << 2) | ((c & 24) >> 1) | (c & 3); }


// fp32 x = hi + lo, both bf16 round-to-nearest-even, packed four to a u32x2.
__device__ __forceinline__ void split4(f32x4 x, u32x2 &hi, u32x2 &lo) {
    const uint32_t h0 = pk_bf16(x[0], x[1]), h1 = pk_bf16(x[2], x[3]);
    hi = u32x2{h0, h1};
    lo = u32x2{pk_bf16(x[0] - __uint_as_float(h0 << 16), x[1] - __uint_as_float(h0 & 0xffff0000u)),
               pk_bf16(x[2] - __uint_as_float(h1 << 16), x[3] - __uint_as_float(h1 & 0xffff0000u))};
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

// Inclusive prefix sum (x) and prefix maximum (z) over the 64 lanes of a wave with DPP:
// shifts by 1, 2, 4 and 8 inside each row of 16 lanes, then the row totals carried by
// the broadcasts of lanes 15 (to rows 1 and 3) and 31 (to rows 2 and 3).  Lanes with no
// source take the identity (0 for the sum, -1 for the maximum).  All 64 lanes active.
__device__ __forceinline__ void wave_scan_sum_max(float &x, int &z) {
#define GDR_SCAN_STEP(ctrl, rmask)                                                                          \
    {                                                                                                       \
        const float y = __builtin_bit_cast(                                                                 \
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, rmask, 0xf, false));   \
        const int zy = __builtin_amdgcn_update_dpp(-1, z, ctrl, rmask, 0xf, false);                         \
        x += y;                                                                                             \
        z = max(z, zy);                                                                                     \
    }
    GDR_SCAN_STEP(0x111, 0xf)  // row_shr:1
    GDR_SCAN_STEP(0x112, 0xf)  // row_shr:2
    GDR_SCAN_STEP(0x114, 0xf)  // row_shr:4
    GDR_SCAN_STEP(0x118, 0xf)  // row_shr:8
    GDR_SCAN_STEP(0x142, 0xa)  // row_bcast:15
    GDR_SCAN_STEP(0x143, 0xc)  // row_bcast:31
#undef GDR_SCAN_STEP
}

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
// The lower-triangular Tm (fp32 rows in Ts, row pitch LT, unit diagonal implied) to the
// record as bf16 rows of 64 in pcol order, 16 bytes per store.
template <int LT>
__device__ __forceinline__ void store_ut(char *dst, const float (*Ts)[LT], const int tid) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {  // 512 pieces of 8 bf16
        const int pc = tid + 256 * m, row = pc >> 3, c0 = (pc & 7) * 8;
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ca = pcol_inv(c0 + 2 * j), cb = pcol_inv(c0 + 2 * j + 1);
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
// GBF16: the gates are bf16 (compile time, so the gate loads carry no branch).
// SEP: the write keys are a tensor of their own (k_w != k).  Without one the UT transform
// runs in place (Tm over the Gram matrix): 22 KB of LDS, five blocks per CU (the
// registers allow five); with one, Tm has its own array, which first holds the key tile.
template <bool GBF16, bool SEP>
__global__ void __launch_bounds__(kThreads, SEP ? 4 : 5) gdr_prep_kernel(ChunkParams p, int NT) {
    constexpr int PT = SEP ? kC + 8 : kC + 4;  // row pitch of Tm
    __shared__ float gl[kC], bl[kC];
    __shared__ int zl[kC];
    __shared__ __align__(16) float As[kC][kC + 4];  // Gram matrix, strictly lower part (first: the write keys)
    __shared__ __align__(16) float Tbuf[SEP ? kC * PT : 4];  // UT transform (first: the keys)
    __shared__ __align__(16) float Xs[4][16][16];  // the four 16 x 16 blocks of A_2:4,0:2 T_0:2,0:2
    float(*Ts)[PT];
    if constexpr (SEP)
        Ts = reinterpret_cast<float(*)[PT]>(&Tbuf[0]);
    else
        Ts = As;

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
    constexpr bool sep = SEP;
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
    // every tile of both row blocks is formed (the masks below zero the ones above the
    // diagonal): products guarded by the wave's block index would each become a branch
    // of their own, with the accumulators copied around it
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
            const bf16x8 kb = as_bf16x8(*reinterpret_cast<const u32x4 *>(&KWs[16 * J + r][8 * ((4 * kk + q) ^ r)]));
            accG[J] = mfma(as_bf16x8(ka[kk]), kb, accG[J]);
            accP[J] = mfma(kb, as_bf16x8(qa[kk]), accP[J]);  // scores transposed
        }
    // cumulative log decay and beta (wave 0), segmented at zero gates: P_t sums log alpha
    // over the chunk's tokens <= t with a zero gate adding 0, and Z_t is the last token
    // <= t whose gate is 0 (-1 if none).  The decay from token s to token t >= s is
    // [Z_t <= s] e^{P_t - P_s}: a hard reset makes it exactly 0 and no infinity is ever
    // subtracted from another.
    if (w == 0) {
        const bool zero = l < n && a_raw == 0.f;
        float la = (l < n && !zero) ? logf(a_raw) : 0.f;
        int z = zero ? l : -1;
        const float be = l < n ? b_raw : 0.f;
        wave_scan_sum_max(la, z);
        gl[l] = la;
        zl[l] = z;
        bl[l] = be;
    }

    __syncthreads();

    // decay / beta weights; Gram to LDS (fp32).  Every LDS read is hoisted ahead of the
    // stores so none waits behind them.  The exponent is clamped at 0, which changes
    // only entries the masks discard (g decreases in t).
    char *rec = static_cast<char *>(p.ws) + ((long)bh * NT + c) * kRecBytes;
    float gG[4], gS[4], bS[4], gQ[4][4], bQ[4][4];
    int zG[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        gG[i] = gl[16 * IG + 4 * q + i];
        zG[i] = zl[16 * IG + 4 * q + i];
        gS[i] = gl[16 * i + r];
        bS[i] = bl[16 * i + r];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            gQ[J][i] = gl[16 * J + 4 * q + i];
            bQ[J][i] = bl[16 * J + 4 * q + i];
        }
    }
    const int tP = 16 * IP + r;  // the scores' token row of this lane
    const float gt = gl[tP];
    const int zt = zl[tP];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        if (J <= IG) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 16 * J + r, t = 16 * IG + 4 * q + i;
                const float v = accG[J][i] * bS[J] * __expf(fminf(gG[i] - gS[J], 0.f));
                As[t][s] = (s < t && t < n && zG[i] <= s) ? v : 0.f;
            }
        }
        // scores: lane (r, q) holds P[tP][s] for s = 16 J + 4 q + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = 16 * J + 4 * q + i;
            const float v = accP[J][i] * bQ[J][i] * __expf(fminf(gt - gQ[J][i], 0.f));
            accP[J][i] = (J <= IP && s <= tP && tP < n && zt <= s) ? v : 0.f;
        }
    }
    // P to the record in the pcol column order straight from the C tiles: tiles 2 kk and
    // 2 kk + 1 give this lane the stored columns 32 kk + 8 q .. + 7 of row tP, as two bf16
    // terms (16 bytes each)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        u32x4 hi, lo;
        split_frag(accP[2 * kk], accP[2 * kk + 1], hi, lo);
        *reinterpret_cast<u32x4 *>(rec + kRecPhi + 2 * (tP * kC + 32 * kk + 8 * q)) = hi;
        *reinterpret_cast<u32x4 *>(rec + kRecPlo + 2 * (tP * kC + 32 * kk + 8 * q)) = lo;
    }
    __syncthreads();

    ut_transform(As, Ts, Xs, w, l);

    // write the rest of the record
    store_ut(rec + kRecT, Ts, tid);
    if (tid < kC) {
        float *gam = reinterpret_cast<float *>(rec + kRecGam);
        float *fac = reinterpret_cast<float *>(rec + kRecFac);
        const int zC = zl[n - 1];
        gam[tid] = zl[tid] < 0 ? __expf(gl[tid]) : 0.f;
        fac[tid] = (tid < n && zC <= tid) ? bl[tid] * __expf(gl[n - 1] - gl[tid]) : 0.f;
        if (tid == 0) *reinterpret_cast<float *>(rec + kRecGC) = zC < 0 ? __expf(gl[n - 1]) : 0.f;
        reinterpret_cast<float *>(rec + kRecGlog)[tid] = gl[tid];
        reinterpret_cast<float *>(rec + kRecBeta)[tid] = bl[tid];
    }
}


// ---------------------------------------------------------------------------
// prep kernel, general gates
// ---------------------------------------------------------------------------
// One 256-thread block per chunk for a forget gate per key channel (ACH) and / or
// beta vectors (BVEC; u = sqrt(beta^k) (.) k, w = sqrt(beta^k) (.) k_w; a scalar beta
// gives u = k, w = beta k_w).  Per key channel i the decay from token s to token
// t >= s inside the chunk is [no zero gate in (s, t]] e^{P_t - P_s}, with P the
// cumulative log decay in which zero gates add 0 (a zero gate is a hard reset).
// The record carries U = u (.) gamma_t, Q = q (.) gamma_t and W = w (.) (decay from t
// to the chunk end) as two bf16 terms each, gamma_t being the decay from the chunk
// start through t -- every factor <= 1 -- plus Tm, P as for the scalar path, and the
// decay over the whole chunk per channel.
// The Gram and score matrices A_ts = sum_i u_ti w_si d_i(s, t) and
// Pm_ts = sum_i q_ti w_si d_i(s, t) take one of two forms, chosen per chunk:
//  * factored (no zero gate in the chunk and every channel's decay inside the chunk
//    within e^{-80}): d_i(s, t) = e^{P_ti} e^{-P_si}, so both matrices are plain
//    products of U (or Q) and What = w (.) e^{-P} on the matrix cores (three bf16
//    terms);
//  * exact (otherwise): every entry is summed over the channels with its own decay
//    factor on the vector ALU, so no factor can overflow and a zero gate cuts the
//    chunk exactly.
template <bool GBF16, bool ACH, bool BVEC>
__global__ void __launch_bounds__(kThreads) gdr_prep_chan_kernel(ChunkParams p, int NT) {
    // the cumulative log decay P[t][i] is dead once the Gram and score entries are
    // formed; the Gram and UT arrays take its place
    __shared__ __align__(16) float pool[kC * (kC + 4) + kC * (kC + 8)];
    __shared__ __align__(16) uint16_t Whs[kC][kD + 8], Wls[kC][kD + 8];  // What, two bf16 terms
    __shared__ __align__(16) float Xs[4][16][16];
    __shared__ uint32_t zbits[2][kD];  // per channel: zero gates among tokens 0..31 | 32..63
    float(*gs)[kD + 4] = reinterpret_cast<float(*)[kD + 4]>(pool);
    float(*As)[kC + 4] = reinterpret_cast<float(*)[kC + 4]>(pool);
    float(*Ts)[kC + 8] = reinterpret_cast<float(*)[kC + 8]>(pool + kC * (kC + 4));
    uint16_t(*Ph)[kC + 8] = reinterpret_cast<uint16_t(*)[kC + 8]>(&Ts[0][0]);
    uint16_t(*Pl)[kC + 8] = reinterpret_cast<uint16_t(*)[kC + 8]>(&Ts[kC / 2][0]);
    float(*Wx)[kD] = reinterpret_cast<float(*)[kD]>(&Whs[0][0]);  // exact form: w in fp32
    static_assert(kC * (kD + 4) <= kC * (kC + 4) + kC * (kC + 8), "pool holds P");
    static_assert(sizeof(float) * kC * kD <= 2 * sizeof(uint16_t) * kC * (kD + 8), "What space holds w");

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

    // P[t][i]: thread (i, half) scans 32 tokens of channel i; the upper half then adds
    // the lower half's total.  Tokens past the chunk end decay by 1.  The chunk takes
    // the factored form unless some channel has a zero gate or leaves [-80, 80].
    bool unsafe = false;
    {
        const int i = tid & (kD - 1), hf = tid >> 7;
        float a[32];
#pragma unroll
        for (int j = 0; j < 32; ++j)
            a[j] = ACH ? ld_gate(p.alpha, tok(32 * hf + j) * kD + i, GBF16) : ld_gate(p.alpha, tok(32 * hf + j), GBF16);
        float run = 0.f;
        uint32_t zb = 0;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const bool valid = 32 * hf + j < n, zero = valid && a[j] == 0.f;
            run += (valid && !zero) ? logf(a[j]) : 0.f;
            zb |= zero ? (1u << j) : 0u;
            gs[32 * hf + j][i] = run;
        }
        zbits[hf][i] = zb;
        __syncthreads();
        if (hf == 1) {
            const float off = gs[31][i];
#pragma unroll
            for (int j = 0; j < 32; ++j) gs[32 + j][i] += off;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const float g = gs[32 * hf + j][i];
            unsafe |= (32 * hf + j < n) && !(g >= -80.f && g <= 80.f);
        }
        unsafe |= zb != 0;
    }
    const bool exact = __syncthreads_or(unsafe);
    // zero gate of channel i among tokens lo .. hi (inclusive; empty when lo > hi)
    auto zero_in = [&](int i, int lo, int hi) -> bool {
        if (lo > hi) return false;
        const uint64_t zm = (uint64_t)zbits[0][i] | ((uint64_t)zbits[1][i] << 32);
        const uint64_t upto = hi >= 63 ? ~0ull : ((1ull << (hi + 1)) - 1);
        return (zm & upto & ~((1ull << lo) - 1)) != 0;
    };
    if (tid < kD) {
        const bool z = zero_in(tid, 0, n - 1);
        reinterpret_cast<float *>(rec + kRcGC)[tid] = z ? 0.f : __expf(gs[n - 1][tid]);
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
            float u8[8], q8[8], wh8[8], wt8[8], wx8[8];
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
                const int ch = k0 + j;
                const float g = gs[t][ch], gq = gs[tp][ch], gC = gs[n - 1][ch];
                // decay from the chunk start through t, and from t to the chunk end
                const float head = zero_in(ch, 0, t) ? 0.f : __expf(g);
                const float headq = zero_in(ch, 0, tp) ? 0.f : __expf(gq);
                const float tail = zero_in(ch, t + 1, n - 1) ? 0.f : __expf(gC - g);
                u8[j] = t < n ? u * head : 0.f;
                wt8[j] = t < n ? wv * tail : 0.f;
                q8[j] = tp < n ? qv * headq : 0.f;
                wh8[j] = (t < n && !exact) ? wv * __expf(-g) : 0.f;
                wx8[j] = t < n ? wv : 0.f;
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
            if (exact) {
#pragma unroll
                for (int j = 0; j < 8; ++j) Wx[t][k0 + j] = wx8[j];
            } else {
                split8(wh8, h8, l8);
                *reinterpret_cast<u32x4 *>(&Whs[t][k0]) = __builtin_bit_cast(u32x4, h8);
                *reinterpret_cast<u32x4 *>(&Wls[t][k0]) = __builtin_bit_cast(u32x4, l8);
            }
        }
    }
    __syncthreads();

    const int IG = w, IP = 3 - w;
    if (!exact) {
        // Gram row block IG = w and score row block IP = 3 - w against What (three bf16
        // products per term pair: hi.hi + hi.lo + lo.hi)
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
                // every tile is formed; the masks below zero the ones above the diagonal
                // (guarded products would each become a branch with the accumulators
                // copied around it)
                accG[J] = mfma(as_bf16x8(uh[kk]), bh8, accG[J]);
                accG[J] = mfma(as_bf16x8(uh[kk]), bl8, accG[J]);
                accG[J] = mfma(as_bf16x8(ul[kk]), bh8, accG[J]);
                accP[J] = mfma(as_bf16x8(qh[kk]), bh8, accP[J]);
                accP[J] = mfma(as_bf16x8(qh[kk]), bl8, accP[J]);
                accP[J] = mfma(as_bf16x8(ql[kk]), bh8, accP[J]);
            }
        __syncthreads();  // P is dead: As and Ts take its place

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
                Ph[tq][pcol(s)] = __builtin_bit_cast(uint16_t, hi);
                Pl[tq][pcol(s)] = __builtin_bit_cast(uint16_t, lo);
            }
        }
    } else {
        // thread: row te = tid / 4, columns s = (tid % 4) + 4 j; each entry summed over
        // the channels with its own decay [no zero in (s, te]] e^{P_te - P_s}
        const int te = tid >> 2, s0 = tid & 3;
        float aA[16], aP[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) aA[j] = aP[j] = 0.f;
        if (te < n) {
            const long rte = tok(te) * kD;
            const float bsc = BVEC ? 0.f : ld_gate(p.beta_k, tok(te), GBF16);
            (void)bsc;
            for (int i = 0; i < kD; ++i) {
                const float sbt = BVEC ? sqrtf(ld_gate(p.beta_k, rte + i, GBF16)) : 1.f;
                const float ut = bf16_to_f32(K[rte + i]) * sbt, qt = bf16_to_f32(Q[rte + i]);
                const float Pt = gs[te][i];
                const uint64_t zm = (uint64_t)zbits[0][i] | ((uint64_t)zbits[1][i] << 32);
                // zero gates of channel i among tokens <= te
                const uint64_t upto = te >= 63 ? ~0ull : ((1ull << (te + 1)) - 1);
                const uint64_t zt = zm & upto;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int s = s0 + 4 * j;
                    // no zero gate of channel i among tokens s + 1 .. te
                    const bool open = (zt & ~((2ull << s) - 1)) == 0;
                    const float d = (s <= te && open) ? __expf(Pt - gs[s][i]) : 0.f;
                    const float wsd = Wx[s][i] * d;
                    aA[j] = (s < te) ? fmaf(ut, wsd, aA[j]) : aA[j];
                    aP[j] = fmaf(qt, wsd, aP[j]);
                }
            }
        }
        __syncthreads();  // P and w are dead: As and Ts take their place
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int s = s0 + 4 * j;
            As[te][s] = (s < te && te < n) ? aA[j] : 0.f;
            const float pv = (s <= te && te < n) ? aP[j] : 0.f;
            const __bf16 hi = (__bf16)pv;
            const __bf16 lo = (__bf16)(pv - (float)hi);
            Ph[te][pcol(s)] = __builtin_bit_cast(uint16_t, hi);
            Pl[te][pcol(s)] = __builtin_bit_cast(uint16_t, lo);
        }
    }
    __syncthreads();
    store_p(rec + kRcPh, rec + kRcPl, Ph, Pl, tid);
    __syncthreads();
    ut_transform(As, Ts, Xs, w, l);
    store_ut(rec + kRcT, Ts, tid);
}


// ---------------------------------------------------------------------------
// state kernel, wave-specialised form
// ---------------------------------------------------------------------------
// Four waves per workgroup, one per SIMD, for value columns j0 .. j0 + 31 of one
// (batch, head).  Waves 0 and 1 ("chain" waves) own value columns
// j0 + 16 w .. j0 + 16 w + 15 for all 64 tokens and 128 key channels and carry
// only the sequential part of a chunk:
//     Y = K S,  R = V - Diag(gamma) Y,  D = Tm R,  S <- gamma_end S + K_w^T (fac D).
// The state, R, D and the weighted residuals never leave the wave: each product
// is a 16-column MFMA whose B operand is built in registers from the C tiles of
// the product before it.  A C tile holds rows 4q .. 4q+3 of its 16 rows in lane
// (r, q), so two vertically adjacent C tiles give lane (r, q) the eight rows
// {4q .. 4q+3, 16+4q .. 16+4q+3} of a 32-row block.  The state's key rows are
// therefore kept in the skey order and Tm's and P's token columns in the pcol order,
// which map those eight rows to eight consecutive keys or stored columns: every A
// operand is one 16-byte LDS read.  The transposed write key comes from the
// row-major key tile with the gfx950 transposing LDS read (ds_read_b64_tr_b16:
// lane j of each 16-lane group receives element j of the 4 rows addressed by its
// group; each lane addresses the 4 consecutive keys of its skey group).
// Waves 2 and 3 ("side" waves) take the rest for the same columns: they copy the
// next chunk's operands global -> LDS (global_load_lds; keys, queries, write keys,
// Tm and the decay factors into the other half of a double buffer at the chunk
// start, V and the two P terms into single buffers once the current ones have
// been read), form O0 = Q S from the state fragments the chain wave leaves in
// LDS, and after the chain wave has published D, form and store
// O = Diag(gamma) O0 + P D.  Two barriers per chunk.
// LDS rows are kept whole; 16-byte pieces are XOR-swizzled by row so that each
// read spreads over the LDS banks.
constexpr int kCW = 32;  // value columns per workgroup

struct WsBuf {
    uint16_t K[kC][kD];   // key rows; piece p of row t stored at piece p ^ (t & 15)
    uint16_t Q[kC][kD];   // query rows, same layout
    uint16_t KW[kC][kD];  // separate write-key rows, same layout
    uint16_t T[kC][kC];   // Tm rows; piece p of row t stored at p ^ ((t >> 1) & 7)
    float G[288];         // record tail: gamma_t | fac_t | gamma_end (+pad) | P_t | beta_t
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


// Fragment of row t (lane row r) of a key-width tile, k step kk: keys 32 kk + 8 q .. + 7
// (the state's key order, skey)
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

    f32x4 S[8];          // chain waves: S[kt][i] = S[skey(kt, q, i)][cw + r]
    u32x4 sfh[4], sfl[4];  // chain waves: the state's B fragments (two bf16 terms), kept for Y
    auto publish_state = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            split_frag(S[2 * kk], S[2 * kk + 1], sfh[kk], sfl[kk]);
            sm.Sx[w][2 * kk][l] = sfh[kk];
            sm.Sx[w][2 * kk + 1][l] = sfl[kk];
        }
    };
    if (chain) {
        if (p.S0) {
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[kt][i] = p.S0[((long)bh * kD + skey(kt, q, i)) * kD + cw + r];
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
            // Y = K S (S as two bf16 terms, the fragments this wave split last)
            f32x4 Y[4];
            {
                u32x4 ka[4][4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) ka[kk][tt] = frag_row(B.K, 16 * tt + r, kk, q);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) Y[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) Y[tt] = mfma(as_bf16x8(ka[kk][tt]), as_bf16x8(sfh[kk]), Y[tt]);
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) Y[tt] = mfma(as_bf16x8(ka[kk][tt]), as_bf16x8(sfl[kk]), Y[tt]);
                }
            }
            // R = V - gamma_t Y (rows past the chunk end zeroed)
            u32x4 rh[2], rl[2];
            {
                f32x4 R[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const f32x4 gam = *reinterpret_cast<const f32x4 *>(&B.G[16 * tt + 4 * q]);
                    // lane (r, q) receives column r of rows 16 tt + 4 q .. + 3
                    const u32x2 v4 = ld_tr(&sm.V[16 * tt + 4 * q + (r >> 2)][16 * w + 4 * (r & 3)]);
                    const f32x4 vf = {__uint_as_float(v4.x << 16), __uint_as_float(v4.x & 0xffff0000u),
                                      __uint_as_float(v4.y << 16), __uint_as_float(v4.y & 0xffff0000u)};
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
                        ta[f] = *reinterpret_cast<const u32x4 *>(&B.T[t][8 * ((4 * kk + q) ^ sw)]);
                    }
                }
                // consecutive products go to different tiles (a product that accumulates onto
                // the one just issued waits for it); each tile still sums hi, lo per k step
                constexpr int f0[4] = {0, 1, 2, 4}, f1[4] = {0, 0, 3, 5};
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) D[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) D[tt] = mfma(as_bf16x8(ta[f0[tt]]), as_bf16x8(rh[0]), D[tt]);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) D[tt] = mfma(as_bf16x8(ta[f0[tt]]), as_bf16x8(rl[0]), D[tt]);
#pragma unroll
                for (int tt = 2; tt < 4; ++tt) D[tt] = mfma(as_bf16x8(ta[f1[tt]]), as_bf16x8(rh[1]), D[tt]);
#pragma unroll
                for (int tt = 2; tt < 4; ++tt) D[tt] = mfma(as_bf16x8(ta[f1[tt]]), as_bf16x8(rl[1]), D[tt]);
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

            // S <- gamma_end S + K_w^T E; A fragments of K_w^T by the transposing read
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
                        const int pc = 4 * (kt >> 1) + a, hf = 4 * (kt & 1);
                        kw[kt][kk] = cat(ld_tr(&KWs[t1][8 * (pc ^ (t1 & 15)) + hf]),
                                         ld_tr(&KWs[t2][8 * (pc ^ (t2 & 15)) + hf]));
                    }
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) S[kt] *= gC;
                // the eight state tiles are independent: the hi products of a k step for all of
                // them, then the lo products (each tile sums hi, lo per k step)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                    for (int kt = 0; kt < 8; ++kt) S[kt] = mfma(as_bf16x8(kw[kt][kk]), as_bf16x8(eh[kk]), S[kt]);
#pragma unroll
                    for (int kt = 0; kt < 8; ++kt) S[kt] = mfma(as_bf16x8(kw[kt][kk]), as_bf16x8(el[kk]), S[kt]);
                }
            }
            publish_state();  // for the next chunk (the side wave read this chunk's before B1)
            if (ckpt_after(p, c)) {
                float *Ck = p.ckpt + ((long)bh * p.nck + (c + 1) / p.seg_chunks - 1) * kD * kD;
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) Ck[(long)(skey(kt, q, i)) * kD + cw + r] = S[kt][i];
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
                    for (int tt = 0; tt < 4; ++tt) qa[kk][tt] = frag_row(B.Q, 16 * tt + r, kk, q);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    sh[kk] = sm.Sx[w][2 * kk][l];
                    sl[kk] = sm.Sx[w][2 * kk + 1][l];
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) O[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) O[tt] = mfma(as_bf16x8(qa[kk][tt]), as_bf16x8(sh[kk]), O[tt]);
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) O[tt] = mfma(as_bf16x8(qa[kk][tt]), as_bf16x8(sl[kk]), O[tt]);
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
                    ph[f] = *reinterpret_cast<const u32x4 *>(&sm.Ph[t][8 * ((4 * kk + q) ^ sw)]);
                    pl[f] = *reinterpret_cast<const u32x4 *>(&sm.Pl[t][8 * ((4 * kk + q) ^ sw)]);
                }
            }
            // B1: D published; V and the P terms of this chunk consumed.  The side wave's
            // own LDS reads are complete (lgkmcnt) and the asm is a compiler memory barrier,
            // but unlike lds_barrier() there is no release fence: that would also wait for
            // the next chunk's copies issued above (they write LDS), holding every wave at
            // B1 until they land; they only need to have landed by B2.
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (c + 1 < p.c1) issue_late(c + 1);

            // O += P D, then stored per lane (4 tokens of one value column per tile)
            {
                u32x4 dh[2], dl[2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    dh[kk] = sm.Dx[w][2 * kk][l];
                    dl[kk] = sm.Dx[w][2 * kk + 1][l];
                }
                // per tile and k step: ph dh, ph dl, pl dh; consecutive products go to
                // different tiles
                constexpr int f0[4] = {0, 1, 2, 4}, f1[4] = {0, 0, 3, 5};
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) O[tt] = mfma(as_bf16x8(ph[f0[tt]]), as_bf16x8(dh[0]), O[tt]);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) O[tt] = mfma(as_bf16x8(ph[f0[tt]]), as_bf16x8(dl[0]), O[tt]);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) O[tt] = mfma(as_bf16x8(pl[f0[tt]]), as_bf16x8(dh[0]), O[tt]);
#pragma unroll
                for (int tt = 2; tt < 4; ++tt) O[tt] = mfma(as_bf16x8(ph[f1[tt]]), as_bf16x8(dh[1]), O[tt]);
#pragma unroll
                for (int tt = 2; tt < 4; ++tt) O[tt] = mfma(as_bf16x8(ph[f1[tt]]), as_bf16x8(dl[1]), O[tt]);
#pragma unroll
                for (int tt = 2; tt < 4; ++tt) O[tt] = mfma(as_bf16x8(pl[f1[tt]]), as_bf16x8(dh[1]), O[tt]);
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
            for (int i = 0; i < 4; ++i) p.ST[((long)bh * kD + skey(kt, q, i)) * kD + cw + r] = S[kt][i];
    }
}


// ---------------------------------------------------------------------------
// state kernel, general gates (wave-specialised, as above)
// ---------------------------------------------------------------------------
// The key-side operands come from the general-gate record with their decay and
// beta applied (U, Q, W as two bf16 terms each), so the products take three bf16
// terms (hi.hi + hi.lo + lo.hi):
//     Y = U S,  R = vh - Y,  D = Tm R,  O = Q S + P D,  S <- Diag(gamma_end) S + W^T D.
// vh = sqrt(beta) (.) v for a beta vector over the value channels (VSCALE).  The
// operand tiles do not fit twice in LDS, so everything is single buffered: after
// the first barrier of chunk c the side waves copy U, Q, Tm, P, V (and beta) of
// chunk c + 1 (all consumed before it); after the second, W and gamma_end, which the
// chain waves read between the two barriers.
struct ChanLds {
    uint16_t Uh[kC][kD], Ul[kC][kD];  // rows; piece p of row t stored at piece p ^ (t & 15)
    uint16_t Qh[kC][kD], Ql[kC][kD];
    uint16_t Wh[kC][kD], Wl[kC][kD];
    uint16_t T[kC][kC];               // rows; piece p of row t stored at p ^ ((t >> 1) & 7)
    uint16_t Ph[kC][kC], Pl[kC][kC];
    uint16_t V[kC][kCW];
    float Bv[kC][kCW];                // beta over the value channels (fp32 or bf16 bits)
    float GC[kD];                     // gamma_end per key channel
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
    // W and gamma_end of chunk c (read by the chain waves between the two barriers)
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
                for (int i = 0; i < 4; ++i) S[kt][i] = p.S0[((long)bh * kD + skey(kt, q, i)) * kD + cw + r];
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
                        ah[tt] = frag_row(sm.Uh, 16 * tt + r, kk, q);
                        al[tt] = frag_row(sm.Ul, 16 * tt + r, kk, q);
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
                        ta[f] = *reinterpret_cast<const u32x4 *>(&sm.T[t][8 * ((4 * kk + q) ^ sw)]);
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

            // S <- Diag(gamma_end) S + W^T D; A fragments of W^T by the transposing read
            {
                const int a = r & 3, m = r >> 2;
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) S[kt] *= *reinterpret_cast<const f32x4 *>(&sm.GC[skey(kt, q, 0)]);
#pragma unroll
                for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const int t1 = 32 * kk + 4 * q + m, t2 = t1 + 16;
                        const int pc = 4 * (kt >> 1) + a, hf = 4 * (kt & 1);
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
                    for (int i = 0; i < 4; ++i) Ck[(long)(skey(kt, q, i)) * kD + cw + r] = S[kt][i];
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
                        ah[tt] = frag_row(sm.Qh, 16 * tt + r, kk, q);
                        al[tt] = frag_row(sm.Ql, 16 * tt + r, kk, q);
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
                    ph[f] = *reinterpret_cast<const u32x4 *>(&sm.Ph[t][8 * ((4 * kk + q) ^ sw)]);
                    pl[f] = *reinterpret_cast<const u32x4 *>(&sm.Pl[t][8 * ((4 * kk + q) ^ sw)]);
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
            for (int i = 0; i < 4; ++i) p.ST[((long)bh * kD + skey(kt, q, i)) * kD + cw + r] = S[kt][i];
    }
}

}  // namespace

bool chunk_mfma_supported(const ChunkParams &p) { return p.io_bf16 && p.dk == kD && p.dv == kD && p.C == kC; }

// scalar forget gate and scalar beta: the scalar record and kernels; anything else
// takes the general-gate record and kernels
static bool general_gates(const ChunkParams &p) { return p.alpha_ch || p.beta_mode != 0; }

size_t chunk_mfma_workspace(const ChunkParams &p) {
    const long NT = (p.T + kC - 1) / kC;
    return (size_t)p.B * p.H * NT * (general_gates(p) ? kRcBytes : kRecBytes);
}

// Chunk blocks of the prefill given an execution context (below): at least this many
// chunks per block, at most kMaxPrepBlocks blocks.
constexpr int kPrepBlockChunks = 128;
constexpr int kMaxPrepBlocks = 16;
static_assert(2 + kMaxPrepBlocks <= kCtxEvents, "one context event per block");

hipError_t launch_chunk_mfma(const ChunkParams &p, const gdr_context *ctx, hipStream_t st) {
    const long nbh = (long)p.B * p.H;
    const int NT = (p.T + kC - 1) / kC;
    if (nbh == 0 || NT == 0) return hipSuccess;
    const long groups = (nbh + 7) / 8;
    const bool gen = general_gates(p);
    const bool g16 = p.gate_bf16 != 0, ach = p.alpha_ch != 0, bvec = p.beta_mode != 0;
    int nt = NT;
    int nb = (int)nbh;
    // the prep of chunks c0 .. c1 - 1 of every (batch, head)
    auto prep = [&](int c0, int c1, hipStream_t s) -> hipError_t {
        ChunkParams arg = p;
        arg.c0 = c0;
        arg.c1 = c1;
        void *args[] = {&arg, &nt};
        const void *fn;
        if (gen) {
            // <GBF16, ACH, BVEC>
            const void *preps[8] = {
                reinterpret_cast<const void *>(&gdr_prep_chan_kernel<false, false, false>),
                reinterpret_cast<const void *>(&gdr_prep_chan_kernel<false, false, true>),
                reinterpret_cast<const void *>(&gdr_prep_chan_kernel<false, true, false>),
                reinterpret_cast<const void *>(&gdr_prep_chan_kernel<false, true, true>),
                reinterpret_cast<const void *>(&gdr_prep_chan_kernel<true, false, false>),
                reinterpret_cast<const void *>(&gdr_prep_chan_kernel<true, false, true>),
                reinterpret_cast<const void *>(&gdr_prep_chan_kernel<true, true, false>),
                reinterpret_cast<const void *>(&gdr_prep_chan_kernel<true, true, true>)};
            fn = preps[(g16 ? 4 : 0) + (ach ? 2 : 0) + (bvec ? 1 : 0)];
        } else {
            const void *preps[4] = {reinterpret_cast<const void *>(&gdr_prep_kernel<false, false>),
                                    reinterpret_cast<const void *>(&gdr_prep_kernel<false, true>),
                                    reinterpret_cast<const void *>(&gdr_prep_kernel<true, false>),
                                    reinterpret_cast<const void *>(&gdr_prep_kernel<true, true>)};
            fn = preps[(g16 ? 2 : 0) + (p.kw != p.k ? 1 : 0)];
        }
        return hipLaunchKernel(fn, dim3((unsigned)(nbh * (c1 - c0))), dim3(kThreads), args, 0, s);
    };
    // the state recurrence over chunks c0 .. c1 - 1, entering with S0
    auto state = [&](int c0, int c1, const float *S0) -> hipError_t {
        ChunkParams arg = p;
        arg.c0 = c0;
        arg.c1 = c1;
        arg.S0 = S0;
        void *args[] = {&arg, &nt, &nb};
        const void *fn;
        if (gen) {
            // <VSCALE, GBF16>
            const void *states[4] = {reinterpret_cast<const void *>(&gdr_state_chan_kernel<false, false>),
                                     reinterpret_cast<const void *>(&gdr_state_chan_kernel<false, true>),
                                     reinterpret_cast<const void *>(&gdr_state_chan_kernel<true, false>),
                                     reinterpret_cast<const void *>(&gdr_state_chan_kernel<true, true>)};
            fn = states[(bvec ? 2 : 0) + (g16 ? 1 : 0)];
        } else {
            fn = p.kw != p.k ? reinterpret_cast<const void *>(&gdr_state_ws_kernel<true>)
                             : reinterpret_cast<const void *>(&gdr_state_ws_kernel<false>);
        }
        return hipLaunchKernel(fn, dim3((unsigned)(groups * 8 * (kD / kCW))), dim3(256), args, 0, st);
    };
    hipError_t e;
    // With an execution context, a long sequence with scalar gates whose state kernel
    // leaves CUs idle (one workgroup per CU and head column block: fewer than 64 (batch,
    // head) pairs) and whose final state is written is cut into chunk blocks: the prep of
    // every block runs on the context's second stream while the state recurrence walks
    // the blocks in order on the caller's stream, one launch per block, each entering with
    // the state the launch before left in ST and waiting only for its own block's prep.
    const int nblk = (ctx && p.ST && !gen && nbh < 64) ? min(kMaxPrepBlocks, NT / kPrepBlockChunks) : 1;
    if (nblk <= 1) {
        if ((e = prep(0, NT, st)) != hipSuccess) return e;
        return state(0, NT, p.S0);
    }
    hipStream_t side = ctx->stream;
    const hipEvent_t fork = ctx->ev[0], *solved = ctx->ev + 2;
    auto bound = [&](int j) { return (int)((long)NT * j / nblk); };
    if ((e = hipEventRecord(fork, st)) != hipSuccess) return e;  // inputs ready on st
    if ((e = hipStreamWaitEvent(side, fork, 0)) != hipSuccess) return e;
    for (int j = 0; j < nblk; ++j) {
        if ((e = prep(bound(j), bound(j + 1), side)) != hipSuccess) return e;
        if ((e = hipEventRecord(solved[j], side)) != hipSuccess) return e;
    }
    // the last wait also joins the second stream back into st
    for (int j = 0; j < nblk; ++j) {
        if ((e = hipStreamWaitEvent(st, solved[j], 0)) != hipSuccess) return e;
        if ((e = state(bound(j), bound(j + 1), j == 0 ? p.S0 : p.ST)) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gdr
