// chunk_mfma.hip -- chunkwise WY / UT-transform prefill on gfx950 bf16 matrix cores.
//
// Serves bf16 q / k / k_w / v, dk == dv == 128, chunk 64, scalar forget gate and
// scalar beta (Gated DeltaNet; OSDN when a write key k_w is given).  Per chunk
// of n <= 64 tokens with g_t the cumulative log-decay inside the chunk
// (u = k, w = beta k_w, vh = v):
//     A  = strictly-lower( beta_s e^{g_t - g_s} k_t . k_w,s )     block Gram matrix
//     Tm = (I + A)^{-1}                                          UT transform
//     P  = lower-incl-diag( beta_s e^{g_t - g_s} q_t . k_w,s )    intra-chunk scores
//     R  = V - Diag(e^g) K S                                     residual before the chunk
//     D  = Tm R                                                  per-token residuals
//     O  = Diag(e^g) Q S + P D
//     S <- e^{g_C} S + sum_s beta_s e^{g_C - g_s} k_w,s D_s^T
// (the WY factors of the pages' chunk-parallel form are Tm Diag(e^g) K and Tm V;
// the write key replaces the key in the Gram matrix and the scores exactly as
// the OSDN page, section 2.1 states; FG2-GDN page, section 3).
//
// Two kernels:
//  * prep  -- one 256-thread block per chunk, fully parallel: the two 64 x 64
//             products on MFMA, the exact-difference decay weights, the UT
//             transform by blocked forward substitution in fp32, and a
//             per-chunk record in the workspace: Tm (bf16), P split into two
//             bf16 terms, e^{g_t}, beta_s e^{g_C - g_s}, e^{g_C}.
//  * state -- one 256-thread block per (batch*head, block of BV value columns),
//             walking the chunks in order with the state held transposed
//             (Z = S^T, BV x 128, fp32) in the accumulators of the four waves.
//             Every product that touches the state or a residual uses a
//             two-term bf16 split of the fp32 operand (hi + lo), so the state
//             path keeps ~16 mantissa bits; raw bf16 inputs are exact MFMA
//             operands and all decay / beta factors are applied in fp32.
//
// MFMA operand layouts (v_mfma_f32_16x16x32_bf16, lane l, r = l % 16, q = l / 16):
//   A (16 x 32): lane holds A[r][8q .. 8q+7];  B (32 x 16): B[8q .. 8q+7][r];
//   C (16 x 16): lane holds C[4q .. 4q+3][r].
#include <stdlib.h>

#include "gdr_device.hpp"
#include "gdr_internal.hpp"

namespace gdr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

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
constexpr int kRecBytes = 25216;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

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

// Workgroup barrier that waits only for this wave's LDS traffic.  __syncthreads()
// also drains outstanding global loads, which would stall on the next chunk's
// prefetch at every barrier; the "memory" clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// prep kernel
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) gdr_prep_kernel(ChunkParams p, int NT) {
    __shared__ float gl[kC], bl[kC];
    __shared__ __align__(16) float As[kC][kC + 4];  // Gram matrix, strictly lower part
    __shared__ __align__(16) float Ts[kC][kC + 8];  // UT transform; first holds the two P terms
    __shared__ float Xs[3][16][17];
    uint16_t(*Ph)[kC + 8] = reinterpret_cast<uint16_t(*)[kC + 8]>(&Ts[0][0]);
    uint16_t(*Pl)[kC + 8] = reinterpret_cast<uint16_t(*)[kC + 8]>(&Ts[kC / 2][0]);

    const int blk = blockIdx.x;
    const int c = blk % NT, bh = blk / NT;
    const int b = bh / p.H, h = bh % p.H;
    const int t0 = c * kC, n = min(kC, p.T - t0);
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 15, q = l >> 4;
    auto tok = [&](int t) -> long { return ((long)b * p.T + t0 + t) * p.H + h; };
    const uint16_t *K = static_cast<const uint16_t *>(p.k);
    const uint16_t *KW = static_cast<const uint16_t *>(p.kw);
    const uint16_t *Q = static_cast<const uint16_t *>(p.q);

    // cumulative log decay and beta (wave 0)
    if (w == 0) {
        float la = 0.f, be = 0.f;
        if (l < n) {
            la = logf(ld_gate(p.alpha, tok(l), p.gate_bf16));
            be = ld_gate(p.beta_k, tok(l), p.gate_bf16);
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(la, off);
            if (l >= off) la += y;
        }
        gl[l] = la;
        bl[l] = be;
    }

    // Gram row-block I = w (tiles J <= w) and score row-block IP = 3 - w (tiles J <= IP)
    const int IG = w, IP = 3 - w;
    // rows past the end of a short chunk read the last valid row; their Gram and
    // score entries are masked below
    auto rowt = [&](int t) -> long { return tok(min(t, n - 1)) * kD; };
    u32x4 ka[4], qa[4];
    {
        const int tg = 16 * IG + r, tp = 16 * IP + r;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            ka[kk] = ld16(K + rowt(tg) + kk * 32 + 8 * q);
            qa[kk] = ld16(Q + rowt(tp) + kk * 32 + 8 * q);
        }
    }
    // all key tiles are loaded before the first product so every load is in flight at once
    u32x4 kb[4][4];
#pragma unroll
    for (int J = 0; J < 4; ++J)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kb[J][kk] = ld16(KW + rowt(16 * J + r) + kk * 32 + 8 * q);
    f32x4 accG[4], accP[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        accG[J] = f32x4{0.f, 0.f, 0.f, 0.f};
        accP[J] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (J <= IG) accG[J] = mfma(as_bf16x8(ka[kk]), as_bf16x8(kb[J][kk]), accG[J]);
            if (J <= IP) accP[J] = mfma(as_bf16x8(qa[kk]), as_bf16x8(kb[J][kk]), accP[J]);
        }
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
            if (J <= IG) {
                const int t = 16 * IG + 4 * q + i;
                As[t][s] = (s < t && t < n) ? accG[J][i] * bS[J] * __expf(gG[i] - gS[J]) : 0.f;
            }
            const int tp = 16 * IP + 4 * q + i;
            float pv = 0.f;
            if (J <= IP && s <= tp && tp < n) pv = accP[J][i] * bS[J] * __expf(gP[i] - gS[J]);
            const __bf16 hi = (__bf16)pv;
            const __bf16 lo = (__bf16)(pv - (float)hi);
            Ph[tp][s] = __builtin_bit_cast(uint16_t, hi);
            Pl[tp][s] = __builtin_bit_cast(uint16_t, lo);
        }
    }
    __syncthreads();
    char *rec = static_cast<char *>(p.ws) + ((long)bh * NT + c) * kRecBytes;
#pragma unroll
    for (int m = 0; m < 2; ++m) {  // P terms to the record, 16 bytes per store
        const int pc = tid + 256 * m, row = pc >> 3, c0 = (pc & 7) * 8;
        *reinterpret_cast<u32x4 *>(rec + kRecPhi + (row * kC + c0) * 2) =
            *reinterpret_cast<const u32x4 *>(&Ph[row][c0]);
        *reinterpret_cast<u32x4 *>(rec + kRecPlo + (row * kC + c0) * 2) =
            *reinterpret_cast<const u32x4 *>(&Pl[row][c0]);
    }
    __syncthreads();

    // diagonal 16 x 16 blocks of (I + A)^{-1}: wave w, lane c < 16 owns column c;
    // row rr of the block is read as four 16-byte loads
    if (l < 16) {
        const int base = 16 * w, cc = l;
        float col[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float a[16];
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(&As[base + rr][base + 4 * m4]);
                a[4 * m4] = x[0];
                a[4 * m4 + 1] = x[1];
                a[4 * m4 + 2] = x[2];
                a[4 * m4 + 3] = x[3];
            }
            float v = rr == cc ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < rr; ++m) v -= a[m] * col[m];
            col[rr] = v;
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) Ts[base + rr][base + cc] = col[rr];
    }
    __syncthreads();
    // off-diagonal blocks by distance d: T_IJ = -T_II * sum_{K=J}^{I-1} A_IK T_KJ
    for (int d = 1; d < 4; ++d) {
        const int nb = 4 - d;
        for (int e = tid; e < nb * 256; e += kThreads) {
            const int J = e >> 8, I = J + d, rr = (e >> 4) & 15, cc = e & 15;
            float x = 0.f;
            for (int Kb = J; Kb < I; ++Kb) {
#pragma unroll
                for (int m4 = 0; m4 < 4; ++m4) {
                    const f32x4 a = *reinterpret_cast<const f32x4 *>(&As[16 * I + rr][16 * Kb + 4 * m4]);
#pragma unroll
                    for (int u = 0; u < 4; ++u) x += a[u] * Ts[16 * Kb + 4 * m4 + u][16 * J + cc];
                }
            }
            Xs[J][rr][cc] = x;
        }
        __syncthreads();
        for (int e = tid; e < nb * 256; e += kThreads) {
            const int J = e >> 8, I = J + d, rr = (e >> 4) & 15, cc = e & 15;
            float x = 0.f;
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) {
                const f32x4 tr = *reinterpret_cast<const f32x4 *>(&Ts[16 * I + rr][16 * I + 4 * m4]);
#pragma unroll
                for (int u = 0; u < 4; ++u) x -= tr[u] * Xs[J][4 * m4 + u][cc];
            }
            Ts[16 * I + rr][16 * J + cc] = x;
        }
        __syncthreads();
    }

    // write the rest of the record
#pragma unroll
    for (int m = 0; m < 2; ++m) {  // Tm: 512 pieces of 8 bf16
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
        *reinterpret_cast<u32x4 *>(rec + kRecT + (row * kC + c0) * 2) = o;
    }
    if (tid < kC) {
        float *gam = reinterpret_cast<float *>(rec + kRecGam);
        float *fac = reinterpret_cast<float *>(rec + kRecFac);
        gam[tid] = __expf(gl[tid]);
        fac[tid] = tid < n ? bl[tid] * __expf(gl[n - 1] - gl[tid]) : 0.f;
        if (tid == 0) *reinterpret_cast<float *>(rec + kRecGC) = __expf(gl[n - 1]);
    }
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two fp32 -> two bf16 (round to nearest even) in one packed conversion
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// fp32 x = hi + lo, both bf16 round-to-nearest-even, packed four to a u32x2.
__device__ __forceinline__ void split4(f32x4 x, u32x2 &hi, u32x2 &lo) {
    const uint32_t h0 = pk_bf16(x[0], x[1]), h1 = pk_bf16(x[2], x[3]);
    hi = u32x2{h0, h1};
    lo = u32x2{pk_bf16(x[0] - __uint_as_float(h0 << 16), x[1] - __uint_as_float(h0 & 0xffff0000u)),
               pk_bf16(x[2] - __uint_as_float(h1 << 16), x[3] - __uint_as_float(h1 & 0xffff0000u))};
}

template <int BV>
__global__ void __launch_bounds__(kThreads) gdr_state_kernel(ChunkParams p, int NT, int nbh) {
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
    const bool sep_kw = p.kw != p.k;

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
            f32x4 rv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float vv = bf16_to_f32(VO[w][4 * q + i][16 * nt + r]);
                rv[i] = 16 * w + 4 * q + i < n ? vv - gam[i] * accY[nt][i] : 0.f;
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

int value_block(long nbh) {
    static const int forced = [] {
        const char *e = getenv("GDR_STATE_BV");
        return e ? atoi(e) : 0;
    }();
    if (forced == 16 || forced == 32) return forced;
    return nbh * (kD / 32) >= 256 ? 32 : 16;
}

}  // namespace

bool chunk_mfma_supported(const ChunkParams &p) {
    return p.io_bf16 && p.dk == kD && p.dv == kD && p.C == kC && !p.alpha_ch && p.beta_mode == 0;
}

size_t chunk_mfma_workspace(const ChunkParams &p) {
    const long NT = (p.T + kC - 1) / kC;
    return (size_t)p.B * p.H * NT * kRecBytes;
}

hipError_t launch_chunk_mfma(const ChunkParams &p, hipStream_t st) {
    const long nbh = (long)p.B * p.H;
    const int NT = (p.T + kC - 1) / kC;
    if (nbh == 0 || NT == 0) return hipSuccess;
    ChunkParams arg = p;
    int nt = NT;
    int nb = (int)nbh;
    {
        void *args[] = {&arg, &nt};
        const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&gdr_prep_kernel),
                                             dim3((unsigned)(nbh * NT)), dim3(kThreads), args, 0, st);
        if (e != hipSuccess) return e;
    }
    void *args[] = {&arg, &nt, &nb};
    const long groups = (nbh + 7) / 8;
    if (value_block(nbh) == 32) {
        return hipLaunchKernel(reinterpret_cast<const void *>(&gdr_state_kernel<32>),
                               dim3((unsigned)(groups * 8 * (kD / 32))), dim3(kThreads), args, 0, st);
    }
    return hipLaunchKernel(reinterpret_cast<const void *>(&gdr_state_kernel<16>),
                           dim3((unsigned)(groups * 8 * (kD / 16))), dim3(kThreads), args, 0, st);
}

}  // namespace gdr
