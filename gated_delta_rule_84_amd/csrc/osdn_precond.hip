// osdn_precond.hip -- OSDN phase 1: the preconditioner scan over the key stream.
//
// OSDN page, sections 2.2 (closed-form hypergradient surrogate, two phases) and
// 2.3 (retention gate of the preconditioner).  For one (batch, head), with the
// diagonal preconditioner d (d_0 given) and, per token t,
//     kw_t = d_t (.) k_t,   u_t = 1 - beta_t <d_t, a_t>,   a_t = k_t (.) k_t
//     d_{t+1} = r_t d_t + e_t a_t,   e_t = c_t u_t,   c_t = eta beta_t / |k_t|^2
// (the online-gradient-descent step on the surrogate; c_t = 0 for a zero key), and
// the per-token loss ratio of phase 2 is u_t^2; q_geo = exp(mean_t log u_t^2).
//
// The update is affine in d, so a chunk of n <= 64 tokens starting from d_0 obeys
//     d_t = P_t d_0 + sum_{j<t} (P_t / P_{j+1}) e_j a_j,       P_t = prod_{i<t} r_i
//     (I + A) e = z,   A_{tj} = c_t beta_t (P_t / P_{j+1}) <a_t, a_j>  (j < t),
//                      z_t = c_t - c_t beta_t P_t <a_t, d_0>.
// Four launches:
//   osdn_chunk_kernel   every chunk in parallel: a, |k|^2, the coefficients, the
//                       decayed Gram matrix and Tm = (I + A)^{-1} (unit lower
//                       triangular: the four 16 x 16 diagonal blocks by forward
//                       substitution, one column per thread, then the off-diagonal
//                       blocks by distance from the diagonal), into a workspace record.
//   osdn_chain_kernel   one workgroup per (batch, head), chunks in order, only what
//                       the next chunk needs: x_t = <a_t, d_0>, e = Tm z and
//                       d_n = P_n d_0 + sum_j (P_n / P_{j+1}) e_j a_j; d_0 and e of
//                       every chunk go to its record.  Four waves carry the chain, four
//                       more stage the next chunk's keys (as k^2) and record head.
//   osdn_emit_kernel    every chunk in parallel again: from d_0 and e, d one token at
//                       a time (a key channel per thread), the write keys, and the
//                       chunk's sum of log loss ratios.
//   osdn_qgeo_kernel    q_geo per (batch, head) from the chunk sums, in chunk order.
// Everything is fp32 (exact products of the stored keys) except the log-ratio
// sums (fp64).  The chain is the only sequential part: three small matrix-vector
// products per chunk, on one workgroup per (batch, head).  For a long sequence and a
// caller-owned execution context, the chunks are cut into blocks: the chunk solve of
// every block and the emission of each finished block run on the context's second
// stream while the chain works through the blocks in order on the caller's stream (it
// occupies one CU per sequence, so the parallel passes fill the others); the chain
// carries d from one block to the next through the next chunk's record.
#include <math.h>

#include "gdr_device.hpp"
#include "gdr_internal.hpp"
#include "gdr_mfma.hpp"
#include "gdr_ut.hpp"

namespace gdr {
namespace {

constexpr int kPL = 64;       // tokens per chunk
constexpr int kPD = 128;      // largest dk
constexpr int kPThreads = 256;

// workspace record of one (b, h, chunk), fp32 words
constexpr int kPrT = 0;                    // [64][64] Tm (row t, column j)
constexpr int kPrC = kPrT + kPL * kPL;     // [64] c_t
constexpr int kPrCb = kPrC + kPL;          // [64] c_t beta_t
constexpr int kPrBeta = kPrCb + kPL;       // [64] beta_t
constexpr int kPrR = kPrBeta + kPL;        // [64] r_t
constexpr int kPrP = kPrR + kPL;           // [64] P_t
constexpr int kPrRho = kPrP + kPL;         // [64] P_n / P_{j+1} (0 past the chunk end)
constexpr int kPrPn = kPrRho + kPL;        // P_n (slot of 64)
constexpr int kPrD0 = kPrPn + kPL;         // [128] d at the chunk start      (chain)
constexpr int kPrE = kPrD0 + kPD;          // [64] e_t                         (chain)
constexpr int kPrLog = kPrE + kPL;         // fp64: sum of log loss ratios      (emit)
constexpr int kPrWords = kPrLog + kPL;     // 4800 words = 19,200 bytes

struct PcParams {
    int B, T, H, dk, io_bf16, gate_bf16, NT;
    int c0, c1;  // the launch covers chunks c0 .. c1 - 1 of every (batch, head)
    float eta;
    const void *k, *beta, *r;
    const float *d0;
    void *kw;
    float *dT, *qgeo;
    float *rec;
};

// retention gates at or below this act as full forgetting (their logarithm stays finite)
constexpr float kRMin = 1e-30f;

// keys of one chunk into LDS as fp32 (rows past the chunk end zero): every
// 16-byte piece of the tile is requested before any is written out.  Loads are
// unconditional (rows clamped to the chunk) so that the compiler can count them;
// pieces past row 63 land in the sink row kPL of kf.
template <bool BF, int PITCH, bool SQ = false>
__device__ __forceinline__ void load_keys(const PcParams &p, float (*kf)[PITCH], long tok0, int n, int tid) {
    // the keys of one chunk into rows of kf (k^2 when SQ); rows past the chunk end and
    // pieces past the 64 rows go to row kPL (the sink) as zeros
    constexpr int es = BF ? 2 : 4;
    const int kpieces = p.dk * es / 16;
    const char *kb = static_cast<const char *>(p.k);
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int e = tid + kPThreads * u, t = min(e / kpieces, n - 1), pc = e % kpieces;
        v[u] = *reinterpret_cast<const u32x4 *>(kb + (tok0 + (long)t * p.H) * p.dk * es + 16 * pc);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int e = tid + kPThreads * u, t = e / kpieces, pc = e % kpieces;
        const int row = min(t, kPL);
        const bool live = t < n;
        constexpr int nv = BF ? 8 : 4;
        float x[nv];
#pragma unroll
        for (int j = 0; j < nv; ++j) {
            const uint32_t wd = v[u][BF ? j >> 1 : j];
            const float f = BF ? __uint_as_float((j & 1) ? (wd & 0xffff0000u) : (wd << 16)) : __uint_as_float(wd);
            x[j] = live ? (SQ ? f * f : f) : 0.f;
        }
        if (PITCH % 4 == 0) {  // 16-byte rows: vector writes
#pragma unroll
            for (int j = 0; j < nv; j += 4)
                *reinterpret_cast<f32x4 *>(&kf[row][nv * pc + j]) = f32x4{x[j], x[j + 1], x[j + 2], x[j + 3]};
        } else {
#pragma unroll
            for (int j = 0; j < nv; ++j) kf[row][nv * pc + j] = x[j];
        }
    }
}

// Lane exchanges on the vector ALU (DPP), in place of shuffles through the LDS unit:
// the value of lane l ^ 1 or l ^ 2 (quad permutes), and of lane l + 4 inside its row of
// 16 (lanes 12 .. 15 of a row receive 0).  All lanes of the wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]
constexpr int kDppShl4 = 0x104;  // row_shl:4

// workgroup barrier that waits only for this wave's LDS operations: global loads
// issued for the next chunk stay in flight across it (the memory clobber keeps the
// compiler from moving memory operations across)
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <bool BF>
__global__ void __launch_bounds__(kPThreads) osdn_chunk_kernel(PcParams p) {
    // row kPL: sink of the key copy; a row pitch of 4 mod 64 words keeps the
    // 16 x 4 fragment reads of the Gram products free of bank conflicts
    __shared__ __attribute__((aligned(16))) float a[kPL + 1][kPD + 4];
    __shared__ __attribute__((aligned(16))) float A[kPL][kPL + 4];   // A (strictly lower)
    __shared__ __attribute__((aligned(16))) float Ti[kPL][kPL + 8];  // Tm, strictly lower part (unit diagonal implicit)
    __shared__ __attribute__((aligned(16))) float Xs[4][16][16];     // UT transform scratch
    __shared__ float nk[kPL], lg[kPL + 1], cb[kPL];
    const int tid = threadIdx.x;
    const int nc = p.c1 - p.c0;
    const int bh = (int)(blockIdx.x / nc), c = p.c0 + (int)(blockIdx.x % nc);
    const int b = bh / p.H, h = bh % p.H, dk = p.dk;
    const int t0 = c * kPL, n = min(kPL, p.T - t0);
    float *rec = p.rec + ((long)bh * p.NT + c) * kPrWords;
    const long tok0 = ((long)b * p.T + t0) * p.H + h;

    // this token's gates are requested together with the keys
    float bt = 0.f, rt = 1.f;
    if (tid < n) {
        const long tk = tok0 + (long)tid * p.H;
        bt = ld_elem(p.beta, tk, p.gate_bf16);
        if (p.r) rt = ld_elem(p.r, tk, p.gate_bf16);
    }
    load_keys<BF, kPD + 4, true>(p, a, tok0, n, tid);
    __syncthreads();
    {  // |k_t|^2 = sum of the row of a = k^2 (4 lanes per row, 16-byte reads)
        const int t = tid >> 2, part = tid & 3;
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int i0 = 32 * part + 4 * m;
            const f32x4 x = *reinterpret_cast<const f32x4 *>(&a[t][min(i0, kPD - 4)]);
#pragma unroll
            for (int y = 0; y < 4; ++y) s4[y] += i0 + y < dk ? x[y] : 0.f;
        }
        float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        s += dpp_mov<kDppXor1>(s);
        s += dpp_mov<kDppXor2>(s);
        if (part == 0) nk[t] = s;
    }
    __syncthreads();  // nk is read by wave 0 below
    if (tid < kPL) {  // one wave: coefficients and the cumulative log retention (scan)
        const int t = tid;
        const float ct = nk[t] > 0.f ? p.eta * bt / nk[t] : 0.f;
        rec[kPrC + t] = ct;
        rec[kPrCb + t] = ct * bt;
        rec[kPrBeta + t] = bt;
        rec[kPrR + t] = rt;
        cb[t] = ct * bt;
        float x = logf(fmaxf(rt, kRMin));  // inclusive prefix sum over the 64 lanes
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off);
            if (t >= off) x += y;
        }
        lg[t + 1] = x;  // log P_{t+1}
        if (t == 0) lg[0] = 0.f;
    }
    __syncthreads();
    if (tid < kPL) {
        const float ln = lg[n];
        rec[kPrP + tid] = expf(lg[tid]);
        rec[kPrRho + tid] = tid < n ? expf(ln - lg[tid + 1]) : 0.f;
        if (tid == 0) rec[kPrPn] = expf(ln);
    }

    // A_{tj} = cb_t (P_t / P_{j+1}) <a_t, a_j> for j < t < n.  The Gram products on fp32
    // matrix cores (v_mfma_f32_16x16x4_f32: lane (r, q) supplies A[r][q] and B[q][r] of a
    // 4-channel step, C tiles hold C[4q .. 4q+3][r]): the ten 16 x 16 tiles on or below
    // the diagonal, three or two per wave, each pass over the channels reading one
    // fragment per tile row and column.
    {
        const int w = tid >> 6, l = tid & 63, r = l & 15, q = l >> 4;
        // tiles (I, J) of wave w: 0: (0,0) (1,0) (1,1); 1: (2,0) (2,1) (2,2); 2: (3,0) (3,1); 3: (3,2) (3,3)
        const int I0 = w == 0 ? 0 : w == 1 ? 2 : 3;
        const int J0 = w < 2 ? 0 : w == 2 ? 0 : 2;
        const int nt = w < 2 ? 3 : 2;
        // tile k of the wave: row I, column J
        auto tI = [&](int k) { return w == 0 ? (k == 0 ? 0 : 1) : I0; };
        auto tJ = [&](int k) { return w == 0 ? (k == 2 ? 1 : 0) : J0 + k; };
        f32x4 acc[3] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        // a wave with two tiles also forms a copy of its first one in the third slot
        // (never stored), so the loop carries no branch; two channel steps per
        // iteration (dk is a multiple of 8), every operand read before the products
        int ra[3], rb[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int kk = k < nt ? k : 0;
            ra[k] = 16 * tI(kk) + r;
            rb[k] = 16 * tJ(kk) + r;
        }
        const int ksteps = dk / 4;
        for (int st = 0; st < ksteps; st += 2) {
            float av[2][3], bv[2][3];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    av[u][k] = a[ra[k]][4 * (st + u) + q];
                    bv[u][k] = a[rb[k]][4 * (st + u) + q];
                }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int k = 0; k < 3; ++k)
                    acc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u][k], bv[u][k], acc[k], 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            if (k < nt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * tI(k) + 4 * q + i, j = 16 * tJ(k) + r;
                    A[t][j] = (j < t && t < n) ? cb[t] * expf(lg[t] - lg[j + 1]) * acc[k][i] : 0.f;
                }
            }
        }
        // the tiles above the diagonal are never read (A is strictly lower)
    }
    __syncthreads();

    // Tm = (I + A)^{-1}: diagonal 16 x 16 blocks by forward substitution, the others by
    // the 2 x 2 block-inverse rule on fp32 matrix cores
    ut_transform(A, Ti, Xs, tid >> 6, tid & 63);
    for (int e4 = tid; e4 < kPL * kPL / 4; e4 += kPThreads) {  // 16-byte stores
        const int t = e4 / (kPL / 4), j0 = 4 * (e4 % (kPL / 4));
        f32x4 v;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int j = j0 + x;
            v[x] = j < t ? Ti[t][j] : (j == t ? 1.f : 0.f);
        }
        *reinterpret_cast<f32x4 *>(rec + kPrT + 4 * e4) = v;
    }
}

template <bool BF>
__global__ void __launch_bounds__(2 * kPThreads) osdn_chain_kernel(PcParams p) {
    // chunk operands, double buffered: a = k^2 (rows of 132 floats: 16-byte aligned,
    // zero past dk; row kPL is a sink), Tm and the vector rows of the record
    constexpr int kKP = kPD + 4;
    __shared__ __attribute__((aligned(16))) float kf[2][kPL + 1][kKP];
    __shared__ __attribute__((aligned(16))) float Tm[2][kPL][kPL + 4];
    __shared__ __attribute__((aligned(16))) float vc[2][7][kPL];  // c, cb, beta, r, P, rho, (Pn in [6][0])
    __shared__ __attribute__((aligned(16))) float d[kPD];
    __shared__ __attribute__((aligned(16))) float zs[kPL], we[kPL];
    // waves 0-3 carry the chain; waves 4-7 ("stagers") copy the chunk after the current
    // one into the other half of the LDS double buffer, so that the chain's waves do
    // nothing between their three barriers per chunk but the chain
    const int tid = threadIdx.x & (kPThreads - 1);
    const bool stager = threadIdx.x >= kPThreads;
    const int bh = blockIdx.x;
    const int b = bh / p.H, h = bh % p.H, dk = p.dk;
    for (int i = threadIdx.x; i < 2 * (kPL + 1) * kKP; i += 2 * kPThreads) (&kf[0][0][0])[i] = 0.f;
    // d at the start of chunk c0: the initial preconditioner, or (a later block of
    // chunks) what the launch for the block before left in chunk c0's record
    if (!stager && tid < kPD) {
        float v = 0.f;
        if (tid < dk)
            v = p.c0 > 0 ? p.rec[((long)bh * p.NT + p.c0) * kPrWords + kPrD0 + tid]
                         : (p.d0 ? p.d0[(long)bh * dk + tid] : 1.f);
        d[tid] = v;
    }

    // stagers: register copies of two chunks ahead (two sets, used alternately): keys
    // (16-byte pieces) and the record head (Tm and the vectors: 1,136 pieces)
    constexpr int ksz = BF ? 2 : 4;  // bytes per key element
    const int kpieces = dk * ksz / 16;
    constexpr int NKP = BF ? 4 : 8;  // key pieces per stager thread (64 rows of at most 128 keys)
    u32x4 kA[NKP], rA[5], kB[NKP], rB[5];
    // this thread's key pieces (row, 16-byte piece) are the same in every chunk
    int prow[NKP], ppc[NKP];
#pragma unroll
    for (int u = 0; u < NKP; ++u) {
        const int e = tid + kPThreads * u;
        prow[u] = e / kpieces;
        ppc[u] = e - prow[u] * kpieces;
    }
    auto load_chunk = [&](int c, u32x4 (&kreg)[NKP], u32x4 (&rreg)[5]) __attribute__((always_inline)) {
        const int t0 = c * kPL, n = min(kPL, p.T - t0);
        const char *kb = static_cast<const char *>(p.k);
#pragma unroll
        for (int u = 0; u < NKP; ++u) {  // unconditional (rows clamped): the compiler counts them
            const int t = min(prow[u], n - 1);
            kreg[u] = *reinterpret_cast<const u32x4 *>(kb + ((((long)b * p.T + t0 + t) * p.H + h) * dk) * ksz + 16 * ppc[u]);
        }
        const float *rec = p.rec + ((long)bh * p.NT + c) * kPrWords;
#pragma unroll
        for (int u = 0; u < 5; ++u) {
            const int w4 = min(tid + kPThreads * u, kPrD0 / 4 - 1);
            rreg[u] = *reinterpret_cast<const u32x4 *>(rec + 4 * w4);
        }
    };
    // the keys of chunk c into buffer bf as k^2, and the record head
    auto store_keys = [&](int c, int bf, const u32x4 (&kreg)[NKP]) __attribute__((always_inline)) {
        const int t0 = c * kPL, n = min(kPL, p.T - t0);
#pragma unroll
        for (int u = 0; u < NKP; ++u) {
            const int t = prow[u], pc = ppc[u];
            const int row = min(t, kPL);
            const bool live = t < n;
            if (BF) {
                f32x4 lo, hi;
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    const float k0 = live ? __uint_as_float(kreg[u][x] << 16) : 0.f;
                    const float k1 = live ? __uint_as_float(kreg[u][x] & 0xffff0000u) : 0.f;
                    const float k2 = live ? __uint_as_float(kreg[u][x + 2] << 16) : 0.f;
                    const float k3 = live ? __uint_as_float(kreg[u][x + 2] & 0xffff0000u) : 0.f;
                    lo[2 * x] = k0 * k0;
                    lo[2 * x + 1] = k1 * k1;
                    hi[2 * x] = k2 * k2;
                    hi[2 * x + 1] = k3 * k3;
                }
                *reinterpret_cast<f32x4 *>(&kf[bf][row][8 * pc]) = lo;
                *reinterpret_cast<f32x4 *>(&kf[bf][row][8 * pc + 4]) = hi;
            } else {
                f32x4 v;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float k0 = live ? __uint_as_float(kreg[u][x]) : 0.f;
                    v[x] = k0 * k0;
                }
                *reinterpret_cast<f32x4 *>(&kf[bf][row][4 * pc]) = v;
            }
        }
    };
    auto store_rec = [&](int bf, const u32x4 (&rreg)[5]) __attribute__((always_inline)) {
        // Tm rows then the vector rows; the clamped duplicate pieces rewrite the last
        // piece with its own value
#pragma unroll
        for (int u = 0; u < 5; ++u) {
            const int w = 4 * min(tid + kPThreads * u, kPrD0 / 4 - 1);
            float *dst = w < kPrC ? &Tm[bf][w / kPL][w % kPL] : &vc[bf][(w - kPrC) / kPL][(w - kPrC) % kPL];
            *reinterpret_cast<f32x4 *>(dst) = __builtin_bit_cast(f32x4, rreg[u]);
        }
    };

    // One chunk of the chain from buffer bf (staged during the previous chunk).  Three
    // barriers.
    auto step = [&](int c, int bf) __attribute__((always_inline)) {
        float *rec = p.rec + ((long)bh * p.NT + c) * kPrWords;
        lds_sync();  // this chunk's operands staged; d of its start complete
        if (tid < dk) rec[kPrD0 + tid] = d[tid];
        // z_t = c_t - cb_t P_t <a_t, d_0>   (4 lanes per token, 32 channels each)
        {
            const int t = tid >> 2, part = tid & 3;
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const f32x4 av = *reinterpret_cast<const f32x4 *>(&kf[bf][t][32 * part + 4 * m]);
                const f32x4 dv = *reinterpret_cast<const f32x4 *>(&d[32 * part + 4 * m]);
#pragma unroll
                for (int x = 0; x < 4; ++x) s4[x] = fmaf(av[x], dv[x], s4[x]);
            }
            float sum = (s4[0] + s4[1]) + (s4[2] + s4[3]);
            sum += dpp_mov<kDppXor1>(sum);
            sum += dpp_mov<kDppXor2>(sum);
            if (part == 0) zs[t] = vc[bf][0][t] - vc[bf][1][t] * vc[bf][4][t] * sum;
        }
        lds_sync();
        // e = Tm z  (4 lanes per token, 16 columns each, 16-byte reads)
        {
            const int t = tid >> 2, part = tid & 3;
            float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int j0 = 16 * part + 4 * m;
                const f32x4 tv = *reinterpret_cast<const f32x4 *>(&Tm[bf][t][j0]);
                const f32x4 zv = *reinterpret_cast<const f32x4 *>(&zs[j0]);
#pragma unroll
                for (int x = 0; x < 4; ++x)  // strictly lower part of Tm (its diagonal is 1)
                    s4[x] = fmaf(j0 + x < t ? tv[x] : 0.f, zv[x], s4[x]);
            }
            float sum = (s4[0] + s4[1]) + (s4[2] + s4[3]);
            sum += dpp_mov<kDppXor1>(sum);
            sum += dpp_mov<kDppXor2>(sum);
            if (part == 0) {
                we[t] = vc[bf][5][t] * (zs[t] + sum);
                rec[kPrE + t] = zs[t] + sum;
            }
        }
        lds_sync();
        // d_n = P_n d_0 + sum_j rho_j e_j a_j: lane (j group g, channel quad m) sums the
        // tokens j = 8 g .. 8 g + 7 for channels 4 m .. 4 m + 3 (16-byte reads); the eight
        // j groups of a quad are adjacent lanes
        {
            const int g = tid & 7, m = tid >> 3;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const f32x4 w0 = *reinterpret_cast<const f32x4 *>(&we[8 * g]);
            const f32x4 w1 = *reinterpret_cast<const f32x4 *>(&we[8 * g + 4]);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const f32x4 av = *reinterpret_cast<const f32x4 *>(&kf[bf][8 * g + jj][4 * m]);
                const float wj = jj < 4 ? w0[jj] : w1[jj - 4];
#pragma unroll
                for (int x = 0; x < 4; ++x) acc[x] = fmaf(wj, av[x], acc[x]);
            }
            // the eight lanes of a quad's token groups: sums over lane pairs, then quads,
            // then the quad four lanes up (only lane g = 0 uses the total)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                acc[x] += dpp_mov<kDppXor1>(acc[x]);
                acc[x] += dpp_mov<kDppXor2>(acc[x]);
                acc[x] += dpp_mov<kDppShl4>(acc[x]);
            }
            if (g == 0 && 4 * m < dk) {
                const float pn = vc[bf][6][0];
                f32x4 dv = *reinterpret_cast<const f32x4 *>(&d[4 * m]);
#pragma unroll
                for (int x = 0; x < 4; ++x) dv[x] = pn * dv[x] + acc[x];
                *reinterpret_cast<f32x4 *>(&d[4 * m]) = dv;
            }
        }
    };

    const int c0 = p.c0, c1 = p.c1;
    if (stager) {
        if (c1 > c0) {
            load_chunk(c0, kA, rA);
            if (c0 + 1 < c1) load_chunk(c0 + 1, kB, rB);
        }
        __syncthreads();  // the buffers are zeroed
        if (c1 > c0) {
            store_keys(c0, 0, kA);
            store_rec(0, rA);
            if (c0 + 2 < c1) load_chunk(c0 + 2, kA, rA);
        }
        // beside chunk c of the chain: stage chunk c + 1 into the buffer chunk c - 1 used
        // (free once the chain's waves reach the chunk's first barrier) from (kn, rn), the
        // keys and the record head in the chain's first two barrier intervals, then refill
        // (kn, rn) with chunk c + 3; the chain's three barriers are matched
        auto stage = [&](int c, u32x4 (&kn)[NKP], u32x4 (&rn)[5]) __attribute__((always_inline)) {
            lds_sync();
            if (c + 1 < c1) store_keys(c + 1, (c + 1 - c0) & 1, kn);
            lds_sync();
            if (c + 1 < c1) store_rec((c + 1 - c0) & 1, rn);
            lds_sync();
            if (c + 3 < c1) load_chunk(c + 3, kn, rn);
        };
        for (int c = c0; c < c1; c += 2) {
            stage(c, kB, rB);
            if (c + 1 < c1) stage(c + 1, kA, rA);
        }
        __syncthreads();
        return;
    }
    __syncthreads();  // the buffers are zeroed
    for (int c = c0; c < c1; ++c) step(c, (c - c0) & 1);
    __syncthreads();
    if (tid < dk) {
        if (c1 < p.NT) p.rec[((long)bh * p.NT + c1) * kPrWords + kPrD0 + tid] = d[tid];  // the next block's start
        else if (p.dT) p.dT[(long)bh * dk + tid] = d[tid];
    }
}

template <bool BF>
__global__ void __launch_bounds__(kPThreads) osdn_emit_kernel(PcParams p) {
    // rows of 132 floats (16-byte aligned, 4 mod 64 words: a column read by 64 lanes
    // touches 64 banks); row kPL of kf is the sink of the key copy
    constexpr int kKP = kPD + 4;
    __shared__ __attribute__((aligned(16))) float kf[kPL + 1][kKP];
    __shared__ __attribute__((aligned(16))) float kw[kPL][kKP];
    __shared__ float vr[kPL], ve[kPL], vb[kPL];
    __shared__ double red[kPThreads / 64];
    const int tid = threadIdx.x;
    const int nc = p.c1 - p.c0;
    const int bh = (int)(blockIdx.x / nc), c = p.c0 + (int)(blockIdx.x % nc);
    const int b = bh / p.H, h = bh % p.H, dk = p.dk;
    const int t0 = c * kPL, n = min(kPL, p.T - t0);
    float *rec = p.rec + ((long)bh * p.NT + c) * kPrWords;
    const long tok0 = ((long)b * p.T + t0) * p.H + h;
    load_keys<BF, kKP>(p, kf, tok0, n, tid);
    if (tid < kPL) {
        vr[tid] = rec[kPrR + tid];
        ve[tid] = rec[kPrE + tid];
        vb[tid] = rec[kPrBeta + tid];
    }
    __syncthreads();
    // d through the chunk, one key channel per thread; kw_t = d_t (.) k_t
    if (tid < dk) {
        float di = rec[kPrD0 + tid];
        float kc[kPL];
#pragma unroll
        for (int t = 0; t < kPL; ++t) kc[t] = kf[t][tid];
        if (n == kPL) {  // a full chunk: no per-token test
#pragma unroll
            for (int t = 0; t < kPL; ++t) {
                kw[t][tid] = di * kc[t];
                di = fmaf(vr[t], di, ve[t] * kc[t] * kc[t]);
            }
        } else {
#pragma unroll
            for (int t = 0; t < kPL; ++t) {
                if (t < n) {
                    kw[t][tid] = di * kc[t];
                    di = fmaf(vr[t], di, ve[t] * kc[t] * kc[t]);
                }
            }
        }
    }
    __syncthreads();
    // u_t = 1 - beta_t <kw_t, k_t>; the chunk's sum of log u_t^2
    double logsum = 0.0;
    {
        const int t = tid >> 2, part = tid & 3;
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int i0 = 32 * part + 4 * m, ic = min(i0, kPD - 4);
            const f32x4 x = *reinterpret_cast<const f32x4 *>(&kw[t][ic]);
            const f32x4 y = *reinterpret_cast<const f32x4 *>(&kf[t][ic]);
#pragma unroll
            for (int z = 0; z < 4; ++z) s4[z] += i0 + z < dk ? x[z] * y[z] : 0.f;
        }
        float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        s += dpp_mov<kDppXor1>(s);
        s += dpp_mov<kDppXor2>(s);
        if (part == 0 && t < n) {
            const double u = 1.0 - (double)vb[t] * (double)s;
            logsum = log(u * u);
        }
    }
    for (int off = 32; off > 0; off >>= 1) logsum += __shfl_xor(logsum, off);
    if ((tid & 63) == 0) red[tid >> 6] = logsum;
    // write keys out as rows (16 bytes per piece)
    {
        constexpr int es = BF ? 2 : 4;
        const int opieces = dk * es / 16;
        for (int e = tid; e < n * opieces; e += kPThreads) {
            const int t = e / opieces, pc = e % opieces;
            char *dst = static_cast<char *>(p.kw) + (tok0 + (long)t * p.H) * dk * es + 16 * pc;
            if (BF) {
                const f32x4 lo = *reinterpret_cast<const f32x4 *>(&kw[t][8 * pc]);
                const f32x4 hi = *reinterpret_cast<const f32x4 *>(&kw[t][8 * pc + 4]);
                uint32_t w[4];
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    w[x] = (uint32_t)f32_to_bf16(lo[2 * x]) | ((uint32_t)f32_to_bf16(lo[2 * x + 1]) << 16);
                    w[x + 2] = (uint32_t)f32_to_bf16(hi[2 * x]) | ((uint32_t)f32_to_bf16(hi[2 * x + 1]) << 16);
                }
                *reinterpret_cast<u32x4 *>(dst) = u32x4{w[0], w[1], w[2], w[3]};
            } else {
                *reinterpret_cast<u32x4 *>(dst) = __builtin_bit_cast(u32x4, *reinterpret_cast<const f32x4 *>(&kw[t][4 * pc]));
            }
        }
    }
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
        for (int w = 0; w < kPThreads / 64; ++w) tot += red[w];
        *reinterpret_cast<double *>(rec + kPrLog) = tot;
    }
}

// q_geo = exp(sum of the chunk sums / T): one workgroup per (batch, head); thread
// i sums chunks i, i + 256, ... and the 256 partial sums are added in a fixed tree
// (the same order on every run)
__global__ void __launch_bounds__(kPThreads) osdn_qgeo_kernel(PcParams p) {
    __shared__ double part[kPThreads];
    const int bh = blockIdx.x, tid = threadIdx.x;
    double tot = 0.0;
    for (int c = tid; c < p.NT; c += kPThreads)
        tot += *reinterpret_cast<const double *>(p.rec + ((long)bh * p.NT + c) * kPrWords + kPrLog);
    part[tid] = tot;
    __syncthreads();
    for (int off = kPThreads / 2; off > 0; off >>= 1) {
        if (tid < off) part[tid] += part[tid + off];
        __syncthreads();
    }
    if (tid == 0) p.qgeo[bh] = p.T > 0 ? (float)exp(part[0] / p.T) : 1.f;
}

}  // namespace

size_t osdn_precond_workspace(int B, int T, int H) {
    const long NT = (T + kPL - 1) / kPL;
    return (size_t)B * H * NT * kPrWords * sizeof(float);
}

namespace {
constexpr int kOsdnBlocks = 32;  // most chunk blocks of a call
static_assert(2 + 2 * kOsdnBlocks <= kCtxEvents, "events of one call");
}  // namespace

hipError_t launch_osdn_precond(int B, int T, int H, int dk, int io_bf16, int gate_bf16, float eta, const void *k,
                               const void *beta, const void *r, const float *d0, void *kw, float *dT, float *qgeo,
                               void *ws, const gdr_context *ctx, hipStream_t st) {
    const long nbh = (long)B * H;
    if (nbh == 0) return hipSuccess;
    PcParams p;
    p.B = B; p.T = T; p.H = H; p.dk = dk; p.io_bf16 = io_bf16; p.gate_bf16 = gate_bf16;
    p.NT = (T + kPL - 1) / kPL;
    p.c0 = 0;
    p.c1 = p.NT;
    p.eta = eta;
    p.k = k; p.beta = beta; p.r = r; p.d0 = d0; p.kw = kw; p.dT = dT; p.qgeo = qgeo;
    p.rec = static_cast<float *>(ws);
    const void *chunk_fn = io_bf16 ? reinterpret_cast<const void *>(&osdn_chunk_kernel<true>)
                                   : reinterpret_cast<const void *>(&osdn_chunk_kernel<false>);
    const void *chain_fn = io_bf16 ? reinterpret_cast<const void *>(&osdn_chain_kernel<true>)
                                   : reinterpret_cast<const void *>(&osdn_chain_kernel<false>);
    const void *emit_fn = io_bf16 ? reinterpret_cast<const void *>(&osdn_emit_kernel<true>)
                                  : reinterpret_cast<const void *>(&osdn_emit_kernel<false>);
    // chunks c0 .. c1 - 1: one block per (batch, head, chunk), or (the chain) one per (batch, head)
    auto launch = [&](const void *fn, int c0, int c1, hipStream_t s) -> hipError_t {
        PcParams a = p;
        a.c0 = c0;
        a.c1 = c1;
        void *args[] = {&a};
        const long grid = fn == chain_fn ? nbh : nbh * (c1 - c0);
        return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(fn == chain_fn ? 2 * kPThreads : kPThreads), args, 0, s);
    };
    auto finish = [&]() -> hipError_t {
        if (!qgeo) return hipSuccess;
        void *args[] = {&p};
        return hipLaunchKernel(reinterpret_cast<const void *>(&osdn_qgeo_kernel), dim3((unsigned)nbh),
                               dim3(kPThreads), args, 0, st);
    };
    hipError_t e;
    const int nblk = ctx && p.NT >= 256 ? min(kOsdnBlocks, p.NT / 64) : 1;
    if (nblk == 1) {
        if (p.NT > 0 && (e = launch(chunk_fn, 0, p.NT, st)) != hipSuccess) return e;
        if ((e = launch(chain_fn, 0, p.NT, st)) != hipSuccess) return e;  // with no chunk: dT = d0
        if (p.NT > 0 && (e = launch(emit_fn, 0, p.NT, st)) != hipSuccess) return e;
        return finish();
    }
    hipStream_t side = ctx->stream;
    const hipEvent_t fork = ctx->ev[0], join = ctx->ev[1], *solved = ctx->ev + 2, *chained = ctx->ev + 2 + kOsdnBlocks;
    auto bound = [&](int j) { return (int)((long)p.NT * j / nblk); };
    // side: every block's chunk solve; caller's stream: the chain, block by block, each
    // after its block's solve; side again: each block's emission after its chain
    if ((e = hipEventRecord(fork, st)) != hipSuccess) return e;  // inputs ready on st
    if ((e = hipStreamWaitEvent(side, fork, 0)) != hipSuccess) return e;
    for (int j = 0; j < nblk; ++j) {
        if ((e = launch(chunk_fn, bound(j), bound(j + 1), side)) != hipSuccess) return e;
        if ((e = hipEventRecord(solved[j], side)) != hipSuccess) return e;
    }
    for (int j = 0; j < nblk; ++j) {
        if ((e = hipStreamWaitEvent(st, solved[j], 0)) != hipSuccess) return e;
        if ((e = launch(chain_fn, bound(j), bound(j + 1), st)) != hipSuccess) return e;
        if ((e = hipEventRecord(chained[j], st)) != hipSuccess) return e;
    }
    for (int j = 0; j < nblk; ++j) {
        if ((e = hipStreamWaitEvent(side, chained[j], 0)) != hipSuccess) return e;
        if ((e = launch(emit_fn, bound(j), bound(j + 1), side)) != hipSuccess) return e;
    }
    if ((e = hipEventRecord(join, side)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(st, join, 0)) != hipSuccess) return e;
    return finish();
}

}  // namespace gdr
