// mc_readout.hip -- Memory-Caching read-out over cached segment states.
//
// Memory Caching: RNNs with Growing Memory, sections 2 and 3: the state at the end
// of every segment is cached, and a token reads the caches of the segments before
// its own besides the online state.  For one (batch b, head h), token t in segment
// j_t = min(floor(t / seg_len), N) adds
//     sum over s < j_t of  g[t, s] * M_s^T q_t                     (gated residual)
// with g == 1 for the plain residual memory.  Memory soup equals the gated form for
// a linear memory, and sparse selective caching is the gated form with most gates
// zero, so one kernel serves all of them.
//
// Two launches:
//   mc_prep_kernel     caches -> workspace: every matrix transposed (rows = value
//                      channels) and split into two bf16 terms (hi + lo).  For the
//                      residual memory it stores the prefix sums P_j = sum_{s < j} M_s
//                      instead (slot j - 1), so each token needs one matrix.
//   mc_readout_kernel  256 tokens of one (b, h) per workgroup, 64 per wave.  The
//                      query tile stays in registers; for each matrix the workgroup
//                      copies its two terms (64 KB) into LDS (double buffered, the
//                      next one in flight while the current one is used), every wave
//                      forms Q M (bf16 MFMA, both terms) per 16-column tile and adds
//                      it to its fp32 accumulators scaled by each token's weight.  A
//                      wave whose 64 tokens all have weight 0 for a matrix skips its
//                      products.  The accumulators go out through LDS as whole rows,
//                      added to o_in and rounded once.
// The contraction is dense (2 x 64 x 128 x 128 flop per token tile and matrix), so
// this is a matrix-core kernel; its bound is MFMA issue.
#include "gdr_device.hpp"
#include "gdr_internal.hpp"
#include "gdr_mfma.hpp"

namespace gdr {
namespace {

constexpr int kMD = 128;            // dk == dv
constexpr int kMTok = 256;          // tokens per workgroup
constexpr int kMPitch = kMD + 4;    // fp32 row pitch of the output staging

struct McLds {
    union {
        uint16_t M[2][2][kMD][kMD];       // [buffer][hi, lo][value column j][key i]; piece p of row j at p ^ (j & 15)
        float Acc[4][64][kMPitch];        // epilogue: each wave's 64 output rows (fp32)
    };
    float W[2][kMTok];                    // per-token weight of the buffer's matrix
};

// ---------------------------------------------------------------------------
// caches -> transposed two-term bf16 matrices (or their prefix sums)
// ---------------------------------------------------------------------------
// grid (B * H, 8, z): block y handles key rows 16 y .. 16 y + 15; block z the caches
// z, z + gridDim.z, ... (the prefix sums run through all caches in one block, z = 1).
// A thread reads 8 consecutive value columns of one key row (coalesced), the strip
// is transposed through LDS, and a thread writes 8 consecutive keys of one value
// row per term.
template <bool PREFIX>
__global__ void __launch_bounds__(256) mc_prep_kernel(const float *__restrict__ ckpt, uint16_t *__restrict__ mt,
                                                      int N) {
    __shared__ float strip[16][kMD + 1];
    const long bh = blockIdx.x;
    const int i0 = 16 * blockIdx.y;
    const int tid = threadIdx.x;
    const int ri = tid >> 4, cj = 8 * (tid & 15);  // read: key row i0 + ri, value columns cj .. cj + 7
    const int wj = tid >> 1, wi = 8 * (tid & 1);   // write: value row wj, keys i0 + wi .. + 7
    float run[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s = blockIdx.z; s < N; s += gridDim.z) {
        const float *src = ckpt + ((bh * N + s) * kMD + i0 + ri) * kMD + cj;
        const float4 a = *reinterpret_cast<const float4 *>(src);
        const float4 c = *reinterpret_cast<const float4 *>(src + 4);
        const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            run[e] = PREFIX ? run[e] + x[e] : x[e];
            strip[ri][cj + e] = run[e];
        }
        __syncthreads();
        u32x4 hi, lo;
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v0 = strip[wi + 2 * e][wj], v1 = strip[wi + 2 * e + 1][wj];
            hw[e] = pk_bf16(v0, v1);
            lw[e] = pk_bf16(v0 - __uint_as_float(hw[e] << 16), v1 - __uint_as_float(hw[e] & 0xffff0000u));
        }
        hi = u32x4{hw[0], hw[1], hw[2], hw[3]};
        lo = u32x4{lw[0], lw[1], lw[2], lw[3]};
        uint16_t *dst = mt + (bh * N + s) * (2L * kMD * kMD) + (long)wj * kMD + i0 + wi;
        *reinterpret_cast<u32x4 *>(dst) = hi;
        *reinterpret_cast<u32x4 *>(dst + kMD * kMD) = lo;
        __syncthreads();  // strip is rewritten by the next matrix
    }
}

struct McParams {
    int B, T, H, N, seg, residual;
    const uint16_t *q;    // [B, T, H, 128] bf16
    const uint16_t *mt;   // [B * H][N][2][128][128] bf16 (prep output)
    const float *gates;   // [B, T, H, N] (gated form)
    const uint16_t *oin;  // may be NULL
    uint16_t *oout;
};

// B fragment (natural order, keys 32 kk + 8 q .. + 7) of transposed-matrix row j
__device__ __forceinline__ u32x4 mt_frag(const uint16_t (*M)[kMD], int j, int kk, int q) {
    return *reinterpret_cast<const u32x4 *>(&M[j][8 * ((4 * kk + q) ^ (j & 15))]);
}

__global__ void __launch_bounds__(256) mc_readout_kernel(McParams p, int ntb, int nbh) {
    __shared__ McLds sm;
    // the blocks of one (b, h) run on one XCD (they share its matrices in L2)
    const int x = blockIdx.x, xcd = x & 7, slot = x >> 3;
    const int bh = (slot / ntb) * 8 + xcd, tb = slot % ntb;
    if (bh >= nbh) return;
    const int b = bh / p.H, h = bh % p.H;
    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, r = l & 15, q = l >> 4;
    const int t0 = tb * kMTok;
    const int tlast = min(t0 + kMTok, p.T) - 1;
    auto seg_of = [&](int t) { return min(t / p.seg, p.N); };
    // matrices this workgroup reads: gated form s in [0, j(tlast)); residual form the
    // prefix slots j - 1 for j in [max(j(t0), 1), j(tlast)]
    int m_lo, m_hi;
    if (p.residual) {
        m_lo = max(seg_of(t0), 1) - 1;
        m_hi = seg_of(tlast);
    } else {
        m_lo = 0;
        m_hi = seg_of(tlast);
    }
    const int nm = max(m_hi - m_lo, 0);

    // this thread's token (weights) and this wave's query fragments (rows clamped)
    const int tw = t0 + tid;
    const int jt = tw < p.T ? seg_of(tw) : 0;
    auto weight_src = [&](int m) -> float {
        if (tw >= p.T) return 0.f;
        if (p.residual) return (jt >= 1 && jt - 1 == m) ? 1.f : 0.f;
        return m < jt ? p.gates[(((long)b * p.T + tw) * p.H + h) * p.N + m] : 0.f;
    };
    u32x4 qa[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int t = min(t0 + 64 * wv + 16 * tt + r, p.T - 1);
        const uint16_t *qr = p.q + (((long)b * p.T + t) * p.H + h) * kMD;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qa[tt][kk] = *reinterpret_cast<const u32x4 *>(qr + 32 * kk + 8 * q);
    }
    f32x4 acc[4][8];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[tt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    // copy of matrix m into buffer bb: 64 KB = 64 copies of 1 KB (4 rows), 16 per wave.
    // Lane l covers row 4 g + l / 16, stored piece l % 16 = global piece ^ (row & 15).
    auto issue = [&](int m, int bb) __attribute__((always_inline)) {
        const uint16_t *src = p.mt + ((long)bh * p.N + m) * (2L * kMD * kMD);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int ci = 16 * wv + u, z = ci >> 5, row = 4 * (ci & 31) + (l >> 4);
            const int gp = (l & 15) ^ (row & 15);
            dma16(src + ((long)z * kMD + row) * kMD + 8 * gp, &sm.M[bb][z][4 * (ci & 31)][0]);
        }
    };

    float wnext = 0.f;
    if (nm > 0) {
        issue(m_lo, 0);
        wnext = weight_src(m_lo);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    for (int i = 0; i < nm; ++i) {
        const int m = m_lo + i, bb = i & 1;
        const float wcur = wnext;
        sm.W[bb][tid] = wcur;
        if (i + 1 < nm) {
            issue(m + 1, bb ^ 1);
            wnext = weight_src(m + 1);
        }
        const bool any = __builtin_amdgcn_ballot_w64(wcur != 0.f) != 0;
        if (any) {
            f32x4 wt[4];  // weights of this lane's C rows 16 tt + 4 q + i
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) wt[tt] = *reinterpret_cast<const f32x4 *>(&sm.W[bb][64 * wv + 16 * tt + 4 * q]);
            const uint16_t(*Mh)[kMD] = sm.M[bb][0];
            const uint16_t(*Ml)[kMD] = sm.M[bb][1];
            // B fragments of the next 16-column tile are read while the current tile's
            // products run (two register sets), so the LDS latency stays hidden
            u32x4 bf[2][8];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf[0][kk] = mt_frag(Mh, r, kk, q);
                bf[0][4 + kk] = mt_frag(Ml, r, kk, q);
            }
            // the products of tile ct go to tmp[ct & 1]; tile ct - 1's gated add runs on the
            // vector ALU while they execute
            f32x4 tmp[2][4];
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const int cur = ct & 1;
                if (ct + 1 < 8) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        bf[cur ^ 1][kk] = mt_frag(Mh, 16 * (ct + 1) + r, kk, q);
                        bf[cur ^ 1][4 + kk] = mt_frag(Ml, 16 * (ct + 1) + r, kk, q);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) tmp[cur][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        tmp[cur][tt] = mfma(as_bf16x8(qa[tt][kk]), as_bf16x8(bf[cur][kk]), tmp[cur][tt]);
                        tmp[cur][tt] = mfma(as_bf16x8(qa[tt][kk]), as_bf16x8(bf[cur][4 + kk]), tmp[cur][tt]);
                    }
                if (ct > 0) {
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) acc[tt][ct - 1] += wt[tt] * tmp[cur ^ 1][tt];
                }
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) acc[tt][7] += wt[tt] * tmp[1][tt];
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next matrix has landed
        __syncthreads();                     // and this buffer is free again
    }

    // epilogue: accumulators -> LDS rows (fp32) -> + o_in -> bf16 rows of 16 bytes
    float(*A)[kMPitch] = sm.Acc[wv];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) A[16 * tt + 4 * q + i][16 * ct + r] = acc[tt][ct][i];
    // each wave reads back only its own rows, and a wave's LDS accesses complete in order
    // all of this lane's o_in pieces are requested before any is used (one memory
    // latency per workgroup, not one per piece); rows past T are clamped on load
    // and not stored
    u32x4 oi[16];
    if (p.oin) {
#pragma unroll
        for (int it = 0; it < 16; ++it) {
            const int pi = 64 * it + l, row = pi >> 4, pc = pi & 15;
            const int t = min(t0 + 64 * wv + row, p.T - 1);
            oi[it] = *reinterpret_cast<const u32x4 *>(p.oin + (((long)b * p.T + t) * p.H + h) * kMD + 8 * pc);
        }
    }
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int pi = 64 * it + l, row = pi >> 4, pc = pi & 15;
        const int t = t0 + 64 * wv + row;
        const f32x4 a0 = *reinterpret_cast<const f32x4 *>(&A[row][8 * pc]);
        const f32x4 a1 = *reinterpret_cast<const f32x4 *>(&A[row][8 * pc + 4]);
        float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        if (p.oin) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] += __uint_as_float(oi[it][e] << 16);
                v[2 * e + 1] += __uint_as_float(oi[it][e] & 0xffff0000u);
            }
        }
        if (t < p.T)
            *reinterpret_cast<u32x4 *>(p.oout + (((long)b * p.T + t) * p.H + h) * kMD + 8 * pc) =
                u32x4{pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3]), pk_bf16(v[4], v[5]), pk_bf16(v[6], v[7])};
    }
}

}  // namespace

size_t mc_readout_workspace(int B, int H, int N) { return (size_t)B * H * N * 2 * kMD * kMD * sizeof(uint16_t); }

hipError_t launch_mc_readout(int B, int T, int H, int N, int seg, const void *q, const float *ckpt,
                             const float *gates, const void *oin, void *oout, void *ws, hipStream_t st) {
    const int nbh = B * H;
    if (nbh == 0 || T == 0) return hipSuccess;
    uint16_t *mt = static_cast<uint16_t *>(ws);
    const bool residual = gates == nullptr;
    if (N > 0) {
        const void *fn = residual ? reinterpret_cast<const void *>(&mc_prep_kernel<true>)
                                  : reinterpret_cast<const void *>(&mc_prep_kernel<false>);
        const float *src = ckpt;
        int n = N;
        void *args[] = {&src, &mt, &n};
        const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)nbh, kMD / 16, residual ? 1u : (unsigned)N),
                                             dim3(256), args, 0, st);
        if (e != hipSuccess) return e;
    }
    McParams p;
    p.B = B; p.T = T; p.H = H; p.N = N; p.seg = seg; p.residual = residual;
    p.q = static_cast<const uint16_t *>(q);
    p.mt = mt;
    p.gates = gates;
    p.oin = static_cast<const uint16_t *>(oin);
    p.oout = static_cast<uint16_t *>(oout);
    int ntb = (T + kMTok - 1) / kMTok;
    const unsigned grid = (unsigned)(8 * ((nbh + 7) / 8) * ntb);
    int nb = nbh;
    void *args[] = {&p, &ntb, &nb};
    return hipLaunchKernel(reinterpret_cast<const void *>(&mc_readout_kernel), dim3(grid), dim3(256), args, 0, st);
}

}  // namespace gdr
