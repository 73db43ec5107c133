// dmem.hip -- delta-mem context pass: token-state, sequence-state and multi-state writes.
//
// delta-mem: Efficient Online Memory for Large Language Models, section 2.A (update
// rule), 2.C (read from the memory before the write) and 2.D (write granularities).
// Per memory (one (batch, head), R x R, row a predicting value component a as M k):
//     read   r_t = M q_t                        (the memory before t's segment is written)
//     write  M <- lambda M + beta (vbar - M kbar) kbar^T     once per segment
// where kbar, vbar are the means of the segment's keys and values and lambda, beta
// the gates stored at its last token (a segment of one token: the per-token write).
// With J sub-states per group (consecutive heads h = g J + j) the group's read is
// the sum of its J reads.
//
// Layout of the work: one lane per memory row -- lane (m, a) of a wave holds row a of
// memory m in registers (R floats), so a wave carries 64 / R memories and the dot
// products M q, M k are per-lane loops with no cross-lane reduction.  The J reads of a
// group sit in adjacent lane groups and are summed by xor shuffles.  Each wave stages
// its memories' inputs through LDS in blocks of 32 tokens (16 for fp32 rows), copied
// buffer -> LDS one block ahead into a double buffer (the copies of one wave serve only
// that wave, so no workgroup barrier is needed).  A segment's write is computed for
// every token and selected where the segment closes (the memories of one wave close
// their segments at different tokens).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr_device.hpp"
#include "gdr_internal.hpp"
#include "gdr_mfma.hpp"

namespace gdr {
namespace {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void *lds_ptr_t;

constexpr int kWaves = 4;     // waves per workgroup

// x + x of lane (l xor 1): a quad permutation [1, 0, 3, 2] on the DPP path (no LDS trip)
__device__ __forceinline__ float add_xor1(float x) {
    const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false);
    return x + __int_as_float(y);
}

// Buffer resource over `bytes` bytes from `base`: loads past the end return 0 (the
// hardware range check), so every token block and every 4-byte gate word can be
// loaded whole.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// Per-wave LDS staging of one block of TB tokens for the wave's MPW memories: the q,
// k, v rows (NP 16-byte pieces each; piece p of the row of (token tl, memory ml) at
// index (tl MPW + ml) NP + p) and the 4-byte words holding each (token, memory)'s
// lambda, beta and segment mark.
template <int R, int L, bool IOB, int TB>
struct Stage {
    static constexpr int MPW = 64 / (R * L);
    static constexpr int NP = R * (IOB ? 2 : 4) / 16;
    u32x4v rows[3][TB * MPW * NP];
    uint32_t lam[TB * MPW], beta[TB * MPW], seg[TB * MPW];
};

// L lanes share one memory row (C = R / L columns each; their partial dot products are
// combined by one shuffle), so that a small batch still gives every SIMD several waves.
template <int R, int L, bool IOB, bool GB, bool SEG, int J>
__global__ void __launch_bounds__(64 * kWaves) dmem_fwd_kernel(DmemParams p) {
    constexpr int es = IOB ? 2 : 4, gs = GB ? 2 : 4;
    constexpr int MPW0 = 64 / (R * L);
    constexpr int TB = (IOB ? 32 : 16) > 64 / MPW0 ? (IOB ? 32 : 16) : 64 / MPW0;  // tokens per staged block
    constexpr int C = R / L;                   // columns of the row held by a lane
    using St = Stage<R, L, IOB, TB>;
    constexpr int MPW = St::MPW, NP = St::NP;  // memories per wave, 16-byte pieces per row
    constexpr int TPI = 64 / (NP * MPW);       // tokens per row copy (one 16-byte piece per lane)
    constexpr int GPI = 64 / MPW;              // tokens per gate copy (one word per lane)
    static_assert(MPW % J == 0, "a group's sub-states share a wave");
    static_assert(TB % TPI == 0 && TB % GPI == 0, "whole copies per block");
    __shared__ St stage[kWaves][2];

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, half = lane % L, a = (lane / L) % R, ml = lane / (L * R);
    const int c0 = C * half;                   // first column of this lane
    const long nmem = (long)p.B * p.H, T = p.T;
    const long m0 = ((long)blockIdx.x * kWaves + wv) * MPW;
    const long m = m0 + ml;
    const bool valid = m < nmem;
    auto memory = [&](long mm, int &b, int &h) {  // lanes past the end work on the last memory
        mm = mm < nmem ? mm : nmem - 1;
        b = (int)(mm / p.H);
        h = (int)(mm % p.H);
    };
    int b, h;
    memory(m, b, h);
    const int G = p.H / J, g = h / J, j = h % J;

    const unsigned row_bytes = (unsigned)(nmem * T * R * es), gate_bytes = (unsigned)(nmem * T * gs);
    const unsigned seg_bytes = (unsigned)(p.B * T);
    // the 4-byte word staged for gate element e (segment mark byte sb): the aligned word
    // holding it, moved back so that it ends inside the tensor (the range check would
    // turn a word reaching past the end into 0); tensors under 4 bytes are read directly
    const bool tiny_g = gate_bytes < 4, tiny_s = seg_bytes < 4;
    auto gword = [&](long e) { return min((unsigned)(e * gs) & ~3u, gate_bytes - 4u); };
    auto sword = [&](long sb) { return min((unsigned)sb & ~3u, seg_bytes - 4u); };
    const __amdgpu_buffer_rsrc_t rq = rsrc(p.q, row_bytes), rk = rsrc(p.k, row_bytes), rv = rsrc(p.v, row_bytes);
    const __amdgpu_buffer_rsrc_t rl = rsrc(p.lam, gate_bytes), rb = rsrc(p.beta, gate_bytes);
    const __amdgpu_buffer_rsrc_t rs = rsrc(p.seg, seg_bytes);
    // this lane's share of the copies: row piece rp of memory rm at token offset rt of
    // each copy, gate word of memory gm at token offset gt
    const int rp = lane % NP, rt = lane / (NP * MPW);
    int rbm, rhm, gbm, ghm;
    memory(m0 + (lane / NP) % MPW, rbm, rhm);
    memory(m0 + lane % MPW, gbm, ghm);
    const int gt = lane / MPW;

    auto copy = [&](long t0, St &st) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < TB / TPI; ++u) {
            const long t = t0 + u * TPI + rt;  // rows past T read 0 (range check)
            const unsigned off = (unsigned)((((long)rbm * T + t) * p.H + rhm) * R * es) + 16u * rp;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_ptr_t)&st.rows[0][u * 64], 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)&st.rows[1][u * 64], 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)&st.rows[2][u * 64], 16, off, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < TB / GPI; ++u) {
            const long t = min(t0 + u * GPI + gt, T - 1);
            if (!tiny_g) {
                const unsigned e = gword(((long)gbm * T + t) * p.H + ghm);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_ptr_t)&st.lam[u * 64], 4, e, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)&st.beta[u * 64], 4, e, 0, 0, 0);
            }
            if (SEG && !tiny_s)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)&st.seg[u * 64], 4, sword((long)gbm * T + t), 0, 0, 0);
        }
    };

    float M[C];
    {
        const float *src = p.M + (((long)b * p.H + h) * R + a) * R + c0;
#pragma unroll
        for (int c = 0; c < C; ++c) M[c] = src[c];
    }
    float ks[C];
#pragma unroll
    for (int c = 0; c < C; ++c) ks[c] = 0.f;
    float vs = 0.f;
    int n = 0;

    copy(0, stage[wv][0]);
    for (long t0 = 0, blk = 0; t0 < T; t0 += TB, ++blk) {
        St &cur = stage[wv][blk & 1];
        // this block's copies have landed and the last block's LDS reads are done (the
        // wave's own copies: no workgroup barrier); the asm is also a compiler memory
        // barrier, so no LDS access moves across it
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        if (t0 + TB < T) copy(t0 + TB, stage[wv][(blk + 1) & 1]);
        const int nt = (int)min((long)TB, T - t0);
        for (int tl = 0; tl < nt; ++tl) {
            const long t = t0 + tl;
            const int ix = tl * MPW + ml;
            // this lane's C columns of the q and k rows, read at a lane-dependent LDS
            // address (no run-time index into registers)
            float qf[C], kf[C];
            {
                constexpr int NW = C * es / 4;  // 4-byte words of the lane's columns
                const uint32_t *qw = reinterpret_cast<const uint32_t *>(&cur.rows[0][ix * NP]) + c0 * es / 4;
                const uint32_t *kw = reinterpret_cast<const uint32_t *>(&cur.rows[1][ix * NP]) + c0 * es / 4;
                uint32_t wq[NW], wk[NW];
#pragma unroll
                for (int i = 0; i < NW; ++i) {
                    wq[i] = qw[i];
                    wk[i] = kw[i];
                }
#pragma unroll
                for (int i = 0; i < NW; ++i) {
                    if (IOB) {
                        qf[2 * i] = __uint_as_float(wq[i] << 16);
                        qf[2 * i + 1] = __uint_as_float(wq[i] & 0xffff0000u);
                        kf[2 * i] = __uint_as_float(wk[i] << 16);
                        kf[2 * i + 1] = __uint_as_float(wk[i] & 0xffff0000u);
                    } else {
                        qf[i] = __uint_as_float(wq[i]);
                        kf[i] = __uint_as_float(wk[i]);
                    }
                }
            }
            const char *vrow = reinterpret_cast<const char *>(&cur.rows[2][ix * NP]);
            const float vf = IOB ? __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(vrow + 2 * a) << 16)
                                 : *reinterpret_cast<const float *>(vrow + 4 * a);
            const long e = ((long)b * T + t) * p.H + h;
            float lam, beta;
            if (tiny_g) {  // uniform
                lam = GB ? __uint_as_float((uint32_t) static_cast<const uint16_t *>(p.lam)[e] << 16) : static_cast<const float *>(p.lam)[e];
                beta = GB ? __uint_as_float((uint32_t) static_cast<const uint16_t *>(p.beta)[e] << 16) : static_cast<const float *>(p.beta)[e];
            } else {
                const uint32_t lw = cur.lam[ix], bw = cur.beta[ix];
                const unsigned sh = GB ? 8u * ((unsigned)(e * gs) - gword(e)) : 0u;  // 0 or 16
                lam = GB ? __uint_as_float(((lw >> sh) & 0xffffu) << 16) : __uint_as_float(lw);
                beta = GB ? __uint_as_float(((bw >> sh) & 0xffffu) << 16) : __uint_as_float(bw);
            }
            // read from the memory before this token's segment is written (two partial
            // sums for a shorter dependency chain)
            float r0 = 0.f, r1 = 0.f;
#pragma unroll
            for (int c = 0; c < C; c += 2) {
                r0 = fmaf(M[c], qf[c], r0);
                r1 = fmaf(M[c + 1], qf[c + 1], r1);
            }
            float rd = r0 + r1;
            if (L == 2) rd = add_xor1(rd);
#pragma unroll
            for (int s = R * L; s < R * L * J; s <<= 1) rd += __shfl_xor(rd, s);
            if (valid && j == 0 && half == 0) {
                const long o = (((long)b * T + t) * G + g) * R + a;
                if (IOB)
                    static_cast<uint16_t *>(p.out)[o] = (uint16_t)(pk_bf16(rd, 0.f) & 0xffffu);  // RNE
                else
                    static_cast<float *>(p.out)[o] = rd;
            }
            // the write, taken where the segment closes
            float kbar[C], vbar;
            bool closes;
            if (SEG) {
#pragma unroll
                for (int c = 0; c < C; ++c) ks[c] += kf[c];
                vs += vf;
                n += 1;
                const long sbyte = (long)b * T + t;
                const unsigned mark = tiny_s ? (unsigned)p.seg[sbyte]
                                             : (cur.seg[ix] >> (8u * ((unsigned)sbyte - sword(sbyte)))) & 0xffu;
                closes = mark != 0 || t == T - 1;
                const float inv = 1.0f / (float)n;  // exactly 1 for a one-token segment
#pragma unroll
                for (int c = 0; c < C; ++c) kbar[c] = ks[c] * inv;
                vbar = vs * inv;
            } else {
                closes = true;
#pragma unroll
                for (int c = 0; c < C; ++c) kbar[c] = kf[c];
                vbar = vf;
            }
            float p0 = 0.f, p1 = 0.f;
#pragma unroll
            for (int c = 0; c < C; c += 2) {
                p0 = fmaf(M[c], kbar[c], p0);
                p1 = fmaf(M[c + 1], kbar[c + 1], p1);
            }
            float pred = p0 + p1;
            if (L == 2) pred = add_xor1(pred);
            const float coef = beta * (vbar - pred);
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const float upd = fmaf(coef, kbar[c], lam * M[c]);
                M[c] = closes ? upd : M[c];
            }
            if (SEG) {
#pragma unroll
                for (int c = 0; c < C; ++c) ks[c] = closes ? 0.f : ks[c];
                vs = closes ? 0.f : vs;
                n = closes ? 0 : n;
            }
        }
    }
    if (valid) {
        float *dst = p.M + (m * R + a) * R + c0;
#pragma unroll
        for (int c = 0; c < C; ++c) dst[c] = M[c];
    }
}

// two lanes per row where a group's sub-states still fit in one wave
template <int R, bool IOB, bool GB, bool SEG>
const void *pick_j(int J) {
    switch (J) {
    case 1: return reinterpret_cast<const void *>(&dmem_fwd_kernel<R, 2, IOB, GB, SEG, 1>);
    case 2: return reinterpret_cast<const void *>(&dmem_fwd_kernel<R, (R * 4 <= 64 ? 2 : 1), IOB, GB, SEG, 2>);
    case 4: return reinterpret_cast<const void *>(&dmem_fwd_kernel<R, (R * 8 <= 64 ? 2 : 1), IOB, GB, SEG, 4>);
    case 8:
        if constexpr (64 / R >= 8) return reinterpret_cast<const void *>(&dmem_fwd_kernel<R, 1, IOB, GB, SEG, 8>);
        return nullptr;
    default: return nullptr;
    }
}

// lanes per row of the kernel pick_j chooses
int lanes_per_row(int R, int J) { return (J == 1 || R * 2 * J <= 64) ? 2 : 1; }

template <int R>
const void *pick(const DmemParams &p) {
    const bool seg = p.seg != nullptr;
    if (p.io_bf16) {
        if (p.gate_bf16) return seg ? pick_j<R, true, true, true>(p.J) : pick_j<R, true, true, false>(p.J);
        return seg ? pick_j<R, true, false, true>(p.J) : pick_j<R, true, false, false>(p.J);
    }
    if (p.gate_bf16) return seg ? pick_j<R, false, true, true>(p.J) : pick_j<R, false, true, false>(p.J);
    return seg ? pick_j<R, false, false, true>(p.J) : pick_j<R, false, false, false>(p.J);
}

}  // namespace

hipError_t launch_dmem(const DmemParams &p, hipStream_t s) {
    const long nmem = (long)p.B * p.H;
    if (nmem == 0 || p.T == 0) return hipSuccess;
    const void *fn = p.R == 8 ? pick<8>(p) : (p.R == 16 ? pick<16>(p) : nullptr);
    if (!fn) return hipErrorInvalidValue;
    const int mpw = 64 / (p.R * lanes_per_row(p.R, p.J));
    const long waves = (nmem + mpw - 1) / mpw;
    const long blocks = (waves + kWaves - 1) / kWaves;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    DmemParams q = p;
    void *args[] = {&q};
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(64 * kWaves), args, 0, s);
}

}  // namespace gdr
