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
// group sit in adjacent lane groups and are summed by xor shuffles.  Tokens are walked
// in blocks of kTB: the next block's rows are loaded while the current block is
// processed.  A segment's write is computed for every token and selected where the
// segment closes (the memories of one wave close their segments at different tokens).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr_device.hpp"
#include "gdr_internal.hpp"

namespace gdr {
namespace {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

constexpr int kTB = 4;        // tokens per block
constexpr int kWaves = 4;     // waves per workgroup

// One token's inputs for one lane, as loaded (bf16 bit patterns or fp32 words).
template <int R, bool IOB>
struct Tok {
    static constexpr int kVec = R * (IOB ? 2 : 4) / 16;  // 16-byte pieces of a row
    u32x4v q[kVec], k[kVec];
    uint32_t v, lam, beta, se;
};

template <int R, bool IOB>
__device__ __forceinline__ void row_to_f32(const u32x4v (&w)[Tok<R, IOB>::kVec], float (&x)[R]) {
#pragma unroll
    for (int i = 0; i < Tok<R, IOB>::kVec; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (IOB) {
                x[8 * i + 2 * j] = __uint_as_float(w[i][j] << 16);
                x[8 * i + 2 * j + 1] = __uint_as_float(w[i][j] & 0xffff0000u);
            } else {
                x[4 * i + j] = __uint_as_float(w[i][j]);
            }
        }
    }
}

__device__ __forceinline__ float word_to_f32(uint32_t w, bool bf16) { return bf16 ? __uint_as_float(w << 16) : __uint_as_float(w); }

template <int R, bool IOB, bool GB, bool SEG, int J>
__global__ void __launch_bounds__(64 * kWaves) dmem_fwd_kernel(DmemParams p) {
    constexpr int MPW = 64 / R;  // memories per wave
    static_assert(MPW % J == 0, "a group's sub-states share a wave");
    const int lane = threadIdx.x & 63, a = lane % R;
    const long nmem = (long)p.B * p.H;
    const long m = ((long)blockIdx.x * kWaves + (threadIdx.x >> 6)) * MPW + lane / R;
    const bool valid = m < nmem;
    const long mm = valid ? m : nmem - 1;  // lanes past the end work on the last memory, store nothing
    const int b = (int)(mm / p.H), h = (int)(mm % p.H);
    const int G = p.H / J, g = h / J, j = h % J;
    const long T = p.T;

    const char *qb = static_cast<const char *>(p.q), *kb = static_cast<const char *>(p.k);
    constexpr int es = IOB ? 2 : 4;
    auto load = [&](long t, Tok<R, IOB> &x) __attribute__((always_inline)) {
        const long e = ((long)b * T + t) * p.H + h;  // token row index
        const u32x4v *qr = reinterpret_cast<const u32x4v *>(qb + e * R * es);
        const u32x4v *kr = reinterpret_cast<const u32x4v *>(kb + e * R * es);
#pragma unroll
        for (int i = 0; i < Tok<R, IOB>::kVec; ++i) {
            x.q[i] = qr[i];
            x.k[i] = kr[i];
        }
        x.v = IOB ? static_cast<const uint16_t *>(p.v)[e * R + a] : static_cast<const uint32_t *>(p.v)[e * R + a];
        x.lam = GB ? static_cast<const uint16_t *>(p.lam)[e] : static_cast<const uint32_t *>(p.lam)[e];
        x.beta = GB ? static_cast<const uint16_t *>(p.beta)[e] : static_cast<const uint32_t *>(p.beta)[e];
        x.se = SEG ? p.seg[(long)b * T + t] : 1u;
    };

    float M[R];
    {
        const float *src = p.M + (mm * R + a) * R;
#pragma unroll
        for (int c = 0; c < R; ++c) M[c] = src[c];
    }
    float ks[R];
#pragma unroll
    for (int c = 0; c < R; ++c) ks[c] = 0.f;
    float vs = 0.f;
    int n = 0;

    Tok<R, IOB> cur[kTB], nxt[kTB];
#pragma unroll
    for (int u = 0; u < kTB; ++u) load(min((long)u, T - 1), cur[u]);
    for (long t0 = 0; t0 < T; t0 += kTB) {
        if (t0 + kTB < T) {
#pragma unroll
            for (int u = 0; u < kTB; ++u) load(min(t0 + kTB + u, T - 1), nxt[u]);
        }
#pragma unroll
        for (int u = 0; u < kTB; ++u) {
            const long t = t0 + u;
            if (t < T) {  // uniform
                float qf[R], kf[R];
                row_to_f32<R, IOB>(cur[u].q, qf);
                row_to_f32<R, IOB>(cur[u].k, kf);
                const float vf = word_to_f32(cur[u].v, IOB);
                const float lam = word_to_f32(cur[u].lam, GB), beta = word_to_f32(cur[u].beta, GB);
                // read from the memory before this token's segment is written
                float rd = 0.f;
#pragma unroll
                for (int c = 0; c < R; ++c) rd = fmaf(M[c], qf[c], rd);
#pragma unroll
                for (int s = R; s < R * J; s <<= 1) rd += __shfl_xor(rd, s);
                if (valid && j == 0) {
                    const long o = (((long)b * T + t) * G + g) * R + a;
                    if (IOB)
                        static_cast<uint16_t *>(p.out)[o] = f32_to_bf16(rd);
                    else
                        static_cast<float *>(p.out)[o] = rd;
                }
                // the write, taken where the segment closes
                float kbar[R], vbar;
                bool closes;
                if (SEG) {
#pragma unroll
                    for (int c = 0; c < R; ++c) ks[c] += kf[c];
                    vs += vf;
                    n += 1;
                    closes = cur[u].se != 0 || t == T - 1;
                    const float fn = (float)n;
#pragma unroll
                    for (int c = 0; c < R; ++c) kbar[c] = ks[c] / fn;
                    vbar = vs / fn;
                } else {
                    closes = true;
#pragma unroll
                    for (int c = 0; c < R; ++c) kbar[c] = kf[c];
                    vbar = vf;
                }
                float pred = 0.f;
#pragma unroll
                for (int c = 0; c < R; ++c) pred = fmaf(M[c], kbar[c], pred);
                const float coef = beta * (vbar - pred);
#pragma unroll
                for (int c = 0; c < R; ++c) {
                    const float upd = fmaf(coef, kbar[c], lam * M[c]);
                    M[c] = closes ? upd : M[c];
                }
                if (SEG) {
#pragma unroll
                    for (int c = 0; c < R; ++c) ks[c] = closes ? 0.f : ks[c];
                    vs = closes ? 0.f : vs;
                    n = closes ? 0 : n;
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kTB; ++u) cur[u] = nxt[u];
    }
    if (valid) {
        float *dst = p.M + (m * R + a) * R;
#pragma unroll
        for (int c = 0; c < R; ++c) dst[c] = M[c];
    }
}

template <int R, bool IOB, bool GB, bool SEG>
const void *pick_j(int J) {
    switch (J) {
    case 1: return reinterpret_cast<const void *>(&dmem_fwd_kernel<R, IOB, GB, SEG, 1>);
    case 2: return reinterpret_cast<const void *>(&dmem_fwd_kernel<R, IOB, GB, SEG, 2>);
    case 4: return reinterpret_cast<const void *>(&dmem_fwd_kernel<R, IOB, GB, SEG, 4>);
    case 8:
        if constexpr (64 / R >= 8) return reinterpret_cast<const void *>(&dmem_fwd_kernel<R, IOB, GB, SEG, 8>);
        return nullptr;
    default: return nullptr;
    }
}

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
    const int mpw = 64 / p.R;
    const long waves = (nmem + mpw - 1) / mpw;
    const long blocks = (waves + kWaves - 1) / kWaves;
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    DmemParams q = p;
    void *args[] = {&q};
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(64 * kWaves), args, 0, s);
}

}  // namespace gdr
