// decode.hip -- one-token gated delta-rule step on a resident fp32 state (gfx950).
//
// Per (batch, head), with u, w, vh the erase key, write key and written value
// (scalar beta: u = k, w = beta k_w, vh = v; beta vectors: sqrt(beta^k) k,
// sqrt(beta^k) k_w, sqrt(beta^v) v):
//     p_u = S^T (alpha (.) u),  p_q = S^T (alpha (.) q)      column reductions
//     delta = vh - p_u                                       residual on the decayed state
//     o = p_q + delta (w . q)                                = S_new^T q
//     S_new = Diag(alpha) S + w delta^T                      written back in place
// This is one step of the gated delta rule [OSDN page, section 1; FG2-GDN page,
// sections 1 and 2.A] with the read-out taken after the write.  Two options give
// the delta-mem step [delta-mem page, section 2.A update rule, section 2.C read]:
// undecayed prediction (p_u = S^T u, the residual against the state before the
// gate) and read before write (o = S^T q, the state before the gate and write).
//
// The step is bound by HBM: the state is read once and written once (8 bytes
// per element) and every other operand is O(dk + dv).  Each thread owns float4
// column groups of R rows and keeps them in registers between the reduction
// and the write-back, so no byte of S is fetched twice.
#include "gdr_device.hpp"
#include "gdr_internal.hpp"

namespace gdr {
namespace {

constexpr int kDecodeThreads = 256;
typedef float nf4 __attribute__((ext_vector_type(4)));

// Square power-of-two states D x D, D in {8, 16, 32, 64, 128}.
//   NC  float4 column groups per row, RT row-threads per head, R rows per thread,
//   TG = NC * RT threads per head, G heads per 256-thread block.
template <int D>
__global__ void __launch_bounds__(kDecodeThreads) decode_sq_kernel(DecodeParams p) {
    constexpr int NC = D / 4;
    constexpr int RT = (D < kDecodeThreads / NC) ? D : kDecodeThreads / NC;
    constexpr int R = D / RT;
    constexpr int TG = NC * RT;
    constexpr int G = kDecodeThreads / TG;
    constexpr int NWG = TG > 64 ? TG / 64 : 1;  // waves per head
    static_assert(R * RT == D && TG * G == kDecodeThreads && TG >= D, "decode tiling");

    // per-head vectors: 0 alpha*u, 1 alpha*q, 2 w, 3 alpha, 4 vh, 5 q
    __shared__ float sv[G][6][D];
    __shared__ float sred[G][NWG][NC][9];

    const int tid = threadIdx.x;
    const int g = tid / TG, tg = tid - g * TG;
    const int cg = tg % NC, rt = tg / NC;
    const long nbh = (long)p.B * p.H;
    const long bh = (long)blockIdx.x * G + g;
    const bool act = bh < nbh;

    float4 s[R];
    float *Sh = p.S + (act ? bh : 0) * (long)D * D;
    if (act) {
#pragma unroll
        for (int m = 0; m < R; ++m)
            s[m] = *reinterpret_cast<const float4 *>(Sh + (long)(rt + m * RT) * D + cg * 4);
    }
    if (act && tg < D) {
        const long vi = bh * D + tg;
        const float kk = ld_elem(p.k, vi, p.io_bf16);
        const float kw = ld_elem(p.kw, vi, p.io_bf16);
        const float qq = ld_elem(p.q, vi, p.io_bf16);
        const float vv = ld_elem(p.v, vi, p.io_bf16);
        const float a = ld_elem(p.alpha, p.alpha_ch ? vi : bh, p.gate_bf16);
        float u, w, vh;
        if (p.beta_mode == 0) {
            u = kk;
            w = ld_elem(p.beta_k, bh, p.gate_bf16) * kw;
            vh = vv;
        } else {
            const float bk = ld_elem(p.beta_k, vi, p.gate_bf16);
            const float sb = sqrtf(bk);
            u = sb * kk;
            w = sb * kw;
            const float bv = p.beta_mode == 2 ? ld_elem(p.beta_v, vi, p.gate_bf16) : bk;
            vh = sqrtf(bv) * vv;
        }
        sv[g][0][tg] = p.undecayed_prediction ? u : a * u;
        sv[g][1][tg] = p.read_before_write ? qq : a * qq;
        sv[g][2][tg] = w;
        sv[g][3][tg] = a;
        sv[g][4][tg] = vh;
        sv[g][5][tg] = qq;
    }
    __syncthreads();

    float red[9];
#pragma unroll
    for (int c = 0; c < 9; ++c) red[c] = 0.f;
    if (act) {
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const int r = rt + m * RT;
            const float ua = sv[g][0][r], qa = sv[g][1][r];
            red[0] += s[m].x * ua; red[1] += s[m].y * ua; red[2] += s[m].z * ua; red[3] += s[m].w * ua;
            red[4] += s[m].x * qa; red[5] += s[m].y * qa; red[6] += s[m].z * qa; red[7] += s[m].w * qa;
            red[8] += sv[g][2][r] * sv[g][5][r];
        }
    }
    // reduce over the row-threads of this head that share the column group
    constexpr int kWaveSpan = TG < 64 ? TG : 64;
#pragma unroll
    for (int off = NC; off < kWaveSpan; off <<= 1) {
#pragma unroll
        for (int c = 0; c < 9; ++c) red[c] += __shfl_xor(red[c], off);
    }
    if constexpr (NWG > 1) {
        const int wv = tg / 64;          // wave inside the head group
        if ((tg % 64) < NC) {
#pragma unroll
            for (int c = 0; c < 9; ++c) sred[g][wv][cg][c] = red[c];
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 9; ++c) {
            float t = 0.f;
#pragma unroll
            for (int x = 0; x < NWG; ++x) t += sred[g][x][cg][c];
            red[c] = t;
        }
    }
    if (!act) return;

    float dl[4], o[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        dl[c] = sv[g][4][cg * 4 + c] - red[c];
        o[c] = p.read_before_write ? red[4 + c] : red[4 + c] + dl[c] * red[8];
    }
    if (rt == 0) {
        const long oi = bh * D + cg * 4;
        if (p.io_bf16) {
            uint2 pk;
            pk.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
            pk.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
            *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.o) + oi) = pk;
        } else {
            *reinterpret_cast<float4 *>(static_cast<float *>(p.o) + oi) = make_float4(o[0], o[1], o[2], o[3]);
        }
    }
#pragma unroll
    for (int m = 0; m < R; ++m) {
        const int r = rt + m * RT;
        const float a = sv[g][3][r], w = sv[g][2][r];
        float4 x = s[m];
        x.x = a * x.x + w * dl[0];
        x.y = a * x.y + w * dl[1];
        x.z = a * x.z + w * dl[2];
        x.w = a * x.w + w * dl[3];
        float *dst = Sh + (long)r * D + cg * 4;
        if constexpr (D >= 64) {
            // large states stream through HBM once per step: a non-temporal store
            // (measured ~20% faster at D = 128) keeps them from displacing anything
            __builtin_nontemporal_store(nf4{x.x, x.y, x.z, x.w}, reinterpret_cast<nf4 *>(dst));
        } else {
            *reinterpret_cast<float4 *>(dst) = x;  // small states stay cache resident
        }
    }
}

// Any dk, dv (multiples of 8, <= 128): one block of 128 threads per head,
// thread j owns value column j and walks the dk rows twice (the second pass
// re-reads the column from cache).
__global__ void __launch_bounds__(128) decode_generic_kernel(DecodeParams p) {
    __shared__ float ua[128], qa[128], ww[128], aa[128], vh[128], wred[2];
    const int dk = p.dk, dv = p.dv;
    const long bh = blockIdx.x;
    const int tid = threadIdx.x;
    float wq = 0.f;
    if (tid < dk) {
        const long vi = bh * dk + tid;
        const float kk = ld_elem(p.k, vi, p.io_bf16);
        const float kw = ld_elem(p.kw, vi, p.io_bf16);
        const float qq = ld_elem(p.q, vi, p.io_bf16);
        const float a = ld_elem(p.alpha, p.alpha_ch ? vi : bh, p.gate_bf16);
        float u, w;
        if (p.beta_mode == 0) {
            u = kk;
            w = ld_elem(p.beta_k, bh, p.gate_bf16) * kw;
        } else {
            const float sb = sqrtf(ld_elem(p.beta_k, vi, p.gate_bf16));
            u = sb * kk;
            w = sb * kw;
        }
        ua[tid] = p.undecayed_prediction ? u : a * u;
        qa[tid] = p.read_before_write ? qq : a * qq;
        ww[tid] = w;
        aa[tid] = a;
        wq = w * qq;
    }
    if (tid < dv) {
        const long vj = bh * dv + tid;
        const float vv = ld_elem(p.v, vj, p.io_bf16);
        float x = vv;
        if (p.beta_mode == 1) x = sqrtf(ld_elem(p.beta_k, bh * dk + tid, p.gate_bf16)) * vv;
        if (p.beta_mode == 2) x = sqrtf(ld_elem(p.beta_v, vj, p.gate_bf16)) * vv;
        vh[tid] = x;
    }
    for (int off = 32; off > 0; off >>= 1) wq += __shfl_xor(wq, off);
    if ((tid & 63) == 0) wred[tid >> 6] = wq;
    __syncthreads();
    wq = wred[0] + wred[1];
    if (tid >= dv) return;
    float *Sh = p.S + bh * (long)dk * dv;
    float pu = 0.f, pq = 0.f;
    for (int i = 0; i < dk; ++i) {
        const float s = Sh[(long)i * dv + tid];
        pu += s * ua[i];
        pq += s * qa[i];
    }
    const float dl = vh[tid] - pu;
    st_elem(p.o, bh * dv + tid, p.read_before_write ? pq : pq + dl * wq, p.io_bf16);
    for (int i = 0; i < dk; ++i) {
        const long e = (long)i * dv + tid;
        Sh[e] = aa[i] * Sh[e] + ww[i] * dl;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, hipStream_t st) {
    const long nbh = (long)p.B * p.H;
    if (nbh == 0) return hipSuccess;
    DecodeParams arg = p;
    void *args[] = {&arg};
    auto launch = [&](const void *fn, int heads_per_block, int threads) {
        const dim3 grid((unsigned)((nbh + heads_per_block - 1) / heads_per_block));
        return hipLaunchKernel(fn, grid, dim3(threads), args, 0, st);
    };
    if (p.dk == p.dv) {
        switch (p.dk) {
        case 128: return launch(reinterpret_cast<const void *>(&decode_sq_kernel<128>), 1, kDecodeThreads);
        case 64:  return launch(reinterpret_cast<const void *>(&decode_sq_kernel<64>), 1, kDecodeThreads);
        case 32:  return launch(reinterpret_cast<const void *>(&decode_sq_kernel<32>), 1, kDecodeThreads);
        case 16:  return launch(reinterpret_cast<const void *>(&decode_sq_kernel<16>), 4, kDecodeThreads);
        case 8:   return launch(reinterpret_cast<const void *>(&decode_sq_kernel<8>), 16, kDecodeThreads);
        default: break;
        }
    }
    return launch(reinterpret_cast<const void *>(&decode_generic_kernel), 1, 128);
}

}  // namespace gdr
