// chunk_valu.hip -- chunkwise WY / UT-transform prefill in fp32 on the vector ALU.
//
// The general kernel: any dk, dv (multiples of 8, <= 128), chunk 16/32/64, bf16 or
// fp32 inputs, every gate and beta layout.  It is the path for fp32 inputs and
// for shapes the matrix-core kernel does not take.
//
// For one chunk of n <= C tokens entering with state S (dk x dv), with
// per-token erase key u, write key w and value vh (scalar beta: u = k,
// w = beta k_w, vh = v; beta vectors: sqrt(beta^k) k, sqrt(beta^k) k_w,
// sqrt(beta^v) v) and d(s, t) the decay from token s to token t >= s inside the
// chunk (per key channel for channel gates), gamma_t = d(start, t):
//     A   = strictly-lower( sum_i u_ti w_si d_i(s, t) )   block Gram matrix
//     Tm  = (I + A)^{-1}                                 forward substitution
//     R   = vh - (gamma u) S                             residual before the chunk's writes
//     Dl  = Tm R                                         per-token residuals of the recurrence
//     P   = lower-incl-diag( sum_i q_ti w_si d_i(s, t) ) intra-chunk scores
//     O   = (gamma q) S + P Dl
//     S  <- Diag(gamma_end) S + (d(., end) w)^T Dl
// which is the recurrence of the pages rewritten per chunk: the WY factors
// are Tm (gamma u) and Tm vh [FG2-GDN page, sections 2.A and 3; OSDN page,
// section 2.1: the write key replaces the key in the Gram matrix and the
// intra-block scores].  Decays are kept segmented at zero gates (a hard reset):
// with P the cumulative log decay in which a zero gate adds 0, d(s, t) =
// [no zero gate in (s, t]] e^{P_t - P_s}.  Every factor is a decay over tokens in
// order, so none exceeds 1: any gate in [0, 1] is taken, however strong the decay.
//
// Mapping: one 256-thread block per (batch*head, block of kVB value columns),
// walking the chunks in order; all chunk operands live in LDS.  Columns of S
// evolve independently given the chunk's Gram inverse, so splitting dv across
// blocks needs no communication (the Gram work is repeated per block).
#include "gdr_device.hpp"
#include "gdr_internal.hpp"

namespace gdr {
namespace {

constexpr int kVB = 16;        // value columns per block
constexpr int kThreads = 256;

__host__ __device__ inline size_t valu_lds_floats(int dk, int C) {
    const int ldk = dk + 1, ldc = C + 1;
    // Ub, Wb, Pg | M | Sb | Rv, Dl | gt, fac, zt | gC | zero masks (two words per channel)
    return (size_t)3 * C * ldk + (size_t)C * ldc + (size_t)dk * kVB + 2 * (size_t)C * kVB + 3 * C + dk + 2 * dk;
}

template <bool CH>
__global__ void __launch_bounds__(kThreads) chunk_valu_kernel(ChunkParams p) {
    extern __shared__ float sm[];
    const int dk = p.dk, dv = p.dv, C = p.C, T = p.T, H = p.H;
    const int ldk = dk + 1, ldc = C + 1;
    float *Ub = sm;                    // [C][ldk] erase keys u, then gamma u; then queries q, then gamma q
    float *Wb = Ub + C * ldk;          // [C][ldk] write keys w, then d(., end) w
    float *Pg = Wb + C * ldk;          // [C][ldk] channel gates: cumulative log decay P
    float *M = Pg + C * ldk;           // [C][ldc] Gram -> inverse -> scores
    float *Sb = M + C * ldc;           // [dk][kVB] state columns of this block
    float *Rv = Sb + dk * kVB;         // [C][kVB] written values -> residuals R
    float *Dl = Rv + C * kVB;          // [C][kVB] residuals of the recurrence
    float *gt = Dl + C * kVB;          // [C] scalar gates: cumulative log decay P
    float *fac = gt + C;               // [C] scalar gates: d(s, end)
    int *zt = reinterpret_cast<int *>(fac + C);  // [C] scalar gates: last zero gate <= t (-1: none)
    float *gC = fac + 2 * C;           // [dk] gamma_end per channel (channel gates)
    uint32_t *zm = reinterpret_cast<uint32_t *>(gC + dk);  // [dk][2] channel gates: zero-gate bits

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H;
    const int j0 = blockIdx.y * kVB;
    const int nv = min(kVB, dv - j0);
    const long s_base = (long)bh * dk * dv;

    for (int e = tid; e < dk * kVB; e += kThreads) {
        const int i = e / kVB, j = e % kVB;
        Sb[e] = (p.S0 && j < nv) ? p.S0[s_base + (long)i * dv + j0 + j] : 0.f;
    }

    // decay of key channel i from token s to token t >= s
    auto dec_ch = [&](int i, int s, int t) -> float {
        const uint64_t bits = (uint64_t)zm[2 * i] | ((uint64_t)zm[2 * i + 1] << 32);
        const uint64_t upto = t >= 63 ? ~0ull : ((1ull << (t + 1)) - 1);
        const uint64_t from = s >= 63 ? 0ull : ~((2ull << s) - 1);  // tokens s + 1 ..
        if (s >= 0 && (bits & upto & from)) return 0.f;
        if (s < 0 && (bits & upto)) return 0.f;
        return expf(Pg[t * ldk + i] - (s >= 0 ? Pg[s * ldk + i] : 0.f));
    };
    auto dec_sc = [&](int s, int t) -> float {  // scalar gates, s = -1: from the chunk start
        if (zt[t] > s) return 0.f;
        return expf(gt[t] - (s >= 0 ? gt[s] : 0.f));
    };

    const int NT = (T + C - 1) / C;
    for (int c = 0; c < NT; ++c) {
        const int t0 = c * C;
        const int n = min(C, T - t0);
        auto tok = [&](int t) -> long { return ((long)b * T + t0 + t) * H + h; };

        // ---- cumulative log decay inside the chunk, segmented at zero gates ------
        if (!CH) {
            if (tid < 64) {
                float x = 0.f;
                int z = -1;
                if (tid < n) {
                    const float a = ld_elem(p.alpha, tok(tid), p.gate_bf16);
                    if (a == 0.f)
                        z = tid;
                    else
                        x = logf(a);
                }
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float y = __shfl_up(x, off);
                    const int zy = __shfl_up(z, off);
                    if (tid >= off) {
                        x += y;
                        z = max(z, zy);
                    }
                }
                if (tid < C) {
                    gt[tid] = x;
                    zt[tid] = z;
                }
            }
        } else {
            if (tid < dk) {
                float acc = 0.f;
                uint32_t z0 = 0, z1 = 0;
                for (int t = 0; t < n; ++t) {
                    const float a = ld_elem(p.alpha, tok(t) * dk + tid, p.gate_bf16);
                    if (a == 0.f) {
                        if (t < 32)
                            z0 |= 1u << t;
                        else
                            z1 |= 1u << (t - 32);
                    } else {
                        acc += logf(a);
                    }
                    Pg[t * ldk + tid] = acc;
                }
                zm[2 * tid] = z0;
                zm[2 * tid + 1] = z1;
            }
        }
        __syncthreads();
        if (!CH && tid < n) fac[tid] = dec_sc(tid, n - 1);
        if (CH && tid < dk) gC[tid] = dec_ch(tid, -1, n - 1);

        // ---- chunk operands: u, w (q comes once u is no longer needed) ------------
        for (int e = tid; e < n * dk; e += kThreads) {
            const int t = e / dk, i = e % dk;
            const long ti = tok(t) * dk + i;
            const float kk = ld_elem(p.k, ti, p.io_bf16);
            const float kw = ld_elem(p.kw, ti, p.io_bf16);
            float u, w;
            if (p.beta_mode == 0) {
                u = kk;
                w = ld_elem(p.beta_k, tok(t), p.gate_bf16) * kw;
            } else {
                const float sb = sqrtf(ld_elem(p.beta_k, ti, p.gate_bf16));
                u = sb * kk;
                w = sb * kw;
            }
            Ub[t * ldk + i] = u;
            Wb[t * ldk + i] = w;
        }
        for (int e = tid; e < n * kVB; e += kThreads) {
            const int t = e / kVB, j = e % kVB;
            float x = 0.f;
            if (j < nv) {
                const long tj = tok(t) * dv + j0 + j;
                x = ld_elem(p.v, tj, p.io_bf16);
                if (p.beta_mode == 1) x *= sqrtf(ld_elem(p.beta_k, tok(t) * dk + j0 + j, p.gate_bf16));
                if (p.beta_mode == 2) x *= sqrtf(ld_elem(p.beta_v, tj, p.gate_bf16));
            }
            Rv[e] = x;
        }
        __syncthreads();

        // ---- Gram matrix (strictly lower) -----------------------------------------
        for (int e = tid; e < n * n; e += kThreads) {
            const int t = e / n, s = e % n;
            float a = 0.f;
            if (s < t) {
                if (CH) {
                    for (int i = 0; i < dk; ++i) a += Ub[t * ldk + i] * Wb[s * ldk + i] * dec_ch(i, s, t);
                } else {
                    for (int i = 0; i < dk; ++i) a += Ub[t * ldk + i] * Wb[s * ldk + i];
                    a *= dec_sc(s, t);
                }
            }
            M[t * ldc + s] = a;
        }
        __syncthreads();

        // ---- (I + A)^{-1} by forward substitution, row by row, in place ----------
        for (int t = 1; t < n; ++t) {
            float val = 0.f;
            const int j = tid;
            if (j < t) {
                val = -M[t * ldc + j];
                for (int s = j + 1; s < t; ++s) val -= M[t * ldc + s] * M[s * ldc + j];
            }
            __syncthreads();
            if (j < t) M[t * ldc + j] = val;
            __syncthreads();
        }

        // ---- R = vh - (gamma u) S ---------------------------------------------------
        if (CH) {
            for (int e = tid; e < n * dk; e += kThreads) {
                const int t = e / dk, i = e % dk;
                Ub[t * ldk + i] *= dec_ch(i, -1, t);
            }
            __syncthreads();
        }
        for (int e = tid; e < n * kVB; e += kThreads) {
            const int t = e / kVB, j = e % kVB;
            float acc = 0.f;
            for (int i = 0; i < dk; ++i) acc += Ub[t * ldk + i] * Sb[i * kVB + j];
            if (!CH) acc *= dec_sc(-1, t);
            Rv[e] -= acc;
        }
        __syncthreads();

        // ---- Dl = Tm R (unit diagonal); queries into Ub ---------------------------
        for (int e = tid; e < n * kVB; e += kThreads) {
            const int t = e / kVB, j = e % kVB;
            float acc = Rv[e];
            for (int s = 0; s < t; ++s) acc += M[t * ldc + s] * Rv[s * kVB + j];
            Dl[e] = acc;
        }
        for (int e = tid; e < n * dk; e += kThreads) {
            const int t = e / dk, i = e % dk;
            Ub[t * ldk + i] = ld_elem(p.q, tok(t) * dk + i, p.io_bf16);
        }
        __syncthreads();

        // ---- intra-chunk scores (lower incl. diagonal) ----------------------------
        for (int e = tid; e < n * n; e += kThreads) {
            const int t = e / n, s = e % n;
            float a = 0.f;
            if (s <= t) {
                if (CH) {
                    for (int i = 0; i < dk; ++i) a += Ub[t * ldk + i] * Wb[s * ldk + i] * dec_ch(i, s, t);
                } else {
                    for (int i = 0; i < dk; ++i) a += Ub[t * ldk + i] * Wb[s * ldk + i];
                    a *= dec_sc(s, t);
                }
            }
            M[t * ldc + s] = a;
        }
        __syncthreads();

        // ---- O = (gamma q) S + P Dl -------------------------------------------------
        if (CH) {
            for (int e = tid; e < n * dk; e += kThreads) {
                const int t = e / dk, i = e % dk;
                Ub[t * ldk + i] *= dec_ch(i, -1, t);
                Wb[t * ldk + i] *= dec_ch(i, t, n - 1);  // for the state update below
            }
            __syncthreads();
        }
        for (int e = tid; e < n * kVB; e += kThreads) {
            const int t = e / kVB, j = e % kVB;
            if (j >= nv) continue;
            float acc = 0.f;
            for (int i = 0; i < dk; ++i) acc += Ub[t * ldk + i] * Sb[i * kVB + j];
            if (!CH) acc *= dec_sc(-1, t);
            for (int s = 0; s <= t; ++s) acc += M[t * ldc + s] * Dl[s * kVB + j];
            st_elem(p.o, tok(t) * dv + j0 + j, acc, p.io_bf16);
        }
        __syncthreads();

        // ---- state update ---------------------------------------------------------
        for (int e = tid; e < dk * kVB; e += kThreads) {
            const int i = e / kVB, j = e % kVB;
            float acc = 0.f;
            if (CH) {
                for (int s = 0; s < n; ++s) acc += Wb[s * ldk + i] * Dl[s * kVB + j];
                Sb[e] = gC[i] * Sb[e] + acc;
            } else {
                for (int s = 0; s < n; ++s) acc += fac[s] * Wb[s * ldk + i] * Dl[s * kVB + j];
                Sb[e] = dec_sc(-1, n - 1) * Sb[e] + acc;
            }
        }
        __syncthreads();
        if (ckpt_after(p, c)) {
            float *Ck = p.ckpt + ((long)bh * p.nck + (c + 1) / p.seg_chunks - 1) * dk * dv;
            for (int e = tid; e < dk * kVB; e += kThreads) {
                const int i = e / kVB, j = e % kVB;
                if (j < nv) Ck[(long)i * dv + j0 + j] = Sb[e];
            }
        }
    }

    if (p.ST) {
        for (int e = tid; e < dk * kVB; e += kThreads) {
            const int i = e / kVB, j = e % kVB;
            if (j < nv) p.ST[s_base + (long)i * dv + j0 + j] = Sb[e];
        }
    }
}

}  // namespace

hipError_t launch_chunk_valu(const ChunkParams &p, hipStream_t st) {
    const long nbh = (long)p.B * p.H;
    if (nbh == 0) return hipSuccess;
    const size_t lds = valu_lds_floats(p.dk, p.C) * sizeof(float);
    const dim3 grid((unsigned)nbh, (p.dv + kVB - 1) / kVB);
    const void *fn = p.alpha_ch ? reinterpret_cast<const void *>(&chunk_valu_kernel<true>)
                                : reinterpret_cast<const void *>(&chunk_valu_kernel<false>);
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    ChunkParams arg = p;
    void *args[] = {&arg};
    return hipLaunchKernel(fn, grid, dim3(kThreads), args, lds, st);
}

size_t chunk_valu_lds_bytes(int dk, int C) { return valu_lds_floats(dk, C) * sizeof(float); }

}  // namespace gdr
