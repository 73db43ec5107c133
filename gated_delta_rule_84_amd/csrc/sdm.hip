// sdm.hip -- Sparse Delta Memory: product-key slot selection and the table pass.
//
// Resumo Técnico: Sparse Delta Memory (SDM), Mecanismo Central items 1-4.  Per
// (batch, head) the memory is a table M of N = n * n slots x dv (fp32).  Per token the
// slot score of i = a * n + b is s1[a] + s2[b] (fp32) from the two half scores of
// the key (write) or of the query (read).  The W best slots by the key are written
//     M[i] <- alpha M[i] + beta w_i (v - alpha M[i])     (w = softmax of their scores)
// and the read-out is sum_r w'_r M[i_r] over the R best slots by the query (softmax
// weights), after the write.  Ranking: higher score first, equal scores by lower slot.
//
// Two launches:
//   sdm_select_kernel  one wave per (token, head, write | read): the top-k of each
//                      half by threshold bisection (order-preserving integer keys of
//                      the fp32 scores), then the k-th largest pair sum of the two
//                      top-k lists by bisection again (per-row counts by binary search:
//                      the pair sums are monotone along a sorted row), the winners
//                      gathered (boundary ties by lower slot), ranked and softmaxed.
//                      topk(s1 (+) s2) = topk(topk(s1) (+) topk(s2)) [same page, item 2].
//                      Selection does not depend on the table, so every token runs
//                      in parallel.
//   sdm_table_kernel   one workgroup per (batch, head), tokens in order: the W rows are
//                      gathered, updated and scattered; after a barrier the read rows of
//                      this token and the write rows of the next token are gathered
//                      together (both see this token's writes), so each token waits on
//                      one memory round trip.  HBM bound: 3 x k x dv x 4 bytes per token.
#include <math.h>
#include <stdint.h>

#include "gdr_device.hpp"
#include "gdr_internal.hpp"
#include "gdr_mfma.hpp"

namespace gdr {
namespace {

constexpr int kSdmMaxN = 1024;   // half-score length
constexpr int kSdmMaxK = 128;    // W, R
constexpr int kSdmDv = 128;
constexpr int kSelWaves = 4;
constexpr int kCandMax = 704;    // >= sum_{i=1..k} floor(k / i) = 645 for k = 128, rounded to 64
constexpr int kCandRegs = kCandMax / 64;
constexpr int kLongRows = 11;    // candidate rows spread over the lanes; later rows have <= k / 12 entries

struct SdmParams {
    int B, T, H, n, W, R, io_bf16, gate_bf16;
    const float *ks, *qs;       // [B, T, H, 2, n]
    const void *v, *alpha, *beta;
    float *M;                   // [B, H, n * n, dv]
    void *o;
    int32_t *widx, *ridx;       // [B, T, H, W], [B, T, H, R]
    float *wwt, *rwt;
};

// Order-preserving integer key of a (sanitised, non-NaN) float: unsigned order ==
// float order, -0 and +0 share a key.
__device__ __forceinline__ uint32_t okey(float x) {
    uint32_t u = __float_as_uint(x);
    u = (u == 0x80000000u) ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_val(uint32_t q) {
    return __uint_as_float((q & 0x80000000u) ? (q & 0x7fffffffu) : ~q);
}
// NaN -> the lowest finite score, +-inf -> +-FLT_MAX: sums of two scores are then never NaN
__device__ __forceinline__ float clean(float x) { return fminf(fmaxf(x, -3.402823466e38f), 3.402823466e38f); }

__device__ __forceinline__ void wsync() {  // order LDS traffic between the lanes of one wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}
__device__ __forceinline__ float wave_fsum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}
__device__ __forceinline__ int wave_imin(int x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = min(x, __shfl_xor(x, off));
    return x;
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, off));
    return x;
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, off));
    return x;
}
__device__ __forceinline__ int wave_excl_scan(int x, int lane) {  // exclusive prefix sum
    int incl = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    return incl - x;
}

// Largest key t with at least k of the keys q at or above it (lo / hi: the smallest and
// largest valid key; invalid entries hold 0, below every valid key).
template <int NQ>
__device__ __forceinline__ uint32_t kth_key(const uint32_t (&q)[NQ], uint32_t lo, uint32_t hi, int k) {
    while (lo < hi) {
        const uint32_t mid = lo + (uint32_t)(((uint64_t)(hi - lo) + 1u) >> 1);
        int c = 0;
#pragma unroll
        for (int u = 0; u < NQ; ++u) c += q[u] >= mid;
        if (wave_sum(c) >= k) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

struct SelWave {
    float hv[2][kSdmMaxK];      // each half's top-k values, best first
    int hi[2][kSdmMaxK];        // and their positions in the half
    uint32_t ck[kCandMax];      // candidate pair keys
    uint16_t cij[kCandMax];     // and their (row, column) in the two top-k lists
    float cv[kSdmMaxK];         // winners (unsorted), then sorted
    int cs[kSdmMaxK];
    float sv[kSdmMaxK];
    int ss[kSdmMaxK];
};

// Rank-sort the k entries (cv, cs) into (sv, ss): higher value first, lower slot on ties.
__device__ __forceinline__ void wave_rank_sort(SelWave &w, int k, int lane) {
    wsync();
    for (int e = lane; e < k; e += 64) {
        const float x = w.cv[e];
        const int sx = w.cs[e];
        int r = 0;
        for (int f = 0; f < k; ++f) {
            const float y = w.cv[f];
            r += (y > x) || (y == x && w.cs[f] < sx);
        }
        w.sv[r] = x;
        w.ss[r] = sx;
    }
    wsync();
}

// Top-k of one half (m values, x[u] holds position 64 u + lane), sorted into w.hv[h],
// w.hi[h] (equal values by lower position).  Returns the key of the best value left out
// (0 if none).
template <int NP>
__device__ uint32_t half_topk(SelWave &w, int h, const float (&x)[NP], int m, int k, int lane) {
    uint32_t q[NP];
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const bool ok = 64 * u + lane < m;
        q[u] = ok ? okey(x[u]) : 0u;
        lo = ok ? min(lo, q[u]) : lo;
        hi = max(hi, q[u]);
    }
    const uint32_t th = kth_key(q, wave_umin(lo), wave_umax(hi), k);
    int ngt = 0, cge = 0;
    uint32_t below = 0u;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const bool gt = q[u] > th;
        const int pos = ngt + wave_excl_scan(gt ? 1 : 0, lane);
        if (gt && pos < k) {
            w.cv[pos] = x[u];
            w.cs[pos] = 64 * u + lane;
        }
        ngt += wave_sum(gt ? 1 : 0);
        cge += q[u] >= th;
        below = q[u] < th ? max(below, q[u]) : below;
    }
    ngt = min(ngt, k);
    int need = k - ngt;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        if (need > 0) {
            const bool eq = q[u] == th;
            const int pos = wave_excl_scan(eq ? 1 : 0, lane);
            if (eq && pos < need) {
                w.cv[ngt + pos] = x[u];
                w.cs[ngt + pos] = 64 * u + lane;
            }
            const int take = min(wave_sum(eq ? 1 : 0), need);
            ngt += take;
            need -= take;
        }
    }
    wave_rank_sort(w, k, lane);
    for (int e = lane; e < k; e += 64) {
        w.hv[h][e] = w.sv[e];
        w.hi[h][e] = w.ss[e];
    }
    return wave_sum(cge) > k ? th : wave_umax(below);
}

// number of j < k with A[i] + B[j] at or above key th (a prefix: the row is nonincreasing)
__device__ __forceinline__ int row_count_ge(const SelWave &w, float ai, int k, uint32_t th) {
    int lo = 0, hi = k;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (okey(ai + w.hv[1][mid]) >= th) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// One wave per (token-head, write | read).  Each half keeps its kh = min(k, n) best.  The
// k best pair sums of the two sorted lists lie among the pairs (i, j) with
// (i + 1)(j + 1) <= k (a pair outside is dominated by more than k pairs that are at least
// as large), so the k-th largest key is found by bisection over those <= 645 candidates,
// held in registers.  Pairs above it are all
// candidates; pairs equal to it are taken by lower slot, from the full rows of the
// grid -- or from every slot of the table when a pair outside the two top-k lists can
// reach it (rounding of the fp32 sums, or ties at a half's boundary).
template <int NP>
__global__ void __launch_bounds__(64 * kSelWaves) sdm_select_kernel(SdmParams p) {
    __shared__ SelWave sel[kSelWaves];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long item = (long)blockIdx.x * kSelWaves + wv;        // (token-head) * 2 + which
    const long ntok = (long)p.B * p.T * p.H;
    if (item >= 2 * ntok) return;
    const long tk = item >> 1;
    const int which = (int)(item & 1);                           // 0 write (key), 1 read (query)
    const int k = which ? p.R : p.W, n = p.n;
    const int kh = min(k, n);                                    // length of each half's list
    SelWave &w = sel[wv];
    const float *src = (which ? p.qs : p.ks) + tk * 2 * n;
    float x0[NP], x1[NP];
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int a = min(64 * u + lane, n - 1);                 // clamped: every load in bounds
        x0[u] = clean(src[a]);
        x1[u] = clean(src[n + a]);
    }
    const uint32_t nx0 = half_topk(w, 0, x0, n, kh, lane);
    const uint32_t nx1 = half_topk(w, 1, x1, n, kh, lane);
    wsync();

    // candidates: rows i < kLongRows spread over the lanes column-wise, later rows one per lane
    const int r0 = min(kh, kLongRows);
    int off = 0;
    for (int i = 0; i < r0; ++i) {
        const int L = min(kh, k / (i + 1));
        for (int j = lane; j < L; j += 64) {
            w.ck[off + j] = okey(w.hv[0][i] + w.hv[1][j]);
            w.cij[off + j] = (uint16_t)((i << 7) | j);
        }
        off += L;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = r0 + 64 * u + lane;
        const int L = i < kh ? min(kh, k / (i + 1)) : 0;
        const int o = off + wave_excl_scan(L, lane);
        for (int j = 0; j < L; ++j) {
            w.ck[o + j] = okey(w.hv[0][i] + w.hv[1][j]);
            w.cij[o + j] = (uint16_t)((i << 7) | j);
        }
        off += wave_sum(L);
    }
    const int nc = off;
    wsync();
    uint32_t cq[kCandRegs];
    uint32_t cmin = 0xffffffffu;
#pragma unroll
    for (int u = 0; u < kCandRegs; ++u) {
        const bool ok = 64 * u + lane < nc;
        cq[u] = ok ? w.ck[64 * u + lane] : 0u;
        cmin = ok ? min(cmin, cq[u]) : cmin;
    }
    const uint32_t th = kth_key(cq, wave_umin(cmin), okey(w.hv[0][0] + w.hv[1][0]), k);

    // pairs strictly above the k-th key
    int ngt = 0;
#pragma unroll
    for (int u = 0; u < kCandRegs; ++u) {
        const bool gt = cq[u] > th;
        const int pos = ngt + wave_excl_scan(gt ? 1 : 0, lane);
        if (gt && pos < k) {
            const int ij = w.cij[64 * u + lane], i = ij >> 7, j = ij & 127;
            w.cv[pos] = w.hv[0][i] + w.hv[1][j];
            w.cs[pos] = w.hi[0][i] * n + w.hi[1][j];
        }
        ngt += wave_sum(gt ? 1 : 0);
    }
    ngt = min(ngt, k);
    const float tv = key_val(th);
    bool outside = false;
    if (kh < n) {
        if (nx0) outside |= okey(key_val(nx0) + w.hv[1][0]) >= th;
        if (nx1) outside |= okey(w.hv[0][0] + key_val(nx1)) >= th;
    }
    if (!outside) {
        // ties at the k-th key inside the grid, by lower slot, one at a time
        int last = -1;
        while (ngt < k) {
            int best = 0x7fffffff;
            for (int i = lane; i < kh; i += 64) {
                const float ai = w.hv[0][i];
                const int g1 = th == 0xffffffffu ? kh : row_count_ge(w, ai, kh, th + 1);
                const int g0 = row_count_ge(w, ai, kh, th);
                for (int j = g1; j < g0; ++j) {
                    const int sl = w.hi[0][i] * n + w.hi[1][j];
                    if (sl > last) best = min(best, sl);
                }
            }
            best = wave_imin(best);
            if (best == 0x7fffffff) best = 0;   // unreachable (the grid holds enough ties); keeps a valid slot
            if (lane == 0) {
                w.cs[ngt] = best;
                w.cv[ngt] = tv;
            }
            last = best;
            ++ngt;
        }
    } else {
        // ties at the k-th key over the whole table, in slot order
        int need = k - ngt;
        for (int a = 0; a < n && need > 0; ++a) {
            const float sa = clean(src[a]);
#pragma unroll
            for (int u = 0; u < NP; ++u) {
                if (need > 0) {
                    const int b = 64 * u + lane;
                    const bool eq = b < n && okey(sa + x1[u]) == th;
                    const int pos = wave_excl_scan(eq ? 1 : 0, lane);
                    if (eq && pos < need) {
                        w.cs[ngt + pos] = a * n + b;
                        w.cv[ngt + pos] = tv;
                    }
                    const int take = min(wave_sum(eq ? 1 : 0), need);
                    ngt += take;
                    need -= take;
                }
            }
        }
    }
    wave_rank_sort(w, k, lane);
    // softmax weights of the sorted winners
    const float mx = w.sv[0];
    float part = 0.f;
    for (int e = lane; e < k; e += 64) part += expf(w.sv[e] - mx);
    const float tot = wave_fsum(part);
    int32_t *oi = (which ? p.ridx : p.widx) + tk * k;
    float *ow = (which ? p.rwt : p.wwt) + tk * k;
    for (int e = lane; e < k; e += 64) {
        oi[e] = w.ss[e];
        ow[e] = expf(w.sv[e] - mx) / tot;
    }
}

// ---------------------------------------------------------------------------
// table pass
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) sdm_table_kernel(SdmParams p) {
    __shared__ float part[8][kSdmDv];
    __shared__ float vv[kSdmDv];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x, b = bh / p.H, h = bh % p.H;
    const long N = (long)p.n * p.n;
    float *Mh = p.M + (long)bh * N * kSdmDv;
    // write rows: thread -> (row tid / 2, 64 columns); read rows: thread -> (column
    // quad tid % 32, rows tid / 32 + 8 r)
    const int wrow = tid >> 1, wcol = 64 * (tid & 1);
    const int rq = tid & 31, rg = tid >> 5;
    auto tok = [&](int t) -> long { return ((long)b * p.T + t) * p.H + h; };
    f32x4 wreg[16];
    int wsl = 0;          // this thread's write slot of the current token
    float wc = 0.f;       // its weight
    auto gather_write = [&](int t) __attribute__((always_inline)) {
        if (wrow < p.W) {
            wsl = p.widx[tok(t) * p.W + wrow];
            wc = p.wwt[tok(t) * p.W + wrow];
            const float *src = Mh + (long)wsl * kSdmDv + wcol;
#pragma unroll
            for (int u = 0; u < 16; ++u) wreg[u] = *reinterpret_cast<const f32x4 *>(src + 4 * u);
        }
    };
    if (p.T > 0) gather_write(0);
    for (int t = 0; t < p.T; ++t) {
        const long tk = tok(t);
        // this token's read slots and weights, requested before the write
        int rsl[16];
        float rw[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int r = rg + 8 * u;
            rsl[u] = r < p.R ? p.ridx[tk * p.R + r] : 0;
            rw[u] = r < p.R ? p.rwt[tk * p.R + r] : 0.f;
        }
        const float a = ld_elem(p.alpha, tk, p.gate_bf16), be = ld_elem(p.beta, tk, p.gate_bf16);
        if (tid < kSdmDv) vv[tid] = ld_elem(p.v, tk * kSdmDv + tid, p.io_bf16);
        __syncthreads();  // v of this token; the previous token's read partials are consumed
        if (wrow < p.W) {
            const float c = be * wc;
            float *dst = Mh + (long)wsl * kSdmDv + wcol;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                f32x4 m = wreg[u] * a;
                const f32x4 vx = *reinterpret_cast<const f32x4 *>(&vv[wcol + 4 * u]);
                m = m + c * (vx - m);
                *reinterpret_cast<f32x4 *>(dst + 4 * u) = m;
            }
        }
        __syncthreads();  // this token's rows are written (and visible to the workgroup)
        // read rows of this token and write rows of the next one, requested together
        f32x4 rreg[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
            rreg[u] = *reinterpret_cast<const f32x4 *>(Mh + (long)rsl[u] * kSdmDv + 4 * rq);
        if (t + 1 < p.T) gather_write(t + 1);
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 16; ++u) acc += rw[u] * rreg[u];
        *reinterpret_cast<f32x4 *>(&part[rg][4 * rq]) = acc;
        __syncthreads();
        if (tid < kSdmDv) {
            float s = 0.f;
#pragma unroll
            for (int g = 0; g < 8; ++g) s += part[g][tid];
            st_elem(p.o, tk * kSdmDv + tid, s, p.io_bf16);
        }
    }
}

}  // namespace

size_t sdm_workspace(int B, int T, int H, int W, int R) {
    return (size_t)B * T * H * (size_t)(W + R) * (sizeof(int32_t) + sizeof(float));
}

hipError_t launch_sdm(int B, int T, int H, int n, int W, int R, int io_bf16, int gate_bf16, const float *ks,
                      const float *qs, const void *v, const void *alpha, const void *beta, float *M, void *o,
                      int32_t *wslots, int32_t *rslots, void *ws, hipStream_t st) {
    const long ntok = (long)B * T * H;
    if (ntok == 0) return hipSuccess;
    SdmParams p;
    p.B = B; p.T = T; p.H = H; p.n = n; p.W = W; p.R = R; p.io_bf16 = io_bf16; p.gate_bf16 = gate_bf16;
    p.ks = ks; p.qs = qs; p.v = v; p.alpha = alpha; p.beta = beta; p.M = M; p.o = o;
    char *w = static_cast<char *>(ws);
    int32_t *wi = reinterpret_cast<int32_t *>(w);
    int32_t *ri = wi + ntok * W;
    float *ww = reinterpret_cast<float *>(ri + ntok * R);
    float *rw = ww + ntok * W;
    p.widx = wslots ? wslots : wi;
    p.ridx = rslots ? rslots : ri;
    p.wwt = ww;
    p.rwt = rw;
    void *args[] = {&p};
    const long items = 2 * ntok;
    const int np = (n + 63) / 64;
    const void *sel = np <= 1 ? reinterpret_cast<const void *>(&sdm_select_kernel<1>)
                      : np <= 2 ? reinterpret_cast<const void *>(&sdm_select_kernel<2>)
                      : np <= 4 ? reinterpret_cast<const void *>(&sdm_select_kernel<4>)
                      : np <= 8 ? reinterpret_cast<const void *>(&sdm_select_kernel<8>)
                                : reinterpret_cast<const void *>(&sdm_select_kernel<16>);
    hipError_t e = hipLaunchKernel(sel,
                                   dim3((unsigned)((items + kSelWaves - 1) / kSelWaves)), dim3(64 * kSelWaves), args, 0,
                                   st);
    if (e != hipSuccess) return e;
    return hipLaunchKernel(reinterpret_cast<const void *>(&sdm_table_kernel), dim3((unsigned)(B * H)), dim3(256), args,
                           0, st);
}

}  // namespace gdr
