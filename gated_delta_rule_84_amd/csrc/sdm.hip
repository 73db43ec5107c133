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
//   sdm_table_kernel   one workgroup per (batch, head, 32 columns), tokens in order: the
//                      W rows are gathered, updated and scattered, the R rows gathered
//                      and summed; the next token's rows are gathered while this one is
//                      processed, with rows written in between forwarded from LDS.
//                      HBM bound: (2 W + R) x dv x 4 bytes per token.
#include <math.h>
#include <stdint.h>

#include <mutex>

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
    int32_t *widx, *ridx;       // [B, T, H, Wp], [B, T, H, Rp]: padded to a multiple of 4
    float *wwt, *rwt;
    int Wp, Rp;
    int32_t *uw, *ur;           // caller's slot outputs [B, T, H, W] / [B, T, H, R] or null
    int t0, t1;                 // the launch covers tokens t0 .. t1 - 1 of every (batch, head)
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

__device__ __forceinline__ float wave_fsum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
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
__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }
// number of set bits of m below this lane
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Largest key t with at least k of the keys q at or above it (lo / hi: the smallest and
// largest valid key; invalid entries hold 0, below every valid key).  Counts by ballot.
template <int NQ>
__device__ __forceinline__ uint32_t kth_key(const uint32_t (&q)[NQ], uint32_t lo, uint32_t hi, int k) {
    while (lo < hi) {
        const uint32_t mid = lo + (uint32_t)(((uint64_t)(hi - lo) + 1u) >> 1);
        int c = 0;
#pragma unroll
        for (int u = 0; u < NQ; ++u) c += popc(__ballot(q[u] >= mid));
        if (c >= k) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Sort key of a scored slot: higher score first, then lower slot (unique per slot).
__device__ __forceinline__ uint64_t skey(uint32_t score_key, int slot) {
    return ((uint64_t)score_key << 32) | (uint32_t)~(uint32_t)slot;
}
__device__ __forceinline__ int skey_slot(uint64_t k) { return (int)~(uint32_t)k; }
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t x, int m) {
    const int lo = __shfl_xor((int)(uint32_t)x, m), hi = __shfl_xor((int)(uint32_t)(x >> 32), m);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
// Bitonic sort, descending, of the 128 keys held as element 2 lane + i in k_i.
__device__ __forceinline__ void bitonic128(uint64_t &k0, uint64_t &k1, int lane) {
#pragma unroll
    for (int size = 2; size <= 128; size <<= 1) {
        const bool up = ((2 * lane) & size) != 0;        // this block sorts ascending
#pragma unroll
        for (int d = size >> 1; d >= 1; d >>= 1) {
            if (d == 1) {
                const uint64_t mx = max(k0, k1), mn = min(k0, k1);
                k0 = up ? mn : mx;
                k1 = up ? mx : mn;
            } else {
                const int ld = d >> 1;
                const uint64_t p0 = shfl_xor64(k0, ld), p1 = shfl_xor64(k1, ld);
                const bool keep_max = ((lane & ld) == 0) != up;
                k0 = keep_max ? max(k0, p0) : min(k0, p0);
                k1 = keep_max ? max(k1, p1) : min(k1, p1);
            }
        }
    }
}

struct SelWave {
    uint64_t kk[kSdmMaxK];      // winners' sort keys, staged for the sort
    float hv[2][kSdmMaxK];      // each half's top-k values, best first
    int hi[2][kSdmMaxK];        // and their positions in the half
    uint32_t ck[kCandMax];      // candidate pair keys
    uint16_t cij[kCandMax];     // and their (row, column) in the two top-k lists
};

// the k staged keys w.kk[0..k) sorted best first into (k0, k1) of element 2 lane + i
__device__ __forceinline__ void sort_staged(SelWave &w, int k, int lane, uint64_t &k0, uint64_t &k1) {
    wsync();
    k0 = 2 * lane < k ? w.kk[2 * lane] : 0ull;
    k1 = 2 * lane + 1 < k ? w.kk[2 * lane + 1] : 0ull;
    bitonic128(k0, k1, lane);
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
        const uint64_t mgt = __ballot(q[u] > th);
        const int pos = ngt + lanes_below(mgt);
        if (q[u] > th && pos < k) w.kk[pos] = skey(q[u], 64 * u + lane);
        ngt += popc(mgt);
        cge += popc(__ballot(q[u] >= th));
        below = q[u] < th ? max(below, q[u]) : below;
    }
    ngt = min(ngt, k);
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        if (ngt < k) {
            const uint64_t meq = __ballot(q[u] == th);
            const int pos = ngt + lanes_below(meq);
            if (q[u] == th && pos < k) w.kk[pos] = skey(q[u], 64 * u + lane);
            ngt = min(ngt + popc(meq), k);
        }
    }
    uint64_t k0, k1;
    sort_staged(w, k, lane, k0, k1);
    if (2 * lane < k) {
        w.hv[h][2 * lane] = key_val((uint32_t)(k0 >> 32));
        w.hi[h][2 * lane] = skey_slot(k0);
    }
    if (2 * lane + 1 < k) {
        w.hv[h][2 * lane + 1] = key_val((uint32_t)(k1 >> 32));
        w.hi[h][2 * lane + 1] = skey_slot(k1);
    }
    return cge > k ? th : wave_umax(below);
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
// held in registers.  Pairs above it are all candidates; pairs equal to it are taken by
// lower slot, from the full rows of the grid -- or from every slot of the table when a
// pair outside the two top-k lists can reach it (rounding of the fp32 sums, or ties at a
// half's boundary).
template <int NP>
__global__ void __launch_bounds__(64 * kSelWaves) sdm_select_kernel(SdmParams p) {
    __shared__ SelWave sel[kSelWaves];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long item = (long)blockIdx.x * kSelWaves + wv;        // (token-head) * 2 + which
    const int len = p.t1 - p.t0;
    if (item >= 2L * p.B * len * p.H) return;
    const long il = item >> 1, bt = il / p.H;                    // (batch, token in range), head
    const long tk = ((bt / len) * p.T + p.t0 + bt % len) * p.H + il % p.H;
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
        const float ai = w.hv[0][i];
        for (int j = lane; j < L; j += 64) {
            w.ck[off + j] = okey(ai + w.hv[1][j]);
            w.cij[off + j] = (uint16_t)((i << 7) | j);
        }
        off += L;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = r0 + 64 * u + lane;
        const int L = i < kh ? min(kh, k / (i + 1)) : 0;
        int incl = L;                                            // inclusive scan of L over the lanes
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        const int o0 = off + incl - L;
        for (int j = 0; j < L; ++j) {
            w.ck[o0 + j] = okey(w.hv[0][i] + w.hv[1][j]);
            w.cij[o0 + j] = (uint16_t)((i << 7) | j);
        }
        off += __shfl(incl, 63);
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
        const uint64_t mgt = __ballot(cq[u] > th);
        const int pos = ngt + lanes_below(mgt);
        if (cq[u] > th && pos < k) {
            const int ij = w.cij[64 * u + lane], i = ij >> 7, j = ij & 127;
            w.kk[pos] = skey(cq[u], w.hi[0][i] * n + w.hi[1][j]);
        }
        ngt += popc(mgt);
    }
    ngt = min(ngt, k);
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
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) best = min(best, __shfl_xor(best, o));
            if (best == 0x7fffffff) best = 0;   // unreachable (the grid holds enough ties); keeps a valid slot
            if (lane == 0) w.kk[ngt] = skey(th, best);
            last = best;
            ++ngt;
        }
    } else {
        // ties at the k-th key over the whole table, in slot order
        for (int a = 0; a < n && ngt < k; ++a) {
            const float sa = clean(src[a]);
#pragma unroll
            for (int u = 0; u < NP; ++u) {
                if (ngt < k) {
                    const int b2 = 64 * u + lane;
                    const bool eq = b2 < n && okey(sa + x1[u]) == th;
                    const uint64_t meq = __ballot(eq);
                    const int pos = ngt + lanes_below(meq);
                    if (eq && pos < k) w.kk[pos] = skey(th, a * n + b2);
                    ngt = min(ngt + popc(meq), k);
                }
            }
        }
    }
    uint64_t k0, k1;
    sort_staged(w, k, lane, k0, k1);
    // softmax weights of the sorted winners (element 2 lane + i)
    const float v0 = key_val((uint32_t)(k0 >> 32)), v1 = key_val((uint32_t)(k1 >> 32));
    const float mx = __shfl(v0, 0);
    const float e0 = 2 * lane < k ? expf(v0 - mx) : 0.f, e1 = 2 * lane + 1 < k ? expf(v1 - mx) : 0.f;
    const float inv = 1.f / wave_fsum(e0 + e1);
    const int kp = which ? p.Rp : p.Wp;
    int32_t *oi = (which ? p.ridx : p.widx) + tk * kp;
    float *ow = (which ? p.rwt : p.wwt) + tk * kp;
    int32_t *ou = which ? p.ur : p.uw;
    const int best = __shfl(skey_slot(k0), 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {                // padding: a valid slot and weight 0
        const int e = 2 * lane + i;
        const int sl = i ? skey_slot(k1) : skey_slot(k0);
        if (e < kp) {
            oi[e] = e < k ? sl : best;
            ow[e] = e < k ? (i ? e1 : e0) * inv : 0.f;
            if (ou && e < k) ou[tk * k + e] = sl;
        }
    }
}

constexpr int kSdmCols = 32;                 // columns per workgroup
constexpr int kSdmGroups = kSdmDv / kSdmCols;
constexpr int kSdmHash = 512;                // >= 4 x the written rows per token
constexpr int kSdmFilterWords = 2048;        // 65,536-bit filter in front of the hash

__device__ __forceinline__ uint32_t sdm_mix(int slot) { return (uint32_t)slot * 0x9E3779B1u; }

__device__ __forceinline__ void lds_barrier() {  // LDS traffic waited for; global memory not
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// vmcnt(0) (loads and stores), as the builtin so that the compiler's own wait
// placement knows every earlier load has landed
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The rows one token wrote, findable by slot: a filter bit per slot hash (a clear bit
// means "not written", the common case: one LDS read), then an exact open-addressing
// hash of slot -> row.
struct SdmTable {
    uint32_t filt[kSdmFilterWords];
    int key[kSdmHash];
    int row[kSdmHash];
};

// row of each of the 4 slots in the token's write list, or -1
__device__ __forceinline__ void sdm_find4(const SdmTable &tb, const int (&slot)[4], int (&res)[4]) {
    uint32_t f[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = tb.filt[sdm_mix(slot[j]) >> 21];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        res[j] = -1;
        const uint32_t m = sdm_mix(slot[j]);
        if ((f[j] >> ((m >> 16) & 31)) & 1u) {
            int h = (int)(m >> 23);
#pragma unroll 1
            for (int i = 0; i < kSdmHash; ++i) {
                const int e = tb.key[h];
                if (e == slot[j]) {
                    res[j] = tb.row[h];
                    break;
                }
                if (e < 0) break;
                h = (h + 1) & (kSdmHash - 1);
            }
        }
    }
}
// returns the hash entry used (kept by the caller to clear it)
__device__ __forceinline__ int sdm_insert(SdmTable &tb, int slot, int r) {
    const uint32_t m = sdm_mix(slot);
    atomicOr(&tb.filt[m >> 21], 1u << ((m >> 16) & 31));
    int h = (int)(m >> 23);
#pragma unroll 1
    for (int i = 0; i < kSdmHash; ++i) {
        if (atomicCAS(&tb.key[h], -1, slot) == -1) {
            tb.row[h] = r;
            return h;
        }
        h = (h + 1) & (kSdmHash - 1);
    }
    return -1;
}
__device__ __forceinline__ void sdm_erase(SdmTable &tb, int slot, int h) {
    const uint32_t m = sdm_mix(slot);
    atomicAnd(&tb.filt[m >> 21], ~(1u << ((m >> 16) & 31)));
    if (h >= 0) tb.key[h] = -1;
}

// ---------------------------------------------------------------------------
// table pass
// ---------------------------------------------------------------------------
// One workgroup per (batch, head, group of 32 columns): the update and the read-out of a
// column touch no other column, so the four column groups of a head run independently.
// Thread (rg = tid / 8, q = tid % 8) holds columns 4q..4q+3 of the group for rows
// 4 rg + j (j < 4) of the token's write list and of its read list.
//
// Tokens are software-pipelined one deep: the rows of token t + 1 are gathered while
// token t is processed, so they can miss token t's writes (still in flight).  Those are
// forwarded from LDS: token t's written rows are kept there with a table of their
// slots, and every gathered row of token t + 1 is looked up in it.  Stores of token t - 1
// are complete before token t + 1's gathers are issued (each wave waits for its own
// stores, then the workgroup barrier), so one token of forwarding suffices, and each
// token costs one memory round trip.  Reads of token t see token t's own writes the same
// way (lookup after the update).
template <int IO_BF, int GATE_BF>
__global__ void __launch_bounds__(256) sdm_table_kernel(SdmParams p) {
    __shared__ __attribute__((aligned(16))) float buf[2][kSdmMaxK][kSdmCols];
    __shared__ SdmTable tabs[2];
    __shared__ __attribute__((aligned(16))) float part[4][kSdmCols];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int q = tid & 7, rg = tid >> 3;
    const int bh = blockIdx.x / kSdmGroups, cg = blockIdx.x % kSdmGroups;
    const int b = bh / p.H, h = bh % p.H;
    const int cb = cg * kSdmCols + 4 * q;                       // this thread's first column
    const long N = (long)p.n * p.n;
    float *Mh = p.M + (long)bh * N * kSdmDv + cb;
    auto tok = [&](int t) -> long { return ((long)b * p.T + t) * p.H + h; };

    for (int i = tid; i < kSdmFilterWords; i += 256) {
        tabs[0].filt[i] = 0u;
        tabs[1].filt[i] = 0u;
    }
    for (int i = tid; i < kSdmHash; i += 256) {
        tabs[0].key[i] = -1;
        tabs[1].key[i] = -1;
    }

    // slots and weights of the 4 consecutive rows this thread holds (the lists are padded
    // to a multiple of 4 with a valid slot and weight 0; rows 4 rg >= W or R are clamped
    // to the first 4 and never used)
    int ws0[4], rs0[4], ws1[4], rs1[4];
    float ww0[4], rw0[4], ww1[4], rw1[4];
    const int wo = min(4 * rg, p.Wp - 4), ro = min(4 * rg, p.Rp - 4);
    auto load_slots = [&](int t, int (&ws)[4], float (&ww)[4], int (&rs)[4], float (&rw)[4]) __attribute__((
                          always_inline)) {
        const long tk = tok(t);
        const u32x4 a = *reinterpret_cast<const u32x4 *>(p.widx + tk * p.Wp + wo);
        const f32x4 c = *reinterpret_cast<const f32x4 *>(p.wwt + tk * p.Wp + wo);
        const u32x4 d = *reinterpret_cast<const u32x4 *>(p.ridx + tk * p.Rp + ro);
        const f32x4 e = *reinterpret_cast<const f32x4 *>(p.rwt + tk * p.Rp + ro);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ws[j] = (int)a[j];
            ww[j] = c[j];
            rs[j] = (int)d[j];
            rw[j] = e[j];
        }
    };
    // v and the gates are kept as loaded (raw bits) and converted only after the wait at
    // the top of their token: converted at the load, they would make the compiler wait
    // for the whole gather in flight.
    struct Rows {
        f32x4 w[4], r[4], vf;
        u32x2 vb;
        uint32_t a, be;
    };
    auto gather = [&](int t, const int (&ws)[4], const int (&rs)[4], Rows &x) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x.w[j] = *reinterpret_cast<const f32x4 *>(Mh + (long)ws[j] * kSdmDv);
            x.r[j] = *reinterpret_cast<const f32x4 *>(Mh + (long)rs[j] * kSdmDv);
        }
        const long tk = tok(t);
        if (IO_BF) x.vb = *reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(p.v) + tk * kSdmDv + cb);
        else x.vf = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(p.v) + tk * kSdmDv + cb);
        if (GATE_BF) {
            x.a = static_cast<const uint16_t *>(p.alpha)[tk];
            x.be = static_cast<const uint16_t *>(p.beta)[tk];
        } else {
            x.a = static_cast<const uint32_t *>(p.alpha)[tk];
            x.be = static_cast<const uint32_t *>(p.beta)[tk];
        }
    };
    // the hash entry this thread filled for each table (thread q < 4 inserts row 4 rg + q)
    int ins_slot[2] = {0, 0}, ins_h[2] = {-2, -2};
    // One token.  (ws, ww, rs, rw) / x: its slots and rows; (wsn, rsn) / xn: the next
    // token's slots (loaded) and rows (gathered here).  All loads are unconditional (token
    // indices clamped) into registers whose last use is behind them.
    auto step = [&](int t, int (&ws)[4], float (&ww)[4], int (&rs)[4], float (&rw)[4], const int (&wsn)[4],
                    const int (&rsn)[4], Rows &x, Rows &xn, const int cur) __attribute__((always_inline)) {
        const int prv = cur ^ 1;
        wait_vmem();          // this token's rows, the next token's slots, own stores of t - 1
        lds_barrier();        // every wave's stores of t - 1 done; table `cur` is empty
        gather(min(t + 1, p.t1 - 1), wsn, rsn, xn);
        uint32_t vb0 = x.vb[0], vb1 = x.vb[1], ab = x.a, bb = x.be;
        asm volatile("" : "+v"(vb0), "+v"(vb1), "+v"(ab), "+v"(bb));
        const f32x4 vv = IO_BF ? f32x4{__uint_as_float(vb0 << 16), __uint_as_float(vb0 & 0xffff0000u),
                                       __uint_as_float(vb1 << 16), __uint_as_float(vb1 & 0xffff0000u)}
                               : x.vf;
        const float a = __uint_as_float(GATE_BF ? ab << 16 : ab), be = __uint_as_float(GATE_BF ? bb << 16 : bb);
        if (t > p.t0) {       // rows written by token t - 1 after their gather was issued
            int pw[4], pr[4];
            sdm_find4(tabs[prv], ws, pw);
            sdm_find4(tabs[prv], rs, pr);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (pw[j] >= 0) x.w[j] = *reinterpret_cast<const f32x4 *>(&buf[prv][pw[j]][4 * q]);
                if (pr[j] >= 0) x.r[j] = *reinterpret_cast<const f32x4 *>(&buf[prv][pr[j]][4 * q]);
            }
        }
        // the gated delta update of the written rows
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * rg + j;
            if (r < p.W) {
                const f32x4 m0 = x.w[j] * a;
                const f32x4 m = m0 + (be * ww[j]) * (vv - m0);
                *reinterpret_cast<f32x4 *>(Mh + (long)ws[j] * kSdmDv) = m;
                *reinterpret_cast<f32x4 *>(&buf[cur][r][4 * q]) = m;
            }
        }
        if (q < 4 && 4 * rg + q < p.W) {
            const int sl = q == 0 ? ws[0] : q == 1 ? ws[1] : q == 2 ? ws[2] : ws[3];
            ins_slot[cur] = sl;
            ins_h[cur] = sdm_insert(tabs[cur], sl, 4 * rg + q);
        }
        lds_barrier();        // token t's rows and table complete; token t - 1's no longer read
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            int pr[4];
            sdm_find4(tabs[cur], rs, pr);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (pr[j] >= 0) x.r[j] = *reinterpret_cast<const f32x4 *>(&buf[cur][pr[j]][4 * q]);
                if (4 * rg + j < p.R) acc += rw[j] * x.r[j];
            }
        }
        if (ins_h[prv] != -2) {   // empty token t - 1's table: it is token t + 1's
            sdm_erase(tabs[prv], ins_slot[prv], ins_h[prv]);
            ins_h[prv] = -2;
        }
        load_slots(min(t + 2, p.t1 - 1), ws, ww, rs, rw);
        // read-out: sum over the rows of the wave sharing q, then over the four waves
#pragma unroll
        for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], off);
        }
        if (lane < 8) *reinterpret_cast<f32x4 *>(&part[wv][4 * lane]) = acc;
        lds_barrier();
        if (tid < kSdmCols) {
            const float o = part[0][tid] + part[1][tid] + part[2][tid] + part[3][tid];
            st_elem(p.o, tok(t) * kSdmDv + cg * kSdmCols + tid, o, IO_BF);
        }
    };
    if (p.t1 <= p.t0) return;
    Rows x0, x1;
    load_slots(p.t0, ws0, ww0, rs0, rw0);
    gather(p.t0, ws0, rs0, x0);
    load_slots(min(p.t0 + 1, p.t1 - 1), ws1, ww1, rs1, rw1);
    for (int t = p.t0;; t += 2) {
        step(t, ws0, ww0, rs0, rw0, ws1, rs1, x0, x1, 0);
        if (t + 1 >= p.t1) break;
        step(t + 1, ws1, ww1, rs1, rw1, ws0, rs0, x1, x0, 1);
        if (t + 2 >= p.t1) break;
    }
}

}  // namespace

size_t sdm_workspace(int B, int T, int H, int W, int R) {
    const size_t wp = (size_t)((W + 3) & ~3), rp = (size_t)((R + 3) & ~3);
    return (size_t)B * T * H * (wp + rp) * (sizeof(int32_t) + sizeof(float));
}

// With a caller-owned execution context, the selection of a block of tokens runs on the
// context's second stream while the table pass works through the blocks before it on
// the caller's stream: the table pass holds one workgroup per CU and is latency bound,
// so the selection's blocks fill the rest of each CU.  The table pass of block j waits
// for the selection of block j only.
namespace {
constexpr int kSdmBlocks = 64;    // most token blocks of a call (blocks of >= 128 tokens)
static_assert(kSdmBlocks + 1 <= kCtxEvents, "events of one call");
}  // namespace

hipError_t launch_sdm(int B, int T, int H, int n, int W, int R, int io_bf16, int gate_bf16, const float *ks,
                      const float *qs, const void *v, const void *alpha, const void *beta, float *M, void *o,
                      int32_t *wslots, int32_t *rslots, void *ws, const gdr_context *ctx, hipStream_t st) {
    const long ntok = (long)B * T * H;
    if (ntok == 0) return hipSuccess;
    SdmParams p;
    p.B = B; p.T = T; p.H = H; p.n = n; p.W = W; p.R = R; p.io_bf16 = io_bf16; p.gate_bf16 = gate_bf16;
    p.ks = ks; p.qs = qs; p.v = v; p.alpha = alpha; p.beta = beta; p.M = M; p.o = o;
    p.Wp = (W + 3) & ~3;
    p.Rp = (R + 3) & ~3;
    int32_t *wi = static_cast<int32_t *>(ws);
    int32_t *ri = wi + ntok * p.Wp;
    float *ww = reinterpret_cast<float *>(ri + ntok * p.Rp);
    float *rw = ww + ntok * p.Wp;
    p.widx = wi;
    p.ridx = ri;
    p.wwt = ww;
    p.rwt = rw;
    p.uw = wslots;
    p.ur = rslots;
    const int np = (n + 63) / 64;
    const void *sel = np <= 1 ? reinterpret_cast<const void *>(&sdm_select_kernel<1>)
                      : np <= 2 ? reinterpret_cast<const void *>(&sdm_select_kernel<2>)
                      : np <= 4 ? reinterpret_cast<const void *>(&sdm_select_kernel<4>)
                      : np <= 8 ? reinterpret_cast<const void *>(&sdm_select_kernel<8>)
                                : reinterpret_cast<const void *>(&sdm_select_kernel<16>);
    const void *tab = io_bf16 ? (gate_bf16 ? reinterpret_cast<const void *>(&sdm_table_kernel<1, 1>)
                                           : reinterpret_cast<const void *>(&sdm_table_kernel<1, 0>))
                              : (gate_bf16 ? reinterpret_cast<const void *>(&sdm_table_kernel<0, 1>)
                                           : reinterpret_cast<const void *>(&sdm_table_kernel<0, 0>));
    auto launch = [&](const void *fn, int t0, int t1, hipStream_t s) -> hipError_t {
        SdmParams a = p;
        a.t0 = t0;
        a.t1 = t1;
        void *args[] = {&a};
        if (fn == tab) return hipLaunchKernel(fn, dim3((unsigned)(B * H * kSdmGroups)), dim3(256), args, 0, s);
        const long items = 2L * B * (t1 - t0) * H;
        return hipLaunchKernel(fn, dim3((unsigned)((items + kSelWaves - 1) / kSelWaves)), dim3(64 * kSelWaves), args,
                               0, s);
    };
    const int nblk = ctx && T >= 1024 ? min(kSdmBlocks, T / 128) : 1;
    if (nblk == 1) {
        const hipError_t e = launch(sel, 0, T, st);
        return e != hipSuccess ? e : launch(tab, 0, T, st);
    }
    hipError_t e;
    hipStream_t side = ctx->stream;
    const hipEvent_t fork = ctx->ev[0], *done = ctx->ev + 1;
    auto bound = [&](int j) { return (int)((long)T * j / nblk); };
    if ((e = hipEventRecord(fork, st)) != hipSuccess) return e;           // inputs ready on st
    if ((e = hipStreamWaitEvent(side, fork, 0)) != hipSuccess) return e;
    for (int j = 0; j < nblk; ++j) {
        if ((e = launch(sel, bound(j), bound(j + 1), side)) != hipSuccess) return e;
        if ((e = hipEventRecord(done[j], side)) != hipSuccess) return e;
    }
    for (int j = 0; j < nblk; ++j) {
        if ((e = hipStreamWaitEvent(st, done[j], 0)) != hipSuccess) return e;
        if ((e = launch(tab, bound(j), bound(j + 1), st)) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gdr
