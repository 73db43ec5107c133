// gdr_ut.hpp -- the UT transform of a strictly lower 64 x 64 matrix on a 256-thread
// workgroup: Tm = (I + A)^{-1}, used by the chunk preparation of the prefill and by the
// chunk solve of the OSDN preconditioner scan.
#pragma once

#include "gdr_mfma.hpp"

namespace gdr {
namespace {

constexpr int kUtN = 64;

// Tm = (I + A)^{-1} for the strictly lower 64 x 64 A in As, into the lower part of
// Ts (fp32, row pitch LT; the unit diagonal and the upper part are not written).
// Ts may be As itself (LT = kUtN + 4): every 16 x 16 block of A is read before the
// block of Tm at the same place is written (the diagonal blocks by the wave that
// inverts them, after its loop; the off-diagonal ones after a barrier that follows
// their last read).  Ends with a barrier; starts reading As, so the caller has
// published it with a barrier.
template <int LT>
__device__ __forceinline__ void ut_transform(float (*As)[kUtN + 4], float (*Ts)[LT], float (*Xs)[16][16],
                                             const int w, const int l) {
    const int r = l & 15, q = l >> 4;
    // diagonal 16 x 16 blocks of (I + A)^{-1}: wave w, lane c < 16 owns column c;
    // row rr of the block is read as four 16-byte loads
    if (l < 16) {
        const int base = 16 * w, cc = l;
        float col[16];
        // row rr + 1 of the block is requested before row rr's dependent chain runs
        // (only its first rr + 1 entries are used: whole 16-byte pieces up to them)
        f32x4 nxt[4] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f},
                        f32x4{0.f, 0.f, 0.f, 0.f}};
        auto load_row = [&](int rr, f32x4 (&x)[4]) __attribute__((always_inline)) {
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4)
                if (4 * m4 < rr) x[m4] = *reinterpret_cast<const f32x4 *>(&As[base + rr][base + 4 * m4]);
        };
        load_row(0, nxt);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float a[16];
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) {
                a[4 * m4] = nxt[m4][0];
                a[4 * m4 + 1] = nxt[m4][1];
                a[4 * m4 + 2] = nxt[m4][2];
                a[4 * m4 + 3] = nxt[m4][3];
            }
            if (rr + 1 < 16) load_row(rr + 1, nxt);
            float v = rr == cc ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < rr; ++m) v -= a[m] * col[m];
            col[rr] = v;
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) Ts[base + rr][base + cc] = col[rr];
    }
    __syncthreads();
    // Off-diagonal 16 x 16 blocks on fp32 matrix cores (v_mfma_f32_16x16x4_f32; lane
    // (r, q) supplies A[r][k] and B[k][r] of k step s, C tiles as for bf16), by the
    // 2 x 2 block inverse [[T_a, 0], [L, T_b]]^-1 lower-left = -T_b L T_a, first on the
    // two 32 x 32 diagonal halves, then on the 64 x 64 matrix.
    {
        // C = M1 M2 for 16 x 16 blocks of LDS matrices (row pitch ld1, ld2)
        auto mm = [&](const float *M1, int ld1, const float *M2, int ld2, f32x4 acc) __attribute__((always_inline)) {
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(M1[r * ld1 + 4 * s4 + q], M2[(4 * s4 + q) * ld2 + r], acc, 0, 0, 0);
            return acc;
        };
        // C = M1 X with X a C tile held in registers: k step s4 takes row 4 q + s4 of X
        auto mmr = [&](const float *M1, int ld1, f32x4 X, f32x4 acc) __attribute__((always_inline)) {
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(M1[r * ld1 + 4 * q + s4], X[s4], acc, 0, 0, 0);
            return acc;
        };
        auto Ab = [&](int I, int J) { return &As[16 * I][16 * J]; };
        auto Tb = [&](int I, int J) { return &Ts[16 * I][16 * J]; };
        constexpr int LA = kUtN + 4;
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        auto storeT = [&](int I, int J, f32x4 v) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) Ts[16 * I + 4 * q + i][16 * J + r] = -v[i];
        };
        // level 1: T_10 (wave 0), T_32 (wave 1); waves 2, 3 start the 64 x 64 level
        f32x4 xa = z, xb = z;
        if (w < 2) {
            const int o = 2 * w;  // block offset of this 32 x 32 half
            const f32x4 x = mm(Ab(o + 1, o), LA, Tb(o, o), LT, z);
            storeT(o + 1, o, mmr(Tb(o + 1, o + 1), LT, x, z));
        } else {
            const int I = w;      // X_I0 (partial) and X_I1 = A_I1 T_11 for block row I = 2, 3
            xa = mm(Ab(I, 0), LA, Tb(0, 0), LT, z);
            xb = mm(Ab(I, 1), LA, Tb(1, 1), LT, z);
        }
        __syncthreads();
        if (w >= 2) {  // X_I0 += A_I1 T_10; publish X_I0, X_I1
            const int I = w;
            xa = mm(Ab(I, 1), LA, Tb(1, 0), LT, xa);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Xs[2 * (I - 2)][4 * q + i][r] = xa[i];
                Xs[2 * (I - 2) + 1][4 * q + i][r] = xb[i];
            }
        }
        __syncthreads();
        {   // T_IJ = -sum_{M=2}^{I} T_IM X_MJ for I = 2 + (w >> 1), J = w & 1
            const int I = 2 + (w >> 1), J = w & 1;
            f32x4 t = mm(Tb(I, 2), LT, &Xs[J][0][0], 16, z);
            if (I == 3) t = mm(Tb(3, 3), LT, &Xs[2 + J][0][0], 16, t);
            storeT(I, J, t);
        }
        __syncthreads();
    }

}

}  // namespace
}  // namespace gdr
