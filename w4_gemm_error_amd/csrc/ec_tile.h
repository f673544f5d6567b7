// ec_tile.h -- internal to libw4ec: the gate / low-rank down-projection
// pass, [T | l] = X [A | w_g], as MFMA tiles (shared by the decode kernel's
// EC workgroups and the prefill prepass).
//
// A is row-major [K, r] (contiguous along the rank), but an MFMA operand
// wants 8 consecutive k per lane; so each 64-deep slice of [A | w_g] is
// staged transposed in LDS (at[c][k]) by the whole workgroup, from 16-byte
// global loads that are prefetched into registers one slice ahead.
#pragma once

#include "w4ec_common.h"

namespace w4ec {

constexpr int EC_KT = 64;                  // k per staged slice
constexpr int EC_LDS_STRIDE = EC_KT + 8;   // halves per transposed row (16-byte aligned rows)
constexpr int EC_MAX_COLS = 272;           // (256 + 1) rounded up to 16
constexpr int EC_LDS_HALVES = EC_MAX_COLS * EC_LDS_STRIDE;
constexpr int EC_THREADS = 256;

__device__ inline int ec_col_blocks(int r) { return (r + 1 + 15) >> 4; }

// One workgroup (EC_THREADS threads) computes, for the 16 rows that the
// calling wavefront's lanes point at (xrow = this lane's row, already
// clamped to a valid token), the fragments of X[:, kbeg:kend) [A|w_g] for
// column blocks cb = cb_first + i * CB_STEP (i < MAXI, cb < CBE), into
// acc[i] (v_mfma_f32_16x16x32 C layout: column 16 cb + (l & 15), rows
// 4 (l >> 4) + v).  kbeg, kend are multiples of 64.  All threads must call.
//
// ACH 16-byte chunks of A per thread are prefetched one slice ahead (enough
// for 8 * ACH columns of A); chunks beyond that are read when stored.
template <int ACT, int CB_STEP, int MAXI, int ACH>
__device__ void ec_tile(const uint16_t* __restrict__ X, int K, int xrow,
                        const uint16_t* __restrict__ A, const uint16_t* __restrict__ w_g, int r,
                        int kbeg, int kend, int cb_first, uint16_t* at, floatx4 (&acc)[MAXI])
{
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int koff = 8 * (l >> 4);
    const int CBE = ec_col_blocks(r);
    const int cols = CBE * 16;
    const bool vec = (r & 7) == 0;
    const int cpr = r >> 3;                 // 16-byte chunks per row of A (vector path)
    const int nch = EC_KT * cpr;            // chunks per slice (<= 64 * 32)

#pragma unroll
    for (int i = 0; i < MAXI; ++i)
        acc[i] = (floatx4){0.f, 0.f, 0.f, 0.f};

    // constant columns: padding beyond the gate, and the gate when absent
    for (int idx = tid; idx < (cols - r) * EC_KT; idx += EC_THREADS) {
        const int c = r + idx / EC_KT, kk = idx % EC_KT;
        if (c > r || !w_g)
            at[c * EC_LDS_STRIDE + kk] = 0;
    }

    const uint16_t* xp = X + (size_t)xrow * K + koff;
    u32x4 ach[ACH];
    uint16_t gv = 0;
    u32x4 xn0, xn1;
    auto gload = [&](int k) {
        if (vec) {
#pragma unroll
            for (int i = 0; i < ACH; ++i) {
                const int ch = tid + EC_THREADS * i;
                if (ch < nch) {
                    const int kk = ch % EC_KT, cc = (ch / EC_KT) * 8;
                    ach[i] = ld16(A + (size_t)(k + kk) * r + cc);
                }
            }
        }
        if (w_g && tid < EC_KT)
            gv = w_g[k + tid];
        xn0 = ld16(xp + k);
        xn1 = ld16(xp + k + 32);
    };
    auto lstore = [&](int k) {
        if (vec) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int ch = tid + EC_THREADS * i;
                if (ch < nch) {
                    const int kk = ch % EC_KT, cc = (ch / EC_KT) * 8;
                    const u32x4 v = (i < ACH) ? ach[i < ACH ? i : 0] : ld16(A + (size_t)(k + kk) * r + cc);
                    const uint32_t w0 = v.x, w1 = v.y, w2 = v.z, w3 = v.w;
                    uint16_t* dst = at + cc * EC_LDS_STRIDE + kk;
                    dst[0 * EC_LDS_STRIDE] = (uint16_t)(w0 & 0xFFFF);
                    dst[1 * EC_LDS_STRIDE] = (uint16_t)(w0 >> 16);
                    dst[2 * EC_LDS_STRIDE] = (uint16_t)(w1 & 0xFFFF);
                    dst[3 * EC_LDS_STRIDE] = (uint16_t)(w1 >> 16);
                    dst[4 * EC_LDS_STRIDE] = (uint16_t)(w2 & 0xFFFF);
                    dst[5 * EC_LDS_STRIDE] = (uint16_t)(w2 >> 16);
                    dst[6 * EC_LDS_STRIDE] = (uint16_t)(w3 & 0xFFFF);
                    dst[7 * EC_LDS_STRIDE] = (uint16_t)(w3 >> 16);
                }
            }
        } else {
            for (int idx = tid; idx < EC_KT * r; idx += EC_THREADS) {
                const int kk = idx / r, c = idx - kk * r;
                at[c * EC_LDS_STRIDE + kk] = A[(size_t)(k + kk) * r + c];
            }
        }
        if (w_g && tid < EC_KT)
            at[r * EC_LDS_STRIDE + tid] = gv;
    };

    if (kbeg < kend)
        gload(kbeg);
    for (int k = kbeg; k < kend; k += EC_KT) {
        __syncthreads();                 // the previous slice has been consumed
        lstore(k);
        const u32x4 x0 = xn0, x1 = xn1;
        __syncthreads();
        if (k + EC_KT < kend)
            gload(k + EC_KT);
#pragma unroll
        for (int i = 0; i < MAXI; ++i) {
            const int cb = cb_first + i * CB_STEP;
            if (cb < CBE) {
                const uint16_t* bp = at + (cb * 16 + (l & 15)) * EC_LDS_STRIDE + koff;
                acc[i] = mfma16x16x32<ACT>(x0, *reinterpret_cast<const u32x4*>(bp), acc[i]);
                acc[i] = mfma16x16x32<ACT>(x1, *reinterpret_cast<const u32x4*>(bp + 32), acc[i]);
            }
        }
    }
}

}  // namespace w4ec
