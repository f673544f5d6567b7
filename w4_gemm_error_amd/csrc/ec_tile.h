// ec_tile.h -- internal to libw4ec: LDS staging of [A | w_g] slices for the
// gate / low-rank down-projection, [T | l] = X [A | w_g], as MFMA tiles
// (shared by the decode kernel's EC workgroups and the prefill prepass).
//
// A is row-major [K, r]: a slice of rows [k0, k0 + kc) is one contiguous
// block, copied verbatim into LDS with direct global-to-LDS 16-byte loads
// (no registers, no per-element index arithmetic).  An MFMA B operand wants
// 8 consecutive k of one column per lane; gfx950's LDS transpose read
// (ds_read_b64_tr_b16) delivers exactly that from the row-major slice: in
// each group of 16 lanes, output lane i, element j is element (i mod 4) of
// the 8 bytes addressed by lane 4 j + i / 4.  So when lane 4 q + u of the
// group points at row k + q, columns n0 + 4 u .. n0 + 4 u + 3, lane i
// receives column n0 + i at rows k .. k + 3.
//
// Column blocks: cb < ec_a_blocks(r) hold 16 columns of A (columns >= r of
// the last block read past the row and are discarded); block ec_a_blocks(r)
// holds the gate vector as its column 0 (all zero when there is no gate,
// i.e. a zero gate logit) and, on request, a column of ones as its column 1
// (the token's sum of activations), zero elsewhere.
#pragma once

#include "w4ec_common.h"

namespace w4ec {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) short4_t lds_short4;

// (slice geometry: ec_pitch, ec_a_blocks, ec_blocks, ec_slice_bytes in w4ec_common.h)

// Bank swizzle of a staged slice.  A fragment read takes, per group of 16
// lanes, 32 bytes (16 columns) from each of four consecutive rows.  When a
// row is a multiple of 128 bytes (r a multiple of 64) those four 32-byte
// pieces would fall on the same eight of the 32 banks; so row k stores its
// 32-byte column pairs in the order p ^ ec_swz(k): then the four rows of a
// read land on four different groups of eight banks (rows of 64 + 128 j
// bytes take (k >> 1) & 1; other pitches are left as they are).  Applies
// to pitches (halves) that are multiples of 32.
__host__ __device__ inline int ec_swz(int k, int pitch)
{
    if (pitch & 31)
        return 0;
    return ((pitch >> 4) & 3) == 0 ? (k & 3) : ((k >> 1) & 1);
}

// 16 bytes from global memory into LDS; lds_base is wavefront-uniform and
// lane l's bytes land at lds_base + 16 l
__device__ inline void copy16_to_lds(const void* src, void* lds_base)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_base, 16, 0, 0);
}

// Stage rows [k0, k0 + kc) of A into at[kc][ec_pitch(r)] and w_g[k0, k0 + kc)
// into wgl[kc] (kc a multiple of 64, <= 512; k0 a multiple of 64), swizzled
// (ec_swz) when SWZ.  Every thread of the NT calls; the caller waits for
// the loads (s_waitcnt vmcnt) and synchronizes before reading.
template <int NT = 256, bool SWZ = false>
__device__ inline void ec_stage(const uint16_t* __restrict__ A, const uint16_t* __restrict__ w_g, int r,
                                int k0, int kc, uint16_t* at, uint16_t* wgl)
{
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    if ((r & 3) == 0) {
        // pitch == r: the LDS slice is the global one, 16-byte chunk by chunk
        // (16-byte aligned: k0 r 2 is a multiple of 128), with each row's
        // 32-byte pairs in swizzled order: LDS chunk j of row k holds global
        // chunk 2 ((j >> 1) ^ ec_swz(k)) + (j & 1)
        const int bytes = kc * r * 2;
        const int cpr = r >> 3;                         // 16-byte chunks per row
        const bool pow2 = (cpr & (cpr - 1)) == 0;
        const int sh = __builtin_ctz(cpr);
        const char* src = reinterpret_cast<const char*>(A + (size_t)k0 * r);
        for (int off = w * 1024; off < bytes; off += NT * 16) {
            const int c = (off >> 4) + l;
            if (16 * c < bytes) {
                if constexpr (SWZ) {
                    const int k = pow2 ? c >> sh : c / cpr, j = c - k * cpr;
                    const int jg = 2 * ((j >> 1) ^ ec_swz(k, r)) + (j & 1);
                    copy16_to_lds(src + 16 * (k * cpr + jg), reinterpret_cast<char*>(at) + off);
                } else {
                    copy16_to_lds(src + 16 * c, reinterpret_cast<char*>(at) + off);
                }
            }
        }
    } else {
        const int pitch = ec_pitch(r);
        for (int idx = tid; idx < kc * r; idx += NT) {
            const int kk = idx / r, c = idx - kk * r;
            const int cs = SWZ ? (((c >> 4) ^ ec_swz(kk, pitch)) << 4) + (c & 15) : c;
            at[kk * pitch + cs] = A[(size_t)(k0 + kk) * r + c];
        }
    }
    if (w_g && w == 0 && 8 * l < kc)
        copy16_to_lds(w_g + k0 + 8 * l, wgl);
}

// B fragment of v_mfma_f32_16x16x32 from a row-major LDS array of 16-bit
// values (pitch halves per row, a multiple of 4), columns c0 .. c0 + 15,
// rows krow .. krow + 31: lane l gets column c0 + (l & 15) at rows
// krow + 8 (l >> 4) + t, t = 0..7.
// the transpose reads of a B fragment, lane l at p (its row and column
// chosen by the caller), the second four rows 4 pitch halves further on
__device__ inline u32x4 tr_bfrag(const uint16_t* p, int pitch)
{
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p);
    const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p + 4 * pitch));
    return (u32x4){(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                   (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                   (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                   (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
}

__device__ inline u32x4 lds_bfrag(const uint16_t* base, int pitch, int c0, int krow)
{
    const int l = threadIdx.x & 63;
    return tr_bfrag(base + (krow + 8 * (l >> 4) + ((l & 15) >> 2)) * pitch + c0 + 4 * (l & 3), pitch);
}

// B fragment for column block cb < ec_a_blocks(r) of the staged slice (rows
// krow .. krow + 31, krow a multiple of 8; the swizzle, when SWZ, is the
// same for rows k and k + 4)
template <bool SWZ = false>
__device__ inline u32x4 ec_bfrag_a(const uint16_t* at, int r, int cb, int krow)
{
    const int l = threadIdx.x & 63;
    const int pitch = ec_pitch(r);
    const int row = krow + 8 * (l >> 4) + ((l & 15) >> 2);
    const int cbs = SWZ ? cb ^ ec_swz(row, pitch) : cb;
    return tr_bfrag(at + row * pitch + 16 * cbs + 4 * (l & 3), pitch);
}

// B fragment of the gate block (column block ec_a_blocks(r)), same rows:
// column 0 is the gate vector (or zero without one), column 1 the ones of
// one2 (two ones in the activation format, or 0), the rest zero.  Every lane
// reads (a valid address) and then selects, so no lane diverges.
__device__ inline u32x4 ec_bfrag_gate(const uint16_t* wgl, bool gate, uint32_t one2, int krow)
{
    const int l = threadIdx.x & 63;
    const u32x4 v = *reinterpret_cast<const u32x4*>(wgl + krow + 8 * (l >> 4));
    const int j = l & 15;
    const bool g = gate && j == 0;
    const uint32_t o = j == 1 ? one2 : 0u;
    return (u32x4){g ? v.x : o, g ? v.y : o, g ? v.z : o, g ? v.w : o};
}

// Column of the [T | l] partial held by lane column j of block cb, or -1
// when that column is discarded (the sum column is not part of it).
__device__ inline int ec_col(int r, int cb, int j)
{
    if (cb == ec_a_blocks(r))
        return j == 0 ? r : -1;
    const int c = 16 * cb + j;
    return c < r ? c : -1;
}

// ---------------------------------------------------------------- vector gate
//
// One gate per rank component (SPEAR summary section 2.1A: W + B diag(gamma(A
// x)) A with gamma a bottleneck MLP, read as gamma = sigmoid(relu(T G1 + c1)
// G2 + c2)), for nt <= VG_TMAX token rows of T held in LDS.  256 threads.
constexpr int VG_HMAX = 64;     // widest bottleneck
constexpr int VG_TMAX = 16;     // token rows per call
constexpr int VG_THREADS = 256;

// Staging of the gate parameters in LDS ([r h | h | h r | r] act values):
// vgate_stage_load issues every load into registers (VG_SREG per thread,
// so at most VG_SREG * VG_THREADS values: vgate_stageable), the caller
// issues its own loads, then vgate_stage_store writes the values to LDS and
// points G1 .. c2 at them.  The parameters do not depend on T, so their
// trip to memory overlaps the one for T.
constexpr int VG_SREG = 16;

__host__ __device__ inline int vgate_stage_elems(int r, int h) { return 2 * r * h + r + h; }
__host__ __device__ inline bool vgate_stageable(int r, int h) { return vgate_stage_elems(r, h) <= VG_SREG * VG_THREADS; }

__device__ inline void vgate_stage_load(const uint16_t* G1, const uint16_t* c1, const uint16_t* G2,
                                        const uint16_t* c2, int r, int h, uint16_t (&v)[VG_SREG])
{
    const int n1 = r * h, tot = vgate_stage_elems(r, h);
#pragma unroll
    for (int k = 0; k < VG_SREG; ++k) {
        const int e = k * VG_THREADS + (int)threadIdx.x;
        v[k] = 0;
        if (e < n1)
            v[k] = G1[e];
        else if (e < n1 + h)
            v[k] = c1[e - n1];
        else if (e < 2 * n1 + h)
            v[k] = G2[e - n1 - h];
        else if (e < tot)
            v[k] = c2[e - 2 * n1 - h];
    }
}

__device__ inline void vgate_stage_store(const uint16_t*& G1, const uint16_t*& c1, const uint16_t*& G2,
                                         const uint16_t*& c2, int r, int h, const uint16_t (&v)[VG_SREG],
                                         uint16_t* dst)
{
    const int n1 = r * h, tot = vgate_stage_elems(r, h);
#pragma unroll
    for (int k = 0; k < VG_SREG; ++k) {
        const int e = k * VG_THREADS + (int)threadIdx.x;
        if (e < tot)
            dst[e] = v[k];
    }
    G1 = dst;
    c1 = dst + n1;
    G2 = dst + n1 + h;
    c2 = dst + 2 * n1 + h;
}

// u[t][i] = relu(sum_c T[t][c] G1[c][i] + c1[i]) into tU ([nt][VG_HMAX]).
// Thread (chunk, i) adds a chunk of the r columns for every row: its G1
// loads are coalesced (neighbouring threads read neighbouring i) and issued
// eight at a time; the chunks' partial sums meet in `red`
// ([nt][VG_THREADS] floats) and are added in chunk order.
template <int ACT>
__device__ void vgate_hidden(const float* tT, int ldT, int nt, int r, int h, const uint16_t* G1,
                             const uint16_t* c1, float* tU, float* red)
{
    const int tid = threadIdx.x;
    const int nch = VG_THREADS / h;
    const int i = tid % h, ch = tid / h;
    if (ch < nch) {
        const int per = (r + nch - 1) / nch;
        const int cb = min(r, ch * per), ce = min(r, cb + per);
        float acc[VG_TMAX];
#pragma unroll
        for (int t = 0; t < VG_TMAX; ++t)
            acc[t] = 0.0f;
        for (int c0 = cb; c0 < ce; c0 += 8) {
            float g[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                g[k] = c0 + k < ce ? act_to_f32<ACT>(G1[(size_t)(c0 + k) * h + i]) : 0.0f;
#pragma unroll
            for (int t = 0; t < VG_TMAX; ++t) {
                if (t < nt) {
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        if (c0 + k < ce)
                            acc[t] += tT[t * ldT + c0 + k] * g[k];
                }
            }
        }
#pragma unroll
        for (int t = 0; t < VG_TMAX; ++t)
            if (t < nt)
                red[(t * nch + ch) * h + i] = acc[t];
    }
    __syncthreads();
    for (int e = tid; e < nt * h; e += VG_THREADS) {
        const int t = e / h, q = e - t * h;
        float u = 0.0f;
        for (int c = 0; c < nch; ++c)
            u += red[(t * nch + c) * h + q];
        u += act_to_f32<ACT>(c1[q]);
        tU[t * VG_HMAX + q] = fmaxf(u, 0.0f);
    }
    __syncthreads();
}

// gamma[t][c] = sigmoid(sum_i u[t][i] G2[i][c] + c2[c]) for the columns c
// of [c_lo, c_hi), one thread per column (G2 loads coalesced, eight at a
// time); out(t, c, gamma) receives each gate.
template <int ACT, typename F>
__device__ void vgate_gates(const float* tU, int nt, int r, int h, const uint16_t* G2, const uint16_t* c2,
                            int c_lo, int c_hi, F&& out)
{
    for (int c = c_lo + (int)threadIdx.x; c < c_hi; c += VG_THREADS) {
        float z[VG_TMAX];
        const float bias = act_to_f32<ACT>(c2[c]);
#pragma unroll
        for (int t = 0; t < VG_TMAX; ++t)
            z[t] = 0.0f;
        for (int i0 = 0; i0 < h; i0 += 8) {
            float g[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                g[k] = i0 + k < h ? act_to_f32<ACT>(G2[(size_t)(i0 + k) * r + c]) : 0.0f;
#pragma unroll
            for (int t = 0; t < VG_TMAX; ++t) {
                if (t < nt) {
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        if (i0 + k < h)
                            z[t] += tU[t * VG_HMAX + i0 + k] * g[k];
                }
            }
        }
#pragma unroll
        for (int t = 0; t < VG_TMAX; ++t)
            if (t < nt)
                out(t, c, sigmoid_f32(z[t] + bias));
    }
}

}  // namespace w4ec
