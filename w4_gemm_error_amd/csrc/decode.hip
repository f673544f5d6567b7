// decode.hip -- the W4 + EC layer for 1..16 tokens in a single kernel launch.
//
// SPEAR (gist.science technical summary, section 2.2A): in the decode phase
// the layer is memory bound, and the EC is folded into the low-bit GEMM's
// epilogue so that no second launch sits on the critical path.  One grid
// does all of it:
//
//  * workgroups [0, P): "EC" role.  Each loads one K-slice of X, A and w_g
//    in a single trip, forms the partial sums of T = X A and of the gate
//    logit X . w_g with MFMAs, and hands them over (below).  They have the
//    lowest ids, so they are dispatched before any main workgroup.
//  * workgroups [P, P + n_main): "main" role.  Each owns CB blocks of 16
//    output columns; its four wavefronts split K.  A wavefront keeps a ring
//    of in-flight 16-byte panel loads (16 columns x 128 k of packed codes per
//    load), turns the codes into (q - z) with a few integer and packed-half
//    operations and accumulates X Wd^T with v_mfma_f32_16x16x32 (the tokens
//    are the 16 MFMA rows); sums are scaled by s whenever the group changes.
//    After an LDS reduction over the wavefronts, the epilogue extends the
//    reduction by the r rank terms, acc += T_g B, as MFMAs, then rounds and
//    stores Y.
//
// Hand-over of the gated rank-r activations T_g = g * T.  While the weight
// stream saturates HBM, every dependent trip to memory costs microseconds,
// and hundreds of workgroups polling or reading one spot pile onto one
// memory channel; so the data is published in DEC_NREP replica slots spread
// over the channels, main workgroup i using slot i mod DEC_NREP.  Each EC
// workgroup writes its partial sums; the last one to arrive adds them in a
// fixed order, applies the gate and writes T_g into every slot, then raises
// each slot's flag.  (Letting every main workgroup add the P partials itself
// instead makes the grid as a whole read megabytes of partial sums, and
// measured slower even for one token.)
// The last reader of a slot returns its control words to zero.  All waits
// are bounded.  Hand-over data moves with device-coherent accesses (see
// w4ec_common.h), so no cache-wide write-back or invalidate is needed.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "ec_tile.h"
#include "w4ec.h"
#include "w4ec_common.h"
#include "w4ec_launch.h"

namespace w4ec {

constexpr int DEC_EC_MAXI = 5;     // column blocks per wavefront in the EC role (17 / 4)
constexpr int DEC_EC_KSMAX = 256;  // k per EC slice (at most)


struct DecodeKArgs {
    const uint16_t* X;
    const uint8_t* codes;
    const uint32_t* sz;
    const uint16_t* A;
    const uint16_t* B;
    const uint16_t* w_g;
    float b_g;
    uint16_t* Y;
    int M, N, K, r, r_pad, G, NB, KB, Npad;
    int P, KS, RC, n_main;
    int stage_first;     // main workgroups stage X before issuing weight loads
    uint32_t* flags;     // [2]: a wait timed out (sticky: every later call's Y is NaN)
    uint32_t spin;       // polls before a bounded wait gives up (0: give up at once)
    uint32_t* partial;   // [P][M][RC] hand-over words
    uint8_t* rep_ctrl;   // DEC_NREP slots of DEC_REP_CTRL_STRIDE bytes: [1] readers done
    uint8_t* rep_data;   // DEC_NREP slots of DEC_REP_DATA_STRIDE bytes: T_g [M][r_pad] as hand-over words
    // vector gate (h > 0): gamma = sigmoid(relu(T G1 + c1) G2 + c2) per rank component
    const uint16_t* G1;  // act [r][h]
    const uint16_t* c1;  // act [h]
    const uint16_t* G2;  // act [h][r]
    const uint16_t* c2;  // act [r]
    int h;
    int vg_staged;       // the gate parameters are copied to LDS (they fit)
    const int32_t* S;    // salient-channel correction: T = X[:, S] (no EC role), or null
    // codebook weights (codebook kernels only): per-channel codebooks of 16
    // fp16 entries and the sparse outlier residual in compressed rows
    const uint16_t* cb;      // [N][16] (per channel), or the library [L][16]
    const int32_t* row_ptr;  // [N + 1]
    const int32_t* col_idx;  // [nnz]
    const uint16_t* val;     // [nnz] fp16
    int nnz;
    const uint8_t* libid;    // library mode: [N][K / 128] each group's entry
    int L;                   // library mode: entries (1 .. CBK_LIB_MAX)
};

// Codebook modes of the decode main role (template parameter CBK)
constexpr int CBK_NONE = 0, CBK_CHANNEL = 1, CBK_LIBRARY = 2;
constexpr int CBK_LIB_MAX = W4EC_XFP_LIB_MAX;   // library entries a workgroup's tables hold

// Codebook lookup of one dword of indices (natural order: byte j holds the
// indices of k = 2j and 2j + 1): t points at the column's entry 0 of a pair
// table laid out [256][16 columns], entry p = cb[p & 15] | cb[p >> 4] << 16,
// so that each byte of w selects one MFMA operand dword.  A column's
// entries sit in 4 of the 64 banks, so only the 4 lanes that read the same
// column's table can conflict.
template <int STRIDE = PANEL_N>
__device__ inline u32x4 cb_lookup(uint32_t w, const uint32_t* t)
{
    return (u32x4){t[(w & 0xFFu) * STRIDE], t[((w >> 8) & 0xFFu) * STRIDE], t[((w >> 16) & 0xFFu) * STRIDE],
                   t[(w >> 24) * STRIDE]};
}
// Library mode: the tables of all the library's entries are laid out
// [entry][256] (t = the group's entry's table, stride 1), so that a read's
// bank follows the index byte alone: many lanes may name one entry.

// eight fp16 values -> bf16 (round to nearest even)
__device__ inline u32x4 f16x8_to_bf16x8(u32x4 v)
{
    auto cv = [](uint32_t p) {
        const float lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xFFFF));
        const float hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(p >> 16));
        return bf16_pair_from_f32(lo, hi);
    };
    return (u32x4){cv(v.x), cv(v.y), cv(v.z), cv(v.w)};
}

__device__ inline uint32_t* rep_word(const DecodeKArgs& a, int slot, int i)
{
    return reinterpret_cast<uint32_t*>(a.rep_ctrl + (size_t)slot * DEC_REP_CTRL_STRIDE) + i;
}

// EC role: every global load of the slice is issued at once -- the X
// fragments into registers, the slice of [A | w_g] straight into LDS -- then
// each wavefront runs the MFMAs for its column blocks (cb = w, w + 4, ...).
template <int ACT, int NS>
__device__ inline void dec_ec_mfma(const u32x4 (&xf)[DEC_EC_KSMAX / 32], const uint16_t* at, const uint16_t* wgl,
                                   int r, bool gate, int w, floatx4 (&acc)[DEC_EC_MAXI])
{
    const int nba = ec_a_blocks(r);
#pragma unroll
    for (int i = 0; i < DEC_EC_MAXI; ++i) {
        const int cb = w + 4 * i;                    // wavefront-uniform
        if (cb > nba)
            break;
        u32x4 bf[NS];
        if (cb < nba) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
                bf[s] = ec_bfrag_a(at, r, cb, 32 * s);
        } else {
#pragma unroll
            for (int s = 0; s < NS; ++s)
                bf[s] = ec_bfrag_gate(wgl, gate, 0u, 32 * s);
        }
#pragma unroll
        for (int s = 0; s < NS; ++s)
            acc[i] = mfma16x16x32<ACT>(xf[s], bf[s], acc[i]);
    }
}

// Vector gate (SPEAR summary section 2.1A: W + B diag(gamma(A x)) A, gamma
// a bottleneck MLP, read as gamma = sigmoid(relu(T G1 + c1) G2 + c2)).  The
// gate of a rank component depends on the token's whole row of T, so the
// reducers split tokens rather than words: reducer j of nred takes token
// j mod M (with more reducers than tokens, the reducers of one token each
// publish a share of its words) or tokens j, j + nred, ... (with fewer).
// Every reducer of a token adds the P slices of the row in slice order and
// runs the bottleneck in fp32, so all of them compute the same gates.
template <int ACT>
__device__ __forceinline__ void decode_vgate_reduce(const DecodeKArgs& a, uint8_t* smem, int j, int nred)
{
    const int tid = threadIdx.x;
    const int M = a.M, r = a.r, h = a.h;
    const int w8 = a.r_pad / 4;                             // 8-byte words of a token's T_g
    const int qs = M * a.RC;                                // words per slice
    float* tT = reinterpret_cast<float*>(smem);             // [r_pad] T of the token
    float* tG = tT + a.r_pad;                               // [r_pad] gamma * T
    float* tU = tG + a.r_pad;                               // [VG_HMAX] bottleneck
    float* red = tU + VG_HMAX;                              // [VG_THREADS] partial sums
    uint64_t* tw = reinterpret_cast<uint64_t*>(red + VG_THREADS);      // [w8], 8-byte aligned
    uint16_t* gst = reinterpret_cast<uint16_t*>(tw + w8);   // staged gate parameters (if they fit)
    const int nrep = min(DEC_NREP, a.n_main);               // slots that have readers
    // Reducer j takes tokens j, j + nred, ...: at most one reducer per
    // token, which publishes all of the token's words.  Reducers without a
    // token read nothing.  (A slot's last reader clears the partial sums once
    // the slot is complete, and it is complete only when every reducer that
    // reads them has written.)  Splitting a token's words over several
    // reducers, each of which reads the whole row and runs the bottleneck,
    // measured slower: every extra reader of the row adds to the traffic
    // that the row's arrival waits behind.
    const int m0 = j, mstep = nred, wb = 0, we = w8;
    if (m0 >= M)
        return;
    // the gate parameters do not depend on T: their loads go out first and
    // overlap the wait for the partial sums
    const uint16_t *G1 = a.G1, *c1 = a.c1, *G2 = a.G2, *c2 = a.c2;
    uint16_t gv[VG_SREG];
    if (a.vg_staged)
        vgate_stage_load(G1, c1, G2, c2, r, h, gv);
    bool staged = false;
    uint32_t it = 0;                                        // bounded wait, shared by all waits
    // a wait that gave up (or a wait limit of 0) publishes NaN for the
    // token instead of sums of partials that had not all landed
    bool lost = a.spin == 0;
    // ng thread groups split the P slices (slice q -> group q mod ng), so
    // that all of them are in flight at once; the groups' sums are added in
    // group order
    const int ng = max(1, DEC_THREADS / a.r_pad);
    for (int m = m0; m < M; m += mstep) {
        __syncthreads();                                    // LDS of the previous token is free
        for (int e = tid; e < ng * a.r_pad; e += DEC_THREADS) {
            const int g = e / a.r_pad, c = e - g * a.r_pad;
            float t = 0.0f;
            if (c < r) {
                const uint32_t* src = a.partial + (size_t)m * a.RC + c;
                for (int q = g; q < a.P; q += 8 * ng) {
                    // eight slices in flight; those not landed yet are loaded again together
                    uint32_t v[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        v[i] = q + i * ng < a.P ? atomic_load_dev(src + (size_t)(q + i * ng) * qs) : 1u;
                    for (;;) {
                        bool miss = false;
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            miss |= v[i] == 0u;
                        if (!miss || lost)
                            break;
                        if (it >= a.spin) {
                            lost = true;
                            break;
                        }
                        ++it;
                        __builtin_amdgcn_s_sleep(1);
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            if (v[i] == 0u)                 // only slices < P can read as zero
                                v[i] = atomic_load_dev(src + (size_t)(q + i * ng) * qs);
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (q + i * ng < a.P)
                            t += hw_dec32(v[i]);
                }
            }
            red[e] = t;
        }
        const bool lost_any = __syncthreads_or(lost) != 0;
        if (lost_any && tid == 0)
            atomic_store_dev(&a.flags[2], 1u);
        for (int c = tid; c < a.r_pad; c += DEC_THREADS) {
            float t = red[c];
            for (int g = 1; g < ng; ++g)
                t += red[g * a.r_pad + c];
            tT[c] = lost_any ? __builtin_nanf("") : t;
        }
        if (a.vg_staged && !staged) {
            vgate_stage_store(G1, c1, G2, c2, r, h, gv, gst);
            staged = true;
        }
        __syncthreads();
        // one copy per address space of the parameters (LDS when staged), so
        // that no access needs a flat (either-space) load
        auto bottleneck = [&](const uint16_t* g1, const uint16_t* b1, const uint16_t* g2, const uint16_t* b2) {
            vgate_hidden<ACT>(tT, 0, 1, r, h, g1, b1, tU, red);
            vgate_gates<ACT>(tU, 1, r, h, g2, b2, 4 * wb, min(r, 4 * we),
                             [&](int, int c, float g) { tG[c] = g * tT[c]; });
        };
        if (staged) {
            const int n1 = r * h;
            bottleneck(gst, gst + n1, gst + n1 + h, gst + 2 * n1 + h);
        } else {
            bottleneck(a.G1, a.c1, a.G2, a.c2);
        }
        __syncthreads();
        for (int i = tid; i < we - wb; i += DEC_THREADS) {
            const int c0 = 4 * (wb + i);
            uint64_t word = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int c = c0 + k;
                word |= (uint64_t)hw_enc16(f32_to_act<ACT>(c < r ? tG[c] : 0.0f)) << (16 * k);
            }
            tw[i] = word;
        }
        __syncthreads();
        const int nw = we - wb;
        for (int i = tid; i < nw * nrep; i += DEC_THREADS) {
            const int slot = i / nw, jj = i - slot * nw;
            st8_dev(reinterpret_cast<uint64_t*>(a.rep_data + (size_t)slot * DEC_REP_DATA_STRIDE) + (size_t)m * w8 + wb + jj,
                    tw[jj]);
        }
    }
}

// Scalar-gate reducers: the last nred EC workgroups, each with a share of
// the M r_pad / 4 words of T_g, for which thread groups split the P slices
// (slice q -> group q mod ng, eight loads in flight per thread).  nred
// starts at M (one token's worth of words each) and doubles, up to
// min(P, DEC_EC_RMAX), while a group would walk more than 16 slices (more
// than two trips).  Fewer pollers get the partial sums sooner: against
// every EC workgroup reducing, 10.4 vs 10.7 us at one token (K = 4096,
// r = 64) and 11.2 vs 11.6 us at four; a single reducer for 16 tokens took
// 18.0 us.
__host__ __device__ inline int dec_scalar_groups(int P, int M, int share)
{
    const int g = DEC_THREADS / (4 * share + M);
    return g < 1 ? 1 : (g < P ? g : P);
}
__host__ __device__ inline int dec_scalar_reducers(int P, int M, int r_pad)
{
    const int cap = P < DEC_EC_RMAX ? P : DEC_EC_RMAX;
    const int n8 = M * r_pad / 4;
    int nred = M < cap ? M : cap;
    for (;;) {
        const int share = (n8 + nred - 1) / nred;
        const int ng = dec_scalar_groups(P, M, share);
        if ((P + ng - 1) / ng <= 16 || nred >= cap)
            return nred;
        nred = 2 * nred < cap ? 2 * nred : cap;
    }
}

template <int ACT>
__device__ __forceinline__ void decode_ec_role(const DecodeKArgs& a, uint8_t* smem)
{
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int p = blockIdx.x;
    const int r = a.r;
    const int M = a.M;
    const int kbeg = p * a.KS;
    const int len = min(a.KS, a.K - kbeg);          // multiple of 64
    const int xrow = min(l & 15, M - 1);
    const bool gate = a.w_g != nullptr;
    uint16_t* at = reinterpret_cast<uint16_t*>(smem);
    uint16_t* wgl = at + len * ec_pitch(r) + 16;
    // The main workgroups sharing this CU wait for these results: give the
    // EC wavefronts the first pick of the CU's issue slots.
    __builtin_amdgcn_s_setprio(3);

    const uint16_t* xp = a.X + (size_t)xrow * a.K + kbeg + 8 * (l >> 4);
    u32x4 xf[DEC_EC_KSMAX / 32];
#pragma unroll
    for (int s = 0; s < DEC_EC_KSMAX / 32; ++s)
        xf[s] = ld16(xp + 32 * min(s, (len >> 5) - 1));   // steps past the slice are never used
    ec_stage(a.A, a.w_g, r, kbeg, len, at, wgl);
    wait_all_mem();
    __syncthreads();

    floatx4 acc[DEC_EC_MAXI];
#pragma unroll
    for (int i = 0; i < DEC_EC_MAXI; ++i)
        acc[i] = (floatx4){0.f, 0.f, 0.f, 0.f};
    switch (len >> 6) {
    case 1: dec_ec_mfma<ACT, 2>(xf, at, wgl, r, gate, w, acc); break;
    case 2: dec_ec_mfma<ACT, 4>(xf, at, wgl, r, gate, w, acc); break;
    case 3: dec_ec_mfma<ACT, 6>(xf, at, wgl, r, gate, w, acc); break;
    default: dec_ec_mfma<ACT, 8>(xf, at, wgl, r, gate, w, acc); break;
    }

    // partial sums -> [P][M][RC] as hand-over words: stored and left, with no
    // wait and no counter; EC workgroup 0 takes each one as it lands
    const int qs = M * a.RC;                               // words per slice
    uint32_t* part = a.partial + (size_t)p * qs;
#pragma unroll
    for (int i = 0; i < DEC_EC_MAXI; ++i) {
        const int cb = w + 4 * i;
        const int c = cb < ec_blocks(r) ? ec_col(r, cb, l & 15) : -1;
        // the vector gate reads only the columns of T: the logit column is
        // not stored (a word no reducer waits for could land after the slot's
        // last reader has cleared the partial sums)
        if (c >= 0 && !(a.h > 0 && c == r)) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = 4 * (l >> 4) + v;
                if (m < M)
                    atomic_store_dev(part + m * a.RC + c, hw_enc32(acc[i][v]));
            }
        }
    }

    // ---- this workgroup's share of the reduction: 8-byte words [w0, w1) of
    // T_g = g * T ([M][r_pad] values, four per word), for which it adds the P
    // slices of its T values and of every token's gate logit.  The last
    // DEC_EC_RMAX EC workgroups reduce: workgroups start in id order, so every
    // slice a reducer waits for belongs to a workgroup that has started, and
    // the waiting workgroups never hold all the CU slots.
    const int red0 = max(0, a.P - DEC_EC_RMAX);
    if (p < red0)
        return;
    if (a.h > 0) {
        __syncthreads();                                    // the slice in LDS is no longer read
        decode_vgate_reduce<ACT>(a, smem, p - red0, a.P - red0);
        return;
    }
    // With the scalar gate only the last dec_scalar_reducers() of those
    // reduce: fewer workgroups polling the partial sums get them sooner.
    const int nred = dec_scalar_reducers(a.P, M, a.r_pad);
    const int rbeg = a.P - nred;
    if (p < rbeg)
        return;
    const int n8 = M * a.r_pad / 4;
    const int share = (n8 + nred - 1) / nred;
    const int w0 = (p - rbeg) * share, w1 = min(n8, w0 + share);
    if (w0 >= w1)
        return;
    const int nw = w1 - w0;
    const int nv = 4 * nw;                                  // T values, then M logits
    const int ne = nv + M;
    // ng thread groups split the P slices (slice q -> group q mod ng); ng
    // depends on the shape only, so every workgroup adds a token's logit in
    // the same order
    const int ng = dec_scalar_groups(a.P, M, share);
    __syncthreads();                                        // the slice in LDS is no longer read
    const int tsum_off = ng > 1 ? ng * ne : 0;
    float* red = reinterpret_cast<float*>(smem);            // [ng][ne] (ng > 1 only)
    float* tsum = red + tsum_off;                           // [ne]
    uint64_t* tw = reinterpret_cast<uint64_t*>(red + ((tsum_off + ne + 1) & ~1));   // [nw], 8-byte aligned
    uint32_t it = 0;                                        // bounded wait, shared by all of this thread's waits
    // a wait that gave up (or a wait limit of 0) publishes NaN for this
    // share instead of sums of partials that had not all landed
    bool lost = a.spin == 0;
    for (int e0 = tid; e0 < ne * ng; e0 += DEC_THREADS) {
        const int g = e0 / ne, e = e0 - g * ne;
        int pe = (e - nv) * a.RC + r;                       // a logit ...
        if (e < nv) {                                       // ... or a T value (none past column r)
            const int v = 4 * w0 + e;
            const int m = v / a.r_pad, c = v - m * a.r_pad;
            pe = c < r ? m * a.RC + c : -1;
        }
        float t = 0.0f;
        if (pe >= 0) {
            const uint32_t* src = a.partial + pe;
            for (int q = g; q < a.P; q += 8 * ng) {
                // eight slices in flight; those not landed yet are loaded again together
                uint32_t v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    v[i] = q + i * ng < a.P ? atomic_load_dev(src + (size_t)(q + i * ng) * qs) : 1u;
                for (;;) {
                    bool miss = false;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        miss |= v[i] == 0u;
                    if (!miss || lost)
                        break;
                    if (it >= a.spin) {
                        lost = true;
                        break;
                    }
                    ++it;
                    __builtin_amdgcn_s_sleep(1);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        if (v[i] == 0u)                     // only slices < P can read as zero
                            v[i] = atomic_load_dev(src + (size_t)(q + i * ng) * qs);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (q + i * ng < a.P)
                        t += hw_dec32(v[i]);
            }
        }
        if (ng > 1)
            red[e0] = t;
        else
            tsum[e] = t;
    }
    const bool lost_any = __syncthreads_or(lost) != 0;
    if (lost_any && tid == 0)
        atomic_store_dev(&a.flags[2], 1u);
    if (ng > 1) {
        for (int e = tid; e < ne; e += DEC_THREADS) {
            float t = red[e];
            for (int g = 1; g < ng; ++g)
                t += red[g * ne + e];
            tsum[e] = t;
        }
    }
    if (lost_any)
        for (int e = tid; e < ne; e += DEC_THREADS)
            tsum[e] = __builtin_nanf("");
    __syncthreads();
    // gate, round to the activation format, pack four values per word
    for (int i = tid; i < nw; i += DEC_THREADS) {
        const int v0 = 4 * (w0 + i);
        const int m = v0 / a.r_pad;
        const float gm = sigmoid_f32(tsum[nv + m] + a.b_g);
        uint64_t word = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = v0 + k - m * a.r_pad;
            word |= (uint64_t)hw_enc16(f32_to_act<ACT>(c < r ? gm * tsum[4 * i + k] : 0.0f)) << (16 * k);
        }
        tw[i] = word;
    }
    __syncthreads();
    const int nrep = min(DEC_NREP, a.n_main);               // slots that have readers
    for (int i = tid; i < nw * nrep; i += DEC_THREADS) {
        const int slot = i / nw, j = i - slot * nw;
        st8_dev(reinterpret_cast<uint64_t*>(a.rep_data + (size_t)slot * DEC_REP_DATA_STRIDE) + w0 + j, tw[j]);
    }
}

// LDS of the main role: the staged activations (during the stream), the
// wavefront reduction (after it) at the same offset, then the B columns,
// the salient-channel operand, and for fractional zero points the chunk
// sums of the activations ([M][K / 128] floats) and the correction
// ([M][CB x 16] floats)
__host__ __device__ inline size_t main_b_offset(int M, int K, bool xlds, int CB)
{
    size_t b = (size_t)4 * CB * 64 * 16;
    if (xlds && (size_t)M * K * 2 > b)
        b = (size_t)M * K * 2;
    return (b + 15) / 16 * 16;
}

__host__ __device__ inline size_t main_frac_offset(int M, int K, bool xlds, int CB, int r_pad, bool ec, bool gather)
{
    const size_t b = main_b_offset(M, K, xlds, CB) + (ec ? (size_t)CB * r_pad * PANEL_N * 2 : 0) +
                     (gather ? (size_t)M * r_pad * 2 : 0);
    return (b + 15) / 16 * 16;
}

template <int ACT, int CB, int XCH, int DEPTH, bool GROUPED, bool STAGE_FIRST, int CBK = CBK_NONE>
__device__ __forceinline__ void decode_main_role(const DecodeKArgs& a, uint8_t* smem)
{
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wavefront-uniform
    const int mb = blockIdx.x - a.P;
    // Workgroups with ids congruent mod 8 run on one XCD; give each such
    // class a contiguous range of column blocks, so that the lines of B,
    // scale/zero and Y that neighbouring blocks share are fetched into one
    // L2 rather than into eight.
    const int q8 = a.n_main >> 3, r8 = a.n_main & 7, c8 = mb & 7;
    const int cb0 = (c8 * q8 + min(c8, r8) + (mb >> 3)) * CB;
    const int M = a.M;
    const int K = a.K;
    const int KB = a.KB;
    const int per = KB >> 2, rem = KB & 3;
    const int kcnt = per + (w < rem ? 1 : 0);
    // a wavefront without panels (K < 512) still issues its (clamped) loads,
    // from panel 0, and multiplies them by zero
    const int kbeg = kcnt > 0 ? w * per + min(w, rem) : 0;
    const int klast = max(kcnt - 1, 0);

    const int row = l & 15;
    const int koff = 8 * (l >> 4);
    const bool xrow = row < M;

    int n_l[CB];
    const uint8_t* wp[CB];      // this lane's 16 bytes of panel (column block, kbeg)
#pragma unroll
    for (int j = 0; j < CB; ++j) {
        const int cb = min(cb0 + j, a.NB - 1);      // a block past the end re-reads the last one (never stored)
        n_l[j] = (cb0 + j) * PANEL_N + (l & 15);
        wp[j] = a.codes + ((size_t)cb * KB + kbeg) * PANEL_BYTES + l * 16;
    }
    const int nsteps = a.r_pad >> 5;
    const uint32_t* szp[CB];    // scale/zero of column n_l[j] (group of panel kbeg)
    const int ppg = a.G / PANEL_K;                   // panels per group
#pragma unroll
    for (int j = 0; j < CB; ++j) {
        const int n = min(n_l[j], a.Npad - 1);
        szp[j] = a.sz + (size_t)((kbeg * PANEL_K) / a.G) * a.Npad + n;
    }
    const uint8_t* idp[CB];     // library mode: column n_l[j]'s group entries, from panel kbeg
    if constexpr (CBK == CBK_LIBRARY) {
#pragma unroll
        for (int j = 0; j < CB; ++j)
            idp[j] = a.libid + (size_t)min(n_l[j], a.N - 1) * KB + kbeg;
    }

    // Loads retire in issue order, so everything consumed before the first
    // panel (scale/zero, the activations staged in LDS) is issued first;
    // then a ring of DEPTH weight panels, consumed one by one as they arrive
    // and refilled unconditionally (indices clamped to the wavefront's last
    // panel, extra panels multiplied by zero) so that the ring's waits stay
    // exact.  STAGE_FIRST stages the activations completely before the first
    // weight load (so that EC loads reach memory ahead of the weight stream);
    // the launch plan currently issues the ring first in every case, which
    // measured faster once the EC reduction ran on few workgroups.
    // (Every load below is issued unconditionally -- indices are clamped and
    // unwanted values zeroed afterwards -- so that the compiler can count the
    // loads in flight and wait for exactly the one it needs.)
    constexpr bool XLDS = XCH > 0;
    // The weights enter the MFMAs with their exponent-trick offsets (one
    // AND-OR per pair); the offsets and the zero point come off per group
    // through the activations' sums.  (fp16 with groups keeps the exact
    // offset subtraction: a group of one panel would pay the sums'
    // transposition on every panel.)
    constexpr bool BIAS = !CBK && (ACT == ACT_BF16 || !GROUPED);
    u32x4 wring[DEPTH][CB];
    u32x4 xring[XLDS ? 1 : DEPTH][4];
    uint32_t szring[GROUPED ? DEPTH : 1][CB];
    uint32_t idring[CBK == CBK_LIBRARY ? DEPTH : 1][CB];   // library mode: the panels' group entries
    uint32_t sz0[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j)
        sz0[j] = *szp[j];
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
    const int nxchunks = XLDS ? M * K / 8 : 1;       // 16-byte chunks of X (XCH per thread suffice)
    // The epilogue's B columns (rows [0, r_pad) of this workgroup's column
    // blocks, 16-byte chunks of 8 columns) are loaded first, so that they do
    // not queue behind the weight stream; they stay in registers during the
    // stream and are parked in LDS after it.
    // Salient channels with X staged in LDS: the indices are this thread's
    // first loads (so waiting for them waits for nothing else), and the
    // gather X[m][S[j]] runs from LDS as soon as X is staged, under the
    // weight stream, into the operand area past the parked B.
    constexpr int SG = 4;                            // gather elements per thread (M <= 4, r_pad <= 256)
    int sg[SG];
    const bool lds_gather = XLDS && a.S != nullptr && a.r > 0;
    if (lds_gather) {
#pragma unroll
        for (int i = 0; i < SG; ++i) {
            const int e = tid + DEC_THREADS * i;
            const int j = e % a.r_pad;
            sg[i] = (e < M * a.r_pad && j < a.r) ? a.S[j] : 0;
        }
    }
    // Codebook weights (XFP summary, sections 2 and 3): the CB x 16
    // columns' codebooks are loaded before the weight stream, converted to
    // the MFMA operand type (bf16 for bf16 activations), and expanded in
    // LDS, past the staged activations, into pair tables [CB][256][16].
    // Thread tid writes entries p = tid / 16 + 16 i (i < 16) of column
    // tid % 16: their low half is codebook entry tid / 16, the high half
    // entry i, and the stores are contiguous.
    uint32_t* ptab = reinterpret_cast<uint32_t*>(smem + main_b_offset(M, K, XLDS, CB));
    u32x4 cbv[CBK ? CB : 1][2];                      // column tid % 16's 16 entries, per block
    uint32_t cblo[CBK ? CB : 1];                     // its entry tid / 16
    // The sparse residual is spread over the whole workgroup: thread tid
    // takes column rc = tid % (CB x 16) of the workgroup and its entries
    // rsub, rsub + RS, ... (rsub = tid / (CB x 16)).  Its row bounds are
    // loaded ahead of everything else, its first RB entries after the ring's
    // first panels, so that the dependent loads run under the weight stream.
    constexpr int CBN = CB * PANEL_N;                // columns per workgroup
    constexpr int RS = DEC_THREADS / CBN;            // threads per column
    constexpr int RB = 4;                            // residual entries per thread and batch
    const int rc = tid % CBN, rsub = tid / CBN;
    const bool rcol_ok = cb0 * PANEL_N + rc < a.N;
    int rb0 = 0, rb1 = 0;
    int rk[RB];
    uint32_t rv[RB];
    u32x4 libv = (u32x4){0u, 0u, 0u, 0u};            // library mode: 16 bytes of the library
    if constexpr (CBK) {
        {
            const int n = min(cb0 * PANEL_N + rc, a.N - 1);
            rb0 = a.row_ptr[n];
            rb1 = a.row_ptr[n + 1];
        }
        if constexpr (CBK == CBK_LIBRARY) {
            if (tid < 2 * a.L)
                libv = ld16(a.cb + (size_t)tid * 8);
        } else {
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const int n = min((cb0 + j) * PANEL_N + (tid & 15), a.N - 1);
                cbv[j][0] = ld16(a.cb + (size_t)n * 16);
                cbv[j][1] = ld16(a.cb + (size_t)n * 16 + 8);
                cblo[j] = a.cb[(size_t)n * 16 + (tid >> 4)];
            }
        }
    }
    u32x4 bstage[2 * CB];
    {
        const int nbch = CB * a.r_pad * 2;
        const bool bvec = ((uintptr_t)a.B & 15) == 0 && (a.N & 7) == 0;
#pragma unroll
        for (int i = 0; i < 2 * CB; ++i) {
            const int ch = tid + DEC_THREADS * i;
            const int j = ch / (2 * a.r_pad), jr = (ch >> 1) - j * a.r_pad;
            const int n0 = (cb0 + j) * PANEL_N + 8 * (ch & 1);
            u32x4 v = (u32x4){0u, 0u, 0u, 0u};
            if (a.r > 0 && ch < nbch && jr < a.r) {
                const uint16_t* src = a.B + (size_t)jr * a.N + n0;
                if (bvec && n0 + 8 <= a.N) {
                    v = ld16(src);
                } else {
                    uint32_t hv[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        hv[t] = n0 + t < a.N ? (uint32_t)src[t] : 0u;
                    v = (u32x4){hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16),
                                hv[6] | (hv[7] << 16)};
                }
            }
            bstage[i] = v;
        }
    }
    u32x4 xstage[XLDS ? XCH : 1];
    const uint16_t* xg = a.X + (size_t)(xrow ? row : 0) * K + (size_t)kbeg * PANEL_K + koff;
    auto issue = [&](int u, int i) {                 // panel i (clamped) into ring slot u
        const int ic = min(i, klast);
        if constexpr (CBK == CBK_LIBRARY) {
#pragma unroll
            for (int j = 0; j < CB; ++j)
                idring[u][j] = idp[j][ic];
        }
        if constexpr (GROUPED) {
            const int gi = ((kbeg + ic) * PANEL_K) / a.G - (kbeg * PANEL_K) / a.G;
#pragma unroll
            for (int j = 0; j < CB; ++j)
                szring[u][j] = szp[j][(size_t)gi * a.Npad];
        }
#pragma unroll
        for (int j = 0; j < CB; ++j)
            wring[u][j] = ld16_stream(wp[j] + (size_t)ic * PANEL_BYTES);
        if constexpr (!XLDS) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                xring[u][s] = ld16(xg + (size_t)ic * PANEL_K + 32 * s);
        }
    };
    auto store_x = [&]() {
#pragma unroll
        for (int i = 0; i < XCH; ++i)
            st16(xs + (size_t)min(tid + DEC_THREADS * i, nxchunks - 1) * 8, xstage[i]);
        lds_barrier();
    };
    if constexpr (XLDS) {
#pragma unroll
        for (int i = 0; i < XCH; ++i)
            xstage[i] = ld16(a.X + (size_t)min(tid + DEC_THREADS * i, nxchunks - 1) * 8);
    }
    // keep the issue order: the scheduler must not sink these loads below the
    // weight loads (each wait would then cover the whole ring)
    __builtin_amdgcn_sched_barrier(0);
    uint16_t* tgl = reinterpret_cast<uint16_t*>(smem + main_b_offset(M, K, XLDS, CB)) + (size_t)CB * a.r_pad * PANEL_N;
    auto gather_lds = [&]() {
        bool bad = false;
#pragma unroll
        for (int i = 0; i < SG; ++i) {
            const int e = tid + DEC_THREADS * i;
            if (e < M * a.r_pad) {
                const int m = e / a.r_pad, j = e - m * a.r_pad;
                int idx = sg[i];
                bad |= j < a.r && (idx < 0 || idx >= K);
                idx = min(max(idx, 0), K - 1);
                tgl[e] = j < a.r ? xs[(size_t)m * K + idx] : (uint16_t)0;
            }
        }
        if (bad)
            atomic_store_dev(&a.flags[3], 1u);
    };
    if constexpr (XLDS && STAGE_FIRST) {
        store_x();
        if (lds_gather)
            gather_lds();
    }
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
        issue(u, u);
        __builtin_amdgcn_sched_barrier(0);   // slot u is issued u-th
    }
    if constexpr (XLDS && !STAGE_FIRST) {
        store_x();
        if (lds_gather)
            gather_lds();
    }
    if constexpr (CBK == CBK_LIBRARY) {
        // the library, staged in LDS past the tables (rounded to bf16 for
        // bf16 activations), then every entry's table: thread tid writes
        // entry byte tid of each, cb[tid & 15] | cb[tid >> 4] << 16
        static_assert(DEC_THREADS == 256, "one table entry per thread and library entry");
        uint16_t* libl = reinterpret_cast<uint16_t*>(ptab + CBK_LIB_MAX * 256);
        if (tid < 2 * a.L)
            st16(libl + tid * 8, ACT == ACT_BF16 ? f16x8_to_bf16x8(libv) : libv);
        lds_barrier();
#pragma unroll 4
        for (int e = 0; e < a.L; ++e)
            ptab[e * 256 + tid] = (uint32_t)libl[e * 16 + (tid & 15)] | ((uint32_t)libl[e * 16 + (tid >> 4)] << 16);
        lds_barrier();
    } else if constexpr (CBK) {
        static_assert(DEC_THREADS == 256, "sixteen pair-table entries per thread and block");
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            u32x4 v0 = cbv[j][0], v1 = cbv[j][1];
            uint32_t lo = cblo[j];
            if constexpr (ACT == ACT_BF16) {
                v0 = f16x8_to_bf16x8(v0);
                v1 = f16x8_to_bf16x8(v1);
                lo = f16x8_to_bf16x8((u32x4){lo, 0u, 0u, 0u}).x & 0xFFFFu;
            }
            const uint32_t e[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            uint32_t* tj = ptab + j * 256 * PANEL_N + tid;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                tj[256 * i] = lo | ((i & 1) ? (e[i >> 1] & 0xFFFF0000u) : (e[i >> 1] << 16));
        }
        lds_barrier();
    }
    if constexpr (CBK) {
        // row bounds clamped to [0, nnz] (an absent column has none), then
        // the first batch (indices clamped into the arrays, which the host
        // makes non-empty; entries past the row are discarded)
        rb0 = rcol_ok ? min(max(rb0, 0), a.nnz) : 0;
        rb1 = rcol_ok ? min(max(rb1, 0), a.nnz) : 0;
        const int elast = max(a.nnz - 1, 0);
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int e = min(rb0 + rsub + RS * i, elast);
            rk[i] = a.col_idx[e];
            rv[i] = a.val[e];
        }
    }

    // Zero points.  Offset codes (BIAS): a group adds s (accg - (oL + z) xL -
    // (oH + z) xH), xL and xH this wavefront's activation sums over the
    // group's panels and the two kinds of k position -- exact in z, any fp16
    // zero point.  Otherwise the codes are offset by the integer part
    // zi = floor(z) exactly (the exponent trick), and a fractional part
    // zf = z - zi leaves -zf * s * (the group's activation sum) per output,
    // which the epilogue subtracts when some zero point is fractional (a
    // slower path; with integer zero points nothing is added).
    floatx4 acc[CB], accg[CB];
    float s_cur[CB];
    DqF16 dqh[CB];
    float dqb[CB];
    float cL[CB], cH[CB];   // BIAS: s (oL + z), s (oH + z)
    // BIAS: this lane's activation sums over the group so far (token l & 15,
    // the lane's k chunks), at the two kinds of k position (offset 1024 /
    // 64 for fp16, both 128 for bf16)
    float plo = 0.0f, phi = 0.0f;
    // ... and their transposition through LDS at a group's end: [4 chunk
    // groups][16 tokens][2] per wavefront
    float* tsum = reinterpret_cast<float*>(smem + main_frac_offset(M, K, XLDS, CB, a.r_pad, a.r > 0,
                                                                   a.r > 0 && a.S != nullptr)) + w * 128;
    bool fz = false;        // a zero point this lane has seen is fractional
    auto set_sz = [&](const uint32_t* v) {
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            s_cur[j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[j] & 0xFFFF));
            const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[j] >> 16));
            if constexpr (BIAS) {
                cL[j] = s_cur[j] * ((ACT == ACT_F16 ? 1024.0f : 128.0f) + z);
                cH[j] = s_cur[j] * ((ACT == ACT_F16 ? 64.0f : 128.0f) + z);
            } else {
                const float zi = floorf(z);
                fz |= z != zi;
                if constexpr (ACT == ACT_F16)
                    dqh[j] = dq_f16_consts(zi);
                else
                    dqb[j] = -(8388608.0f + zi);
            }
        }
    };
    // the end of a group: its partial sums, scaled, into acc.  With offset
    // codes the activation sums go through LDS from the lanes that hold them
    // (token l & 15) to those whose accumulator rows they are (tokens
    // 4 (l >> 4) + v), the four chunk groups added in order; only this
    // wavefront touches its area, and its LDS accesses complete in order.
    auto flush = [&]() {
        float sxl[4] = {0.f, 0.f, 0.f, 0.f}, sxh[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BIAS) {
            tsum[((l >> 4) * 16 + (l & 15)) * 2] = plo;
            tsum[((l >> 4) * 16 + (l & 15)) * 2 + 1] = phi;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const floatx4 t0 = *reinterpret_cast<const floatx4*>(tsum + (g * 16 + 4 * (l >> 4)) * 2);
                const floatx4 t1 = *reinterpret_cast<const floatx4*>(tsum + (g * 16 + 4 * (l >> 4)) * 2 + 4);
                sxl[0] += t0[0]; sxh[0] += t0[1];
                sxl[1] += t0[2]; sxh[1] += t0[3];
                sxl[2] += t1[0]; sxh[2] += t1[1];
                sxl[3] += t1[2]; sxh[3] += t1[3];
            }
            plo = 0.0f;
            phi = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            if constexpr (BIAS) {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[j][v] += s_cur[j] * accg[j][v] - (cL[j] * sxl[v] + cH[j] * sxh[v]);
            } else {
                acc[j] += s_cur[j] * accg[j];
            }
            accg[j] = (floatx4){0.f, 0.f, 0.f, 0.f};
        }
    };
#pragma unroll
    for (int j = 0; j < CB; ++j) {
        acc[j] = (floatx4){0.f, 0.f, 0.f, 0.f};
        accg[j] = acc[j];
    }
    set_sz(sz0);
    if constexpr (CBK) {
#pragma unroll
        for (int j = 0; j < CB; ++j)
            s_cur[j] = 1.0f;                         // the codebook entries are the weights
    }
    int left_in_group = ppg - (kbeg % ppg);          // panels until the group changes

    // lanes of absent tokens read token M - 1's row (the same address in all
    // of them: an LDS broadcast) and multiply zeros
    const uint16_t* xl = xs + (size_t)min(row, M - 1) * K + (size_t)kbeg * PANEL_K + koff;
    // one chunk of DEPTH panels; REFILL: the ring is refilled for the next
    // chunk (only while one follows, so no panel is loaded twice)
    auto chunk = [&](int i0, auto refill_tag) {
        constexpr bool REFILL = decltype(refill_tag)::value;
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            const int i = i0 + u;
            const bool valid = i < kcnt;                // wavefront-uniform
            u32x4 wv[CB];
            u32x4 xf[4];
#pragma unroll
            for (int j = 0; j < CB; ++j)
                wv[j] = wring[u][j];
            uint32_t szv[CB];
            if constexpr (GROUPED) {
#pragma unroll
                for (int j = 0; j < CB; ++j)
                    szv[j] = szring[u][j];
            }
            uint32_t tl[CB];                            // library mode: the panel's entries' tables
            if constexpr (CBK == CBK_LIBRARY) {
                // (an entry past the library is clamped to its last)
#pragma unroll
                for (int j = 0; j < CB; ++j)
                    tl[j] = min(idring[u][j], (uint32_t)(a.L - 1)) << 8;
            }
            if constexpr (XLDS) {
                const int ic = min(i, klast);
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    xf[s] = *reinterpret_cast<const u32x4*>(xl + (size_t)ic * PANEL_K + 32 * s);
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    xf[s] = xring[u][s];
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
                xf[s] = (valid && xrow) ? xf[s] : (u32x4){0u, 0u, 0u, 0u};
            if constexpr (REFILL) {
                issue(u, i + DEPTH);
                __builtin_amdgcn_sched_barrier(0);  // refill slot u as soon as it is consumed
            }
            if constexpr (GROUPED) {
                if (valid && left_in_group == ppg && i > 0) {
                    flush();
                    set_sz(szv);
                }
            }
            if constexpr (BIAS) {
                // (zero for a panel past the wavefront's last and for absent tokens)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    plo = act_dot2_ones<ACT>(xf[s].x, plo);
                    plo = act_dot2_ones<ACT>(xf[s].z, plo);
                    phi = act_dot2_ones<ACT>(xf[s].y, phi);
                    phi = act_dot2_ones<ACT>(xf[s].w, phi);
                }
            }
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const uint32_t w0 = wv[j].x, w1 = wv[j].y, w2 = wv[j].z, w3 = wv[j].w;
                const uint32_t ws[4] = {w0, w1, w2, w3};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    u32x4 bq;
                    if constexpr (CBK == CBK_LIBRARY)
                        bq = cb_lookup<1>(ws[s], ptab + tl[j]);
                    else if constexpr (CBK)
                        bq = cb_lookup(ws[s], ptab + j * 256 * PANEL_N + (l & 15));
                    else if constexpr (BIAS)
                        bq = ACT == ACT_F16 ? dequant_f16_biased(ws[s]) : bf16_biased(ws[s]);
                    else if constexpr (ACT == ACT_F16)
                        bq = dequant_f16(ws[s], dqh[j]);
                    else
                        bq = dequant_bf16(ws[s], dqb[j]);
                    accg[j] = mfma16x16x32<ACT>(xf[s], bq, accg[j]);
                }
            }
            if constexpr (GROUPED) {
                if (--left_in_group == 0)
                    left_in_group = ppg;
            }
        }
    };
    int i0 = 0;
    for (; i0 + DEPTH < kcnt; i0 += DEPTH)
        chunk(i0, std::true_type{});
    chunk(i0, std::false_type{});
    flush();

    // sparse outlier residual: this thread's share of column rc, for every
    // token, sum x[m][k] * val (X from LDS while it is still staged there)
    // into rpart[rsub][m][rc] past the pair tables; the prefetched batch,
    // then any further ones.  Added to the outputs in the final reduction,
    // in a fixed order.
    float* rpart = reinterpret_cast<float*>(ptab + (CBK == CBK_LIBRARY ? CBK_LIB_MAX * 256 + 256 : CB * 256 * PANEL_N));
    if constexpr (CBK) {
        auto add_batch = [&](const int* kk, const uint32_t* vb, int eb, bool first) {
            int k[RB];
            float v[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const bool ok = eb + RS * i < rb1;
                k[i] = ok ? min(max(kk[i], 0), K - 1) : 0;
                v[i] = ok ? (float)__builtin_bit_cast(_Float16, (uint16_t)vb[i]) : 0.0f;
            }
            for (int m = 0; m < M; ++m) {
                float sum = first ? 0.0f : rpart[(rsub * M + m) * CBN + rc];
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    const uint16_t xb = XLDS ? xs[(size_t)m * K + k[i]] : a.X[(size_t)m * K + k[i]];
                    sum += act_to_f32<ACT>(xb) * v[i];
                }
                rpart[(rsub * M + m) * CBN + rc] = sum;
            }
        };
        add_batch(rk, rv, rb0 + rsub, true);
        for (int eb = rb0 + rsub + RS * RB; eb < rb1; eb += RS * RB) {
            int kk[RB];
            uint32_t vb[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const int e = min(eb + RS * i, a.nnz - 1);
                kk[i] = a.col_idx[e];
                vb[i] = a.val[e];
            }
            add_batch(kk, vb, eb, false);
        }
    }

    // park B in LDS ([CB][r_pad][16] halves, past the staged activations and
    // the reduction buffer; read after the barrier below)
    uint16_t* bl = reinterpret_cast<uint16_t*>(smem + main_b_offset(M, K, XLDS, CB));
    if (a.r > 0) {
#pragma unroll
        for (int i = 0; i < 2 * CB; ++i) {
            const int ch = tid + DEC_THREADS * i;
            if (ch < CB * a.r_pad * 2)
                st16(bl + (size_t)ch * 8, bstage[i]);
        }
    }

    // ---- reduce the four K shares (fixed order); LDS is reused from here on.
    // The barrier also tells whether some lane of the workgroup saw a
    // fractional zero point.
    bool anyfrac = false;
    if constexpr (CBK || BIAS)
        __syncthreads();
    else
        anyfrac = __syncthreads_or(fz) != 0;
    floatx4* red = reinterpret_cast<floatx4*>(smem);                       // [4][CB][64]
#pragma unroll
    for (int j = 0; j < CB; ++j)
        red[(w * CB + j) * 64 + l] = acc[j];

    // Fractional zero points (a slower path, taken once the partial sums are
    // parked and few registers are live): each token's activation sums over
    // 128-k chunks, xck[m][kb] (from global memory: the staged copy is being
    // overwritten), then for this workgroup's columns the correction
    // corr[m][c] = sum_g s_g (z_g - floor z_g) sum_{k in g} x[m][k], groups and
    // chunks added in order; the epilogue subtracts it (zero without a
    // fractional zero point).
    float* xck = reinterpret_cast<float*>(smem + main_frac_offset(M, K, XLDS, CB, a.r_pad,
                                                                  a.r > 0, a.r > 0 && a.S != nullptr));
    float* corr = xck + M * KB;                                            // [M][CB x 16]
    if (anyfrac) {
#pragma unroll 1
        for (int e = tid; e < M * KB; e += DEC_THREADS) {
            const int m = e / KB, kb = e - m * KB;
            const uint16_t* src = a.X + (size_t)m * K + kb * PANEL_K;
            float t = 0.0f;
#pragma unroll 1
            for (int c = 0; c < PANEL_K; c += 8) {
                const u32x4 v = ld16(src + c);
                const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    t += act_to_f32<ACT>((uint16_t)(u[i] & 0xFFFF));
                    t += act_to_f32<ACT>((uint16_t)(u[i] >> 16));
                }
            }
            xck[e] = t;
        }
        __syncthreads();                                    // uniform: anyfrac is the workgroup's
        const int cpg = a.G / PANEL_K;                       // chunks per group
#pragma unroll 1
        for (int e = tid; e < M * CB * PANEL_N; e += DEC_THREADS) {
            const int m = e / (CB * PANEL_N), c = e - m * (CB * PANEL_N);
            const int nc = min(cb0 * PANEL_N + c, a.Npad - 1);
            float t = 0.0f;
#pragma unroll 1
            for (int g = 0; g < K / a.G; ++g) {
                const uint32_t v = a.sz[(size_t)g * a.Npad + nc];
                const float sg = (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFF));
                const float zg = (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
                float xsum = 0.0f;
#pragma unroll 1
                for (int q = 0; q < cpg; ++q)
                    xsum += xck[m * KB + g * cpg + q];
                t += sg * (zg - floorf(zg)) * xsum;
            }
            corr[e] = t;
        }
    } else if constexpr (!CBK && !BIAS) {
        for (int e = tid; e < M * CB * PANEL_N; e += DEC_THREADS)
            corr[e] = 0.0f;
    }

    // ---- gated rank-r activations from this workgroup's replica slot, in
    // the MFMA A-operand layout (row = token l & 15, ranks 32 rs + koff + t),
    // taken as soon as every word has landed; a wavefront with an epilogue
    // waits for them while the others are done
    const int slot = mb % DEC_NREP;
    uint64_t* sdata = reinterpret_cast<uint64_t*>(a.rep_data + (size_t)slot * DEC_REP_DATA_STRIDE);
    u32x4 af[8];
    bool lost = false;      // this wavefront's wait for T_g gave up: its outputs are NaN
    uint32_t sticky = 0;    // a wait gave up in an earlier call on this workspace: NaN too
    // salient channels (SERQ summary, section 2): the operand is the gather
    // X[token][S[j]], made by the whole workgroup into LDS ([M][r_pad], past
    // the parked B) -- no EC role and no hand-over.  An index outside [0, K)
    // is clamped and raises flags[3].
    if (a.r > 0 && a.S && !lds_gather) {
        bool bad = false;
#pragma unroll 4
        for (int e = tid; e < M * a.r_pad; e += DEC_THREADS) {
            const int m = e / a.r_pad, j = e - m * a.r_pad;
            uint16_t v = 0;
            if (j < a.r) {
                int idx = a.S[j];
                bad |= idx < 0 || idx >= K;
                idx = min(max(idx, 0), K - 1);
                v = a.X[(size_t)m * K + idx];
            }
            tgl[e] = v;
        }
        if (bad)
            atomic_store_dev(&a.flags[3], 1u);
    } else if (a.r > 0 && w < CB && !a.S) {
        const uint64_t* src = sdata + (row * a.r_pad + koff) / 4;
        uint32_t it = 0;
        sticky = atomic_load_dev(&a.flags[2]);            // alongside the first poll
        lost = a.spin == 0;
        // read all of them, and again while any has not landed (a wait limit
        // of 0 gives up at once)
        for (; !lost;) {
            bool miss = false;
#pragma unroll
            for (int rs = 0; rs < 8; ++rs) {
                if (rs < nsteps) {
                    uint64_t lo = 0, hi = 0;
                    if (xrow) {
                        lo = ld8_dev(src + 8 * rs);
                        hi = ld8_dev(src + 8 * rs + 1);
                        miss |= (hw_missing16(lo) | hw_missing16(hi)) != 0;
                        lo = ~lo;
                        hi = ~hi;
                    }
                    af[rs] = (u32x4){(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
                }
            }
            if (__builtin_amdgcn_ballot_w64(miss) == 0)
                break;
            if (it >= a.spin) {
                lost = true;
                break;
            }
            ++it;
            __builtin_amdgcn_s_sleep(1);
        }
        if (lost && l == 0)
            atomic_store_dev(&a.flags[2], 1u);
    }
    __syncthreads();
    if (a.r > 0 && a.S && w < CB) {
#pragma unroll
        for (int rs = 0; rs < 8; ++rs)
            if (rs < nsteps)
                af[rs] = xrow ? *reinterpret_cast<const u32x4*>(tgl + (size_t)row * a.r_pad + 32 * rs + koff)
                              : (u32x4){0u, 0u, 0u, 0u};
    }

#pragma unroll
    for (int j = 0; j < CB; ++j) {
        if ((j & 3) != w)
            continue;
        floatx4 tot = red[(0 * CB + j) * 64 + l];
        tot += red[(1 * CB + j) * 64 + l];
        tot += red[(2 * CB + j) * 64 + l];
        tot += red[(3 * CB + j) * 64 + l];
        const int n = n_l[j];

        if constexpr (CBK) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = 4 * (l >> 4) + v;
                if (m < M) {
                    float rs = 0.0f;
#pragma unroll
                    for (int u = 0; u < RS; ++u)
                        rs += rpart[(u * M + m) * CBN + j * PANEL_N + (l & 15)];
                    tot[v] += rs;
                }
            }
        }
        if (a.r > 0) {
            const uint16_t* bj = bl + (size_t)j * a.r_pad * PANEL_N;
            u32x4 bfr[8];
#pragma unroll
            for (int rs = 0; rs < 8; ++rs)
                if (rs < nsteps)
                    bfr[rs] = lds_bfrag(bj, PANEL_N, 0, 32 * rs);
#pragma unroll
            for (int rs = 0; rs < 8; ++rs)
                if (rs < nsteps)
                    tot = mfma16x16x32<ACT>(af[rs], bfr[rs], tot);
        }
        if constexpr (!CBK && !BIAS) {
            // fractional zero points (zero otherwise: read unconditionally,
            // so that the compiler keeps one copy of this loop)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                tot[v] -= corr[min(4 * (l >> 4) + v, M - 1) * (CB * PANEL_N) + j * PANEL_N + (l & 15)];
        }
        if (n < a.N) {
            // a wait that gave up here, or one that did in an earlier call on
            // this workspace (whose hand-over state is then not to be
            // trusted), turns the outputs into NaN rather than wrong numbers
            const bool poison = lost || sticky != 0u;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = 4 * (l >> 4) + v;
                if (m < M)
                    a.Y[(size_t)m * a.N + n] = poison ? act_nan<ACT>() : f32_to_act<ACT>(tot[v]);
            }
        }
    }

    // The last reader of a slot returns the slot, and its share of the EC
    // partial sums (whose reduction finished before any slot was written),
    // to zero for the next call.
    if (a.r > 0 && !a.S) {
        __shared__ int s_last;
        if (tid == 0) {
            const int readers = a.n_main / DEC_NREP + (slot < a.n_main % DEC_NREP ? 1 : 0);
            s_last = atomic_add_dev(rep_word(a, slot, 1), 1u) == (uint32_t)(readers - 1);
        }
        __syncthreads();
        if (s_last) {
            if (tid == 0)
                atomic_store_dev(rep_word(a, slot, 1), 0u);
            const int n8 = M * a.r_pad / 4;
            for (int i = tid; i < n8; i += DEC_THREADS)
                st8_dev(sdata + i, 0ull);
            const int nrep = min(DEC_NREP, a.n_main);
            const int np = a.P * M * a.RC;
            for (int i = slot * DEC_THREADS + tid; i < np; i += nrep * DEC_THREADS)
                atomic_store_dev(a.partial + i, 0u);
        }
    }
}

// Two column blocks per workgroup (activations staged in LDS): the grid
// holds ~450 workgroups, which fit the CUs in one round at two wavefronts
// per SIMD, i.e. within 256 registers.
template <int ACT, int CB, int XCH, int DEPTH, bool GROUPED, bool STAGE_FIRST, int CBK = CBK_NONE>
__global__ __launch_bounds__(DEC_THREADS, 2)
void decode_kernel(DecodeKArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t dsmem[];
    if constexpr (CBK) {
        decode_main_role<ACT, CB, XCH, DEPTH, false, false, CBK>(a, dsmem);   // no EC role
    } else {
        if ((int)blockIdx.x < a.P)
            decode_ec_role<ACT>(a, dsmem);
        else
            decode_main_role<ACT, CB, XCH, DEPTH, GROUPED, STAGE_FIRST>(a, dsmem);
    }
}


static size_t main_lds_bytes(const DecodePlan& p, int M, int K, int r, bool gather)
{
    // past the other regions: the fractional-zero-point sums and correction,
    // or (offset codes) the transposition areas of the four wavefronts
    return main_frac_offset(M, K, p.xlds, p.CB, p.r_pad, r > 0, r > 0 && gather) +
           std::max((size_t)M * (K / PANEL_K + p.CB * PANEL_N) * sizeof(float), (size_t)4 * 128 * sizeof(float));
}

// LDS of the EC role: the staged slice and gate vector, then the final reduction
static size_t ec_lds_bytes(const DecodePlan& p, int M, int r)
{
    if (p.P == 0)
        return 0;
    const size_t at = (size_t)ec_slice_bytes(r, p.KS) + (size_t)p.KS * 2;
    // the reduction's share: [ng][ne] sums (<= 256 floats, or none), [ne] totals, [nw] words
    const int nred = dec_scalar_reducers(p.P, M, p.r_pad);
    const int share = (M * p.r_pad / 4 + nred - 1) / nred;
    const size_t fin = ((size_t)DEC_THREADS + 4 * share + M + 2) * 4 + (size_t)share * 8;
    // vector gate: [r_pad] T, [r_pad] gated T, [VG_HMAX] bottleneck,
    // [VG_THREADS] partial sums, [r_pad / 4] words, then (when they fit in
    // what the slice needs anyway) the gate parameters
    const size_t vg = ((size_t)2 * p.r_pad + VG_HMAX + VG_THREADS) * 4 + (size_t)p.r_pad / 4 * 8;
    return (std::max(at, std::max(fin, vg)) + 15) / 16 * 16;
}

template <int ACT, int CB, int XCH, int DEPTH, bool GROUPED, bool STAGE_FIRST, int CBK = CBK_NONE>
static hipError_t launch_decode_t(const DecodeKArgs& k, const DecodePlan& p, hipStream_t st)
{
    auto kern = decode_kernel<ACT, CB, XCH, DEPTH, GROUPED, STAGE_FIRST, CBK>;
    // codebook tables (per channel [CB][256][16], or the library's
    // [CBK_LIB_MAX][256] and the staged library) and the residual's sums
    const size_t tables = CBK == CBK_LIBRARY ? (size_t)CBK_LIB_MAX * 256 * 4 + 1024 : (size_t)CB * PANEL_N * 256 * 4;
    const size_t lds = std::max(main_lds_bytes(p, k.M, k.K, k.r, k.S != nullptr) + (CBK ? tables + (size_t)DEC_THREADS * k.M * 4 : 0),
                                ec_lds_bytes(p, k.M, k.r));
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(kern, dim3(k.P + k.n_main), dim3(DEC_THREADS), lds, st, k);
    return hipGetLastError();
}

template <int ACT, bool GROUPED, bool STAGE_FIRST>
static hipError_t launch_decode_grp(const DecodeKArgs& k, const DecodePlan& p, hipStream_t st)
{
    if (p.xlds) {
        // two column blocks: each workgroup stages X once for twice the
        // weights.  With one block, a token at 4096 k staged 8 KB of X from
        // L2 per 32 KB of weights, and the call measured 0.3-0.4 us slower.
        const size_t xch = ((size_t)k.M * k.K / 8 + DEC_THREADS - 1) / DEC_THREADS;
        if (xch <= 2)
            return launch_decode_t<ACT, 2, 2, 8, GROUPED, STAGE_FIRST>(k, p, st);
        return launch_decode_t<ACT, 2, DEC_XLDS_CHUNKS, 8, GROUPED, STAGE_FIRST>(k, p, st);
    }
    if (p.CB == 2)
        return launch_decode_t<ACT, 2, 0, 4, GROUPED, false>(k, p, st);
    if (p.CB == 1)
        return launch_decode_t<ACT, 1, 0, 4, GROUPED, false>(k, p, st);
    // four column blocks: a ring of two steps keeps the registers at two waves per SIMD
    return launch_decode_t<ACT, 4, 0, 2, GROUPED, false>(k, p, st);
}

template <int ACT>
static hipError_t launch_decode_act(const DecodeKArgs& k, const DecodePlan& p, hipStream_t st)
{
    // (the plan always issues the weight ring before staging X)
    if (k.G != k.K)
        return launch_decode_grp<ACT, true, false>(k, p, st);
    return launch_decode_grp<ACT, false, false>(k, p, st);
}

template <int ACT, int MODE>
static hipError_t launch_decode_xfp_act(const DecodeKArgs& k, const DecodePlan& p, hipStream_t st)
{
    if (p.xlds) {
        const size_t xch = ((size_t)k.M * k.K / 8 + DEC_THREADS - 1) / DEC_THREADS;
        if (xch <= 2)
            return launch_decode_t<ACT, 2, 2, 8, false, false, MODE>(k, p, st);
        return launch_decode_t<ACT, 2, DEC_XLDS_CHUNKS, 8, false, false, MODE>(k, p, st);
    }
    if (p.CB == 1)
        return launch_decode_t<ACT, 1, 0, 4, false, false, MODE>(k, p, st);
    if (p.CB == 2)
        return launch_decode_t<ACT, 2, 0, 4, false, false, MODE>(k, p, st);
    if constexpr (MODE == CBK_LIBRARY) {
        // the panels' entry ids take the registers of two more column blocks:
        // two blocks per workgroup, a ring of four steps
        DecodePlan q = p;
        q.CB = 2;
        q.n_main = (k.NB + 1) / 2;
        DecodeKArgs kq = k;
        kq.n_main = q.n_main;
        return launch_decode_t<ACT, 2, 0, 4, false, false, MODE>(kq, q, st);
    } else {
        return launch_decode_t<ACT, 4, 0, 2, false, false, MODE>(k, p, st);
    }
}

// Codebook weights with a sparse outlier residual: the main role alone (no
// EC), the codebook lookup in place of the affine dequantization.
hipError_t launch_decode_xfp(const XfpArgs& x, const DecodePlan& p, hipStream_t st)
{
    BlobGeom g = blob_geom(x.N, x.K, x.K);
    DecodeKArgs k{};
    k.X = (const uint16_t*)x.X;
    k.codes = (const uint8_t*)x.packed + g.codes_off;
    k.sz = (const uint32_t*)((const char*)x.packed + g.sz_off);
    k.Y = (uint16_t*)x.Y;
    k.M = x.M; k.N = x.N; k.K = x.K; k.r = 0; k.r_pad = 0; k.G = x.K;
    k.NB = g.NB; k.KB = g.KB; k.Npad = g.Npad;
    k.P = 0; k.KS = 0; k.RC = 1; k.n_main = p.n_main;
    k.stage_first = 0;
    k.cb = x.cb; k.row_ptr = x.row_ptr; k.col_idx = x.col_idx; k.val = x.val; k.nnz = x.nnz;
    k.libid = x.libid; k.L = x.L;
    if (x.nnz == 0) {
        // the kernel loads entry 0 unconditionally (and discards it): point
        // the empty arrays at the row pointers, which always exist
        k.col_idx = x.row_ptr;
        k.val = reinterpret_cast<const uint16_t*>(x.row_ptr);
    }
    if (x.libid) {
        if (x.act == ACT_F16)
            return launch_decode_xfp_act<ACT_F16, CBK_LIBRARY>(k, p, st);
        return launch_decode_xfp_act<ACT_BF16, CBK_LIBRARY>(k, p, st);
    }
    if (x.act == ACT_F16)
        return launch_decode_xfp_act<ACT_F16, CBK_CHANNEL>(k, p, st);
    return launch_decode_xfp_act<ACT_BF16, CBK_CHANNEL>(k, p, st);
}

hipError_t launch_decode(const LayerArgs& a, const DecodePlan& p, hipStream_t st)
{
    BlobGeom g = blob_geom(a.N, a.K, a.G);
    DecodeKArgs k;
    k.X = (const uint16_t*)a.X;
    k.codes = (const uint8_t*)a.packed + g.codes_off;
    k.sz = (const uint32_t*)((const char*)a.packed + g.sz_off);
    k.A = (const uint16_t*)a.A;
    k.B = (const uint16_t*)a.B;
    k.w_g = (const uint16_t*)a.w_g;
    k.b_g = a.b_g;
    k.Y = (uint16_t*)a.Y;
    k.M = a.M; k.N = a.N; k.K = a.K; k.r = a.r; k.r_pad = p.r_pad; k.G = a.G;
    k.NB = g.NB; k.KB = g.KB; k.Npad = g.Npad;
    k.P = p.P; k.KS = p.KS; k.RC = p.RC; k.n_main = p.n_main;
    k.stage_first = p.stage_first;
    k.flags = (uint32_t*)(a.ws + p.off_flags);
    k.spin = a.spin;
    k.partial = (uint32_t*)(a.ws + p.off_partial);
    k.rep_ctrl = (uint8_t*)(a.ws + p.off_rep_ctrl);
    k.rep_data = (uint8_t*)(a.ws + p.off_rep_data);
    k.G1 = (const uint16_t*)a.G1; k.c1 = (const uint16_t*)a.c1;
    k.G2 = (const uint16_t*)a.G2; k.c2 = (const uint16_t*)a.c2;
    k.h = a.r > 0 ? a.h : 0;
    k.vg_staged = 0;
    k.S = a.S;
    if (k.h > 0) {
        // stage the gate parameters when they fit in the EC role's LDS
        const size_t base = ((size_t)2 * p.r_pad + VG_HMAX + VG_THREADS) * 4 + (size_t)p.r_pad / 4 * 8;
        k.vg_staged = vgate_stageable(a.r, a.h) &&
                      base + (size_t)vgate_stage_elems(a.r, a.h) * 2 <= ec_lds_bytes(p, a.M, a.r);
    }
    if (a.act == ACT_F16)
        return launch_decode_act<ACT_F16>(k, p, st);
    return launch_decode_act<ACT_BF16>(k, p, st);
}


// ---------------------------------------------------------------- no-allocation state
//
// The decode hand-over state of w4ec_linear_decode_noalloc: a static device
// array, one copy per GPU, held until the process ends.  On the host the
// array's name is a stand-in, never a device address, so it is not passed
// to any kernel: the first call on a device, with that device current, takes
// the address with hipGetSymbolAddress, clears the array with a fill kernel
// on the caller's stream (capturable: no memset node), and keeps the address
// for every later call on that device.  Calls that overlap in time on one
// device share the array and race.
static __device__ __align__(256) uint8_t scratch[W4EC_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES];
}  // namespace

hipError_t noalloc_scratch(void** out, hipStream_t st)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!ptr)
            return hipErrorInvalidSymbol;
        e = launch_zero_fill(ptr, W4EC_NOALLOC_SCRATCH_BYTES, st);
        if (e != hipSuccess)
            return e;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace w4ec
