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
#include <type_traits>

#include "ec_tile.h"
#include "w4ec_common.h"
#include "w4ec_launch.h"

namespace w4ec {

constexpr int DEC_THREADS = 256;
constexpr int DEC_EC_MAXI = 5;     // column blocks per wavefront in the EC role (17 / 4)
constexpr int DEC_XLDS_CHUNKS = 8; // 16-byte chunks of staged activations per thread
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
    uint32_t* flags;     // [0] EC arrivals, [2] a wait timed out
    float* partial;      // [P][16][RC]
    uint8_t* rep_ctrl;   // DEC_NREP slots of DEC_REP_CTRL_STRIDE bytes: [0] ready, [1] readers done
    uint8_t* rep_data;   // DEC_NREP slots of rep_data_stride bytes
    size_t rep_data_stride;
};

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

template <int ACT>
__device__ void decode_ec_role(const DecodeKArgs& a, uint8_t* smem)
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
    const int nrep = min(DEC_NREP, a.n_main);       // slots that have readers

    // partial sums -> [P][16][RC]; the last EC workgroup reduces them
    float* part = a.partial + (size_t)p * 16 * a.RC;
#pragma unroll
    for (int i = 0; i < DEC_EC_MAXI; ++i) {
        const int cb = w + 4 * i;
        const int c = cb < ec_blocks(r) ? ec_col(r, cb, l & 15) : -1;
        if (c >= 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = 4 * (l >> 4) + v;
                if (m < M)
                    st4_dev(part + m * a.RC + c, acc[i][v]);
            }
        }
    }
    wait_all_mem();
    __syncthreads();
    __shared__ uint32_t s_old;
    if (tid == 0)
        s_old = atomic_add_dev(&a.flags[0], 1u);
    __syncthreads();
    if (s_old != (uint32_t)(a.P - 1))
        return;
    if (tid == 0)
        atomic_store_dev(&a.flags[0], 0u);
    float* red = reinterpret_cast<float*>(smem);            // [ng][ne] (ng > 1 only: <= 256 floats)
    float* tsum = red + DEC_THREADS;                        // [M][RC]
    float* gl = tsum + 16 * a.RC;                           // [16]
    uint16_t* tg = reinterpret_cast<uint16_t*>(gl + 16);    // [M][r_pad]
    const int ne = M * a.RC;
    // ng thread groups split the P slices (slice q -> group q mod ng); each
    // thread keeps 8 loads in flight, and the groups' sums are added in
    // group order, so the result does not depend on timing
    const int ng = max(1, min(a.P, DEC_THREADS / ne));
    const size_t qs = (size_t)16 * a.RC;
    for (int e0 = tid; e0 < ne * ng; e0 += DEC_THREADS) {
        const int g = e0 / ne, e = e0 - g * ne;
        const float* src = a.partial + e;
        float t = 0.0f;
        int q = g;
        for (; q + 7 * ng < a.P; q += 8 * ng) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = ld4_dev(src + (size_t)(q + i * ng) * qs);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                t += v[i];
        }
        for (; q < a.P; q += ng)
            t += ld4_dev(src + (size_t)q * qs);
        if (ng > 1)
            red[e0] = t;
        else
            tsum[e] = t;
    }
    if (ng > 1) {
        __syncthreads();
        for (int e = tid; e < ne; e += DEC_THREADS) {
            float t = red[e];
            for (int g = 1; g < ng; ++g)
                t += red[g * ne + e];
            tsum[e] = t;
        }
    }
    __syncthreads();
    if (tid < M)
        gl[tid] = sigmoid_f32(tsum[tid * a.RC + r] + a.b_g);
    __syncthreads();
    const int nt = M * a.r_pad;
    for (int e = tid; e < nt; e += DEC_THREADS) {
        const int m = e / a.r_pad, c = e - m * a.r_pad;
        tg[e] = f32_to_act<ACT>(c < r ? gl[m] * tsum[m * a.RC + c] : 0.0f);
    }
    __syncthreads();
    const int n8 = nt / 4;                                  // 8-byte words of T_g
    const uint64_t* tg8 = reinterpret_cast<const uint64_t*>(tg);
    const int sstep = n8 <= DEC_THREADS ? DEC_THREADS / n8 : 1;   // thread -> (word, slots s0 + j sstep)
    const int s0 = n8 <= DEC_THREADS ? tid / n8 : 0;
    if (s0 < sstep) {
        for (int i = tid - s0 * n8; i < n8; i += DEC_THREADS) {
            const uint64_t v = tg8[i];
            for (int slot = s0; slot < nrep; slot += sstep) {
                uint64_t* dst = reinterpret_cast<uint64_t*>(a.rep_data + (size_t)slot * a.rep_data_stride);
                __hip_atomic_store(dst + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    wait_all_mem();
    __syncthreads();
    if (tid < nrep)
        atomic_store_dev(rep_word(a, tid, 0), 1u);
}

template <int ACT, int CB, int XCH, int DEPTH, bool GROUPED, bool STAGE_FIRST>
__device__ void decode_main_role(const DecodeKArgs& a, uint8_t* smem)
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

    // Loads retire in issue order, so everything consumed before the first
    // panel (scale/zero, the activations staged in LDS) is issued first;
    // then a ring of DEPTH weight panels, consumed one by one as they arrive
    // and refilled unconditionally (indices clamped to the wavefront's last
    // panel, extra panels multiplied by zero) so that the ring's waits stay
    // exact.  With an EC to wait for, the activations are staged completely
    // before the first weight load, which lets the EC workgroups' loads reach
    // memory ahead of the weight stream.
    // (Every load below is issued unconditionally -- indices are clamped and
    // unwanted values zeroed afterwards -- so that the compiler can count the
    // loads in flight and wait for exactly the one it needs.)
    constexpr bool XLDS = XCH > 0;
    u32x4 wring[DEPTH][CB];
    u32x4 xring[XLDS ? 1 : DEPTH][4];
    uint32_t szring[GROUPED ? DEPTH : 1][CB];
    uint32_t sz0[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j)
        sz0[j] = *szp[j];
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
    const int nxchunks = XLDS ? M * K / 8 : 1;       // 16-byte chunks of X (XCH per thread suffice)
    u32x4 xstage[XLDS ? XCH : 1];
    const uint16_t* xg = a.X + (size_t)(xrow ? row : 0) * K + (size_t)kbeg * PANEL_K + koff;
    auto issue = [&](int u, int i) {                 // panel i (clamped) into ring slot u
        const int ic = min(i, klast);
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
    if constexpr (XLDS && STAGE_FIRST)
        store_x();
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
        issue(u, u);
        __builtin_amdgcn_sched_barrier(0);   // slot u is issued u-th
    }
    if constexpr (XLDS && !STAGE_FIRST)
        store_x();

    floatx4 acc[CB], accg[CB];
    float s_cur[CB];
    DqF16 dqh[CB];
    float dqb[CB];
    auto set_sz = [&](const uint32_t* v) {
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            s_cur[j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[j] & 0xFFFF));
            const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[j] >> 16));
            if constexpr (ACT == ACT_F16)
                dqh[j] = dq_f16_consts(z);
            else
                dqb[j] = -(8388608.0f + z);
        }
    };
#pragma unroll
    for (int j = 0; j < CB; ++j) {
        acc[j] = (floatx4){0.f, 0.f, 0.f, 0.f};
        accg[j] = acc[j];
    }
    set_sz(sz0);
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
#pragma unroll
                    for (int j = 0; j < CB; ++j) {
                        acc[j] += s_cur[j] * accg[j];
                        accg[j] = (floatx4){0.f, 0.f, 0.f, 0.f};
                    }
                    set_sz(szv);
                }
            }
#pragma unroll
            for (int j = 0; j < CB; ++j) {
                const uint32_t w0 = wv[j].x, w1 = wv[j].y, w2 = wv[j].z, w3 = wv[j].w;
                const uint32_t ws[4] = {w0, w1, w2, w3};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    u32x4 bq;
                    if constexpr (ACT == ACT_F16)
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

#pragma unroll
    for (int j = 0; j < CB; ++j)
        acc[j] += s_cur[j] * accg[j];

    // B fragments for the epilogue (rank rows 32 rs + koff + t, column n),
    // issued now so that they arrive during the reductions below
    u32x4 bfr[CB][8];
    if (a.r > 0) {
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            if ((j & 3) != w)
                continue;
#pragma unroll
            for (int rs = 0; rs < 8; ++rs) {
                if (rs < nsteps) {
                    uint32_t hv[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const int jr = 32 * rs + koff + t;
                        hv[t] = (jr < a.r && n_l[j] < a.N) ? (uint32_t)a.B[(size_t)jr * a.N + n_l[j]] : 0u;
                    }
                    bfr[j][rs] = (u32x4){hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16),
                                         hv[4] | (hv[5] << 16), hv[6] | (hv[7] << 16)};
                }
            }
        }
    }

    // ---- reduce the four K shares (fixed order); LDS is reused from here on
    __syncthreads();
    floatx4* red = reinterpret_cast<floatx4*>(smem);                       // [4][CB][64]
#pragma unroll
    for (int j = 0; j < CB; ++j)
        red[(w * CB + j) * 64 + l] = acc[j];

    // ---- gated rank-r activations from this workgroup's replica slot
    const int slot = mb % DEC_NREP;
    const uint8_t* sdata = a.rep_data + (size_t)slot * a.rep_data_stride;
    if (a.r > 0 && tid == 0) {
        uint32_t it = 0;
        while (atomic_load_dev(rep_word(a, slot, 0)) == 0u) {
            __builtin_amdgcn_s_sleep(2);
            if (++it >= SPIN_LIMIT) {
                atomic_store_dev(&a.flags[2], 1u);
                break;
            }
        }
    }
    __syncthreads();

#pragma unroll
    for (int j = 0; j < CB; ++j) {
        if ((j & 3) != w)
            continue;
        floatx4 tot = red[(0 * CB + j) * 64 + l];
        tot += red[(1 * CB + j) * 64 + l];
        tot += red[(2 * CB + j) * 64 + l];
        tot += red[(3 * CB + j) * 64 + l];
        const int n = n_l[j];
        if (a.r > 0) {
#pragma unroll
            for (int rs = 0; rs < 8; ++rs) {
                if (rs < nsteps) {
                    u32x4 af = (u32x4){0u, 0u, 0u, 0u};
                    if (xrow) {
                        const uint64_t* src = reinterpret_cast<const uint64_t*>(
                            sdata + ((size_t)row * a.r_pad + 32 * rs + koff) * 2);
                        const uint64_t lo = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        const uint64_t hi = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        af = (u32x4){(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
                    }
                    tot = mfma16x16x32<ACT>(af, bfr[j][rs], tot);
                }
            }
        }
        if (n < a.N) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = 4 * (l >> 4) + v;
                if (m < M)
                    a.Y[(size_t)m * a.N + n] = f32_to_act<ACT>(tot[v]);
            }
        }
    }

    // the last reader of a slot clears it for the next call
    if (a.r > 0) {
        __syncthreads();
        if (tid == 0) {
            const int readers = a.n_main / DEC_NREP + (slot < a.n_main % DEC_NREP ? 1 : 0);
            const uint32_t old = atomic_add_dev(rep_word(a, slot, 1), 1u);
            if (old == (uint32_t)(readers - 1)) {
                atomic_store_dev(rep_word(a, slot, 0), 0u);
                atomic_store_dev(rep_word(a, slot, 1), 0u);
            }
        }
    }
}

template <int ACT, int CB, int XCH, int DEPTH, bool GROUPED, bool STAGE_FIRST>
__global__ __launch_bounds__(DEC_THREADS)
void decode_kernel(DecodeKArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t dsmem[];
    if ((int)blockIdx.x < a.P)
        decode_ec_role<ACT>(a, dsmem);
    else
        decode_main_role<ACT, CB, XCH, DEPTH, GROUPED, STAGE_FIRST>(a, dsmem);
}

// activations of at most this many bytes are staged in LDS by the main role
// (8 chunks of 16 bytes per thread)
constexpr size_t DEC_XLDS_MAX_BYTES = (size_t)DEC_XLDS_CHUNKS * 16 * DEC_THREADS;

bool decode_use_xlds(int M, int K) { return M <= 4 && (size_t)M * K * 2 <= DEC_XLDS_MAX_BYTES; }

// LDS of the main role: the staged activations, then (after the stream)
// the wavefront reduction
static size_t main_lds_bytes(const DecodePlan& p, int M, int K, int r)
{
    size_t b = (size_t)4 * p.CB * 64 * 16;
    if (p.xlds)
        b = std::max(b, (size_t)M * K * 2);
    return (b + 15) / 16 * 16;
}

// LDS of the EC role: the staged slice and gate vector, then the final reduction
static size_t ec_lds_bytes(const DecodePlan& p, int r)
{
    if (p.P == 0)
        return 0;
    const size_t at = (size_t)ec_slice_bytes(r, p.KS) + (size_t)p.KS * 2;
    const size_t fin = (size_t)DEC_THREADS * 4 + (size_t)16 * (r + 1) * 4 + 64 + (size_t)16 * p.r_pad * 2;
    return (std::max(at, fin) + 15) / 16 * 16;
}

template <int ACT, int CB, int XCH, int DEPTH, bool GROUPED, bool STAGE_FIRST>
static hipError_t launch_decode_t(const DecodeKArgs& k, const DecodePlan& p, hipStream_t st)
{
    auto kern = decode_kernel<ACT, CB, XCH, DEPTH, GROUPED, STAGE_FIRST>;
    const size_t lds = std::max(main_lds_bytes(p, k.M, k.K, k.r), ec_lds_bytes(p, k.r));
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
        const size_t xch = ((size_t)k.M * k.K / 8 + DEC_THREADS - 1) / DEC_THREADS;
        if (xch <= 2)
            return launch_decode_t<ACT, 1, 2, 8, GROUPED, STAGE_FIRST>(k, p, st);
        return launch_decode_t<ACT, 1, DEC_XLDS_CHUNKS, 8, GROUPED, STAGE_FIRST>(k, p, st);
    }
    if (p.CB == 1)
        return launch_decode_t<ACT, 1, 0, 4, GROUPED, false>(k, p, st);
    return launch_decode_t<ACT, 2, 0, 4, GROUPED, false>(k, p, st);
}

template <int ACT>
static hipError_t launch_decode_act(const DecodeKArgs& k, const DecodePlan& p, hipStream_t st)
{
    if (k.G != k.K)
        return p.stage_first ? launch_decode_grp<ACT, true, true>(k, p, st)
                             : launch_decode_grp<ACT, true, false>(k, p, st);
    return p.stage_first ? launch_decode_grp<ACT, false, true>(k, p, st)
                         : launch_decode_grp<ACT, false, false>(k, p, st);
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
    k.partial = (float*)(a.ws + p.off_partial);
    k.rep_ctrl = (uint8_t*)(a.ws + p.off_rep_ctrl);
    k.rep_data = (uint8_t*)(a.ws + p.off_rep_data);
    k.rep_data_stride = p.rep_data_stride;
    if (a.act == ACT_F16)
        return launch_decode_act<ACT_F16>(k, p, st);
    return launch_decode_act<ACT_BF16>(k, p, st);
}

}  // namespace w4ec
