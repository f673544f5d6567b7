// prefill.hip -- the W4 + EC layer for many tokens: a prepass for the gate
// and X A, then a tiled MFMA GEMM whose epilogue applies the gated rank-r
// correction.
//
// SPEAR (gist.science technical summary, section 2.2A) describes the
// prefill phase as compute bound.  The page runs the EC beside the GEMM in a
// separate kernel; this library instead folds the gated correction into the
// GEMM epilogue as r extra terms of the reduction (T_g B), and keeps the only
// part that needs a full pass over K -- the gate logit X . w_g and T = X A --
// in a prepass that reads X once for all r + 1 columns.
//
// GEMM tiling for gfx950 (wave64, 16x16x32 MFMA, 160 KB LDS per CU):
//  * workgroup tile BM x 256 (BM = 64 or 128 tokens), 4 wavefronts; wavefront
//    w owns columns [64 w, 64 w + 64) of the tile for all BM rows, so every
//    packed weight is loaded and dequantized exactly once per tile, straight
//    from HBM into registers (one 16-byte load per lane per 16 x 128 panel);
//  * the X tile (BM x 128 per step) is staged in LDS, double buffered, with
//    16-byte chunks XOR-swizzled by row so the MFMA A-operand reads are free
//    of bank conflicts; all four wavefronts read it;
//  * split-K when the tile count alone cannot fill the 256 CUs: partial fp32
//    tiles go to the workspace and the last-arriving workgroup of a tile adds
//    them in a fixed order, then runs the epilogue;
//  * tile ids are remapped so that the workgroups an XCD receives (block ids
//    congruent mod 8) share rows of X and columns of W in that XCD's L2.
#include "ec_tile.h"
#include "w4ec_common.h"
#include "w4ec_launch.h"

namespace w4ec {

constexpr int PF_THREADS = 256;
constexpr int PF_BN = 256;

// ---------------------------------------------------------------- prepass

struct PrepassKArgs {
    const uint16_t* X;
    const uint16_t* A;
    const uint16_t* w_g;
    float b_g;
    int M, K, r, r_pad, kc, ks;
    floatx4* partial;   // [mt][ks][4 wavefronts][17 column blocks][64 lanes]
    uint32_t* cnt;      // [mt]
    uint16_t* tg;       // [Mpad][r_pad], activation format
};

constexpr int PRE_MAXI = 17;   // (256 + 1 + 15) / 16 column blocks of [A | w_g]

// 64 tokens x one K slice per workgroup (wavefront w: tokens 16 w .. 16 w + 15).
// With a split over K, the last workgroup of a token tile adds the slices'
// fragments in a fixed order.  It then applies the gate and stores
// T_g = g * T in the activation format for the GEMM epilogue.
template <int ACT>
__global__ __launch_bounds__(PF_THREADS)
void prepass_kernel(PrepassKArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t at[EC_LDS_HALVES];
    __shared__ float gsh[64];
    __shared__ uint32_t s_old;
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = tid >> 6;
    const int mt = blockIdx.x;
    const int kz = blockIdx.y;
    const int m0 = mt * 64;
    const int kbeg = kz * a.kc;
    const int kend = min(a.K, kbeg + a.kc);
    const int xrow = min(m0 + 16 * w + (l & 15), a.M - 1);
    const int CBE = ec_col_blocks(a.r);

    floatx4 acc[PRE_MAXI];
    ec_tile<ACT, 1, PRE_MAXI, 8>(a.X, a.K, xrow, a.A, a.w_g, a.r, kbeg, kend, 0, at, acc);

    if (a.ks > 1) {
        floatx4* mine = a.partial + ((size_t)(mt * a.ks + kz) * 4 + w) * PRE_MAXI * 64;
#pragma unroll
        for (int i = 0; i < PRE_MAXI; ++i)
            if (i < CBE)
                st16_dev(mine + i * 64 + l, acc[i]);
        wait_all_mem();
        __syncthreads();
        if (tid == 0)
            s_old = atomic_add_dev(&a.cnt[mt], 1u);
        __syncthreads();
        if (s_old != (uint32_t)(a.ks - 1))
            return;
        if (tid == 0)
            atomic_store_dev(&a.cnt[mt], 0u);
#pragma unroll
        for (int i = 0; i < PRE_MAXI; ++i) {
            if (i < CBE) {
                floatx4 t = (floatx4){0.f, 0.f, 0.f, 0.f};
                for (int z = 0; z < a.ks; ++z)
                    t += (z == kz) ? acc[i]
                                   : ld16_dev(a.partial + ((size_t)(mt * a.ks + z) * 4 + w) * PRE_MAXI * 64 + i * 64 + l);
                acc[i] = t;
            }
        }
    }

    // gate: column r lives in block r / 16, lanes with (l & 15) == r % 16
    const int cg = a.r >> 4;
#pragma unroll
    for (int i = 0; i < PRE_MAXI; ++i) {
        if (i == cg && (l & 15) == (a.r & 15)) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                gsh[16 * w + 4 * (l >> 4) + v] = sigmoid_f32(acc[i][v] + a.b_g);
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PRE_MAXI; ++i) {
        const int c = i * 16 + (l & 15);
        if (i < CBE && c < a.r_pad) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int mloc = 16 * w + 4 * (l >> 4) + v;
                const float val = c < a.r ? gsh[mloc] * acc[i][v] : 0.0f;
                a.tg[(size_t)(m0 + mloc) * a.r_pad + c] = f32_to_act<ACT>(val);
            }
        }
    }
    const int c0 = CBE * 16;
    for (int e = tid; e < 64 * (a.r_pad - c0); e += PF_THREADS) {
        const int mloc = e / (a.r_pad - c0), c = c0 + e % (a.r_pad - c0);
        a.tg[(size_t)(m0 + mloc) * a.r_pad + c] = 0;
    }
}

// ---------------------------------------------------------------- GEMM

struct GemmKArgs {
    const uint16_t* X;
    const uint8_t* codes;
    const uint32_t* sz;
    const uint16_t* B;
    const uint16_t* tg;
    uint16_t* Y;
    floatx4* partial;  // [tile][ksplit][4][RB][4][64] fragments
    uint32_t* cnt;     // [mt*nt]
    int M, N, K, r, r_pad, G, NB, KB, Npad, mt, nt, ksplit, Mpad;
};

__device__ inline void tile_of(int bid, int mt, int nt, int& tm, int& tn)
{
    const int T = mt * nt;
    int t = bid;
    if ((T & 7) == 0) {
        // block ids congruent mod 8 land on one XCD: give each XCD a
        // contiguous run of the grouped raster below
        t = (bid & 7) * (T >> 3) + (bid >> 3);
    }
    const int GM = 4;  // M tiles per raster group
    const int group = t / (GM * nt);
    const int first = group * GM;
    const int gm = min(GM, mt - first);
    const int in = t - group * GM * nt;
    tm = first + in % gm;
    tn = in / gm;
}

template <int ACT, int BM, bool GROUPED>
__global__ __launch_bounds__(PF_THREADS, 1)
void prefill_gemm_kernel(GemmKArgs a)
{
    constexpr int RB = BM / 16;            // 16-row blocks per tile
    constexpr int XROW_BYTES = PANEL_K * 2; // 256 bytes per staged row
    constexpr int XLOADS = BM * XROW_BYTES / 16 / PF_THREADS;  // 16-byte loads per thread per step
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][BM * XROW_BYTES];
    __shared__ uint32_t s_old;

    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = tid >> 6;
    int tm, tn;
    tile_of(blockIdx.x, a.mt, a.nt, tm, tn);
    const int kz = blockIdx.y;
    const int m0 = tm * BM;
    const int n0 = tn * PF_BN;
    const int cbw = n0 / PANEL_N + 4 * w;   // first column block of this wavefront

    const int kb0 = (int)(((long)kz * a.KB) / a.ksplit);
    const int kb1 = (int)(((long)(kz + 1) * a.KB) / a.ksplit);

    // X tile staging: thread -> (row, chunk) for each of its loads
    const uint16_t* xsrc[XLOADS];
    int xdst[XLOADS];
#pragma unroll
    for (int i = 0; i < XLOADS; ++i) {
        const int rr = i * (PF_THREADS / 16) + (tid >> 4);
        const int ch = tid & 15;
        const int gm = min(m0 + rr, a.M - 1);
        xsrc[i] = a.X + (size_t)gm * a.K + ch * 8;
        xdst[i] = rr * XROW_BYTES + ((ch ^ (rr & 15)) << 4);
    }

    floatx4 acc[RB][4];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = (floatx4){0.f, 0.f, 0.f, 0.f};

    int n_j[4];
    bool colok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        n_j[j] = (cbw + j) * PANEL_N + (l & 15);
        colok[j] = (cbw + j) < a.NB;
    }

    // per-channel zero points (and, when grouped, per-group scale/zero)
    DqF16 dqh[4];
    float dqb[4];
    half2_t sh2[4];
    float sf[4];
    auto load_sz = [&](int grp) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t v = colok[j] ? a.sz[(size_t)grp * a.Npad + n_j[j]] : 0u;
            const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFF));
            const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
            sf[j] = (float)s;
            sh2[j] = (half2_t){s, s};
            dqh[j] = dq_f16_consts(z);
            dqb[j] = -(8388608.0f + z);
        }
    };
    int cur_g = (kb0 * PANEL_K) / a.G;
    load_sz(cur_g);

    u32x4 xr[XLOADS];
    u32x4 wv[4], wn[4];
    auto load_x = [&](int kb) {
#pragma unroll
        for (int i = 0; i < XLOADS; ++i)
            xr[i] = ld16(xsrc[i] + (size_t)kb * PANEL_K);
    };
    auto load_w = [&](int kb, u32x4* dst) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            dst[j] = colok[j] ? ld16_stream(a.codes + ((size_t)(cbw + j) * a.KB + kb) * PANEL_BYTES + l * 16)
                              : (u32x4){0u, 0u, 0u, 0u};
    };
    auto store_x = [&](int buf) {
#pragma unroll
        for (int i = 0; i < XLOADS; ++i)
            st16(&xs[buf][xdst[i]], xr[i]);
    };

    if (kb0 < kb1) {
        load_x(kb0);
        load_w(kb0, wv);
        store_x(0);
    }
    __syncthreads();

    for (int kb = kb0; kb < kb1; ++kb) {
        const int cur = (kb - kb0) & 1;
        const bool more = kb + 1 < kb1;
        if (more) {
            load_x(kb + 1);
            load_w(kb + 1, wn);
        }
        if constexpr (GROUPED) {
            const int grp = (kb * PANEL_K) / a.G;
            if (grp != cur_g) {
                cur_g = grp;
                load_sz(grp);
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4 af[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int rr = rb * 16 + (l & 15);
                const int ch = 4 * s + (l >> 4);
                af[rb] = *reinterpret_cast<const u32x4*>(&xs[cur][rr * XROW_BYTES + ((ch ^ (l & 15)) << 4)]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u32x4 bq;
                if constexpr (ACT == ACT_F16) {
                    if constexpr (GROUPED)
                        bq = dequant_f16_scaled(wv[j][s], dqh[j], sh2[j]);
                    else
                        bq = dequant_f16(wv[j][s], dqh[j]);
                } else {
                    if constexpr (GROUPED)
                        bq = dequant_bf16_scaled(wv[j][s], dqb[j], sf[j]);
                    else
                        bq = dequant_bf16(wv[j][s], dqb[j]);
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc[rb][j] = mfma16x16x32<ACT>(af[rb], bq, acc[rb][j]);
            }
        }
        if (more) {
            store_x(cur ^ 1);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                wv[j] = wn[j];
        }
        __syncthreads();
    }

    // ---- split-K hand-over: the last workgroup of the tile sums the partials
    // (fragment layout [tile][split][wavefront][RB][4][64 lanes], 16 bytes per lane)
    if (a.ksplit > 1) {
        const int tile = tm * a.nt + tn;
        auto frag = [&](int z, int rb, int j) -> size_t {
            return ((((size_t)tile * a.ksplit + z) * 4 + w) * RB * 4 + rb * 4 + j) * 64 + l;
        };
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                st16_dev(a.partial + frag(kz, rb, j), acc[rb][j]);
        wait_all_mem();
        __syncthreads();
        if (tid == 0)
            s_old = atomic_add_dev(&a.cnt[tile], 1u);
        __syncthreads();
        if (s_old != (uint32_t)(a.ksplit - 1))
            return;
        if (tid == 0)
            atomic_store_dev(&a.cnt[tile], 0u);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                floatx4 t = (floatx4){0.f, 0.f, 0.f, 0.f};
                for (int z = 0; z < a.ksplit; ++z)
                    t += (z == kz) ? acc[rb][j] : ld16_dev(a.partial + frag(z, rb, j));
                acc[rb][j] = t;
            }
    }

    // ---- epilogue: per-channel scale, gated rank-r correction, store
    if constexpr (!GROUPED) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[rb][j] *= sf[j];
    }
    if (a.r > 0) {
        const int koff = 8 * (l >> 4);
        const int nsteps = a.r_pad >> 5;
        for (int rs = 0; rs < nsteps; ++rs) {
            u32x4 bfr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t hv[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int jr = 32 * rs + koff + t;
                    hv[t] = (jr < a.r && n_j[j] < a.N) ? (uint32_t)a.B[(size_t)jr * a.N + n_j[j]] : 0u;
                }
                bfr[j] = (u32x4){hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16),
                                 hv[4] | (hv[5] << 16), hv[6] | (hv[7] << 16)};
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int m = m0 + rb * 16 + (l & 15);
                const u32x4 af = ld16(a.tg + (size_t)m * a.r_pad + 32 * rs + koff);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[rb][j] = mfma16x16x32<ACT>(af, bfr[j], acc[rb][j]);
            }
        }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n_j[j];
            if (n >= a.N)
                continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + rb * 16 + 4 * (l >> 4) + v;
                if (m < a.M)
                    a.Y[(size_t)m * a.N + n] = f32_to_act<ACT>(acc[rb][j][v]);
            }
        }
}

template <int ACT, int BM, bool GROUPED>
static hipError_t launch_gemm_t(const GemmKArgs& k, hipStream_t st)
{
    dim3 grid(k.mt * k.nt, k.ksplit);
    hipLaunchKernelGGL((prefill_gemm_kernel<ACT, BM, GROUPED>), grid, dim3(PF_THREADS), 0, st, k);
    return hipGetLastError();
}

template <int ACT>
static hipError_t launch_gemm_act(const GemmKArgs& k, int BM, bool grouped, hipStream_t st)
{
    if (BM == 64)
        return grouped ? launch_gemm_t<ACT, 64, true>(k, st) : launch_gemm_t<ACT, 64, false>(k, st);
    return grouped ? launch_gemm_t<ACT, 128, true>(k, st) : launch_gemm_t<ACT, 128, false>(k, st);
}

hipError_t launch_prefill(const LayerArgs& a, const PrefillPlan& p, hipStream_t st)
{
    BlobGeom g = blob_geom(a.N, a.K, a.G);
    uint16_t* tg = (uint16_t*)(a.ws + p.off_tg);
    if (a.r > 0) {
        PrepassKArgs q;
        q.X = (const uint16_t*)a.X;
        q.A = (const uint16_t*)a.A;
        q.w_g = (const uint16_t*)a.w_g;
        q.b_g = a.b_g;
        q.M = a.M; q.K = a.K; q.r = a.r; q.r_pad = p.r_pad;
        q.kc = p.pre_kc; q.ks = p.pre_ks;
        q.partial = (floatx4*)(a.ws + p.off_pre_partial);
        q.cnt = (uint32_t*)(a.ws + p.off_pre_cnt);
        q.tg = tg;
        dim3 grid(p.pre_mt, p.pre_ks);
        if (a.act == ACT_F16)
            hipLaunchKernelGGL(prepass_kernel<ACT_F16>, grid, dim3(PF_THREADS), 0, st, q);
        else
            hipLaunchKernelGGL(prepass_kernel<ACT_BF16>, grid, dim3(PF_THREADS), 0, st, q);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    GemmKArgs k;
    k.X = (const uint16_t*)a.X;
    k.codes = (const uint8_t*)a.packed + g.codes_off;
    k.sz = (const uint32_t*)((const char*)a.packed + g.sz_off);
    k.B = (const uint16_t*)a.B;
    k.tg = tg;
    k.Y = (uint16_t*)a.Y;
    k.partial = (floatx4*)(a.ws + p.off_gemm_partial);
    k.cnt = (uint32_t*)(a.ws + p.off_gemm_cnt);
    k.M = a.M; k.N = a.N; k.K = a.K; k.r = a.r; k.r_pad = p.r_pad; k.G = a.G;
    k.NB = g.NB; k.KB = g.KB; k.Npad = g.Npad;
    k.mt = p.mt; k.nt = p.nt; k.ksplit = p.ksplit; k.Mpad = p.Mpad;
    const bool grouped = a.G != a.K;
    if (a.act == ACT_F16)
        return launch_gemm_act<ACT_F16>(k, p.BM, grouped, st);
    return launch_gemm_act<ACT_BF16>(k, p.BM, grouped, st);
}

}  // namespace w4ec
