// prefill.hip -- the W4 + EC layer for many tokens: a prepass for the gate
// and X A, then a tiled MFMA GEMM whose epilogue applies the gated rank-r
// correction.
//
// SPEAR (gist.science technical summary, section 2.2A) describes the
// prefill phase as compute bound.  The page runs the EC beside the GEMM in a
// separate kernel; this library instead folds the gated correction into the
// GEMM epilogue as r extra terms of the reduction (T_g B), and keeps the only
// part that needs a full pass over K -- the gate logit X . w_g and T = X A --
// in a prepass that reads X once for all r + 1 columns (K-sliced partial
// sums), followed by a small kernel that adds the slices and applies the
// gate.
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
    int M, K, r, kc, ks;
    floatx4* partial;   // [pre_mt][ks][4 wavefronts][ec_blocks(r)][64 lanes]
};

constexpr int PRE_MAXB = 17;   // column blocks of [A | w_g] (r <= 256), gate block included
constexpr int PRE_MAXS = 16;   // 32-k steps per workgroup (kc <= 512)

// One workgroup: 64 tokens (wavefront w: tokens 16 w .. 16 w + 15) x one K
// slice of at most 512.  Every load is issued at once -- the X fragments
// into registers, the slice of [A | w_g] straight into LDS -- then each
// wavefront runs the MFMAs for all column blocks and stores its fragments.
// The slices are added by ec_reduce_kernel, in slice order.
template <int ACT>
__global__ __launch_bounds__(PF_THREADS)
void prepass_kernel(PrepassKArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t psmem[];
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int mt = blockIdx.x;
    const int z = blockIdx.y;
    const int kbeg = z * a.kc;
    const int len = min(a.kc, a.K - kbeg);          // multiple of 64
    const int xrow = min(mt * 64 + 16 * w + (l & 15), a.M - 1);
    const int nb = ec_blocks(a.r);
    const bool gate = a.w_g != nullptr;
    uint16_t* at = reinterpret_cast<uint16_t*>(psmem);
    uint16_t* wgl = at + len * ec_pitch(a.r) + 16;

    const uint16_t* xp = a.X + (size_t)xrow * a.K + kbeg + 8 * (l >> 4);
    u32x4 xf[PRE_MAXS];
#pragma unroll
    for (int s = 0; s < PRE_MAXS; ++s)
        if (32 * s < len)
            xf[s] = ld16(xp + 32 * s);
    ec_stage(a.A, a.w_g, a.r, kbeg, len, at, wgl);
    wait_all_mem();
    __syncthreads();

    floatx4 acc[PRE_MAXB];
#pragma unroll
    for (int cb = 0; cb < PRE_MAXB; ++cb) {
        acc[cb] = (floatx4){0.f, 0.f, 0.f, 0.f};
        if (cb < nb) {
#pragma unroll
            for (int s = 0; s < PRE_MAXS; ++s)
                if (32 * s < len)
                    acc[cb] = mfma16x16x32<ACT>(xf[s], ec_bfrag(at, wgl, a.r, gate, cb, 32 * s), acc[cb]);
        }
    }
    floatx4* mine = a.partial + ((size_t)(mt * a.ks + z) * 4 + w) * nb * 64;
#pragma unroll
    for (int cb = 0; cb < PRE_MAXB; ++cb)
        if (cb < nb)
            mine[cb * 64 + l] = acc[cb];
}

struct EcReduceKArgs {
    const floatx4* partial;
    uint16_t* tg;       // [Mpad][r_pad], activation format
    float b_g;
    int r, r_pad, ks;
};

// One workgroup per 16 tokens: adds the K slices' fragments in slice order,
// applies the gate and stores T_g = g * T (zero in columns r .. r_pad - 1).
template <int ACT>
__global__ __launch_bounds__(PF_THREADS)
void ec_reduce_kernel(EcReduceKArgs a)
{
    constexpr int TP = 260;                          // LDS row of T: r + 1 <= 257 columns
    __shared__ float tl[16][TP];
    __shared__ float gl[16];
    const int tid = threadIdx.x;
    const int rb = blockIdx.x;                       // rows 16 rb .. 16 rb + 15
    const int mt = rb >> 2, w = rb & 3;
    const int ne = ec_blocks(a.r) * 64;              // fragments per slice of this row block
    const floatx4* base = a.partial + ((size_t)mt * a.ks * 4 + w) * ne;
    const size_t zs = (size_t)4 * ne;
    for (int e = tid; e < ne; e += PF_THREADS) {
        const floatx4* src = base + e;
        floatx4 t = (floatx4){0.f, 0.f, 0.f, 0.f};
        int z = 0;
        for (; z + 8 <= a.ks; z += 8) {
            floatx4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = src[(size_t)(z + i) * zs];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                t += v[i];
        }
        for (; z < a.ks; ++z)
            t += src[(size_t)z * zs];
        const int l = e & 63;
        const int c = ec_col(a.r, e >> 6, l & 15);
        if (c >= 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                tl[4 * (l >> 4) + v][c] = t[v];
        }
    }
    __syncthreads();
    if (tid < 16)
        gl[tid] = sigmoid_f32(tl[tid][a.r] + a.b_g);
    __syncthreads();
    for (int row = 0; row < 16; ++row)
        for (int c = tid; c < a.r_pad; c += PF_THREADS)
            a.tg[(size_t)(16 * rb + row) * a.r_pad + c] = f32_to_act<ACT>(c < a.r ? gl[row] * tl[row][c] : 0.0f);
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

size_t prepass_lds_bytes(int r, int kc)
{
    return (size_t)ec_slice_bytes(r, kc) + (size_t)kc * 2;
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
        q.M = a.M; q.K = a.K; q.r = a.r;
        q.kc = p.pre_kc; q.ks = p.pre_ks;
        q.partial = (floatx4*)(a.ws + p.off_pre_partial);
        const size_t lds = prepass_lds_bytes(a.r, p.pre_kc);
        auto pk = a.act == ACT_F16 ? prepass_kernel<ACT_F16> : prepass_kernel<ACT_BF16>;
        if (lds > 64 * 1024) {
            hipError_t e = hipFuncSetAttribute((const void*)pk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess)
                return e;
        }
        hipLaunchKernelGGL(pk, dim3(p.pre_mt, p.pre_ks), dim3(PF_THREADS), lds, st, q);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        EcReduceKArgs rq;
        rq.partial = q.partial;
        rq.tg = tg;
        rq.b_g = a.b_g;
        rq.r = a.r; rq.r_pad = p.r_pad; rq.ks = p.pre_ks;
        auto rk = a.act == ACT_F16 ? ec_reduce_kernel<ACT_F16> : ec_reduce_kernel<ACT_BF16>;
        hipLaunchKernelGGL(rk, dim3(p.pre_mt * 4), dim3(PF_THREADS), 0, st, rq);
        e = hipGetLastError();
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
