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
//  * workgroup tile BM x 256 (BM = 64 or 128 tokens), 8 wavefronts (two per
//    SIMD); wavefront w owns columns [32 w, 32 w + 32) of the tile for all BM
//    rows, so every packed weight is loaded and dequantized exactly once per
//    tile, straight from HBM into registers (one 16-byte load per lane per
//    16 x 128 panel), through a ring of four 128-k steps in flight;
//  * the X tile (BM x 128 per step) is loaded two steps ahead into registers
//    and written to an LDS double buffer, with 16-byte chunks XOR-swizzled by
//    row so the MFMA A-operand reads are free of bank conflicts; all eight
//    wavefronts read it;
//  * with bf16 and one zero point per column, the weights enter the MFMAs as
//    128 + q and the epilogue subtracts (128 + z) times the token's sum of
//    activations (from the prepass), which saves the per-element subtract
//    that bf16 lacks in packed form;
//  * split-K when the tile count alone cannot fill the 256 CUs: partial fp32
//    tiles go to the workspace and the last-arriving workgroup of a tile adds
//    them in a fixed order, then runs the epilogue;
//  * tile ids are remapped so that the workgroups an XCD receives (block ids
//    congruent mod 8) share rows of X and columns of W in that XCD's L2.
#include <atomic>
#include <type_traits>

#include "ec_tile.h"
#include "w4ec_common.h"
#include "w4ec_launch.h"

namespace w4ec {

constexpr int PF_THREADS = 256;
constexpr int PF_BN = 256;
// GEMM: 8 wavefronts (two per SIMD, so that one's dequantization and loads
// run under the other's MFMAs), each owning JW = 2 column blocks (32
// columns) of the 256-column tile for all BM rows
constexpr int GEMM_THREADS = 512;
constexpr int NW = GEMM_THREADS / 64;
constexpr int JW = PF_BN / PANEL_N / NW;

// ---------------------------------------------------------------- prepass

struct PrepassKArgs {
    const uint16_t* X;
    const uint16_t* A;
    const uint16_t* w_g;
    uint32_t one2;      // two ones in the activation format: also sum each token's activations (else 0)
    int M, K, r, kc, ks;
    int nch;            // chunks of kc per workgroup (its slice: nch kc, the chunks one after another)
    floatx4* partial;   // [pre_mt][ks][4 wavefronts][ec_blocks(r)][64 lanes]
};

constexpr int PRE_MAXB = 17;   // column blocks of [A | w_g] (r <= 256), gate block included
constexpr int PRE_MAXS = 16;   // 32-k steps per workgroup (kc <= 512)

// adds this chunk's products into acc (the caller zeroes it once)
template <int ACT, int NS>
__device__ inline void prepass_mfma(const u32x4 (&xf)[PRE_MAXS], const uint16_t* at, const uint16_t* wgl, int r,
                                    bool gate, uint32_t one2, int nb, floatx4 (&acc)[PRE_MAXB])
{
    const int nba = ec_a_blocks(r);
#pragma unroll
    for (int cb = 0; cb < PRE_MAXB; ++cb) {
        if (cb < nb) {
            u32x4 bf[NS];
            if (cb < nba) {
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    bf[s] = ec_bfrag_a<true>(at, r, cb, 32 * s);
            } else {
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    bf[s] = ec_bfrag_gate(wgl, gate, one2, 32 * s);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s)
                acc[cb] = mfma16x16x32<ACT>(xf[s], bf[s], acc[cb]);
        }
    }
}

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
    const int xrow = min(mt * 64 + 16 * w + (l & 15), a.M - 1);
    const int nb = ec_blocks(a.r);
    const bool gate = a.w_g != nullptr;
    uint16_t* at = reinterpret_cast<uint16_t*>(psmem);

    floatx4 acc[PRE_MAXB];
#pragma unroll
    for (int cb = 0; cb < PRE_MAXB; ++cb)
        acc[cb] = (floatx4){0.f, 0.f, 0.f, 0.f};
    // the slice's chunks one after another (one, unless the grid would
    // otherwise take several rounds of workgroups)
    for (int c = 0; c < a.nch; ++c) {
        const int kbeg = (z * a.nch + c) * a.kc;
        if (kbeg >= a.K)
            break;                                      // uniform
        const int len = min(a.kc, a.K - kbeg);          // multiple of 64
        uint16_t* wgl = at + len * ec_pitch(a.r) + 16;
        if (c > 0)
            __syncthreads();                            // the previous chunk's LDS reads are done
        const uint16_t* xp = a.X + (size_t)xrow * a.K + kbeg + 8 * (l >> 4);
        u32x4 xf[PRE_MAXS];
#pragma unroll
        for (int s = 0; s < PRE_MAXS; ++s)            // steps past the chunk are never used
            xf[s] = ld16(xp + 32 * min(s, (len >> 5) - 1));
        ec_stage<PF_THREADS, true>(a.A, a.w_g, a.r, kbeg, len, at, wgl);
        wait_all_mem();
        __syncthreads();

        // per column block (wavefront-uniform branch), all fragment reads of
        // the chunk first, then the MFMAs; the step count is a template
        // argument, so no MFMA of the chain sits behind a branch
        switch (len >> 6) {
        case 1: prepass_mfma<ACT, 2>(xf, at, wgl, a.r, gate, a.one2, nb, acc); break;
        case 2: prepass_mfma<ACT, 4>(xf, at, wgl, a.r, gate, a.one2, nb, acc); break;
        case 3: prepass_mfma<ACT, 6>(xf, at, wgl, a.r, gate, a.one2, nb, acc); break;
        case 4: prepass_mfma<ACT, 8>(xf, at, wgl, a.r, gate, a.one2, nb, acc); break;
        case 5: prepass_mfma<ACT, 10>(xf, at, wgl, a.r, gate, a.one2, nb, acc); break;
        case 6: prepass_mfma<ACT, 12>(xf, at, wgl, a.r, gate, a.one2, nb, acc); break;
        case 7: prepass_mfma<ACT, 14>(xf, at, wgl, a.r, gate, a.one2, nb, acc); break;
        default: prepass_mfma<ACT, 16>(xf, at, wgl, a.r, gate, a.one2, nb, acc); break;
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
    float* rowsum;      // [Mpad] sums of each token's activations, or null
    float b_g;
    int r, r_pad, ks;
    const uint16_t* G1; // vector gate: act [r][h], [h], [h][r], [r]
    const uint16_t* c1;
    const uint16_t* G2;
    const uint16_t* c2;
    int h;
    int vg_staged;      // the gate parameters are copied to (dynamic) LDS
};

// One workgroup per (16 tokens, column block of T): adds the K slices'
// fragments of that block and of the gate block in slice order, applies
// the gate and stores its 16 columns of T_g = g * T (zero past r).
template <int ACT>
__global__ __launch_bounds__(PF_THREADS)
void ec_reduce_kernel(EcReduceKArgs a)
{
    __shared__ float tl[2][4][64][4];                // [block: mine, gate][quarter of the slices][lane][v]
    __shared__ float gl[16];
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int q = tid >> 6;                          // wavefront: a quarter of the slices
    const int rb = blockIdx.x;                       // rows 16 rb .. 16 rb + 15
    const int cb = blockIdx.y;                       // column block of T (of ec_a_blocks(r))
    const int mt = rb >> 2, w = rb & 3;
    const int nb = ec_blocks(a.r);
    const int ne = nb * 64;                          // fragments per slice of this row block
    const floatx4* base = a.partial + ((size_t)mt * a.ks * 4 + w) * ne;
    const size_t zs = (size_t)4 * ne;
    // wavefront q adds slices q, q + 4, ... of both blocks (fixed order,
    // ascending); the loads of both blocks for up to eight slices each go
    // out together, so that a batch costs one trip to memory
    const floatx4* src0 = base + cb * 64 + l;
    const floatx4* src1 = base + (nb - 1) * 64 + l;
    floatx4 t0 = (floatx4){0.f, 0.f, 0.f, 0.f}, t1 = t0;
    for (int z0 = q; z0 < a.ks; z0 += 32) {
        floatx4 v0[8], v1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int z = min(z0 + 4 * i, a.ks - 1);          // past the last slice: re-read it, unused
            v0[i] = src0[(size_t)z * zs];
            v1[i] = src1[(size_t)z * zs];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (z0 + 4 * i < a.ks) {
                t0 += v0[i];
                t1 += v1[i];
            }
        }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        tl[0][q][l][v] = t0[v];
        tl[1][q][l][v] = t1[v];
    }
    __syncthreads();
    // gate logits of the 16 rows: lane column 0 of the gate block (row
    // 4 g + v lives in lane 16 g, element v); their sums: lane column 1
    if (tid < 16) {
        const int lane = (tid >> 2) * 16;
        const int v = tid & 3;
        const float lg = ((tl[1][0][lane][v] + tl[1][1][lane][v]) + tl[1][2][lane][v]) + tl[1][3][lane][v];
        gl[tid] = sigmoid_f32(lg + a.b_g);
        if (a.rowsum && cb == 0)
            a.rowsum[16 * rb + tid] =
                ((tl[1][0][lane + 1][v] + tl[1][1][lane + 1][v]) + tl[1][2][lane + 1][v]) + tl[1][3][lane + 1][v];
    }
    __syncthreads();
    // this block's 16 columns for the 16 rows: lane l holds column l & 15, rows 4 (l >> 4) + v
    if (tid < 64) {
        const int c = 16 * cb + (l & 15);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = 4 * (l >> 4) + v;
            const float t = ((tl[0][0][l][v] + tl[0][1][l][v]) + tl[0][2][l][v]) + tl[0][3][l][v];
            if (c < a.r_pad)
                a.tg[(size_t)(16 * rb + row) * a.r_pad + c] = f32_to_act<ACT>(c < a.r ? gl[row] * t : 0.0f);
        }
    }
    // columns of r_pad past the last block of A (r <= 16 (r_pad / 16 - 1) only when r_pad > 16 blocks)
    if (cb == ec_a_blocks(a.r) - 1) {
        for (int e = tid; e < 16 * a.r_pad; e += PF_THREADS) {
            const int row = e / a.r_pad, c = e - row * a.r_pad;
            if (c >= 16 * (cb + 1))
                a.tg[(size_t)(16 * rb + row) * a.r_pad + c] = 0;
        }
    }
}

// Vector gate (one gate per rank component; SPEAR summary section 2.1A,
// W + B diag(gamma(A x)) A with gamma a bottleneck MLP, read as
// gamma = sigmoid(relu(T G1 + c1) G2 + c2)).  One workgroup per 4 tokens
// (the 16 lanes of each MFMA fragment that hold them): it adds every column
// block of T over the K slices in slice order, runs the bottleneck for the
// 4 tokens in fp32 and stores T_g = gamma * T.
constexpr int VG_RMAX = 256;    // largest rank
constexpr int VG_NT = 4;        // tokens per workgroup

template <int ACT>
__global__ __launch_bounds__(PF_THREADS)
void ec_reduce_vgate_kernel(EcReduceKArgs a)
{
    static_assert(PF_THREADS == VG_THREADS, "the bottleneck helpers assume 256 threads");
    __shared__ float tT[VG_NT][VG_RMAX + 1];         // T of the 4 tokens (columns < r)
    __shared__ float tU[VG_NT * VG_HMAX];            // bottleneck activations
    __shared__ float red[VG_NT * VG_THREADS];        // the bottleneck's partial sums
    extern __shared__ __attribute__((aligned(16))) uint16_t gst[];   // staged gate parameters
    const int tid = threadIdx.x;
    // the gate parameters do not depend on T: their loads go out first and
    // overlap those of the partial sums
    const uint16_t *G1 = a.G1, *c1 = a.c1, *G2 = a.G2, *c2 = a.c2;
    uint16_t gv[VG_SREG];
    if (a.vg_staged)
        vgate_stage_load(G1, c1, G2, c2, a.r, a.h, gv);
    const int rb = blockIdx.x >> 2, grp = blockIdx.x & 3;   // rows 16 rb + 4 grp .. + 3
    const int mt = rb >> 2, w = rb & 3;
    const int nb = ec_blocks(a.r), nba = ec_a_blocks(a.r);
    const int ne = nb * 64;                          // fragments per slice of this row block
    const floatx4* base = a.partial + ((size_t)mt * a.ks * 4 + w) * ne;
    const size_t zs = (size_t)4 * ne;
    const int r = a.r, h = a.h;
    // e = (column block e / 16, column e % 16): lane 16 grp + column holds
    // rows 4 grp + v of that column
    for (int e = tid; e < nb * 16; e += PF_THREADS) {
        const int cb = e >> 4, col = e & 15;
        if (cb >= nba && !(a.rowsum && col == 1))
            continue;                                // the gate logit column is not used here
        const floatx4* src = base + cb * 64 + grp * 16 + col;
        floatx4 t = (floatx4){0.f, 0.f, 0.f, 0.f};
        for (int z0 = 0; z0 < a.ks; z0 += 8) {
            floatx4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = z0 + i < a.ks ? src[(size_t)(z0 + i) * zs] : (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 8; ++i)
                t += v[i];
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            if (cb < nba) {
                if (16 * cb + col < r)
                    tT[v][16 * cb + col] = t[v];
            } else {
                a.rowsum[16 * rb + 4 * grp + v] = t[v];   // the column of ones: activation sums
            }
        }
    }
    if (a.vg_staged)
        vgate_stage_store(G1, c1, G2, c2, r, h, gv, gst);
    __syncthreads();
    uint16_t* tg = a.tg + (size_t)(16 * rb + 4 * grp) * a.r_pad;
    // one copy per address space of the parameters (LDS when staged), so
    // that no access needs a flat (either-space) load
    auto bottleneck = [&](const uint16_t* g1, const uint16_t* b1, const uint16_t* g2, const uint16_t* b2) {
        vgate_hidden<ACT>(&tT[0][0], VG_RMAX + 1, VG_NT, r, h, g1, b1, tU, red);
        vgate_gates<ACT>(tU, VG_NT, r, h, g2, b2, 0, r, [&](int t, int c, float g) {
            tg[(size_t)t * a.r_pad + c] = f32_to_act<ACT>(g * tT[t][c]);
        });
    };
    if (a.vg_staged) {
        const int n1 = r * h;
        bottleneck(gst, gst + n1, gst + n1 + h, gst + 2 * n1 + h);
    } else {
        bottleneck(a.G1, a.c1, a.G2, a.c2);
    }
    const int pad = a.r_pad - r;
    for (int e = tid; e < VG_NT * pad; e += PF_THREADS)
        tg[(size_t)(e / pad) * a.r_pad + r + e % pad] = f32_to_act<ACT>(0.0f);
}

// ---------------------------------------------------------------- salient channels
//
// Single-factor correction over salient input channels (SERQ summary,
// section 2): T_g is the gather X[:, S] of s channels, laid out like the
// gated rank-r activations ([rows][r_pad], zero past s and past M), so the
// GEMM's epilogue adds T_g R unchanged.  An index outside [0, K) is clamped
// and raises flags[3].
struct GatherKArgs {
    const uint16_t* X;
    const int32_t* S;
    uint16_t* tg;
    uint32_t* flags;
    int M, K, s, r_pad, rows;
};

__global__ __launch_bounds__(PF_THREADS)
void serq_gather_kernel(GatherKArgs a)
{
    const int e = blockIdx.x * PF_THREADS + threadIdx.x;
    if (e >= a.rows * a.r_pad)
        return;
    const int m = e / a.r_pad, j = e - m * a.r_pad;
    uint16_t v = 0;
    if (m < a.M && j < a.s) {
        int idx = a.S[j];
        if (idx < 0 || idx >= a.K) {
            atomic_store_dev(&a.flags[3], 1u);
            idx = min(max(idx, 0), a.K - 1);
        }
        v = a.X[(size_t)m * a.K + idx];
    }
    a.tg[e] = v;
}

// ---------------------------------------------------------------- unfused EC
//
// The correction as a kernel of its own, for the unfused and semi-fused
// prefill forms (SPEAR summary section 2.2A runs the EC beside the low-bit
// GEMM and adds it afterwards): Y += T_g B, with T_g [rows][r_pad] from the
// gate step and Y already holding the plain W4 product.  One workgroup per
// 64 x 64 tile of Y; the B tile is staged in LDS and read back as MFMA
// operands, T_g rows are the other operand, Y is read, added to and rounded
// once more.
constexpr int APPLY_TM = 64, APPLY_TN = 64;
constexpr int APPLY_BP = APPLY_TN + 16;   // halves per staged B row

struct ApplyKArgs {
    uint16_t* Y;
    const uint16_t* B;
    const uint16_t* tg;
    int M, N, r, r_pad;
};

template <int ACT>
__global__ __launch_bounds__(PF_THREADS)
void ec_apply_kernel(ApplyKArgs a)
{
    __shared__ __attribute__((aligned(16))) uint16_t bl[256 * APPLY_BP];   // r_pad <= 256 rows
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = tid >> 6;
    const int n0 = blockIdx.x * APPLY_TN;
    const int m0 = blockIdx.y * APPLY_TM;
    // B rows [0, r_pad) x columns [n0, n0 + 64): zero past r and past N
    for (int e = tid; e < a.r_pad * (APPLY_TN / 8); e += PF_THREADS) {
        const int j = e / (APPLY_TN / 8), c8 = e - j * (APPLY_TN / 8);
        const int n = n0 + 8 * c8;
        uint16_t v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
            v[t] = (j < a.r && n + t < a.N) ? a.B[(size_t)j * a.N + n + t] : (uint16_t)0;
        u32x4 q = (u32x4){v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                          v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16)};
        st16(bl + (size_t)j * APPLY_BP + 8 * c8, q);
    }
    __syncthreads();
    const int row = m0 + 16 * w + (l & 15);            // A-operand row of this lane
    const uint16_t* tr = a.tg + (size_t)row * a.r_pad + 8 * (l >> 4);
    floatx4 acc[APPLY_TN / 16];
#pragma unroll
    for (int j = 0; j < APPLY_TN / 16; ++j)
        acc[j] = (floatx4){0.f, 0.f, 0.f, 0.f};
    for (int rs = 0; rs < a.r_pad / 32; ++rs) {
        const u32x4 af = ld16(tr + 32 * rs);
#pragma unroll
        for (int j = 0; j < APPLY_TN / 16; ++j)
            acc[j] = mfma16x16x32<ACT>(af, lds_bfrag(bl, APPLY_BP, 16 * j, 32 * rs), acc[j]);
    }
#pragma unroll
    for (int j = 0; j < APPLY_TN / 16; ++j) {
        const int n = n0 + 16 * j + (l & 15);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = m0 + 16 * w + 4 * (l >> 4) + v;
            if (m < a.M && n < a.N) {
                uint16_t* y = a.Y + (size_t)m * a.N + n;
                *y = f32_to_act<ACT>(act_to_f32<ACT>(*y) + acc[j][v]);
            }
        }
    }
}

hipError_t launch_prefill_ec_apply(const ApplyArgs& a, const PrefillPlan& p, hipStream_t st)
{
    ApplyKArgs k;
    k.Y = (uint16_t*)a.Y;
    k.B = (const uint16_t*)a.B;
    k.tg = (const uint16_t*)(a.ws + p.off_tg);
    k.M = a.M; k.N = a.N; k.r = a.r; k.r_pad = p.r_pad;
    dim3 grid((a.N + APPLY_TN - 1) / APPLY_TN, (a.M + APPLY_TM - 1) / APPLY_TM);
    if (a.act == ACT_F16)
        hipLaunchKernelGGL(ec_apply_kernel<ACT_F16>, grid, dim3(PF_THREADS), 0, st, k);
    else
        hipLaunchKernelGGL(ec_apply_kernel<ACT_BF16>, grid, dim3(PF_THREADS), 0, st, k);
    return hipGetLastError();
}

// ---------------------------------------------------------------- GEMM

struct GemmKArgs {
    const uint16_t* X;
    const uint8_t* codes;
    const uint32_t* sz;
    const uint16_t* B;
    uint16_t* tg;      // [Mpad][r_pad] T_g, activation format
    float* rowsum;     // bf16 per-channel: sums of each token's activations over K
    uint16_t* Y;
    floatx4* partial;  // [tile][ksplit][NW][RB][JW][64] fragments
    uint32_t* cnt;     // [mt*nt]
    // Fused EC (ec_q > 0): the workgroups make T_g (and the activation sums)
    // themselves.  Every workgroup is resident at once; the first ec_q of
    // each row of tiles compute a K range of [T | l] = X [A | w_g] for the
    // row's tokens before their main loop, and after it they hand out the
    // reduction of those pieces among themselves, 16 tokens x 16 ranks at a
    // time; the epilogue waits (bounded) for all of its row's units.
    const uint16_t* A;
    const uint16_t* w_g;
    float b_g;
    uint32_t one2;     // two ones in the activation format: also sum the activations (else 0)
    floatx4* ecp;      // [mt][ec_q][BM / 16][ec_blocks(r)][64] fragments
    uint32_t* eccnt;   // [4][mt]: pieces done, units handed out, units done, workgroups done
    uint32_t* flags;   // workspace flags: [1] a fused-EC wait gave up (sticky until reset)
    uint32_t spin;     // polls before a bounded wait gives up
    int ec_q, ec_kc;   // pieces per row of tiles; k per LDS slice of [A | w_g]
    int M, N, K, r, r_pad, G, NB, KB, Npad, mt, nt, ksplit, Mpad;
};

// Work item of a workgroup: its tile (tm, tn) and K split kz.  Workgroups
// whose linear ids are congruent mod 8 run on one XCD; each XCD gets a
// contiguous run of the work items in split-major order, so that with a K
// split it holds one split's K range of many tiles (its L2 then fetches
// that range of X and of the weights once, instead of every range of the
// tiles it holds); the tiles of a split run in a grouped raster (GM M tiles
// by all N tiles), so that neighbouring items share activations and weights.
__device__ inline void work_of(int mt, int nt, int ksplit, int& tm, int& tn, int& kz)
{
    const int T = mt * nt;
    const int W = T * ksplit;
    const int bid = blockIdx.x + blockIdx.y * gridDim.x;
    const int wi = (W & 7) == 0 ? (bid & 7) * (W >> 3) + (bid >> 3) : bid;
    kz = wi / T;
    const int t = wi - kz * T;
    const int GM = 8;  // M tiles per raster group (2, 4, 16 measured slower at 4096 tokens)
    const int group = t / (GM * nt);
    const int first = group * GM;
    const int gm = min(GM, mt - first);
    const int in = t - group * GM * nt;
    tm = first + in % gm;
    tn = in / gm;
}

// ---------------------------------------------------------------- fused EC
//
// SPEAR (gist.science technical summary, section 2.1A): the gate logit
// x w_g and the rank-r projection X A come from one pass over X; the
// correction g (X A) B is added in the epilogue.  Here the pass over X is
// spread over the GEMM's own workgroups (all resident: a plan of at most
// one workgroup per CU), so that no separate launch precedes the GEMM.

__device__ inline float ld_dev_f32(const float* p)
{
    return __uint_as_float(atomic_load_dev(reinterpret_cast<const uint32_t*>(p)));
}

// byte offset of piece q's fragment (row block rb, column block cb) of tile row tm
__device__ inline uint32_t ecp_off(const GemmKArgs& a, int rbk, int tm, int q, int rb, int cb)
{
    const int l = threadIdx.x & 63;
    return (uint32_t)(((((size_t)tm * a.ec_q + q) * rbk + rb) * ec_blocks(a.r) + cb) * 64 + l) * 16u;
}

__device__ inline __amdgpu_buffer_rsrc_t ecp_rsrc(const GemmKArgs& a, int rbk)
{
    return dev_rsrc(a.ecp, (uint32_t)((size_t)a.mt * a.ec_q * rbk * ec_blocks(a.r) * 64 * 16));
}

// Bounded wait (thread 0 of the workgroup) until *p >= target; true when it
// gave up (at once with a wait limit of 0, or after an earlier wait of the
// fused EC gave up on this workspace: flags[1], sticky until reset).
__device__ inline bool ec_wait_ge(const GemmKArgs& a, const uint32_t* p, uint32_t target)
{
    bool lost = a.spin == 0 || atomic_load_dev(&a.flags[1]) != 0;
    for (uint32_t it = 0; !lost && atomic_load_dev(p) < target; ++it) {
        if (it >= a.spin)
            lost = true;
        else
            __builtin_amdgcn_s_sleep(1);
    }
    if (lost)
        atomic_store_dev(&a.flags[1], 1u);
    return lost;
}

// Producer: piece q of tile row tm, rows m0 .. m0 + BM - 1 of [T | l] over
// the K range [k0, k1) (64-multiples, about K / ec_q, at most ec_kc), with
// that range of [A | w_g] in LDS.  Wavefront w takes row block w mod (BM /
// 16) and, with two wavefronts per row block, every other column block;
// each block is one chain of MFMAs, stored as soon as it is done.  The LDS
// is not in use yet, nor are the main loop's registers.
template <int ACT, int NS>
__device__ __forceinline__ void ec_piece_blocks(const GemmKArgs& a, const u32x4 (&xf)[PRE_MAXS], const uint16_t* at,
                                                const uint16_t* wgl, int cb0, int cbstep, __amdgpu_buffer_rsrc_t rs,
                                                uint32_t off0)
{
    const int nb = ec_blocks(a.r), nba = ec_a_blocks(a.r);
    const bool gate = a.w_g != nullptr;
#pragma unroll 1
    for (int cb = cb0; cb < nb; cb += cbstep) {        // wavefront-uniform
        u32x4 bf[NS];
        if (cb < nba) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
                bf[s] = ec_bfrag_a<true>(at, a.r, cb, 32 * s);
        } else {
#pragma unroll
            for (int s = 0; s < NS; ++s)
                bf[s] = ec_bfrag_gate(wgl, gate, a.one2, 32 * s);
        }
        floatx4 acc = (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s)
            acc = mfma16x16x32<ACT>(xf[s], bf[s], acc);
        st16_sc1(rs, off0 + (uint32_t)cb * 1024u, acc);
    }
}

template <int ACT, int BM>
__device__ __forceinline__ void ec_produce(const GemmKArgs& a, int tm, int q, int m0, uint8_t* smem)
{
    constexpr int RBK = BM / 16;
    constexpr int WPR = NW / RBK;
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rb = w % RBK, part = w / RBK;
    const int K64 = a.K >> 6;
    const int k0 = 64 * (int)((long long)q * K64 / a.ec_q);
    const int k1 = 64 * (int)((long long)(q + 1) * K64 / a.ec_q);
    const int ns = (k1 - k0) >> 5;                     // 32-k steps (even, 2 .. 16)
    uint16_t* at = reinterpret_cast<uint16_t*>(smem);
    uint16_t* wgl = at + (k1 - k0) * ec_pitch(a.r) + 16;
    const uint16_t* xp = a.X + (size_t)min(m0 + 16 * rb + (l & 15), a.M - 1) * a.K + k0 + 8 * (l >> 4);
    u32x4 xf[PRE_MAXS];
#pragma unroll
    for (int s = 0; s < PRE_MAXS; ++s)                 // steps past the range are never used
        xf[s] = ld16(xp + 32 * min(s, ns - 1));
    ec_stage<GEMM_THREADS, true>(a.A, a.w_g, a.r, k0, k1 - k0, at, wgl);
    wait_all_mem();
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rs = ecp_rsrc(a, RBK);
    const uint32_t off0 = ecp_off(a, RBK, tm, q, rb, 0);
    switch (ns >> 1) {
    case 1: ec_piece_blocks<ACT, 2>(a, xf, at, wgl, part, WPR, rs, off0); break;
    case 2: ec_piece_blocks<ACT, 4>(a, xf, at, wgl, part, WPR, rs, off0); break;
    case 3: ec_piece_blocks<ACT, 6>(a, xf, at, wgl, part, WPR, rs, off0); break;
    case 4: ec_piece_blocks<ACT, 8>(a, xf, at, wgl, part, WPR, rs, off0); break;
    case 5: ec_piece_blocks<ACT, 10>(a, xf, at, wgl, part, WPR, rs, off0); break;
    case 6: ec_piece_blocks<ACT, 12>(a, xf, at, wgl, part, WPR, rs, off0); break;
    case 7: ec_piece_blocks<ACT, 14>(a, xf, at, wgl, part, WPR, rs, off0); break;
    default: ec_piece_blocks<ACT, 16>(a, xf, at, wgl, part, WPR, rs, off0); break;
    }
}

// Reducer: after its main loop a workgroup takes units (row block, column
// block of T) of its tile row from the row's dispenser until none is left,
// so that the workgroups that finish first do the work.  A unit adds the
// pieces' fragments of its block and of the gate block in a fixed order
// (wavefront w adds pieces w, w + 8, ...; then wavefront 0 adds the eight
// sums in order), applies the gate and stores 16 tokens x 16 ranks of T_g
// (and, for the first column block, the tokens' activation sums) with
// device-coherent stores; then it counts the unit as done.
template <int ACT, int BM>
__device__ __forceinline__ void ec_reduce_units(const GemmKArgs& a, int tm, int m0, uint8_t* smem, uint32_t& s_u)
{
    constexpr int RBK = BM / 16;
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nb = ec_blocks(a.r), nba = ec_a_blocks(a.r);
    const int ucb = nba > 0 ? nba : 1;                 // units per row block (r = 0: the sums alone)
    const uint32_t U = (uint32_t)(RBK * ucb);
    uint32_t* cnt_piece = a.eccnt;
    uint32_t* cnt_grab = a.eccnt + a.mt;
    uint32_t* cnt_unit = a.eccnt + 2 * a.mt;
    floatx4* red = reinterpret_cast<floatx4*>(smem);  // [NW][2][64]
    uint16_t* tgl = reinterpret_cast<uint16_t*>(red + NW * 2 * 64);   // [16][16]
    const __amdgpu_buffer_rsrc_t rs = ecp_rsrc(a, RBK);
    const __amdgpu_buffer_rsrc_t tgs = dev_rsrc(a.tg, (uint32_t)((size_t)a.Mpad * a.r_pad * 2));
    bool waited = false, lost = false;
    for (;;) {
        if (tid == 0)
            s_u = atomic_add_dev(&cnt_grab[tm], 1u);
        __syncthreads();
        const uint32_t u = s_u;
        if (u >= U)
            break;
        if (!waited) {
            // every piece of the row has been stored (long done in practice)
            __syncthreads();
            if (tid == 0)
                s_u = ec_wait_ge(a, &cnt_piece[tm], (uint32_t)a.ec_q) ? 1u : 0u;
            __syncthreads();
            lost = s_u != 0;
            waited = true;
        }
        const int rb = (int)u / ucb;
        const int cbt = nba > 0 ? (int)u - rb * ucb : nb - 1;
        floatx4 t = (floatx4){0.f, 0.f, 0.f, 0.f}, gsum = t;
        for (int q0 = w; q0 < a.ec_q; q0 += 4 * NW) {
            floatx4 vt[4], vg[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = min(q0 + NW * i, a.ec_q - 1);   // past the last piece: re-read it, unused
                vt[i] = ld16_sc1(rs, ecp_off(a, RBK, tm, q, rb, cbt));
                vg[i] = ld16_sc1(rs, ecp_off(a, RBK, tm, q, rb, nb - 1));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (q0 + NW * i < a.ec_q) {
                    t += vt[i];
                    gsum += vg[i];
                }
            }
        }
        red[(w * 2) * 64 + l] = t;
        red[(w * 2 + 1) * 64 + l] = gsum;
        __syncthreads();
        if (w == 0) {
            floatx4 T = red[l], Gb = red[64 + l];
#pragma unroll
            for (int v = 1; v < NW; ++v) {
                T += red[(v * 2) * 64 + l];
                Gb += red[(v * 2 + 1) * 64 + l];
            }
            // lane l: column l & 15 of the block, rows 4 (l >> 4) + v; the
            // gate logits of those rows sit in lane 16 (l >> 4) (column 0),
            // their activation sums in lane 16 (l >> 4) + 1
            const float nan = __builtin_nanf("");
            if (nba > 0) {
                const int c = 16 * cbt + (l & 15);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float lg = __shfl(Gb[v], l & 48);
                    const float g = sigmoid_f32(lg + a.b_g);
                    tgl[(4 * (l >> 4) + v) * 16 + (l & 15)] = f32_to_act<ACT>(lost ? nan : c < a.r ? g * T[v] : 0.0f);
                }
                if (l < 32) {
                    const int row = l >> 1, c8 = 8 * (l & 1);
                    const u32x4 val = *reinterpret_cast<const u32x4*>(tgl + row * 16 + c8);
                    const uint32_t off = (uint32_t)(((size_t)(m0 + 16 * rb + row) * a.r_pad) * 2);
                    st16_sc1(tgs, off + (16 * cbt + c8) * 2, __builtin_bit_cast(floatx4, val));
                    // ranks of r_pad past the last block of A: zero
                    if (cbt == nba - 1 && 16 * nba < a.r_pad)
                        st16_sc1(tgs, off + (16 * nba + c8) * 2, (floatx4){0.f, 0.f, 0.f, 0.f});
                }
            }
            if (a.one2 != 0 && cbt == (nba > 0 ? 0 : nb - 1) && (l & 15) == 1) {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    atomic_store_dev(reinterpret_cast<uint32_t*>(a.rowsum + m0 + 16 * rb + 4 * (l >> 4) + v),
                                     __float_as_uint(lost ? nan : Gb[v]));
            }
            wait_all_mem();
            if (l == 0)
                atomic_add_dev(&cnt_unit[tm], 1u);
        }
    }
}

constexpr int YT_PITCH = GEMM_YT_PITCH;   // halves per LDS row of the output tile (256 + 8: staggered banks)

template <int BM>
constexpr int gemm_lds_bytes()
{
    return gemm_lds_bytes_of(BM);
}

// The end of a GEMM tile: the split-K hand-over (the last workgroup of a
// tile adds the partial sums), the zero-point terms and scales, the gated
// rank-r correction, and the store.  NWV wavefronts, each owning 16 / NWV
// column blocks of the 256-column tile for all BM rows; `smem` is an LDS
// region of LDSB bytes that the main loop no longer uses.
// The gated rank-r correction as r more terms of a tile's reduction:
// acc += T_g[m0, m0 + BM) B[:, n0, n0 + 256).  The rank dimension goes in
// chunks of RCH ranks, as many as the LDS region of LDSB bytes holds: B rows
// padded to 272 halves, so that their transpose read is free of bank
// conflicts, T_g rows to RCH + 8.  load() sends the loads of 128 ranks (NCH
// chunks) out together into registers; apply() parks each chunk in LDS and
// reads it back as MFMA operands (loading ranks past 128 itself).  `fused`:
// T_g was written during this kernel, so it is read past this XCD's L2.
template <int ACT, int BM, int NWV, int LDSB>
struct GemmEc {
    static constexpr int GEMM_THREADS = 64 * NWV;
    static constexpr int JW = 16 / NWV;
    static constexpr int RB = BM / 16;
    static constexpr int BP = PF_BN + 16;               // halves per LDS row of B
    static constexpr int RCH = 128 * BP * 2 + BM * 136 * 2 <= LDSB ? 128 : 64 * BP * 2 + BM * 72 * 2 <= LDSB ? 64 : 32;
    static constexpr int TP = RCH + 8;                  // halves per LDS row of T_g
    static constexpr int BCH = RCH * (PF_BN / 8) / GEMM_THREADS;      // 16-byte B chunks per thread
    static constexpr int TCH = (BM * (RCH / 8) + GEMM_THREADS - 1) / GEMM_THREADS;
    static constexpr int NCH = 128 / RCH;               // chunks loaded together
    static_assert(RCH * BP * 2 + BM * TP * 2 <= LDSB, "EC staging fits the LDS");
    u32x4 bva[NCH][BCH], tva[NCH][TCH];

    // chunk [c0, c0 + RCH) of B's rows for the tile's 256 columns and of
    // T_g's columns for its BM tokens (zero past r and past r_pad, where
    // nothing is loaded)
    __device__ __forceinline__ void load_chunk(const GemmKArgs& a, int c0, int m0, int n0, bool fused,
                                               u32x4 (&bv)[BCH], u32x4 (&tv)[TCH])
    {
        const int tid = threadIdx.x;
        const bool bvec = ((uintptr_t)a.B & 15) == 0 && (a.N & 7) == 0;
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int ch = tid + GEMM_THREADS * i;
            const int jr = c0 + (ch >> 5), n = n0 + 8 * (ch & 31);
            u32x4 v = (u32x4){0u, 0u, 0u, 0u};
            if (jr < a.r) {
                const uint16_t* src = a.B + (size_t)jr * a.N + n;
                if (bvec && n + 8 <= a.N) {
                    v = ld16(src);
                } else {
                    uint32_t hv[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        hv[t] = n + t < a.N ? (uint32_t)src[t] : 0u;
                    v = (u32x4){hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16),
                                hv[6] | (hv[7] << 16)};
                }
            }
            bv[i] = v;
        }
        if (fused) {
            const __amdgpu_buffer_rsrc_t tgs = dev_rsrc(a.tg, (uint32_t)((size_t)a.Mpad * a.r_pad * 2));
#pragma unroll
            for (int i = 0; i < TCH; ++i) {
                const int ch = min(tid + GEMM_THREADS * i, BM * (RCH / 8) - 1);
                const int rr = ch / (RCH / 8), cc = ch - rr * (RCH / 8);
                tv[i] = c0 + 8 * cc < a.r_pad ? __builtin_bit_cast(u32x4, ld16_sc1(tgs, (uint32_t)(((size_t)(m0 + rr) * a.r_pad + c0 + 8 * cc) * 2)))
                                              : (u32x4){0u, 0u, 0u, 0u};
            }
        } else {
#pragma unroll
            for (int i = 0; i < TCH; ++i) {
                const int ch = min(tid + GEMM_THREADS * i, BM * (RCH / 8) - 1);
                const int rr = ch / (RCH / 8), cc = ch - rr * (RCH / 8);
                tv[i] = c0 + 8 * cc < a.r_pad ? ld16(a.tg + (size_t)(m0 + rr) * a.r_pad + c0 + 8 * cc)
                                              : (u32x4){0u, 0u, 0u, 0u};
            }
        }
    }

    // ranks [g0, g0 + 128)
    __device__ __forceinline__ void load(const GemmKArgs& a, int g0, int m0, int n0, bool fused)
    {
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            load_chunk(a, g0 + c * RCH, m0, n0, fused, bva[c], tva[c]);
    }

    // after load(a, 0, ...): every rank into acc (LDSB bytes of LDS at smem
    // free for it; a barrier ends each chunk)
    __device__ __forceinline__ void apply(const GemmKArgs& a, floatx4 (&acc)[RB][JW], int m0, int n0, uint8_t* smem,
                                          bool fused)
    {
        const int tid = threadIdx.x;
        const int l = tid & 63;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
        uint16_t* bl = reinterpret_cast<uint16_t*>(smem);
        uint16_t* tl = bl + RCH * BP;
        const int koff = 8 * (l >> 4);
        for (int g0 = 0; g0 < a.r_pad; g0 += NCH * RCH) {
            if (g0 > 0)
                load(a, g0, m0, n0, fused);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int c0 = g0 + c * RCH;
                if (c0 >= a.r_pad)
                    break;
#pragma unroll
                for (int i = 0; i < BCH; ++i) {
                    const int ch = tid + GEMM_THREADS * i;
                    st16(bl + (ch >> 5) * BP + 8 * (ch & 31), bva[c][i]);
                }
#pragma unroll
                for (int i = 0; i < TCH; ++i) {
                    const int ch = tid + GEMM_THREADS * i;
                    if (ch < BM * (RCH / 8)) {
                        const int rr = ch / (RCH / 8), cc = ch - rr * (RCH / 8);
                        st16(tl + rr * TP + 8 * cc, tva[c][i]);
                    }
                }
                __syncthreads();
                const int ns = min(RCH, a.r_pad - c0) >> 5;
                for (int rs = 0; rs < ns; ++rs) {
                    u32x4 bfr[JW];
#pragma unroll
                    for (int j = 0; j < JW; ++j)
                        bfr[j] = lds_bfrag(bl, BP, 16 * (JW * w + j), 32 * rs);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        const u32x4 af = *reinterpret_cast<const u32x4*>(tl + (rb * 16 + (l & 15)) * TP + 32 * rs + koff);
#pragma unroll
                        for (int j = 0; j < JW; ++j)
                            acc[rb][j] = mfma16x16x32<ACT>(af, bfr[j], acc[rb][j]);
                    }
                }
                __syncthreads();                        // before the next chunk or another use of the LDS
            }
        }
    }
};

template <int ACT, int BM, bool GROUPED, int NWV, int LDSB>
__device__ __forceinline__ void gemm_tail(const GemmKArgs& a, floatx4 (&acc)[BM / 16][16 / NWV], const float (&sf)[16 / NWV],
                                          const float (&zf)[16 / NWV], const uint32_t* const (&szsrc)[16 / NWV], int tm,
                                          int tn, int kz, int m0, int n0, uint8_t* smem, uint32_t& s_old, uint32_t& s_ec,
                                          const float* rsl)
{
    constexpr int GEMM_THREADS = 64 * NWV;
    constexpr int NW = NWV;
    constexpr int JW = 16 / NWV;
    constexpr int RB = BM / 16;
    constexpr bool BIAS = ACT == ACT_BF16 && !GROUPED;
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool fused = BM == 64 && a.ec_q > 0;
    // The gated rank-r correction's operands (its first 128 ranks) are
    // loaded as early as the tile allows, so that their trip to memory
    // overlaps the others of the tail: at once for a tile done in one piece;
    // for a split tile, by its last workgroup together with the other
    // splits' partial sums (128-token tiles: after those, the registers do
    // not hold both); with the fused EC after its wait.  A chunk of ranks
    // per trip, after everything else, cost 1-2 us per chunk.
    GemmEc<ACT, BM, NWV, LDSB> ec;
    if (BM == 64 && a.r > 0 && !fused && a.ksplit == 1)
        ec.load(a, 0, m0, n0, false);

    // ---- split-K hand-over: the last workgroup of the tile sums the partials
    // (fragment layout [tile][split][wavefront][RB][JW][64 lanes], 16 bytes per lane)
    if (a.ksplit > 1) {
        const int tile = tm * a.nt + tn;
        // byte offset of a fragment, within the region of all tiles' partials
        auto frag = [&](int z, int rb, int j) -> uint32_t {
            return (uint32_t)(((((size_t)tile * a.ksplit + z) * NW + w) * RB * JW + rb * JW + j) * 64 + l) * 16u;
        };
        const __amdgpu_buffer_rsrc_t prs =
            dev_rsrc(a.partial, (uint32_t)((size_t)a.mt * a.nt * a.ksplit * NW * RB * JW * 64 * 16));
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int j = 0; j < JW; ++j)
                st16_sc1(prs, frag(kz, rb, j), acc[rb][j]);
        wait_all_mem();
        __syncthreads();
        if (tid == 0)
            s_old = atomic_add_dev(&a.cnt[tile], 1u);
        __syncthreads();
        if (s_old != (uint32_t)(a.ksplit - 1))
            return;
        if (tid == 0)
            atomic_store_dev(&a.cnt[tile], 0u);
        if (BM == 64 && a.r > 0 && !fused)
            ec.load(a, 0, m0, n0, false);
        // splits added in order (from zero, as a plain sum would); the other
        // splits' fragments are loaded SB splits at a time, all in flight at
        // once (o-th other split: o, or o + 1 past this workgroup's own)
        constexpr int SB = BM == 64 ? 3 : 1;
        floatx4 sum[RB][JW];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int j = 0; j < JW; ++j)
                sum[rb][j] = (floatx4){0.f, 0.f, 0.f, 0.f};
        bool own = false;                               // this workgroup's partial added
        for (int o0 = 0; o0 < a.ksplit - 1; o0 += SB) {
            floatx4 t[SB][RB][JW];
#pragma unroll
            for (int s = 0; s < SB; ++s) {
                const int z = o0 + s + (o0 + s >= kz ? 1 : 0);
                if (z < a.ksplit) {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                        for (int j = 0; j < JW; ++j)
                            t[s][rb][j] = ld16_sc1(prs, frag(z, rb, j));
                }
            }
#pragma unroll
            for (int s = 0; s < SB; ++s) {
                const int z = o0 + s + (o0 + s >= kz ? 1 : 0);
                if (z < a.ksplit) {
                    if (!own && kz < z) {
                        own = true;
#pragma unroll
                        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                            for (int j = 0; j < JW; ++j)
                                sum[rb][j] += acc[rb][j];
                    }
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                        for (int j = 0; j < JW; ++j)
                            sum[rb][j] += t[s][rb][j];
                }
            }
        }
        if (!own) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int j = 0; j < JW; ++j)
                    sum[rb][j] += acc[rb][j];
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int j = 0; j < JW; ++j)
                acc[rb][j] = sum[rb][j];
    }
    if (BM != 64 && a.r > 0 && !fused)
        ec.load(a, 0, m0, n0, false);

    // ---- fused EC: wait (bounded) until every unit of this tile row is done;
    // a wait that gave up stores NaN
    bool eclost = false;
    if (fused) {
        const int ucb = ec_a_blocks(a.r) > 0 ? ec_a_blocks(a.r) : 1;
        if (tid == 0)
            s_ec = ec_wait_ge(a, a.eccnt + 2 * a.mt + tm, (uint32_t)(RB * ucb)) ? 1u : 0u;
        __syncthreads();
        eclost = s_ec != 0;
        if (a.r > 0)
            ec.load(a, 0, m0, n0, true);
    }

    // ---- epilogue: per-channel zero point (bf16) and scale, gated rank-r
    // correction.  The activation sums come from the LDS copy made at the
    // tile's start (rsl), or with the fused EC from memory, read past this
    // XCD's L2 (they were written during this kernel).
    if constexpr (BIAS) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = rb * 16 + 4 * (l >> 4) + v;
                const float sx = rsl ? rsl[row] : fused ? ld_dev_f32(a.rowsum + m0 + row) : a.rowsum[m0 + row];
#pragma unroll
                for (int j = 0; j < JW; ++j)
                    acc[rb][j][v] -= (128.0f + zf[j]) * sx;
            }
        }
        if (rsl)
            __syncthreads();                            // the LDS is reused below
    }
    if constexpr (ACT == ACT_F16 && !GROUPED) {
        // a fractional zero point among the tile's columns (the other forms
        // take it in the dequantization or the bf16 zero-point term)
        bool fz = false;
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(*szsrc[j] >> 16));
            fz |= z != floorf(z);
        }
        if (__syncthreads_or(fz)) {
            // fractional zero points (a slower path): subtract (z - zi) times
            // each token's sum of activations over K, computed here from X
            // (TPR threads per token, each a contiguous share of K, added in
            // a fixed order)
            constexpr int TPR = GEMM_THREADS / BM;
            float* rs = reinterpret_cast<float*>(smem);          // [TPR][BM], then [BM]
            {
                const int row = tid / TPR, part = tid - row * TPR;
                const int len = a.K / TPR;                       // a multiple of 16
                const uint16_t* xs = a.X + (size_t)min(m0 + row, a.M - 1) * a.K + (size_t)part * len;
                float t = 0.0f;
#pragma unroll 1
                for (int k = 0; k < len; k += 8) {
                    const u32x4 v = ld16(xs + k);
                    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const half2_t h = h2_of(u[i]);
                        t += (float)h.x;
                        t += (float)h.y;
                    }
                }
                rs[part * BM + row] = t;
            }
            __syncthreads();
            if (tid < BM) {
                float t = rs[tid];
                for (int q = 1; q < TPR; ++q)
                    t += rs[q * BM + tid];
                rs[TPR * BM + tid] = t;
            }
            __syncthreads();
            float zfr[JW];                              // z - floor(z) of this lane's columns
#pragma unroll
            for (int j = 0; j < JW; ++j) {
                const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(*szsrc[j] >> 16));
                zfr[j] = z - floorf(z);
            }
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float sx = rs[TPR * BM + rb * 16 + 4 * (l >> 4) + v];
#pragma unroll
                    for (int j = 0; j < JW; ++j)
                        acc[rb][j][v] -= zfr[j] * sx;
                }
            __syncthreads();                            // before the epilogue reuses the LDS
        }
    }
    if constexpr (!GROUPED) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int j = 0; j < JW; ++j)
                acc[rb][j] *= sf[j];
    }
    if (a.r > 0)
        ec.apply(a, acc, m0, n0, smem, fused);

    // ---- store: round to the activation format into an LDS tile, then
    // write whole rows of the tile with 16-byte stores (in passes of RBP
    // row blocks when the region holds fewer than BM rows)
    constexpr int RBP = LDSB / (16 * YT_PITCH * 2) < RB ? LDSB / (16 * YT_PITCH * 2) : RB;
    static_assert(RBP >= 1, "one row block of the output tile fits the LDS");
    uint16_t* yt = reinterpret_cast<uint16_t*>(smem);   // [RBP * 16][YT_PITCH]
    const bool vec = (a.N & 7) == 0;
#pragma unroll
    for (int rp = 0; rp < RB; rp += RBP) {
        if (rp > 0)
            __syncthreads();                            // the previous pass has read its rows
#pragma unroll
        for (int rb = rp; rb < rp + RBP && rb < RB; ++rb)
#pragma unroll
            for (int j = 0; j < JW; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    yt[((rb - rp) * 16 + 4 * (l >> 4) + v) * YT_PITCH + 16 * JW * w + 16 * j + (l & 15)] =
                        f32_to_act<ACT>(eclost ? __builtin_nanf("") : acc[rb][j][v]);
        __syncthreads();
        const int nrow = (rp + RBP <= RB ? RBP : RB - rp) * 16;
        for (int e = tid; e < nrow * (PF_BN / 8); e += GEMM_THREADS) {
            const int row = e >> 5, c8 = (e & 31) * 8;
            const int m = m0 + rp * 16 + row, n = n0 + c8;
            if (m >= a.M || n >= a.N)
                continue;
            const uint16_t* src = yt + row * YT_PITCH + c8;
            uint16_t* dst = a.Y + (size_t)m * a.N + n;
            if (vec) {
                st16(dst, *reinterpret_cast<const u32x4*>(src));
            } else {
                for (int t = 0; t < 8 && n + t < a.N; ++t)
                    dst[t] = src[t];
            }
        }
    }
}

template <int ACT, int BM, bool GROUPED>
__global__ __launch_bounds__(GEMM_THREADS, BM == 64 ? 2 : 1)
void prefill_gemm_kernel(GemmKArgs a)
{
    constexpr int RB = BM / 16;            // 16-row blocks per tile
    constexpr int XROW_BYTES = PANEL_K * 2; // 256 bytes per staged row
    // bf16 with one zero point per column: the weights enter the MFMAs as
    // 128 + c (one AND-OR per pair; bf16 has no packed subtract) and the
    // epilogue subtracts (128 + z) times the token's activation sum
    constexpr bool BIAS = ACT == ACT_BF16 && !GROUPED;
    constexpr int XLOADS = BM * XROW_BYTES / 16 / GEMM_THREADS;  // 16-byte loads per thread per step
    // weight ring: D 128-k steps per wavefront (even, so that the two
    // activation register sets below alternate with the ring slots); four
    // steps keep ~64 KB of weights in flight per CU
    constexpr int D = 4;
    // activation register sets: the activations of step i are loaded XS
    // steps ahead.  Loads retire in issue order, so the wait for them also
    // waits for every weight load issued before them: their distance bounds
    // the weight ring's.  Four sets (as deep as the ring) where the
    // registers allow.
    constexpr int XS = BM == 64 ? 4 : 2;
    static_assert(D % XS == 0, "activation sets must divide the ring");
    constexpr int LDSB = BM == 64 ? gemm_smem_bytes_of(BM) : gemm_lds_bytes<BM>();
    static_assert(2 * BM * XROW_BYTES + BM * 4 <= LDSB, "the activation sums fit beside the X buffers");
    __shared__ __attribute__((aligned(16))) uint8_t smem[LDSB];
    __shared__ uint32_t s_old, s_ec;

    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    int tm, tn, kz;
    work_of(a.mt, a.nt, a.ksplit, tm, tn, kz);
    const int m0 = tm * BM;
    const int n0 = tn * PF_BN;
    const int cbw = n0 / PANEL_N + JW * w;  // first column block of this wavefront

    const int kb0 = (int)(((long)kz * a.KB) / a.ksplit);
    const int nk = (int)(((long)(kz + 1) * a.KB) / a.ksplit) - kb0;   // >= 1 steps of 128 k

    // X tile staging: thread -> (row, chunk) for each of its loads; 16-byte
    // chunks XOR-swizzled by row in LDS
    const uint16_t* xsrc[XLOADS];
    int xdst[XLOADS];
#pragma unroll
    for (int i = 0; i < XLOADS; ++i) {
        const int rr = i * (GEMM_THREADS / 16) + (tid >> 4);
        const int ch = tid & 15;
        const int gm = min(m0 + rr, a.M - 1);
        xsrc[i] = a.X + (size_t)gm * a.K + (size_t)kb0 * PANEL_K + ch * 8;
        xdst[i] = rr * XROW_BYTES + ((ch ^ (rr & 15)) << 4);
    }

    int n_j[JW];
    bool colok[JW];
    const uint8_t* wsrc[JW];    // this lane's 16 bytes of the first panel of each column block
    const uint32_t* szsrc[JW];  // scale/zero of this lane's column, group of step 0
#pragma unroll
    for (int j = 0; j < JW; ++j) {
        n_j[j] = (cbw + j) * PANEL_N + (l & 15);
        colok[j] = (cbw + j) < a.NB;
        const int cb = min(cbw + j, a.NB - 1);       // past the end: re-read the last block, never stored
        wsrc[j] = a.codes + ((size_t)cb * a.KB + kb0) * PANEL_BYTES + l * 16;
        szsrc[j] = a.sz + (size_t)((kb0 * PANEL_K) / a.G) * a.Npad + min(n_j[j], a.Npad - 1);
    }

    floatx4 acc[RB][JW];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < JW; ++j)
            acc[i][j] = (floatx4){0.f, 0.f, 0.f, 0.f};

    // scale/zero of the current group: fp16 codes are offset by the integer
    // part zi = floor(z) exactly; the fractional part z - zi enters as
    // -(z - zi) s in the fp16 grouped dequantization, and as a correction by
    // the tokens' activation sums in the fp16 per-channel epilogue; bf16
    // grouped weights are q s - z s (exact operands, one rounding), and the
    // bf16 per-channel epilogue subtracts (128 + z) times the sums
    DqF16 dqh[JW];
    half2_t sh2[JW], ch2[JW];   // fp16 grouped: s and -(z - zi) s
    float sf[JW];
    float zf[JW];        // bf16 per-channel: z; bf16 grouped: -z s
    // The constants are formed in fp16 from the packed dword: zi = floor(z)
    // exactly, -(1024 + zi) and -(64 + zi) exactly (|z| <= 1024), and
    // (zi - z) s rounded once (zi - z is exact) -- -0 for an integer zero
    // point, so that those products are unchanged.
    auto set_sz = [&](const uint32_t* v) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)(v[j] & 0xFFFF));
            const _Float16 zh = __builtin_bit_cast(_Float16, (uint16_t)(v[j] >> 16));
            const _Float16 zi = __builtin_floorf16(zh);
            const _Float16 ch = (zi - zh) * sv;
            const _Float16 a = (_Float16)-1024.0f - zi, b = (_Float16)-64.0f - zi;
            sh2[j] = (half2_t){sv, sv};
            ch2[j] = (half2_t){ch, ch};
            dqh[j].off_lo = (half2_t){a, a};
            dqh[j].off_hi = (half2_t){b, b};
            if constexpr (ACT == ACT_BF16) {
                const float z = (float)zh;
                sf[j] = (float)sv;
                zf[j] = GROUPED ? -z * (float)sv : z;
            } else {
                sf[j] = (float)sv;
            }
        }
    };

    // Every load below is unconditional (indices clamped to the last step),
    // so the compiler can count the loads in flight and wait for exactly
    // the one it needs: the weight ring keeps D - 1 steps in flight behind
    // the one being multiplied.
    u32x4 wr[D][JW];
    uint32_t szr[GROUPED ? D : 1][JW];
    uint32_t szcur[JW] = {};    // scale/zero of the current group (grouped)
    u32x4 xr[XS][XLOADS];       // activations of steps i + 1, ..., i + XS
    auto issue_w1 = [&](int u, int i, int j) __attribute__((always_inline)) {
        const int ic = min(i, nk - 1);
        if constexpr (GROUPED) {
            const int gi = ((kb0 + ic) * PANEL_K) / a.G - (kb0 * PANEL_K) / a.G;
            szr[u][j] = szsrc[j][(size_t)gi * a.Npad];
        }
        wr[u][j] = ld16_stream(wsrc[j] + (size_t)ic * PANEL_BYTES);
    };
    auto issue_w = [&](int u, int i) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < JW; ++j)
            issue_w1(u, i, j);
    };
    // part p of 2 (XLOADS / 2 loads each, or all of them with part == -1)
    auto load_x = [&](int set, int i, int part = -1) __attribute__((always_inline)) {
        const int ic = min(i, nk - 1);
        constexpr int PER = XLOADS >= 2 ? XLOADS / 2 : 1;
#pragma unroll
        for (int x = 0; x < XLOADS; ++x)
            if (part < 0 || x / PER == part)
                xr[set][x] = ld16(xsrc[x] + (size_t)ic * PANEL_K);
    };
    auto store_x = [&](int set, int buf) __attribute__((always_inline)) {
        uint8_t* dst = smem + buf * (BM * XROW_BYTES);   // arithmetic, not a choice between captures
#pragma unroll
        for (int x = 0; x < XLOADS; ++x)
            st16(dst + xdst[x], xr[set][x]);
    };

    // fused EC (64-token tiles only, a single row of them): this
    // workgroup's piece, stored and counted before the main loop's first
    // loads go out (its registers are free then)
    constexpr bool FUSED = BM == 64;
    if (FUSED && a.ec_q > 0) {
        const int q = kz * a.nt + tn;
        if (q < a.ec_q) {
            ec_produce<ACT, BM>(a, tm, q, m0, smem);
            wait_all_mem();
            __syncthreads();
            if (tid == 0)
                atomic_add_dev(&a.eccnt[tm], 1u);
        }
    }
    if constexpr (!GROUPED) {
        uint32_t v[JW];
#pragma unroll
        for (int j = 0; j < JW; ++j)
            v[j] = *szsrc[j];
        set_sz(v);
    }
#pragma unroll
    for (int xs = 0; xs < XS; ++xs) {
        load_x(xs, xs);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < D; ++u) {
        issue_w(u, u);
        __builtin_amdgcn_sched_barrier(0);
    }
    // bf16 with one zero point per column: the tokens' activation sums,
    // copied to the end of the LDS (past the X buffers) for the epilogue,
    // which then makes no trip to memory for them
    const bool fused = FUSED && a.ec_q > 0;
    float* rsl = nullptr;
    if constexpr (BIAS) {
        if (!fused) {
            rsl = reinterpret_cast<float*>(smem + LDSB - BM * 4);
            if (tid < BM)
                rsl[tid] = a.rowsum[m0 + tid];
        }
    }
    store_x(0, 0);
    __syncthreads();

    const int ppg = a.G / PANEL_K;                   // steps per group
    // hook(s) runs before the MFMAs of k-step s: it spreads the step's global
    // loads over the step, so that they never arrive at the vector cache as
    // one burst that stalls the wavefront at its issue
    auto compute = [&](int i, const u32x4 (&wv)[JW], auto hook) __attribute__((always_inline)) {
        const uint8_t* xsb = smem + (i & 1) * (BM * XROW_BYTES);
        auto read_a = [&](int s, u32x4 (&af)[RB]) __attribute__((always_inline)) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int rr = rb * 16 + (l & 15);
                const int ch = 4 * s + (l >> 4);
                af[rb] = *reinterpret_cast<const u32x4*>(xsb + rr * XROW_BYTES + ((ch ^ (l & 15)) << 4));
            }
        };
        // A operands of the next k-step are read from LDS while the current
        // one's MFMAs run
        u32x4 afc[RB], afn[RB];
        read_a(0, afc);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            __builtin_amdgcn_sched_barrier(0);
            hook(s);
            __builtin_amdgcn_sched_barrier(0);   // keep this k-step's loads here
            if (s < 3)
                read_a(s + 1, afn);
#pragma unroll
            for (int j = 0; j < JW; ++j) {
                const uint32_t q = wv[j][s];
                u32x4 bq;
                if constexpr (ACT == ACT_F16) {
                    if constexpr (GROUPED)
                        bq = dequant_f16_scaled(q, dqh[j], sh2[j], ch2[j]);
                    else
                        bq = dequant_f16(q, dqh[j]);
                } else {
                    if constexpr (GROUPED)
                        bq = dequant_bf16_scaled(q, sf[j], zf[j]);
                    else
                        bq = bf16_biased(q);
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    acc[rb][j] = mfma16x16x32<ACT>(afc[rb], bq, acc[rb][j]);
            }
            if (s < 3) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    afc[rb] = afn[rb];
            }
        }
    };
    // one chunk of D steps; REFILL: the ring slot of each step is refilled
    // with the step D later (only while a full chunk follows)
    auto chunk = [&](int i0, auto refill_tag) __attribute__((always_inline)) {
        constexpr bool REFILL = decltype(refill_tag)::value;
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int i = i0 + u;                           // i0 is a multiple of D: i & 1 == u & 1
            u32x4 wv[JW];                                   // this step's panels: slot u is free to refill
#pragma unroll
            for (int j = 0; j < JW; ++j)
                wv[j] = wr[u][j];
            // k-steps 0 and 1: half each of the activations of step i + XS
            // (into the set stored one step ago); k-steps 2 and 3, when
            // refilling: one column block each of the weights of step i + D.
            // The weights go after the activations, so that the wait for
            // these activations (at the end of step i + XS - 1) does not
            // also wait for them.
            static_assert(JW == 2, "one column block per late k-step");
            auto hook = [&](int s) __attribute__((always_inline)) {
                if (s < 2)
                    load_x(u % XS, i + XS, s);
                if constexpr (REFILL) {
                    if (s >= 2)
                        issue_w1(u, i + D, s - 2);
                }
            };
            if (REFILL || i < nk) {                         // uniform; always true while refilling
                if constexpr (GROUPED) {
                    // a new group's scale/zero, selected without a branch
                    // (a branch here made the compiler drain every load in
                    // flight at each step)
                    const bool chg = i == 0 || ((kb0 + i) % ppg) == 0;
                    uint32_t v[JW];
#pragma unroll
                    for (int j = 0; j < JW; ++j) {
                        v[j] = chg ? szr[u][j] : szcur[j];
                        szcur[j] = v[j];
                    }
                    set_sz(v);
                }
                compute(i, wv, hook);
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    hook(s);
            }
            store_x((u + 1) % XS, (u + 1) & 1);            // step i + 1, loaded XS - 1 steps ago
            __syncthreads();
        }
    };
    int i0 = 0;
    for (; i0 + D < nk; i0 += D)
        chunk(i0, std::true_type{});
    chunk(i0, std::false_type{});

    if (FUSED && a.ec_q > 0)
        ec_reduce_units<ACT, BM>(a, tm, m0, smem, s_ec);
    gemm_tail<ACT, BM, GROUPED, 8, LDSB>(a, acc, sf, zf, szsrc, tm, tn, kz, m0, n0, smem, s_old, s_ec, rsl);
    // fused EC: the last workgroup of the tile row to be done with the
    // counters returns them to zero
    if (FUSED && a.ec_q > 0 && tid == 0) {
        if (atomic_add_dev(&a.eccnt[3 * a.mt + tm], 1u) == (uint32_t)(a.nt * a.ksplit - 1)) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                atomic_store_dev(&a.eccnt[c * a.mt + tm], 0u);
        }
    }
}

template <int ACT, int BM, bool GROUPED>
static hipError_t launch_gemm_t(const GemmKArgs& k, hipStream_t st)
{
    dim3 grid(k.mt * k.nt, k.ksplit);
    hipLaunchKernelGGL((prefill_gemm_kernel<ACT, BM, GROUPED>), grid, dim3(GEMM_THREADS), 0, st, k);
    return hipGetLastError();
}

template <int ACT>
static hipError_t launch_gemm_act(const GemmKArgs& k, int BM, bool grouped, hipStream_t st)
{
    if (BM == 64)
        return grouped ? launch_gemm_t<ACT, 64, true>(k, st) : launch_gemm_t<ACT, 64, false>(k, st);
    return grouped ? launch_gemm_t<ACT, 128, true>(k, st) : launch_gemm_t<ACT, 128, false>(k, st);
}


// The gate / X A prepass and its reduction: T_g (and, for the GEMM's bf16
// per-channel zero-point term, each token's activation sum) in the workspace.
static hipError_t launch_prefill_ec_part(const LayerArgs& a, const PrefillPlan& p, bool sums, hipStream_t st)
{
    uint16_t* tg = (uint16_t*)(a.ws + p.off_tg);
    float* rowsum = (float*)(a.ws + p.off_rowsum);
    {
        PrepassKArgs q;
        q.X = (const uint16_t*)a.X;
        q.A = (const uint16_t*)a.A;
        q.w_g = (const uint16_t*)a.w_g;
        q.one2 = !sums ? 0u : 0x3F803F80u;                   // bf16 ones
        q.M = a.M; q.K = a.K; q.r = a.r;
        q.kc = p.pre_kc; q.ks = p.pre_ks; q.nch = p.pre_nch;
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
        rq.rowsum = sums ? rowsum : nullptr;
        rq.b_g = a.b_g;
        rq.r = a.r; rq.r_pad = p.r_pad; rq.ks = p.pre_ks;
        rq.G1 = (const uint16_t*)a.G1; rq.c1 = (const uint16_t*)a.c1;
        rq.G2 = (const uint16_t*)a.G2; rq.c2 = (const uint16_t*)a.c2;
        rq.h = a.h;
        if (a.r > 0 && a.h > 0) {
            auto vk = a.act == ACT_F16 ? ec_reduce_vgate_kernel<ACT_F16> : ec_reduce_vgate_kernel<ACT_BF16>;
            const size_t gbytes = (size_t)vgate_stage_elems(a.r, a.h) * 2;
            rq.vg_staged = vgate_stageable(a.r, a.h);    // at most 8 KB
            hipLaunchKernelGGL(vk, dim3(p.pre_mt * 16), dim3(PF_THREADS), rq.vg_staged ? gbytes : 0, st, rq);
        } else {
            auto rk = a.act == ACT_F16 ? ec_reduce_kernel<ACT_F16> : ec_reduce_kernel<ACT_BF16>;
            hipLaunchKernelGGL(rk, dim3(p.pre_mt * 4, a.r > 0 ? ec_a_blocks(a.r) : 1), dim3(PF_THREADS), 0, st, rq);
        }
        return hipGetLastError();
    }
}

hipError_t launch_prefill_ec_gate(const LayerArgs& a, const PrefillPlan& p, hipStream_t st)
{
    return launch_prefill_ec_part(a, p, false, st);
}

// Compute units of the current device (looked up once per device).
static hipError_t resident_cus(int* out)
{
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    int n = dev < 64 ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (n == 0) {
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
        if (dev < 64)
            cache[dev].store(n, std::memory_order_relaxed);
    }
    *out = n;
    return hipSuccess;
}

hipError_t launch_prefill(const LayerArgs& a, const PrefillPlan& p, hipStream_t st)
{
    BlobGeom g = blob_geom(a.N, a.K, a.G);
    uint16_t* tg = (uint16_t*)(a.ws + p.off_tg);
    const bool sums = a.act == ACT_BF16 && a.G == a.K;   // the GEMM's bf16 zero-point term
    float* rowsum = (float*)(a.ws + p.off_rowsum);
    if (a.S) {
        // salient channels: activation sums only if the GEMM needs them
        // (the prepass without a compensator), then the gather
        if (sums) {
            LayerArgs b = a;
            b.r = 0; b.A = nullptr; b.w_g = nullptr; b.S = nullptr;
            hipError_t e = launch_prefill_ec_part(b, p, true, st);   // its slices fit r = 0 too
            if (e != hipSuccess)
                return e;
        }
        GatherKArgs ga;
        ga.X = (const uint16_t*)a.X;
        ga.S = a.S;
        ga.tg = tg;
        ga.flags = (uint32_t*)(a.ws + p.off_flags);
        ga.M = a.M; ga.K = a.K; ga.s = a.r; ga.r_pad = p.r_pad;
        ga.rows = p.pre_mt * 64;
        const int n = ga.rows * ga.r_pad;
        hipLaunchKernelGGL(serq_gather_kernel, dim3((n + PF_THREADS - 1) / PF_THREADS), dim3(PF_THREADS), 0, st, ga);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    // the fused EC needs every workgroup resident at once (one per CU: the
    // GEMM's workgroups hold a CU's registers)
    bool fused = false;
    if (!a.S && a.h == 0 && (a.r > 0 || sums) && p.ec_q > 0) {
        int cus = 0;
        hipError_t e = resident_cus(&cus);
        if (e != hipSuccess)
            return e;
        fused = (long long)p.mt * p.nt * p.ksplit <= cus;
    }
    if (!a.S && !fused && (a.r > 0 || sums)) {
        hipError_t e = launch_prefill_ec_part(a, p, sums, st);
        if (e != hipSuccess)
            return e;
    }
    GemmKArgs k;
    k.X = (const uint16_t*)a.X;
    k.codes = (const uint8_t*)a.packed + g.codes_off;
    k.sz = (const uint32_t*)((const char*)a.packed + g.sz_off);
    k.B = (const uint16_t*)a.B;
    k.tg = tg;
    k.rowsum = rowsum;
    k.Y = (uint16_t*)a.Y;
    k.partial = (floatx4*)(a.ws + p.off_gemm_partial);
    k.cnt = (uint32_t*)(a.ws + p.off_gemm_cnt);
    k.A = (const uint16_t*)a.A;
    k.w_g = (const uint16_t*)a.w_g;
    k.b_g = a.b_g;
    k.one2 = !sums ? 0u : 0x3F803F80u;                   // bf16 ones
    k.ecp = (floatx4*)(a.ws + p.off_pre_partial);
    k.eccnt = (uint32_t*)(a.ws + p.off_ec_cnt);
    k.flags = (uint32_t*)(a.ws + p.off_flags);
    k.spin = a.spin;
    k.ec_q = fused ? p.ec_q : 0;
    k.ec_kc = p.ec_kc;
    k.M = a.M; k.N = a.N; k.K = a.K; k.r = a.r; k.r_pad = p.r_pad; k.G = a.G;
    k.NB = g.NB; k.KB = g.KB; k.Npad = g.Npad;
    k.mt = p.mt; k.nt = p.nt; k.ksplit = p.ksplit; k.Mpad = p.Mpad;
    const bool grouped = a.G != a.K;
    if (a.act == ACT_F16)
        return launch_gemm_act<ACT_F16>(k, p.BM, grouped, st);
    return launch_gemm_act<ACT_BF16>(k, p.BM, grouped, st);
}

}  // namespace w4ec
