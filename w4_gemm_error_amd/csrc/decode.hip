// decode.hip -- the W4 + EC layer for 1..16 tokens in a single kernel launch.
//
// SPEAR (gist.science technical summary, section 2.2A): in the decode phase
// the layer is memory bound, and the EC is folded into the low-bit GEMM's
// epilogue so that no second launch sits on the critical path.  Here one
// grid does all of it:
//
//  * workgroups [0, P): "EC" role.  Each reads one K-slice of X, A and w_g
//    and writes partial sums of T = X A and of the gate logit X . w_g.  The
//    last of them to finish (arrival counter) adds the P partials in a fixed
//    order, applies the sigmoid gate and stores T_g = g * T in the
//    activation format, then raises a ready flag.
//  * workgroups [P, P + n_main): "main" role.  Each owns CB blocks of 16
//    output columns; its four wavefronts split K.  A wavefront streams its
//    share of the packed weights with one 16-byte load per lane per panel
//    (16 columns x 128 k), turns the codes into (q - z) with a few integer
//    and packed-half operations, and accumulates X Wd^T with
//    v_mfma_f32_16x16x32 (X rows are the 16 MFMA rows; unused rows are zero).
//    Per-group sums are scaled by s when the group changes.  After an LDS
//    reduction over the wavefronts, the epilogue waits for the ready flag
//    and extends the reduction by the r rank terms: acc += T_g B, again as
//    MFMAs, then rounds and stores Y.
//
// The EC workgroups have the lowest ids, so they are dispatched before any
// main workgroup can occupy the GPU while waiting; the wait is bounded.
// The last main workgroup returns the counters to zero.
#include "w4ec_common.h"
#include "w4ec_launch.h"

namespace w4ec {

constexpr int DEC_THREADS = 256;
constexpr int EC_KS_MAX = 256;

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
    uint32_t* flags;   // [0] EC arrivals, [1] ready, [2] main done, [3] wait timed out
    float* partial;    // [P][16][RC]
    uint16_t* tg;      // [16][r_pad], activation format
};

template <int ACT>
__device__ void decode_ec_role(const DecodeKArgs& a, float* smem)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int b = blockIdx.x;
    const int M = a.M;
    const int k0 = b * a.KS;
    const int len = min(a.KS, a.K - k0);
    float* xs = smem;                        // [16][EC_KS_MAX]
    float* redT = smem + 16 * EC_KS_MAX;     // [4][16][64]
    float* gsum = redT + 4 * 16 * 64;        // [4][16]
    float* gsh = gsum + 64;                  // [16]

    for (int idx = tid; idx < M * len; idx += DEC_THREADS) {
        int m = idx / len, kk = idx - m * len;
        xs[m * EC_KS_MAX + kk] = act_to_f32<ACT>(a.X[(size_t)m * a.K + k0 + kk]);
    }
    __syncthreads();

    // gate logit partial: thread t takes k0 + t
    {
        float wv = 0.0f;
        if (a.w_g && tid < len)
            wv = act_to_f32<ACT>(a.w_g[k0 + tid]);
        for (int m = 0; m < M; ++m) {
            float v = (tid < len) ? xs[m * EC_KS_MAX + tid] * wv : 0.0f;
            for (int off = 32; off > 0; off >>= 1)
                v += __shfl_xor(v, off);
            if (lane == 0)
                gsum[wave * 16 + m] = v;
        }
    }

    // T partial: lane = column, wavefront = k phase (k0 + wave + 4i)
    for (int c0 = 0; c0 < a.r; c0 += 64) {
        const int c = c0 + lane;
        float acc[16];
#pragma unroll
        for (int m = 0; m < 16; ++m)
            acc[m] = 0.0f;
        if (c < a.r) {
            for (int kk = wave; kk < len; kk += 4) {
                float av = act_to_f32<ACT>(a.A[(size_t)(k0 + kk) * a.r + c]);
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    if (m < M)
                        acc[m] += xs[m * EC_KS_MAX + kk] * av;
            }
        }
#pragma unroll
        for (int m = 0; m < 16; ++m)
            redT[(wave * 16 + m) * 64 + lane] = acc[m];
        __syncthreads();
        float* part = a.partial + (size_t)b * 16 * a.RC;
        for (int idx = tid; idx < M * 64; idx += DEC_THREADS) {
            int m = idx >> 6, cl = idx & 63;
            if (c0 + cl < a.r) {
                float s = redT[(0 * 16 + m) * 64 + cl] + redT[(1 * 16 + m) * 64 + cl] +
                          redT[(2 * 16 + m) * 64 + cl] + redT[(3 * 16 + m) * 64 + cl];
                part[m * a.RC + c0 + cl] = s;
            }
        }
        __syncthreads();
    }
    if (tid < M) {
        float s = gsum[0 * 16 + tid] + gsum[1 * 16 + tid] + gsum[2 * 16 + tid] + gsum[3 * 16 + tid];
        a.partial[(size_t)b * 16 * a.RC + tid * a.RC + a.r] = s;
    }

    // hand over: the last EC workgroup reduces all slices
    fence_release();
    __syncthreads();
    __shared__ uint32_t s_old;
    if (tid == 0)
        s_old = atomic_add_acq_rel(&a.flags[0], 1u);
    __syncthreads();
    if (s_old != (uint32_t)(a.P - 1))
        return;
    fence_acquire();
    if (tid < 16) {
        float g = 0.0f;
        if (tid < M) {
            float l = 0.0f;
            for (int p = 0; p < a.P; ++p)
                l += a.partial[((size_t)p * 16 + tid) * a.RC + a.r];
            g = sigmoid_f32(l + a.b_g);
        }
        gsh[tid] = g;
    }
    __syncthreads();
    for (int idx = tid; idx < 16 * a.r_pad; idx += DEC_THREADS) {
        int m = idx / a.r_pad, j = idx - m * a.r_pad;
        float v = 0.0f;
        if (m < M && j < a.r) {
            float t = 0.0f;
            for (int p = 0; p < a.P; ++p)
                t += a.partial[((size_t)p * 16 + m) * a.RC + j];
            v = gsh[m] * t;
        }
        a.tg[idx] = f32_to_act<ACT>(v);
    }
    fence_release();
    __syncthreads();
    if (tid == 0)
        atomic_store_release(&a.flags[1], 1u);
}

template <int ACT, int CB, int U>
__device__ void decode_main_role(const DecodeKArgs& a, float* smem)
{
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int w = tid >> 6;
    const int cb0 = (blockIdx.x - a.P) * CB;
    const int M = a.M;
    const int KB = a.KB;

    // this wavefront's panels along K
    const int per = KB >> 2, rem = KB & 3;
    const int kbeg = w * per + min(w, rem);
    const int kcnt = per + (w < rem ? 1 : 0);

    const int row = l & 15;
    const int koff = 8 * (l >> 4);
    const bool xrow = row < M;
    const uint16_t* xp = a.X + (size_t)(xrow ? row : 0) * a.K + koff;

    floatx4 acc[CB], accg[CB];
    float s_cur[CB];
    DqF16 dqh[CB];
    float dqb[CB];
    int n_l[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) {
        acc[j] = (floatx4){0.f, 0.f, 0.f, 0.f};
        accg[j] = acc[j];
        s_cur[j] = 0.0f;
        dqh[j] = dq_f16_consts(0.0f);
        dqb[j] = 0.0f;
        n_l[j] = (cb0 + j) * PANEL_N + (l & 15);
    }
    int cur_g = -1;

    for (int kc = 0; kc < kcnt; kc += U) {
        u32x4 xf[U][4];
        u32x4 wq[U][CB];
        uint32_t szv[U][CB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (kc + u < kcnt) {
                const int kb = kbeg + kc + u;
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    xf[u][s] = xrow ? ld16(xp + (size_t)kb * PANEL_K + 32 * s) : (u32x4){0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (kc + u < kcnt) {
                const int kb = kbeg + kc + u;
                const int grp = (kb * PANEL_K) / a.G;
#pragma unroll
                for (int j = 0; j < CB; ++j) {
                    if (cb0 + j < a.NB) {
                        wq[u][j] = ld16_stream(a.codes + ((size_t)(cb0 + j) * KB + kb) * PANEL_BYTES + l * 16);
                        szv[u][j] = a.sz[(size_t)grp * a.Npad + n_l[j]];
                    } else {
                        wq[u][j] = (u32x4){0u, 0u, 0u, 0u};
                        szv[u][j] = 0u;
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (kc + u < kcnt) {
                const int kb = kbeg + kc + u;
                const int grp = (kb * PANEL_K) / a.G;
                if (grp != cur_g) {
#pragma unroll
                    for (int j = 0; j < CB; ++j) {
                        acc[j] += s_cur[j] * accg[j];
                        accg[j] = (floatx4){0.f, 0.f, 0.f, 0.f};
                        const uint32_t v = szv[u][j];
                        s_cur[j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFF));
                        const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
                        if constexpr (ACT == ACT_F16)
                            dqh[j] = dq_f16_consts(z);
                        else
                            dqb[j] = -(8388608.0f + z);
                    }
                    cur_g = grp;
                }
#pragma unroll
                for (int j = 0; j < CB; ++j) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        u32x4 bq;
                        if constexpr (ACT == ACT_F16)
                            bq = dequant_f16(wq[u][j][s], dqh[j]);
                        else
                            bq = dequant_bf16(wq[u][j][s], dqb[j]);
                        accg[j] = mfma16x16x32<ACT>(xf[u][s], bq, accg[j]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < CB; ++j)
        acc[j] += s_cur[j] * accg[j];

    // reduce the four K shares (fixed order)
    floatx4* red = reinterpret_cast<floatx4*>(smem);   // [4][CB][64]
#pragma unroll
    for (int j = 0; j < CB; ++j)
        red[(w * CB + j) * 64 + l] = acc[j];
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
            // B fragment rows koff + t of each 32-deep rank step, column n
            u32x4 bfr[8];
            const int nsteps = a.r_pad >> 5;
#pragma unroll
            for (int rs = 0; rs < 8; ++rs) {
                if (rs < nsteps) {
                    uint32_t hv[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const int jr = 32 * rs + koff + t;
                        hv[t] = (jr < a.r && n < a.N) ? (uint32_t)a.B[(size_t)jr * a.N + n] : 0u;
                    }
                    bfr[rs] = (u32x4){hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16),
                                      hv[4] | (hv[5] << 16), hv[6] | (hv[7] << 16)};
                }
            }
            // wait (bounded) for T_g
            if (l == 0) {
                uint32_t it = 0;
                while (atomic_load_acquire(&a.flags[1]) == 0u) {
                    __builtin_amdgcn_s_sleep(2);
                    if (++it >= SPIN_LIMIT) {
                        atomic_store_relaxed(&a.flags[3], 1u);
                        break;
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
            fence_acquire();
#pragma unroll
            for (int rs = 0; rs < 8; ++rs) {
                if (rs < nsteps) {
                    u32x4 af = ld16(a.tg + (size_t)row * a.r_pad + 32 * rs + koff);
                    tot = mfma16x16x32<ACT>(af, bfr[rs], tot);
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

    if (a.r > 0) {
        __syncthreads();
        if (tid == 0) {
            uint32_t old = atomic_add_acq_rel(&a.flags[2], 1u);
            if (old == (uint32_t)(a.n_main - 1)) {
                atomic_store_relaxed(&a.flags[0], 0u);
                atomic_store_relaxed(&a.flags[1], 0u);
                atomic_store_release(&a.flags[2], 0u);
            }
        }
    }
}

template <int ACT, int CB, int U>
__global__ __launch_bounds__(DEC_THREADS)
void decode_kernel(DecodeKArgs a)
{
    // EC role: 16 x 256 staged activations + 4 x 16 x 64 reduction + small;
    // main role: 4 x CB x 64 float4.
    __shared__ float smem[16 * EC_KS_MAX + 4 * 16 * 64 + 64 + 16];
    static_assert(4 * CB * 64 * 4 <= 16 * EC_KS_MAX + 4 * 16 * 64, "main-role LDS");
    if ((int)blockIdx.x < a.P)
        decode_ec_role<ACT>(a, smem);
    else
        decode_main_role<ACT, CB, U>(a, smem);
}

template <int ACT, int CB>
static hipError_t launch_decode_t(const DecodeKArgs& k, hipStream_t st)
{
    dim3 grid(k.P + k.n_main);
    hipLaunchKernelGGL((decode_kernel<ACT, CB, 4>), grid, dim3(DEC_THREADS), 0, st, k);
    return hipGetLastError();
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
    k.flags = (uint32_t*)(a.ws + p.off_flags);
    k.partial = (float*)(a.ws + p.off_partial);
    k.tg = (uint16_t*)(a.ws + p.off_tg);
    if (a.act == ACT_F16) {
        if (p.CB == 1) return launch_decode_t<ACT_F16, 1>(k, st);
        return launch_decode_t<ACT_F16, 2>(k, st);
    }
    if (p.CB == 1) return launch_decode_t<ACT_BF16, 1>(k, st);
    return launch_decode_t<ACT_BF16, 2>(k, st);
}

}  // namespace w4ec
