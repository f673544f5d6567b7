// api.cpp -- the C ABI of libw4ec (declared in include/w4ec.h): argument
// validation, launch plans, workspace sizing and dispatch to the kernels.
// Validation makes no HIP call, so every argument error is reported before
// anything touches the device.
#include "w4ec.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <new>

#include "w4ec_common.h"
#include "w4ec_launch.h"

using namespace w4ec;

namespace {

constexpr int MAX_RANK = 256;
constexpr int DECODE_MAX_M = 16;
constexpr int TARGET_WGS = 256;   // one workgroup per CU for the large-tile kernels

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_weight_shape(int N, int K, int G)
{
    if (N <= 0 || K <= 0 || G <= 0)
        return W4EC_ERR_INVALID_ARG;
    if (K % PANEL_K != 0)
        return W4EC_ERR_UNSUPPORTED;
    if (G != K && (G % PANEL_K != 0 || K % G != 0))
        return W4EC_ERR_UNSUPPORTED;
    if ((long long)N * K > (1LL << 40))
        return W4EC_ERR_UNSUPPORTED;
    return W4EC_OK;
}

// Workspace layout, shared by both entry points so that one workspace can
// serve decode and prefill calls in any order:
//   [0, CTRL_BYTES)   state that every call returns to zero and that no
//                     call overwrites with anything else: decode flags,
//                     split-K tile counters, the decode replica slots'
//                     counters and data, the decode EC partial sums (decode
//                     hand-over words announce themselves by being nonzero)
//   [CTRL_BYTES, ...) per-call data of the prefill kernels (partial sums,
//                     gated activations), fully written before it is read
//                     within a call
constexpr size_t CTRL_BYTES = W4EC_WS_STATE_BYTES;

constexpr size_t OFF_DEC_FLAGS = 0;           // 256 B
constexpr size_t OFF_GEMM_CNT = 256 + 1024;   // split-K tile counters, <= 256 of them
constexpr size_t OFF_EC_CNT = 4 << 10;        // fused-EC counters, 4 per row of tiles, <= 256 rows
constexpr size_t OFF_DEC_REP = 64 << 10;      // DEC_NREP decode slots of DEC_REP_CTRL_STRIDE bytes
constexpr size_t OFF_DEC_REP_DATA = 256 << 10;  // DEC_NREP slots of DEC_REP_DATA_STRIDE bytes
constexpr size_t OFF_DEC_PARTIAL = 512 << 10;   // decode EC partial sums, up to CTRL_BYTES
static_assert(OFF_GEMM_CNT + 256 * 4 <= OFF_EC_CNT && OFF_EC_CNT + 4 * 256 * 4 <= OFF_DEC_REP, "control region");
static_assert(OFF_DEC_REP + DEC_NREP * DEC_REP_CTRL_STRIDE <= OFF_DEC_REP_DATA, "control region");
static_assert(OFF_DEC_REP_DATA + DEC_NREP * DEC_REP_DATA_STRIDE <= OFF_DEC_PARTIAL, "control region");

DecodePlan make_decode_plan(int M, int N, int K, int r)
{
    DecodePlan p{};
    const int NB = (N + PANEL_N - 1) / PANEL_N;
    p.RC = r + 1;
    p.r_pad = (r + 31) / 32 * 32;
    if (r > 0) {
        // each EC workgroup loads its whole slice in one trip (KS a multiple
        // of 64, <= DEC_EC_KS); the slice and its gate vector in LDS stay
        // within 40 KB, so that 4 workgroups fit on a CU
        int ks = DEC_EC_KS;
        while (ks > 64 && (((ks * ((r + 3) & ~3) + 16) * 2 + ks * 2) > 40960))
            ks -= 64;
        p.KS = ks;
        p.P = (K + p.KS - 1) / p.KS;
    }
    p.xlds = decode_use_xlds(M, K);
    // column blocks per workgroup: two when X is staged in LDS (X staged once
    // for twice the weights); one for a few tokens with a long K; for more
    // tokens four, so that each activation fragment loaded from L2 feeds
    // four blocks' MFMAs -- unless that leaves too few workgroups: below 512
    // column blocks (N < 8192) two (N = 4096, 12 tokens, K = 14336, G = 128:
    // 27.8 -> 22.6 us; 8 tokens at K = 4096: 10.1 -> 9.5 us; from N = 8192
    // on, four measured faster)
    p.CB = p.xlds ? 2 : (M <= 4 ? 1 : (NB >= 512 ? 4 : 2));
    p.n_main = (NB + p.CB - 1) / p.CB;
    // X is staged after the weight ring is issued, also with an EC: since the
    // EC reduction runs on few reducers its chain no longer gains from
    // having memory to itself first (10.3 against 10.45 us at one token,
    // the same at four and sixteen)
    p.stage_first = 0;
    p.off_flags = OFF_DEC_FLAGS;
    p.off_rep_ctrl = OFF_DEC_REP;
    p.off_rep_data = OFF_DEC_REP_DATA;
    p.off_partial = OFF_DEC_PARTIAL;
    // the EC partial sums must fit the control region (K up to ~60k at
    // r = 256 and 16 tokens, far more at lower rank or fewer tokens)
    p.ok = r == 0 || OFF_DEC_PARTIAL + (size_t)p.P * M * p.RC * 4 <= CTRL_BYTES;
    p.bytes = CTRL_BYTES;
    return p;
}

constexpr size_t PRE_LDS_MAX = 80 << 10;

PrefillPlan make_prefill_plan(int M, int N, int K, int r)
{
    PrefillPlan p{};
    const int NB = (N + PANEL_N - 1) / PANEL_N;
    const int KB = K / PANEL_K;
    p.BN = 256;
    p.nt = (NB * PANEL_N + p.BN - 1) / p.BN;
    p.BM = M <= 64 ? 64 : 128;
    // With few tiles the K split that fills the chip writes and reads
    // ksplit x M x N fp32 partial sums; when 128-token tiles would need a
    // split of 4 or more, 64-token tiles halve that traffic.
    if (p.BM == 128 && (long long)((M + 127) / 128) * p.nt * 4 <= TARGET_WGS)
        p.BM = 64;
    p.mt = (M + p.BM - 1) / p.BM;
    p.ksplit = 1;
    // split K only while the workgroups still fit in one round (one per CU)
    while ((long long)p.mt * p.nt * p.ksplit * 2 <= TARGET_WGS && KB / (2 * p.ksplit) >= 4 && p.ksplit < 16)
        p.ksplit *= 2;
    p.Mpad = p.mt * p.BM;
    p.r_pad = (r + 31) / 32 * 32;
    // prepass: 64-token tiles x K slices of at most 512, each slice of
    // [A | w_g] held in LDS at once (two workgroups per CU)
    p.pre_mt = (M + 63) / 64;
    // (the prepass also runs with r == 0 for bf16 per-channel weights: the
    // GEMM then needs each token's activation sum)
    p.pre_ks = 1;
    p.pre_kc = K;
    {
        int kcmax = 512;
        while (kcmax > 64 && prepass_lds_bytes(r, kcmax) > PRE_LDS_MAX)
            kcmax -= 64;
        const int ks = (K + kcmax - 1) / kcmax;
        p.pre_kc = ((K + ks - 1) / ks + 63) / 64 * 64;
        p.pre_ks = (K + p.pre_kc - 1) / p.pre_kc;
        // a grid of more than one round of workgroups (two per CU): each
        // takes several chunks of K one after another, so that the grid fits
        // one round and writes fewer partial sums (up to four chunks)
        p.pre_nch = 1;
        while (p.pre_nch < 4 && (long long)p.pre_mt * ((p.pre_ks + p.pre_nch - 1) / p.pre_nch) > 2 * TARGET_WGS)
            p.pre_nch *= 2;
        p.pre_ks = (p.pre_ks + p.pre_nch - 1) / p.pre_nch;
    }
    // tile counters exist only for split work, which is chosen only while the
    // workgroup count is below TARGET_WGS: at most 256 of them
    p.off_gemm_cnt = OFF_GEMM_CNT;
    p.off_ec_cnt = OFF_EC_CNT;
    p.off_flags = OFF_DEC_FLAGS;
    // Fused EC for a single row of 64-token tiles (M <= 64), when every
    // workgroup is resident at once: the prepass would have one workgroup
    // per K slice only, so the GEMM's workgroups do it instead.  Each of the
    // first ec_q workgroups computes [T | l] for the row's tokens over about
    // K / ec_q of K, a range whose rows of [A | w_g] fit the GEMM's LDS at
    // once (at most ec_kc of them).  (With more rows of tiles the prepass
    // kernels measured faster: the pieces' reduction, a chain of trips to
    // memory after the main loop, then costs more than the launches.)
    p.ec_q = 0;
    {
        p.ec_kc = 512;
        while (p.ec_kc > 64 && prepass_lds_bytes(r, p.ec_kc) > (size_t)GEMM_EC_LDS)
            p.ec_kc -= 64;
        const long long W = (long long)p.mt * p.nt * p.ksplit;
        const int K64 = K / 64;
        const int q = std::min(p.nt * p.ksplit, K64);
        const int piece = 64 * ((K64 + q - 1) / q);
        if (M <= 64 && p.BM == 64 && W <= TARGET_WGS && piece <= p.ec_kc)
            p.ec_q = q;
    }

    size_t off = CTRL_BYTES;
    p.off_pre_partial = off;   // the prepass's partial sums, or the fused EC's pieces
    off = align_up(off + std::max((size_t)p.pre_mt * p.pre_ks * 4, (size_t)p.mt * p.ec_q * (p.BM / 16)) *
                             ((r + 15) / 16 + 1) * 64 * 16,
                   256);
    p.off_tg = off;
    if (r > 0)
        off = align_up(off + (size_t)p.Mpad * p.r_pad * 2, 256);
    p.off_rowsum = off;
    off = align_up(off + (size_t)std::max(p.Mpad, p.pre_mt * 64) * sizeof(float), 256);
    p.off_gemm_partial = off;
    if (p.ksplit > 1)
        off = align_up(off + (size_t)p.ksplit * p.Mpad * p.nt * p.BN * sizeof(float), 256);
    p.bytes = off;
    return p;
}

int check_layer_args(const void* X, const void* packed, const void* A, const void* B,
                     const void* w_g, const void* Y, int M, int N, int K, int r, int G, int act,
                     const void* ws, size_t ws_bytes, size_t need)
{
    if (M <= 0 || r < 0)
        return W4EC_ERR_INVALID_ARG;
    int rc = check_weight_shape(N, K, G);
    if (rc != W4EC_OK)
        return rc;
    if (r > MAX_RANK)
        return W4EC_ERR_UNSUPPORTED;
    if (act != W4EC_FP16 && act != W4EC_BF16)
        return W4EC_ERR_INVALID_ARG;
    if (!X || !packed || !Y)
        return W4EC_ERR_INVALID_ARG;
    if (r > 0 && (!A || !B))
        return W4EC_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(Y, 16) || !aligned(packed, 256))
        return W4EC_ERR_INVALID_ARG;
    if (r > 0 && (!aligned(A, 16) || !aligned(B, 2) || !aligned(w_g, 16)))
        return W4EC_ERR_INVALID_ARG;
    if (X == Y || packed == Y || (r > 0 && (A == Y || B == Y)))
        return W4EC_ERR_INVALID_ARG;
    if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256)))
        return W4EC_ERR_WORKSPACE;
    return W4EC_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? W4EC_OK : W4EC_ERR_HIP; }

// polls a bounded wait makes before it gives up (w4ec_set_wait_limit)
std::atomic<uint32_t> g_wait_limit{SPIN_LIMIT};

}  // namespace

extern "C" {

const char* w4ec_status_str(int status)
{
    switch (status) {
    case W4EC_OK: return "W4EC_OK";
    case W4EC_ERR_INVALID_ARG: return "W4EC_ERR_INVALID_ARG";
    case W4EC_ERR_UNSUPPORTED: return "W4EC_ERR_UNSUPPORTED";
    case W4EC_ERR_WORKSPACE: return "W4EC_ERR_WORKSPACE";
    case W4EC_ERR_HIP: return "W4EC_ERR_HIP";
    case W4EC_ERR_TIMED_OUT: return "W4EC_ERR_TIMED_OUT";
    case W4EC_ERR_BAD_INDEX: return "W4EC_ERR_BAD_INDEX";
    default: return "W4EC_UNKNOWN_STATUS";
    }
}

size_t w4ec_packed_bytes(int N, int K, int group_size)
{
    if (check_weight_shape(N, K, group_size) != W4EC_OK)
        return 0;
    return blob_geom(N, K, group_size).bytes;
}

int w4ec_quantize_rtn(const float* W, int N, int K, int group_size, uint8_t* q_canon,
                      uint16_t* scale, uint16_t* zero, void* stream)
{
    if (N <= 0 || K <= 0 || group_size <= 0 || K % 2 != 0 || group_size % 2 != 0 || K % group_size != 0)
        return W4EC_ERR_INVALID_ARG;
    if (!W || !q_canon || !scale || !zero)
        return W4EC_ERR_INVALID_ARG;
    if (!aligned(W, 4) || !aligned(scale, 2) || !aligned(zero, 2))
        return W4EC_ERR_INVALID_ARG;
    if (K / group_size > 65535 || N > 65535 * 64)
        return W4EC_ERR_UNSUPPORTED;
    if (N > 65535)
        return W4EC_ERR_UNSUPPORTED;
    return hip_status(launch_rtn_quantize(W, N, K, group_size, q_canon, scale, zero, (hipStream_t)stream));
}

int w4ec_pack(const uint8_t* q_canon, const uint16_t* scale, const uint16_t* zero,
              int N, int K, int group_size, void* packed, void* stream)
{
    int rc = check_weight_shape(N, K, group_size);
    if (rc != W4EC_OK)
        return rc;
    if (!q_canon || !scale || !zero || !packed)
        return W4EC_ERR_INVALID_ARG;
    if (!aligned(packed, 256) || !aligned(scale, 2) || !aligned(zero, 2))
        return W4EC_ERR_INVALID_ARG;
    return hip_status(launch_pack(q_canon, scale, zero, N, K, group_size, packed, (hipStream_t)stream));
}

int w4ec_pack_xfp(const uint8_t* idx_canon, int N, int K, void* packed, void* stream)
{
    int rc = check_weight_shape(N, K, K);
    if (rc != W4EC_OK)
        return rc;
    if (!idx_canon || !packed || !aligned(packed, 256))
        return W4EC_ERR_INVALID_ARG;
    return hip_status(launch_pack(idx_canon, nullptr, nullptr, N, K, K, packed, (hipStream_t)stream));
}

int w4ec_unpack(const void* packed, int N, int K, int group_size, uint8_t* q_canon,
                uint16_t* scale, uint16_t* zero, void* stream)
{
    int rc = check_weight_shape(N, K, group_size);
    if (rc != W4EC_OK)
        return rc;
    if (!packed || !q_canon || !scale || !zero)
        return W4EC_ERR_INVALID_ARG;
    if (!aligned(packed, 256) || !aligned(scale, 2) || !aligned(zero, 2))
        return W4EC_ERR_INVALID_ARG;
    return hip_status(launch_unpack(packed, N, K, group_size, q_canon, scale, zero, (hipStream_t)stream));
}

size_t w4ec_workspace_bytes(int M, int N, int K, int r, int group_size)
{
    if (M <= 0 || r < 0 || r > MAX_RANK || check_weight_shape(N, K, group_size) != W4EC_OK)
        return 0;
    size_t b = make_prefill_plan(M, N, K, r).bytes;
    if (M <= DECODE_MAX_M) {
        size_t d = make_decode_plan(M, N, K, r).bytes;
        if (d > b)
            b = d;
    }
    return b;
}

}  // extern "C"

namespace {

constexpr int VGATE_MAX_H = 64;   // widest bottleneck of the vector gate

struct VGate {
    const void* G1;
    const void* c1;
    const void* G2;
    const void* c2;
    int h;
};

// Vector-gate parameters, checked only when there is a compensator (r > 0).
int check_vgate(const VGate* v, int r)
{
    if (!v || r == 0)
        return W4EC_OK;
    if (v->h < 1)
        return W4EC_ERR_INVALID_ARG;
    if (v->h > VGATE_MAX_H)
        return W4EC_ERR_UNSUPPORTED;
    if (!v->G1 || !v->c1 || !v->G2 || !v->c2)
        return W4EC_ERR_INVALID_ARG;
    if (!aligned(v->G1, 2) || !aligned(v->c1, 2) || !aligned(v->G2, 2) || !aligned(v->c2, 2))
        return W4EC_ERR_INVALID_ARG;
    return W4EC_OK;
}

LayerArgs layer_args(const void* X, const void* packed, const void* A, const void* B,
                     const void* w_g, float b_g, void* Y, int M, int N, int K, int r,
                     int group_size, int act_dtype, void* workspace, const VGate* vg)
{
    LayerArgs a{X, packed, r > 0 ? A : nullptr, r > 0 ? B : nullptr, r > 0 ? w_g : nullptr,
                b_g, Y, M, N, K, r, group_size, act_dtype, (char*)workspace};
    a.spin = g_wait_limit.load(std::memory_order_relaxed);
    if (vg && r > 0) {
        a.w_g = nullptr;                 // the vector gate replaces the scalar one
        a.G1 = vg->G1; a.c1 = vg->c1; a.G2 = vg->G2; a.c2 = vg->c2;
        a.h = vg->h;
    }
    return a;
}

int decode_entry(const void* X, const void* packed, const void* A, const void* B,
                 const void* w_g, float b_g, void* Y, int M, int N, int K, int r,
                 int group_size, int act_dtype, void* workspace, size_t workspace_bytes,
                 void* stream, const VGate* vg, const int32_t* S = nullptr, bool noalloc = false)
{
    if (M > DECODE_MAX_M)
        return W4EC_ERR_UNSUPPORTED;
    DecodePlan p{};
    size_t need = 0;
    if (M > 0 && r >= 0 && r <= MAX_RANK && check_weight_shape(N, K, group_size) == W4EC_OK) {
        p = make_decode_plan(M, N, K, r);
        if (!p.ok)
            return W4EC_ERR_UNSUPPORTED;
        // a caller's workspace must hold the whole state region; the static
        // area (noalloc) only the bytes this shape touches: the control
        // words and replica slots, then the EC partial sums
        need = r == 0 ? 0 : noalloc ? OFF_DEC_PARTIAL + (size_t)p.P * M * p.RC * sizeof(uint32_t) : p.bytes;
    }
    int rc = check_layer_args(X, packed, A, B, vg ? nullptr : w_g, Y, M, N, K, r, group_size,
                              act_dtype, workspace, workspace_bytes, noalloc ? 0 : need);
    if (rc != W4EC_OK)
        return rc;
    rc = check_vgate(vg, r);
    if (rc != W4EC_OK)
        return rc;
    if (!vg && w_g && !((uintptr_t)w_g % 2 == 0))
        return W4EC_ERR_INVALID_ARG;
    if (noalloc && need > 0) {
        if (need > W4EC_NOALLOC_SCRATCH_BYTES)
            return W4EC_ERR_UNSUPPORTED;
        const hipError_t e = noalloc_scratch(&workspace, (hipStream_t)stream);
        if (e == hipErrorInvalidDevice)
            return W4EC_ERR_UNSUPPORTED;
        if (e != hipSuccess)
            return W4EC_ERR_HIP;
    }
    LayerArgs a = layer_args(X, packed, A, B, w_g, b_g, Y, M, N, K, r, group_size, act_dtype,
                             need > 0 ? workspace : nullptr, vg);
    if (S && r > 0) {
        // salient channels: the main workgroups gather their own operand,
        // no EC workgroups and no hand-over
        a.S = S;
        a.A = nullptr;
        a.w_g = nullptr;
        p.P = 0;
        p.stage_first = 0;
    }
    return hip_status(launch_decode(a, p, (hipStream_t)stream));
}

int prefill_entry(const void* X, const void* packed, const void* A, const void* B,
                  const void* w_g, float b_g, void* Y, int M, int N, int K, int r,
                  int group_size, int act_dtype, void* workspace, size_t workspace_bytes,
                  void* stream, const VGate* vg, const int32_t* S = nullptr)
{
    PrefillPlan p{};
    size_t need = 0;
    if (M > 0 && r >= 0 && r <= MAX_RANK && check_weight_shape(N, K, group_size) == W4EC_OK) {
        p = make_prefill_plan(M, N, K, r);
        const bool sums = act_dtype == W4EC_BF16 && group_size == K;   // bf16 zero-point term
        need = (r > 0 || p.ksplit > 1 || sums) ? p.bytes : 0;
    }
    int rc = check_layer_args(X, packed, A, B, vg ? nullptr : w_g, Y, M, N, K, r, group_size,
                              act_dtype, workspace, workspace_bytes, need);
    if (rc != W4EC_OK)
        return rc;
    rc = check_vgate(vg, r);
    if (rc != W4EC_OK)
        return rc;
    if (!vg && w_g && !((uintptr_t)w_g % 2 == 0))
        return W4EC_ERR_INVALID_ARG;
    LayerArgs a = layer_args(X, packed, A, B, w_g, b_g, Y, M, N, K, r, group_size, act_dtype,
                             need > 0 ? workspace : nullptr, vg);
    if (S && r > 0) {
        a.S = S;
        a.A = nullptr;
        a.w_g = nullptr;
    }
    return hip_status(launch_prefill(a, p, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int w4ec_linear_decode(const void* X, const void* packed, const void* A, const void* B,
                       const void* w_g, float b_g, void* Y, int M, int N, int K, int r,
                       int group_size, int act_dtype, void* workspace, size_t workspace_bytes,
                       void* stream)
{
    return decode_entry(X, packed, A, B, w_g, b_g, Y, M, N, K, r, group_size, act_dtype,
                        workspace, workspace_bytes, stream, nullptr);
}

int w4ec_linear_decode_noalloc(const void* X, const void* packed, const void* A, const void* B,
                               const void* w_g, float b_g, void* Y, int M, int N, int K, int r,
                               int group_size, int act_dtype, void* stream)
{
    return decode_entry(X, packed, A, B, w_g, b_g, Y, M, N, K, r, group_size, act_dtype, nullptr, 0,
                        stream, nullptr, nullptr, true);
}

int w4ec_linear_prefill(const void* X, const void* packed, const void* A, const void* B,
                        const void* w_g, float b_g, void* Y, int M, int N, int K, int r,
                        int group_size, int act_dtype, void* workspace, size_t workspace_bytes,
                        void* stream)
{
    return prefill_entry(X, packed, A, B, w_g, b_g, Y, M, N, K, r, group_size, act_dtype,
                         workspace, workspace_bytes, stream, nullptr);
}

// The prefill plan's EC regions (prepass partial sums, T_g) depend on M, K
// and r only; any N gives the same offsets.
static PrefillPlan ec_plan(int M, int K, int r) { return make_prefill_plan(M, 16, K, r); }

size_t w4ec_prefill_ec_workspace_bytes(int M, int K, int r)
{
    if (M <= 0 || r < 1 || r > MAX_RANK || K <= 0 || K % PANEL_K != 0)
        return 0;
    const PrefillPlan p = ec_plan(M, K, r);
    return p.off_tg + (size_t)((M + 63) / 64 * 64) * p.r_pad * 2;
}

int w4ec_prefill_ec_gate(const void* X, const void* A, const void* w_g, float b_g, int M, int K,
                         int r, int act_dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    if (M <= 0 || r < 1 || K <= 0)
        return W4EC_ERR_INVALID_ARG;
    if (K % PANEL_K != 0 || r > MAX_RANK)
        return W4EC_ERR_UNSUPPORTED;
    if (act_dtype != W4EC_FP16 && act_dtype != W4EC_BF16)
        return W4EC_ERR_INVALID_ARG;
    if (!X || !A || !aligned(X, 16) || !aligned(A, 16) || !aligned(w_g, 16))
        return W4EC_ERR_INVALID_ARG;
    const size_t need = w4ec_prefill_ec_workspace_bytes(M, K, r);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return W4EC_ERR_WORKSPACE;
    LayerArgs a{X, nullptr, A, nullptr, w_g, b_g, nullptr, M, 16, K, r, K, act_dtype, (char*)workspace};
    return hip_status(launch_prefill_ec_gate(a, ec_plan(M, K, r), (hipStream_t)stream));
}

int w4ec_prefill_ec_apply(void* Y, const void* B, int M, int N, int K, int r, int act_dtype,
                          const void* workspace, size_t workspace_bytes, void* stream)
{
    if (M <= 0 || N <= 0 || r < 1 || K <= 0)
        return W4EC_ERR_INVALID_ARG;
    if (K % PANEL_K != 0 || r > MAX_RANK)
        return W4EC_ERR_UNSUPPORTED;
    if (act_dtype != W4EC_FP16 && act_dtype != W4EC_BF16)
        return W4EC_ERR_INVALID_ARG;
    if (!Y || !B || !aligned(Y, 2) || !aligned(B, 2) || Y == B)
        return W4EC_ERR_INVALID_ARG;
    const size_t need = w4ec_prefill_ec_workspace_bytes(M, K, r);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return W4EC_ERR_WORKSPACE;
    ApplyArgs a{Y, B, M, N, r, act_dtype, (char*)workspace};
    return hip_status(launch_prefill_ec_apply(a, ec_plan(M, K, r), (hipStream_t)stream));
}

// Salient-channel correction: the layer's checks with R standing in for A
// (it is the operand whose presence r > 0 requires), plus S.
static int check_serq(const int32_t* S, const void* R, int s)
{
    if (s > 0 && (!S || !R || !aligned(S, 4) || !aligned(R, 2)))
        return W4EC_ERR_INVALID_ARG;
    return W4EC_OK;
}

int w4ec_linear_decode_serq(const void* X, const void* packed, const int32_t* S, const void* R,
                            void* Y, int M, int N, int K, int s, int group_size, int act_dtype,
                            void* workspace, size_t workspace_bytes, void* stream)
{
    int rc = check_serq(S, R, s);
    if (rc != W4EC_OK)
        return rc;
    return decode_entry(X, packed, s > 0 ? X : nullptr, R, nullptr, 0.0f, Y, M, N, K, s, group_size,
                        act_dtype, workspace, workspace_bytes, stream, nullptr, S);
}

int w4ec_linear_prefill_serq(const void* X, const void* packed, const int32_t* S, const void* R,
                             void* Y, int M, int N, int K, int s, int group_size, int act_dtype,
                             void* workspace, size_t workspace_bytes, void* stream)
{
    int rc = check_serq(S, R, s);
    if (rc != W4EC_OK)
        return rc;
    return prefill_entry(X, packed, s > 0 ? X : nullptr, R, nullptr, 0.0f, Y, M, N, K, s, group_size,
                         act_dtype, workspace, workspace_bytes, stream, nullptr, S);
}

int w4ec_linear_decode_vgate(const void* X, const void* packed, const void* A, const void* B,
                             const void* G1, const void* c1, const void* G2, const void* c2,
                             int h, void* Y, int M, int N, int K, int r, int group_size,
                             int act_dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    const VGate vg{G1, c1, G2, c2, h};
    return decode_entry(X, packed, A, B, nullptr, 0.0f, Y, M, N, K, r, group_size, act_dtype,
                        workspace, workspace_bytes, stream, &vg);
}

int w4ec_linear_prefill_vgate(const void* X, const void* packed, const void* A, const void* B,
                              const void* G1, const void* c1, const void* G2, const void* c2,
                              int h, void* Y, int M, int N, int K, int r, int group_size,
                              int act_dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    const VGate vg{G1, c1, G2, c2, h};
    return prefill_entry(X, packed, A, B, nullptr, 0.0f, Y, M, N, K, r, group_size, act_dtype,
                         workspace, workspace_bytes, stream, &vg);
}

int w4ec_linear_decode_xfp(const void* X, const void* packed, const uint16_t* codebook,
                           const int32_t* row_ptr, const int32_t* col_idx, const uint16_t* val,
                           int nnz, void* Y, int M, int N, int K, int act_dtype, void* stream)
{
    if (M <= 0 || nnz < 0)
        return W4EC_ERR_INVALID_ARG;
    if (M > DECODE_MAX_M)
        return W4EC_ERR_UNSUPPORTED;
    int rc = check_weight_shape(N, K, K);
    if (rc != W4EC_OK)
        return rc;
    if (act_dtype != W4EC_FP16 && act_dtype != W4EC_BF16)
        return W4EC_ERR_INVALID_ARG;
    if (!X || !packed || !codebook || !row_ptr || !Y || (nnz > 0 && (!col_idx || !val)))
        return W4EC_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(Y, 16) || !aligned(packed, 256) || !aligned(codebook, 16) ||
        !aligned(row_ptr, 4) || !aligned(col_idx, 4) || !aligned(val, 2))
        return W4EC_ERR_INVALID_ARG;
    if (X == Y || packed == Y || codebook == Y)
        return W4EC_ERR_INVALID_ARG;
    const XfpArgs x{X, packed, codebook, row_ptr, col_idx, val, nnz, Y, M, N, K, act_dtype};
    return hip_status(launch_decode_xfp(x, make_decode_plan(M, N, K, 0), (hipStream_t)stream));
}

int w4ec_linear_decode_xfp_lib(const void* X, const void* packed, const uint16_t* library, int L,
                               const uint8_t* libid, const int32_t* row_ptr, const int32_t* col_idx,
                               const uint16_t* val, int nnz, void* Y, int M, int N, int K, int act_dtype,
                               void* stream)
{
    if (M <= 0 || nnz < 0 || L < 1)
        return W4EC_ERR_INVALID_ARG;
    if (M > DECODE_MAX_M || L > W4EC_XFP_LIB_MAX)
        return W4EC_ERR_UNSUPPORTED;
    int rc = check_weight_shape(N, K, K);
    if (rc != W4EC_OK)
        return rc;
    if (act_dtype != W4EC_FP16 && act_dtype != W4EC_BF16)
        return W4EC_ERR_INVALID_ARG;
    if (!X || !packed || !library || !libid || !row_ptr || !Y || (nnz > 0 && (!col_idx || !val)))
        return W4EC_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(Y, 16) || !aligned(packed, 256) || !aligned(library, 16) ||
        !aligned(row_ptr, 4) || !aligned(col_idx, 4) || !aligned(val, 2))
        return W4EC_ERR_INVALID_ARG;
    if (X == Y || packed == Y || library == Y || (const void*)libid == Y)
        return W4EC_ERR_INVALID_ARG;
    XfpArgs x{X, packed, library, row_ptr, col_idx, val, nnz, Y, M, N, K, act_dtype};
    x.libid = libid;
    x.L = L;
    return hip_status(launch_decode_xfp(x, make_decode_plan(M, N, K, 0), (hipStream_t)stream));
}

void w4ec_set_wait_limit(uint32_t polls)
{
    g_wait_limit.store(polls, std::memory_order_relaxed);
}

uint32_t w4ec_wait_limit(void)
{
    return g_wait_limit.load(std::memory_order_relaxed);
}

int w4ec_workspace_status(const void* workspace, size_t workspace_bytes, void* stream)
{
    if (!workspace || workspace_bytes < OFF_DEC_FLAGS + 16 || !aligned(workspace, 256))
        return W4EC_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    uint32_t f[4] = {0, 0, 0, 0};
    hipError_t e = hipMemcpyAsync(f, (const char*)workspace + OFF_DEC_FLAGS, sizeof f, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess)
        e = hipStreamSynchronize(st);
    if (e != hipSuccess)
        return W4EC_ERR_HIP;
    if (f[1] || f[2])
        return W4EC_ERR_TIMED_OUT;
    if (f[3])
        return W4EC_ERR_BAD_INDEX;
    return W4EC_OK;
}

int w4ec_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream)
{
    if (!src || !sink || !aligned(src, 16) || !aligned(sink, 4) || bytes % 16 != 0)
        return W4EC_ERR_INVALID_ARG;
    if (bytes == 0)
        return W4EC_OK;
    return hip_status(launch_stream_read(src, bytes, sink, (hipStream_t)stream));
}

int w4ec_workspace_reset(void* workspace, size_t workspace_bytes, void* stream)
{
    if (!workspace || !aligned(workspace, 256) || workspace_bytes % 16 != 0)
        return W4EC_ERR_WORKSPACE;
    const size_t n = std::min(workspace_bytes, CTRL_BYTES);
    return hip_status(launch_zero_fill(workspace, n, (hipStream_t)stream));
}

}  // extern "C"
