// abi_checks.cpp -- the host side of libw4ec (argument validation, launch
// plans, workspace sizing) run under AddressSanitizer and
// UndefinedBehaviorSanitizer, with no GPU.  It links api.cpp against stub
// launchers that check what each plan would hand a kernel (every region
// inside the workspace the caller sized with w4ec_workspace_bytes, every
// tile of the output covered) instead of launching anything; the pointers
// passed are aligned fakes that nothing dereferences.
//
// Built and run by tests/test_sanitizers.py (host-only compilation, sanitizers
// on the host code only).  Prints "abi checks ok: N calls" and exits 0, or
// names the first failed check and exits 1.
#include "w4ec.h"

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "w4ec_common.h"
#include "w4ec_launch.h"

namespace {

int g_fail = 0;
long g_calls = 0;
long g_launches = 0;
size_t g_ws_bytes = 0;     // workspace bytes the current call was given
bool g_noalloc = false;    // the current call uses the static state array
long g_scratch_lookups = 0;

#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        if (!(cond)) {                                                    \
            if (g_fail++ < 20) {                                          \
                std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
                std::fprintf(stderr, __VA_ARGS__);                        \
                std::fprintf(stderr, "\n");                               \
            }                                                             \
        }                                                                 \
    } while (0)

constexpr size_t STATE = W4EC_WS_STATE_BYTES;

void* fake(uintptr_t base) { return reinterpret_cast<void*>(base); }

}  // namespace

// ---------------------------------------------------------------- stub launchers
namespace w4ec {

hipError_t launch_rtn_quantize(const float*, int N, int K, int G, uint8_t*, uint16_t*, uint16_t*, hipStream_t)
{
    ++g_launches;
    CHECK(N > 0 && K > 0 && G > 0 && K % G == 0, "rtn N=%d K=%d G=%d", N, K, G);
    return hipSuccess;
}

hipError_t launch_pack(const uint8_t*, const uint16_t*, const uint16_t*, int N, int K, int G, void*, hipStream_t)
{
    ++g_launches;
    CHECK(N > 0 && K % PANEL_K == 0 && K % G == 0, "pack N=%d K=%d G=%d", N, K, G);
    return hipSuccess;
}

hipError_t launch_unpack(const void*, int N, int K, int G, uint8_t*, uint16_t*, uint16_t*, hipStream_t)
{
    ++g_launches;
    CHECK(N > 0 && K % PANEL_K == 0 && K % G == 0, "unpack N=%d K=%d G=%d", N, K, G);
    return hipSuccess;
}

hipError_t launch_decode(const LayerArgs& a, const DecodePlan& p, hipStream_t)
{
    ++g_launches;
    CHECK(a.M >= 1 && a.M <= 16, "decode M=%d", a.M);
    CHECK(p.n_main * p.CB * PANEL_N >= a.N, "decode columns: n_main %d CB %d N %d", p.n_main, p.CB, a.N);
    CHECK((p.n_main - 1) * p.CB * PANEL_N < a.N, "decode: a workgroup with no column");
    CHECK(!p.xlds || (a.M <= 4 && (size_t)a.M * a.K * 2 <= DEC_XLDS_MAX_BYTES), "decode xlds M=%d K=%d", a.M, a.K);
    if (a.r > 0) {
        CHECK(a.ws != nullptr && g_ws_bytes >= (g_noalloc ? W4EC_NOALLOC_SCRATCH_BYTES : STATE),
              "decode r=%d without a state region", a.r);
        if (a.S == nullptr) {
            CHECK(p.P >= 1 && p.KS % 64 == 0 && (long)p.P * p.KS >= a.K && (long)(p.P - 1) * p.KS < a.K,
                  "decode EC slices P=%d KS=%d K=%d", p.P, p.KS, a.K);
            CHECK(p.off_partial + (size_t)p.P * a.M * p.RC * 4 <= (g_noalloc ? W4EC_NOALLOC_SCRATCH_BYTES : STATE),
                  "decode partials outside the state region");
        }
        CHECK(p.r_pad >= a.r && p.r_pad % 32 == 0 && (size_t)a.M * p.r_pad * 2 <= DEC_REP_DATA_STRIDE,
              "decode T_g slot r_pad=%d M=%d", p.r_pad, a.M);
    }
    CHECK(a.spin == w4ec_wait_limit(), "decode wait limit %u", a.spin);
    return hipSuccess;
}

static void check_prefill_plan(const LayerArgs& a, const PrefillPlan& p, bool gemm)
{
    CHECK(p.BM == 64 || p.BM == 128, "BM=%d", p.BM);
    CHECK(p.mt * p.BM >= a.M && (p.mt - 1) * p.BM < a.M && p.Mpad == p.mt * p.BM, "M tiles mt=%d BM=%d M=%d", p.mt, p.BM, a.M);
    if (gemm) {
        CHECK(p.nt * p.BN >= a.N && (p.nt - 1) * p.BN < a.N, "N tiles nt=%d N=%d", p.nt, a.N);
        CHECK(p.ksplit >= 1 && p.ksplit <= a.K / PANEL_K, "ksplit=%d K=%d", p.ksplit, a.K);
        if (p.ksplit > 1)
            CHECK(p.mt * p.nt <= 256, "split tiles %d > 256 counters", p.mt * p.nt);
    }
    // each prepass workgroup takes pre_nch chunks of pre_kc: the slices
    // cover K and none is empty
    const long slice = (long)p.pre_nch * p.pre_kc;
    CHECK(p.pre_kc % 64 == 0 && p.pre_nch >= 1 && p.pre_nch <= 4 && (long)p.pre_ks * slice >= a.K &&
              (long)(p.pre_ks - 1) * slice < a.K,
          "prepass slices ks=%d nch=%d kc=%d K=%d", p.pre_ks, p.pre_nch, p.pre_kc, a.K);
    CHECK(p.pre_nch == 1 || (long)p.pre_mt * p.pre_ks <= 512 || p.pre_nch == 4, "prepass chunks beyond one round");
    CHECK(prepass_lds_bytes(a.r, p.pre_kc) <= (80u << 10), "prepass LDS");
    CHECK(p.off_pre_partial >= STATE && p.off_tg >= p.off_pre_partial && p.off_rowsum >= p.off_tg &&
          p.off_gemm_partial >= p.off_rowsum && p.bytes >= p.off_gemm_partial, "region order");
    CHECK(p.off_pre_partial + (size_t)p.pre_mt * p.pre_ks * 4 * ec_blocks(a.r) * 64 * 16 <= p.off_tg, "prepass partials");
    if (a.r > 0)
        CHECK(p.off_tg + (size_t)std::max(p.Mpad, p.pre_mt * 64) * p.r_pad * 2 <= p.off_rowsum ||
                  p.Mpad >= p.pre_mt * 64, "T_g region");
    if (gemm && p.ksplit > 1)
        CHECK(p.off_gemm_partial + (size_t)p.ksplit * p.Mpad * p.nt * p.BN * 4 <= p.bytes, "split-K partials");
}

hipError_t launch_prefill(const LayerArgs& a, const PrefillPlan& p, hipStream_t)
{
    ++g_launches;
    check_prefill_plan(a, p, true);
    if (a.ws)
        CHECK(p.bytes <= g_ws_bytes, "prefill plan %zu > workspace %zu", p.bytes, g_ws_bytes);
    else
        CHECK(a.r == 0 && p.ksplit == 1 && !(a.act == W4EC_BF16 && a.G == a.K), "prefill needs a workspace");
    return hipSuccess;
}

hipError_t launch_prefill_ec_gate(const LayerArgs& a, const PrefillPlan& p, hipStream_t)
{
    ++g_launches;
    check_prefill_plan(a, p, false);
    return hipSuccess;
}

hipError_t launch_prefill_ec_apply(const ApplyArgs& a, const PrefillPlan& p, hipStream_t)
{
    ++g_launches;
    CHECK(p.r_pad >= a.r && p.off_tg + (size_t)((a.M + 63) / 64 * 64) * p.r_pad * 2 <= g_ws_bytes, "apply T_g");
    return hipSuccess;
}

hipError_t launch_decode_xfp(const XfpArgs& x, const DecodePlan& p, hipStream_t)
{
    ++g_launches;
    CHECK(x.M >= 1 && x.M <= 16 && p.n_main * p.CB * PANEL_N >= x.N, "xfp plan");
    return hipSuccess;
}

hipError_t launch_zero_fill(void*, size_t bytes, hipStream_t)
{
    ++g_launches;
    CHECK(bytes % 16 == 0 && bytes <= g_ws_bytes && bytes <= STATE, "zero fill %zu", bytes);
    return hipSuccess;
}

hipError_t launch_stream_read(const void*, size_t bytes, uint32_t*, hipStream_t)
{
    ++g_launches;
    CHECK(bytes % 16 == 0 && bytes > 0, "stream read %zu", bytes);
    return hipSuccess;
}

hipError_t noalloc_scratch(void** out, hipStream_t)
{
    ++g_scratch_lookups;
    CHECK(g_noalloc, "state array looked up outside a noalloc call");
    *out = reinterpret_cast<void*>(uintptr_t(0x78000000));
    return hipSuccess;
}

}  // namespace w4ec

// ---------------------------------------------------------------- driver

namespace {

const uintptr_t X = 0x10000000, PK = 0x20000000, A = 0x30000000, B = 0x40000000, WG = 0x50000000,
                Y = 0x60000000, WS = 0x70000000;

int layer(bool decode, int M, int N, int K, int r, int G, int act, size_t ws_bytes,
          uintptr_t x = X, uintptr_t y = Y, uintptr_t ws = WS)
{
    ++g_calls;
    g_ws_bytes = ws_bytes;
    auto fn = decode ? w4ec_linear_decode : w4ec_linear_prefill;
    return fn(fake(x), fake(PK), r ? fake(A) : nullptr, r ? fake(B) : nullptr, r ? fake(WG) : nullptr, 0.5f,
              fake(y), M, N, K, r, G, act, ws ? fake(ws) : nullptr, ws_bytes, nullptr);
}

void expect(int got, int want, const char* what)
{
    CHECK(got == want, "%s: got %s, want %s", what, w4ec_status_str(got), w4ec_status_str(want));
}

}  // namespace

int main()
{
    // ---- argument errors: reported before any launch
    const long l0 = g_launches;
    expect(layer(true, 0, 512, 512, 8, 512, 0, 1 << 26), W4EC_ERR_INVALID_ARG, "M = 0");
    expect(layer(true, 17, 512, 512, 8, 512, 0, 1 << 26), W4EC_ERR_UNSUPPORTED, "decode M = 17");
    expect(layer(false, 4, 512, 100, 8, 100, 0, 1 << 26), W4EC_ERR_UNSUPPORTED, "K % 128");
    expect(layer(false, 4, 512, 512, 8, 64, 0, 1 << 26), W4EC_ERR_UNSUPPORTED, "G = 64");
    expect(layer(false, 4, 512, 512, 257, 512, 0, 1 << 26), W4EC_ERR_UNSUPPORTED, "r = 257");
    expect(layer(false, 4, 512, 512, 8, 512, 2, 1 << 26), W4EC_ERR_INVALID_ARG, "act = 2");
    expect(layer(false, 4, 0, 512, 8, 512, 0, 1 << 26), W4EC_ERR_INVALID_ARG, "N = 0");
    expect(layer(true, 4, 512, 512, 8, 512, 0, 1 << 26, X + 2), W4EC_ERR_INVALID_ARG, "misaligned X");
    expect(layer(true, 4, 512, 512, 8, 512, 0, 1 << 26, X, X), W4EC_ERR_INVALID_ARG, "Y aliases X");
    expect(layer(true, 4, 512, 512, 8, 512, 0, 1024), W4EC_ERR_WORKSPACE, "small workspace");
    expect(layer(true, 4, 512, 512, 8, 512, 0, 1 << 26, X, Y, WS + 16), W4EC_ERR_WORKSPACE, "misaligned workspace");
    expect(layer(true, 4, 512, 512, 8, 512, 0, 1 << 26, X, Y, 0), W4EC_ERR_WORKSPACE, "no workspace");
    expect(layer(false, 4, 512, 512, -1, 512, 0, 1 << 26), W4EC_ERR_INVALID_ARG, "r = -1");
    ++g_calls;
    expect(w4ec_pack(nullptr, nullptr, nullptr, 16, 128, 128, fake(PK), nullptr), W4EC_ERR_INVALID_ARG, "pack nulls");
    expect(w4ec_workspace_status(nullptr, 0, nullptr), W4EC_ERR_WORKSPACE, "status without workspace");
    expect(w4ec_workspace_reset(fake(WS + 16), 256, nullptr), W4EC_ERR_WORKSPACE, "reset misaligned");
    expect(w4ec_stream_read(fake(WS), 24, reinterpret_cast<uint32_t*>(fake(WS)), nullptr), W4EC_ERR_INVALID_ARG,
           "stream read of a partial chunk");
    expect(w4ec_stream_read(fake(WS + 8), 256, reinterpret_cast<uint32_t*>(fake(WS)), nullptr),
           W4EC_ERR_INVALID_ARG, "stream read misaligned");
    expect(w4ec_stream_read(fake(WS), 256, nullptr, nullptr), W4EC_ERR_INVALID_ARG, "stream read without sink");
    expect(w4ec_linear_decode_vgate(fake(X), fake(PK), fake(A), fake(B), fake(WG), fake(WG + 4096), fake(WG + 8192),
                                    fake(WG + 12288), 65, fake(Y), 1, 512, 512, 32, 512, 0, fake(WS), 1 << 26, nullptr),
           W4EC_ERR_UNSUPPORTED, "vgate h = 65");
    expect(w4ec_linear_decode_xfp(fake(X), fake(PK), nullptr, static_cast<const int32_t*>(fake(A)), nullptr, nullptr, 0,
                                  fake(Y), 1, 512, 512, 0,
                                  nullptr), W4EC_ERR_INVALID_ARG, "xfp without codebooks");
    CHECK(g_launches == l0, "an invalid call launched");
    expect(w4ec_stream_read(fake(WS), 256, reinterpret_cast<uint32_t*>(fake(WS)), nullptr), W4EC_OK, "stream read");
    CHECK(g_launches == l0 + 1, "stream read launches once");
    expect(w4ec_stream_read(fake(WS), 0, reinterpret_cast<uint32_t*>(fake(WS)), nullptr), W4EC_OK, "empty stream read");
    CHECK(g_launches == l0 + 1, "an empty stream read launches nothing");

    // ---- wait limit round trip
    const uint32_t lim = w4ec_wait_limit();
    w4ec_set_wait_limit(7);
    CHECK(w4ec_wait_limit() == 7, "wait limit");
    expect(layer(true, 1, 512, 512, 8, 512, 0, w4ec_workspace_bytes(1, 512, 512, 8, 512)), W4EC_OK, "decode at limit 7");
    w4ec_set_wait_limit(lim);

    // ---- valid shapes: every plan fits the workspace the caller sized
    const int Ns[] = {16, 48, 272, 4096, 14336, 28672};
    const int Ks[] = {128, 512, 4096, 8192, 14336, 20480};
    const int Rs[] = {0, 1, 8, 64, 128, 256};
    const int Md[] = {1, 2, 4, 5, 16};
    const int Mp[] = {1, 17, 64, 65, 128, 200, 256, 2048, 4096};
    for (int N : Ns)
        for (int K : Ks)
            for (int r : Rs)
                for (int grouped = 0; grouped < 2; ++grouped)
                    for (int act = 0; act < 2; ++act) {
                        const int G = grouped ? 128 : K;
                        for (int M : Md) {
                            const size_t ws = w4ec_workspace_bytes(M, N, K, r, G);
                            const int rc = layer(true, M, N, K, r, G, act, ws);
                            CHECK(rc == W4EC_OK || (rc == W4EC_ERR_UNSUPPORTED && r > 128 && K > 16384),
                                  "decode M=%d N=%d K=%d r=%d G=%d: %s", M, N, K, r, G, w4ec_status_str(rc));
                        }
                        for (int M : Mp) {
                            const size_t ws = w4ec_workspace_bytes(M, N, K, r, G);
                            expect(layer(false, M, N, K, r, G, act, ws), W4EC_OK, "prefill");
                            if (r > 0) {
                                ++g_calls;
                                const size_t we = w4ec_prefill_ec_workspace_bytes(M, K, r);
                                g_ws_bytes = we;
                                expect(w4ec_prefill_ec_gate(fake(X), fake(A), fake(WG), 0.f, M, K, r, act, fake(WS),
                                                            we, nullptr), W4EC_OK, "ec gate");
                                expect(w4ec_prefill_ec_apply(fake(Y), fake(B), M, N, K, r, act, fake(WS), we, nullptr),
                                       W4EC_OK, "ec apply");
                            }
                        }
                    }
    // ---- the no-allocation decode: same argument checks, the state array
    // only for r > 0, and shapes whose state would not fit it refused
    g_noalloc = true;
    g_ws_bytes = W4EC_NOALLOC_SCRATCH_BYTES;
    {
        const long l1 = g_launches, s1 = g_scratch_lookups;
        ++g_calls;
        expect(w4ec_linear_decode_noalloc(fake(X), fake(PK), fake(A), fake(B), fake(WG), 0.f, fake(Y), 17, 512, 512,
                                          8, 512, 0, nullptr), W4EC_ERR_UNSUPPORTED, "noalloc M = 17");
        expect(w4ec_linear_decode_noalloc(fake(X + 2), fake(PK), fake(A), fake(B), fake(WG), 0.f, fake(Y), 4, 512, 512,
                                          8, 512, 0, nullptr), W4EC_ERR_INVALID_ARG, "noalloc misaligned X");
        expect(w4ec_linear_decode_noalloc(fake(X), fake(PK), fake(A), fake(B), fake(WG), 0.f, fake(Y), 16, 256, 16384,
                                          256, 16384, 0, nullptr), W4EC_ERR_UNSUPPORTED, "noalloc state too large");
        CHECK(g_launches == l1 && g_scratch_lookups == s1, "a refused noalloc call launched or looked up the array");
        expect(w4ec_linear_decode_noalloc(fake(X), fake(PK), fake(A), fake(B), fake(WG), 0.f, fake(Y), 16, 14336, 4096,
                                          256, 4096, 1, nullptr), W4EC_OK, "noalloc 16 tokens rank 256");
        expect(w4ec_linear_decode_noalloc(fake(X), fake(PK), nullptr, nullptr, nullptr, 0.f, fake(Y), 1, 4096, 4096,
                                          0, 128, 0, nullptr), W4EC_OK, "noalloc without rank");
        CHECK(g_scratch_lookups == s1 + 1, "the state array is looked up only with a rank");
    }
    g_noalloc = false;
    g_ws_bytes = STATE;
    expect(w4ec_workspace_reset(fake(WS), STATE, nullptr), W4EC_OK, "reset");
    if (g_fail) {
        std::fprintf(stderr, "%d check(s) failed\n", g_fail);
        return 1;
    }
    std::printf("abi checks ok: %ld calls, %ld launches checked\n", g_calls, g_launches);
    return 0;
}
