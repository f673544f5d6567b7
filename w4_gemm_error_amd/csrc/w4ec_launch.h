// w4ec_launch.h -- internal host-side launchers (one per kernel family).
// The C ABI in api.cpp validates arguments, builds a plan and calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w4ec_common.h"

namespace w4ec {

hipError_t launch_rtn_quantize(const float* W, int N, int K, int G, uint8_t* qc,
                               uint16_t* scale, uint16_t* zero, hipStream_t st);
// scale == zero == NULL: the codebook blob (indices in natural nibble order,
// group_size K, scale 1 and zero 0)
hipError_t launch_pack(const uint8_t* qc, const uint16_t* scale, const uint16_t* zero,
                       int N, int K, int G, void* packed, hipStream_t st);
hipError_t launch_unpack(const void* packed, int N, int K, int G, uint8_t* qc,
                         uint16_t* scale, uint16_t* zero, hipStream_t st);

struct LayerArgs {
    const void* X;
    const void* packed;
    const void* A;
    const void* B;
    const void* w_g;
    float b_g;
    void* Y;
    int M, N, K, r, G, act;
    char* ws;
    // vector gate (h > 0): one gate per rank component, from a bottleneck of
    // width h on T = X A; w_g and b_g are then unused
    const void* G1;   // act [r][h]
    const void* c1;   // act [h]
    const void* G2;   // act [h][r]
    const void* c2;   // act [r]
    int h;
    // single-factor correction over salient channels (S non-null): T_g is
    // the gather X[:, S] (r = s channels), B is the factor R; no gate
    const int32_t* S; // [s] input-channel indices
    uint32_t spin;    // polls before a bounded wait gives up (0: at once)
};

hipError_t launch_decode(const LayerArgs& a, const DecodePlan& p, hipStream_t st);
hipError_t launch_prefill(const LayerArgs& a, const PrefillPlan& p, hipStream_t st);

// unfused / semi-fused prefill pieces: T_g into the workspace, then Y += T_g B
struct ApplyArgs {
    void* Y;
    const void* B;
    int M, N, r, act;
    char* ws;
};
hipError_t launch_prefill_ec_gate(const LayerArgs& a, const PrefillPlan& p, hipStream_t st);

// codebook weights with a sparse outlier residual (decode)
struct XfpArgs {
    const void* X;
    const void* packed;       // the 4-bit indices, packed as codes by w4ec_pack
    const uint16_t* cb;       // [N][16] fp16
    const int32_t* row_ptr;   // [N + 1]
    const int32_t* col_idx;   // [nnz]
    const uint16_t* val;      // [nnz] fp16
    int nnz;
    void* Y;
    int M, N, K, act;
    // shared-library mode (libid non-null): cb is the library [L][16] and
    // libid [N][K / 128] names each group's entry
    const uint8_t* libid = nullptr;
    int L = 0;
};
hipError_t launch_decode_xfp(const XfpArgs& x, const DecodePlan& p, hipStream_t st);
hipError_t launch_prefill_ec_apply(const ApplyArgs& a, const PrefillPlan& p, hipStream_t st);
// bytes (a multiple of 16, 16-byte aligned) set to zero by a kernel (no
// hipMemsetAsync node when a caller captures the stream into a graph)
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t st);
// the streaming-read reference: bytes (a multiple of 16) from src, one XOR
// word per workgroup (512 of them) into sink
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);
// The static state array of w4ec_linear_decode_noalloc on the current
// device (W4EC_NOALLOC_SCRATCH_BYTES bytes): its device address, looked up
// and cleared (a fill kernel on `st`) by the first call on each device.
// hipErrorInvalidDevice beyond the devices it keeps addresses for.
hipError_t noalloc_scratch(void** out, hipStream_t st);

}  // namespace w4ec
