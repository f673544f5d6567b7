/*
 * w4ec.h -- C ABI of libw4ec: a weight-only 4-bit linear layer with an
 * input-adaptive low-rank error compensator (EC), for AMD Instinct MI355X
 * (gfx950) on one GPU.
 *
 * The operation (SPEAR, "A System for Post-Quantization Error-Adaptive
 * Recovery Enabling Efficient Low-Bit LLM Serving"; gist.science technical
 * summary, section 2.1A "input-adaptive error compensators").  The page
 * writes the effective weight as the 4-bit weight plus a gated rank-r product
 * B diag(gate(A x)) A; this library takes the gate as one scalar per token,
 * g = sigmoid(x . w_g + b_g), with the page's scale alpha folded into B:
 *
 *   Y[m,n] = sum_k X[m,k] Wd[n,k]  +  g[m] * sum_j T[m,j] B[j,n]
 *   Wd[n,k] = (q[n,k] - z[n,k/G]) * s[n,k/G]       q in 0..15 (4-bit codes)
 *   T[m,j]  = sum_k X[m,k] A[k,j]
 *   g[m]    = 1 / (1 + exp(-(sum_k X[m,k] w_g[k] + b_g)))
 *
 * Section 2.2A of the same summary splits the work by phase: a decode step
 * (few tokens, memory bound) runs the EC inside the low-bit GEMM's epilogue
 * in a single kernel -> w4ec_linear_decode; a prefill step (many tokens,
 * compute bound) -> w4ec_linear_prefill, here also with the gated correction
 * fused into the GEMM epilogue (an extension of the reduction by r terms)
 * after a prepass that computes the gate and X A in one read of X.
 *
 * Conventions for every call:
 *  - Pointers named as "device" are HIP device pointers owned by the caller.
 *    The library never allocates or frees memory and keeps no state between
 *    calls except what the caller's workspace holds.
 *  - All arrays are row-major and contiguous.  X, Y, A, w_g and the workspace
 *    must be 16-byte aligned; the packed blob 256-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous on it unless stated otherwise.
 *  - Activations X, Y and the EC parameters A, B, w_g share one dtype
 *    (`act_dtype`: W4EC_FP16 or W4EC_BF16); scale and zero are always fp16
 *    (passed as uint16_t bit patterns).  Accumulation is fp32.
 *  - Shapes: N >= 1; K a multiple of 128; group_size G == K (one scale/zero
 *    per output channel) or a multiple of 128 that divides K; 0 <= r <= 256.
 *  - Errors are returned as w4ec_status values before anything is launched;
 *    a failed launch returns W4EC_ERR_HIP.  No C++ exception crosses the ABI.
 *  - Y must not alias any input.  The same inputs give a bit-identical Y
 *    (all cross-workgroup sums run in a fixed order; no float atomics).
 */
#ifndef W4EC_H_
#define W4EC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4EC_OK = 0,
    W4EC_ERR_INVALID_ARG = -1,  /* null pointer, bad shape, misalignment, bad zero point */
    W4EC_ERR_UNSUPPORTED = -2,  /* shape outside what the library supports (see above) */
    W4EC_ERR_WORKSPACE = -3,    /* workspace missing or smaller than w4ec_workspace_bytes */
    W4EC_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed           */
    W4EC_ERR_TIMED_OUT = -5,    /* w4ec_workspace_status: a bounded wait gave up        */
    W4EC_ERR_BAD_INDEX = -6     /* w4ec_workspace_status: a salient-channel index was   */
                                /* outside [0, K) and was clamped                       */
} w4ec_status;

typedef enum { W4EC_FP16 = 0, W4EC_BF16 = 1 } w4ec_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* w4ec_status_str(int status);

/* Size in bytes of the packed device blob for an N x K layer with group size
 * G (codes, scales and zero points in the layout the kernels read).
 * Returns 0 for unsupported shapes. */
size_t w4ec_packed_bytes(int N, int K, int group_size);

/* Round-to-nearest asymmetric int4 quantization on the GPU -- the per-channel
 * RTN baseline of the SPEAR summary's results (section 3.1), here also per
 * group of G input features.  Per row n and group:
 *   lo = min(min w, 0), hi = max(max w, 0), s = fp16((hi - lo) / 15)
 *   z = clamp(rint(-lo / s), 0, 15), q = clamp(rint(w / s) + z, 0, 15)
 * computed in float64 (s clamped to the largest finite half; a group whose s
 * rounds to 0 gets s = 1, z = 0).  W must be finite.
 *   W      device, float32 [N, K]
 *   q_canon device, uint8 [N, K/2]: code k in the low nibble of byte k/2 when
 *          k is even, in the high nibble when k is odd
 *   scale, zero  device, fp16 bits [N, K/G]  (zero is an integer 0..15)   */
int w4ec_quantize_rtn(const float* W, int N, int K, int group_size,
                      uint8_t* q_canon, uint16_t* scale, uint16_t* zero,
                      void* stream);

/* Re-lay canonical codes and fp16 scale/zero into the device blob.  Weights
 * are prepared once, offline (the 2:4-sparsity-versus-quantization summary,
 * "Is 2:4 Sparsity Still Worth It?", chiosa.app, section on space and
 * compute parity, counts index and scale bytes with the weights and prepares
 * them offline).  Zero points need not be integers: the SPEAR summary's
 * results (section 3.1) cover quantizers beside RTN (GPTQ, AWQ, OmniQuant)
 * whose zero points are arbitrary; any fp16 z with |z| <= 1024 is exact (the
 * kernels take floor(z) exactly and correct for the fraction).  A zero point
 * that is not finite or lies beyond +-1024 is stored as NaN: the outputs that
 * use it are NaN, and w4ec_unpack returns NaN for it.  Asynchronous.
 *   q_canon device uint8 [N, K/2]; scale, zero device fp16 bits [N, K/G];
 *   packed  device, w4ec_packed_bytes(N, K, G) bytes, 256-byte aligned.   */
int w4ec_pack(const uint8_t* q_canon, const uint16_t* scale, const uint16_t* zero,
              int N, int K, int group_size, void* packed, void* stream);

/* Inverse of w4ec_pack (a test hook): blob -> canonical codes and fp16
 * scale/zero, same layouts as w4ec_pack's inputs; exact except for zero
 * points that w4ec_pack stored as NaN.  Asynchronous. */
int w4ec_unpack(const void* packed, int N, int K, int group_size,
                uint8_t* q_canon, uint16_t* scale, uint16_t* zero, void* stream);

/* Workspace bytes needed by w4ec_linear_decode / w4ec_linear_prefill for
 * this shape (the larger of the two when both apply; at least
 * W4EC_WS_STATE_BYTES when r > 0).  The workspace holds the gated rank-r
 * activations, partial sums and the counters through which workgroups hand
 * over partial results.  It must be zero-filled once when allocated (or
 * passed to w4ec_workspace_reset).  Its first W4EC_WS_STATE_BYTES bytes hold
 * hand-over state that every call returns to zero, so the workspace can be
 * reused by later calls on the same stream, of any shape and either phase,
 * without clearing.  Two calls that overlap in time must not share a
 * workspace.
 *
 * Failures inside a call.  The decode kernel's workgroups hand partial
 * results to each other and wait for them with bounded waits (a wait gives
 * up after w4ec_wait_limit() polls, about a second by default), so a broken
 * hand-over can never hang the GPU.  So do the prefill GEMM's workgroups
 * when they compute the gated rank-r activations themselves (at most 64
 * tokens, when all of them fit on the device at once).  A wait that gives
 * up records it in the workspace and turns the outputs that depend on it
 * into NaN; the call itself has already returned W4EC_OK.  From then on
 * that phase's hand-over state in the workspace is not to be trusted:
 * every later call of that phase that waits on it writes NaN into the
 * outputs that depend on it, until w4ec_workspace_reset; the other phase
 * stays correct.  A
 * salient-channel index outside [0, K) (w4ec_linear_*_serq) is also
 * recorded, without the NaN outputs.  w4ec_workspace_status reports both. */
#define W4EC_WS_STATE_BYTES ((size_t)16 << 20)
size_t w4ec_workspace_bytes(int M, int N, int K, int r, int group_size);

/* What the calls so far on this workspace recorded: W4EC_OK,
 * W4EC_ERR_TIMED_OUT (a bounded wait gave up: the results of that call
 * where they depend on it, and of every later call of that phase that waits
 * on this workspace, are NaN) or
 * W4EC_ERR_BAD_INDEX (a salient-channel index was clamped).  Synchronizes
 * `stream` and reads 16 bytes of the workspace.  W4EC_ERR_WORKSPACE for a
 * missing or misaligned (256 B) workspace. */
int w4ec_workspace_status(const void* workspace, size_t workspace_bytes, void* stream);

/* Zero the workspace's state region (its first W4EC_WS_STATE_BYTES bytes,
 * or all of it when smaller) with a kernel on `stream` (asynchronous; no
 * memset node in a captured graph): the recovery after a recorded failure,
 * and an alternative to zero-filling a new workspace.  workspace_bytes must
 * be a multiple of 16. */
int w4ec_workspace_reset(void* workspace, size_t workspace_bytes, void* stream);

/* Polls a bounded wait makes before it gives up, for every later launch in
 * this process (default 4194304, about a second).  0 makes every wait give
 * up at once, as if it had timed out: a way to exercise the failure path
 * above from the host, with every kernel still exiting normally.  Not
 * thread-safe with respect to launches already being prepared. */
void w4ec_set_wait_limit(uint32_t polls);
uint32_t w4ec_wait_limit(void);

/* The layer, decode phase: 1 <= M <= 16 tokens, one kernel launch.
 *   X     device act [M, K]          packed  device blob from w4ec_pack
 *   A     device act [K, r]          B       device act [r, N]
 *   w_g   device act [K], or NULL (then x . w_g = 0 and g = sigmoid(b_g);
 *         b_g = -INFINITY closes the gate, +INFINITY opens it fully)
 *   b_g   gate bias (fp32, by value)
 *   Y     device act [M, N] (output)
 *   r     EC rank; r == 0 is the plain W4 layer (A, B, w_g ignored, may be NULL)
 * Returns W4EC_ERR_UNSUPPORTED for M > 16, and for shapes whose EC partial
 * sums exceed the workspace's state region (only with r near 256, 16
 * tokens and K beyond about 60000). */
int w4ec_linear_decode(const void* X, const void* packed, const void* A, const void* B,
                       const void* w_g, float b_g, void* Y,
                       int M, int N, int K, int r, int group_size, int act_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/* w4ec_linear_decode without a workspace argument and without allocating:
 * for callers that cannot call hipMalloc (code under HIP graph capture,
 * serving loops, harnesses that forbid allocation).  The decode hand-over
 * state lives in a static device array of W4EC_NOALLOC_SCRATCH_BYTES bytes
 * that the library holds on each GPU it runs on until the process ends.
 * The first call on a device (with that device current) looks up the
 * array's address and clears it with a kernel on `stream`; later calls
 * reuse it, each returning the state to zero as with a workspace.
 * Arguments, results and errors as for w4ec_linear_decode, plus
 * W4EC_ERR_UNSUPPORTED when the shape's state would exceed the array
 * (512 KiB + 4 * ceil(K / KS) * M * (r + 1) bytes, KS <= 256 the EC slice
 * width: with K = 4096 any M <= 16 and r <= 256 fits).  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, two host threads) race and must not be issued.  A bounded wait
 * that gives up is recorded in the array as in a workspace, and every later
 * call of this entry point on that GPU then writes NaN into all of Y (there
 * is no reset for the array).  r == 0 touches no state at all. */
#define W4EC_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
int w4ec_linear_decode_noalloc(const void* X, const void* packed, const void* A, const void* B,
                               const void* w_g, float b_g, void* Y,
                               int M, int N, int K, int r, int group_size, int act_dtype,
                               void* stream);

/* The layer, prefill phase: any M >= 1 (tiled MFMA GEMM, three launches:
 * the gate / X A prepass over K slices, the reduction of its slices with the
 * gate, then the GEMM with the gated correction in its epilogue; for bf16
 * activations with one zero point per channel the prepass also sums each
 * token's activations, which the GEMM's zero-point term uses, so it runs
 * even when r == 0).  Arguments as for w4ec_linear_decode. */
int w4ec_linear_prefill(const void* X, const void* packed, const void* A, const void* B,
                        const void* w_g, float b_g, void* Y,
                        int M, int N, int K, int r, int group_size, int act_dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/* The layer with a vector gate: one gate per rank component instead of one
 * per token.  The SPEAR summary (section 2.1A) writes the compensated weight
 * as W + alpha B diag(gamma(A x)) A, with gamma a small bottleneck MLP on
 * the rank-r projection; it names neither the MLP's activation nor its
 * width.  This library reads gamma as a two-layer bottleneck of width h with
 * a ReLU and a sigmoid output (alpha folded into B, as above):
 *
 *   T[m,j]     = sum_k X[m,k] A[k,j]
 *   u[m,i]     = max(0, sum_j T[m,j] G1[j,i] + c1[i])          0 <= i < h
 *   gamma[m,j] = 1 / (1 + exp(-(sum_i u[m,i] G2[i,j] + c2[j])))
 *   Y[m,n]     = sum_k X[m,k] Wd[n,k] + sum_j gamma[m,j] T[m,j] B[j,n]
 *
 *   G1  device act [r, h]     c1  device act [h]
 *   G2  device act [h, r]     c2  device act [r]     (2-byte aligned)
 *   h   bottleneck width, 1 <= h <= 64 (W4EC_ERR_UNSUPPORTED above)
 * The bottleneck runs in fp32 on the fp32 sums of T; T_g = gamma * T is
 * rounded to the activation type, as in the scalar form.  Other arguments,
 * limits, workspace and error behaviour as w4ec_linear_decode /
 * w4ec_linear_prefill; with r == 0 the gate arguments are ignored. */
int w4ec_linear_decode_vgate(const void* X, const void* packed, const void* A, const void* B,
                             const void* G1, const void* c1, const void* G2, const void* c2,
                             int h, void* Y, int M, int N, int K, int r, int group_size,
                             int act_dtype, void* workspace, size_t workspace_bytes, void* stream);

int w4ec_linear_prefill_vgate(const void* X, const void* packed, const void* A, const void* B,
                              const void* G1, const void* c1, const void* G2, const void* c2,
                              int h, void* Y, int M, int N, int K, int r, int group_size,
                              int act_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Single-factor correction over salient input channels (SERQ summary,
 * "SERQ: Saliency-Aware Low-Rank Error Reconstruction for LLM Quantization",
 * section 2): the quantized product plus the activation channels of the
 * salient weight rows times one low-rank factor R,
 *
 *   Y[m,n] = sum_k X[m,k] Wd[n,k] + sum_j X[m, S[j]] R[j,n]      j < s
 *
 * read in the W4A16 setting of this library (X and R in the activation
 * type; no activation or R quantization).  The page's offline permutation
 * makes the salient channels one contiguous block; any index list works.
 *   S  device int32 [s], channel indices in [0, K) (duplicates allowed);
 *      an index outside that range is clamped to it and leaves a nonzero
 *      word in the workspace's state region (the result is then undefined)
 *   R  device act [s, N] (2-byte aligned)
 *   s  0 <= s <= 256; s == 0 is the plain W4 layer (S, R ignored)
 * The decode form needs no EC workgroups: each output workgroup gathers its
 * operand from X itself.  Workspace as w4ec_workspace_bytes(M, N, K, s, G);
 * other arguments and limits as w4ec_linear_decode / w4ec_linear_prefill. */
int w4ec_linear_decode_serq(const void* X, const void* packed, const int32_t* S, const void* R,
                            void* Y, int M, int N, int K, int s, int group_size, int act_dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

int w4ec_linear_prefill_serq(const void* X, const void* packed, const int32_t* S, const void* R,
                             void* Y, int M, int N, int K, int s, int group_size, int act_dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Unfused and semi-fused prefill (the SPEAR summary, section 2.2A, runs the
 * EC beside the low-bit GEMM in the prefill phase and adds its product
 * afterwards).  These two calls split the EC off the fused prefill so that a
 * caller can run
 *     w4ec_prefill_ec_gate  (X -> T_g in its workspace), on one stream,
 *     w4ec_linear_prefill with r = 0 (Y = X Wd^T), on another, then
 *     w4ec_prefill_ec_apply (Y += T_g B) after both,
 * e.g. as a graph with a fork and a join.  The result equals the fused
 * layer's up to one more rounding of Y to the activation type.
 *
 * w4ec_prefill_ec_workspace_bytes: workspace for the two EC calls (their
 * own; a concurrent GEMM needs a different one).  0 for unsupported shapes.
 *
 * w4ec_prefill_ec_gate: T_g = g * (X A) with g = sigmoid(X w_g + b_g), as in
 * w4ec_linear_prefill, into the workspace.
 *   X device act [M, K]; A device act [K, r]; w_g device act [K] or NULL;
 *   1 <= r <= 256; K a multiple of 128.
 *
 * w4ec_prefill_ec_apply: Y += T_g B, with T_g from the last
 * w4ec_prefill_ec_gate on this workspace (same M, K, r) and Y [M, N] holding
 * the plain W4 product.  B device act [r, N]; Y device act [M, N], read and
 * written; the workspace is only read.
 * Both return W4EC_ERR_WORKSPACE for a missing, misaligned (256 B) or too
 * small workspace, and validate before launching anything. */
size_t w4ec_prefill_ec_workspace_bytes(int M, int K, int r);
int w4ec_prefill_ec_gate(const void* X, const void* A, const void* w_g, float b_g, int M, int K,
                         int r, int act_dtype, void* workspace, size_t workspace_bytes, void* stream);
int w4ec_prefill_ec_apply(void* Y, const void* B, int M, int N, int K, int r, int act_dtype,
                          const void* workspace, size_t workspace_bytes, void* stream);

/* Codebook indices, canonical uint8 [N][K/2] (even k in the low nibble,
 * values 0..15), device -> the blob that w4ec_linear_decode_xfp reads
 * (w4ec_packed_bytes(N, K, K) bytes, 256-byte aligned): the panel layout of
 * w4ec_pack with the eight indices of each dword in natural order (byte j
 * holds those of k = 2j and 2j + 1), so that each byte selects one entry
 * of a 256-entry table of codebook pairs.  w4ec_unpack does not read it.
 * Asynchronous.  Returns W4EC_ERR_UNSUPPORTED unless K is a multiple of
 * 128. */
int w4ec_pack_xfp(const uint8_t* idx_canon, int N, int K, void* packed, void* stream);

/* Codebook weights with a sparse outlier residual, decode (XFP summary,
 * "XFP: Quality-Targeted Adaptive Codebook Quantization with Sparse Outlier
 * Separation for LLM Inference", sections 2 and 3: the outliers kept apart
 * at full precision, every other weight an index into a learned codebook of
 * 16 entries), in the W4A16 setting of this library, with one codebook per
 * output channel (a per-layer codebook is the case of identical rows):
 *
 *   Wh[n,k] = codebook[n][idx[n,k]] + (sum of val[e] over the entries e of
 *             row n with col_idx[e] == k)
 *   Y[m,n]  = sum_k X[m,k] Wh[n,k]
 *
 *   X        device act [M, K], 16-byte aligned; 1 <= M <= 16
 *   packed   device blob from w4ec_pack_xfp of the 4-bit indices idx
 *   codebook device fp16 [N][16], 16-byte aligned; with bf16 activations
 *            each entry is rounded to bf16 before it is multiplied
 *   row_ptr  device int32 [N + 1]; row n's entries are
 *            [row_ptr[n], row_ptr[n+1]) (clamped to [0, nnz]; a decreasing
 *            pair is an empty row)
 *   col_idx  device int32 [nnz], each in [0, K) (an index outside is
 *            clamped to that range; the result is then undefined)
 *   val      device fp16 [nnz], the residual values
 *   nnz      number of residual entries (>= 0; col_idx and val may be NULL
 *            when it is 0)
 *   Y        device act [M, N] (output), 16-byte aligned
 * K must be a multiple of 128.  No workspace.  Returns W4EC_ERR_UNSUPPORTED
 * for M > 16; W4EC_ERR_INVALID_ARG for missing or misaligned pointers and
 * Y aliasing an input.  Asynchronous on stream. */
int w4ec_linear_decode_xfp(const void* X, const void* packed, const uint16_t* codebook,
                           const int32_t* row_ptr, const int32_t* col_idx, const uint16_t* val,
                           int nnz, void* Y, int M, int N, int K, int act_dtype, void* stream);

/* Codebook weights from a shared library (XFP summary, section 2,
 * "adaptive learned codebooks", shared-library mode): the layer keeps L
 * codebooks of 16 fp16 entries, and each group of 128 consecutive weights of
 * an output channel (along K) names the entry it uses; the sparse fp16
 * outlier residual is as in w4ec_linear_decode_xfp:
 *
 *   Wh[n,k] = library[libid[n][k / 128]][idx[n,k]] + (sum of val[e] over the
 *             entries e of row n with col_idx[e] == k)
 *   Y[m,n]  = sum_k X[m,k] Wh[n,k]
 *
 *   X        device act [M, K], 16-byte aligned; 1 <= M <= 16
 *   packed   device blob from w4ec_pack_xfp of the 4-bit indices idx
 *   library  device fp16 [L][16], 16-byte aligned, 1 <= L <= W4EC_XFP_LIB_MAX;
 *            with bf16 activations each entry is rounded to bf16 before it
 *            is multiplied
 *   libid    device uint8 [N][K/128], each group's entry (one past the
 *            library is clamped to entry L - 1; the result is then undefined)
 *   row_ptr, col_idx, val, nnz, Y as w4ec_linear_decode_xfp.
 * The workgroups hold the whole library's pair tables in LDS (32 KB for 32
 * entries) instead of one table per output channel.  K must be a multiple
 * of 128.  No workspace.  Returns W4EC_ERR_UNSUPPORTED for M > 16 or
 * L > W4EC_XFP_LIB_MAX; W4EC_ERR_INVALID_ARG for L < 1, missing or
 * misaligned pointers and Y aliasing an input.  Asynchronous on stream. */
#define W4EC_XFP_LIB_MAX 32
int w4ec_linear_decode_xfp_lib(const void* X, const void* packed, const uint16_t* library, int L,
                               const uint8_t* libid, const int32_t* row_ptr, const int32_t* col_idx,
                               const uint16_t* val, int nnz, void* Y, int M, int N, int K, int act_dtype,
                               void* stream);

/* Streaming-read reference (a measurement hook, not part of the layer):
 * reads `bytes` from `src` with the plainest access pattern the library
 * knows for HBM -- 512 workgroups of 256 threads, workgroup w reading the
 * 16-byte chunks [w c, (w + 1) c) with c = ceil(bytes / 16 / 512), sixteen
 * non-temporal 16-byte loads in flight per thread -- and writes one 32-bit
 * XOR of its chunks' words per workgroup into sink[0 .. 511], so that no
 * load can be dropped.  The duration of this kernel for a byte count is the HBM
 * read time actually attainable on the device, against which the decode's
 * fraction of the 8 TB/s roofline can be read (the decode streams the same
 * packed weights in one pass).
 *   src   device, 16-byte aligned; bytes a multiple of 16 (0 launches nothing)
 *   sink  device uint32 [512], 4-byte aligned (output)
 * W4EC_ERR_INVALID_ARG for a missing or misaligned pointer or a byte count
 * that is not a multiple of 16.  Asynchronous on stream. */
int w4ec_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4EC_H_ */
