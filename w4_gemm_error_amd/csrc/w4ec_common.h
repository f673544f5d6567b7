// w4ec_common.h -- internal to libw4ec: device types, the packed blob layout,
// int4 dequantization and MFMA wrappers for gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4ec {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { ACT_F16 = 0, ACT_BF16 = 1 };

// ------------------------------------------------------------ blob layout
//
// header (256 B) | codes | scale/zero
//
// codes: panels of 16 output columns x 128 input features, 1024 bytes each,
// ordered [column block cb][k block kb].  Inside a panel, lane l (0..63) of
// a wavefront owns bytes [16 l, 16 l + 16): four dwords, dword s (0..3)
// holding the 8 codes of column 16 cb + (l & 15) at
//   k = 128 kb + 32 s + 8 (l >> 4) + t,  t = 0..7.
// That is exactly the B operand of v_mfma_f32_16x16x32_{f16,bf16} for four
// consecutive 32-deep steps, so one 16-byte load per lane feeds 4 MFMAs.
// Within a dword, code t sits in nibble (t even ? t/2 : 4 + t/2): masking
// with 0x000F000F / 0x00F000F0 after shifts of 0 and 8 then yields the
// pairs (t0,t1) (t2,t3) (t4,t5) (t6,t7) in the two halves of a register.
//
// scale/zero: for group gi and column n (padded to a multiple of 16),
// one dword at index gi * Npad + n: fp16 scale in the low half, fp16 zero in
// the high half.  Padded columns hold codes 0 and scale = zero = 0.
constexpr int PANEL_K = 128;
constexpr int PANEL_N = 16;
constexpr int PANEL_BYTES = 1024;
constexpr size_t HEADER_BYTES = 256;
constexpr uint32_t BLOB_MAGIC = 0x43453457u;  // "W4EC"

// zero-point flags of a blob, recorded by the pack kernel (the kernels
// read the zero points themselves)
constexpr uint32_t ZF_FRAC = 1u;   // some zero point is not an integer
constexpr uint32_t ZF_BAD = 2u;    // some zero point is not finite or |z| > ZMAX: stored as NaN
constexpr float ZMAX = 1024.0f;    // the exact integer offsets hold for |z| <= ZMAX

struct BlobHeader {
    uint32_t magic;
    int32_t N, K, G;
    uint32_t zflags;     // ZF_FRAC | ZF_BAD
};

__host__ __device__ inline int nibble_of(int t) { return (t & 1) ? 4 + (t >> 1) : (t >> 1); }

struct BlobGeom {
    int N, K, G, NB, KB, Npad, NG;
    size_t codes_off, sz_off, bytes;
};

__host__ __device__ inline BlobGeom blob_geom(int N, int K, int G)
{
    BlobGeom g;
    g.N = N; g.K = K; g.G = G;
    g.NB = (N + PANEL_N - 1) / PANEL_N;
    g.KB = K / PANEL_K;
    g.Npad = g.NB * PANEL_N;
    g.NG = K / G;
    g.codes_off = HEADER_BYTES;
    g.sz_off = g.codes_off + (size_t)g.NB * g.KB * PANEL_BYTES;
    g.bytes = g.sz_off + (size_t)g.NG * g.Npad * 4;
    return g;
}

// ------------------------------------------------------------ memory helpers

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Streamed once per call: ask for non-temporal (streaming) caching.
__device__ inline u32x4 ld16_stream(const void* p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <int ACT> __device__ inline float act_to_f32(uint16_t v)
{
    if constexpr (ACT == ACT_F16) {
        return (float)__builtin_bit_cast(_Float16, v);
    } else {
        return __uint_as_float((uint32_t)v << 16);
    }
}

// A quiet NaN in the activation format.
template <int ACT> __device__ inline uint16_t act_nan() { return ACT == ACT_F16 ? 0x7E00u : 0x7FC0u; }

// float -> act bits, round to nearest even.
template <int ACT> __device__ inline uint16_t f32_to_act(float f)
{
    if constexpr (ACT == ACT_F16) {
        return __builtin_bit_cast(uint16_t, (_Float16)f);
    } else {
        __bf16 b = (__bf16)f;
        return __builtin_bit_cast(uint16_t, b);
    }
}

// ------------------------------------------------------------ MFMA

template <int ACT> __device__ inline floatx4 mfma16x16x32(u32x4 a, u32x4 b, floatx4 c)
{
    if constexpr (ACT == ACT_F16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                      __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
}

// ------------------------------------------------------------ dequant
//
// One dword of 8 codes (blob nibble order) -> 8 operand values in natural
// k order, as four registers of two 16-bit values.
//
// fp16: (0x6400 | c) is the half 1024 + c, and (0x5400 | c << 4) is the
// half 64 + c (exponent 21: the nibble in mantissa bits 4..7 counts whole
// units); both are exact.  Subtracting 1024 + z, or 64 + z, gives c - z
// exactly for an integer zero point z in 0..15.  Each half pair is built
// with one AND-OR, written out because the compiler splits it into two
// instructions; its result only feeds packed adds, never an MFMA operand
// directly.
struct DqF16 {
    half2_t off_lo;  // -(1024 + z)
    half2_t off_hi;  // -(64 + z)
};

__device__ inline DqF16 dq_f16_consts(float z)
{
    DqF16 c;
    _Float16 a = (_Float16)(-(1024.0f + z));
    _Float16 b = (_Float16)(-(64.0f + z));
    c.off_lo = (half2_t){a, a};
    c.off_hi = (half2_t){b, b};
    return c;
}

// (a & mask) | b.  Only for values that a VALU instruction consumes next:
// the compiler does not see what the asm writes, so it cannot keep the wait
// states an MFMA reading it directly would need.
__device__ inline uint32_t and_or(uint32_t a, uint32_t mask, uint32_t b)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(b));
    return r;
}

// Elements go through a scalar first: clang reads the wrong lane when
// __builtin_bit_cast is applied directly to an ext-vector element access.
__device__ inline half2_t h2_of(uint32_t v) { return __builtin_bit_cast(half2_t, v); }
__device__ inline uint32_t u32_of(half2_t v) { return __builtin_bit_cast(uint32_t, v); }

__device__ inline u32x4 dequant_f16(uint32_t w, const DqF16& c)
{
    const uint32_t w8 = w >> 8;
    const half2_t p0 = h2_of(and_or(w, 0x000F000Fu, 0x64006400u)) + c.off_lo;
    const half2_t p1 = h2_of(and_or(w, 0x00F000F0u, 0x54005400u)) + c.off_hi;
    const half2_t p2 = h2_of(and_or(w8, 0x000F000Fu, 0x64006400u)) + c.off_lo;
    const half2_t p3 = h2_of(and_or(w8, 0x00F000F0u, 0x54005400u)) + c.off_hi;
    u32x4 r;
    r.x = u32_of(p0);
    r.y = u32_of(p1);
    r.z = u32_of(p2);
    r.w = u32_of(p3);
    return r;
}

// Same, times the scale s, plus c2 = -(z - zi) s for a zero point z with
// integer part zi (the consts hold zi): (q - zi) s - (z - zi) s in one fused
// multiply-add, rounded once to fp16.  With an integer zero point c2 = -0
// and this is the rounded product (q - z) s.  sc holds {s, c2}.

__device__ inline u32x4 dequant_f16_scaled(uint32_t w, const DqF16& c, half2_t s2, half2_t c2)
{
    const u32x4 q = dequant_f16(w, c);
    const uint32_t q0 = q.x, q1 = q.y, q2 = q.z, q3 = q.w;
    u32x4 r;
    r.x = u32_of(__builtin_elementwise_fma(h2_of(q0), s2, c2));
    r.y = u32_of(__builtin_elementwise_fma(h2_of(q1), s2, c2));
    r.z = u32_of(__builtin_elementwise_fma(h2_of(q2), s2, c2));
    r.w = u32_of(__builtin_elementwise_fma(h2_of(q3), s2, c2));
    return r;
}

// The codes with their exponent-trick offsets left in: 1024 + c for the
// codes at bits 0-3 and 8-11 of each half of the dword (MFMA k positions 0,
// 1, 4, 5 of the eight), 64 + c for those at bits 4-7 and 12-15 (positions
// 2, 3, 6, 7).  Exact, one AND-OR per pair; the caller takes the offsets and
// the zero point off afterwards, as (offset + z) times the activations'
// sums over those positions.
// A constant the compiler keeps in a register (an empty asm hides its
// value): with both operands in registers, (a & m) | b is one v_and_or_b32,
// where two literals would take an AND and an OR.
__device__ inline uint32_t reg_const(uint32_t c)
{
    asm("" : "+v"(c));
    return c;
}

__device__ inline u32x4 dequant_f16_biased(uint32_t w)
{
    const uint32_t w8 = w >> 8;
    const uint32_t m0 = reg_const(0x000F000Fu), m1 = reg_const(0x00F000F0u);
    const uint32_t b0 = reg_const(0x64006400u), b1 = reg_const(0x54005400u);
    return (u32x4){(w & m0) | b0, (w & m1) | b1, (w8 & m0) | b0, (w8 & m1) | b1};
}

// c + a.lo + a.hi in fp32 (a pair of activations; products with one are exact)
template <int ACT>
__device__ inline float act_dot2_ones(uint32_t a, float c)
{
    if constexpr (ACT == ACT_F16) {
        return __builtin_amdgcn_fdot2(h2_of(a), (half2_t){(_Float16)1.0f, (_Float16)1.0f}, c, false);
    } else {
        typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a), __builtin_bit_cast(bf162_t, 0x3F803F80u),
                                               c, false);
    }
}

// bf16: build 2^23 + c as a float (0x4B000000 | c), subtract 2^23 + z
// exactly, and keep the upper half of the float -- exact for the small
// integer c - z (and for (c - z) * s the bf16 conversion rounds to nearest
// even).
__device__ inline uint32_t bf16_pair_from_f32(float lo, float hi)
{
    __bf16 a = (__bf16)lo;
    __bf16 b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ inline float nib_f32(uint32_t w, int p, float off)
{
    return __uint_as_float(0x4B000000u | ((w >> (4 * p)) & 0xFu)) + off;
}

// off = -(2^23 + z)
__device__ inline u32x4 dequant_bf16(uint32_t w, float off)
{
    u32x4 r;
    r.x = bf16_pair_from_f32(nib_f32(w, 0, off), nib_f32(w, 4, off));
    r.y = bf16_pair_from_f32(nib_f32(w, 1, off), nib_f32(w, 5, off));
    r.z = bf16_pair_from_f32(nib_f32(w, 2, off), nib_f32(w, 6, off));
    r.w = bf16_pair_from_f32(nib_f32(w, 3, off), nib_f32(w, 7, off));
    return r;
}

// bf16 (0x4300 | c) is 128 + c exactly, built per pair; the caller removes
// 128 + z afterwards.  Written in plain C, not with and_or: these values
// are MFMA operands, and the compiler must see the instructions that write
// them to keep the VALU-to-MFMA wait states.
__device__ inline u32x4 bf16_biased(uint32_t w)
{
    const uint32_t w8 = w >> 8;
    const uint32_t m = reg_const(0x000F000Fu), b = reg_const(0x43004300u);
    u32x4 r;
    r.x = (w & m) | b;
    r.y = ((w >> 4) & m) | b;
    r.z = (w8 & m) | b;
    r.w = ((w8 >> 4) & m) | b;
    return r;
}

// q s + c in fp32 with c = -z s, then rounded to bf16.  z s is exact in fp32
// (two fp16 values carry at most 22 significant bits), so the fused
// multiply-add rounds (q - z) s once, for any fp16 zero point z.
__device__ inline float nib_val(uint32_t w, int p) { return (float)((w >> (4 * p)) & 0xFu); }

__device__ inline u32x4 dequant_bf16_scaled(uint32_t w, float s, float c)
{
    u32x4 r;
    r.x = bf16_pair_from_f32(fmaf(nib_val(w, 0), s, c), fmaf(nib_val(w, 4), s, c));
    r.y = bf16_pair_from_f32(fmaf(nib_val(w, 1), s, c), fmaf(nib_val(w, 5), s, c));
    r.z = bf16_pair_from_f32(fmaf(nib_val(w, 2), s, c), fmaf(nib_val(w, 6), s, c));
    r.w = bf16_pair_from_f32(fmaf(nib_val(w, 3), s, c), fmaf(nib_val(w, 7), s, c));
    return r;
}

// ------------------------------------------------------------ gate

__device__ inline float sigmoid_f32(float l)
{
    if (l >= 0.0f)
        return 1.0f / (1.0f + expf(-l));
    float e = expf(l);
    return e / (1.0f + e);
}

// ------------------------------------------------------------ cross-workgroup hand-over
//
// Partial results handed from one workgroup to another (possibly on another
// XCD, with its own L2) are written and read with device-scope coherent
// accesses (relaxed agent-scope atomics: global loads / stores with the sc1
// bit), which gfx950 keeps coherent across XCDs per access.  The writer
// waits for its stores to complete (s_waitcnt 0) and meets its workgroup at
// a barrier before one thread bumps the arrival counter; a reader issues its
// loads only after it has seen the counter.  No whole-cache write-back or
// invalidate (what agent-scope fences compile to) is needed on either side.

__device__ inline void st4_dev(float* p, float v)
{
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float ld4_dev(const float* p)
{
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
}

__device__ inline void st16_dev(floatx4* p, floatx4 v)
{
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
    const uint64_t lo = (uint64_t)__float_as_uint(v.x) | ((uint64_t)__float_as_uint(v.y) << 32);
    const uint64_t hi = (uint64_t)__float_as_uint(v.z) | ((uint64_t)__float_as_uint(v.w) << 32);
    __hip_atomic_store(q, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline floatx4 ld16_dev(const floatx4* p)
{
    const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (floatx4){__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                     __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32))};
}

// 16-byte device-coherent accesses through a buffer resource (base and size
// wave-uniform, byte offset per lane): sc1 stores write through to memory and
// sc1 loads read past this XCD's L2, like the relaxed agent-scope atomics
// above, but as one contiguous 16-byte access per lane (two strided 8-byte
// accesses write whole 32-byte sectors for 8 bytes each).  Offsets at or
// past `bytes` read as zero and are not written.
__device__ inline __amdgpu_buffer_rsrc_t dev_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int CPOL_SC1 = 16;
__device__ inline void st16_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off, floatx4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, CPOL_SC1);
}
__device__ inline floatx4 ld16_sc1(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CPOL_SC1));
}

// Self-announcing hand-over words.  A value is stored as the bit complement
// of its encoding, so the zero word that a cleared buffer holds means "not
// written yet" and a reader can take each value as soon as it lands, with no
// flag, counter or store acknowledgement in between.  The one encoding whose
// complement is zero is an all-ones NaN; it is replaced by another NaN.
__device__ inline uint32_t hw_enc32(float v)
{
    const uint32_t b = __float_as_uint(v);
    return ~(b == 0xFFFFFFFFu ? 0xFFC00000u : b);
}
__device__ inline float hw_dec32(uint32_t w) { return __uint_as_float(~w); }
// 16-bit values (fp16 or bf16; 0xFFC0 is a NaN in both)
__device__ inline uint16_t hw_enc16(uint16_t b) { return (uint16_t)~(b == 0xFFFFu ? 0xFFC0u : b); }
// nonzero iff a word of four 16-bit values holds one not written yet (a
// zero lane)
__device__ inline uint64_t hw_missing16(uint64_t w)
{
    return (w - 0x0001000100010001ull) & ~w & 0x8000800080008000ull;
}

__device__ inline uint64_t ld8_dev(const uint64_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void st8_dev(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// all of this thread's outstanding memory operations have completed
__device__ inline void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Workgroup barrier for data exchanged through LDS only: waits for this
// wavefront's LDS operations (lgkmcnt 0) but, unlike __syncthreads(), not for
// its global loads in flight (the s_waitcnt immediate keeps vmcnt and expcnt
// at their maximum).
__device__ inline void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
}

__device__ inline uint32_t atomic_add_dev(uint32_t* p, uint32_t v)
{
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint32_t atomic_load_dev(const uint32_t* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void atomic_store_dev(uint32_t* p, uint32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A bounded wait: every waiter gives up after this many polls (roughly a
// second) so that a broken hand-over can never hang the GPU; it then records
// the failure in the workspace and its results become NaN.  The host can
// lower the limit (w4ec_set_wait_limit); 0 makes every wait give up at once.
constexpr uint32_t SPIN_LIMIT = 1u << 22;

// ------------------------------------------------------------ launch plans
// (shared by the host dispatch and the workspace sizing)

// Geometry of a staged [A | w_g] slice (the decode EC role and the prefill
// prepass): halves per LDS row of an A slice (the transpose read needs 8-byte
// aligned rows); column blocks of A, and the total with the gate block; LDS
// bytes of a slice of kc rows (plus slack for the last block's over-read).
__host__ __device__ inline int ec_pitch(int r) { return (r + 3) & ~3; }
__host__ __device__ inline int ec_a_blocks(int r) { return (r + 15) >> 4; }
__host__ __device__ inline int ec_blocks(int r) { return ec_a_blocks(r) + 1; }
__host__ __device__ inline int ec_slice_bytes(int r, int kc) { return (kc * ec_pitch(r) + 16) * 2; }
// LDS of a prepass workgroup: the slice and its gate vector
inline size_t prepass_lds_bytes(int r, int kc) { return (size_t)ec_slice_bytes(r, kc) + (size_t)kc * 2; }
// LDS of a prefill GEMM workgroup of BM tokens: two staged 128-k steps of X,
// or the rounded output tile (rows of GEMM_YT_PITCH halves), whichever is
// larger
constexpr int GEMM_YT_PITCH = 264;
__host__ __device__ constexpr int gemm_lds_bytes_of(int BM)
{
    return (2 * BM * PANEL_K * 2 > BM * GEMM_YT_PITCH * 2) ? 2 * BM * PANEL_K * 2 : BM * GEMM_YT_PITCH * 2;
}
// LDS array of a 64-token GEMM workgroup: at least the main loop's and the
// epilogue's, and room for a fused-EC slice of [A | w_g] (a workgroup holds
// a CU's registers, so its LDS costs no occupancy)
constexpr int GEMM_EC_LDS = 128 << 10;
__host__ __device__ constexpr int gemm_smem_bytes_of(int BM)
{
    return gemm_lds_bytes_of(BM) > GEMM_EC_LDS ? gemm_lds_bytes_of(BM) : GEMM_EC_LDS;
}

constexpr int DEC_THREADS = 256;     // threads per decode workgroup
constexpr int DEC_XLDS_CHUNKS = 8;   // 16-byte chunks of staged activations per decode thread
// the decode main role stages X in LDS for at most 4 tokens and this many bytes
constexpr size_t DEC_XLDS_MAX_BYTES = (size_t)DEC_XLDS_CHUNKS * 16 * DEC_THREADS;
inline bool decode_use_xlds(int M, int K) { return M <= 4 && (size_t)M * K * 2 <= DEC_XLDS_MAX_BYTES; }

constexpr int DEC_EC_KS = 256;   // at most this many k per decode EC workgroup
constexpr int DEC_EC_RMAX = 128; // at most this many decode EC workgroups reduce (half the CUs)
constexpr int DEC_NREP = 32;                    // replica slots of the decode hand-over
constexpr size_t DEC_REP_CTRL_STRIDE = 4096;    // control words of one slot (own page)
constexpr size_t DEC_REP_DATA_STRIDE = 8192;    // T_g of one slot: up to 16 tokens x 256 ranks x 2 bytes

struct DecodePlan {
    int P;          // EC workgroups (K slices) -- 0 when r == 0
    int KS;         // k per EC slice (multiple of 64)
    int RC;         // partial columns: r (low rank) + 1 (gate logit)
    int r_pad;      // r rounded up to 32
    int CB;         // column blocks per main workgroup
    int n_main;     // main workgroups
    bool xlds;      // main workgroups stage the activations in LDS
    int stage_first;  // main workgroups stage X before issuing weight loads
    bool ok;        // the shape fits the workspace's control region
    size_t off_flags, off_partial, off_rep_ctrl, off_rep_data, bytes;
};

struct PrefillPlan {
    int BM;         // tokens per GEMM tile (64 or 128)
    int BN;         // columns per GEMM tile (256)
    int mt, nt;     // tiles along M and N
    int ksplit;     // GEMM split over K
    int pre_mt;     // prepass tiles of 64 tokens
    int pre_ks;     // prepass split over K
    int pre_kc;     // k per prepass chunk (multiple of 64, <= 512)
    int pre_nch;    // chunks per prepass workgroup (its K slice: pre_nch pre_kc)
    int r_pad, Mpad;
    int ec_q;       // fused EC: pieces of [T | l] per row of tiles (0: the prepass kernels instead)
    int ec_kc;      // fused EC: k per LDS slice of [A | w_g] (multiple of 64, <= 512)
    size_t off_flags, off_gemm_cnt, off_ec_cnt, off_pre_partial, off_tg, off_rowsum, off_gemm_partial, bytes;
};

}  // namespace w4ec
