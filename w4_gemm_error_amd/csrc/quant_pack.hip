// quant_pack.hip -- offline weight preparation on the GPU: RTN int4
// quantization into canonical codes, and the canonical <-> blob re-layout.
#include <algorithm>

#include "w4ec_common.h"
#include "w4ec_launch.h"

namespace w4ec {

// ---------------------------------------------------------------- fp16 <-> double

// binary16 bits -> double (exact).
__device__ inline double half_bits_to_f64(uint16_t h)
{
    return (double)(float)__builtin_bit_cast(_Float16, h);
}

// double -> binary16 bits, round to nearest even, working on the bit
// pattern of the double: keep the top 11 significant bits (fewer for
// results in the subnormal range) and round on the dropped remainder.
__device__ inline uint16_t f64_to_half_bits_rne(double x)
{
    uint64_t u = (uint64_t)__double_as_longlong(x);
    uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    if (a >= 0x7FF0000000000000ull)                        // inf / nan
        return sign | (a > 0x7FF0000000000000ull ? 0x7E00 : 0x7C00);
    int ebits = (int)(a >> 52);
    if (ebits == 0)                                        // double zero / subnormal
        return sign;
    int eh = ebits - 1023 + 15;                            // biased half exponent
    uint64_t mant = (a & 0xFFFFFFFFFFFFFull) | (1ull << 52);
    if (eh >= 31)
        return sign | 0x7C00;
    if (eh < -11)                                          // below half of the smallest subnormal
        return sign;
    int shift = (eh >= 1) ? 42 : 43 - eh;                  // bits dropped from the 53-bit significand
    uint64_t kept = mant >> shift;
    uint64_t rem = mant & ((1ull << shift) - 1);
    uint64_t halfway = 1ull << (shift - 1);
    if (rem > halfway || (rem == halfway && (kept & 1)))
        ++kept;
    if (eh >= 1) {
        if (kept == 2048) {                                // carried into the next binade
            kept = 1024;
            ++eh;
            if (eh >= 31)
                return sign | 0x7C00;
        }
        return sign | (uint16_t)(eh << 10) | (uint16_t)(kept & 0x3FF);
    }
    return sign | (uint16_t)kept;                          // subnormal (1024 encodes 2^-14)
}

// ---------------------------------------------------------------- RTN

constexpr int QT = 128;  // threads per (row, group)

__global__ __launch_bounds__(QT)
void rtn_quantize_kernel(const float* __restrict__ W, int N, int K, int G,
                         uint8_t* __restrict__ qc, uint16_t* __restrict__ scale,
                         uint16_t* __restrict__ zero)
{
    const int n = blockIdx.y;
    const int gi = blockIdx.x;
    const int NG = K / G;
    const float* w = W + (size_t)n * K + (size_t)gi * G;
    __shared__ float s_lo[QT], s_hi[QT];
    __shared__ double s_scale;
    __shared__ int s_zero;

    float lo = 0.0f, hi = 0.0f;
    for (int k = threadIdx.x; k < G; k += QT) {
        float v = w[k];
        lo = fminf(lo, v);
        hi = fmaxf(hi, v);
    }
    s_lo[threadIdx.x] = lo;
    s_hi[threadIdx.x] = hi;
    __syncthreads();
    for (int off = QT / 2; off > 0; off >>= 1) {
        if (threadIdx.x < off) {
            s_lo[threadIdx.x] = fminf(s_lo[threadIdx.x], s_lo[threadIdx.x + off]);
            s_hi[threadIdx.x] = fmaxf(s_hi[threadIdx.x], s_hi[threadIdx.x + off]);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        double dlo = (double)s_lo[0], dhi = (double)s_hi[0];
        uint16_t sh = 0;
        if (dhi > dlo)
            sh = f64_to_half_bits_rne((dhi - dlo) / 15.0);
        if (sh == 0x7C00)
            sh = 0x7BFF;
        double s;
        int z;
        if (sh == 0) {
            sh = 0x3C00;
            s = 1.0;
            z = 0;
        } else {
            s = half_bits_to_f64(sh);
            double zz = rint(-dlo / s);
            z = (int)(zz < 0.0 ? 0.0 : (zz > 15.0 ? 15.0 : zz));
        }
        scale[(size_t)n * NG + gi] = sh;
        zero[(size_t)n * NG + gi] = f64_to_half_bits_rne((double)z);
        s_scale = s;
        s_zero = z;
    }
    __syncthreads();
    const double s = s_scale;
    const double z = (double)s_zero;
    uint8_t* out = qc + (size_t)n * (K / 2) + (size_t)gi * (G / 2);
    for (int b = threadIdx.x; b < G / 2; b += QT) {
        double q0 = rint((double)w[2 * b] / s) + z;
        double q1 = rint((double)w[2 * b + 1] / s) + z;
        int c0 = (int)(q0 < 0.0 ? 0.0 : (q0 > 15.0 ? 15.0 : q0));
        int c1 = (int)(q1 < 0.0 ? 0.0 : (q1 > 15.0 ? 15.0 : q1));
        out[b] = (uint8_t)(c0 | (c1 << 4));
    }
}

// ---------------------------------------------------------------- pack / unpack

// One thread per blob dword (8 codes).  natural: code t of the dword in
// nibble t (the codebook layout, whose bytes are pairs of consecutive k),
// else in the nibble that the affine dequantization expects.
__global__ void pack_codes_kernel(const uint8_t* __restrict__ qc, int N, int K,
                                  int NB, int KB, uint32_t* __restrict__ codes, int natural)
{
    size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t total = (size_t)NB * KB * (PANEL_BYTES / 4);
    if (idx >= total)
        return;
    int s = (int)(idx & 3);
    int l = (int)((idx >> 2) & 63);
    size_t panel = idx >> 8;
    int kb = (int)(panel % KB);
    int cb = (int)(panel / KB);
    int n = cb * PANEL_N + (l & 15);
    int k0 = kb * PANEL_K + 32 * s + 8 * (l >> 4);
    uint32_t word = 0;
    if (n < N) {
        const uint8_t* src = qc + (size_t)n * (K / 2) + (k0 >> 1);
        for (int t = 0; t < 8; ++t) {
            uint32_t byte = src[t >> 1];
            uint32_t c = (t & 1) ? (byte >> 4) : (byte & 0xF);
            word |= c << (4 * (natural ? t : nibble_of(t)));
        }
    }
    codes[idx] = word;
}

__global__ void pack_sz_kernel(const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero,
                               int N, int NG, int Npad, uint32_t* __restrict__ sz,
                               BlobHeader* __restrict__ hdr)
{
    size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)NG * Npad)
        return;
    int gi = (int)(idx / Npad);
    int n = (int)(idx % Npad);
    uint32_t v = 0;
    if (n < N && !scale) {
        v = 0x3C00u;                                 // scale 1, zero 0 (codebook blob)
    } else if (n < N) {
        uint16_t s = scale[(size_t)n * NG + gi];
        uint16_t z = zero[(size_t)n * NG + gi];
        float zf = (float)__builtin_bit_cast(_Float16, z);
        // any zero point is accepted; the kernels take its integer part
        // exactly and correct for a fractional part, which needs |z| <= ZMAX.
        // One outside that range (or not finite) is stored as NaN, which
        // turns the outputs that use it into NaN.
        const uint32_t f = !(fabsf(zf) <= ZMAX) ? ZF_BAD : (zf != floorf(zf) ? ZF_FRAC : 0u);
        if (f)
            atomicOr(&hdr->zflags, f);
        if (f & ZF_BAD)
            z = 0x7E00u;
        v = (uint32_t)s | ((uint32_t)z << 16);
    }
    sz[idx] = v;
}

__global__ void write_header_kernel(BlobHeader* hdr, int N, int K, int G)
{
    if (threadIdx.x == 0 && blockIdx.x == 0) {
        hdr->magic = BLOB_MAGIC;
        hdr->N = N;
        hdr->K = K;
        hdr->G = G;
        hdr->zflags = 0;
    }
}

// One thread per canonical byte (2 codes).
__global__ void unpack_codes_kernel(const uint32_t* __restrict__ codes, int N, int K, int KB,
                                    uint8_t* __restrict__ qc)
{
    size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)N * (K / 2))
        return;
    int n = (int)(idx / (K / 2));
    int k = 2 * (int)(idx % (K / 2));
    int cb = n / PANEL_N, kb = k / PANEL_K, kin = k % PANEL_K;
    int s = kin / 32, kr = kin % 32;
    int l = (n % PANEL_N) + 16 * (kr / 8);
    int t = kr % 8;
    uint32_t word = codes[((size_t)cb * KB + kb) * (PANEL_BYTES / 4) + (size_t)l * 4 + s];
    uint32_t c0 = (word >> (4 * nibble_of(t))) & 0xF;
    uint32_t c1 = (word >> (4 * nibble_of(t + 1))) & 0xF;
    qc[idx] = (uint8_t)(c0 | (c1 << 4));
}

__global__ void unpack_sz_kernel(const uint32_t* __restrict__ sz, int N, int NG, int Npad,
                                 uint16_t* __restrict__ scale, uint16_t* __restrict__ zero)
{
    size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)N * NG)
        return;
    int n = (int)(idx / NG);
    int gi = (int)(idx % NG);
    uint32_t v = sz[(size_t)gi * Npad + n];
    scale[idx] = (uint16_t)(v & 0xFFFF);
    zero[idx] = (uint16_t)(v >> 16);
}

// ---------------------------------------------------------------- launchers

static inline unsigned blocks_for(size_t n, unsigned t) { return (unsigned)((n + t - 1) / t); }

hipError_t launch_rtn_quantize(const float* W, int N, int K, int G, uint8_t* qc,
                               uint16_t* scale, uint16_t* zero, hipStream_t st)
{
    dim3 grid(K / G, N);
    hipLaunchKernelGGL(rtn_quantize_kernel, grid, dim3(QT), 0, st, W, N, K, G, qc, scale, zero);
    return hipGetLastError();
}

hipError_t launch_pack(const uint8_t* qc, const uint16_t* scale, const uint16_t* zero,
                       int N, int K, int G, void* packed, hipStream_t st)
{
    BlobGeom g = blob_geom(N, K, G);
    char* base = (char*)packed;
    BlobHeader* hdr = (BlobHeader*)base;
    hipLaunchKernelGGL(write_header_kernel, dim3(1), dim3(64), 0, st, hdr, N, K, G);
    size_t nw = (size_t)g.NB * g.KB * (PANEL_BYTES / 4);
    hipLaunchKernelGGL(pack_codes_kernel, dim3(blocks_for(nw, 256)), dim3(256), 0, st,
                       qc, N, K, g.NB, g.KB, (uint32_t*)(base + g.codes_off), scale ? 0 : 1);
    size_t ns = (size_t)g.NG * g.Npad;
    hipLaunchKernelGGL(pack_sz_kernel, dim3(blocks_for(ns, 256)), dim3(256), 0, st,
                       scale, zero, N, g.NG, g.Npad, (uint32_t*)(base + g.sz_off), hdr);
    return hipGetLastError();
}

hipError_t launch_unpack(const void* packed, int N, int K, int G, uint8_t* qc,
                         uint16_t* scale, uint16_t* zero, hipStream_t st)
{
    BlobGeom g = blob_geom(N, K, G);
    const char* base = (const char*)packed;
    size_t nb = (size_t)N * (K / 2);
    hipLaunchKernelGGL(unpack_codes_kernel, dim3(blocks_for(nb, 256)), dim3(256), 0, st,
                       (const uint32_t*)(base + g.codes_off), N, K, g.KB, qc);
    size_t ns = (size_t)N * g.NG;
    hipLaunchKernelGGL(unpack_sz_kernel, dim3(blocks_for(ns, 256)), dim3(256), 0, st,
                       (const uint32_t*)(base + g.sz_off), N, g.NG, g.Npad, scale, zero);
    return hipGetLastError();
}

// ---------------------------------------------------------------- workspace reset

__global__ __launch_bounds__(256) void zero_fill_kernel(u32x4* p, size_t n16)
{
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
        p[i] = (u32x4){0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------- streaming-read reference
//
// The plainest read of a buffer: STREAM_WGS workgroups of 256 threads, each
// workgroup a contiguous share of the 16-byte chunks (ceil(n / STREAM_WGS)),
// each thread with STREAM_BATCH 16-byte non-temporal loads in flight at once
// (one round trip for a ~32 MB buffer), folding the data into one XOR word
// per workgroup so that no load can be dropped.  Its duration is the
// attainable HBM read time for a byte count, the reference for the decode's
// fraction of the roofline.
constexpr int STREAM_WGS = 512;
constexpr int STREAM_BATCH = 16;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16, uint32_t* sink)
{
    __shared__ uint32_t part[4];
    const size_t per = (n16 + STREAM_WGS - 1) / STREAM_WGS;
    const size_t lo = (size_t)blockIdx.x * per;
    const size_t hi = lo + per < n16 ? lo + per : n16;
    u32x4 acc = (u32x4){0u, 0u, 0u, 0u};
    for (size_t b = lo + threadIdx.x; b < hi; b += 256 * STREAM_BATCH) {
        u32x4 v[STREAM_BATCH];
#pragma unroll
        for (int u = 0; u < STREAM_BATCH; ++u) {         // past the share: re-read its last chunk, unused
            const size_t i = b + 256 * (size_t)u;
            v[u] = ld16_stream(src + (i < hi ? i : hi - 1));
        }
#pragma unroll
        for (int u = 0; u < STREAM_BATCH; ++u)
            if (b + 256 * (size_t)u < hi)
                acc ^= v[u];
    }
    uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        x ^= (uint32_t)__shfl_xor((int)x, o);
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0)
        sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st)
{
    hipLaunchKernelGGL(stream_read_kernel, dim3(STREAM_WGS), dim3(256), 0, st, (const u32x4*)src, bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t st)
{
    const size_t n16 = bytes / 16;
    if (n16 == 0)
        return hipSuccess;
    const size_t wgs = std::min<size_t>((n16 + 255) / 256, 2048);
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)wgs), dim3(256), 0, st, (u32x4*)p, n16);
    return hipGetLastError();
}

}  // namespace w4ec
