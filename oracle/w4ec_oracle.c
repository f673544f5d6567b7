/*
 * w4ec_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
 *
 * A plain, slow, float64 CPU reference for the weight-only 4-bit linear layer
 * with an input-adaptive error compensator (EC).  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load this file's
 * library; the GPU library never links, includes or calls it, and the two
 * share no code.
 *
 * What it computes (SPEAR, "A System for Post-Quantization Error-Adaptive
 * Recovery" -- gist.science technical summary, section 2.1A "input-adaptive
 * error compensators": the effective weight is the quantized weight plus a
 * gated low-rank product of an down-projection A and an up-projection B; the
 * gate is a per-token scalar, sigmoid(x . w_g + b_g), with the scale alpha
 * taken as 1 and folded into B):
 *
 *   q[n,k]  = nibble k of row n of the canonical code array
 *   Wd[n,k] = (q[n,k] - z[n,k/G]) * s[n,k/G]                 (asymmetric int4)
 *   Y0[m,n] = sum_k X[m,k] * Wd[n,k]                          (plain W4 layer)
 *   T[m,j]  = sum_k X[m,k] * A[k,j]                           (rank-r down-proj)
 *   l[m]    = sum_k X[m,k] * w_g[k] + b_g ;  g[m] = 1/(1+exp(-l[m]))
 *   C[m,n]  = sum_j T[m,j] * B[j,n]                           (rank-r up-proj)
 *   Y[m,n]  = Y0[m,n] + g[m] * C[m,n]
 *
 * Every sum is a naive loop with its index ascending, in float64, on inputs
 * widened exactly from fp16 / bf16.  No blocking, no reordering, no fusion.
 *
 * The round-to-nearest (RTN) quantizer follows the per-channel RTN baseline
 * that the SPEAR summary's results section (3.1) names as its W4 setting:
 * per row (or per group of G input features) the range [min(w,0), max(w,0)]
 * is mapped onto the 16 codes; the scale is rounded to fp16 before the zero
 * point and the codes are derived from it, so the stored parameters
 * reproduce the codes.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared -ffp-contract=off (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- formats */

/* IEEE-754 binary16 -> double, exact (every half is a double). */
double w4o_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* zero / subnormal */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);     /* 1.m * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 -> double, exact: a bf16 is the upper half of a binary32. */
double w4o_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* double -> binary16 with round-to-nearest-even, from the definition:
 * pick the quantum (spacing) of the binade the value falls in, round the
 * value to a whole number of quanta, then encode.  Overflow gives infinity
 * (values at or above 65520 round up to 2^16). */
uint16_t w4o_double_to_half(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isnan(x))
        return 0x7e00;
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7c00;
    int e2;
    frexp(a, &e2);                       /* a = f * 2^e2, f in [0.5, 1) */
    int p = e2 - 1;                      /* a in [2^p, 2^(p+1)) */
    int qexp = (p < -14) ? -24 : p - 10; /* quantum 2^qexp */
    double n = rint(ldexp(a, -qexp));    /* whole quanta, ties to even */
    double v = ldexp(n, qexp);
    if (v >= 65536.0)
        return sign | 0x7c00;
    if (v < ldexp(1.0, -14))             /* subnormal: n quanta of 2^-24 */
        return sign | (uint16_t)n;       /* n == 1024 encodes 2^-14 */
    frexp(v, &e2);
    p = e2 - 1;
    uint16_t mant = (uint16_t)(ldexp(v, 10 - p) - 1024.0);
    return sign | (uint16_t)((p + 15) << 10) | mant;
}

static double act_to_double(uint16_t v, int act_bf16)
{
    return act_bf16 ? w4o_bf16_to_double(v) : w4o_half_to_double(v);
}

/* ---------------------------------------------------------------- codes */

/* Canonical code array: uint8 [N][K/2]; byte k/2 of row n holds code k in
 * its low nibble when k is even and in its high nibble when k is odd. */
static int code_at(const uint8_t* qc, int K, int n, int k)
{
    uint8_t byte = qc[(size_t)n * (size_t)(K / 2) + (size_t)(k >> 1)];
    return (k & 1) ? (byte >> 4) : (byte & 0x0f);
}

/* Expand the canonical array into one code per byte (uint8 [N][K]). */
void w4o_unpack_codes(const uint8_t* qc, int N, int K, uint8_t* q)
{
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            q[(size_t)n * K + k] = (uint8_t)code_at(qc, K, n, k);
}

/* ---------------------------------------------------------------- RTN */

/* Round-to-nearest asymmetric int4 quantization of W (float32 [N][K]) with
 * one (scale, zero) pair per row and group of G consecutive input features.
 * Outputs: canonical codes qc [N][K/2], scale and zero as binary16 bits
 * [N][K/G].  Every step is in float64:
 *   lo = min(min_k w, 0), hi = max(max_k w, 0)
 *   s  = fp16((hi - lo) / 15)   (clamped to the largest finite half)
 *   z  = clamp(rint(-lo / s), 0, 15)
 *   q  = clamp(rint(w / s) + z, 0, 15)
 * A group whose range is zero, or so small that s rounds to zero in fp16,
 * gets s = 1, z = 0 (all its codes are then 0). */
void w4o_rtn_quantize(const float* W, int N, int K, int G,
                      uint8_t* qc, uint16_t* scale, uint16_t* zero)
{
    int ngroups = K / G;
    memset(qc, 0, (size_t)N * (size_t)(K / 2));
    for (int n = 0; n < N; ++n) {
        for (int gi = 0; gi < ngroups; ++gi) {
            const float* w = W + (size_t)n * K + (size_t)gi * G;
            double lo = 0.0, hi = 0.0;
            for (int k = 0; k < G; ++k) {
                double v = (double)w[k];
                if (v < lo) lo = v;
                if (v > hi) hi = v;
            }
            uint16_t sh = 0;
            if (hi > lo)
                sh = w4o_double_to_half((hi - lo) / 15.0);
            if (sh == 0x7c00)
                sh = 0x7bff;
            double s;
            int z;
            if (sh == 0) {
                sh = 0x3c00; /* 1.0 */
                s = 1.0;
                z = 0;
            } else {
                s = w4o_half_to_double(sh);
                double zz = rint(-lo / s);
                z = (int)(zz < 0.0 ? 0.0 : (zz > 15.0 ? 15.0 : zz));
            }
            scale[(size_t)n * ngroups + gi] = sh;
            zero[(size_t)n * ngroups + gi] = w4o_double_to_half((double)z);
            for (int k = 0; k < G; ++k) {
                double qq = rint((double)w[k] / s) + (double)z;
                int q = (int)(qq < 0.0 ? 0.0 : (qq > 15.0 ? 15.0 : qq));
                int kk = gi * G + k;
                size_t byte = (size_t)n * (size_t)(K / 2) + (size_t)(kk >> 1);
                qc[byte] |= (uint8_t)((kk & 1) ? (q << 4) : q);
            }
        }
    }
}

/* ---------------------------------------------------------------- forward */

/* Gate: logistic function in a form that does not overflow; +inf -> 1,
 * -inf -> 0 exactly. */
static double sigmoid(double l)
{
    if (l >= 0.0)
        return 1.0 / (1.0 + exp(-l));
    double e = exp(l);
    return e / (1.0 + e);
}

/* The full layer for a subset of tokens.
 *
 *   X      act bits [M][K]        (act_bf16: 0 = fp16, 1 = bf16)
 *   qc     canonical codes [N][K/2]
 *   scale, zero  fp16 bits [N][K/G]
 *   A      act bits [K][r]   B act bits [r][N]   w_g act bits [K] or NULL
 *   b_g    gate bias
 *   rows   token indices to evaluate (NULL: all M, in order), n_rows of them
 * Outputs, indexed by position i in `rows` (any may be NULL except Y):
 *   Y, Y0, C [n_rows][N];  T [n_rows][r];  g [n_rows]
 * Returns 0, or -1 on bad arguments or allocation failure. */
int w4o_forward(int M, int N, int K, int r, int G, int act_bf16,
                const uint16_t* X, const uint8_t* qc,
                const uint16_t* scale, const uint16_t* zero,
                const uint16_t* A, const uint16_t* B, const uint16_t* w_g,
                double b_g, const int* rows, int n_rows,
                double* Y, double* Y0, double* T, double* g, double* C)
{
    if (M < 0 || N <= 0 || K <= 0 || r < 0 || G <= 0 || K % G || K % 2 || !Y)
        return -1;
    if (!rows)
        n_rows = M;
    if (n_rows <= 0)
        return 0;
    int ngroups = K / G;

    double* xd = (double*)malloc(sizeof(double) * (size_t)n_rows * K);
    double* td = (double*)malloc(sizeof(double) * (size_t)n_rows * (r > 0 ? r : 1));
    double* gd = (double*)malloc(sizeof(double) * (size_t)n_rows);
    if (!xd || !td || !gd) {
        free(xd); free(td); free(gd);
        return -1;
    }
    for (int i = 0; i < n_rows; ++i) {
        int m = rows ? rows[i] : i;
        if (m < 0 || m >= M) {
            free(xd); free(td); free(gd);
            return -1;
        }
        for (int k = 0; k < K; ++k)
            xd[(size_t)i * K + k] = act_to_double(X[(size_t)m * K + k], act_bf16);
    }

    /* T = X A and the gate, one token at a time. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n_rows; ++i) {
        const double* x = xd + (size_t)i * K;
        for (int j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += x[k] * act_to_double(A[(size_t)k * r + j], act_bf16);
            td[(size_t)i * r + j] = acc;
        }
        double l = 0.0;
        if (w_g)
            for (int k = 0; k < K; ++k)
                l += x[k] * act_to_double(w_g[k], act_bf16);
        l += b_g;
        gd[i] = sigmoid(l);
    }

    /* One output feature at a time: dequantize row n of W, then every token. */
    int bad = 0;
#pragma omp parallel
    {
        double* wd = (double*)malloc(sizeof(double) * (size_t)K);
        double* bc = (double*)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
        if (!wd || !bc) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 8)
        for (int n = 0; n < N; ++n) {
            if (!wd || !bc)
                continue;
            for (int k = 0; k < K; ++k) {
                int gi = k / G;
                double s = w4o_half_to_double(scale[(size_t)n * ngroups + gi]);
                double z = w4o_half_to_double(zero[(size_t)n * ngroups + gi]);
                wd[k] = ((double)code_at(qc, K, n, k) - z) * s;
            }
            for (int j = 0; j < r; ++j)
                bc[j] = act_to_double(B[(size_t)j * N + n], act_bf16);
            for (int i = 0; i < n_rows; ++i) {
                const double* x = xd + (size_t)i * K;
                double y0 = 0.0;
                for (int k = 0; k < K; ++k)
                    y0 += x[k] * wd[k];
                double c = 0.0;
                for (int j = 0; j < r; ++j)
                    c += td[(size_t)i * r + j] * bc[j];
                size_t o = (size_t)i * N + n;
                Y[o] = y0 + gd[i] * c;
                if (Y0) Y0[o] = y0;
                if (C) C[o] = c;
            }
        }
        free(wd);
        free(bc);
    }
    if (T)
        memcpy(T, td, sizeof(double) * (size_t)n_rows * r);
    if (g)
        memcpy(g, gd, sizeof(double) * (size_t)n_rows);
    free(xd);
    free(td);
    free(gd);
    return bad ? -1 : 0;
}

/* The layer with a vector gate: one gate per rank component, for a subset
 * of tokens.  The SPEAR summary (section 2.1A) writes the compensated weight
 * as W + alpha B diag(gamma(A x)) A, with gamma a small bottleneck MLP on the
 * rank-r projection; it names neither the MLP's activation nor its width.
 * Read here as a two-layer bottleneck of width h with a ReLU, and a sigmoid
 * on its output so that each component is a gate in (0, 1) like the scalar
 * gate; alpha is folded into B as in w4o_forward:
 *
 *   T[m,j]     = sum_k X[m,k] * A[k,j]
 *   u[m,i]     = max(0, sum_j T[m,j] * G1[j,i] + c1[i])          i < h
 *   gamma[m,j] = sigmoid(sum_i u[m,i] * G2[i,j] + c2[j])         j < r
 *   C[m,n]     = sum_j gamma[m,j] * T[m,j] * B[j,n]
 *   Y[m,n]     = Y0[m,n] + C[m,n]
 *
 *   G1 act bits [r][h], c1 act bits [h], G2 act bits [h][r], c2 act bits [r]
 * Other arguments and outputs as w4o_forward, with gamma [n_rows][r] in
 * place of g.  Returns 0, or -1 on bad arguments or allocation failure. */
int w4o_forward_vgate(int M, int N, int K, int r, int G, int act_bf16, int h,
                      const uint16_t* X, const uint8_t* qc,
                      const uint16_t* scale, const uint16_t* zero,
                      const uint16_t* A, const uint16_t* B,
                      const uint16_t* G1, const uint16_t* c1,
                      const uint16_t* G2, const uint16_t* c2,
                      const int* rows, int n_rows,
                      double* Y, double* Y0, double* T, double* gamma, double* C)
{
    if (M < 0 || N <= 0 || K <= 0 || r <= 0 || h <= 0 || G <= 0 || K % G || K % 2 || !Y)
        return -1;
    if (!A || !B || !G1 || !c1 || !G2 || !c2)
        return -1;
    if (!rows)
        n_rows = M;
    if (n_rows <= 0)
        return 0;
    int ngroups = K / G;

    double* xd = (double*)malloc(sizeof(double) * (size_t)n_rows * K);
    double* td = (double*)malloc(sizeof(double) * (size_t)n_rows * r);
    double* gd = (double*)malloc(sizeof(double) * (size_t)n_rows * r);
    double* ud = (double*)malloc(sizeof(double) * (size_t)n_rows * h);
    if (!xd || !td || !gd || !ud) {
        free(xd); free(td); free(gd); free(ud);
        return -1;
    }
    for (int i = 0; i < n_rows; ++i) {
        int m = rows ? rows[i] : i;
        if (m < 0 || m >= M) {
            free(xd); free(td); free(gd); free(ud);
            return -1;
        }
        for (int k = 0; k < K; ++k)
            xd[(size_t)i * K + k] = act_to_double(X[(size_t)m * K + k], act_bf16);
    }

    /* T = X A, then the bottleneck and the gate of every rank component,
     * one token at a time. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < n_rows; ++i) {
        const double* x = xd + (size_t)i * K;
        double* t = td + (size_t)i * r;
        double* u = ud + (size_t)i * h;
        for (int j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += x[k] * act_to_double(A[(size_t)k * r + j], act_bf16);
            t[j] = acc;
        }
        for (int q = 0; q < h; ++q) {
            double acc = 0.0;
            for (int j = 0; j < r; ++j)
                acc += t[j] * act_to_double(G1[(size_t)j * h + q], act_bf16);
            acc += act_to_double(c1[q], act_bf16);
            u[q] = acc > 0.0 ? acc : 0.0;
        }
        for (int j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int q = 0; q < h; ++q)
                acc += u[q] * act_to_double(G2[(size_t)q * r + j], act_bf16);
            acc += act_to_double(c2[j], act_bf16);
            gd[(size_t)i * r + j] = sigmoid(acc);
        }
    }

    /* One output feature at a time: dequantize row n of W, then every token. */
    int bad = 0;
#pragma omp parallel
    {
        double* wd = (double*)malloc(sizeof(double) * (size_t)K);
        double* bc = (double*)malloc(sizeof(double) * (size_t)r);
        if (!wd || !bc) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 8)
        for (int n = 0; n < N; ++n) {
            if (!wd || !bc)
                continue;
            for (int k = 0; k < K; ++k) {
                int gi = k / G;
                double s = w4o_half_to_double(scale[(size_t)n * ngroups + gi]);
                double z = w4o_half_to_double(zero[(size_t)n * ngroups + gi]);
                wd[k] = ((double)code_at(qc, K, n, k) - z) * s;
            }
            for (int j = 0; j < r; ++j)
                bc[j] = act_to_double(B[(size_t)j * N + n], act_bf16);
            for (int i = 0; i < n_rows; ++i) {
                const double* x = xd + (size_t)i * K;
                double y0 = 0.0;
                for (int k = 0; k < K; ++k)
                    y0 += x[k] * wd[k];
                double c = 0.0;
                for (int j = 0; j < r; ++j)
                    c += gd[(size_t)i * r + j] * td[(size_t)i * r + j] * bc[j];
                size_t o = (size_t)i * N + n;
                Y[o] = y0 + c;
                if (Y0) Y0[o] = y0;
                if (C) C[o] = c;
            }
        }
        free(wd);
        free(bc);
    }
    if (T)
        memcpy(T, td, sizeof(double) * (size_t)n_rows * r);
    if (gamma)
        memcpy(gamma, gd, sizeof(double) * (size_t)n_rows * r);
    free(xd);
    free(td);
    free(gd);
    free(ud);
    return bad ? -1 : 0;
}

/* Single-factor correction over salient input channels (SERQ summary,
 * section 2, "saliency-aware error reconstruction"): the output is the
 * quantized product plus the salient activation channels times one
 * low-rank factor R, Y ~ X W + X_s R.  Read in the W4A16 setting of this
 * library: X and R stay in the activation type (no activation or R
 * quantization), and the salient channels are a list of input-channel
 * indices S (an offline permutation makes them a contiguous block; any list,
 * duplicates included, is accepted):
 *
 *   C[m,n] = sum_j X[m, S[j]] * R[j,n]        j < s
 *   Y[m,n] = Y0[m,n] + C[m,n]
 *
 *   S int32 [s] with 0 <= S[j] < K;  R act bits [s][N]
 * Other arguments and outputs as w4o_forward (Y0 and C may be NULL).
 * Returns 0, or -1 on bad arguments or allocation failure. */
int w4o_forward_serq(int M, int N, int K, int s, int G, int act_bf16,
                     const uint16_t* X, const uint8_t* qc,
                     const uint16_t* scale, const uint16_t* zero,
                     const int32_t* S, const uint16_t* R,
                     const int* rows, int n_rows,
                     double* Y, double* Y0, double* C)
{
    if (M < 0 || N <= 0 || K <= 0 || s < 0 || G <= 0 || K % G || K % 2 || !Y)
        return -1;
    if (s > 0 && (!S || !R))
        return -1;
    for (int j = 0; j < s; ++j)
        if (S[j] < 0 || S[j] >= K)
            return -1;
    if (!rows)
        n_rows = M;
    if (n_rows <= 0)
        return 0;
    int ngroups = K / G;
    double* xd = (double*)malloc(sizeof(double) * (size_t)n_rows * K);
    if (!xd)
        return -1;
    for (int i = 0; i < n_rows; ++i) {
        int m = rows ? rows[i] : i;
        if (m < 0 || m >= M) {
            free(xd);
            return -1;
        }
        for (int k = 0; k < K; ++k)
            xd[(size_t)i * K + k] = act_to_double(X[(size_t)m * K + k], act_bf16);
    }
    int bad = 0;
#pragma omp parallel
    {
        double* wd = (double*)malloc(sizeof(double) * (size_t)K);
        if (!wd) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 8)
        for (int n = 0; n < N; ++n) {
            if (!wd)
                continue;
            for (int k = 0; k < K; ++k) {
                int gi = k / G;
                double sc = w4o_half_to_double(scale[(size_t)n * ngroups + gi]);
                double z = w4o_half_to_double(zero[(size_t)n * ngroups + gi]);
                wd[k] = ((double)code_at(qc, K, n, k) - z) * sc;
            }
            for (int i = 0; i < n_rows; ++i) {
                const double* x = xd + (size_t)i * K;
                double y0 = 0.0;
                for (int k = 0; k < K; ++k)
                    y0 += x[k] * wd[k];
                double c = 0.0;
                for (int j = 0; j < s; ++j)
                    c += x[S[j]] * act_to_double(R[(size_t)j * N + n], act_bf16);
                size_t o = (size_t)i * N + n;
                Y[o] = y0 + c;
                if (Y0) Y0[o] = y0;
                if (C) C[o] = c;
            }
        }
        free(wd);
    }
    free(xd);
    return bad ? -1 : 0;
}

/* Codebook weights with a sparse outlier residual (XFP summary, section 2,
 * "sparse outlier separation" and "adaptive learned codebooks", per-channel
 * mode): every weight is an index into its output channel's codebook of
 * 2^4 fp16 entries, plus an fp16 residual at the few outlier positions:
 *
 *   Wh[n,k] = cb[n][idx[n,k]] + sum of val[e] over the entries e of row n
 *             whose column is k (compressed sparse rows: row_ptr, col_idx)
 *   Y[m,n]  = sum_k X[m,k] * Wh[n,k]
 *
 *   idx   canonical 4-bit array [N][K/2] (as the W4 codes)
 *   cb    fp16 bits [N][16]
 *   row_ptr int32 [N+1], col_idx int32 [nnz] in [0, K), val fp16 bits [nnz]
 * rows / n_rows as w4o_forward.  Returns 0, or -1 on bad arguments. */
int w4o_forward_xfp(int M, int N, int K, int act_bf16,
                    const uint16_t* X, const uint8_t* qc, const uint16_t* cb,
                    const int32_t* row_ptr, const int32_t* col_idx, const uint16_t* val,
                    const int* rows, int n_rows, double* Y)
{
    if (M < 0 || N <= 0 || K <= 0 || K % 2 || !Y || !X || !qc || !cb || !row_ptr)
        return -1;
    if (row_ptr[0] != 0)
        return -1;
    for (int n = 0; n < N; ++n) {
        if (row_ptr[n + 1] < row_ptr[n])
            return -1;
        for (int e = row_ptr[n]; e < row_ptr[n + 1]; ++e)
            if (col_idx[e] < 0 || col_idx[e] >= K)
                return -1;
    }
    if (!rows)
        n_rows = M;
    if (n_rows <= 0)
        return 0;
    double* xd = (double*)malloc(sizeof(double) * (size_t)n_rows * K);
    if (!xd)
        return -1;
    for (int i = 0; i < n_rows; ++i) {
        int m = rows ? rows[i] : i;
        if (m < 0 || m >= M) {
            free(xd);
            return -1;
        }
        for (int k = 0; k < K; ++k)
            xd[(size_t)i * K + k] = act_to_double(X[(size_t)m * K + k], act_bf16);
    }
    int bad = 0;
#pragma omp parallel
    {
        double* wd = (double*)malloc(sizeof(double) * (size_t)K);
        if (!wd) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 8)
        for (int n = 0; n < N; ++n) {
            if (!wd)
                continue;
            for (int k = 0; k < K; ++k)
                wd[k] = w4o_half_to_double(cb[(size_t)n * 16 + code_at(qc, K, n, k)]);
            for (int e = row_ptr[n]; e < row_ptr[n + 1]; ++e)
                wd[col_idx[e]] += w4o_half_to_double(val[e]);
            for (int i = 0; i < n_rows; ++i) {
                const double* x = xd + (size_t)i * K;
                double y = 0.0;
                for (int k = 0; k < K; ++k)
                    y += x[k] * wd[k];
                Y[(size_t)i * N + n] = y;
            }
        }
        free(wd);
    }
    free(xd);
    return bad ? -1 : 0;
}

/* Codebook weights from a shared library (XFP summary, section 2, "adaptive
 * learned codebooks", shared-library mode): the layer keeps L codebooks of
 * 2^4 fp16 entries, and each group of 128 consecutive weights of an output
 * channel (along K) names the library entry it uses; the sparse fp16
 * residual is as in w4o_forward_xfp:
 *
 *   Wh[n,k] = lib[libid[n][k / 128]][idx[n,k]] + sum of val[e] over the
 *             entries e of row n whose column is k
 *   Y[m,n]  = sum_k X[m,k] * Wh[n,k]
 *
 *   idx    canonical 4-bit array [N][K/2]
 *   lib    fp16 bits [L][16], 1 <= L <= 256
 *   libid  uint8 [N][K/128], each < L
 *   row_ptr, col_idx, val, rows, n_rows as w4o_forward_xfp.
 * K a multiple of 128.  Returns 0, or -1 on bad arguments. */
int w4o_forward_xfp_lib(int M, int N, int K, int act_bf16,
                        const uint16_t* X, const uint8_t* qc, const uint16_t* lib, int L,
                        const uint8_t* libid, const int32_t* row_ptr, const int32_t* col_idx,
                        const uint16_t* val, const int* rows, int n_rows, double* Y)
{
    if (M < 0 || N <= 0 || K <= 0 || K % 128 || !Y || !X || !qc || !lib || !libid || !row_ptr)
        return -1;
    if (L < 1 || L > 256 || row_ptr[0] != 0)
        return -1;
    const int ng = K / 128;
    for (int n = 0; n < N; ++n) {
        if (row_ptr[n + 1] < row_ptr[n])
            return -1;
        for (int e = row_ptr[n]; e < row_ptr[n + 1]; ++e)
            if (col_idx[e] < 0 || col_idx[e] >= K)
                return -1;
        for (int g = 0; g < ng; ++g)
            if (libid[(size_t)n * ng + g] >= L)
                return -1;
    }
    if (!rows)
        n_rows = M;
    if (n_rows <= 0)
        return 0;
    double* xd = (double*)malloc(sizeof(double) * (size_t)n_rows * K);
    if (!xd)
        return -1;
    for (int i = 0; i < n_rows; ++i) {
        int m = rows ? rows[i] : i;
        if (m < 0 || m >= M) {
            free(xd);
            return -1;
        }
        for (int k = 0; k < K; ++k)
            xd[(size_t)i * K + k] = act_to_double(X[(size_t)m * K + k], act_bf16);
    }
    int bad = 0;
#pragma omp parallel
    {
        double* wd = (double*)malloc(sizeof(double) * (size_t)K);
        if (!wd) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 8)
        for (int n = 0; n < N; ++n) {
            if (!wd)
                continue;
            for (int k = 0; k < K; ++k) {
                const int entry = libid[(size_t)n * ng + k / 128];
                wd[k] = w4o_half_to_double(lib[(size_t)entry * 16 + code_at(qc, K, n, k)]);
            }
            for (int e = row_ptr[n]; e < row_ptr[n + 1]; ++e)
                wd[col_idx[e]] += w4o_half_to_double(val[e]);
            for (int i = 0; i < n_rows; ++i) {
                const double* x = xd + (size_t)i * K;
                double y = 0.0;
                for (int k = 0; k < K; ++k)
                    y += x[k] * wd[k];
                Y[(size_t)i * N + n] = y;
            }
        }
        free(wd);
    }
    free(xd);
    return bad ? -1 : 0;
}

/* Threads an OpenMP region of this library will use. */
int w4o_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
