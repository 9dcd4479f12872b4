/*
 * CPU oracle for the dense fp16 NT GEMM  C = A * B^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or helper with the
 * HIP library.
 *
 * What it computes (Tilus "Hopper matmul" tutorial pages):
 *   - "2. Multi-Stage Software Pipelining", The Full Kernel: A is viewed as
 *     fp16 [m_size, k_size] and B as fp16 [n_size, k_size], both row-major;
 *     the MMA consumes B transposed; the accumulator is fp32 initialised to
 *     0.0; at the end it is cast to fp16 and stored to C fp16 [m_size, n_size].
 *   - "6. Register Reallocation, Multicast, and a Persistent Kernel", opening
 *     paragraphs: accumulation stays fp32 in every version (like-for-like
 *     with the vendor library).
 *
 * The oracle evaluates the exact definition instead of any particular fp32
 * summation order:
 *
 *     C[i][j] = fp16_rne( sum_{k=0}^{K-1} double(A[i][k]) * double(B[j][k]) )
 *
 * with one fp64 accumulator per output element, k ascending, starting at
 * +0.0.  A product of two fp16 values has at most 22 significant bits, so it
 * is exact in fp64; the fp64 sum then differs from the exact real sum by far
 * less than half an fp16 ulp for every shape we test, so one final
 * round-to-nearest-even gives the correctly rounded result of the exact sum
 * (up to exact-tie coincidences).  Any fp32-accumulating kernel is an
 * approximation of this value.
 *
 * Readings taken where the pages are silent:
 *   - the cast to fp16 rounds to nearest, ties to even (IEEE default);
 *   - results with magnitude >= 65520 become +-inf; fp16 subnormals are kept
 *     (gradual underflow down to 2^-24) both in inputs and in the output;
 *   - K = 0 gives the empty sum +0.0; M = 0 or N = 0 computes nothing.
 *
 * fp16 values travel as raw uint16 bit patterns.  The two conversions below
 * are written from the IEEE binary16 definition (1 sign bit, 5 exponent bits
 * with bias 15, 10 fraction bits).
 *
 * No -ffast-math: the build uses -O2 -ffp-contract=off so each "+=" is one
 * correctly rounded fp64 addition.
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>

/* binary16 bit pattern -> exact double. */
static double f16_bits_to_double(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double mag;
    if (expo == 0) {
        /* zero or subnormal: frac * 2^-24 */
        mag = ldexp((double)frac, -24);
    } else if (expo == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        /* normal: (1024 + frac) * 2^(expo - 15 - 10) */
        mag = ldexp((double)(1024 + frac), expo - 25);
    }
    return sign ? -mag : mag;
}

/* Round a non-negative double holding a value in [0, 2^53) to the nearest
 * integer, ties to the even integer.  Written out so that it does not depend
 * on the floating-point environment's rounding mode. */
static double round_half_even(double q)
{
    const double fl = floor(q);
    const double rem = q - fl; /* exact: q and fl share the exponent range */
    if (rem > 0.5) return fl + 1.0;
    if (rem < 0.5) return fl;
    /* exact tie: pick the even neighbour */
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* double -> binary16 bit pattern, round to nearest, ties to even. */
static uint16_t double_to_f16_bits_rne(double x)
{
    if (isnan(x)) return 0x7e00;
    const uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
    const double ax = fabs(x);
    /* 65504 is the largest finite half; the midpoint to the next binade
     * (65536) is 65520 and it ties to the even neighbour, 65536 = overflow. */
    if (ax >= 65520.0) return (uint16_t)(sign | 0x7c00);
    if (ax == 0.0) return sign;

    int e2;
    frexp(ax, &e2);        /* ax = m * 2^e2, m in [0.5, 1) */
    int e = e2 - 1;        /* ax in [2^e, 2^(e+1)) */
    if (e < -14) {
        /* subnormal range: count units of 2^-24 */
        const double q = round_half_even(ldexp(ax, 24));
        /* q == 1024 rounds up into the smallest normal, whose bit pattern is
         * exactly 0x0400, so no special case is needed. */
        return (uint16_t)(sign | (uint16_t)q);
    }
    /* normal range: 11-bit significand in [1024, 2048) */
    double q = round_half_even(ldexp(ax, 10 - e));
    if (q == 2048.0) {
        q = 1024.0;
        e += 1;
    }
    if (e > 15) return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(q - 1024.0));
}

/* Exposed so that the tests can pin the conversions on their own. */
double oracle_f16_to_f64(uint16_t h) { return f16_bits_to_double(h); }
uint16_t oracle_f64_to_f16(double x) { return double_to_f16_bits_rne(x); }

/* The exact sum for one output element, before the fp16 rounding. */
static double dot_row(const double *a_row, const double *b_row, int64_t K)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += a_row[k] * b_row[k];
    return s;
}

/* Decode an fp16 matrix to doubles once (a pure representation change). */
static void decode(const uint16_t *src, double *dst, int64_t count)
{
    for (int64_t t = 0; t < count; ++t) dst[t] = f16_bits_to_double(src[t]);
}

/*
 * Full oracle: C[M,N] (fp16 bits) from A[M,K], B[N,K] (fp16 bits).
 * `c_sum`, when not NULL, receives the unrounded fp64 sums [M,N].
 * `a_dbl` / `b_dbl` are caller-provided scratch of M*K and N*K doubles.
 * Output elements are independent, so rows are spread over threads; the sum
 * for one element is always the same sequential loop.
 */
void oracle_gemm_f16_nt(int64_t M, int64_t N, int64_t K,
                        const uint16_t *A, const uint16_t *B, uint16_t *C,
                        double *c_sum, double *a_dbl, double *b_dbl,
                        int nthreads)
{
    if (M <= 0 || N <= 0) return;
    decode(A, a_dbl, M * K);
    decode(B, b_dbl, N * K);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            const double s = dot_row(a_dbl + i * K, b_dbl + j * K, K);
            C[i * N + j] = double_to_f16_bits_rne(s);
            if (c_sum) c_sum[i * N + j] = s;
        }
    }
}

/*
 * Sampled oracle for shapes too large to evaluate whole: the same definition
 * evaluated only at the `count` positions (rows[t], cols[t]).
 */
void oracle_gemm_f16_nt_sampled(int64_t M, int64_t N, int64_t K,
                                const uint16_t *A, const uint16_t *B,
                                const int64_t *rows, const int64_t *cols,
                                int64_t count, uint16_t *out, double *out_sum,
                                int nthreads)
{
    (void)M;
    (void)N;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (int64_t t = 0; t < count; ++t) {
        const uint16_t *a = A + rows[t] * K;
        const uint16_t *b = B + cols[t] * K;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += f16_bits_to_double(a[k]) * f16_bits_to_double(b[k]);
        out[t] = double_to_f16_bits_rne(s);
        if (out_sum) out_sum[t] = s;
    }
}

/* Array forms of the two conversions, for the pins that sweep all patterns. */
void oracle_f16_to_f64_array(const uint16_t *src, double *dst, int64_t count)
{
    for (int64_t t = 0; t < count; ++t) dst[t] = f16_bits_to_double(src[t]);
}

void oracle_f64_to_f16_array(const double *src, uint16_t *dst, int64_t count)
{
    for (int64_t t = 0; t < count; ++t) dst[t] = double_to_f16_bits_rne(src[t]);
}
