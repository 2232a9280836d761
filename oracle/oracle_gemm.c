/*
 * CPU oracle for the persistent tile-scheduled GEMM -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load
 * this library.  It shares no code, header or constant with the HIP path.
 *
 * What it computes (pages: "[Feature] Introduce tile scheduler #2441", diff of
 * examples/gemm_sm100/gemm_tcgen5mma_ws_persistent.py, where C = A @ B with
 * A[M,K], B[K,N] row-major and the result compared against torch `a @ b` in
 * main(); and the tilelang lowering blog, section 1.1, whose gemm reads
 * A[M,K], B[K,N] and writes C[M,N]):
 *
 *   C64[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]    (ascending k, binary64)
 *
 * followed by a single round-to-nearest-ties-to-even of C64 into the output
 * format (IEEE 754-2008 binary16, or bfloat16 = 8-bit exponent, 7-bit fraction).
 *
 * The inputs are the already-rounded fp16/bf16 arrays widened to binary64 (an
 * exact conversion done by the caller); every product of two such values is
 * exact in binary64, only the running sum rounds.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Plain triple loop, i-k-j order so each C64[i][j] still sums in ascending k.
 * OpenMP splits rows; each row is summed by one thread in the same order. */
void oracle_gemm_f64(int64_t M, int64_t N, int64_t K,
                     const double* A, const double* B, double* C)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double* c = C + i * N;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = A[i * K + k];
            const double* b = B + k * N;
            for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
        }
    }
}

/* The same definition evaluated at `count` chosen (row, col) positions only:
 * out[t] = sum_k A[rows[t]][k] * B[k][cols[t]], ascending k.  Used where the
 * full product is too large for the CPU (sampled checks). */
void oracle_gemm_entries_f64(int64_t N, int64_t K,
                             const double* A, const double* B,
                             int64_t count, const int64_t* rows, const int64_t* cols,
                             double* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const double* a = A + rows[t] * K;
        const int64_t j = cols[t];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += a[k] * B[k * N + j];
        out[t] = s;
    }
}

/* Round one binary64 value to the nearest value of a binary format with
 * p significand bits (hidden bit included), exponent field width ebits,
 * normal exponents emin..emax (bias = emax), ties to even.  This follows the
 * IEEE 754 definition directly: write |x| = mant * 2^e2 with an integer
 * 53-bit mant, pick the format's quantum 2^q at that magnitude (the subnormal
 * quantum below emin), round mant * 2^(e2-q) to an integer n, then encode
 * n * 2^q.  Results beyond the largest finite value become infinity. */
static uint16_t round_binary(double x, int p, int ebits, int emin, int emax)
{
    const int fbits = p - 1;
    const uint16_t sign_bit = (uint16_t)(1u << (ebits + fbits));
    const uint16_t exp_ones = (uint16_t)(((1u << ebits) - 1u) << fbits);
    uint16_t sign = signbit(x) ? sign_bit : 0;

    if (isnan(x)) return (uint16_t)(sign | exp_ones | (1u << (fbits - 1)));
    if (isinf(x)) return (uint16_t)(sign | exp_ones);
    const double ax = fabs(x);
    if (ax == 0.0) return sign;

    int e2;
    const double fr = frexp(ax, &e2);              /* ax = fr * 2^e2, fr in [0.5,1) */
    const uint64_t mant = (uint64_t)ldexp(fr, 53); /* exact integer in [2^52, 2^53) */
    e2 -= 53;                                      /* ax = mant * 2^e2             */
    const int ex = e2 + 52;                        /* floor(log2(ax))               */
    int q = (ex > emin ? ex : emin) - fbits;       /* quantum exponent              */
    const int shift = q - e2;                      /* > 0 for the formats used here */

    uint64_t n;
    if (shift >= 64) {
        n = 0;                                     /* below half the smallest step */
    } else {
        const uint64_t whole = mant >> shift;
        const uint64_t rem = mant & ((1ull << shift) - 1ull);
        const uint64_t half = 1ull << (shift - 1);
        n = whole;
        if (rem > half || (rem == half && (whole & 1ull))) n += 1;
    }
    if (n == (1ull << p)) { n >>= 1; q += 1; }     /* carried into the next binade */
    if (n == 0) return sign;
    if (n >= (1ull << fbits)) {                    /* normal */
        const int E = q + fbits;
        if (E > emax) return (uint16_t)(sign | exp_ones);
        const uint64_t biased = (uint64_t)(E + emax);
        return (uint16_t)(sign | (biased << fbits) | (n - (1ull << fbits)));
    }
    return (uint16_t)(sign | n);                   /* subnormal, biased exponent 0 */
}

/* fmt: 1 = IEEE binary16 (fp16), 2 = bfloat16. */
uint16_t oracle_round_one(double x, int fmt)
{
    if (fmt == 1) return round_binary(x, 11, 5, -14, 15);
    return round_binary(x, 8, 8, -126, 127);
}

void oracle_round_array(const double* x, uint16_t* out, int64_t n, int fmt)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_one(x[i], fmt);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of later oracle calls (n >= 1); timing only, the sums do not depend on it. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
