/*
 * CPU oracle for the block-scaled (MX) FP8 GEMM -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load
 * this code.  It shares no code, header or constant with the HIP path.
 *
 * What it computes.  The tile-scheduler page ("[Feature] Introduce tile
 * scheduler #2441", PR overview and the changed-file list) names an MXFP8
 * block-scaled persistent GEMM (examples/blockscaled_gemm_sm100/
 * gemm_mxfp8_blockscaled_1d1d.py, with scale factors SFA and SFB) but does not
 * print its formats.  They are taken from the OCP Microscaling (MX) Formats
 * specification v1.0:
 *   * an element is FP8 E4M3: sign bit, 4 exponent bits (bias 7), 3 mantissa
 *     bits; exponent field 0 encodes subnormals 2^-6 * m/8; S.1111.111 is NaN;
 *     there are no infinities (largest finite value 448);
 *   * a scale is E8M0: 8 exponent bits, value 2^(e - 127); 0xFF is NaN;
 *   * a block is 32 consecutive elements along K sharing one scale, and the
 *     dot product of two MX vectors is sum over blocks of
 *     scale_a * scale_b * sum_{k in block} a_k * b_k.
 * Layout (a reading; the page's "1d1d" = one-dimensional blocks along K for
 * both operands): A[M][K] and B[N][K] element codes, both K-contiguous;
 * SFA[M][K/32] and SFB[N][K/32] scale codes.
 *
 *   C64[i][j] = sum_{k=0}^{K-1} x(A[i][k]) * s(SFA[i][k/32]) * x(B[j][k]) * s(SFB[j][k/32])
 *
 * in binary64, ascending k.  Every product is exact in binary64 (at most 8
 * significant bits, magnitudes in [2^-272, 2^272]); only the running sum
 * rounds, so grouping a term as (x(a) s(sa)) (x(b) s(sb)) gives the same
 * value as any other order of its four factors.  The
 * caller rounds C64 once to the output format (oracle_round_array).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* OCP FP8 E4M3 element -> binary64 (NaN for S.1111.111). */
double oracle_e4m3_decode(uint8_t c)
{
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);          /* 2^-6 * m/8 */
    else
        v = ldexp(8.0 + (double)m, e - 10); /* 2^(e-7) * (1 + m/8) */
    return s ? -v : v;
}

/* OCP E8M0 scale -> binary64 (NaN for 0xFF). */
double oracle_e8m0_decode(uint8_t c)
{
    if (c == 255) return NAN;
    return ldexp(1.0, (int)c - 127);
}

/* One operand element with its block scale applied: x(code) * s(scale code).
 * Exact in binary64: at most 4 significant bits, magnitude in [2^-136, 2^136]. */
static double mx_value(uint8_t code, uint8_t scale)
{
    return oracle_e4m3_decode(code) * oracle_e8m0_decode(scale);
}

/* C[M][N] = the MX product above; K % 32 == 0.
 * Each operand is decoded once (row r, column k -> x * s, exact), B into
 * K-major order; then the plain i-k-j triple loop of the fp16/bf16 oracle, so
 * every C64[i][j] is still summed in ascending k.  Since each decoded value
 * and each product of two of them is exact, the sum is the same binary64
 * sequence as the per-term formula above, bit for bit.  Returns 0, or -1
 * when the decoded copies cannot be allocated. */
int oracle_mx_gemm_f64(int64_t M, int64_t N, int64_t K, const uint8_t* A, const uint8_t* SFA,
                       const uint8_t* B, const uint8_t* SFB, double* C)
{
    const int64_t KB = K / 32;
    double* xa = (double*)malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(double));
    double* xbt = (double*)malloc((size_t)(K * N > 0 ? K * N : 1) * sizeof(double));
    if (!xa || !xbt) { free(xa); free(xbt); return -1; }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k) xa[i * K + k] = mx_value(A[i * K + k], SFA[i * KB + k / 32]);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j) xbt[k * N + j] = mx_value(B[j * K + k], SFB[j * KB + k / 32]);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double* c = C + i * N;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = xa[i * K + k];
            const double* b = xbt + k * N;
            for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
        }
    }
    free(xa);
    free(xbt);
    return 0;
}

/* The same at `count` chosen (row, col) positions, term by term. */
void oracle_mx_gemm_entries_f64(int64_t K, const uint8_t* A, const uint8_t* SFA, const uint8_t* B,
                                const uint8_t* SFB, int64_t count, const int64_t* rows,
                                const int64_t* cols, double* out)
{
    const int64_t KB = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        const uint8_t* a = A + rows[t] * K;
        const uint8_t* sa = SFA + rows[t] * KB;
        const uint8_t* b = B + cols[t] * K;
        const uint8_t* sb = SFB + cols[t] * KB;
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += mx_value(a[k], sa[k / 32]) * mx_value(b[k], sb[k / 32]);
        out[t] = s;
    }
}
