/*
 * Plain fp64 reference for the routed LoRA delta.  TEST INFRASTRUCTURE ONLY:
 * tests, the smoke check and the benchmark's CPU-baseline leg call it; the
 * product library never links or loads it.
 *
 * The computation is the formula of TensorFold PR #47 (third commit message):
 * the delta scale * B @ (A @ x) is added to a projection's fp32 partial sum.
 * Orientation is PEFT's (xLLM PR #2014, "New subsystems", LoRAAdapterLoader):
 * lora_A is [rank, in_features], lora_B is [out_features, rank].  Under tensor
 * parallelism A is cut by input columns (TensorFold PR #47, first commit
 * message), so a GPU's share reads columns [a_col0, a_col0 + h_in) of A.
 *
 * Every input value is decoded exactly to binary64, every product of two
 * decoded values is exact in binary64, and sums run in the plain index order
 * of the definition: u_k = sum_i A[k][i] x[i] (i ascending), then
 * d_o = scale * sum_k B[o][k] u_k (k ascending).
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared lora_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the upper half of an IEEE-754 binary32 word. */
double oracle_bf16_value(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_fp16_value(uint16_t bits)
{
    int sign = bits >> 15;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(frac | 0x400), expo - 25); /* (1.frac) * 2^(expo-15) */
    return sign ? -v : v;
}

static double decode(uint16_t bits, int kind)
{
    return kind == 2 ? oracle_fp16_value(bits) : oracle_bf16_value(bits);
}

/*
 * Delta of one adapter on one output slice, for a list of rows.
 *
 *   rows[p]   row of x this entry reads (p = 0 .. n_rows-1)
 *   x         [*, ldx] bits, x_kind 1 = bf16, 2 = fp16; row t holds the h_in
 *             input features this GPU sees
 *   A         [rank, lda] bf16 bits; this GPU's share is columns
 *             [a_col0, a_col0 + h_in)
 *   B         [h_out, ldb] bf16 bits, columns [0, rank)
 *   out       [n_rows, ldo] binary64; entry p receives the delta at columns
 *             [out_col0, out_col0 + h_out)
 *
 * Returns 0, or -1 when scratch memory cannot be had.
 */
int oracle_slice_delta(int64_t n_rows, const int64_t *rows,
                       int64_t h_in, const uint16_t *x, int64_t ldx, int32_t x_kind,
                       int64_t rank, const uint16_t *A, int64_t lda, int64_t a_col0,
                       int64_t h_out, const uint16_t *B, int64_t ldb,
                       double scale, double *out, int64_t ldo, int64_t out_col0)
{
    double *u = (double *)malloc((size_t)(rank > 0 ? rank : 1) * sizeof(double));
    double *xr = (double *)malloc((size_t)(h_in > 0 ? h_in : 1) * sizeof(double));
    if (!u || !xr) {
        free(u);
        free(xr);
        return -1;
    }
    for (int64_t p = 0; p < n_rows; ++p) {
        const uint16_t *xt = x + rows[p] * ldx;
        for (int64_t i = 0; i < h_in; ++i)
            xr[i] = decode(xt[i], x_kind);
        /* shrink: u = A x over this GPU's columns */
        for (int64_t k = 0; k < rank; ++k) {
            const uint16_t *ak = A + k * lda + a_col0;
            double s = 0.0;
            for (int64_t i = 0; i < h_in; ++i)
                s += oracle_bf16_value(ak[i]) * xr[i];
            u[k] = s;
        }
        /* expand: d = scale * B u */
        double *op = out + p * ldo + out_col0;
        for (int64_t o = 0; o < h_out; ++o) {
            const uint16_t *bo = B + o * ldb;
            double s = 0.0;
            for (int64_t k = 0; k < rank; ++k)
                s += oracle_bf16_value(bo[k]) * u[k];
            op[o] = scale * s;
        }
    }
    free(u);
    free(xr);
    return 0;
}

/*
 * The base projection of a lane for a list of rows: out[p][o] =
 * sum_i W[o][i] x[rows[p]][i], i ascending, in binary64 from exact decodes.
 * This is the fp32 partial sum that the delta above is added to (TensorFold
 * PR #47, third commit message and PR body "What this changes": the delta
 * lands in the projection's partial sum before the cross-rank reduction).  W
 * is the linear layer's weight in its usual [out_features, in_features]
 * orientation, bf16; under tensor parallelism a row-parallel layer's GPU
 * holds the columns of its input share, which is what W holds here.
 *
 *   x    [*, ldx] bits, x_kind 1 = bf16, 2 = fp16; row t holds h_in features
 *   W    [h_out, ldw] bf16 bits, columns [0, h_in)
 *   out  [n_rows, ldo] binary64, columns [0, h_out)
 *
 * Returns 0, or -1 when scratch memory cannot be had.
 */
int oracle_linear_rows(int64_t n_rows, const int64_t *rows, int64_t h_in, const uint16_t *x,
                       int64_t ldx, int32_t x_kind, int64_t h_out, const uint16_t *W,
                       int64_t ldw, double *out, int64_t ldo)
{
    double *xr = (double *)malloc((size_t)(h_in > 0 ? h_in : 1) * sizeof(double));
    if (!xr) return -1;
    for (int64_t p = 0; p < n_rows; ++p) {
        const uint16_t *xt = x + rows[p] * ldx;
        for (int64_t i = 0; i < h_in; ++i)
            xr[i] = decode(xt[i], x_kind);
        double *op = out + p * ldo;
        for (int64_t o = 0; o < h_out; ++o) {
            const uint16_t *wo = W + o * ldw;
            double s = 0.0;
            for (int64_t i = 0; i < h_in; ++i)
                s += oracle_bf16_value(wo[i]) * xr[i];
            op[o] = s;
        }
    }
    free(xr);
    return 0;
}
