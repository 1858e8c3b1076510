// Load-time fold of an adapter's A onto a transformed input (gfx950).
//
// A projection may read its input in another representation x' = M x (the
// packed shared expert's down projection reads the rotated, scaled fp16
// hidden state its expert kernels leave behind); an adapter of that
// projection is then stored with A' = A M^-1, so that A' x' = A x (TensorFold
// PR #47, first commit message: the shared expert's A is rewritten once at
// load to read the rotated hidden state).  The caller passes F = M^-1.
//
// dst[k][c] = bf16(sum_i A[k][a_col0 + i] * F[i][c]) for k < rank, c < h_in:
// an fp32 fma chain over i ascending, rounded to nearest even.  Each thread
// owns one column c for kFoldRanks ranks, so a row of F is read once per
// kFoldRanks ranks; A's rows are staged in LDS in chunks of kFoldChunk.
#include "kernels_common.h"

namespace lora {
namespace {

constexpr int kFoldCols = 256;
constexpr int kFoldRanks = 8;
constexpr int kFoldChunk = 512;

__device__ inline float bf16_value(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Nearest bf16 of an fp32 value, ties to even (NaN stays a quiet NaN).
__device__ inline uint16_t bf16_nearest(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__global__ __launch_bounds__(kFoldCols) void k_fold_a(uint16_t *__restrict__ dst,
                                                      const uint16_t *__restrict__ src,
                                                      int64_t lda, int64_t a_col0, int rank,
                                                      int h_in, const float *__restrict__ F,
                                                      int64_t ldf)
{
    __shared__ float a_s[kFoldRanks][kFoldChunk];
    const int c = blockIdx.x * kFoldCols + threadIdx.x;
    const int k0 = blockIdx.y * kFoldRanks;
    float acc[kFoldRanks];
#pragma unroll
    for (int kk = 0; kk < kFoldRanks; ++kk) acc[kk] = 0.f;
    for (int i0 = 0; i0 < h_in; i0 += kFoldChunk) {
        const int n = min(kFoldChunk, h_in - i0);
        __syncthreads();
        for (int t = threadIdx.x; t < kFoldRanks * kFoldChunk; t += kFoldCols) {
            const int kk = t / kFoldChunk, ii = t - kk * kFoldChunk;
            a_s[kk][ii] = k0 + kk < rank && ii < n
                              ? bf16_value(src[(int64_t)(k0 + kk) * lda + a_col0 + i0 + ii])
                              : 0.f;
        }
        __syncthreads();
        if (c < h_in) {
            for (int ii = 0; ii < n; ++ii) {
                const float f = F[(int64_t)(i0 + ii) * ldf + c];
#pragma unroll
                for (int kk = 0; kk < kFoldRanks; ++kk) acc[kk] = fmaf(a_s[kk][ii], f, acc[kk]);
            }
        }
    }
    if (c < h_in) {
#pragma unroll
        for (int kk = 0; kk < kFoldRanks; ++kk)
            if (k0 + kk < rank) dst[(int64_t)(k0 + kk) * h_in + c] = bf16_nearest(acc[kk]);
    }
}

}  // namespace

hipError_t launch_fold_a(uint16_t *dst, const uint16_t *src, int64_t lda, int64_t a_col0,
                         int rank, int h_in, const float *F, int64_t ldf, hipStream_t s)
{
    if (rank < 1 || h_in < 1 || ldf < h_in) return hipErrorInvalidValue;
    const dim3 grid((h_in + kFoldCols - 1) / kFoldCols, (rank + kFoldRanks - 1) / kFoldRanks);
    hipLaunchKernelGGL(k_fold_a, grid, dim3(kFoldCols), 0, s, dst, src, lda, a_col0, rank, h_in,
                       F, ldf);
    return hipGetLastError();
}

}  // namespace lora
