// Decode path: gathered GEMV shrink and expand on the vector ALUs (gfx950).
//
// Decode rows of one adapter slot are grouped into segments of up to
// kDecodeSegRows rows.  The shrink reads each A tile once per segment and
// reuses it for all rows of the segment; the expand reads each B^T tile once
// per segment.  Both keep a per-row summation order fixed by the lane's
// widths and the adapter's rank (TensorFold PR #47, third commit message:
// fp32 sums in a fixed order, so a row's bits depend only on its own input and
// its own adapter).
//
// Shrink order for u[k] = sum_i A[k][i] x[i] over h_in:
//   h_in is cut into sub-chunks of kSubChunk = 512 elements; sub-chunk q
//   belongs to part q % kParts.  Within a part, lane l of a wave accumulates
//   elements [512 q + 8 l, 512 q + 8 l + 8) of its sub-chunks, q ascending,
//   four bf16 pair-dot steps per sub-chunk (pairs 0-1, 2-3, 4-5, 6-7), into one
//   fp32 sum.  The 64 lane sums are combined by a fixed reduce-scatter
//   butterfly (lane masks 32, 16, 8, 4, 2, 1), and the part sums as
//   (p0 + p1) + (p2 + p3).  v = fp32(scale * u).
//   An fp16 input is split exactly into two bf16 values x = hi + lo (fp16
//   carries 11 significant bits) and each pair-dot step is done for hi, then lo.
// Expand order: d[o] = fma chain over k = 0 .. rank-1 starting from 0, then
//   y[o] = y[o] + d[o].
#include "lora_internal.h"

namespace lora {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Exact split of two packed fp16 values into packed bf16 hi and lo words.
__device__ __forceinline__ void split_f16x2(uint32_t w, uint32_t &hi, uint32_t &lo)
{
    const float f0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    const float f1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    const uint32_t u0 = __float_as_uint(f0), u1 = __float_as_uint(f1);
    const uint32_t t0 = u0 & 0xffff0000u, t1 = u1 & 0xffff0000u;
    const float l0 = f0 - __uint_as_float(t0);
    const float l1 = f1 - __uint_as_float(t1);
    hi = (u0 >> 16) | t1;
    lo = (__float_as_uint(l0) >> 16) | (__float_as_uint(l1) & 0xffff0000u);
}

__device__ __forceinline__ uint4 ld16(const uint16_t *p)
{
    return *reinterpret_cast<const uint4 *>(p);
}

// In lane L: the sum over the wave's 64 lanes of val[L].  Fixed butterfly.
__device__ __forceinline__ float wave_reduce_scatter64(float (&val)[64], int lane)
{
#pragma unroll
    for (int s = 0; s < 6; ++s) {
        const int m = 32 >> s;
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < m; ++i) {
            const float send = upper ? val[i] : val[m + i];
            const float keep = upper ? val[m + i] : val[i];
            val[i] = keep + __shfl_xor(send, m, 64);
        }
    }
    return val[0];
}

template <bool FP16X>
__global__ __launch_bounds__(256) void k_shrink_gemv(LaneGeom g, PoolDev p, RoutingDev r,
                                                      int kb_per_slice,
                                                      const uint16_t *__restrict__ x,
                                                      int64_t ldx, float *__restrict__ v)
{
    constexpr int C = kDecodeSegRows;
    const int per_seg = g.n_slices * kb_per_slice;
    const int task = blockIdx.x;
    const int si = task / per_seg;
    const int rem = task - si * per_seg;
    const int j = rem / kb_per_slice;
    const int kb = rem - j * kb_per_slice;
    const int4 sd = r.seg[si];
    const int slot = sd.x;
    const int rank = p.rank[slot * kMetaStride + j];
    const int k0 = kb * kKBlock;
    if (k0 >= rank) return;
    const int n_rows = sd.z;
    const int kn = min(kKBlock, rank - k0);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;

    const uint16_t *Ab =
        p.A + (int64_t)(slot - 1) * g.a_slot_stride + ((int64_t)j * g.rank_pad + k0) * g.h_in;
    const uint16_t *xr[C];
#pragma unroll
    for (int c = 0; c < C; ++c) xr[c] = x + (int64_t)r.row_idx[sd.y + min(c, n_rows - 1)] * ldx;

    float acc[C][kKBlock];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int k = 0; k < kKBlock; ++k) acc[c][k] = 0.f;

    const int n_sub = (g.h_in + kSubChunk - 1) / kSubChunk;
    for (int q = wave; q < n_sub; q += kParts) {
        const int e = q * kSubChunk + lane * 8;
        if (e < g.h_in) {
            uint32_t xw[C][FP16X ? 8 : 4];
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if (c < n_rows) {
                    const uint4 t = ld16(xr[c] + e);
                    if constexpr (FP16X) {
                        split_f16x2(t.x, xw[c][0], xw[c][4]);
                        split_f16x2(t.y, xw[c][1], xw[c][5]);
                        split_f16x2(t.z, xw[c][2], xw[c][6]);
                        split_f16x2(t.w, xw[c][3], xw[c][7]);
                    } else {
                        xw[c][0] = t.x;
                        xw[c][1] = t.y;
                        xw[c][2] = t.z;
                        xw[c][3] = t.w;
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < kKBlock; ++k) {
                if (k < kn) {
                    const uint4 a = ld16(Ab + (int64_t)k * g.h_in + e);
                    const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        if (c < n_rows) {
                            float s = acc[c][k];
#pragma unroll
                            for (int m = 0; m < 4; ++m) {
                                s = dot2_bf16(aw[m], xw[c][m], s);
                                if constexpr (FP16X) s = dot2_bf16(aw[m], xw[c][4 + m], s);
                            }
                            acc[c][k] = s;
                        }
                    }
                }
            }
        }
    }

    float val[64];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int k = 0; k < kKBlock; ++k) val[c * kKBlock + k] = acc[c][k];
    const float red = wave_reduce_scatter64(val, lane);

    __shared__ float part[kParts][64];
    part[wave][lane] = red;
    __syncthreads();
    if (wave == 0) {
        const float u = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
        const int c = lane / kKBlock;
        const int k = lane % kKBlock;
        if (c < n_rows && k < kn) {
            const float scale = p.scale[slot * kMetaStride + j];
            v[(int64_t)(sd.y + c) * g.v_stride + j * g.rank_pad + k0 + k] = scale * u;
        }
    }
}

__global__ __launch_bounds__(64) void k_expand_gemv(LaneGeom g, PoolDev p, RoutingDev r,
                                                     int tiles_per_slice,
                                                     const float *__restrict__ v,
                                                     float *__restrict__ y, int64_t ldy)
{
    constexpr int C = kDecodeSegRows;
    const int per_seg = g.n_slices * tiles_per_slice;
    const int task = blockIdx.x;
    const int si = task / per_seg;
    const int rem = task - si * per_seg;
    const int j = rem / tiles_per_slice;
    const int tile = rem - j * tiles_per_slice;
    const int hj = g.h_out[j];
    if (tile * kExpandTile >= hj) return;
    const int4 sd = r.seg[si];
    const int slot = sd.x;
    const int n_rows = sd.z;
    const int rank = p.rank[slot * kMetaStride + j];

    __shared__ float4 vs[LORA_MAX_RANK][2];   // vs[k] = v of rows 0..7 at rank k
    float *vsf = reinterpret_cast<float *>(vs);
    for (int i = threadIdx.x; i < rank * C; i += 64) {
        const int k = i / C, c = i % C;
        vsf[i] = c < n_rows ? v[(int64_t)(sd.y + c) * g.v_stride + j * g.rank_pad + k] : 0.f;
    }
    __syncthreads();

    const int o0 = tile * kExpandTile + threadIdx.x * 8;
    if (o0 >= hj) return;
    const uint16_t *bt =
        p.Bt + (int64_t)(slot - 1) * g.bt_slot_stride + g.bt_slice_off[j] + o0;
    float acc[C][8];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;

    for (int k = 0; k < rank; ++k) {
        const uint4 b = ld16(bt + (int64_t)k * hj);
        const float bf[8] = {__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u),
                             __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xffff0000u),
                             __uint_as_float(b.z << 16), __uint_as_float(b.z & 0xffff0000u),
                             __uint_as_float(b.w << 16), __uint_as_float(b.w & 0xffff0000u)};
        const float4 va = vs[k][0], vb = vs[k][1];
        const float vc[C] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (c < n_rows) {
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[c][e] = __builtin_fmaf(bf[e], vc[c], acc[c][e]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
        if (c < n_rows) {
            const int t = r.row_idx[sd.y + c];
            float4 *yp = reinterpret_cast<float4 *>(y + (int64_t)t * ldy + g.col_off[j] + o0);
            float4 a = yp[0], b = yp[1];
            a.x += acc[c][0];
            a.y += acc[c][1];
            a.z += acc[c][2];
            a.w += acc[c][3];
            b.x += acc[c][4];
            b.y += acc[c][5];
            b.z += acc[c][6];
            b.w += acc[c][7];
            yp[0] = a;
            yp[1] = b;
        }
    }
}

// ---- pool maintenance ----

__global__ void k_pack_a(uint16_t *dst, const uint16_t *src, int64_t lda, int64_t a_col0,
                         int rank, int h_in, int64_t total)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t k = i / h_in, c = i - k * h_in;
    dst[i] = k < rank ? src[k * lda + a_col0 + c] : (uint16_t)0;
}

__global__ void k_pack_bt(uint16_t *dst, const uint16_t *src, int64_t ldb, int rank, int h_out,
                          int64_t total)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t k = i / h_out, o = i - k * h_out;
    dst[i] = k < rank ? src[o * ldb + k] : (uint16_t)0;
}

__global__ void k_pack_bn(uint16_t *dst, const uint16_t *src, int64_t ldb, int rank,
                          int rank_pad, int64_t total)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int64_t o = i / rank_pad, k = i - o * rank_pad;
    dst[i] = k < rank ? src[o * ldb + k] : (uint16_t)0;
}

__global__ void k_set_meta(int32_t *rank_tab, float *scale_tab, int slot, int n_slices,
                           int4 ranks, float4 scales)
{
    const int j = threadIdx.x;
    if (j >= kMetaStride) return;
    const int rk[4] = {ranks.x, ranks.y, ranks.z, ranks.w};
    const float sc[4] = {scales.x, scales.y, scales.z, scales.w};
    rank_tab[slot * kMetaStride + j] = j < n_slices ? rk[j] : 0;
    scale_tab[slot * kMetaStride + j] = j < n_slices ? sc[j] : 0.f;
}

__global__ void k_clear_meta(int32_t *rank_tab, float *scale_tab, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    rank_tab[i] = 0;
    scale_tab[i] = 0.f;
}

}  // namespace

hipError_t launch_shrink_gemv(const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                              int n_seg, int kb_per_slice, const void *x, int64_t ldx, float *v,
                              hipStream_t s)
{
    const int64_t blocks = (int64_t)n_seg * g.n_slices * kb_per_slice;
    if (blocks <= 0) return hipSuccess;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const uint16_t *xp = static_cast<const uint16_t *>(x);
    if (g.x_fp16)
        hipLaunchKernelGGL(k_shrink_gemv<true>, dim3((unsigned)blocks), dim3(256), 0, s, g, p, r,
                           kb_per_slice, xp, ldx, v);
    else
        hipLaunchKernelGGL(k_shrink_gemv<false>, dim3((unsigned)blocks), dim3(256), 0, s, g, p, r,
                           kb_per_slice, xp, ldx, v);
    return hipGetLastError();
}

hipError_t launch_expand_gemv(const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                              int n_seg, int tiles_per_slice, const float *v, float *y,
                              int64_t ldy, hipStream_t s)
{
    const int64_t blocks = (int64_t)n_seg * g.n_slices * tiles_per_slice;
    if (blocks <= 0) return hipSuccess;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_expand_gemv, dim3((unsigned)blocks), dim3(64), 0, s, g, p, r,
                       tiles_per_slice, v, y, ldy);
    return hipGetLastError();
}

hipError_t launch_pack_a(uint16_t *dst, const uint16_t *src, int64_t lda, int64_t a_col0,
                         int rank, int rank_pad, int h_in, hipStream_t s)
{
    const int64_t total = (int64_t)rank_pad * h_in;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_pack_a, dim3((unsigned)blocks), dim3(256), 0, s, dst, src, lda, a_col0,
                       rank, h_in, total);
    return hipGetLastError();
}

hipError_t launch_pack_bt(uint16_t *dst, const uint16_t *src, int64_t ldb, int rank,
                          int rank_pad, int h_out, hipStream_t s)
{
    const int64_t total = (int64_t)rank_pad * h_out;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_pack_bt, dim3((unsigned)blocks), dim3(256), 0, s, dst, src, ldb, rank,
                       h_out, total);
    return hipGetLastError();
}

hipError_t launch_pack_bn(uint16_t *dst, const uint16_t *src, int64_t ldb, int rank,
                          int rank_pad, int h_out, hipStream_t s)
{
    const int64_t total = (int64_t)rank_pad * h_out;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_pack_bn, dim3((unsigned)blocks), dim3(256), 0, s, dst, src, ldb, rank,
                       rank_pad, total);
    return hipGetLastError();
}

hipError_t launch_set_meta(int32_t *rank_tab, float *scale_tab, int slot, int n_slices,
                           const int32_t *ranks, const float *scales, hipStream_t s)
{
    int4 rk = make_int4(0, 0, 0, 0);
    float4 sc = make_float4(0.f, 0.f, 0.f, 0.f);
    int *rp = &rk.x;
    float *sp = &sc.x;
    for (int j = 0; j < n_slices && j < 4; ++j) {
        rp[j] = ranks[j];
        sp[j] = scales[j];
    }
    hipLaunchKernelGGL(k_set_meta, dim3(1), dim3(64), 0, s, rank_tab, scale_tab, slot, n_slices,
                       rk, sc);
    return hipGetLastError();
}

hipError_t launch_clear_meta(int32_t *rank_tab, float *scale_tab, int n_rows, hipStream_t s)
{
    const int n = n_rows * kMetaStride;
    hipLaunchKernelGGL(k_clear_meta, dim3((n + 255) / 256), dim3(256), 0, s, rank_tab,
                       scale_tab, n);
    return hipGetLastError();
}

}  // namespace lora
