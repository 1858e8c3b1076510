// Prefill path: shrink and expand of a prompt chunk on the matrix cores (gfx950).
//
// A prefill segment is up to kPrefillSegRows contiguous rows of one sequence
// with one adapter slot (TensorFold PR #47, third commit message: prompt
// chunks run one slot for all their rows), so the shrink is the dense product
// [rows x h_in] x [h_in x rank] and the expand [rows x rank] x [rank x h_j].
// Both use v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Each wave owns
// 16 rows of the segment.
//
// Shrink:  u^T[k][t] = sum over K-steps of 32 (ascending) of one MFMA with
//          the pool's A rows as the first operand and x rows as the second.
//          An fp16 x is split exactly into bf16 hi + lo and each K-step does
//          the hi product, then the lo product.  v = fp32(scale * u).
// Expand:  d^T[o][t] = sum over K-steps of 32 (ascending) of two MFMAs,
//          B rows times v_hi then B rows times v_lo, where v = v_hi + v_lo with
//          v_hi = bf16(v) and v_lo = bf16(v - v_hi) (both nearest-even), which
//          carries about 16 significant bits of the fp32 v into the bf16
//          products.  Then y = y + d.
// Every output element depends only on its own row of x (or v) and the
// adapter's factors, and a sequence is cut into segments by its own length
// only, so a row's bits do not depend on the rest of the batch.
#include "kernels_common.h"

namespace lora {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16x16x32(uint4 a, uint4 b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Exact split of eight packed fp16 values into packed bf16 hi and lo parts.
__device__ __forceinline__ void split_f16x8(uint4 w, uint4 &hi, uint4 &lo)
{
    uint32_t in[4] = {w.x, w.y, w.z, w.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float f0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(in[m] & 0xffffu));
        const float f1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(in[m] >> 16));
        const uint32_t u0 = __float_as_uint(f0), u1 = __float_as_uint(f1);
        const uint32_t t0 = u0 & 0xffff0000u, t1 = u1 & 0xffff0000u;
        const float l0 = f0 - __uint_as_float(t0);
        const float l1 = f1 - __uint_as_float(t1);
        h[m] = (u0 >> 16) | t1;
        l[m] = (__float_as_uint(l0) >> 16) | (__float_as_uint(l1) & 0xffff0000u);
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

__device__ __forceinline__ uint32_t bf16_bits(float f)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two-term bf16 form of eight fp32 values: hi = bf16(f), lo = bf16(f - hi).
__device__ __forceinline__ void split_f32x8(const float (&f)[8], uint4 &hi, uint4 &lo)
{
    uint32_t h[8], l[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        h[m] = bf16_bits(f[m]);
        l[m] = bf16_bits(f[m] - __uint_as_float(h[m] << 16));
    }
    hi = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                    h[6] | (h[7] << 16));
    lo = make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16),
                    l[6] | (l[7] << 16));
}

template <bool FP16X, int NT>
__global__ __launch_bounds__(256) void k_shrink_mfma(LaneGeom g, PoolDev p, RoutingDev r,
                                                      int seg_begin,
                                                      const uint16_t *__restrict__ x,
                                                      int64_t ldx, float *__restrict__ v)
{
    const int task = blockIdx.x;
    const int si = seg_begin + task / g.n_slices;
    const int j = task % g.n_slices;
    const Seg sd = load_seg(r.seg, si);
    const int slot = sd.slot();
    const int n_rows = sd.n_rows();
    const int rank = sd.rank(j);
    const int ntiles = (rank + 15) / 16;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r0 = wave * 16;
    if (r0 >= n_rows || ntiles > NT) return;
    const int li = lane & 15, lg = lane >> 4;
    const int row = r0 + li;
    const bool row_ok = row < n_rows;
    const uint16_t *xrow = x + (int64_t)(sd.first_row() + (row_ok ? row : r0)) * ldx;
    const uint16_t *Ab = p.A + (int64_t)(slot - 1) * g.a_slot_stride +
                         (int64_t)j * g.rank_pad * g.h_in + (int64_t)li * g.h_in;
    const int64_t tile_stride = (int64_t)16 * g.h_in;

    f32x4_t acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll 2
    for (int k0 = 0; k0 < g.h_in; k0 += 32) {
        const int e = k0 + lg * 8;
        const bool e_ok = e < g.h_in;
        const uint4 xv = (row_ok && e_ok) ? ld16(xrow + e) : zero;
        uint4 xhi = xv, xlo = zero;
        if constexpr (FP16X) split_f16x8(xv, xhi, xlo);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (nt < ntiles) {
                const uint4 av = e_ok ? ld16(Ab + nt * tile_stride + e) : zero;
                acc[nt] = mfma16x16x32(av, xhi, acc[nt]);
                if constexpr (FP16X) acc[nt] = mfma16x16x32(av, xlo, acc[nt]);
            }
        }
    }

    if (row_ok) {
        const float scale = p.scale[slot * kMetaStride + j];
        float *vr = v + (int64_t)(sd.v_row() + row) * g.v_stride + j * g.rank_pad + 4 * lg;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            if (nt < ntiles) {
                float4 o;
                o.x = scale * acc[nt][0];
                o.y = scale * acc[nt][1];
                o.z = scale * acc[nt][2];
                o.w = scale * acc[nt][3];
                *reinterpret_cast<float4 *>(vr + nt * 16) = o;
            }
        }
    }
}

template <int NS>
__global__ __launch_bounds__(256) void k_expand_mfma(LaneGeom g, PoolDev p, RoutingDev r,
                                                      int seg_begin, int tiles_per_slice,
                                                      const float *__restrict__ v,
                                                      float *__restrict__ y, int64_t ldy)
{
    const int per_seg = g.n_slices * tiles_per_slice;
    const int task = blockIdx.x;
    const int si = seg_begin + task / per_seg;
    const int rem = task % per_seg;
    const int j = rem / tiles_per_slice;
    const int tile = rem - j * tiles_per_slice;
    const int hj = g.h_out[j];
    const int o_base = tile * (NS * 16);
    if (o_base >= hj) return;
    const Seg sd = load_seg(r.seg, si);
    const int slot = sd.slot();
    const int n_rows = sd.n_rows();
    const int rank = sd.rank(j);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r0 = wave * 16;
    if (r0 >= n_rows) return;
    const int li = lane & 15, lg = lane >> 4;
    const int row = r0 + li;
    const bool row_ok = row < n_rows;
    const float *vrow =
        v + (int64_t)(sd.v_row() + (row_ok ? row : r0)) * g.v_stride + j * g.rank_pad;
    const uint16_t *Bn = p.Bn + (int64_t)(slot - 1) * g.bt_slot_stride + g.bt_slice_off[j];

    f32x4_t acc[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const uint4 zero = make_uint4(0, 0, 0, 0);
    for (int k0 = 0; k0 < rank; k0 += 32) {
        const int kk = k0 + lg * 8;
        float vf[8];
        if (row_ok && kk + 8 <= rank) {
            const float4 a = *reinterpret_cast<const float4 *>(vrow + kk);
            const float4 b = *reinterpret_cast<const float4 *>(vrow + kk + 4);
            vf[0] = a.x; vf[1] = a.y; vf[2] = a.z; vf[3] = a.w;
            vf[4] = b.x; vf[5] = b.y; vf[6] = b.z; vf[7] = b.w;
        } else {
#pragma unroll
            for (int m = 0; m < 8; ++m) vf[m] = (row_ok && kk + m < rank) ? vrow[kk + m] : 0.f;
        }
        uint4 vhi, vlo;
        split_f32x8(vf, vhi, vlo);
        const bool k_ok = kk + 8 <= g.rank_pad;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int o = o_base + s * 16 + li;
            const uint4 bv = (k_ok && o < hj) ? ld16(Bn + (int64_t)o * g.rank_pad + kk) : zero;
            acc[s] = mfma16x16x32(bv, vhi, acc[s]);
            acc[s] = mfma16x16x32(bv, vlo, acc[s]);
        }
    }

    if (row_ok) {
        const int t = sd.first_row() + row;
        float *yrow = y + (int64_t)t * ldy + g.col_off[j];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int oc = o_base + s * 16 + 4 * lg;
            if (oc < hj) {
                float4 *yp = reinterpret_cast<float4 *>(yrow + oc);
                float4 yv = *yp;
                yv.x += acc[s][0];
                yv.y += acc[s][1];
                yv.z += acc[s][2];
                yv.w += acc[s][3];
                *yp = yv;
            }
        }
    }
}

}  // namespace

hipError_t launch_shrink_mfma(const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                              int seg_begin, int n_seg, int nt_per_slice, const void *x,
                              int64_t ldx, float *v, hipStream_t s)
{
    const int64_t blocks = (int64_t)n_seg * g.n_slices;
    if (blocks <= 0 || nt_per_slice <= 0) return hipSuccess;
    if (blocks > INT32_MAX || nt_per_slice > 16) return hipErrorInvalidConfiguration;
    const uint16_t *xp = static_cast<const uint16_t *>(x);
    const dim3 grid((unsigned)blocks), block(256);
#define LAUNCH_SHRINK(F, N) \
    hipLaunchKernelGGL((k_shrink_mfma<F, N>), grid, block, 0, s, g, p, r, seg_begin, xp, ldx, v)
    if (g.x_fp16) {
        if (nt_per_slice <= 4) LAUNCH_SHRINK(true, 4);
        else if (nt_per_slice <= 8) LAUNCH_SHRINK(true, 8);
        else LAUNCH_SHRINK(true, 16);
    } else {
        if (nt_per_slice <= 4) LAUNCH_SHRINK(false, 4);
        else if (nt_per_slice <= 8) LAUNCH_SHRINK(false, 8);
        else LAUNCH_SHRINK(false, 16);
    }
#undef LAUNCH_SHRINK
    return hipGetLastError();
}

hipError_t launch_expand_mfma(const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                              int seg_begin, int n_seg, int tiles_per_slice, const float *v,
                              float *y, int64_t ldy, hipStream_t s)
{
    const int64_t blocks = (int64_t)n_seg * g.n_slices * tiles_per_slice;
    if (blocks <= 0) return hipSuccess;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_expand_mfma<kMfmaExpandCols / 16>), dim3((unsigned)blocks), dim3(256),
                       0, s, g, p, r, seg_begin, tiles_per_slice, v, y, ldy);
    return hipGetLastError();
}

}  // namespace lora
