// Decode-path device code of the GEMV shrink and expand kernels.
//
// Shrink order for u[k] = sum_i A[k][i] x[i] over h_in:
//   h_in is cut into sub-chunks of kSubChunk = 512 elements; sub-chunk q
//   belongs to part q % 8.  Within a part, lane l of a wave accumulates
//   elements [512 q + 8 l, 512 q + 8 l + 8) of its sub-chunks, q ascending,
//   four bf16 pair-dot steps per sub-chunk (pairs 0-1, 2-3, 4-5, 6-7), into one
//   fp32 sum (elements past h_in count as zero).  The 64 lane sums are combined
//   by a fixed reduce-scatter butterfly (partners L^32, L^16, L^8, L^7, L^2,
//   L^1); the part sums as q0 = (p0 + p1) + (p2 + p3), q1 = (p4 + p5) + (p6 + p7),
//   u = q0 + q1, and v = fp32(scale * u).
//   An fp16 input is split exactly into two bf16 values x = hi + lo (fp16
//   carries 11 significant bits) and each pair-dot step is done for hi, then lo.
// Expand order: d[o] = fma chain over k = 0 .. rank-1 starting from 0, then
//   y[o] = y[o] + d[o].
#pragma once

#include "kernels_common.h"

namespace lora {


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

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Halving step across lanes L and L ^ M (M = 32 or 16) by a swap of register
// halves: afterwards every lane holds its own half plus its partner's copy of
// it (lanes with bit M clear keep entries [0, M), the others [M, 2M)).
template <int M>
__device__ __forceinline__ void halve_swap(float (&val)[64])
{
#pragma unroll
    for (int i = 0; i < M; ++i) {
        uint32_t a = __float_as_uint(val[i]), b = __float_as_uint(val[M + i]);
        if constexpr (M == 32) {
            const auto t = __builtin_amdgcn_permlane32_swap(a, b, false, false);
            a = t[0];
            b = t[1];
        } else {
            const auto t = __builtin_amdgcn_permlane16_swap(a, b, false, false);
            a = t[0];
            b = t[1];
        }
        val[i] = __uint_as_float(a) + __uint_as_float(b);
    }
}

// Halving step across lanes L and P(L) for a lane pairing P given by a DPP
// control, where P(L) differs from L in bit BIT (and possibly in lower bits).
template <int M, int BIT, int CTRL>
__device__ __forceinline__ void halve_dpp(float (&val)[64], int lane)
{
    const bool upper = (lane & BIT) != 0;
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const float lo = val[i], hi = val[M + i];
        const float send = upper ? lo : hi;
        const float keep = upper ? hi : lo;
        val[i] = keep + dpp<CTRL>(send);
    }
}

// In lane L: the sum over the wave's 64 lanes of val[L].  Fixed butterfly:
// partners L^32, L^16 (register-half swaps), then L^8 (row rotate by 8),
// L^7 (half-row mirror), L^2, L^1 (quad permutes); lane L keeps, at each step,
// the half selected by its own bit 5, 4, 3, 2, 1, 0.
__device__ __forceinline__ float wave_reduce_scatter64(float (&val)[64], int lane)
{
    halve_swap<32>(val);
    halve_swap<16>(val);
    halve_dpp<8, 8, 0x128>(val, lane);   // row_ror:8
    halve_dpp<4, 4, 0x141>(val, lane);   // row_half_mirror
    halve_dpp<2, 2, 0x4E>(val, lane);    // quad_perm [2,3,0,1]
    halve_dpp<1, 1, 0xB1>(val, lane);    // quad_perm [1,0,3,2]
    return val[0];
}

// One wave's share of a shrink step: x of the segment's rows and A of the
// task's ranks at one 8-element column group of a sub-chunk.
struct ShrinkTile {
    uint4 x[kDecodeSegRows];
    uint4 a[kKBlock];
};

// Only the first R rows are loaded and multiplied (the others' sums stay 0).
template <bool FP16X, int R>
__device__ __forceinline__ void shrink_tile_fma(const ShrinkTile &t, bool valid,
                                                float (&acc)[kDecodeSegRows][kKBlock])
{
    constexpr int C = R;
    uint32_t xw[C][FP16X ? 8 : 4];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const uint4 u = valid ? t.x[c] : make_uint4(0, 0, 0, 0);
        if constexpr (FP16X) {
            split_f16x2(u.x, xw[c][0], xw[c][4]);
            split_f16x2(u.y, xw[c][1], xw[c][5]);
            split_f16x2(u.z, xw[c][2], xw[c][6]);
            split_f16x2(u.w, xw[c][3], xw[c][7]);
        } else {
            xw[c][0] = u.x;
            xw[c][1] = u.y;
            xw[c][2] = u.z;
            xw[c][3] = u.w;
        }
    }
#pragma unroll
    for (int k = 0; k < kKBlock; ++k) {
        const uint32_t aw[4] = {t.a[k].x, t.a[k].y, t.a[k].z, t.a[k].w};
#pragma unroll
        for (int c = 0; c < C; ++c) {
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

// One wave's part sum for the 8 x 8 (row, rank) block of a shrink task:
// part `part` of h_in, reduced over the wave; lane L returns the value of
// (row L / 8, rank k0 + L % 8).  With R < 8 only rows 0 .. R-1 are loaded
// and multiplied and the other rows sum to 0: every (row, rank) value has
// its own chain of pair-dots and its own path through the butterfly, so the
// computed rows get the same bits as with R = 8 (for segments of at most R
// rows, at a fraction of the loads and products).
template <bool FP16X, int R = kDecodeSegRows>
__device__ __forceinline__ float shrink_part(const LaneGeom &g, const PoolDev &p, const Seg &sd,
                                             int j, int k0, int kn, int part, int lane,
                                             const uint16_t *__restrict__ x, int64_t ldx)
{
    constexpr int C = kDecodeSegRows;
    // Rows past the segment and ranks past the adapter's rank re-read the last
    // valid row (a cache hit); their sums are computed and discarded.
    const uint16_t *Ab = p.A + (int64_t)(sd.slot() - 1) * g.a_slot_stride +
                         ((int64_t)j * g.rank_pad + k0) * g.h_in;
    const uint16_t *ar[kKBlock];
#pragma unroll
    for (int k = 0; k < kKBlock; ++k) ar[k] = Ab + (int64_t)min(k, kn - 1) * g.h_in;
    const uint16_t *xr[C] = {x + (int64_t)sd.row<0>() * ldx, x + (int64_t)sd.row<1>() * ldx,
                             x + (int64_t)sd.row<2>() * ldx, x + (int64_t)sd.row<3>() * ldx,
                             x + (int64_t)sd.row<4>() * ldx, x + (int64_t)sd.row<5>() * ldx,
                             x + (int64_t)sd.row<6>() * ldx, x + (int64_t)sd.row<7>() * ldx};
    float acc[C][kKBlock];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int k = 0; k < kKBlock; ++k) acc[c][k] = 0.f;
    // All loads of a sub-chunk are issued before its products.
    const int n_sub = (g.h_in + kSubChunk - 1) / kSubChunk;
    for (int q = part; q < n_sub; q += kParts) {
        const int e_raw = q * kSubChunk + lane * 8;
        const int e = min(e_raw, g.h_in - 8);
        ShrinkTile t;
#pragma unroll
        for (int c = 0; c < R; ++c) t.x[c] = ld16(xr[c] + e);
#pragma unroll
        for (int k = 0; k < kKBlock; ++k) t.a[k] = ld16(ar[k] + e);
        shrink_tile_fma<FP16X, R>(t, e_raw < g.h_in, acc);
    }
    float val[64];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int k = 0; k < kKBlock; ++k) val[c * kKBlock + k] = acc[c][k];
    return wave_reduce_scatter64(val, lane);
}

__device__ __forceinline__ void widen_bf16x8(uint4 b, float (&f)[8])
{
    f[0] = __uint_as_float(b.x << 16);
    f[1] = __uint_as_float(b.x & 0xffff0000u);
    f[2] = __uint_as_float(b.y << 16);
    f[3] = __uint_as_float(b.y & 0xffff0000u);
    f[4] = __uint_as_float(b.z << 16);
    f[5] = __uint_as_float(b.z & 0xffff0000u);
    f[6] = __uint_as_float(b.w << 16);
    f[7] = __uint_as_float(b.w & 0xffff0000u);
}

// B^T of LC = 8 or 4 adjacent columns of one rank, as one 16- or 8-byte load.
template <int LC> struct BLoad;
template <> struct BLoad<8> {
    typedef uint4 T;
    __device__ static void widen(T b, float (&f)[8]) { widen_bf16x8(b, f); }
};
template <> struct BLoad<4> {
    typedef uint2 T;
    __device__ static void widen(T b, float (&f)[4])
    {
        f[0] = __uint_as_float(b.x << 16);
        f[1] = __uint_as_float(b.x & 0xffff0000u);
        f[2] = __uint_as_float(b.y << 16);
        f[3] = __uint_as_float(b.y & 0xffff0000u);
    }
};

// Expand of C rows of a decode segment over LC (8 or 4) columns per lane.
//   yp[c]    y of segment row c at this lane's columns (valid for every c)
//   n_rows   rows of the C that belong to the segment (may exceed C, rows
//            from C on being another wave's, or be <= 0: nothing is stored)
//   bt       B^T of the slice at this lane's columns: bt[k * hj]
//   wait     called once, after the loads of the first two B blocks and of y
//            are issued and before v is first read
//   vsrc     vsrc(c, kb, out) fills out[0..8) with v of row c, ranks kb..kb+7
//            (ranks at or past `rank` must come back as zero)
// y[row c][cols] += sum_k B[k] v[c][k] for c < n_rows, when store is true.
template <int C, int LC, class Wait, class VSrc>
__device__ __forceinline__ void expand_rows(float *const (&yp)[C], int n_rows,
                                            const uint16_t *bt, int hj, int rank, bool store,
                                            Wait wait, VSrc vsrc)
{
    static_assert(LC == 8 || LC == 4, "8 or 4 columns per lane");
    typedef typename BLoad<LC>::T BV;
    // Ranks in blocks of 8 (pool rows past the rank are zero and in bounds;
    // v past the rank is zero), the next block's B loads in flight.  Loads
    // complete in issue order, so the first two B blocks (rows 0..15, inside
    // rank_pad) are issued before y: their products then run while y is
    // still on its way from HBM.
    BV b0[8], b1[8];
    auto load_b = [&](BV (&b)[8], int kb) {
#pragma unroll
        for (int k = 0; k < 8; ++k) b[k] = *reinterpret_cast<const BV *>(bt + (int64_t)(kb + k) * hj);
    };
    load_b(b0, 0);
    load_b(b1, 8);
    __builtin_amdgcn_sched_barrier(0);   // keeps the y loads behind them
    float4 ya[C], yb[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        ya[c] = reinterpret_cast<const float4 *>(yp[c])[0];
        if constexpr (LC == 8) yb[c] = reinterpret_cast<const float4 *>(yp[c])[1];
    }
    float acc[C][LC];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int e = 0; e < LC; ++e) acc[c][e] = 0.f;
    auto fma_b = [&](const BV (&b)[8], int kb) {
        float vk[C][8];
#pragma unroll
        for (int c = 0; c < C; ++c) vsrc(c, kb, vk[c]);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float bf[LC];
            BLoad<LC>::widen(b[k], bf);
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int e = 0; e < LC; ++e) acc[c][e] = __builtin_fmaf(bf[e], vk[c][k], acc[c][e]);
        }
    };
    wait();
    // ranks 0..15 peeled (constant kb, so a caller's vsrc can serve them from
    // registers), then blocks of 16
    fma_b(b0, 0);
    if (rank > 8) {
        if (rank > 16) load_b(b0, 16);
        fma_b(b1, 8);
        if (rank > 24) load_b(b1, 24);
        for (int kb = 16; kb < rank; kb += 16) {
            fma_b(b0, kb);
            if (kb + 8 >= rank) break;
            if (kb + 16 < rank) load_b(b0, kb + 16);
            fma_b(b1, kb + 8);
            if (kb + 24 < rank) load_b(b1, kb + 24);
        }
    }
    if (store) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (c < n_rows) {
                float4 a = ya[c];
                a.x += acc[c][0];
                a.y += acc[c][1];
                a.z += acc[c][2];
                a.w += acc[c][3];
                reinterpret_cast<float4 *>(yp[c])[0] = a;
                if constexpr (LC == 8) {
                    float4 b = yb[c];
                    b.x += acc[c][4];
                    b.y += acc[c][5];
                    b.z += acc[c][6];
                    b.w += acc[c][7];
                    reinterpret_cast<float4 *>(yp[c])[1] = b;
                }
            }
        }
    }
}

}  // namespace lora
