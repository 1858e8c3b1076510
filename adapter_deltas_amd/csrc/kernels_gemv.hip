// Decode path: gathered GEMV shrink and expand on the vector ALUs (gfx950).
//
// Decode rows of one adapter slot are grouped into segments of up to
// kDecodeSegRows rows.  The shrink reads each A tile once per segment and
// reuses it for all rows of the segment; the expand reads each B^T tile once
// per segment.  Both keep a per-row summation order fixed by the lane's
// widths and the adapter's rank (TensorFold PR #47, third commit message:
// fp32 sums in a fixed order, so a row's bits depend only on its own input and
// its own adapter); the order is spelled out in kernels_decode.h.
#include "kernels_decode.h"

#include <algorithm>

namespace lora {
namespace {

// W waves per task (1, 2, 4 or 8): wave w sums parts w, w + W, ... of the 8,
// each reduced on its own, so the bits do not depend on W.
//
// The prologue has no branch before the descriptor and count loads are
// issued, and the scale load follows them, so the first data loads wait for
// about two scalar round trips rather than a chain of them.
//
// vsplit > 0: v is written in the split form of the base projection's
// epilogue (rows of vsplit bf16) instead of fp32.
//
// TAB: the task is read from `tasks` (one word per live task: decode
// segment, slice, rank block), so no workgroup is launched for a rank block
// past its segment's rank; a slice past the pool's count ends the task.
template <bool FP16X, int W, bool TAB>
__global__ __launch_bounds__(64 * W) void k_shrink_gemv(LaneGeom g, PoolDev p, RoutingDev r,
                                                         int n_tasks, int kb_per_slice,
                                                         const uint16_t *__restrict__ x,
                                                         int64_t ldx, float *__restrict__ v,
                                                         int vsplit, const int32_t *tasks)
{
    touch_args(n_tasks, g, p, r, ldx);
    const int task = TAB ? xcd_task(blockIdx.x, n_tasks)
                         : seg_task(r, blockIdx.x, n_tasks, g.n_slices * kb_per_slice);
    if (task >= n_tasks) return;
    int si, j, kb;
    if constexpr (TAB) {
        typedef const __attribute__((address_space(4))) int32_t cint;
        const int w = *(cint *)(tasks + task);
        si = w & 0xffffff;
        j = (w >> 24) & 3;
        kb = (int)((uint32_t)w >> 26);
        if (j >= g.n_slices) return;
    } else {
        const int per_seg = g.n_slices * kb_per_slice;
        si = task / per_seg;
        const int rem = task - si * per_seg;
        j = rem / kb_per_slice;
        kb = rem - j * kb_per_slice;
    }
    Seg sd;
    if (!decode_seg(r, si, sd)) return;
    // past the count a device-built descriptor is stale: its slot is read
    // only after the check
    const float scale = p.scale[sd.slot() * kMetaStride + j];
    const int rank = sd.rank(j);
    const int k0 = kb * kKBlock;
    if (k0 >= rank) return;
    const int kn = min(kKBlock, rank - k0);
    const int wave = W == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int n_sub = (g.h_in + kSubChunk - 1) / kSubChunk;

    // rows past the segment are not multiplied (same bits for the others)
    const int nr = sd.n_rows();
    __shared__ float part[kParts][64];
#pragma unroll
    for (int pp = 0; pp < kParts / W; ++pp) {
        const int pt = wave + pp * W;
        // a part with no sub-chunk sums to zero
        float u = 0.f;
        if (pt < n_sub) {
            if (nr <= 2) u = shrink_part<FP16X, 2>(g, p, sd, j, k0, kn, pt, lane, x, ldx);
            else if (nr <= 4) u = shrink_part<FP16X, 4>(g, p, sd, j, k0, kn, pt, lane, x, ldx);
            else u = shrink_part<FP16X, 8>(g, p, sd, j, k0, kn, pt, lane, x, ldx);
        }
        part[pt][lane] = u;
    }
    __syncthreads();
    if (wave == 0) {
        const float q0 = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
        const float q1 = (part[4][lane] + part[5][lane]) + (part[6][lane] + part[7][lane]);
        const int c = lane / kKBlock;
        const int k = lane % kKBlock;
        if (c < sd.n_rows() && k < kn) {
            const float val = scale * (q0 + q1);
            if (vsplit) {
                const float one[1] = {val};
                store_vsplit<1>(reinterpret_cast<uint16_t *>(v), vsplit, vsplit_groups(g.rank_pad),
                                sd.v_row() + c, j, k0 + k, one);
            } else {
                v[(int64_t)(sd.v_row() + c) * g.v_stride + j * g.rank_pad + k0 + k] = val;
            }
        }
    }
}


// Prologue as in k_shrink_gemv; the slice's widths and offsets are taken from
// the arguments by selects.
// A task is (segment, slice, 64 LC columns), LC = 8 or 4 columns per lane;
// each of its 8 / C waves expands C segment rows.  C and LC change which
// wave computes an output, never its sum.
template <int C, int LC>
__global__ __launch_bounds__(64 * (kDecodeSegRows / C)) void k_expand_gemv(LaneGeom g, PoolDev p,
                                                                   RoutingDev r, int n_tasks,
                                                                   int tiles_per_seg,
                                                                   const float *__restrict__ v,
                                                                   float *__restrict__ y,
                                                                   int64_t ldy)
{
    constexpr int kExpandWaves = kDecodeSegRows / C;
    constexpr int TILE = 64 * LC;
    touch_args(n_tasks, g, p, r, ldy);
    const int task = seg_task(r, blockIdx.x, n_tasks, tiles_per_seg);
    if (task >= n_tasks) return;
    const int si = task / tiles_per_seg;
    int j, tile;
    slice_tile<TILE>(g, task - si * tiles_per_seg, j, tile);
    const int hj = pick4(g.h_out, j);
    const int col_off = pick4(g.col_off, j);
    const int64_t bt_off = pick4(g.bt_slice_off, j);
    Seg sd;
    const bool live = decode_seg(r, si, sd);
    if (!live) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int c0 = wave * C;                    // first segment row of this wave
    const int n_rows = sd.n_rows() - c0;        // rows of this wave (may be <= 0)
    if (n_rows <= 0) return;
    const int rank = sd.rank(j);
    const int o0 = tile * TILE + lane * LC;
    const bool col_ok = o0 < hj;
    const int oc = col_ok ? o0 : hj - LC;
    // token rows c0 .. c0 + C - 1 of the segment (wave-uniform selection)
    const int all[kDecodeSegRows] = {sd.row<0>(), sd.row<1>(), sd.row<2>(), sd.row<3>(),
                                     sd.row<4>(), sd.row<5>(), sd.row<6>(), sd.row<7>()};
    float *yp[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        int t = all[c];
#pragma unroll
        for (int w = 1; w < kExpandWaves; ++w)
            if (wave == w) t = all[w * C + c];
        yp[c] = y + (int64_t)t * ldy + col_off + oc;
    }
    const uint16_t *bt = p.Bt + (int64_t)(sd.slot() - 1) * g.bt_slot_stride + bt_off + oc;
    // v is read-only here and the same for every lane: constant-space reads
    // become scalar loads.
    typedef const __attribute__((address_space(4))) float cfloat;
    const int64_t vrow0 = (int64_t)(sd.v_row() + c0) * g.v_stride + j * g.rank_pad;
    auto vrow = [&](int c) {
        return (cfloat *)(v + vrow0 + (int64_t)min(c, n_rows - 1) * g.v_stride);
    };
    // v of ranks 0..15 (inside rank_pad) is requested here, ahead of the B and
    // y loads, so that it is not the last operand to arrive
    float vp[C][16];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        cfloat *vr = vrow(c);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const float t = vr[k];
            vp[c][k] = k < rank ? t : 0.f;
        }
    }
    auto vsrc = [&](int c, int kb, float (&out)[8]) {
        if (kb < 16) {
#pragma unroll
            for (int k = 0; k < 8; ++k) out[k] = kb == 0 ? vp[c][k] : vp[c][8 + k];
            return;
        }
        cfloat *vr = vrow(c);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float t = vr[kb + k];
            out[k] = kb + k < rank ? t : 0.f;
        }
    };
    expand_rows<C, LC>(yp, n_rows, bt, hj, rank, col_ok, [] {}, vsrc);
}

// Shrink and expand of decode segments in one launch, for ranks up to
// kFusedMaxRank.  A task is the expand's (segment, slice, 512 columns); its
// eight waves first compute the segment's v for the slice exactly as
// k_shrink_gemv does (wave w sums part w with shrink_part, the parts are
// combined in the same order, v = fp32(scale * u)) into LDS, while the
// task's y rows and first B blocks are already loading, and then expand one
// segment row each with expand_rows.  Every value is the one the two kernels
// produce, so the result is bit-identical to lora_shrink then lora_expand.
// The column tiles of a slice recompute the same v and re-read the slice's
// A: cheap next to a second launch while those bytes are few (8 rows x 64
// columns: 6.2 -> 5.0 us per call), too costly for a 4096-wide slice (8
// tiles: 12 -> 21 us) or for many segments over a wide h_in (a MoE gate_up
// with 768-wide slices: 35 -> 163 us).
template <bool FP16X>
__global__ __launch_bounds__(64 * kParts) void k_delta_gemv(LaneGeom g, PoolDev p, RoutingDev r,
                                                            int n_tasks, int tiles_per_seg,
                                                            const uint16_t *__restrict__ x,
                                                            int64_t ldx, float *__restrict__ y,
                                                            int64_t ldy)
{
    constexpr int KB = kFusedMaxRank / kKBlock;   // rank blocks at most
    static_assert(kParts == kDecodeSegRows, "one part and one row per wave");
    touch_args(n_tasks, g, p, r, ldy);
    const int task = seg_task(r, blockIdx.x, n_tasks, tiles_per_seg);
    if (task >= n_tasks) return;
    const int si = task / tiles_per_seg;
    int j, tile;
    slice_tile<kExpandTile>(g, task - si * tiles_per_seg, j, tile);
    const int hj = pick4(g.h_out, j);
    const int col_off = pick4(g.col_off, j);
    const int64_t bt_off = pick4(g.bt_slice_off, j);
    Seg sd;
    const bool live = decode_seg(r, si, sd);
    if (!live) return;       // the whole workgroup
    const float scale = p.scale[sd.slot() * kMetaStride + j];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int rank = sd.rank(j);
    const int n_kb = (rank + kKBlock - 1) / kKBlock;
    const int o0 = tile * kExpandTile + lane * 8;
    const bool col_ok = o0 < hj;
    const int oc = col_ok ? o0 : hj - 8;
    // this wave's segment row (past the segment: the descriptor's repeat of
    // the last row, loaded but not stored)
    const int all[kDecodeSegRows] = {sd.row<0>(), sd.row<1>(), sd.row<2>(), sd.row<3>(),
                                     sd.row<4>(), sd.row<5>(), sd.row<6>(), sd.row<7>()};
    int trow = all[0];
#pragma unroll
    for (int w = 1; w < kDecodeSegRows; ++w)
        if (wave == w) trow = all[w];
    float *const yp[1] = {y + (int64_t)trow * ldy + col_off + oc};
    const uint16_t *bt = p.Bt + (int64_t)(sd.slot() - 1) * g.bt_slot_stride + bt_off + oc;

    __shared__ float part[KB][kParts][64];
    __shared__ float vl[kDecodeSegRows][KB * kKBlock];
    const int n_sub = (g.h_in + kSubChunk - 1) / kSubChunk;
    auto shrink = [&] {
        for (int kb = 0; kb < n_kb; ++kb) {
            const int k0 = kb * kKBlock;
            // a part with no sub-chunk sums to zero
            part[kb][wave][lane] =
                wave < n_sub ? shrink_part<FP16X>(g, p, sd, j, k0, min(kKBlock, rank - k0), wave,
                                                  lane, x, ldx)
                             : 0.f;
        }
        __syncthreads();
        if ((int)threadIdx.x < n_kb * 64) {
            const int kb = threadIdx.x >> 6, l = threadIdx.x & 63;
            const float q0 = (part[kb][0][l] + part[kb][1][l]) + (part[kb][2][l] + part[kb][3][l]);
            const float q1 = (part[kb][4][l] + part[kb][5][l]) + (part[kb][6][l] + part[kb][7][l]);
            vl[l / kKBlock][kb * kKBlock + l % kKBlock] = scale * (q0 + q1);
        }
        __syncthreads();
    };
    auto vsrc = [&](int, int kb, float (&out)[8]) {
#pragma unroll
        for (int k = 0; k < 8; ++k) out[k] = kb + k < rank ? vl[wave][kb + k] : 0.f;
    };
    expand_rows<1, 8>(yp, sd.n_rows() - wave, bt, hj, rank, col_ok, shrink, vsrc);
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
                              int vsplit, hipStream_t s, const int32_t *tasks, int n_tasks)
{
    const int64_t blocks = tasks ? n_tasks : (int64_t)n_seg * g.n_slices * kb_per_slice;
    if (blocks <= 0) return hipSuccess;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const uint16_t *xp = static_cast<const uint16_t *>(x);
    // Waves per task: enough for the sub-chunks of h_in, at most one per
    // part, and fewer as the grid grows (a wave then sums several parts in
    // turn; the sums do not change).  A small grid needs every wave it can
    // get, a large one keeps more, smaller workgroups resident per CU.
    // Measured shrink per call with 8 / 4 / 2 waves: decode_mix (162 tasks)
    // 5.7 / 6.8 / 9.3 us, many_tenants (1160) 29.4 / 25.0 / 36.6, moe_decode
    // (about 3500) 23.0 / 23.0 / 21.8.
    const int n_sub = (g.h_in + kSubChunk - 1) / kSubChunk;
    const int w_max = blocks < 512 ? 8 : blocks < 2048 ? 4 : 2;
    const int w = std::min(w_max, n_sub >= 8 ? 8 : n_sub >= 4 ? 4 : n_sub >= 2 ? 2 : 1);
    const int64_t n_blocks =
        tasks ? blocks : seg_grid(r, n_seg, (int64_t)g.n_slices * kb_per_slice);
    if (n_blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)n_blocks), block(64 * w);
#define LAUNCH_SHRINK(F, W)                                                                   \
    do {                                                                                      \
        if (tasks)                                                                            \
            hipLaunchKernelGGL((k_shrink_gemv<F, W, true>), grid, block, 0, s, g, p, r,       \
                               (int)blocks, kb_per_slice, xp, ldx, v, vsplit, tasks);         \
        else                                                                                  \
            hipLaunchKernelGGL((k_shrink_gemv<F, W, false>), grid, block, 0, s, g, p, r,      \
                               (int)blocks, kb_per_slice, xp, ldx, v, vsplit, tasks);         \
    } while (0)
    if (g.x_fp16) {
        if (w == 8) LAUNCH_SHRINK(true, 8);
        else if (w == 4) LAUNCH_SHRINK(true, 4);
        else if (w == 2) LAUNCH_SHRINK(true, 2);
        else LAUNCH_SHRINK(true, 1);
    } else {
        if (w == 8) LAUNCH_SHRINK(false, 8);
        else if (w == 4) LAUNCH_SHRINK(false, 4);
        else if (w == 2) LAUNCH_SHRINK(false, 2);
        else LAUNCH_SHRINK(false, 1);
    }
#undef LAUNCH_SHRINK
    return hipGetLastError();
}

hipError_t launch_delta_gemv(const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                             int n_seg, const void *x, int64_t ldx, float *y, int64_t ldy,
                             hipStream_t s)
{
    const int tiles_per_seg = lane_tiles(g, kExpandTile);
    const int64_t blocks = (int64_t)n_seg * tiles_per_seg;
    if (blocks <= 0) return hipSuccess;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const uint16_t *xp = static_cast<const uint16_t *>(x);
    const int64_t n_blocks = seg_grid(r, n_seg, tiles_per_seg);
    if (n_blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)n_blocks), block(64 * kParts);
    if (g.x_fp16)
        hipLaunchKernelGGL(k_delta_gemv<true>, grid, block, 0, s, g, p, r, (int)blocks,
                           tiles_per_seg, xp, ldx, y, ldy);
    else
        hipLaunchKernelGGL(k_delta_gemv<false>, grid, block, 0, s, g, p, r, (int)blocks,
                           tiles_per_seg, xp, ldx, y, ldy);
    return hipGetLastError();
}

hipError_t launch_expand_gemv(const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                              int n_seg, int rows_per_wave, int lane_cols, const float *v,
                              float *y, int64_t ldy, hipStream_t s)
{
    // only live tiles: ceil(h_j / columns per task) for each slice j
    const int tiles_per_seg = lane_tiles(g, 64 * lane_cols);
    const int64_t blocks = (int64_t)n_seg * tiles_per_seg;
    if (blocks <= 0) return hipSuccess;
    const int64_t n_blocks = seg_grid(r, n_seg, tiles_per_seg);
    if (n_blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)n_blocks);
#define LAUNCH_EXPAND(C, LC)                                                                      \
    hipLaunchKernelGGL((k_expand_gemv<C, LC>), grid, dim3(64 * (kDecodeSegRows / C)), 0, s, g, p, \
                       r, (int)blocks, tiles_per_seg, v, y, ldy)
    if (rows_per_wave == 4 && lane_cols == 8) LAUNCH_EXPAND(4, 8);
    else if (rows_per_wave == 4 && lane_cols == 4) LAUNCH_EXPAND(4, 4);
    else if (rows_per_wave == 2 && lane_cols == 8) LAUNCH_EXPAND(2, 8);
    else if (rows_per_wave == 2 && lane_cols == 4) LAUNCH_EXPAND(2, 4);
    else return hipErrorInvalidValue;
#undef LAUNCH_EXPAND
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
