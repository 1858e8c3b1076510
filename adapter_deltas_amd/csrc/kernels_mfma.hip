// Prefill path: shrink and expand of a prompt chunk on the matrix cores (gfx950).
//
// A prefill segment is up to kPrefillSegRows contiguous rows of one sequence
// with one adapter slot (TensorFold PR #47, third commit message: prompt
// chunks run one slot for all their rows), so the shrink is the dense product
// [rows x h_in] x [h_in x rank] and the expand [rows x rank] x [rank x h_j].
// Both use v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Each wave owns
// 16 rows of the segment.
//
// Shrink:  h_in is cut into pairs of K-steps of 32 (64 elements, loaded as
//          whole 128-byte rows); pair p belongs to part p % 4.
//          S_w[t][k] = MFMA chain over the K-steps of part w's pairs,
//          ascending, with the pool's A rows as the first operand and x rows
//          as the second;
//          u = (S_0 + S_1) + (S_2 + S_3) and v = fp32(scale * u).  An fp16 x
//          is split exactly into bf16 hi + lo and each K-step does the hi
//          product, then the lo product.  The order depends on h_in only.
// Expand:  d^T[o][t] = sum over K-steps of 32 (ascending) of two MFMAs,
//          B rows times v_hi then B rows times v_lo, where v = v_hi + v_lo with
//          v_hi = bf16(v) and v_lo = bf16(v - v_hi) (both nearest-even), which
//          carries about 16 significant bits of the fp32 v into the bf16
//          products.  Then y = y + d.
// Every output element depends only on its own row of x (or v) and the
// adapter's factors, and a sequence is cut into segments by its own length
// only, so a row's bits do not depend on the rest of the batch.
#include "kernels_common.h"

#include <type_traits>

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

constexpr int kShrinkParts = 4;     // waves of a shrink task: one K-part each
constexpr int kRowTiles = kPrefillSegRows / 16;

// Position of 16-byte chunk c of a staged 128-byte row: an XOR swizzle, so
// the 16 rows an operand read takes one chunk index from, and the 8 rows a
// load instruction writes, fall in different bank groups.
__device__ __forceinline__ int chunk_pos(int row, int c) { return c ^ (row & 7); }

// Shrink task: RT 16-row tiles of one prefill segment and up to NG 16-rank
// tiles.  A segment's rank tiles are numbered across its slices (slice 0's
// tiles, then slice 1's, ...), and a task takes `cnt` consecutive ones from
// number c0, so one task can cover the tiles of several slices and read the
// segment's x rows once for all of them.  Wave w owns K-part w.  Each pair of
// K-steps loads the segment's x rows and the tiles' A rows as whole 128-byte
// lines (eight consecutive lanes read one row's 64 elements, eight rows per
// instruction: a load of 16 rows x 64 bytes ran at half the rate), and
// reorders them through the wave's own LDS into the MFMA operand layout
// (lane l: row l % 16, elements 8 (l / 16) .. + 7 of the K-step).
// Tasks come from a host-built table (word: segment | c0 << 24 |
// (cnt - 1) << 30, whole segments; block b takes word b, laid out for XCD
// b % 8) when the routing has one for the lane's slice count; otherwise from
// the block index: row chunk, slice, group of NG tiles.  Either way a
// (row, rank) sum is the same.
// vsplit > 0: v is written in the split form of the base projection's
// epilogue (rows of vsplit bf16) instead of fp32.
template <bool FP16X, int NG, int RT, bool GATHER>
__device__ __forceinline__ void shrink_mfma_task(const LaneGeom &g, const PoolDev &p,
                                                 const RoutingDev &r, int task, int seg_begin,
                                                 int groups_per_slice,
                                                 const uint32_t *__restrict__ tab,
                                                 const uint16_t *__restrict__ x, int64_t ldx,
                                                 float *__restrict__ v, int vsplit)
{
    constexpr int ROWS = 16 * RT;
    static_assert(kRowTiles % RT == 0, "row chunks tile the segment");
    int si, rc, c0 = 0, cnt = 0, jb = 0, grp = 0;
    if (tab) {
        const uint32_t w = tab[task];
        if (w == (uint32_t)kMfmaTaskNone) return;   // an empty place of the table
        si = seg_begin + (int)(w & 0xffffffu);
        rc = 0;
        c0 = (int)((w >> 24) & 63u);
        cnt = (int)(w >> 30) + 1;
    } else {
        // task order within a segment: row chunk, slice, rank group
        const int per_chunk = g.n_slices * groups_per_slice;
        const int per_seg = per_chunk * (kRowTiles / RT);
        si = seg_begin + task / per_seg;
        const int rem = task % per_seg;
        rc = rem / per_chunk;
        const int rem2 = rem - rc * per_chunk;
        jb = rem2 / groups_per_slice;
        grp = rem2 - jb * groups_per_slice;
    }
    if (r.counts && si - seg_begin >= r.counts[kCntGather]) return;   // device-built routing
    const Seg sd = load_seg(r.seg, si);
    const int rb = rc * ROWS;                       // first segment row of the task
    const int n_rows = sd.n_rows() - rb;            // rows of the task, if positive
    if (n_rows <= 0) return;
    // rank tiles of each slice (none past the lane's slices)
    int ntj[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ntj[j] = j < g.n_slices ? (sd.rank(j) + 15) / 16 : 0;
    if (!tab) {
        const int t0 = grp * NG;
        if (t0 >= ntj[jb]) return;
        c0 = (jb > 0 ? ntj[0] : 0) + (jb > 1 ? ntj[1] : 0) + (jb > 2 ? ntj[2] : 0) + t0;
        cnt = min(NG, ntj[jb] - t0);
    }
    // tile i of the task: slice tj[i], rank tile tt[i]; the live ones
    // (i < nt_here) come first
    int tj[NG], tt[NG], nt_here = 0;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        int c = c0 + i, j = 0;
        if (c >= ntj[0]) {
            c -= ntj[0];
            j = 1;
            if (c >= ntj[1]) {
                c -= ntj[1];
                j = 2;
                if (c >= ntj[2]) {
                    c -= ntj[2];
                    j = 3;
                }
            }
        }
        const bool live = i < cnt && c < ntj[j];
        tj[i] = live ? j : 0;
        tt[i] = live ? c : 0;
        nt_here += live ? 1 : 0;
    }
    if (nt_here == 0) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int lb = lane >> 3, lc = lane & 7;        // load layout: row lb, chunk lc
    const int li = lane & 15, lg = lane >> 4;       // operand layout: row li, chunk lg

    // Row pointers of the load layout (8 rows of 128 bytes per instruction).
    // Rows past the segment read its last row and A rows past rank_pad the
    // last padded row: their products only reach outputs that are not stored.
    const uint16_t *xr[2 * RT];
#pragma unroll
    for (int i = 0; i < 2 * RT; ++i) {
        const int sr = rb + min(8 * i + lb, n_rows - 1);       // segment row
        const int tok = GATHER ? r.rows[sd.v_row() + sr] : sd.first_row() + sr;
        xr[i] = x + (int64_t)tok * ldx;
    }
    const uint16_t *a_slot = p.A + (int64_t)(sd.slot() - 1) * g.a_slot_stride;

    __shared__ uint4 lds[kShrinkParts][(RT + NG) * 16][8];   // per wave: x rows, then A rows
    uint4(*const lw)[8] = lds[wave];

    f32x4_t acc[RT][NG];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int nt = 0; nt < NG; ++nt) acc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // K-step pairs (64 elements) p = wave, wave + 4, ...; loads run DP pairs
    // ahead.  The loop is branch-free so the loads stay in flight: every load
    // has a valid (clamped) address, and pairs past h_in and the padding
    // pairs that round a wave's count up to a multiple of the depth multiply
    // zeros.  The loop is instantiated for the task's count of live rank
    // tiles NTH (the rank tiles past the segment's rank are neither loaded
    // nor multiplied), so no branch sits between its products: a branch per
    // product had every product wait for its own LDS read.
    constexpr int DP = 2;                           // K-step pairs of loads in flight
    const int n_pairs = (g.h_in + 63) / 64;
    const int my_steps = (n_pairs - wave + kShrinkParts - 1) / kShrinkParts;
    auto run = [&](auto nth_c) {
        constexpr int NTH = decltype(nth_c)::value;
        const uint16_t *ar[2 * NTH];
#pragma unroll
        for (int i = 0; i < 2 * NTH; ++i)
            ar[i] = a_slot + ((int64_t)tj[i / 2] * g.rank_pad +
                              min(16 * tt[i / 2] + 8 * (i % 2) + lb, g.rank_pad - 1)) * g.h_in;
        uint4 xs[DP][2 * RT], as[DP][2 * NTH];
        const uint4 zero = make_uint4(0, 0, 0, 0);
        auto load = [&](uint4 (&xt)[2 * RT], uint4 (&at)[2 * NTH], int step) {
            const int e = min((wave + kShrinkParts * step) * 64 + 8 * lc, g.h_in - 8);
#pragma unroll
            for (int i = 0; i < 2 * RT; ++i) xt[i] = ld16(xr[i] + e);
#pragma unroll
            for (int i = 0; i < 2 * NTH; ++i) at[i] = ld16(ar[i] + e);
        };
        auto mma = [&](const uint4 (&xt)[2 * RT], const uint4 (&at)[2 * NTH], int step) {
            // chunks past h_in are staged as zeros, in both operands
            const uint32_t m =
                (wave + kShrinkParts * step) * 64 + 8 * lc < g.h_in ? ~0u : 0u;
            auto keep = [&](uint4 w) { return make_uint4(w.x & m, w.y & m, w.z & m, w.w & m); };
#pragma unroll
            for (int i = 0; i < 2 * RT; ++i) {
                const int row = 8 * i + lb;
                lw[row][chunk_pos(row, lc)] = keep(xt[i]);
            }
#pragma unroll
            for (int i = 0; i < 2 * NTH; ++i) {
                const int row = 16 * RT + 8 * i + lb;
                lw[row][chunk_pos(row, lc)] = keep(at[i]);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int h = 0; h < 2; ++h) {             // the pair's two K-steps
                const int cq = 4 * h + lg;
                uint4 af[NTH];
#pragma unroll
                for (int nt = 0; nt < NTH; ++nt) {
                    const int row = 16 * (RT + nt) + li;
                    af[nt] = lw[row][chunk_pos(row, cq)];
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const int row = 16 * rt + li;
                    const uint4 xv = lw[row][chunk_pos(row, cq)];
                    uint4 xhi = xv, xlo = zero;
                    if constexpr (FP16X) split_f16x8(xv, xhi, xlo);
#pragma unroll
                    for (int nt = 0; nt < NTH; ++nt) {
                        acc[rt][nt] = mfma16x16x32(af[nt], xhi, acc[rt][nt]);
                        if constexpr (FP16X) acc[rt][nt] = mfma16x16x32(af[nt], xlo, acc[rt][nt]);
                    }
                }
            }
            // the next step's writes stay behind these reads
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        };
        // The scheduling fences keep every load group in source order, in the
        // first fill as in the loop, and each refill after the step that reads
        // the registers it overwrites.  The loads of a pass are then consumed
        // in the next pass and stay in flight across the loop's back edge.
#pragma unroll
        for (int st = 0; st < DP; ++st) {
            load(xs[st], as[st], st);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int base = 0; base < my_steps; base += DP) {
#pragma unroll
            for (int st = 0; st < DP; ++st) {
                mma(xs[st], as[st], base + st);
                __builtin_amdgcn_sched_barrier(0);
                load(xs[st], as[st], base + st + DP);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    if (nt_here >= NG) run(std::integral_constant<int, NG>{});
    else if constexpr (NG > 1) {
        if (nt_here == 1) run(std::integral_constant<int, 1>{});
        else if constexpr (NG > 2) {
            if (nt_here == 2) run(std::integral_constant<int, 2>{});
            else run(std::integral_constant<int, 3>{});
        }
    }

    // u = (S0 + S1) + (S2 + S3), one 16-rank tile at a time through the
    // staging LDS.  Lane l holds, per (rt, nt),
    // u^T[rank 16 nt + 4 lg + i][row 16 rt + li].
    static_assert(sizeof(lds) >= kShrinkParts * ROWS * 16 * sizeof(float),
                  "reduction tile fits the staging LDS");
    float(*const red)[ROWS][16] = reinterpret_cast<float(*)[ROWS][16]>(&lds[0][0][0]);
    static_assert(kShrinkParts == 4, "the combine below adds four parts");
    const int orow = threadIdx.x >> 2, ok4 = (threadIdx.x & 3) * 4;
    float *const vrow = v + (int64_t)(sd.v_row() + rb + orow) * g.v_stride + ok4;
#pragma unroll
    for (int nt = 0; nt < NG; ++nt) {
        if (nt >= nt_here) break;                   // the same for the whole workgroup
        const float scale = p.scale[sd.slot() * kMetaStride + tj[nt]];
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float4 d;
            d.x = acc[rt][nt][0];
            d.y = acc[rt][nt][1];
            d.z = acc[rt][nt][2];
            d.w = acc[rt][nt][3];
            *reinterpret_cast<float4 *>(&red[wave][16 * rt + li][4 * lg]) = d;
        }
        __syncthreads();
        if (orow < n_rows && orow < ROWS) {
            float4 u;
            float *uf = &u.x;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float t[kShrinkParts];
#pragma unroll
                for (int w = 0; w < kShrinkParts; ++w) t[w] = red[w][orow][ok4 + i];
                uf[i] = scale * ((t[0] + t[1]) + (t[2] + t[3]));
            }
            if (vsplit) {
                const float four[4] = {u.x, u.y, u.z, u.w};
                store_vsplit<4>(reinterpret_cast<uint16_t *>(v), vsplit, vsplit_groups(g.rank_pad),
                                sd.v_row() + rb + orow, tj[nt], 16 * tt[nt] + ok4, four);
            } else {
                *reinterpret_cast<float4 *>(vrow + tj[nt] * g.rank_pad + 16 * tt[nt]) = u;
            }
        }
    }
}

template <bool FP16X, int NG, int RT, bool GATHER>
__global__ __launch_bounds__(64 * kShrinkParts, 2) void k_shrink_mfma(
    LaneGeom g, PoolDev p, RoutingDev r, int n_tasks, int seg_begin, int groups_per_slice,
    const uint32_t *__restrict__ tab, const uint16_t *__restrict__ x, int64_t ldx,
    float *__restrict__ v, int vsplit)
{
    touch_args(n_tasks, g, p, r, ldx);
    // a table is laid out for the dispatch (word b is a task of XCD b % 8,
    // each XCD's heaviest first); the block-index tasks are grouped per XCD
    const int task = tab ? (int)blockIdx.x : xcd_task(blockIdx.x, n_tasks);
    shrink_mfma_task<FP16X, NG, RT, GATHER>(g, p, r, task, seg_begin, groups_per_slice, tab, x,
                                            ldx, v, vsplit);
}

// A task is one 128-column tile of one slice over a group of consecutive
// prefill segments.  The tile's B rows (128 outputs x 32*NK ranks, zero past
// the slot's rank) are staged in LDS once and kept while the slot stays the
// same, so a group that covers one prompt reads its B tile from HBM once.
// Wave w multiplies rows 16w .. 16w + 15 of each segment; with WAVES = 1 a
// workgroup is one wave and every segment has at most 16 rows (gather
// segments cut that small for batches of small (adapter, expert) groups, so
// no wave of a workgroup idles on an empty row block).
template <int NK, bool GATHER, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(WAVES == 1 ? (NK <= 2 ? 2 : 1) : NK == 1 ? 3 : NK <= 4 ? 2 : 1)))
void k_expand_mfma(LaneGeom g, PoolDev p, RoutingDev r, int n_tasks,
                                                      int seg_begin, int seg_end, int group,
                                                      int tiles_per_grp,
                                                      const float *__restrict__ v,
                                                      float *__restrict__ y, int64_t ldy)
{
    constexpr int NS = kMfmaExpandCols / 16;      // 16-column MFMA tiles of a task
    constexpr int COLS = kMfmaExpandCols;
    constexpr int LDT = COLS + 4;                 // padded LDS row of d
    constexpr int KR = 32 * NK;                   // staged ranks
    constexpr int LDB = KR + 8;                   // padded LDS row of B (bf16)
    constexpr int CPR = KR / 8;                   // 16-byte chunks per staged B row
    static_assert(COLS == 128, "two rows of y per wave instruction");
    touch_args(n_tasks, g, p, r, ldy);
    const int task = xcd_task(blockIdx.x, n_tasks);
    const int grp = task / tiles_per_grp;
    int j, tile;
    slice_tile<COLS>(g, task - grp * tiles_per_grp, j, tile);
    const int hj = pick4(g.h_out, j);
    const int col_off = pick4(g.col_off, j);
    const int64_t bt_off = pick4(g.bt_slice_off, j);
    const int o_base = tile * COLS;
    const int s_first = seg_begin + grp * group;
    int s_last = min(s_first + group, seg_end);
    if (r.counts) s_last = min(s_last, seg_begin + r.counts[kCntGather]);   // device-built routing
    if (s_first >= s_last) return;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int r0 = wave * 16;
    const int yc = o_base + 4 * (lane & 31);
    const bool yc_ok = yc < hj;

    __shared__ __align__(16) uint16_t bs[COLS][LDB];
    __shared__ __align__(16) float dt[WAVES][16][LDT];

    // y of this wave's 16 rows of a segment, two whole 128-column rows per
    // instruction: lane l takes row 2q + l/32, columns 4 * (l % 32) .. + 3.
    // Loads are branch-free: rows past the segment read one of its rows and
    // columns past the slice its last four columns (h_out is a multiple of 8);
    // only the stores are masked.
    auto y_row = [&](int q) { return r0 + 2 * q + (lane >> 5); };
    const int ycol = col_off + min(yc, hj - 4);
    // token row of this lane's y row q of segment sd
    auto y_tok = [&](Seg sd, int q) -> int {
        const int last = sd.n_rows() - 1;
        if constexpr (GATHER) {
            // the wave's 16 entries of the row table, through scalar loads
            // (entries past the segment are read but not used)
            typedef const __attribute__((address_space(4))) int32_t cint;
            cint *t = (cint *)(r.rows + sd.v_row() + r0);
            const int e0 = t[2 * q], e1 = t[2 * q + 1], first = t[0];
            return y_row(q) <= last ? ((lane >> 5) ? e1 : e0) : first;
        } else {
            return sd.first_row() + min(y_row(q), last);
        }
    };
    // v of row r0 + li, ranks 32 ks + 8 lg .. + 7 (raw; the rank and row
    // masks are applied when the rows are used).  The addresses stay inside
    // the row.
    auto load_v = [&](Seg sd, float4 (&vr)[2 * NK]) {
        const float *vrow = v + (int64_t)(sd.v_row() + min(r0 + li, sd.n_rows() - 1)) * g.v_stride +
                            j * g.rank_pad;
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
            const int kc = min(32 * ks + 8 * lg, g.rank_pad - 8);
            vr[2 * ks] = *reinterpret_cast<const float4 *>(vrow + kc);
            vr[2 * ks + 1] = *reinterpret_cast<const float4 *>(vrow + kc + 4);
        }
    };
    // Rows of the next segment that load while the current one is worked on:
    // y always, v too when it is small (up to 64 ranks).  v is loaded before
    // y since it is needed first and loads complete in issue order.
    constexpr bool kPrefetchV = NK <= 2;
    auto load_rows = [&](Seg sd, float4 (&yv)[8], float4 (&vr)[2 * NK]) {
        if constexpr (kPrefetchV) load_v(sd, vr);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            yv[q] = *reinterpret_cast<const float4 *>(y + (int64_t)y_tok(sd, q) * ldy + ycol);
    };

    int staged = 0;                               // slot whose B tile is in bs
    // B tile of a slot into bs: PER 16-byte chunks per thread, loaded in
    // batches (of up to 8, or 4) whose loads are all issued before the first
    // LDS write (a loop of load-then-write waited out one load latency per
    // chunk: eight for a rank-128 tile).  Every load reads a clamped address in the
    // slot's rows; chunks past the slice or the rank are written as zeros.
    constexpr int PER = COLS * CPR / (64 * WAVES);
    constexpr int BMAX = WAVES == 1 ? 4 : 8;    // the one-wave forms hold more registers
    constexpr int BATCH = PER < BMAX ? PER : BMAX;
    static_assert(PER % BATCH == 0, "whole batches");
    auto stage_b = [&](Seg sd) {           // uniform over the workgroup
        const int slot = sd.slot();
        if (slot == staged) return;
        const int rank = sd.rank(j);
        const uint16_t *Bn = p.Bn + (int64_t)(slot - 1) * g.bt_slot_stride + bt_off;
        __syncthreads();
#pragma unroll 1
        for (int b0 = 0; b0 < PER; b0 += BATCH) {
            uint4 w[BATCH];
#pragma unroll
            for (int i = 0; i < BATCH; ++i) {
                const int c = (int)threadIdx.x + (b0 + i) * 64 * WAVES;
                const int ol = c / CPR, kc = (c - ol * CPR) * 8;
                const int o = min(o_base + ol, hj - 1);
                w[i] = ld16(Bn + (int64_t)o * g.rank_pad + min(kc, g.rank_pad - 8));
            }
#pragma unroll
            for (int i = 0; i < BATCH; ++i) {
                const int c = (int)threadIdx.x + (b0 + i) * 64 * WAVES;
                const int ol = c / CPR, kc = (c - ol * CPR) * 8;
                const uint32_t m = (o_base + ol < hj && kc < rank) ? ~0u : 0u;
                *reinterpret_cast<uint4 *>(&bs[ol][kc]) =
                    make_uint4(w[i].x & m, w[i].y & m, w[i].z & m, w[i].w & m);
            }
        }
        __syncthreads();
        staged = slot;
    };
    // The one-wave form with up to 32 ranks also loads the next segment's B
    // tile into registers while the current segment is worked on (its
    // segments are mostly of different slots; LDS allows 2 waves per SIMD,
    // so the registers are there): CHL chunks of 16 bytes per lane.
    constexpr bool kPrefetchB = WAVES == 1 && NK == 1;
    constexpr int CHL = kPrefetchB ? COLS * CPR / 64 : 1;
    auto load_b_regs = [&](Seg sd, uint4 (&bq)[CHL]) {
        const int rank = sd.rank(j);
        const uint16_t *Bn =
            p.Bn + (int64_t)(sd.slot() - 1) * g.bt_slot_stride + bt_off;
#pragma unroll
        for (int i = 0; i < CHL; ++i) {
            const int c = lane + 64 * i;
            const int ol = c / CPR, kc = (c - ol * CPR) * 8;
            const int o = o_base + ol;
            bq[i] = (o < hj && kc < rank) ? ld16(Bn + (int64_t)o * g.rank_pad + kc)
                                          : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_b = [&](Seg sd, const uint4 (&bq)[CHL]) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < CHL; ++i) {
            const int c = lane + 64 * i;
            const int ol = c / CPR, kc = (c - ol * CPR) * 8;
            *reinterpret_cast<uint4 *>(&bs[ol][kc]) = bq[i];
        }
        __syncthreads();
        staged = sd.slot();
    };

    // One set of B registers suffices: a segment's prefetched tile goes to
    // LDS at the start of its step, before the next one is loaded.
    uint4 bq[CHL];

    // One segment: multiply with the rows loaded into (yv, vf) while the rows
    // of the next segment of the group load into (yn, vn) (and, with
    // kPrefetchB, its B tile into bq when its slot differs).
    auto step = [&](int si, Seg sd, float4 (&yv)[8], float4 (&vr)[2 * NK],
                    float4 (&yn)[8], float4 (&vn)[2 * NK]) {
        const bool act = r0 < sd.n_rows();
        if constexpr (!kPrefetchV)      // the group's first v loads with its first y
            if (act && si != s_first) load_v(sd, vr);
        if constexpr (kPrefetchB) {
            if (sd.slot() != staged) store_b(sd, bq);
        } else {
            stage_b(sd);
        }
        f32x4_t acc[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (act) {
            // v is zero past the rank and for rows past the segment; K-steps
            // past the rank multiply zeros and leave acc unchanged.
            const int rank = sd.rank(j);
            const bool row_ok = r0 + li < sd.n_rows();
#pragma unroll
            for (int ks = 0; ks < NK; ++ks) {
                const int kk = 32 * ks + 8 * lg;
                const float4 a = vr[2 * ks], b = vr[2 * ks + 1];
                const float t[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                float f[8];
#pragma unroll
                for (int m = 0; m < 8; ++m) f[m] = (row_ok && kk + m < rank) ? t[m] : 0.f;
                uint4 vhi, vlo;
                split_f32x8(f, vhi, vlo);
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const uint4 bv =
                        *reinterpret_cast<const uint4 *>(&bs[16 * s + li][32 * ks + 8 * lg]);
                    acc[s] = mfma16x16x32(bv, vhi, acc[s]);
                    acc[s] = mfma16x16x32(bv, vlo, acc[s]);
                }
            }
        }
        if (si + 1 < s_last) {
            const Seg nx = load_seg(r.seg, si + 1);
            if (r0 < nx.n_rows()) load_rows(nx, yn, vn);
            if constexpr (kPrefetchB)
                if (nx.slot() != sd.slot()) load_b_regs(nx, bq);
        }
        if (act) {
            // d of (row li, columns 16 s + 4 lg ..) -> LDS -> the y layout.
            // The first barrier keeps the previous segment's reads of dt
            // ahead of these writes.
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                float4 d;
                d.x = acc[s][0];
                d.y = acc[s][1];
                d.z = acc[s][2];
                d.w = acc[s][3];
                *reinterpret_cast<float4 *>(&dt[wave][li][16 * s + 4 * lg]) = d;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float4 d = *reinterpret_cast<const float4 *>(
                    &dt[wave][2 * q + (lane >> 5)][4 * (lane & 31)]);
                float4 o = yv[q];
                o.x += d.x;
                o.y += d.y;
                o.z += d.z;
                o.w += d.w;
                if (yc_ok && y_row(q) < sd.n_rows())
                    *reinterpret_cast<float4 *>(y + (int64_t)y_tok(sd, q) * ldy + ycol) = o;
            }
        }
    };

    // Two register sets alternate, so no set is copied while its loads are
    // in flight.
    float4 ya[8], yb[8];
    float4 va[2 * NK], vb[2 * NK];
    {
        const Seg sd = load_seg(r.seg, s_first);
        if (r0 < sd.n_rows()) {
            if constexpr (!kPrefetchV) load_v(sd, va);
            load_rows(sd, ya, va);
        }
        if constexpr (kPrefetchB) load_b_regs(sd, bq);
    }
    for (int si = s_first; si < s_last; si += 2) {
        step(si, load_seg(r.seg, si), ya, va, yb, vb);
        if (si + 1 >= s_last) break;
        step(si + 1, load_seg(r.seg, si + 1), yb, vb, ya, va);
    }
}

}  // namespace

template <int NG, int RT>
static void launch_shrink_t(bool fp16, bool gather, dim3 grid, hipStream_t s, const LaneGeom &g,
                            const PoolDev &p, const RoutingDev &r, int seg_begin, int groups,
                            const uint32_t *tab, const uint16_t *x, int64_t ldx, float *v,
                            int vsplit)
{
    const dim3 block(64 * kShrinkParts);
    if (fp16 && gather)
        hipLaunchKernelGGL((k_shrink_mfma<true, NG, RT, true>), grid, block, 0, s, g, p, r,
                           (int)grid.x, seg_begin, groups, tab, x, ldx, v, vsplit);
    else if (fp16)
        hipLaunchKernelGGL((k_shrink_mfma<true, NG, RT, false>), grid, block, 0, s, g, p, r,
                           (int)grid.x, seg_begin, groups, tab, x, ldx, v, vsplit);
    else if (gather)
        hipLaunchKernelGGL((k_shrink_mfma<false, NG, RT, true>), grid, block, 0, s, g, p, r,
                           (int)grid.x, seg_begin, groups, tab, x, ldx, v, vsplit);
    else
        hipLaunchKernelGGL((k_shrink_mfma<false, NG, RT, false>), grid, block, 0, s, g, p, r,
                           (int)grid.x, seg_begin, groups, tab, x, ldx, v, vsplit);
}

template <int NG>
static void launch_shrink_ng(int rt, bool fp16, bool gather, dim3 grid, hipStream_t s,
                             const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                             int seg_begin, int groups, const uint16_t *x, int64_t ldx, float *v,
                             int vsplit)
{
    if (rt == 1)
        launch_shrink_t<NG, 1>(fp16, gather, grid, s, g, p, r, seg_begin, groups, nullptr, x,
                               ldx, v, vsplit);
    else if (rt == 2)
        launch_shrink_t<NG, 2>(fp16, gather, grid, s, g, p, r, seg_begin, groups, nullptr, x,
                               ldx, v, vsplit);
    else
        launch_shrink_t<NG, 4>(fp16, gather, grid, s, g, p, r, seg_begin, groups, nullptr, x,
                               ldx, v, vsplit);
}

hipError_t launch_shrink_mfma(const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                              bool gather, int seg_begin, int n_seg, int nt_per_slice,
                              const void *x, int64_t ldx, float *v, int vsplit, hipStream_t s,
                              const uint32_t *tab, int n_tab, int tab_tiles, int tab_rows)
{
    if (n_seg <= 0) return hipSuccess;
    const uint16_t *xp = static_cast<const uint16_t *>(x);
    const bool fp16 = g.x_fp16 != 0;
    if (tab && n_tab > 0) {
        // host-built tasks of whole segments: the smallest tile and row
        // counts that cover the table (fewer registers, more workgroups per
        // compute unit)
        static_assert(kShrinkMaxTiles == 4 && kRowTiles == 4, "template sizes 1, 2, 4");
        const int ng = tab_tiles <= 1 ? 1 : tab_tiles <= 2 ? 2 : 4;
        const int rt = tab_rows <= 16 ? 1 : tab_rows <= 32 ? 2 : 4;
        const dim3 grid((unsigned)n_tab);
        auto go = [&](auto ng_c) {
            constexpr int NG = decltype(ng_c)::value;
            if (rt == 1)
                launch_shrink_t<NG, 1>(fp16, gather, grid, s, g, p, r, seg_begin, 0, tab, xp, ldx,
                                       v, vsplit);
            else if (rt == 2)
                launch_shrink_t<NG, 2>(fp16, gather, grid, s, g, p, r, seg_begin, 0, tab, xp, ldx,
                                       v, vsplit);
            else
                launch_shrink_t<NG, 4>(fp16, gather, grid, s, g, p, r, seg_begin, 0, tab, xp, ldx,
                                       v, vsplit);
        };
        if (ng == 1) go(std::integral_constant<int, 1>{});
        else if (ng == 2) go(std::integral_constant<int, 2>{});
        else go(std::integral_constant<int, 4>{});
        return hipGetLastError();
    }
    // Task shape: whole segments and up to 4 rank tiles (x and A read the
    // fewest times), made finer -- rows first, then ranks -- while the grid
    // is under kShrinkMinBlocks workgroups.
    int ng = nt_per_slice <= 1 ? 1 : nt_per_slice <= 2 ? 2 : 4, rt = kRowTiles;
    auto blocks_of = [&](int ng_, int rt_) {
        return (int64_t)n_seg * g.n_slices * ((nt_per_slice + ng_ - 1) / ng_) * (kRowTiles / rt_);
    };
    while (blocks_of(ng, rt) < kShrinkMinBlocks && (ng > 1 || rt > 1)) {
        if (rt > 1 && (rt >= ng || ng == 1)) rt /= 2;
        else ng /= 2;
    }
    const int groups = (nt_per_slice + ng - 1) / ng;
    const int64_t blocks = blocks_of(ng, rt);
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    if (ng == 1)
        launch_shrink_ng<1>(rt, fp16, gather, grid, s, g, p, r, seg_begin, groups, xp, ldx, v,
                                vsplit);
    else if (ng == 2)
        launch_shrink_ng<2>(rt, fp16, gather, grid, s, g, p, r, seg_begin, groups, xp, ldx, v,
                                vsplit);
    else
        launch_shrink_ng<4>(rt, fp16, gather, grid, s, g, p, r, seg_begin, groups, xp, ldx, v,
                                vsplit);
    return hipGetLastError();
}

template <int NK>
static void launch_expand_nk(bool gather, bool one_wave, dim3 grid, hipStream_t s,
                             const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                             int seg_begin, int seg_end, int group, int tiles_per_grp,
                             const float *v, float *y, int64_t ldy)
{
    if (gather && one_wave)
        hipLaunchKernelGGL((k_expand_mfma<NK, true, 1>), grid, dim3(64), 0, s, g, p, r,
                           (int)grid.x, seg_begin, seg_end, group, tiles_per_grp, v, y, ldy);
    else if (gather)
        hipLaunchKernelGGL((k_expand_mfma<NK, true, 4>), grid, dim3(256), 0, s, g, p, r,
                           (int)grid.x, seg_begin, seg_end, group, tiles_per_grp, v, y, ldy);
    else
        hipLaunchKernelGGL((k_expand_mfma<NK, false, 4>), grid, dim3(256), 0, s, g, p, r,
                           (int)grid.x, seg_begin, seg_end, group, tiles_per_grp, v, y, ldy);
}

hipError_t launch_expand_mfma(const LaneGeom &g, const PoolDev &p, const RoutingDev &r,
                              bool gather, int seg_begin, int n_seg, int group, int max_rank,
                              int max_seg_rows, const float *v, float *y, int64_t ldy,
                              hipStream_t s)
{
    if (n_seg <= 0) return hipSuccess;
    if (group < 1 || max_rank < 1 || max_rank > 256) return hipErrorInvalidValue;
    if (max_seg_rows < 1 || max_seg_rows > kPrefillSegRows) return hipErrorInvalidValue;
    const int64_t groups = (n_seg + group - 1) / group;
    // only live tiles: ceil(h_j / 128) for each slice j
    const int tiles_per_grp = lane_tiles(g, kMfmaExpandCols);
    const int64_t blocks = groups * tiles_per_grp;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    const int seg_end = seg_begin + n_seg;
    const int nk = (max_rank + 31) / 32;
    // one wave per workgroup when no gather segment has more than 16 rows
    const bool one_wave = gather && max_seg_rows <= 16;
    if (nk <= 1)
        launch_expand_nk<1>(gather, one_wave, grid, s, g, p, r, seg_begin, seg_end, group,
                            tiles_per_grp, v, y, ldy);
    else if (nk <= 2)
        launch_expand_nk<2>(gather, one_wave, grid, s, g, p, r, seg_begin, seg_end, group,
                            tiles_per_grp, v, y, ldy);
    else if (nk <= 4)
        launch_expand_nk<4>(gather, one_wave, grid, s, g, p, r, seg_begin, seg_end, group,
                            tiles_per_grp, v, y, ldy);
    else
        launch_expand_nk<8>(gather, one_wave, grid, s, g, p, r, seg_begin, seg_end, group,
                            tiles_per_grp, v, y, ldy);
    return hipGetLastError();
}

}  // namespace lora
