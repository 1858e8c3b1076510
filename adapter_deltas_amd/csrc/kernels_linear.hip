// The base projection with the delta in its accumulator (gfx950).
//
// y[t] = x[t] W^T for every row t of the batch, and for a row t with adapter
// slot s != 0 the delta of each slice is added to the fp32 accumulator before
// the single store of y (TensorFold PR #47, third commit message and PR body
// "What this changes": the delta lands in the projection's fp32 partial sum,
// before the cross-rank reduction).  The shrink's v is made by the shrink
// kernels beforehand, in the routing's active-row order.
//
// Product:  v_mfma_f32_16x16x32_bf16 with W rows as the first operand and x
//           rows as the second, so lane l of a 16 x 16 result holds four
//           consecutive output features (4 (l / 16) .. + 3) of one row
//           (l % 16) and stores them as one 16-byte write.  Each output sums
//           its K-steps of 32 in ascending order, from zero.
// Delta:    as K-steps after the product's, in the same accumulator: per
//           distinct slot of the tile's rows, slice and group of 16 ranks,
//           one 32-wide step of B rows against (v_hi, v_lo) of those ranks
//           (v = v_hi + v_lo, both bf16, written so by the shrink), with every
//           other row, column and rank read as zero.  Each output sums its own
//           product terms, then its own delta steps in a fixed order, plus
//           steps of exact zeros.
// A row's bits depend on its own x row, W and its adapter only.
#include "kernels_common.h"

#include <algorithm>
#include <type_traits>
#include <utility>

namespace lora {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16x16x32(uint4 a, uint4 b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int kBK = 64;            // K elements per tile: 8 chunks of 16 bytes per row
constexpr int kChunks = kBK / 8;
constexpr int kThreads = 256;      // 4 waves, 2 x 2 over (features, rows)

// Position of 16-byte chunk c of LDS row r: rows are 128 bytes, and the XOR
// puts the chunks 8 consecutive lanes read (rows r .. r + 7, one chunk
// index) in 8 different bank groups.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 7); }

// A tile is BN output features x BM rows of the batch.  Each XCD takes a
// consecutive range of tasks (xcd_task), and inside it tasks go through the
// tiles in groups of kGroupM row tiles: the group's row tiles for one feature
// tile, then for the next, so the W and x tiles that run at the same time on
// an XCD are few and stay in its L2.
//
// Main loop: K-tiles of kBK; the global loads of tile kt + D are issued while
// tile kt is multiplied (D register sets in flight), then each set is moved to
// one of two LDS buffers, with its masks applied.  The loop is branch-free: it
// runs a multiple of D tiles, and a tile past the last loads zeros.
//
// The delta, as K-steps after the product's: for each distinct slot s among
// the tile's rows (ascending), each slice j the tile's columns touch and each
// group k of 16 ranks the slot has on that slice, one step of 32: W rows
// B[s][j][o][16 k ..] (output-major) for both halves, x rows v_hi of those
// ranks in the first half and v_lo in the second, from the split v the shrink
// wrote.  Two steps make a K-tile.  A row of another slot, a column of another
// slice and a rank past the slot's rank read as zero, so each output's sum
// gets exactly its own row's delta terms, always at the same positions of the
// same steps whatever the other rows are, and exact zeros from the rest.
constexpr int kGroupM = 8;

__device__ __forceinline__ void tile_of(int task, int n_tiles, int m_tiles, int &tn, int &tm)
{
    const int per_group = kGroupM * n_tiles;
    const int grp = task / per_group;
    const int in = task - grp * per_group;
    const int gm = min(kGroupM, m_tiles - grp * kGroupM);   // row tiles in this group
    tn = in / gm;
    tm = grp * kGroupM + (in - tn * gm);
}

// f(integral_constant<int, i>) for i = 0 .. N - 1, in order, at compile time.
template <class F, int... I>
__device__ __forceinline__ void unroll_seq(F f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void unroll(F f)
{
    unroll_seq(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ int wave_min(int v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m));
    return v;
}

// One delta step in a word: slot (17 bits), slice j (2), 16-rank group k (4),
// the slot's rank on slice j (9 bits, <= 256).
__device__ __forceinline__ uint32_t step_word(int slot, int j, int k, int rank)
{
    return (uint32_t)slot | ((uint32_t)j << 17) | ((uint32_t)k << 19) | ((uint32_t)rank << 23);
}

__device__ __forceinline__ int pick_rank(const int4 &rk, int j)
{
    return j == 0 ? rk.x : j == 1 ? rk.y : j == 2 ? rk.z : rk.w;
}

// The chunk, or zeros (masks, so no select of aggregates goes through memory).
__device__ __forceinline__ uint4 keep_if(uint4 w, bool ok)
{
    const uint32_t m = ok ? ~0u : 0u;
    return make_uint4(w.x & m, w.y & m, w.z & m, w.w & m);
}

// Zeroes the bf16 values of a 16-byte chunk from position n_ok on (0..8).
__device__ __forceinline__ uint4 keep_first(uint4 w, int n_ok)
{
    uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = 2 * i < n_ok ? 0xffffu : 0u;
        const uint32_t hi = 2 * i + 1 < n_ok ? 0xffff0000u : 0u;
        q[i] &= lo | hi;
    }
    return make_uint4(q[0], q[1], q[2], q[3]);
}

template <int BN, int BM, bool DELTA>
__global__ __launch_bounds__(kThreads, 2) void k_linear(LaneGeom g, PoolDev p, LinearArgs a,
                                                      int n_tasks, int n_tiles, int m_tiles)
{
    constexpr int NI = BN / 32, MI = BM / 32;              // 16-wide tiles per wave
    constexpr int ROWS = BN + BM;                          // LDS rows per K-tile
    constexpr int NL = ROWS * kChunks / kThreads;          // 16-byte loads per thread
    // K-tiles of loads in flight (64 x 64 tiles on decode_mix QKV, per call:
    // 3 -> 40.4 us, 4 -> 39.2, 6 -> 41.9, 8 -> 41.4: the tile's L2 traffic,
    // not its loads in flight, sets the time)
    constexpr int D = NL <= 4 ? 3 : 2;
    constexpr int LDT = BN + 4;                            // padded row of the output tile
    constexpr int CPL = BN / 64;                           // epilogue columns per lane
    constexpr int RPW = BM / (kThreads / 64);              // epilogue rows per wave
    static_assert(ROWS * kChunks % kThreads == 0, "loads tile the threads");
    static_assert(CPL == 1 || CPL == 2, "64 or 128 columns");
    static_assert(RPW <= 64 && BM <= 128, "one lane per epilogue row");
    constexpr int kStageBytes = 2 * ROWS * kChunks * 16;
    constexpr int kTileBytes = BM * LDT * 4;
    __shared__ __align__(16) unsigned char smem[kStageBytes > kTileBytes ? kStageBytes
                                                                         : kTileBytes];
    uint4(*const lds)[ROWS][kChunks] = reinterpret_cast<uint4(*)[ROWS][kChunks]>(smem);
    float(*const tile)[LDT] = reinterpret_cast<float(*)[LDT]>(smem);
    // the tile's delta steps (see step_word), and their count
    __shared__ uint32_t d_step[DELTA ? kLinearMaxSteps : 1];
    __shared__ int d_count;

    int tn, tm;
    tile_of(xcd_task(blockIdx.x, n_tasks), n_tiles, m_tiles, tn, tm);
    const int n0 = tn * BN, m0 = tm * BM;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wn = wave >> 1, wm = wave & 1;

    // The epilogue rows of this wave are the RPW consecutive tile rows
    // wave * RPW + i; lane i < RPW holds that row's token.
    const int e_row0 = wave * RPW;
    int my_t = 0;
    {
        const int m = m0 + e_row0 + lane;
        if (lane < RPW && m < a.M) my_t = a.rows ? a.rows[m] : m;
    }

    // Load layout: thread tid loads chunk tid % 8 of tile rows tid / 8 + 32 i.
    // Rows past N or M read the last valid row; their products reach only
    // outputs that are not stored.
    const int lc = tid & 7;
    const uint16_t *src[NL];
    int lrow[NL];
    int xslot[NL];          // delta: the slot of the x row (0 for W rows and base rows)
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int r = (tid >> 3) + 32 * i;
        lrow[i] = r;
        xslot[i] = 0;
        if (r < BN) {
            src[i] = a.W + (int64_t)min(n0 + r, a.N - 1) * a.ldw;
        } else {
            const int m = min(m0 + r - BN, a.M - 1);
            const int t = a.rows ? a.rows[m] : m;
            src[i] = a.x + (int64_t)t * a.ldx;
            if constexpr (DELTA)
                if (m0 + r - BN < a.n_delta) xslot[i] = a.row_meta[4 * (m0 + r - BN)];
        }
    }
    const int KT = (a.K + kBK - 1) / kBK;

    uint4 st[D][NL];
    // Product tiles: loads read a clamped address; masks are applied when a
    // set is written to LDS, so nothing waits for a load before it is needed.
    auto load_base = [&](uint4 (&dst)[NL], int kt) __attribute__((always_inline)) {
        const int ec = min(kt * kBK + lc * 8, a.K - 8);
#pragma unroll
        for (int i = 0; i < NL; ++i) dst[i] = ld16(src[i] + ec);
    };
    // The first product tiles are in flight while the slots are found.
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (d < KT) load_base(st[d], d);

    // Delta steps of the tile: its slices [j_lo, j_hi], distinct slots, and
    // per (slot, slice) one step per 16 ranks.
    auto slice_of = [&](int col) __attribute__((always_inline)) {
        return (g.n_slices > 1 && col >= g.col_off[1]) + (g.n_slices > 2 && col >= g.col_off[2]) +
               (g.n_slices > 3 && col >= g.col_off[3]);
    };
    const int j_lo = slice_of(n0), j_hi = slice_of(min(n0 + BN - 1, a.N - 1));
    int n_steps = 0;
    if constexpr (DELTA) {
        if (wave == 0) {
            // each lane holds the slots and ranks of rows lane and lane + 64,
            // from the routing's per-row table (one load each)
            int sa = 0, sb = 0;
            int4 ra = make_int4(0, 0, 0, 0), rb = make_int4(0, 0, 0, 0);
            auto unpack = [](int4 w, int &slot, int4 &rk) {
                slot = w.x;
                rk = make_int4(w.y & 0xffff, (int)((uint32_t)w.y >> 16), w.z & 0xffff,
                               (int)((uint32_t)w.z >> 16));
            };
            {
                const int ma = m0 + lane, mb = m0 + lane + 64;
                if (lane < BM && ma < a.n_delta)
                    unpack(*reinterpret_cast<const int4 *>(a.row_meta + 4 * ma), sa, ra);
                if (lane + 64 < BM && mb < a.n_delta)
                    unpack(*reinterpret_cast<const int4 *>(a.row_meta + 4 * mb), sb, rb);
            }
            // the distinct nonzero slots, ascending, by repeated minimum; the
            // steps of each are written at once, lane l writing its step l
            int last = 0, base = 0;
            for (;;) {
                const int c = wave_min(min(sa > last ? sa : INT32_MAX, sb > last ? sb : INT32_MAX));
                if (c == INT32_MAX) break;
                const uint64_t ha = __builtin_amdgcn_ballot_w64(sa == c);
                const uint64_t hb = __builtin_amdgcn_ballot_w64(sb == c);
                int4 rk;
                if (ha) {
                    const int l = (int)__builtin_ctzll(ha);
                    rk = make_int4(__builtin_amdgcn_readlane(ra.x, l), __builtin_amdgcn_readlane(ra.y, l),
                                   __builtin_amdgcn_readlane(ra.z, l), __builtin_amdgcn_readlane(ra.w, l));
                } else {
                    const int l = (int)__builtin_ctzll(hb);
                    rk = make_int4(__builtin_amdgcn_readlane(rb.x, l), __builtin_amdgcn_readlane(rb.y, l),
                                   __builtin_amdgcn_readlane(rb.z, l), __builtin_amdgcn_readlane(rb.w, l));
                }
                // lane l: step l of this slot (slice j, group k), at most 4 x 16
                int rest = lane, j = -1, k = 0, rank = 0;
                for (int jj = j_lo; jj <= j_hi; ++jj) {
                    const int rj = pick_rank(rk, jj), nk = (rj + 15) / 16;
                    if (j < 0 && rest < nk) {
                        j = jj;
                        k = rest;
                        rank = rj;
                    }
                    rest -= nk;
                }
                if (j >= 0 && base + lane < kLinearMaxSteps)
                    d_step[base + lane] = step_word(c, j, k, rank);
                for (int jj = j_lo; jj <= j_hi; ++jj) base += (pick_rank(rk, jj) + 15) / 16;
                last = c;
            }
            if (lane == 0) d_count = min(base, kLinearMaxSteps);
        }
        __syncthreads();
        n_steps = __builtin_amdgcn_readfirstlane(d_count);
    }
    const int T_d = (n_steps + 1) / 2;       // delta K-tiles, two steps each
    const int KT_all = KT + T_d;
    const int G = vsplit_groups(g.rank_pad);
    const int vs_len = g.n_slices * G * 32;
    const uint16_t *vs = reinterpret_cast<const uint16_t *>(a.v);

    // per-slice widths and offsets, selected by slice below
    const int hj_[4] = {g.h_out[0], g.h_out[1], g.h_out[2], g.h_out[3]};
    const int cj_[4] = {g.col_off[0], g.col_off[1], g.col_off[2], g.col_off[3]};
    const int64_t bo_[4] = {g.bt_slice_off[0], g.bt_slice_off[1], g.bt_slice_off[2],
                            g.bt_slice_off[3]};
    auto sel = [](int j, auto v0, auto v1, auto v2, auto v3) __attribute__((always_inline)) {
        return j == 0 ? v0 : j == 1 ? v1 : j == 2 ? v2 : v3;
    };

    // This thread's 16 bytes of a delta tile: step h of its two, chunk q of
    // the step's four (ranks 8 (q & 1) .., v_hi for q < 2, v_lo after).
    // Past the last step: slot 0 (reads any valid address, moves zeros).
    const int h = lc >> 2, q = lc & 3;
    struct Step { int s, j, k, rank; };
    auto step_of = [&](int kt) __attribute__((always_inline)) {
        const int si = 2 * (kt - KT) + h;
        const uint32_t w = si < n_steps ? d_step[si] : 0u;
        return Step{(int)(w & 0x1ffffu), (int)((w >> 17) & 3u), (int)((w >> 19) & 15u),
                    (int)(w >> 23)};
    };

    auto load = [&](uint4 (&dst)[NL], int kt) __attribute__((always_inline)) {
        if (kt < KT || kt >= KT_all) {           // the product's tile (or past the last)
            load_base(dst, kt);
        } else {
            const Step dt = step_of(kt);
            const int hj = sel(dt.j, hj_[0], hj_[1], hj_[2], hj_[3]);
            const int cj = sel(dt.j, cj_[0], cj_[1], cj_[2], cj_[3]);
            const int64_t bo = sel(dt.j, bo_[0], bo_[1], bo_[2], bo_[3]);
            const uint16_t *bn = p.Bn + (int64_t)(max(dt.s, 1) - 1) * g.bt_slot_stride + bo +
                                 16 * dt.k + 8 * (q & 1);
            const uint16_t *vc = vs + (dt.j * G + dt.k) * 32 + 8 * q;
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int r = lrow[i];
                if (r < BN) {
                    const int ol = min(max(n0 + r - cj, 0), hj - 1);
                    dst[i] = ld16(bn + (int64_t)ol * g.rank_pad);
                } else {
                    const int m = min(m0 + r - BN, a.n_delta - 1);
                    dst[i] = ld16(vc + (int64_t)m * vs_len);
                }
            }
        }
    };
    auto store = [&](const uint4 (&from)[NL], int kt, int buf) __attribute__((always_inline)) {
        if (kt < KT) {
            const bool ok = kt * kBK + lc * 8 < a.K;   // K is a multiple of 8: whole chunks
#pragma unroll
            for (int i = 0; i < NL; ++i)
                lds[buf][lrow[i]][swz(lrow[i], lc)] = keep_if(from[i], ok);
        } else if (kt < KT_all) {
            const Step dt = step_of(kt);
            const int hj = sel(dt.j, hj_[0], hj_[1], hj_[2], hj_[3]);
            const int cj = sel(dt.j, cj_[0], cj_[1], cj_[2], cj_[3]);
            const int kb = 16 * dt.k + 8 * (q & 1);        // first rank of this chunk
            const bool live = dt.s != 0;
            const int n_ok = min(max(dt.rank - kb, 0), 8);
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int r = lrow[i];
                uint4 w;
                if (r < BN) {
                    const int ol = n0 + r - cj;
                    const bool ok = live && n0 + r < a.N && ol >= 0 && ol < hj && kb < dt.rank;
                    w = keep_if(from[i], ok);
                } else {
                    const bool ok = live && m0 + r - BN < a.n_delta && xslot[i] == dt.s;
                    w = keep_first(from[i], ok ? n_ok : 0);
                }
                lds[buf][r][swz(r, lc)] = w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < NL; ++i)
                lds[buf][lrow[i]][swz(lrow[i], lc)] = make_uint4(0, 0, 0, 0);
        }
    };

    f32x4_t acc[NI][MI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) acc[ni][mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int li = lane & 15, lg = lane >> 4;
    auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            const int cq = ks * 4 + lg;
            uint4 wf[NI], xf[MI];
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                const int r = wn * (BN / 2) + 16 * ni + li;
                wf[ni] = lds[buf][r][swz(r, cq)];
            }
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const int r = BN + wm * (BM / 2) + 16 * mi + li;
                xf[mi] = lds[buf][r][swz(r, cq)];
            }
#pragma unroll
            for (int ni = 0; ni < NI; ++ni)
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
                    acc[ni][mi] = mfma16x16x32(wf[ni], xf[mi], acc[ni][mi]);
        }
    };

    // Register set kt % D holds K-tile kt from its load until its move to LDS;
    // the loop is unrolled by D so every set is named at compile time.
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (d >= KT) load(st[d], d);
    store(st[0], 0, 0);
    __syncthreads();
    // Product iterations whose loads and moves are all product tiles run a
    // loop with no branch in it; the last ones and the delta tiles follow.
    auto step_base = [&](auto slot, int kt) __attribute__((always_inline)) {
        constexpr int S = decltype(slot)::value;
        load_base(st[S], kt + D);
        __builtin_amdgcn_sched_barrier(0);
        compute(kt & 1);
        __builtin_amdgcn_sched_barrier(0);
        const bool ok = (kt + 1) * kBK + lc * 8 < a.K;
#pragma unroll
        for (int i = 0; i < NL; ++i)
            lds[(kt + 1) & 1][lrow[i]][swz(lrow[i], lc)] = keep_if(st[(S + 1) % D][i], ok);
        __syncthreads();
    };
    auto step = [&](auto slot, int kt) __attribute__((always_inline)) {
        constexpr int S = decltype(slot)::value;
        load(st[S], kt + D);
        __builtin_amdgcn_sched_barrier(0);
        compute(kt & 1);
        __builtin_amdgcn_sched_barrier(0);
        store(st[(S + 1) % D], kt + 1, (kt + 1) & 1);
        __syncthreads();
    };
    int kt = 0;
    for (; kt + 2 * D <= KT; kt += D) {
        unroll<D>([&](auto c) __attribute__((always_inline)) { step_base(c, kt + c.value); });
    }
    const int KTD = (KT_all + D - 1) / D * D;
    for (; kt < KTD; kt += D) {
        unroll<D>([&](auto c) __attribute__((always_inline)) { step(c, kt + c.value); });
    }

    // Accumulator tile to LDS: lane holds, per (ni, mi), outputs
    // 16 ni + 4 lg + i (i = 0..3) of tile row 16 mi + li of its wave's quarter.
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int r = wm * (BM / 2) + 16 * mi + li;
            const int c = wn * (BN / 2) + 16 * ni + 4 * lg;
            *reinterpret_cast<float4 *>(&tile[r][c]) =
                make_float4(acc[ni][mi][0], acc[ni][mi][1], acc[ni][mi][2], acc[ni][mi][3]);
        }
    __syncthreads();

    // Rows: lane covers columns o = n0 + CPL lane .. + CPL - 1; every row of
    // the tile is stored once, whole 256- or 512-byte row pieces per wave.
    const int oc = CPL * lane;
    const int o = n0 + oc;
    const int n_rows = max(0, min(RPW, a.M - (m0 + e_row0)));   // valid rows of the wave
    if (o < a.N) {
        for (int r = 0; r < n_rows; ++r) {
            const int t = __builtin_amdgcn_readlane(my_t, r);
            float *yp = a.y + (int64_t)t * a.ldy + o;
            if constexpr (CPL == 2)
                *reinterpret_cast<float2 *>(yp) =
                    make_float2(tile[e_row0 + r][oc], tile[e_row0 + r][oc + 1]);
            else
                *yp = tile[e_row0 + r][oc];
        }
    }
}

template <int BN, int BM>
void launch_t(const LaneGeom &g, const PoolDev &p, const LinearArgs &a, hipStream_t s)
{
    const int n_tiles = (a.N + BN - 1) / BN, m_tiles = (a.M + BM - 1) / BM;
    const int n_tasks = n_tiles * m_tiles;
    if (a.n_delta > 0)
        hipLaunchKernelGGL((k_linear<BN, BM, true>), dim3(n_tasks), dim3(kThreads), 0, s, g, p,
                           a, n_tasks, n_tiles, m_tiles);
    else
        hipLaunchKernelGGL((k_linear<BN, BM, false>), dim3(n_tasks), dim3(kThreads), 0, s, g,
                           p, a, n_tasks, n_tiles, m_tiles);
}


// The largest tile that still gives the chip at least two workgroups per
// CU; small batches (decode) take 64 x 64 tiles.
constexpr int64_t kWantTasks = 512;
int64_t linear_tasks(int64_t M, int64_t N, int bn, int bm)
{
    return ((N + bn - 1) / bn) * ((M + bm - 1) / bm);
}

}  // namespace

int linear_tile_rows(int64_t M, int64_t N)
{
    return linear_tasks(M, N, 128, 128) >= kWantTasks ? 128 : 64;
}

hipError_t launch_linear(const LaneGeom &g, const PoolDev &p, const LinearArgs &a,
                         hipStream_t s)
{
    if (a.M <= 0) return hipSuccess;
    if (a.K < 8 || a.K % 8 || a.N < 8 || a.N % 8) return hipErrorInvalidValue;
    if (linear_tasks(a.M, a.N, 64, 64) > INT32_MAX) return hipErrorInvalidConfiguration;
    if (linear_tasks(a.M, a.N, 128, 128) >= kWantTasks) launch_t<128, 128>(g, p, a, s);
    else if (linear_tasks(a.M, a.N, 128, 64) >= kWantTasks) launch_t<128, 64>(g, p, a, s);
    else launch_t<64, 64>(g, p, a, s);
    return hipGetLastError();
}

}  // namespace lora
