// The base projection with the delta in its epilogue (gfx950).
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
// Delta:    for each 16-row group and slot, d^T[o][t] = sum over rank steps of
//           32 (ascending, from zero) of two MFMAs, B rows times v_hi then B
//           rows times v_lo, with v = v_hi + v_lo split into bf16 (nearest
//           even); then y = acc + d.  That is the prefill expand's arithmetic,
//           so on a row the routing sends to the matrix cores (prefill and
//           gather rows) the result equals lora_delta_apply applied to this
//           kernel's base product, bit for bit.  A 16-column group that
//           straddles a slice edge (slice widths are multiples of 8, not 16)
//           takes an fp32 fma chain over the ranks instead.
// A row's bits depend on its own x row, W and its adapter only.
#include "kernels_common.h"

#include <algorithm>
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
// one of two LDS buffers.  The loop is branch-free: it runs a multiple of D
// tiles, and a tile past K loads zeros (adding exact zeros to every sum).
// Epilogue: the accumulator tile goes through LDS to a row layout; wave w then
// takes rows w, w + 4, ... and, per row, its lanes take the tile's columns
// (CPL consecutive columns each), adding the row's delta with B^T loaded
// coalesced along the columns.  Each row's token, slot and ranks are loaded
// into the wave's lanes when the kernel starts and read back with readlane.
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

template <int BN, int BM, bool DELTA>
__global__ __launch_bounds__(kThreads) void k_linear(LaneGeom g, PoolDev p, LinearArgs a,
                                                      int n_tasks, int n_tiles, int m_tiles)
{
    constexpr int NI = BN / 32, MI = BM / 32;              // 16-wide tiles per wave
    constexpr int ROWS = BN + BM;                          // LDS rows per K-tile
    constexpr int NL = ROWS * kChunks / kThreads;          // 16-byte loads per thread
    constexpr int D = NL <= 4 ? 3 : 2;                     // K-tiles of loads in flight
    constexpr int LDT = BN + 4;                            // padded row of the output tile
    constexpr int CPL = BN / 64;                           // epilogue columns per lane
    constexpr int RPW = BM / (kThreads / 64);              // epilogue rows per wave
    static_assert(ROWS * kChunks % kThreads == 0, "loads tile the threads");
    static_assert(CPL == 1 || CPL == 2, "64 or 128 columns");
    static_assert(RPW <= 64, "one lane per epilogue row");
    constexpr int kStageBytes = 2 * ROWS * kChunks * 16;
    constexpr int kTileBytes = BM * LDT * 4;
    __shared__ __align__(16) unsigned char smem[kStageBytes > kTileBytes ? kStageBytes
                                                                         : kTileBytes];
    uint4(*const lds)[ROWS][kChunks] = reinterpret_cast<uint4(*)[ROWS][kChunks]>(smem);
    float(*const tile)[LDT] = reinterpret_cast<float(*)[LDT]>(smem);

    int tn, tm;
    tile_of(xcd_task(blockIdx.x, n_tasks), n_tiles, m_tiles, tn, tm);
    const int n0 = tn * BN, m0 = tm * BM;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wn = wave >> 1, wm = wave & 1;

    // The slot and ranks of the rows this lane holds in the accumulator
    // layout (row 16 mi + li of the wave's row half), for the delta.
    int ms[MI];
    int4 mrk[MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
        ms[mi] = 0;
        mrk[mi] = make_int4(0, 0, 0, 0);
        if constexpr (DELTA) {
            const int m = m0 + wm * (BM / 2) + 16 * mi + (lane & 15);
            if (m < a.n_delta) {
                ms[mi] = a.tok_slot[a.rows ? a.rows[m] : m];
                mrk[mi] = *reinterpret_cast<const int4 *>(p.rank + ms[mi] * kMetaStride);
            }
        }
    }

    // The epilogue rows of this wave are the RPW consecutive tile rows
    // wave * RPW + i; lane i < RPW holds that row's token, slot and the rank of
    // each slice, loaded now and used at the end.
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
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int r = (tid >> 3) + 32 * i;
        lrow[i] = r;
        if (r < BN) {
            src[i] = a.W + (int64_t)min(n0 + r, a.N - 1) * a.ldw;
        } else {
            const int m = min(m0 + r - BN, a.M - 1);
            const int t = a.rows ? a.rows[m] : m;
            src[i] = a.x + (int64_t)t * a.ldx;
        }
    }
    const int KT = (a.K + kBK - 1) / kBK;
    uint4 st[D][NL];
    // Loads read a clamped address; the chunks past K are zeroed when the set
    // is written to LDS, so nothing waits for a load before it is needed.
    auto load = [&](uint4 (&dst)[NL], int kt) {
        const int ec = min(kt * kBK + lc * 8, a.K - 8);
#pragma unroll
        for (int i = 0; i < NL; ++i) dst[i] = ld16(src[i] + ec);
    };
    auto store = [&](const uint4 (&from)[NL], int kt, int buf) {
        const bool ok = kt * kBK + lc * 8 < a.K;   // K is a multiple of 8: whole chunks
#pragma unroll
        for (int i = 0; i < NL; ++i)
            lds[buf][lrow[i]][swz(lrow[i], lc)] = ok ? from[i] : make_uint4(0, 0, 0, 0);
    };

    f32x4_t acc[NI][MI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) acc[ni][mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int li = lane & 15, lg = lane >> 4;
    auto compute = [&](int buf) {
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
    // the loop is unrolled by D so every set is named at compile time, and
    // every step runs (tiles past K are zeros), so no load waits behind a
    // branch.
#pragma unroll
    for (int d = 0; d < D; ++d) load(st[d], d);
    store(st[0], 0, 0);
    __syncthreads();
    auto step = [&](auto slot, int kt) {
        constexpr int S = decltype(slot)::value;
        load(st[S], kt + D);
        __builtin_amdgcn_sched_barrier(0);
        compute(kt & 1);
        __builtin_amdgcn_sched_barrier(0);
        store(st[(S + 1) % D], kt + 1, (kt + 1) & 1);
        __syncthreads();
    };
    const int KTD = (KT + D - 1) / D * D;
    for (int kt = 0; kt < KTD; kt += D) {
        step(std::integral_constant<int, 0>{}, kt);
        step(std::integral_constant<int, 1>{}, kt + 1);
        if constexpr (D > 2) step(std::integral_constant<int, 2>{}, kt + 2);
    }

    if constexpr (DELTA) {
        auto slice_of = [&](int col) {
            return (g.n_slices > 1 && col >= g.col_off[1]) + (g.n_slices > 2 && col >= g.col_off[2]) +
                   (g.n_slices > 3 && col >= g.col_off[3]);
        };
        auto pick_rank = [](const int4 &rk, int j) {
            return j == 0 ? rk.x : j == 1 ? rk.y : j == 2 ? rk.z : rk.w;
        };
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            const int m_row = m0 + wm * (BM / 2) + 16 * mi + li;   // this lane's row
            const int vrow = min(m_row, max(a.n_delta, 1) - 1);    // a readable v row
            // one pass per distinct slot among the group's 16 rows (lanes
            // 0..15 hold them; usually one, as rows come grouped by adapter)
            uint64_t pend = __builtin_amdgcn_ballot_w64(lane < 16 && ms[mi] != 0);
            while (pend) {
                const int lead = (int)__builtin_ctzll(pend);
                const int s = __builtin_amdgcn_readlane(ms[mi], lead);
                const bool in = ms[mi] == s;                      // this lane's row has slot s
                pend &= ~__builtin_amdgcn_ballot_w64(lane < 16 && in);
                int4 rk;
                rk.x = __builtin_amdgcn_readlane(mrk[mi].x, lead);
                rk.y = __builtin_amdgcn_readlane(mrk[mi].y, lead);
                rk.z = __builtin_amdgcn_readlane(mrk[mi].z, lead);
                rk.w = __builtin_amdgcn_readlane(mrk[mi].w, lead);
                // per column group: its slice, whether it straddles a slice
                // edge, and its B and v rows
                int jn[NI], rn[NI];
                bool mf[NI];
                const uint16_t *bn[NI];
                const float *vn[NI];
                int rmax = 0;
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    const int c0 = n0 + wn * (BN / 2) + 16 * ni;    // the 16-column group
                    const int j = slice_of(min(c0, a.N - 1));
                    jn[ni] = j;
                    mf[ni] = c0 < a.N && slice_of(min(c0 + 15, a.N - 1)) == j;
                    rn[ni] = pick_rank(rk, j);
                    rmax = max(rmax, mf[ni] ? rn[ni] : 0);
                    bn[ni] = p.Bn + (int64_t)(s - 1) * g.bt_slot_stride + pick4(g.bt_slice_off, j) +
                             (int64_t)(min(c0 + li, a.N - 1) - pick4(g.col_off, j)) * g.rank_pad;
                    vn[ni] = a.v + (int64_t)vrow * g.v_stride + j * g.rank_pad;
                }
                // matrix cores: the prefill expand's chain per column group,
                // B rows from the output-major copy (zero past the rank); each
                // rank step's loads for every group are issued before its MFMAs
                f32x4_t d[NI];
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) d[ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                for (int ks = 0; ks * 32 < rmax; ++ks) {
                    const int kk = 32 * ks + 8 * lg;
                    const int kc = min(kk, g.rank_pad - 8);       // inside the row
                    uint4 bv[NI];
                    float4 va[NI], vb[NI];
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) {
                        bv[ni] = ld16(bn[ni] + kc);
                        va[ni] = *reinterpret_cast<const float4 *>(vn[ni] + kc);
                        vb[ni] = *reinterpret_cast<const float4 *>(vn[ni] + kc + 4);
                    }
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) {
                        if (!mf[ni] || ks * 32 >= rn[ni]) continue;   // uniform
                        const float t[8] = {va[ni].x, va[ni].y, va[ni].z, va[ni].w,
                                            vb[ni].x, vb[ni].y, vb[ni].z, vb[ni].w};
                        float f[8];
#pragma unroll
                        for (int q = 0; q < 8; ++q) f[q] = (in && kk + q < rn[ni]) ? t[q] : 0.f;
                        uint4 vhi, vlo;
                        split_f32x8(f, vhi, vlo);
                        d[ni] = mfma16x16x32(bv[ni], vhi, d[ni]);
                        d[ni] = mfma16x16x32(bv[ni], vlo, d[ni]);
                    }
                }
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    const int c0 = n0 + wn * (BN / 2) + 16 * ni;
                    if (!in || c0 >= a.N) continue;
                    if (mf[ni]) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) acc[ni][mi][q] += d[ni][q];
                    } else {
                        // a group across a slice edge: per output, an fp32 fma
                        // chain over its slice's ranks from 0, then y = acc + d
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int o = c0 + 4 * lg + q;
                            if (o >= a.N) continue;
                            const int jq = slice_of(o);
                            const int rank = pick_rank(rk, jq);
                            const uint16_t *bt = p.Bt + (int64_t)(s - 1) * g.bt_slot_stride +
                                                 pick4(g.bt_slice_off, jq) + (o - pick4(g.col_off, jq));
                            const int hq = pick4(g.h_out, jq);
                            const float *vq = a.v + (int64_t)vrow * g.v_stride + jq * g.rank_pad;
                            float dq = 0.f;
                            for (int k = 0; k < rank; ++k)
                                dq = __builtin_fmaf(__uint_as_float((uint32_t)bt[(int64_t)k * hq] << 16),
                                                    vq[k], dq);
                            acc[ni][mi][q] += dq;
                        }
                    }
                }
            }
        }
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

}  // namespace

hipError_t launch_linear(const LaneGeom &g, const PoolDev &p, const LinearArgs &a,
                         hipStream_t s)
{
    if (a.M <= 0) return hipSuccess;
    if (a.K < 8 || a.K % 8 || a.N < 8 || a.N % 8) return hipErrorInvalidValue;
    // The largest tile that still gives the chip at least two workgroups per
    // CU; small batches (decode) take 64 x 64 tiles.
    auto tasks = [&](int bn, int bm) {
        return (int64_t)((a.N + bn - 1) / bn) * ((a.M + bm - 1) / bm);
    };
    constexpr int64_t kWant = 512;
    if (tasks(64, 64) > INT32_MAX) return hipErrorInvalidConfiguration;
    if (tasks(128, 128) >= kWant) launch_t<128, 128>(g, p, a, s);
    else if (tasks(128, 64) >= kWant) launch_t<128, 64>(g, p, a, s);
    else launch_t<64, 64>(g, p, a, s);
    return hipGetLastError();
}

}  // namespace lora
