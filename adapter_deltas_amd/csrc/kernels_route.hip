// Device-side routing of a decode batch (gfx950).
//
// Input: one slot per token row (0 = base), every row a decode row.  One
// workgroup sorts the active rows by (path, slot, row), four keys per thread in
// registers (strides across waves through LDS), finds each slot's run start
// with a max-scan and numbers the segments with a sum-scan, then writes the
// same kinds of segment the host planner writes: for adapters whose largest
// slice rank is below LORA_GATHER_MIN_RANK, decode segments of up to
// kDecodeSegRows rows (GEMV path); for the others, gather segments of up to
// kPrefillSegRows rows (matrix-core path).  Each row's path depends only on its
// adapter, and a row's bits do not depend on which segment it lands in, so
// the delta equals the one a host-built routing gives, bit for bit.
//
// The segment table has room for max_dec decode segments, then max_gather
// gather segments; the exact counts go to `counts` for the kernels to read.
#include <utility>

#include "kernels_common.h"

namespace lora {
namespace {

constexpr uint32_t kNoKey = 0xffffffffu;
constexpr int kRowBits = 13;                 // row index bits of a sort key
constexpr int kSlotBits = 16;                // slot bits above them, then the path bit
constexpr int kRouteRowsPerThread = 4;       // sort keys per thread (8 in the largest form)
static_assert(LORA_DEVICE_ROUTING_MAX_TOKENS <= (1 << kRowBits), "rows fit the key");
static_assert((kDecodeSegRows & (kDecodeSegRows - 1)) == 0 &&
                  (kPrefillSegRows & (kPrefillSegRows - 1)) == 0,
              "segment sizes are powers of two");

// Inclusive prefix sums of x.x and x.y over lanes 0..lane of the wave.
__device__ inline int2 wave_prefix_sum2(int2 x, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int a = __shfl_up(x.x, d, 64), b = __shfl_up(x.y, d, 64);
        if (lane >= d) {
            x.x += a;
            x.y += b;
        }
    }
    return x;
}

// Inclusive prefix maximum of x over lanes 0..lane of the wave.
__device__ inline int wave_prefix_max(int x, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int a = __shfl_up(x, d, 64);
        if (lane >= d) x = max(x, a);
    }
    return x;
}

// Exclusive prefix sums of x (two fields) over the block's threads, and the
// block totals.  Every thread must call it; `part` holds one entry per wave.
template <int NW>
__device__ inline int2 block_exclusive_sum2(int2 x, int lane, int wave, int2 *part, int2 &total)
{
    const int2 incl = wave_prefix_sum2(x, lane);
    int2 before = make_int2(0, 0);
    if constexpr (NW == 1) {
        total = make_int2(__shfl(incl.x, 63, 64), __shfl(incl.y, 63, 64));
    } else {
        if (lane == 63) part[wave] = incl;
        __syncthreads();
        total = make_int2(0, 0);
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int2 v = part[w];
            if (w < wave) {
                before.x += v.x;
                before.y += v.y;
            }
            total.x += v.x;
            total.y += v.y;
        }
        __syncthreads();
    }
    return make_int2(before.x + incl.x - x.x, before.y + incl.y - x.y);
}

// Maximum of x over the threads before this one (0 for thread 0; x >= 0).
template <int NW>
__device__ inline int block_exclusive_max(int x, int lane, int wave, int *part)
{
    const int incl = wave_prefix_max(x, lane);
    int excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0;
    if constexpr (NW > 1) {
        if (lane == 63) part[wave] = incl;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NW; ++w)
            if (w < wave) excl = max(excl, part[w]);
        __syncthreads();
    }
    return excl;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// The value of lane `lane ^ M` (M = 1, 2, 4, 8, 16 or 32), without LDS:
// quad permutes and row rotates for partners in the same 16-lane row,
// register-half swaps for the others.
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x, int lane)
{
    if constexpr (M == 1) {
        return dpp_u32<0xB1>(x);                           // quad_perm [1,0,3,2]
    } else if constexpr (M == 2) {
        return dpp_u32<0x4E>(x);                           // quad_perm [2,3,0,1]
    } else if constexpr (M == 4) {
        const uint32_t a = dpp_u32<0x124>(x);              // row_ror:4, from lane - 4
        const uint32_t b = dpp_u32<0x12C>(x);              // row_ror:12, from lane + 4
        return (lane & 4) ? a : b;
    } else if constexpr (M == 8) {
        return dpp_u32<0x128>(x);                          // row_ror:8
    } else if constexpr (M == 16) {
        const auto t = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane & 16) ? t[0] : t[1];
    } else {
        static_assert(M == 32, "partner within the wave");
        const auto t = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane & 32) ? t[0] : t[1];
    }
}

// Puts the smaller of a and b first when `up`, the larger otherwise.
__device__ inline void order2(uint32_t &a, uint32_t &b, bool up)
{
    const uint32_t lo = min(a, b), hi = max(a, b);
    a = up ? lo : hi;
    b = up ? hi : lo;
}

// One compare-exchange stage of a bitonic merge of SIZE positions, then the
// smaller strides of the same merge.  Thread t holds positions E t .. E t +
// E - 1; strides below E stay in the thread, below 64 E in the wave, larger
// ones go through LDS (`key`, E entries per thread).
template <int E, int SIZE, int STRIDE>
__device__ __forceinline__ void bitonic_stage(uint32_t (&k)[E], int tid, int lane, uint32_t *key)
{
    static_assert(E == 4 || E == 8, "four or eight keys per thread");
    const int p0 = tid * E;
    if constexpr (STRIDE >= 64 * E) {
        const bool up = (p0 & SIZE) == 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; e += 4)
            *reinterpret_cast<uint4 *>(&key[p0 + e]) = make_uint4(k[e], k[e + 1], k[e + 2], k[e + 3]);
        __syncthreads();
        const bool keep_min = ((p0 & STRIDE) == 0) == up;
#pragma unroll
        for (int e = 0; e < E; e += 4) {
            const uint4 o = *reinterpret_cast<const uint4 *>(&key[(p0 ^ STRIDE) + e]);
            k[e] = keep_min ? min(k[e], o.x) : max(k[e], o.x);
            k[e + 1] = keep_min ? min(k[e + 1], o.y) : max(k[e + 1], o.y);
            k[e + 2] = keep_min ? min(k[e + 2], o.z) : max(k[e + 2], o.z);
            k[e + 3] = keep_min ? min(k[e + 3], o.w) : max(k[e + 3], o.w);
        }
    } else if constexpr (STRIDE >= E) {
        const bool up = (p0 & SIZE) == 0;
        const bool keep_min = ((tid & (STRIDE / E)) == 0) == up;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t o = lane_xor<STRIDE / E>(k[e], lane);
            k[e] = keep_min ? min(k[e], o) : max(k[e], o);
        }
    } else {
        // partners inside the thread: e and e + STRIDE; the direction of a
        // pair comes from its position's SIZE bit
#pragma unroll
        for (int e = 0; e < E; ++e)
            if ((e & STRIDE) == 0) order2(k[e], k[e + STRIDE], ((p0 + e) & SIZE) == 0);
    }
    if constexpr (STRIDE > 1) bitonic_stage<E, SIZE, STRIDE / 2>(k, tid, lane, key);
}

// Bitonic sort, ascending, of the first n_sort positions (a power of two,
// uniform): merges of 2, 4, ... n_sort positions.  Positions past n_sort are
// sorted among themselves only.
template <int E, int ROWS, int SIZE = 2>
__device__ __forceinline__ void bitonic_sort(uint32_t (&k)[E], int n_sort, int tid, int lane,
                                             uint32_t *key)
{
    if (SIZE > n_sort) return;
    bitonic_stage<E, SIZE, SIZE / 2>(k, tid, lane, key);
    if constexpr (SIZE < ROWS) bitonic_sort<E, ROWS, SIZE * 2>(k, n_sort, tid, lane, key);
}

// f(integral_constant<int, e>) for e = 0 .. E - 1, unrolled at compile time.
template <class F, int... I>
__device__ __forceinline__ void for_each_key(F f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}

// THREADS threads route up to E * THREADS rows.  Thread t holds the keys of
// sorted positions E t .. E t + E - 1 in registers.  With MOE the rows are the
// dispatched (token, expert) rows of an expert projection and `tok_slot`
// holds each token's adapter slot; a row's slot is its (adapter, expert)
// pool slot.
template <int THREADS, int E, bool MOE>
__global__ __launch_bounds__(THREADS) void k_route_decode(
    const int32_t *__restrict__ tok_slot, int n_tok, MoeDispatch moe,
    const int4 *__restrict__ rank_rows, int max_slots, int max_dec, int max_gather,
    int32_t *__restrict__ seg, int32_t *__restrict__ rows, int32_t *__restrict__ tok,
    int32_t *__restrict__ counts)
{
    constexpr int ROWS = THREADS * E;
    constexpr int NW = THREADS / 64;
    constexpr uint32_t kRowMask = (1u << kRowBits) - 1;
    __shared__ __align__(16) uint32_t key[ROWS];
    __shared__ int2 part2[NW];
    __shared__ int part1[NW];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p0 = tid * E;
    const uint32_t gather_key = 1u << (kRowBits + kSlotBits);
    auto pre = [](uint32_t k) { return k >> kRowBits; };   // (path, slot) of a key
    // the sort covers the next power of two >= n_tok (at least 2) positions
    int n_sort = 2;
    while (n_sort < n_tok) n_sort <<= 1;

    // Keys path << 28 | slot << 12 | row, one per row; base and invalid rows
    // get kNoKey and sort last.  All slot loads, then all rank loads (rank
    // row 0 is zero), so the dependent global reads are paid once each.
    // sl = -1 marks a row that names no valid slot.
    int sl[E];
    if constexpr (MOE) {
        int t[E], x[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool row = p0 + e < n_tok;
            t[e] = row ? moe.row_token[p0 + e] : 0;
            x[e] = row ? moe.row_expert[p0 + e] : 0;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool row = p0 + e < n_tok;
            const bool t_ok = t[e] >= 0 && t[e] < moe.n_tokens;
            const int a = row && t_ok ? tok_slot[t[e]] : 0;
            const bool ok = t_ok && x[e] >= 0 && x[e] < moe.n_experts && a >= 0 &&
                            a <= moe.n_adapter_slots;
            sl[e] = !row ? 0 : !ok ? -1 : a == 0 ? 0 : (a - 1) * moe.n_experts + x[e] + 1;
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) sl[e] = p0 + e < n_tok ? tok_slot[p0 + e] : 0;
    }
    int4 rk[E];
#pragma unroll
    for (int e = 0; e < E; ++e) rk[e] = rank_rows[sl[e] >= 1 && sl[e] <= max_slots ? sl[e] : 0];
    uint32_t k[E];
    int n_ok = 0, n_ok_decode = 0, n_bad = 0, n_unedited = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = p0 + e, s = sl[e];
        const int4 r = rk[e];
        // a slot holds factors iff its slice-0 rank is set
        const bool g = max(max(r.x, r.y), max(r.z, r.w)) >= kGatherMinRank;
        const bool in_range = s >= 1 && s <= max_slots;
        const bool ok = in_range && r.x > 0 && (g ? max_gather : max_dec) > 0;
        if (i < n_tok) tok[i] = ok ? s : 0;
        k[e] = ok ? (g ? gather_key : 0u) | (uint32_t)s << kRowBits | (uint32_t)i : kNoKey;
        n_ok += ok;
        n_ok_decode += ok && !g;
        // an (adapter, expert) slot without factors: the adapter leaves that
        // expert alone; any other slot that is not 0 and not usable is invalid
        const bool unedited = MOE && in_range && r.x == 0;
        n_unedited += unedited;
        n_bad += s != 0 && !ok && !unedited;
    }
    int2 cnt;
    block_exclusive_sum2<NW>(make_int2(n_ok | n_ok_decode << 16, n_bad | n_unedited << 16), lane,
                             wave, part2, cnt);
    const int na = cnt.x & 0xffff;          // active rows
    const int n_invalid = cnt.y & 0xffff;
    const int n_unedited_rows = cnt.y >> 16;

    bitonic_sort<E, ROWS>(k, n_sort, tid, lane, key);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; e += 4)
        *reinterpret_cast<uint4 *>(&key[p0 + e]) = make_uint4(k[e], k[e + 1], k[e + 2], k[e + 3]);
    __syncthreads();
    // the ranks of each sorted row's slot, needed by the descriptors at the
    // end (loaded after the barrier, which would wait for them)
    int4 srk[E];
#pragma unroll
    for (int e = 0; e < E; ++e) srk[e] = rank_rows[k[e] != kNoKey ? pre(k[e]) & 0xffff : 0];

    // Run starts (first position of each (path, slot) run) by a max-scan;
    // a segment starts every 8th (decode) or 64th (gather) row of a run.
    const uint32_t prev = p0 > 0 ? key[p0 - 1] : kNoKey;
    int run_start[E];
    {
        int m = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t before = e == 0 ? prev : k[e - 1];
            if (p0 + e < na && pre(before) != pre(k[e])) m = p0 + e;
            run_start[e] = m;
        }
        const int excl = block_exclusive_max<NW>(m, lane, wave, part1);
#pragma unroll
        for (int e = 0; e < E; ++e) run_start[e] = max(run_start[e], excl);
    }
    int flag[E];
    int n_flag = 0, n_flag_decode = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int size = k[e] >= gather_key ? kPrefillSegRows : kDecodeSegRows;
        flag[e] = p0 + e < na && ((p0 + e - run_start[e]) & (size - 1)) == 0;
        n_flag += flag[e];
        n_flag_decode += flag[e] && k[e] < gather_key;
    }
    int2 seg_total;
    const int2 seg_before = block_exclusive_sum2<NW>(
        make_int2(n_flag | n_flag_decode << 16, 0), lane, wave, part2, seg_total);
    const int ord = seg_before.x & 0xffff;  // segments before this thread's positions
    const int total = seg_total.x & 0xffff;
    const int n_dec = seg_total.x >> 16;    // decode segments come first

    // first position whose key's (path, slot) is >= q
    auto lower = [&](uint32_t q) {
        int lo = 0, hi = na;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (pre(key[mid]) < q) lo = mid + 1;
            else hi = mid;
        }
        return lo;
    };
    // row p of the sorted order, and the descriptor of the segment starting
    // there (flag), the ord-th segment; by value, so no register array is
    // indexed at run time
    auto emit = [&](int p, uint32_t kp, bool fl, int4 ranks, int ord) {
        if (p < na) rows[p] = (int32_t)(kp & kRowMask);
        if (!fl) return;
        const bool g = kp >= gather_key;
        const int s = (int)(pre(kp) & 0xffff);
        // (the bounds hold for every mixture; the test only guards memory)
        const bool room = g ? ord - n_dec >= 0 && ord - n_dec < max_gather : ord < max_dec;
        if (!room) return;
        int4 *d = reinterpret_cast<int4 *>(seg + (int64_t)(g ? max_dec + (ord - n_dec) : ord) * kSegWords);
        int n;
        int r[kDecodeSegRows];
        if (!g) {
            // the run's next rows (positions past the run hold other keys)
            uint32_t nk[kDecodeSegRows];
#pragma unroll
            for (int c = 0; c < kDecodeSegRows; ++c) nk[c] = p + c < ROWS ? key[p + c] : kNoKey;
            n = 0;
            int last = 0;
#pragma unroll
            for (int c = 0; c < kDecodeSegRows; ++c)
                if (pre(nk[c]) == pre(kp) && n == c) {
                    n = c + 1;
                    last = (int)(nk[c] & kRowMask);
                }
#pragma unroll
            for (int c = 0; c < kDecodeSegRows; ++c) r[c] = c < n ? (int)(nk[c] & kRowMask) : last;
        } else {
            n = min(kPrefillSegRows, lower(pre(kp) + 1) - p);
#pragma unroll
            for (int c = 0; c < kDecodeSegRows; ++c) r[c] = 0;
        }
        d[0] = make_int4(s, p, n, g ? kSegGather : kSegDecode);
        d[1] = ranks;
        d[2] = make_int4(r[0], r[1], r[2], r[3]);
        d[3] = make_int4(r[4], r[5], r[6], r[7]);
    };
    int ordv[E];                            // segments before position p0 + e
    ordv[0] = ord;
#pragma unroll
    for (int e = 1; e < E; ++e) ordv[e] = ordv[e - 1] + flag[e - 1];
    for_each_key([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        emit(p0 + e, k[e], flag[e], srk[e], ordv[e]);
    }, std::make_integer_sequence<int, E>{});
    if (tid == 0) {
        counts[kCntActive] = na;
        counts[kCntDecode] = n_dec;
        counts[kCntPrefill] = 0;
        counts[kCntGather] = total - n_dec;
        counts[kCntInvalid] = n_invalid;
        counts[kCntUnedited] = n_unedited_rows;
    }
}

}  // namespace

hipError_t launch_route_decode(const int32_t *tok_slot, int n_tok, const MoeDispatch *moe,
                               const int32_t *rank_tab, int max_slots, int max_dec,
                               int max_gather, int32_t *seg, int32_t *rows, int32_t *tok,
                               int32_t *counts, hipStream_t s)
{
    static_assert(kMetaStride == 4, "one int4 of ranks per slot");
    static_assert(kSegWords == 16, "a descriptor is four int4 values");
    if (n_tok < 0 || n_tok > LORA_DEVICE_ROUTING_MAX_TOKENS) return hipErrorInvalidValue;
    if (reinterpret_cast<uintptr_t>(rank_tab) % 16 || reinterpret_cast<uintptr_t>(seg) % 16)
        return hipErrorInvalidValue;
    const int4 *rr = reinterpret_cast<const int4 *>(rank_tab);
    const MoeDispatch d = moe ? *moe : MoeDispatch{nullptr, nullptr, 0, 1, 0};
    auto launch = [&](auto kernel, int threads) {
        hipLaunchKernelGGL(kernel, dim3(1), dim3(threads), 0, s, tok_slot, n_tok, d, rr,
                           max_slots, max_dec, max_gather, seg, rows, tok, counts);
    };
    // the smallest workgroup whose threads hold the rows: every thread runs
    // every stage of the sort, so a half-empty workgroup costs twice the
    // compare-exchange work (2048 MoE rows: 18 us on 1024 threads)
    constexpr int E = kRouteRowsPerThread;
    if (n_tok <= 64 * E)
        moe ? launch(k_route_decode<64, E, true>, 64) : launch(k_route_decode<64, E, false>, 64);
    else if (n_tok <= 128 * E)
        moe ? launch(k_route_decode<128, E, true>, 128)
            : launch(k_route_decode<128, E, false>, 128);
    else if (n_tok <= 256 * E)
        moe ? launch(k_route_decode<256, E, true>, 256)
            : launch(k_route_decode<256, E, false>, 256);
    else if (n_tok <= 512 * E)
        moe ? launch(k_route_decode<512, E, true>, 512)
            : launch(k_route_decode<512, E, false>, 512);
    else if (n_tok <= 1024 * E)
        moe ? launch(k_route_decode<1024, E, true>, 1024)
            : launch(k_route_decode<1024, E, false>, 1024);
    else
        moe ? launch(k_route_decode<1024, 2 * E, true>, 1024)
            : launch(k_route_decode<1024, 2 * E, false>, 1024);
    return hipGetLastError();
}

}  // namespace lora
