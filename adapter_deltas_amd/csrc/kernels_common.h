// Device helpers shared by the gfx950 kernels.
#pragma once

#include "lora_internal.h"

namespace lora {

// A segment descriptor held as four uniform int4 values.
struct Seg {
    int4 h;    // slot, first active row, rows, kind
    int4 rk;   // rank of slices 0..3
    int4 lo;   // token rows 0..3
    int4 hi;   // token rows 4..7
    __device__ int slot() const { return h.x; }
    __device__ int v_row() const { return h.y; }
    __device__ int n_rows() const { return h.z; }
    __device__ int rank(int j) const
    {
        return j == 0 ? rk.x : j == 1 ? rk.y : j == 2 ? rk.z : rk.w;
    }
    // token row c of a decode segment (entries past n_rows repeat the last row)
    template <int c>
    __device__ int row() const
    {
        static_assert(c >= 0 && c < 8, "row index");
        if constexpr (c == 0) return lo.x;
        else if constexpr (c == 1) return lo.y;
        else if constexpr (c == 2) return lo.z;
        else if constexpr (c == 3) return lo.w;
        else if constexpr (c == 4) return hi.x;
        else if constexpr (c == 5) return hi.y;
        else if constexpr (c == 6) return hi.z;
        else return hi.w;
    }
    // first token row of a prefill segment
    __device__ int first_row() const { return lo.x; }
};

// Descriptors are read-only while kernels run, so they are read through the
// constant address space: a uniform index then gives scalar loads, which
// neither take vector registers nor wait behind the vector loads in flight.
// The 64-byte descriptor is read as one 16-word load, so that no part of it
// is fetched later than another.
__device__ __forceinline__ Seg load_seg(const int32_t *seg, int si)
{
    typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
    typedef const __attribute__((address_space(4))) i32x16 cvec;
    const i32x16 d = *(cvec *)(seg + (int64_t)si * kSegWords);
    return Seg{make_int4(d[0], d[1], d[2], d[3]), make_int4(d[4], d[5], d[6], d[7]),
               make_int4(d[8], d[9], d[10], d[11]), make_int4(d[12], d[13], d[14], d[15])};
}

// Workgroups are handed to the 8 XCDs round-robin by block id, and each XCD
// has its own L2.  This bijection on [0, n) gives XCD x the consecutive task
// range of its share, so tasks that read the same rows or factor tiles (which
// sit next to each other in task order) share an L2.  Placement only changes
// speed, never results.
__device__ __forceinline__ int xcd_task(int b, int n)
{
    // XCD x < n % 8 has q + 1 tasks, the others q (written without a branch,
    // so that loads after it are not held behind one)
    const int q = n / kXcds, rem = n % kXcds;
    const int xcd = b % kXcds, local = b / kXcds;
    return xcd * q + min(xcd, rem) + local;
}

// A device-built routing knows its segment count only on the device: a
// launch covers a bound, and the live segments are a prefix of it.  Dealt out
// by xcd_task, that prefix would sit on the first few XCDs only; here `deal`
// tasks (whole segments: r.spread of them, `per` tasks each) go to the XCDs
// in turn, deal d to XCD d % 8, so the prefix spreads over every XCD while a
// segment's tasks, and those of the next few segments, share an L2.  The
// grid is seg_grid(): 8 * deal * ceil(n / (8 * spread)) blocks, a bijection
// onto the tasks below that, of which those from n * per on are empty.
__device__ __forceinline__ int spread_task(int b, int deal)
{
    const int xcd = b % kXcds, l = b / kXcds;
    const int i = l / deal;
    return (xcd + kXcds * i) * deal + (l - i * deal);
}

// Task of block b in a launch of n tasks, `per` to a segment (see seg_grid).
__device__ __forceinline__ int seg_task(const RoutingDev &r, int b, int n, int per)
{
    return r.spread > 0 ? spread_task(b, r.spread * per) : xcd_task(b, n);
}

// Slice j and tile within the slice of tile number `rem` of a segment, by
// compares and selects on the widths in the kernel arguments, so every task
// of a launch is a live tile and none waits for a table load to find that out.
template <int TILE>
__device__ __forceinline__ void slice_tile(const LaneGeom &g, int rem, int &j, int &tile)
{
    const int c1 = (g.h_out[0] + TILE - 1) / TILE;
    const int c2 = c1 + (g.h_out[1] + TILE - 1) / TILE;
    const int c3 = c2 + (g.h_out[2] + TILE - 1) / TILE;
    j = (rem >= c1) + (rem >= c2) + (rem >= c3);
    tile = rem - (rem >= c3 ? c3 : rem >= c2 ? c2 : rem >= c1 ? c1 : 0);
}

// Entry j (0..3) of a 4-entry array held in the kernel arguments, taken by
// selects: indexing the argument segment with a runtime value would make the
// load of the entry wait for that value, one more dependent scalar load
// before the kernel's first data load.
// The empty statement makes the four values opaque, so the compiler neither
// turns the selects back into a load through a selected address nor into
// branches.
template <class T>
__device__ __forceinline__ T pick4(const T (&a)[4], int j)
{
    T a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
    asm("" : "+s"(a0), "+s"(a1), "+s"(a2), "+s"(a3));
    const T lo = (j & 1) ? a1 : a0;
    const T hi = (j & 1) ? a3 : a2;
    return (j & 2) ? hi : lo;
}

// The kernel arguments of the decode kernels (lane geometry, pool and
// routing views, then the call's own scalars) span four 64-byte lines.  Left
// to itself the compiler loads each argument at its first use, so a line
// first needed deep in the prologue costs one more miss in series.  This
// asks for one argument of each line at entry, so the four lines are fetched
// together and later argument loads hit the scalar cache.  The task count
// passes through the same statement, so the task arithmetic (and everything
// after it) is placed behind the one wait.
__device__ __forceinline__ void touch_args(int &n_tasks, const LaneGeom &g, const PoolDev &p,
                                           const RoutingDev &r, int64_t last)
{
    asm volatile("" : "+s"(n_tasks) : "s"(g.h_in), "s"(g.bt_slot_stride), "s"(p.scale),
                 "s"(r.counts), "s"(last));
}

// Descriptor of decode segment si into sd, and whether si is one of the
// batch's decode segments: with device-built routing the grid covers the
// bound on the count and the tasks past the count end here.  The count and
// the descriptor (inside the table for any si of the grid) are both loaded
// before either is waited for, and the result depends on both, so neither
// load is moved behind the other's branch.  With host-built routing there is
// no count and an arbitrary readable word stands in for it.
__device__ __forceinline__ bool decode_seg(const RoutingDev &r, int si, Seg &sd)
{
    typedef const __attribute__((address_space(4))) int32_t cint;
    const int32_t *cp = r.counts ? r.counts + kCntDecode : r.seg;
    const int raw = *(cint *)cp;
    sd = load_seg(r.seg, si);
    const int n_dec = r.counts ? raw : INT32_MAX;
    return si < n_dec && sd.n_rows() > 0;
}

// v in the split form (vsplit_groups) is written by store_vsplit.
__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Stores n (1 or 4) consecutive ranks k .. k + n - 1 (within one group of 16)
// of row p, slice j; a row holds row_len bf16.
template <int N>
__device__ __forceinline__ void store_vsplit(uint16_t *vs, int row_len, int groups, int p, int j,
                                             int k, const float (&val)[N])
{
    uint16_t *at = vs + (int64_t)p * row_len + (j * groups + k / 16) * 32 + k % 16;
    uint16_t hi[N], lo[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        hi[i] = bf16_rne(val[i]);
        lo[i] = bf16_rne(val[i] - __uint_as_float((uint32_t)hi[i] << 16));
    }
    if constexpr (N == 4) {
        *reinterpret_cast<uint2 *>(at) =
            make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
        *reinterpret_cast<uint2 *>(at + 16) =
            make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
    } else {
        at[0] = hi[0];
        at[16] = lo[0];
    }
}

__device__ __forceinline__ uint4 ld16(const uint16_t *p)
{
    return *reinterpret_cast<const uint4 *>(p);
}

}  // namespace lora
