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
__device__ __forceinline__ Seg load_seg(const int32_t *seg, int si)
{
    typedef const __attribute__((address_space(4))) int32_t cint;
    cint *p = (cint *)(seg + (int64_t)si * kSegWords);
    return Seg{make_int4(p[0], p[1], p[2], p[3]), make_int4(p[4], p[5], p[6], p[7]),
               make_int4(p[8], p[9], p[10], p[11]), make_int4(p[12], p[13], p[14], p[15])};
}

// Workgroups are handed to the 8 XCDs round-robin by block id, and each XCD
// has its own L2.  This bijection on [0, n) gives XCD x the consecutive task
// range of its share, so tasks that read the same rows or factor tiles (which
// sit next to each other in task order) share an L2.  Placement only changes
// speed, never results.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_task(int b, int n)
{
    const int q = n / kXcds, rem = n % kXcds;
    const int xcd = b % kXcds, local = b / kXcds;
    return xcd < rem ? xcd * (q + 1) + local : rem * (q + 1) + (xcd - rem) * q + local;
}

__device__ __forceinline__ uint4 ld16(const uint16_t *p)
{
    return *reinterpret_cast<const uint4 *>(p);
}

}  // namespace lora
