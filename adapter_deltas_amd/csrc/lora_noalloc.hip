// lora_delta_apply_noalloc: the delta with v kept in a static device array of
// the library instead of a caller workspace, for callers that cannot allocate
// device memory.  The kernels are lora_delta_apply's own; only the home of v
// differs.
#include <mutex>

#include "lora_internal.h"

namespace {

constexpr int64_t kScratchBytes = LORA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte lines");

// One copy per GPU, held until the process ends.  In host code this name is
// only a handle for hipGetSymbolAddress: kernels are given the device address
// looked up below, never the name.
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float *g_scratch_ptr[kMaxDevices];   // device address of scratch per device (null: not yet)

// Device address of `scratch` on device `dev`, looked up once per device
// with that device current (the caller's current device is restored).
int32_t scratch_on(int dev, float **out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return lora::fail(LORA_ERR_ARG, "device %d outside 0..%d", dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return lora::hip_fail(e, "hipGetDevice");
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return lora::hip_fail(e, "hipSetDevice");
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return lora::hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return lora::fail(LORA_ERR_HIP, "hipGetSymbolAddress gave a null address");
        g_scratch_ptr[dev] = static_cast<float *>(p);
    }
    *out = g_scratch_ptr[dev];
    return LORA_OK;
}

}  // namespace

extern "C" int32_t lora_delta_apply_noalloc(const lora_pool *pool, const lora_routing *routing,
                                            const void *x, int64_t ldx, float *y, int64_t ldy,
                                            void *stream)
{
    int64_t need = 0;
    if (int32_t rc = lora_workspace_bytes(pool, routing, &need)) return rc;
    lora_routing_info info{};
    lora_routing_get_info(routing, &info);
    if (info.n_active == 0) return LORA_OK;
    if (need > kScratchBytes)
        return lora::fail(LORA_ERR_CAPACITY,
                          "this batch needs %lld bytes of workspace, more than the %lld bytes "
                          "of the static scratch; use lora_delta_apply with a workspace",
                          (long long)need, (long long)kScratchBytes);
    // the GPU the work runs on is the stream's (the current one for the null stream)
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = -1;
    hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return lora::hip_fail(e, "finding the stream's device");
    float *v = nullptr;
    if (int32_t rc = scratch_on(dev, &v)) return rc;
    return lora::delta_apply_ws(pool, routing, x, ldx, y, ldy, v, kScratchBytes, st);
}
