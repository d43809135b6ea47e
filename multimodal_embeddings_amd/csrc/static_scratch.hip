// static_scratch.hip -- the allocation-free variant of the attention step (internal to libube).
//
// ube_step_attention allocates device memory for the item bounds and the 256-token
// tile list of every call. ube_step_attention_static keeps them in `scratch`, a
// fixed device array of the library: each GPU holds its own copy from the moment
// the code object is loaded until the process ends. Host code never passes the
// array's name to a kernel or a copy (on the host it names a stand-in, not device
// memory); it resolves the array's device address once per GPU with
// hipGetSymbolAddress, with that GPU current, and uses that address only.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "ube_steps.h"

namespace {

constexpr size_t kScratchInts = (size_t)1 << 18;  // 1 MiB of int32
constexpr int kMaxDevices = 64;

static __device__ __align__(256) int scratch[kScratchInts];

std::mutex g_mu;                    // guards the address table and the host staging
int *g_scratch_ptr[kMaxDevices] = {};
int g_host[kScratchInts];           // host image of what goes into `scratch` (no allocation per call)

// Device address of `scratch` on the current GPU (resolved on the first call there). NULL on failure.
int *scratch_on_current_device(hipError_t *err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess || !p) {
            if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        g_scratch_ptr[dev] = (int *)p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" ube_status_t ube_step_attention_static(void const *q, void const *k, size_t ldqk, void const *vt,
                                                  size_t ldvt, void *o, size_t ldo, uint32_t const *cu_host,
                                                  size_t count, size_t heads, void *stream) {
    if (!q || !k || !vt || !o || !cu_host || !heads || count >= kScratchInts) return ube_status_invalid_argument_k;
    size_t ntiles = 0;
    for (size_t i = 0; i < count; ++i) {
        if (cu_host[i + 1] < cu_host[i] || cu_host[i + 1] > 0x7fffff00u) return ube_status_invalid_argument_k;
        ntiles += (cu_host[i + 1] - cu_host[i] + ube::kTileTokens - 1) / ube::kTileTokens;
    }
    const size_t tiles_at = (count + 2) & ~(size_t)1;  // int2 entries start 8-byte aligned
    if (tiles_at + 2 * ntiles > kScratchInts) return ube_status_invalid_argument_k;
    if (ldvt < (size_t)cu_host[count] + ube::kRowPad) return ube_status_invalid_argument_k;

    std::lock_guard<std::mutex> lock(g_mu);
    hipError_t e = hipSuccess;
    int *dev = scratch_on_current_device(&e);
    if (!dev) return ube_status_device_k;
    for (size_t i = 0; i <= count; ++i) g_host[i] = (int)cu_host[i];
    size_t t = 0;
    for (size_t i = 0; i < count; ++i)
        for (uint32_t s = cu_host[i]; s < cu_host[i + 1]; s += ube::kTileTokens, ++t) {
            g_host[tiles_at + 2 * t] = (int)i;
            g_host[tiles_at + 2 * t + 1] = (int)s;
        }
    hipStream_t st = (hipStream_t)stream;
    e = hipMemcpyAsync(dev, g_host, (tiles_at + 2 * ntiles) * sizeof(int), hipMemcpyHostToDevice, st);
    if (e == hipSuccess)
        e = ube::launch_attention((const uint16_t *)q, (const uint16_t *)k, (int)ldqk, (const uint16_t *)vt, (int)ldvt,
                                  (uint16_t *)o, (int)ldo, dev, (const int2 *)(dev + tiles_at), (int)ntiles,
                                  (int)heads, st);
    // the host image is reused by the next call, and the next call on this GPU overwrites `scratch`
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e == hipSuccess) return ube_status_success_k;
    return e == hipErrorInvalidValue ? ube_status_invalid_argument_k : ube_status_device_k;
}
