// noalloc.hip -- hypic_seam_advance_noalloc: hypic_seam_advance with its window records and
// blocked-scan buffers in a static device array of the library instead of a caller
// workspace, for callers that cannot allocate device memory.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "api_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;   // HYPIC_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == HYPIC_NOALLOC_SCRATCH_BYTES, "header and library disagree on the scratch size");

// One copy per device, held while the library is loaded.  In host code this name stands
// for the host-side shadow, not a device address: kernels get the address returned by
// hipGetSymbolAddress for the device they run on.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on device `dev`, looked up once per device with that
// device current (and the caller's current device restored).
hypic_status scratch_on(int dev, void** out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return hypic::api_error(HYPIC_E_UNSUPPORTED, "hypic_seam_advance_noalloc: device index out of range");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess)
            return hypic::api_error(HYPIC_E_DEVICE, "hypic_seam_advance_noalloc: hipGetDevice failed");
        if (cur != dev && hipSetDevice(dev) != hipSuccess)
            return hypic::api_error(HYPIC_E_DEVICE, "hypic_seam_advance_noalloc: hipSetDevice failed");
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) {
            char msg[256];
            snprintf(msg, sizeof msg, "hypic_seam_advance_noalloc: hipGetSymbolAddress failed (HIP error %d, %s)",
                     (int)e, hipGetErrorString(e));
            return hypic::api_error(HYPIC_E_DEVICE, msg);
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return HYPIC_OK;
}

}  // namespace

extern "C" hypic_status hypic_seam_advance_noalloc(const hypic_dims* dims, int32_t n_chain, int32_t n_step,
                                                   int32_t w, const int64_t* seam_start, int64_t n_tokens,
                                                   const void* q, const void* k, const void* v, const void* g,
                                                   const void* beta, float scale, const int32_t* pair_id,
                                                   int32_t n_pair, const void* T_cache, const float* S_cache,
                                                   float* S_run, float* out, void* stream)
{
    const size_t need = hypic_seam_workspace_bytes(dims, n_chain, n_step, w);
    if (need > kScratchBytes) {
        char msg[256];
        snprintf(msg, sizeof msg,
                 "hypic_seam_advance_noalloc: the call needs %zu bytes of scratch, the library's static scratch "
                 "holds %zu (use hypic_seam_advance with a workspace)", need, kScratchBytes);
        return hypic::api_error(HYPIC_E_INVALID, msg);
    }
    int dev = -1;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess)
        return hypic::api_error(HYPIC_E_DEVICE, "hypic_seam_advance_noalloc: the stream's device is unknown");
    void* ws = nullptr;
    if (hypic_status s = scratch_on(dev, &ws)) return s;
    return hypic::seam_advance_with(dims, n_chain, n_step, w, seam_start, n_tokens, q, k, v, g, beta, scale,
                                    pair_id, n_pair, T_cache, S_cache, S_run, out, ws, kScratchBytes, stream);
}
