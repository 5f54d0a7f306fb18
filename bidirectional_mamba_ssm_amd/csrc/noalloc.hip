// bimamba_ssd_fwd_noalloc: the bidirectional scan with no device allocation,
// for callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc). Its workspace is a static
// device array of kScratchBytes, held by every device the library runs on
// until the process ends; calls that overlap on one device share it and
// race. Nothing in it needs clearing: every kernel writes what it later
// reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/bimamba.h"
#include "internal.hpp"

namespace {

constexpr size_t kScratchBytes = BIMAMBA_NOALLOC_SCRATCH_BYTES;

// One copy per device, at its own address on each.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch`, per device (looked up once)

// The current device's address of `scratch`. Host code uses this address,
// never the array's name (a host-side stand-in, not a device address).
int scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return bm::api_fail(BIMAMBA_EHIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices)
        return bm::api_fail(BIMAMBA_EUNSUPPORTED, "device index beyond 63");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return bm::api_fail(BIMAMBA_EHIP, "hipGetSymbolAddress of the scan's static workspace failed");
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return BIMAMBA_OK;
}

}  // namespace

extern "C" {

int bimamba_ssd_fwd_noalloc(const bimamba_shape *s, const bimamba_dir *fwd,
                            const bimamba_dir *bwd, const int32_t *cu_seqlens, int nseq,
                            const float *init_state, float *final_state, float *y,
                            bimamba_stream stream) {
    // every argument first, with no HIP call (the shape must fit the buffer)
    int rc = bm::ssd_fwd_impl(s, fwd, bwd, cu_seqlens, nseq, init_state, final_state, y, nullptr,
                              nullptr, kScratchBytes, stream, kScratchBytes, true);
    if (rc) return rc;
    void *ws = nullptr;
    if ((rc = scratch_address(&ws))) return rc;
    return bm::ssd_fwd_impl(s, fwd, bwd, cu_seqlens, nseq, init_state, final_state, y, nullptr,
                            ws, kScratchBytes, stream, kScratchBytes, false);
}

}  // extern "C"
