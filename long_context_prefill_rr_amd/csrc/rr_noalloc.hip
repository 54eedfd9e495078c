// rr_noalloc.hip -- rr_prefill_noalloc: the whole sparse prefill with its
// workspace in a library-owned device array, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The workspace rr_prefill takes from the caller (block scores, pooled-key
// planes, per-(row, block) statistics, the V transpose) lives here in
// `scratch`, a file-scope device array of kScratchBytes.  Every GPU the
// library runs on holds its own copy until the process ends.  In host code
// the array's name only stands in for the symbol: its device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, on the first call made there, and only that address is handed to
// the kernels.  No kernel of the prefill reads workspace it has not written
// in the same call, so nothing is cleared between calls.
#include <mutex>

#include "rr.h"
#include "rr_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB, as stated in rr.h
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_lock;
void *g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (looked up once
// per device, under the lock); nullptr if the lookup fails.
void *scratch_on_current_device(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" {

size_t rr_noalloc_scratch_bytes(void) { return kScratchBytes; }

int rr_prefill_noalloc(const uint16_t *Q, const uint16_t *K, const uint16_t *V, int L, int Hq,
                       int Hkv, int d, int B, int S, float tau, void *O, int o_dtype,
                       int32_t *counts, int32_t *block_idx, void *stream) {
    const int rc = rr::check_prefill_args(Q, K, V, L, Hq, Hkv, d, B, S, tau, O, o_dtype, counts,
                                          block_idx);
    if (rc != RR_OK) return rc;
    if (rr_prefill_workspace_bytes(L, Hq, Hkv, d, B, S) > kScratchBytes) return RR_E_WORKSPACE;
    // The kernels run on the stream's device and must get that device's
    // copy of the array: require the stream to belong to the current device.
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return RR_E_HIP;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return RR_E_HIP;
        if (sdev != dev) return RR_E_UNSUPPORTED;
    }
    void *ws = scratch_on_current_device(dev);
    if (!ws) return RR_E_HIP;
    return rr::run_prefill(Q, K, V, L, Hq, Hkv, d, B, S, tau, O, o_dtype, counts, block_idx, ws,
                           stream);
}

}  // extern "C"
