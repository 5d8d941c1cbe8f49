// bd_lmhead_conf_noalloc: the LM-head confidence call with its scratch
// memory (the per-workgroup partial states that the merge kernel combines)
// in a library-owned device array instead of a caller workspace, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The array lives in this file.  In host code its name is only a host-side
// stand-in, so its device address is fetched once per device (with that
// device current) through hipGetSymbolAddress and kept in a table; every use
// goes through that address.  Each GPU holds its own copy of the array until
// the process ends, shared by every call on that GPU.
#include <mutex>

#include "bd_internal.h"

namespace {

// Three partial arrays (max, sum, index) of at most 256 workgroups x 64
// positions x 4 bytes each: the largest workspace of the bf16 LM head.
constexpr size_t kScratchBytes = 3 * 256 * 64 * 4;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device.
hipError_t scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" bd_status bd_lmhead_conf_noalloc(bd_dtype dt, const void* h, const void* W,
                                            int32_t B, int32_t d, int32_t V, float* conf,
                                            int32_t* argmax, hipStream_t stream) {
    const bd::Finish f{conf, argmax, false, 0.f, nullptr, nullptr, nullptr};
    const bd_status s = bd::lmhead_args_status(dt, h, W, B, d, V, f);
    if (s != BD_OK) return s;
    if (bd::lmhead_ws_bytes_dt(dt, B, d, V) > kScratchBytes) return BD_E_WORKSPACE;
    void* ws = nullptr;
    if (scratch_on_current_device(&ws) != hipSuccess) return BD_E_DEVICE;
    return bd::launch_lmhead(dt, h, W, B, d, V, f, ws, stream) == hipSuccess ? BD_OK
                                                                              : BD_E_LAUNCH;
}
