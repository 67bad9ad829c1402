// moe_ffn_nvfp4_static: moe_ffn_nvfp4 with its workspace in a file-scope device array instead of
// a caller-allocated buffer, for callers that cannot allocate device memory.
//
// The array lives in every GPU the library is loaded on, until the process ends. Host code never
// passes the array's name to a kernel (on the host it is only a stand-in, not a device address):
// its device address is looked up once per device with hipGetSymbolAddress, with that device
// current, and that address is what the kernels receive.
#include <mutex>

#include "moe_internal.h"

// The workspace array (one per GPU). Its name is used only in the symbol lookup below.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_WS_BYTES];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` on each device (null: not looked up)

// Device address of this device's copy of the scratch array, looked up on the device's first
// call with the device current. Returns null on failure.
void *scratch_for(int dev) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev]) return g_scratch[dev];
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) {
        (void)hipGetLastError();
        return nullptr;
    }
    g_scratch[dev] = p;
    return p;
}

}  // namespace

extern "C" int moe_ffn_nvfp4_static(const uint16_t *x, const float *topk_w, const int32_t *offsets,
                                    const int32_t *pair_ids, const int32_t *active,
                                    const int32_t *counts, moe_bank gate, moe_bank up,
                                    moe_bank down, int32_t T, int32_t k, int32_t E, int32_t H,
                                    int32_t F, float *y, int32_t path, moe_stream_t stream) {
    // host-checkable conditions first, so that nothing touches a device on a rejected call
    if (T < 0 || k < 1 || E < 1 || H < 64 || F < 64 || H % 64 || F % 64) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (moe_ffn_nvfp4_ws(T, k, E, H, F) > (size_t)MOE_STATIC_WS_BYTES) return MOE_EWS;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int dev = -1;
    if (s != nullptr) {
        hipDevice_t d;
        if (hipStreamGetDevice(s, &d) != hipSuccess) return MOE_ELAUNCH;
        dev = (int)d;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return MOE_ELAUNCH;
    }
    if (dev < 0 || dev >= kMaxDevices) return MOE_ELAUNCH;
    void *ws = scratch_for(dev);
    if (!ws) return MOE_ELAUNCH;
    return moe_ffn_nvfp4(x, topk_w, offsets, pair_ids, active, counts, gate, up, down, T, k, E, H,
                         F, y, path, ws, (size_t)MOE_STATIC_WS_BYTES, stream);
}
