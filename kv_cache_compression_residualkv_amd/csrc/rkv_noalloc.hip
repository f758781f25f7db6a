// rkv_encode without any allocation: the workspace is a static device array of this
// library (one per GPU the library runs on), for callers that cannot allocate.
#include <hip/hip_runtime.h>

#include <mutex>

#include "rkv.h"

namespace {

// The encode's scratch: candidate lists, the rescan queue, mean rows and hidden planes.
// Each GPU holds its own copy at its own address until the process ends.
__device__ __align__(256) unsigned char scratch[RKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The address of this device's copy of `scratch` (looked up on the first call on the
// device, with that device current). The array's host-side name is not a device address.
rkv_status device_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RKV_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RKV_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return RKV_OK;
}

}  // namespace

extern "C" rkv_status rkv_encode_noalloc(const rkv_config* cfg, const rkv_weights* w, rkv_cache* cache,
                                         const void* kv, int32_t kv_len, const int32_t* rows, const int32_t* pos,
                                         int32_t n, void* stream) {
    if (!cfg || !cache) return RKV_ERR_INVALID_ARG;
    const rkv_status cs = rkv_validate_config(cfg);
    if (cs != RKV_OK) return cs;
    if (n == 0) return rkv_encode_ex(cfg, w, cache, kv, kv_len, rows, pos, n, nullptr, 0, stream, nullptr);
    // an invalid cache gives 0 here and is reported by rkv_encode_ex
    const size_t need = rkv_encode_workspace_bytes(cfg, cache->batch, n, cache->cap_ref);
    if (need > (size_t)RKV_NOALLOC_SCRATCH_BYTES) return RKV_ERR_WORKSPACE;
    void* ws = nullptr;
    const rkv_status st = device_scratch(&ws);
    if (st != RKV_OK) return st;
    return rkv_encode_ex(cfg, w, cache, kv, kv_len, rows, pos, n, ws, (size_t)RKV_NOALLOC_SCRATCH_BYTES, stream,
                         nullptr);
}
