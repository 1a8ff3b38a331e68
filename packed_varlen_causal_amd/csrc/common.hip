// Status strings, version and cached device properties for libpvc.
#include <mutex>
#include <unordered_map>

#include "pvc_internal.h"

namespace pvc {

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    static std::mutex mu;
    static std::unordered_map<int, int> cache;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    cache[dev] = prop.multiProcessorCount;
    return prop.multiProcessorCount;
}

}  // namespace pvc

extern "C" const char* pvc_status_string(pvc_status status) {
    switch (status) {
        case PVC_OK: return "ok";
        case PVC_ERR_NULL: return "a required pointer is NULL";
        case PVC_ERR_INVALID_ARG: return "an argument is out of range";
        case PVC_ERR_UNSUPPORTED: return "unsupported shape (head_dim or layout)";
        case PVC_ERR_WORKSPACE: return "workspace missing or too small";
        case PVC_ERR_HIP: return "HIP runtime error";
        case PVC_ERR_SCRATCH_LIMIT: return "more tokens than the allocation-free entry point's static scratch holds";
        default: return "unknown status";
    }
}

extern "C" const char* pvc_version(void) { return "pvc 0.1.0 gfx950"; }
