// Internal helpers shared by the libpvc translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pvc.h"

namespace pvc {

// Launch bookkeeping: every entry point checks the launch and maps a HIP
// failure to PVC_ERR_HIP.
inline pvc_status launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? PVC_OK : PVC_ERR_HIP;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Number of compute units of the current device, cached per device.
int device_cu_count();

// 256-byte alignment for every region carved out of a caller workspace.
constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Device error word update (no-op for a NULL word).
__device__ inline void raise_error(uint32_t* word, uint32_t bits) {
    if (word != nullptr && bits != 0u) atomicOr(word, bits);
}

// bf16 <-> fp32 (bit patterns).  fp32 -> bf16 rounds to nearest even; inputs
// here are finite.
__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// Binary search: the largest r in [0, nseg) with cu[r] <= i, for a sorted cu.
// With a malformed cu the result is still in [0, nseg).
__device__ inline int32_t upper_segment(const int32_t* __restrict__ cu, int32_t nseg, int64_t i) {
    int32_t lo = 0, hi = nseg - 1;
    while (lo < hi) {
        int32_t mid = (lo + hi + 1) >> 1;
        if (int64_t(cu[mid]) <= i) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace pvc
