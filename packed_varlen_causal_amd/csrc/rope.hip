// Rotary position embedding over a packed THD buffer with positions reset per
// segment ([vllbc] THD RoPE recovers local positions from cu_seqlens;
// [charlestar] "nine tokens, three identities": p_i = i - cu_r; [opworld]
// "pitfall two": reset positions per document).
//
// Rotate-half pairing (j, j + d/2), or with the interleaved flag the pairing
// (2j, 2j + 1) of the RoFormer construction; angle theta_j = fp32(p) * f_j with the fp32
// frequency table f_j = base^(-2j/d) computed on the host in double.  The angle
// stays that one fp32 product; sin, cos and the rotation are evaluated in
// double and the result is rounded once to bf16.  fp32 rotation would lose
// the result's leading bits whenever x_j cos and x_{j+d/2} sin nearly cancel;
// in double the single bf16 rounding is the only one that matters.  The kernel
// is bound by HBM traffic, and an fp64 FMA costs the same issue slot as an
// unpacked fp32 one on this chip, so the wider arithmetic is free here.
//
// Double -> bf16 rounding: round to odd at fp32 precision (24 bits), then
// round to nearest even at bf16 precision (8 bits); with at least two spare
// bits the pair equals one direct round-to-nearest-even of the double.
//
// Work layout: one thread owns one token, eight consecutive pairs (16 bytes of
// each half-row; interleaved: four pairs, one 16-byte piece) and
// kHeadsPerThread heads of q and of k.  It evaluates its
// eight sin/cos pairs once and streams the heads; the d/16 threads of a token
// together read and write whole 2*d-byte head rows, so every access is a
// coalesced 16-byte vector.  The kernel moves 2 B in + 2 B out per element and
// is bound by HBM bandwidth.
#include <math.h>

#include "pvc_internal.h"

namespace pvc {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kHeadsPerThread = 8;
constexpr int kMaxHalf = 128;

struct RopeFreqs {
    float f[kMaxHalf];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Round a double to bf16, nearest even, through fp32 round-to-odd.
__device__ inline uint32_t f64_to_bf16_bits(double y) {
    const float f = (float)y;                          // nearest even at fp32
    uint32_t fb = __float_as_uint(f);
    const double back = (double)f;
    if (back != y) {
        if (fabs(back) > fabs(y)) fb -= 1u;            // undo an outward rounding: truncate
        fb |= 1u;                                      // sticky bit: round to odd
    }
    fb += 0x7FFFu + ((fb >> 16) & 1u);                 // nearest even at bf16
    return fb >> 16;
}

// Round a double to fp16, nearest even (subnormals included), through fp32
// round-to-odd (24 bits against fp16's 11).
__device__ inline uint32_t f64_to_f16_bits(double y) {
    const float f = (float)y;
    uint32_t fb = __float_as_uint(f);
    const double back = (double)f;
    if (back != y) {
        if (fabs(back) > fabs(y)) fb -= 1u;
        fb |= 1u;
    }
    const _Float16 h = (_Float16)__uint_as_float(fb);     // v_cvt_f16_f32: nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// 16-bit element codec: bf16 (F16 = false) or fp16.
template <bool F16>
__device__ inline double in16(uint16_t b) {
    if constexpr (F16) return (double)(float)__builtin_bit_cast(_Float16, b);
    else return (double)bf16_to_f32(b);
}
template <bool F16>
__device__ inline uint32_t out16(double y) {
    if constexpr (F16) return f64_to_f16_bits(y);
    else return f64_to_bf16_bits(y);
}

template <bool F16>
__device__ inline void rotate8(const u32x4& a, const u32x4& b, const double* c, const double* s,
                               u32x4& ya, u32x4& yb) {
    // a holds x_j .. x_{j+7}, b holds x_{j+d/2} .. x_{j+d/2+7}; two bf16 per dword
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t ra = 0, rb = 0;
#pragma unroll
        for (int hlf = 0; hlf < 2; ++hlf) {
            const int e = 2 * w + hlf;
            const double x1 = in16<F16>(uint16_t(a[w] >> (16 * hlf)));
            const double x2 = in16<F16>(uint16_t(b[w] >> (16 * hlf)));
            const double y1 = x1 * c[e] - x2 * s[e];
            const double y2 = x2 * c[e] + x1 * s[e];
            ra |= out16<F16>(y1) << (16 * hlf);
            rb |= out16<F16>(y2) << (16 * hlf);
        }
        ya[w] = ra;
        yb[w] = rb;
    }
}

// Interleaved pairs: a holds x_{2j} .. x_{2j+7} (pairs j .. j+3, one per dword).
template <bool F16>
__device__ inline u32x4 rotate4_interleaved(const u32x4& a, const double* c, const double* s) {
    u32x4 y;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const double x1 = in16<F16>(uint16_t(a[w]));
        const double x2 = in16<F16>(uint16_t(a[w] >> 16));
        y[w] = out16<F16>(x1 * c[w] - x2 * s[w]) | (out16<F16>(x2 * c[w] + x1 * s[w]) << 16);
    }
    return y;
}

// head_dim a multiple of 16: vectorized path.
template <bool INTERLEAVED, bool F16>
__global__ __launch_bounds__(kRopeThreads) void rope_vec_kernel(
        const uint16_t* q_in, uint16_t* q_out, const uint16_t* k_in, uint16_t* k_out, int64_t T,
        int32_t H, int32_t D, const int32_t* __restrict__ cu, int32_t nseg, RopeFreqs freqs,
        uint32_t* dev_error) {
    // 16-byte pieces a thread owns per head row: two 8-pair halves (rotate-half)
    // or one 4-pair piece (interleaved)
    const int chunks = INTERLEAVED ? D >> 3 : D >> 4;
    const int hgroups = (H + kHeadsPerThread - 1) / kHeadsPerThread;
    const int64_t gid = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
    const int64_t per_token = (int64_t)chunks * hgroups;
    const int64_t i = gid / per_token;
    if (i >= T) return;
    const int rem = (int)(gid - i * per_token);
    const int hg = rem / chunks;
    const int ch = rem - hg * chunks;

    const int32_t r = upper_segment(cu, nseg, i);
    const int64_t st = cu[r], en = cu[r + 1];
    const bool ok = st <= i && i < en;
    if (!ok && ch == 0 && hg == 0) raise_error(dev_error, i >= en ? PVC_DEV_TOTAL : PVC_DEV_NOT_INCREASING);
    const float p = ok ? (float)(i - st) : 0.0f;     // malformed cu: identity (copy through)

    constexpr int NP = INTERLEAVED ? 4 : 8;           // pairs per thread
    double c[NP], s[NP];
    const int j0 = ch * NP;
#pragma unroll
    for (int e = 0; e < NP; ++e) {
        const float theta = p * freqs.f[j0 + e];      // one fp32 product
        sincos((double)theta, &s[e], &c[e]);
    }
    const int half = D >> 1;
    const int h_lo = hg * kHeadsPerThread;
    const int h_hi = min(H, h_lo + kHeadsPerThread);
#pragma unroll 1
    for (int t = 0; t < 2; ++t) {
        const uint16_t* src = t == 0 ? q_in : k_in;
        uint16_t* dst = t == 0 ? q_out : k_out;
        if (src == nullptr) break;
        for (int h = h_lo; h < h_hi; ++h) {
            const int64_t row = (i * H + h) * (int64_t)D;
            if constexpr (INTERLEAVED) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(src + row + 2 * j0);
                *reinterpret_cast<u32x4*>(dst + row + 2 * j0) = rotate4_interleaved<F16>(a, c, s);
            } else {
                const u32x4 a = *reinterpret_cast<const u32x4*>(src + row + j0);
                const u32x4 b = *reinterpret_cast<const u32x4*>(src + row + half + j0);
                u32x4 ya, yb;
                rotate8<F16>(a, b, c, s, ya, yb);
                *reinterpret_cast<u32x4*>(dst + row + j0) = ya;
                *reinterpret_cast<u32x4*>(dst + row + half + j0) = yb;
            }
        }
    }
}

// Any even head_dim: one thread per (token, pair), heads looped.
template <bool INTERLEAVED, bool F16>
__global__ __launch_bounds__(kRopeThreads) void rope_scalar_kernel(
        const uint16_t* q_in, uint16_t* q_out, const uint16_t* k_in, uint16_t* k_out, int64_t T,
        int32_t H, int32_t D, const int32_t* __restrict__ cu, int32_t nseg, RopeFreqs freqs,
        uint32_t* dev_error) {
    const int half = D >> 1;
    const int64_t gid = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
    const int64_t i = gid / half;
    if (i >= T) return;
    const int j = (int)(gid - i * half);
    const int32_t r = upper_segment(cu, nseg, i);
    const int64_t st = cu[r], en = cu[r + 1];
    const bool ok = st <= i && i < en;
    if (!ok && j == 0) raise_error(dev_error, i >= en ? PVC_DEV_TOTAL : PVC_DEV_NOT_INCREASING);
    const float p = ok ? (float)(i - st) : 0.0f;
    const float theta = p * freqs.f[j];
    double sn, cs;
    sincos((double)theta, &sn, &cs);
    for (int t = 0; t < 2; ++t) {
        const uint16_t* src = t == 0 ? q_in : k_in;
        uint16_t* dst = t == 0 ? q_out : k_out;
        if (src == nullptr) break;
        for (int h = 0; h < H; ++h) {
            const int64_t row = (i * H + h) * (int64_t)D;
            const int64_t e1 = INTERLEAVED ? row + 2 * j : row + j;
            const int64_t e2 = INTERLEAVED ? row + 2 * j + 1 : row + half + j;
            const double x1 = in16<F16>(src[e1]);
            const double x2 = in16<F16>(src[e2]);
            dst[e1] = (uint16_t)out16<F16>(x1 * cs - x2 * sn);
            dst[e2] = (uint16_t)out16<F16>(x2 * cs + x1 * sn);
        }
    }
}

}  // namespace
}  // namespace pvc

using namespace pvc;

namespace {

template <bool INTERLEAVED, bool F16>
void rope_launch(bool vec, int64_t nblk, hipStream_t s, const uint16_t* qi, uint16_t* qo, const uint16_t* ki,
                 uint16_t* ko, int64_t T, int32_t H, int32_t D, const int32_t* cu, int32_t nseg,
                 const RopeFreqs& freqs, uint32_t* dev_error) {
    if (vec)
        hipLaunchKernelGGL((rope_vec_kernel<INTERLEAVED, F16>), dim3((unsigned)nblk), dim3(kRopeThreads), 0, s, qi,
                           qo, ki, ko, T, H, D, cu, nseg, freqs, dev_error);
    else
        hipLaunchKernelGGL((rope_scalar_kernel<INTERLEAVED, F16>), dim3((unsigned)nblk), dim3(kRopeThreads), 0, s,
                           qi, qo, ki, ko, T, H, D, cu, nseg, freqs, dev_error);
}

pvc_status rope_apply(const void* q_in, void* q_out, const void* k_in, void* k_out, int64_t total_tokens,
                      int32_t heads, int32_t head_dim, const int32_t* cu_seqlens, int32_t nseg, float base,
                      bool interleaved, bool f16, uint32_t* dev_error, void* stream) {
    if (q_in == nullptr || q_out == nullptr || cu_seqlens == nullptr) return PVC_ERR_NULL;
    if ((k_in == nullptr) != (k_out == nullptr)) return PVC_ERR_NULL;
    if (total_tokens < 1 || total_tokens > 0x7fffffffLL || heads < 1 || nseg < 1)
        return PVC_ERR_INVALID_ARG;
    if (!(base > 0.0f) || base != base) return PVC_ERR_INVALID_ARG;
    if (head_dim < 2 || head_dim > 2 * kMaxHalf || (head_dim & 1)) return PVC_ERR_UNSUPPORTED;

    RopeFreqs freqs;
    for (int j = 0; j < head_dim / 2; ++j)
        freqs.f[j] = (float)pow((double)base, -2.0 * j / (double)head_dim);
    hipStream_t s = as_stream(stream);
    const auto* qi = static_cast<const uint16_t*>(q_in);
    auto* qo = static_cast<uint16_t*>(q_out);
    const auto* ki = static_cast<const uint16_t*>(k_in);
    auto* ko = static_cast<uint16_t*>(k_out);
    const bool aligned = ((reinterpret_cast<uintptr_t>(q_in) | reinterpret_cast<uintptr_t>(q_out) |
                           reinterpret_cast<uintptr_t>(k_in) | reinterpret_cast<uintptr_t>(k_out)) & 15u) == 0;
    const bool vec = head_dim % 16 == 0 && aligned;
    int64_t threads;
    if (vec) {
        const int64_t hgroups = (heads + kHeadsPerThread - 1) / kHeadsPerThread;
        threads = total_tokens * (head_dim / (interleaved ? 8 : 16)) * hgroups;
    } else {
        threads = total_tokens * (head_dim / 2);
    }
    const int64_t nblk = (threads + kRopeThreads - 1) / kRopeThreads;
    const int64_t T = total_tokens;
    if (interleaved) {
        if (f16) rope_launch<true, true>(vec, nblk, s, qi, qo, ki, ko, T, heads, head_dim, cu_seqlens, nseg, freqs, dev_error);
        else rope_launch<true, false>(vec, nblk, s, qi, qo, ki, ko, T, heads, head_dim, cu_seqlens, nseg, freqs, dev_error);
    } else {
        if (f16) rope_launch<false, true>(vec, nblk, s, qi, qo, ki, ko, T, heads, head_dim, cu_seqlens, nseg, freqs, dev_error);
        else rope_launch<false, false>(vec, nblk, s, qi, qo, ki, ko, T, heads, head_dim, cu_seqlens, nseg, freqs, dev_error);
    }
    return launch_status();
}

}  // namespace

extern "C" pvc_status pvc_rope_thd_apply(const void* q_in, void* q_out, const void* k_in, void* k_out,
                                         int64_t total_tokens, int32_t heads, int32_t head_dim,
                                         const int32_t* cu_seqlens, int32_t nseg, float base,
                                         uint32_t* dev_error, void* stream) {
    return rope_apply(q_in, q_out, k_in, k_out, total_tokens, heads, head_dim, cu_seqlens, nseg, base, false,
                      false, dev_error, stream);
}

extern "C" pvc_status pvc_rope_thd_apply_interleaved(const void* q_in, void* q_out, const void* k_in,
                                                     void* k_out, int64_t total_tokens, int32_t heads,
                                                     int32_t head_dim, const int32_t* cu_seqlens, int32_t nseg,
                                                     float base, uint32_t* dev_error, void* stream) {
    return rope_apply(q_in, q_out, k_in, k_out, total_tokens, heads, head_dim, cu_seqlens, nseg, base, true,
                      false, dev_error, stream);
}

extern "C" pvc_status pvc_rope_thd_apply_ex(const void* q_in, void* q_out, const void* k_in, void* k_out,
                                            int64_t total_tokens, int32_t heads, int32_t head_dim,
                                            const int32_t* cu_seqlens, int32_t nseg, float base, int32_t flags,
                                            uint32_t* dev_error, void* stream) {
    if (flags & ~(PVC_ROPE_INTERLEAVED | PVC_ROPE_F16)) return PVC_ERR_INVALID_ARG;
    return rope_apply(q_in, q_out, k_in, k_out, total_tokens, heads, head_dim, cu_seqlens, nseg, base,
                      (flags & PVC_ROPE_INTERLEAVED) != 0, (flags & PVC_ROPE_F16) != 0, dev_error, stream);
}
