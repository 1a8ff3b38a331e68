// Packed cross-entropy over the rows of a THD buffer, for gfx950.
//
// For logits z [T, V] (bf16, fp16 or fp32, row stride ld) and the pre-shifted labels
// that pack_build writes (label[i] is the token row i predicts; the ignore
// index on each segment's last row and on pad segments), this computes what
// [charlestar] "cross-boundary prediction pairs" keeps for the training loop:
// the cross-entropy summed over the valid targets and the int64 count of
// valid targets, and optionally
//   - each row's loss (0 for a row that is not a target),
//   - per-segment loss sums S_r and target counts n_r over cu_seqlens, from
//     which the caller forms either average of [charlestar] "packing should
//     not choose the weight of long samples",
//   - the gradient of the loss sum, scale * (softmax(z_i) - onehot(y_i)), zero
//     on ignored rows, fused into the same pass (in place over the logits if
//     the caller wants).
//
// Kernels:
//   ce_row_kernel      one 256-thread workgroup per row.  A row of up to 16
//                      16-byte vectors per thread is loaded once and kept in
//                      registers: each thread's max, then exp2 of every
//                      element against it (fp32, the scale log2(e) folded into
//                      one FMA), and the gradient from the same registers.
//                      Longer rows stream in chunks with a running (max, sum)
//                      and are re-read (from L2) for the gradient.  The
//                      (max, sum) pairs of the 256 threads meet through lane
//                      shuffles and LDS; loss = max + ln(sum) - z_y.
//                      HBM-bound: 2V bytes per bf16 row read once (plus 2V
//                      written with the gradient).
//   ce_reduce_kernel   4096 rows per workgroup: fp64 sum of the row losses and
//                      int64 count of valid labels, in a fixed order.
//   ce_final_kernel    one workgroup adds the partials in a fixed order.
//   ce_segment_kernel  one wave per segment: fp64 sum and int64 count over
//                      [cu_r, cu_r+1), in a fixed order.
// No floating-point atomics: the results do not depend on scheduling.
#include <math.h>

#include "pvc_internal.h"

namespace pvc {
namespace {

constexpr int kCeThreads = 256;
constexpr int kCeRowsPerBlock = 4096;        // rows per ce_reduce_kernel workgroup
constexpr int kCeChunk = 4;                  // 16-byte vectors per thread per chunk
constexpr int kCeResident = 16;              // vectors per thread of a register-resident row
constexpr float kL2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Values per 16-byte vector and their fp32 form; DT is the logits' element
// type code (PVC_OUT_BF16, PVC_OUT_F32 or PVC_OUT_F16).
template <int DT>
struct Vec;
template <>
struct Vec<PVC_OUT_BF16> {
    static constexpr int N = 8;
    __device__ static void unpack(const u32x4& w, float (&x)[N]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
    __device__ static float scalar(const void* p, int64_t i) {
        return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    }
};
template <>
struct Vec<PVC_OUT_F16> {
    static constexpr int N = 8;
    __device__ static float h(uint32_t b) { return (float)__builtin_bit_cast(_Float16, uint16_t(b)); }
    __device__ static void unpack(const u32x4& w, float (&x)[N]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = h(w[i] & 0xFFFFu);
            x[2 * i + 1] = h(w[i] >> 16);
        }
    }
    __device__ static float scalar(const void* p, int64_t i) { return h(static_cast<const uint16_t*>(p)[i]); }
};
template <>
struct Vec<PVC_OUT_F32> {
    static constexpr int N = 4;
    __device__ static void unpack(const u32x4& w, float (&x)[N]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
    }
    __device__ static float scalar(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
};

// Running (max, sum of exp(x - max)) of a set of values; max = -inf means
// "nothing finite seen yet" and keeps sum at 0.
struct MaxSum {
    float m = -INFINITY;
    float s = 0.0f;
};

__device__ inline float safe_base(float m) { return m == -INFINITY ? 0.0f : m; }

__device__ inline MaxSum merge(MaxSum a, MaxSum b) {
    const float m = fmaxf(a.m, b.m);
    const float base = safe_base(m);
    MaxSum r;
    r.m = m;
    r.s = a.s * __builtin_amdgcn_exp2f((a.m - base) * kL2e) + b.s * __builtin_amdgcn_exp2f((b.m - base) * kL2e);
    return r;
}

// Merge across the 256 threads of the workgroup; every thread gets the result.
__device__ inline MaxSum block_merge(MaxSum v, float* shm, float* shs) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        MaxSum o;
        o.m = __shfl_xor(v.m, off);
        o.s = __shfl_xor(v.s, off);
        v = merge(v, o);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        shm[wave] = v.m;
        shs[wave] = v.s;
    }
    __syncthreads();
    MaxSum r;
    r.m = shm[0];
    r.s = shs[0];
#pragma unroll
    for (int w = 1; w < kCeThreads / 64; ++w) {
        MaxSum o;
        o.m = shm[w];
        o.s = shs[w];
        r = merge(r, o);
    }
    return r;
}

// A row is a target when its label is not the ignore index and names a
// class: the rule of pack_build's loss mask (label != ignore index), with
// out-of-range labels excluded as well.
__device__ inline bool ce_target(int32_t y, int32_t ignore, int32_t V) { return y != ignore && y >= 0 && y < V; }

struct CeParams {
    const void* logits;
    int64_t ld;
    const int32_t* labels;
    int64_t T;
    int32_t V;
    int32_t ignore;
    float* row_loss;             // [T] (caller's or the workspace)
    void* grad;                  // nullable
    int64_t grad_ld;
    float grad_scale;
    uint32_t* dev_error;
};

// One row per workgroup.  VEC: the row start is 16-byte aligned, so the first
// floor(V / N) * N values are read as vectors and the rest one by one.
// RES: the vectors of the row fit in registers (at most kCeResident per
// thread): they are loaded once, the thread's max is taken over all of them
// before any exponential, and the gradient pass reads them from registers
// instead of from memory again.
// A 16-bit gradient value: bf16 or fp16, nearest even.
template <int GRAD>
__device__ inline uint32_t enc16(float g) {
    if constexpr (GRAD == 3) return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)g);
    else return (uint32_t)f32_to_bf16_rne(g);
}

template <int IN_DT, int GRAD /* 0 none, 1 bf16, 2 fp32, 3 fp16 */, bool RES>
__global__ __launch_bounds__(kCeThreads) void ce_row_kernel(CeParams p, bool vec) {
    using VT = Vec<IN_DT>;
    constexpr bool IN_F32 = IN_DT == PVC_OUT_F32;
    constexpr int N = VT::N;
    __shared__ float shm[kCeThreads / 64], shs[kCeThreads / 64];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int V = p.V;
    const char* rowp = static_cast<const char*>(p.logits) + row * p.ld * (IN_F32 ? 4 : 2);
    const int32_t y = p.labels[row];
    const bool valid = ce_target(y, p.ignore, V);
    if (tid == 0 && y != p.ignore && !(y >= 0 && y < V)) raise_error(p.dev_error, PVC_DEV_LABEL);

    // ---- pass 1: running max and sum of exp
    MaxSum acc;
    const int nvec = vec ? V / N : 0;
    const u32x4* vp = reinterpret_cast<const u32x4*>(rowp);
    u32x4 res[RES ? kCeResident : 1];
    if constexpr (RES) {
#pragma unroll
        for (int i = 0; i < kCeResident; ++i) {
            const int vi = i * kCeThreads + tid;
            res[i] = vi < nvec ? vp[vi] : u32x4{0u, 0u, 0u, 0u};
        }
        float cm = -INFINITY;
#pragma unroll
        for (int i = 0; i < kCeResident; ++i) {
            if (i * kCeThreads + tid < nvec) {
                float x[N];
                VT::unpack(res[i], x);
#pragma unroll
                for (int e = 0; e < N; ++e) cm = fmaxf(cm, x[e]);
            }
        }
        const float nb = -safe_base(cm) * kL2e;
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < kCeResident; ++i) {
            if (i * kCeThreads + tid < nvec) {
                float x[N];
                VT::unpack(res[i], x);
#pragma unroll
                for (int e = 0; e < N; ++e) s += __builtin_amdgcn_exp2f(fmaf(x[e], kL2e, nb));
            }
        }
        acc.m = cm;
        acc.s = s;
    }
    for (int c0 = 0; !RES && c0 < nvec; c0 += kCeChunk * kCeThreads) {
        float x[kCeChunk][N];
        float cm = -INFINITY;
#pragma unroll
        for (int i = 0; i < kCeChunk; ++i) {
            const int vi = c0 + i * kCeThreads + tid;
            if (vi < nvec) {
                VT::unpack(vp[vi], x[i]);
            } else {
#pragma unroll
                for (int e = 0; e < N; ++e) x[i][e] = -INFINITY;
            }
#pragma unroll
            for (int e = 0; e < N; ++e) cm = fmaxf(cm, x[i][e]);
        }
        const float mn = fmaxf(acc.m, cm);
        const float base = safe_base(mn);
        float s = acc.s * __builtin_amdgcn_exp2f((acc.m - base) * kL2e);
        const float nb = -base * kL2e;
#pragma unroll
        for (int i = 0; i < kCeChunk; ++i)
#pragma unroll
            for (int e = 0; e < N; ++e) s += __builtin_amdgcn_exp2f(fmaf(x[i][e], kL2e, nb));
        acc.m = mn;
        acc.s = s;
    }
    for (int i = nvec * N + tid; i < V; i += kCeThreads) {
        MaxSum one;
        one.m = VT::scalar(rowp, i);
        one.s = 1.0f;
        acc = merge(acc, one);
    }
    // the target's logit is read before the barrier: with the gradient
    // written in place, pass 2 may overwrite it
    const float zy = (tid == 0 && valid) ? VT::scalar(rowp, y) : 0.0f;
    const MaxSum tot = block_merge(acc, shm, shs);
    const float base = safe_base(tot.m);
    const float l2s = __builtin_amdgcn_logf(tot.s);          // log2 of sum exp(z - base)
    if (tid == 0) p.row_loss[row] = valid ? (base + l2s * kLn2) - zy : 0.0f;

    // ---- pass 2: gradient scale * (softmax - onehot), zero on ignored rows
    if constexpr (GRAD != 0) {
        const float sc = valid ? p.grad_scale : 0.0f;
        char* growp = static_cast<char*>(p.grad) + row * p.grad_ld * (GRAD == 2 ? 4 : 2);
        auto gval = [&](float x, int idx) -> float {
            const float pr = __builtin_amdgcn_exp2f(fmaf(x - base, kL2e, -l2s));
            return sc * (pr - (idx == y ? 1.0f : 0.0f));
        };
        auto emit = [&](int vi, const u32x4& wv) {
            float x[N];
            VT::unpack(wv, x);
            if constexpr (GRAD == 2) {
#pragma unroll
                for (int q = 0; q < N / 4; ++q)
                    reinterpret_cast<f32x4*>(growp)[vi * (N / 4) + q] =
                            f32x4{gval(x[4 * q], vi * N + 4 * q), gval(x[4 * q + 1], vi * N + 4 * q + 1),
                                  gval(x[4 * q + 2], vi * N + 4 * q + 2), gval(x[4 * q + 3], vi * N + 4 * q + 3)};
            } else {
                uint32_t w[N / 2];
#pragma unroll
                for (int q = 0; q < N / 2; ++q)
                    w[q] = enc16<GRAD>(gval(x[2 * q], vi * N + 2 * q)) |
                           (enc16<GRAD>(gval(x[2 * q + 1], vi * N + 2 * q + 1)) << 16);
                if constexpr (N == 8) {
                    reinterpret_cast<u32x4*>(growp)[vi] = u32x4{w[0], w[1], w[2], w[3]};
                } else {
                    reinterpret_cast<uint32_t*>(growp)[2 * vi] = w[0];
                    reinterpret_cast<uint32_t*>(growp)[2 * vi + 1] = w[1];
                }
            }
        };
        if constexpr (RES) {
#pragma unroll
            for (int i = 0; i < kCeResident; ++i)
                if (i * kCeThreads + tid < nvec) emit(i * kCeThreads + tid, res[i]);
        } else {
            for (int vi = tid; vi < nvec; vi += kCeThreads) emit(vi, vp[vi]);
        }
        for (int i = nvec * N + tid; i < V; i += kCeThreads) {
            const float g = gval(VT::scalar(rowp, i), i);
            if constexpr (GRAD == 2) reinterpret_cast<float*>(growp)[i] = g;
            else reinterpret_cast<uint16_t*>(growp)[i] = (uint16_t)enc16<GRAD>(g);
        }
    }
}

// fp64 / int64 tree over the 256 threads of a workgroup (fixed order).
__device__ inline void block_sum(double& s, long long& c, double* shs, long long* shc) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        s += __shfl_xor(s, off);
        c += __shfl_xor(c, off);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        shs[wave] = s;
        shc[wave] = c;
    }
    __syncthreads();
    s = shs[0];
    c = shc[0];
#pragma unroll
    for (int w = 1; w < kCeThreads / 64; ++w) {
        s += shs[w];
        c += shc[w];
    }
}

__global__ __launch_bounds__(kCeThreads) void ce_reduce_kernel(const float* __restrict__ row_loss,
                                                               const int32_t* __restrict__ labels, int64_t T,
                                                               int32_t V, int32_t ignore, double* __restrict__ psum,
                                                               long long* __restrict__ pcount) {
    __shared__ double shs[kCeThreads / 64];
    __shared__ long long shc[kCeThreads / 64];
    double s = 0.0;
    long long c = 0;
    const int64_t r0 = (int64_t)blockIdx.x * kCeRowsPerBlock;
    for (int i = threadIdx.x; i < kCeRowsPerBlock; i += kCeThreads) {
        const int64_t r = r0 + i;
        if (r < T) {
            const int32_t y = labels[r];
            s += (double)row_loss[r];
            c += ce_target(y, ignore, V) ? 1 : 0;
        }
    }
    block_sum(s, c, shs, shc);
    if (threadIdx.x == 0) {
        psum[blockIdx.x] = s;
        pcount[blockIdx.x] = c;
    }
}

__global__ __launch_bounds__(kCeThreads) void ce_final_kernel(const double* __restrict__ psum,
                                                              const long long* __restrict__ pcount, int64_t nblk,
                                                              double* __restrict__ loss_sum,
                                                              int64_t* __restrict__ target_count) {
    __shared__ double shs[kCeThreads / 64];
    __shared__ long long shc[kCeThreads / 64];
    double s = 0.0;
    long long c = 0;
    for (int64_t i = threadIdx.x; i < nblk; i += kCeThreads) {
        s += psum[i];
        c += pcount[i];
    }
    block_sum(s, c, shs, shc);
    if (threadIdx.x == 0) {
        *loss_sum = s;
        *target_count = c;
    }
}

// One wave per segment [cu_r, cu_r+1), clamped into [0, T]; malformed cu
// entries set the usual error bits.
__global__ __launch_bounds__(kCeThreads) void ce_segment_kernel(const float* __restrict__ row_loss,
                                                                const int32_t* __restrict__ labels, int64_t T,
                                                                int32_t V, int32_t ignore, const int32_t* __restrict__ cu,
                                                                int32_t nseg, double* __restrict__ seg_loss,
                                                                int64_t* __restrict__ seg_count,
                                                                uint32_t* dev_error) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * (kCeThreads / 64) + (threadIdx.x >> 6);
    if (r >= nseg) return;
    const int64_t a_raw = cu[r], b_raw = cu[r + 1];
    if (lane == 0) {
        uint32_t err = 0;
        if (b_raw <= a_raw) err |= PVC_DEV_NOT_INCREASING;
        if (r == 0 && a_raw != 0) err |= PVC_DEV_CU0;
        if (r == nseg - 1 && b_raw != T) err |= PVC_DEV_TOTAL;
        raise_error(dev_error, err);
    }
    const int64_t a = min<int64_t>(max<int64_t>(a_raw, 0), T);
    const int64_t b = min<int64_t>(max<int64_t>(b_raw, a), T);
    double s = 0.0;
    long long c = 0;
    for (int64_t i = a + lane; i < b; i += 64) {
        const int32_t y = labels[i];
        s += (double)row_loss[i];
        c += ce_target(y, ignore, V) ? 1 : 0;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        s += __shfl_xor(s, off);
        c += __shfl_xor(c, off);
    }
    if (lane == 0) {
        if (seg_loss != nullptr) seg_loss[r] = s;
        if (seg_count != nullptr) seg_count[r] = c;
    }
}

struct CeLayout {
    size_t rows, psum, pcount, total;
    int64_t nblk;
};

CeLayout ce_layout(int64_t T) {
    CeLayout L;
    L.nblk = (T + kCeRowsPerBlock - 1) / kCeRowsPerBlock;
    L.rows = 0;
    L.psum = align_up((size_t)T * sizeof(float));
    L.pcount = L.psum + align_up((size_t)L.nblk * sizeof(double));
    L.total = L.pcount + align_up((size_t)L.nblk * sizeof(long long));
    return L;
}

bool ce_aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

bool ce_overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

template <int IN_DT, bool RES>
void launch_rows2(const CeParams& prm, bool vec, int grad, hipStream_t s) {
    const dim3 g((unsigned)prm.T), b(kCeThreads);
    if (grad == 0) hipLaunchKernelGGL((ce_row_kernel<IN_DT, 0, RES>), g, b, 0, s, prm, vec);
    else if (grad == 1) hipLaunchKernelGGL((ce_row_kernel<IN_DT, 1, RES>), g, b, 0, s, prm, vec);
    else if (grad == 2) hipLaunchKernelGGL((ce_row_kernel<IN_DT, 2, RES>), g, b, 0, s, prm, vec);
    else hipLaunchKernelGGL((ce_row_kernel<IN_DT, 3, RES>), g, b, 0, s, prm, vec);
}

template <int IN_DT>
void launch_rows(const CeParams& prm, bool vec, int grad, hipStream_t s) {
    constexpr int N = IN_DT == PVC_OUT_F32 ? 4 : 8;
    if (vec && prm.V / N <= kCeResident * kCeThreads) launch_rows2<IN_DT, true>(prm, vec, grad, s);
    else launch_rows2<IN_DT, false>(prm, vec, grad, s);
}

inline bool ce_dtype_ok(int32_t t) { return t == PVC_OUT_BF16 || t == PVC_OUT_F32 || t == PVC_OUT_F16; }

}  // namespace
}  // namespace pvc

using namespace pvc;

extern "C" size_t pvc_ce_workspace_size(int64_t total_tokens) {
    if (total_tokens < 1 || total_tokens > 0x7fffffffLL) return 0;
    return ce_layout(total_tokens).total;
}

extern "C" pvc_status pvc_packed_ce_loss(const void* logits, int32_t logits_dtype, int64_t ld,
                                         const int32_t* labels, int64_t total_tokens, int32_t vocab,
                                         int32_t ignore_index, const int32_t* cu_seqlens, int32_t nseg,
                                         double* loss_sum, int64_t* target_count, float* row_loss,
                                         double* seg_loss, int64_t* seg_count, void* grad, int32_t grad_dtype,
                                         int64_t grad_ld, float grad_scale, void* workspace,
                                         size_t workspace_bytes, uint32_t* dev_error, void* stream) {
    if (logits == nullptr || labels == nullptr || loss_sum == nullptr || target_count == nullptr ||
        workspace == nullptr)
        return PVC_ERR_NULL;
    if ((seg_loss != nullptr || seg_count != nullptr) && cu_seqlens == nullptr) return PVC_ERR_NULL;
    if (total_tokens < 1 || total_tokens > 0x7fffffffLL || vocab < 1 || ld < vocab) return PVC_ERR_INVALID_ARG;
    if (!ce_dtype_ok(logits_dtype)) return PVC_ERR_INVALID_ARG;
    if (grad != nullptr) {
        if (!ce_dtype_ok(grad_dtype)) return PVC_ERR_INVALID_ARG;
        if (grad_ld < vocab || !isfinite(grad_scale)) return PVC_ERR_INVALID_ARG;
    }
    if (cu_seqlens != nullptr && (nseg < 1 || nseg > total_tokens)) return PVC_ERR_INVALID_ARG;
    const CeLayout L = ce_layout(total_tokens);
    if (workspace_bytes < L.total) return PVC_ERR_WORKSPACE;
    if (!ce_aligned16(workspace)) return PVC_ERR_INVALID_ARG;
    const size_t esz = logits_dtype == PVC_OUT_F32 ? 4 : 2;
    const size_t in_bytes = (size_t)((total_tokens - 1) * ld + vocab) * esz;
    if (grad != nullptr) {
        const size_t gsz = grad_dtype == PVC_OUT_F32 ? 4 : 2;
        const size_t g_bytes = (size_t)((total_tokens - 1) * grad_ld + vocab) * gsz;
        // in place (the same buffer, dtype and stride) or apart from the logits
        const bool same = grad == logits && grad_dtype == logits_dtype && grad_ld == ld;
        if (!same && ce_overlaps(grad, g_bytes, logits, in_bytes)) return PVC_ERR_INVALID_ARG;
        if (ce_overlaps(grad, g_bytes, workspace, L.total)) return PVC_ERR_INVALID_ARG;
    }
    char* ws = static_cast<char*>(workspace);
    CeParams prm{};
    prm.logits = logits;
    prm.ld = ld;
    prm.labels = labels;
    prm.T = total_tokens;
    prm.V = vocab;
    prm.ignore = ignore_index;
    prm.row_loss = row_loss != nullptr ? row_loss : reinterpret_cast<float*>(ws + L.rows);
    prm.grad = grad;
    prm.grad_ld = grad_ld;
    prm.grad_scale = grad_scale;
    prm.dev_error = dev_error;
    // 16-byte vectors when every row start (of the logits and of the
    // gradient) is 16-byte aligned, else one value at a time
    const bool vec = ce_aligned16(logits) && (ld * esz) % 16 == 0 &&
                     (grad == nullptr ||
                      (ce_aligned16(grad) && (grad_ld * (grad_dtype == PVC_OUT_F32 ? 4 : 2)) % 16 == 0));
    const int gmode = grad == nullptr ? 0 : grad_dtype == PVC_OUT_F32 ? 2 : grad_dtype == PVC_OUT_F16 ? 3 : 1;
    hipStream_t s = as_stream(stream);
    if (logits_dtype == PVC_OUT_F32) launch_rows<PVC_OUT_F32>(prm, vec, gmode, s);
    else if (logits_dtype == PVC_OUT_F16) launch_rows<PVC_OUT_F16>(prm, vec, gmode, s);
    else launch_rows<PVC_OUT_BF16>(prm, vec, gmode, s);
    double* psum = reinterpret_cast<double*>(ws + L.psum);
    long long* pcount = reinterpret_cast<long long*>(ws + L.pcount);
    hipLaunchKernelGGL(ce_reduce_kernel, dim3((unsigned)L.nblk), dim3(kCeThreads), 0, s, prm.row_loss, labels,
                       total_tokens, vocab, ignore_index, psum, pcount);
    hipLaunchKernelGGL(ce_final_kernel, dim3(1), dim3(kCeThreads), 0, s, psum, pcount, L.nblk, loss_sum,
                       target_count);
    if (seg_loss != nullptr || seg_count != nullptr) {
        const unsigned blocks = (unsigned)((nseg + kCeThreads / 64 - 1) / (kCeThreads / 64));
        hipLaunchKernelGGL(ce_segment_kernel, dim3(blocks), dim3(kCeThreads), 0, s, prm.row_loss, labels,
                           total_tokens, vocab, ignore_index, cu_seqlens, nseg, seg_loss, seg_count, dev_error);
    }
    return launch_status();
}
