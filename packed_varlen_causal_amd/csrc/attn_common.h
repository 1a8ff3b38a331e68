// Shared pieces of the attention kernels (forward and backward) for gfx950:
// tile geometry, the plan layout, MFMA and lane helpers, the untracked
// global -> LDS load, and the LDS swizzles.
#pragma once

#include <math.h>

#include <type_traits>

#include "pvc_internal.h"

namespace pvc {
namespace attn {

constexpr int kWaves = 4;       // waves per workgroup, 32 query rows each
constexpr int kBM = 32 * kWaves; // query rows per tile
constexpr int kBN = 32;         // keys per LDS stage (32 or 64)
constexpr int kRing = 2;        // LDS stages per K/V ring; kRing - 1 are in flight
constexpr int kThreads = 64 * kWaves;
constexpr int kCheckThreads = 1024;
constexpr int kNumXcd = 8;
constexpr int32_t kPlanMagic = 0x31435650;   // "PVC1"

// Plan header (int32 slots).  HDR_FOLDED: the plan of separate query / key
// boundaries, whose row ranges already hold the causal limit (the kernels
// then run without their own diagonal); HDR_TK: rows of K and V;
// HDR_MAXLEN: the longest (query) segment, which picks the forward's item order.
enum { HDR_MAGIC = 0, HDR_T = 1, HDR_CAUSAL = 2, HDR_NTILES = 3, HDR_ERR = 4, HDR_VALID = 5, HDR_FOLDED = 6,
       HDR_TK = 7, HDR_MAXLEN = 8 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct PlanLayout {
    size_t header, rows, qseg, order, total;
    int64_t ntiles;
};

inline PlanLayout plan_layout(int64_t T) {
    PlanLayout L;
    L.ntiles = (T + kBM - 1) / kBM;
    size_t off = 0;
    L.header = off;
    off += align_up(16 * sizeof(int32_t));
    L.rows = off;
    off += align_up((size_t)T * sizeof(int2));
    // the query segment of each row, for plans whose row ranges are key rows
    // (tile order only)
    L.qseg = off;
    off += align_up((size_t)T * sizeof(int2));
    // the start order of the 32-row query tiles (grouped-head forward over a
    // plan of separate query / key boundaries)
    L.order = off;
    off += align_up((size_t)((T + 31) / 32) * sizeof(int32_t));
    L.total = off;
    return L;
}

typedef __attribute__((address_space(3))) char lds_char;

// One direct global -> LDS load of 16 bytes per lane: lane l's bytes at
// base + off land at LDS address lds + 16 l.  Written as inline assembly so
// that the compiler does not track it: with the builtin, it waits for every
// such load to finish before the next LDS read, even when the read is from
// another buffer, which serialises the prefetch with the compute.  The caller
// waits for the loads itself (s_waitcnt vmcnt) before a barrier.  M0 holds
// the LDS address; no compiled code in this file uses M0.  The LDS pointer
// itself is an operand, so the compiler sees the buffer written.
__device__ inline void lds_dma16(const void* base, uint32_t off, lds_char* lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds)
                 : "memory");
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>)
template <int N, typename F> __device__ __attribute__((always_inline)) inline void static_for(F&& f) {
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

__device__ inline f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The 16-bit element type of q, k, v (and of a 16-bit output): bf16 or fp16.
// Operands are loaded as raw 16-byte vectors; the type matters only to the
// MFMA, the probability rounding (nearest even either way), the row-sum dot
// and the output rounding.
template <bool F16>
struct Elt;
template <>
struct Elt<false> {
    using x8 = bf16x8;
    using x2 = bf16x2;
    __device__ static x2 pair(float a, float b) { return x2{(__bf16)a, (__bf16)b}; }
    __device__ static f32x16 mfma(const x8& a, const x8& b, const f32x16& c) { return mfma32(a, b, c); }
    __device__ static float sum2(const x2& a, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(a, x2{(__bf16)1.0f, (__bf16)1.0f}, c, false);
    }
    __device__ static float dot2(const x2& a, const x2& b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
    }
};
template <>
struct Elt<true> {
    using x8 = f16x8;
    using x2 = f16x2;
    __device__ static x2 pair(float a, float b) { return x2{(_Float16)a, (_Float16)b}; }
    __device__ static f32x16 mfma(const x8& a, const x8& b, const f32x16& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static float sum2(const x2& a, float c) {
        return __builtin_amdgcn_fdot2(a, x2{(_Float16)1.0f, (_Float16)1.0f}, c, false);
    }
    __device__ static float dot2(const x2& a, const x2& b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }
};

// Max over the lane pair (l, l^32): v_permlane32_swap hands each lane its
// partner's value without a round trip through LDS.
__device__ inline float lane_pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float lane_pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// LDS tiles hold 64 keys x D bf16 with no padding, so each 1 KiB written by one
// direct global->LDS load is contiguous.  Bank conflicts are removed by XOR
// swizzles on the column chunks instead:
//   K: 16-byte chunks, chunk ^ fk(row); the MFMA A-operand read (one row per
//      lane, one 16-byte chunk) then covers distinct banks for any 8 or 16
//      consecutive rows;
//   V: 32-byte chunks, chunk ^ fv(row); the transposing read (four rows x one
//      32-byte chunk per 16 lanes, and the next chunk for the next 16 lanes)
//      covers distinct banks.
template <int D> __device__ inline int k_swz(int row) {
    if constexpr (D == 128) return row & 15;
    else return (row & 7) ^ ((row >> 3) & 1);
}
template <int D> __device__ inline int v_swz(int row) {
    if constexpr (D == 128) return ((row & 3) << 1) | ((row >> 1) & 1);
    else return row & 3;
}
// Tiles the backward reads both ways (row by row as an A operand, and through
// the transposing read): 16-byte chunks, chunk ^ ft(row).  A row read serves
// 16 consecutive rows per pass, so ft must be one-to-one on them; a
// transposing read serves 4 rows per pass, each spanning 4 consecutive
// chunks (64 bytes), so those 4 rows must land in different 64-byte groups.
// At d = 128 (a row is exactly the 64 banks) ft swaps the row's two low 2-bit
// fields; at d = 64 (two rows per 64 banks, split by parity) ft maps rows of
// one parity one-to-one onto the 8 chunks, with bit 2 taken from row bit 1.
template <int D> __device__ inline int t_swz(int row) {
    if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | (((row >> 3) & 1) << 1) | ((row >> 2) & 1);
}

}  // namespace attn
}  // namespace pvc
