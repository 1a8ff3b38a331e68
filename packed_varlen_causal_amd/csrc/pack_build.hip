// Packing metadata kernels: prefix sum of sample lengths (cu_seqlens), per-token
// segment ids, positions, pre-shifted labels and loss mask, the int64 target
// count, and the cu_seqlens validator.
//
// Definitions ([charlestar] "nine tokens, three identities"; [vllbc] "three
// things"; [m020] "06 positions and labels"; [compass] "implementation notes"):
//   cu[0] = 0, cu[r+1] = cu[r] + len[r]; segment(i) = r with cu[r] <= i < cu[r+1];
//   position(i) = i - cu[r]; label(i) = token[i+1] if i+1 < cu[r+1] and r is not
//   a pad segment, else the ignore index; loss_mask = label != ignore.
//
// Work layout.  The scan runs in chunks of 8192 lengths per 1024-thread block
// (one block when nseg <= 8192, else reduce / top-scan / apply).  The token
// kernel splits the buffer into blocks of 2048 consecutive tokens (1024 up to
// 2^20 tokens, so that small buffers still spread over the chip), taken in
// turn by a grid of four 256-thread workgroups per CU.  For each block the
// workgroup finds the segments of its first and last token (a 128-way
// parallel search of cu_seqlens, or above 2^20 tokens a map the scan writes)
// and stages that slice (at most 2049 entries, because every segment holds a
// token) in LDS.  Each thread then takes groups of 4 consecutive tokens: one
// search of the LDS slice per group, 16-byte loads of the token ids and
// 16-byte stores of ids, positions and labels (4 bytes of loss mask),
// contiguous across the wave.  The target count needs one atomic add per
// workgroup: with one per block, the 131,072 same-address adds of a 2^28
// token buffer took half the kernel's time.
// Traffic: 4 B read + 13 B written per token; bound by HBM.
#include <algorithm>

#include "pvc_internal.h"

namespace pvc {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanIPT = 8;
constexpr int kScanChunk = kScanThreads * kScanIPT;

constexpr int kTokThreads = 256;
// Up to this many tokens a token-kernel block takes 1024 tokens, above 2048.
constexpr int kSmallTokens = 1 << 20;

// Inclusive block scan, one value per thread: a shuffle scan inside each
// wave, then every thread adds the totals of the waves before its own.  On
// return sh[blockDim.x - 1] holds the block total (callers read it).
__device__ long long block_inclusive_scan(long long x, long long* sh) {
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const long long y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    long long carry = 0;
    for (int w = 0; w < wave; ++w) carry += sh[w];
    x += carry;
    __syncthreads();                               // every wave has read the totals
    if (t == (int)blockDim.x - 1) sh[t] = x;
    __syncthreads();
    return x;
}

struct ChunkResult {
    long long sum;
    int max_len;
    uint32_t err;
};

// Scan lengths[base .. base+kScanChunk) with a carry-in; optionally write the
// exclusive prefix sums to cu.  Every thread gets the chunk's sum, max, error.
// With blk_seg, each segment also writes its index at every token-kernel
// block (tok_block tokens) that starts inside it: blk_seg[b] is then the
// segment of token b * tok_block, for the blocks b below nblk.
__device__ ChunkResult scan_chunk(const int32_t* __restrict__ lengths, int32_t nseg, int64_t base,
                                  long long carry, int32_t* __restrict__ cu, bool write,
                                  int32_t* __restrict__ blk_seg = nullptr, int32_t tok_block = 1,
                                  int64_t nblk = 0) {
    __shared__ long long sh[kScanThreads];
    __shared__ int s_max;
    __shared__ unsigned s_err;
    const int t = threadIdx.x;
    if (t == 0) { s_max = 0; s_err = 0; }
    long long vals[kScanIPT];
    long long local = 0;
    int mx = 0;
    uint32_t err = 0;
#pragma unroll
    for (int k = 0; k < kScanIPT; ++k) {
        const int64_t idx = base + (int64_t)t * kScanIPT + k;
        int32_t L = 0;
        if (idx < nseg) {
            L = lengths[idx];
            if (L <= 0) err |= PVC_DEV_LENGTH;
        }
        vals[k] = local;
        local += L;
        mx = max(mx, L);
    }
    const long long incl = block_inclusive_scan(local, sh);
    const long long excl = incl - local;
    if (write) {
#pragma unroll
        for (int k = 0; k < kScanIPT; ++k) {
            const int64_t idx = base + (int64_t)t * kScanIPT + k;
            if (idx < nseg) cu[idx] = (int32_t)(carry + excl + vals[k]);
        }
        if (blk_seg != nullptr) {
            for (int k = 0; k < kScanIPT; ++k) {
                const int64_t idx = base + (int64_t)t * kScanIPT + k;
                if (idx >= nseg) break;
                const int64_t c0 = carry + excl + vals[k];
                const int64_t c1 = c0 + (k + 1 < kScanIPT ? vals[k + 1] - vals[k] : local - vals[k]);
                for (int64_t b = (max<int64_t>(c0, 0) + tok_block - 1) / tok_block; b < nblk && b * tok_block < c1; ++b)
                    blk_seg[b] = (int32_t)idx;
            }
        }
    }
    atomicMax(&s_max, mx);
    if (err) atomicOr(&s_err, err);
    __syncthreads();
    ChunkResult res{sh[blockDim.x - 1], s_max, s_err};
    __syncthreads();
    return res;
}

__device__ void finish_scan(long long total, int max_len, uint32_t err, int32_t nseg, int64_t T,
                            int32_t* cu, int64_t* num_targets, int32_t* max_seqlen,
                            uint32_t* dev_error) {
    if (total > 0x7fffffffLL) err |= PVC_DEV_RANGE;
    if (total != T) err |= PVC_DEV_TOTAL;
    cu[nseg] = (int32_t)total;
    if (max_seqlen) *max_seqlen = max_len;
    if (num_targets) *num_targets = 0;
    raise_error(dev_error, err);
}

__global__ __launch_bounds__(kScanThreads) void scan_single_kernel(
        const int32_t* __restrict__ lengths, int32_t nseg, int64_t T, int32_t* __restrict__ cu,
        int64_t* num_targets, int32_t* max_seqlen, uint32_t* dev_error, int32_t* __restrict__ blk_seg,
        int32_t tok_block, int64_t nblk) {
    ChunkResult r = scan_chunk(lengths, nseg, 0, 0, cu, true, blk_seg, tok_block, nblk);
    if (threadIdx.x == 0) finish_scan(r.sum, r.max_len, r.err, nseg, T, cu, num_targets, max_seqlen, dev_error);
}

__global__ __launch_bounds__(kScanThreads) void scan_reduce_kernel(
        const int32_t* __restrict__ lengths, int32_t nseg, long long* part_sum, int* part_max,
        uint32_t* dev_error) {
    ChunkResult r = scan_chunk(lengths, nseg, (int64_t)blockIdx.x * kScanChunk, 0, nullptr, false);
    if (threadIdx.x == 0) {
        part_sum[blockIdx.x] = r.sum;
        part_max[blockIdx.x] = r.max_len;
        raise_error(dev_error, r.err);
    }
}

// One block: exclusive scan of the chunk sums (in place), then the totals.
__global__ __launch_bounds__(kScanThreads) void scan_top_kernel(
        long long* part_sum, const int* part_max, int32_t nchunks, int32_t nseg, int64_t T,
        int32_t* cu, int64_t* num_targets, int32_t* max_seqlen, uint32_t* dev_error) {
    __shared__ long long sh[kScanThreads];
    __shared__ int s_max;
    const int t = threadIdx.x;
    if (t == 0) s_max = 0;
    long long carry = 0;
    int mx = 0;
    for (int base = 0; base < nchunks; base += kScanThreads) {
        const int idx = base + t;
        const long long x = idx < nchunks ? part_sum[idx] : 0;
        if (idx < nchunks) mx = max(mx, part_max[idx]);
        const long long incl = block_inclusive_scan(x, sh);
        if (idx < nchunks) part_sum[idx] = carry + incl - x;
        carry += sh[kScanThreads - 1];
        __syncthreads();
    }
    atomicMax(&s_max, mx);
    __syncthreads();
    if (t == 0) finish_scan(carry, s_max, 0u, nseg, T, cu, num_targets, max_seqlen, dev_error);
}

__global__ __launch_bounds__(kScanThreads) void scan_apply_kernel(
        const int32_t* __restrict__ lengths, int32_t nseg, const long long* part_sum,
        int32_t* __restrict__ cu, int32_t* __restrict__ blk_seg, int32_t tok_block, int64_t nblk) {
    scan_chunk(lengths, nseg, (int64_t)blockIdx.x * kScanChunk, part_sum[blockIdx.x], cu, true, blk_seg,
               tok_block, nblk);
}

// The segments of two tokens a and b (a in threads 0..127, b in 128..255),
// found together by 128-way narrowing: each round probes 128 evenly spaced
// entries of cu in the remaining range, in parallel, and keeps the interval
// after the last probe that is <= the token.  About 4 rounds for 4 million
// segments instead of 22 dependent loads per search.  On a malformed cu the
// result is still some index in [0, nseg-1]; callers check it.
__device__ void block_segments_of(const int32_t* __restrict__ cu, int32_t nseg, int64_t a, int64_t b,
                                  int32_t& ra, int32_t& rb) {
    __shared__ int32_t s_lo[2], s_hi[2];
    __shared__ int32_t s_cnt[4];
    const int t = threadIdx.x;
    const int w = t >> 6;                    // waves 0,1 search a; 2,3 search b
    const int which = t >> 7;
    const int k = t & 127;
    if (t < 2) {
        s_lo[t] = 0;
        s_hi[t] = nseg - 1;
    }
    __syncthreads();
    while (s_lo[0] < s_hi[0] || s_lo[1] < s_hi[1]) {    // uniform
        const int32_t lo = s_lo[which], hi = s_hi[which];
        const int32_t step = (int32_t)(((int64_t)hi - lo + 1 + 127) / 128);
        const int64_t r = (int64_t)lo + (int64_t)k * step;
        const int64_t target = which ? b : a;
        const bool pred = lo < hi && r <= hi && (int64_t)cu[r] <= target;
        const unsigned long long m = __ballot(pred);
        if ((t & 63) == 0) s_cnt[w] = __popcll(m);
        __syncthreads();
        if (t < 2 && s_lo[t] < s_hi[t]) {
            const int cnt = s_cnt[2 * t] + s_cnt[2 * t + 1];
            const int32_t l0 = s_lo[t], h0 = s_hi[t];
            const int32_t st = (int32_t)(((int64_t)h0 - l0 + 1 + 127) / 128);
            if (cnt == 0) {
                s_hi[t] = l0;
            } else {
                s_lo[t] = l0 + (cnt - 1) * st;
                s_hi[t] = (int32_t)min<int64_t>((int64_t)l0 + (int64_t)cnt * st - 1, h0);
            }
        }
        __syncthreads();
    }
    ra = s_lo[0];
    rb = s_lo[1];
    __syncthreads();
}

// A bounded grid of workgroups loops over token blocks of 1024 kR tokens.
// For each block the workgroup stages its slice of cu_seqlens in LDS (found
// by the parallel search, or read from the scan's block map), then each
// thread handles groups of 4 consecutive tokens: one segment search in the
// slice per group, the group's tokens and the next one read as a 16-byte
// vector and one scalar, and each output written as one 16-byte (ids,
// positions, labels) or 4-byte (loss mask) store.  Round g of the kR rounds
// covers the block's tokens [1024 g, 1024 g + 1024), thread t the group at 4t
// of that range, so every load and store instruction of a wave covers one
// contiguous span.  VEC: the pointers allow those vector accesses; otherwise
// the same work goes one element at a time.  A malformed cu (a block's slice
// that does not fit) falls back to a global binary search per token.  The
// target count adds up per workgroup, then one atomic add each.
template <int kR, bool VEC>
__global__ __launch_bounds__(kTokThreads) void pack_tokens_kernel(
        const int32_t* __restrict__ cu, const uint8_t* __restrict__ is_pad,
        const int32_t* __restrict__ tokens, int32_t nseg, int64_t T, int32_t ignore_index,
        int32_t* __restrict__ seg_out, int32_t* __restrict__ pos_out,
        int32_t* __restrict__ lab_out, uint8_t* __restrict__ mask_out,
        int64_t* num_targets, uint32_t* dev_error, const int32_t* __restrict__ blk_seg) {
    constexpr int kRound = kTokThreads * 4;
    constexpr int kTokBlock = kRound * kR;
    __shared__ int32_t s_cu[kTokBlock + 2];
    __shared__ int32_t s_lo, s_n;
    __shared__ unsigned s_cnt, s_err;
    const int64_t nblk = (T + kTokBlock - 1) / kTokBlock;
    if (threadIdx.x == 0) {
        s_cnt = 0;
        s_err = 0;
    }
    unsigned cnt = 0;
    uint32_t err = 0;
    // token blocks blockIdx.x, + gridDim.x, ...: the grid is bounded so that
    // the workgroups' target counts meet in a few hundred atomic adds rather
    // than one per token block (same-address atomics serialise)
    for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        const int64_t b0 = blk * kTokBlock;
        const int64_t b_last = min(b0 + kTokBlock, T) - 1;
        int32_t lo, hi;
        if (blk_seg != nullptr) {
            // the scan's map: the segments of this block's first token and of
            // the next block's (which bounds this block's last); any value is
            // clamped
            lo = min(max(blk_seg[blk], 0), nseg - 1);
            hi = blk + 1 < nblk ? min(max(blk_seg[blk + 1], lo), nseg - 1) : nseg - 1;
        } else {
            block_segments_of(cu, nseg, b0, b_last, lo, hi);
        }
        if (threadIdx.x == 0) {
            int32_t n = hi - lo + 2;                       // entries cu[lo .. hi+1]
            if (n < 2 || n > kTokBlock + 2) n = 0;         // malformed cu: search globally
            s_lo = lo;
            s_n = n;
        }
        __syncthreads();
        const int32_t n = s_n, slo = s_lo;
        for (int e = threadIdx.x; e < n; e += kTokThreads) s_cu[e] = cu[slo + e];
        __syncthreads();

#pragma unroll
        for (int g = 0; g < kR; ++g) {
            const int64_t i = b0 + (int64_t)g * kRound + 4 * threadIdx.x;
            if (i >= T) break;
            const bool full = i + 3 < T;
            int32_t tk[5] = {0, 0, 0, 0, 0};
            if (tokens != nullptr) {
                if (VEC && full) {
                    const int4 v = *reinterpret_cast<const int4*>(tokens + i);
                    tk[0] = v.x; tk[1] = v.y; tk[2] = v.z; tk[3] = v.w;
                } else {
                    for (int k = 0; k < 4 && i + k < T; ++k) tk[k] = tokens[i + k];
                }
                if (i + 4 < T) tk[4] = tokens[i + 4];
            }
            // the group's first segment; later tokens of the group step forward
            int32_t rl = 0, r = 0;
            int64_t st = 0, en = 0;
            if (n) {
                rl = upper_segment(s_cu, n - 1, i);
                r = slo + rl;
                st = s_cu[rl];
                en = s_cu[rl + 1];
            }
            int32_t so[4], po[4], lb[4];
            uint32_t mk = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t ii = i + k;
                so[k] = -1;
                po[k] = 0;
                lb[k] = ignore_index;
                if (ii >= T) continue;
                if (n) {
                    while (ii >= en && rl + 2 < n) {       // at most three steps: a group holds 4 tokens
                        ++rl;
                        ++r;
                        st = en;
                        en = s_cu[rl + 1];
                    }
                } else {
                    r = upper_segment(cu, nseg, ii);
                    st = cu[r];
                    en = cu[r + 1];
                }
                const bool ok = st <= ii && ii < en;
                if (!ok) err |= (ii >= en) ? PVC_DEV_TOTAL : PVC_DEV_NOT_INCREASING;
                if (ok && ii + 1 < en && ii + 1 < T && tokens != nullptr && !(is_pad != nullptr && is_pad[r]))
                    lb[k] = tk[k + 1];
                so[k] = ok ? r : -1;
                po[k] = ok ? (int32_t)(ii - st) : 0;
                const bool m = lb[k] != ignore_index;
                mk |= (uint32_t)m << (8 * k);
                cnt += m;
            }
            if (VEC && full) {
                if (seg_out) *reinterpret_cast<int4*>(seg_out + i) = make_int4(so[0], so[1], so[2], so[3]);
                if (pos_out) *reinterpret_cast<int4*>(pos_out + i) = make_int4(po[0], po[1], po[2], po[3]);
                if (lab_out) *reinterpret_cast<int4*>(lab_out + i) = make_int4(lb[0], lb[1], lb[2], lb[3]);
                if (mask_out) *reinterpret_cast<uint32_t*>(mask_out + i) = mk;
            } else {
                for (int k = 0; k < 4 && i + k < T; ++k) {
                    if (seg_out) seg_out[i + k] = so[k];
                    if (pos_out) pos_out[i + k] = po[k];
                    if (lab_out) lab_out[i + k] = lb[k];
                    if (mask_out) mask_out[i + k] = (uint8_t)((mk >> (8 * k)) & 1u);
                }
            }
        }
        __syncthreads();                                   // s_cu and s_n are read before the next block's
    }
    if (cnt) atomicAdd(&s_cnt, cnt);
    if (err) atomicOr(&s_err, err);
    __syncthreads();
    if (threadIdx.x == 0) {
        if (num_targets && s_cnt)
            atomicAdd(reinterpret_cast<unsigned long long*>(num_targets), (unsigned long long)s_cnt);
        raise_error(dev_error, s_err);
    }
}

// num_targets = 0 ahead of pack_tokens_kernel's atomic adds, when no scan
// kernel (which clears it) runs first.
__global__ void zero_count_kernel(int64_t* num_targets) {
    if (threadIdx.x == 0) *num_targets = 0;
}

constexpr int kValThreads = 256;

__global__ __launch_bounds__(kValThreads) void validate_kernel(
        const int32_t* __restrict__ cu, int32_t nseg, int64_t T, int32_t max_seqlen,
        const int32_t* __restrict__ lengths, uint32_t* dev_error) {
    __shared__ unsigned s_err;
    if (threadIdx.x == 0) s_err = 0;
    __syncthreads();
    const int64_t r = (int64_t)blockIdx.x * kValThreads + threadIdx.x;
    uint32_t e = 0;
    if (r < nseg) {
        const int64_t a = cu[r], b = cu[r + 1];
        if (b <= a) e |= PVC_DEV_NOT_INCREASING;
        if (b - a > max_seqlen) e |= PVC_DEV_MAXSEQ;
        if (lengths != nullptr && b - a != (int64_t)lengths[r]) e |= PVC_DEV_MISMATCH;
    }
    if (r == 0) {
        if (cu[0] != 0) e |= PVC_DEV_CU0;
        if ((int64_t)cu[nseg] != T) e |= PVC_DEV_TOTAL;
    }
    if (e) atomicOr(&s_err, e);
    __syncthreads();
    if (threadIdx.x == 0) raise_error(dev_error, s_err);
}

bool aligned_to(const void* p, uintptr_t n) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % n) == 0; }

template <int kR>
void launch_tokens_r(hipStream_t s, bool vec, const int32_t* cu, const uint8_t* is_pad, const int32_t* tokens,
                     int32_t nseg, int64_t T, int32_t ignore_index, int32_t* seg_out, int32_t* pos_out,
                     int32_t* lab_out, uint8_t* mask_out, int64_t* num_targets, uint32_t* dev_error,
                     const int32_t* blk_seg) {
    const int64_t blocks = (T + kTokThreads * 4 * kR - 1) / (kTokThreads * 4 * kR);
    // four workgroups per CU, each looping over token blocks
    const int64_t nblk = std::min<int64_t>(blocks, std::max(1, device_cu_count()) * 4);
    if (vec)
        hipLaunchKernelGGL((pack_tokens_kernel<kR, true>), dim3((unsigned)nblk), dim3(kTokThreads), 0, s, cu, is_pad,
                           tokens, nseg, T, ignore_index, seg_out, pos_out, lab_out, mask_out, num_targets, dev_error,
                           blk_seg);
    else
        hipLaunchKernelGGL((pack_tokens_kernel<kR, false>), dim3((unsigned)nblk), dim3(kTokThreads), 0, s, cu, is_pad,
                           tokens, nseg, T, ignore_index, seg_out, pos_out, lab_out, mask_out, num_targets, dev_error,
                           blk_seg);
}

// Tokens per block of the per-token kernel for a buffer of T tokens.
inline int32_t tok_block(int64_t T) { return T <= kSmallTokens ? kTokThreads * 4 : kTokThreads * 8; }
inline int64_t tok_blocks(int64_t T) { return (T + tok_block(T) - 1) / tok_block(T); }

// blk_seg: NULL (each block searches cu for its segment range) or the scan's
// block map for tok_block(T).
void launch_tokens(hipStream_t s, const int32_t* cu, const uint8_t* is_pad, const int32_t* tokens, int32_t nseg,
                   int64_t T, int32_t ignore_index, int32_t* seg_out, int32_t* pos_out, int32_t* lab_out,
                   uint8_t* mask_out, int64_t* num_targets, uint32_t* dev_error, const int32_t* blk_seg) {
    // 16-byte vectors for the token ids and the int32 outputs, 4 bytes for the mask
    const bool vec = aligned_to(tokens, 16) && aligned_to(seg_out, 16) && aligned_to(pos_out, 16) &&
                     aligned_to(lab_out, 16) && aligned_to(mask_out, 4);
    // 1024 tokens per block up to 2^20 tokens (small buffers still spread over
    // the chip), 2048 above
    if (T <= kSmallTokens)
        launch_tokens_r<1>(s, vec, cu, is_pad, tokens, nseg, T, ignore_index, seg_out, pos_out, lab_out, mask_out,
                           num_targets, dev_error, blk_seg);
    else
        launch_tokens_r<2>(s, vec, cu, is_pad, tokens, nseg, T, ignore_index, seg_out, pos_out, lab_out, mask_out,
                           num_targets, dev_error, blk_seg);
}

}  // namespace
}  // namespace pvc

using namespace pvc;

// total_tokens is part of the query so that callers size the workspace from
// the same arguments they pass to pvc_pack_build; the scan's partials depend
// on the segment count only.
namespace {
// The workspace: the scan's per-chunk partials (more than one chunk of
// segments), then the per-token kernel's block map (buffers above
// kSmallTokens tokens, whose blocks would otherwise each search cu).
struct PackLayout {
    size_t partials, map, total;
};
PackLayout pack_layout(int32_t nseg, int64_t T) {
    PackLayout L{0, 0, 0};
    if (nseg > kScanChunk) {
        const size_t nch = ((size_t)nseg + kScanChunk - 1) / kScanChunk;
        L.total = align_up(nch * sizeof(long long)) + align_up(nch * sizeof(int));
    }
    L.map = L.total;
    if (T > kSmallTokens && T <= 0x7fffffffLL) L.total += align_up((size_t)tok_blocks(T) * sizeof(int32_t));
    return L;
}
}  // namespace

extern "C" size_t pvc_pack_build_workspace_size(int32_t nseg, int64_t total_tokens) {
    if (nseg < 1) return 0;
    return pack_layout(nseg, total_tokens).total;
}

extern "C" pvc_status pvc_pack_build(const int32_t* lengths, const uint8_t* is_pad,
                                     const int32_t* tokens, int32_t nseg, int64_t total_tokens,
                                     int32_t ignore_index, int32_t* cu_seqlens, int32_t* segment_ids,
                                     int32_t* position_ids, int32_t* shifted_labels,
                                     uint8_t* loss_mask, int64_t* num_targets, int32_t* max_seqlen,
                                     uint32_t* dev_error, void* workspace, size_t workspace_bytes,
                                     void* stream) {
    if (lengths == nullptr || cu_seqlens == nullptr) return PVC_ERR_NULL;
    if ((shifted_labels != nullptr || loss_mask != nullptr || num_targets != nullptr) && tokens == nullptr)
        return PVC_ERR_NULL;
    if (nseg < 1 || total_tokens < 1 || total_tokens > 0x7fffffffLL) return PVC_ERR_INVALID_ARG;
    const PackLayout PL = pack_layout(nseg, total_tokens);
    if (PL.total > 0 && (workspace == nullptr || workspace_bytes < PL.total)) return PVC_ERR_WORKSPACE;
    hipStream_t s = as_stream(stream);
    const bool per_token = segment_ids || position_ids || shifted_labels || loss_mask || num_targets;
    int32_t* blk_seg = (per_token && PL.total > PL.map) ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + PL.map)
                                                        : nullptr;
    const int64_t nblk = blk_seg ? tok_blocks(total_tokens) : 0;

    if (nseg <= kScanChunk) {
        hipLaunchKernelGGL(scan_single_kernel, dim3(1), dim3(kScanThreads), 0, s, lengths, nseg,
                           total_tokens, cu_seqlens, num_targets, max_seqlen, dev_error, blk_seg,
                           tok_block(total_tokens), nblk);
    } else {
        const int32_t nch = (int32_t)(((int64_t)nseg + kScanChunk - 1) / kScanChunk);
        char* ws = static_cast<char*>(workspace);
        long long* part_sum = reinterpret_cast<long long*>(ws);
        int* part_max = reinterpret_cast<int*>(ws + align_up(nch * sizeof(long long)));
        hipLaunchKernelGGL(scan_reduce_kernel, dim3(nch), dim3(kScanThreads), 0, s, lengths, nseg,
                           part_sum, part_max, dev_error);
        hipLaunchKernelGGL(scan_top_kernel, dim3(1), dim3(kScanThreads), 0, s, part_sum, part_max, nch,
                           nseg, total_tokens, cu_seqlens, num_targets, max_seqlen, dev_error);
        hipLaunchKernelGGL(scan_apply_kernel, dim3(nch), dim3(kScanThreads), 0, s, lengths, nseg,
                           part_sum, cu_seqlens, blk_seg, tok_block(total_tokens), nblk);
    }
    if (per_token)
        launch_tokens(s, cu_seqlens, is_pad, tokens, nseg, total_tokens, ignore_index, segment_ids, position_ids,
                      shifted_labels, loss_mask, num_targets, dev_error, blk_seg);
    return launch_status();
}

extern "C" pvc_status pvc_pack_tokens(const int32_t* cu_seqlens, const uint8_t* is_pad, const int32_t* tokens,
                                      int32_t nseg, int64_t total_tokens, int32_t ignore_index,
                                      int32_t* segment_ids, int32_t* position_ids, int32_t* shifted_labels,
                                      uint8_t* loss_mask, int64_t* num_targets, uint32_t* dev_error, void* stream) {
    if (cu_seqlens == nullptr) return PVC_ERR_NULL;
    if ((shifted_labels != nullptr || loss_mask != nullptr || num_targets != nullptr) && tokens == nullptr)
        return PVC_ERR_NULL;
    if (nseg < 1 || total_tokens < 1 || total_tokens > 0x7fffffffLL) return PVC_ERR_INVALID_ARG;
    hipStream_t s = as_stream(stream);
    if (num_targets != nullptr) hipLaunchKernelGGL(zero_count_kernel, dim3(1), dim3(64), 0, s, num_targets);
    if (segment_ids || position_ids || shifted_labels || loss_mask || num_targets)
        launch_tokens(s, cu_seqlens, is_pad, tokens, nseg, total_tokens, ignore_index, segment_ids, position_ids,
                      shifted_labels, loss_mask, num_targets, dev_error, nullptr);
    return launch_status();
}

extern "C" pvc_status pvc_validate_cu_seqlens(const int32_t* cu_seqlens, int32_t nseg,
                                              int64_t total_tokens, int32_t max_seqlen,
                                              const int32_t* lengths, uint32_t* dev_error,
                                              void* stream) {
    if (cu_seqlens == nullptr || dev_error == nullptr) return PVC_ERR_NULL;
    if (nseg < 1 || total_tokens < 1 || total_tokens > 0x7fffffffLL || max_seqlen < 1)
        return PVC_ERR_INVALID_ARG;
    const int64_t nblk = ((int64_t)nseg + kValThreads - 1) / kValThreads;
    hipLaunchKernelGGL(validate_kernel, dim3((unsigned)nblk), dim3(kValThreads), 0, as_stream(stream),
                       cu_seqlens, nseg, total_tokens, max_seqlen, lengths, dev_error);
    return launch_status();
}
