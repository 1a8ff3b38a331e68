// Block-diagonal causal attention over a packed THD buffer, for gfx950.
//
// Definition ([charlestar] "EOS is content": allow(i,j) = same segment and
// p_j <= p_i, additive -inf mask applied before the softmax,
// O = softmax(Q K^T / sqrt(d) + M) V; [compass] "cross-contamination":
// block-diagonal visibility; [opworld] "pitfall one": the varlen kernel skips
// cross-document blocks instead of masking them).
//
// Plan (device-side only, no host synchronization):
//   every token i gets its segment's key range [cu[r], cu[r+1]) by binary
//   search (8 B per token), and one workgroup validates cu_seqlens and seals
//   the header; one launch (plan_fused_kernel, its last workgroup doing the
//   check) up to 16,384 segments, else plan_rows_kernel + plan_check_kernel.
// Query tiles are aligned to the buffer, not to segments: tile w covers rows
// [128w, 128w+128).  A tile may hold the tail of one segment and the head of
// the next, or many short segments; every row carries its own key range, so
// tiles need no per-segment padding.
//
// Forward kernel: one 256-thread workgroup (four wave64s) per (head, tile).
// Wave w owns query rows [128w' + 32w, +32).  Keys stream through LDS in
// stages of 32: K and V go from global memory straight into LDS (no register
// round trip), double buffered, so stage st+1 is in flight while stage st is
// computed.  Per 32-key stage a wave
//   S^T = K Q^T      8 (d=128) v_mfma_f32_32x32x16_bf16, K from LDS as the A
//                    operand, Q^T held in registers as the B operand; each
//                    lane then owns one query and 16 of the 32 keys
//   mask             only on blocks that cross a segment edge or the diagonal
//   online softmax   running max and sum per query in exp2 units; the row max
//                    needs one lane-pair exchange (lane l <-> l^32)
//   O^T += V^T P^T   the probabilities, rounded to bf16, are already in the B
//                    operand layout; the V^T operand comes from row-major V in
//                    LDS through the transposing LDS read (ds_read_b64_tr_b16)
// A wave skips every 32-key stage that lies wholly outside its rows' segments
// or above their diagonal, so cross-segment and above-diagonal blocks are never
// computed.  The running max moves only when a row's new maximum exceeds it by
// more than 2^8 (in probability), which leaves most stages without a rescale
// of the accumulator.  LDS rows are unpadded; XOR swizzles on 16- and 32-byte
// column chunks keep the operand reads free of bank conflicts.
//
// Grid to hardware: workgroups are dealt round-robin to the 8 XCDs, so the
// block index is remapped to give each XCD a contiguous range of the
// (head, tile) space; an XCD then works through a few heads, and the query
// tiles that share a head's K/V run together on one L2.  The segments go in
// buffer order and each segment's tiles from its end to its start, so the
// heaviest tiles of a segment (its last rows see the most keys) are
// dispatched first; when segments span more than two tiles, each segment's
// run of tiles comes once for every head of the XCD before the next
// segment's, so no head's long samples start near the end of the launch.  A
// global longest-first order was measured slower: it separates the tiles of
// a segment and loses their K/V reuse in L2.
#include <math.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "attn_common.h"

namespace pvc {
namespace {

using namespace attn;

// ------------------------------------------------------------------ plan

// Row i's key range: its segment [cu[r], cu[r+1]) (clamped into [0, T)), or
// {i, i+1} for a row outside every segment of a malformed cu.
__device__ inline int2 plan_row(const int32_t* __restrict__ cu, int32_t nseg, int64_t T, int64_t i) {
    const int32_t r = upper_segment(cu, nseg, i);
    const int64_t st = max<int64_t>(cu[r], 0), en = min<int64_t>(cu[r + 1], T);
    const bool ok = st <= i && i < en;
    return ok ? make_int2((int)st, (int)en) : make_int2((int)i, (int)(i + 1));
}

// Padded storage: segment r's L_r = cu[r+1] - cu[r] tokens sit at rows
// [cu_p[r], cu_p[r] + L_r) of a slot that ends at cu_p[r+1]; the rest of the
// slot is padding, whose rows get an empty key range {i, i} (no key, output 0).
__device__ inline int2 plan_row_padded(const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_p,
                                       int32_t nseg, int64_t T, int64_t i) {
    const int32_t r = upper_segment(cu_p, nseg, i);
    const int64_t st = min<int64_t>(max<int64_t>(cu_p[r], 0), T);
    const int64_t len = (int64_t)cu[r + 1] - cu[r];
    const int64_t en = min<int64_t>(max<int64_t>(st + len, st), T);
    const bool ok = st <= i && i < en;
    return ok ? make_int2((int)st, (int)en) : make_int2((int)i, (int)i);
}

__global__ __launch_bounds__(256) void plan_rows_kernel(const int32_t* __restrict__ cu,
                                                        const int32_t* __restrict__ cu_p, int32_t nseg,
                                                        int64_t T, int2* __restrict__ rows) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= T) return;
    rows[i] = cu_p == nullptr ? plan_row(cu, nseg, T, i) : plan_row_padded(cu, cu_p, nseg, T, i);
}

// Validates cu (and, for padded storage, cu_p) and seals the plan header;
// one workgroup of any size.
__device__ void plan_check_block(const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_p, int32_t nseg,
                                 int64_t T, int32_t max_seqlen, int32_t causal, int32_t* __restrict__ header,
                                 int32_t ntiles, uint32_t* dev_error) {
    __shared__ unsigned s_err;
    __shared__ int s_max;
    const int t = threadIdx.x;
    if (t == 0) {
        s_err = 0;
        s_max = 0;
    }
    __syncthreads();
    // the cu_seqlens contract
    uint32_t err = 0;
    int64_t mx = 0;
    for (int64_t r = t; r < nseg; r += blockDim.x) {
        const int64_t a = cu[r], b = cu[r + 1];
        if (b <= a) err |= PVC_DEV_NOT_INCREASING;
        if (b - a > max_seqlen) err |= PVC_DEV_MAXSEQ;
        if (cu_p != nullptr && (int64_t)cu_p[r + 1] - cu_p[r] < b - a) err |= PVC_DEV_PADDED;
        mx = max(mx, b - a);
    }
    if (mx > 0) atomicMax(&s_max, (int)min<int64_t>(mx, 0x7fffffff));
    if (t == 0) {
        if (cu[0] != 0) err |= PVC_DEV_CU0;
        if (cu_p == nullptr) {
            if ((int64_t)cu[nseg] != T) err |= PVC_DEV_TOTAL;
        } else {
            if (cu_p[0] != 0) err |= PVC_DEV_CU0;
            if ((int64_t)cu_p[nseg] != T) err |= PVC_DEV_TOTAL;
        }
    }
    if (err) atomicOr(&s_err, err);
    __syncthreads();
    if (t == 0) {
        header[HDR_MAGIC] = kPlanMagic;
        header[HDR_T] = (int32_t)T;
        header[HDR_CAUSAL] = causal ? 1 : 0;
        header[HDR_NTILES] = ntiles;
        header[HDR_ERR] = (int32_t)s_err;
        header[HDR_VALID] = s_err == 0 ? 1 : 0;
        header[HDR_FOLDED] = 0;
        header[HDR_TK] = (int32_t)T;
        header[HDR_MAXLEN] = s_max;
        raise_error(dev_error, s_err);
    }
}

__global__ __launch_bounds__(kCheckThreads) void plan_check_kernel(
        const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_p, int32_t nseg, int64_t T,
        int32_t max_seqlen, int32_t causal, int32_t* __restrict__ header, int32_t ntiles, uint32_t* dev_error) {
    plan_check_block(cu, cu_p, nseg, T, max_seqlen, causal, header, ntiles, dev_error);
}

// Rows and check in one launch: workgroups [0, G - 1) write the row ranges,
// the last one validates and seals (the header and the rows are both complete
// when the launch ends, before any kernel that reads the plan).
__global__ __launch_bounds__(256) void plan_fused_kernel(const int32_t* __restrict__ cu,
                                                         const int32_t* __restrict__ cu_p, int32_t nseg, int64_t T,
                                                         int32_t max_seqlen, int32_t causal,
                                                         int32_t* __restrict__ header, int32_t ntiles,
                                                         int2* __restrict__ rows, uint32_t* dev_error) {
    if (blockIdx.x == gridDim.x - 1) {
        plan_check_block(cu, cu_p, nseg, T, max_seqlen, causal, header, ntiles, dev_error);
        return;
    }
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= T) return;
    rows[i] = cu_p == nullptr ? plan_row(cu, nseg, T, i) : plan_row_padded(cu, cu_p, nseg, T, i);
}

// Up to this many segments the check shares the rows' launch (a 256-thread
// workgroup); beyond, it runs alone with 1024 threads.
constexpr int32_t kFusedCheckSegs = 16384;

// The self-attention plan, plain (cu_p NULL) or padded storage.
void launch_plan(const int32_t* cu, const int32_t* cu_p, int32_t nseg, int64_t T, int32_t max_seqlen,
                 int32_t causal, int32_t* header, int32_t ntiles, int2* rows, uint32_t* dev_error, hipStream_t s) {
    const int64_t nblk = (T + 255) / 256;
    if (nseg <= kFusedCheckSegs) {
        hipLaunchKernelGGL(plan_fused_kernel, dim3((unsigned)(nblk + 1)), dim3(256), 0, s, cu, cu_p, nseg, T,
                           max_seqlen, causal, header, ntiles, rows, dev_error);
    } else {
        hipLaunchKernelGGL(plan_rows_kernel, dim3((unsigned)nblk), dim3(256), 0, s, cu, cu_p, nseg, T, rows);
        hipLaunchKernelGGL(plan_check_kernel, dim3(1), dim3(kCheckThreads), 0, s, cu, cu_p, nseg, T, max_seqlen,
                           causal, header, ntiles, dev_error);
    }
}

// Separate query and key boundaries (requests of an inference prefill):
// query a of request r (rows [cu_q[r], cu_q[r+1])) sees keys
// [cu_k[r], cu_k[r] + n) with n = min(Lk, a + Lk - Lq + 1) when causal (the
// bottom-right alignment: the last query sees every key) and n = Lk
// otherwise; n <= 0 gives an empty range (output 0).
__global__ __launch_bounds__(256) void plan_rows_qk_kernel(const int32_t* __restrict__ cu_q,
                                                           const int32_t* __restrict__ cu_k, int32_t nseg,
                                                           int64_t Tq, int64_t Tk, int32_t causal,
                                                           int2* __restrict__ rows, int2* __restrict__ qseg) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= Tq) return;
    const int32_t r = upper_segment(cu_q, nseg, i);
    // the request's query rows, clamped into [0, Tq] like every range read
    // from device data: the forward's tile order is decoded from them
    const int64_t qs = min<int64_t>(max<int64_t>(cu_q[r], 0), Tq);
    const int64_t qe = min<int64_t>(max<int64_t>(cu_q[r + 1], qs), Tq);
    const int64_t ks = min<int64_t>(max<int64_t>(cu_k[r], 0), Tk);
    const int64_t ke = min<int64_t>(max<int64_t>(cu_k[r + 1], ks), Tk);
    const int64_t Lk = ke - ks;
    const int64_t n = causal ? min<int64_t>(Lk, (i - qs) + Lk - (qe - qs) + 1) : Lk;
    const bool ok = qs <= i && i < qe;
    rows[i] = ok ? make_int2((int)ks, (int)(ks + max<int64_t>(n, 0))) : make_int2((int)ks, (int)ks);
    qseg[i] = ok ? make_int2((int)qs, (int)qe) : make_int2((int)i, (int)i);
}

// ---- start order of the grouped-head forward's 32-row query tiles.
// A tile belongs to the request of its first row.  Each request's run of
// tiles is cut into chunks of kOrderChunk tiles from its last (heaviest)
// tile down, and the chunks start in decreasing order of the key span of
// their heaviest tile (ties in buffer order): the longest tiles start first,
// as in longest-processing-time-first list scheduling, while a chunk's tiles
// stay neighbours that read their request's K / V together through L2.
// Inference prefills mix requests whose tiles differ in length by 100x
// (cached prefixes); in buffer order a long request near the end of the
// buffer starts its tiles last and the XCD finishes on them alone.
constexpr int kOrderChunk = 16;
constexpr int kOrderMaxChunks = 2048;    // beyond: the buffer order below

// The buffer order: requests in buffer order, each request's tiles from its
// last to its first (a position outside every run is a run of one).
__device__ inline int mirrored_tile(const int2* __restrict__ qseg, int nt, int pos) {
    const int2 sr = qseg[(int64_t)pos * 32];
    int64_t ta = max<int64_t>((sr.x + 31LL) / 32, 0);
    int64_t tb = min<int64_t>((sr.y + 31LL) / 32, nt);
    if (!(pos >= ta && pos < tb)) {
        ta = pos;
        tb = pos + 1;
    }
    return (int)(ta + tb - 1 - pos);
}

// Keys a 32-row tile's waves stream: from its first row's range start to
// its last row's range end (ranges of a folded plan grow with the row).
__device__ inline int tile_span(const int2* __restrict__ rows, int64_t Tq, int64_t tile) {
    const int64_t a = tile * 32, b = min<int64_t>(a + 31, Tq - 1);
    return max(rows[b].y - rows[a].x, 0);
}

// Exclusive prefix sum of v over the workgroup's threads (thread order),
// and the total.  Every thread of the kCheckThreads-thread workgroup calls it.
__device__ inline int block_excl_sum(int v, int* s_wave, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kCheckThreads / 64; ++w) {
        const int cw = s_wave[w];
        off += w < wave ? cw : 0;
        tot += cw;
    }
    __syncthreads();
    total = tot;
    return off + x - v;
}

// order[pos] = the tile that starts at position pos, for every position of
// [0, nt): a permutation of the tiles.  Sorted when the plan is valid and it
// has at most kOrderMaxChunks chunks, else the buffer order.
__device__ void build_tile_order(const int2* __restrict__ rows, const int2* __restrict__ qseg, int64_t Tq, int nt,
                                 bool valid, int32_t* __restrict__ order) {
    __shared__ int s_w[kOrderMaxChunks], s_hi[kOrderMaxChunks], s_n[kOrderMaxChunks], s_rank[kOrderMaxChunks],
            s_off[kOrderMaxChunks];
    __shared__ int s_wave[kCheckThreads / 64];
    const int t = threadIdx.x;
    // more tiles than chunks x chunk size leave too many chunks anyway
    if (valid && (int64_t)nt <= (int64_t)kOrderChunk * kOrderMaxChunks) {
        // tile x heads a chunk when it lies a multiple of kOrderChunk below
        // its run's last tile; the chunk is [x - n + 1, x]
        int nc = 0, covered = 0;                          // workgroup-uniform
        for (int base = 0; base < nt; base += kCheckThreads) {
            const int x = base + t;
            bool head = false;
            int n = 0, w = 0;
            if (x < nt) {
                const int2 sr = qseg[(int64_t)x * 32];
                const int64_t ta = max<int64_t>((sr.x + 31LL) / 32, 0);
                const int64_t tb = min<int64_t>((sr.y + 31LL) / 32, nt);
                if (x >= ta && x < tb && (tb - 1 - x) % kOrderChunk == 0) {
                    head = true;
                    n = (int)min<int64_t>(kOrderChunk, x + 1 - ta);
                    for (int i = 0; i < n; ++i) w = max(w, tile_span(rows, Tq, x - i));
                }
            }
            int heads, tiles;
            const int slot = nc + block_excl_sum(head ? 1 : 0, s_wave, heads);
            block_excl_sum(n, s_wave, tiles);
            if (head && slot < kOrderMaxChunks) {
                s_w[slot] = w;
                s_hi[slot] = x + 1;
                s_n[slot] = n;
            }
            nc += heads;
            covered += tiles;
        }
        // the chunks cover every tile once when the plan is valid
        if (nc <= kOrderMaxChunks && covered == nt) {
            __syncthreads();
            // rank: larger span first, ties by buffer position (a permutation)
            for (int ci = t; ci < nc; ci += kCheckThreads) {
                const int w = s_w[ci];
                int r = 0;
                for (int d = 0; d < nc; ++d) {
                    const int wd = s_w[d];
                    r += (wd > w) | ((wd == w) & (d < ci));
                }
                s_rank[ci] = r;
                s_off[r] = s_n[ci];
            }
            __syncthreads();
            // first position of each rank: exclusive sum, two ranks per thread
            const int a0 = 2 * t < nc ? s_off[2 * t] : 0;
            const int a1 = 2 * t + 1 < nc ? s_off[2 * t + 1] : 0;
            int total;
            const int e = block_excl_sum(a0 + a1, s_wave, total);
            if (2 * t < nc) s_off[2 * t] = e;
            if (2 * t + 1 < nc) s_off[2 * t + 1] = e + a0;
            __syncthreads();
            for (int ci = t; ci < nc; ci += kCheckThreads) {
                const int b = s_off[s_rank[ci]], hi = s_hi[ci], n = s_n[ci];
                for (int i = 0; i < n; ++i) order[b + i] = hi - 1 - i;
            }
            return;
        }
    }
    for (int pos = t; pos < nt; pos += kCheckThreads) order[pos] = mirrored_tile(qseg, nt, pos);
}

__global__ __launch_bounds__(kCheckThreads) void plan_check_qk_kernel(
        const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int32_t nseg, int64_t Tq, int64_t Tk,
        int32_t max_q, int32_t max_k, int32_t causal, int32_t* __restrict__ header, int32_t ntiles,
        const int2* __restrict__ rows, const int2* __restrict__ qseg, int32_t* __restrict__ order,
        uint32_t* dev_error) {
    __shared__ unsigned s_err;
    __shared__ int s_max;
    const int t = threadIdx.x;
    if (t == 0) {
        s_err = 0;
        s_max = 0;
    }
    __syncthreads();
    uint32_t err = 0;
    int64_t mx = 0;
    for (int64_t r = t; r < nseg; r += kCheckThreads) {
        const int64_t a = cu_q[r], b = cu_q[r + 1], ka = cu_k[r], kb = cu_k[r + 1];
        if (b <= a || kb <= ka) err |= PVC_DEV_NOT_INCREASING;
        if (b - a > max_q || kb - ka > max_k) err |= PVC_DEV_MAXSEQ;
        mx = max(mx, b - a);
    }
    if (mx > 0) atomicMax(&s_max, (int)min<int64_t>(mx, 0x7fffffff));
    if (t == 0) {
        if (cu_q[0] != 0 || cu_k[0] != 0) err |= PVC_DEV_CU0;
        if ((int64_t)cu_q[nseg] != Tq || (int64_t)cu_k[nseg] != Tk) err |= PVC_DEV_TOTAL;
    }
    if (err) atomicOr(&s_err, err);
    __syncthreads();
    // (the row ranges are complete: plan_rows_qk_kernel ran before on the stream)
    build_tile_order(rows, qseg, Tq, (int)((Tq + 31) / 32), s_err == 0, order);
    if (t == 0) {
        header[HDR_MAGIC] = kPlanMagic;
        header[HDR_T] = (int32_t)Tq;
        header[HDR_CAUSAL] = causal ? 1 : 0;
        header[HDR_NTILES] = ntiles;
        header[HDR_ERR] = (int32_t)s_err;
        header[HDR_VALID] = s_err == 0 ? 1 : 0;
        header[HDR_FOLDED] = 1;
        header[HDR_TK] = (int32_t)Tk;
        header[HDR_MAXLEN] = s_max;
        raise_error(dev_error, s_err);
    }
}

// --------------------------------------------------------------- forward

struct AttnParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    void* out;
    float* lse;
    const int32_t* header;     // THD: plan header
    const int2* rows;          // THD: per-row key range
    const int2* qseg;          // THD: per-row query segment (tile order of folded plans)
    const int32_t* order;      // grouped heads: start order of the 32-row tiles
    const int32_t* seqlens;    // SBHD: valid length per sample
    int64_t T;                 // THD: query rows
    int64_t Tk;                // THD: key / value rows
    int32_t H;                 // query heads
    int32_t group;             // query heads per key / value head
    int32_t folded;            // the plan's row ranges hold the causal limit
    int32_t causal_flag;       // causal as the caller asked (checked against the plan)
    int32_t ntiles;            // THD: 128-row tiles (the plan's); SBHD: tiles per sample
    int32_t ntiles_q;          // grouped heads (QH > 1): 32-row query tiles
    int32_t items;             // heads x tiles (x batch for SBHD); head groups x 32-row tiles (QH > 1)
    int32_t head_block;        // THD: heads interleaved per segment run (item order)
    int32_t B, L;              // SBHD: batch and padded length
    float scale_log2;          // log2(e) / sqrt(d)
    uint32_t* dev_error;
};

// Threshold (log2 units) by which a row's running max may lag before the
// accumulator is rescaled: probabilities stay below 2^8.
constexpr float kRescaleSlack = 8.0f;

// QH > 1 (grouped key / value heads, QH a divisor of the group size): the
// workgroup's waves are QH = 4 query heads of one key / value head on the
// same 32 query rows, so each K / V stage is staged once for four heads, the
// waves see identical key ranges (no wave waits at a stage barrier with
// nothing to compute), and a tile is 32 rows.  QH == 1: four waves of one
// head on 128 rows.
template <int D, bool CAUSAL, bool OUT_F32, bool SBHD, bool F16, int QH = 1>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void attn_fwd_kernel(AttnParams p) {
    static_assert(D == 64 || D == 128, "head_dim");
    static_assert(QH == 1 || (QH == kWaves && !SBHD), "grouped heads: one wave per query head");
    constexpr int BM = QH == 1 ? kBM : 32;    // query rows per tile
    using E = Elt<F16>;                      // bf16 or fp16 inputs
    using x8 = typename E::x8;
    using x2 = typename E::x2;
    constexpr int NS = D / 16;               // MFMA k-steps for q.k
    constexpr int ND = D / 32;               // 32-wide d blocks of the output
    constexpr int ROW_B = D * 2;             // bytes per key row in LDS
    constexpr int TILE_B = kBN * ROW_B;      // bytes per K (or V) stage
    constexpr int CHUNKS = TILE_B / 1024;    // 1 KiB direct loads per tile
    constexpr int CPW = CHUNKS / kWaves;     // ... per wave
    static_assert(CPW >= 1 && CPW * kWaves == CHUNKS, "staging split");
    constexpr int ROWS_PER_CHUNK = 1024 / ROW_B;
    constexpr int L16 = ROW_B / 16;          // 16-byte pieces per row
    constexpr int NH = kBN / 32;              // 32-key halves per stage
    static_assert(NH == 1 || NH == 2, "stage size");
    // one LDS block: kRing K stages, then kRing V stages (and, after the last
    // stage, the output tile of every wave)
    __shared__ __attribute__((aligned(1024))) uint16_t sKV[2 * kRing * kBN * D];

    // ---- which (head, tile): XCD-contiguous remap of the block index
    const int nblk = gridDim.x;
    const int per_xcd = nblk / kNumXcd;
    const int logical = QH > 1 ? (int)blockIdx.x : (blockIdx.x % kNumXcd) * per_xcd + blockIdx.x / kNumXcd;
    if (logical >= p.items) return;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int head, b = 0, r0, r1, last_row;
    int4 hd0 = {0, 0, 0, 0}, hd1 = {0, 0, 0, 0};      // THD: the plan header
    int seg_lo = 0;
    if constexpr (SBHD) {
        const int per_head = p.B * p.ntiles;
        head = logical / per_head;
        const int rem = logical - head * per_head;
        b = rem / p.ntiles;
        const int tile = p.ntiles - 1 - (rem - b * p.ntiles);   // heavy tiles first
        r0 = tile * kBM;
        r1 = min(r0 + kBM, p.L);
        last_row = p.L - 1;
    } else if constexpr (QH > 1) {
        // Items position-major: block b runs head group b % G at position
        // b / G of the plan's tile order (heaviest chunks first).  Blocks go
        // to the XCDs round-robin, so with a multiple of 8 groups an XCD runs
        // whole groups (their K / V stays in one L2) and with fewer it runs
        // an even share of every group's positions.  Grouped heads run on
        // plans of separate boundaries only (folded: each row's keys are its
        // own range, k_lo below), so no segment start is needed here.
        hd0 = *reinterpret_cast<const int4*>(p.header);
        hd1 = *reinterpret_cast<const int4*>(p.header + 4);
        const int nt = p.ntiles_q;
        const int G = p.H / QH;
        const int grp = logical % G;
        const int pos = logical / G;
        const int tile = min(max(p.order[pos], 0), nt - 1);
        head = grp * QH + wave;
        r0 = tile * BM;
        r1 = (int)min<int64_t>((int64_t)r0 + BM, p.T);
        last_row = (int)(p.Tk - 1);
    } else {
        // Segments in buffer order, and inside each segment its tiles from
        // last to first: a segment's later tiles have the longer key ranges,
        // so they start first, and the workgroups an XCD runs together are
        // neighbours that share K/V in its L2.  The tiles whose first row lies
        // in segment s are [ceil(start_s / BM), ceil(end_s / BM)); position
        // pos of that run takes the tile mirrored in it.
        // (A plan of separate key boundaries keeps the query segments apart:
        // its row ranges are key rows.)
        // Heads go in blocks of head_block (one block per XCD when the head
        // count is a multiple of 8); inside a block, a segment's tiles for
        // every head of the block come together, so the heavy tiles of all
        // of an XCD's heads start early instead of its last head's starting
        // near the end.  Item i of a block of hx heads: position
        // p = i / hx lies in the run [ta, tb) of its segment, whose items
        // are [hx ta, hx tb); the offset in that run gives the head and the
        // mirrored tile.  Positions the plan does not place in a run (a
        // padding row's empty range) form runs of one.  Every head and tile
        // stays in range whatever the plan holds; a plan that is not sealed
        // computes and writes nothing.
        // When no segment spans more than two tiles every tile is light and
        // the blocks are single heads (the plain head-major order).  The
        // plan header and the segment lookups of both orders are loaded
        // together, so the decode costs one memory round trip.
        hd0 = *reinterpret_cast<const int4*>(p.header);
        hd1 = *reinterpret_cast<const int4*>(p.header + 4);
        const int maxlen = p.header[HDR_MAXLEN];
        const int2* seg_of = p.folded ? p.qseg : p.rows;
        const int hm_head = logical / p.ntiles;                 // head-major
        const int hm_pos = logical - hm_head * p.ntiles;
        const int per_block = p.head_block * p.ntiles;          // interleaved
        const int hblk = logical / per_block;
        const int h0 = hblk * p.head_block;
        const int hx = min(p.head_block, p.H - h0);
        const int i = logical - hblk * per_block;               // < hx * ntiles
        const int il_pos = i / hx;
        const int2 sr_hm = seg_of[(int64_t)hm_pos * kBM];       // segment of the first row at pos
        const int2 sr_il = seg_of[(int64_t)il_pos * kBM];
        const bool il = maxlen > 2 * kBM && p.head_block > 1;
        const int pos = il ? il_pos : hm_pos;
        const int2 sr = il ? sr_il : sr_hm;
        // (plan ranges lie in [0, T]; the clamp keeps ta >= 0 regardless)
        int ta = max((sr.x + kBM - 1) / kBM, 0);
        int tb = min((sr.y + kBM - 1) / kBM, p.ntiles);
        if (!(pos >= ta && pos < tb)) {
            ta = pos;
            tb = pos + 1;
        }
        int tile;
        if (il) {
            const int run = tb - ta;
            const int local = i - hx * ta;
            const int hl = local / run;
            head = h0 + hl;
            tile = tb - 1 - (local - hl * run);
        } else {
            head = hm_head;
            tile = ta + tb - 1 - pos;
        }
        // a self-attention plan: the tile's first row lies in segment sr, so
        // its keys start at sr.x (the first row's range) with no further load
        seg_lo = sr.x;
        r0 = tile * kBM;
        r1 = (int)min<int64_t>((int64_t)r0 + kBM, p.T);
        last_row = (int)(p.Tk - 1);
    }
    const int H = p.H;
    const int seq_len = SBHD ? p.seqlens[b] : 0;

    // token row -> element offset of (row, head, 0)
    auto row_off = [&](int row) -> int64_t {
        if constexpr (SBHD) return (((int64_t)row * p.B + b) * H + head) * D;
        else return ((int64_t)row * H + head) * D;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int c = lane & 31;
    const int g = lane >> 5;

    // ---- wave and lane row ranges (grouped heads: every wave on the tile's rows)
    const int wr0 = QH == 1 ? r0 + 32 * wave : r0;
    const int wr1 = min(wr0 + 32, r1);
    const bool wave_active = wr0 < r1;
    const int row = min(wr0 + c, r1 - 1);
    int start_l, end_l, w_lo, w_hi, max_start, min_end;
    if constexpr (SBHD) {
        start_l = 0;
        end_l = seq_len;
        w_lo = 0;
        w_hi = CAUSAL ? wr1 : p.L;
        max_start = 0;
        min_end = seq_len;
    } else {
        const int2 mine = p.rows[row];
        start_l = mine.x;
        end_l = mine.y;
        const int2 first = p.rows[min(wr0, r1 - 1)];
        const int2 last = p.rows[max(wr1 - 1, 0)];
        w_lo = first.x;
        w_hi = CAUSAL ? wr1 : last.y;
        max_start = last.x;
        min_end = first.y;
    }
    int k_lo, k_hi;
    if constexpr (SBHD) {
        k_lo = 0;
        k_hi = CAUSAL ? r1 : p.L;
    } else {
        k_lo = p.folded ? p.rows[r0].x : seg_lo;
        k_hi = CAUSAL ? r1 : p.rows[r1 - 1].y;
    }

    // ---- Q^T operand in registers: lane (c, g) holds Q[row][16s + 8g .. +8]
    x8 qreg[NS];
    {
        const uint16_t* qp = p.q + row_off(row) + 8 * g;
#pragma unroll
        for (int s = 0; s < NS; ++s) qreg[s] = *reinterpret_cast<const x8*>(qp + 16 * s);
    }
    // The plan header was read with the decode.  Every load so far stays
    // inside its buffer whatever the plan holds; a stale or failed plan
    // turns the tile into no stages and no output, so no K/V address is ever
    // formed from plan data that was not sealed.
    bool plan_ok = true;
    if constexpr (!SBHD) {
        const bool sealed = (hd0.x == kPlanMagic) & (hd0.y == (int32_t)p.T) & (hd0.z == p.causal_flag) &
                            (hd0.w == p.ntiles) & (hd1.z == p.folded) & (hd1.w == (int32_t)p.Tk);
        plan_ok = sealed & (hd1.y == 1);
        if (!sealed && threadIdx.x == 0) raise_error(p.dev_error, PVC_DEV_PLAN);
    }
    const int nstages = plan_ok ? (k_hi - k_lo + kBN - 1) / kBN : 0;

    // ---- direct global -> LDS staging.  Wave w writes the 1 KiB chunks
    // w, w + kWaves, w + 2 kWaves, ... of each tile; lane l of a chunk lands
    // at byte 16*l, so it fetches the 16-byte piece the swizzle puts there.
    // Consecutive chunks of one wave are 16 (or 32) rows apart, which leaves
    // the swizzle unchanged, so one per-lane offset serves all of them and a
    // chunk only moves the uniform base pointer.
    constexpr int CHUNK_ROWS = kWaves * ROWS_PER_CHUNK;     // rows between a wave's chunks
    static_assert(CHUNK_ROWS % 16 == 0, "swizzle period");
    // elements per key row, and the key / value head this query head reads
    const int64_t row_stride = SBHD ? (int64_t)p.B * H * D : (int64_t)(H / p.group) * D;
    const int64_t head_off = SBHD ? ((int64_t)b * H + head) * D : (int64_t)(head / p.group) * D;
    const int fetch_rr = wave * ROWS_PER_CHUNK + lane / L16;   // row of chunk 0 in the stage
    uint32_t k_loff, v_loff;
    {
        const int phys = lane % L16;
        const int kpiece = phys ^ k_swz<D>(fetch_rr);
        const int vpiece = (((phys >> 1) ^ v_swz<D>(fetch_rr)) << 1) | (phys & 1);
        k_loff = (uint32_t)((fetch_rr * row_stride + kpiece * 8) * 2);
        v_loff = (uint32_t)((fetch_rr * row_stride + vpiece * 8) * 2);
    }
    // one stage of K (or V) into LDS buffer `buf`
    // Addresses are a uniform base (SGPR pair) plus a 32-bit per-lane offset.
    // dst is the stage buffer's LDS byte address.
    auto fetch_rows = [&](const uint16_t* src, lds_char* dst, uint32_t loff, int kt) {
        const char* base = reinterpret_cast<const char*>(src) + ((int64_t)kt * row_stride + head_off) * 2;
        const int64_t chunk_step = (int64_t)CHUNK_ROWS * row_stride * 2;
        if (kt + kBN - 1 <= last_row) {                                     // uniform
#pragma unroll
            for (int i = 0; i < CPW; ++i) lds_dma16(base + i * chunk_step, loff, dst + (wave + kWaves * i) * 1024);
        } else {
            // rows past the buffer's end re-read its last row (their scores are
            // masked); offsets are taken from the first row that exists, so
            // they stay non-negative even for a stage that starts past the end
            const int base_row = min(kt, last_row);
            const char* b0 = reinterpret_cast<const char*>(src) + ((int64_t)base_row * row_stride + head_off) * 2;
            const uint32_t piece = loff - (uint32_t)(fetch_rr * row_stride * 2);
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                const int rr = min(kt + fetch_rr + i * CHUNK_ROWS, last_row) - base_row;   // 0 .. kBN-1
                lds_dma16(b0, (uint32_t)(rr * row_stride * 2) + piece, dst + (wave + kWaves * i) * 1024);
            }
        }
    };
    auto fetch = [&](const uint16_t* src, lds_char* dst, uint32_t loff, int stage) {
        fetch_rows(src, dst, loff, k_lo + stage * kBN);
    };

    // ---- LDS read offsets.  Every swizzle term depends on the lane only, so
    // each operand read is a per-lane base plus a compile-time offset.
    //   K (A operand of S^T): row 32h + c, 16-byte piece (2s + g) ^ k_swz(c)
    //   V (transposing read): row 32h + 16ks + 8hh + 4g + li/4, 32-byte chunk
    //   (2j + chi) ^ v_swz(li/4), 8-byte piece li%4
    uint32_t k_roff[NS], v_roff[ND];
    {
        const int li = lane & 15;
        const int chi = (lane >> 4) & 1;
#pragma unroll
        for (int s = 0; s < NS; ++s) k_roff[s] = c * ROW_B + (((2 * s + g) ^ k_swz<D>(c)) << 4);
        const int vr = 4 * g + (li >> 2);
#pragma unroll
        for (int j = 0; j < ND; ++j)
            v_roff[j] = vr * ROW_B + (((2 * j + chi) ^ v_swz<D>(vr)) << 5) + ((li & 3) << 3);
    }

    // ---- running state (one query per lane; the lane pair (c, 0)/(c, 1)
    // shares the query and keeps identical m, disjoint halves of l and acc rows)
    f32x16 acc[ND];
#pragma unroll
    for (int j = 0; j < ND; ++j) acc[j] = f32x16(0.0f);
    float m_run = -INFINITY;
    float l_run = 0.0f;
    const float sl2 = p.scale_log2;

    // ---- per-stage work.  A wave takes part in stage st only if some key of
    // the stage is visible to one of its rows; it masks only stages that
    // cross a segment edge or its diagonal.
    auto stage_active = [&](int st) -> bool {
        const int kt = k_lo + st * kBN;
        return wave_active && st >= 0 && st < nstages && kt < w_hi && kt + kBN > w_lo;
    };
    auto stage_full = [&](int st) -> bool {
        const int kt = k_lo + st * kBN;
        return kt >= max_start && kt + kBN <= min_end && (!CAUSAL || kt + kBN - 1 <= wr0);
    };
    char* const kbase = reinterpret_cast<char*>(&sKV[0]);
    char* const vbase = kbase + kRing * TILE_B;

    // K operand: key 32h + c of the stage in buffer kb, k-step s
    auto kop = [&](const char* kb, int h, int s) -> x8 {
        return *reinterpret_cast<const x8*>(kb + k_roff[s] + 32 * h * ROW_B);
    };
    // V^T operand (d block j, 16-key step ks of half h) through the transposing read
    auto vop = [&](const char* vb, int h, int ks, int j) -> x8 {
        const char* vp = vb + v_roff[j] + (32 * h + 16 * ks) * ROW_B;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * ROW_B));
        return __builtin_bit_cast(x8, (short __attribute__((ext_vector_type(8)))){
            lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };
    // S^T of one stage: one 32-key block per half, chains interleaved
    auto qk = [&](const char* kb, f32x16 (&S)[NH]) {
#pragma unroll
        for (int h = 0; h < NH; ++h) S[h] = f32x16(0.0f);
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int h = 0; h < NH; ++h) S[h] = E::mfma(kop(kb, h, s), qreg[s], S[h]);
    };
    // O^T += V^T P^T for one stage; P[h][ks] holds the bf16 probabilities of
    // keys 32h + 16ks + 8(e/4) + 4g + e%4 of this lane's query
    auto pv = [&](const char* vb, const x8 (&P)[NH][2]) {
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < ND; ++j) acc[j] = E::mfma(vop(vb, h, ks, j), P[h][ks], acc[j]);
    };
    // eight bf16 pairs of one 32-key half into the two B operands of P.V
    auto pack = [&](const x2 (&pk)[8], x8 (&out)[2]) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            out[ks] = x8{pk[4 * ks][0], pk[4 * ks][1], pk[4 * ks + 1][0], pk[4 * ks + 1][1],
                             pk[4 * ks + 2][0], pk[4 * ks + 2][1], pk[4 * ks + 3][0], pk[4 * ks + 3][1]};
    };
    auto prob_pair = [&](const f32x16& S, int i, float m_use) -> x2 {
        return E::pair(__builtin_amdgcn_exp2f(fmaf(S[2 * i], sl2, -m_use)),
                       __builtin_amdgcn_exp2f(fmaf(S[2 * i + 1], sl2, -m_use)));
    };
    // stage max in exp2 units, shared by the lane pair
    auto stage_max = [&](const f32x16 (&S)[NH]) {
        float mx = S[0][0];
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int r = (h == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, S[h][r]);
        return lane_pair_max(mx) * sl2;
    };
    // -inf for keys outside the lane's segment or above its diagonal.  Score
    // (h, r) belongs to key kt + 4g + C with C = 32h + 8(r/4) + r%4; the
    // lane's visible keys [start_l, vis_end) become bounds on C per stage.
    const int vis_end = CAUSAL ? min(end_l, row + 1) : end_l;
    auto mask = [&](int st, f32x16 (&S)[NH]) {
        const int x0 = k_lo + st * kBN + 4 * g;
        const int lo = start_l - x0, hi = vis_end - x0;
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int C = 32 * h + 8 * (r >> 2) + (r & 3);
                S[h][r] = ((C >= lo) & (C < hi)) ? S[h][r] : -INFINITY;
            }
    };
    // softmax of one stage: mask, running max (with rescale), probabilities
    auto softmax_stage = [&](int st, f32x16 (&S)[NH], x8 (&P)[NH][2]) {
        if (!stage_full(st)) mask(st, S);
        const float m_st = stage_max(S);
        // move the running max only when it would lag by more than the slack;
        // lanes that keep their max scale by exactly 1 (their m_run may still
        // be -inf when all their keys so far were masked)
        const bool grow = m_st > m_run + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(grow)) {
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_st) : 1.0f;
#pragma unroll
            for (int j = 0; j < ND; ++j) acc[j] *= alpha;
            l_run *= alpha;
            m_run = grow ? m_st : m_run;
        }
        const float m_use = m_run == -INFINITY ? 0.0f : m_run;
        x2 pk[NH][8];
        float rs = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                pk[h][i] = prob_pair(S[h], i, m_use);
                rs = E::sum2(pk[h][i], rs);
            }
        l_run += rs;
#pragma unroll
        for (int h = 0; h < NH; ++h) pack(pk[h], P[h]);
    };

    // ---- stages in order through a ring of kRing K and V buffers: stage st
    // is computed from buffer st % kRing while stages st+1 .. st+kRing-1 are
    // in flight.  The loop is unrolled by kRing so every buffer address is a
    // compile-time offset.
    constexpr int LPS = 2 * CPW;                  // direct loads per stage and wave
    static_assert((kRing - 2) * LPS <= 63, "vmcnt range");
    // s_waitcnt vmcnt(n) for the stages still allowed in flight (expcnt and
    // lgkmcnt left open; vmcnt is split over bits 3:0 and 15:14)
    auto wait_stages = [&](int ahead) {
        static_for<kRing - 1>([&](auto n) {
            constexpr int v = decltype(n)::value * LPS;
            if (ahead == decltype(n)::value)
                __builtin_amdgcn_s_waitcnt(0x0F70 | (v & 15) | ((v >> 4) << 14));
        });
    };
    lds_char* const k_lds = (lds_char*)kbase;
    lds_char* const v_lds = (lds_char*)vbase;
    auto fetch_stage = [&](int stage, int slot) {
        fetch(p.k, k_lds + slot * TILE_B, k_loff, stage);
        fetch(p.v, v_lds + slot * TILE_B, v_loff, stage);
    };
    static_for<kRing - 1>([&](auto i) {
        if (decltype(i)::value < nstages) fetch_stage(decltype(i)::value, decltype(i)::value);
    });
    for (int st0 = 0; st0 < nstages; st0 += kRing) {
        static_for<kRing>([&](auto I) {
            constexpr int SLOT = decltype(I)::value;
            const int st = st0 + SLOT;
            if (st >= nstages) return;
            // stage st has landed for this wave, then for all; stage st-1 is consumed
            wait_stages(min(kRing - 2, nstages - 1 - st));
            __syncthreads();
            if (st + kRing - 1 < nstages) fetch_stage(st + kRing - 1, (SLOT + kRing - 1) % kRing);
            if (stage_active(st)) {
                f32x16 S[NH];
                x8 P[NH][2];
                qk(kbase + SLOT * TILE_B, S);
                softmax_stage(st, S, P);
                pv(vbase + SLOT * TILE_B, P);
            }
        });
    }

    // ---- epilogue: lane (c, g) holds O^T rows d = 32j + 8(r/4) + 4g + r%4
    if (!plan_ok) return;                                  // uniform: nothing was computed
    const float l = lane_pair_sum(l_run);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;          // a padding row has no key: output 0
    const bool row_ok = wave_active && wr0 + c < r1;
    if constexpr (OUT_F32) {
        if (row_ok) {
            const int64_t ob = row_off(row);
#pragma unroll
            for (int j = 0; j < ND; ++j)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int d0 = 32 * j + 8 * rq + 4 * g;
                    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + ob + d0) =
                            f32x4{acc[j][4 * rq] * inv, acc[j][4 * rq + 1] * inv, acc[j][4 * rq + 2] * inv,
                                  acc[j][4 * rq + 3] * inv};
                }
        }
    } else {
        // The bf16 tile goes through LDS so that every store instruction
        // writes whole rows (16 consecutive lanes x 16 B = one 256-byte row
        // at d=128) instead of 16-byte pieces of 32 rows.  Each wave uses its
        // own 32-row slice of the stage buffers, free once all waves are past
        // the last stage; 16-byte chunks are XOR-swizzled by row.
        constexpr int CPR = ROW_B / 16;                    // 16-byte chunks per row
        static_assert(kWaves * 32 * ROW_B <= 2 * kRing * TILE_B, "output tile fits the stage buffers");
        __syncthreads();
        char* const ob_lds = kbase + wave * 32 * ROW_B;
#pragma unroll
        for (int j = 0; j < ND; ++j)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const x2 a = E::pair(acc[j][4 * rq] * inv, acc[j][4 * rq + 1] * inv);
                const x2 bb = E::pair(acc[j][4 * rq + 2] * inv, acc[j][4 * rq + 3] * inv);
                const int chunk = (4 * j + rq) ^ (c & (CPR - 1));
                *reinterpret_cast<u32x2*>(ob_lds + c * ROW_B + chunk * 16 + g * 8) =
                        u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, bb)};
            }
        if (wave_active) {
            constexpr int RPI = 64 / CPR;                  // rows per 64-lane store
#pragma unroll
            for (int i = 0; i < 32 / RPI; ++i) {
                const int r = i * RPI + lane / CPR;
                const int k = lane % CPR;
                const u32x4 v = *reinterpret_cast<const u32x4*>(ob_lds + r * ROW_B + ((k ^ (r & (CPR - 1))) << 4));
                if (wr0 + r < r1)
                    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + row_off(wr0 + r) + k * 8) = v;
            }
        }
    }
    if constexpr (!SBHD) {
        if (p.lse != nullptr && g == 0 && row_ok)
            p.lse[(int64_t)head * p.T + row] = (m_run + __log2f(l)) * 0.69314718055994530942f;
    }
}

template <int D, bool SBHD, bool F16, int QH = 1>
pvc_status launch_fwd_t(const AttnParams& prm, bool causal, bool out_f32, hipStream_t s) {
    const int64_t grid = ((int64_t)prm.items + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (grid > 0x7fffffffLL) return PVC_ERR_INVALID_ARG;
    dim3 g((unsigned)grid), blk(kThreads);
    if constexpr (QH > 1) {
        // folded plans only: the causal limit is in the row ranges
        if (causal) return PVC_ERR_INVALID_ARG;
        if (out_f32) hipLaunchKernelGGL((attn_fwd_kernel<D, false, true, SBHD, F16, QH>), g, blk, 0, s, prm);
        else hipLaunchKernelGGL((attn_fwd_kernel<D, false, false, SBHD, F16, QH>), g, blk, 0, s, prm);
        return launch_status();
    }
    if (causal) {
        if (out_f32) hipLaunchKernelGGL((attn_fwd_kernel<D, true, true, SBHD, F16>), g, blk, 0, s, prm);
        else hipLaunchKernelGGL((attn_fwd_kernel<D, true, false, SBHD, F16>), g, blk, 0, s, prm);
    } else {
        if (out_f32) hipLaunchKernelGGL((attn_fwd_kernel<D, false, true, SBHD, F16>), g, blk, 0, s, prm);
        else hipLaunchKernelGGL((attn_fwd_kernel<D, false, false, SBHD, F16>), g, blk, 0, s, prm);
    }
    return launch_status();
}

// out_dtype: PVC_OUT_BF16 / PVC_OUT_F32 for bf16 inputs, PVC_OUT_F16 /
// PVC_OUT_F16_F32 for fp16 inputs.
inline bool io_valid(int32_t t) { return t == PVC_OUT_BF16 || t == PVC_OUT_F32 || t == PVC_OUT_F16 || t == PVC_OUT_F16_F32; }
inline bool io_f16(int32_t t) { return t == PVC_OUT_F16 || t == PVC_OUT_F16_F32; }
inline bool io_f32(int32_t t) { return t == PVC_OUT_F32 || t == PVC_OUT_F16_F32; }

template <int D, int QH = 1>
pvc_status launch_thd(const AttnParams& prm, bool causal, int32_t out_dtype, hipStream_t s) {
    if (io_f16(out_dtype)) return launch_fwd_t<D, false, true, QH>(prm, causal, io_f32(out_dtype), s);
    return launch_fwd_t<D, false, false, QH>(prm, causal, io_f32(out_dtype), s);
}

// Heads per block of the item order: one block per XCD when the head count
// divides by the XCD count, else single heads.
inline int32_t head_block(int32_t heads) { return heads % kNumXcd == 0 ? heads / kNumXcd : 1; }

// Per-lane staging offsets span one 32-row stage in 32 bits (32 * 2^24 * 2 B).
constexpr int64_t kMaxRowElems = (int64_t)1 << 24;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

}  // namespace
}  // namespace pvc

using namespace pvc;

extern "C" size_t pvc_attn_workspace_size(int64_t total_tokens, int32_t nseg) {
    (void)nseg;
    if (total_tokens < 1 || total_tokens > 0x7fffffffLL) return 0;
    return plan_layout(total_tokens).total;
}

// The forward's workspace is its plan, which depends on the tokens only.
extern "C" size_t pvc_varlen_attn_fwd_workspace_size(int64_t total_tokens, int32_t nseg, int32_t max_seqlen,
                                                     int32_t heads, int32_t head_dim) {
    (void)max_seqlen;
    (void)heads;
    (void)head_dim;
    return pvc_attn_workspace_size(total_tokens, nseg);
}

extern "C" pvc_status pvc_attn_plan(const int32_t* cu_seqlens, int32_t nseg, int64_t total_tokens,
                                    int32_t max_seqlen, int32_t causal, void* workspace,
                                    size_t workspace_bytes, uint32_t* dev_error, void* stream) {
    if (cu_seqlens == nullptr || workspace == nullptr) return PVC_ERR_NULL;
    if (nseg < 1 || total_tokens < 1 || total_tokens > 0x7fffffffLL || max_seqlen < 1)
        return PVC_ERR_INVALID_ARG;
    const PlanLayout L = plan_layout(total_tokens);
    if (workspace_bytes < L.total) return PVC_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    auto* header = reinterpret_cast<int32_t*>(ws + L.header);
    auto* rows = reinterpret_cast<int2*>(ws + L.rows);
    launch_plan(cu_seqlens, nullptr, nseg, total_tokens, max_seqlen, causal ? 1 : 0, header, (int32_t)L.ntiles, rows,
                dev_error, as_stream(stream));
    return launch_status();
}

extern "C" pvc_status pvc_attn_plan_padded(const int32_t* cu_seqlens, const int32_t* cu_seqlens_padded,
                                           int32_t nseg, int64_t total_rows, int32_t max_seqlen, int32_t causal,
                                           void* workspace, size_t workspace_bytes, uint32_t* dev_error,
                                           void* stream) {
    if (cu_seqlens == nullptr || cu_seqlens_padded == nullptr || workspace == nullptr) return PVC_ERR_NULL;
    if (nseg < 1 || total_rows < 1 || total_rows > 0x7fffffffLL || max_seqlen < 1) return PVC_ERR_INVALID_ARG;
    const PlanLayout L = plan_layout(total_rows);
    if (workspace_bytes < L.total) return PVC_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    auto* header = reinterpret_cast<int32_t*>(ws + L.header);
    auto* rows = reinterpret_cast<int2*>(ws + L.rows);
    launch_plan(cu_seqlens, cu_seqlens_padded, nseg, total_rows, max_seqlen, causal ? 1 : 0, header,
                (int32_t)L.ntiles, rows, dev_error, as_stream(stream));
    return launch_status();
}

namespace {

// Host checks of the self-attention forward (nothing is enqueued before they pass).
pvc_status fwd_args(const void* q, const void* k, const void* v, void* out, int64_t total_tokens, int32_t heads,
                    int32_t head_dim, int32_t out_dtype, const void* workspace, size_t workspace_bytes) {
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || workspace == nullptr)
        return PVC_ERR_NULL;
    if (total_tokens < 1 || total_tokens > 0x7fffffffLL || heads < 1) return PVC_ERR_INVALID_ARG;
    if (!io_valid(out_dtype)) return PVC_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return PVC_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PVC_ERR_INVALID_ARG;
    const PlanLayout L = plan_layout(total_tokens);
    if (workspace_bytes < L.total) return PVC_ERR_WORKSPACE;
    const size_t in_bytes = (size_t)total_tokens * heads * head_dim * 2;
    const size_t out_bytes = in_bytes * (io_f32(out_dtype) ? 2 : 1);
    if (overlaps(out, out_bytes, q, in_bytes) || overlaps(out, out_bytes, k, in_bytes) ||
        overlaps(out, out_bytes, v, in_bytes))
        return PVC_ERR_INVALID_ARG;
    if (L.ntiles * (int64_t)heads > 0x7ffffff0LL) return PVC_ERR_INVALID_ARG;
    if ((int64_t)heads * head_dim > kMaxRowElems) return PVC_ERR_INVALID_ARG;
    return PVC_OK;
}

}  // namespace

extern "C" pvc_status pvc_varlen_attn_fwd_planned(const void* q, const void* k, const void* v, void* out,
                                                  float* lse, int64_t total_tokens, int32_t heads,
                                                  int32_t head_dim, int32_t causal, int32_t out_dtype,
                                                  const void* workspace, size_t workspace_bytes,
                                                  uint32_t* dev_error, void* stream) {
    const pvc_status chk = fwd_args(q, k, v, out, total_tokens, heads, head_dim, out_dtype, workspace,
                                    workspace_bytes);
    if (chk != PVC_OK) return chk;
    const PlanLayout L = plan_layout(total_tokens);
    const char* ws = static_cast<const char*>(workspace);
    AttnParams prm{};
    prm.q = static_cast<const uint16_t*>(q);
    prm.k = static_cast<const uint16_t*>(k);
    prm.v = static_cast<const uint16_t*>(v);
    prm.out = out;
    prm.lse = lse;
    prm.header = reinterpret_cast<const int32_t*>(ws + L.header);
    prm.rows = reinterpret_cast<const int2*>(ws + L.rows);
    prm.qseg = reinterpret_cast<const int2*>(ws + L.qseg);
    prm.T = total_tokens;
    prm.Tk = total_tokens;
    prm.H = heads;
    prm.group = 1;
    prm.folded = 0;
    prm.causal_flag = causal != 0 ? 1 : 0;
    prm.ntiles = (int32_t)L.ntiles;
    prm.items = (int32_t)(L.ntiles * heads);
    prm.head_block = head_block(heads);
    prm.scale_log2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
    prm.dev_error = dev_error;
    hipStream_t s = as_stream(stream);
    if (head_dim == 128) return launch_thd<128>(prm, causal != 0, out_dtype, s);
    return launch_thd<64>(prm, causal != 0, out_dtype, s);
}

extern "C" pvc_status pvc_attn_plan_qk(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t nseg,
                                       int64_t total_q, int64_t total_k, int32_t max_seqlen_q,
                                       int32_t max_seqlen_k, int32_t causal, void* workspace,
                                       size_t workspace_bytes, uint32_t* dev_error, void* stream) {
    if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr || workspace == nullptr) return PVC_ERR_NULL;
    if (nseg < 1 || total_q < 1 || total_q > 0x7fffffffLL || total_k < 1 || total_k > 0x7fffffffLL ||
        max_seqlen_q < 1 || max_seqlen_k < 1)
        return PVC_ERR_INVALID_ARG;
    const PlanLayout L = plan_layout(total_q);
    if (workspace_bytes < L.total) return PVC_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    auto* header = reinterpret_cast<int32_t*>(ws + L.header);
    auto* rows = reinterpret_cast<int2*>(ws + L.rows);
    auto* qseg = reinterpret_cast<int2*>(ws + L.qseg);
    hipStream_t s = as_stream(stream);
    const int64_t nblk = (total_q + 255) / 256;
    hipLaunchKernelGGL(plan_rows_qk_kernel, dim3((unsigned)nblk), dim3(256), 0, s, cu_seqlens_q, cu_seqlens_k,
                       nseg, total_q, total_k, causal ? 1 : 0, rows, qseg);
    hipLaunchKernelGGL(plan_check_qk_kernel, dim3(1), dim3(kCheckThreads), 0, s, cu_seqlens_q, cu_seqlens_k, nseg,
                       total_q, total_k, max_seqlen_q, max_seqlen_k, causal ? 1 : 0, header, (int32_t)L.ntiles,
                       rows, qseg, reinterpret_cast<int32_t*>(ws + L.order), dev_error);
    return launch_status();
}

extern "C" pvc_status pvc_varlen_attn_fwd_qk_planned(const void* q, const void* k, const void* v, void* out,
                                                     float* lse, int64_t total_q, int64_t total_k, int32_t heads,
                                                     int32_t kv_heads, int32_t head_dim, int32_t causal,
                                                     int32_t out_dtype, const void* workspace,
                                                     size_t workspace_bytes, uint32_t* dev_error, void* stream) {
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || workspace == nullptr)
        return PVC_ERR_NULL;
    if (total_q < 1 || total_q > 0x7fffffffLL || total_k < 1 || total_k > 0x7fffffffLL || heads < 1 ||
        kv_heads < 1 || heads % kv_heads != 0)
        return PVC_ERR_INVALID_ARG;
    if (!io_valid(out_dtype)) return PVC_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return PVC_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PVC_ERR_INVALID_ARG;
    const PlanLayout L = plan_layout(total_q);
    if (workspace_bytes < L.total) return PVC_ERR_WORKSPACE;
    const size_t q_bytes = (size_t)total_q * heads * head_dim * 2;
    const size_t kv_bytes = (size_t)total_k * kv_heads * head_dim * 2;
    const size_t out_bytes = q_bytes * (io_f32(out_dtype) ? 2 : 1);
    if (overlaps(out, out_bytes, q, q_bytes) || overlaps(out, out_bytes, k, kv_bytes) ||
        overlaps(out, out_bytes, v, kv_bytes))
        return PVC_ERR_INVALID_ARG;
    if (L.ntiles * (int64_t)heads > 0x7ffffff0LL) return PVC_ERR_INVALID_ARG;
    if ((int64_t)heads * head_dim > kMaxRowElems) return PVC_ERR_INVALID_ARG;
    const char* ws = static_cast<const char*>(workspace);
    AttnParams prm{};
    prm.q = static_cast<const uint16_t*>(q);
    prm.k = static_cast<const uint16_t*>(k);
    prm.v = static_cast<const uint16_t*>(v);
    prm.out = out;
    prm.lse = lse;
    prm.header = reinterpret_cast<const int32_t*>(ws + L.header);
    prm.rows = reinterpret_cast<const int2*>(ws + L.rows);
    prm.qseg = reinterpret_cast<const int2*>(ws + L.qseg);
    prm.order = reinterpret_cast<const int32_t*>(ws + L.order);
    prm.T = total_q;
    prm.Tk = total_k;
    prm.H = heads;
    prm.group = heads / kv_heads;
    prm.folded = 1;
    prm.causal_flag = causal != 0 ? 1 : 0;
    prm.ntiles = (int32_t)L.ntiles;
    prm.items = (int32_t)(L.ntiles * heads);
    prm.head_block = head_block(heads);
    prm.scale_log2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
    prm.dev_error = dev_error;
    hipStream_t s = as_stream(stream);
    // the causal limit is in the plan's row ranges: the kernel runs without its own diagonal
    if (prm.group % kWaves == 0) {
        // four query heads of one key / value head per workgroup, 32-row tiles
        prm.ntiles_q = (int32_t)((total_q + 31) / 32);
        prm.items = (int32_t)((int64_t)prm.ntiles_q * (heads / kWaves));
        if (head_dim == 128) return launch_thd<128, kWaves>(prm, false, out_dtype, s);
        return launch_thd<64, kWaves>(prm, false, out_dtype, s);
    }
    if (head_dim == 128) return launch_thd<128>(prm, false, out_dtype, s);
    return launch_thd<64>(prm, false, out_dtype, s);
}

extern "C" pvc_status pvc_varlen_attn_fwd(const void* q, const void* k, const void* v, void* out,
                                          float* lse, const int32_t* cu_seqlens, int32_t nseg,
                                          int64_t total_tokens, int32_t max_seqlen, int32_t heads,
                                          int32_t head_dim, int32_t causal, int32_t out_dtype,
                                          void* workspace, size_t workspace_bytes, uint32_t* dev_error,
                                          void* stream) {
    // the forward's own checks first, so that a refused call enqueues no plan either
    pvc_status st = fwd_args(q, k, v, out, total_tokens, heads, head_dim, out_dtype, workspace, workspace_bytes);
    if (st != PVC_OK) return st;
    st = pvc_attn_plan(cu_seqlens, nseg, total_tokens, max_seqlen, causal, workspace, workspace_bytes, dev_error,
                       stream);
    if (st != PVC_OK) return st;
    return pvc_varlen_attn_fwd_planned(q, k, v, out, lse, total_tokens, heads, head_dim, causal,
                                       out_dtype, workspace, workspace_bytes, dev_error, stream);
}

extern "C" pvc_status pvc_padded_attn_fwd_sbhd(const void* q, const void* k, const void* v, void* out,
                                               const int32_t* seqlens, int32_t batch, int32_t max_len,
                                               int32_t heads, int32_t head_dim, int32_t causal,
                                               int32_t out_dtype, void* stream) {
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || seqlens == nullptr)
        return PVC_ERR_NULL;
    if (batch < 1 || max_len < 1 || heads < 1) return PVC_ERR_INVALID_ARG;
    if (out_dtype != PVC_OUT_BF16 && out_dtype != PVC_OUT_F32) return PVC_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return PVC_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PVC_ERR_INVALID_ARG;
    const int64_t elems = (int64_t)max_len * batch * heads * head_dim;
    if (elems > (int64_t)1 << 46) return PVC_ERR_INVALID_ARG;
    const size_t bytes = (size_t)elems * 2;
    const size_t out_bytes = bytes * (out_dtype == PVC_OUT_F32 ? 2 : 1);
    if (overlaps(out, out_bytes, q, bytes) || overlaps(out, out_bytes, k, bytes) ||
        overlaps(out, out_bytes, v, bytes))
        return PVC_ERR_INVALID_ARG;
    if ((int64_t)batch * heads * head_dim > kMaxRowElems) return PVC_ERR_INVALID_ARG;
    const int64_t tiles = (max_len + kBM - 1) / kBM;
    const int64_t items = tiles * batch * heads;
    if (items > 0x7ffffff0LL) return PVC_ERR_INVALID_ARG;
    AttnParams prm{};
    prm.q = static_cast<const uint16_t*>(q);
    prm.k = static_cast<const uint16_t*>(k);
    prm.v = static_cast<const uint16_t*>(v);
    prm.out = out;
    prm.seqlens = seqlens;
    prm.H = heads;
    prm.ntiles = (int32_t)tiles;
    prm.items = (int32_t)items;
    prm.group = 1;
    prm.B = batch;
    prm.L = max_len;
    prm.scale_log2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
    hipStream_t s = as_stream(stream);
    const bool f32 = out_dtype == PVC_OUT_F32;
    if (head_dim == 128) return launch_fwd_t<128, true, false>(prm, causal != 0, f32, s);
    return launch_fwd_t<64, true, false>(prm, causal != 0, f32, s);
}

// ------------------------------------------------ allocation-free forward
//
// pvc_varlen_attn_fwd with its plan in a library-owned device array instead
// of a caller workspace, for callers that cannot allocate.  The array holds
// the plan layout of kNoAllocMaxTokens tokens (16 MiB + 256 B); each GPU the
// library runs on gets its own copy,
// kept until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the device symbol): the
// device address comes from hipGetSymbolAddress, once per device, and is
// cached per device.  Every call on one GPU shares that GPU's array, so
// calls that overlap on one GPU (different streams, or other host threads)
// race on the plan; calls ordered on one stream do not.  Nothing in it needs
// clearing: each call's plan launch rewrites the header and every row the
// forward reads before the forward runs.

namespace {
constexpr int64_t kNoAllocMaxTokens = (int64_t)1 << 20;
// plan_layout(kNoAllocMaxTokens).total: the header, two int2 planes and the
// tile order (one int32 per 32 rows)
constexpr size_t kNoAllocBytes =
        kAlign + 2 * (size_t)kNoAllocMaxTokens * sizeof(int2) + (size_t)kNoAllocMaxTokens / 32 * sizeof(int32_t);
constexpr int kNoAllocMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];
static_assert(kNoAllocBytes % kAlign == 0, "the plan layout's regions are 256-byte aligned");

namespace {
std::atomic<void*> g_scratch_ptr[kNoAllocMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch`, looked up on the first call on
// that device (with that device current) and cached.
pvc_status noalloc_scratch(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) return PVC_ERR_HIP;
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (ptr == nullptr) {
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return PVC_ERR_HIP;
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return PVC_OK;
}
}  // namespace

extern "C" int64_t pvc_noalloc_max_tokens(void) { return kNoAllocMaxTokens; }

extern "C" pvc_status pvc_varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                                                  float* lse, const int32_t* cu_seqlens, int32_t nseg,
                                                  int64_t total_tokens, int32_t max_seqlen, int32_t heads,
                                                  int32_t head_dim, int32_t causal, int32_t out_dtype,
                                                  uint32_t* dev_error, void* stream) {
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || cu_seqlens == nullptr) return PVC_ERR_NULL;
    if (total_tokens < 1) return PVC_ERR_INVALID_ARG;
    // the size limit before any HIP call
    if (total_tokens > kNoAllocMaxTokens || plan_layout(total_tokens).total > kNoAllocBytes)
        return PVC_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    const pvc_status st = noalloc_scratch(&ws);
    if (st != PVC_OK) return st;
    // the remaining checks, the plan and the forward: pvc_varlen_attn_fwd
    return pvc_varlen_attn_fwd(q, k, v, out, lse, cu_seqlens, nseg, total_tokens, max_seqlen, heads, head_dim,
                               causal, out_dtype, ws, kNoAllocBytes, dev_error, stream);
}
