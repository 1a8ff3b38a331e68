// Backward of block-diagonal causal attention over a packed THD buffer, for
// gfx950.
//
// For an upstream gradient dO of O = softmax(Q K^T / sqrt(d) + M) V (the
// forward of [charlestar] "EOS is content"), with P the masked softmax and
// s = 1/sqrt(d):
//   dV = P^T dO,  dP = dO V^T,  D_i = dO_i . O_i,  dS = P o (dP - D),
//   dQ = s dS K,  dK = s dS^T Q.
// P is recomputed from Q, K and the forward's log-sum-exp, so nothing of size
// T x T is stored.  Two launches, both on the forward's plan (per-row key
// ranges, 128-row tiles, the forward's XCD-contiguous item order):
//   bwd_dq_kernel     query-major like the forward: a wave holds Q^T and dO^T
//                     of its 32 rows in registers, forms D_i = dO_i . O_i and
//                     lse_i * log2(e) for them and stores both in a padded
//                     scratch buffer for the second launch, and streams
//                     32-key stages of K and V through LDS; per stage S^T = K Q^T and
//                     dP^T = V dO^T (MFMA, K and V as A operands),
//                     dS^T = P^T o (dP^T - D) in registers, and
//                     dQ^T += K^T dS^T with K^T from the transposing LDS read;
//   bwd_dkdv_kernel   key-major, one workgroup per CU taking its XCD's items
//                     from a counter (the next item's loads go out before the
//                     current item's stores): a wave holds K^T and V^T of its
//                     32 keys and streams 64-query stages (two 32-query
//                     halves) of Q, dO, lse and D through a ring of three
//                     buffers; per half
//                     S = Q K^T and dP = dO V^T (lane = key), P and dS in
//                     registers, dV^T += dO^T P and dK^T += Q^T dS with Q^T and
//                     dO^T from the transposing LDS read.  Both halves' S and
//                     dP are issued first, so one half's MFMA chains overlap
//                     the other half's exponentials.  One wave per SIMD
//                     (about 370 registers: the two fp32 accumulators alone
//                     take 128).
// Every product rounds its probability operand (P or dS) to the input type
// (bf16 or fp16) and accumulates in fp32.  Each output element is written
// once by one workgroup and no atomic touches a value (the only atomic is the
// dK/dV ticket), so results do not depend on scheduling.  Stages that lie
// wholly outside a wave's segments or on the wrong side of its diagonal are
// skipped, as in the forward.  The dQ kernel recomputes S and dP, which the
// dK/dV kernel also computes: seven products per score instead of five, the
// price of writing every gradient once without accumulating atomics.
#include "attn_common.h"

#include <algorithm>

namespace pvc {
namespace {

using namespace attn;

struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* out;
    const uint16_t* dout;
    const float* lse;          // [H, T], natural log (the forward's)
    float* scratch;            // [2][H][Tp]: lse * log2(e), then D
    int32_t* queue;            // dK/dV item counters, one per XCD (kQueueStride ints apart), after the planes
    void* dq;
    void* dk;
    void* dv;
    const int32_t* header;
    const int2* rows;
    int64_t T;
    int64_t Tp;                // padded row count of the scratch planes
    int32_t H;
    int32_t ntiles;
    int32_t items;
    int32_t head_block;        // heads interleaved per segment run (item order)
    float scale_log2;          // log2(e) / sqrt(d)
    float scale;               // 1 / sqrt(d)
    uint32_t* dev_error;
};

constexpr float kLog2e = 1.4426950408889634f;

// Scratch rows per head: T rounded up to 32 rows plus 128, so every block of
// up to 128 rows a stage reads lies inside the plane.
constexpr int kScratchPad = 4 * kBN;
inline int64_t scratch_rows(int64_t T) { return (T + kBN - 1) / kBN * kBN + kScratchPad; }
// The dK/dV work queue: one counter per XCD, 64 bytes apart, after the planes.
constexpr int kQueueStride = 16;
constexpr size_t kQueueBytes = (size_t)kNumXcd * kQueueStride * sizeof(int32_t);
inline size_t planes_bytes(int64_t T, int32_t H) { return align_up((size_t)2 * H * scratch_rows(T) * sizeof(float)); }

// Stage geometry.  Measured alternatives: two key halves per dQ stage and
// 2- vs 3-deep dQ rings within 2%; one query half per dK/dV stage 6% slower
// on long segments; a 2-deep dK/dV ring 7% slower on mid-length segments.
constexpr int kDqHalves = 1;      // 32-key halves per dQ stage
constexpr int kDqRing = 2;        // stage buffers of the dQ kernel
constexpr int kDkdvRing = 3;      // stage buffers of the dK/dV kernel
constexpr int kDkdvHalves = 2;    // 32-query halves per dK/dV stage

// s_waitcnt vmcnt(LPS * ahead) for ahead < RING - 1 (expcnt and lgkmcnt left
// open; vmcnt is split over bits 3:0 and 15:14): every stage but the newest
// `ahead` ones has landed for this wave
template <int RING, int LPS>
__device__ __attribute__((always_inline)) inline void wait_stages(int ahead) {
    static_assert((RING - 2) * LPS <= 63, "vmcnt range");
    static_for<RING - 1>([&](auto n) {
        constexpr int v = decltype(n)::value * LPS;
        if (ahead == decltype(n)::value) __builtin_amdgcn_s_waitcnt(0x0F70 | (v & 15) | ((v >> 4) << 14));
    });
}

// ------------------------------------------------------------- shared pieces

// Block index -> logical (head, tile) item: the forward's XCD-contiguous mapping.
__device__ inline int xcd_logical() {
    const int per_xcd = gridDim.x / kNumXcd;
    return (blockIdx.x % kNumXcd) * per_xcd + blockIdx.x / kNumXcd;
}

// Logical item -> (head, tile) in the forward's item order: heads in blocks
// of head_block when some segment spans more than two tiles (else single
// heads), and inside a block a segment's run of tiles for every head of the
// block together.  MIRROR takes a run's tiles from last to first (query tiles:
// the last is the heaviest), else first to last (key tiles: the first is
// seen by every later query).  Heads and tiles stay in range whatever the
// plan holds; an unsealed plan computes nothing.
template <bool MIRROR>
__device__ inline void item_of(const BwdParams& p, int logical, int& head, int& tile) {
    const int hb = p.header[HDR_MAXLEN] > 2 * kBM ? p.head_block : 1;
    const int per_block = hb * p.ntiles;
    const int hblk = logical / per_block;
    const int h0 = hblk * hb;
    const int hx = min(hb, p.H - h0);
    const int i = logical - hblk * per_block;            // < hx * ntiles
    const int pos = i / hx;
    const int2 sr = p.rows[(int64_t)pos * kBM];          // segment of the first row at pos
    int ta = max((sr.x + kBM - 1) / kBM, 0);
    int tb = min((sr.y + kBM - 1) / kBM, p.ntiles);
    if (!(pos >= ta && pos < tb)) {
        ta = pos;
        tb = pos + 1;
    }
    const int run = tb - ta;
    const int local = i - hx * ta;
    const int hl = local / run;
    const int off = local - hl * run;
    head = h0 + hl;
    tile = MIRROR ? tb - 1 - off : ta + off;
}

// Plan header check, read in one piece (see the forward).
__device__ inline bool plan_sealed(const BwdParams& p, bool causal, bool& sealed) {
    const int4 h0 = *reinterpret_cast<const int4*>(p.header);
    const int4 h1 = *reinterpret_cast<const int4*>(p.header + 4);
    // a self-attention plan only: no separate key boundaries
    sealed = (h0.x == kPlanMagic) & (h0.y == (int32_t)p.T) & (h0.z == (causal ? 1 : 0)) & (h0.w == p.ntiles) &
             (h1.z == 0) & (h1.w == (int32_t)p.T);
    return sealed & (h1.y == 1);
}

// ------------------------------------------------------------------ dQ

template <int D, bool CAUSAL, bool OUT_F32, bool F16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdParams p) {
    using E = Elt<F16>;                      // bf16 or fp16 inputs
    using x8 = typename E::x8;
    using x2 = typename E::x2;
    static_assert(D == 64 || D == 128, "head_dim");
    static_assert(kBN == 32, "32-key halves");
    constexpr int NH = kDqHalves;
    constexpr int SKEYS = NH * kBN;                 // keys per stage
    constexpr int NS = D / 16;
    constexpr int ND = D / 32;
    constexpr int ROW_B = D * 2;
    constexpr int TILE_B = kBN * ROW_B;
    constexpr int CHUNKS = TILE_B / 1024;
    constexpr int CPW = CHUNKS / kWaves;
    static_assert(CPW >= 1 && CPW * kWaves == CHUNKS, "staging split");
    constexpr int ROWS_PER_CHUNK = 1024 / ROW_B;
    constexpr int L16 = ROW_B / 16;
    constexpr int CHUNK_ROWS = kWaves * ROWS_PER_CHUNK;
    static_assert(CHUNK_ROWS % 16 == 0, "swizzle period");
    __shared__ __attribute__((aligned(1024))) uint16_t sKV[2 * kDqRing * SKEYS * D];

    const int logical = xcd_logical();
    if (logical >= p.items) return;
    // the dK/dV launch that follows takes its items from these counters
    if (blockIdx.x == 0 && threadIdx.x < kNumXcd * kQueueStride) p.queue[threadIdx.x] = 0;
    // (head, tile) in the forward's order: a segment's heaviest (last) query
    // tile starts first
    int head, tile;
    item_of<true>(p, logical, head, tile);
    const int r0 = tile * kBM;
    const int r1 = (int)min<int64_t>((int64_t)r0 + kBM, p.T);
    const int last_row = (int)(p.T - 1);
    const int H = p.H;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 31;
    const int g = lane >> 5;
    const int wr0 = r0 + 32 * wave;
    const int wr1 = min(wr0 + 32, r1);
    const bool wave_active = wr0 < r1;
    const int row = min(wr0 + c, r1 - 1);

    const int2 mine = p.rows[row];
    const int start_l = mine.x, end_l = mine.y;
    const int2 first = p.rows[min(wr0, r1 - 1)];
    const int2 last = p.rows[max(wr1 - 1, 0)];
    const int w_lo = first.x;
    const int w_hi = CAUSAL ? wr1 : last.y;
    const int max_start = last.x;
    const int min_end = first.y;
    const int k_lo = p.rows[r0].x;
    const int k_hi = CAUSAL ? r1 : p.rows[r1 - 1].y;

    auto row_off = [&](int r) -> int64_t { return ((int64_t)r * H + head) * D; };
    // Q^T and dO^T B operands: lane (c, g) holds X[row][16s + 8g .. +8]
    x8 qreg[NS], doreg[NS];
    {
        const uint16_t* qp = p.q + row_off(row) + 8 * g;
        const uint16_t* gp = p.dout + row_off(row) + 8 * g;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            qreg[s] = *reinterpret_cast<const x8*>(qp + 16 * s);
            doreg[s] = *reinterpret_cast<const x8*>(gp + 16 * s);
        }
    }
    // lse in log2 units and D = dO . O of the lane's row (the lane pair holds
    // the two halves of the row), stored once per row for the dK/dV launch.
    // A padding row (no key: LSE -inf) gets +inf, so its recomputed
    // probabilities exp2(s - lse) are 0 rather than NaN.  The scratch rows
    // past T, which dK/dV stages also read, are zeroed by the workgroups of
    // the last tile.
    float lse2, dlt;
    {
        const float l = p.lse[(int64_t)head * p.T + row];
        lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
        const uint16_t* op = p.out + row_off(row) + 8 * g;
        float part = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const x8 o = *reinterpret_cast<const x8*>(op + 16 * s);
            const x8 d = doreg[s];
            part = E::dot2(__builtin_shufflevector(o, o, 0, 1), __builtin_shufflevector(d, d, 0, 1), part);
            part = E::dot2(__builtin_shufflevector(o, o, 2, 3), __builtin_shufflevector(d, d, 2, 3), part);
            part = E::dot2(__builtin_shufflevector(o, o, 4, 5), __builtin_shufflevector(d, d, 4, 5), part);
            part = E::dot2(__builtin_shufflevector(o, o, 6, 7), __builtin_shufflevector(d, d, 6, 7), part);
        }
        dlt = lane_pair_sum(part);
        if (g == 0 && wave_active && wr0 + c < r1) {
            p.scratch[(int64_t)head * p.Tp + row] = lse2;
            p.scratch[((int64_t)H + head) * p.Tp + row] = dlt;
        }
        if (tile == p.ntiles - 1 && tid < p.Tp - p.T) {
            p.scratch[(int64_t)head * p.Tp + p.T + tid] = 0.0f;
            p.scratch[((int64_t)H + head) * p.Tp + p.T + tid] = 0.0f;
        }
    }
    bool sealed;
    const bool plan_ok = plan_sealed(p, CAUSAL, sealed);
    if (!sealed && tid == 0) raise_error(p.dev_error, PVC_DEV_PLAN);
    const int nstages = plan_ok ? (k_hi - k_lo + SKEYS - 1) / SKEYS : 0;

    // ---- K and V stages, both with the swizzle for tiles read both ways
    // (both are read as A operands row by row; K is also read transposed)
    const int64_t row_stride = (int64_t)H * D;
    const int64_t head_off = (int64_t)head * D;
    const int fetch_rr = wave * ROWS_PER_CHUNK + lane / L16;
    const uint32_t loff =
            (uint32_t)((fetch_rr * row_stride + ((lane % L16) ^ t_swz<D>(fetch_rr)) * 8) * 2);
    char* const kbase = reinterpret_cast<char*>(&sKV[0]);
    char* const vbase = kbase + kDqRing * NH * TILE_B;
    auto fetch_rows = [&](const uint16_t* src, lds_char* dst, int kt) {
        const char* base = reinterpret_cast<const char*>(src) + ((int64_t)kt * row_stride + head_off) * 2;
        const int64_t chunk_step = (int64_t)CHUNK_ROWS * row_stride * 2;
        if (kt + kBN - 1 <= last_row) {
#pragma unroll
            for (int i = 0; i < CPW; ++i) lds_dma16(base + i * chunk_step, loff, dst + (wave + kWaves * i) * 1024);
        } else {
            // rows past the buffer's end re-read its last row (masked later)
            const int base_row = min(kt, last_row);
            const char* b0 = reinterpret_cast<const char*>(src) + ((int64_t)base_row * row_stride + head_off) * 2;
            const uint32_t piece = loff - (uint32_t)(fetch_rr * row_stride * 2);
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                const int rr = min(kt + fetch_rr + i * CHUNK_ROWS, last_row) - base_row;
                lds_dma16(b0, (uint32_t)(rr * row_stride * 2) + piece, dst + (wave + kWaves * i) * 1024);
            }
        }
    };
    lds_char* const k_lds = (lds_char*)kbase;
    lds_char* const v_lds = (lds_char*)vbase;
    auto fetch_stage = [&](int st, int slot) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            fetch_rows(p.k, k_lds + (slot * NH + h) * TILE_B, k_lo + st * SKEYS + h * kBN);
            fetch_rows(p.v, v_lds + (slot * NH + h) * TILE_B, k_lo + st * SKEYS + h * kBN);
        }
    };

    // ---- LDS read offsets (16-byte piece ^ t_swz(row))
    //   row read (A operand): row c, piece 2s + g
    //   transposing read: rows 16ks + 8hh + 4g + li/4, d = 32j + 16chi + 4(li%4)
    uint32_t r_off[NS], t_off[ND][2];
    {
        const int li = lane & 15;
        const int chi = (lane >> 4) & 1;
#pragma unroll
        for (int s = 0; s < NS; ++s) r_off[s] = c * ROW_B + (((2 * s + g) ^ t_swz<D>(c)) << 4);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int rl = 4 * g + (li >> 2) + 8 * hh;
#pragma unroll
            for (int j = 0; j < ND; ++j)
                t_off[j][hh] = rl * ROW_B + (((4 * j + 2 * chi + ((li & 3) >> 1)) ^ t_swz<D>(rl)) << 4) +
                               ((li & 1) << 3);
        }
    }
    auto rop = [&](const char* b, int s) { return *reinterpret_cast<const x8*>(b + r_off[s]); };
    auto top = [&](const char* b, int ks, int j) -> x8 {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + t_off[j][0] + 16 * ks * ROW_B));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + t_off[j][1] + 16 * ks * ROW_B));
        return __builtin_bit_cast(x8, (short __attribute__((ext_vector_type(8)))){
            lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };

    f32x16 acc[ND];
#pragma unroll
    for (int j = 0; j < ND; ++j) acc[j] = f32x16(0.0f);
    const float sl2 = p.scale_log2;
    const int vis_end = CAUSAL ? min(end_l, row + 1) : end_l;

    auto stage_active = [&](int st) -> bool {
        const int kt = k_lo + st * SKEYS;
        return wave_active && kt < w_hi && kt + SKEYS > w_lo;
    };
    auto half_full = [&](int kt) -> bool {
        return kt >= max_start && kt + kBN <= min_end && (!CAUSAL || kt + kBN - 1 <= wr0);
    };
    // one stage: S^T and dP^T of every half first, so one half's MFMA chains
    // overlap the other's exponentials
    auto stage = [&](int st, int slot) __attribute__((always_inline)) {
        f32x16 S[NH], dP[NH];
        x8 ka[NH][NS], va[NH][NS];
#pragma unroll
        for (int s = 0; s < NS; ++s)
            static_for<NH>([&](auto H_) {
                constexpr int h = decltype(H_)::value;
                ka[h][s] = rop(kbase + (slot * NH + h) * TILE_B, s);
                va[h][s] = rop(vbase + (slot * NH + h) * TILE_B, s);
            });
        static_for<NH>([&](auto H_) {
            constexpr int h = decltype(H_)::value;
            S[h] = f32x16(0.0f);
            dP[h] = f32x16(0.0f);
        });
#pragma unroll
        for (int s = 0; s < NS; ++s)
            static_for<NH>([&](auto H_) {
                constexpr int h = decltype(H_)::value;
                S[h] = E::mfma(ka[h][s], qreg[s], S[h]);
                dP[h] = E::mfma(va[h][s], doreg[s], dP[h]);
            });
        // the K and V operand reads run 4 ahead of their MFMAs (mask 0x100 =
        // LDS read, 0x008 = MFMA); with two waves per SIMD a shorter lead
        // than the dK/dV kernel's suffices (8 measured slower here)
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        static_for<2 * NH * NS - 4>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        });
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        static_for<NH>([&](auto H_) {
            constexpr int h = decltype(H_)::value;
            const int kt = k_lo + st * SKEYS + h * kBN;
            if (!half_full(kt)) {
                const int x0 = kt + 4 * g;
                const int lo = start_l - x0, hi = vis_end - x0;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int C = 8 * (r >> 2) + (r & 3);
                    S[h][r] = ((C >= lo) & (C < hi)) ? S[h][r] : -INFINITY;
                }
            }
            // dS^T = P^T o (dP^T - D); keys 16ks + 8(e/4) + 4g + e%4 of pack ks
            x2 pk[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(S[h][2 * i], sl2, -lse2));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(S[h][2 * i + 1], sl2, -lse2));
                pk[i] = E::pair(p0 * (dP[h][2 * i] - dlt), p1 * (dP[h][2 * i + 1] - dlt));
            }
            x8 ds[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                ds[ks] = x8{pk[4 * ks][0], pk[4 * ks][1], pk[4 * ks + 1][0], pk[4 * ks + 1][1],
                                pk[4 * ks + 2][0], pk[4 * ks + 2][1], pk[4 * ks + 3][0], pk[4 * ks + 3][1]};
            const char* kb = kbase + (slot * NH + h) * TILE_B;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < ND; ++j) acc[j] = E::mfma(top(kb, ks, j), ds[ks], acc[j]);   // dQ^T += K^T dS^T
        });
    };

    // stages through a ring of kDqRing K and V buffers: stage st is computed
    // while stages st+1 .. st+kDqRing-1 are in flight
    constexpr int RING = kDqRing;
    static_for<RING - 1>([&](auto i) {
        if (decltype(i)::value < nstages) fetch_stage(decltype(i)::value, decltype(i)::value);
    });
    for (int st0 = 0; st0 < nstages; st0 += RING) {
        static_for<RING>([&](auto I) {
            constexpr int SLOT = decltype(I)::value;
            const int st = st0 + SLOT;
            if (st >= nstages) return;
            wait_stages<RING, 2 * NH * CPW>(min(RING - 2, nstages - 1 - st));   // stage st has landed
            __syncthreads();
            if (st + RING - 1 < nstages) fetch_stage(st + RING - 1, (SLOT + RING - 1) % RING);
            if (stage_active(st)) stage(st, SLOT);
        });
    }

    // ---- epilogue: dQ = s (dQ^T)^T; lane (c, g) holds rows d = 32j + 8(r/4) + 4g + r%4
    if (!plan_ok) return;
    const float sc = p.scale;
    const bool row_ok = wave_active && wr0 + c < r1;
    if constexpr (OUT_F32) {
        if (row_ok) {
            float* o = static_cast<float*>(p.dq) + row_off(row);
#pragma unroll
            for (int j = 0; j < ND; ++j)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq)
                    *reinterpret_cast<f32x4*>(o + 32 * j + 8 * rq + 4 * g) =
                            f32x4{acc[j][4 * rq] * sc, acc[j][4 * rq + 1] * sc, acc[j][4 * rq + 2] * sc,
                                  acc[j][4 * rq + 3] * sc};
        }
    } else {
        // through LDS for whole-row stores, as in the forward
        constexpr int CPR = ROW_B / 16;
        static_assert(kBM * ROW_B <= 2 * kDqRing * NH * TILE_B, "output tile fits the stage buffers");
        __syncthreads();
        char* const ob = kbase + wave * 32 * ROW_B;
#pragma unroll
        for (int j = 0; j < ND; ++j)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const x2 a = E::pair(acc[j][4 * rq] * sc, acc[j][4 * rq + 1] * sc);
                const x2 b = E::pair(acc[j][4 * rq + 2] * sc, acc[j][4 * rq + 3] * sc);
                const int chunk = (4 * j + rq) ^ (c & (CPR - 1));
                *reinterpret_cast<u32x2*>(ob + c * ROW_B + chunk * 16 + g * 8) =
                        u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
            }
        if (wave_active) {
            constexpr int RPI = 64 / CPR;
#pragma unroll
            for (int i = 0; i < 32 / RPI; ++i) {
                const int r = i * RPI + lane / CPR;
                const int kk = lane % CPR;
                const u32x4 val = *reinterpret_cast<const u32x4*>(ob + r * ROW_B + ((kk ^ (r & (CPR - 1))) << 4));
                if (wr0 + r < r1)
                    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.dq) + row_off(wr0 + r) + kk * 8) = val;
            }
        }
    }
}

// --------------------------------------------------------------- dK, dV

template <int D, bool CAUSAL, bool OUT_F32, bool F16, int NH>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdParams p) {
    using E = Elt<F16>;                      // bf16 or fp16 inputs
    using x8 = typename E::x8;
    using x2 = typename E::x2;
    static_assert(D == 64 || D == 128, "head_dim");
    static_assert(kBN == 32, "32-query halves");
    constexpr int SROWS = NH * kBN;               // query rows per stage
    static_assert(SROWS <= kScratchPad, "the lse / D planes are padded past T by kScratchPad rows");
    constexpr int NS = D / 16;
    constexpr int ND = D / 32;
    constexpr int ROW_B = D * 2;
    constexpr int TILE_B = kBN * ROW_B;
    constexpr int CHUNKS = TILE_B / 1024;
    constexpr int CPW = CHUNKS / kWaves;
    static_assert(CPW >= 1 && CPW * kWaves == CHUNKS, "staging split");
    constexpr int ROWS_PER_CHUNK = 1024 / ROW_B;
    constexpr int L16 = ROW_B / 16;
    constexpr int CHUNK_ROWS = kWaves * ROWS_PER_CHUNK;
    static_assert(CHUNK_ROWS % 16 == 0, "swizzle period");
    // Q stages, then dO stages (NH 32-row halves each); per stage and half
    // 32 lse values and 32 D values
    __shared__ __attribute__((aligned(1024))) uint16_t sQO[2 * kDkdvRing * SROWS * D];
    __shared__ __attribute__((aligned(16))) float sLD[kDkdvRing][NH][2][kBN];

    // ---- work queue.  One workgroup per CU takes the (head, key tile) items
    // of its XCD in order from a counter at the end of the scratch buffer
    // (zeroed by the dQ launch).  After an item's last stage the next item's
    // decode, K / V registers and first stages are issued before the
    // current item's epilogue, so those loads overlap its stores and no CU
    // waits for a new workgroup.  Key tiles go in buffer order inside each
    // run: a segment's first key tiles are seen by all its later queries,
    // so they are its heaviest and start first.
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 31;
    const int g = lane >> 5;
    const int last_row = (int)(p.T - 1);
    const int H = p.H;
    bool sealed;
    const bool plan_ok = plan_sealed(p, CAUSAL, sealed);
    if (!sealed && tid == 0) raise_error(p.dev_error, PVC_DEV_PLAN);
    if (!plan_ok) return;                                 // uniform: nothing is computed
    const int xcd = blockIdx.x % kNumXcd;
    const int per_xcd = (p.items + kNumXcd - 1) / kNumXcd;
    int* const ctr = p.queue + kQueueStride * xcd;
    __shared__ int s_tk[2];
    // ticket j of this XCD's queue -> item, or -1 when the queue is drained
    auto item_at = [&](int j) -> int {
        return (unsigned)j < (unsigned)per_xcd && xcd * per_xcd + j < p.items ? xcd * per_xcd + j : -1;
    };

    struct Item {
        int head, r0, r1, kw0, kw1, key, lo_j, hi_j, w_qlo, w_qhi, full_lo, full_hi, q_lo, nstages;
        bool wave_active;
    };
    auto decode = [&](int logical) -> Item {
        Item it;
        int tile;
        item_of<false>(p, logical, it.head, tile);
        it.r0 = tile * kBM;
        it.r1 = (int)min<int64_t>((int64_t)it.r0 + kBM, p.T);
        it.kw0 = it.r0 + 32 * wave;                       // this wave's keys [kw0, kw1)
        it.kw1 = min(it.kw0 + 32, it.r1);
        it.wave_active = it.kw0 < it.r1;
        it.key = min(it.kw0 + c, it.r1 - 1);
        // queries that may see key j: [lo_j, hi_j) = [causal ? j : start_j, end_j)
        const int2 mine = p.rows[it.key];
        it.lo_j = CAUSAL ? it.key : mine.x;
        it.hi_j = mine.y;
        const int2 first = p.rows[min(it.kw0, it.r1 - 1)];
        const int2 last = p.rows[max(it.kw1 - 1, 0)];
        it.w_qlo = CAUSAL ? it.kw0 : first.x;             // smallest lo_j of the wave
        it.w_qhi = last.y;                                 // largest hi_j
        it.full_lo = CAUSAL ? it.kw1 - 1 : last.x;        // largest lo_j
        it.full_hi = first.y;                              // smallest hi_j
        // non-causal stages start on a multiple of 4 rows, so each 16-byte
        // piece of the lse / D planes a stage loads is aligned
        it.q_lo = CAUSAL ? it.r0 : (p.rows[it.r0].x & ~3);
        const int q_hi = p.rows[it.r1 - 1].y;
        it.nstages = (q_hi - it.q_lo + SROWS - 1) / SROWS;
        return it;
    };
    auto row_off = [&](int r, int head) -> int64_t { return ((int64_t)r * H + head) * D; };
    // K^T and V^T B operands: lane (c, g) holds X[key][16s + 8g .. +8]
    x8 kreg[NS], vreg[NS];
    auto load_kv = [&](const Item& it) {
        const uint16_t* kp = p.k + row_off(it.key, it.head) + 8 * g;
        const uint16_t* vp = p.v + row_off(it.key, it.head) + 8 * g;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            kreg[s] = *reinterpret_cast<const x8*>(kp + 16 * s);
            vreg[s] = *reinterpret_cast<const x8*>(vp + 16 * s);
        }
    };

    // ---- Q and dO stages (swizzled by t_swz), lse and D blocks (128 bytes each)
    const int64_t row_stride = (int64_t)H * D;
    const int fetch_rr = wave * ROWS_PER_CHUNK + lane / L16;
    const uint32_t loff =
            (uint32_t)((fetch_rr * row_stride + ((lane % L16) ^ t_swz<D>(fetch_rr)) * 8) * 2);
    char* const qbase = reinterpret_cast<char*>(&sQO[0]);
    char* const obase = qbase + kDkdvRing * NH * TILE_B;
    auto fetch_rows = [&](const uint16_t* src, lds_char* dst, int kt, int64_t head_off) {
        const char* base = reinterpret_cast<const char*>(src) + ((int64_t)kt * row_stride + head_off) * 2;
        const int64_t chunk_step = (int64_t)CHUNK_ROWS * row_stride * 2;
        if (kt + kBN - 1 <= last_row) {
#pragma unroll
            for (int i = 0; i < CPW; ++i) lds_dma16(base + i * chunk_step, loff, dst + (wave + kWaves * i) * 1024);
        } else {
            const int base_row = min(kt, last_row);
            const char* b0 = reinterpret_cast<const char*>(src) + ((int64_t)base_row * row_stride + head_off) * 2;
            const uint32_t piece = loff - (uint32_t)(fetch_rr * row_stride * 2);
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                const int rr = min(kt + fetch_rr + i * CHUNK_ROWS, last_row) - base_row;
                lds_dma16(b0, (uint32_t)(rr * row_stride * 2) + piece, dst + (wave + kWaves * i) * 1024);
            }
        }
    };
    lds_char* const q_lds = (lds_char*)qbase;
    lds_char* const o_lds = (lds_char*)obase;
    lds_char* const ld_lds = (lds_char*)&sLD[0][0][0];
    // the lse and D values of a stage are 16 NH pieces of 16 bytes, laid out
    // [half][plane][8 pieces]; every wave loads 4 NH of them (lanes 0 ..
    // 4 NH - 1), so all waves issue the same number of loads per stage.
    // Piece P = 4 NH wave + lane holds rows qt + 32 (P / 16) + 4 (P % 8) .. +3
    // of plane (P / 8) % 2 (the planes are padded by kScratchPad rows past T,
    // so every piece lies inside them).
    const char* const sbase = reinterpret_cast<const char*>(p.scratch);
    constexpr int PPW = 4 * NH;                      // pieces per wave
    const int piece = PPW * wave + (lane & (PPW - 1));
    auto fetch_stage = [&](const Item& it, int st, int slot) {
        const int64_t head_off = (int64_t)it.head * D;
        const int64_t piece_row = ((piece >> 3) & 1 ? (int64_t)H + it.head : (int64_t)it.head) * p.Tp +
                                  (piece >> 4) * kBN + 4 * (piece & 7);
        const int qt = it.q_lo + st * SROWS;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            fetch_rows(p.q, q_lds + (slot * NH + h) * TILE_B, qt + h * kBN, head_off);
            fetch_rows(p.dout, o_lds + (slot * NH + h) * TILE_B, qt + h * kBN, head_off);
        }
        // the LDS destination is wave-uniform; readfirstlane keeps it scalar
        const int ld_dst = __builtin_amdgcn_readfirstlane((slot * NH * 2 * kBN + PPW * 4 * wave) * 4);
        if (lane < PPW) lds_dma16(sbase, (uint32_t)((piece_row + qt) * 4), ld_lds + ld_dst);
    };

    uint32_t r_off[NS], t_off[ND][2];
    {
        const int li = lane & 15;
        const int chi = (lane >> 4) & 1;
#pragma unroll
        for (int s = 0; s < NS; ++s) r_off[s] = c * ROW_B + (((2 * s + g) ^ t_swz<D>(c)) << 4);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int rl = 4 * g + (li >> 2) + 8 * hh;
#pragma unroll
            for (int j = 0; j < ND; ++j)
                t_off[j][hh] = rl * ROW_B + (((4 * j + 2 * chi + ((li & 3) >> 1)) ^ t_swz<D>(rl)) << 4) +
                               ((li & 1) << 3);
        }
    }
    auto rop = [&](const char* b, int s) { return *reinterpret_cast<const x8*>(b + r_off[s]); };
    auto top = [&](const char* b, int ks, int j) -> x8 {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + t_off[j][0] + 16 * ks * ROW_B));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + t_off[j][1] + 16 * ks * ROW_B));
        return __builtin_bit_cast(x8, (short __attribute__((ext_vector_type(8)))){
            lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };

    f32x16 accV[ND], accK[ND];
    const float sl2 = p.scale_log2;

    auto stage_active = [&](const Item& it, int st) -> bool {
        const int qt = it.q_lo + st * SROWS;
        return it.wave_active && qt + SROWS > it.w_qlo && qt < it.w_qhi;
    };
    auto half_full = [&](const Item& it, int qt) -> bool { return qt >= it.full_lo && qt + kBN <= it.full_hi; };
    auto pack = [&](const x2 (&pk)[8], x8 (&outp)[2]) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            outp[ks] = x8{pk[4 * ks][0], pk[4 * ks][1], pk[4 * ks + 1][0], pk[4 * ks + 1][1],
                              pk[4 * ks + 2][0], pk[4 * ks + 2][1], pk[4 * ks + 3][0], pk[4 * ks + 3][1]};
    };
    // one stage: S = Q K^T and dP = dO V^T for every half first, so the
    // MFMA chains of one half overlap the exp / pack work of the other
    auto stage = [&](const Item& it, int st, int slot) __attribute__((always_inline)) {
        const int qt = it.q_lo + st * SROWS;
        f32x16 S[NH], dP[NH];
        x8 qa[NH][NS], oa[NH][NS];
#pragma unroll
        for (int s = 0; s < NS; ++s)
            static_for<NH>([&](auto H_) {
                constexpr int h = decltype(H_)::value;
                qa[h][s] = rop(qbase + (slot * NH + h) * TILE_B, s);
                oa[h][s] = rop(obase + (slot * NH + h) * TILE_B, s);
            });
        static_for<NH>([&](auto H_) {
            constexpr int h = decltype(H_)::value;
            S[h] = f32x16(0.0f);
            dP[h] = f32x16(0.0f);
        });
#pragma unroll
        for (int s = 0; s < NS; ++s)
            static_for<NH>([&](auto H_) {
                constexpr int h = decltype(H_)::value;
                S[h] = E::mfma(qa[h][s], kreg[s], S[h]);
                dP[h] = E::mfma(oa[h][s], vreg[s], dP[h]);
            });
        // schedule: the LDS reads of the A operands run 8 ahead of the MFMAs
        // that take them (mask 0x100 = LDS read, 0x008 = MFMA), so one wave
        // per SIMD does not stall on each read's latency; without the fence
        // the compiler issues each read just before its product
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
        static_for<2 * NH * NS - 8>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        });
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        static_for<NH>([&](auto H_) {
            constexpr int h = decltype(H_)::value;
            // lane = key c; register r = query qt + 32h + 8(r/4) + 4g + r%4
            const int qh = qt + h * kBN;
            if (!half_full(it, qh)) {
                const int x0 = qh + 4 * g;
                const int lo = it.lo_j - x0, hi = it.hi_j - x0;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int C = 8 * (r >> 2) + (r & 3);
                    S[h][r] = ((C >= lo) & (C < hi)) ? S[h][r] : -INFINITY;
                }
            }
            const float* ld = &sLD[slot][h][0][0];
            f32x4 l4[4], d4[4];
#pragma unroll
            for (int kq = 0; kq < 4; ++kq) {
                l4[kq] = *reinterpret_cast<const f32x4*>(ld + 8 * kq + 4 * g);
                d4[kq] = *reinterpret_cast<const f32x4*>(ld + kBN + 8 * kq + 4 * g);
            }
            x2 pp[8], pd[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r0_ = 2 * i, r1_ = 2 * i + 1;
                const float p0 = __builtin_amdgcn_exp2f(fmaf(S[h][r0_], sl2, -l4[r0_ >> 2][r0_ & 3]));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(S[h][r1_], sl2, -l4[r1_ >> 2][r1_ & 3]));
                pp[i] = E::pair(p0, p1);
                pd[i] = E::pair(p0 * (dP[h][r0_] - d4[r0_ >> 2][r0_ & 3]),
                                p1 * (dP[h][r1_] - d4[r1_ >> 2][r1_ & 3]));
            }
            x8 Pb[2], Db[2];
            pack(pp, Pb);
            pack(pd, Db);
            const char* qb = qbase + (slot * NH + h) * TILE_B;
            const char* ob = obase + (slot * NH + h) * TILE_B;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < ND; ++j) {
                    accV[j] = E::mfma(top(ob, ks, j), Pb[ks], accV[j]);   // dV^T += dO^T P
                    accK[j] = E::mfma(top(qb, ks, j), Db[ks], accK[j]);   // dK^T += Q^T dS
                }
        });
    };

    constexpr int RING = kDkdvRing;
    static_assert(NH == 2, "the epilogue stages two waves' rows in each Q or dO buffer of the last ring slot");
    static_assert(kBM * ROW_B <= 2 * NH * TILE_B, "output tile fits one ring slot of Q and dO");
    const float sc = p.scale;
    // one item's dV and dK: lane (c, g) holds rows d = 32j + 8(r/4) + 4g + r%4
    // of dV^T and dK^T for key kw0 + c.  The bf16 tile goes through the last
    // ring slot (the next item's first stages fill the others).
    auto epilogue = [&](const Item& it) {
        if constexpr (OUT_F32) {
            if (it.wave_active && it.kw0 + c < it.kw1) {
                float* ov = static_cast<float*>(p.dv) + row_off(it.key, it.head);
                float* ok = static_cast<float*>(p.dk) + row_off(it.key, it.head);
#pragma unroll
                for (int j = 0; j < ND; ++j)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        const int d0 = 32 * j + 8 * rq + 4 * g;
                        *reinterpret_cast<f32x4*>(ov + d0) =
                                f32x4{accV[j][4 * rq], accV[j][4 * rq + 1], accV[j][4 * rq + 2], accV[j][4 * rq + 3]};
                        *reinterpret_cast<f32x4*>(ok + d0) =
                                f32x4{accK[j][4 * rq] * sc, accK[j][4 * rq + 1] * sc, accK[j][4 * rq + 2] * sc,
                                      accK[j][4 * rq + 3] * sc};
                    }
            }
        } else {
            constexpr int CPR = ROW_B / 16;
            char* const ob = (wave < 2 ? qbase : obase) + (RING - 1) * NH * TILE_B + (wave & 1) * TILE_B;
            auto emit = [&](const f32x16 (&acc)[ND], float mul, uint16_t* dst) {
                __syncthreads();                           // the staging rows are free
#pragma unroll
                for (int j = 0; j < ND; ++j)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        const x2 a = E::pair(acc[j][4 * rq] * mul, acc[j][4 * rq + 1] * mul);
                        const x2 b = E::pair(acc[j][4 * rq + 2] * mul, acc[j][4 * rq + 3] * mul);
                        const int chunk = (4 * j + rq) ^ (c & (CPR - 1));
                        *reinterpret_cast<u32x2*>(ob + c * ROW_B + chunk * 16 + g * 8) =
                                u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
                    }
                if (it.wave_active) {
                    constexpr int RPI = 64 / CPR;
#pragma unroll
                    for (int i = 0; i < 32 / RPI; ++i) {
                        const int r = i * RPI + lane / CPR;
                        const int kk = lane % CPR;
                        const u32x4 val =
                                *reinterpret_cast<const u32x4*>(ob + r * ROW_B + ((kk ^ (r & (CPR - 1))) << 4));
                        if (it.kw0 + r < it.kw1) *reinterpret_cast<u32x4*>(dst + row_off(it.kw0 + r, it.head) + kk * 8) = val;
                    }
                }
            };
            emit(accV, 1.0f, static_cast<uint16_t*>(p.dv));
            emit(accK, sc, static_cast<uint16_t*>(p.dk));
        }
    };
    auto prefetch = [&](const Item& it) {
        static_for<RING - 1>([&](auto i) {
            if (decltype(i)::value < it.nstages) fetch_stage(it, decltype(i)::value, decltype(i)::value);
        });
    };

    if (tid == 0) s_tk[0] = atomicAdd(ctr, 1);
    __syncthreads();
    const int first = item_at(s_tk[0]);
    if (first < 0) return;                                // uniform: the queue is drained
    // The next ticket is taken two stages before an item ends, so the queue
    // hands items out in the order workgroups finish (as a dispatcher would)
    // and the XCD's active key tiles stay neighbours that share Q / dO in L2.
    int nxt = 0;
    Item cur = decode(first);
    load_kv(cur);
    prefetch(cur);
    for (int n = 0;; ++n) {
#pragma unroll
        for (int j = 0; j < ND; ++j) {
            accV[j] = f32x16(0.0f);
            accK[j] = f32x16(0.0f);
        }
        for (int st0 = 0; st0 < cur.nstages; st0 += RING) {
            static_for<RING>([&](auto I) {
                constexpr int SLOT = decltype(I)::value;
                const int st = st0 + SLOT;
                if (st >= cur.nstages) return;
                // stage st has landed.  An item's first wait is for every
                // outstanding load and store: the previous item's stores were
                // issued after this item's first stages.
                if (st == 0) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
                else wait_stages<RING, 2 * NH * CPW + 1>(min(RING - 2, cur.nstages - 1 - st));
                __syncthreads();
                if (st + RING - 1 < cur.nstages) fetch_stage(cur, st + RING - 1, (SLOT + RING - 1) % RING);
                if (st == max(cur.nstages - 2, 0) && tid == 0) nxt = atomicAdd(ctr, 1);
                if (stage_active(cur, st)) stage(cur, st, SLOT);
            });
        }
        if (cur.nstages == 0 && tid == 0) nxt = atomicAdd(ctr, 1);
        if (tid == 0) s_tk[(n + 1) & 1] = nxt;
        __syncthreads();                                  // the ring is consumed and the ticket visible
        const int following = item_at(s_tk[(n + 1) & 1]);
        Item next = cur;
        if (following >= 0) {
            next = decode(following);
            load_kv(next);
            prefetch(next);
        }
        epilogue(cur);
        if (following < 0) break;
        cur = next;
    }
}

// ------------------------------------------------------------------- host


// dQ first: it writes the lse / D planes that dK/dV reads.
template <int D, bool F16>
pvc_status launch_bwd(const BwdParams& prm, bool causal, bool out_f32, hipStream_t s) {
    static_assert(kThreads >= kBN - 1 + kScratchPad, "the last tile's workgroup zeroes every scratch row past T");
    static_assert(kThreads >= kNumXcd * kQueueStride, "the first dQ workgroup zeroes the queue");
    const int64_t grid = ((int64_t)prm.items + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (grid > 0x7fffffffLL) return PVC_ERR_INVALID_ARG;
    dim3 g((unsigned)grid), blk(kThreads);
    // dK/dV: one workgroup per CU (its register use allows no more), a
    // multiple of the XCD count so every XCD's queue has workgroups
    const int64_t per_cu = std::max<int64_t>(kNumXcd, device_cu_count() / kNumXcd * kNumXcd);
    dim3 gk((unsigned)std::min<int64_t>(grid, per_cu));
    if (causal) {
        if (out_f32) {
            hipLaunchKernelGGL((bwd_dq_kernel<D, true, true, F16>), g, blk, 0, s, prm);
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, true, F16, kDkdvHalves>), gk, blk, 0, s, prm);
        } else {
            hipLaunchKernelGGL((bwd_dq_kernel<D, true, false, F16>), g, blk, 0, s, prm);
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, false, F16, kDkdvHalves>), gk, blk, 0, s, prm);
        }
    } else {
        if (out_f32) {
            hipLaunchKernelGGL((bwd_dq_kernel<D, false, true, F16>), g, blk, 0, s, prm);
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, true, F16, kDkdvHalves>), gk, blk, 0, s, prm);
        } else {
            hipLaunchKernelGGL((bwd_dq_kernel<D, false, false, F16>), g, blk, 0, s, prm);
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, false, F16, kDkdvHalves>), gk, blk, 0, s, prm);
        }
    }
    return launch_status();
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

constexpr int64_t kMaxRowElems = (int64_t)1 << 24;

}  // namespace
}  // namespace pvc

using namespace pvc;
using namespace pvc::attn;

extern "C" size_t pvc_attn_bwd_scratch_size(int64_t total_tokens, int32_t heads) {
    if (total_tokens < 1 || total_tokens > 0x7fffffffLL || heads < 1) return 0;
    return planes_bytes(total_tokens, heads) + kQueueBytes;
}

extern "C" pvc_status pvc_varlen_attn_bwd_planned(const void* q, const void* k, const void* v, const void* out,
                                                  const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                                  int64_t total_tokens, int32_t heads, int32_t head_dim,
                                                  int32_t causal, int32_t grad_dtype, const void* workspace,
                                                  size_t workspace_bytes, void* scratch, size_t scratch_bytes,
                                                  uint32_t* dev_error, void* stream) {
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || dout == nullptr || lse == nullptr ||
        dq == nullptr || dk == nullptr || dv == nullptr || workspace == nullptr || scratch == nullptr)
        return PVC_ERR_NULL;
    if (total_tokens < 1 || total_tokens > 0x7fffffffLL || heads < 1) return PVC_ERR_INVALID_ARG;
    if (grad_dtype != PVC_OUT_BF16 && grad_dtype != PVC_OUT_F32 && grad_dtype != PVC_OUT_F16 &&
        grad_dtype != PVC_OUT_F16_F32)
        return PVC_ERR_INVALID_ARG;
    const bool f16 = grad_dtype == PVC_OUT_F16 || grad_dtype == PVC_OUT_F16_F32;
    const bool f32 = grad_dtype == PVC_OUT_F32 || grad_dtype == PVC_OUT_F16_F32;
    if (head_dim != 64 && head_dim != 128) return PVC_ERR_UNSUPPORTED;
    const void* in16[] = {q, k, v, out, dout, dq, dk, dv, lse, scratch};
    for (const void* ptr : in16)
        if (!aligned16(ptr)) return PVC_ERR_INVALID_ARG;
    const PlanLayout L = plan_layout(total_tokens);
    if (workspace_bytes < L.total) return PVC_ERR_WORKSPACE;
    if (scratch_bytes < pvc_attn_bwd_scratch_size(total_tokens, heads)) return PVC_ERR_WORKSPACE;
    if ((int64_t)heads * head_dim > kMaxRowElems) return PVC_ERR_INVALID_ARG;
    if (L.ntiles * (int64_t)heads > 0x7ffffff0LL) return PVC_ERR_INVALID_ARG;
    // the lse / D blocks are addressed by 32-bit byte offsets into the scratch
    if ((int64_t)2 * heads * scratch_rows(total_tokens) * 4 >= ((int64_t)1 << 32)) return PVC_ERR_INVALID_ARG;
    const size_t in_bytes = (size_t)total_tokens * heads * head_dim * 2;
    const size_t g_bytes = in_bytes * (f32 ? 2 : 1);
    const void* ins[] = {q, k, v, out, dout};
    void* outs[] = {dq, dk, dv};
    for (void* o : outs) {
        for (const void* i : ins)
            if (overlaps(o, g_bytes, i, in_bytes)) return PVC_ERR_INVALID_ARG;
        if (overlaps(o, g_bytes, scratch, scratch_bytes)) return PVC_ERR_INVALID_ARG;
    }
    if (overlaps(dq, g_bytes, dk, g_bytes) || overlaps(dq, g_bytes, dv, g_bytes) || overlaps(dk, g_bytes, dv, g_bytes))
        return PVC_ERR_INVALID_ARG;
    const char* ws = static_cast<const char*>(workspace);
    BwdParams prm{};
    prm.q = static_cast<const uint16_t*>(q);
    prm.k = static_cast<const uint16_t*>(k);
    prm.v = static_cast<const uint16_t*>(v);
    prm.out = static_cast<const uint16_t*>(out);
    prm.dout = static_cast<const uint16_t*>(dout);
    prm.lse = lse;
    prm.scratch = static_cast<float*>(scratch);
    prm.queue = reinterpret_cast<int32_t*>(static_cast<char*>(scratch) + planes_bytes(total_tokens, heads));
    prm.dq = dq;
    prm.dk = dk;
    prm.dv = dv;
    prm.header = reinterpret_cast<const int32_t*>(ws + L.header);
    prm.rows = reinterpret_cast<const int2*>(ws + L.rows);
    prm.T = total_tokens;
    prm.Tp = scratch_rows(total_tokens);
    prm.H = heads;
    prm.ntiles = (int32_t)L.ntiles;
    prm.items = (int32_t)(L.ntiles * heads);
    prm.head_block = heads % kNumXcd == 0 ? heads / kNumXcd : 1;
    prm.scale_log2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
    prm.scale = (float)(1.0 / sqrt((double)head_dim));
    prm.dev_error = dev_error;
    hipStream_t s = as_stream(stream);
    if (f16) {
        if (head_dim == 128) return launch_bwd<128, true>(prm, causal != 0, f32, s);
        return launch_bwd<64, true>(prm, causal != 0, f32, s);
    }
    if (head_dim == 128) return launch_bwd<128, false>(prm, causal != 0, f32, s);
    return launch_bwd<64, false>(prm, causal != 0, f32, s);
}
