/*
 * pvc.h — C ABI of libpvc: packed variable-length causal attention on
 * AMD Instinct MI355X (gfx950).
 *
 * One packed buffer holds several independent samples back to back with no
 * batch dimension (the THD layout: token-major [total_tokens, heads, head_dim]).
 * Sample boundaries come from cu_seqlens, the prefix sum of the sample
 * lengths: segment r is the token range [cu[r], cu[r+1]).  Attention is
 * block-diagonal: a query sees only keys of its own segment, and with causal
 * masking only keys at or before it.  Rotary positions restart at every
 * segment: token i of segment r has position i - cu[r].
 *
 * Page tags used in the citations below (the pages specify the method):
 *   [vllbc]      blog.vllbc.top  "long-context training: remove padding"
 *   [compass]    brenchcc.github.io/llm-compass  "Sequence Packing"
 *   [m020]       xuujii.github.io/ai-infra-kb  M020 "length grouping, de-padding, packing"
 *   [opworld]    operatorworld.com  "packing and document boundaries"
 *   [charlestar] charlestar.github.io  "sequence packing and variable-length attention"
 *
 * Conventions for every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates no memory; entry points that need scratch space take a caller
 *     workspace and report its size through a *_workspace_size query.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously; no entry point synchronizes the stream
 *     or copies anything back to the host.
 *   - The return value is a pvc_status for errors the host can see from the
 *     arguments alone (null pointers, sizes, unsupported shapes, a too-small
 *     workspace, a failed launch).  Nothing is enqueued when it is not PVC_OK.
 *   - Errors that depend on device data (a malformed cu_seqlens) are OR-ed into
 *     the caller's 32-bit device error word `dev_error` (PVC_DEV_* bits) when
 *     that pointer is non-NULL; the caller zeroes it beforehand and reads it
 *     after synchronizing.  Kernels clamp every index they derive from device
 *     data, so bad data yields a set bit and unspecified outputs, never an
 *     out-of-bounds access.
 *   - bf16 tensors are IEEE bfloat16 bit patterns, row major, contiguous.
 *   - cu_seqlens values and total_tokens fit in int32 ([charlestar] "nine
 *     tokens, three identities": the interface takes int32 prefix sums).
 *   - No global mutable state; per-device properties are cached once.
 *   - Calls on different streams that write the same buffers race; the
 *     library adds no ordering of its own beyond the stream.
 */
#ifndef PVC_H
#define PVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */

typedef int32_t pvc_status;
enum {
    PVC_OK = 0,
    PVC_ERR_NULL = 1,          /* a required pointer is NULL */
    PVC_ERR_INVALID_ARG = 2,   /* a size or flag is out of range */
    PVC_ERR_UNSUPPORTED = 3,   /* a shape the kernels do not implement (e.g. head_dim) */
    PVC_ERR_WORKSPACE = 4,     /* workspace NULL or smaller than the size query */
    PVC_ERR_HIP = 5,           /* the HIP runtime reported an error (launch, device) */
    PVC_ERR_SCRATCH_LIMIT = 6  /* an allocation-free entry point got more tokens than
                                  its library-owned scratch holds */
};

/* Bits of the device error word.  The cu_seqlens contract is the one listed
 * in [charlestar] "nine tokens, three identities": cu[0] == 0, strictly
 * increasing (every length positive), cu[nseg] == total_tokens, max_seqlen
 * equal to the largest difference, all values representable in int32. */
enum {
    PVC_DEV_CU0 = 1u,             /* cu[0] != 0 */
    PVC_DEV_NOT_INCREASING = 2u,  /* some cu[r+1] <= cu[r] */
    PVC_DEV_TOTAL = 4u,           /* cu[nseg] (or the sum of lengths) != total_tokens */
    PVC_DEV_MAXSEQ = 8u,          /* a segment is longer than max_seqlen (a larger
                                     max_seqlen is accepted) */
    PVC_DEV_LENGTH = 16u,         /* pack_build: a sample length <= 0 */
    PVC_DEV_MISMATCH = 32u,       /* validate: cu disagrees with the given lengths
                                     ([charlestar]: [0,4,5,9] looks like a prefix sum
                                     of [3,2,4] but moves b0 into A) */
    PVC_DEV_RANGE = 64u,          /* the sum of lengths does not fit in int32 */
    PVC_DEV_PLAN = 128u,          /* attention run with a plan built for other arguments */
    PVC_DEV_LABEL = 256u,         /* packed CE: a label outside [0, vocab) that is not
                                     the ignore index (the row is not a target) */
    PVC_DEV_PADDED = 512u         /* cu_seqlens_padded: a slot shorter than its segment */
};

/* Static text for a status code (never NULL). */
const char* pvc_status_string(pvc_status status);

/* Library version string, e.g. "pvc 0.1.0 gfx950". */
const char* pvc_version(void);

/* ------------------------------------------------------------ pack_build */

/* Bytes of device workspace pvc_pack_build needs for `nseg` samples and
 * `total_tokens` tokens (0: no workspace needed).  Above 8192 samples it
 * holds the scan's per-chunk partials; above 2^20 tokens, the segment at
 * which each 2048-token block of the per-token pass starts (written by the
 * scan, so those blocks need not search cu_seqlens). */
size_t pvc_pack_build_workspace_size(int32_t nseg, int64_t total_tokens);

/*
 * Packing metadata for one buffer of `nseg` samples laid end to end.
 *
 * Computes, for r < nseg and i < total_tokens:
 *   cu_seqlens[0] = 0, cu_seqlens[r+1] = cu_seqlens[r] + lengths[r]
 *       ([vllbc] "three things": prefix sum of the lengths; [charlestar]
 *        "nine tokens, three identities")
 *   segment_ids[i]   = the r with cu[r] <= i < cu[r+1]
 *   position_ids[i]  = i - cu[segment_ids[i]]            (reset per segment)
 *   shifted_labels[i]= tokens[i+1] when i+1 < cu[r+1] and !is_pad[r], else
 *                      ignore_index: next-token targets aligned to the input
 *                      position, so a sample's last token predicts nothing
 *                      ([m020] "06 positions and labels"; [charlestar]
 *                      "cross-boundary prediction pairs": the pre-shifted form)
 *   loss_mask[i]     = shifted_labels[i] != ignore_index
 *   *num_targets     = sum of loss_mask (int64; [charlestar] "distributed
 *                      denominator": an int64 count of valid targets)
 *   *max_seqlen      = max(lengths)  (the longest segment, not the total)
 * A segment with is_pad[r] != 0 is a pad tail: it keeps its own entry in
 * cu_seqlens and all its labels are ignore_index ([compass] "implementation
 * notes": the pad tail is closed off as its own segment with labels -100).
 *
 * lengths   [nseg] int32, every value > 0 (else PVC_DEV_LENGTH)
 * is_pad    [nseg] uint8 or NULL (no pad segments)
 * tokens    [total_tokens] int32 token ids; must not equal ignore_index.  May be
 *           NULL when shifted_labels and loss_mask are NULL.
 * total_tokens  the caller's T; the device checks sum(lengths) == T
 *           (PVC_DEV_TOTAL; tokens past the last segment get segment -1,
 *           position 0 and an ignored label)
 * outputs   cu_seqlens [nseg+1] required; segment_ids, position_ids,
 *           shifted_labels [T] int32, loss_mask [T] uint8, num_targets (int64
 *           scalar), max_seqlen (int32 scalar) each optional (NULL = skip)
 * Bit-exact: integer results only.
 */
pvc_status pvc_pack_build(const int32_t* lengths, const uint8_t* is_pad,
                          const int32_t* tokens, int32_t nseg, int64_t total_tokens,
                          int32_t ignore_index, int32_t* cu_seqlens, int32_t* segment_ids,
                          int32_t* position_ids, int32_t* shifted_labels, uint8_t* loss_mask,
                          int64_t* num_targets, int32_t* max_seqlen, uint32_t* dev_error,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * The per-token half of pvc_pack_build on an existing cu_seqlens [nseg+1]
 * (device): segment_ids, position_ids, shifted_labels, loss_mask and
 * num_targets exactly as defined there ([charlestar] "nine tokens, three
 * identities"; [m020] "06 positions and labels"), for callers whose
 * boundaries already exist, or that run this pass apart from the prefix sum
 * (say, on a second stream beside RoPE, which needs only cu_seqlens).
 * Arguments, optional outputs and errors as for pvc_pack_build; a token
 * outside every segment of a malformed cu gets segment -1, position 0 and an
 * ignored label, and sets PVC_DEV_TOTAL or PVC_DEV_NOT_INCREASING.
 * num_targets is cleared by this call (a one-thread kernel ahead of the pass).
 */
pvc_status pvc_pack_tokens(const int32_t* cu_seqlens, const uint8_t* is_pad, const int32_t* tokens,
                           int32_t nseg, int64_t total_tokens, int32_t ignore_index, int32_t* segment_ids,
                           int32_t* position_ids, int32_t* shifted_labels, uint8_t* loss_mask,
                           int64_t* num_targets, uint32_t* dev_error, void* stream);

/*
 * Check a caller-supplied cu_seqlens [nseg+1] against the contract above and
 * OR the failing PVC_DEV_* bits into *dev_error (required here).  With
 * `lengths` [nseg] non-NULL it also checks cu[r+1] - cu[r] == lengths[r]
 * (PVC_DEV_MISMATCH).
 */
pvc_status pvc_validate_cu_seqlens(const int32_t* cu_seqlens, int32_t nseg,
                                   int64_t total_tokens, int32_t max_seqlen,
                                   const int32_t* lengths, uint32_t* dev_error, void* stream);

/* -------------------------------------------------------------- RoPE */

/*
 * Rotary position embedding with positions reset per segment, on q and
 * (optionally) k, never v ([charlestar] "varlen interface": q and k carry the
 * rotation before attention; [vllbc] THD RoPE recovers local positions from
 * cu_seqlens; [opworld] "pitfall two": reset positions per document).
 *
 * Token i finds its segment r by binary search in cu_seqlens, position
 * p = i - cu[r].  For each head and pair j < head_dim/2 (rotate-half pairing):
 *   f_j   = base^(-2j/head_dim), computed in double and rounded to fp32
 *   theta = fp32(p) * f_j                 (one fp32 product)
 *   y_j          = x_j cos(theta) - x_{j+d/2} sin(theta)
 *   y_{j+d/2}    = x_{j+d/2} cos(theta) + x_j sin(theta)
 * with sin, cos and the rotation in double and one rounding to bf16 (nearest
 * even).  Position 0 is the identity, bit for bit.
 *
 * q_in/q_out  [total_tokens, heads, head_dim] bf16; q_out may equal q_in
 * k_in/k_out  same shape, both NULL to rotate q only; k_out may equal k_in
 * head_dim    even, 2..256
 * A token outside every segment (malformed cu) is copied unrotated and sets
 * PVC_DEV_TOTAL or PVC_DEV_NOT_INCREASING.
 */
pvc_status pvc_rope_thd_apply(const void* q_in, void* q_out, const void* k_in, void* k_out,
                              int64_t total_tokens, int32_t heads, int32_t head_dim,
                              const int32_t* cu_seqlens, int32_t nseg, float base,
                              uint32_t* dev_error, void* stream);

/* pvc_rope_thd_apply with the interleaved pairing (x_{2j}, x_{2j+1}) of the
 * RoFormer construction that [charlestar] "positions and RoPE" cites, in place
 * of rotate-half: y_{2j} = x_{2j} cos - x_{2j+1} sin, y_{2j+1} = x_{2j+1} cos +
 * x_{2j} sin, theta_j = fp32(p) * f_j as above.  Same arguments, precision,
 * alignment rules and errors. */
pvc_status pvc_rope_thd_apply_interleaved(const void* q_in, void* q_out, const void* k_in, void* k_out,
                                          int64_t total_tokens, int32_t heads, int32_t head_dim,
                                          const int32_t* cu_seqlens, int32_t nseg, float base,
                                          uint32_t* dev_error, void* stream);

/* Flags of pvc_rope_thd_apply_ex. */
enum { PVC_ROPE_INTERLEAVED = 1, PVC_ROPE_F16 = 2 };

/* pvc_rope_thd_apply with flags: PVC_ROPE_INTERLEAVED selects the
 * interleaved pairing; PVC_ROPE_F16 makes q and k fp16 ([charlestar]
 * "varlen interface": fp16 or bf16 inputs), the one rounding of the double
 * rotation going to fp16 (nearest even, subnormals kept) instead of bf16.
 * Unknown flag bits -> PVC_ERR_INVALID_ARG; otherwise as pvc_rope_thd_apply. */
pvc_status pvc_rope_thd_apply_ex(const void* q_in, void* q_out, const void* k_in, void* k_out,
                                 int64_t total_tokens, int32_t heads, int32_t head_dim,
                                 const int32_t* cu_seqlens, int32_t nseg, float base, int32_t flags,
                                 uint32_t* dev_error, void* stream);

/* ------------------------------------------------------- attention */

/* Element types of the attention entry points (out_dtype / grad_dtype) and of
 * the cross-entropy logits.  PVC_OUT_BF16 / PVC_OUT_F32: bf16 inputs, bf16 or
 * fp32 output.  PVC_OUT_F16 / PVC_OUT_F16_F32: fp16 inputs ([charlestar]
 * "varlen interface": q, k, v in fp16 or bf16), fp16 or fp32 output.  Entry
 * points that take only some of them say so. */
enum { PVC_OUT_BF16 = 0, PVC_OUT_F32 = 1, PVC_OUT_F16 = 2, PVC_OUT_F16_F32 = 3 };

/* Bytes of workspace for a plan over `total_tokens` tokens in `nseg` segments. */
size_t pvc_attn_workspace_size(int64_t total_tokens, int32_t nseg);

/* The workspace query of pvc_varlen_attn_fwd with the arguments of that call
 * ([charlestar] "varlen interface": total tokens, segments, max_seqlen, heads,
 * head_dim).  The workspace is the plan, which depends on total_tokens only:
 * the result equals pvc_attn_workspace_size(total_tokens, nseg). */
size_t pvc_varlen_attn_fwd_workspace_size(int64_t total_tokens, int32_t nseg, int32_t max_seqlen,
                                          int32_t heads, int32_t head_dim);

/*
 * Build the tile plan for one cu_seqlens: every row's key range (its
 * segment), from which the attention kernels derive the same-segment,
 * on-or-below-diagonal blocks they compute ([charlestar] "EOS is content":
 * allow(i,j) = same segment and p_j <= p_i; [opworld] "pitfall one":
 * cross-document blocks are pure waste, which the varlen kernel never
 * computes).  Query tiles of 128 rows run segment by segment in buffer order,
 * each segment's tiles from its end (the heaviest) to its start; with a head
 * count that is a multiple of 8 and a segment longer than two tiles, each
 * segment's run of tiles comes once for every head an XCD owns before the
 * next segment's.  The plan records its longest segment for that choice.
 * cu_seqlens is read on the device only; it is validated as
 * pvc_validate_cu_seqlens would (without lengths) and an invalid cu yields an
 * empty plan plus the error bits.  The plan depends only on
 * (cu_seqlens, nseg, total_tokens, causal), so one plan serves every layer
 * and head that shares the boundaries.
 */
pvc_status pvc_attn_plan(const int32_t* cu_seqlens, int32_t nseg, int64_t total_tokens,
                         int32_t max_seqlen, int32_t causal, void* workspace,
                         size_t workspace_bytes, uint32_t* dev_error, void* stream);

/*
 * The plan for padded storage: logical boundaries apart from storage offsets
 * (the cu_seqlens_padded of Megatron's packed-sequence parameters that [vllbc]
 * "five steps" describes).  Segment r has L_r = cu_seqlens[r+1] -
 * cu_seqlens[r] tokens, stored at rows [cu_seqlens_padded[r],
 * cu_seqlens_padded[r] + L_r) of its slot [cu_seqlens_padded[r],
 * cu_seqlens_padded[r+1]); the rest of the slot is padding.  q, k, v and the
 * outputs of the attention entry points are then [total_rows, heads, d] in
 * that storage; a padding row attends to nothing and is attended by nothing:
 * its output is 0, its LSE -inf, its gradients 0.  (RoPE needs no variant:
 * pvc_rope_thd_apply with cu_seqlens_padded counts positions from each slot's
 * start, which is right for the real tokens.)
 * cu_seqlens_padded [nseg + 1] int32 on the device: cu_seqlens_padded[0] == 0
 * (else PVC_DEV_CU0), each slot at least as long as its segment (else
 * PVC_DEV_PADDED), cu_seqlens_padded[nseg] == total_rows (else PVC_DEV_TOTAL);
 * cu_seqlens as for pvc_attn_plan except that its last entry is the number of
 * real tokens.  The workspace is pvc_attn_workspace_size(total_rows, nseg).
 * Use the plan with total_tokens = total_rows.
 */
pvc_status pvc_attn_plan_padded(const int32_t* cu_seqlens, const int32_t* cu_seqlens_padded, int32_t nseg,
                                int64_t total_rows, int32_t max_seqlen, int32_t causal, void* workspace,
                                size_t workspace_bytes, uint32_t* dev_error, void* stream);

/*
 * The plan for separate query and key boundaries: an inference prefill of
 * independent requests, each with its own keys ([m020] "07 train vs infer":
 * variable-length kernels organise the requests; every request keeps its own
 * KV).  Request r has queries [cu_seqlens_q[r], cu_seqlens_q[r+1]) and keys
 * [cu_seqlens_k[r], cu_seqlens_k[r+1]) (a cached prefix plus its new tokens,
 * for example).  Causal alignment is bottom-right: query a of a request sees
 * keys b <= a + Lk - Lq, so its last query sees every key and Lq == Lk is the
 * ordinary causal mask ([charlestar] "varlen interface" notes that
 * non-square alignment is a separate convention; this is the reading taken).
 * A query that sees no key outputs 0 with LSE -inf.  Both cu arrays
 * [nseg + 1] int32 on the device, strictly increasing from 0 to total_q /
 * total_k, segments at most max_seqlen_q / max_seqlen_k (else the usual error
 * bits and an empty plan).  Workspace pvc_attn_workspace_size(total_q, nseg).
 * The plan also fixes the start order of the forward's 32-row query tiles:
 * each request's tiles in chunks of 16 from its end (the heaviest) down, the
 * chunks longest-first by the keys of their heaviest tile (with more than
 * 2,048 chunks: request by request, each from its end to its start).  The
 * order changes when work starts, never a result.  Used by
 * pvc_varlen_attn_fwd_qk_planned
 * only (a forward: the backward entry refuses this plan).
 */
pvc_status pvc_attn_plan_qk(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t nseg,
                            int64_t total_q, int64_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int32_t causal, void* workspace, size_t workspace_bytes, uint32_t* dev_error,
                            void* stream);

/*
 * Attention forward over a plan of pvc_attn_plan_qk, with grouped key /
 * value heads: q and out [total_q, heads, head_dim], k and v
 * [total_k, kv_heads, head_dim] (bf16, contiguous, 16-byte aligned); query
 * head h reads key / value head h / (heads / kv_heads); heads a multiple of
 * kv_heads.  causal must be the plan's.  lse [heads, total_q] fp32 (natural
 * log), nullable.  out_dtype, head_dim and the errors as for
 * pvc_varlen_attn_fwd_planned; a plan built for other arguments sets
 * PVC_DEV_PLAN and nothing is written.
 */
pvc_status pvc_varlen_attn_fwd_qk_planned(const void* q, const void* k, const void* v, void* out, float* lse,
                                          int64_t total_q, int64_t total_k, int32_t heads, int32_t kv_heads,
                                          int32_t head_dim, int32_t causal, int32_t out_dtype,
                                          const void* workspace, size_t workspace_bytes, uint32_t* dev_error,
                                          void* stream);

/*
 * Attention forward with an existing plan:
 *   out[i,h,:] = sum_j softmax_j(q_i.k_j / sqrt(head_dim) + M_ij) v_j
 * with M_ij = 0 where segment(i) == segment(j) and (j <= i or !causal), -inf
 * elsewhere, applied before normalising ([charlestar] "EOS is content": the
 * masked softmax equation; [compass] "cross-contamination": block-diagonal
 * mask).  causal == 0 lets a query see its whole segment.  The softmax scale is
 * fixed at 1/sqrt(head_dim) ([charlestar]: QK^T / sqrt(d)).
 *
 * q, k, v    [total_tokens, heads, head_dim] (same head count), bf16 for
 *            out_dtype PVC_OUT_BF16 / PVC_OUT_F32, fp16 for PVC_OUT_F16 /
 *            PVC_OUT_F16_F32
 * out        [total_tokens, heads, head_dim], in the input type (PVC_OUT_BF16,
 *            PVC_OUT_F16) or fp32 (PVC_OUT_F32, PVC_OUT_F16_F32: the same
 *            schedule and accumulators, written before the final rounding);
 *            must not alias q, k or v
 * lse        NULL or [heads, total_tokens] fp32: natural-log sum of exponentials
 *            of the scaled scores of each row
 * head_dim   64 or 128; heads * head_dim at most 2^24 (PVC_ERR_INVALID_ARG)
 * total_tokens and causal must be those the plan was built with; otherwise
 * PVC_DEV_PLAN is set and nothing is written.
 * Arithmetic: MFMA products in the input type with fp32 accumulation;
 * probabilities are rounded to the input type (nearest even) for the P.V
 * product and the row sums use those rounded values.  Deterministic: no
 * atomics, results do not depend on scheduling.
 */
pvc_status pvc_varlen_attn_fwd_planned(const void* q, const void* k, const void* v, void* out,
                                       float* lse, int64_t total_tokens, int32_t heads,
                                       int32_t head_dim, int32_t causal, int32_t out_dtype,
                                       const void* workspace, size_t workspace_bytes,
                                       uint32_t* dev_error, void* stream);

/*
 * pvc_attn_plan followed by pvc_varlen_attn_fwd_planned: the varlen interface
 * of [charlestar] "varlen interface" for self-attention (one cu_seqlens for q
 * and k, max_seqlen = the longest segment, no dropout).
 */
pvc_status pvc_varlen_attn_fwd(const void* q, const void* k, const void* v, void* out,
                               float* lse, const int32_t* cu_seqlens, int32_t nseg,
                               int64_t total_tokens, int32_t max_seqlen, int32_t heads,
                               int32_t head_dim, int32_t causal, int32_t out_dtype,
                               void* workspace, size_t workspace_bytes, uint32_t* dev_error,
                               void* stream);

/*
 * pvc_varlen_attn_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same plan and forward, with the plan kept in a
 * library-owned static device array instead of a caller workspace.  No
 * hipMalloc, hipFree or other allocating call is made; the first call on a
 * device looks the array's address up (hipGetSymbolAddress) and caches it.
 * Limit: total_tokens <= pvc_noalloc_max_tokens() (2^20), else
 * PVC_ERR_SCRATCH_LIMIT before any HIP call.  Each GPU holds one 16 MiB
 * array until the process ends, shared by every call on that GPU: calls that
 * overlap on one GPU (other streams, other host threads) race on it and must
 * be serialised by the caller; calls in order on one stream are safe.
 * Arguments, results, determinism and the other errors are those of
 * pvc_varlen_attn_fwd; its outputs are bit-identical to that call's.
 */
int64_t pvc_noalloc_max_tokens(void);
pvc_status pvc_varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                                       const int32_t* cu_seqlens, int32_t nseg, int64_t total_tokens,
                                       int32_t max_seqlen, int32_t heads, int32_t head_dim, int32_t causal,
                                       int32_t out_dtype, uint32_t* dev_error, void* stream);

/*
 * Attention backward with an existing plan (the one the forward used): the
 * gradients of the forward above for an upstream gradient dout,
 *   dV = P^T dO,  dS = P o (dO V^T - D),  D_i = dO_i . O_i,
 *   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),
 * with P the masked softmax of the forward (the calculus of [charlestar]
 * "EOS is content": the masked-softmax equation; masked pairs have P = 0, so
 * no gradient crosses a segment boundary).  P is recomputed from q, k and lse.
 *
 * q, k, v, out, dout  [total_tokens, heads, head_dim], all bf16 (grad_dtype
 *             PVC_OUT_BF16 / PVC_OUT_F32) or all fp16 (PVC_OUT_F16 /
 *             PVC_OUT_F16_F32: [charlestar] "varlen interface", q, k, v in fp16
 *             or bf16); out is the forward's 16-bit output for these q, k, v
 * lse         [heads, total_tokens] fp32, the forward's log-sum-exp (natural log)
 * dq, dk, dv  [total_tokens, heads, head_dim], in the input type (PVC_OUT_BF16,
 *             PVC_OUT_F16) or fp32 (PVC_OUT_F32, PVC_OUT_F16_F32: the same
 *             schedule before the final rounding); must not alias each other,
 *             the inputs or the scratch
 * scratch     device buffer of pvc_attn_bwd_scratch_size bytes (overwritten)
 * head_dim    64 or 128; 2 * heads * (total_tokens + 159) * 4 bytes must stay
 *             below 4 GiB (PVC_ERR_INVALID_ARG otherwise)
 * total_tokens and causal must be those the plan was built with; otherwise
 * PVC_DEV_PLAN is set and no gradient is written (the scratch still is).  All
 * pointers 16-byte aligned.
 * Arithmetic: MFMA products in the input type with fp32 accumulation; P and
 * dS are rounded to the input type (nearest even) for their products.
 * Deterministic: every gradient element is written once by one workgroup and
 * no atomic touches a value (the only atomic hands out dK/dV work items).
 */
size_t pvc_attn_bwd_scratch_size(int64_t total_tokens, int32_t heads);
pvc_status pvc_varlen_attn_bwd_planned(const void* q, const void* k, const void* v, const void* out,
                                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                       int64_t total_tokens, int32_t heads, int32_t head_dim,
                                       int32_t causal, int32_t grad_dtype, const void* workspace,
                                       size_t workspace_bytes, void* scratch, size_t scratch_bytes,
                                       uint32_t* dev_error, void* stream);

/*
 * Padded comparison layout, for measurement: the same attention kernel on a
 * padded SBHD buffer [max_len, batch, heads, head_dim] (bf16) in which sample
 * b occupies rows s < seqlens[b].  Every sample is processed over all max_len
 * rows; keys at or beyond seqlens[b] are masked to -inf but still computed, and
 * padded query rows are computed too ([vllbc] "padding waste": the key-padding
 * mask sets scores to -inf without removing the token, the kernel still sees
 * L).  Only blocks wholly above the causal diagonal are skipped.  out has the
 * input's shape; its padded rows hold attention over the sample's valid keys.
 * seqlens [batch] int32 on the device, each in 1..max_len.  out_dtype
 * PVC_OUT_BF16 or PVC_OUT_F32 (bf16 inputs); batch * heads * head_dim at most
 * 2^24.
 */
pvc_status pvc_padded_attn_fwd_sbhd(const void* q, const void* k, const void* v, void* out,
                                    const int32_t* seqlens, int32_t batch, int32_t max_len,
                                    int32_t heads, int32_t head_dim, int32_t causal,
                                    int32_t out_dtype, void* stream);

/* ------------------------------------------------------ packed cross-entropy */

/* Workspace bytes of pvc_packed_ce_loss for total_tokens rows (0 if out of
 * range). */
size_t pvc_ce_workspace_size(int64_t total_tokens);

/* Cross-entropy over the rows of a packed buffer: the loss summed over the
 * valid targets and the int64 count of valid targets, kept apart rather than
 * averaged ([charlestar] "cross-boundary prediction pairs": reduction "sum"
 * with the ignore index, then the count of labels that are not ignored; no
 * class weights, no label smoothing).  Optionally per-row losses, per-segment
 * sums and counts (the S_r and n_r of [charlestar] "packing should not choose
 * the weight of long samples", for a token or a sample average) and the
 * gradient of the loss sum.
 *
 * logits       [total_tokens rows, vocab] on the device, row stride ld
 *              elements (ld >= vocab); bf16 (logits_dtype PVC_OUT_BF16),
 *              fp16 (PVC_OUT_F16) or fp32 (PVC_OUT_F32).  Rows whose starts are 16-byte aligned are
 *              read as 16-byte vectors, others one value at a time.
 * labels       [total_tokens] int32: the pre-shifted labels of pvc_pack_build
 *              (label[i] is the target of row i; ignore_index where row i
 *              predicts nothing).  A label outside [0, vocab) other than
 *              ignore_index makes the row a non-target and sets
 *              PVC_DEV_LABEL.
 * cu_seqlens   [nseg + 1] int32 (nullable unless seg_loss / seg_count are
 *              given); a malformed cu sets PVC_DEV_CU0 / NOT_INCREASING /
 *              TOTAL and its entries are clamped into [0, total_tokens].
 * loss_sum     [1] fp64 out: the sum of the valid rows' losses.  Each row's
 *              loss is computed in fp32 (log-sum-exp with the row max
 *              subtracted); the sums run in fp64 in a fixed order, so the
 *              result does not depend on scheduling.
 * target_count [1] int64 out: the number of target rows, those whose label
 *              is not ignore_index and lies in [0, vocab) (an ignore_index
 *              inside [0, vocab) still marks a row as ignored).
 * row_loss     [total_tokens] fp32 out, nullable: each row's loss, 0 for a
 *              row that is not a target.
 * seg_loss, seg_count  [nseg] fp64 / int64 out, nullable: the sums over
 *              [cu_r, cu_{r+1}).
 * grad         nullable: [total_tokens, vocab], row stride grad_ld, bf16, fp16
 *              or fp32 (grad_dtype, the same codes): grad_scale * (softmax(z_i) - onehot(y_i)) on
 *              target rows, 0 on the others.  May be the logits buffer itself
 *              (same dtype and stride: computed in place); otherwise it must
 *              not overlap the logits.  grad_scale finite (for example 1/N or
 *              W/N of [charlestar] "the distributed denominator").
 * workspace    >= pvc_ce_workspace_size(total_tokens) bytes, 16-byte aligned.
 * Device outputs are written on `stream`; nothing is synchronized.
 * Errors: NULL required pointer -> PVC_ERR_NULL; total_tokens outside
 * [1, 2^31), vocab < 1, ld < vocab, an unknown dtype, a non-finite scale,
 * nseg outside [1, total_tokens], overlapping outputs -> PVC_ERR_INVALID_ARG;
 * a small workspace -> PVC_ERR_WORKSPACE.
 */
pvc_status pvc_packed_ce_loss(const void* logits, int32_t logits_dtype, int64_t ld, const int32_t* labels,
                              int64_t total_tokens, int32_t vocab, int32_t ignore_index,
                              const int32_t* cu_seqlens, int32_t nseg, double* loss_sum,
                              int64_t* target_count, float* row_loss, double* seg_loss, int64_t* seg_count,
                              void* grad, int32_t grad_dtype, int64_t grad_ld, float grad_scale,
                              void* workspace, size_t workspace_bytes, uint32_t* dev_error, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PVC_H */
