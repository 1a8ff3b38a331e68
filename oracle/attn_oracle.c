/*
 * CPU oracle for packed variable-length attention, fp64.  TEST INFRASTRUCTURE
 * ONLY: the tests, the package smoke check and the benchmark's CPU-baseline leg
 * may load this; the GPU library never does, and this file shares nothing with it.
 *
 * What it computes is the plain definition, written out with no blocking,
 * fusion or reordering:
 *   - segment r of the packed buffer is the half-open token range [cu[r], cu[r+1])
 *     ([charlestar] "nine tokens, three identities": prefix sums of the lengths);
 *   - query i of segment r may see key j iff j is in the same segment and, for
 *     causal attention, j <= i ([charlestar] "EOS is content": the allow()
 *     equation; [compass] "cross-contamination": the block-diagonal mask);
 *   - o_i = softmax(q_i K^T / sqrt(d) + M_i) V with the additive mask M = 0 on
 *     allowed keys and -inf elsewhere, applied before normalising
 *     ([charlestar] "EOS is content": the softmax equation);
 *   - lse_i = m + ln(sum_j exp(s_ij - m)), natural log.
 * Non-causal attention (causal == 0) lets every query see its whole segment.
 *
 * Inputs are bf16 bit patterns (uint16), [T, H, d] row major; each value is
 * decoded exactly to double.  Every sum runs in index order in double.
 *
 * Page tags:
 *   [charlestar] charlestar.github.io "sequence packing and variable-length attention"
 *   [compass]    brenchcc.github.io/llm-compass "Sequence Packing"
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Segment r holding token i: the r with cu[r] <= i < cu[r+1]; -1 if none. */
static int32_t segment_of(const int32_t* cu, int32_t nseg, int64_t i) {
    for (int32_t r = 0; r < nseg; ++r)
        if ((int64_t)cu[r] <= i && i < (int64_t)cu[r + 1]) return r;
    return -1;
}

/*
 * Attention for a list of query rows, all heads.
 *   rows[0..nrows)  token indices of the queries to evaluate
 *   out   [nrows, heads, head_dim] doubles
 *   lse   [nrows, heads] doubles (may be NULL)
 *   scratch  at least max_seqlen doubles (scores of one row)
 * Returns 0, or -1 if a row lies outside every segment.
 */
int oracle_attn_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const int32_t* cu, int32_t nseg, int32_t heads, int32_t head_dim,
                     int32_t causal, const int64_t* rows, int64_t nrows,
                     double* out, double* lse, double* scratch) {
    const double inv_sqrt_d = 1.0 / sqrt((double)head_dim);
    for (int64_t n = 0; n < nrows; ++n) {
        const int64_t i = rows[n];
        const int32_t r = segment_of(cu, nseg, i);
        if (r < 0) return -1;
        const int64_t j_begin = cu[r];
        const int64_t j_end = causal ? i + 1 : (int64_t)cu[r + 1];
        for (int32_t h = 0; h < heads; ++h) {
            const uint16_t* qi = q + (i * heads + h) * (int64_t)head_dim;
            /* scores of the allowed keys; masked keys contribute exp(-inf) = 0 */
            double m = -INFINITY;
            for (int64_t j = j_begin; j < j_end; ++j) {
                const uint16_t* kj = k + (j * heads + h) * (int64_t)head_dim;
                double dot = 0.0;
                for (int32_t c = 0; c < head_dim; ++c)
                    dot += bf16_to_double(qi[c]) * bf16_to_double(kj[c]);
                const double s = dot * inv_sqrt_d;
                scratch[j - j_begin] = s;
                if (s > m) m = s;
            }
            double denom = 0.0;
            for (int64_t j = j_begin; j < j_end; ++j) {
                const double w = exp(scratch[j - j_begin] - m);
                scratch[j - j_begin] = w;
                denom += w;
            }
            /* o_i[c] = sum_j w_j v_j[c] / denom; each sum still runs over j in order */
            double* oi = out + (n * heads + h) * (int64_t)head_dim;
            for (int32_t c = 0; c < head_dim; ++c) oi[c] = 0.0;
            for (int64_t j = j_begin; j < j_end; ++j) {
                const uint16_t* vj = v + (j * heads + h) * (int64_t)head_dim;
                const double w = scratch[j - j_begin];
                for (int32_t c = 0; c < head_dim; ++c) oi[c] += w * bf16_to_double(vj[c]);
            }
            for (int32_t c = 0; c < head_dim; ++c) oi[c] /= denom;
            if (lse) lse[n * heads + h] = m + log(denom);
        }
    }
    return 0;
}

/*
 * Gradients of the attention above for one segment and one head, fp64.
 *
 * For a scalar loss with upstream gradient dO = dL/dO, the chain rule through
 * o_i = sum_j p_ij v_j and the softmax p_ij = exp(s_ij) / sum_l exp(s_il) over
 * the allowed keys gives, with s_ij = q_i . k_j / sqrt(d):
 *   dV_j = sum_i p_ij dO_i
 *   dP_ij = dO_i . v_j,   D_i = sum_j p_ij dP_ij = dO_i . o_i
 *   dS_ij = p_ij (dP_ij - D_i)             (softmax Jacobian; masked p_ij = 0)
 *   dQ_i = sum_j dS_ij k_j / sqrt(d),  dK_j = sum_i dS_ij q_i / sqrt(d).
 * Masked pairs have p_ij = 0 and contribute nothing; keys of other segments
 * never enter, so a segment's gradients equal those of the segment alone.
 *
 *   q, k, v, dout  the segment's first row of this head; row stride ld
 *                  elements ([T, H, d] row major: ld = H * d); n rows
 *   dq, dk, dv     outputs with the same layout, overwritten
 *   scratch        at least 2 n + d doubles
 * Every sum runs in index order in double.
 */
void oracle_attn_bwd_segment(const double* q, const double* k, const double* v, const double* dout,
                             int64_t n, int32_t d, int64_t ld, int32_t causal, double* dq,
                             double* dk, double* dv, double* scratch) {
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    double* p = scratch;          /* p_ij of one query row */
    double* ds = scratch + n;     /* dS_ij of one query row */
    double* o = scratch + 2 * n;  /* o_i */
    for (int64_t j = 0; j < n; ++j)
        for (int32_t c = 0; c < d; ++c) {
            dk[j * ld + c] = 0.0;
            dv[j * ld + c] = 0.0;
        }
    for (int64_t i = 0; i < n; ++i) {
        const int64_t j_end = causal ? i + 1 : n;
        const double* qi = q + i * ld;
        const double* gi = dout + i * ld;
        double m = -INFINITY;
        for (int64_t j = 0; j < j_end; ++j) {
            double dot = 0.0;
            for (int32_t c = 0; c < d; ++c) dot += qi[c] * k[j * ld + c];
            p[j] = dot * inv_sqrt_d;
            if (p[j] > m) m = p[j];
        }
        double denom = 0.0;
        for (int64_t j = 0; j < j_end; ++j) {
            p[j] = exp(p[j] - m);
            denom += p[j];
        }
        for (int64_t j = 0; j < j_end; ++j) p[j] /= denom;
        for (int32_t c = 0; c < d; ++c) o[c] = 0.0;
        for (int64_t j = 0; j < j_end; ++j)
            for (int32_t c = 0; c < d; ++c) o[c] += p[j] * v[j * ld + c];
        double D = 0.0;
        for (int32_t c = 0; c < d; ++c) D += gi[c] * o[c];
        for (int64_t j = 0; j < j_end; ++j) {
            double dp = 0.0;
            for (int32_t c = 0; c < d; ++c) dp += gi[c] * v[j * ld + c];
            ds[j] = p[j] * (dp - D);
        }
        double* dqi = dq + i * ld;
        for (int32_t c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < j_end; ++j) acc += ds[j] * k[j * ld + c];
            dqi[c] = acc * inv_sqrt_d;
        }
        for (int64_t j = 0; j < j_end; ++j)
            for (int32_t c = 0; c < d; ++c) {
                dk[j * ld + c] += ds[j] * qi[c] * inv_sqrt_d;
                dv[j * ld + c] += p[j] * gi[c];
            }
    }
}
