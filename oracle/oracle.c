/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU reference of what the context-parallel attention
 * path computes.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the product library never does, and the two
 * share no code, headers or tables.
 *
 * Sources (the pages this follows, cited by title and section):
 *   [P1] "Breaking the Long-Sequence Inference Bottleneck: A Deep Dive into
 *        vLLM's Distributed Context Parallelism Architecture"
 *   [P3] "vLLM DCP and PCP: Decode and Prefill Context Parallelism"
 *
 * Everything is computed from the *logical* per-request sequences, never from
 * a paged cache, so a wrong slot map, block walk or merge on the device side
 * shows up as a mismatch here.  No blocking, fusion or reordering beyond what
 * the definitions state: scores are formed, the maximum found, the softmax
 * normaliser summed, then the weighted value sum taken.
 *
 * Pinned by tests/test_oracle_pins.py against the pages' worked examples,
 * closed forms, invariants and torch's fp64 scaled_dot_product_attention.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_FP8_E4M3FN 2

/* ------------------------------------------------------------------------ */
/* Element decoding                                                          */
/* ------------------------------------------------------------------------ */

/* bfloat16: the upper 16 bits of an IEEE-754 binary32. */
double oracle_decode_bf16(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit float E4M3 ("fn": finite, no infinities): 1 sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits.  Exponent field 0 encodes subnormals
 * m/8 * 2^(1-7); exponent 15 with mantissa 7 is NaN; every other code is a
 * finite normal number (1 + m/8) * 2^(e-7), so the largest is 448. */
double oracle_decode_e4m3fn(uint8_t bits) {
    int sign = (bits >> 7) & 1;
    int e = (bits >> 3) & 0xF;
    int m = bits & 0x7;
    double mag;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, 1 - 7);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

static double load_elem(const void *base, int64_t idx, int dtype, double scale) {
    switch (dtype) {
    case OR_F32: return (double)((const float *)base)[idx];
    case OR_BF16: return oracle_decode_bf16(((const uint16_t *)base)[idx]);
    case OR_FP8_E4M3FN: return oracle_decode_e4m3fn(((const uint8_t *)base)[idx]) * scale;
    default: return NAN;
    }
}

/* ------------------------------------------------------------------------ */
/* Ownership and paging                                                      */
/* ------------------------------------------------------------------------ */

/* [P1] section 2, "Interleave Size: Controlling the interleaving granularity":
 * the owner of position t is floor(t / interleave_size) mod CP_size. */
int64_t oracle_owner(int64_t t, int64_t N, int64_t I) { return (t / I) % N; }

/* Local KV length of each request on rank r: the number of positions
 * t in [0, L) that rank r owns ([P3] Deep Dive 5, get_dcp_local_seq_lens).
 * Counted, not derived. */
void oracle_local_lens(int64_t B, const int32_t *seq_lens, int64_t rank, int64_t N,
                       int64_t I, int32_t *out) {
    for (int64_t b = 0; b < B; ++b) {
        int64_t n = 0;
        for (int64_t t = 0; t < seq_lens[b]; ++t)
            if (oracle_owner(t, N, I) == rank) ++n;
        out[b] = (int32_t)n;
    }
}

/* Slot mapping on rank r ([P1] section 2, "Diagram: Actual mapping of the
 * Block Table and Slot Mapping"): a token that rank r does not own maps to -1
 * (the cache write skips it).  An owned token is stored at its local index
 * l = number of positions before it that rank r also owns (counted by a scan
 * of the request), in the physical block block_table[req][l / bs] at offset
 * l mod bs.  A local index past the block table's width maps to -2.
 *
 * req[j], pos[j] describe token j; positions of one request need not be
 * sorted or complete. */
void oracle_slot_map(int64_t T, const int32_t *req, const int32_t *pos,
                     const int32_t *block_table, int64_t bt_stride, int64_t max_blocks,
                     int64_t rank, int64_t N, int64_t I, int64_t bs, int64_t *slot_out) {
    /* per request: the largest position asked about, then one counting scan */
    int64_t nreq = 0;
    for (int64_t j = 0; j < T; ++j)
        if (req[j] + 1 > nreq) nreq = req[j] + 1;
    int64_t *maxpos = (int64_t *)calloc((size_t)(nreq > 0 ? nreq : 1), sizeof(int64_t));
    for (int64_t b = 0; b < nreq; ++b) maxpos[b] = -1;
    for (int64_t j = 0; j < T; ++j)
        if (pos[j] > maxpos[req[j]]) maxpos[req[j]] = pos[j];
    int64_t **count_before = (int64_t **)calloc((size_t)(nreq > 0 ? nreq : 1), sizeof(int64_t *));
    for (int64_t b = 0; b < nreq; ++b) {
        if (maxpos[b] < 0) continue;
        count_before[b] = (int64_t *)malloc((size_t)(maxpos[b] + 1) * sizeof(int64_t));
        int64_t seen = 0;
        for (int64_t t = 0; t <= maxpos[b]; ++t) {
            count_before[b][t] = seen;
            if (oracle_owner(t, N, I) == rank) ++seen;
        }
    }
    for (int64_t j = 0; j < T; ++j) {
        int64_t t = pos[j];
        if (oracle_owner(t, N, I) != rank) {
            slot_out[j] = -1;
            continue;
        }
        int64_t l = count_before[req[j]][t];
        int64_t blk = l / bs;
        if (blk >= max_blocks) {
            slot_out[j] = -2;
            continue;
        }
        int64_t phys = block_table[req[j] * bt_stride + blk];
        slot_out[j] = phys * bs + (l % bs);
    }
    for (int64_t b = 0; b < nreq; ++b) free(count_before[b]);
    free(count_before);
    free(maxpos);
}

/* ------------------------------------------------------------------------ */
/* Attention                                                                 */
/* ------------------------------------------------------------------------ */

/* Exact softmax attention of query rows over one logical key/value sequence,
 * restricted to a key set.  [P3] Deep Dive 6, "Deriving the partial and global
 * outputs": for a query q and key set K,
 *     s_j = scale * (q . k_j),   L = log sum_j exp(s_j),
 *     o   = sum_j exp(s_j) v_j / exp(L).
 * (The pages use scale = 1/sqrt(d); here it is an argument.)
 *
 * Query row i, head h (h in heads[], or 0..Hq-1 if heads is NULL) reads key
 * head g = floor(h * Hkv / Hq) and the key set
 *     { t : key_begin[i] <= t < key_end[i],
 *           and, if shard_N > 0, floor(t / shard_I) mod shard_N == shard_r }.
 * An empty set gives o = 0 and L = -inf.
 *
 * Element (token t, head g, column d) of q/k/v lives at index
 *     t * tok_stride + g * head_stride + d   of its array.
 * fp8 elements are decoded and multiplied by the array's scale.
 *
 * out: [n_q][n_heads][Dv], lse: [n_q][n_heads], both fp64, natural log. */
void oracle_attention(int64_t n_q, int64_t Hq, int64_t Hkv, int64_t Dk, int64_t Dv,
                      const int32_t *heads, int64_t n_heads,
                      const void *q, int q_dtype, int64_t q_tok_stride, int64_t q_head_stride,
                      const void *k, int k_dtype, int64_t k_tok_stride, int64_t k_head_stride,
                      double k_scale,
                      const void *v, int v_dtype, int64_t v_tok_stride, int64_t v_head_stride,
                      double v_scale,
                      const int64_t *key_begin, const int64_t *key_end,
                      int64_t shard_N, int64_t shard_I, int64_t shard_r,
                      double scale, double *out, double *lse) {
    int64_t nh = heads ? n_heads : Hq;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int64_t i = 0; i < n_q; ++i) {
        for (int64_t hi = 0; hi < nh; ++hi) {
            int64_t h = heads ? heads[hi] : hi;
            int64_t g = h * Hkv / Hq;
            int64_t lo = key_begin[i], hi_end = key_end[i];
            int64_t n = hi_end > lo ? hi_end - lo : 0;
            double *o = out + (i * nh + hi) * Dv;
            double *qrow = (double *)malloc((size_t)Dk * sizeof(double));
            double *s = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
            char *in_set = (char *)malloc((size_t)(n > 0 ? n : 1));
            for (int64_t d = 0; d < Dk; ++d)
                qrow[d] = load_elem(q, i * q_tok_stride + h * q_head_stride + d, q_dtype, 1.0);
            /* scores over the key set */
            int64_t count = 0;
            double m = -INFINITY;
            for (int64_t j = 0; j < n; ++j) {
                int64_t t = lo + j;
                in_set[j] = (shard_N <= 0) || (oracle_owner(t, shard_N, shard_I) == shard_r);
                if (!in_set[j]) continue;
                double dot = 0.0;
                for (int64_t d = 0; d < Dk; ++d)
                    dot += qrow[d] * load_elem(k, t * k_tok_stride + g * k_head_stride + d,
                                               k_dtype, k_scale);
                s[j] = scale * dot;
                if (s[j] > m) m = s[j];
                ++count;
            }
            for (int64_t d = 0; d < Dv; ++d) o[d] = 0.0;
            if (count == 0) {
                lse[i * nh + hi] = -INFINITY;
            } else {
                /* L = log sum exp(s_j), evaluated as m + log sum exp(s_j - m) */
                double z = 0.0;
                for (int64_t j = 0; j < n; ++j)
                    if (in_set[j]) z += exp(s[j] - m);
                double L = m + log(z);
                lse[i * nh + hi] = L;
                /* o = sum_j exp(s_j - L) v_j */
                for (int64_t j = 0; j < n; ++j) {
                    if (!in_set[j]) continue;
                    int64_t t = lo + j;
                    double w = exp(s[j] - L);
                    for (int64_t d = 0; d < Dv; ++d)
                        o[d] += w * load_elem(v, t * v_tok_stride + g * v_head_stride + d,
                                              v_dtype, v_scale);
                }
            }
            free(in_set);
            free(s);
            free(qrow);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Exact merge of partial results                                            */
/* ------------------------------------------------------------------------ */

/* [P3] Deep Dive 6, "Deriving the partial and global outputs": with
 * l = max_i L_i and a_i = exp(L_i - l),
 *     O = sum_i a_i o_i / sum_i a_i,   L = l + log sum_i a_i.
 * A part with L_i = -inf (empty key set) gets weight 0; if every part is
 * -inf the result is O = 0, L = -inf.
 * part_out: [n_parts][rows][Dv], part_lse: [n_parts][rows]. */
void oracle_lse_merge(int64_t n_parts, int64_t rows, int64_t Dv, const double *part_out,
                      const double *part_lse, double *out, double *lse) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double l = -INFINITY;
        for (int64_t i = 0; i < n_parts; ++i)
            if (part_lse[i * rows + r] > l) l = part_lse[i * rows + r];
        double *o = out + r * Dv;
        for (int64_t d = 0; d < Dv; ++d) o[d] = 0.0;
        if (l == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double asum = 0.0;
        for (int64_t i = 0; i < n_parts; ++i) {
            double Li = part_lse[i * rows + r];
            if (Li == -INFINITY) continue;
            double a = exp(Li - l);
            asum += a;
            const double *oi = part_out + (i * rows + r) * Dv;
            for (int64_t d = 0; d < Dv; ++d) o[d] += a * oi[d];
        }
        for (int64_t d = 0; d < Dv; ++d) o[d] /= asum;
        lse[r] = l + log(asum);
    }
}

/* Threads of the OpenMP loops above (for timing the oracle at a stated core
 * count; the results do not depend on it: every (query row, head) is computed
 * by one thread in the same order). */
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int oracle_max_threads(void) { return omp_get_max_threads(); }
