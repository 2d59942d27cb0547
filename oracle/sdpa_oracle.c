/*
 * Plain fp64 CPU oracle for fused scaled dot-product attention (forward and
 * backward).  TEST INFRASTRUCTURE ONLY: the GPU library never links, loads or
 * calls this file, and this file includes nothing from the GPU library.
 *
 * What it computes is the plain definition, not a tiled algorithm:
 *
 *   forward (Composable Kernel "fmha_bwd_kernel.hpp Source File", formula
 *   comment at the head of the file, lines S, S', S'', P; PyTorch "MHA.cpp",
 *   run_cudnn_SDP_fprop, which returns O and fp32 softmax stats [b,h,s_q]):
 *     s_ij  = scale * sum_c Q_ic K_jc + Bias_ij          (allowed j only)
 *     P_ij  = exp(s_ij - m_i) / l_i,  m_i = max_j s_ij,  l_i = sum_j exp(s_ij - m_i)
 *     LSE_i = m_i + ln l_i                               (natural log)
 *     Z_ij  = keep(b,h,i,j) / (1 - p)   if p > 0, else 1
 *     O_ie  = sum_j P_ij Z_ij V_je
 *
 *   backward (same formula comment, lines dV, dP, D, dS'', dBias, dK, dQ):
 *     D_i    = sum_e dO_ie O_ie                         (O from this oracle, fp64)
 *     dV_je  = sum_i P_ij Z_ij dO_ie
 *     dP_ij  = Z_ij sum_e dO_ie V_je
 *     dS_ij  = P_ij (dP_ij - D_i)
 *     dBias  = dS
 *     dQ_ic  = scale sum_j dS_ij K_jc
 *     dK_jc  = scale sum_i dS_ij Q_ic
 *
 * Readings of points the pages leave open (each is also listed in the design
 * notes of the repository):
 *   - "causal" is the top-left mask: j is visible from i iff j <= i (the
 *     oneDNN micro SDPA host driver, init_conf_common, names both top-left and
 *     bottom-right kinds; the CK mask object is built with a top-left flag).
 *   - The general mask is a band around the diagonal (CK builds its mask
 *     from a left / right window and the top-left flag, in
 *     FmhaBwdDQDKDVKernel's operator()): j is visible from i iff
 *     lo <= j - i - off <= hi, with off = 0 (top-left) or s_kv - s_q
 *     (bottom-right), lo = -window_left and hi = window_right (either side
 *     unbounded when not given), and causal meaning hi <= 0.
 *   - A row with no visible key has O_i = 0, LSE_i = -inf and zero gradients
 *     (oneDNN's softmax_inf_as_zero flag).
 *   - ALiBi (CK's FmhaBwdAlibiKargs: one fp32 slope per batch and head, and
 *     the position encoding built in FmhaBwdDQDKDVKernel's operator() from
 *     the mask, or bottom-right aligned when there is no mask) adds
 *       -slope * |j - i - off|
 *     to s_ij, with off the mask's alignment (s_kv - s_q bottom-right, 0
 *     top-left; s_kv - s_q without a mask).  It takes the place of Bias.
 *   - Dropout multiplies the normalised P after the row statistics are taken;
 *     LSE comes from the undropped P (CK's init_dropout keeps 1/(1-p) as the
 *     rescale and passes the undropped probability to the D preprocess).
 *   - The keep decision is the counter-based Philox4x32-10 block function of
 *     Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as
 *     1, 2, 3" (SC'11), keyed as documented at keep_bit() below, with an 8-bit
 *     threshold as in CK's init_dropout (p_undrop_in_uint8_t).
 *
 * Every function here is a loop nest over the definition; the only ordering
 * choice is the ascending index order of each sum.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11, section 3.3 and Table 2).            */
/* One round: two 32x32->64 multiplies of counter words 0 and 2 by the      */
/* published multipliers, the high halves XORed with the other two counter  */
/* words and the round key, then a fixed word permutation.  The key is      */
/* advanced by the Weyl constants (golden ratio and sqrt(3)-1) per round.   */
/* ------------------------------------------------------------------------ */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                          uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t prod0 = (uint64_t)PHILOX_M0 * (uint64_t)c0;
        uint64_t prod1 = (uint64_t)PHILOX_M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
        uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += PHILOX_W0;
        k1 += PHILOX_W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Drop threshold: the 8-bit value round(256 p), computed in fp64 from the
 * caller's fp32 probability.  An element is kept iff its random byte is at
 * least this value, so the kept fraction is (256 - threshold) / 256. */
int oracle_drop_threshold(float p) {
    double t = floor(256.0 * (double)p + 0.5);
    if (t < 0.0) t = 0.0;
    if (t > 255.0) t = 255.0;
    return (int)t;
}

/* Keep bit for element (i, j) of head (b, h):
 *   counter = (j >> 2, i >> 2, b*H + h, low 32 bits of offset)
 *   key     = (low 32 bits of seed, high 32 bits of seed)
 *   byte    = (word[i & 3] >> (8 * (j & 3))) & 0xff
 * so one block-function call covers a 4x4 patch of (i, j). */
int oracle_keep_bit(uint64_t seed, uint64_t offset, uint32_t bh, int64_t i,
                    int64_t j, int threshold) {
    uint32_t ctr[4] = {(uint32_t)(j >> 2), (uint32_t)(i >> 2), bh,
                       (uint32_t)(offset & 0xffffffffu)};
    uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
    uint32_t r[4];
    oracle_philox4x32_10(ctr, key, r);
    uint32_t byte = (r[i & 3] >> (8 * (j & 3))) & 0xffu;
    return byte >= (uint32_t)threshold;
}

/* ------------------------------------------------------------------------ */
/* One attention head.  All matrices are row-major with the given leading   */
/* dimensions (elements between consecutive rows); lse and dvec are dense.  */
/* ------------------------------------------------------------------------ */
typedef struct {
    int64_t sq, skv, dqk, dv;
    double scale;
    int32_t causal;
    float p_drop;
    uint64_t seed, offset;
    uint32_t bh; /* b * H + h: the head's index in the dropout counter */
    const double *q, *k, *v, *bias, *dout;
    int64_t ld_q, ld_k, ld_v, ld_bias, ld_do;
    double *o, *lse, *dq, *dk, *dv_out, *dbias, *dvec;
    int64_t ld_o, ld_dq, ld_dk, ld_dv, ld_dbias;
    uint8_t *keep; /* optional [sq][skv] keep bits (allowed (i,j) only) */
    int64_t ld_keep;
    /* General band mask (when band != 0; `causal` is then ignored): key j is
     * visible from row i iff band_lo <= j - i - band_off <= band_hi.
     * band_off = s_kv - s_q aligns the diagonal to the bottom-right corner,
     * 0 to the top-left; band_lo / band_hi bound a sliding window (CK's
     * window_size_left/right with its top-left / bottom-right mask kinds,
     * oneDNN's top-left and bottom-right causal kinds). */
    int32_t band;
    int64_t band_off, band_lo, band_hi;
    /* ALiBi (when alibi != 0): s_ij += -alibi_slope * |j - i - alibi_off| */
    int32_t alibi;
    double alibi_slope;
    int64_t alibi_off;
} oracle_head_t;

/* Visible keys of row i: the contiguous range [*first, *last]; empty when
 * *first > *last.  Without a band: all keys, or top-left causal j <= i. */
static void visible_range(const oracle_head_t *h, int64_t i, int64_t *first, int64_t *last) {
    int64_t f = 0, l = h->skv - 1;
    if (h->band) {
        int64_t lo = i + h->band_off + h->band_lo, hi = i + h->band_off + h->band_hi;
        if (lo > f) f = lo;
        if (hi < l) l = hi;
    } else if (h->causal && i < l) {
        l = i;
    }
    *first = f;
    *last = l;
}

/* Row i of the forward: fills s[0..last] with P_ij (probabilities, undropped)
 * and returns LSE_i.  Returns -inf and leaves s untouched if no key is visible. */
static double row_probs(const oracle_head_t *h, int64_t i, double *s) {
    int64_t first, last;
    visible_range(h, i, &first, &last);
    if (first > last) return -INFINITY;
    const double *qi = h->q + i * h->ld_q;
    for (int64_t j = first; j <= last; ++j) {
        const double *kj = h->k + j * h->ld_k;
        double acc = 0.0;
        for (int64_t c = 0; c < h->dqk; ++c) acc += qi[c] * kj[c];
        s[j] = h->scale * acc + (h->bias ? h->bias[i * h->ld_bias + j] : 0.0);
        if (h->alibi) s[j] -= h->alibi_slope * fabs((double)(j - i - h->alibi_off));
    }
    double m = -INFINITY;
    for (int64_t j = first; j <= last; ++j)
        if (s[j] > m) m = s[j];
    double l = 0.0;
    for (int64_t j = first; j <= last; ++j) l += exp(s[j] - m);
    for (int64_t j = first; j <= last; ++j) s[j] = exp(s[j] - m) / l;
    return m + log(l);
}

/* Z_ij for the visible keys of row i (1 everywhere when p == 0). */
static void row_dropout(const oracle_head_t *h, int64_t i, int64_t first, int64_t last, double *z) {
    if (h->p_drop <= 0.0f) {
        for (int64_t j = first; j <= last; ++j) z[j] = 1.0;
        return;
    }
    int thr = oracle_drop_threshold(h->p_drop);
    double rescale = 1.0 / (1.0 - (double)h->p_drop);
    for (int64_t j = first; j <= last; ++j)
        z[j] = oracle_keep_bit(h->seed, h->offset, h->bh, i, j, thr) ? rescale : 0.0;
}

static void head_fwd(const oracle_head_t *h, double *s, double *z) {
    for (int64_t i = 0; i < h->sq; ++i) {
        double *oi = h->o + i * h->ld_o;
        int64_t first, last;
        visible_range(h, i, &first, &last);
        double lse = row_probs(h, i, s);
        if (h->lse) h->lse[i] = lse;
        for (int64_t e = 0; e < h->dv; ++e) oi[e] = 0.0;
        if (first > last) continue;
        row_dropout(h, i, first, last, z);
        if (h->keep)
            for (int64_t j = first; j <= last; ++j)
                h->keep[i * h->ld_keep + j] = z[j] != 0.0;
        for (int64_t j = first; j <= last; ++j) {
            const double *vj = h->v + j * h->ld_v;
            double w = s[j] * z[j];
            for (int64_t e = 0; e < h->dv; ++e) oi[e] += w * vj[e];
        }
    }
}

/* Backward of one head.  Sums over i (dK, dV) run in ascending i, one row of
 * P at a time; sums over j (dQ) and over e (D, dP) run in ascending order. */
static void head_bwd(const oracle_head_t *h, double *s, double *z, double *oi) {
    for (int64_t j = 0; j < h->skv; ++j) {
        for (int64_t c = 0; c < h->dqk; ++c) h->dk[j * h->ld_dk + c] = 0.0;
        for (int64_t e = 0; e < h->dv; ++e) h->dv_out[j * h->ld_dv + e] = 0.0;
    }
    for (int64_t i = 0; i < h->sq; ++i) {
        double *dqi = h->dq + i * h->ld_dq;
        for (int64_t c = 0; c < h->dqk; ++c) dqi[c] = 0.0;
        if (h->dbias)
            for (int64_t j = 0; j < h->skv; ++j) h->dbias[i * h->ld_dbias + j] = 0.0;
        int64_t first, last;
        visible_range(h, i, &first, &last);
        double lse = row_probs(h, i, s);
        if (first > last) {
            if (h->dvec) h->dvec[i] = 0.0;
            if (h->o) for (int64_t e = 0; e < h->dv; ++e) h->o[i * h->ld_o + e] = 0.0;
            if (h->lse) h->lse[i] = lse;
            continue;
        }
        row_dropout(h, i, first, last, z);
        /* O_i from this oracle's own forward definition */
        for (int64_t e = 0; e < h->dv; ++e) oi[e] = 0.0;
        for (int64_t j = first; j <= last; ++j) {
            const double *vj = h->v + j * h->ld_v;
            double w = s[j] * z[j];
            for (int64_t e = 0; e < h->dv; ++e) oi[e] += w * vj[e];
        }
        const double *doi = h->dout + i * h->ld_do;
        double D = 0.0;
        for (int64_t e = 0; e < h->dv; ++e) D += doi[e] * oi[e];
        if (h->dvec) h->dvec[i] = D;
        if (h->o) for (int64_t e = 0; e < h->dv; ++e) h->o[i * h->ld_o + e] = oi[e];
        if (h->lse) h->lse[i] = lse;
        const double *qi = h->q + i * h->ld_q;
        for (int64_t j = first; j <= last; ++j) {
            const double *vj = h->v + j * h->ld_v;
            const double *kj = h->k + j * h->ld_k;
            double pz = s[j] * z[j];
            /* dV_j += P_ij Z_ij dO_i */
            double *dvj = h->dv_out + j * h->ld_dv;
            for (int64_t e = 0; e < h->dv; ++e) dvj[e] += pz * doi[e];
            /* dP_ij = Z_ij (dO_i . V_j);  dS_ij = P_ij (dP_ij - D_i) */
            double dot = 0.0;
            for (int64_t e = 0; e < h->dv; ++e) dot += doi[e] * vj[e];
            double dS = s[j] * (z[j] * dot - D);
            if (h->dbias) h->dbias[i * h->ld_dbias + j] = dS;
            /* dQ_i += scale dS_ij K_j ;  dK_j += scale dS_ij Q_i */
            double *dkj = h->dk + j * h->ld_dk;
            for (int64_t c = 0; c < h->dqk; ++c) {
                dqi[c] += h->scale * dS * kj[c];
                dkj[c] += h->scale * dS * qi[c];
            }
        }
    }
}

static int64_t max_skv(const oracle_head_t *heads, int64_t n) {
    int64_t m = 1;
    for (int64_t t = 0; t < n; ++t) {
        if (heads[t].skv > m) m = heads[t].skv;
        if (heads[t].dv > m) m = heads[t].dv;
    }
    return m;
}

/* Forward over a list of heads (batch mode and varlen both reduce to a list
 * of independent heads).  threads <= 0 means the OpenMP default. */
void oracle_fwd(const oracle_head_t *heads, int64_t n, int threads) {
    int64_t w = max_skv(heads, n);
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)w);
        double *z = (double *)malloc(sizeof(double) * (size_t)w);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n; ++t) head_fwd(&heads[t], s, z);
        free(s);
        free(z);
    }
}

void oracle_bwd(const oracle_head_t *heads, int64_t n, int threads) {
    int64_t w = max_skv(heads, n);
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)w);
        double *z = (double *)malloc(sizeof(double) * (size_t)w);
        double *oi = (double *)malloc(sizeof(double) * (size_t)w);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < n; ++t) head_bwd(&heads[t], s, z, oi);
        free(s);
        free(z);
        free(oi);
    }
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
