/*
 * CPU oracle for the compressed branch of Native Sparse Attention (NSA).
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  The product (the HIP library and
 * its Python binding) never calls it, and it shares no code, header, table or
 * helper with the product.
 *
 * What it computes is the plain definition, step by step, in the order the
 * two operator pages give it:
 *
 *   - "aclnnNsaCompress" (CANN operator page), section "Formula": the
 *     compressed keys of a sequence of length t are phi applied to the windows
 *     k_{id+1 : id+l} for 0 <= i <= floor((t-l)/d).  phi is read as a
 *     per-window-position weighted sum with a weight of shape [l, N]: a
 *     scalar per (window position, head), broadcast over the head dim.
 *
 *   - "mindspore.ops.nsa_compress_attention" (MindSpore operator page),
 *     steps 1-7: scaled QK^T, attention mask, softmax -> P_cmp,
 *     attentionOut = P_cmp . value, the importance-score remap
 *     P_slc[j] = sum_{m<l'/d} sum_{n<l/d} P_cmp[l'/d*j - m - n],
 *     the sum of P_slc over the query heads of a KV-head group, the top-k
 *     mask and the top-k indices.
 *
 *   - the selected-block attention that consumes the top-k indices, whose
 *     interface only is given ("lite_boost.ops.rain_fusion_attention"); its
 *     reading is stated at nsa_oracle_select_attention below.
 *
 * Arithmetic is float64 on inputs that are bfloat16 or float16 bit patterns
 * (the two element types the MindSpore page allows for query, key and value)
 * widened exactly.  The one decision that floating point turns into integers (which
 * blocks the top-k picks) is taken on the importance scores rounded to
 * float32, the precision the GPU kernels take it in.
 *
 * Readings of points the pages leave open (each also listed in the design
 * notes of the repository):
 *   - a compressed block i is visible to the query at local position t iff
 *     i*d + l - 1 <= t (the last token of its window is not in the future),
 *     unless an explicit atten_mask is given;
 *   - select block j is a top-k candidate iff j*l' <= t, unless an explicit
 *     topk_mask is given; picks beyond the number of candidates are -1;
 *   - explicit masks (the MindSpore page's optional bool atten_mask and
 *     topk_mask of shape (S1, S2); polarity unstated): one matrix shared by
 *     all sequences, indexed by (local query position t, local compressed
 *     entry i or select block j); a true element masks its pair out, and
 *     the mask given replaces that step's positional rule;
 *   - query head h belongs to KV head floor(h / (N1/N2));
 *   - a remap index outside [0, number of compressed blocks) adds 0;
 *   - l/d in the remap's upper limit is floor(l/d); l'/d is an integer
 *     (the page requires l' % d == 0);
 *   - the number of select blocks of a sequence of length T is ceil(T/l');
 *   - a query with no visible block has output 0, softmax max -inf and
 *     softmax sum 0;
 *   - top-k order: descending score, ties to the lower block index.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#else
#include <time.h>
#endif

/* ---- stage timers (instrumentation for the CPU baseline; no arithmetic) ---
 * Thread-seconds spent in each stage since the last reset: 0 = compression,
 * 1 = scores, mask, softmax and output (steps 1-3), 2 = remap and group sum
 * (steps 4-5), 3 = top-k mask and selection (steps 6-7). */
static double g_stage_s[4];

static double now_s(void)
{
#ifdef _OPENMP
    return omp_get_wtime();
#else
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
#endif
}

void nsa_oracle_stage_reset(void)
{
    for (int i = 0; i < 4; ++i)
        g_stage_s[i] = 0.0;
}

void nsa_oracle_stage_seconds(double* out4)
{
    for (int i = 0; i < 4; ++i)
        out4[i] = g_stage_s[i];
}

/* ---- bfloat16 ------------------------------------------------------------ */

/* Widen a bfloat16 bit pattern: it is the top half of a float32. */
double nsa_oracle_bf16_to_double(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16, ties to even (one rounding step,
 * straight from double).  bfloat16 keeps 8 significant bits and float32's
 * exponent range; below 2^-126 its spacing is fixed at 2^-133. */
uint16_t nsa_oracle_double_to_bf16(double x)
{
    if (isnan(x))
        return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double ax = fabs(x);
    if (ax == 0.0)
        return sign;
    if (isinf(ax))
        return (uint16_t)(sign | 0x7F80);
    int e;
    frexp(ax, &e);                 /* ax = m * 2^e, m in [0.5, 1) */
    int qexp = e - 8;              /* spacing of 8 significant bits */
    if (qexp < -133)
        qexp = -133;               /* subnormal range */
    double r = nearbyint(ldexp(ax, -qexp));  /* default mode: nearest, ties even */
    double y = ldexp(r, qexp);
    const double bf16_max = 3.3895313892515355e38;  /* (2 - 2^-7) * 2^127 */
    if (y > bf16_max)
        return (uint16_t)(sign | 0x7F80);
    float f = (float)y;            /* exact: y has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

void nsa_oracle_round_to_bf16(const double* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = nsa_oracle_double_to_bf16(x[i]);
}

/* ---- float16 (IEEE 754 binary16) ------------------------------------------ */

/* Widen a binary16 bit pattern from its definition: 1 sign bit, 5 exponent
 * bits with bias 15, 10 fraction bits.  Exponent field 0 holds zero and the
 * subnormals f * 2^-24; field 31 holds the infinities and NaNs. */
double nsa_oracle_f16_to_double(uint16_t h)
{
    double sign = (h & 0x8000) ? -1.0 : 1.0;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    if (e == 0)
        return sign * ldexp((double)f, -24);
    if (e == 31)
        return f == 0 ? sign * INFINITY : NAN;
    return sign * ldexp((double)(1024 + f), e - 25);
}

/* Round a double to the nearest binary16, ties to even (one rounding step,
 * straight from double).  binary16 keeps 11 significant bits down to 2^-14
 * and a fixed spacing of 2^-24 below; anything that rounds above the largest
 * finite value 65504 becomes infinity. */
uint16_t nsa_oracle_double_to_f16(double x)
{
    if (isnan(x))
        return 0x7E00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double ax = fabs(x);
    if (ax == 0.0)
        return sign;
    if (isinf(ax))
        return (uint16_t)(sign | 0x7C00);
    int e;
    frexp(ax, &e);                 /* ax = m * 2^e, m in [0.5, 1) */
    int qexp = e - 11;             /* spacing of 11 significant bits */
    if (qexp < -24)
        qexp = -24;                /* subnormal range */
    double r = nearbyint(ldexp(ax, -qexp));  /* default mode: nearest, ties even */
    double y = ldexp(r, qexp);
    if (y > 65504.0)
        return (uint16_t)(sign | 0x7C00);
    if (y < ldexp(1.0, -14))       /* subnormal (or zero): y = r * 2^-24 */
        return (uint16_t)(sign | (uint16_t)r);
    int ey;
    double my = frexp(y, &ey);     /* y = my * 2^ey, my in [0.5, 1) */
    int field = ey - 1 + 15;       /* y = 1.f * 2^(ey-1) */
    int frac = (int)(ldexp(my, 11) - 1024.0);
    return (uint16_t)(sign | (uint16_t)(field << 10) | (uint16_t)frac);
}

void nsa_oracle_round_to_f16(const double* x, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = nsa_oracle_double_to_f16(x[i]);
}

/* Element types of q, k, v and the weight: 0 = bfloat16, 1 = float16. */
static double widen(int dtype, uint16_t h)
{
    return dtype == 1 ? nsa_oracle_f16_to_double(h) : nsa_oracle_bf16_to_double(h);
}

int nsa_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- step A: compression (aclnnNsaCompress, "Formula") -------------------- */

/* Number of windows of a length-T sequence: i runs from 0 to floor((T-l)/d),
 * and there is none when T < l. */
int64_t nsa_oracle_n_cmp(int64_t T, int64_t l, int64_t d)
{
    if (T < l)
        return 0;
    return (T - l) / d + 1;
}

static int64_t seq_start(const int64_t* prefix, int64_t b)
{
    return b == 0 ? 0 : prefix[b - 1];
}

/* x: [T, N, D] (TND, sequences back to back, lengths given as prefix
 * sums act_seq_len[B]); w: [l, N]; both of element type dtype (0 = bfloat16,
 * 1 = float16); out: [sum_b n_cmp_b, N, D] double.
 * out[i, h, e] = sum_{p<l} w[p, h] * x[start + i*d + p, h, e]: the 1-based
 * window k_{id+1 : id+l} is rows i*d .. i*d+l-1 counted from 0. */
int nsa_oracle_compress(const uint16_t* x, const uint16_t* w, const int64_t* act_seq_len,
                        int64_t B, int64_t N, int64_t D, int64_t l, int64_t d, int dtype,
                        double* out)
{
    if (B < 1 || N < 1 || D < 1 || l < 1 || d < 1 || dtype < 0 || dtype > 1)
        return -1;
    const double t_start = now_s();
    int64_t out_row = 0;
    for (int64_t b = 0; b < B; ++b) {
        int64_t start = seq_start(act_seq_len, b);
        int64_t T = act_seq_len[b] - start;
        if (T < 0)
            return -2;
        int64_t n = nsa_oracle_n_cmp(T, l, d);
        for (int64_t i = 0; i < n; ++i) {
            for (int64_t h = 0; h < N; ++h) {
                for (int64_t e = 0; e < D; ++e) {
                    double acc = 0.0;
                    for (int64_t p = 0; p < l; ++p) {
                        double wp = widen(dtype, w[p * N + h]);
                        double xv = widen(dtype, x[((start + i * d + p) * N + h) * D + e]);
                        acc += wp * xv;
                    }
                    out[((out_row + i) * N + h) * D + e] = acc;
                }
            }
        }
        out_row += n;
    }
    g_stage_s[0] += now_s() - t_start;
    return 0;
}

/* ---- steps 1-7 of nsa_compress_attention ---------------------------------- */

/* Which sequence a global token belongs to, and its local position. */
static int64_t find_seq(const int64_t* act_seq_qlen, int64_t B, int64_t tg, int64_t* t_local)
{
    for (int64_t b = 0; b < B; ++b) {
        if (tg < act_seq_qlen[b]) {
            *t_local = tg - seq_start(act_seq_qlen, b);
            return b;
        }
    }
    return -1;
}

/* Steps 1-3 for one (token, query head): scores s_i = scale * <q, k_i> over
 * the visible compressed blocks, the softmax P_cmp and the output
 * sum_i P_i v_i.  P receives P_cmp for every i < n_cmp (0 where masked). */
static void attend_one_head(const uint16_t* qh, const uint16_t* kc, const uint16_t* vc,
                            int64_t cmp0, int64_t n_cmp, int64_t t, int64_t g,
                            int64_t N2, int64_t D1, int64_t D2, double scale,
                            int64_t l, int64_t d, int dtype, const uint8_t* amask_row,
                            double* s, double* P, double* out_h, double* m_out, double* L_out)
{
    /* step 1: QK = scale * query . key^T, then the attention mask (the row
     * of an explicit mask when one is given, else the positional rule). */
    double m = -INFINITY;
    int any = 0;
    for (int64_t i = 0; i < n_cmp; ++i) {
        int visible = amask_row ? (amask_row[i] == 0) : (i * d + l - 1 <= t);
        if (!visible) {
            s[i] = -INFINITY;
            continue;
        }
        const uint16_t* ki = kc + ((cmp0 + i) * N2 + g) * D1;
        double dot = 0.0;
        for (int64_t e = 0; e < D1; ++e)
            dot += widen(dtype, qh[e]) * widen(dtype, ki[e]);
        s[i] = scale * dot;
        if (!any || s[i] > m)
            m = s[i];
        any = 1;
    }
    /* step 2: P_cmp = Softmax(QK), natural base. */
    double L = 0.0;
    for (int64_t i = 0; i < n_cmp; ++i)
        L += (s[i] == -INFINITY) ? 0.0 : exp(s[i] - m);
    for (int64_t i = 0; i < n_cmp; ++i)
        P[i] = (s[i] == -INFINITY) ? 0.0 : exp(s[i] - m) / L;
    /* step 3: attentionOut = P_cmp . value. */
    for (int64_t e = 0; e < D2; ++e) {
        double acc = 0.0;
        for (int64_t i = 0; i < n_cmp; ++i) {
            acc += P[i] * widen(dtype, vc[((cmp0 + i) * N2 + g) * D2 + e]);
        }
        out_h[e] = acc;
    }
    *m_out = any ? m : -INFINITY;
    *L_out = any ? L : 0.0;
}

/* Step 4 for one head: P_slc[j] = sum_{m=0}^{R-1} sum_{n=0}^{L2-1} P[R*j - m - n],
 * R = l'/d and L2 = floor(l/d); indices outside [0, n_cmp) add nothing. */
static void remap_one_head(const double* P, int64_t n_cmp, int64_t S_sel,
                           int64_t R, int64_t L2, double* Pslc_h)
{
    for (int64_t j = 0; j < S_sel; ++j) {
        double acc = 0.0;
        for (int64_t m = 0; m < R; ++m) {
            for (int64_t n = 0; n < L2; ++n) {
                int64_t idx = R * j - m - n;
                if (idx >= 0 && idx < n_cmp)
                    acc += P[idx];
            }
        }
        Pslc_h[j] = acc;
    }
}

/* Steps 6-7 for one (token, KV head): candidates are the j with j*l' <= t;
 * pick the `count` largest scores (descending, ties to the lower j) by
 * repeated selection; slots left over hold -1. */
static void topk_one_group(const double* Pslc_g, int64_t S_sel, int64_t t, int64_t lsel,
                           int64_t count, const uint8_t* tmask_row, unsigned char* taken,
                           int32_t* idx_out)
{
    for (int64_t j = 0; j < S_sel; ++j)   /* topk_mask: not a candidate */
        taken[j] = tmask_row ? (tmask_row[j] != 0) : !(j * lsel <= t);
    for (int64_t k = 0; k < count; ++k) {
        int64_t best = -1;
        float best_v = 0.0f;
        for (int64_t j = 0; j < S_sel; ++j) {
            if (taken[j])
                continue;
            float v = (float)Pslc_g[j];
            if (best < 0 || v > best_v) {
                best = j;
                best_v = v;
            }
        }
        if (best >= 0)
            taken[best] = 1;
        idx_out[k] = (int32_t)best;
    }
}

/*
 * Compressed attention, importance scores and top-k for the listed tokens.
 *
 * q_rows   : [n_tok, N1, D1], the query rows of the listed tokens
 * tokens   : [n_tok] global token indices into the TND query tensor
 * kc, vc   : [T2, N2, D1] and [T2, N2, D2] compressed keys / values
 * dtype    : element type of q_rows, kc and vc: 0 = bfloat16, 1 = float16
 * act_seq_qlen, act_cmp_seq_kvlen : [B] prefix sums of the query and the
 *            compressed lengths of each sequence
 * out      : [n_tok, N1, D2]; smax, ssum: [n_tok, N1]
 * pslc     : [n_tok, N2, s_stride] group-summed importance scores before the
 *            top-k mask, j < ceil(T_b/l'), zero beyond
 * topk     : [n_tok, N2, count] int32
 * atten_mask, am_rows, am_cols : NULL, or a [am_rows, am_cols] byte matrix
 *            (non-zero = masked out) indexed by (local t, compressed entry i);
 *            it needs a row for every local position and a column for every
 *            compressed entry of each sequence
 * topk_mask, tm_rows, tm_cols : NULL, or the same for (local t, select block j)
 * Returns 0, or a negative code for arguments it cannot evaluate.
 */
int nsa_oracle_attention_masked(const uint16_t* q_rows, const int64_t* tokens, int64_t n_tok,
                                const uint16_t* kc, const uint16_t* vc,
                                const int64_t* act_seq_qlen, const int64_t* act_seq_kvlen,
                                const int64_t* act_cmp_seq_kvlen,
                                int64_t B, int64_t N1, int64_t N2, int64_t D1, int64_t D2,
                                double scale, int64_t l, int64_t d, int64_t lsel, int64_t count,
                                int dtype, const uint8_t* atten_mask, int64_t am_rows,
                                int64_t am_cols, const uint8_t* topk_mask, int64_t tm_rows,
                                int64_t tm_cols, double* out, double* smax, double* ssum,
                                double* pslc, int64_t s_stride, int32_t* topk)
{
    if (N2 < 1 || N1 % N2 != 0 || d < 1 || lsel % d != 0 || count < 1 || B < 1 ||
        dtype < 0 || dtype > 1)
        return -1;
    const int64_t G = N1 / N2;
    const int64_t R = lsel / d;
    const int64_t L2 = l / d;
    int64_t n_cmp_max = 0, s_sel_max = 0;
    for (int64_t b = 0; b < B; ++b) {
        int64_t nc = act_cmp_seq_kvlen[b] - seq_start(act_cmp_seq_kvlen, b);
        int64_t T = act_seq_kvlen ? act_seq_kvlen[b] - seq_start(act_seq_kvlen, b)
                                  : act_seq_qlen[b] - seq_start(act_seq_qlen, b);
        int64_t ss = (T + lsel - 1) / lsel;
        if (nc > n_cmp_max) n_cmp_max = nc;
        if (ss > s_sel_max) s_sel_max = ss;
    }
    if (s_stride < s_sel_max)
        return -2;
    int64_t T_max = 0;
    for (int64_t b = 0; b < B; ++b) {
        int64_t T = act_seq_qlen[b] - seq_start(act_seq_qlen, b);
        if (T > T_max) T_max = T;
    }
    if ((atten_mask && (am_rows < T_max || am_cols < n_cmp_max)) ||
        (topk_mask && (tm_rows < T_max || tm_cols < s_sel_max)))
        return -5;
    for (int64_t k = 0; k < n_tok; ++k) {
        int64_t tl = 0;
        if (find_seq(act_seq_qlen, B, tokens[k], &tl) < 0)
            return -3;
    }
    int err = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(n_cmp_max + 1));
        double* P = (double*)malloc(sizeof(double) * (size_t)(n_cmp_max + 1));
        double* Ph = (double*)malloc(sizeof(double) * (size_t)(s_sel_max + 1));
        unsigned char* taken = (unsigned char*)malloc((size_t)(s_sel_max + 1));
        double st_attn = 0.0, st_remap = 0.0, st_topk = 0.0;   /* this thread's stage times */
        if (!s || !P || !Ph || !taken) {
#pragma omp atomic write
            err = -4;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t k = 0; k < n_tok; ++k) {
                int64_t t = 0;
                int64_t b = find_seq(act_seq_qlen, B, tokens[k], &t);
                int64_t T = act_seq_qlen[b] - seq_start(act_seq_qlen, b);
                /* chunked prefill: the queries are the last T of the sequence's
                 * Tkv key/value tokens, so local query t sits at position
                 * pos = Tkv - T + t for both causal rules (bottom-right
                 * alignment); select blocks follow the key/value tokens */
                int64_t Tkv = act_seq_kvlen ? act_seq_kvlen[b] - seq_start(act_seq_kvlen, b) : T;
                int64_t pos = Tkv - T + t;
                int64_t cmp0 = seq_start(act_cmp_seq_kvlen, b);
                int64_t n_cmp = act_cmp_seq_kvlen[b] - cmp0;
                int64_t S_sel = (Tkv + lsel - 1) / lsel;
                double* pslc_k = pslc + k * N2 * s_stride;
                for (int64_t x = 0; x < N2 * s_stride; ++x)
                    pslc_k[x] = 0.0;
                for (int64_t h = 0; h < N1; ++h) {
                    int64_t g = h / G;
                    const double t0 = now_s();
                    attend_one_head(q_rows + (k * N1 + h) * D1, kc, vc, cmp0, n_cmp, pos, g,
                                    N2, D1, D2, scale, l, d, dtype,
                                    atten_mask ? atten_mask + t * am_cols : NULL, s, P,
                                    out + (k * N1 + h) * D2,
                                    smax + k * N1 + h, ssum + k * N1 + h);
                    const double t1 = now_s();
                    /* step 4, then step 5: heads of a group summed in order. */
                    remap_one_head(P, n_cmp, S_sel, R, L2, Ph);
                    for (int64_t j = 0; j < S_sel; ++j)
                        pslc_k[g * s_stride + j] += Ph[j];
                    st_attn += t1 - t0;
                    st_remap += now_s() - t1;
                }
                const double t2 = now_s();
                for (int64_t g = 0; g < N2; ++g)
                    topk_one_group(pslc_k + g * s_stride, S_sel, pos, lsel, count,
                                   topk_mask ? topk_mask + t * tm_cols : NULL, taken,
                                   topk + (k * N2 + g) * count);
                st_topk += now_s() - t2;
            }
        }
#pragma omp critical(nsa_oracle_stage)
        {
            g_stage_s[1] += st_attn;
            g_stage_s[2] += st_remap;
            g_stage_s[3] += st_topk;
        }
        free(s);
        free(P);
        free(Ph);
        free(taken);
    }
    return err;
}

/* The same without explicit masks: the positional rules throughout. */
int nsa_oracle_attention(const uint16_t* q_rows, const int64_t* tokens, int64_t n_tok,
                         const uint16_t* kc, const uint16_t* vc,
                         const int64_t* act_seq_qlen, const int64_t* act_cmp_seq_kvlen, int64_t B,
                         int64_t N1, int64_t N2, int64_t D1, int64_t D2, double scale,
                         int64_t l, int64_t d, int64_t lsel, int64_t count, int dtype,
                         double* out, double* smax, double* ssum,
                         double* pslc, int64_t s_stride, int32_t* topk)
{
    return nsa_oracle_attention_masked(q_rows, tokens, n_tok, kc, vc, act_seq_qlen, NULL,
                                       act_cmp_seq_kvlen, B, N1, N2, D1, D2, scale, l, d, lsel,
                                       count, dtype, NULL, 0, 0, NULL, 0, 0, out, smax, ssum,
                                       pslc, s_stride, topk);
}

/* ---- selected-block attention (the consumer of topk_indices) --------------
 *
 * The pages define this step only through an interface ("lite_boost.ops.
 * rain_fusion_attention": per query, a -1 padded list of KV block indices
 * to attend to, returning the output and the softmax log-sum-exp).  Reading
 * taken, the plainest one the rest supports: query token t (local position
 * in its sequence), query head h of KV group g = floor(h / (N1/N2)), attends
 * to the raw keys s of its own sequence with s <= t whose select block
 * floor(s / l') is listed in topk[t, g, 0..count) (entries outside
 * [0, ceil(T/l')) and repeats add nothing); softmax of scale * q.k over
 * those keys, applied to v.  A query with no such key has output 0 and
 * log-sum-exp -inf.
 *
 * q [T, N1, D1], k [T, N2, D1], v [T, N2, D2] (element type dtype), TND with
 * prefix sums act_seq_qlen[B]; topk [T, N2, count] int32.  Outputs: out
 * [T, N1, D2] and lse [T, N1] (natural log of sum_s exp(score_s)), double.
 * Only the listed tokens (global indices) are evaluated: out and lse have
 * n_tok rows.
 */
int nsa_oracle_select_attention_kv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const int32_t* topk, const int64_t* tokens, int64_t n_tok,
                                   const int64_t* act_seq_qlen, const int64_t* act_seq_kvlen, int64_t B,
                                   int64_t N1, int64_t N2, int64_t D1, int64_t D2, double scale,
                                   int64_t lsel, int64_t count, int dtype, double* out, double* lse)
{
    if (N2 < 1 || N1 % N2 != 0 || lsel < 1 || count < 1 || B < 1 || dtype < 0 || dtype > 1)
        return -1;
    const int64_t G = N1 / N2;
    int64_t T_max = 0;   /* longest key/value sequence */
    for (int64_t b = 0; b < B; ++b) {
        int64_t T = act_seq_qlen[b] - seq_start(act_seq_qlen, b);
        int64_t Tkv = act_seq_kvlen ? act_seq_kvlen[b] - seq_start(act_seq_kvlen, b) : T;
        if (Tkv < T)
            return -2;
        if (Tkv > T_max) T_max = Tkv;
    }
    for (int64_t i = 0; i < n_tok; ++i) {
        int64_t tl = 0;
        if (find_seq(act_seq_qlen, B, tokens[i], &tl) < 0)
            return -3;
    }
    const int64_t S_max = (T_max + lsel - 1) / lsel;
    int err = 0;
#pragma omp parallel
    {
        unsigned char* sel = (unsigned char*)malloc((size_t)(S_max + 1));
        double* s = (double*)malloc(sizeof(double) * (size_t)(T_max + 1));
        if (!sel || !s) {
#pragma omp atomic write
            err = -4;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < n_tok; ++i) {
                int64_t tq = 0;
                const int64_t b = find_seq(act_seq_qlen, B, tokens[i], &tq);
                const int64_t T = act_seq_qlen[b] - seq_start(act_seq_qlen, b);
                /* keys and values of the sequence start at s0 and number Tkv;
                 * chunked prefill puts query tq at position t = Tkv - T + tq */
                const int64_t s0 = act_seq_kvlen ? seq_start(act_seq_kvlen, b) : seq_start(act_seq_qlen, b);
                const int64_t Tkv = act_seq_kvlen ? act_seq_kvlen[b] - s0 : T;
                const int64_t t = Tkv - T + tq;
                const int64_t S = (Tkv + lsel - 1) / lsel;
                for (int64_t g = 0; g < N2; ++g) {
                    /* the listed blocks of (t, g), as a set */
                    for (int64_t j = 0; j < S; ++j)
                        sel[j] = 0;
                    const int32_t* row = topk + (tokens[i] * N2 + g) * count;
                    for (int64_t c = 0; c < count; ++c)
                        if (row[c] >= 0 && row[c] < S)
                            sel[row[c]] = 1;
                    for (int64_t hh = 0; hh < G; ++hh) {
                        const int64_t h = g * G + hh;
                        const uint16_t* qh = q + (tokens[i] * N1 + h) * D1;
                        double m = -INFINITY;
                        for (int64_t x = 0; x <= t; ++x) {
                            s[x] = -INFINITY;
                            if (!sel[x / lsel])
                                continue;
                            const uint16_t* kx = k + ((s0 + x) * N2 + g) * D1;
                            double dot = 0.0;
                            for (int64_t e = 0; e < D1; ++e)
                                dot += widen(dtype, qh[e]) * widen(dtype, kx[e]);
                            s[x] = scale * dot;
                            if (s[x] > m)
                                m = s[x];
                        }
                        double* o = out + (i * N1 + h) * D2;
                        for (int64_t e = 0; e < D2; ++e)
                            o[e] = 0.0;
                        if (m == -INFINITY) {
                            lse[i * N1 + h] = -INFINITY;
                            continue;
                        }
                        double L = 0.0;
                        for (int64_t x = 0; x <= t; ++x)
                            if (s[x] != -INFINITY)
                                L += exp(s[x] - m);
                        for (int64_t x = 0; x <= t; ++x) {
                            if (s[x] == -INFINITY)
                                continue;
                            const double p = exp(s[x] - m) / L;
                            const uint16_t* vx = v + ((s0 + x) * N2 + g) * D2;
                            for (int64_t e = 0; e < D2; ++e)
                                o[e] += p * widen(dtype, vx[e]);
                        }
                        lse[i * N1 + h] = m + log(L);
                    }
                }
            }
        }
        free(sel);
        free(s);
    }
    return err;
}

int nsa_oracle_select_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const int32_t* topk, const int64_t* tokens, int64_t n_tok,
                                const int64_t* act_seq_qlen, int64_t B, int64_t N1, int64_t N2,
                                int64_t D1, int64_t D2, double scale, int64_t lsel, int64_t count,
                                int dtype, double* out, double* lse)
{
    return nsa_oracle_select_attention_kv(q, k, v, topk, tokens, n_tok, act_seq_qlen, NULL, B, N1, N2, D1, D2,
                                          scale, lsel, count, dtype, out, lse);
}

/* ---- backward of compression and compressed attention ---------------------
 *
 * The pages state the training use of the operator (the softmax max and sum
 * outputs are kept for it) but give no backward formulas; these are the
 * derivatives of the forward definitions above, taken with respect to the
 * loss's gradient dout of attention_out only (softmax_max / softmax_sum are
 * statistics, the top-k indices carry no gradient).  Per query row (t, h)
 * with visible blocks i, P_i the softmax, O = sum_i P_i vc_i:
 *   dvc_i += P_i * dout,   dP_i = dout . vc_i,   Dlt = sum_i P_i dP_i,
 *   dS_i = P_i (dP_i - Dlt),   dq = scale sum_i dS_i kc_i,
 *   dkc_i += scale dS_i q.
 * The forward is recomputed from its definition in float64.
 */
int nsa_oracle_attention_backward_kv(const uint16_t* q, const uint16_t* kc, const uint16_t* vc,
                                     const uint16_t* dout, const int64_t* act_seq_qlen,
                                     const int64_t* act_seq_kvlen, const int64_t* act_cmp_seq_kvlen,
                                     int64_t B, int64_t N1, int64_t N2, int64_t D1, int64_t D2,
                                     double scale, int64_t l, int64_t d, int dtype, double* dq,
                                     double* dkc, double* dvc)
{
    if (N2 < 1 || N1 % N2 != 0 || d < 1 || l < 1 || B < 1 || dtype < 0 || dtype > 1)
        return -1;
    const int64_t G = N1 / N2;
    const int64_t T1 = act_seq_qlen[B - 1], T2 = act_cmp_seq_kvlen[B - 1];
    for (int64_t x = 0; x < T1 * N1 * D1; ++x)
        dq[x] = 0.0;
    for (int64_t x = 0; x < T2 * N2 * D1; ++x)
        dkc[x] = 0.0;
    for (int64_t x = 0; x < T2 * N2 * D2; ++x)
        dvc[x] = 0.0;
    int64_t n_cmp_max = 1;
    for (int64_t b = 0; b < B; ++b) {
        int64_t nc = act_cmp_seq_kvlen[b] - seq_start(act_cmp_seq_kvlen, b);
        if (nc > n_cmp_max) n_cmp_max = nc;
    }
    int err = 0;
    /* one (sequence, KV head) per iteration: its dkc / dvc rows and its
     * queries' dq rows are written by it alone */
#pragma omp parallel
    {
        double* P = (double*)malloc(sizeof(double) * (size_t)n_cmp_max);
        double* dP = (double*)malloc(sizeof(double) * (size_t)n_cmp_max);
        if (!P || !dP) {
#pragma omp atomic write
            err = -4;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bg = 0; bg < B * N2; ++bg) {
                const int64_t b = bg / N2, g = bg % N2;
                const int64_t q0 = seq_start(act_seq_qlen, b), T = act_seq_qlen[b] - q0;
                const int64_t c0 = seq_start(act_cmp_seq_kvlen, b);
                const int64_t nc = act_cmp_seq_kvlen[b] - c0;
                /* chunked prefill: query t sits at position Tkv - T + t */
                const int64_t Tkv = act_seq_kvlen ? act_seq_kvlen[b] - seq_start(act_seq_kvlen, b) : T;
                for (int64_t t = 0; t < T; ++t) {
                    const int64_t pos = Tkv - T + t;
                    int64_t nv = 0;
                    while (nv < nc && nv * d + l - 1 <= pos)
                        ++nv;
                    if (nv == 0)
                        continue;
                    for (int64_t hh = 0; hh < G; ++hh) {
                        const int64_t h = g * G + hh;
                        const uint16_t* qh = q + ((q0 + t) * N1 + h) * D1;
                        const uint16_t* doh = dout + ((q0 + t) * N1 + h) * D2;
                        double m = -INFINITY;
                        for (int64_t i = 0; i < nv; ++i) {
                            const uint16_t* ki = kc + ((c0 + i) * N2 + g) * D1;
                            double dot = 0.0;
                            for (int64_t e = 0; e < D1; ++e)
                                dot += widen(dtype, qh[e]) * widen(dtype, ki[e]);
                            P[i] = scale * dot;
                            if (P[i] > m)
                                m = P[i];
                        }
                        double L = 0.0;
                        for (int64_t i = 0; i < nv; ++i) {
                            P[i] = exp(P[i] - m);
                            L += P[i];
                        }
                        double Dlt = 0.0;
                        for (int64_t i = 0; i < nv; ++i) {
                            P[i] /= L;
                            const uint16_t* vi = vc + ((c0 + i) * N2 + g) * D2;
                            double acc = 0.0;
                            for (int64_t e = 0; e < D2; ++e)
                                acc += widen(dtype, doh[e]) * widen(dtype, vi[e]);
                            dP[i] = acc;
                            Dlt += P[i] * acc;
                        }
                        double* dqh = dq + ((q0 + t) * N1 + h) * D1;
                        for (int64_t i = 0; i < nv; ++i) {
                            const double dS = P[i] * (dP[i] - Dlt);
                            const uint16_t* ki = kc + ((c0 + i) * N2 + g) * D1;
                            double* dki = dkc + ((c0 + i) * N2 + g) * D1;
                            double* dvi = dvc + ((c0 + i) * N2 + g) * D2;
                            for (int64_t e = 0; e < D1; ++e) {
                                dqh[e] += scale * dS * widen(dtype, ki[e]);
                                dki[e] += scale * dS * widen(dtype, qh[e]);
                            }
                            for (int64_t e = 0; e < D2; ++e)
                                dvi[e] += P[i] * widen(dtype, doh[e]);
                        }
                    }
                }
            }
        }
        free(P);
        free(dP);
    }
    return err;
}

int nsa_oracle_attention_backward(const uint16_t* q, const uint16_t* kc, const uint16_t* vc,
                                  const uint16_t* dout, const int64_t* act_seq_qlen,
                                  const int64_t* act_cmp_seq_kvlen, int64_t B, int64_t N1,
                                  int64_t N2, int64_t D1, int64_t D2, double scale, int64_t l,
                                  int64_t d, int dtype, double* dq, double* dkc, double* dvc)
{
    return nsa_oracle_attention_backward_kv(q, kc, vc, dout, act_seq_qlen, NULL, act_cmp_seq_kvlen, B, N1, N2, D1,
                                            D2, scale, l, d, dtype, dq, dkc, dvc);
}

/* Backward of the compression: y[i, n, :] = sum_p w[p, n] x[start + i*d + p, n, :]
 * gives dx[start + i*d + p, n, :] += w[p, n] dy[i, n, :] and
 * dw[p, n] = sum over sequences, windows i and dims e of
 * dy[i, n, e] * x[start + i*d + p, n, e].  Rows in no window get 0. */
int nsa_oracle_compress_backward(const uint16_t* x, const uint16_t* w, const double* dy,
                                 const int64_t* act_seq_len, int64_t B, int64_t N, int64_t D,
                                 int64_t l, int64_t d, int dtype, double* dx, double* dw)
{
    if (B < 1 || N < 1 || D < 1 || l < 1 || d < 1 || dtype < 0 || dtype > 1)
        return -1;
    const int64_t T = act_seq_len[B - 1];
    for (int64_t k = 0; k < T * N * D; ++k)
        dx[k] = 0.0;
    for (int64_t k = 0; k < l * N; ++k)
        dw[k] = 0.0;
    int64_t out_row = 0;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t start = seq_start(act_seq_len, b);
        const int64_t n = nsa_oracle_n_cmp(act_seq_len[b] - start, l, d);
        for (int64_t i = 0; i < n; ++i) {
            for (int64_t h = 0; h < N; ++h) {
                const double* dyi = dy + ((out_row + i) * N + h) * D;
                for (int64_t p = 0; p < l; ++p) {
                    const int64_t row = start + i * d + p;
                    const double wp = widen(dtype, w[p * N + h]);
                    double acc = 0.0;
                    for (int64_t e = 0; e < D; ++e) {
                        dx[(row * N + h) * D + e] += wp * dyi[e];
                        acc += dyi[e] * widen(dtype, x[(row * N + h) * D + e]);
                    }
                    dw[p * N + h] += acc;
                }
            }
        }
        out_row += n;
    }
    return 0;
}
