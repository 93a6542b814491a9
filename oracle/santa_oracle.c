/*
 * santa_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU implementation of what the decode-step stochastic
 * sparse attention path computes.  It exists to check the GPU library and to
 * serve as the timed CPU baseline; nothing in the product path may link, load
 * or call it.  It shares no code, header, table or helper with the GPU
 * library: every conversion and every step below is written out here again.
 *
 * Source of the method: the web page "Stochastic Sparse Attention for
 * Memory-Bound Inference" (ICML 2026 paper notes on SANTA).  Sections cited:
 *   [one-line summary]   the estimator and the 1.5x claim
 *   [framework]          the overall framework and its flowchart
 *   [key design 1]       AV as an expectation; Eq. (4) estimator; S2ANTA-strat
 *                        and S2ANTA-sys (one offset U ~ Unif[0,1/S),
 *                        thresholds U + m/S, indices by inverting the CDF)
 *   [key design 2]       S2ANTA-prop: tile partition functions, a global
 *                        reducer, per-tile budgets proportional to tile mass
 *   [key design 3]       S2ANTA-flash: S/(number of tiles) local samples per
 *                        tile, rescaled by the true tile mass at merge time
 *   [key design 4]       Bernoulli qK^T: the query scaled into [-1, 1], its
 *                        magnitudes taken as Bernoulli probabilities, ternary
 *                        queries, an unbiased score estimate, sparse feature
 *                        reads of K; [ablations] the mean group query for GQA
 *
 * Readings taken where the page is silent (each is listed in the design
 * notes as well):
 *   R1  samples are drawn with multiplicity (systematic thresholds can hit the
 *       same token more than once; each hit counts);
 *   R2  m runs over 0..S-1, so every threshold lies in [0,1);
 *   R3  J = min{ j : F(j) > t }  (left-closed CDF cells [F(j-1), F(j)));
 *       if rounding leaves no such j, J is the last token with nonzero mass;
 *   R4  prop's per-tile budget is the number of global thresholds that fall
 *       in the tile's CDF interval, so prop equals untiled systematic
 *       sampling;
 *   R5  the tile length T is given in tokens; n_t = ceil(n_k / T);
 *   R6  flash uses one offset per head, scaled to the per-tile budget:
 *       u_f = U * n_t in [0, 1/S_f), S_f = S / n_t;
 *   R10 GQA maps q head h to KV head h / (Hq / Hkv);
 *   R11 a request with zero keys is empty: output 0, indices -1, budgets 0;
 *   R15 Bernoulli qK^T: "B" is the number of independent ternary draws that
 *       are averaged; the scale into [-1, 1] is a = max_i |q_i|; draw r takes
 *       z_i = sign(q_i) when fl32(u_{r,i} * a) < |q_i|, else 0 (the decision
 *       is taken in fp32, as the GPU takes it);
 *   R16 the mean group query is the fp32 mean of the group's G queries, summed
 *       in head order and multiplied by 1/G; all G heads then share its
 *       ternary draws and therefore its scores.
 *
 * All arithmetic is IEEE double.  Inputs (bf16 or fp32) are widened exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* problem description (the oracle's own; not the GPU library's struct) */
/* ------------------------------------------------------------------ */
typedef struct {
    int batch, num_q_heads, num_kv_heads, head_dim;
    int max_seq_len;          /* contiguous: KV rows per (b, kv head)       */
    const int *seq_lens;      /* host [batch] or NULL (all = max_seq_len)   */
    int q_fmt, kv_fmt;        /* storage: 0 fp32, 1 bf16 bit patterns        */
                              /* (uint16), 2 OCP e4m3 bytes (uint8)          */
    int page_size;            /* 0: contiguous [B,Hkv,max_seq_len,d]        */
    const int *page_table;    /* host [batch, max_pages] (paged only)       */
    int max_pages;
    float scale;              /* softmax scale exactly as the GPU gets it   */
    int tile_len;             /* T, tokens per tile                         */
} oracle_problem;

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static double widen_bf16(uint16_t bits)
{
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* OCP e4m3 (the 8-bit float of the OCP FP8 formats): sign, a 4-bit
   exponent with bias 7, a 3-bit mantissa; exponent field 0 holds the
   subnormals m/8 * 2^-6, and S.1111.111 is NaN (there are no infinities). */
static double widen_e4m3(uint8_t bits)
{
    int sign = bits >> 7, e = (bits >> 3) & 15, m = bits & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

static double load_val(const void *base, size_t i, int fmt)
{
    if (fmt == 1)
        return widen_bf16(((const uint16_t *)base)[i]);
    if (fmt == 2)
        return widen_e4m3(((const uint8_t *)base)[i]);
    return (double)((const float *)base)[i];
}

static int seq_len_of(const oracle_problem *p, int b)
{
    return p->seq_lens ? p->seq_lens[b] : p->max_seq_len;
}

/* Element offset of row (b, kv head g, token j) in K or V. */
static size_t kv_row_offset(const oracle_problem *p, int b, int g, int j)
{
    size_t d = (size_t)p->head_dim;
    if (p->page_size == 0)
        return (((size_t)b * p->num_kv_heads + g) * p->max_seq_len + j) * d;
    int page = p->page_table[(size_t)b * p->max_pages + j / p->page_size];
    return (((size_t)page * p->num_kv_heads + g) * p->page_size + j % p->page_size) * d;
}

static int kv_head_of(const oracle_problem *p, int h)
{
    return h / (p->num_q_heads / p->num_kv_heads);   /* R10 */
}

/* ------------------------------------------------------------------ */
/* O1 -- scores.  x_j = scale * <q_h, K_j>   [framework: score stage]   */
/* ------------------------------------------------------------------ */
void oracle_logits(const oracle_problem *p, const void *q, const void *k,
                   int b, int h, double *x)
{
    int d = p->head_dim, g = kv_head_of(p, h), n = seq_len_of(p, b);
    size_t qoff = ((size_t)b * p->num_q_heads + h) * d;
    for (int j = 0; j < n; ++j) {
        size_t koff = kv_row_offset(p, b, g, j);
        double dot = 0.0;
        for (int i = 0; i < d; ++i)
            dot += load_val(q, qoff + i, p->q_fmt) * load_val(k, koff + i, p->kv_fmt);
        x[j] = (double)p->scale * dot;
    }
}

static int lengths_ok(const oracle_problem *p);

/* ------------------------------------------------------------------ */
/* O13 -- Bernoulli qK^T [key design 4].  a = max_i |q_i| scales the    */
/* query into [-1, 1]; |q_i| / a is the probability that a ternary draw */
/* keeps feature i, with the sign of q_i (R15).  Summing `draws` draws  */
/* gives integer coefficients c_i in [-draws, draws]; the score         */
/* estimate is (a / draws) * sum_i c_i K_{j,i}, unbiased since          */
/* E[c_i] = draws * q_i / a.  Only features with c_i != 0 are read.     */
/*   qf [d] the query in fp32; u [draws, d] uniforms in [0,1).           */
/* Writes c[d] and *a_out; returns the number of features with c != 0,  */
/* or -1 if a uniform lies outside [0,1).                               */
/* ------------------------------------------------------------------ */
int oracle_bernoulli_coefs(const float *qf, int d, const float *u, int draws, int *c, float *a_out)
{
    float a = 0.0f;
    for (int i = 0; i < d; ++i) {
        float m = fabsf(qf[i]);
        if (m > a) a = m;
    }
    int nz = 0, bad = 0;
    for (int i = 0; i < d; ++i) {
        float mag = fabsf(qf[i]);
        int sgn = qf[i] > 0.0f ? 1 : (qf[i] < 0.0f ? -1 : 0);
        int kept = 0;
        for (int r = 0; r < draws; ++r) {
            float ur = u[(size_t)r * d + i];
            if (!(ur >= 0.0f && ur < 1.0f)) bad = 1;
            float prod = ur * a;                 /* one fp32 rounding */
            if (prod < mag) kept += 1;
        }
        c[i] = sgn * kept;
        if (c[i] != 0) nz += 1;
    }
    *a_out = a;
    return bad ? -1 : nz;
}

/* The query that head h's Bernoulli draws are taken from (fp32): its own
   (exact widening), or with the mean group query (R16) the fp32 mean of the
   group's G queries, summed in head order. */
static void bernoulli_query(const oracle_problem *p, const void *q, int group_mean, int b, int h,
                            float *qf)
{
    int d = p->head_dim, G = p->num_q_heads / p->num_kv_heads;
    if (!group_mean) {
        size_t off = ((size_t)b * p->num_q_heads + h) * d;
        for (int i = 0; i < d; ++i) qf[i] = (float)load_val(q, off + i, p->q_fmt);
        return;
    }
    int h0 = kv_head_of(p, h) * G;
    for (int i = 0; i < d; ++i) {
        float s = (float)load_val(q, ((size_t)b * p->num_q_heads + h0) * d + i, p->q_fmt);
        for (int hh = 1; hh < G; ++hh)
            s = s + (float)load_val(q, ((size_t)b * p->num_q_heads + h0 + hh) * d + i, p->q_fmt);
        qf[i] = s * (1.0f / (float)G);
    }
}

/* Uniforms of head h: [B, Hq, draws, d] per head, or [B, Hkv, draws, d]
   with the mean group query (one set per group). */
static const float *bernoulli_uniforms(const oracle_problem *p, const float *ub, int draws,
                                       int group_mean, int b, int h)
{
    int d = p->head_dim;
    size_t owner = group_mean ? (size_t)b * p->num_kv_heads + kv_head_of(p, h)
                              : (size_t)b * p->num_q_heads + h;
    return ub + owner * (size_t)draws * d;
}

/* Estimated scores of head h of request b:
     x_j = scale * (a / draws) * sum_i c_i K_{j,i}     (fp64 sum)
   Returns the number of features head h reads, or -1 on a bad uniform. */
int oracle_bernoulli_logits(const oracle_problem *p, const void *q, const void *k, int draws,
                            int group_mean, const float *ub, int b, int h, double *x)
{
    int d = p->head_dim, g = kv_head_of(p, h), n = seq_len_of(p, b);
    float *qf = (float *)malloc(sizeof(float) * (size_t)d);
    int *c = (int *)malloc(sizeof(int) * (size_t)d);
    float a = 0.0f;
    bernoulli_query(p, q, group_mean, b, h, qf);
    int nz = oracle_bernoulli_coefs(qf, d, bernoulli_uniforms(p, ub, draws, group_mean, b, h),
                                    draws, c, &a);
    double coef = (double)p->scale * ((double)a / (double)draws);
    for (int j = 0; j < n; ++j) {
        size_t koff = kv_row_offset(p, b, g, j);
        double dot = 0.0;
        for (int i = 0; i < d; ++i)
            if (c[i] != 0) dot += (double)c[i] * load_val(k, koff + i, p->kv_fmt);
        x[j] = coef * dot;
    }
    free(qf);
    free(c);
    return nz;
}

/* Features of K that KV group (b, g) reads: the union over the group's
   heads of { i : c_i != 0 } (one query with the mean group query).
   nread [B*Hkv].  Returns 0, or -1 on bad arguments or uniforms. */
int oracle_bernoulli_features(const oracle_problem *p, const void *q, int draws, int group_mean,
                              const float *ub, int *nread)
{
    if (draws < 1 || !lengths_ok(p)) return -1;
    int d = p->head_dim, G = p->num_q_heads / p->num_kv_heads, status = 0;
    float *qf = (float *)malloc(sizeof(float) * (size_t)d);
    int *c = (int *)malloc(sizeof(int) * (size_t)d);
    char *any = (char *)malloc((size_t)d);
    for (int b = 0; b < p->batch; ++b)
        for (int g = 0; g < p->num_kv_heads; ++g) {
            memset(any, 0, (size_t)d);
            for (int hl = 0; hl < (group_mean ? 1 : G); ++hl) {
                int h = g * G + hl;
                float a;
                bernoulli_query(p, q, group_mean, b, h, qf);
                if (oracle_bernoulli_coefs(qf, d, bernoulli_uniforms(p, ub, draws, group_mean, b, h),
                                           draws, c, &a) < 0)
                    status = -3;
                for (int i = 0; i < d; ++i)
                    if (c[i] != 0) any[i] = 1;
            }
            int cnt = 0;
            for (int i = 0; i < d; ++i) cnt += any[i];
            nread[(size_t)b * p->num_kv_heads + g] = cnt;
        }
    free(qf);
    free(c);
    free(any);
    return status;
}

/* ------------------------------------------------------------------ */
/* O2 -- softmax weights.  e_j = exp(x_j - max x), returns Z = sum e.  */
/* A_j = e_j / Z is the categorical distribution of [key design 1].    */
/* ------------------------------------------------------------------ */
double oracle_softmax_weights(const double *x, int n, double *e, double *max_out)
{
    double m = -INFINITY;
    for (int j = 0; j < n; ++j)
        if (x[j] > m) m = x[j];
    double z = 0.0;
    for (int j = 0; j < n; ++j) {
        e[j] = exp(x[j] - m);
        z += e[j];
    }
    if (max_out) *max_out = m;
    return z;
}

/* ------------------------------------------------------------------ */
/* O3 + O5 + O7 -- invert the CDF of weights w at sorted thresholds t.  */
/*   F(j) = (w_0 + ... + w_j) / sum(w),  F(n-1) := 1                    */
/*   J_m  = min{ j : F(j) > t_m }       (R3)                            */
/*   delta_m = distance from t_m to the nearer edge of J_m's cell       */
/* [key design 1]: J_m = F^{-1}(T_m).                                    */
/* Returns 0, or -1 if the thresholds are not sorted or out of [0,1).   */
/* ------------------------------------------------------------------ */
int oracle_invert_cdf(const double *w, int n, const double *t, int count,
                      int *idx, double *delta)
{
    double *F = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!F) return -2;
    double z = 0.0;
    for (int j = 0; j < n; ++j) z += w[j];
    double run = 0.0;
    int last_nonzero = -1;
    for (int j = 0; j < n; ++j) {
        run += w[j];
        F[j] = run / z;
        if (w[j] > 0.0) last_nonzero = j;
    }
    if (n > 0) F[n - 1] = 1.0;

    int j = 0;
    for (int m = 0; m < count; ++m) {
        if (t[m] < 0.0 || t[m] >= 1.0 || (m > 0 && t[m] < t[m - 1])) {
            free(F);
            return -1;
        }
        while (j < n && !(F[j] > t[m])) ++j;
        int J = (j < n) ? j : last_nonzero;
        /* only the last cell, whose edge is forced to 1, can be reached by
           a token of zero mass; R3 sends it to the last token with mass */
        if (J >= 0 && !(w[J] > 0.0)) J = last_nonzero;
        idx[m] = J;
        if (delta) {
            double lo = (J > 0) ? F[J - 1] : 0.0;
            double a = t[m] - lo, c = F[J] - t[m];
            delta[m] = a < c ? a : c;
        }
    }
    free(F);
    return 0;
}

/* ------------------------------------------------------------------ */
/* O3 -- the CDF cell of a given token: [F(j-1), F(j)) with F(-1) = 0,  */
/* F(j) = (w_0 + ... + w_j) / sum(w) and F(n-1) := 1, the cells that    */
/* oracle_invert_cdf inverts [key design 1: J_m = F^{-1}(T_m)].  A       */
/* threshold selects token j exactly when it lies in j's cell; where     */
/* several tokens are correct (a threshold within rounding of an edge),  */
/* they are the tokens whose cells lie that close to it.  Tokens outside */
/* [0, n) get NaN edges.                                                 */
/* ------------------------------------------------------------------ */
int oracle_cell_edges(const double *w, int n, const int *tok, int count, double *lo, double *hi)
{
    double *F = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!F) return -2;
    double z = 0.0;
    for (int j = 0; j < n; ++j) z += w[j];
    double run = 0.0;
    for (int j = 0; j < n; ++j) {
        run += w[j];
        F[j] = run / z;
    }
    if (n > 0) F[n - 1] = 1.0;
    for (int m = 0; m < count; ++m) {
        int j = tok[m];
        if (j < 0 || j >= n) {
            lo[m] = NAN;
            hi[m] = NAN;
            continue;
        }
        lo[m] = (j > 0) ? F[j - 1] : 0.0;
        hi[m] = F[j];
    }
    free(F);
    return 0;
}

/* O4 -- systematic thresholds t_m = U + m/S, m = 0..S-1 (R2) [key design 1] */
void oracle_sys_thresholds(double U, int S, double *t)
{
    for (int m = 0; m < S; ++m) t[m] = U + (double)m / (double)S;
}

/* O12 -- stratified thresholds t_m = (m + u_m)/S, one uniform per stratum  */
/* [key design 1: S2ANTA-strat draws an independent offset in each of the   */
/* S equal-mass strata].                                                    */
void oracle_strat_thresholds(const double *u01, int S, double *t)
{
    for (int m = 0; m < S; ++m) t[m] = ((double)m + u01[m]) / (double)S;
}

/* O12 -- i.i.d. thresholds: S independent uniforms on [0,1), sorted so the  */
/* CDF can be inverted in one sweep [key design 1: Eq. (4), i_s ~ A iid].     */
static int cmp_double(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x > y) - (x < y);
}
void oracle_iid_thresholds(const double *u01, int S, double *t)
{
    memcpy(t, u01, sizeof(double) * (size_t)S);
    qsort(t, (size_t)S, sizeof(double), cmp_double);
}

/* O6 -- (1/S) * sum_m V[J_m], fp64.  Repeated indices count each time (R1). */
static void mean_of_rows(const oracle_problem *p, const void *v, int b, int g,
                         const int *idx, int count, double *out)
{
    int d = p->head_dim;
    for (int i = 0; i < d; ++i) out[i] = 0.0;
    for (int m = 0; m < count; ++m) {
        size_t off = kv_row_offset(p, b, g, idx[m]);
        for (int i = 0; i < d; ++i) out[i] += load_val(v, off + i, p->kv_fmt);
    }
    for (int i = 0; i < d; ++i) out[i] /= (double)count;
}

/* Reading R11 (empty requests): a request with no keys has no distribution
   to sample from; its output rows are 0, it selects no token (index -1) and
   every tile budget is 0.  Lengths must lie in [0, max_seq_len]. */
static int lengths_ok(const oracle_problem *p)
{
    if (p->batch <= 0 || p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->head_dim <= 0 ||
        p->tile_len <= 0 || p->num_q_heads % p->num_kv_heads)
        return 0;
    for (int b = 0; b < p->batch; ++b) {
        int n = seq_len_of(p, b);
        if (n < 0 || n > p->max_seq_len) return 0;
    }
    return 1;
}

static int num_tiles(const oracle_problem *p, int n)
{
    return (n + p->tile_len - 1) / p->tile_len;   /* R5 */
}

static int max_tiles(const oracle_problem *p)
{
    int best = 0;
    for (int b = 0; b < p->batch; ++b) {
        int nt = num_tiles(p, seq_len_of(p, b));
        if (nt > best) best = nt;
    }
    return best;
}

/* ------------------------------------------------------------------ */
/* S2ANTA-prop with a choice of threshold generator (O1-O8, O12).       */
/* By R4 prop equals untiled sampling at the same thresholds: tiles     */
/* change how the thresholds are located, not which tokens they select  */
/* [key design 2].  The generator is that of key design 1:              */
/*   kind 0  S2ANTA-sys:   u [B*Hq], one offset per head in [0, 1/S);   */
/*                         t_m = U + m/S                                */
/*   kind 1  S2ANTA-strat: u [B*Hq*S], one uniform in [0,1) per stratum; */
/*                         t_m = (m + u_m)/S                            */
/*   kind 2  i.i.d.:       u [B*Hq*S], uniforms in [0,1); t = sorted u  */
/* (thresholds formed in fp64 from the fp32 inputs).                    */
/*   out      [B*Hq*d] estimate (1/S) sum V[J_m]                        */
/*   idx      [B*Hq*S] selected token per threshold (NULL allowed)     */
/*   delta    [B*Hq*S] boundary distance per threshold (NULL allowed)  */
/*   tile_cnt [B*Hq*max_nt] thresholds per tile, S_t (NULL allowed)    */
/* Returns 0, or a negative code on bad arguments.                      */
/* ------------------------------------------------------------------ */
typedef struct {
    int draws, group_mean;
    const float *ub;
} bernoulli_args;

/* Optional cell query (all four NULL, or all given): for every head and
   threshold position m, cell_thr gets the threshold t_m and [cell_lo,
   cell_hi) the CDF cell of the token cell_tok names at m (any token, e.g.
   one chosen by another implementation), by oracle_cell_edges. */
typedef struct {
    const int *tok;
    double *thr, *lo, *hi;
} cell_query;

static int prop_core(const oracle_problem *p, const void *q, const void *k, const void *v,
                     int S, int kind, const float *u, const bernoulli_args *bern, double *out,
                     int *idx, double *delta, int *tile_cnt, const cell_query *cq)
{
    if (S <= 0 || kind < 0 || kind > 2 || !lengths_ok(p)) return -1;
    if (bern && bern->draws < 1) return -1;
    int H = p->num_q_heads, d = p->head_dim, mnt = max_tiles(p);
    int status = 0;
    int nheads = p->batch * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < nheads; ++bh) {
        int b = bh / H, h = bh % H, g = kv_head_of(p, h), n = seq_len_of(p, b);
        if (n == 0) {                                   /* R11 */
            for (int i = 0; i < d; ++i) out[(size_t)bh * d + i] = 0.0;
            for (int m = 0; m < S; ++m) {
                if (idx) idx[(size_t)bh * S + m] = -1;
                if (delta) delta[(size_t)bh * S + m] = INFINITY;
            }
            if (tile_cnt)
                for (int i = 0; i < mnt; ++i) tile_cnt[(size_t)bh * mnt + i] = 0;
            if (cq)
                for (int m = 0; m < S; ++m) {
                    size_t o = (size_t)bh * S + m;
                    cq->thr[o] = NAN;
                    cq->lo[o] = NAN;
                    cq->hi[o] = NAN;
                }
            continue;
        }
        double *x = (double *)malloc(sizeof(double) * (size_t)n);
        double *e = (double *)malloc(sizeof(double) * (size_t)n);
        double *t = (double *)malloc(sizeof(double) * (size_t)S);
        double *u01 = (double *)malloc(sizeof(double) * (size_t)S);
        int *J = (int *)malloc(sizeof(int) * (size_t)S);
        double *dl = (double *)malloc(sizeof(double) * (size_t)S);
        if (bern) {
            if (oracle_bernoulli_logits(p, q, k, bern->draws, bern->group_mean, bern->ub, b, h, x) < 0) {
#pragma omp atomic write
                status = -3;
            }
        } else {
            oracle_logits(p, q, k, b, h, x);
        }
        oracle_softmax_weights(x, n, e, NULL);
        if (kind == 0) {
            double U = (double)u[bh];
            if (!(U >= 0.0 && U < 1.0 / (double)S)) {
#pragma omp atomic write
                status = -3;
            }
            oracle_sys_thresholds(U, S, t);
        } else {
            for (int m = 0; m < S; ++m) {
                u01[m] = (double)u[(size_t)bh * S + m];
                if (!(u01[m] >= 0.0 && u01[m] < 1.0)) {
#pragma omp atomic write
                    status = -3;
                    u01[m] = 0.0;
                }
            }
            if (kind == 1)
                oracle_strat_thresholds(u01, S, t);
            else
                oracle_iid_thresholds(u01, S, t);
        }
        if (oracle_invert_cdf(e, n, t, S, J, dl) != 0) {
            /* rejected thresholds: the call fails; no row is read */
#pragma omp atomic write
            status = -4;
            for (int m = 0; m < S; ++m) {
                J[m] = 0;
                dl[m] = NAN;
            }
        }
        mean_of_rows(p, v, b, g, J, S, out + (size_t)bh * d);
        if (idx) memcpy(idx + (size_t)bh * S, J, sizeof(int) * (size_t)S);
        if (delta) memcpy(delta + (size_t)bh * S, dl, sizeof(double) * (size_t)S);
        if (tile_cnt) {
            int *tc = tile_cnt + (size_t)bh * mnt;
            for (int i = 0; i < mnt; ++i) tc[i] = 0;
            for (int m = 0; m < S; ++m) tc[J[m] / p->tile_len] += 1;
        }
        if (cq) {
            size_t o = (size_t)bh * S;
            memcpy(cq->thr + o, t, sizeof(double) * (size_t)S);
            oracle_cell_edges(e, n, cq->tok + o, S, cq->lo + o, cq->hi + o);
        }
        free(x); free(e); free(t); free(u01); free(J); free(dl);
    }
    return status;
}

int oracle_santa_prop_sampler(const oracle_problem *p, const void *q, const void *k,
                              const void *v, int S, int kind, const float *u, double *out,
                              int *idx, double *delta, int *tile_cnt)
{
    return prop_core(p, q, k, v, S, kind, u, NULL, out, idx, delta, tile_cnt, NULL);
}

/* S2ANTA-sys prop: the systematic generator of the function above. */
int oracle_santa_prop(const oracle_problem *p, const void *q, const void *k,
                      const void *v, int S, const float *u, double *out,
                      int *idx, double *delta, int *tile_cnt)
{
    return prop_core(p, q, k, v, S, 0, u, NULL, out, idx, delta, tile_cnt, NULL);
}

/* S2ANTA-prop (systematic thresholds) on Bernoulli qK^T scores (O13 in
   place of O1; key design 4 composed with key design 2).  ub as for
   oracle_bernoulli_logits; other arguments as for oracle_santa_prop. */
int oracle_santa_prop_bernoulli(const oracle_problem *p, const void *q, const void *k,
                                const void *v, int S, const float *u, int draws, int group_mean,
                                const float *ub, double *out, int *idx, double *delta,
                                int *tile_cnt)
{
    bernoulli_args ba = {draws, group_mean, ub};
    return prop_core(p, q, k, v, S, 0, u, &ba, out, idx, delta, tile_cnt, NULL);
}

/* Cells of given tokens in prop's (untiled) CDF, with the thresholds of
   the chosen generator; on Bernoulli scores when draws > 0 (then kind must
   be 0).  tok [B*Hq*S]; thr, lo, hi [B*Hq*S] (NaN for empty requests).
   Arguments otherwise as for oracle_santa_prop_sampler and
   oracle_santa_prop_bernoulli. */
int oracle_prop_cells(const oracle_problem *p, const void *q, const void *k, int S, int kind,
                      const float *u, int draws, int group_mean, const float *ub, const int *tok,
                      double *thr, double *lo, double *hi)
{
    if (S <= 0 || !lengths_ok(p) || (draws > 0 && kind != 0)) return -1;
    double *out = (double *)malloc(sizeof(double) * (size_t)p->batch * p->num_q_heads * p->head_dim);
    if (!out) return -2;
    /* the estimate itself is not needed: V is replaced by K, which has the
       same layout, so no V argument is required */
    bernoulli_args ba = {draws, group_mean, ub};
    cell_query cq = {tok, thr, lo, hi};
    int rc = prop_core(p, q, k, k, S, kind, u, draws > 0 ? &ba : NULL, out, NULL, NULL, NULL, &cq);
    free(out);
    return rc;
}

/* ------------------------------------------------------------------ */
/* S2ANTA-flash (O9) [key design 3].  Every tile behaves as if it held  */
/* all the mass: it samples S_f = S/n_t tokens from its own softmax     */
/* with thresholds u_f + m/S_f (R6), averages them into o_t, and the    */
/* merge weighs o_t by the tile's true share p_t = Z_t e^{m_t-M} / Z.   */
/*   idx   [B*Hq*S] tile-major: tile t's samples at t*S_f..t*S_f+S_f-1  */
/*   ptile [B*Hq*n_t] p_t (NULL allowed), for replay                    */
/* Requires uniform sequence length and S % n_t == 0.                   */
/* ------------------------------------------------------------------ */
/* The generators of key design 1, applied to each tile's own softmax with
   its S_f = S/n_t samples:
     kind 0  systematic: u [B*Hq], one offset U per head in [0, 1/S);
             local thresholds u_f + m/S_f, u_f = U n_t (R6)
     kind 1  stratified: u [B*Hq*S] in [0,1), tile-major (tile t's uniforms
             at t*S_f .. t*S_f + S_f - 1); local thresholds (m + u_m)/S_f
     kind 2  i.i.d.: u as for kind 1; local thresholds = the tile's
             uniforms, sorted */
static int flash_core(const oracle_problem *p, const void *q, const void *k, const void *v,
                      int S, int kind, const float *u, double *out, int *idx, double *delta,
                      double *ptile, const cell_query *cq)
{
    if (p->seq_lens || !lengths_ok(p) || kind < 0 || kind > 2) return -1;
    int n = p->max_seq_len, nt = num_tiles(p, n);
    if (S <= 0 || S % nt) return -1;
    int Sf = S / nt, H = p->num_q_heads, d = p->head_dim, T = p->tile_len;
    int status = 0;
    int nheads = p->batch * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < nheads; ++bh) {
        int b = bh / H, h = bh % H, g = kv_head_of(p, h);
        double *x = (double *)malloc(sizeof(double) * (size_t)n);
        double *e = (double *)malloc(sizeof(double) * (size_t)T);
        double *mt = (double *)malloc(sizeof(double) * (size_t)nt);
        double *zt = (double *)malloc(sizeof(double) * (size_t)nt);
        double *ot = (double *)malloc(sizeof(double) * (size_t)nt * d);
        double *t = (double *)malloc(sizeof(double) * (size_t)Sf);
        double *u01 = (double *)malloc(sizeof(double) * (size_t)Sf);
        int *J = (int *)malloc(sizeof(int) * (size_t)Sf);
        double *dl = (double *)malloc(sizeof(double) * (size_t)Sf);
        oracle_logits(p, q, k, b, h, x);
        double uf = 0.0;
        if (kind == 0) {
            double U = (double)u[bh];
            if (!(U >= 0.0 && U < 1.0 / (double)S)) {
#pragma omp atomic write
                status = -3;
            }
            uf = U * (double)nt;
        }
        for (int tt = 0; tt < nt; ++tt) {
            int j0 = tt * T, len = (n - j0 < T) ? n - j0 : T;
            zt[tt] = oracle_softmax_weights(x + j0, len, e, &mt[tt]);
            if (kind == 0) {
                oracle_sys_thresholds(uf, Sf, t);
            } else {
                for (int m = 0; m < Sf; ++m) {
                    u01[m] = (double)u[(size_t)bh * S + (size_t)tt * Sf + m];
                    if (!(u01[m] >= 0.0 && u01[m] < 1.0)) {
#pragma omp atomic write
                        status = -3;
                        u01[m] = 0.0;
                    }
                }
                if (kind == 1)
                    oracle_strat_thresholds(u01, Sf, t);
                else
                    oracle_iid_thresholds(u01, Sf, t);
            }
            if (oracle_invert_cdf(e, len, t, Sf, J, dl) != 0) {
                /* rejected thresholds: the call fails; no row is read */
#pragma omp atomic write
                status = -4;
                for (int m = 0; m < Sf; ++m) {
                    J[m] = 0;
                    dl[m] = NAN;
                }
            }
            if (cq) {
                /* the tile's own CDF: the cell of the named token relative
                   to the tile (NaN if the token lies outside the tile) */
                size_t o = (size_t)bh * S + (size_t)tt * Sf;
                for (int m = 0; m < Sf; ++m) {
                    int jl = cq->tok[o + m] - j0;
                    cq->thr[o + m] = t[m];
                    oracle_cell_edges(e, len, &jl, 1, cq->lo + o + m, cq->hi + o + m);
                }
            }
            for (int m = 0; m < Sf; ++m) J[m] += j0;
            mean_of_rows(p, v, b, g, J, Sf, ot + (size_t)tt * d);
            if (idx) memcpy(idx + (size_t)bh * S + (size_t)tt * Sf, J, sizeof(int) * (size_t)Sf);
            if (delta) memcpy(delta + (size_t)bh * S + (size_t)tt * Sf, dl, sizeof(double) * (size_t)Sf);
        }
        double M = -INFINITY;
        for (int tt = 0; tt < nt; ++tt) if (mt[tt] > M) M = mt[tt];
        double Z = 0.0;
        for (int tt = 0; tt < nt; ++tt) Z += zt[tt] * exp(mt[tt] - M);
        double *o = out + (size_t)bh * d;
        for (int i = 0; i < d; ++i) o[i] = 0.0;
        for (int tt = 0; tt < nt; ++tt) {
            double pt = zt[tt] * exp(mt[tt] - M) / Z;
            if (ptile) ptile[(size_t)bh * nt + tt] = pt;
            for (int i = 0; i < d; ++i) o[i] += pt * ot[(size_t)tt * d + i];
        }
        free(x); free(e); free(mt); free(zt); free(ot); free(t); free(u01); free(J); free(dl);
    }
    return status;
}

int oracle_santa_flash_sampler(const oracle_problem *p, const void *q, const void *k,
                               const void *v, int S, int kind, const float *u, double *out,
                               int *idx, double *delta, double *ptile)
{
    return flash_core(p, q, k, v, S, kind, u, out, idx, delta, ptile, NULL);
}

/* S2ANTA-flash with systematic thresholds. */
int oracle_santa_flash(const oracle_problem *p, const void *q, const void *k,
                       const void *v, int S, const float *u, double *out,
                       int *idx, double *delta, double *ptile)
{
    return flash_core(p, q, k, v, S, 0, u, out, idx, delta, ptile, NULL);
}

/* Cells of given tokens in flash's tile-local CDFs: position m belongs to
   tile m / S_f (tile-major, as flash's indices), its threshold is the
   tile's local one and [lo, hi) is the named token's cell in that tile's
   own CDF (NaN if the token is not in the tile).  tok, thr, lo, hi
   [B*Hq*S]; other arguments as for oracle_santa_flash_sampler. */
int oracle_flash_cells(const oracle_problem *p, const void *q, const void *k, int S, int kind,
                       const float *u, const int *tok, double *thr, double *lo, double *hi)
{
    if (S <= 0 || !lengths_ok(p)) return -1;
    double *out = (double *)malloc(sizeof(double) * (size_t)p->batch * p->num_q_heads * p->head_dim);
    if (!out) return -2;
    cell_query cq = {tok, thr, lo, hi};
    /* K stands in for V (same layout); the estimate is not needed */
    int rc = flash_core(p, q, k, k, S, kind, u, out, NULL, NULL, NULL, &cq);
    free(out);
    return rc;
}

/* ------------------------------------------------------------------ */
/* O10 -- exact attention output AV = sum_j A_j V_j  [key design 1: the */
/* quantity the estimators are unbiased for].                           */
/* ------------------------------------------------------------------ */
int oracle_exact(const oracle_problem *p, const void *q, const void *k,
                 const void *v, double *out)
{
    if (!lengths_ok(p)) return -1;
    int H = p->num_q_heads, d = p->head_dim;
    int nheads = p->batch * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < nheads; ++bh) {
        int b = bh / H, h = bh % H, g = kv_head_of(p, h), n = seq_len_of(p, b);
        double *o = out + (size_t)bh * d;
        for (int i = 0; i < d; ++i) o[i] = 0.0;
        if (n == 0) continue;                           /* R11 */
        double *x = (double *)malloc(sizeof(double) * (size_t)n);
        double *e = (double *)malloc(sizeof(double) * (size_t)n);
        oracle_logits(p, q, k, b, h, x);
        double Z = oracle_softmax_weights(x, n, e, NULL);
        for (int j = 0; j < n; ++j) {
            double a = e[j] / Z;
            size_t off = kv_row_offset(p, b, g, j);
            for (int i = 0; i < d; ++i) o[i] += a * load_val(v, off + i, p->kv_fmt);
        }
        free(x); free(e);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* O11 -- replay: the estimate a given index set produces, in fp64.     */
/*   prop/sys: out = (1/S) sum_m V[idx_m]                               */
/*   flash (ptile != NULL): out = sum_t p_t (1/S_f) sum V[idx in tile t]*/
/* ------------------------------------------------------------------ */
int oracle_replay(const oracle_problem *p, const void *v, int S, const int *idx,
                  const double *ptile, int ntile, double *out)
{
    if (S <= 0 || !lengths_ok(p)) return -1;
    int H = p->num_q_heads, d = p->head_dim;
    int nheads = p->batch * H;
    if (ptile && (ntile <= 0 || S % ntile)) return -1;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < nheads; ++bh) {
        int b = bh / H, h = bh % H, g = kv_head_of(p, h), n = seq_len_of(p, b);
        const int *I = idx + (size_t)bh * S;
        int bad = 0;
        double *o = out + (size_t)bh * d;
        if (n == 0) {                                   /* R11 */
            for (int m = 0; m < S; ++m)
                if (I[m] != -1) bad = 1;
            for (int i = 0; i < d; ++i) o[i] = 0.0;
            if (bad) {
#pragma omp atomic write
                status = -2;
            }
            continue;
        }
        for (int m = 0; m < S; ++m)
            if (I[m] < 0 || I[m] >= n) bad = 1;
        if (bad) {
#pragma omp atomic write
            status = -2;
            continue;
        }
        if (!ptile) {
            mean_of_rows(p, v, b, g, I, S, o);
        } else {
            int Sf = S / ntile;
            double *ot = (double *)malloc(sizeof(double) * (size_t)d);
            for (int i = 0; i < d; ++i) o[i] = 0.0;
            for (int tt = 0; tt < ntile; ++tt) {
                mean_of_rows(p, v, b, g, I + (size_t)tt * Sf, Sf, ot);
                double pt = ptile[(size_t)bh * ntile + tt];
                for (int i = 0; i < d; ++i) o[i] += pt * ot[i];
            }
            free(ot);
        }
    }
    return status;
}

/* ------------------------------------------------------------------ */
/* Estimator on explicit weights: (1/count) sum_m V[J_m] for thresholds */
/* t (any of the three samplers).  V is [n, d] fp64.                    */
/* ------------------------------------------------------------------ */
int oracle_estimate_from_weights(const double *w, int n, const double *V, int d,
                                 const double *t, int count, double *out)
{
    int *J = (int *)malloc(sizeof(int) * (size_t)count);
    int rc = oracle_invert_cdf(w, n, t, count, J, NULL);
    if (rc == 0) {
        for (int i = 0; i < d; ++i) out[i] = 0.0;
        for (int m = 0; m < count; ++m)
            for (int i = 0; i < d; ++i) out[i] += V[(size_t)J[m] * d + i];
        for (int i = 0; i < d; ++i) out[i] /= (double)count;
    }
    free(J);
    return rc;
}

/* ------------------------------------------------------------------ */
/* E_U and the trace of Cov_U of the systematic estimator, exactly.     */
/* As U sweeps [0, 1/S) a threshold U + m/S crosses a cell edge F(j)    */
/* only where U = F(j) mod (1/S); between such points every J_m is      */
/* fixed.  Summing the (constant) estimate over those intervals, each   */
/* weighted by its probability length*S, gives the expectation exactly  */
/* (up to fp64 rounding of the breakpoints).                            */
/* ------------------------------------------------------------------ */
int oracle_sys_moments(const double *w, int n, const double *V, int d, int S,
                       double *mean, double *var_trace)
{
    double inv = 1.0 / (double)S;
    double *bp = (double *)malloc(sizeof(double) * (size_t)(n + 2));
    double z = 0.0, run = 0.0;
    for (int j = 0; j < n; ++j) z += w[j];
    int nb = 0;
    bp[nb++] = 0.0;
    bp[nb++] = inv;
    for (int j = 0; j < n - 1; ++j) {
        run += w[j];
        double F = run / z;
        double r = F - floor(F * (double)S) / (double)S;
        if (r < 0.0) r = 0.0;
        if (r < inv) bp[nb++] = r;
    }
    qsort(bp, (size_t)nb, sizeof(double), cmp_double);
    double *t = (double *)malloc(sizeof(double) * (size_t)S);
    double *est = (double *)malloc(sizeof(double) * (size_t)d);
    double second = 0.0;
    for (int i = 0; i < d; ++i) mean[i] = 0.0;
    int rc = 0;
    for (int k = 0; k + 1 < nb; ++k) {
        double a = bp[k], c = bp[k + 1];
        if (!(c > a)) continue;
        double Umid = 0.5 * (a + c);
        oracle_sys_thresholds(Umid, S, t);
        if (oracle_estimate_from_weights(w, n, V, d, t, S, est) != 0) { rc = -1; break; }
        double prob = (c - a) * (double)S;
        double sq = 0.0;
        for (int i = 0; i < d; ++i) {
            mean[i] += prob * est[i];
            sq += est[i] * est[i];
        }
        second += prob * sq;
    }
    if (var_trace) {
        double mm = 0.0;
        for (int i = 0; i < d; ++i) mm += mean[i] * mean[i];
        *var_trace = second - mm;
    }
    free(bp); free(t); free(est);
    return rc;
}

/* ------------------------------------------------------------------ */
/* E over u_f of the flash estimator on explicit weights, exactly.      */
/* Tiles of length T; every tile's local estimator is piecewise         */
/* constant in u_f in [0, 1/S_f) with breakpoints G_t(j) mod 1/S_f; the */
/* union of those breakpoints makes every tile constant at once.        */
/* ------------------------------------------------------------------ */
int oracle_flash_moments(const double *w, int n, const double *V, int d, int S,
                         int T, double *mean, double *var_trace)
{
    int nt = (n + T - 1) / T;
    if (S % nt) return -1;
    int Sf = S / nt;
    double inv = 1.0 / (double)Sf;
    double *bp = (double *)malloc(sizeof(double) * (size_t)(n + 2));
    int nb = 0;
    bp[nb++] = 0.0;
    bp[nb++] = inv;
    double Z = 0.0;
    for (int j = 0; j < n; ++j) Z += w[j];
    for (int tt = 0; tt < nt; ++tt) {
        int j0 = tt * T, len = (n - j0 < T) ? n - j0 : T;
        double zt = 0.0, run = 0.0;
        for (int j = 0; j < len; ++j) zt += w[j0 + j];
        if (!(zt > 0.0)) continue;
        for (int j = 0; j < len - 1; ++j) {
            run += w[j0 + j];
            double G = run / zt;
            double r = G - floor(G * (double)Sf) / (double)Sf;
            if (r < 0.0) r = 0.0;
            if (r < inv) bp[nb++] = r;
        }
    }
    qsort(bp, (size_t)nb, sizeof(double), cmp_double);
    double *t = (double *)malloc(sizeof(double) * (size_t)Sf);
    double *ot = (double *)malloc(sizeof(double) * (size_t)d);
    double *est = (double *)malloc(sizeof(double) * (size_t)d);
    double second = 0.0;
    for (int i = 0; i < d; ++i) mean[i] = 0.0;
    int rc = 0;
    for (int k = 0; k + 1 < nb && rc == 0; ++k) {
        double a = bp[k], c = bp[k + 1];
        if (!(c > a)) continue;
        double umid = 0.5 * (a + c);
        oracle_sys_thresholds(umid, Sf, t);
        for (int i = 0; i < d; ++i) est[i] = 0.0;
        for (int tt = 0; tt < nt; ++tt) {
            int j0 = tt * T, len = (n - j0 < T) ? n - j0 : T;
            double zt = 0.0;
            for (int j = 0; j < len; ++j) zt += w[j0 + j];
            if (!(zt > 0.0)) continue;
            if (oracle_estimate_from_weights(w + j0, len, V + (size_t)j0 * d, d, t, Sf, ot) != 0) { rc = -1; break; }
            for (int i = 0; i < d; ++i) est[i] += (zt / Z) * ot[i];
        }
        double prob = (c - a) * (double)Sf, sq = 0.0;
        for (int i = 0; i < d; ++i) {
            mean[i] += prob * est[i];
            sq += est[i] * est[i];
        }
        second += prob * sq;
    }
    if (var_trace) {
        double mm = 0.0;
        for (int i = 0; i < d; ++i) mm += mean[i] * mean[i];
        *var_trace = second - mm;
    }
    free(bp); free(t); free(ot); free(est);
    return rc;
}

/* Number of OpenMP threads the parallel loops above use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
