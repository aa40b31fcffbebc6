/*
 * Oracle for jagged GDPA / JFA — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 loop nests of what the jagged attention path computes.
 * Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this file's library; the product path never does.
 * It shares no code, header or constant with the GPU library.
 *
 * What is computed (the pages never write the formula out; the formula below
 * is the plain reading of their words):
 *   - "GEM Training: How Meta Doubled the Efficiency..." (globalainews.in),
 *     section "What to watch": the attention-like modules are two matrix
 *     products with an element-wise activation between them, GELU or SiLU
 *     taking the place of softmax (GDPA).
 *   - same page, section "What happened": JFA is FlashAttention run directly
 *     on variable-length jagged tensors, with custom attention biases,
 *     asymmetric query / key-value lengths and a backward pass.
 *
 * For sample b with Lq query rows and Lk key rows, head h, sample-local
 * indices i (query) and j (key):
 *   X[i][j]  = scale * <q_i, k_j> + bias(h, i, j)
 *   valid    = (j < Lk) and (not causal or j <= i + Lk - Lq)
 *              and, with a window w > 0 (sliding-window attention, named on
 *              "Meta redesigns AI training infrastructure...", section "Custom
 *              Kernels and 5D Parallelism..."; the pages give no definition):
 *              i' - j < w and (causal or j - i' < w), where i' = i + Lk - Lq
 *              is the query's aligned position
 *   GDPA:  O_i = sum_{valid j} act(X_ij) v_j                 (no normalisation)
 *   JFA:   O_i = sum_{valid j} softmax_j(X_i.) v_j,  LSE_i = log sum_j exp X_ij
 *          (a row with no valid key: O_i = 0, LSE_i = -inf)
 * Bias kinds: REL    table[h][clamp(i - j, lo, hi) - lo]
 *             KEYPOS table[h][clamp(j, lo, hi) - lo]
 *
 * Backward, with upstream gradient dO and L = <O, dO>:
 *   dP_ij = <dO_i, v_j>
 *   GDPA:  dX_ij = dP_ij act'(X_ij),   dV_j = sum_i act(X_ij) dO_i
 *   JFA:   dX_ij = P_ij (dP_ij - sum_k P_ik dP_ik),  dV_j = sum_i P_ij dO_i
 *   dQ_i = scale sum_j dX_ij k_j,   dK_j = scale sum_i dX_ij q_i
 *   bias table (the pages list custom attention biases among what the jagged
 *   kernels support, "GEM Training...", section "What happened"; the table
 *   enters X additively, so dL/dtable sums dX over the pairs that read each
 *   entry):  dTable[h][c] = sum over samples and valid pairs (i, j) whose
 *   index (REL: clamp(i - j, lo, hi) - lo; KEYPOS: clamp(j, lo, hi) - lo) is c
 *   of dX_ij
 *
 * Rotary position embedding (optional, rope_base > 0).  The pages name a
 * rotary embedding fused into their block-attention kernel ("Meta redesigns AI
 * training infrastructure...", section "Custom Kernels and 5D Parallelism for
 * Trillion-Parameter Scale") without defining it; this is the rotation of
 * RoFormer (Su et al.) in its split-half form.  A query or key row at
 * sample-local position t (query i, key j; row r of a shared query block) is
 * turned pair by pair before the scores are formed: element d < D/2 and
 * element d + D/2 rotate by the angle t * rope_base^(-2d/D),
 *   x'_d = x_d cos a - x_{d+D/2} sin a,   x'_{d+D/2} = x_d sin a + x_{d+D/2} cos a.
 * X uses the turned rows; V is not turned.  The gradients returned are with
 * respect to the rows as given, so dQ_i and dK_j are the gradients of the
 * turned rows turned back (the rotation's transpose is the turn by -a).
 * With bf16 operands (rope_bf16 = 1) the turned rows are themselves operands
 * of bf16 products, so they are bf16 values: each element of the exact turn
 * (computed in double) is rounded to the nearest bf16 value, ties to even -- a
 * quantisation step with a plain definition, taken here straight from the
 * double, with no intermediate precision.  The gradients then follow the
 * rounded rows (the rounding is held fixed).
 *
 * Inputs are float32 arrays (bf16 values are exactly representable in
 * float32); all arithmetic is double.  Layout is token-major [T, H, D] with
 * int32 offsets [B+1]; a NULL q_off means one block of lq_fixed query rows
 * shared by every sample ([lq_fixed, H, D]) whose forward output still has one
 * row block per sample ([B * lq_fixed, H, D]).  Outputs are double arrays;
 * every element is written.
 *
 * Pinned by the CPU test suite against padded dense attention with an explicit
 * mask, per-sample library attention, central finite differences of the
 * forward pass and hand-derived closed forms.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ACT_SILU = 0, ACT_GELU_TANH = 1, ACT_GELU_ERF = 2 };
enum { BIAS_NONE = 0, BIAS_REL = 1, BIAS_KEYPOS = 2 };

/* SiLU(x) = x * sigmoid(x); derivative sigma (1 + x (1 - sigma)). */
static double silu(double x) { return x / (1.0 + exp(-x)); }
static double silu_grad(double x) {
    double s = 1.0 / (1.0 + exp(-x));
    return s * (1.0 + x * (1.0 - s));
}

/* GELU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))). */
static const double GELU_C = 0.7978845608028654; /* sqrt(2/pi) */
static double gelu_tanh(double x) {
    double t = tanh(GELU_C * (x + 0.044715 * x * x * x));
    return 0.5 * x * (1.0 + t);
}
static double gelu_tanh_grad(double x) {
    double t = tanh(GELU_C * (x + 0.044715 * x * x * x));
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * GELU_C * (1.0 + 3.0 * 0.044715 * x * x);
}

/* GELU, exact form: x Phi(x), Phi the standard normal CDF; derivative Phi + x phi. */
static double gelu_erf(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }
static double gelu_erf_grad(double x) {
    double cdf = 0.5 * (1.0 + erf(x / sqrt(2.0)));
    double pdf = exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
    return cdf + x * pdf;
}

static double act_f(int act, double x) {
    switch (act) {
    case ACT_SILU: return silu(x);
    case ACT_GELU_TANH: return gelu_tanh(x);
    default: return gelu_erf(x);
    }
}
static double act_grad(int act, double x) {
    switch (act) {
    case ACT_SILU: return silu_grad(x);
    case ACT_GELU_TANH: return gelu_tanh_grad(x);
    default: return gelu_erf_grad(x);
    }
}

typedef struct {
    const float *q, *k, *v;
    const int32_t *q_off, *kv_off;
    int32_t lq_fixed;
    int B, H, D;
    double scale;
    int act;
    int causal;
    int window;
    int bias_kind;
    const float *bias_table;
    int bias_lo, bias_hi;
    double rope_base;            /* 0: no rotary embedding */
    int rope_bf16;               /* turned rows rounded to bf16 (bf16 operands) */
    double *qrot, *krot;         /* turned copies of q and k (rotary embedding only) */
} problem;

static int64_t clampi(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

static double bias_at(const problem *p, int h, int64_t i, int64_t j) {
    int64_t width = (int64_t)p->bias_hi - p->bias_lo + 1;
    const float *row = p->bias_table + (int64_t)h * width;
    switch (p->bias_kind) {
    case BIAS_REL: return row[clampi(i - j, p->bias_lo, p->bias_hi) - p->bias_lo];
    case BIAS_KEYPOS: return row[clampi(j, p->bias_lo, p->bias_hi) - p->bias_lo];
    default: return 0.0;
    }
}

static int is_valid(const problem *p, int64_t i, int64_t j, int64_t lq, int64_t lk) {
    if (j < 0 || j >= lk) return 0;
    const int64_t ia = i + lk - lq;  /* the query's position aligned to the keys */
    if (p->causal && j > ia) return 0;
    if (p->window > 0 && (ia - j >= p->window || (!p->causal && j - ia >= p->window))) return 0;
    return 1;
}

typedef struct { int64_t qs, lq, ks, lk, o0; } sample;

/* Rows of sample b: query rows start at global row qs (lq of them), key rows
 * at ks (lk of them); output rows start at o0. */
static sample sample_rows(const problem *p, int b) {
    sample s;
    if (p->q_off) { s.qs = p->q_off[b]; s.lq = (int64_t)p->q_off[b + 1] - p->q_off[b]; s.o0 = s.qs; }
    else { s.qs = 0; s.lq = p->lq_fixed; s.o0 = (int64_t)b * p->lq_fixed; }
    s.ks = p->kv_off[b];
    s.lk = (int64_t)p->kv_off[b + 1] - p->kv_off[b];
    return s;
}

static const float *row_of(const problem *p, const float *base, int64_t row, int h) {
    return base + (row * p->H + h) * (int64_t)p->D;
}

/* Element d of query row `row` (global), head h, as the scores see it: turned
 * by the rotary embedding when there is one. */
static double q_at(const problem *p, int64_t row, int h, int d) {
    const int64_t e = (row * p->H + h) * (int64_t)p->D + d;
    return p->qrot ? p->qrot[e] : (double)p->q[e];
}
static double k_at(const problem *p, int64_t row, int h, int d) {
    const int64_t e = (row * p->H + h) * (int64_t)p->D + d;
    return p->krot ? p->krot[e] : (double)p->k[e];
}

/* Rotary embedding of one row x[0..D) at position t: pair (d, d + D/2) turns
 * by sign * t * base^(-2d/D) (sign -1: the inverse turn). */
static void rope_turn(double *x, int D, double base, double t, int sign) {
    const int half = D / 2;
    for (int d = 0; d < half; ++d) {
        const double a = sign * t * pow(base, -2.0 * d / D);
        const double c = cos(a), sn = sin(a);
        const double x0 = x[d], x1 = x[d + half];
        x[d] = x0 * c - x1 * sn;
        x[d + half] = x0 * sn + x1 * c;
    }
}

/* Nearest bf16 value of a double, ties to even: 8 significant bits, the
 * exponent range of float32 (normal down to 2^-126, below it a fixed step of
 * 2^-133), magnitudes that round past the largest finite bf16 value become
 * infinite.  Written from the definition of rounding to a p-bit significand. */
static double bf16_nearest(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    frexp(x, &e);                /* 2^(e-1) <= |x| < 2^e */
    int q = e - 8;               /* the bf16 step at |x|: 2^(e-1-7) */
    if (q < -133) q = -133;
    const double r = ldexp(nearbyint(ldexp(x, -q)), q);  /* default rounding: to nearest, ties even */
    const double bf16_max = ldexp(255.0, 120);           /* (2 - 2^-7) 2^127 */
    return fabs(r) > bf16_max ? copysign(INFINITY, x) : r;
}

/* The exact turn of one row (in double), each element rounded to bf16. */
static void rope_turn_bf16(const float *x, double *y, int D, double base, double t) {
    for (int d = 0; d < D; ++d) y[d] = (double)x[d];
    rope_turn(y, D, base, t, 1);
    for (int d = 0; d < D; ++d) y[d] = bf16_nearest(y[d]);
}

/* Turned copy of a [rows, H, D] tensor: row r of sample b sits at position
 * r - off[b]; with off NULL (a shared query block) row r sits at position r. */
static double *rope_copy(const float *x, const int32_t *off, int B, int64_t rows, int H, int D,
                         double base, int round_bf16) {
    double *y = (double *)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1) * H * D);
    if (!y) return NULL;
    for (int64_t e = 0; e < rows * H * D; ++e) y[e] = (double)x[e];
    for (int b = 0; b < (off ? B : 1); ++b) {
        const int64_t r0 = off ? off[b] : 0, r1 = off ? off[b + 1] : rows;
        for (int64_t r = r0; r < r1; ++r)
            for (int h = 0; h < H; ++h) {
                const int64_t e = (r * H + h) * (int64_t)D;
                if (round_bf16) rope_turn_bf16(x + e, y + e, D, base, (double)(r - r0));
                else rope_turn(y + e, D, base, (double)(r - r0), 1);
            }
    }
    return y;
}

static double score(const problem *p, int h, const sample *s, int64_t i, int64_t j) {
    double dot = 0.0;
    for (int d = 0; d < p->D; ++d) dot += q_at(p, s->qs + i, h, d) * k_at(p, s->ks + j, h, d);
    return p->scale * dot + bias_at(p, h, i, j);
}

static double *orow(const problem *p, double *base, int64_t row, int h) {
    return base + (row * p->H + h) * (int64_t)p->D;
}

/* Per-row softmax statistics of JFA over the valid keys: m = max, l = sum exp(X - m). */
static int row_stats(const problem *p, int h, const sample *s, int64_t i, double *m_out, double *l_out) {
    double m = -INFINITY;
    int any = 0;
    for (int64_t j = 0; j < s->lk; ++j) {
        if (!is_valid(p, i, j, s->lq, s->lk)) continue;
        double x = score(p, h, s, i, j);
        if (x > m) m = x;
        any = 1;
    }
    double l = 0.0;
    if (any)
        for (int64_t j = 0; j < s->lk; ++j)
            if (is_valid(p, i, j, s->lq, s->lk)) l += exp(score(p, h, s, i, j) - m);
    *m_out = m;
    *l_out = l;
    return any;
}

/* Global query row r (0 <= r < rows of the output) -> its sample. */
static int sample_of_out_row(const problem *p, int64_t r) {
    if (!p->q_off) return (int)(r / p->lq_fixed);
    int lo = 0, hi = p->B - 1; /* last b with q_off[b] <= r */
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (p->q_off[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

static int sample_of_key_row(const problem *p, int64_t r) {
    int lo = 0, hi = p->B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (p->kv_off[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

/* Forward of one query row i of sample b, head h.  softmax = 0: GDPA, 1: JFA. */
static void fwd_row(const problem *p, int softmax, int b, int h, int64_t i, double *o, double *lse) {
    sample s = sample_rows(p, b);
    const int D = p->D;
    double *oi = orow(p, o, s.o0 + i, h);
    for (int d = 0; d < D; ++d) oi[d] = 0.0;
    double m = 0.0, l = 1.0;
    if (softmax) {
        int any = row_stats(p, h, &s, i, &m, &l);
        if (lse) lse[(s.o0 + i) * p->H + h] = any ? m + log(l) : -INFINITY;
        if (!any) return;
    }
    for (int64_t j = 0; j < s.lk; ++j) {
        if (!is_valid(p, i, j, s.lq, s.lk)) continue;
        double x = score(p, h, &s, i, j);
        double w = softmax ? exp(x - m) / l : act_f(p->act, x);
        const float *vj = row_of(p, p->v, s.ks + j, h);
        for (int d = 0; d < D; ++d) oi[d] += w * (double)vj[d];
    }
}

/* Weight W_ij (act(X) or softmax P) and dX_ij of one valid pair, given the
 * row's softmax statistics m, l and delta = sum_k P_ik dP_ik (JFA only). */
static void pair_bwd(const problem *p, int softmax, int h, const sample *s, int64_t i, int64_t j,
                     const float *doi, double m, double l, double delta, double *w, double *dx) {
    double x = score(p, h, s, i, j);
    const float *vj = row_of(p, p->v, s->ks + j, h);
    double dp = 0.0;
    for (int d = 0; d < p->D; ++d) dp += (double)doi[d] * (double)vj[d];
    if (softmax) {
        *w = exp(x - m) / l;
        *dx = *w * (dp - delta);
    } else {
        *w = act_f(p->act, x);
        *dx = dp * act_grad(p->act, x);
    }
}

/* Softmax statistics of query row i (JFA): m, l, and delta_i = sum_j P_ij dP_ij;
 * with oabs non-NULL also sum_d |dO_id| |O_id| (O_i = sum_j P_ij v_j). */
static int row_bwd_stats(const problem *p, int h, const sample *s, int64_t i, const float *doi,
                         double *m, double *l, double *delta, double *oabs) {
    if (!row_stats(p, h, s, i, m, l)) return 0;
    double dl = 0.0, o[128];
    for (int d = 0; d < p->D && oabs; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < s->lk; ++j) {
        if (!is_valid(p, i, j, s->lq, s->lk)) continue;
        double w, dx;
        pair_bwd(p, 1, h, s, i, j, doi, *m, *l, 0.0, &w, &dx);  /* dx = P_ij dP_ij here */
        dl += dx;
        if (oabs) {
            const float *vj = row_of(p, p->v, s->ks + j, h);
            for (int d = 0; d < p->D; ++d) o[d] += w * (double)vj[d];
        }
    }
    *delta = dl;
    if (oabs) {
        double a = 0.0;
        for (int d = 0; d < p->D; ++d) a += fabs((double)doi[d]) * fabs(o[d]);
        *oabs = a;
    }
    return 1;
}

static int nthreads_or_default(int nthreads) {
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

static problem make_problem(const float *q, const float *k, const float *v, const int32_t *q_off,
                            int32_t lq_fixed, const int32_t *kv_off, int B, int H, int D, double scale,
                            int act, int causal, int window, double rope_base, int bias_kind,
                            const float *bias_table, int bias_lo, int bias_hi) {
    problem p;
    p.q = q; p.k = k; p.v = v; p.q_off = q_off; p.kv_off = kv_off; p.lq_fixed = lq_fixed;
    p.B = B; p.H = H; p.D = D; p.scale = scale; p.act = act; p.causal = causal; p.window = window;
    p.bias_kind = bias_table ? bias_kind : BIAS_NONE; p.bias_table = bias_table;
    p.bias_lo = bias_lo; p.bias_hi = bias_hi;
    p.rope_base = fabs(rope_base);
    p.rope_bf16 = rope_base < 0.0;
    p.qrot = p.krot = NULL;
    return p;
}

/* Turned copies of q and k when the problem has a rotary embedding. */
static int rope_prepare(problem *p) {
    if (!(p->rope_base > 0.0)) return 0;
    const int64_t tq = p->q_off ? (int64_t)p->q_off[p->B] : p->lq_fixed;
    p->qrot = rope_copy(p->q, p->q_off, p->B, tq, p->H, p->D, p->rope_base, p->rope_bf16);
    p->krot = rope_copy(p->k, p->kv_off, p->B, (int64_t)p->kv_off[p->B], p->H, p->D, p->rope_base,
                        p->rope_bf16);
    return (p->qrot && p->krot) ? 0 : 2;
}
static void rope_release(problem *p) {
    free(p->qrot);
    free(p->krot);
    p->qrot = p->krot = NULL;
}

static int64_t out_rows(const problem *p) {
    return p->q_off ? (int64_t)p->q_off[p->B] : (int64_t)p->B * p->lq_fixed;
}

/* Every output row (all heads) is independent: parallel over rows. */
static void run_fwd(const problem *p, int softmax, double *o, double *lse, int nthreads) {
    const int64_t n = out_rows(p) * p->H;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads_or_default(nthreads))
    for (int64_t u = 0; u < n; ++u) {
        const int64_t r = u / p->H;
        const int h = (int)(u % p->H);
        const int b = sample_of_out_row(p, r);
        const int64_t o0 = p->q_off ? p->q_off[b] : (int64_t)b * p->lq_fixed;
        fwd_row(p, softmax, b, h, r - o0, o, lse);
    }
}

/* Backward: (1) per query row, the softmax statistics (JFA); (2) dQ per query
 * row, summing over its keys; (3) dK and dV per key row, summing over the
 * query rows that see it.  Each output row is written by one iteration, so
 * every phase is parallel over rows and needs no reduction across threads. */
/* Rounding-noise scale of one gradient row (optional outputs nq, nk), the sum
 * of two parts:
 *  - with terms t_d = scale dX_ij x_jd summed over j, max_d sqrt(sum_j t_d^2)
 *    times dx_unit, the unit roundoff of the dX operands (2^-8 for bf16): the
 *    error a sum of those terms carries when each dX_ij is rounded before it is
 *    multiplied;
 *  - (JFA) scale max_d sum_j P_ij |delta-error_i| |x_jd| with the error of delta
 *    taken as delta_unit sum_d |dO_id| |O_id| (2^-16 for an output held to 16
 *    significant bits: a bf16 value plus its bf16 residual), which decides rows
 *    whose exact dX vanishes (a row with one visible key).
 * With the rotary embedding the row is turned back afterwards, which mixes
 * elements d and d + D/2, so pairs are combined. */
static double noise_of(const double *ss, const double *pd, int D, int turned, double scale, double dx_unit,
                       double delta_unit) {
    double mx = 0.0, mp = 0.0;
    for (int d = 0; d < D; ++d) {
        const int e = d < D / 2 ? d + D / 2 : d - D / 2;
        const double v = ss[d] + (turned ? ss[e] : 0.0);
        const double w = pd[d] + (turned ? pd[e] : 0.0);
        if (v > mx) mx = v;
        if (w > mp) mp = w;
    }
    return dx_unit * sqrt(mx) + scale * delta_unit * mp;
}

static int run_bwd(const problem *p, int softmax, const float *dout, double *dq, double *dk,
                   double *dv, double *nq, double *nk, double dx_unit, double delta_unit, int nthreads) {
    if (!p->q_off) return 1;
    const int64_t tq = p->q_off[p->B], tk = p->kv_off[p->B];
    const int H = p->H, D = p->D;
    double *st = NULL; /* per (row, head): m, l, delta, valid, sum_d |dO| |O| */
    if (softmax) {
        st = (double *)malloc(sizeof(double) * 5 * (size_t)(tq > 0 ? tq : 1) * H);
        if (!st) return 2;
    }
    const int nt = nthreads_or_default(nthreads);
    if (softmax) {
#pragma omp parallel for schedule(dynamic, 16) num_threads(nt)
        for (int64_t u = 0; u < tq * H; ++u) {
            const int64_t r = u / H;
            const int h = (int)(u % H);
            const int b = sample_of_out_row(p, r);
            sample s = sample_rows(p, b);
            double *sr = st + 5 * u;
            sr[4] = 0.0;
            sr[3] = row_bwd_stats(p, h, &s, r - s.qs, row_of(p, dout, r, h), &sr[0], &sr[1], &sr[2],
                                  (nq || nk) ? &sr[4] : NULL);
        }
    }
#pragma omp parallel for schedule(dynamic, 16) num_threads(nt)
    for (int64_t u = 0; u < tq * H; ++u) {
        const int64_t r = u / H;
        const int h = (int)(u % H);
        const int b = sample_of_out_row(p, r);
        sample s = sample_rows(p, b);
        const int64_t i = r - s.qs;
        double *dqi = orow(p, dq, r, h);
        double ss[128], pd[128];
        for (int d = 0; d < D; ++d) { dqi[d] = 0.0; ss[d] = 0.0; pd[d] = 0.0; }
        if (nq) nq[u] = 0.0;
        const double *sr = softmax ? st + 5 * u : NULL;
        if (softmax && sr[3] == 0.0) continue;
        const float *doi = row_of(p, dout, r, h);
        for (int64_t j = 0; j < s.lk; ++j) {
            if (!is_valid(p, i, j, s.lq, s.lk)) continue;
            double w, dx;
            pair_bwd(p, softmax, h, &s, i, j, doi, sr ? sr[0] : 0.0, sr ? sr[1] : 1.0,
                     sr ? sr[2] : 0.0, &w, &dx);
            for (int d = 0; d < D; ++d) {
                const double kd = k_at(p, s.ks + j, h, d);
                const double t = p->scale * dx * kd;
                dqi[d] += t;
                ss[d] += t * t;
                if (sr) pd[d] += w * sr[4] * fabs(kd);
            }
        }
        if (p->qrot) rope_turn(dqi, D, p->rope_base, (double)i, -1);
        if (nq) nq[u] = noise_of(ss, pd, D, p->qrot != NULL, p->scale, dx_unit, delta_unit);
    }
#pragma omp parallel for schedule(dynamic, 16) num_threads(nt)
    for (int64_t u = 0; u < tk * H; ++u) {
        const int64_t r = u / H;
        const int h = (int)(u % H);
        const int b = sample_of_key_row(p, r);
        sample s = sample_rows(p, b);
        const int64_t j = r - s.ks;
        double *dkj = orow(p, dk, r, h), *dvj = orow(p, dv, r, h);
        double ss[128], pd[128];
        for (int d = 0; d < D; ++d) { dkj[d] = 0.0; dvj[d] = 0.0; ss[d] = 0.0; pd[d] = 0.0; }
        for (int64_t i = 0; i < s.lq; ++i) {
            if (!is_valid(p, i, j, s.lq, s.lk)) continue;
            const double *sr = softmax ? st + 5 * ((s.qs + i) * H + h) : NULL;
            const float *doi = row_of(p, dout, s.qs + i, h);
            double w, dx;
            pair_bwd(p, softmax, h, &s, i, j, doi, sr ? sr[0] : 0.0, sr ? sr[1] : 1.0,
                     sr ? sr[2] : 0.0, &w, &dx);
            for (int d = 0; d < D; ++d) {
                const double qd = q_at(p, s.qs + i, h, d);
                const double t = p->scale * dx * qd;
                dkj[d] += t;
                ss[d] += t * t;
                if (sr) pd[d] += w * sr[4] * fabs(qd);
                dvj[d] += w * (double)doi[d];
            }
        }
        if (p->krot) rope_turn(dkj, D, p->rope_base, (double)j, -1);
        if (nk) nk[u] = noise_of(ss, pd, D, p->krot != NULL, p->scale, dx_unit, delta_unit);
    }
    free(st);
    return 0;
}

/* Gradient of L with respect to the bias table: each (sample, head) adds the
 * dX of its valid pairs to the entry the pair reads, into its own row of
 * partial sums; the rows are then added sample by sample in order. */
static int run_dbias(const problem *p, int softmax, const float *dout, double *dtable, int nthreads) {
    if (!p->q_off || p->bias_kind == BIAS_NONE) return 1;
    const int B = p->B, H = p->H;
    const int64_t W = (int64_t)p->bias_hi - p->bias_lo + 1;
    double *part = (double *)calloc((size_t)(B > 0 ? B : 1) * H * W, sizeof(double));
    if (!part) return 2;
    const int nt = nthreads_or_default(nthreads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t u = 0; u < (int64_t)B * H; ++u) {
        const int b = (int)(u / H), h = (int)(u % H);
        sample s = sample_rows(p, b);
        double *row = part + u * W;
        for (int64_t i = 0; i < s.lq; ++i) {
            const float *doi = row_of(p, dout, s.qs + i, h);
            double m = 0.0, l = 1.0, delta = 0.0;
            if (softmax && !row_bwd_stats(p, h, &s, i, doi, &m, &l, &delta, NULL)) continue;
            for (int64_t j = 0; j < s.lk; ++j) {
                if (!is_valid(p, i, j, s.lq, s.lk)) continue;
                double w, dx;
                pair_bwd(p, softmax, h, &s, i, j, doi, m, l, delta, &w, &dx);
                const int64_t pos = p->bias_kind == BIAS_REL ? i - j : j;
                row[clampi(pos, p->bias_lo, p->bias_hi) - p->bias_lo] += dx;
            }
        }
    }
    for (int64_t c = 0; c < (int64_t)H * W; ++c) dtable[c] = 0.0;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int64_t c = 0; c < W; ++c) dtable[(int64_t)h * W + c] += part[((int64_t)b * H + h) * W + c];
    free(part);
    return 0;
}

/* ------------------------------------------------------------ exported API */
/* act: 0 SiLU, 1 GELU (tanh form), 2 GELU (erf form).
 * bias_kind: 0 none, 1 REL (query minus key), 2 KEYPOS (key position).
 * rope_base: 0 for no rotary embedding, else the base of its angles; a negative
 * value -b means base b with the turned rows rounded to bf16 (rope_bf16).
 * nthreads <= 0: OpenMP default.  Return 0 on success. */

int ref_gdpa_fwd(const float *q, const float *k, const float *v, double *o, const int32_t *q_off,
                 int32_t lq_fixed, const int32_t *kv_off, int B, int H, int D, double scale, int act,
                 int causal, int window, double rope_base, int bias_kind, const float *bias_table,
                 int bias_lo, int bias_hi, int nthreads) {
    problem p = make_problem(q, k, v, q_off, lq_fixed, kv_off, B, H, D, scale, act, causal, window, rope_base,
                             bias_kind, bias_table, bias_lo, bias_hi);
    if (rope_prepare(&p)) { rope_release(&p); return 2; }
    run_fwd(&p, 0, o, NULL, nthreads);
    rope_release(&p);
    return 0;
}

/* lse: [total_q_out, H] (token-major, like the outputs). */
int ref_attn_fwd(const float *q, const float *k, const float *v, double *o, double *lse,
                 const int32_t *q_off, int32_t lq_fixed, const int32_t *kv_off, int B, int H, int D,
                 double scale, int causal, int window, double rope_base, int bias_kind,
                 const float *bias_table, int bias_lo, int bias_hi, int nthreads) {
    problem p = make_problem(q, k, v, q_off, lq_fixed, kv_off, B, H, D, scale, ACT_SILU, causal, window,
                             rope_base, bias_kind, bias_table, bias_lo, bias_hi);
    if (rope_prepare(&p)) { rope_release(&p); return 2; }
    run_fwd(&p, 1, o, lse, nthreads);
    rope_release(&p);
    return 0;
}

int ref_gdpa_bwd(const float *q, const float *k, const float *v, const float *dout, double *dq,
                 double *dk, double *dv, const int32_t *q_off, const int32_t *kv_off, int B, int H,
                 int D, double scale, int act, int causal, int window, double rope_base, int bias_kind,
                 const float *bias_table, int bias_lo, int bias_hi, int nthreads) {
    problem p = make_problem(q, k, v, q_off, 0, kv_off, B, H, D, scale, act, causal, window, rope_base,
                             bias_kind, bias_table, bias_lo, bias_hi);
    if (!q_off) return 1;
    if (rope_prepare(&p)) { rope_release(&p); return 2; }
    const int rc = run_bwd(&p, 0, dout, dq, dk, dv, NULL, NULL, 0.0, 0.0, nthreads);
    rope_release(&p);
    return rc;
}

int ref_attn_bwd(const float *q, const float *k, const float *v, const float *dout, double *dq,
                 double *dk, double *dv, const int32_t *q_off, const int32_t *kv_off, int B, int H,
                 int D, double scale, int causal, int window, double rope_base, int bias_kind,
                 const float *bias_table, int bias_lo, int bias_hi, int nthreads) {
    problem p = make_problem(q, k, v, q_off, 0, kv_off, B, H, D, scale, ACT_SILU, causal, window, rope_base,
                             bias_kind, bias_table, bias_lo, bias_hi);
    if (!q_off) return 1;
    if (rope_prepare(&p)) { rope_release(&p); return 2; }
    const int rc = run_bwd(&p, 1, dout, dq, dk, dv, NULL, NULL, 0.0, 0.0, nthreads);
    rope_release(&p);
    return rc;
}

/* As ref_gdpa_bwd / ref_attn_bwd (softmax 0 / 1), also writing the rounding-noise
 * scale of every dQ row (nq [total_q, H]) and dK row (nk [total_k, H]) for the
 * given unit roundoffs of dX and of delta (see noise_of). */
int ref_bwd_noise(int softmax, const float *q, const float *k, const float *v, const float *dout,
                  double *dq, double *dk, double *dv, double *nq, double *nk, const int32_t *q_off,
                  const int32_t *kv_off, int B, int H, int D, double scale, int act, int causal,
                  int window, double rope_base, int bias_kind, const float *bias_table, int bias_lo,
                  int bias_hi, double dx_unit, double delta_unit, int nthreads) {
    problem p = make_problem(q, k, v, q_off, 0, kv_off, B, H, D, scale, act, causal, window, rope_base,
                             bias_kind, bias_table, bias_lo, bias_hi);
    if (!q_off || D > 128) return 1;
    if (rope_prepare(&p)) { rope_release(&p); return 2; }
    const int rc = run_bwd(&p, softmax, dout, dq, dk, dv, nq, nk, dx_unit, delta_unit, nthreads);
    rope_release(&p);
    return rc;
}

/* dL/dtable [H][bias_hi - bias_lo + 1] of L = <O, dout> (needs a bias kind). */
int ref_gdpa_dbias(const float *q, const float *k, const float *v, const float *dout, double *dtable,
                   const int32_t *q_off, const int32_t *kv_off, int B, int H, int D, double scale,
                   int act, int causal, int window, double rope_base, int bias_kind,
                   const float *bias_table, int bias_lo, int bias_hi, int nthreads) {
    problem p = make_problem(q, k, v, q_off, 0, kv_off, B, H, D, scale, act, causal, window, rope_base,
                             bias_kind, bias_table, bias_lo, bias_hi);
    if (!q_off) return 1;
    if (rope_prepare(&p)) { rope_release(&p); return 2; }
    const int rc = run_dbias(&p, 0, dout, dtable, nthreads);
    rope_release(&p);
    return rc;
}

int ref_attn_dbias(const float *q, const float *k, const float *v, const float *dout, double *dtable,
                   const int32_t *q_off, const int32_t *kv_off, int B, int H, int D, double scale,
                   int causal, int window, double rope_base, int bias_kind, const float *bias_table,
                   int bias_lo, int bias_hi, int nthreads) {
    problem p = make_problem(q, k, v, q_off, 0, kv_off, B, H, D, scale, ACT_SILU, causal, window, rope_base,
                             bias_kind, bias_table, bias_lo, bias_hi);
    if (!q_off) return 1;
    if (rope_prepare(&p)) { rope_release(&p); return 2; }
    const int rc = run_dbias(&p, 1, dout, dtable, nthreads);
    rope_release(&p);
    return rc;
}

/* One entry c of head h of the GDPA table gradient, summed sample by sample.
 * An interior entry is read by one relative position (REL: j = i - (lo + c))
 * or one key (KEYPOS: j = lo + c) per query row, so only those pairs are
 * visited; the end entries (c = 0 or c = hi - lo) scan every pair of a row. */
int ref_gdpa_dbias_entry(const float *q, const float *k, const float *v, const float *dout,
                         double *out, const int32_t *q_off, const int32_t *kv_off, int B, int H,
                         int D, double scale, int act, int causal, int window, double rope_base,
                         int bias_kind, const float *bias_table, int bias_lo, int bias_hi, int h, int c,
                         int nthreads) {
    problem p = make_problem(q, k, v, q_off, 0, kv_off, B, H, D, scale, act, causal, window, rope_base,
                             bias_kind, bias_table, bias_lo, bias_hi);
    const int64_t W = (int64_t)bias_hi - bias_lo + 1;
    if (!q_off || p.bias_kind == BIAS_NONE || h < 0 || h >= H || c < 0 || c >= W) return 1;
    if (rope_prepare(&p)) { rope_release(&p); return 2; }
    const int interior = c > 0 && c < W - 1;
    double *per_b = (double *)calloc((size_t)(B > 0 ? B : 1), sizeof(double));
    if (!per_b) { rope_release(&p); return 2; }
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads_or_default(nthreads))
    for (int b = 0; b < B; ++b) {
        sample s = sample_rows(&p, b);
        double acc = 0.0;
        for (int64_t i = 0; i < s.lq; ++i) {
            const float *doi = row_of(&p, dout, s.qs + i, h);
            int64_t j0 = 0, j1 = s.lk;
            if (interior) {
                j0 = p.bias_kind == BIAS_REL ? i - (bias_lo + c) : (int64_t)bias_lo + c;
                j1 = j0 + 1;
            }
            for (int64_t j = j0 < 0 ? 0 : j0; j < j1 && j < s.lk; ++j) {
                if (!is_valid(&p, i, j, s.lq, s.lk)) continue;
                const int64_t pos = p.bias_kind == BIAS_REL ? i - j : j;
                if (clampi(pos, bias_lo, bias_hi) - bias_lo != c) continue;
                double w, dx;
                pair_bwd(&p, 0, h, &s, i, j, doi, 0.0, 1.0, 0.0, &w, &dx);
                acc += dx;
            }
        }
        per_b[b] = acc;
    }
    double tot = 0.0;
    for (int b = 0; b < B; ++b) tot += per_b[b];
    *out = tot;
    free(per_b);
    rope_release(&p);
    return 0;
}

/* The turned copy of a [rows, H, D] tensor (positions from off as above;
 * rope_base negative: the bf16-rounded variant), exported so the tests can pin
 * the turn on its own. */
int ref_rope(const float *x, double *out, const int32_t *off, int B, int64_t rows, int H, int D,
             double rope_base) {
    double *y = rope_copy(x, off, B, rows, H, D, fabs(rope_base), rope_base < 0.0);
    if (!y) return 2;
    memcpy(out, y, sizeof(double) * (size_t)rows * H * D);
    free(y);
    return 0;
}

/* Element-wise activation and derivative, exported so the tests can pin them
 * against library implementations. */
void ref_act(int act, const double *x, double *y, double *dy, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        y[i] = act_f(act, x[i]);
        dy[i] = act_grad(act, x[i]);
    }
}

int ref_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
