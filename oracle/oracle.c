/*
 * CPU oracle of the quantised MoE layer.  TEST INFRASTRUCTURE ONLY: loaded
 * by the tests, the smoke check and the benchmark's CPU-baseline leg, never
 * by the product path.  See oracle.h for the sources and conventions.
 *
 * Pins (tests/test_oracle_pins.py) tie every function here to something
 * other than itself: brute-force subset search and full sorts for the
 * router, closed forms and hand-made round-half-even vectors for the
 * quantiser, int64 brute force and a dequantise-then-matmul path for the
 * integer dots, a dense SwiGLU for the single-expert layer, linearity in
 * routed_scaling_factor, and a stable sort for the permutation.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* threads an OpenMP region of the oracle uses (1 without OpenMP) */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* sets the thread count of later OpenMP regions (timing only: every result
 * is the same for any count, each output's arithmetic order being fixed) */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_code(int wbits, const uint8_t *row, int j)
{
    if (wbits == 8)
        return (int)(int8_t)row[j];
    if (wbits == 4) {
        int nib = (j & 1) ? (row[j >> 1] >> 4) : (row[j >> 1] & 15);
        return nib >= 8 ? nib - 16 : nib;
    }
    /* wbits == 2 */
    int f = (row[j >> 2] >> (2 * (j & 3))) & 3;
    return f >= 2 ? f - 4 : f;
}

static size_t row_bytes(int wbits, int in_dim) { return (size_t)in_dim * wbits / 8; }

/* ------------------------------------------------------------------------
 * Router.  GeekNews #31297, "implemented features": a DeepSeek-V3-style
 * sigmoid router, noaux_tc, with routed_scaling_factor; wpnews.pro spec
 * table: 8 of 256 experts active per token.
 *
 * reading: the noaux_tc steps are those of DeepSeek-V3's router: score
 *   s = sigmoid(x . W_e); the correction bias is added for selection only,
 *   c = s + bias; a group's score is the sum of its two largest c (its only
 *   c when a group holds one expert); the topk_group best groups are kept
 *   and the others excluded outright; the top_k largest c among the kept
 *   experts are selected; their weights are the unbiased s normalised to sum
 *   to one, times routed_scaling_factor.
 * reading: the router reads the unquantised fp32 x; z, s and c are fp64.
 * reading: ties go to the lower group / expert index; the k outputs are in
 *   selection order (c descending, index ascending).
 */
void oracle_router_scores(const oracle_shape *sh, const float *x, const float *gate_w,
                          const float *bias, double *s, double *c)
{
    const int H = sh->hidden, E = sh->n_experts;
    for (int e = 0; e < E; e++) {
        double z = 0.0;
        for (int j = 0; j < H; j++)
            z += (double)x[j] * (double)gate_w[(size_t)e * H + j];
        s[e] = 1.0 / (1.0 + exp(-z));
        c[e] = s[e] + (double)bias[e];
    }
}

int oracle_route(const oracle_shape *sh, const float *x, int T, const float *gate_w,
                 const float *bias, int32_t *idx, float *w, double *margins)
{
    const int E = sh->n_experts, G = sh->n_group, tg = sh->topk_group, k = sh->top_k;
    if (E <= 0 || G <= 0 || E % G || tg < 1 || tg > G || k < 1 || k > tg * (E / G))
        return -1;
    const int m = E / G;
    int bad = 0;

    #pragma omp parallel for schedule(dynamic)
    for (int t = 0; t < T; t++) {
        double *s = malloc(sizeof(double) * E), *c = malloc(sizeof(double) * E);
        double *gscore = malloc(sizeof(double) * G);
        char *gkeep = calloc(G, 1), *taken = calloc(E, 1);
        if (!s || !c || !gscore || !gkeep || !taken) { bad = 1; goto next; }

        oracle_router_scores(sh, x + (size_t)t * sh->hidden, gate_w, bias, s, c);

        /* group score: sum of the two largest biased scores of the group */
        for (int g = 0; g < G; g++) {
            double b1 = -INFINITY, b2 = -INFINITY;
            for (int e = g * m; e < (g + 1) * m; e++) {
                if (c[e] > b1) { b2 = b1; b1 = c[e]; }
                else if (c[e] > b2) b2 = c[e];
            }
            gscore[g] = (m >= 2) ? b1 + b2 : b1;
        }
        /* keep the topk_group best groups (score desc, index asc) */
        double last_kept_g = INFINITY;
        for (int r = 0; r < tg; r++) {
            int best = -1;
            for (int g = 0; g < G; g++)
                if (!gkeep[g] && (best < 0 || gscore[g] > gscore[best])) best = g;
            gkeep[best] = 1;
            last_kept_g = gscore[best];
        }
        double best_dropped_g = -INFINITY;
        for (int g = 0; g < G; g++)
            if (!gkeep[g] && gscore[g] > best_dropped_g) best_dropped_g = gscore[g];

        /* top_k experts of the kept groups (c desc, index asc) */
        double sum = 0.0;
        for (int i = 0; i < k; i++) {
            int best = -1;
            for (int e = 0; e < E; e++)
                if (gkeep[e / m] && !taken[e] && (best < 0 || c[e] > c[best])) best = e;
            taken[best] = 1;
            idx[(size_t)t * k + i] = best;
            sum += s[best];
        }
        double best_left = -INFINITY;
        for (int e = 0; e < E; e++)
            if (gkeep[e / m] && !taken[e] && c[e] > best_left) best_left = c[e];

        /* adaptive expert top-p (GeekNews #31297, useful options; yodev.dev
           colibrì page, useful knobs: the --topp option, 30-40% fewer expert
           reads).  The pages name the knob only; the reading: keep the
           shortest prefix of the selection (selection order, at least one
           expert) whose share of the selection's summed s reaches p, the
           shares s_i / sum added in slot order in fp64, then renormalise
           over the kept prefix.  Dropped slots report expert -1 and weight 0. */
        int kept = k;
        if (sh->top_p > 0.0 && sh->top_p < 1.0) {
            double cum = 0.0;
            kept = 0;
            while (kept < k) {
                cum += s[idx[(size_t)t * k + kept]] / sum;
                kept++;
                if (cum >= sh->top_p) break;
            }
            sum = 0.0;
            for (int i = 0; i < kept; i++) sum += s[idx[(size_t)t * k + i]];
        }
        for (int i = 0; i < k; i++)
            w[(size_t)t * k + i] = (i < kept) ? (float)(s[idx[(size_t)t * k + i]] / sum * sh->rsf) : 0.0f;

        if (margins) {
            margins[2 * t + 0] = c[idx[(size_t)t * k + k - 1]] - best_left;  /* +inf if none left */
            margins[2 * t + 1] = last_kept_g - best_dropped_g;              /* +inf if tg == G  */
        }
        for (int i = kept; i < k; i++) idx[(size_t)t * k + i] = -1;
    next:
        free(s); free(c); free(gscore); free(gkeep); free(taken);
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------
 * Activation quantisation.  GeekNews #31297, "implemented features": the
 * integer-dot kernels take Q8_0-style int8 activations.
 *
 * reading: blocks of 32 consecutive elements along a row; per block
 *   amax = max |x|, d = amax / 127 as an fp32 IEEE division (the scale is
 *   kept in fp32, not fp16 as in Q8_0 proper); q = rint(x / d) with an fp32
 *   division and round-half-to-even, clamped to [-127, 127]; an all-zero
 *   block has d = 0 and q = 0.  No flush-to-zero: a subnormal d is kept.
 *   Inputs must be finite.
 */
void oracle_quant_act(const float *x, int T, int D, int8_t *q, float *d)
{
    const int nb = D / 32;
    for (int t = 0; t < T; t++)
        for (int b = 0; b < nb; b++) {
            const float *xb = x + (size_t)t * D + 32 * b;
            int8_t *qb = q + (size_t)t * D + 32 * b;
            float amax = 0.0f;
            for (int j = 0; j < 32; j++)
                if (fabsf(xb[j]) > amax) amax = fabsf(xb[j]);
            float db = amax / 127.0f;
            d[(size_t)t * nb + b] = db;
            for (int j = 0; j < 32; j++) {
                float v = (db == 0.0f) ? 0.0f : rintf(xb[j] / db);
                if (v > 127.0f) v = 127.0f;
                if (v < -127.0f) v = -127.0f;
                qb[j] = (int8_t)v;
            }
        }
}

/* ------------------------------------------------------------------------
 * Integer block dots.  GeekNews #31297, "implemented features": the matmul
 * multiplies int8 activations by int8 / packed int4 / packed int2 weight
 * codes with integer arithmetic; per-row weight scales and the activation
 * block scales are applied after the integer sums.
 *   out[t][r][b] = sum_{j<32} code[r][32b + j] * q[t][32b + j]   (int32)
 */
void oracle_block_dots(int wbits, const uint8_t *codes, int rows, int D, const int8_t *q,
                       int T, int32_t *out)
{
    const int nb = D / 32;
    const size_t rb = row_bytes(wbits, D);
    #pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; r++)
        for (int t = 0; t < T; t++)
            for (int b = 0; b < nb; b++) {
                int64_t acc = 0;
                for (int j = 32 * b; j < 32 * b + 32; j++)
                    acc += (int64_t)oracle_code(wbits, codes + r * rb, j) * q[(size_t)t * D + j];
                out[((size_t)t * rows + r) * nb + b] = (int32_t)acc;
            }
}

/*   y[t][r] = (float)( s_w[r] * sum_b d[t][b] * I[t][r][b] )   all in fp64
 * (each term d * I is exact in fp64: a 24-bit mantissa times |I| < 2^20) */
void oracle_matvec(int wbits, const uint8_t *codes, const float *s_w, int rows, int D,
                   const int8_t *q, const float *d, int T, float *y)
{
    const int nb = D / 32;
    const size_t rb = row_bytes(wbits, D);
    #pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; r++)
        for (int t = 0; t < T; t++) {
            double acc = 0.0;
            for (int b = 0; b < nb; b++) {
                int64_t blk = 0;
                for (int j = 32 * b; j < 32 * b + 32; j++)
                    blk += (int64_t)oracle_code(wbits, codes + r * rb, j) * q[(size_t)t * D + j];
                acc += (double)d[(size_t)t * nb + b] * (double)blk;
            }
            y[(size_t)t * rows + r] = (float)((double)s_w[r] * acc);
        }
}

/* Cross-check path: dequantise both operands to fp64 (W = s_w * code,
 * x = d * q) and take the plain dot product; equals oracle_matvec before
 * its final fp32 rounding, up to fp64 summation order. */
void oracle_dequant_matmul(int wbits, const uint8_t *codes, const float *s_w, int rows, int D,
                           const int8_t *q, const float *d, int T, double *y)
{
    const int nb = D / 32;
    const size_t rb = row_bytes(wbits, D);
    for (int t = 0; t < T; t++)
        for (int r = 0; r < rows; r++) {
            double acc = 0.0;
            for (int j = 0; j < D; j++) {
                double wf = (double)s_w[r] * oracle_code(wbits, codes + r * rb, j);
                double xf = (double)d[(size_t)t * nb + j / 32] * q[(size_t)t * D + j];
                acc += wf * xf;
            }
            y[(size_t)t * rows + r] = acc;
        }
}

/* ------------------------------------------------------------------------
 * One SwiGLU expert on quantised activations (q, d over H):
 *   g = W_gate x, u = W_up x                     (oracle_matvec)
 *   h = (float)( silu(g) * u ),  silu(z) = z / (1 + exp(-z))   in fp64
 *   (qh, dh) = quant(h) over I                   (oracle_quant_act)
 *   y = W_down h                                 (oracle_matvec)
 * reading: the expert's hidden activation h is itself quantised to int8
 *   before the down projection, since the pages' integer-dot design feeds
 *   int8 activations to every expert matmul.
 * qh / dh (nullable) receive the intermediate codes and scales.
 */
int oracle_expert_ffn(const oracle_shape *sh, const oracle_expert *ex, const int8_t *q,
                      const float *d, int T, float *y, int8_t *qh, float *dh)
{
    const int H = sh->hidden, I = sh->inter;
    float *g = malloc(sizeof(float) * (size_t)T * I), *u = malloc(sizeof(float) * (size_t)T * I);
    float *h = malloc(sizeof(float) * (size_t)T * I);
    int8_t *qh_ = malloc((size_t)T * I);
    float *dh_ = malloc(sizeof(float) * (size_t)T * (I / 32));
    int rc = 0;
    if (!g || !u || !h || !qh_ || !dh_) { rc = -2; goto out; }

    oracle_matvec(sh->wbits, ex->gate, ex->gate_s, I, H, q, d, T, g);
    oracle_matvec(sh->wbits, ex->up, ex->up_s, I, H, q, d, T, u);
    for (size_t i = 0; i < (size_t)T * I; i++) {
        double gz = (double)g[i];
        double silu = gz / (1.0 + exp(-gz));
        h[i] = (float)(silu * (double)u[i]);
    }
    oracle_quant_act(h, T, I, qh_, dh_);
    oracle_matvec(sh->wbits, ex->down, ex->down_s, H, I, qh_, dh_, T, y);
    if (qh) memcpy(qh, qh_, (size_t)T * I);
    if (dh) memcpy(dh, dh_, sizeof(float) * (size_t)T * (I / 32));
out:
    free(g); free(u); free(h); free(qh_); free(dh_);
    return rc;
}

/* ------------------------------------------------------------------------
 * Weighted combine.  wpnews.pro spec table: 8 active + 1 shared expert.
 *   out[t] = (float)( sum_{i<k} w[t][i] * y_i[t] + y_shared[t] )   in fp64,
 * slots in order, then the shared expert.
 * reading: the shared expert has weight 1 and is not scaled by
 *   routed_scaling_factor.
 * y_slots is [T][k][H]; y_shared [T][H] or NULL.
 */
int oracle_combine(const oracle_shape *sh, int T, const float *w, const float *y_slots,
                   const float *y_shared, float *out)
{
    const int H = sh->hidden, k = sh->top_k;
    for (int t = 0; t < T; t++)
        for (int r = 0; r < H; r++) {
            double acc = 0.0;
            for (int i = 0; i < k; i++)
                acc += (double)w[(size_t)t * k + i] * (double)y_slots[((size_t)t * k + i) * H + r];
            if (y_shared) acc += (double)y_shared[(size_t)t * H + r];
            out[(size_t)t * H + r] = (float)acc;
        }
    return 0;
}

/* ------------------------------------------------------------------------
 * The MoE layer: route x, quantise x, run each token's k routed experts and
 * the shared expert, combine.  Tokens are independent; GeekNews #31297's
 * batch-union MoE (each unique expert read once per batch and applied to
 * every position routed to it) changes the schedule, not the result, so
 * the oracle runs token by token.
 * routed[e] points at expert e (it may be NULL for an expert no token
 * selects: the call fails with -3 if a selected expert is missing).
 */
int oracle_layer_forward(const oracle_shape *sh, const float *x, int T, const float *gate_w,
                         const float *bias, const oracle_expert *const *routed,
                         const oracle_expert *shared, float *y, int32_t *idx, float *w)
{
    const int H = sh->hidden, k = sh->top_k;
    int rc = oracle_route(sh, x, T, gate_w, bias, idx, w, NULL);
    if (rc) return rc;
    for (int i = 0; i < T * k; i++)
        if (idx[i] >= 0 && !routed[idx[i]]) return -3;
    if (sh->n_shared && !shared) return -3;

    int8_t *q = malloc((size_t)H);
    float *d = malloc(sizeof(float) * (H / 32));
    float *ys = malloc(sizeof(float) * (size_t)k * H), *ysh = malloc(sizeof(float) * H);
    if (!q || !d || !ys || !ysh) { rc = -2; goto out; }
    for (int t = 0; t < T; t++) {
        oracle_quant_act(x + (size_t)t * H, 1, H, q, d);
        for (int i = 0; i < k; i++) {
            if (idx[(size_t)t * k + i] < 0) {  /* dropped by top-p: weight 0, nothing read */
                memset(ys + (size_t)i * H, 0, sizeof(float) * H);
                continue;
            }
            if ((rc = oracle_expert_ffn(sh, routed[idx[(size_t)t * k + i]], q, d, 1,
                                        ys + (size_t)i * H, NULL, NULL))) goto out;
        }
        if (sh->n_shared && (rc = oracle_expert_ffn(sh, shared, q, d, 1, ysh, NULL, NULL))) goto out;
        oracle_combine(sh, 1, w + (size_t)t * k, ys, sh->n_shared ? ysh : NULL, y + (size_t)t * H);
    }
out:
    free(q); free(d); free(ys); free(ysh);
    return rc;
}

/* ------------------------------------------------------------------------
 * RMSNorm of the 75-layer decode stack, x_{l+1} = x_l + MoE_l(RMSNorm(x_l)).
 * reading: out = x / sqrt(mean(x^2) + eps) * g, mean over H, sum of squares
 *   and the scaling in fp64, one fp32 rounding at the end.
 */
void oracle_rmsnorm(const float *x, const float *g, double eps, int T, int H, float *out)
{
    for (int t = 0; t < T; t++) {
        double ss = 0.0;
        for (int j = 0; j < H; j++) ss += (double)x[(size_t)t * H + j] * (double)x[(size_t)t * H + j];
        double r = 1.0 / sqrt(ss / H + eps);
        for (int j = 0; j < H; j++)
            out[(size_t)t * H + j] = (float)((double)x[(size_t)t * H + j] * r * (double)g[j]);
    }
}

/* ------------------------------------------------------------------------
 * Token permutation for the batch-union schedule (GeekNews #31297,
 * "implemented features": each unique expert of a prefill / verify batch is
 * read once and applied to every position routed to it).
 * Assignment a = t*k + i routes token t to expert idx[a].  Rows are grouped
 * by expert: off[e] .. off[e+1]-1 hold the assignments of expert e in
 * ascending a (a counting sort, stable); perm[row] = a, inv[a] = row.
 * reading: an assignment adaptive top-p dropped (expert -1) gets no row and
 *   inv = -1; rows 0 .. off[E]-1 hold the kept ones.
 */
int oracle_permute(const int32_t *idx, int T, int k, int E, int32_t *perm, int32_t *off,
                   int32_t *inv)
{
    const int n = T * k;
    for (int e = 0; e <= E; e++) off[e] = 0;
    for (int a = 0; a < n; a++) {
        if (idx[a] == -1) continue;                 /* dropped by top-p: no row */
        if (idx[a] < 0 || idx[a] >= E) return -1;
        off[idx[a] + 1]++;
    }
    for (int e = 0; e < E; e++) off[e + 1] += off[e];
    int32_t *fill = malloc(sizeof(int32_t) * (E > 0 ? E : 1));
    if (!fill) return -2;
    for (int e = 0; e < E; e++) fill[e] = off[e];
    for (int a = 0; a < n; a++) {
        if (idx[a] < 0) { inv[a] = -1; continue; }
        int row = fill[idx[a]]++;
        perm[row] = a;
        inv[a] = row;
    }
    free(fill);
    return 0;
}

/* ---------------------------------------------------------------- MTP draft verification
 * GeekNews #31297, implemented features: the multi-token-prediction head
 * drafts tokens, the main model verifies them in one batched forward, and
 * rejection sampling keeps sampled output lossless; useful options: --temp T
 * (0 = greedy).  The yodev.dev page: greedy output is identical to plain
 * greedy decoding.
 * reading: the pages name rejection sampling but not its rule; the rule
 * taken is speculative sampling (Leviathan, Kalman & Matias, ICML 2023;
 * Chen et al. 2023): draft x_i, drawn from q_i, is kept when
 * u_i * q_i(x_i) < p_i(x_i); at the first refusal the emitted token is drawn
 * from max(0, p_i - q_i) renormalised (from p_i itself if that has no mass);
 * when every draft is kept it is drawn from p_D.  p and q are the softmax
 * of the logits divided by the temperature; nucleus filtering is not
 * applied.  Draws use inverse CDFs in ascending token order with the given
 * uniforms; greedy (tau = 0) keeps drafts while they equal the target's
 * argmax (lowest index on ties) and emits the argmax at the first mismatch. */

/* softmax(z / tau) of one row into out[V], fp64, max subtracted */
static void softmax_row(const float *z, int V, double tau, double *out)
{
    float m = z[0];
    for (int x = 1; x < V; x++) if (z[x] > m) m = z[x];
    double s = 0.0;
    for (int x = 0; x < V; x++) {
        out[x] = exp(((double)z[x] - (double)m) / tau);
        s += out[x];
    }
    for (int x = 0; x < V; x++) out[x] /= s;
}

static int argmax_row(const float *z, int V)
{
    int a = 0;
    for (int x = 1; x < V; x++) if (z[x] > z[a]) a = x;
    return a;
}

/* smallest x whose cumulative weight exceeds u * (total weight); margin =
 * distance of the target from the nearest cumulative boundary, relative to
 * the total */
static int inverse_cdf(const double *w, int V, double u, double *margin)
{
    double W = 0.0;
    for (int x = 0; x < V; x++) W += w[x];
    const double t = u * W;
    double c = 0.0;
    int last = -1;
    for (int x = 0; x < V; x++) {
        if (w[x] <= 0.0) continue;
        const double c0 = c;
        c += w[x];
        last = x;
        if (c > t) {
            double m = (t - c0 < c - t) ? t - c0 : c - t;
            if (margin) *margin = m / W;
            return x;
        }
    }
    if (margin) *margin = 0.0;  /* rounding left t at or above the total */
    return last;
}

int oracle_mtp_accept(int B, int D, int V, const int32_t *draft, const float *p_logits,
                      const float *q_logits, double tau, const double *u, int32_t *n_acc,
                      int32_t *next, double *margins)
{
    if (B < 0 || D < 0 || V < 1 || tau < 0.0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (int b = 0; b < B; b++) {
        const int32_t *dr = draft + (size_t)b * D;
        const float *pb = p_logits + (size_t)b * (D + 1) * V;
        const float *qb = q_logits + (size_t)b * D * V;
        const double *ub = u + (size_t)b * (D + 1);
        double mg = 1.0;
        int n = D, nx = -1;
        if (tau == 0.0) {
            for (int i = 0; i < D; i++) {
                const int a = argmax_row(pb + (size_t)i * V, V);
                if (a != dr[i]) { n = i; nx = a; break; }
            }
            if (nx < 0) nx = argmax_row(pb + (size_t)D * V, V);
        } else {
            double *P = malloc(sizeof(double) * V), *Q = malloc(sizeof(double) * V);
            if (!P || !Q) { bad = 1; free(P); free(Q); continue; }
            for (int i = 0; i < D && nx < 0; i++) {
                const int x = dr[i];
                if (x < 0 || x >= V) { bad = 1; break; }
                softmax_row(pb + (size_t)i * V, V, tau, P);
                softmax_row(qb + (size_t)i * V, V, tau, Q);
                const double lhs = ub[i] * Q[x], rhs = P[x];
                const double m = fabs(rhs - lhs) / (rhs > lhs ? rhs : lhs > 0.0 ? lhs : 1.0);
                if (m < mg) mg = m;
                if (lhs < rhs) continue;  /* kept */
                n = i;
                double R = 0.0;
                for (int y = 0; y < V; y++) {
                    Q[y] = P[y] > Q[y] ? P[y] - Q[y] : 0.0;  /* the residual, in place */
                    R += Q[y];
                }
                double m2;
                nx = inverse_cdf(R > 0.0 ? Q : P, V, ub[D], &m2);
                if (m2 < mg) mg = m2;
            }
            if (nx < 0 && !bad) {
                double m2;
                softmax_row(pb + (size_t)D * V, V, tau, P);
                nx = inverse_cdf(P, V, ub[D], &m2);
                if (m2 < mg) mg = m2;
            }
            free(P);
            free(Q);
        }
        n_acc[b] = n;
        next[b] = nx;
        if (margins) margins[b] = mg;
    }
    return bad ? -2 : 0;
}
