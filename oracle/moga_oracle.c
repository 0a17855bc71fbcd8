/*
 * CPU oracle for the MoGA + STGA forward path.  TEST INFRASTRUCTURE ONLY:
 * only the tests, the package smoke check and the benchmark's CPU-baseline leg
 * may load or call it.  It shares no code, header, table or helper with the
 * HIP library, and the HIP library never calls it.
 *
 * Everything here is the plain definition written out, in fp64, one query row
 * at a time.  Page citations use the page's site and section:
 *   [N]  papernotes.org ICLR 2026 note "MoGA: Mixture-of-Groups Attention for
 *        End-to-End Long Video Generation", section 方法详解 / 关键设计 1-4.
 *   [T]  jxzklqfsx.com Chinese translation of the paper, section 方法
 *        (混合分組注意力, 組平衡損失, 時空分組注意力).
 *   [B]  xugj520.cn blog on MoGA, §2.2-2.3 (router), §3.2 (STGA boundary
 *        frames), §9 (augment_kv=2).
 * Readings where the pages are silent are marked READING and listed with the
 * design notes.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC moga_oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Router  ([N] key design 1; [B] §2.3)                                       */
/*   r = x W (linear, no bias); p(i|x) = softmax(r)_i; g(x) = argmax_i p(i|x) */
/* READING: the argmax is taken over the logits (softmax is monotone), the    */
/* first maximum wins on an exact tie.  pin[t] >= 0 forces g(t) = pin[t].     */
/* gap[t] = top-1 minus top-2 logit (INFINITY when M = 1).                    */
/* ------------------------------------------------------------------------- */
int oracle_route(const float *x, const float *w, int64_t n, int d, int m,
                 const int32_t *pin, int32_t *group_id, double *p_sel, double *gap,
                 double *prob_sum, int64_t *counts, double *probs /* NULL or [n][m] */)
{
    if (n < 0 || d < 1 || m < 1 || m > 256) return -1;
    double *p_all = probs ? probs : (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * m);
    if (!p_all) return -2;

#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        double r[256];
        double rmax = -INFINITY, r2 = -INFINITY;
        int best = 0;
        for (int i = 0; i < m; ++i) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j)
                acc += (double)x[t * (int64_t)d + j] * (double)w[(int64_t)j * m + i];
            r[i] = acc;
        }
        for (int i = 0; i < m; ++i) {
            if (r[i] > rmax) { r2 = rmax; rmax = r[i]; best = i; }
            else if (r[i] > r2) { r2 = r[i]; }
        }
        double z = 0.0;
        for (int i = 0; i < m; ++i) z += exp(r[i] - rmax);
        for (int i = 0; i < m; ++i) p_all[t * (int64_t)m + i] = exp(r[i] - rmax) / z;
        int g = (pin && pin[t] >= 0) ? pin[t] : best;
        group_id[t] = g;
        p_sel[t] = p_all[t * (int64_t)m + g];
        gap[t] = (m == 1) ? INFINITY : rmax - r2;
    }
    for (int i = 0; i < m; ++i) { prob_sum[i] = 0.0; counts[i] = 0; }
    for (int64_t t = 0; t < n; ++t) {
        for (int i = 0; i < m; ++i) prob_sum[i] += p_all[t * (int64_t)m + i];
        counts[group_id[t]] += 1;
    }
    if (!probs) free(p_all);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Group boundaries and the permutation ([N] key design 2)                    */
/*   n_i = #{t : g(t) = i};  cu[0] = 0, cu[i+1] = cu[i] + n_i;                */
/*   perm lists group 0's tokens, then group 1's, ... each in ascending t.    */
/* READING: ascending token order inside a group and ascending group id.      */
/* ------------------------------------------------------------------------- */
int oracle_groups(const int32_t *group_id, int64_t n, int m, int64_t *cu, int64_t *perm)
{
    if (n < 0 || m < 1) return -1;
    int64_t j = 0;
    cu[0] = 0;
    for (int i = 0; i < m; ++i) {
        for (int64_t t = 0; t < n; ++t)
            if (group_id[t] == i) perm[j++] = t;
        cu[i + 1] = j;
    }
    return j == n ? 0 : -3; /* an id outside [0, m) leaves perm short */
}

/* ------------------------------------------------------------------------- */
/* Group-balancing loss ([N] key design 3)                                    */
/*   F_i = n_i / N;  P_i = mean over all tokens of p(i|x);                    */
/*   L_gb = alpha * M * sum_i F_i P_i.                                        */
/* READING: P_i averages p(i|x) over every token (the MoE load-balancing     */
/* convention the pages say the loss is borrowed from).                       */
/* ------------------------------------------------------------------------- */
double oracle_balance_loss(const int64_t *counts, const double *prob_sum, int64_t n, int m,
                           double alpha, double *F, double *P)
{
    double acc = 0.0;
    for (int i = 0; i < m; ++i) {
        double f = (double)counts[i] / (double)n;
        double p = prob_sum[i] / (double)n;
        if (F) F[i] = f;
        if (P) P[i] = p;
        acc += f * p;
    }
    return alpha * (double)m * acc;
}

/* ------------------------------------------------------------------------- */
/* One attention row: out = sum_u softmax_u(scale <q, k_u>) v_u over the key   */
/* list, in fp64, max-subtracted.                                              */
/* ------------------------------------------------------------------------- */
static void attend_row(const float *qrow, const float *kh, const float *vh, int hd,
                       const int64_t *keys, int64_t nk, double scale, double *s, double *out)
{
    double smax = -INFINITY;
    for (int64_t a = 0; a < nk; ++a) {
        const float *kr = kh + keys[a] * (int64_t)hd;
        double acc = 0.0;
        for (int c = 0; c < hd; ++c) acc += (double)qrow[c] * (double)kr[c];
        s[a] = scale * acc;
        if (s[a] > smax) smax = s[a];
    }
    double z = 0.0;
    for (int64_t a = 0; a < nk; ++a) { s[a] = exp(s[a] - smax); z += s[a]; }
    for (int c = 0; c < hd; ++c) out[c] = 0.0;
    for (int64_t a = 0; a < nk; ++a) {
        const float *vr = vh + keys[a] * (int64_t)hd;
        double wgt = s[a] / z;
        for (int c = 0; c < hd; ++c) out[c] += wgt * (double)vr[c];
    }
}

/* ------------------------------------------------------------------------- */
/* MoGA attention rows ([N] key design 1)                                     */
/*   MoGA(x_t) = p(g(t)|x_t) * SA(q_t, K_{g(t)}, V_{g(t)})                    */
/* with the key set {u : g(u) = g(t)}.  q/k/v hold n_heads_in heads, each      */
/* [n][hd]; row r asks for head rows_h[r] (an index into those), token        */
/* rows_t[r].  p_sel NULL means no probability scale.  Returns the number of   */
/* (query, key) pairs evaluated, or a negative value on bad arguments.         */
/* ------------------------------------------------------------------------- */
int64_t oracle_moga_attn(const float *q, const float *k, const float *v, int64_t n, int hd,
                         const int32_t *group_id, int m, const double *p_sel, double scale,
                         int64_t n_rows, const int32_t *rows_h, const int64_t *rows_t, double *out)
{
    if (n < 1 || hd < 1 || m < 1) return -1;
    int64_t *cnt = (int64_t *)calloc((size_t)m + 1, sizeof(int64_t));
    int64_t *members = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    if (!cnt || !members) { free(cnt); free(members); return -2; }
    /* member lists of every group, ascending token order */
    int64_t j = 0;
    for (int i = 0; i < m; ++i) {
        cnt[i] = j;
        for (int64_t t = 0; t < n; ++t)
            if (group_id[t] == i) members[j++] = t;
    }
    cnt[m] = j;
    int64_t pairs = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : pairs)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t t = rows_t[r];
        int g = group_id[t];
        int64_t nk = cnt[g + 1] - cnt[g];
        double *s = (double *)malloc(sizeof(double) * (size_t)nk);
        const int64_t hoff = (int64_t)rows_h[r] * n * hd;
        attend_row(q + hoff + t * hd, k + hoff, v + hoff, hd, members + cnt[g], nk, scale, s,
                   out + r * (int64_t)hd);
        double ps = p_sel ? p_sel[t] : 1.0;
        for (int c = 0; c < hd; ++c) out[r * (int64_t)hd + c] *= ps;
        pairs += nk;
        free(s);
    }
    free(cnt);
    free(members);
    return pairs;
}

/* ------------------------------------------------------------------------- */
/* STGA key sets ([N] key design 4; [T] 時空分組注意力; [B] §3.2, §9)           */
/* Token t sits in frame f = t / (H W) at (y, x), frame-major (READING).      */
/* Temporal groups: same shot s, same chunk c = (f - start_s) / T (chunks      */
/* start at each shot's first frame; a short last chunk is its own group,     */
/* READING), same spatial window (y / win_h, x / win_w).  Keys and values     */
/* (never queries) of the FIRST chunk of shot s > 0 also take the last `aug`   */
/* frames of shot s-1, and those of the LAST chunk of shot s < S-1 the first   */
/* `aug` frames of shot s+1, same window, clipped to the neighbour shot        */
/* (READING: only chunks that touch a shot boundary are augmented).           */
/* Per-frame groups: every token of frame f.                                  */
/* Fills keys[] and returns their count.                                       */
/* ------------------------------------------------------------------------- */
typedef struct {
    int frames, height, width, n_shots, win_h, win_w, t_group, aug;
    const int32_t *shot_start;
} oracle_grid;

static int64_t stga_keys(const oracle_grid *G, int mode, int64_t t, int64_t *keys)
{
    const int64_t hw = (int64_t)G->height * G->width;
    const int f = (int)(t / hw);
    const int y = (int)((t % hw) / G->width);
    const int x = (int)(t % G->width);
    int64_t nk = 0;
    if (mode == 1) { /* per-frame group */
        for (int64_t u = 0; u < hw; ++u) keys[nk++] = (int64_t)f * hw + u;
        return nk;
    }
    int s = 0;
    while (s + 1 < G->n_shots && G->shot_start[s + 1] <= f) ++s;
    const int s0 = G->shot_start[s], s1 = G->shot_start[s + 1];
    const int c = (f - s0) / G->t_group;
    const int n_chunks = (s1 - s0 + G->t_group - 1) / G->t_group;
    const int y0 = (y / G->win_h) * G->win_h, x0 = (x / G->win_w) * G->win_w;
    int lo = s0 + c * G->t_group;
    int hi = lo + G->t_group < s1 ? lo + G->t_group : s1;
    /* frame ranges: [a0,a1) borrowed from the previous shot, [lo,hi) own, [b0,b1) next shot */
    int a0 = lo, a1 = lo, b0 = hi, b1 = hi;
    if (c == 0 && s > 0) {
        int prev0 = G->shot_start[s - 1];
        a0 = s0 - G->aug < prev0 ? prev0 : s0 - G->aug;
        a1 = s0;
    }
    if (c == n_chunks - 1 && s + 1 < G->n_shots) {
        int next1 = G->shot_start[s + 2];
        b0 = s1;
        b1 = s1 + G->aug > next1 ? next1 : s1 + G->aug;
    }
    int ranges[3][2] = {{a0, a1}, {lo, hi}, {b0, b1}};
    for (int rg = 0; rg < 3; ++rg)
        for (int ff = ranges[rg][0]; ff < ranges[rg][1]; ++ff)
            for (int yy = y0; yy < y0 + G->win_h; ++yy)
                for (int xx = x0; xx < x0 + G->win_w; ++xx)
                    keys[nk++] = (int64_t)ff * hw + (int64_t)yy * G->width + xx;
    return nk;
}

static int grid_ok(const oracle_grid *G)
{
    if (G->frames < 1 || G->height < 1 || G->width < 1 || G->n_shots < 1) return 0;
    if (G->win_h < 1 || G->win_w < 1 || G->height % G->win_h || G->width % G->win_w) return 0;
    if (G->t_group < 1 || G->aug < 0) return 0;
    if (G->shot_start[0] != 0 || G->shot_start[G->n_shots] != G->frames) return 0;
    for (int s = 0; s < G->n_shots; ++s)
        if (G->shot_start[s + 1] <= G->shot_start[s]) return 0;
    return 1;
}

/* STGA attention rows; mode 0 = temporal groups, 1 = per-frame groups.        */
int64_t oracle_stga_attn(const float *q, const float *k, const float *v, int hd, int frames,
                         int height, int width, int n_shots, const int32_t *shot_start,
                         int win_h, int win_w, int t_group, int aug, int mode, double scale,
                         int64_t n_rows, const int32_t *rows_h, const int64_t *rows_t,
                         double *out)
{
    oracle_grid G = {frames, height, width, n_shots, win_h, win_w, t_group, aug, shot_start};
    if (!grid_ok(&G) || hd < 1) return -1;
    const int64_t n = (int64_t)frames * height * width;
    const int64_t max_keys = (int64_t)height * width * (t_group + 2 * aug) + (int64_t)height * width;
    int64_t pairs = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(+ : pairs)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)max_keys);
        double *s = (double *)malloc(sizeof(double) * (size_t)max_keys);
        int64_t t = rows_t[r];
        int64_t nk = stga_keys(&G, mode, t, keys);
        const int64_t hoff = (int64_t)rows_h[r] * n * hd;
        attend_row(q + hoff + t * hd, k + hoff, v + hoff, hd, keys, nk, scale, s,
                   out + r * (int64_t)hd);
        pairs += nk;
        free(keys);
        free(s);
    }
    return pairs;
}

/* Number of (query, key) pairs of one head: the sum over tokens of the key-set size. */
int64_t oracle_stga_pairs(int frames, int height, int width, int n_shots,
                          const int32_t *shot_start, int win_h, int win_w, int t_group, int aug,
                          int mode)
{
    oracle_grid G = {frames, height, width, n_shots, win_h, win_w, t_group, aug, shot_start};
    if (!grid_ok(&G)) return -1;
    const int64_t n = (int64_t)frames * height * width;
    const int64_t max_keys = (int64_t)height * width * (t_group + 2 * aug) + (int64_t)height * width;
    int64_t pairs = 0;
#pragma omp parallel for schedule(static) reduction(+ : pairs)
    for (int64_t t = 0; t < n; ++t) {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)max_keys);
        pairs += stga_keys(&G, mode, t, keys);
        free(keys);
    }
    return pairs;
}

/* Key list of one token (for tests of the grouping itself). */
int64_t oracle_stga_key_list(int frames, int height, int width, int n_shots,
                             const int32_t *shot_start, int win_h, int win_w, int t_group,
                             int aug, int mode, int64_t t, int64_t *keys)
{
    oracle_grid G = {frames, height, width, n_shots, win_h, win_w, t_group, aug, shot_start};
    if (!grid_ok(&G)) return -1;
    return stga_keys(&G, mode, t, keys);
}

/* ------------------------------------------------------------------------- */
/* Variable-length segment attention ([N] key design 2: the grouped rows are   */
/* handed to a varlen attention call described by per-segment offsets).        */
/* Query row i of segment s (cu_q[s] <= i < cu_q[s+1]) attends to the key rows */
/* [cu_k[s], cu_k[s+1]).  READING: a segment with no keys yields zeros.        */
/* q holds [heads][len_q][hd], k and v [heads][len_k][hd].  Rows that belong   */
/* to no segment return -1 in seg_of_row and are left as zeros.                */
/* ------------------------------------------------------------------------- */
int64_t oracle_varlen_attn(const float *q, const float *k, const float *v, int64_t len_q,
                           int64_t len_k, int hd, int n_seg, const int64_t *cu_q,
                           const int64_t *cu_k, const double *row_scale, double scale,
                           int64_t n_rows, const int32_t *rows_h, const int64_t *rows_i,
                           double *out)
{
    if (hd < 1 || n_seg < 1) return -1;
    for (int s = 0; s < n_seg; ++s)
        if (cu_q[s] > cu_q[s + 1] || cu_k[s] > cu_k[s + 1] || cu_q[s] < 0 || cu_k[s] < 0 ||
            cu_q[s + 1] > len_q || cu_k[s + 1] > len_k)
            return -1;
    int64_t pairs = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(+ : pairs)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t i = rows_i[r];
        double *o = out + r * (int64_t)hd;
        for (int c = 0; c < hd; ++c) o[c] = 0.0;
        int seg = -1;
        for (int s = 0; s < n_seg; ++s)
            if (cu_q[s] <= i && i < cu_q[s + 1]) { seg = s; break; }
        if (seg < 0) continue;
        const int64_t nk = cu_k[seg + 1] - cu_k[seg];
        if (nk == 0) continue;
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)nk);
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)nk);
        for (int64_t a = 0; a < nk; ++a) keys[a] = cu_k[seg] + a;
        const int64_t h = rows_h[r];
        attend_row(q + (h * len_q + i) * hd, k + h * len_k * hd, v + h * len_k * hd, hd, keys, nk,
                   scale, s_buf, o);
        if (row_scale)
            for (int c = 0; c < hd; ++c) o[c] *= row_scale[i];
        pairs += nk;
        free(keys);
        free(s_buf);
    }
    return pairs;
}

/* ========================================================================= */
/* Backward of the MoGA forward ([N] key design 1: the router is made          */
/* differentiable through the p(g(x)|x) factor; key design 3: L_gb).           */
/*                                                                             */
/* With the routing g held fixed (the argmax and the counts n_i, hence F_i,    */
/* are piecewise constant in x), for upstream gradients d_out of              */
/* out_t = p_t * O'_t (p_t = p(g_t|x_t), O'_t = SA(q_t, K_G, V_G), per head)   */
/* and d_loss of L_gb:                                                         */
/*   dO'_t = p_t d_out_t;  P_tu = softmax_u(scale <q_t,k_u>) over u in G(t)    */
/*   D_t = <dO'_t, O'_t>;  dP_tu = <dO'_t, v_u>;  dS_tu = P_tu (dP_tu - D_t)   */
/*   dq_t = scale sum_u dS_tu k_u;  dk_u = scale sum_t dS_tu q_t;              */
/*   dv_u = sum_t P_tu dO'_t                                                   */
/*   dp_t = sum_heads <d_out_t, O'_t>                                          */
/*   a_ti = [i = g_t] dp_t + d_loss * alpha * M * F_i / n                      */
/*          (dL_gb / dp(i|x_t), since P_i = (1/n) sum_t p(i|x_t))              */
/*   dr_ti = p_ti (a_ti - sum_j a_tj p_tj)   (softmax backward)                */
/*   dW = x^T dr;  dx = dr W^T                                                 */
/* lse_t = log sum_u exp(scale <q_t,k_u>) per head (the softmax normaliser).   */
/* All of q, k, v, d_out hold n_heads heads of [n][hd].  Plain loops, fp64.    */
/* ========================================================================= */
static void group_members(const int32_t *group_id, int64_t n, int m, int64_t *cnt,
                          int64_t *members)
{
    int64_t j = 0;
    for (int i = 0; i < m; ++i) {
        cnt[i] = j;
        for (int64_t t = 0; t < n; ++t)
            if (group_id[t] == i) members[j++] = t;
    }
    cnt[m] = j;
}

/* router probabilities p [n][m] in fp64 */
static void router_probs(const float *x, const float *w, int64_t n, int d, int m, double *p)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        double *pt = p + t * m;
        double mx = -INFINITY;
        for (int i = 0; i < m; ++i) {
            double r = 0.0;
            for (int c = 0; c < d; ++c) r += (double)x[t * d + c] * (double)w[(int64_t)c * m + i];
            pt[i] = r;
            if (r > mx) mx = r;
        }
        double z = 0.0;
        for (int i = 0; i < m; ++i) { pt[i] = exp(pt[i] - mx); z += pt[i]; }
        for (int i = 0; i < m; ++i) pt[i] /= z;
    }
}

/* router part for one token: a_ti, then dr_t (softmax backward) and dx_t = dr_t W^T, from its
 * probabilities p_t [m] over all groups, its group g, dp_t and F [m] */
static void router_bwd_token(const double *pt, int g, double dpt, const double *F, int m, int d,
                             const float *w, int64_t n, double d_loss, double alpha,
                             double *dr_t, double *dx_t)
{
    double a[256], dot = 0.0;
    for (int i = 0; i < m; ++i) {
        a[i] = (i == g ? dpt : 0.0) + d_loss * alpha * (double)m * F[i] / (double)n;
        dot += a[i] * pt[i];
    }
    for (int i = 0; i < m; ++i) dr_t[i] = pt[i] * (a[i] - dot);
    for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int i = 0; i < m; ++i) acc += dr_t[i] * (double)w[(int64_t)c * m + i];
        dx_t[c] = acc;
    }
}

/* scores, probabilities and O' of one query row against a key list; returns lse */
static double softmax_row(const float *qrow, const float *kh, const float *vh, int hd,
                          const int64_t *keys, int64_t nk, double scale, double *P, double *o)
{
    double smax = -INFINITY;
    for (int64_t a = 0; a < nk; ++a) {
        const float *kr = kh + keys[a] * (int64_t)hd;
        double acc = 0.0;
        for (int c = 0; c < hd; ++c) acc += (double)qrow[c] * (double)kr[c];
        P[a] = scale * acc;
        if (P[a] > smax) smax = P[a];
    }
    double z = 0.0;
    for (int64_t a = 0; a < nk; ++a) { P[a] = exp(P[a] - smax); z += P[a]; }
    for (int c = 0; c < hd; ++c) o[c] = 0.0;
    for (int64_t a = 0; a < nk; ++a) {
        P[a] /= z;
        const float *vr = vh + keys[a] * (int64_t)hd;
        for (int c = 0; c < hd; ++c) o[c] += P[a] * (double)vr[c];
    }
    return smax + log(z);
}

int oracle_moga_backward(const float *x, const float *w, int64_t n, int d, int m, int n_heads,
                         int hd, const float *q, const float *k, const float *v,
                         const int32_t *group_id, const float *d_out, double d_loss,
                         double alpha, double scale, double *dq, double *dk, double *dv,
                         double *dx, double *dw, double *dp, double *lse)
{
    if (n < 1 || d < 1 || m < 1 || n_heads < 1 || hd < 1) return -1;
    for (int64_t t = 0; t < n; ++t)
        if (group_id[t] < 0 || group_id[t] >= m) return -3;
    int64_t *cnt = (int64_t *)calloc((size_t)m + 1, sizeof(int64_t));
    int64_t *members = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    double *p = (double *)malloc(sizeof(double) * (size_t)n * m);
    double *dpart = (double *)calloc((size_t)n * n_heads, sizeof(double)); /* <d_out, O'> per head */
    if (!cnt || !members || !p || !dpart) { free(cnt); free(members); free(p); free(dpart); return -2; }
    group_members(group_id, n, m, cnt, members);
    router_probs(x, w, n, d, m, p);
    const size_t E = (size_t)n_heads * n * hd;
    memset(dq, 0, sizeof(double) * E);
    memset(dk, 0, sizeof(double) * E);
    memset(dv, 0, sizeof(double) * E);

    /* attention part: one (head, group) at a time; a group's rows only touch its own keys */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t hg = 0; hg < (int64_t)n_heads * m; ++hg) {
        const int h = (int)(hg / m), g = (int)(hg % m);
        const int64_t nk = cnt[g + 1] - cnt[g];
        if (nk == 0) continue;
        const int64_t *keys = members + cnt[g];
        const int64_t hoff = (int64_t)h * n * hd;
        const float *qh = q + hoff, *kh = k + hoff, *vh = v + hoff, *gh = d_out + hoff;
        double *P = (double *)malloc(sizeof(double) * (size_t)nk);
        double *o = (double *)malloc(sizeof(double) * (size_t)hd);
        double *dO = (double *)malloc(sizeof(double) * (size_t)hd);
        for (int64_t a = 0; a < nk; ++a) {
            const int64_t t = keys[a];
            double l = softmax_row(qh + t * hd, kh, vh, hd, keys, nk, scale, P, o);
            if (lse) lse[(int64_t)h * n + t] = l;
            const double pt = p[t * m + g];
            double Dt = 0.0, part = 0.0;
            for (int c = 0; c < hd; ++c) {
                dO[c] = pt * (double)gh[t * hd + c];
                Dt += dO[c] * o[c];
                part += (double)gh[t * hd + c] * o[c];
            }
            dpart[t * n_heads + h] = part;
            for (int64_t b = 0; b < nk; ++b) {
                const int64_t u = keys[b];
                double dP = 0.0;
                for (int c = 0; c < hd; ++c) dP += dO[c] * (double)vh[u * hd + c];
                const double dS = P[b] * (dP - Dt);
                for (int c = 0; c < hd; ++c) {
                    dq[hoff + t * hd + c] += scale * dS * (double)kh[u * hd + c];
                    dk[hoff + u * hd + c] += scale * dS * (double)qh[t * hd + c];
                    dv[hoff + u * hd + c] += P[b] * dO[c];
                }
            }
        }
        free(P); free(o); free(dO);
    }

    /* router part */
    double *F = (double *)malloc(sizeof(double) * (size_t)m);
    double *dr = (double *)malloc(sizeof(double) * (size_t)n * m);
    for (int i = 0; i < m; ++i) F[i] = (double)(cnt[i + 1] - cnt[i]) / (double)n;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        double dpt = 0.0;
        for (int h = 0; h < n_heads; ++h) dpt += dpart[t * n_heads + h];
        if (dp) dp[t] = dpt;
        router_bwd_token(p + t * m, group_id[t], dpt, F, m, d, w, n, d_loss, alpha, dr + t * m,
                         dx + t * d);
    }
#pragma omp parallel for schedule(static)
    for (int c = 0; c < d; ++c)
        for (int i = 0; i < m; ++i) {
            double acc = 0.0;
            for (int64_t t = 0; t < n; ++t) acc += (double)x[t * d + c] * dr[t * m + i];
            dw[(int64_t)c * m + i] = acc;
        }
    free(F); free(dr); free(cnt); free(members); free(p); free(dpart);
    return 0;
}

/* dq (and D, lse) of selected rows only: row r is head rows_h[r] (an index into the heads of
 * q/k/v/d_out), token rows_t[r].  p_sel[t] = p(g_t|x_t).  Same definitions as above. */
int oracle_moga_dq_rows(const float *q, const float *k, const float *v, const float *d_out,
                        int64_t n, int hd, const int32_t *group_id, int m, const double *p_sel,
                        double scale, int64_t n_rows, const int32_t *rows_h,
                        const int64_t *rows_t, double *dq, double *D, double *lse)
{
    if (n < 1 || hd < 1 || m < 1) return -1;
    int64_t *cnt = (int64_t *)calloc((size_t)m + 1, sizeof(int64_t));
    int64_t *members = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    if (!cnt || !members) { free(cnt); free(members); return -2; }
    group_members(group_id, n, m, cnt, members);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t t = rows_t[r];
        const int g = group_id[t];
        const int64_t nk = cnt[g + 1] - cnt[g];
        const int64_t *keys = members + cnt[g];
        const int64_t hoff = (int64_t)rows_h[r] * n * hd;
        double *P = (double *)malloc(sizeof(double) * (size_t)nk);
        double *o = (double *)malloc(sizeof(double) * (size_t)hd);
        double *dO = (double *)malloc(sizeof(double) * (size_t)hd);
        double l = softmax_row(q + hoff + t * hd, k + hoff, v + hoff, hd, keys, nk, scale, P, o);
        double Dt = 0.0;
        for (int c = 0; c < hd; ++c) {
            dO[c] = p_sel[t] * (double)d_out[hoff + t * hd + c];
            Dt += dO[c] * o[c];
        }
        for (int c = 0; c < hd; ++c) dq[r * hd + c] = 0.0;
        for (int64_t b = 0; b < nk; ++b) {
            const int64_t u = keys[b];
            double dP = 0.0;
            for (int c = 0; c < hd; ++c) dP += dO[c] * (double)v[hoff + u * hd + c];
            const double dS = P[b] * (dP - Dt);
            for (int c = 0; c < hd; ++c) dq[r * hd + c] += scale * dS * (double)k[hoff + u * hd + c];
        }
        if (D) D[r] = Dt;
        if (lse) lse[r] = l;
        free(P); free(o); free(dO);
    }
    free(cnt); free(members);
    return 0;
}

/* The router part above for selected tokens only: x_rows [n_rows][d] are those tokens' router
 * inputs, g_rows their groups, dp_rows their dp_t; counts [m] and n are the whole problem's
 * (F_i = counts_i / n).  Writes dr [n_rows][m] and dx [n_rows][d]. */
int oracle_router_bwd_rows(const float *x_rows, const float *w, int64_t n_rows, int d, int m,
                           const int32_t *g_rows, const double *dp_rows, const int64_t *counts,
                           int64_t n, double d_loss, double alpha, double *dr, double *dx)
{
    if (n_rows < 0 || d < 1 || m < 1 || m > 256 || n < 1) return -1;
    double *p = (double *)malloc(sizeof(double) * (size_t)(n_rows > 0 ? n_rows : 1) * m);
    double *F = (double *)malloc(sizeof(double) * (size_t)m);
    if (!p || !F) { free(p); free(F); return -2; }
    router_probs(x_rows, w, n_rows, d, m, p);
    for (int i = 0; i < m; ++i) F[i] = (double)counts[i] / (double)n;
    for (int64_t r = 0; r < n_rows; ++r)
        router_bwd_token(p + r * m, g_rows[r], dp_rows[r], F, m, d, w, n, d_loss, alpha,
                         dr + r * m, dx + r * d);
    free(p); free(F);
    return 0;
}

/* dk and dv of selected KEY rows only: row r is head rows_h[r] (an index into the heads of
 * q/k/v/d_out), key token rows_t[r].  Same definitions as oracle_moga_backward: for a key u of
 * group G, dv_u = sum over the queries t of G of P_tu dO'_t and
 * dk_u = scale sum_t P_tu (dP_tu - D_t) q_t, with dO'_t = p_t d_out_t, dP_tu = <dO'_t, v_u>,
 * and P_tu, D_t = <dO'_t, O'_t> from each query's whole softmax row over G.  Every query of G
 * is needed, so the work per (head, group) is |G|^2 hd whatever the number of sampled keys. */
int oracle_moga_dkdv_rows(const float *q, const float *k, const float *v, const float *d_out,
                          int64_t n, int hd, const int32_t *group_id, int m,
                          const double *p_sel, double scale, int64_t n_rows,
                          const int32_t *rows_h, const int64_t *rows_t, double *dk, double *dv)
{
    if (n < 1 || hd < 1 || m < 1 || n_rows < 0) return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows_t[r] < 0 || rows_t[r] >= n || group_id[rows_t[r]] < 0 || group_id[rows_t[r]] >= m)
            return -3;
    int64_t *cnt = (int64_t *)calloc((size_t)m + 1, sizeof(int64_t));
    int64_t *members = (int64_t *)malloc(sizeof(int64_t) * (size_t)n);
    if (!cnt || !members) { free(cnt); free(members); return -2; }
    group_members(group_id, n, m, cnt, members);
    for (int64_t r = 0; r < n_rows * hd; ++r) { dk[r] = 0.0; dv[r] = 0.0; }
    int rc = 0;
    /* one (head, group) pair at a time: the softmax statistics of all its queries, then the
     * sampled keys of that pair */
    for (int64_t r0 = 0; r0 < n_rows && rc == 0; ++r0) {
        const int h = rows_h[r0], g = group_id[rows_t[r0]];
        int first = 1;
        for (int64_t r1 = 0; r1 < r0; ++r1)
            if (rows_h[r1] == h && group_id[rows_t[r1]] == g) { first = 0; break; }
        if (!first) continue;
        const int64_t nk = cnt[g + 1] - cnt[g];
        const int64_t *keys = members + cnt[g];
        const int64_t hoff = (int64_t)h * n * hd;
        double *lse = (double *)malloc(sizeof(double) * (size_t)nk);
        double *D = (double *)malloc(sizeof(double) * (size_t)nk);
        if (!lse || !D) { free(lse); free(D); rc = -2; break; }
#pragma omp parallel
        {
            double *P = (double *)malloc(sizeof(double) * (size_t)nk);
            double *o = (double *)malloc(sizeof(double) * (size_t)hd);
#pragma omp for schedule(dynamic, 16)
            for (int64_t a = 0; a < nk; ++a) {
                const int64_t t = keys[a];
                lse[a] = softmax_row(q + hoff + t * hd, k + hoff, v + hoff, hd, keys, nk, scale, P,
                                     o);
                double Dt = 0.0;
                for (int c = 0; c < hd; ++c)
                    Dt += p_sel[t] * (double)d_out[hoff + t * hd + c] * o[c];
                D[a] = Dt;
            }
            free(P);
            free(o);
        }
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = r0; r < n_rows; ++r) {
            if (rows_h[r] != h || group_id[rows_t[r]] != g) continue;
            const int64_t u = rows_t[r];
            const float *ku = k + hoff + u * hd, *vu = v + hoff + u * hd;
            for (int64_t a = 0; a < nk; ++a) {
                const int64_t t = keys[a];
                const float *qt = q + hoff + t * hd, *gt = d_out + hoff + t * hd;
                double s = 0.0, dP = 0.0;
                for (int c = 0; c < hd; ++c) {
                    s += (double)qt[c] * (double)ku[c];
                    dP += p_sel[t] * (double)gt[c] * (double)vu[c];
                }
                const double P = exp(scale * s - lse[a]);
                const double dS = P * (dP - D[a]);
                for (int c = 0; c < hd; ++c) {
                    dv[r * hd + c] += P * p_sel[t] * (double)gt[c];
                    dk[r * hd + c] += scale * dS * (double)qt[c];
                }
            }
        }
        free(lse);
        free(D);
    }
    free(cnt);
    free(members);
    return rc;
}

/* ========================================================================= */
/* Backward of one STGA branch ([N] key design 4; the branches enter the      */
/* layer output through the mean, so their upstream gradient is the mean's).  */
/* For O_t = softmax_u(scale <q_t, k_u>) v_u over the branch's key set of t  */
/* and J = sum_t <G_t, O_t> (G = d_out, per head):                            */
/*   P_tu = softmax over set(t);  D_t = <G_t, O_t>;  dP_tu = <G_t, v_u>;      */
/*   dS_tu = P_tu (dP_tu - D_t);  dq_t = scale sum_{u in set(t)} dS_tu k_u;   */
/*   dk_u = scale sum_{t : u in set(t)} dS_tu q_t;  dv_u = sum_t P_tu G_t.    */
/* A key can sit in several key sets (a boundary frame is borrowed by the     */
/* neighbouring shot's chunk), so dk, dv add over every query that uses it.   */
/* mode 0 = temporal groups, 1 = per-frame groups; tensors [n_heads][n][hd];  */
/* lse [n_heads][n] gets each query's log-normaliser.  Plain loops in fp64.   */
/* ========================================================================= */
int oracle_stga_backward(const float *q, const float *k, const float *v, const float *d_out,
                         int n_heads, int hd, int frames, int height, int width, int n_shots,
                         const int32_t *shot_start, int win_h, int win_w, int t_group, int aug,
                         int mode, double scale, double *dq, double *dk, double *dv, double *lse)
{
    oracle_grid G = {frames, height, width, n_shots, win_h, win_w, t_group, aug, shot_start};
    if (!grid_ok(&G) || hd < 1 || n_heads < 1) return -1;
    const int64_t n = (int64_t)frames * height * width;
    const int64_t max_keys = (int64_t)height * width * (t_group + 2 * aug) + (int64_t)height * width;
    const size_t E = (size_t)n_heads * n * hd;
    memset(dq, 0, sizeof(double) * E);
    memset(dk, 0, sizeof(double) * E);
    memset(dv, 0, sizeof(double) * E);
    /* one head per thread: keys of several queries meet in dk, dv */
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < n_heads; ++h) {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)max_keys);
        double *P = (double *)malloc(sizeof(double) * (size_t)max_keys);
        double *o = (double *)malloc(sizeof(double) * (size_t)hd);
        const int64_t hoff = (int64_t)h * n * hd;
        const float *qh = q + hoff, *kh = k + hoff, *vh = v + hoff, *gh = d_out + hoff;
        for (int64_t t = 0; t < n; ++t) {
            const int64_t nk = stga_keys(&G, mode, t, keys);
            const double l = softmax_row(qh + t * hd, kh, vh, hd, keys, nk, scale, P, o);
            if (lse) lse[(int64_t)h * n + t] = l;
            double Dt = 0.0;
            for (int c = 0; c < hd; ++c) Dt += (double)gh[t * hd + c] * o[c];
            for (int64_t b = 0; b < nk; ++b) {
                const int64_t u = keys[b];
                double dP = 0.0;
                for (int c = 0; c < hd; ++c) dP += (double)gh[t * hd + c] * (double)vh[u * hd + c];
                const double dS = P[b] * (dP - Dt);
                for (int c = 0; c < hd; ++c) {
                    dq[hoff + t * hd + c] += scale * dS * (double)kh[u * hd + c];
                    dk[hoff + u * hd + c] += scale * dS * (double)qh[t * hd + c];
                    dv[hoff + u * hd + c] += P[b] * (double)gh[t * hd + c];
                }
            }
        }
        free(keys); free(P); free(o);
    }
    return 0;
}

/* The same gradients for selected rows only (full-size tests): row r is head rows_h[r] (an
 * index into the heads of q/k/v/d_out), token rows_t[r]; dq and lse are that token's as a
 * query, dk and dv as a key.  The queries whose key set can hold key u lie in u's spatial
 * window (per-frame: u's frame) within t_group + aug frames of u; each candidate's key set is
 * built and searched for u, so the sum runs over exactly the queries that use u. */
int oracle_stga_bwd_rows(const float *q, const float *k, const float *v, const float *d_out,
                         int hd, int frames, int height, int width, int n_shots,
                         const int32_t *shot_start, int win_h, int win_w, int t_group, int aug,
                         int mode, double scale, int64_t n_rows, const int32_t *rows_h,
                         const int64_t *rows_t, double *dq, double *dk, double *dv, double *lse)
{
    oracle_grid G = {frames, height, width, n_shots, win_h, win_w, t_group, aug, shot_start};
    if (!grid_ok(&G) || hd < 1) return -1;
    const int64_t n = (int64_t)frames * height * width, hw = (int64_t)height * width;
    const int64_t max_keys = (int64_t)height * width * (t_group + 2 * aug) + (int64_t)height * width;
    int rc = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)max_keys);
        double *P = (double *)malloc(sizeof(double) * (size_t)max_keys);
        double *o = (double *)malloc(sizeof(double) * (size_t)hd);
        const int64_t hoff = (int64_t)rows_h[r] * n * hd;
        const float *qh = q + hoff, *kh = k + hoff, *vh = v + hoff, *gh = d_out + hoff;
        const int64_t u = rows_t[r];
        double *dqr = dq + r * hd, *dkr = dk + r * hd, *dvr = dv + r * hd;
        for (int c = 0; c < hd; ++c) { dqr[c] = 0.0; dkr[c] = 0.0; dvr[c] = 0.0; }
        /* as a query */
        {
            const int64_t nk = stga_keys(&G, mode, u, keys);
            const double l = softmax_row(qh + u * hd, kh, vh, hd, keys, nk, scale, P, o);
            if (lse) lse[r] = l;
            double Dt = 0.0;
            for (int c = 0; c < hd; ++c) Dt += (double)gh[u * hd + c] * o[c];
            for (int64_t b = 0; b < nk; ++b) {
                double dP = 0.0;
                for (int c = 0; c < hd; ++c) dP += (double)gh[u * hd + c] * (double)vh[keys[b] * hd + c];
                const double dS = P[b] * (dP - Dt);
                for (int c = 0; c < hd; ++c) dqr[c] += scale * dS * (double)kh[keys[b] * hd + c];
            }
        }
        /* as a key: every query t whose key set holds u */
        const int fu = (int)(u / hw);
        const int yu = (int)((u % hw) / width), xu = (int)(u % width);
        const int span = mode == 1 ? 0 : t_group + aug;
        const int f_lo = fu - span < 0 ? 0 : fu - span;
        const int f_hi = fu + span >= frames ? frames - 1 : fu + span;
        const int y0 = mode == 1 ? 0 : (yu / win_h) * win_h, y1 = mode == 1 ? height : y0 + win_h;
        const int x0 = mode == 1 ? 0 : (xu / win_w) * win_w, x1 = mode == 1 ? width : x0 + win_w;
        for (int f = f_lo; f <= f_hi; ++f)
            for (int y = y0; y < y1; ++y)
                for (int x = x0; x < x1; ++x) {
                    const int64_t t = (int64_t)f * hw + (int64_t)y * width + x;
                    const int64_t nk = stga_keys(&G, mode, t, keys);
                    int64_t bu = -1;
                    for (int64_t b = 0; b < nk; ++b)
                        if (keys[b] == u) { bu = b; break; }
                    if (bu < 0) continue;
                    softmax_row(qh + t * hd, kh, vh, hd, keys, nk, scale, P, o);
                    double Dt = 0.0, dP = 0.0;
                    for (int c = 0; c < hd; ++c) {
                        Dt += (double)gh[t * hd + c] * o[c];
                        dP += (double)gh[t * hd + c] * (double)vh[u * hd + c];
                    }
                    const double dS = P[bu] * (dP - Dt);
                    for (int c = 0; c < hd; ++c) {
                        dkr[c] += scale * dS * (double)qh[t * hd + c];
                        dvr[c] += P[bu] * (double)gh[t * hd + c];
                    }
                }
        free(keys); free(P); free(o);
    }
    return rc;
}
