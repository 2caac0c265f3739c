/*
 * Plain fp64 CPU oracle for 3D-RoPE exact self-attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header, table or constant with the
 * HIP library.
 *
 * What it computes follows the ReGenVC pages (arXiv 2607.28144):
 *  - the decoder is a diffusion transformer whose attention runs over the
 *    video-latent token sequence, split into heads (blog summary,
 *    "Methodology - deep read", the USP paragraph on Ulysses and Ring);
 *  - the sequence-parallel scheme keeps attention exact and numerically
 *    equivalent (blog summary, "Technical innovations", USP bullet), so the
 *    target is exact softmax(Q K^T * scale) V over all keys, non-causal;
 *  - FlashAttention and FlashAttention-2 are the cited attention kernels
 *    (index page, "Builds on"): both compute that same exact result.
 * The pages name no rotary convention; the readings taken here are:
 *  - token n of a T x H x W latent grid sits at t = n / (H W),
 *    h = (n / W) mod H, w = n mod W (row-major, t slowest), origin 0;
 *  - the head_dim/2 rotation pairs are split into three consecutive chunks
 *    of pairs_t, pairs_h, pairs_w pairs for the t, h and w axes;
 *  - pair i of axis a with local index j rotates by pos_a * base^(-j/P_a),
 *    each axis being an independent 1D rotary ladder of its own width;
 *  - the pair is the adjacent interleaved couple (x[2i], x[2i+1]), rotated
 *    counter-clockwise, i.e. multiplied by exp(+i phi) as a complex number;
 *  - Q and K are rotated, V is not.
 *
 * Every loop below is the definition written out, in double precision, with
 * no blocking and no online softmax.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Latent coordinates of token n (row-major, t slowest). */
void oracle_token_coords(int64_t n, int64_t grid_h, int64_t grid_w,
                         int64_t *t, int64_t *h, int64_t *w) {
    *w = n % grid_w;
    *h = (n / grid_w) % grid_h;
    *t = n / (grid_w * grid_h);
}

/* Rotate one head_dim vector x at position pos[3] = (t, h, w) into y. */
static void rope_row(const double *x, double *y, int head_dim,
                     const double pos[3], const int pairs[3], double base) {
    int npairs = head_dim / 2;
    for (int i = 0; i < npairs; ++i) {
        int axis, j;
        if (i < pairs[0]) {
            axis = 0;
            j = i;
        } else if (i < pairs[0] + pairs[1]) {
            axis = 1;
            j = i - pairs[0];
        } else {
            axis = 2;
            j = i - pairs[0] - pairs[1];
        }
        double theta = pow(base, -(double)j / (double)pairs[axis]);
        double phi = pos[axis] * theta;
        double c = cos(phi), s = sin(phi);
        double a = x[2 * i], b = x[2 * i + 1];
        y[2 * i] = a * c - b * s;
        y[2 * i + 1] = a * s + b * c;
    }
}

static int pairs_ok(int head_dim, int pt, int ph, int pw) {
    return head_dim > 0 && head_dim % 2 == 0 && pt > 0 && ph > 0 && pw > 0 &&
           pt + ph + pw == head_dim / 2;
}

/*
 * Rotate rows of x [rows][head_dim] at explicit positions pos [rows][3]
 * (t, h, w; any real values). Returns 0, or -1 on a bad argument.
 */
int oracle_rope_positions(const double *x, double *y, int64_t rows,
                          int head_dim, const double *pos, int pairs_t,
                          int pairs_h, int pairs_w, double base) {
    if (!x || !y || !pos || rows < 0 || base <= 0.0 ||
        !pairs_ok(head_dim, pairs_t, pairs_h, pairs_w))
        return -1;
    int pairs[3] = {pairs_t, pairs_h, pairs_w};
    for (int64_t r = 0; r < rows; ++r)
        rope_row(x + r * head_dim, y + r * head_dim, head_dim, pos + 3 * r,
                 pairs, base);
    return 0;
}

/*
 * Rotate x [heads][T*H*W][head_dim] over the latent grid into y.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_rope_grid(const double *x, double *y, int heads, int head_dim,
                     int grid_t, int grid_h, int grid_w, int pairs_t,
                     int pairs_h, int pairs_w, double base) {
    if (!x || !y || heads < 1 || grid_t < 1 || grid_h < 1 || grid_w < 1 ||
        base <= 0.0 || !pairs_ok(head_dim, pairs_t, pairs_h, pairs_w))
        return -1;
    int64_t n_tokens = (int64_t)grid_t * grid_h * grid_w;
    int pairs[3] = {pairs_t, pairs_h, pairs_w};
#pragma omp parallel for collapse(2) schedule(static)
    for (int hd = 0; hd < heads; ++hd)
        for (int64_t n = 0; n < n_tokens; ++n) {
            int64_t t, h, w;
            oracle_token_coords(n, grid_h, grid_w, &t, &h, &w);
            double pos[3] = {(double)t, (double)h, (double)w};
            int64_t off = ((int64_t)hd * n_tokens + n) * head_dim;
            rope_row(x + off, y + off, head_dim, pos, pairs, base);
        }
    return 0;
}

/*
 * Exact softmax attention, optionally with the log-sum-exp of the scores.
 *   q : [heads][n_q][head_dim]     (any subset of query rows, already rotated)
 *   k : [heads][n_kv][head_dim]    v : [heads][n_kv][head_dim]
 *   o : [heads][n_q][head_dim]     lse : [heads][n_q] or NULL
 * For each (head, query row m): s_n = scale * <q_m, k_n> over all n_kv keys,
 * p_n = exp(s_n - max s) / sum exp(s - max s), o_m = sum_n p_n v_n and
 * lse_m = log sum_n exp(s_n) = max s + log sum exp(s - max s). The LSE is what
 * the Ring half of USP needs to combine attention over separate key chunks
 * exactly (blog summary, "Methodology - deep read", USP paragraph: Ring
 * passes key/value blocks around; "Technical innovations": the result stays
 * exact).
 * Returns 0, or -1 on a bad argument, -2 if memory runs out.
 */
int oracle_attention_lse(const double *q, const double *k, const double *v,
                         double *o, double *lse, int heads, int64_t n_q,
                         int64_t n_kv, int head_dim, double scale) {
    if (!q || !k || !v || !o || heads < 1 || n_q < 0 || n_kv < 1 ||
        head_dim < 1)
        return -1;
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)n_kv);
        double *acc = (double *)malloc(sizeof(double) * (size_t)head_dim);
        if (!s || !acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for collapse(2) schedule(dynamic, 4)
        for (int hd = 0; hd < heads; ++hd)
            for (int64_t m = 0; m < n_q; ++m) {
                if (!s || !acc) continue;
                const double *qm = q + ((int64_t)hd * n_q + m) * head_dim;
                const double *kh = k + (int64_t)hd * n_kv * head_dim;
                const double *vh = v + (int64_t)hd * n_kv * head_dim;
                double mx = -INFINITY;
                for (int64_t n = 0; n < n_kv; ++n) {
                    const double *kn = kh + n * head_dim;
                    double dot = 0.0;
                    for (int c = 0; c < head_dim; ++c) dot += qm[c] * kn[c];
                    s[n] = scale * dot;
                    if (s[n] > mx) mx = s[n];
                }
                double den = 0.0;
                for (int c = 0; c < head_dim; ++c) acc[c] = 0.0;
                for (int64_t n = 0; n < n_kv; ++n) {
                    double p = exp(s[n] - mx);
                    den += p;
                    const double *vn = vh + n * head_dim;
                    for (int c = 0; c < head_dim; ++c) acc[c] += p * vn[c];
                }
                double *om = o + ((int64_t)hd * n_q + m) * head_dim;
                for (int c = 0; c < head_dim; ++c) om[c] = acc[c] / den;
                if (lse) lse[(int64_t)hd * n_q + m] = mx + log(den);
            }
        free(s);
        free(acc);
    }
    return failed ? -2 : 0;
}

/* Exact softmax attention without the LSE (see oracle_attention_lse). */
int oracle_attention(const double *q, const double *k, const double *v,
                     double *o, int heads, int64_t n_q, int64_t n_kv,
                     int head_dim, double scale) {
    return oracle_attention_lse(q, k, v, o, NULL, heads, n_q, n_kv, head_dim,
                                scale);
}

/*
 * Combine attention results over disjoint key sets into the result over
 * their union. Part i holds o_i = sum_{n in K_i} e^{s_n} v_n / Z_i and
 * lse_i = log Z_i with Z_i = sum_{n in K_i} e^{s_n}; over the union,
 * Z = sum_i Z_i, so lse = log sum_i e^{lse_i} and o = sum_i (Z_i / Z) o_i.
 * A part with lse_i = -inf (no keys) has weight 0.
 *   o_parts   : nparts arrays [rows][head_dim]
 *   lse_parts : nparts arrays [rows]
 *   o : [rows][head_dim], lse : [rows] or NULL
 * Returns 0, or -1 on a bad argument (including a row where every part is
 * -inf).
 */
int oracle_merge(const double *const *o_parts, const double *const *lse_parts,
                 int nparts, int64_t rows, int head_dim, double *o,
                 double *lse) {
    if (!o_parts || !lse_parts || nparts < 1 || rows < 0 || head_dim < 1 || !o)
        return -1;
    for (int i = 0; i < nparts; ++i)
        if (!o_parts[i] || !lse_parts[i]) return -1;
    int bad = 0;
    for (int64_t r = 0; r < rows; ++r) {
        double mx = -INFINITY;
        for (int i = 0; i < nparts; ++i)
            if (lse_parts[i][r] > mx) mx = lse_parts[i][r];
        if (mx == -INFINITY) {
            bad = 1;
            continue;
        }
        double z = 0.0;
        for (int i = 0; i < nparts; ++i) z += exp(lse_parts[i][r] - mx);
        double *orow = o + r * head_dim;
        for (int c = 0; c < head_dim; ++c) orow[c] = 0.0;
        for (int i = 0; i < nparts; ++i) {
            double w = exp(lse_parts[i][r] - mx) / z;
            const double *oi = o_parts[i] + r * head_dim;
            for (int c = 0; c < head_dim; ++c) orow[c] += w * oi[c];
        }
        if (lse) lse[r] = mx + log(z);
    }
    return bad ? -1 : 0;
}

/* Number of threads a parallel region of this library will use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
