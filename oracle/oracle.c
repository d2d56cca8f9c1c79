/*
 * Plain fp64 CPU oracle for spacetime attention, patchify and 3D RoPE.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it. It shares no source with the HIP library.
 *
 * Every routine is the plain definition of what it computes, written as
 * nested loops in double precision, with no tiling, fusion or reordering
 * beyond that definition. Inputs and outputs are double arrays (bf16 or fp32
 * inputs arrive as exact double copies of their values). OpenMP parallelises only the outermost
 * independent loop; each output element is computed by one thread in a fixed
 * order, so results do not depend on the thread count.
 *
 * Layouts (the token order of "How AI Generates Video: Inside Sora and Wan2.1
 * on a Real GPU", section 7, where a query at grid (t,h,w) has flat index
 * t*Hp*Wp + h*Wp + w):
 *   latent   x[b][c][t][y][x]            NCTHW, (B, C, Tl, Hl, Wl)
 *   weight   w[o][c][i][j][k]            Conv3d layout, (Dout, C, pt, ph, pw)
 *   tokens   tok[b][n][o]                token-major, n = (t*Hp + h)*Wp + w
 *   q/k/v/o  a[b][n][head][d]            token-major, (B, N, heads, D)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_E_ARG 1        /* null pointer or non-positive size */
#define ORACLE_E_ROPE_SPLIT 2 /* t_dim + h_dim + w_dim != D, or an odd part */
#define ORACLE_E_MODE 3
#define ORACLE_E_NOMEM 4

enum { ORACLE_FULL = 0, ORACLE_SPATIAL = 1, ORACLE_TEMPORAL = 2 };

/* ------------------------------------------------------------------------
 * Patchify: a Conv3d whose stride equals its kernel (pt, ph, pw).
 *
 * "Video and 3D Generation" cheatsheet, "Tiny video DiT" (Conv3d, stride
 * equals kernel); "How AI Generates Video ...", section 4 (each 1x2x2 brick
 * of 16 channels, 64 numbers, is linearly mapped to a 1,536-wide token).
 * For token (t,h,w) and output channel o:
 *   tok[b][n][o] = bias[o] + sum_{c,i,j,k} W[o][c][i][j][k] *
 *                  x[b][c][t*pt+i][h*ph+j][w*pw+k]
 * The token grid is T = Tl/pt, Hp = Hl/ph, Wp = Wl/pw (floor division, as a
 * strided convolution with no padding drops a remainder).
 * ------------------------------------------------------------------------ */
int oracle_patchify(const double *x, const double *w, const double *bias, double *tok,
                    int B, int C, int Tl, int Hl, int Wl, int pt, int ph, int pw, int Dout)
{
    if (!x || !w || !tok || B <= 0 || C <= 0 || Tl <= 0 || Hl <= 0 || Wl <= 0 ||
        pt <= 0 || ph <= 0 || pw <= 0 || Dout <= 0)
        return ORACLE_E_ARG;
    const int T = Tl / pt, Hp = Hl / ph, Wp = Wl / pw;
    if (T <= 0 || Hp <= 0 || Wp <= 0)
        return ORACLE_E_ARG;
    const int64_t N = (int64_t)T * Hp * Wp;

    #pragma omp parallel for schedule(static)
    for (int64_t bn = 0; bn < (int64_t)B * N; ++bn) {
        const int b = (int)(bn / N);
        const int64_t n = bn % N;
        const int t = (int)(n / ((int64_t)Hp * Wp));
        const int h = (int)((n / Wp) % Hp);
        const int ww = (int)(n % Wp);
        for (int o = 0; o < Dout; ++o) {
            double acc = bias ? bias[o] : 0.0;
            for (int c = 0; c < C; ++c)
                for (int i = 0; i < pt; ++i)
                    for (int j = 0; j < ph; ++j)
                        for (int k = 0; k < pw; ++k) {
                            const int64_t wi = ((((int64_t)o * C + c) * pt + i) * ph + j) * pw + k;
                            const int64_t xi =
                                ((((int64_t)b * C + c) * Tl + (t * pt + i)) * Hl + (h * ph + j)) * Wl +
                                (ww * pw + k);
                            acc += w[wi] * x[xi];
                        }
            tok[bn * Dout + o] = acc;
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * 3D factorised rotary position embedding.
 *
 * "How AI Generates Video ...", section 4 ("How 3D Factorized RoPE Encodes
 * (t', h, w)"): each head vector of width D is cut into three consecutive
 * segments of widths (d_t, d_h, d_w) = (44, 42, 42) for D = 128. Inside
 * segment a, element pairs (2j, 2j+1) are read as one complex number and
 * multiplied by exp(i * p_a * f_{a,j}), where p_a is the token's grid index
 * on that axis (t, h or w, counted from 0) and the pair frequency is
 * f_{a,j} = theta^(-2j / d_a), theta = 10,000, with the axis's own width d_a
 * in the exponent. The "Video and 3D Generation" cheatsheet
 * ("Troubleshooting") makes a split that does not sum to D an error.
 * Applied to every head of every token; y must not overlap x.
 * ------------------------------------------------------------------------ */
/* Rotate every head of one token at grid position pos = (t, h, w). */
static void rope_token(const double *x, double *y, const int pos[3], int heads, int D, const int width[3],
                       double theta)
{
    for (int hd = 0; hd < heads; ++hd) {
        const int64_t base = (int64_t)hd * D;
        int off = 0;
        for (int a = 0; a < 3; ++a) {
            for (int j = 0; j < width[a] / 2; ++j) {
                const double freq = pow(theta, -2.0 * (double)j / (double)width[a]);
                const double ang = (double)pos[a] * freq;
                const double c = cos(ang), s = sin(ang);
                const double re = x[base + off + 2 * j];
                const double im = x[base + off + 2 * j + 1];
                /* (re + i*im) * (c + i*s) */
                y[base + off + 2 * j] = re * c - im * s;
                y[base + off + 2 * j + 1] = re * s + im * c;
            }
            off += width[a];
        }
    }
}

int oracle_rope3d(const double *x, double *y, int B, int T, int Hp, int Wp, int heads, int D,
                  int d_t, int d_h, int d_w, double theta)
{
    if (!x || !y || B <= 0 || T <= 0 || Hp <= 0 || Wp <= 0 || heads <= 0 || D <= 0)
        return ORACLE_E_ARG;
    if (d_t < 0 || d_h < 0 || d_w < 0 || d_t + d_h + d_w != D || (d_t % 2) || (d_h % 2) || (d_w % 2))
        return ORACLE_E_ROPE_SPLIT;
    const int64_t N = (int64_t)T * Hp * Wp;
    const int width[3] = {d_t, d_h, d_w};

    #pragma omp parallel for schedule(static)
    for (int64_t bn = 0; bn < (int64_t)B * N; ++bn) {
        const int64_t n = bn % N;
        const int pos[3] = {(int)(n / ((int64_t)Hp * Wp)), (int)((n / Wp) % Hp), (int)(n % Wp)};
        rope_token(x + bn * heads * D, y + bn * heads * D, pos, heads, D, width, theta);
    }
    return ORACLE_OK;
}

/* The same rotation for a list of tokens: row r of x and y ([B][nrows][heads]
 * [D]) holds token rows[r] of the (T, Hp, Wp) grid, whose indices give the
 * position. */
int oracle_rope3d_rows(const double *x, double *y, const int64_t *rows, int64_t nrows, int B, int T, int Hp,
                       int Wp, int heads, int D, int d_t, int d_h, int d_w, double theta)
{
    if (!x || !y || !rows || nrows <= 0 || B <= 0 || T <= 0 || Hp <= 0 || Wp <= 0 || heads <= 0 || D <= 0)
        return ORACLE_E_ARG;
    if (d_t < 0 || d_h < 0 || d_w < 0 || d_t + d_h + d_w != D || (d_t % 2) || (d_h % 2) || (d_w % 2))
        return ORACLE_E_ROPE_SPLIT;
    const int64_t N = (int64_t)T * Hp * Wp;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= N)
            return ORACLE_E_ARG;
    const int width[3] = {d_t, d_h, d_w};

    #pragma omp parallel for schedule(static)
    for (int64_t br = 0; br < (int64_t)B * nrows; ++br) {
        const int64_t n = rows[br % nrows];
        const int pos[3] = {(int)(n / ((int64_t)Hp * Wp)), (int)((n / Wp) % Hp), (int)(n % Wp)};
        rope_token(x + br * heads * D, y + br * heads * D, pos, heads, D, width, theta);
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * Softmax attention over a key set, for one query row:
 *   l_m = scale * <q_n, k_m>        for m in the key set of n
 *   M   = max_m l_m
 *   o_n = sum_m exp(l_m - M) v_m / sum_m exp(l_m - M)
 * computed in two passes in double precision.
 *
 * Key sets (the divided-attention split of the "Video and 3D Generation"
 * cheatsheet, "Formulas and numbers", and of "Video as a 3D signal",
 * "Patches and attention"):
 *   full      all N tokens of the clip (every token sees every token,
 *             "Video Diffusion Models, in depth", Step 3);
 *   spatial   the HpWp tokens of the query's own latent frame t;
 *   temporal  the T tokens at the query's own patch position (h, w).
 * The softmax scale defaults to 1/sqrt(D) when scale <= 0 (the scaling the
 * attention probe of "How AI Generates Video ...", section 7, applies).
 *
 * rows: optional list of nrows query tokens (each in [0, N)); the output is
 * then o[b][r][head][d] for r < nrows. With rows == NULL every token is a
 * query and nrows must equal N.
 * ------------------------------------------------------------------------ */
int oracle_attention(const double *q, const double *k, const double *v, double *o,
                     int B, int T, int Hp, int Wp, int heads, int D, double scale, int mode,
                     const int64_t *rows, int64_t nrows)
{
    if (!q || !k || !v || !o || B <= 0 || T <= 0 || Hp <= 0 || Wp <= 0 || heads <= 0 || D <= 0)
        return ORACLE_E_ARG;
    if (mode != ORACLE_FULL && mode != ORACLE_SPATIAL && mode != ORACLE_TEMPORAL)
        return ORACLE_E_MODE;
    const int64_t HW = (int64_t)Hp * Wp;
    const int64_t N = (int64_t)T * HW;
    if (rows == NULL && nrows != N)
        return ORACLE_E_ARG;
    if (nrows <= 0)
        return ORACLE_E_ARG;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= N)
                return ORACLE_E_ARG;
    if (scale <= 0.0)
        scale = 1.0 / sqrt((double)D);
    const int64_t nkeys = (mode == ORACLE_FULL) ? N : (mode == ORACLE_SPATIAL ? HW : T);
    int failed = 0;

    #pragma omp parallel
    {
        double *logit = (double *)malloc(sizeof(double) * (size_t)nkeys);
        int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)nkeys);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        if (!logit || !key || !acc) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for schedule(dynamic, 4) collapse(3)
        for (int b = 0; b < B; ++b)
            for (int hd = 0; hd < heads; ++hd)
                for (int64_t r = 0; r < nrows; ++r) {
                    if (!logit || !key || !acc)
                        continue;
                    const int64_t n = rows ? rows[r] : r;
                    const int64_t t = n / HW, p = n % HW;
                    /* The key set of query n. */
                    for (int64_t m = 0; m < nkeys; ++m)
                        key[m] = (mode == ORACLE_FULL) ? m
                                 : (mode == ORACLE_SPATIAL) ? t * HW + m
                                                            : m * HW + p;
                    const double *qn = q + (((int64_t)b * N + n) * heads + hd) * D;
                    /* Pass 1: logits and their maximum. */
                    double M = -INFINITY;
                    for (int64_t m = 0; m < nkeys; ++m) {
                        const double *km = k + (((int64_t)b * N + key[m]) * heads + hd) * D;
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d)
                            dot += qn[d] * km[d];
                        logit[m] = scale * dot;
                        if (logit[m] > M)
                            M = logit[m];
                    }
                    /* Pass 2: exponentials, their sum and the weighted values. */
                    double sum = 0.0;
                    for (int d = 0; d < D; ++d)
                        acc[d] = 0.0;
                    for (int64_t m = 0; m < nkeys; ++m) {
                        const double wgt = exp(logit[m] - M);
                        const double *vm = v + (((int64_t)b * N + key[m]) * heads + hd) * D;
                        sum += wgt;
                        for (int d = 0; d < D; ++d)
                            acc[d] += wgt * vm[d];
                    }
                    double *on = o + (((int64_t)b * nrows + r) * heads + hd) * D;
                    for (int d = 0; d < D; ++d)
                        on[d] = acc[d] / sum;
                }
        free(logit);
        free(key);
        free(acc);
    }
    return failed ? ORACLE_E_NOMEM : ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * Cross-attention: queries of one token set attend to all keys of another.
 *
 * "How AI Generates Video ...", section 5, attn2: the video tokens supply the
 * queries and the text-prompt tokens (512 UMT5 embeddings, projected to the
 * model width) supply the keys and values; "Video Diffusion Models, in
 * depth", Step 3, likewise has the video tokens read the text embeddings.
 *   l_m = scale * <q_n, k_m>  for m = 0..Nk-1
 *   o_n = sum_m exp(l_m - M) v_m / sum_m exp(l_m - M),  M = max_m l_m
 * q, o: [B][Nq][heads][D]; k, v: [B][Nk][heads][D]. rows as in
 * oracle_attention (a list of nrows query tokens, or NULL for all Nq).
 * ------------------------------------------------------------------------ */
int oracle_cross_attention(const double *q, const double *k, const double *v, double *o,
                           int B, int Nq, int Nk, int heads, int D, double scale,
                           const int64_t *rows, int64_t nrows)
{
    if (!q || !k || !v || !o || B <= 0 || Nq <= 0 || Nk <= 0 || heads <= 0 || D <= 0)
        return ORACLE_E_ARG;
    if (rows == NULL && nrows != Nq)
        return ORACLE_E_ARG;
    if (nrows <= 0)
        return ORACLE_E_ARG;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= Nq)
                return ORACLE_E_ARG;
    if (scale <= 0.0)
        scale = 1.0 / sqrt((double)D);
    int failed = 0;

    #pragma omp parallel
    {
        double *logit = (double *)malloc(sizeof(double) * (size_t)Nk);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        if (!logit || !acc) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for schedule(dynamic, 4) collapse(3)
        for (int b = 0; b < B; ++b)
            for (int hd = 0; hd < heads; ++hd)
                for (int64_t r = 0; r < nrows; ++r) {
                    if (!logit || !acc)
                        continue;
                    const int64_t n = rows ? rows[r] : r;
                    const double *qn = q + (((int64_t)b * Nq + n) * heads + hd) * D;
                    double M = -INFINITY;
                    for (int m = 0; m < Nk; ++m) {
                        const double *km = k + (((int64_t)b * Nk + m) * heads + hd) * D;
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d)
                            dot += qn[d] * km[d];
                        logit[m] = scale * dot;
                        if (logit[m] > M)
                            M = logit[m];
                    }
                    double sum = 0.0;
                    for (int d = 0; d < D; ++d)
                        acc[d] = 0.0;
                    for (int m = 0; m < Nk; ++m) {
                        const double wgt = exp(logit[m] - M);
                        const double *vm = v + (((int64_t)b * Nk + m) * heads + hd) * D;
                        sum += wgt;
                        for (int d = 0; d < D; ++d)
                            acc[d] += wgt * vm[d];
                    }
                    double *on = o + (((int64_t)b * nrows + r) * heads + hd) * D;
                    for (int d = 0; d < D; ++d)
                        on[d] = acc[d] / sum;
                }
        free(logit);
        free(acc);
    }
    return failed ? ORACLE_E_NOMEM : ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * Windowed spacetime attention: the (T, Hp, Wp) token grid is cut into
 * non-overlapping windows of wt x wh x ww tokens (the last window along an
 * axis is cut short by the grid), and each token attends to the tokens of its
 * own window. This restricts attention to local spacetime windows, the lever
 * "Video Diffusion Models, in depth" ("Inference: where the time goes")
 * names against the quadratic term. Windows (1, Hp, Wp) give the spatial
 * pass, (T, 1, 1) the temporal pass and (T, Hp, Wp) full attention.
 *   key set of (t, h, w) = {(t', h', w') : t'/wt = t/wt, h'/wh = h/wh, w'/ww = w/ww}
 * q/k/v/o and rows as in oracle_attention.
 * ------------------------------------------------------------------------ */
int oracle_window_attention(const double *q, const double *k, const double *v, double *o,
                            int B, int T, int Hp, int Wp, int heads, int D, int wt, int wh, int ww,
                            double scale, const int64_t *rows, int64_t nrows)
{
    if (!q || !k || !v || !o || B <= 0 || T <= 0 || Hp <= 0 || Wp <= 0 || heads <= 0 || D <= 0 ||
        wt <= 0 || wh <= 0 || ww <= 0)
        return ORACLE_E_ARG;
    const int64_t HW = (int64_t)Hp * Wp;
    const int64_t N = (int64_t)T * HW;
    if (rows == NULL && nrows != N)
        return ORACLE_E_ARG;
    if (nrows <= 0)
        return ORACLE_E_ARG;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= N)
                return ORACLE_E_ARG;
    if (scale <= 0.0)
        scale = 1.0 / sqrt((double)D);
    int failed = 0;

    #pragma omp parallel
    {
        double *logit = (double *)malloc(sizeof(double) * (size_t)N);
        int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)N);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        if (!logit || !key || !acc) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for schedule(dynamic, 4) collapse(3)
        for (int b = 0; b < B; ++b)
            for (int hd = 0; hd < heads; ++hd)
                for (int64_t r = 0; r < nrows; ++r) {
                    if (!logit || !key || !acc)
                        continue;
                    const int64_t n = rows ? rows[r] : r;
                    const int t = (int)(n / HW), h = (int)((n / Wp) % Hp), w = (int)(n % Wp);
                    /* The key set: every token whose window indices match. */
                    int64_t nk = 0;
                    for (int64_t m = 0; m < N; ++m) {
                        const int tm = (int)(m / HW), hm = (int)((m / Wp) % Hp), wm = (int)(m % Wp);
                        if (tm / wt == t / wt && hm / wh == h / wh && wm / ww == w / ww)
                            key[nk++] = m;
                    }
                    const double *qn = q + (((int64_t)b * N + n) * heads + hd) * D;
                    double M = -INFINITY;
                    for (int64_t i = 0; i < nk; ++i) {
                        const double *km = k + (((int64_t)b * N + key[i]) * heads + hd) * D;
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d)
                            dot += qn[d] * km[d];
                        logit[i] = scale * dot;
                        if (logit[i] > M)
                            M = logit[i];
                    }
                    double sum = 0.0;
                    for (int d = 0; d < D; ++d)
                        acc[d] = 0.0;
                    for (int64_t i = 0; i < nk; ++i) {
                        const double wgt = exp(logit[i] - M);
                        const double *vm = v + (((int64_t)b * N + key[i]) * heads + hd) * D;
                        sum += wgt;
                        for (int d = 0; d < D; ++d)
                            acc[d] += wgt * vm[d];
                    }
                    double *on = o + (((int64_t)b * nrows + r) * heads + hd) * D;
                    for (int d = 0; d < D; ++d)
                        on[d] = acc[d] / sum;
                }
        free(logit);
        free(key);
        free(acc);
    }
    return failed ? ORACLE_E_NOMEM : ORACLE_OK;
}

/* Number of threads OpenMP will use for the routines above. */
int oracle_num_threads(void)
{
    int n = 1;
    #pragma omp parallel
    {
        #pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
