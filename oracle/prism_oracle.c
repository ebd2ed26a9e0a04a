/*
 * prism_oracle.c -- plain, slow CPU oracle for Prism's dynamic block-sparse video
 * self-attention (one layer, one head at a time, float64 throughout).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no source with the HIP library
 * and includes none of its headers.
 *
 * Sources (pages about arXiv 2610.05416, "Prism: Dynamic Sparse Attention for Native 2K
 * Joint Video-Audio Generation Model Training"):
 *   [digest]  nanless audio-paper-digest post: sections "Prism 的整体流程是怎样的"
 *             (pipeline, Fig. 2), "每个宏区如何估计视觉变化与音频影响" (guidance, Eq. g_d),
 *             "信息密度如何决定块体积与具体边长" (density, Eq. rho_raw, Eq. J),
 *             "混合块选择如何为每个查询定稀疏度" (selection), "模型如何训练与哪些参数更新"
 *             (training: no gradient through the plan, 64-token units).
 *   [review]  xyznot.com review, "Метод" items 1 (variation indicator: sigma^2_{v,d},
 *             r_{v,d}, g_d), 2 (volume and shape quantisation, closed form l*_d),
 *             3 (hybrid Top-k / Top-p).
 *
 * Conventions (readings where the pages are silent; each is listed in the design notes):
 *   - grid T x H x W, token n = (t*H + h)*W + w (raster, w fastest); zones are 8x8x8
 *     boxes in raster order; local coordinates (i, j, l) in [0,8)^3;
 *   - a block shape is stored as its log2 edges packed as lT*16 + lH*4 + lW;
 *   - variances are population variances (1/Z_d); an all-zero variance total gives
 *     shares of 0; the rho and a-bar normalisers are per call (per head for rho);
 *   - tiers: rho >= tau128 -> 64, tau256 <= rho < tau128 -> 128, else 256;
 *   - shape ties: candidates within 1e-9 of the minimum squared log2 distance are tied,
 *     and the first in lexicographic (b_T, b_H, b_W) order wins;
 *   - blocks inside a zone in raster order of block coordinates, tokens inside a block
 *     in raster order; zones in raster order;
 *   - selection order is (P descending, block index ascending); the Top-p prefix is the
 *     shortest one whose mass is >= p (it includes the crossing block); the union with
 *     Top-k is the prefix of length max(k, n_p), capped at the number of blocks.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ZE 8          /* macro-zone edge along T, H and W ([digest] pipeline, Fig. 2) */
#define ZV 512        /* tokens per zone */
#define TIE_TOL 1e-9  /* shape-distance tie tolerance */

static int idx_token(int H, int W, int t, int h, int w) { return (t * H + h) * W + w; }

/* ------------------------------------------------------------------------------------
 * Zone statistics of V for one head ([review] item 1, sigma^2_{v,d};
 * [digest] density section, Eq. rho_raw).
 * v: [N][D] float64.  out: [Z][4] = sigma2_T, sigma2_H, sigma2_W, rho_raw.
 * dmode selects the terms of rho_raw for the density ablation ([digest] ablation
 * section: spatial only or temporal only): 1 spatial, 2 temporal, otherwise both.
 * ---------------------------------------------------------------------------------- */
int orc_zone_stats(int T, int H, int W, int D, const double *v, int dmode, double *out)
{
    if (T % ZE || H % ZE || W % ZE || D <= 0) return -1;
    int nzt = T / ZE, nzh = H / ZE, nzw = W / ZE;
    double *pt = malloc(sizeof(double) * ZE), *ph = malloc(sizeof(double) * ZE),
           *pw = malloc(sizeof(double) * ZE);
    int m = 0;
    for (int zt = 0; zt < nzt; ++zt)
        for (int zh = 0; zh < nzh; ++zh)
            for (int zw = 0; zw < nzw; ++zw, ++m) {
                double s2[3] = {0, 0, 0}, spatial = 0, temporal = 0;
                for (int c = 0; c < D; ++c) {
                    /* axis profiles: mean over the other two axes */
                    for (int a = 0; a < ZE; ++a) pt[a] = ph[a] = pw[a] = 0;
                    for (int i = 0; i < ZE; ++i)
                        for (int j = 0; j < ZE; ++j)
                            for (int l = 0; l < ZE; ++l) {
                                double x = v[(size_t)idx_token(H, W, zt * ZE + i, zh * ZE + j,
                                                                zw * ZE + l) * D + c];
                                pt[i] += x;
                                ph[j] += x;
                                pw[l] += x;
                            }
                    double mu = 0;
                    for (int a = 0; a < ZE; ++a) {
                        pt[a] /= (ZE * ZE);
                        ph[a] /= (ZE * ZE);
                        pw[a] /= (ZE * ZE);
                        mu += pt[a];
                    }
                    mu /= ZE;
                    /* directional variance of each profile about the zone mean (1/Z_d) */
                    double vt = 0, vh = 0, vw = 0;
                    for (int a = 0; a < ZE; ++a) {
                        vt += (pt[a] - mu) * (pt[a] - mu);
                        vh += (ph[a] - mu) * (ph[a] - mu);
                        vw += (pw[a] - mu) * (pw[a] - mu);
                    }
                    s2[0] += vt / ZE;
                    s2[1] += vh / ZE;
                    s2[2] += vw / ZE;
                    /* intra-zone spatial variance about the per-frame mean */
                    double sp = 0;
                    for (int i = 0; i < ZE; ++i)
                        for (int j = 0; j < ZE; ++j)
                            for (int l = 0; l < ZE; ++l) {
                                double x = v[(size_t)idx_token(H, W, zt * ZE + i, zh * ZE + j,
                                                                zw * ZE + l) * D + c];
                                sp += (x - pt[i]) * (x - pt[i]);
                            }
                    spatial += sp / ZV;
                    /* temporal frame-difference term over the Z_T - 1 consecutive pairs */
                    double td = 0;
                    for (int i = 0; i + 1 < ZE; ++i) td += (pt[i + 1] - pt[i]) * (pt[i + 1] - pt[i]);
                    temporal += td / (ZE - 1);
                }
                out[4 * m + 0] = s2[0] / D;
                out[4 * m + 1] = s2[1] / D;
                out[4 * m + 2] = s2[2] / D;
                out[4 * m + 3] = (dmode == 2 ? 0.0 : spatial / D) + (dmode == 1 ? 0.0 : temporal / D);
            }
    free(pt);
    free(ph);
    free(pw);
    return 0;
}

/* ------------------------------------------------------------------------------------
 * Zone statistics of the audio-to-video norm field a ([digest] guidance section;
 * [review] item 1).  The zone mean and the directional variance of the axis profiles of
 * the scalar field, built the same way as for V.
 * a: [N].  out: [Z][4] = mean, sigma2_T, sigma2_H, sigma2_W.
 * ---------------------------------------------------------------------------------- */
int orc_audio_stats(int T, int H, int W, const double *a, double *out)
{
    if (T % ZE || H % ZE || W % ZE) return -1;
    int nzt = T / ZE, nzh = H / ZE, nzw = W / ZE, m = 0;
    for (int zt = 0; zt < nzt; ++zt)
        for (int zh = 0; zh < nzh; ++zh)
            for (int zw = 0; zw < nzw; ++zw, ++m) {
                double pt[ZE] = {0}, ph[ZE] = {0}, pw[ZE] = {0}, mu = 0;
                for (int i = 0; i < ZE; ++i)
                    for (int j = 0; j < ZE; ++j)
                        for (int l = 0; l < ZE; ++l) {
                            double x = a[idx_token(H, W, zt * ZE + i, zh * ZE + j, zw * ZE + l)];
                            pt[i] += x;
                            ph[j] += x;
                            pw[l] += x;
                        }
                for (int q = 0; q < ZE; ++q) {
                    pt[q] /= (ZE * ZE);
                    ph[q] /= (ZE * ZE);
                    pw[q] /= (ZE * ZE);
                    mu += pt[q];
                }
                mu /= ZE;
                double vt = 0, vh = 0, vw = 0;
                for (int q = 0; q < ZE; ++q) {
                    vt += (pt[q] - mu) * (pt[q] - mu);
                    vh += (ph[q] - mu) * (ph[q] - mu);
                    vw += (pw[q] - mu) * (pw[q] - mu);
                }
                out[4 * m + 0] = mu;
                out[4 * m + 1] = vt / ZE;
                out[4 * m + 2] = vh / ZE;
                out[4 * m + 3] = vw / ZE;
            }
    return 0;
}

/* Candidate pool C_B ([digest] density section; [review] item 2): power-of-two edges
 * with log2 edge in [min_edge_log2, 3] along each axis and product 2^S.  Listed in
 * lexicographic (b_T, b_H, b_W) order; returns the count. */
int orc_shape_pool(int S, int min_edge_log2, int *cand /* [..][3] log2 edges */)
{
    int n = 0;
    for (int a = min_edge_log2; a <= 3; ++a)
        for (int b = min_edge_log2; b <= 3; ++b)
            for (int c = min_edge_log2; c <= 3; ++c)
                if (a + b + c == S) {
                    cand[3 * n + 0] = a;
                    cand[3 * n + 1] = b;
                    cand[3 * n + 2] = c;
                    ++n;
                }
    return n;
}

/* ------------------------------------------------------------------------------------
 * Per-zone plan for one head: normalisations, variation indicator g_d ([digest] Eq. g_d;
 * [review] item 1), volume tier B(m) from the density thresholds ([digest] density
 * section; [review] item 2), continuous optimum l*_d of the shape loss J under
 * prod b_d = B ([digest] Eq. J; [review] item 2 closed form) and log2-space nearest
 * candidate.
 *   vstats [Z][4] from orc_zone_stats, astats [Z][4] from orc_audio_stats or NULL
 *   (first layer: no cached A2V norm, video guidance only).
 *   shape_out [Z]: packed log2 edges.  diag [Z][12] (optional): rho, abar, g_T, g_H, g_W,
 *   l*_T, l*_H, l*_W, B, tier margin, shape margin, best distance.
 * Ablation settings ([digest] ablation section): alpha is the exponent of the mapping
 * b_d ~ g_d^-alpha (the Lagrange optimum of J gives 1/2); fixed > 0 gives every zone that
 * packed shape (the fixed-shape baseline; no shape decision, margin reported as 1e300);
 * dmode 3 takes the volume tier from the normalised A2V intensity a_bar instead of rho.
 * ---------------------------------------------------------------------------------- */
int orc_zone_plan(int Z, const double *vstats, const double *astats, double tau128,
                  double tau256, double eps, int min_edge_log2, double alpha, int fixed,
                  int dmode, int *shape_out, double *diag)
{
    if (Z <= 0 || min_edge_log2 < 0 || min_edge_log2 > 2) return -1;
    if (fixed > 0) {
        int fa = (fixed >> 4) & 3, fb = (fixed >> 2) & 3, fc = fixed & 3, fs = fa + fb + fc;
        if (fixed > 63 || fa < min_edge_log2 || fb < min_edge_log2 || fc < min_edge_log2 ||
            fs < 6 || fs > 8)
            return -1;
    }
    double rho_max = 0, a_max = 0;
    for (int m = 0; m < Z; ++m) {
        if (vstats[4 * m + 3] > rho_max) rho_max = vstats[4 * m + 3];
        if (astats && astats[4 * m + 0] > a_max) a_max = astats[4 * m + 0];
    }
    int cand[3 * 64];
    for (int m = 0; m < Z; ++m) {
        const double *vs = vstats + 4 * m;
        double rho = rho_max > 0 ? vs[3] / rho_max : 0.0;
        double vsum = vs[0] + vs[1] + vs[2];
        double r[3];
        for (int d = 0; d < 3; ++d) r[d] = vsum > 0 ? vs[d] / vsum : 0.0;
        double abar = 0, va[3] = {0, 0, 0};
        if (astats) {
            const double *as = astats + 4 * m;
            abar = a_max > 0 ? as[0] / a_max : 0.0;
            double asum = as[1] + as[2] + as[3];
            for (int d = 0; d < 3; ++d) va[d] = asum > 0 ? as[1 + d] / asum : 0.0;
        }
        if (dmode == 3) rho = abar;
        double g[3];
        for (int d = 0; d < 3; ++d) g[d] = r[d] + abar * va[d] + eps;

        int S;
        if (rho >= tau128) S = 6;
        else if (rho >= tau256) S = 7;
        else S = 8;

        double lg[3];
        for (int d = 0; d < 3; ++d) lg[d] = log2(g[d]);
        double lstar[3];
        for (int d = 0; d < 3; ++d)
            lstar[d] = -alpha * lg[d] + (S + alpha * lg[0] + alpha * lg[1] + alpha * lg[2]) / 3.0;

        int nc;
        if (fixed > 0) {
            S = ((fixed >> 4) & 3) + ((fixed >> 2) & 3) + (fixed & 3);
            cand[0] = (fixed >> 4) & 3;
            cand[1] = (fixed >> 2) & 3;
            cand[2] = fixed & 3;
            nc = 1;
        } else {
            nc = orc_shape_pool(S, min_edge_log2, cand);
        }
        double dist[64], best = INFINITY;
        for (int c = 0; c < nc; ++c) {
            double e0 = lstar[0] - cand[3 * c + 0];
            double e1 = lstar[1] - cand[3 * c + 1];
            double e2 = lstar[2] - cand[3 * c + 2];
            dist[c] = e0 * e0 + e1 * e1 + e2 * e2;
            if (dist[c] < best) best = dist[c];
        }
        int win = -1;
        double second = INFINITY;
        for (int c = 0; c < nc; ++c) {
            if (dist[c] <= best + TIE_TOL) {
                if (win < 0) win = c;
            } else if (dist[c] < second) {
                second = dist[c];
            }
        }
        shape_out[m] = cand[3 * win + 0] * 16 + cand[3 * win + 1] * 4 + cand[3 * win + 2];
        if (diag) {
            double *o = diag + 12 * m;
            o[0] = rho;
            o[1] = abar;
            o[2] = g[0];
            o[3] = g[1];
            o[4] = g[2];
            o[5] = lstar[0];
            o[6] = lstar[1];
            o[7] = lstar[2];
            o[8] = (double)(1 << S);
            double tm = fabs(rho - tau128), tm2 = fabs(rho - tau256);
            o[9] = tm < tm2 ? tm : tm2;
            o[10] = fixed > 0 ? 1e300 : second - best;
            o[11] = best;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------
 * Block-contiguous permutation ([digest] summary and pipeline: tokens are rearranged so
 * that each block is contiguous; Q, K and V share it).
 *   perm [N]: permuted position -> token; inv [N]: token -> permuted position;
 *   blk_start [nb], blk_size [nb]: permuted offset and token count of each block;
 *   blk_of [N]: permuted position -> block.  Returns nb, or -1.
 * ---------------------------------------------------------------------------------- */
int orc_permutation(int T, int H, int W, const int *shape, int *perm, int *inv,
                    int *blk_start, int *blk_size, int *blk_of)
{
    if (T % ZE || H % ZE || W % ZE) return -1;
    int nzt = T / ZE, nzh = H / ZE, nzw = W / ZE, m = 0, pos = 0, nb = 0;
    for (int zt = 0; zt < nzt; ++zt)
        for (int zh = 0; zh < nzh; ++zh)
            for (int zw = 0; zw < nzw; ++zw, ++m) {
                int bt = 1 << ((shape[m] >> 4) & 3), bh = 1 << ((shape[m] >> 2) & 3),
                    bw = 1 << (shape[m] & 3);
                for (int gt = 0; gt < ZE / bt; ++gt)
                    for (int gh = 0; gh < ZE / bh; ++gh)
                        for (int gw = 0; gw < ZE / bw; ++gw) {
                            blk_start[nb] = pos;
                            blk_size[nb] = bt * bh * bw;
                            for (int i = 0; i < bt; ++i)
                                for (int j = 0; j < bh; ++j)
                                    for (int l = 0; l < bw; ++l) {
                                        int tok = idx_token(H, W, zt * ZE + gt * bt + i,
                                                            zh * ZE + gh * bh + j,
                                                            zw * ZE + gw * bw + l);
                                        perm[pos] = tok;
                                        inv[tok] = pos;
                                        blk_of[pos] = nb;
                                        ++pos;
                                    }
                            ++nb;
                        }
            }
    return nb;
}

/* Block mean pooling ([digest] obstacles and selection sections: each block is
 * represented by the mean of its tokens).  x [N][D]; out [nb][D]. */
int orc_block_means(int D, const double *x, const int *perm, int nb, const int *blk_start,
                    const int *blk_size, double *out)
{
    for (int b = 0; b < nb; ++b)
        for (int c = 0; c < D; ++c) {
            double s = 0;
            for (int r = 0; r < blk_size[b]; ++r) s += x[(size_t)perm[blk_start[b] + r] * D + c];
            out[(size_t)b * D + c] = s / blk_size[b];
        }
    return 0;
}

/* Block relevance ([digest] selection section; [review] item 3): s_ij = scale * qbar_i .
 * kbar_j and P_i = softmax over every key block of the head.  s, P: [nb][nb]. */
int orc_block_probs(int nb, int D, const double *qbar, const double *kbar, double scale,
                    double *s, double *P)
{
    for (int i = 0; i < nb; ++i) {
        double mx = -INFINITY;
        for (int j = 0; j < nb; ++j) {
            double acc = 0;
            for (int c = 0; c < D; ++c) acc += qbar[(size_t)i * D + c] * kbar[(size_t)j * D + c];
            s[(size_t)i * nb + j] = scale * acc;
            if (s[(size_t)i * nb + j] > mx) mx = s[(size_t)i * nb + j];
        }
        double z = 0;
        for (int j = 0; j < nb; ++j) z += exp(s[(size_t)i * nb + j] - mx);
        for (int j = 0; j < nb; ++j) P[(size_t)i * nb + j] = exp(s[(size_t)i * nb + j] - mx) / z;
    }
    return 0;
}

static const double *g_sort_row;
static int cmp_desc(const void *a, const void *b)
{
    int ia = *(const int *)a, ib = *(const int *)b;
    double pa = g_sort_row[ia], pb = g_sort_row[ib];
    if (pa > pb) return -1;
    if (pa < pb) return 1;
    return ia < ib ? -1 : (ia > ib);
}
static int cmp_int(const void *a, const void *b)
{
    int x = *(const int *)a, y = *(const int *)b;
    return x < y ? -1 : (x > y);
}

/* ------------------------------------------------------------------------------------
 * Hybrid Top-k union Top-p selection per query block ([digest] selection section;
 * [review] item 3).  P [nb][nb] rows from orc_block_probs.
 *   count [nb]; cols [nb][nb] (row i holds count[i] key blocks, ascending);
 *   diag [nb][4] (optional): n_p, cumulative mass after n_p - 1 blocks, after n_p blocks,
 *   and the sort position count[i] - 1's block index.
 * ---------------------------------------------------------------------------------- */
int orc_select(int nb, const double *P, int top_k, double top_p, int *count, int *cols,
               double *diag)
{
    int *ord = malloc(sizeof(int) * (size_t)nb);
    for (int i = 0; i < nb; ++i) {
        const double *row = P + (size_t)i * nb;
        for (int j = 0; j < nb; ++j) ord[j] = j;
        g_sort_row = row;
        qsort(ord, (size_t)nb, sizeof(int), cmp_desc);
        int np = nb;
        double cum = 0, before = 0, after = 0;
        for (int r = 0; r < nb; ++r) {
            before = cum;
            cum += row[ord[r]];
            if (cum >= top_p) {
                np = r + 1;
                after = cum;
                break;
            }
            after = cum;
        }
        int n = top_k > np ? top_k : np;
        if (n > nb) n = nb;
        if (n < 1) n = 1;
        count[i] = n;
        int *dst = cols + (size_t)i * nb;
        memcpy(dst, ord, sizeof(int) * (size_t)n);
        if (diag) {
            diag[4 * i + 0] = np;
            diag[4 * i + 1] = before;
            diag[4 * i + 2] = after;
            diag[4 * i + 3] = ord[n - 1];
        }
        qsort(dst, (size_t)n, sizeof(int), cmp_int);
    }
    free(ord);
    return 0;
}

/* Key tokens of one query token under the plan: the union of its query block's selected
 * key blocks.  Fills keys[] (token indices) and returns their number. */
static int key_tokens(int x, const int *perm, const int *inv, const int *blk_start,
                      const int *blk_size, const int *blk_of, const int *count,
                      const int *cols, int nb, int *keys)
{
    int i = blk_of[inv[x]], nk = 0;
    for (int r = 0; r < count[i]; ++r) {
        int j = cols[(size_t)i * nb + r];
        for (int u = 0; u < blk_size[j]; ++u) keys[nk++] = perm[blk_start[j] + u];
    }
    return nk;
}

/* ------------------------------------------------------------------------------------
 * Exact attention over the selected key blocks ([digest] selection section: full query
 * tokens against the keys and values of the chosen blocks, softmax over those keys;
 * [review] item 3).  Results are in original token order (the inverse permutation is
 * implied by indexing by token).  No causal mask.
 *   q, k, v [N][D]; rows [nrows] (token indices) or NULL for all N;
 *   o [N][D], lse [N]: written for the listed rows only.
 *   mo [N][D] or NULL: sum_y P_xy |v_y - o_x| per channel, the size of the change in o_x
 *   when every weight P_xy is perturbed by a relative amount of at most 1 and the
 *   weights are renormalised (first order); a tolerance for an implementation that rounds
 *   the weights scales it by that rounding's unit roundoff.
 * ---------------------------------------------------------------------------------- */
int orc_attn_fwd(int N, int D, const double *q, const double *k, const double *v,
                 const int *perm, const int *inv, const int *blk_start, const int *blk_size,
                 const int *blk_of, int nb, const int *count, const int *cols, double scale,
                 const int *rows, int nrows, double *o, double *lse, double *mo)
{
    int total = rows ? nrows : N;
#pragma omp parallel
    {
        int *keys = malloc(sizeof(int) * (size_t)N);
        double *s = malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 16)
        for (int r = 0; r < total; ++r) {
            int x = rows ? rows[r] : r;
            int nk = key_tokens(x, perm, inv, blk_start, blk_size, blk_of, count, cols, nb, keys);
            double mx = -INFINITY;
            for (int y = 0; y < nk; ++y) {
                double acc = 0;
                for (int c = 0; c < D; ++c) acc += q[(size_t)x * D + c] * k[(size_t)keys[y] * D + c];
                s[y] = scale * acc;
                if (s[y] > mx) mx = s[y];
            }
            double z = 0;
            for (int y = 0; y < nk; ++y) z += exp(s[y] - mx);
            double l = mx + log(z);
            lse[x] = l;
            for (int c = 0; c < D; ++c) o[(size_t)x * D + c] = 0;
            for (int y = 0; y < nk; ++y) {
                double p = exp(s[y] - l);
                for (int c = 0; c < D; ++c) o[(size_t)x * D + c] += p * v[(size_t)keys[y] * D + c];
            }
            if (mo) {
                double *m = mo + (size_t)x * D;
                const double *ox = o + (size_t)x * D;
                for (int c = 0; c < D; ++c) m[c] = 0;
                for (int y = 0; y < nk; ++y) {
                    double p = exp(s[y] - l);
                    for (int c = 0; c < D; ++c) m[c] += p * fabs(v[(size_t)keys[y] * D + c] - ox[c]);
                }
            }
        }
        free(keys);
        free(s);
    }
    return 0;
}

/* ------------------------------------------------------------------------------------
 * Gradients of the sparse attention with the plan held constant ([digest] training
 * section: the shape assignment and the selection statistics pass no gradient; only the
 * attention over the selected blocks does).
 *   P_xy = exp(scale q_x.k_y - lse_x), delta_x = do_x . o_x,
 *   dv_y += P_xy do_x, dS_xy = P_xy (do_x . v_y - delta_x),
 *   dq_x += scale dS_xy k_y, dk_y += scale dS_xy q_x.
 * o and lse are recomputed here in float64.  rows: the query tokens whose terms are
 * summed (NULL = all; no token listed twice); with an upstream gradient that is zero on
 * every other token this is the full gradient.  dq, dk, dv [N][D] are overwritten (dq
 * only on the listed rows).  dq is summed one query row at a time, dk and dv one key
 * token at a time (each sum over its own terms only), so rows and key tokens are
 * independent and are spread over OpenMP threads.
 *
 * mq, mk, mv [N][D] (all three or none): how far each gradient moves, to first order,
 * when every weight P_xy and every dS_xy is perturbed by a relative amount of at most 1
 * (a tolerance for an implementation that rounds them scales this by that rounding's
 * unit roundoff).  With S_x = sum_y |dS_xy|, the bound on the change of delta_x that the
 * weights' perturbation causes through o_x:
 *   mv_y = sum_x P_xy |do_x|,
 *   mq_x = scale sum_y (|dS_xy| + P_xy S_x) |k_y|,
 *   mk_y = scale sum_x (|dS_xy| + P_xy S_x) |q_x|   (per channel).
 * ---------------------------------------------------------------------------------- */
int orc_attn_bwd(int N, int D, const double *q, const double *k, const double *v,
                 const double *dout, const int *perm, const int *inv, const int *blk_start,
                 const int *blk_size, const int *blk_of, int nb, const int *count,
                 const int *cols, double scale, const int *rows, int nrows, double *dq,
                 double *dk, double *dv, double *mq, double *mk, double *mv)
{
    int total = rows ? nrows : N;
    double *lse = malloc(sizeof(double) * (size_t)N);
    double *delta = malloc(sizeof(double) * (size_t)N);
    double *sabs = malloc(sizeof(double) * (size_t)N);
    memset(dq, 0, sizeof(double) * (size_t)N * D);
    memset(dk, 0, sizeof(double) * (size_t)N * D);
    memset(dv, 0, sizeof(double) * (size_t)N * D);
    if (mq) {
        memset(mq, 0, sizeof(double) * (size_t)N * D);
        memset(mk, 0, sizeof(double) * (size_t)N * D);
        memset(mv, 0, sizeof(double) * (size_t)N * D);
    }
    /* Query side, one listed row x at a time: lse_x, o_x, delta_x, dS_xy over the row's
     * key tokens, dq_x = scale sum_y dS_xy k_y, and S_x. */
#pragma omp parallel
    {
        int *keys = malloc(sizeof(int) * (size_t)N);
        double *s = malloc(sizeof(double) * (size_t)N);
        double *dsv = malloc(sizeof(double) * (size_t)N);
        double *o = malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 16)
        for (int r = 0; r < total; ++r) {
            int x = rows ? rows[r] : r;
            const double *qx = q + (size_t)x * D, *dox = dout + (size_t)x * D;
            int nk = key_tokens(x, perm, inv, blk_start, blk_size, blk_of, count, cols, nb, keys);
            double mx = -INFINITY;
            for (int y = 0; y < nk; ++y) {
                double acc = 0;
                for (int c = 0; c < D; ++c) acc += qx[c] * k[(size_t)keys[y] * D + c];
                s[y] = scale * acc;
                if (s[y] > mx) mx = s[y];
            }
            double z = 0;
            for (int y = 0; y < nk; ++y) z += exp(s[y] - mx);
            double l = mx + log(z);
            for (int c = 0; c < D; ++c) o[c] = 0;
            for (int y = 0; y < nk; ++y) {
                double p = exp(s[y] - l);
                for (int c = 0; c < D; ++c) o[c] += p * v[(size_t)keys[y] * D + c];
            }
            double dl = 0;
            for (int c = 0; c < D; ++c) dl += dox[c] * o[c];
            double sa = 0;
            for (int y = 0; y < nk; ++y) {
                const double *vy = v + (size_t)keys[y] * D;
                double p = exp(s[y] - l);
                double dp = 0;
                for (int c = 0; c < D; ++c) dp += dox[c] * vy[c];
                dsv[y] = p * (dp - dl);
                sa += fabs(dsv[y]);
            }
            for (int y = 0; y < nk; ++y) {
                const double *ky = k + (size_t)keys[y] * D;
                for (int c = 0; c < D; ++c) dq[(size_t)x * D + c] += scale * dsv[y] * ky[c];
                if (mq) {
                    double w = scale * (fabs(dsv[y]) + exp(s[y] - l) * sa);
                    for (int c = 0; c < D; ++c) mq[(size_t)x * D + c] += w * fabs(ky[c]);
                }
            }
            lse[x] = l;
            delta[x] = dl;
            sabs[x] = sa;
        }
        free(keys);
        free(s);
        free(dsv);
        free(o);
    }

    /* Key side: dv_y = sum_x P_xy do_x and dk_y = scale sum_x dS_xy q_x, summed over the
     * listed rows x whose query block selected y's block.  The listed rows are grouped by
     * their query block, and each key block gets the ascending list of query blocks that
     * selected it and hold listed rows; P_xy and dS_xy are formed again from lse_x and
     * delta_x exactly as on the query side. */
    int *rptr = calloc((size_t)nb + 1, sizeof(int));
    int *rlist = malloc(sizeof(int) * (size_t)(total > 0 ? total : 1));
    for (int r = 0; r < total; ++r) rptr[blk_of[inv[rows ? rows[r] : r]] + 1]++;
    for (int i = 0; i < nb; ++i) rptr[i + 1] += rptr[i];
    int *fill = malloc(sizeof(int) * (size_t)(nb > 0 ? nb : 1));
    for (int i = 0; i < nb; ++i) fill[i] = rptr[i];
    for (int r = 0; r < total; ++r) {
        int x = rows ? rows[r] : r;
        rlist[fill[blk_of[inv[x]]]++] = x;
    }
    int *cptr = calloc((size_t)nb + 1, sizeof(int));
    for (int i = 0; i < nb; ++i)
        if (rptr[i + 1] > rptr[i])
            for (int e = 0; e < count[i]; ++e) cptr[cols[(size_t)i * nb + e] + 1]++;
    for (int j = 0; j < nb; ++j) cptr[j + 1] += cptr[j];
    int *clist = malloc(sizeof(int) * (size_t)(cptr[nb] > 0 ? cptr[nb] : 1));
    for (int j = 0; j < nb; ++j) fill[j] = cptr[j];
    for (int i = 0; i < nb; ++i)
        if (rptr[i + 1] > rptr[i])
            for (int e = 0; e < count[i]; ++e) {
                int j = cols[(size_t)i * nb + e];
                clist[fill[j]++] = i;
            }
#pragma omp parallel for schedule(dynamic, 1)
    for (int j = 0; j < nb; ++j) {
        for (int u = 0; u < blk_size[j]; ++u) {
            int y = perm[blk_start[j] + u];
            const double *ky = k + (size_t)y * D, *vy = v + (size_t)y * D;
            double *dky = dk + (size_t)y * D, *dvy = dv + (size_t)y * D;
            for (int e = cptr[j]; e < cptr[j + 1]; ++e) {
                int i = clist[e];
                for (int r = rptr[i]; r < rptr[i + 1]; ++r) {
                    int x = rlist[r];
                    const double *qx = q + (size_t)x * D, *dox = dout + (size_t)x * D;
                    double acc = 0;
                    for (int c = 0; c < D; ++c) acc += qx[c] * ky[c];
                    double p = exp(scale * acc - lse[x]);
                    double dp = 0;
                    for (int c = 0; c < D; ++c) dp += dox[c] * vy[c];
                    double ds = p * (dp - delta[x]);
                    for (int c = 0; c < D; ++c) {
                        dvy[c] += p * dox[c];
                        dky[c] += scale * ds * qx[c];
                    }
                    if (mq) {
                        double w = scale * (fabs(ds) + p * sabs[x]);
                        for (int c = 0; c < D; ++c) {
                            mv[(size_t)y * D + c] += p * fabs(dox[c]);
                            mk[(size_t)y * D + c] += w * fabs(qx[c]);
                        }
                    }
                }
            }
        }
    }
    free(rptr);
    free(rlist);
    free(fill);
    free(cptr);
    free(clist);
    free(lse);
    free(delta);
    free(sabs);
    return 0;
}

/* ------------------------------------------------------------------------------------
 * The A2V norm field ([digest] guidance section: the audio injection strength of a video
 * position is the vector length of its audio-to-video cross-attention output):
 *   out[i] = sqrt(sum_c x[rows[i]][c]^2), x: [N][C] float64, rows: the n row indices.
 * ---------------------------------------------------------------------------------- */
int orc_row_norms(int C, const double *x, const int64_t *rows, int n, double *out)
{
    if (C <= 0 || n < 0) return -1;
    for (int i = 0; i < n; ++i) {
        const double *r = x + (size_t)rows[i] * C;
        double s = 0;
        for (int c = 0; c < C; ++c) s += r[c] * r[c];
        out[i] = sqrt(s);
    }
    return 0;
}
