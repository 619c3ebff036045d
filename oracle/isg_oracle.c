/*
 * isg_oracle.c -- plain, slow CPU oracle for group-shared importance-sampled
 * permuted block-sparse attention (InstaGen).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load or call this library.  It shares no source, header,
 * table or helper with the HIP library; it is written from the method as the
 * InstaGen pages describe it:
 *
 *   [A] InstaGen, acceptodds.com page, abstract (block choice by per-query
 *       votes on product-quantised scores; a random sample of the skipped
 *       tokens, one per query cluster, scaled to stand in for everything
 *       skipped; exact and sampled keys in one attention kernel).
 *   [B] InstaGen, Paper Reading AI Learner page, abstract (block selection as
 *       importance sampling: an exactly computed set of high-scoring keys, the
 *       rest estimated from a sample whose draw probabilities follow the
 *       estimated attention, each term divided by its draw probability; one
 *       sample per query cluster, used by all of its queries).
 *   [F3] InstaGen, thelatestinai.com page, Figure 3: (a) Q and K partitioned
 *       by clustering, (b) centroid scores turned into a per-(query group,
 *       key group) probability pi, (c) the best key group never dropped and
 *       the other keys drawn with probability pi and weight 1/pi, (d) one key
 *       set per query group, so the work is dense blocks.
 *   [F2] same page, Figure 2: Cq = 100 / Ck = 500, budgets E+S from 4+4 % to
 *       32+32 % of the keys.
 *
 * Where the pages leave a step open the reading taken is stated at the step.
 * Arithmetic is fp64 unless a step is defined in fp32 on purpose (the centroid
 * scores and the proposal quantisation, which decide integers and must be
 * reproducible bit for bit).  Build with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------- */
/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw: "Parallel random numbers: as easy
 * as 1, 2, 3", SC'11).  Round: two 64x64->128 products of words 0 and 2 with
 * the multipliers; the new words are (hi1 ^ w1 ^ k0, lo1, hi0 ^ w3 ^ k1, lo0);
 * the key is bumped by the Weyl constants between rounds. */
void orc_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4])
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
    uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += W0; k1 += W1; }
        unsigned __int128 p0 = (unsigned __int128)M0 * x0;
        unsigned __int128 p1 = (unsigned __int128)M1 * x2;
        uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        uint64_t n0 = hi1 ^ x1 ^ k0, n1 = lo1, n2 = hi0 ^ x3 ^ k1, n3 = lo0;
        x0 = n0; x1 = n1; x2 = n2; x3 = n3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* Proposal weights on a 2^(-1/256) grid: tbl[k] = round(2^31 * 2^(-k/256)). */
void orc_proposal_table(uint32_t tbl[256])
{
    for (int k = 0; k < 256; ++k)
        tbl[k] = (uint32_t)llround(exp2(31.0 - (double)k / 256.0));
}

/* ------------------------------------------------------------------------- */
/* k-means (Lloyd), [F3](a): the pages only say Q and K are clustered into
 * groups.  Reading: Euclidean k-means on the raw vectors, ties to the lowest
 * index, empty cluster keeps its previous centroid. */

/* labels[t] = argmin_j sum_k (x_tk - c_jk)^2, fp64; optional best squared distance. */
void orc_kmeans_assign(const float *x, int64_t n, int d, int64_t row_stride,
                       const float *cent, int C, int32_t *labels, double *best_d2)
{
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        const float *xt = x + t * row_stride;
        int best = 0;
        double bd = INFINITY;
        for (int j = 0; j < C; ++j) {
            double s = 0.0;
            for (int k = 0; k < d; ++k) {
                double df = (double)xt[k] - (double)cent[(int64_t)j * d + k];
                s += df * df;
            }
            if (s < bd) { bd = s; best = j; }
        }
        labels[t] = best;
        if (best_d2) best_d2[t] = bd;
    }
}

/* Squared distance of one row to one centroid, fp64 (used by the near-tie rule). */
double orc_sqdist(const float *xrow, const float *crow, int d)
{
    double s = 0.0;
    for (int k = 0; k < d; ++k) {
        double df = (double)xrow[k] - (double)crow[k];
        s += df * df;
    }
    return s;
}

/* c_j = fp64 mean of the members of j (token order), rounded to fp32;
 * an empty cluster keeps cent_prev[j].  counts may be NULL. */
void orc_kmeans_update(const float *x, int64_t n, int d, int64_t row_stride,
                       const int32_t *labels, int C, const float *cent_prev,
                       float *cent_out, int32_t *counts)
{
    double *sum = (double *)calloc((size_t)C * d, sizeof(double));
    int64_t *cnt = (int64_t *)calloc((size_t)C, sizeof(int64_t));
    for (int64_t t = 0; t < n; ++t) {
        int j = labels[t];
        cnt[j] += 1;
        for (int k = 0; k < d; ++k) sum[(int64_t)j * d + k] += (double)x[t * row_stride + k];
    }
    for (int j = 0; j < C; ++j) {
        for (int k = 0; k < d; ++k) {
            int64_t o = (int64_t)j * d + k;
            cent_out[o] = cnt[j] > 0 ? (float)(sum[o] / (double)cnt[j]) : cent_prev[o];
        }
        if (counts) counts[j] = (int32_t)cnt[j];
    }
    free(sum);
    free(cnt);
}

/* Stable counting sort of token ids by label; offsets = exclusive prefix of counts. */
void orc_stable_sort(const int32_t *labels, int64_t n, int C, int32_t *perm, int32_t *offsets)
{
    int64_t *next = (int64_t *)calloc((size_t)C + 1, sizeof(int64_t));
    for (int64_t t = 0; t < n; ++t) next[labels[t] + 1] += 1;
    for (int j = 0; j < C; ++j) next[j + 1] += next[j];
    for (int j = 0; j <= C; ++j) offsets[j] = (int32_t)next[j];
    for (int64_t t = 0; t < n; ++t) perm[next[labels[t]]++] = (int32_t)t;
    free(next);
}

/* Whole clustering step per (b, h) on contiguous [B,H,N,d] fp32 input:
 * init (init_mode 0: c_j = x_{floor(j*N/C)}; 1: given), `iters` rounds of
 * (assign, update), stable sort by the last labels, gather x (and companion,
 * e.g. V for K) into sorted order.  x_perm / companion / companion_perm may be NULL. */
void orc_cluster(const float *x, int B, int H, int N, int d, int C, int iters, int init_mode,
                 const float *companion, float *centroids, int32_t *labels, int32_t *perm,
                 int32_t *offsets, float *x_perm, float *companion_perm)
{
    for (int bh = 0; bh < B * H; ++bh) {
        const float *xh = x + (int64_t)bh * N * d;
        float *ch = centroids + (int64_t)bh * C * d;
        int32_t *lh = labels + (int64_t)bh * N;
        if (init_mode == 0)
            for (int j = 0; j < C; ++j)
                memcpy(ch + (int64_t)j * d, xh + ((int64_t)j * N / C) * d, sizeof(float) * d);
        float *tmp = (float *)malloc(sizeof(float) * (size_t)C * d);
        for (int it = 0; it < iters; ++it) {
            orc_kmeans_assign(xh, N, d, d, ch, C, lh, NULL);
            orc_kmeans_update(xh, N, d, d, lh, C, ch, tmp, NULL);
            memcpy(ch, tmp, sizeof(float) * (size_t)C * d);
        }
        free(tmp);
        int32_t *ph = perm + (int64_t)bh * N;
        orc_stable_sort(lh, N, C, ph, offsets + (int64_t)bh * (C + 1));
        for (int r = 0; r < N; ++r) {
            if (x_perm)
                memcpy(x_perm + ((int64_t)bh * N + r) * d, xh + (int64_t)ph[r] * d, sizeof(float) * d);
            if (companion && companion_perm)
                memcpy(companion_perm + ((int64_t)bh * N + r) * d,
                       companion + ((int64_t)bh * N + ph[r]) * d, sizeof(float) * d);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Centroid scores and pi, [F3](b), [B].
 * S_ij = (fp32 fused-multiply-add chain over k = 0..d-1 of cq_ik * ck_jk) * scale,
 * all in fp32 so that both implementations reach the same bits.
 * Reading of pi: a key's estimated attention is exp(S_ij), so group j's mass is
 * n_j exp(S_ij): pi_ij = n_j e^{S_ij} / sum_{j'} n_j' e^{S_ij'} (fp64); empty -> 0. */
void orc_probs(const float *cq, const float *ck, const int32_t *k_offsets, int B, int H,
               int Cq, int Ck, int d, float scale, float *scores, double *pi)
{
    for (int bh = 0; bh < B * H; ++bh) {
        const int32_t *ko = k_offsets + (int64_t)bh * (Ck + 1);
        for (int i = 0; i < Cq; ++i) {
            const float *qi = cq + ((int64_t)bh * Cq + i) * d;
            float *Si = scores + ((int64_t)bh * Cq + i) * Ck;
            for (int j = 0; j < Ck; ++j) {
                const float *kj = ck + ((int64_t)bh * Ck + j) * d;
                float acc = 0.0f;
                for (int k = 0; k < d; ++k) acc = fmaf(qi[k], kj[k], acc);
                Si[j] = acc * scale;
            }
            if (!pi) continue;
            double *pii = pi + ((int64_t)bh * Cq + i) * Ck;
            double mx = -INFINITY, tot = 0.0;
            for (int j = 0; j < Ck; ++j)
                if (ko[j + 1] > ko[j] && Si[j] > mx) mx = Si[j];
            for (int j = 0; j < Ck; ++j) {
                int nj = ko[j + 1] - ko[j];
                pii[j] = nj > 0 ? (double)nj * exp((double)Si[j] - mx) : 0.0;
                tot += pii[j];
            }
            for (int j = 0; j < Ck; ++j) pii[j] /= tot;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Exact set and shared sample, [B], [F3](c), [A].
 *
 * Exact set: non-empty key groups ordered by (score desc, j asc) -- by
 * (votes desc, score desc, j asc) in votes mode -- the first is always taken
 * (the best group is never dropped), the following ones while the running key
 * count stays <= exact_keys; the walk stops at the first group that would
 * exceed it.  Output: group ids ascending.
 *
 * Sample of the skipped region (every non-empty group not in the exact set,
 * M keys): if M == 0 nothing; if M <= m every skipped key once, offset 0;
 * otherwise m i.i.d. draws with replacement.  A draw picks group j with
 * probability W_j / T (W_j = n_j u_j, T = sum W) and a key uniformly inside it,
 * so the per-key probability is p = u_j / T and the logit offset is
 * ln(1 / (m p)) = ln T - ln u_j - ln m, which makes the exp-weighted sums over
 * the sample unbiased estimates of the sums over the skipped region.
 *
 * u_ij ~ exp(S_ij - Smax_i) quantised on a 2^(-1/256) grid with floor 1
 * (importance mode), u = 1 (uniform mode).  Draw t uses Philox4x64-10 with
 * key (seed, call_id) and counter (floor(t/2) + 1, i, h, b); words 2(t%2) and
 * 2(t%2)+1 form a 128-bit uniform r, z = floor(r T / 2^128). */
static int g_cmp_mode;            /* set before qsort; qsort here is serial */
static const float *g_cmp_S;      /* scores, or pi for the top-p rule */
static const int32_t *g_cmp_V;
static int cmp_rank(const void *a, const void *b)
{
    int ja = *(const int *)a, jb = *(const int *)b;
    if (g_cmp_mode == 2 && g_cmp_V[ja] != g_cmp_V[jb]) return g_cmp_V[ja] > g_cmp_V[jb] ? -1 : 1;
    if (g_cmp_S[ja] != g_cmp_S[jb]) return g_cmp_S[ja] > g_cmp_S[jb] ? -1 : 1;
    return ja < jb ? -1 : (ja > jb ? 1 : 0);
}

static uint64_t draw_z(uint64_t seed, uint64_t call_id, int b, int h, int i, int64_t t, uint64_t T)
{
    uint64_t ctr[4] = {(uint64_t)(t / 2) + 1, (uint64_t)i, (uint64_t)h, (uint64_t)b};
    uint64_t key[2] = {seed, call_id};
    uint64_t w[4];
    orc_philox4x64_10(ctr, key, w);
    uint64_t rhi = w[2 * (t % 2)], rlo = w[2 * (t % 2) + 1];
    /* floor((rhi * 2^64 + rlo) * T / 2^128) */
    unsigned __int128 a = (unsigned __int128)rhi * T;
    unsigned __int128 c = (unsigned __int128)rlo * T;
    unsigned __int128 mid = (unsigned __int128)(uint64_t)a + (uint64_t)(c >> 64);
    return (uint64_t)(a >> 64) + (uint64_t)(mid >> 64);
}

/* Exact set, then the sample.  Budget rule (pi == NULL), [B], [F3](c): groups by
 * (S desc, j asc) -- (votes desc, S desc, j asc) in votes mode -- the first
 * always, then while the running key count stays <= exact_keys.  Top-p rule
 * (pi != NULL; the SVG2-style sizing that [B] allows, since the method wraps any
 * block-sparse selector): groups by (pi desc, j asc), taken one by one until the
 * fp64 running sum of pi, added in that order, reaches top_p. */
static void select_core(const float *scores, const float *pi, double top_p, const int32_t *k_offsets,
                        const int32_t *votes, int B, int H, int Cq, int Ck, int exact_keys, int m, int mode,
                        uint64_t seed, uint64_t call_id, int32_t *exact_groups, int32_t *n_exact,
                        int32_t *sample_idx, float *sample_bias, int32_t *n_sample)
{
    uint32_t tbl[256];
    orc_proposal_table(tbl);
    int *order = (int *)malloc(sizeof(int) * Ck);
    int *taken = (int *)malloc(sizeof(int) * Ck);
    uint64_t *W = (uint64_t *)malloc(sizeof(uint64_t) * Ck);
    uint64_t *U = (uint64_t *)malloc(sizeof(uint64_t) * Ck);
    for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
        int64_t bh = (int64_t)b * H + h;
        const int32_t *ko = k_offsets + bh * (Ck + 1);
        for (int i = 0; i < Cq; ++i) {
            int64_t gi = bh * Cq + i;
            const float *S = scores + gi * Ck;
            int n_ne = 0;
            for (int j = 0; j < Ck; ++j)
                if (ko[j + 1] > ko[j]) order[n_ne++] = j;
            g_cmp_mode = mode; g_cmp_S = pi ? pi + gi * Ck : S; g_cmp_V = votes ? votes + gi * Ck : NULL;
            qsort(order, (size_t)n_ne, sizeof(int), cmp_rank);
            memset(taken, 0, sizeof(int) * Ck);
            if (pi) {
                double mass = 0.0;
                for (int p = 0; p < n_ne; ++p) {
                    int j = order[p];
                    taken[j] = 1;
                    mass += (double)pi[gi * Ck + j];
                    if (mass >= top_p) break;
                }
            } else {
                int64_t cum = 0;
                for (int p = 0; p < n_ne; ++p) {
                    int j = order[p];
                    int nj = ko[j + 1] - ko[j];
                    if (p > 0 && cum + nj > exact_keys) break;
                    cum += nj;
                    taken[j] = 1;
                }
            }
            int ne = 0;
            int32_t *eg = exact_groups + gi * Ck;
            for (int j = 0; j < Ck; ++j) eg[j] = -1;
            for (int j = 0; j < Ck; ++j) if (taken[j]) eg[ne++] = j;
            n_exact[gi] = ne;

            int64_t M = 0;
            float smax = -INFINITY;
            for (int j = 0; j < Ck; ++j)
                if (ko[j + 1] > ko[j] && !taken[j]) {
                    M += ko[j + 1] - ko[j];
                    if (S[j] > smax) smax = S[j];
                }
            int32_t *si = sample_idx + gi * (int64_t)m;
            float *sb = sample_bias + gi * (int64_t)m;
            if (M == 0) { n_sample[gi] = 0; continue; }
            if (M <= m) {
                int64_t t = 0;
                for (int j = 0; j < Ck; ++j)
                    if (ko[j + 1] > ko[j] && !taken[j])
                        for (int r = ko[j]; r < ko[j + 1]; ++r) { si[t] = r; sb[t] = 0.0f; ++t; }
                n_sample[gi] = (int32_t)M;
                continue;
            }
            uint64_t T = 0;
            for (int j = 0; j < Ck; ++j) {
                W[j] = 0; U[j] = 0;
                if (!(ko[j + 1] > ko[j]) || taken[j]) continue;
                uint64_t u = 1;
                if (mode != 1) {
                    float diff = smax - S[j];
                    float prod = diff * 369.32993f;      /* 256 * log2(e) */
                    float rr = rintf(prod);
                    int a = (int)rr;
                    if (a < 0) a = 0;
                    if (a > 7936) a = 7936;
                    int sh = a >> 8;
                    if (sh > 31) sh = 31;
                    u = (uint64_t)(tbl[a & 255] >> sh);
                    if (u < 1) u = 1;
                }
                U[j] = u;
                W[j] = (uint64_t)(ko[j + 1] - ko[j]) * u;
                T += W[j];
            }
            double lnT = log((double)T), lnm = log((double)m);
            for (int64_t t = 0; t < m; ++t) {
                uint64_t z = draw_z(seed, call_id, b, h, i, t, T);
                uint64_t P = 0;
                int j = 0;
                for (j = 0; j < Ck; ++j) {
                    if (W[j] == 0) continue;
                    if (z < P + W[j]) break;
                    P += W[j];
                }
                si[t] = ko[j] + (int32_t)((z - P) / U[j]);
                sb[t] = (float)(lnT - log((double)U[j]) - lnm);
            }
            n_sample[gi] = m;
        }
    }
    free(order); free(taken); free(W); free(U);
}

void orc_select_sample(const float *scores, const int32_t *k_offsets, const int32_t *votes,
                       int B, int H, int Cq, int Ck, int N, int exact_keys, int m, int mode,
                       uint64_t seed, uint64_t call_id, int32_t *exact_groups, int32_t *n_exact,
                       int32_t *sample_idx, float *sample_bias, int32_t *n_sample)
{
    (void)N;
    select_core(scores, NULL, 0.0, k_offsets, votes, B, H, Cq, Ck, exact_keys, m, mode, seed, call_id,
                exact_groups, n_exact, sample_idx, sample_bias, n_sample);
}

void orc_select_sample_topp(const float *scores, const float *pi, const int32_t *k_offsets, int B, int H,
                            int Cq, int Ck, int N, float top_p, int m, int mode, uint64_t seed,
                            uint64_t call_id, int32_t *exact_groups, int32_t *n_exact, int32_t *sample_idx,
                            float *sample_bias, int32_t *n_sample)
{
    (void)N;
    select_core(scores, pi, (double)top_p, k_offsets, NULL, B, H, Cq, Ck, 0, m, mode, seed, call_id,
                exact_groups, n_exact, sample_idx, sample_bias, n_sample);
}

/* ------------------------------------------------------------------------- */
/* Attention over the exact + sampled columns of a query group, [A], [F3](d).
 * For query row r of group i the columns are every key of every exact group
 * (offset 0) followed by the samples (row k_t, offset b_t):
 *   l = scale * <q_r, k> + offset,  O_r = sum e^l v / sum e^l,  LSE_r = ln sum e^l.
 * fp64 throughout; group_mask (nullable, [B,H,Cq]) restricts the work to some groups. */
static void attend_row(const float *q, const float *kh, const float *vh, int d, double scale,
                       const int32_t *cols, const float *offs, int64_t ncol, double *o, double *lse,
                       double *l)
{
    double mu = -INFINITY;
    for (int64_t c = 0; c < ncol; ++c) {
        const float *k = kh + (int64_t)cols[c] * d;
        double s = 0.0;
        for (int e = 0; e < d; ++e) s += (double)q[e] * (double)k[e];
        l[c] = scale * s + (offs ? (double)offs[c] : 0.0);
        if (l[c] > mu) mu = l[c];
    }
    double D = 0.0;
    for (int e = 0; e < d; ++e) o[e] = 0.0;
    for (int64_t c = 0; c < ncol; ++c) {
        double w = exp(l[c] - mu);
        D += w;
        const float *v = vh + (int64_t)cols[c] * d;
        for (int e = 0; e < d; ++e) o[e] += w * (double)v[e];
    }
    for (int e = 0; e < d; ++e) o[e] /= D;
    *lse = mu + log(D);
}

void orc_attention(const float *q_p, const float *k_p, const float *v_p, int B, int H, int N,
                   int d, int Cq, int Ck, const int32_t *q_offsets, const int32_t *k_offsets,
                   const int32_t *exact_groups, const int32_t *n_exact, const int32_t *sample_idx,
                   const float *sample_bias, const int32_t *n_sample, int m, float scale,
                   const uint8_t *group_mask, double *o_p, double *lse_p)
{
    int64_t G = (int64_t)B * H * Cq;
    #pragma omp parallel for schedule(dynamic)
    for (int64_t gi = 0; gi < G; ++gi) {
        if (group_mask && !group_mask[gi]) continue;
        int64_t bh = gi / Cq;
        int i = (int)(gi % Cq);
        const int32_t *qo = q_offsets + bh * (Cq + 1);
        const int32_t *ko = k_offsets + bh * (Ck + 1);
        if (qo[i + 1] == qo[i]) continue;
        int64_t ncol = 0;
        for (int e = 0; e < n_exact[gi]; ++e) {
            int j = exact_groups[gi * Ck + e];
            ncol += ko[j + 1] - ko[j];
        }
        ncol += n_sample[gi];
        int32_t *cols = (int32_t *)malloc(sizeof(int32_t) * (size_t)(ncol + 1));
        float *offs = (float *)malloc(sizeof(float) * (size_t)(ncol + 1));
        double *l = (double *)malloc(sizeof(double) * (size_t)(ncol + 1));
        int64_t c = 0;
        for (int e = 0; e < n_exact[gi]; ++e) {
            int j = exact_groups[gi * Ck + e];
            for (int r = ko[j]; r < ko[j + 1]; ++r) { cols[c] = r; offs[c] = 0.0f; ++c; }
        }
        for (int t = 0; t < n_sample[gi]; ++t) {
            cols[c] = sample_idx[gi * (int64_t)m + t];
            offs[c] = sample_bias[gi * (int64_t)m + t];
            ++c;
        }
        const float *kh = k_p + bh * (int64_t)N * d, *vh = v_p + bh * (int64_t)N * d;
        for (int r = qo[i]; r < qo[i + 1]; ++r)
            attend_row(q_p + (bh * N + r) * (int64_t)d, kh, vh, d, (double)scale, cols, offs, ncol,
                       o_p + (bh * N + r) * (int64_t)d, lse_p + bh * N + r, l);
        free(cols); free(offs); free(l);
    }
}

/* Textbook softmax attention over every key with no offset (the all-selected case).
 * rows (nullable) restricts the work to rows[0..nrows) of every head. */
void orc_dense(const float *q, const float *k, const float *v, int B, int H, int N, int d,
               float scale, const int32_t *rows, int nrows, double *o, double *lse)
{
    int64_t R = rows ? nrows : N;
    int32_t *cols = (int32_t *)malloc(sizeof(int32_t) * (size_t)N);
    for (int c = 0; c < N; ++c) cols[c] = c;
    #pragma omp parallel
    {
        double *l = (double *)malloc(sizeof(double) * (size_t)N);
        #pragma omp for schedule(static) collapse(2)
        for (int64_t bh = 0; bh < (int64_t)B * H; ++bh)
            for (int64_t rr = 0; rr < R; ++rr) {
                int64_t r = rows ? rows[rr] : rr;
                attend_row(q + (bh * N + r) * (int64_t)d, k + bh * (int64_t)N * d,
                           v + bh * (int64_t)N * d, d, (double)scale, cols, NULL, N,
                           o + (bh * R + rr) * (int64_t)d, lse + bh * R + rr, l);
            }
        free(l);
    }
    free(cols);
}

/* Output rows back to token order: o[perm_q[r]] = o_p[r] (and the LSE). */
void orc_unpermute(const double *o_p, const double *lse_p, const int32_t *perm_q, int B, int H,
                   int N, int d, double *o, double *lse)
{
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh)
        for (int r = 0; r < N; ++r) {
            int64_t dst = bh * N + perm_q[bh * N + r];
            memcpy(o + dst * d, o_p + (bh * N + r) * (int64_t)d, sizeof(double) * d);
            if (lse && lse_p) lse[dst] = lse_p[bh * N + r];
        }
}

/* ------------------------------------------------------------------------- */
/* Product-quantised per-query voting, [A] (queries and keys are product-
 * quantised so that every query, not only the centroid, can afford its own
 * block scores; each query picks its top blocks and the group keeps the blocks
 * picked most often).  The pages
 * give no formula; the reading taken (parity unpinned by the pages):
 *   codes: k-means of each d/P-dim subspace into Cc codewords (as orc_cluster);
 *   Kbar_{j,s} = mean over the keys of group j of their subspace-s codeword;
 *   M_s[a][j]  = scale * <cw^q_{s,a}, Kbar_{j,s}>   (fp32 fma chain over the dims);
 *   score(q,j) = sum_s M_s[code_s(q)][j]           (fp32, s ascending);
 *   each query ranks the non-empty key groups by (score desc, j asc), takes the
 *   first always and the following ones while the key count stays <= exact_keys
 *   (the exact-set rule), and votes for every group it takes;
 *   votes[i][j] = number of queries of group i that voted for j.
 * Layouts: codes [P,B,H,N] (token order), codebooks [P,B,H,Cc,ds], ds = d/P. */
void orc_pq_kbar(const int32_t *k_codes, const float *k_cb, const int32_t *perm_k, const int32_t *k_offsets,
                 int B, int H, int N, int P, int Cc, int ds, int Ck, float *kbar)
{
    int d = P * ds;
    double *acc = (double *)malloc(sizeof(double) * (size_t)d);
    for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
        int64_t bh = (int64_t)b * H + h;
        const int32_t *ko = k_offsets + bh * (Ck + 1);
        for (int j = 0; j < Ck; ++j) {
            for (int e = 0; e < d; ++e) acc[e] = 0.0;
            int n = ko[j + 1] - ko[j];
            for (int r = ko[j]; r < ko[j + 1]; ++r) {
                int t = perm_k[bh * N + r];
                for (int s = 0; s < P; ++s) {
                    int code = k_codes[(((int64_t)s * B + b) * H + h) * N + t];
                    const float *cw = k_cb + ((((int64_t)s * B + b) * H + h) * Cc + code) * ds;
                    for (int e = 0; e < ds; ++e) acc[s * ds + e] += (double)cw[e];
                }
            }
            float *out = kbar + (bh * Ck + j) * d;
            for (int e = 0; e < d; ++e) out[e] = n > 0 ? (float)(acc[e] / n) : 0.0f;
        }
    }
    free(acc);
}

void orc_pq_tables(const float *q_cb, const float *kbar, int B, int H, int P, int Cc, int ds, int Ck,
                   float scale, float *tables)
{
    int d = P * ds;
    for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
        int64_t bh = (int64_t)b * H + h;
        for (int s = 0; s < P; ++s)
            for (int a = 0; a < Cc; ++a) {
                const float *cw = q_cb + ((((int64_t)s * B + b) * H + h) * Cc + a) * ds;
                for (int j = 0; j < Ck; ++j) {
                    const float *kb = kbar + (bh * Ck + j) * d + s * ds;
                    float acc = 0.0f;
                    for (int e = 0; e < ds; ++e) acc = fmaf(cw[e], kb[e], acc);
                    tables[(((bh * P + s) * Cc) + a) * Ck + j] = acc * scale;
                }
            }
    }
}

static const float *g_vote_score;
static int cmp_vote(const void *a, const void *b)
{
    int ja = *(const int *)a, jb = *(const int *)b;
    if (g_vote_score[ja] != g_vote_score[jb]) return g_vote_score[ja] > g_vote_score[jb] ? -1 : 1;
    return ja < jb ? -1 : (ja > jb ? 1 : 0);
}

void orc_pq_votes(const int32_t *q_codes, const float *tables, const int32_t *perm_q, const int32_t *q_offsets,
                  const int32_t *k_offsets, int B, int H, int N, int P, int Cc, int Cq, int Ck, int exact_keys,
                  int32_t *votes)
{
    float *score = (float *)malloc(sizeof(float) * Ck);
    int *order = (int *)malloc(sizeof(int) * Ck);
    for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
        int64_t bh = (int64_t)b * H + h;
        const int32_t *qo = q_offsets + bh * (Cq + 1);
        const int32_t *ko = k_offsets + bh * (Ck + 1);
        for (int i = 0; i < Cq; ++i) {
            int32_t *vi = votes + (bh * Cq + i) * Ck;
            for (int j = 0; j < Ck; ++j) vi[j] = 0;
            for (int r = qo[i]; r < qo[i + 1]; ++r) {
                int t = perm_q[bh * N + r];
                for (int j = 0; j < Ck; ++j) {
                    float acc = 0.0f;
                    for (int s = 0; s < P; ++s) {
                        int code = q_codes[(((int64_t)s * B + b) * H + h) * N + t];
                        acc += tables[(((bh * P + s) * Cc) + code) * Ck + j];
                    }
                    score[j] = acc;
                }
                int n_ne = 0;
                for (int j = 0; j < Ck; ++j)
                    if (ko[j + 1] > ko[j]) order[n_ne++] = j;
                g_vote_score = score;
                qsort(order, (size_t)n_ne, sizeof(int), cmp_vote);
                int64_t cum = 0;
                for (int p = 0; p < n_ne; ++p) {
                    int j = order[p];
                    int nj = ko[j + 1] - ko[j];
                    if (p > 0 && cum + nj > exact_keys) break;
                    cum += nj;
                    vi[j] += 1;
                }
            }
        }
    }
    free(score);
    free(order);
}
