/*
 * oracle.c -- plain, slow fp64 CPU reference for dense descriptor matching.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library. The product (the HIP
 * library and its Python binding) never calls it and shares no code with it.
 *
 * Sources (cited by page title and section):
 *  [MASt3R-note]  "MASt3R" (Leroy 2024) note on cv-learn.com, section
 *                 手法とアーキテクチャ: the matching-head paragraph (unit-norm
 *                 D1, D2 in R^{H x W x d}) and the 高速相互マッチング(FRM)
 *                 paragraph (reciprocal set M, grid seeds, NN round trips
 *                 U^t -> V^t -> U^{t+1}, keep converged cycles, O(kWH)).
 *  [FRM-listing]  "DUSt3R和MASt3R论文阅读" (Staskaer blog), section
 *                 "MASt3R matching": the quoted fast_reciprocal_NNs routine
 *                 from MASt3R-SfM (seed grid, not-yet-converged mask,
 *                 forward/backward queries, tests against the previous
 *                 iteration, max_iter, converged = not active, merge).
 *
 * Readings where the pages leave a step open:
 *  - NN(x) is the argmax of the dot product over ALL pixels of the other map,
 *    lowest index on ties (the pages' matcher is a brute-force distance
 *    matcher; for unit vectors ||a-b||^2 = 2 - 2 a.b).
 *  - Arithmetic: stored values are decoded exactly to double, scores are
 *    accumulated in double in component order c = 0..d-1.
 *  - "margin" of a query = best score minus the best score over the other
 *    indices (0 for exact duplicates).
 *
 * Every function below is pinned by the CPU tests against numpy's argmax on the
 * full score matrix, closed forms (seed counts, identity and pure-shift maps),
 * a hand-worked trajectory fixture and invariants (reciprocity, FRM within M,
 * symmetry of M); see tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* IEEE 754 binary16: sign, 5-bit exponent (bias 15), 10-bit fraction. */
static double half_to_double(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* zero / subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);    /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32 pattern. */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Decode n stored elements into doubles (exact for all three formats). */
int orc_decode(const void *src, int dtype, int64_t n, double *out)
{
    if (dtype == ORC_F32) {
        const float *s = (const float *)src;
        for (int64_t i = 0; i < n; ++i) out[i] = (double)s[i];
    } else if (dtype == ORC_F16) {
        const uint16_t *s = (const uint16_t *)src;
        for (int64_t i = 0; i < n; ++i) out[i] = half_to_double(s[i]);
    } else if (dtype == ORC_BF16) {
        const uint16_t *s = (const uint16_t *)src;
        for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_double(s[i]);
    } else {
        return -1;
    }
    return 0;
}

/* score(a, b) = sum_c a[c] * b[c], in double, c ascending. */
static double dot(const double *a, const double *b, int d)
{
    double s = 0.0;
    for (int c = 0; c < d; ++c) s += a[c] * b[c];
    return s;
}

/* Score of the Euclidean metric: minus the squared distance, in double, c
 * ascending, so that the nearest point is the one of maximum score. The pages
 * match 3D points (d = 3) by this distance ("DUSt3R和MASt3R论文阅读", section
 * MASt3R matching: K-d trees for x in R^3). */
static double neg_sqdist(const double *a, const double *b, int d)
{
    double s = 0.0;
    for (int c = 0; c < d; ++c) {
        const double t = a[c] - b[c];
        s -= t * t;
    }
    return s;
}

enum { ORC_DOT = 0, ORC_L2 = 1 };

/* Brute-force NN of one query over all n rows of R: the smallest index that
 * attains the maximum score, the maximum s1 and the best score s2 over every
 * other index (s2 == s1 when the maximum is attained twice). The score is the
 * dot product (ORC_DOT) or minus the squared Euclidean distance (ORC_L2). */
static void nn_one_m(const double *q, const double *R, int64_t n, int d, int metric,
                     int32_t *idx, double *s1, double *s2)
{
    int32_t best = -1;
    double b1 = -INFINITY, b2 = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double s = metric == ORC_L2 ? neg_sqdist(q, R + j * d, d) : dot(q, R + j * d, d);
        if (s > b1) { b2 = b1; b1 = s; best = (int32_t)j; }
        else if (s > b2) { b2 = s; }
    }
    *idx = best; *s1 = b1; *s2 = b2;
}

static void nn_one(const double *q, const double *R, int64_t n, int d, int32_t *idx, double *s1, double *s2)
{
    nn_one_m(q, R, n, d, ORC_DOT, idx, s1, s2);
}

/* NN for a list of queries: row qrows[a] of Q (or row a when qrows is NULL). */
void orc_nn_m(const double *Q, const int32_t *qrows, int64_t nq,
              const double *R, int64_t nr, int d, int metric,
              int32_t *idx, double *s1, double *s2)
{
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t a = 0; a < nq; ++a) {
        int64_t r = qrows ? qrows[a] : a;
        nn_one_m(Q + r * d, R, nr, d, metric, &idx[a], &s1[a], &s2[a]);
    }
}

void orc_nn(const double *Q, const int32_t *qrows, int64_t nq,
            const double *R, int64_t nr, int d,
            int32_t *idx, double *s1, double *s2)
{
    orc_nn_m(Q, qrows, nq, R, nr, d, ORC_DOT, idx, s1, s2);
}

/* Seed grid [FRM-listing]: rows y = S/2, S/2 + S, ... < H and columns
 * x = S/2, S/2 + S, ... < W, linear index p = x + W*y, unique and ascending.
 * Returns k; writes the indices when out != NULL. */
int64_t orc_seed_grid(int H, int W, int S, int32_t *out)
{
    int64_t k = 0;
    if (S <= 0) return -1;
    for (int y = S / 2; y < H; y += S)
        for (int x = S / 2; x < W; x += S) {
            if (out) out[k] = x + W * y;
            ++k;
        }
    return k;
}

/* Fast Reciprocal Matching [MASt3R-note, FRM-listing].
 *
 * State per seed a: u[a] (pixel of image 1), v[a] (pixel of image 2, -1
 * before the first query), the copies u_old / v_old kept from the previous
 * iteration, and the not-yet-converged flag.
 *
 * One iteration:
 *   forward : for each active a, v[a] <- NN2(D1[u[a]]);
 *             a stays active only if v[a] differs from v_old[a];
 *   backward: for each still-active a, u[a] <- NN1(D2[v[a]]);
 *             a stays active only if u[a] differs from u_old[a];
 *   count the iteration; stop once max_iter iterations have run;
 *   otherwise v_old <- v, u_old <- u.
 * The loop also stops as soon as no seed is active. Converged = not active.
 *
 * Extra per-seed outputs for checking: score[a] = score(u[a], v[a]) as found
 * by the last forward query; conv_iter[a] = iteration in which a stopped being
 * active (-1 if never); ambiguous[a] = 1 if any query on a's path had a
 * margin below tau; n_fwd[t] / n_bwd[t] (when not NULL, max_iter entries) =
 * number of forward / backward queries made in iteration t + 1, i.e. the work
 * the loop does. Returns the number of iterations run.
 *
 * Options of the same routine [FRM-listing]:
 *   fwd_test = 0  (the basin variant): the forward test is skipped, so a seed
 *                 only stops when its backward query returns the pixel it
 *                 started the iteration from;
 *   basin         (NULL or int32[N1], filled with -1 by the caller): every
 *                 backward query of an active seed records, at the pixel the
 *                 seed occupied before the query (u_old), the pixel it moved
 *                 to;
 *   u_old_out     (NULL or int32[k]): the u_old copies as they stand when the
 *                 loop ends -- u at the start of the last iteration if the
 *                 loop stopped at max_iter, the final u if it stopped because
 *                 no seed was active (the copy is refreshed after every
 *                 iteration that does not hit max_iter). */
int orc_frm_ex(const double *D1, int64_t N1, const double *D2, int64_t N2, int d, int metric,
               const int32_t *seeds, int64_t k, int max_iter, double tau, int fwd_test,
               int32_t *basin, int32_t *u_old_out,
               int32_t *u, int32_t *v, double *score, int32_t *conv_iter,
               uint8_t *active, uint8_t *ambiguous, int64_t *n_fwd, int64_t *n_bwd)
{
    int32_t *u_old = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k ? k : 1));
    int32_t *v_old = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k ? k : 1));
    if (!u_old || !v_old) { free(u_old); free(v_old); return -1; }
    for (int64_t a = 0; a < k; ++a) {
        u[a] = seeds[a]; v[a] = -1;
        u_old[a] = u[a]; v_old[a] = v[a];
        active[a] = 1; conv_iter[a] = -1; ambiguous[a] = 0; score[a] = NAN;
    }
    for (int t = 0; t < max_iter; ++t) {
        if (n_fwd) n_fwd[t] = 0;
        if (n_bwd) n_bwd[t] = 0;
    }
    int niter = 0;
    for (;;) {
        int64_t n_active = 0;
        for (int64_t a = 0; a < k; ++a) n_active += active[a];
        if (n_active == 0) break;
        if (n_fwd) n_fwd[niter] = n_active;

        /* forward queries: image 1 -> image 2 */
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t a = 0; a < k; ++a) {
            if (!active[a]) continue;
            int32_t j; double s1, s2;
            nn_one_m(D1 + (int64_t)u[a] * d, D2, N2, d, metric, &j, &s1, &s2);
            v[a] = j; score[a] = s1;
            if (s1 - s2 < tau) ambiguous[a] = 1;
        }
        for (int64_t a = 0; a < k; ++a)
            if (fwd_test && active[a] && v[a] == v_old[a]) { active[a] = 0; conv_iter[a] = niter + 1; }

        /* backward queries: image 2 -> image 1 */
        if (n_bwd)
            for (int64_t a = 0; a < k; ++a) n_bwd[niter] += active[a];
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t a = 0; a < k; ++a) {
            if (!active[a]) continue;
            int32_t i; double s1, s2;
            nn_one_m(D2 + (int64_t)v[a] * d, D1, N1, d, metric, &i, &s1, &s2);
            u[a] = i;
            if (s1 - s2 < tau) ambiguous[a] = 1;
        }
        if (basin)
            for (int64_t a = 0; a < k; ++a)
                if (active[a]) basin[u_old[a]] = u[a];
        for (int64_t a = 0; a < k; ++a)
            if (active[a] && u[a] == u_old[a]) { active[a] = 0; conv_iter[a] = niter + 1; }

        niter += 1;
        if (niter >= max_iter) break;
        for (int64_t a = 0; a < k; ++a) { v_old[a] = v[a]; u_old[a] = u[a]; }
    }
    if (u_old_out)
        for (int64_t a = 0; a < k; ++a) u_old_out[a] = u_old[a];
    free(u_old); free(v_old);
    return niter;
}

/* The grid-seed routine with its defaults: forward test on, no basin. */
int orc_frm(const double *D1, int64_t N1, const double *D2, int64_t N2, int d,
            const int32_t *seeds, int64_t k, int max_iter, double tau,
            int32_t *u, int32_t *v, double *score, int32_t *conv_iter,
            uint8_t *active, uint8_t *ambiguous, int64_t *n_fwd, int64_t *n_bwd)
{
    return orc_frm_ex(D1, N1, D2, N2, d, ORC_DOT, seeds, k, max_iter, tau, 1, NULL, NULL, u, v, score, conv_iter,
                      active, ambiguous, n_fwd, n_bwd);
}

/* Which seeds the routine keeps, and the image-1 pixel it reports for each
 * [FRM-listing, end of the routine]:
 *   pixel_tol == 0: kept = not active at exit; reported pixel = u;
 *   pixel_tol >  0: kept = the Euclidean distance, in pixels of the W1-wide
 *                   image, between u_old (as the loop left it) and u is below
 *                   pixel_tol; reported pixel = u_old when report_old (seeds
 *                   given as explicit starts), else u. */
void orc_frm_select(const int32_t *u, const int32_t *u_old, const uint8_t *active, int64_t k, int W1,
                    double pixel_tol, int report_old, uint8_t *keep, int32_t *rep_i)
{
    for (int64_t a = 0; a < k; ++a) {
        if (pixel_tol > 0) {
            const double dy = (double)(u_old[a] / W1 - u[a] / W1);
            const double dx = (double)(u_old[a] % W1 - u[a] % W1);
            keep[a] = sqrt(dy * dy + dx * dx) < pixel_tol;
            rep_i[a] = report_old ? u_old[a] : u[a];
        } else {
            keep[a] = !active[a];
            rep_i[a] = u[a];
        }
    }
}

static int cmp_pair(const void *pa, const void *pb)
{
    const int64_t *a = (const int64_t *)pa, *b = (const int64_t *)pb;
    if (a[0] != b[0]) return a[0] < b[0] ? -1 : 1;
    if (a[1] != b[1]) return a[1] < b[1] ? -1 : 1;
    return 0;
}

/* Collect the converged seeds' (u, v, score) into unique pairs sorted by u
 * (then v) -- the "keep unique correspondences, sorted by the image-1
 * index" step that closes [FRM-listing]. Returns the pair count. */
int64_t orc_merge(const int32_t *u, const int32_t *v, const double *score, const uint8_t *active,
                  int64_t k, int32_t *out_i, int32_t *out_j, double *out_s)
{
    int64_t *buf = (int64_t *)malloc(sizeof(int64_t) * 3 * (size_t)(k ? k : 1));
    if (!buf) return -1;
    int64_t m = 0;
    for (int64_t a = 0; a < k; ++a) {
        if (active[a]) continue;
        buf[3 * m] = u[a]; buf[3 * m + 1] = v[a];
        memcpy(&buf[3 * m + 2], &score[a], sizeof(double));
        ++m;
    }
    qsort(buf, (size_t)m, 3 * sizeof(int64_t), cmp_pair);
    int64_t n = 0;
    for (int64_t t = 0; t < m; ++t) {
        if (n > 0 && buf[3 * t] == out_i[n - 1] && buf[3 * t + 1] == out_j[n - 1]) continue;
        out_i[n] = (int32_t)buf[3 * t]; out_j[n] = (int32_t)buf[3 * t + 1];
        memcpy(&out_s[n], &buf[3 * t + 2], sizeof(double));
        ++n;
    }
    free(buf);
    return n;
}

/* Exhaustive reciprocal (mutual) nearest neighbours [MASt3R-note]:
 * M = {(i, j) : j = NN2(D1_i) and i = NN1(D2_j)}, ascending in i.
 * nn12 / s12 / m12 (size N1) and nn21 / s21 / m21 (size N2) receive both NN
 * tables with scores and margins. Returns |M|. */
int64_t orc_mutual_m(const double *D1, int64_t N1, const double *D2, int64_t N2, int d, int metric,
                     int32_t *nn12, double *s12, double *m12,
                     int32_t *nn21, double *s21, double *m21,
                     int32_t *out_i, int32_t *out_j, double *out_s)
{
    double *t1 = (double *)malloc(sizeof(double) * (size_t)(N1 > N2 ? N1 : N2));
    if (!t1) return -1;
    orc_nn_m(D1, NULL, N1, D2, N2, d, metric, nn12, s12, t1);
    for (int64_t i = 0; i < N1; ++i) m12[i] = s12[i] - t1[i];
    orc_nn_m(D2, NULL, N2, D1, N1, d, metric, nn21, s21, t1);
    for (int64_t j = 0; j < N2; ++j) m21[j] = s21[j] - t1[j];
    free(t1);
    int64_t n = 0;
    for (int64_t i = 0; i < N1; ++i) {
        int32_t j = nn12[i];
        if (nn21[j] == (int32_t)i) {
            out_i[n] = (int32_t)i; out_j[n] = j; out_s[n] = s12[i];
            ++n;
        }
    }
    return n;
}

int64_t orc_mutual(const double *D1, int64_t N1, const double *D2, int64_t N2, int d,
                   int32_t *nn12, double *s12, double *m12,
                   int32_t *nn21, double *s21, double *m21,
                   int32_t *out_i, int32_t *out_j, double *out_s)
{
    return orc_mutual_m(D1, N1, D2, N2, d, ORC_DOT, nn12, s12, m12, nn21, s21, m21, out_i, out_j, out_s);
}
