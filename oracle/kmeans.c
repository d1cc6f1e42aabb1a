/* Lloyd k-means in double precision (oracle; test infrastructure only).
 *
 * Source: the Sparse-VideoGen project write-up, section "Three generations of
 * the same idea".  SVG2 clusters tokens for its semantic-aware permutation
 * and ships a batched flash k-means kernel.  The pages give no variant.
 * Reading: plain Lloyd iterations from caller-given initial centroids.
 *   Assign step: each point goes to the centroid at the smallest squared
 *   Euclidean distance, sum over c of (x_c - m_c)^2.  Ties go to the lowest
 *   centroid index.
 *   Update step: each centroid becomes the mean of its points.  A centroid
 *   with no points keeps its value.
 * There is no early stop.  The output is the assignment of the last
 * iteration, the centroids updated from it, and the cluster sizes.
 *
 * The assign step of each point is independent, so points are split across
 * threads.  Each distance is summed over c in index order.  Each mean is
 * summed over points in index order.  No sum is reordered.
 *
 * Decision audit (optional, min_f32_ratio != NULL).  A float32 evaluation of
 * a squared distance, as (x - m).(x - m) or as |m|^2 - 2 x.m plus |x|^2, with
 * m rounded to float32 and its sums taken in any order, is off by at most
 * B = (d + 4) u (|x|^2 + |m|^2 + 2 sum_c |x_c m_c|), u = 2^-24, to first
 * order in u (the standard
 * bound for a length-d dot product, gamma_d <= d u / (1 - d u), plus the
 * roundings of m, of |m|^2 and of the final combination).  The float32
 * argmin then equals this one whenever every other centroid j beats the
 * winner a by D_j - D_a > B_j + B_a.  The audit reports the smallest
 * (D_j - D_a) / (B_j + B_a) over all points, iterations and j != a; a
 * centroid whose row equals the winner's bit for bit is skipped (it ties in
 * every precision and the lower index wins on both sides).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <float.h>
#include <math.h>

int oracle_lloyd_kmeans(const double *x, int64_t n, int32_t d, int32_t k,
                        const int32_t *init_idx, int32_t iters,
                        int32_t *assign, double *centroids, int64_t *sizes,
                        double *min_rel_margin, double *min_f32_ratio)
{
    if (n <= 0 || d <= 0 || k <= 0 || iters < 1) return 1;
    for (int32_t j = 0; j < k; ++j) {
        if (init_idx[j] < 0 || init_idx[j] >= n) return 2;
        memcpy(centroids + (int64_t)j * d, x + (int64_t)init_idx[j] * d, sizeof(double) * d);
    }
    double *sums = (double *)malloc(sizeof(double) * (size_t)k * d);
    if (!sums) return 3;
    double margin = DBL_MAX, ratio = DBL_MAX;
    for (int32_t it = 0; it < iters; ++it) {
        double it_margin = DBL_MAX, it_ratio = DBL_MAX;
        #pragma omp parallel for schedule(static) reduction(min:it_margin, it_ratio)
        for (int64_t i = 0; i < n; ++i) {
            const double *xi = x + i * d;
            double best = DBL_MAX, second = DBL_MAX;
            int32_t arg = 0;
            for (int32_t j = 0; j < k; ++j) {
                const double *cj = centroids + (int64_t)j * d;
                double s = 0.0;
                for (int32_t c = 0; c < d; ++c) {
                    double diff = xi[c] - cj[c];
                    s += diff * diff;
                }
                if (s < best) { second = best; best = s; arg = j; }
                else if (s < second) { second = s; }
            }
            assign[i] = arg;
            double denom = best > 1e-300 ? best : 1e-300;
            double m = k > 1 ? (second - best) / denom : DBL_MAX;
            if (m < it_margin) it_margin = m;
            if (min_f32_ratio && k > 1) {
                const double u = 1.0 / 16777216.0;
                const double *ca = centroids + (int64_t)arg * d;
                double xx = 0.0, ba = 0.0;
                for (int32_t c = 0; c < d; ++c) xx += xi[c] * xi[c];
                for (int32_t c = 0; c < d; ++c) ba += ca[c] * ca[c] + 2.0 * fabs(xi[c] * ca[c]);
                ba = (d + 4) * u * (xx + ba);
                for (int32_t j = 0; j < k; ++j) {
                    if (j == arg) continue;
                    const double *cj = centroids + (int64_t)j * d;
                    if (memcmp(cj, ca, sizeof(double) * d) == 0) continue;
                    double dj = 0.0, bj = 0.0;
                    for (int32_t c = 0; c < d; ++c) {
                        double diff = xi[c] - cj[c];
                        dj += diff * diff;
                        bj += cj[c] * cj[c] + 2.0 * fabs(xi[c] * cj[c]);
                    }
                    bj = (d + 4) * u * (xx + bj);
                    double r = (dj - best) / (ba + bj);
                    if (r < it_ratio) it_ratio = r;
                }
            }
        }
        if (it_margin < margin) margin = it_margin;
        if (it_ratio < ratio) ratio = it_ratio;
        memset(sums, 0, sizeof(double) * (size_t)k * d);
        for (int32_t j = 0; j < k; ++j) sizes[j] = 0;
        for (int64_t i = 0; i < n; ++i) {
            int32_t a = assign[i];
            sizes[a] += 1;
            double *sa = sums + (int64_t)a * d;
            const double *xi = x + i * d;
            for (int32_t c = 0; c < d; ++c) sa[c] += xi[c];
        }
        for (int32_t j = 0; j < k; ++j) {
            if (sizes[j] == 0) continue;
            for (int32_t c = 0; c < d; ++c)
                centroids[(int64_t)j * d + c] = sums[(int64_t)j * d + c] / (double)sizes[j];
        }
    }
    free(sums);
    if (min_rel_margin) *min_rel_margin = margin;
    if (min_f32_ratio) *min_f32_ratio = ratio;
    return 0;
}
