/*
 * Oracle: the building blocks of the decoder layers around the link step, in fp64 with explicit
 * loops.
 *
 * TEST INFRASTRUCTURE ONLY. Compiled into the checker library that tests, the smoke check and the
 * benchmark's CPU-baseline leg call; the product path never links or loads it, and it shares no
 * code with it.
 *
 *   oracle_linear   out[i][j] = sum_k a[i][k] * w[j][k]      (a [m][k], w [n][k]: y = a W^T)
 *   oracle_rmsnorm  out[i][e] = x[i][e] / sqrt(mean_e x[i][e]^2 + eps) * w[e]
 *
 * The recomputed rows run through a Llama-class decoder layer at link time (EPIC, atlas.scime.ai
 * summary, "Approach", "Key results" and "Limitations": 7-9B models); oracle/model.py composes
 * the layer from these and the oracle link attention.
 */
#include <math.h>
#include <stdint.h>

void oracle_linear(int m, int n, int k, const double *a, const double *w, double *out)
{
    #pragma omp parallel for schedule(static)
    for (int i = 0; i < m; ++i)
        for (int j = 0; j < n; ++j) {
            double s = 0.0;
            for (int t = 0; t < k; ++t)
                s += a[(int64_t)i * k + t] * w[(int64_t)j * k + t];
            out[(int64_t)i * n + j] = s;
        }
}

void oracle_rmsnorm(int rows, int dm, const double *x, const double *w, double eps, double *out)
{
    #pragma omp parallel for schedule(static)
    for (int i = 0; i < rows; ++i) {
        double ss = 0.0;
        for (int e = 0; e < dm; ++e)
            ss += x[(int64_t)i * dm + e] * x[(int64_t)i * dm + e];
        const double inv = 1.0 / sqrt(ss / dm + eps);
        for (int e = 0; e < dm; ++e)
            out[(int64_t)i * dm + e] = x[(int64_t)i * dm + e] * inv * w[e];
    }
}
