/*
 * Oracle: causal RoPE attention of the recomputed rows over a linked cache,
 * in fp64 with explicit loops.
 *
 * TEST INFRASTRUCTURE ONLY. This file is compiled into a checker library that
 * tests, the smoke check and the benchmark's CPU-baseline leg call; the
 * product path never links or loads it, and it shares no code with it.
 *
 * What it computes (one request):
 *   - every key t carries an absolute position key_pos[t] in the linked
 *     prompt; every query row r carries row_pos[r];
 *   - keys are stored without positional encoding and rotary position
 *     embedding is applied at the linked position at attention time (MEPIC,
 *     searcharxiv.org abstract: positional encodings removed from stored KV,
 *     RoPE fused into attention): key t is rotated by key_rot[t], which is
 *     key_pos[t] for such a key (key_rot NULL); key_rot may be negative, a
 *     rotation by a negative angle. A key that already carries a
 *     rotation at its position s inside its segment, as a chunk compiled from
 *     position 0 leaves it (EPIC, atlas.scime.ai summary, "Approach"), is
 *     rotated by the segment's linked start instead; the two rotations
 *     compose to one at the key's absolute position;
 *   - rotation pairs dimension i with i + d/2 ("rotate half"), angle
 *     pos * theta^(-2i/d), no frequency scaling;
 *   - row r, query head h attends key head g = h / (Hq/Hkv) over every key
 *     with key_pos <= row_pos[r] (causal, inclusive); scores are the dot
 *     product of the rotated vectors divided by sqrt(d); softmax is formed in
 *     two passes (maximum, then exponentials), and the output is the
 *     softmax-weighted sum of the values;
 *   - lse = max + ln(sum of exponentials), the natural log of the softmax
 *     denominator of the scaled scores.
 * Which rows are recomputed and what the merged cache holds is decided by the
 * oracle planner (EPIC, atlas.scime.ai summary, "Approach").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

static void rotate(const double *x, double *y, int d, int64_t pos, const double *inv_freq)
{
    int half = d / 2;
    for (int i = 0; i < half; ++i) {
        double angle = (double)pos * inv_freq[i];
        double c = cos(angle);
        double s = sin(angle);
        y[i] = x[i] * c - x[i + half] * s;
        y[i + half] = x[i + half] * c + x[i] * s;
    }
}

/* Returns 0 on success, -1 on invalid arguments, -2 when memory runs out. */
int oracle_link_attention(int n_keys, int n_kv_heads, int n_q_heads, int head_dim,
                          const double *k, const double *v, const int64_t *key_pos,
                          const int64_t *key_rot, int n_rows, const double *q, const int64_t *row_pos,
                          double rope_theta, double *out, double *lse)
{
    if (n_keys < 0 || n_rows < 0 || n_kv_heads <= 0 || n_q_heads <= 0 || head_dim <= 0 ||
        head_dim % 2 != 0 || n_q_heads % n_kv_heads != 0 || rope_theta <= 0.0)
        return -1;
    if (n_rows == 0)
        return 0;
    const int d = head_dim;
    const int group = n_q_heads / n_kv_heads;
    double *inv_freq = malloc(sizeof(double) * (size_t)(d / 2));
    double *k_rot = malloc(sizeof(double) * ((size_t)n_keys * n_kv_heads * d + 1));
    if (!inv_freq || !k_rot) {
        free(inv_freq);
        free(k_rot);
        return -2;
    }
    for (int i = 0; i < d / 2; ++i)
        inv_freq[i] = pow(rope_theta, -2.0 * i / d);

    #pragma omp parallel for schedule(static)
    for (int t = 0; t < n_keys; ++t)
        for (int g = 0; g < n_kv_heads; ++g)
            rotate(k + ((size_t)t * n_kv_heads + g) * d, k_rot + ((size_t)t * n_kv_heads + g) * d,
                   d, key_rot ? key_rot[t] : key_pos[t], inv_freq);

    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    int failed = 0;
    #pragma omp parallel
    {
        double *scores = malloc(sizeof(double) * ((size_t)n_keys + 1));
        double *q_rot = malloc(sizeof(double) * (size_t)d);
        double *acc = malloc(sizeof(double) * (size_t)d);
        if (!scores || !q_rot || !acc) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for schedule(dynamic, 1)
        for (long item = 0; item < (long)n_rows * n_q_heads; ++item) {
            if (!scores || !q_rot || !acc)
                continue;
            int r = (int)(item / n_q_heads);
            int h = (int)(item % n_q_heads);
            int g = h / group;
            int64_t p = row_pos[r];
            rotate(q + ((size_t)r * n_q_heads + h) * d, q_rot, d, p, inv_freq);

            double m = -INFINITY;
            for (int t = 0; t < n_keys; ++t) {
                if (key_pos[t] > p)
                    continue;
                const double *kt = k_rot + ((size_t)t * n_kv_heads + g) * d;
                double s = 0.0;
                for (int e = 0; e < d; ++e)
                    s += q_rot[e] * kt[e];
                s *= inv_sqrt_d;
                scores[t] = s;
                if (s > m)
                    m = s;
            }
            double denom = 0.0;
            for (int e = 0; e < d; ++e)
                acc[e] = 0.0;
            for (int t = 0; t < n_keys; ++t) {
                if (key_pos[t] > p)
                    continue;
                double w = exp(scores[t] - m);
                denom += w;
                const double *vt = v + ((size_t)t * n_kv_heads + g) * d;
                for (int e = 0; e < d; ++e)
                    acc[e] += w * vt[e];
            }
            double *o = out + ((size_t)r * n_q_heads + h) * d;
            if (denom > 0.0) {
                for (int e = 0; e < d; ++e)
                    o[e] = acc[e] / denom;
                if (lse)
                    lse[(size_t)r * n_q_heads + h] = m + log(denom);
            } else {
                /* no key at or before the row's position */
                for (int e = 0; e < d; ++e)
                    o[e] = NAN;
                if (lse)
                    lse[(size_t)r * n_q_heads + h] = -INFINITY;
            }
        }
        free(scores);
        free(q_rot);
        free(acc);
    }
    free(inv_freq);
    free(k_rot);
    return failed ? -2 : 0;
}
