/*
 * CPU oracle for Prefix Sliding attention.  TEST INFRASTRUCTURE ONLY: only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg load
 * it.  It shares no code with the GPU library and is plain, slow and direct:
 * every function below is the definition written out, in double precision.
 *
 * Sources (pages on "Prefix Sliding for efficient test-time scaling"):
 *  - njhaofan.com article, section "PrefixSliding如何丢掉中间Token？": the task
 *    prefix is always kept, the most recent W tokens form a sliding window,
 *    older middle tokens leave the KV cache; a 100-token prefix with a
 *    4096-token window retains at most about 4196 tokens.
 *  - agihunt.info summary, paragraphs on the memory cap and on position
 *    encodings (Continue PE: position IDs keep climbing, stored rotated keys
 *    stay valid).
 *  - papers.ananclaw.com explainer, section "核心方法" (PREFIX block kept,
 *    WINDOW block of the last W tokens, the middle evicted).
 *
 * Readings taken where the pages are silent (listed again in the design
 * notes): the current token is inside its own window (i-W < j <= i, W keys
 * counting itself); prefix queries are causal (j <= i); prefix and window
 * overlap is a plain set union; softmax scale is supplied by the caller
 * (1/sqrt(d) in every test); query head h reads kv head floor(h*Hkv/Hq).
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>

/* Key at position j is visible to the query at position i. */
int oracle_visible(int64_t i, int64_t j, int64_t P, int64_t W) {
    if (j < 0 || j > i) return 0;
    return j < P || j > i - W;
}

/* Number of visible keys for the query at position i: counts directly. */
int64_t oracle_visible_count(int64_t i, int64_t P, int64_t W) {
    int64_t c = 0;
    for (int64_t j = 0; j <= i; ++j) c += oracle_visible(i, j, P, W);
    return c;
}

/*
 * Masked softmax attention over an explicit list of keys.
 *
 *  q    [nq][hq][d]   float32 query rows (inputs are exact in float32)
 *  qpos [nq]          position of each query row
 *  k, v [nk][hkv][d]  float32 key / value rows
 *  kpos [nk]          position of each key row (the list may hold any keys,
 *                     including ones the rule hides; they are skipped, never
 *                     multiplied by zero, so their values cannot leak)
 *  out  [nq][hq][d]   double output
 *  lse  [nq][hq]      double log-sum-exp of the scaled scores (natural log)
 *
 * For query (t, h) with i = qpos[t] and g = floor(h*hkv/hq):
 *   s_j = scale * <q[t][h], k[j][g]>   for every listed j with visible(i, kpos[j])
 *   m   = max_j s_j
 *   out = sum_j exp(s_j - m) v[j][g] / sum_j exp(s_j - m)
 *   lse = m + ln sum_j exp(s_j - m)
 * A query with no visible key gets out = NaN, lse = -inf.
 */
void oracle_attention(int64_t nq, int hq, int hkv, int d,
                      const float* q, const int64_t* qpos,
                      int64_t nk, const float* k, const float* v, const int64_t* kpos,
                      int64_t P, int64_t W, double scale,
                      double* out, double* lse, int n_threads) {
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int64_t th = 0; th < nq * hq; ++th) {
        const int64_t t = th / hq;
        const int h = (int)(th % hq);
        const int g = (int)(((int64_t)h * hkv) / hq);
        const int64_t i = qpos[t];
        const float* qr = q + (t * hq + h) * (int64_t)d;
        double* o = out + (t * hq + h) * (int64_t)d;

        /* pass 1: maximum score over visible keys */
        double m = -INFINITY;
        int64_t nvis = 0;
        for (int64_t j = 0; j < nk; ++j) {
            if (!oracle_visible(i, kpos[j], P, W)) continue;
            const float* kr = k + (j * hkv + g) * (int64_t)d;
            double s = 0.0;
            for (int e = 0; e < d; ++e) s += (double)qr[e] * (double)kr[e];
            s *= scale;
            if (s > m) m = s;
            ++nvis;
        }
        for (int e = 0; e < d; ++e) o[e] = 0.0;
        if (nvis == 0) {
            for (int e = 0; e < d; ++e) o[e] = NAN;
            lse[th] = -INFINITY;
            continue;
        }
        /* pass 2: normaliser and weighted sum of values */
        double l = 0.0;
        for (int64_t j = 0; j < nk; ++j) {
            if (!oracle_visible(i, kpos[j], P, W)) continue;
            const float* kr = k + (j * hkv + g) * (int64_t)d;
            const float* vr = v + (j * hkv + g) * (int64_t)d;
            double s = 0.0;
            for (int e = 0; e < d; ++e) s += (double)qr[e] * (double)kr[e];
            s *= scale;
            double p = exp(s - m);
            l += p;
            for (int e = 0; e < d; ++e) o[e] += p * (double)vr[e];
        }
        for (int e = 0; e < d; ++e) o[e] /= l;
        lse[th] = m + log(l);
    }
}

/*
 * Tile class by exhaustive enumeration of every (query, key) pair of a query
 * tile with positions [i0, i1] and a key tile with positions [j0, j1]:
 *   0 = SKIP   (no pair visible: the tile contributes nothing)
 *   1 = FULL   (every pair visible: no elementwise mask needed)
 *   2 = MASKED (some pairs visible, some not)
 * This is the two-level filter the agihunt.info summary and the njhaofan.com
 * article (section "PrefixSliding如何丢掉中间Token？") describe for the kernel:
 * tiles wholly outside prefix and window are skipped, straddling tiles are
 * masked elementwise.
 */
int oracle_tile_class(int64_t i0, int64_t i1, int64_t j0, int64_t j1, int64_t P, int64_t W) {
    int64_t vis = 0, tot = 0;
    for (int64_t i = i0; i <= i1; ++i)
        for (int64_t j = j0; j <= j1; ++j) {
            vis += oracle_visible(i, j, P, W);
            ++tot;
        }
    if (vis == 0) return 0;
    if (vis == tot) return 1;
    return 2;
}

/*
 * Gradient of oracle_attention with respect to q, k and v, for the trainer
 * side (the agihunt.info summary, paragraph on RL, and the njhaofan.com
 * article, passage on truncated backpropagation: the trainer takes the last
 * few windows of a rollout and backpropagates through the masked attention).
 * The pages give no formula; this is the derivative of the definition above,
 * written out.  For query (t, h), g = floor(h*hkv/hq), visible keys J,
 * p_j = softmax_J(s)_j, upstream gradient dO = dout[t][h]:
 *   dp_j = <dO, v[j][g]>
 *   D    = sum_{j in J} p_j dp_j            (= <dO, out[t][h]>)
 *   ds_j = p_j (dp_j - D)
 *   dq[t][h]  += scale * sum_j ds_j k[j][g]
 *   dk[j][g]  += scale * ds_j q[t][h]
 *   dv[j][g]  += p_j dO
 * Hidden keys get nothing (they are skipped).  Outputs are overwritten.
 * Parallel over kv heads: every write of one thread stays in its kv head.
 * With delta_in non-null, D of query (t, h) is taken from delta_in[t*hq + h]
 * instead (the same formulas with the row term given).
 */
static void attention_bwd_impl(int64_t nq, int hq, int hkv, int d,
                               const float* q, const int64_t* qpos,
                               int64_t nk, const float* k, const float* v, const int64_t* kpos,
                               const float* dout, int64_t P, int64_t W, double scale, const double* delta_in,
                               double* dq, double* dk, double* dv, int n_threads) {
    for (int64_t x = 0; x < nq * hq * (int64_t)d; ++x) dq[x] = 0.0;
    for (int64_t x = 0; x < nk * hkv * (int64_t)d; ++x) { dk[x] = 0.0; dv[x] = 0.0; }
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int g = 0; g < hkv; ++g) {
        for (int64_t t = 0; t < nq; ++t)
            for (int h = 0; h < hq; ++h) {
                if ((int)(((int64_t)h * hkv) / hq) != g) continue;
                const int64_t i = qpos[t];
                const float* qr = q + (t * hq + h) * (int64_t)d;
                const float* dor = dout + (t * hq + h) * (int64_t)d;
                double* dqr = dq + (t * hq + h) * (int64_t)d;
                /* scores and their maximum */
                double m = -INFINITY;
                int64_t nvis = 0;
                for (int64_t j = 0; j < nk; ++j) {
                    if (!oracle_visible(i, kpos[j], P, W)) continue;
                    const float* kr = k + (j * hkv + g) * (int64_t)d;
                    double s = 0.0;
                    for (int e = 0; e < d; ++e) s += (double)qr[e] * (double)kr[e];
                    s *= scale;
                    if (s > m) m = s;
                    ++nvis;
                }
                if (nvis == 0) continue;
                /* probabilities p_j and dp_j over the visible keys */
                double l = 0.0, D = 0.0;
                for (int64_t j = 0; j < nk; ++j) {
                    if (!oracle_visible(i, kpos[j], P, W)) continue;
                    const float* kr = k + (j * hkv + g) * (int64_t)d;
                    double s = 0.0;
                    for (int e = 0; e < d; ++e) s += (double)qr[e] * (double)kr[e];
                    l += exp(s * scale - m);
                }
                for (int64_t j = 0; j < nk; ++j) {
                    if (!oracle_visible(i, kpos[j], P, W)) continue;
                    const float* kr = k + (j * hkv + g) * (int64_t)d;
                    const float* vr = v + (j * hkv + g) * (int64_t)d;
                    double s = 0.0, dpj = 0.0;
                    for (int e = 0; e < d; ++e) s += (double)qr[e] * (double)kr[e];
                    for (int e = 0; e < d; ++e) dpj += (double)dor[e] * (double)vr[e];
                    D += exp(s * scale - m) / l * dpj;
                }
                if (delta_in) D = delta_in[t * hq + h];
                for (int64_t j = 0; j < nk; ++j) {
                    if (!oracle_visible(i, kpos[j], P, W)) continue;
                    const float* kr = k + (j * hkv + g) * (int64_t)d;
                    const float* vr = v + (j * hkv + g) * (int64_t)d;
                    double* dkr = dk + (j * hkv + g) * (int64_t)d;
                    double* dvr = dv + (j * hkv + g) * (int64_t)d;
                    double s = 0.0, dpj = 0.0;
                    for (int e = 0; e < d; ++e) s += (double)qr[e] * (double)kr[e];
                    for (int e = 0; e < d; ++e) dpj += (double)dor[e] * (double)vr[e];
                    const double pj = exp(s * scale - m) / l;
                    const double dsj = pj * (dpj - D);
                    for (int e = 0; e < d; ++e) {
                        dqr[e] += scale * dsj * (double)kr[e];
                        dkr[e] += scale * dsj * (double)qr[e];
                        dvr[e] += pj * (double)dor[e];
                    }
                }
            }
    }
}

void oracle_attention_bwd(int64_t nq, int hq, int hkv, int d,
                          const float* q, const int64_t* qpos,
                          int64_t nk, const float* k, const float* v, const int64_t* kpos,
                          const float* dout, int64_t P, int64_t W, double scale,
                          double* dq, double* dk, double* dv, int n_threads) {
    attention_bwd_impl(nq, hq, hkv, d, q, qpos, nk, k, v, kpos, dout, P, W, scale, (const double*)0, dq, dk, dv,
                       n_threads);
}

/*
 * The gradient above with the row term D of every query supplied by the
 * caller (delta [nq][hq]).  A trainer that stores its forward output in a
 * narrow type forms D = <dO, out> from the stored output; evaluating the
 * exact formulas with that D separates the error the stored output carries
 * into D from the error of the rest of a backward computation.
 */
void oracle_attention_bwd_delta(int64_t nq, int hq, int hkv, int d,
                                const float* q, const int64_t* qpos,
                                int64_t nk, const float* k, const float* v, const int64_t* kpos,
                                const float* dout, int64_t P, int64_t W, double scale, const double* delta,
                                double* dq, double* dk, double* dv, int n_threads) {
    attention_bwd_impl(nq, hq, hkv, d, q, qpos, nk, k, v, kpos, dout, P, W, scale, delta, dq, dk, dv, n_threads);
}

/*
 * Rotary turn of rows by a number of positions: the re-encoding Reset PE
 * performs on retained keys when it gives them new positions (agihunt.info
 * summary, paragraph on position encodings; njhaofan.com article, passage
 * comparing ContinuePE and ResetPE).  Rotary encoding turns the half-split
 * pair (x_e, x_{e+d/2}), e < d/2, by the angle pos * base^(-2e/d), so moving
 * a key from position p to p + delta turns each pair by delta * base^(-2e/d):
 *   out_e       = x_e cos(t) - x_{e+d/2} sin(t)
 *   out_{e+d/2} = x_e sin(t) + x_{e+d/2} cos(t),   t = delta * base^(-2e/d).
 *  x     [n][d] float32 rows;  delta [n] positions per row;  out [n][d] double.
 */
void oracle_rope_turn(int64_t n, int d, const float* x, const int64_t* delta, double base, double* out) {
    const int half = d / 2;
    for (int64_t r = 0; r < n; ++r) {
        const float* xr = x + r * (int64_t)d;
        double* o = out + r * (int64_t)d;
        for (int e = 0; e < half; ++e) {
            const double t = (double)delta[r] * pow(base, -2.0 * e / (double)d);
            const double c = cos(t), s = sin(t);
            const double x0 = xr[e], x1 = xr[e + half];
            o[e] = x0 * c - x1 * s;
            o[e + half] = x0 * s + x1 * c;
        }
    }
}
