/*
 * Oracle for causal kernelized linear attention: plain FP64, one token at a time.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * do.  It shares no code, header, table or helper with the HIP library.
 *
 * What it computes follows the page "Linear attention：把历史写进状态"
 * (hs-black.github.io/posts/linear-attention):
 *   - feature map phi = ELU(x)+1 (section "关键改写：让求和先发生"), with ELU's
 *     scale 1, i.e. phi(x) = x+1 for x > 0 and exp(x) for x <= 0;
 *   - the two accumulators S (r x dv, feature-major) and z (r), starting from
 *     whatever state the caller passes (zero for a fresh sequence, section
 *     "每来一个 token，更新两个累加器"), updated first and read second so that
 *     y_t includes token t (same section);
 *   - the scalar forget gate of section "加一个门": the old S and z are both
 *     multiplied by alpha_t before token t is written (alpha == NULL means
 *     alpha_t = 1, the plain accumulating form of section "公式里的每个维度");
 *   - the read-out y_t = (phi(q_t)^T S_t) / (phi(q_t)^T z_t + eps), with eps added
 *     to the denominator (section "ε 是数值保护"), never max(den, eps).
 * The same page's minimal FP64 loop (section "最小递推里，每一行都有张量意义")
 * is exactly this recurrence with alpha = 1.
 *
 * Sums run left to right over the feature index.  Build without fast-math and
 * without floating-point contraction so that the arithmetic is what is written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_PHI_ELU1 0        /* phi(x) = ELU(x) + 1 */
#define ORACLE_PHI_IDENTITY 1    /* the inputs already are features (worked examples) */
#define ORACLE_PHI_RELU1 2       /* phi(x) = max(x, 0) + 1 */
#define ORACLE_PHI_RELU_EPS 3    /* phi(x) = max(x, 0) + 1e-5 */
#define ORACLE_PHI_SIGMOID_EPS 4 /* phi(x) = 1 / (1 + exp(-x)) + 1e-5 */

double oracle_phi(double x)
{
    return x > 0.0 ? x + 1.0 : exp(x);
}

/*
 * The other positive feature maps the pages use:
 *   - max(x, 0) + 1: the teaching map of the datawhalechina chapter "Linear Attention and
 *     Recurrent State" (Step 4, its positive feature map: positive by construction, so
 *     the normaliser never vanishes);
 *   - max(x, 0) + 1e-5 and sigmoid(x) + 1e-5: the selectable maps of the pluggable
 *     linear-attention module of the page "线性注意力架构演进：从 Transformer 瓶颈到高效
 *     推理" (ai-master.cc, its third replacement plan, whose feature-map switch offers
 *     elu, relu and sigmoid).
 */
double oracle_phi_mode(double x, int32_t phi_mode)
{
    switch (phi_mode) {
    case ORACLE_PHI_IDENTITY:
        return x;
    case ORACLE_PHI_RELU1:
        return (x > 0.0 ? x : 0.0) + 1.0;
    case ORACLE_PHI_RELU_EPS:
        return (x > 0.0 ? x : 0.0) + 1e-5;
    case ORACLE_PHI_SIGMOID_EPS:
        return 1.0 / (1.0 + exp(-x)) + 1e-5;
    default:
        return oracle_phi(x);
    }
}

static int known_phi_mode(int32_t phi_mode)
{
    return phi_mode >= ORACLE_PHI_ELU1 && phi_mode <= ORACLE_PHI_SIGMOID_EPS;
}

static double apply_feature_map(double x, int32_t phi_mode)
{
    return oracle_phi_mode(x, phi_mode);
}

/*
 * One sequence (one head).  Row-major arrays:
 *   q, k  [T, r]      raw queries/keys (phi is applied here)
 *   v     [T, dv]
 *   alpha [T] or NULL
 *   S     [r, dv]     in: state before token 0, out: state after token T-1
 *   z     [r]         in/out like S
 *   y     [T, dv]     out
 *   den   [T] or NULL out: phi(q_t)^T z_t without eps (for denominator monitoring)
 * Returns 0, or -1 on a bad argument or allocation failure (then nothing is written).
 */
int oracle_recurrence(int64_t T, int32_t r, int32_t dv,
                      const double *q, const double *k, const double *v,
                      const double *alpha, double eps, int32_t phi_mode,
                      double *S, double *z, double *y, double *den)
{
    if (T < 1 || r < 1 || dv < 1 || !q || !k || !v || !S || !z || !y)
        return -1;
    if (!known_phi_mode(phi_mode))
        return -1;

    double *qf = (double *)malloc(sizeof(double) * (size_t)r);
    double *kf = (double *)malloc(sizeof(double) * (size_t)r);
    if (!qf || !kf) {
        free(qf);
        free(kf);
        return -1;
    }

    for (int64_t t = 0; t < T; ++t) {
        const double a = alpha ? alpha[t] : 1.0;
        for (int32_t i = 0; i < r; ++i) {
            qf[i] = apply_feature_map(q[t * r + i], phi_mode);
            kf[i] = apply_feature_map(k[t * r + i], phi_mode);
        }

        /* write: S <- a*S + phi(k_t) v_t^T,  z <- a*z + phi(k_t) */
        for (int32_t i = 0; i < r; ++i) {
            for (int32_t j = 0; j < dv; ++j)
                S[(int64_t)i * dv + j] = a * S[(int64_t)i * dv + j] + kf[i] * v[t * dv + j];
            z[i] = a * z[i] + kf[i];
        }

        /* read: numerator phi(q_t)^T S_t, denominator phi(q_t)^T z_t + eps */
        double d = 0.0;
        for (int32_t i = 0; i < r; ++i)
            d += qf[i] * z[i];
        if (den)
            den[t] = d;
        for (int32_t j = 0; j < dv; ++j) {
            double num = 0.0;
            for (int32_t i = 0; i < r; ++i)
                num += qf[i] * S[(int64_t)i * dv + j];
            y[t * dv + j] = num / (d + eps);
        }
    }

    free(qf);
    free(kf);
    return 0;
}

/*
 * Non-causal form: every query reads the state that holds the whole sequence.  This is
 * the associative-order evaluation of the page "线性注意力架构演进" (ai-master.cc): its
 * LinearAttention class's parallel training form and its pluggable module both form
 * K~^T V and the key sum once and read each query against them.  With S0 = z0 = 0 it
 * equals unmasked attention with weights phi(q_t).phi(k_i).  The epsilon convention is
 * the one of the read-out above: eps is added to the denominator.
 *   S <- S0 + sum_t phi(k_t) v_t^T,   z <- z0 + sum_t phi(k_t)     (t = 0 .. T-1)
 *   y_t = (phi(q_t)^T S) / (phi(q_t)^T z + eps)                      for every t
 * Arrays as for oracle_recurrence; S and z are in/out (in: the state before the
 * sequence, out: the state after it).  den [T] or NULL receives phi(q_t)^T z.
 */
int oracle_noncausal(int64_t T, int32_t r, int32_t dv,
                     const double *q, const double *k, const double *v,
                     double eps, int32_t phi_mode,
                     double *S, double *z, double *y, double *den)
{
    if (T < 1 || r < 1 || dv < 1 || !q || !k || !v || !S || !z || !y)
        return -1;
    if (!known_phi_mode(phi_mode))
        return -1;
    double *qf = (double *)malloc(sizeof(double) * (size_t)r);
    if (!qf)
        return -1;

    /* write every token into the state */
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t i = 0; i < r; ++i) {
            const double kf = apply_feature_map(k[t * r + i], phi_mode);
            for (int32_t j = 0; j < dv; ++j)
                S[(int64_t)i * dv + j] = S[(int64_t)i * dv + j] + kf * v[t * dv + j];
            z[i] = z[i] + kf;
        }
    }

    /* read every query against the full state */
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t i = 0; i < r; ++i)
            qf[i] = apply_feature_map(q[t * r + i], phi_mode);
        double d = 0.0;
        for (int32_t i = 0; i < r; ++i)
            d += qf[i] * z[i];
        if (den)
            den[t] = d;
        for (int32_t j = 0; j < dv; ++j) {
            double num = 0.0;
            for (int32_t i = 0; i < r; ++i)
                num += qf[i] * S[(int64_t)i * dv + j];
            y[t * dv + j] = num / (d + eps);
        }
    }
    free(qf);
    return 0;
}

/*
 * Delta rule (same page, section "Delta rule：先读旧答案，再写误差", and its
 * "key 的范数决定了纠错力度" derivation S' = S + beta k (v - k^T S)): a fast-weight
 * memory without the normaliser of the linear-attention read-out.  Per step t:
 *   prediction p_t = S^T k_t        (the memory's current answer for key k_t)
 *   error      e_t = v_t - p_t
 *   write      S <- S + beta_t k_t e_t^T
 *   read       y_t = S^T q_t        (after the write, as in the accumulating form)
 * Keys and queries enter as given: the page's delta examples use raw (unit) keys and
 * apply no feature map.  The read-out with a query is not printed by the page; reading
 * it after the write mirrors the update-then-read order of the accumulating form.
 *
 * Row-major arrays: q, k [T, r]; v [T, dv]; beta [T]; S [r, dv] in/out; y [T, dv] out;
 * pred [T, dv] or NULL (out: p_t, the prediction before the write).
 * Returns 0, or -1 on a bad argument or allocation failure (then nothing is written).
 */
int oracle_delta_steps(int64_t T, int32_t r, int32_t dv,
                       const double *q, const double *k, const double *v, const double *beta,
                       double *S, double *y, double *pred)
{
    if (T < 1 || r < 1 || dv < 1 || !q || !k || !v || !beta || !S || !y)
        return -1;
    double *e = (double *)malloc(sizeof(double) * (size_t)dv);
    if (!e)
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        const double *kt = k + t * r, *qt = q + t * r;
        for (int32_t j = 0; j < dv; ++j) {
            double p = 0.0;
            for (int32_t i = 0; i < r; ++i)
                p += kt[i] * S[(int64_t)i * dv + j];
            if (pred)
                pred[t * dv + j] = p;
            e[j] = v[t * dv + j] - p;
        }
        for (int32_t i = 0; i < r; ++i)
            for (int32_t j = 0; j < dv; ++j)
                S[(int64_t)i * dv + j] = S[(int64_t)i * dv + j] + beta[t] * kt[i] * e[j];
        for (int32_t j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int32_t i = 0; i < r; ++i)
                acc += qt[i] * S[(int64_t)i * dv + j];
            y[t * dv + j] = acc;
        }
    }
    free(e);
    return 0;
}

/*
 * Softmax attention decode, the comparator of the datawhalechina chapter "Linear
 * Attention and Recurrent State" (Step 5: an explicit K/V history against the fixed
 * recurrent state).  The row it computes is the one of the hs-black.github.io page,
 * section "先看普通 attention 在读什么": the query scores every history key, the scores
 * are normalised by softmax, and the values are summed with those weights:
 *   s_i = scale * (q . k_i),   w_i = exp(s_i - max_j s_j),   y = sum_i w_i v_i / sum_i w_i
 * for i = 0 .. L-1 (subtracting the maximum leaves the weights unchanged and keeps exp
 * finite).  One head: q [r]; K [L, r]; V [L, dv]; y [dv] out; w [L] or NULL (out: the
 * normalised weights).  Returns 0, or -1 on a bad argument.
 */
int oracle_softmax_decode(int64_t L, int32_t r, int32_t dv, const double *q, const double *K,
                          const double *V, double scale, double *y, double *w)
{
    if (L < 1 || r < 1 || dv < 1 || !q || !K || !V || !y)
        return -1;
    double *s = (double *)malloc(sizeof(double) * (size_t)L);
    if (!s)
        return -1;
    double mx = -INFINITY;
    for (int64_t i = 0; i < L; ++i) {
        double acc = 0.0;
        for (int32_t c = 0; c < r; ++c)
            acc += q[c] * K[i * r + c];
        s[i] = scale * acc;
        if (s[i] > mx)
            mx = s[i];
    }
    double sum = 0.0;
    for (int64_t i = 0; i < L; ++i) {
        s[i] = exp(s[i] - mx);
        sum += s[i];
    }
    for (int32_t j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < L; ++i)
            acc += s[i] * V[i * dv + j];
        y[j] = acc / sum;
    }
    if (w)
        for (int64_t i = 0; i < L; ++i)
            w[i] = s[i] / sum;
    free(s);
    return 0;
}
