/*
 * oracle.c -- plain, slow fp64 CPU oracle for CLiS attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this file's library.  The HIP library never links,
 * includes or calls it, and it shares no code with the HIP library.
 *
 * Source: the pages "CLiS: Plug-and-Play Attention Acceleration for Video
 * Diffusion on TPUs via Certified Stabilization" (abstract; Algorithm 1 "CLiS
 * forward pass for one dense attention head"; Figure 3 on exp2 limits;
 * Figure 5(a) on the loop-invariant stabilizer).  Cited below as [CLiS ...].
 *
 * Everything is fp64 on already-decoded inputs (the Python wrapper decodes
 * bf16/fp32 to fp64 exactly).  Every function handles one (batch, head) pair;
 * rows are independent, so callers may split row ranges across threads
 * without changing any result.
 *
 * What this computes:
 *  - softmax attention by its definition (the CLiS output is exactly this:
 *    the stabilizer changes only the floating-point path) [CLiS abstract];
 *  - the certification statistics of Algorithm 1, steps 1-7, and the flag;
 *  - the fixed per-row stabilizer mu_i = c * (q_i . kbar), c = scale*log2(e)
 *    (the reading taken where the pages' Algorithm 1 extract stops);
 *  - two self-check evaluations of the same output: with the fixed stabilizer
 *    [CLiS Figure 5(a)], and with online softmax over key blocks
 *    [CLiS abstract: running maxima and accumulator rescaling];
 *  - each row's log-sum-exp (natural log) of its scores, the statistic a
 *    fused attention forward hands to its backward pass;
 *  - the unnormalized fixed-stabilizer sums over a key range, whose values
 *    over disjoint ranges add because the stabilizer does not change
 *    [CLiS Figure 5(a)].
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define LOG2E 1.442695040888963407359924681001892137

/* Scores of query row i against keys [0, nk): s_j = scale * sum_c q_ic k_jc. */
static void row_scores(const double* q, const double* k, int64_t i, int64_t nk, int d,
                       double scale, double* s) {
  const double* qi = q + i * (int64_t)d;
  for (int64_t j = 0; j < nk; ++j) {
    const double* kj = k + j * (int64_t)d;
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += qi[c] * kj[c];
    s[j] = scale * acc;
  }
}

/* Keys visible to row i: all of them, or 0..i under a causal mask. */
static int64_t visible_keys(int64_t i, int64_t nk, int causal) {
  if (!causal) return nk;
  return (i + 1 < nk) ? i + 1 : nk;
}

/*
 * Softmax attention by definition for the listed query rows [CLiS abstract:
 * the method leaves the attention output unchanged].  For row i:
 *   s_j = scale * q_i . k_j over the visible keys,
 *   o_i = sum_j exp(s_j) v_j / sum_j exp(s_j).
 * The row maximum is subtracted inside exp only to keep fp64 in range; it does
 * not change the value.  out is [nrows][d].  Returns 0, or -1 on allocation
 * failure.
 */
int oracle_attention_rows(const double* q, const double* k, const double* v,
                          int64_t nq, int64_t nk, int d, double scale, int causal,
                          const int64_t* rows, int64_t nrows, double* out) {
  (void)nq;
  double* s = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
  if (!s) return -1;
  for (int64_t t = 0; t < nrows; ++t) {
    const int64_t i = rows[t];
    const int64_t n = visible_keys(i, nk, causal);
    double* o = out + t * (int64_t)d;
    row_scores(q, k, i, n, d, scale, s);
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) m = s[j] > m ? s[j] : m;
    double l = 0.0;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      const double w = exp(s[j] - m);
      l += w;
      const double* vj = v + j * (int64_t)d;
      for (int c = 0; c < d; ++c) o[c] += w * vj[c];
    }
    for (int c = 0; c < d; ++c) o[c] /= l;
  }
  free(s);
  return 0;
}

/* Per-head certification record (fields as in Algorithm 1). */
typedef struct {
  double kappa;      /* step 3: max_r ||k_r - kbar||_2                  */
  double qnorm_max;  /* max_r ||q_r||_2                                 */
  double bound;      /* step 4: B_h = max_r BoundUp(q_r, kappa)         */
  double maxabs_v;   /* step 5: max_{j,r} |V_jr|                        */
  double u_exp;      /* Figure 3: log2 of the largest finite exp2 output */
  double u_acc;      /* Figure 3: log2 of the accumulator's largest value */
  int32_t G;         /* step 5 */
  int32_t L;         /* step 6: ceil(log2 N_k) */
  int32_t A;         /* step 6 */
  int32_t C;         /* step 7 */
  int32_t cert;      /* 1: certified, 0: falls back to online softmax */
  int32_t pad;
} oracle_cert_t;

/* ceil(log2 x) for finite x > 0, exactly: x = f * 2^e with f in [0.5, 1). */
static int32_t ceil_log2_exact(double x) {
  int e;
  const double f = frexp(x, &e);
  return (f == 0.5) ? e - 1 : e;
}

/* max that keeps a NaN once one is seen (inputs with NaN never certify). */
static double max_keep_nan(double acc, double x) {
  if (isnan(acc) || isnan(x)) return NAN;
  return x > acc ? x : acc;
}

/*
 * Figure 3 limits.  exp2(x) is finite in a format while x stays below log2 of
 * that format's largest finite value.  P (the exp2 output) is stored in bf16
 * on the bf16 path and fp32 on the fp32 path; the accumulators are fp32.
 */
static double log2_max_finite(int bf16) {
  const double fmax = bf16 ? 0x1.fep127 /* (2 - 2^-7) * 2^127 */ : (double)FLT_MAX;
  return log2(fmax);
}

/*
 * Algorithm 1, steps 1-7, for one head, plus the fixed stabilizer per row.
 *   s1  kbar = (1/N_k) sum_r k_r
 *   s2  centred keys k_r - kbar (not stored)
 *   s3  kappa = max_r ||k_r - kbar||_2  (exact fp64 value; the pages ask
 *       only for a conservative bound, and this is the tightest one)
 *   s4  B_h = max_r BoundUp(q_r, kappa), BoundUp(q, kappa) = c ||q||_2 kappa,
 *       c = scale * log2(e): by Cauchy-Schwarz it bounds the exp2 argument
 *       c q.(k - kbar) of every score of row r
 *   s5  G = ceil(log2 max(1, max |V|))
 *   s6  A = ceil(log2 N_k) + G
 *   s7  C = min(floor(U_exp), ceil(U_acc - A) - 1)
 *   cert = (B_h finite) and (B_h <= C)
 *   mu_r = c * (q_r . kbar)   (log2 units; exp2 arguments become c q.(k-kbar))
 * kbar is [d], mu is [nq].  p_bf16 selects the exp2 output format for U_exp.
 */
int oracle_certify_head(const double* q, const double* k, const double* v,
                        int64_t nq, int64_t nk, int d, double scale, int p_bf16,
                        double* kbar, double* mu, oracle_cert_t* rec) {
  const double c2 = scale * LOG2E;

  /* s1 */
  for (int c = 0; c < d; ++c) kbar[c] = 0.0;
  for (int64_t j = 0; j < nk; ++j)
    for (int c = 0; c < d; ++c) kbar[c] += k[j * (int64_t)d + c];
  for (int c = 0; c < d; ++c) kbar[c] /= (double)nk;

  /* s2, s3 */
  double kappa = 0.0;
  for (int64_t j = 0; j < nk; ++j) {
    double ss = 0.0;
    for (int c = 0; c < d; ++c) {
      const double t = k[j * (int64_t)d + c] - kbar[c];
      ss += t * t;
    }
    kappa = max_keep_nan(kappa, sqrt(ss));
  }

  /* s4 */
  double qmax = 0.0, bound = 0.0;
  for (int64_t r = 0; r < nq; ++r) {
    double ss = 0.0;
    for (int c = 0; c < d; ++c) ss += q[r * (int64_t)d + c] * q[r * (int64_t)d + c];
    const double qn = sqrt(ss);
    qmax = max_keep_nan(qmax, qn);
    bound = max_keep_nan(bound, c2 * qn * kappa);
  }

  /* s5 */
  double vmax = 0.0;
  for (int64_t j = 0; j < nk * (int64_t)d; ++j) vmax = max_keep_nan(vmax, fabs(v[j]));
  /* A non-finite max |V| has no finite exponent; 128 (one past every finite
   * fp32 value) drives C below zero, so such a head never certifies. */
  const int32_t G = isfinite(vmax) ? ceil_log2_exact(vmax > 1.0 ? vmax : 1.0) : 128;

  /* s6 */
  const int32_t L = ceil_log2_exact((double)nk);
  const int32_t A = L + G;

  /* s7 */
  const double u_exp = log2_max_finite(p_bf16);
  const double u_acc = log2_max_finite(0);
  const double c_exp = floor(u_exp);
  const double c_acc = ceil(u_acc - (double)A) - 1.0;
  const int32_t C = (int32_t)(c_exp < c_acc ? c_exp : c_acc);

  const int32_t cert = (isfinite(bound) && bound <= (double)C) ? 1 : 0;

  for (int64_t r = 0; r < nq; ++r) {
    double dot = 0.0;
    for (int c = 0; c < d; ++c) dot += q[r * (int64_t)d + c] * kbar[c];
    mu[r] = c2 * dot;
  }

  rec->kappa = kappa;
  rec->qnorm_max = qmax;
  rec->bound = bound;
  rec->maxabs_v = vmax;
  rec->u_exp = u_exp;
  rec->u_acc = u_acc;
  rec->G = G;
  rec->L = L;
  rec->A = A;
  rec->C = C;
  rec->cert = cert;
  rec->pad = 0;
  return 0;
}

/*
 * Self-check: the output evaluated with a fixed per-row stabilizer, as the
 * method's KV loop does [CLiS Figure 5(a), abstract]:
 *   o_i = sum_j 2^{x_ij} v_j / sum_j 2^{x_ij},  x_ij = c (q_i . k_j) - mu_i.
 * With mu_i from oracle_certify_head this must equal oracle_attention_rows.
 * Also reports the largest exp2 argument of each row (max_x, [nrows]) and the
 * largest |accumulator| reached by the sum and the weighted sum (max_acc,
 * [nrows]) so tests can check the certificate's promise.
 */
int oracle_fixed_mu_rows(const double* q, const double* k, const double* v,
                         int64_t nq, int64_t nk, int d, double scale, int causal,
                         const double* mu, const int64_t* rows, int64_t nrows,
                         double* out, double* max_x, double* max_acc) {
  (void)nq;
  const double c2 = scale * LOG2E;
  double* s = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
  if (!s) return -1;
  for (int64_t t = 0; t < nrows; ++t) {
    const int64_t i = rows[t];
    const int64_t n = visible_keys(i, nk, causal);
    double* o = out + t * (int64_t)d;
    row_scores(q, k, i, n, d, 1.0, s);
    double l = 0.0, xm = -INFINITY, am = 0.0;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      const double x = c2 * s[j] - mu[i];
      xm = x > xm ? x : xm;
      const double p = exp2(x);
      l += p;
      const double* vj = v + j * (int64_t)d;
      for (int c = 0; c < d; ++c) {
        o[c] += p * vj[c];
        const double a = fabs(o[c]);
        am = a > am ? a : am;
      }
      am = l > am ? l : am;
    }
    for (int c = 0; c < d; ++c) o[c] /= l;
    if (max_x) max_x[t] = xm;
    if (max_acc) max_acc[t] = am;
  }
  free(s);
  return 0;
}

/*
 * Self-check: online softmax over key blocks of `block` keys [CLiS abstract:
 * the baseline keeps a running maximum and rescales its accumulators].
 * Per block: m' = max(m, block max), alpha = 2^{m - m'}, l = alpha l + sum p,
 * o = alpha o + sum p v, with p = 2^{c s - m'}.  With tau > 0 the rescale is
 * lazy (the conditional rescaling of FlashAttention-4, which the pages name as
 * a comparator): the stabilizer in use changes only when a block's maximum
 * exceeds it by more than tau, so every weight stays at most 2^tau.  tau = 0 is
 * the eager form.  Both must equal the definition.
 */
int oracle_online_rows(const double* q, const double* k, const double* v,
                       int64_t nq, int64_t nk, int d, double scale, int causal, int64_t block,
                       double tau, const int64_t* rows, int64_t nrows, double* out) {
  (void)nq;
  const double c2 = scale * LOG2E;
  double* s = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
  if (!s) return -1;
  if (block < 1) block = 1;
  for (int64_t t = 0; t < nrows; ++t) {
    const int64_t i = rows[t];
    const int64_t n = visible_keys(i, nk, causal);
    double* o = out + t * (int64_t)d;
    row_scores(q, k, i, n, d, 1.0, s);
    double m = -INFINITY, l = 0.0;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int64_t j0 = 0; j0 < n; j0 += block) {
      const int64_t j1 = (j0 + block < n) ? j0 + block : n;
      double mb = -INFINITY;
      for (int64_t j = j0; j < j1; ++j) mb = (c2 * s[j] > mb) ? c2 * s[j] : mb;
      const double mn = (mb > m + tau) ? mb : m;
      const double alpha = exp2(m - mn);
      l *= alpha;
      for (int c = 0; c < d; ++c) o[c] *= alpha;
      for (int64_t j = j0; j < j1; ++j) {
        const double p = exp2(c2 * s[j] - mn);
        l += p;
        const double* vj = v + j * (int64_t)d;
        for (int c = 0; c < d; ++c) o[c] += p * vj[c];
      }
      m = mn;
    }
    for (int c = 0; c < d; ++c) o[c] /= l;
  }
  free(s);
  return 0;
}

/*
 * Log-sum-exp of each listed row's scores, natural log:
 *   lse_i = ln sum_j exp(s_j),  s_j = scale * q_i . k_j over the visible keys.
 * Evaluated as m + ln sum_j exp(s_j - m), m the row maximum (the shift keeps
 * fp64 in range; it does not change the value).  lse is [nrows].  Returns 0,
 * or -1 on allocation failure.
 */
int oracle_lse_rows(const double* q, const double* k, int64_t nq, int64_t nk, int d, double scale,
                    int causal, const int64_t* rows, int64_t nrows, double* lse) {
  (void)nq;
  double* s = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
  if (!s) return -1;
  for (int64_t t = 0; t < nrows; ++t) {
    const int64_t i = rows[t];
    const int64_t n = visible_keys(i, nk, causal);
    row_scores(q, k, i, n, d, scale, s);
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) m = s[j] > m ? s[j] : m;
    double sum = 0.0;
    for (int64_t j = 0; j < n; ++j) sum += exp(s[j] - m);
    lse[t] = m + log(sum);
  }
  free(s);
  return 0;
}

/*
 * Unnormalized fixed-stabilizer sums of each listed row over the keys
 * [k0, k1) that it sees [CLiS Figure 5(a): with mu_i fixed before the loop,
 * the weights 2^{x_ij} of disjoint key ranges simply add]:
 *   acc_i = sum_{j in [k0, k1), visible} 2^{x_ij} v_j,
 *   l_i   = sum_{j in [k0, k1), visible} 2^{x_ij},
 *   x_ij  = c (q_i . k_j) - mu_i,  c = scale * log2(e).
 * k and v hold the whole head (key j is row j); acc is [nrows][d], l is
 * [nrows]; an empty range gives zeros.  Returns 0.
 */
int oracle_fixed_mu_partial_rows(const double* q, const double* k, const double* v,
                                 int64_t nq, int64_t nk, int d, double scale, int causal,
                                 const double* mu, int64_t k0, int64_t k1,
                                 const int64_t* rows, int64_t nrows, double* acc, double* l) {
  (void)nq;
  const double c2 = scale * LOG2E;
  if (k0 < 0) k0 = 0;
  for (int64_t t = 0; t < nrows; ++t) {
    const int64_t i = rows[t];
    const int64_t n = visible_keys(i, nk, causal);
    const int64_t end = k1 < n ? k1 : n;
    double* a = acc + t * (int64_t)d;
    const double* qi = q + i * (int64_t)d;
    double sum = 0.0;
    for (int c = 0; c < d; ++c) a[c] = 0.0;
    for (int64_t j = k0; j < end; ++j) {
      const double* kj = k + j * (int64_t)d;
      double dot = 0.0;
      for (int c = 0; c < d; ++c) dot += qi[c] * kj[c];
      const double p = exp2(c2 * dot - mu[i]);
      sum += p;
      const double* vj = v + j * (int64_t)d;
      for (int c = 0; c < d; ++c) a[c] += p * vj[c];
    }
    l[t] = sum;
  }
  return 0;
}
