/*
 * Reference oracle for exact attention -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 CPU implementation of what the attention hot path
 * computes.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline leg may load this library; the product path never does.  It shares
 * no source, header, table or helper with the HIP library.
 *
 * What it computes (sources are the pages on IO-aware exact attention):
 *  - "Dao and colleagues: IO-aware exact attention with FlashAttention"
 *    (research record; fields "summary" and "boundary"): the method computes
 *    EXACT attention -- tiling and recomputation change memory traffic, not
 *    the result and not the quadratic arithmetic.  The oracle is therefore the
 *    plain definition, with the full score row S and probability row P
 *    materialised in fp64 (no tiling, no online rescaling):
 *        s_ij = scale * <q_i, k_j>
 *        P_ij = exp(s_ij - m_i) / sum_j' exp(s_ij' - m_i)   over allowed j
 *        O_i  = sum_j P_ij v_j,     LSE_i = m_i + ln(sum_j exp(s_ij - m_i))
 *  - "Flash Attention and Efficient Transformer Mechanisms" (article, the
 *    paragraph on block computation): the blockwise result equals standard
 *    attention exactly; nothing is approximated.
 *  - The backward is the calculus derivative of that definition (the pages
 *    say only that the backward recomputes attention from saved statistics;
 *    they print no formula):
 *        D_i   = sum_c dO_ic O_ic
 *        dP_ij = <dO_i, v_j>,   dS_ij = P_ij (dP_ij - D_i)
 *        dQ_i  = scale sum_j dS_ij k_j
 *        dK_j  = scale sum_i dS_ij q_i,   dV_j = sum_i P_ij dO_i
 *
 * Readings where the pages are silent:
 *  - causal mask is bottom-right aligned: key j is visible to query row i iff
 *    j <= i + diag with diag = Sk - Sq (equals the usual j <= i when Sq = Sk);
 *  - a row with no visible key has O = 0 and LSE = -inf;
 *  - LSE is the natural-log log-sum-exp of the scaled, masked scores.
 *
 * Layout: one attention head at a time; every matrix is dense row-major
 * [rows][d] in fp64.  Rows are parallelised with OpenMP; the arithmetic of
 * each row is sequential in j and c.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static int visible(int64_t i, int64_t j, int64_t diag, int causal) {
  return !causal || j <= i + diag;
}

static double dot(const double* a, const double* b, int64_t d) {
  double s = 0.0;
  for (int64_t c = 0; c < d; c++) s += a[c] * b[c];
  return s;
}

/*
 * Probability row of query row `i` (position i in its sequence) against all
 * sk keys.  Writes s[j] (scaled score, or -inf where masked) and p[j].
 * Returns 0 and leaves m/l untouched if no key is visible.
 */
static int prob_row(const double* qi, int64_t i, int64_t sk, int64_t d,
                    const double* k, int64_t diag, int causal, double scale,
                    double* s, double* p, double* m_out, double* l_out) {
  int any = 0;
  double m = -INFINITY;
  for (int64_t j = 0; j < sk; j++) {
    if (visible(i, j, diag, causal)) {
      s[j] = scale * dot(qi, k + j * d, d);
      if (!any || s[j] > m) m = s[j];
      any = 1;
    } else {
      s[j] = -INFINITY;
    }
  }
  if (!any) {
    for (int64_t j = 0; j < sk; j++) p[j] = 0.0;
    return 0;
  }
  double l = 0.0;
  for (int64_t j = 0; j < sk; j++) {
    p[j] = visible(i, j, diag, causal) ? exp(s[j] - m) : 0.0;
    l += p[j];
  }
  for (int64_t j = 0; j < sk; j++) p[j] /= l;
  *m_out = m;
  *l_out = l;
  return 1;
}

/*
 * Forward for nq query rows of one head.
 *   q    [nq][d]     query rows
 *   pos  [nq]        position of each row inside its sequence (for the mask)
 *   k, v [sk][d]     keys and values of the head's kv head
 *   diag             Sk - Sq of the sequence (bottom-right causal alignment)
 *   o    [nq][d]     output rows;  lse [nq] natural-log LSE
 *   p_out            optional [nq][sk] probability matrix (NULL: not stored)
 */
void oracle_head_fwd(int64_t nq, int64_t sk, int64_t d, const double* q,
                     const int64_t* pos, int64_t diag, int causal,
                     double scale, const double* k, const double* v,
                     double* o, double* lse, double* p_out) {
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(sk > 0 ? sk : 1));
    double* p = (double*)malloc(sizeof(double) * (size_t)(sk > 0 ? sk : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nq; r++) {
      double m = 0.0, l = 0.0;
      double* orow = o + r * d;
      if (!prob_row(q + r * d, pos[r], sk, d, k, diag, causal, scale, s, p,
                    &m, &l)) {
        for (int64_t c = 0; c < d; c++) orow[c] = 0.0;
        lse[r] = -INFINITY;
      } else {
        for (int64_t c = 0; c < d; c++) {
          double acc = 0.0;
          for (int64_t j = 0; j < sk; j++) acc += p[j] * v[j * d + c];
          orow[c] = acc;
        }
        lse[r] = m + log(l);
      }
      if (p_out) memcpy(p_out + r * sk, p, sizeof(double) * (size_t)sk);
    }
    free(s);
    free(p);
  }
}

/*
 * Forward and backward of one kv head and the nh query heads that share it
 * (grouped-query attention; nh = 1 is ordinary multi-head attention).
 *   q, dout   [nh][sq][d]     do_ is the incoming gradient dL/dO
 *   k, v      [sk][d]
 *   o         [nh][sq][d]     forward output (recomputed here in fp64)
 *   lse       [nh][sq]
 *   dq        [nh][sq][d]
 *   dk, dv    [sk][d]         summed over the nh query heads
 * P and dS of each query head are materialised as full sq x sk matrices.
 */
void oracle_group_bwd(int64_t nh, int64_t sq, int64_t sk, int64_t d,
                      const double* q, const double* k, const double* v,
                      const double* dout, int causal, double scale, double* o,
                      double* lse, double* dq, double* dk, double* dv) {
  const int64_t diag = sk - sq;
  double* P = (double*)malloc(sizeof(double) * (size_t)(sq * sk > 0 ? sq * sk : 1));
  double* dS = (double*)malloc(sizeof(double) * (size_t)(sq * sk > 0 ? sq * sk : 1));
  for (int64_t x = 0; x < sk * d; x++) { dk[x] = 0.0; dv[x] = 0.0; }
  for (int64_t h = 0; h < nh; h++) {
    const double* qh = q + h * sq * d;
    const double* doh = dout + h * sq * d;
    double* oh = o + h * sq * d;
    double* dqh = dq + h * sq * d;
#pragma omp parallel
    {
      double* s = (double*)malloc(sizeof(double) * (size_t)(sk > 0 ? sk : 1));
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < sq; i++) {
        double m = 0.0, l = 0.0;
        double* pi = P + i * sk;
        double* dsi = dS + i * sk;
        int any = prob_row(qh + i * d, i, sk, d, k, diag, causal, scale, s, pi,
                           &m, &l);
        /* forward output and LSE */
        for (int64_t c = 0; c < d; c++) {
          double acc = 0.0;
          for (int64_t j = 0; j < sk; j++) acc += pi[j] * v[j * d + c];
          oh[i * d + c] = acc;
        }
        lse[h * sq + i] = any ? m + log(l) : -INFINITY;
        /* D_i = <dO_i, O_i> */
        double Di = dot(doh + i * d, oh + i * d, d);
        /* dP_ij = <dO_i, v_j>;  dS_ij = P_ij (dP_ij - D_i) */
        for (int64_t j = 0; j < sk; j++) {
          double dPij = dot(doh + i * d, v + j * d, d);
          dsi[j] = pi[j] * (dPij - Di);
        }
        /* dQ_i = scale * sum_j dS_ij k_j */
        for (int64_t c = 0; c < d; c++) {
          double acc = 0.0;
          for (int64_t j = 0; j < sk; j++) acc += dsi[j] * k[j * d + c];
          dqh[i * d + c] = scale * acc;
        }
      }
      free(s);
    }
    /* dV_j += sum_i P_ij dO_i;  dK_j += scale * sum_i dS_ij q_i */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < sk; j++) {
      for (int64_t c = 0; c < d; c++) {
        double av = 0.0, ak = 0.0;
        for (int64_t i = 0; i < sq; i++) {
          av += P[i * sk + j] * doh[i * d + c];
          ak += dS[i * sk + j] * qh[i * d + c];
        }
        dv[j * d + c] += av;
        dk[j * d + c] += scale * ak;
      }
    }
  }
  free(P);
  free(dS);
}
