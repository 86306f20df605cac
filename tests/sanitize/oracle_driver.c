/* Host driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of
 * the fp64 oracle (test infrastructure).  Runs oracle_head_fwd and
 * oracle_group_bwd on small seeded inputs, including the degenerate shapes
 * (no keys, no visible key, one query row, d = 1), and checks the properties
 * that need no second implementation: probability rows sum to 1, LSE is
 * -inf exactly for rows with no visible key, O of such rows is 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_head_fwd(int64_t nq, int64_t sk, int64_t d, const double* q, const int64_t* pos,
                     int64_t diag, int causal, double scale, const double* k, const double* v,
                     double* o, double* lse, double* p_out);
void oracle_group_bwd(int64_t nh, int64_t sq, int64_t sk, int64_t d, const double* q,
                      const double* k, const double* v, const double* dout, int causal,
                      double scale, double* o, double* lse, double* dq, double* dk, double* dv);

static uint64_t rng = 88172645463325252ull;
static double uniform(void) {
  rng ^= rng << 13, rng ^= rng >> 7, rng ^= rng << 17;
  return (double)(rng >> 11) * 0x1.0p-53 * 2.0 - 1.0;
}
static double* filled(int64_t n) {
  double* x = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; i++) x[i] = uniform();
  return x;
}

static int check_fwd(int64_t sq, int64_t sk, int64_t d, int causal) {
  double *q = filled(sq * d), *k = filled(sk * d), *v = filled(sk * d);
  double *o = filled(sq * d), *lse = filled(sq), *p = filled(sq * sk);
  int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(sq > 0 ? sq : 1));
  for (int64_t i = 0; i < sq; i++) pos[i] = i;
  oracle_head_fwd(sq, sk, d, q, pos, sk - sq, causal, 0.5, k, v, o, lse, p);
  int bad = 0;
  for (int64_t i = 0; i < sq; i++) {
    double sum = 0.0;
    for (int64_t j = 0; j < sk; j++) sum += p[i * sk + j];
    const int any = sk > 0 && (!causal || i + sk - sq >= 0);
    if (any ? fabs(sum - 1.0) > 1e-12 || !isfinite(lse[i]) : (sum != 0.0 || lse[i] != -INFINITY)) bad++;
    for (int64_t c = 0; c < d && !any; c++) bad += o[i * d + c] != 0.0;
  }
  free(q), free(k), free(v), free(o), free(lse), free(p), free(pos);
  return bad;
}

static int check_bwd(int64_t nh, int64_t sq, int64_t sk, int64_t d, int causal) {
  double *q = filled(nh * sq * d), *k = filled(sk * d), *v = filled(sk * d), *g = filled(nh * sq * d);
  double *o = filled(nh * sq * d), *lse = filled(nh * sq), *dq = filled(nh * sq * d);
  double *dk = filled(sk * d), *dv = filled(sk * d);
  oracle_group_bwd(nh, sq, sk, d, q, k, v, g, causal, 0.25, o, lse, dq, dk, dv);
  int bad = 0;
  /* sum_j dK_j = 0 (every row of dS sums to zero) */
  for (int64_t c = 0; c < d; c++) {
    double s = 0.0, a = 0.0;
    for (int64_t j = 0; j < sk; j++) s += dk[j * d + c], a += fabs(dk[j * d + c]);
    bad += fabs(s) > 1e-12 * (1.0 + a);
  }
  for (int64_t x = 0; x < nh * sq * d; x++) bad += !isfinite(dq[x]) || !isfinite(o[x]);
  free(q), free(k), free(v), free(g), free(o), free(lse), free(dq), free(dk), free(dv);
  return bad;
}

int main(void) {
  const int64_t shapes[][3] = {{1, 1, 1}, {3, 0, 4}, {0, 5, 4}, {5, 3, 2}, {3, 5, 8},
                               {17, 17, 16}, {40, 9, 1}, {9, 40, 3}};
  int bad = 0, n = 0;
  for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); s++)
    for (int causal = 0; causal < 2; causal++) {
      bad += check_fwd(shapes[s][0], shapes[s][1], shapes[s][2], causal);
      bad += check_bwd(1 + (int64_t)s % 3, shapes[s][0], shapes[s][1], shapes[s][2], causal);
      n += 2;
    }
  printf("oracle driver: %d cases, %d failures\n", n, bad);
  return bad != 0;
}
