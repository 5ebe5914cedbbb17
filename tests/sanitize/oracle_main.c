/* Sanitizer driver for the fp64 oracle (test infrastructure): runs every
 * entry point of oracle/gla_oracle.c on small seeded inputs, with and without
 * the optional arguments, over several thread counts and edge shapes, and
 * checks the outputs are finite.  Built with -fsanitize=address,undefined by
 * tests/test_sanitizers.py; any invalid access or undefined behaviour aborts
 * with the sanitizer's report. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gla_oracle_fwd(int, int, int, int, int, const double *, const double *, const double *,
                   const double *, const double *, double *, double *, int);
int gla_oracle_bwd(int, int, int, int, int, const double *, const double *, const double *,
                   const double *, const double *, const double *, const double *, double *,
                   double *, double *, double *, double *, int);
int ggla_oracle_fwd(int, int, int, int, int, const double *, const double *, const double *,
                    const double *, const double *, const double *, double *, double *, int);
int ggla_oracle_bwd(int, int, int, int, int, const double *, const double *, const double *,
                    const double *, const double *, const double *, const double *,
                    const double *, double *, double *, double *, double *, double *,
                    double *, int);

static uint64_t rng = 0x9e3779b97f4a7c15ull;
static double urand(void) { /* xorshift64*, uniform in [-1, 1) */
  rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
  return (double)((rng * 0x2545f4914f6cdd1dull) >> 11) / 4503599627370496.0 - 1.0;
}
/* exactly n doubles on the heap, so that any access past them is reported */
static double *arr(size_t n, int gate) {
  double *p = (double *)malloc((n ? n : 1) * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = gate ? -0.05 * (1.0 + urand()) : urand();
  return p;
}
static int finite(const double *p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static int run(int B, int H, int L, int dk, int dv, int with_h0, int with_dhT, int threads) {
  const size_t BH = (size_t)B * H, nk = BH * L * dk, nv = BH * L * dv, ns = BH * dk * dv;
  double *q = arr(nk, 0), *k = arr(nk, 0), *v = arr(nv, 0), *a = arr(nk, 1), *b = arr(nv, 1);
  double *h0 = with_h0 ? arr(ns, 0) : NULL, *dhT = with_dhT ? arr(ns, 0) : NULL;
  double *o = arr(nv, 0), *hT = arr(ns, 0), *dout = arr(nv, 0);
  double *dq = arr(nk, 0), *dk_ = arr(nk, 0), *dv_ = arr(nv, 0), *da = arr(nk, 0), *db = arr(nv, 0);
  double *dh0 = arr(ns, 0);
  int bad = 0;
  bad |= gla_oracle_fwd(B, H, L, dk, dv, q, k, v, a, h0, o, hT, threads) != 0;
  bad |= !finite(o, nv) || !finite(hT, ns);
  bad |= gla_oracle_bwd(B, H, L, dk, dv, q, k, v, a, h0, dout, dhT, dq, dk_, dv_, da,
                        with_h0 ? dh0 : NULL, threads) != 0;
  bad |= !finite(dq, nk) || !finite(dk_, nk) || !finite(dv_, nv) || !finite(da, nk);
  bad |= ggla_oracle_fwd(B, H, L, dk, dv, q, k, v, a, b, h0, o, hT, threads) != 0;
  bad |= ggla_oracle_bwd(B, H, L, dk, dv, q, k, v, a, b, h0, dout, dhT, dq, dk_, dv_, da, db,
                         with_h0 ? dh0 : NULL, threads) != 0;
  bad |= !finite(db, nv) || !finite(da, nk);
  double *all[] = {q, k, v, a, b, h0, dhT, o, hT, dout, dq, dk_, dv_, da, db, dh0};
  for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) free(all[i]);
  if (bad) fprintf(stderr, "failed: B%d H%d L%d dk%d dv%d h0 %d dhT %d threads %d\n", B, H, L,
                   dk, dv, with_h0, with_dhT, threads);
  return bad;
}

int main(void) {
  int bad = 0;
  bad |= run(1, 1, 17, 16, 32, 0, 0, 1);
  bad |= run(2, 3, 33, 16, 48, 1, 1, 4);
  bad |= run(1, 2, 1, 32, 16, 1, 0, 3);
  bad |= run(3, 1, 64, 8, 8, 0, 1, 8);
  bad |= run(1, 1, 0, 16, 16, 1, 1, 2);   /* empty sequence: hT = h0 */
  bad |= run(0, 2, 10, 16, 16, 0, 0, 2);  /* empty batch */
  /* argument errors are reported, not dereferenced */
  bad |= gla_oracle_fwd(-1, 1, 1, 1, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1) != -1;
  bad |= gla_oracle_fwd(1, 1, 4, 4, 4, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1) != -1;
  printf(bad ? "oracle sanitizer run FAILED\n" : "oracle sanitizer run clean\n");
  return bad;
}
