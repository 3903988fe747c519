/* The float64 oracle's token-recurrent forward and reverse pass (oracle/recurrent.c, included
 * here as one translation unit), built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_host_sanitizers.py (CPU only): random trajectories sharing feature rows, initial
 * states, state captures at every position; every output must be finite. */
#include "../../oracle/recurrent.c"

#include <stdio.h>

static uint64_t st = 88172645463325252ull;
static double urand(void) { /* xorshift64 in [-1, 1) */
  st ^= st << 13;
  st ^= st >> 7;
  st ^= st << 17;
  return (double)(st >> 11) / 4503599627370496.0 - 1.0;
}

static int all_finite(const double *x, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) return 0;
  return 1;
}

int main(void) {
  const int H = 2, dk = 8, dv = 4, R = 40;
  const int64_t n = 3, offsets[4] = {0, 17, 17 + 33, 17 + 33 + 5};
  const int64_t P = offsets[3];
  int64_t nodes[55];
  for (int64_t i = 0; i < P; ++i) nodes[i] = (i * 7) % R;
  double *q = malloc(sizeof(double) * R * H * dk), *k = malloc(sizeof(double) * R * H * dk);
  double *g = malloc(sizeof(double) * R * H * dk), *v = malloc(sizeof(double) * R * H * dv);
  double *beta = malloc(sizeof(double) * R * H), *S0 = malloc(sizeof(double) * n * H * dk * dv);
  for (int i = 0; i < R * H * dk; ++i) {
    q[i] = urand();
    k[i] = urand() * 0.3;
    g[i] = -fabs(urand()) * (i % 5 == 0 ? 200.0 : 1.0); /* some steep channels */
  }
  for (int i = 0; i < R * H * dv; ++i) v[i] = urand();
  for (int i = 0; i < R * H; ++i) beta[i] = 0.5 + 0.5 * urand();
  for (int i = 0; i < n * H * dk * dv; ++i) S0[i] = 0.1 * urand();
  traj_in in = {n, offsets, nodes, H, dk, dv, q, k, v, g, beta, S0};
  /* a capture after every position of every trajectory */
  int64_t cap_off[4], *cap_pos = malloc(sizeof(int64_t) * P), *cap_out = malloc(sizeof(int64_t) * P);
  cap_off[0] = 0;
  for (int64_t x = 0, c = 0; x < n; ++x) {
    for (int64_t a = 1; a <= offsets[x + 1] - offsets[x]; ++a, ++c) {
      cap_pos[c] = a;
      cap_out[c] = c;
    }
    cap_off[x + 1] = cap_off[x] + (offsets[x + 1] - offsets[x]);
  }
  double *o = calloc(P * H * dv, sizeof(double)), *cs = calloc(P * H * dk * dv, sizeof(double));
  int rc = oracle_fwd(&in, o, cap_off, cap_pos, cap_out, cs, 3);
  double *dO = malloc(sizeof(double) * P * H * dv);
  for (int i = 0; i < P * H * dv; ++i) dO[i] = urand();
  double *dq = calloc(P * H * dk, sizeof(double)), *dkk = calloc(P * H * dk, sizeof(double));
  double *dvv = calloc(P * H * dv, sizeof(double)), *dg = calloc(P * H * dk, sizeof(double));
  double *db = calloc(P * H, sizeof(double)), *dS0 = calloc(n * H * dk * dv, sizeof(double));
  double *lam = calloc(P * H * dk * dv, sizeof(double));
  rc |= oracle_bwd(&in, dO, dq, dkk, dvv, dg, db, dS0, cap_off, cap_pos, cap_out, lam, 3);
  const int ok = rc == 0 && all_finite(o, P * H * dv) && all_finite(cs, P * H * dk * dv) &&
                 all_finite(dq, P * H * dk) && all_finite(dkk, P * H * dk) && all_finite(dvv, P * H * dv) &&
                 all_finite(dg, P * H * dk) && all_finite(db, P * H) && all_finite(dS0, n * H * dk * dv) &&
                 all_finite(lam, P * H * dk * dv);
  printf("oracle check rc %d %s\n", rc, ok ? "finite" : "NON-FINITE");
  free(q); free(k); free(g); free(v); free(beta); free(S0); free(cap_pos); free(cap_out);
  free(o); free(cs); free(dO); free(dq); free(dkk); free(dvv); free(dg); free(db); free(dS0); free(lam);
  return ok ? 0 : 1;
}
