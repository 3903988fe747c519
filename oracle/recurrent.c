/*
 * Oracle: gated delta rule, token by token, float64 -- TEST INFRASTRUCTURE.
 * Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may load
 * this library; it shares no code with the HIP path.
 *
 * The recurrence is the KDA-style gated delta rule that the HARTS pages cite
 * as equation (1) (close-reading blog, section 7.1; thelatestinai page,
 * Figure 1(b): linear attention consumes a recurrent state and produces a
 * branch-specific next state), per head, with S of size dk x dv:
 *
 *     S'_t = diag(exp(g_t)) S_{t-1}
 *     S_t  = S'_t - beta_t k_t (k_t^T S'_t - v_t^T)
 *     o_t  = S_t^T q_t
 *
 * g_t is a per-channel log-decay (length dk), beta_t a scalar per head.  No
 * output scale is applied.  Each trajectory runs independently from its own
 * initial state (zero unless given) -- the trajectory-expanded execution the
 * pages use as their baseline.
 *
 * Reverse pass: L = sum_t <dO_t, o_t>.  With lambda = dL/dS_t carried
 * backwards (lambda = 0 after the last token), for token t:
 *
 *     lambda += q_t dO_t^T ;  dq_t = S_t dO_t ;  kappa = k_t^T lambda
 *     r = v_t - S'_t^T k_t ;  dv_t = beta_t kappa ;  dbeta_t = kappa . r
 *     dk_t = beta_t (lambda r - S'_t kappa)
 *     dS' = lambda - beta_t k_t kappa^T ;  dg_t = rowsum(dS' .* S'_t)
 *     lambda <- diag(exp(g_t)) dS'
 *
 * States are checkpointed every CKPT tokens and recomputed inside each block
 * during the reverse sweep; recomputation repeats the same float64 operations
 * in the same order, so it changes no value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define CKPT 64

typedef struct {
  int64_t n_traj;
  const int64_t *offsets; /* [n_traj+1] into positions */
  const int64_t *nodes;   /* [P] feature row of each position */
  int H, dk, dv;
  const double *q, *k, *v, *g, *beta; /* per feature row: [*, H, dk|dv], beta [*, H] */
  const double *S0;                   /* [n_traj, H, dk, dv] or NULL (zero) */
} traj_in;

/* one token forward: S (dk x dv) in place; Sp receives S'_t when non-NULL */
static void step_fwd(int dk, int dv, double *S, double *Sp, const double *q, const double *k,
                     const double *v, const double *g, double beta, double *o, double *tmp) {
  for (int c = 0; c < dk; ++c) {
    double e = exp(g[c]);
    for (int j = 0; j < dv; ++j) S[c * dv + j] *= e;
  }
  if (Sp) memcpy(Sp, S, sizeof(double) * dk * dv);
  /* tmp = S'^T k - v  (length dv) */
  for (int j = 0; j < dv; ++j) tmp[j] = -v[j];
  for (int c = 0; c < dk; ++c) {
    double kc = k[c];
    for (int j = 0; j < dv; ++j) tmp[j] += kc * S[c * dv + j];
  }
  for (int c = 0; c < dk; ++c) {
    double bk = beta * k[c];
    for (int j = 0; j < dv; ++j) S[c * dv + j] -= bk * tmp[j];
  }
  if (o) {
    for (int j = 0; j < dv; ++j) o[j] = 0.0;
    for (int c = 0; c < dk; ++c) {
      double qc = q[c];
      for (int j = 0; j < dv; ++j) o[j] += qc * S[c * dv + j];
    }
  }
}

/*
 * Forward.  o: [P, H, dv] per position.  Captures: for trajectory x, cap_off
 * [n_traj+1] indexes (cap_pos, cap_out); the state after cap_pos tokens of x is
 * written to cap_state[cap_out] ([*, H, dk, dv]).
 */
int oracle_fwd(const traj_in *in, double *o, const int64_t *cap_off, const int64_t *cap_pos,
               const int64_t *cap_out, double *cap_state, int nthreads) {
  const int H = in->H, dk = in->dk, dv = in->dv;
  const int64_t ntask = in->n_traj * H;
  int err = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double *S = (double *)malloc(sizeof(double) * dk * dv);
    double *tmp = (double *)malloc(sizeof(double) * (dv > dk ? dv : dk));
    if (!S || !tmp) err = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t task = 0; task < ntask; ++task) {
      if (!S || !tmp) continue;
      int64_t x = task / H;
      int h = (int)(task % H);
      int64_t p0 = in->offsets[x], p1 = in->offsets[x + 1];
      if (in->S0)
        memcpy(S, in->S0 + (x * H + h) * (int64_t)dk * dv, sizeof(double) * dk * dv);
      else
        memset(S, 0, sizeof(double) * dk * dv);
      int64_t ci = cap_off ? cap_off[x] : 0, ce = cap_off ? cap_off[x + 1] : 0;
      for (int64_t t = 0; t <= p1 - p0; ++t) {
        for (int64_t c = ci; c < ce; ++c)
          if (cap_pos[c] == t)
            memcpy(cap_state + (cap_out[c] * H + h) * (int64_t)dk * dv, S, sizeof(double) * dk * dv);
        if (t == p1 - p0) break;
        int64_t nd = in->nodes[p0 + t];
        step_fwd(dk, dv, S, NULL, in->q + (nd * H + h) * dk, in->k + (nd * H + h) * dk,
                 in->v + (nd * H + h) * dv, in->g + (nd * H + h) * dk, in->beta[nd * H + h],
                 o ? o + ((p0 + t) * H + h) * dv : NULL, tmp);
      }
    }
    free(S);
    free(tmp);
  }
  return err;
}

/*
 * Reverse pass.  dO: [P, H, dv] per position.  Per-position gradients dq, dk,
 * dv_, dg: [P, H, dk|dv], dbeta [P, H].  dS0 (nullable): [n_traj, H, dk, dv].
 * Captures of lambda = dL/dS_a after a tokens, as in oracle_fwd.
 */
int oracle_bwd(const traj_in *in, const double *dO, double *dq, double *dk_, double *dv_, double *dg,
               double *dbeta, double *dS0, const int64_t *cap_off, const int64_t *cap_pos,
               const int64_t *cap_out, double *cap_lambda, int nthreads) {
  const int H = in->H, dk = in->dk, dv = in->dv;
  const int64_t ntask = in->n_traj * H;
  const int64_t SS = (int64_t)dk * dv;
  int err = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double *blk = (double *)malloc(sizeof(double) * SS * (CKPT + 1));
    double *lam = (double *)malloc(sizeof(double) * SS);
    double *Sp = (double *)malloc(sizeof(double) * SS);
    double *dSp = (double *)malloc(sizeof(double) * SS);
    double *tmp = (double *)malloc(sizeof(double) * (dv > dk ? dv : dk));
    double *kap = (double *)malloc(sizeof(double) * dv);
    double *r = (double *)malloc(sizeof(double) * dv);
    int ok = blk && lam && Sp && dSp && tmp && kap && r;
    if (!ok) err = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t task = 0; task < ntask; ++task) {
      if (!ok) continue;
      int64_t x = task / H;
      int h = (int)(task % H);
      int64_t p0 = in->offsets[x], L = in->offsets[x + 1] - p0;
      int64_t nck = L / CKPT + 1;
      double *ck = (double *)malloc(sizeof(double) * SS * nck);
      if (!ck) { err = 1; continue; }
      /* forward sweep: checkpoint the state after t tokens for t = 0, CKPT, ... */
      double *S = blk;
      if (in->S0) memcpy(S, in->S0 + (x * H + h) * SS, sizeof(double) * SS);
      else memset(S, 0, sizeof(double) * SS);
      for (int64_t t = 0; t < L; ++t) {
        if (t % CKPT == 0) memcpy(ck + (t / CKPT) * SS, S, sizeof(double) * SS);
        int64_t nd = in->nodes[p0 + t];
        step_fwd(dk, dv, S, NULL, NULL, in->k + (nd * H + h) * dk, in->v + (nd * H + h) * dv,
                 in->g + (nd * H + h) * dk, in->beta[nd * H + h], NULL, tmp);
      }
      if (L % CKPT == 0) memcpy(ck + (L / CKPT) * SS, S, sizeof(double) * SS);
      memset(lam, 0, sizeof(double) * SS);
      int64_t ci = cap_off ? cap_off[x] : 0, ce = cap_off ? cap_off[x + 1] : 0;
      for (int64_t c = ci; c < ce; ++c)
        if (cap_pos[c] == L) memcpy(cap_lambda + (cap_out[c] * H + h) * SS, lam, sizeof(double) * SS);
      /* reverse sweep, block by block */
      for (int64_t b0 = ((L - 1) / CKPT) * CKPT; L > 0 && b0 >= 0; b0 -= CKPT) {
        int64_t b1 = b0 + CKPT < L ? b0 + CKPT : L;
        memcpy(blk, ck + (b0 / CKPT) * SS, sizeof(double) * SS);
        for (int64_t t = b0; t < b1; ++t) {
          int64_t nd = in->nodes[p0 + t];
          memcpy(blk + (t - b0 + 1) * SS, blk + (t - b0) * SS, sizeof(double) * SS);
          step_fwd(dk, dv, blk + (t - b0 + 1) * SS, NULL, NULL, in->k + (nd * H + h) * dk,
                   in->v + (nd * H + h) * dv, in->g + (nd * H + h) * dk, in->beta[nd * H + h], NULL, tmp);
        }
        for (int64_t t = b1 - 1; t >= b0; --t) {
          int64_t nd = in->nodes[p0 + t], P = p0 + t;
          const double *q = in->q + (nd * H + h) * dk, *k = in->k + (nd * H + h) * dk;
          const double *v = in->v + (nd * H + h) * dv, *g = in->g + (nd * H + h) * dk;
          double beta = in->beta[nd * H + h];
          const double *Sprev = blk + (t - b0) * SS, *Snew = blk + (t - b0 + 1) * SS;
          const double *d_o = dO + (P * H + h) * dv;
          /* S'_t */
          for (int c = 0; c < dk; ++c) {
            double e = exp(g[c]);
            for (int j = 0; j < dv; ++j) Sp[c * dv + j] = Sprev[c * dv + j] * e;
          }
          /* lambda += q dO^T ; dq = S_t dO */
          for (int c = 0; c < dk; ++c) {
            double acc = 0.0;
            for (int j = 0; j < dv; ++j) {
              lam[c * dv + j] += q[c] * d_o[j];
              acc += Snew[c * dv + j] * d_o[j];
            }
            dq[(P * H + h) * dk + c] = acc;
          }
          /* kappa = k^T lambda ; r = v - S'^T k */
          for (int j = 0; j < dv; ++j) { kap[j] = 0.0; r[j] = v[j]; }
          for (int c = 0; c < dk; ++c)
            for (int j = 0; j < dv; ++j) {
              kap[j] += k[c] * lam[c * dv + j];
              r[j] -= Sp[c * dv + j] * k[c];
            }
          double db = 0.0;
          for (int j = 0; j < dv; ++j) {
            dv_[(P * H + h) * dv + j] = beta * kap[j];
            db += kap[j] * r[j];
          }
          dbeta[P * H + h] = db;
          /* dk = beta (lambda r - S' kappa) */
          for (int c = 0; c < dk; ++c) {
            double a = 0.0, b = 0.0;
            for (int j = 0; j < dv; ++j) {
              a += lam[c * dv + j] * r[j];
              b += Sp[c * dv + j] * kap[j];
            }
            dk_[(P * H + h) * dk + c] = beta * (a - b);
          }
          /* dS' = lambda - beta k kappa^T ; dg = rowsum(dS' .* S') ; lambda = diag(e^g) dS' */
          for (int c = 0; c < dk; ++c) {
            double acc = 0.0, e = exp(g[c]);
            for (int j = 0; j < dv; ++j) {
              double d = lam[c * dv + j] - beta * k[c] * kap[j];
              acc += d * Sp[c * dv + j];
              lam[c * dv + j] = e * d;
            }
            dg[(P * H + h) * dk + c] = acc;
          }
          for (int64_t c = ci; c < ce; ++c)
            if (cap_pos[c] == t) memcpy(cap_lambda + (cap_out[c] * H + h) * SS, lam, sizeof(double) * SS);
        }
      }
      if (dS0) memcpy(dS0 + (x * H + h) * SS, lam, sizeof(double) * SS);
      free(ck);
    }
    free(blk); free(lam); free(Sp); free(dSp); free(tmp); free(kap); free(r);
  }
  return err;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
