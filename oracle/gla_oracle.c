/*
 * gla_oracle.c -- fp64 CPU oracle for Gated Linear Attention (GLA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (per batch b, head h; all arithmetic in double):
 *
 *   Forward: the GLA recurrence with the row gate G_t = alpha_t^T 1
 *   ("Gated Linear Attention Transformers with Hardware-Efficient Training",
 *   papercache.org notes, §4.1 "recurrent form" and the one-line summary
 *   S_t = (alpha_t^T 1) ⊙ S_{t-1} + k_t^T v_t; zako-mio deep-reading report,
 *   ch. 2.3, the gate row-gating Diag(alpha_t)):
 *
 *       S_0 = h0 (zeros when h0 == NULL)
 *       for t = 1..L:
 *           S_t[i][j] = exp(a_t[i]) * S_{t-1}[i][j] + k_t[i] * v_t[j]
 *           o_t[j]    = sum_i q_t[i] * S_t[i][j]
 *       hT = S_L
 *
 *   a_t = log alpha_t (the "log forget gate" of the notes' App. B listing)
 *   indexes the d_k rows of the state.  The output includes the current
 *   token (o_t = q_t S_t, same notes §2.1 for the ungated case), the decay is
 *   applied to S_{t-1} before the outer product is added, and S_0 may be a
 *   previous segment's state (§2.2 chunkwise form).
 *
 *   Backward: back-propagation through time of the same recurrence for a
 *   loss L with dL/do_t = do_t and dL/dhT = dhT (zeros when NULL):
 *
 *       dS = dhT
 *       for t = L..1:
 *           dq_t[i]      = sum_j S_t[i][j] * do_t[j]
 *           dS[i][j]    += q_t[i] * do_t[j]            (now dL/dS_t)
 *           dk_t[i]      = sum_j dS[i][j] * v_t[j]
 *           dv_t[j]      = sum_i dS[i][j] * k_t[i]
 *           dloga_t[i]   = exp(a_t[i]) * sum_j dS[i][j] * S_{t-1}[i][j]
 *           dS[i][j]    *= exp(a_t[i])                 (now dL/dS_{t-1})
 *       dh0 = dS
 *
 *   This is the chain rule applied to the recurrence above, nothing more; it
 *   does not use the pages' closed-form gate gradient, which the tests check
 *   against it.  States S_t are recomputed from checkpoints kept every
 *   OR_CKPT steps (recomputation repeats the identical double operations in
 *   the identical order, so the values are bit-identical to storing them).
 *
 * Layouts (row-major, contiguous, double):
 *   q, k, dq, dk, log_alpha, dlog_alpha : [B][H][L][dk]
 *   v, o, dout, dv                      : [B][H][L][dv]
 *   h0, hT, dhT, dh0                    : [B][H][dk][dv]
 *
 * Threads: one (b,h) pair per task, tasks split over `nthreads` pthreads.
 * Each task's arithmetic is independent of the split.
 *
 * General gate (ggla_oracle_fwd / ggla_oracle_bwd): the same recurrence with
 * the outer-product gate G_t = alpha_t^T beta_t of the notes' App. C
 * ("general form"), beta_t acting on the d_v columns:
 *
 *           S_t[i][j] = exp(a_t[i]) * exp(b_t[j]) * S_{t-1}[i][j] + k_t[i] * v_t[j]
 *
 * with b_t = log beta_t, laid out [B][H][L][dv] like v.  Its BPTT adds
 *           dlogb_t[j] = sum_i dS[i][j] * G_t[i][j] * S_{t-1}[i][j]
 * and decays dS by G_t[i][j].  With log_beta == NULL both functions are the
 * row-gated ones above, operation for operation.
 *
 * Return value: 0 on success, -1 on bad arguments, -2 on allocation failure.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define OR_CKPT 64

typedef struct {
  int B, H, L, dk, dv;
  const double *q, *k, *v, *la, *lb, *h0, *dout, *dhT;
  double *o, *hT, *dq, *dkk, *dvv, *dla, *dlb, *dh0;
  int next;            /* next (b,h) task index, guarded by mu */
  int failed;
  pthread_mutex_t mu;
} or_job;

static int or_take(or_job *J) {
  pthread_mutex_lock(&J->mu);
  int t = J->next++;
  pthread_mutex_unlock(&J->mu);
  return t;
}

/* One recurrence step: S <- diag(exp(a)) S + k^T v, or with a column gate b
 * (not NULL): S[i][j] <- exp(a[i]) exp(b[j]) S[i][j] + k[i] v[j]. */
static void or_step(double *S, const double *a, const double *b, const double *kt,
                    const double *vt, int dk, int dv) {
  for (int i = 0; i < dk; ++i) {
    double g = exp(a[i]);
    double *row = S + (size_t)i * dv;
    if (b)
      for (int j = 0; j < dv; ++j) row[j] = (g * exp(b[j])) * row[j] + kt[i] * vt[j];
    else
      for (int j = 0; j < dv; ++j) row[j] = g * row[j] + kt[i] * vt[j];
  }
}

/* log beta of token t, or NULL for the row-gated recurrence */
static const double *or_lb(const or_job *J, size_t vo, int t) {
  return J->lb ? J->lb + vo + (size_t)t * J->dv : NULL;
}

static void or_fwd_head(or_job *J, int bh) {
  const int L = J->L, dk = J->dk, dv = J->dv;
  const size_t qo = (size_t)bh * L * dk, vo = (size_t)bh * L * dv;
  const size_t so = (size_t)bh * dk * dv;
  double *S = (double *)malloc(sizeof(double) * dk * dv);
  if (!S) { J->failed = 1; return; }
  if (J->h0) memcpy(S, J->h0 + so, sizeof(double) * dk * dv);
  else memset(S, 0, sizeof(double) * dk * dv);
  for (int t = 0; t < L; ++t) {
    const double *qt = J->q + qo + (size_t)t * dk;
    or_step(S, J->la + qo + (size_t)t * dk, or_lb(J, vo, t), J->k + qo + (size_t)t * dk,
            J->v + vo + (size_t)t * dv, dk, dv);
    double *ot = J->o + vo + (size_t)t * dv;
    for (int j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
      const double *row = S + (size_t)i * dv;
      for (int j = 0; j < dv; ++j) ot[j] += qt[i] * row[j];
    }
  }
  if (J->hT) memcpy(J->hT + so, S, sizeof(double) * dk * dv);
  free(S);
}

static void or_bwd_head(or_job *J, int bh) {
  const int L = J->L, dk = J->dk, dv = J->dv;
  const size_t qo = (size_t)bh * L * dk, vo = (size_t)bh * L * dv;
  const size_t so = (size_t)bh * dk * dv, SS = (size_t)dk * dv;
  const int nck = (L + OR_CKPT - 1) / OR_CKPT;
  /* ck[c] = S_{c*OR_CKPT}; seg[r] = S_{c*OR_CKPT + r}, r = 0..OR_CKPT */
  double *ck = (double *)malloc(sizeof(double) * SS * (nck + 1));
  double *seg = (double *)malloc(sizeof(double) * SS * (OR_CKPT + 1));
  double *dS = (double *)malloc(sizeof(double) * SS);
  if (!ck || !seg || !dS) { free(ck); free(seg); free(dS); J->failed = 1; return; }

  double *S = ck;
  if (J->h0) memcpy(S, J->h0 + so, sizeof(double) * SS);
  else memset(S, 0, sizeof(double) * SS);
  for (int c = 0; c < nck; ++c) {
    double *next = ck + SS * (c + 1);
    memcpy(next, ck + SS * c, sizeof(double) * SS);
    int t1 = (c + 1) * OR_CKPT < L ? (c + 1) * OR_CKPT : L;
    for (int t = c * OR_CKPT; t < t1; ++t)
      or_step(next, J->la + qo + (size_t)t * dk, or_lb(J, vo, t),
              J->k + qo + (size_t)t * dk, J->v + vo + (size_t)t * dv, dk, dv);
  }

  if (J->dhT) memcpy(dS, J->dhT + so, sizeof(double) * SS);
  else memset(dS, 0, sizeof(double) * SS);

  for (int c = nck - 1; c >= 0; --c) {
    int t0 = c * OR_CKPT;
    int t1 = (c + 1) * OR_CKPT < L ? (c + 1) * OR_CKPT : L;
    memcpy(seg, ck + SS * c, sizeof(double) * SS);
    for (int t = t0; t < t1; ++t) {
      memcpy(seg + SS * (t - t0 + 1), seg + SS * (t - t0), sizeof(double) * SS);
      or_step(seg + SS * (t - t0 + 1), J->la + qo + (size_t)t * dk, or_lb(J, vo, t),
              J->k + qo + (size_t)t * dk, J->v + vo + (size_t)t * dv, dk, dv);
    }
    for (int t = t1 - 1; t >= t0; --t) {
      const double *St = seg + SS * (t - t0 + 1);     /* S_t (after token t) */
      const double *Sp = seg + SS * (t - t0);         /* S_{t-1}             */
      const double *qt = J->q + qo + (size_t)t * dk;
      const double *kt = J->k + qo + (size_t)t * dk;
      const double *vt = J->v + vo + (size_t)t * dv;
      const double *at = J->la + qo + (size_t)t * dk;
      const double *dot = J->dout + vo + (size_t)t * dv;
      double *dqt = J->dq + qo + (size_t)t * dk;
      double *dkt = J->dkk + qo + (size_t)t * dk;
      double *dvt = J->dvv + vo + (size_t)t * dv;
      double *dat = J->dla + qo + (size_t)t * dk;
      for (int i = 0; i < dk; ++i) {
        double s = 0.0;
        for (int j = 0; j < dv; ++j) s += St[(size_t)i * dv + j] * dot[j];
        dqt[i] = s;
      }
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] += qt[i] * dot[j];
      for (int i = 0; i < dk; ++i) {
        double s = 0.0;
        for (int j = 0; j < dv; ++j) s += dS[(size_t)i * dv + j] * vt[j];
        dkt[i] = s;
      }
      for (int j = 0; j < dv; ++j) dvt[j] = 0.0;
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) dvt[j] += dS[(size_t)i * dv + j] * kt[i];
      const double *bt = or_lb(J, vo, t);
      if (!bt) {
        for (int i = 0; i < dk; ++i) {
          double g = exp(at[i]), s = 0.0;
          for (int j = 0; j < dv; ++j) s += dS[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];
          dat[i] = g * s;
          for (int j = 0; j < dv; ++j) dS[(size_t)i * dv + j] *= g;
        }
      } else {
        double *dbt = J->dlb + vo + (size_t)t * dv;
        for (int j = 0; j < dv; ++j) dbt[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
          double g = exp(at[i]), s = 0.0;
          for (int j = 0; j < dv; ++j) {
            double G = g * exp(bt[j]);
            double c = dS[(size_t)i * dv + j] * G * Sp[(size_t)i * dv + j];
            s += c;
            dbt[j] += c;
            dS[(size_t)i * dv + j] *= G;
          }
          dat[i] = s;
        }
      }
    }
  }
  if (J->dh0) memcpy(J->dh0 + so, dS, sizeof(double) * SS);
  free(ck); free(seg); free(dS);
}

static void *or_fwd_worker(void *p) {
  or_job *J = (or_job *)p;
  for (int t = or_take(J); t < J->B * J->H; t = or_take(J)) or_fwd_head(J, t);
  return NULL;
}

static void *or_bwd_worker(void *p) {
  or_job *J = (or_job *)p;
  for (int t = or_take(J); t < J->B * J->H; t = or_take(J)) or_bwd_head(J, t);
  return NULL;
}

static int or_run(or_job *J, void *(*fn)(void *), int nthreads) {
  int tasks = J->B * J->H;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > tasks) nthreads = tasks;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  int started = 0;
  pthread_mutex_init(&J->mu, NULL);
  for (int i = 1; i < nthreads; ++i) {
    pthread_t t;
    if (pthread_create(&t, NULL, fn, J) == 0) th[started++] = t;
  }
  fn(J);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  pthread_mutex_destroy(&J->mu);
  return J->failed ? -2 : 0;
}

int gla_oracle_fwd(int B, int H, int L, int dk, int dv,
                   const double *q, const double *k, const double *v,
                   const double *log_alpha, const double *h0,
                   double *o, double *hT, int nthreads) {
  if (B < 0 || H < 0 || L < 0 || dk <= 0 || dv <= 0) return -1;
  if (B * H == 0) return 0;
  if ((L > 0) && (!q || !k || !v || !log_alpha || !o)) return -1;
  or_job J;
  memset(&J, 0, sizeof(J));
  J.B = B; J.H = H; J.L = L; J.dk = dk; J.dv = dv;
  J.q = q; J.k = k; J.v = v; J.la = log_alpha; J.h0 = h0; J.o = o; J.hT = hT;
  return or_run(&J, or_fwd_worker, nthreads);
}

int gla_oracle_bwd(int B, int H, int L, int dk, int dv,
                   const double *q, const double *k, const double *v,
                   const double *log_alpha, const double *h0,
                   const double *dout, const double *dhT,
                   double *dq, double *dkk, double *dvv, double *dlog_alpha,
                   double *dh0, int nthreads) {
  if (B < 0 || H < 0 || L < 0 || dk <= 0 || dv <= 0) return -1;
  if (B * H == 0) return 0;
  if ((L > 0) && (!q || !k || !v || !log_alpha || !dout || !dq || !dkk ||
                  !dvv || !dlog_alpha))
    return -1;
  or_job J;
  memset(&J, 0, sizeof(J));
  J.B = B; J.H = H; J.L = L; J.dk = dk; J.dv = dv;
  J.q = q; J.k = k; J.v = v; J.la = log_alpha; J.h0 = h0;
  J.dout = dout; J.dhT = dhT;
  J.dq = dq; J.dkk = dkk; J.dvv = dvv; J.dla = dlog_alpha; J.dh0 = dh0;
  return or_run(&J, or_bwd_worker, nthreads);
}

int ggla_oracle_fwd(int B, int H, int L, int dk, int dv,
                    const double *q, const double *k, const double *v,
                    const double *log_alpha, const double *log_beta, const double *h0,
                    double *o, double *hT, int nthreads) {
  if (B < 0 || H < 0 || L < 0 || dk <= 0 || dv <= 0) return -1;
  if (B * H == 0) return 0;
  if ((L > 0) && (!q || !k || !v || !log_alpha || !log_beta || !o)) return -1;
  or_job J;
  memset(&J, 0, sizeof(J));
  J.B = B; J.H = H; J.L = L; J.dk = dk; J.dv = dv;
  J.q = q; J.k = k; J.v = v; J.la = log_alpha; J.lb = log_beta; J.h0 = h0;
  J.o = o; J.hT = hT;
  return or_run(&J, or_fwd_worker, nthreads);
}

int ggla_oracle_bwd(int B, int H, int L, int dk, int dv,
                    const double *q, const double *k, const double *v,
                    const double *log_alpha, const double *log_beta, const double *h0,
                    const double *dout, const double *dhT,
                    double *dq, double *dkk, double *dvv, double *dlog_alpha,
                    double *dlog_beta, double *dh0, int nthreads) {
  if (B < 0 || H < 0 || L < 0 || dk <= 0 || dv <= 0) return -1;
  if (B * H == 0) return 0;
  if ((L > 0) && (!q || !k || !v || !log_alpha || !log_beta || !dout || !dq || !dkk ||
                  !dvv || !dlog_alpha || !dlog_beta))
    return -1;
  or_job J;
  memset(&J, 0, sizeof(J));
  J.B = B; J.H = H; J.L = L; J.dk = dk; J.dv = dv;
  J.q = q; J.k = k; J.v = v; J.la = log_alpha; J.lb = log_beta; J.h0 = h0;
  J.dout = dout; J.dhT = dhT;
  J.dq = dq; J.dkk = dkk; J.dvv = dvv; J.dla = dlog_alpha; J.dlb = dlog_beta; J.dh0 = dh0;
  return or_run(&J, or_bwd_worker, nthreads);
}
