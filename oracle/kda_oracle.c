/*
 * KDA oracle: a plain, slow, token-by-token fp64 CPU implementation of the
 * Kimi Delta Attention recurrence.  TEST INFRASTRUCTURE ONLY: the tests, the
 * smoke check and the benchmark's CPU-baseline leg may call it; the product
 * path (libkda) never does, and the two share no code.
 *
 * What it computes (the definition, written out):
 *
 *   "Kimi K3 Technical Report review" (jw9603.github.io), section 3.2, update
 *   equation:  S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *   readout o_t = S_t^T q_t (the post-update state), S_t in R^{d_k x d_v}.
 *
 *   Same page, section 3.3 (delta form), which this file follows step by step:
 *     Sbar = Diag(alpha_t) S_{t-1}                     (decay: row i scaled by alpha_t[i],
 *                                                      the Diag example of section 3.2)
 *     x    = Sbar^T k_t                                (what the memory predicts for k_t)
 *     S_t  = Sbar + beta_t k_t (v_t - x)^T             (correct only the error)
 *     o_t  = S_t^T q_t
 *
 * Decay happens before the write, and the prediction uses the decayed state.
 * The second page ("Kimi 모델 분석", rlaope.github.io, KDA section) writes the
 * transition as Diag(alpha)(I - beta k k^T) acting on a d_v x d_k state from the
 * right; transposed, that is the same operator.  Read literally as a left
 * multiplication of a d_k x d_v state it would write before decaying; that
 * reading is kept here only behind `order = KDA_ORACLE_ORDER_LITERAL_P2`, so a
 * test can show the GPU path matches the first reading and not the second.
 *
 * Inputs are taken in the dtype the GPU consumed (fp32, or bf16 as raw 16-bit
 * patterns) and widened exactly to fp64 per element, so input rounding is not
 * counted as error.  All arithmetic is fp64.
 *
 * Parallelism: one work item is (sequence b, head h, block of state columns).
 * Column j of S_t depends only on column j of S_{t-1} and on v_t[j] (every
 * step above acts on columns independently), so column blocks are independent
 * and each thread runs the plain recurrence on its own columns.  Results do not
 * depend on the thread count.
 *
 * `mutation` plants one deliberate mistake (test use only, default 0 = none), so
 * the pin tests can show each plausible mistake is caught by at least one pin.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KDA_ORACLE_F32 0
#define KDA_ORACLE_BF16 1
#define KDA_ORACLE_F64 2

#define KDA_ORACLE_ORDER_PAGE1 0
#define KDA_ORACLE_ORDER_LITERAL_P2 1

enum {
  MUT_NONE = 0,
  MUT_NO_DECAY = 1,          /* skip Diag(alpha) */
  MUT_DELTA_SIGN = 2,        /* S += beta k (x - v)^T */
  MUT_READ_PRE_UPDATE = 3,   /* o from Sbar instead of S_t */
  MUT_DECAY_COLUMNS = 4,     /* alpha indexed by the state column (mod d_k) */
  MUT_PREDICT_UNDECAYED = 5, /* x = S_{t-1}^T k instead of Sbar^T k */
  MUT_DROP_BETA = 6,         /* beta treated as 1 */
  MUT_READ_WITH_K = 7,       /* readout uses k instead of q */
};

static double load_elem(const void *p, int dtype, int64_t idx) {
  if (dtype == KDA_ORACLE_F32) return (double)((const float *)p)[idx];
  if (dtype == KDA_ORACLE_F64) return ((const double *)p)[idx];
  /* bf16: the top 16 bits of an IEEE binary32 */
  uint32_t bits = (uint32_t)((const uint16_t *)p)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

typedef struct {
  const void *q, *k, *v, *alpha, *beta, *S0;
  int qkv_dtype, alpha_dtype, beta_dtype, s0_dtype;
  double *o;   /* [n_sel][T][d_v] or NULL */
  double *S_T; /* [n_sel][d_k][d_v] or NULL */
  int B, T, H, dk, dv;
  const int *heads; /* selected (b*H + h) ids, or NULL for all */
  int n_sel;
  int col_block;
  int order, mutation;
  /* work distribution */
  int n_items;
  int next_item;
  pthread_mutex_t lock;
} job_t;

/* Run the recurrence for one (sequence, head) on state columns [j0, j1). */
static void run_item(job_t *jb, int sel, int j0, int j1) {
  const int bh = jb->heads ? jb->heads[sel] : sel;
  const int b = bh / jb->H, h = bh % jb->H;
  const int dk = jb->dk, dv = jb->dv, nj = j1 - j0;
  double *S = (double *)calloc((size_t)dk * nj, sizeof(double));
  double *kv = (double *)malloc(sizeof(double) * dk);
  double *qv = (double *)malloc(sizeof(double) * dk);
  double *av = (double *)malloc(sizeof(double) * dk);
  double *vv = (double *)malloc(sizeof(double) * nj);
  double *x = (double *)malloc(sizeof(double) * nj);
  double *y = (double *)malloc(sizeof(double) * nj);

  if (jb->S0) {
    const int64_t base = (int64_t)bh * dk * dv;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < nj; ++j)
        S[(int64_t)i * nj + j] = load_elem(jb->S0, jb->s0_dtype, base + (int64_t)i * dv + j0 + j);
  }

  for (int t = 0; t < jb->T; ++t) {
    /* token-major layout [B][T][H][d] */
    const int64_t tok = ((int64_t)b * jb->T + t) * jb->H + h;
    for (int i = 0; i < dk; ++i) {
      kv[i] = load_elem(jb->k, jb->qkv_dtype, tok * dk + i);
      qv[i] = load_elem(jb->q, jb->qkv_dtype, tok * dk + i);
      av[i] = load_elem(jb->alpha, jb->alpha_dtype, tok * dk + i);
    }
    for (int j = 0; j < nj; ++j) vv[j] = load_elem(jb->v, jb->qkv_dtype, tok * dv + j0 + j);
    double beta = load_elem(jb->beta, jb->beta_dtype, tok);
    if (jb->mutation == MUT_DROP_BETA) beta = 1.0;

    if (jb->order == KDA_ORACLE_ORDER_LITERAL_P2) {
      /* S_t = Diag(alpha)(I - beta k k^T) S_{t-1} + beta k v^T, read as a left
         multiplication: write-then-decay. Used only to show the two readings differ. */
      for (int j = 0; j < nj; ++j) x[j] = 0.0;
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < nj; ++j) x[j] += kv[i] * S[(int64_t)i * nj + j];
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < nj; ++j) S[(int64_t)i * nj + j] -= beta * kv[i] * x[j];
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < nj; ++j) S[(int64_t)i * nj + j] *= av[i];
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < nj; ++j) S[(int64_t)i * nj + j] += beta * kv[i] * vv[j];
    } else {
      if (jb->mutation == MUT_PREDICT_UNDECAYED) {
        for (int j = 0; j < nj; ++j) x[j] = 0.0;
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < nj; ++j) x[j] += kv[i] * S[(int64_t)i * nj + j];
      }
      /* 1. decay: Sbar = Diag(alpha_t) S_{t-1}; row i (key channel i) scaled by alpha_t[i] */
      if (jb->mutation != MUT_NO_DECAY) {
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < nj; ++j) {
            const double a = (jb->mutation == MUT_DECAY_COLUMNS) ? av[(j0 + j) % dk] : av[i];
            S[(int64_t)i * nj + j] *= a;
          }
      }
      /* 2. predict: x = Sbar^T k_t */
      if (jb->mutation != MUT_PREDICT_UNDECAYED) {
        for (int j = 0; j < nj; ++j) x[j] = 0.0;
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < nj; ++j) x[j] += kv[i] * S[(int64_t)i * nj + j];
      }
      if (jb->mutation == MUT_READ_PRE_UPDATE) {
        for (int j = 0; j < nj; ++j) y[j] = 0.0;
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < nj; ++j) y[j] += S[(int64_t)i * nj + j] * qv[i];
      }
      /* 3. write: S_t = Sbar + beta_t k_t (v_t - x)^T */
      for (int j = 0; j < nj; ++j) {
        const double err = (jb->mutation == MUT_DELTA_SIGN) ? (x[j] - vv[j]) : (vv[j] - x[j]);
        x[j] = beta * err;
      }
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < nj; ++j) S[(int64_t)i * nj + j] += kv[i] * x[j];
    }

    /* 4. read: o_t = S_t^T q_t */
    if (jb->o) {
      if (jb->mutation != MUT_READ_PRE_UPDATE) {
        const double *rd = (jb->mutation == MUT_READ_WITH_K) ? kv : qv;
        for (int j = 0; j < nj; ++j) y[j] = 0.0;
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < nj; ++j) y[j] += S[(int64_t)i * nj + j] * rd[i];
      }
      double *orow = jb->o + ((int64_t)sel * jb->T + t) * dv + j0;
      for (int j = 0; j < nj; ++j) orow[j] = y[j];
    }
  }

  if (jb->S_T) {
    double *dst = jb->S_T + (int64_t)sel * dk * dv;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < nj; ++j) dst[(int64_t)i * dv + j0 + j] = S[(int64_t)i * nj + j];
  }
  free(S); free(kv); free(qv); free(av); free(vv); free(x); free(y);
}

static void *worker(void *arg) {
  job_t *jb = (job_t *)arg;
  const int nblk = (jb->dv + jb->col_block - 1) / jb->col_block;
  for (;;) {
    pthread_mutex_lock(&jb->lock);
    const int item = jb->next_item++;
    pthread_mutex_unlock(&jb->lock);
    if (item >= jb->n_items) break;
    const int sel = item / nblk, blk = item % nblk;
    const int j0 = blk * jb->col_block;
    const int j1 = (j0 + jb->col_block < jb->dv) ? j0 + jb->col_block : jb->dv;
    run_item(jb, sel, j0, j1);
  }
  return NULL;
}

/*
 * Forward over T tokens for the selected heads.
 *   q, k, alpha: [B][T][H][d_k]; v: [B][T][H][d_v]; beta: [B][T][H]  (token-major)
 *   S0: [B][H][d_k][d_v] or NULL (zeros)
 *   o: [n_sel][T][d_v] fp64 or NULL; S_T: [n_sel][d_k][d_v] fp64 or NULL
 *   heads: n_sel ids (b*H + h), or NULL with n_sel = B*H
 *   col_block: state columns per work item (<= 0: all of d_v)
 * Returns 0 on success, -1 on bad arguments.
 */
int kda_oracle_forward(const void *q, const void *k, const void *v, int qkv_dtype,
                       const void *alpha, int alpha_dtype, const void *beta, int beta_dtype,
                       const void *S0, int s0_dtype, double *o, double *S_T,
                       int B, int T, int H, int dk, int dv,
                       const int *heads, int n_sel, int col_block,
                       int order, int mutation, int nthreads) {
  if (B < 1 || H < 1 || T < 0 || dk < 1 || dv < 1) return -1;
  if (T > 0 && (!q || !k || !v || !alpha || !beta)) return -1;
  if (!heads) n_sel = B * H;
  if (n_sel < 0) return -1;
  for (int s = 0; heads && s < n_sel; ++s)
    if (heads[s] < 0 || heads[s] >= B * H) return -1;
  job_t jb;
  memset(&jb, 0, sizeof jb);
  jb.q = q; jb.k = k; jb.v = v; jb.alpha = alpha; jb.beta = beta; jb.S0 = S0;
  jb.qkv_dtype = qkv_dtype; jb.alpha_dtype = alpha_dtype; jb.beta_dtype = beta_dtype;
  jb.s0_dtype = s0_dtype; jb.o = o; jb.S_T = S_T;
  jb.B = B; jb.T = T; jb.H = H; jb.dk = dk; jb.dv = dv;
  jb.heads = heads; jb.n_sel = n_sel;
  jb.col_block = (col_block <= 0 || col_block > dv) ? dv : col_block;
  jb.order = order; jb.mutation = mutation;
  jb.n_items = n_sel * ((dv + jb.col_block - 1) / jb.col_block);
  pthread_mutex_init(&jb.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > jb.n_items) nthreads = jb.n_items > 0 ? jb.n_items : 1;
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
  for (int i = 1; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &jb);
  worker(&jb);
  for (int i = 1; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&jb.lock);
  return 0;
}

/*
 * One decode step for B*H independent states: exactly one iteration of the
 * recurrence above, applied to S in place.
 *   q, k, alpha: [B][H][d_k]; v: [B][H][d_v]; beta: [B][H]
 *   S: [B][H][d_k][d_v] fp64, updated in place; o: [B][H][d_v] fp64 (or NULL)
 */
int kda_oracle_decode_step(const void *q, const void *k, const void *v, int qkv_dtype,
                           const void *alpha, int alpha_dtype, const void *beta, int beta_dtype,
                           double *S, double *o, int B, int H, int dk, int dv,
                           int col_block, int nthreads) {
  if (!S) return -1;
  /* A decode token is a length-1 sequence in the [B][T=1][H][d] layout. */
  return kda_oracle_forward(q, k, v, qkv_dtype, alpha, alpha_dtype, beta, beta_dtype,
                            S, KDA_ORACLE_F64, o, S, B, 1, H, dk, dv, NULL, B * H,
                            col_block, KDA_ORACLE_ORDER_PAGE1, MUT_NONE, nthreads);
}
