/*
 * Driver for the sanitizer build of the oracle (gcc with AddressSanitizer and
 * UndefinedBehaviorSanitizer).  It runs the oracle's entry points over every
 * input dtype, head selection, column blocking and thread count on small
 * inputs, the worked example of the "Kimi K3 Technical Report review"
 * (jw9603.github.io), section 3.4, and the argument rejections; any invalid
 * memory access or undefined behaviour aborts the run.  Exit 0: clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_forward(const void *q, const void *k, const void *v, int qkv_dtype, const void *alpha,
                       int alpha_dtype, const void *beta, int beta_dtype, const void *S0, int s0_dtype,
                       double *o, double *S_T, int B, int T, int H, int dk, int dv, const int *heads, int n_sel,
                       int col_block, int order, int mutation, int nthreads);
int kda_oracle_decode_step(const void *q, const void *k, const void *v, int qkv_dtype, const void *alpha,
                           int alpha_dtype, const void *beta, int beta_dtype, double *S, double *o, int B, int H,
                           int dk, int dv, int col_block, int nthreads);

static uint64_t rng = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in [0, 1) */
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (double)(rng >> 11) * (1.0 / 9007199254740992.0);
}
static uint16_t to_bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static int fail(const char *what) {
  fprintf(stderr, "oracle sanitizer driver: %s\n", what);
  return 1;
}

int main(void) {
  enum { B = 2, T = 37, H = 3, DK = 16, DV = 8 };
  const size_t ntk = (size_t)B * T * H * DK, ntv = (size_t)B * T * H * DV, nt = (size_t)B * T * H;
  float *qf = malloc(ntk * 4), *kf = malloc(ntk * 4), *vf = malloc(ntv * 4), *af = malloc(ntk * 4);
  float *bf = malloc(nt * 4), *s0 = malloc((size_t)B * H * DK * DV * 4);
  uint16_t *qb = malloc(ntk * 2), *kb = malloc(ntk * 2), *vb = malloc(ntv * 2);
  double *ad = malloc(ntk * 8);
  for (size_t i = 0; i < ntk; ++i) {
    qf[i] = (float)(urand() - 0.5);
    kf[i] = (float)(urand() - 0.5);
    af[i] = (float)(0.6 + 0.4 * urand());
    ad[i] = af[i];
    qb[i] = to_bf16_bits(qf[i]);
    kb[i] = to_bf16_bits(kf[i]);
  }
  for (size_t i = 0; i < ntv; ++i) {
    vf[i] = (float)(urand() - 0.5);
    vb[i] = to_bf16_bits(vf[i]);
  }
  for (size_t i = 0; i < nt; ++i) bf[i] = (float)urand();
  for (size_t i = 0; i < (size_t)B * H * DK * DV; ++i) s0[i] = (float)(0.1 * (urand() - 0.5));

  double *o = malloc((size_t)B * H * T * DV * 8), *st = malloc((size_t)B * H * DK * DV * 8);
  const int heads[3] = {5, 0, 3};
  const int cbs[3] = {0, 3, 8}, ths[3] = {1, 2, 5};
  for (int dt = 0; dt < 2; ++dt)
    for (int c = 0; c < 3; ++c)
      for (int sel = 0; sel < 2; ++sel) {
        const void *q = dt ? (const void *)qb : qf, *k = dt ? (const void *)kb : kf, *v = dt ? (const void *)vb : vf;
        const int rc = kda_oracle_forward(q, k, v, dt, c == 1 ? (const void *)ad : af, c == 1 ? 2 : 0, bf, 0,
                                          sel ? s0 : NULL, 0, o, st, B, T, H, DK, DV, sel ? heads : NULL,
                                          sel ? 3 : B * H, cbs[c], c == 2, 0, ths[c]);
        if (rc != 0) return fail("forward rejected valid arguments");
        for (size_t i = 0; i < (size_t)(sel ? 3 : B * H) * DK * DV; ++i)
          if (!isfinite(st[i])) return fail("non-finite state");
      }
  for (int mut = 1; mut <= 7; ++mut)
    if (kda_oracle_forward(qf, kf, vf, 0, af, 0, bf, 0, s0, 0, o, st, B, T, H, DK, DV, NULL, B * H, 4, 0, mut, 3))
      return fail("forward rejected a planted mistake");
  /* T = 0, no outputs wanted */
  if (kda_oracle_forward(NULL, NULL, NULL, 0, NULL, 0, NULL, 0, s0, 0, NULL, st, B, 0, H, DK, DV, NULL, B * H, 0, 0, 0,
                         2))
    return fail("forward rejected T = 0");

  /* the worked example: unit key e0, Sbar^T k = 0.2, v = 0.8, beta = 0.5 -> 0.5 */
  {
    float q4[4] = {1, 0, 0, 0}, k4[4] = {1, 0, 0, 0}, v1[1] = {0.8f}, a4[4] = {1, 1, 1, 1}, b1[1] = {0.5f};
    float S4[4] = {0.2f, 0.7f, -0.3f, 0.1f};
    double o1[1], S1[4];
    if (kda_oracle_forward(q4, k4, v1, 0, a4, 0, b1, 0, S4, 0, o1, S1, 1, 1, 1, 4, 1, NULL, 1, 0, 0, 0, 1))
      return fail("worked example rejected");
    if (fabs(o1[0] - 0.5) > 1e-7) return fail("worked example does not read back 0.5");
  }

  /* decode: one step in place over B*H states */
  double *S = malloc((size_t)B * H * DK * DV * 8);
  for (size_t i = 0; i < (size_t)B * H * DK * DV; ++i) S[i] = s0[i];
  double od[B * H * DV];
  if (kda_oracle_decode_step(qb, kb, vb, 1, af, 0, bf, 0, S, od, B, H, DK, DV, 3, 4)) return fail("decode rejected");

  /* rejections */
  const int bad_heads[1] = {B * H};
  if (kda_oracle_forward(qf, kf, vf, 0, af, 0, bf, 0, NULL, 0, o, st, B, T, H, DK, DV, bad_heads, 1, 0, 0, 0, 1) != -1)
    return fail("out-of-range head accepted");
  if (kda_oracle_forward(qf, kf, vf, 0, af, 0, bf, 0, NULL, 0, o, st, 0, T, H, DK, DV, NULL, 0, 0, 0, 0, 1) != -1)
    return fail("B = 0 accepted");
  if (kda_oracle_forward(NULL, kf, vf, 0, af, 0, bf, 0, NULL, 0, o, st, B, T, H, DK, DV, NULL, B * H, 0, 0, 0, 1) != -1)
    return fail("missing q accepted");
  if (kda_oracle_decode_step(qb, kb, vb, 1, af, 0, bf, 0, NULL, od, B, H, DK, DV, 0, 1) != -1)
    return fail("decode without a state accepted");

  free(qf); free(kf); free(vf); free(af); free(bf); free(s0); free(qb); free(kb); free(vb); free(ad);
  free(o); free(st); free(S);
  puts("oracle sanitizer driver: clean");
  return 0;
}
