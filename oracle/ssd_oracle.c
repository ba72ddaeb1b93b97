/*
 * SSD forward oracle: the token-by-token selective state-space recurrence in
 * plain C, double precision throughout.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link or call
 * this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (page "ops-transformer MambaV2 算子套件", §1.1 and §1.3;
 * tensor semantics from page "Mamba-2 SSD for Ascend NPU", "Implementation"):
 * for every batch row b and head h independently, with group g = h / (H/G),
 *
 *   delta_t = clamp(softplus(dt[b,t,h] + dt_bias[h]), dt_min, dt_max)
 *             (softplus only when dt_softplus is set)
 *   S       = initial_state[b,h]  (P x N), or zero
 *   for t = 0 .. L-1:
 *       S      = exp(delta_t * A[h]) * S + delta_t * x[b,t,h,:] (outer) B[b,t,g,:]
 *       y      = S . C[b,t,g,:] + D[h] * x[b,t,h,:]
 *       y      = y * silu(z[b,t,h,:])          (only when z is given)
 *       out[b,t,h,:] = y
 *   final_state[b,h] = S
 *
 * The discretisation A_bar = exp(delta*A), B_bar x = delta*B*x is the plain
 * reading of "A_bar, B_bar from the step size" in §1.1 of the second page;
 * D is added before the gate, which multiplies last.
 *
 * Layouts (row-major, dense): x, z, out [B,L,H,P]; dt [B,L,H]; A, D,
 * dt_bias [H]; B, C [B,L,G,N]; initial_state, final_state [B,H,P,N].
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double softplus_d(double u) {
  /* log(1 + e^u); for large u it equals u to double precision. */
  return u > 30.0 ? u : log1p(exp(u));
}

static double silu_d(double v) { return v / (1.0 + exp(-v)); }

/* One (b, h) sequence.  S is caller-provided scratch of P*N doubles. */
static void recur_one(int64_t b, int64_t h, int64_t L, int64_t H, int64_t P,
                      int64_t N, int64_t G, const double *x, const double *dt,
                      const double *A, const double *Bm, const double *Cm,
                      const double *D, const double *z, const double *dt_bias,
                      const double *h0, int dt_softplus, double dt_min,
                      double dt_max, double *out, double *final_state,
                      double *S) {
  const int64_t g = h / (H / G);
  if (h0)
    memcpy(S, h0 + (b * H + h) * P * N, (size_t)(P * N) * sizeof(double));
  else
    memset(S, 0, (size_t)(P * N) * sizeof(double));
  const double a_h = A[h];
  const double d_h = D ? D[h] : 0.0;
  const double bias = dt_bias ? dt_bias[h] : 0.0;
  for (int64_t t = 0; t < L; ++t) {
    double delta = dt[(b * L + t) * H + h] + bias;
    if (dt_softplus) delta = softplus_d(delta);
    if (delta < dt_min) delta = dt_min;
    if (delta > dt_max) delta = dt_max;
    const double decay = exp(delta * a_h);
    const double *xt = x + ((b * L + t) * H + h) * P;
    const double *bt = Bm + ((b * L + t) * G + g) * N;
    const double *ct = Cm + ((b * L + t) * G + g) * N;
    double *yt = out + ((b * L + t) * H + h) * P;
    for (int64_t p = 0; p < P; ++p) {
      double *Sp = S + p * N;
      const double dx = delta * xt[p];
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        Sp[n] = decay * Sp[n] + dx * bt[n];
        acc += Sp[n] * ct[n];
      }
      double y = acc + d_h * xt[p];
      if (z) y *= silu_d(z[((b * L + t) * H + h) * P + p]);
      yt[p] = y;
    }
  }
  if (final_state)
    memcpy(final_state + (b * H + h) * P * N, S,
           (size_t)(P * N) * sizeof(double));
}

/*
 * Runs the recurrence for the (b, h) pairs listed in `pairs` (2*npairs
 * int64: b0,h0,b1,h1,...), or for all B*H pairs when pairs is NULL.  Only
 * those pairs' slices of `out` / `final_state` are written.  Optional
 * pointers (D, z, dt_bias, h0, final_state) may be NULL.  nthreads <= 0 uses
 * the OpenMP default.  Returns 0 on success, 1 on a bad argument, 2 when out
 * of memory.
 */
int ssd_oracle_f64(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t N,
                   int64_t G, const double *x, const double *dt,
                   const double *A, const double *Bm, const double *Cm,
                   const double *D, const double *z, const double *dt_bias,
                   const double *h0, int dt_softplus, double dt_min,
                   double dt_max, const int64_t *pairs, int64_t npairs,
                   double *out, double *final_state, int nthreads) {
  if (Bsz < 1 || L < 1 || H < 1 || P < 1 || N < 1 || G < 1 || H % G != 0)
    return 1;
  if (!x || !dt || !A || !Bm || !Cm || !out) return 1;
  const int64_t total = pairs ? npairs : Bsz * H;
  if (pairs) {
    for (int64_t i = 0; i < npairs; ++i)
      if (pairs[2 * i] < 0 || pairs[2 * i] >= Bsz || pairs[2 * i + 1] < 0 ||
          pairs[2 * i + 1] >= H)
        return 1;
  }
  int err = 0;
#ifdef _OPENMP
  /* a clause, not omp_set_num_threads: the thread count of one call must
     not leak into later calls */
  const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
  {
    double *S = (double *)malloc((size_t)(P * N) * sizeof(double));
    if (!S) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      err = 2;
    }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t i = 0; i < total; ++i) {
      if (!S) continue;
      const int64_t b = pairs ? pairs[2 * i] : i / H;
      const int64_t h = pairs ? pairs[2 * i + 1] : i % H;
      recur_one(b, h, L, H, P, N, G, x, dt, A, Bm, Cm, D, z, dt_bias, h0,
                dt_softplus, dt_min, dt_max, out, final_state, S);
    }
    free(S);
  }
  return err;
}

/*
 * The same recurrence in single precision: a float instance of recur_one and
 * of the driver above, statement for statement (expf, log1pf for the
 * softplus).  It is not a parity reference -- the fp64 function is -- but the
 * CPU baseline the benchmark times: the plain recurrence at the precision of
 * the GPU's public tensors.
 */
static float softplus_f(float u) { return u > 15.0f ? u : log1pf(expf(u)); }

static float silu_f(float v) { return v / (1.0f + expf(-v)); }

static void recur_one_f32(int64_t b, int64_t h, int64_t L, int64_t H, int64_t P,
                          int64_t N, int64_t G, const float *x, const float *dt,
                          const float *A, const float *Bm, const float *Cm,
                          const float *D, const float *z, const float *dt_bias,
                          const float *h0, int dt_softplus, float dt_min,
                          float dt_max, float *out, float *final_state,
                          float *S) {
  const int64_t g = h / (H / G);
  if (h0)
    memcpy(S, h0 + (b * H + h) * P * N, (size_t)(P * N) * sizeof(float));
  else
    memset(S, 0, (size_t)(P * N) * sizeof(float));
  const float a_h = A[h];
  const float d_h = D ? D[h] : 0.0f;
  const float bias = dt_bias ? dt_bias[h] : 0.0f;
  for (int64_t t = 0; t < L; ++t) {
    float delta = dt[(b * L + t) * H + h] + bias;
    if (dt_softplus) delta = softplus_f(delta);
    if (delta < dt_min) delta = dt_min;
    if (delta > dt_max) delta = dt_max;
    const float decay = expf(delta * a_h);
    const float *xt = x + ((b * L + t) * H + h) * P;
    const float *bt = Bm + ((b * L + t) * G + g) * N;
    const float *ct = Cm + ((b * L + t) * G + g) * N;
    float *yt = out + ((b * L + t) * H + h) * P;
    for (int64_t p = 0; p < P; ++p) {
      float *Sp = S + p * N;
      const float dx = delta * xt[p];
      float acc = 0.0f;
      for (int64_t n = 0; n < N; ++n) {
        Sp[n] = decay * Sp[n] + dx * bt[n];
        acc += Sp[n] * ct[n];
      }
      float y = acc + d_h * xt[p];
      if (z) y *= silu_f(z[((b * L + t) * H + h) * P + p]);
      yt[p] = y;
    }
  }
  if (final_state)
    memcpy(final_state + (b * H + h) * P * N, S,
           (size_t)(P * N) * sizeof(float));
}

/* Single-precision counterpart of ssd_oracle_f64 (same arguments and return
 * codes, float tensors). */
int ssd_oracle_f32(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t N,
                   int64_t G, const float *x, const float *dt, const float *A,
                   const float *Bm, const float *Cm, const float *D,
                   const float *z, const float *dt_bias, const float *h0,
                   int dt_softplus, float dt_min, float dt_max,
                   const int64_t *pairs, int64_t npairs, float *out,
                   float *final_state, int nthreads) {
  if (Bsz < 1 || L < 1 || H < 1 || P < 1 || N < 1 || G < 1 || H % G != 0)
    return 1;
  if (!x || !dt || !A || !Bm || !Cm || !out) return 1;
  const int64_t total = pairs ? npairs : Bsz * H;
  if (pairs) {
    for (int64_t i = 0; i < npairs; ++i)
      if (pairs[2 * i] < 0 || pairs[2 * i] >= Bsz || pairs[2 * i + 1] < 0 ||
          pairs[2 * i + 1] >= H)
        return 1;
  }
  int err = 0;
#ifdef _OPENMP
  /* a clause, not omp_set_num_threads: the thread count of one call must
     not leak into later calls */
  const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
  {
    float *S = (float *)malloc((size_t)(P * N) * sizeof(float));
    if (!S) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      err = 2;
    }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t i = 0; i < total; ++i) {
      if (!S) continue;
      const int64_t b = pairs ? pairs[2 * i] : i / H;
      const int64_t h = pairs ? pairs[2 * i + 1] : i % H;
      recur_one_f32(b, h, L, H, P, N, G, x, dt, A, Bm, Cm, D, z, dt_bias, h0,
                    dt_softplus, dt_min, dt_max, out, final_state, S);
    }
    free(S);
  }
  return err;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int ssd_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
