/*
 * CPU oracle for causal sliding-window multi-head attention with rotary
 * position embedding (RoPE), in float64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes (Voxtral Realtime 2602 audio encoder; transcribe.cpp
 * "Voxtral" family notes, section Architecture, Voxtral Realtime 2602): each
 * encoder frame is a query that attends causally to the most recent W frames
 * (itself included), W = 750, with RoPE (theta = 1e6, head_dim 64) applied to
 * queries and keys, 32 heads, plain multi-head (no grouping).  The streaming
 * form (same page, "Streaming schedule": 4 encoder frames per step) appends
 * frames to a W-slot ring of rotated keys and values.
 *
 * Readings where the pages are silent:
 *   - window: keys j with t-W+1 <= j <= t (W keys including the query);
 *   - RoPE: half-split pairing (i, i+D/2), frequency f_i = theta^(-2i/D),
 *     angle = position * f_i, computed in float64;
 *   - scale: 1/sqrt(D) unless given;
 *   - bf16 contract: in bf16 mode the rotated q and k are rounded to bfloat16
 *     (nearest, ties to even) before the scores, as the storage dtype of a
 *     rotated tensor is bf16; everything after that is exact float64.
 *
 * Every function here is pinned by CPU tests against brute force, a library
 * attention routine, closed forms and invariants (tests/test_oracle_pins.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <fenv.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- bfloat16 rounding, written from the definition of the format ------
 * bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and the float32
 * exponent range.  Nearest representable value, ties to the even
 * significand; below the smallest normal (2^-126) the spacing stays 2^-133. */
double oracle_bf16_round(double x) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  int e;
  double m = frexp(fabs(x), &e); /* |x| = m * 2^e, m in [0.5, 1) */
  /* significand of 8 bits: value = N * 2^(e-8), N in [128, 256) */
  int shift = 8;
  if (e - 1 < -126) shift = 8 - (-126 - (e - 1)); /* subnormal range: fewer bits */
  double scaled = ldexp(m, shift);
  double n = nearbyint(scaled); /* default rounding mode: nearest, ties to even */
  double r = ldexp(n, e - shift);
  if (r > 3.3895313892515355e38) r = INFINITY; /* beyond the largest bf16 */
  return x < 0 ? -r : r;
}

void oracle_bf16_round_array(double *x, int64_t n) {
  for (int64_t i = 0; i < n; ++i) x[i] = oracle_bf16_round(x[i]);
}

/* ---- RoPE (half-split pairing) -------------------------------------------
 * Rotates vector x (length D) for absolute position p:
 *   x'[i]       = x[i] cos(a_i) - x[i+D/2] sin(a_i)
 *   x'[i+D/2]   = x[i+D/2] cos(a_i) + x[i] sin(a_i)
 * with a_i = p * theta^(-2i/D), i = 0 .. D/2-1. */
static void rope_vec(double *x, int64_t D, int64_t p, double theta) {
  int64_t half = D / 2;
  for (int64_t i = 0; i < half; ++i) {
    double f = pow(theta, -2.0 * (double)i / (double)D);
    double a = (double)p * f;
    double c = cos(a), s = sin(a);
    double x0 = x[i], x1 = x[i + half];
    x[i] = x0 * c - x1 * s;
    x[i + half] = x1 * c + x0 * s;
  }
}

/* Rotate rows of x [B,T,H,D] in place; row (b,t,*) sits at position pos[b*T+t]
 * (pos == NULL means position t).  If bf16 != 0 the results are rounded to
 * bfloat16. */
void oracle_rope(double *x, int64_t B, int64_t T, int64_t H, int64_t D,
                 const int64_t *pos, double theta, int bf16) {
  for (int64_t b = 0; b < B; ++b)
    for (int64_t t = 0; t < T; ++t) {
      int64_t p = pos ? pos[b * T + t] : t;
      for (int64_t h = 0; h < H; ++h) {
        double *row = x + ((b * T + t) * H + h) * D;
        rope_vec(row, D, p, theta);
        if (bf16)
          for (int64_t d = 0; d < D; ++d) row[d] = oracle_bf16_round(row[d]);
      }
    }
}

/* Softmax attention of one query over a set of key rows given by pointer
 * lists: o = sum_j softmax_j(scale * q.k_j) v_j.  Two passes: max, then
 * normalised exponentials. */
static void attend(const double *q, const double *const *keys, const double *const *vals,
                   int64_t nk, int64_t D, double scale, double *s, double *o) {
  double m = -INFINITY;
  for (int64_t j = 0; j < nk; ++j) {
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d) acc += q[d] * keys[j][d];
    s[j] = scale * acc;
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < nk; ++j) {
    s[j] = exp(s[j] - m);
    l += s[j];
  }
  for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
  for (int64_t j = 0; j < nk; ++j) {
    double w = s[j] / l;
    for (int64_t d = 0; d < D; ++d) o[d] += w * vals[j][d];
  }
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
  return nthreads;
#else
  (void)nthreads;
  return 1;
#endif
}

/* Whole-chunk prefill.
 * q,k,v,o: [B,T,H,D] float64.  pos: [B*T] absolute positions or NULL (= t).
 * Query t attends to keys j = max(0,t-W+1) .. t of the same (b,h).
 * rope_applied != 0: q and k are already rotated (no rotation, no rounding).
 * Returns 0, or -1 on bad arguments / allocation failure. */
int oracle_prefill(const double *q, const double *k, const double *v, double *o,
                   int64_t B, int64_t T, int64_t H, int64_t D, int64_t W,
                   const int64_t *pos, double theta, double scale, int bf16,
                   int rope_applied, int nthreads) {
  if (B < 0 || T < 0 || H < 1 || D < 2 || (D & 1) || W < 1) return -1;
  if (B == 0 || T == 0) return 0;
  size_t n = (size_t)(B * T * H * D);
  double *qr = (double *)malloc(n * sizeof(double));
  double *kr = (double *)malloc(n * sizeof(double));
  if (!qr || !kr) { free(qr); free(kr); return -1; }
  memcpy(qr, q, n * sizeof(double));
  memcpy(kr, k, n * sizeof(double));
  if (!rope_applied) {
    oracle_rope(qr, B, T, H, D, pos, theta, bf16);
    oracle_rope(kr, B, T, H, D, pos, theta, bf16);
  }
  int nt = set_threads(nthreads);
  int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nt) reduction(| : err)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h) {
      int64_t cap = W < T ? W : T;
      double *s = (double *)malloc((size_t)cap * sizeof(double));
      const double **kp = (const double **)malloc((size_t)cap * sizeof(double *));
      const double **vp = (const double **)malloc((size_t)cap * sizeof(double *));
      if (!s || !kp || !vp) { err |= 1; free(s); free(kp); free(vp); continue; }
      for (int64_t t = 0; t < T; ++t) {
        int64_t j0 = t - W + 1 < 0 ? 0 : t - W + 1;
        int64_t nk = 0;
        for (int64_t j = j0; j <= t; ++j, ++nk) {
          kp[nk] = kr + ((b * T + j) * H + h) * D;
          vp[nk] = v + ((b * T + j) * H + h) * D;
        }
        attend(qr + ((b * T + t) * H + h) * D, kp, vp, nk, D, scale, s,
               o + ((b * T + t) * H + h) * D);
      }
      free(s); free(kp); free(vp);
    }
  free(qr);
  free(kr);
  return err ? -1 : 0;
}

/* One streaming step for S streams with n new frames each.
 * q_new,k_new,v_new,o: [S,n,H,D].  ring_k (rotated keys), ring_v: [S,H,W,D];
 * slot j of a ring holds the frame at position p with p mod W == j.
 * pos[S]: absolute position of the first new frame (= frames seen so far).
 * New query i (position P+i) attends to ring frames at positions
 * max(0, P+i-W+1) .. P-1 and to new frames P .. P+i.  Reads the ring only.
 * Requires 1 <= n <= W.  Returns 0 or -1. */
int oracle_stream_step(const double *q_new, const double *k_new, const double *v_new,
                       const double *ring_k, const double *ring_v, const int64_t *pos,
                       double *o, int64_t S, int64_t n, int64_t H, int64_t D, int64_t W,
                       double theta, double scale, int bf16, int rope_applied, int nthreads) {
  if (S < 0 || n < 1 || n > W || H < 1 || D < 2 || (D & 1) || W < 1) return -1;
  if (S == 0) return 0;
  size_t cnt = (size_t)(S * n * H * D);
  double *qr = (double *)malloc(cnt * sizeof(double));
  double *kr = (double *)malloc(cnt * sizeof(double));
  int64_t *p = (int64_t *)malloc((size_t)(S * n) * sizeof(int64_t));
  if (!qr || !kr || !p) { free(qr); free(kr); free(p); return -1; }
  memcpy(qr, q_new, cnt * sizeof(double));
  memcpy(kr, k_new, cnt * sizeof(double));
  for (int64_t s = 0; s < S; ++s)
    for (int64_t i = 0; i < n; ++i) p[s * n + i] = pos[s] + i;
  if (!rope_applied) {
    oracle_rope(qr, S, n, H, D, p, theta, bf16);
    oracle_rope(kr, S, n, H, D, p, theta, bf16);
  }
  int nt = set_threads(nthreads);
  int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nt) reduction(| : err)
  for (int64_t s = 0; s < S; ++s)
    for (int64_t h = 0; h < H; ++h) {
      int64_t cap = W + n;
      double *sc = (double *)malloc((size_t)cap * sizeof(double));
      const double **kp = (const double **)malloc((size_t)cap * sizeof(double *));
      const double **vp = (const double **)malloc((size_t)cap * sizeof(double *));
      if (!sc || !kp || !vp) { err |= 1; free(sc); free(kp); free(vp); continue; }
      int64_t P = pos[s];
      for (int64_t i = 0; i < n; ++i) {
        int64_t lo = P + i - W + 1 < 0 ? 0 : P + i - W + 1;
        int64_t nk = 0;
        for (int64_t pp = lo; pp < P; ++pp, ++nk) { /* history from the ring */
          int64_t slot = pp % W;
          kp[nk] = ring_k + ((s * H + h) * W + slot) * D;
          vp[nk] = ring_v + ((s * H + h) * W + slot) * D;
        }
        /* new frames P .. P+i: all inside the window because n <= W */
        for (int64_t jj = 0; jj <= i; ++jj, ++nk) {
          kp[nk] = kr + ((s * n + jj) * H + h) * D;
          vp[nk] = v_new + ((s * n + jj) * H + h) * D;
        }
        attend(qr + ((s * n + i) * H + h) * D, kp, vp, nk, D, scale, sc,
               o + ((s * n + i) * H + h) * D);
      }
      free(sc); free(kp); free(vp);
    }
  free(qr); free(kr); free(p);
  return err ? -1 : 0;
}

/* Append n new frames per stream: rotate k_new (unless rope_applied; bf16
 * rounding in bf16 mode), write rotated k and raw v to slot (pos[s]+i) mod W,
 * then pos[s] += n.  Requires 1 <= n <= W.  Returns 0 or -1. */
int oracle_ring_append(double *ring_k, double *ring_v, const double *k_new, const double *v_new,
                       int64_t *pos, int64_t S, int64_t n, int64_t H, int64_t D, int64_t W,
                       double theta, int bf16, int rope_applied) {
  if (S < 0 || n < 1 || n > W || H < 1 || D < 2 || (D & 1) || W < 1) return -1;
  double *row = (double *)malloc((size_t)D * sizeof(double));
  if (!row) return -1;
  for (int64_t s = 0; s < S; ++s) {
    for (int64_t i = 0; i < n; ++i) {
      int64_t p = pos[s] + i;
      int64_t slot = p % W;
      for (int64_t h = 0; h < H; ++h) {
        const double *src = k_new + ((s * n + i) * H + h) * D;
        memcpy(row, src, (size_t)D * sizeof(double));
        if (!rope_applied) {
          rope_vec(row, D, p, theta);
          if (bf16)
            for (int64_t d = 0; d < D; ++d) row[d] = oracle_bf16_round(row[d]);
        }
        memcpy(ring_k + ((s * H + h) * W + slot) * D, row, (size_t)D * sizeof(double));
        memcpy(ring_v + ((s * H + h) * W + slot) * D, v_new + ((s * n + i) * H + h) * D,
               (size_t)D * sizeof(double));
      }
    }
    pos[s] += n;
  }
  free(row);
  return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
