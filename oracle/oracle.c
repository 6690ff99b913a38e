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
 * The text decoder of the same model (same page and section) uses the same
 * attention with grouped queries: 32 query heads over 8 key/value heads,
 * head_dim 128, a sliding window of 8192 tokens and RoPE theta 1e6, decoded
 * one token at a time over a ring of the same kind.  The functions below
 * take the grouped form as the general one (oracle_gqa_*); the multi-head
 * entry points are that form with as many key/value heads as query heads.
 *
 * Readings where the pages are silent:
 *   - window: keys j with t-W+1 <= j <= t (W keys including the query);
 *   - RoPE: half-split pairing (i, i+D/2), frequency f_i = theta^(-2i/D),
 *     angle = position * f_i, computed in float64;
 *   - scale: 1/sqrt(D) unless given;
 *   - grouping: query head h reads key/value head h / (Hq/Hkv), i.e. each
 *     key/value head serves Hq/Hkv consecutive query heads (the
 *     repeat_interleave layout the Core AI page names for its decoder);
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

/* Whole-chunk prefill, grouped-query form.
 * q,o: [B,T,Hq,D]; k,v: [B,T,Hkv,D] float64.  pos: [B*T] absolute positions
 * or NULL (= t).  Query t of query head h attends to keys j = max(0,t-W+1)
 * .. t of key/value head h / (Hq/Hkv), same b.  With Hkv == Hq this is plain
 * multi-head attention (the audio encoder); the text decoder of the same
 * model groups 32 query heads over 8 key/value heads (transcribe.cpp
 * "Voxtral" family notes, Architecture), each key/value head serving Hq/Hkv
 * consecutive query heads.
 * rope_applied != 0: q and k are already rotated (no rotation, no rounding).
 * Returns 0, or -1 on bad arguments (Hq % Hkv != 0 included) or allocation
 * failure. */
int oracle_gqa_prefill(const double *q, const double *k, const double *v, double *o,
                       int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, int64_t W,
                       const int64_t *pos, double theta, double scale, int bf16,
                       int rope_applied, int nthreads) {
  if (B < 0 || T < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 2 || (D & 1) || W < 1) return -1;
  if (B == 0 || T == 0) return 0;
  const int64_t G = Hq / Hkv;
  size_t nq = (size_t)(B * T * Hq * D), nkv = (size_t)(B * T * Hkv * D);
  double *qr = (double *)malloc(nq * sizeof(double));
  double *kr = (double *)malloc(nkv * sizeof(double));
  if (!qr || !kr) { free(qr); free(kr); return -1; }
  memcpy(qr, q, nq * sizeof(double));
  memcpy(kr, k, nkv * sizeof(double));
  if (!rope_applied) {
    oracle_rope(qr, B, T, Hq, D, pos, theta, bf16);
    oracle_rope(kr, B, T, Hkv, D, pos, theta, bf16);
  }
  int nt = set_threads(nthreads);
  int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nt) reduction(| : err)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < Hq; ++h) {
      const int64_t hk = h / G;
      int64_t cap = W < T ? W : T;
      double *s = (double *)malloc((size_t)cap * sizeof(double));
      const double **kp = (const double **)malloc((size_t)cap * sizeof(double *));
      const double **vp = (const double **)malloc((size_t)cap * sizeof(double *));
      if (!s || !kp || !vp) { err |= 1; free(s); free(kp); free(vp); continue; }
      for (int64_t t = 0; t < T; ++t) {
        int64_t j0 = t - W + 1 < 0 ? 0 : t - W + 1;
        int64_t nk = 0;
        for (int64_t j = j0; j <= t; ++j, ++nk) {
          kp[nk] = kr + ((b * T + j) * Hkv + hk) * D;
          vp[nk] = v + ((b * T + j) * Hkv + hk) * D;
        }
        attend(qr + ((b * T + t) * Hq + h) * D, kp, vp, nk, D, scale, s,
               o + ((b * T + t) * Hq + h) * D);
      }
      free(s); free(kp); free(vp);
    }
  free(qr);
  free(kr);
  return err ? -1 : 0;
}

/* Multi-head prefill: q,k,v,o [B,T,H,D]; oracle_gqa_prefill with Hkv = H. */
int oracle_prefill(const double *q, const double *k, const double *v, double *o,
                   int64_t B, int64_t T, int64_t H, int64_t D, int64_t W,
                   const int64_t *pos, double theta, double scale, int bf16,
                   int rope_applied, int nthreads) {
  return oracle_gqa_prefill(q, k, v, o, B, T, H, H, D, W, pos, theta, scale, bf16,
                            rope_applied, nthreads);
}

/* One streaming step for S streams with n new frames each, grouped-query form.
 * q_new,o: [S,n,Hq,D]; k_new,v_new: [S,n,Hkv,D].  ring_k (rotated keys),
 * ring_v: [S,Hkv,W,D]; slot j of a ring holds the frame at position p with
 * p mod W == j.  pos[S]: absolute position of the first new frame (= frames
 * seen so far).  New query i (position P+i) of query head h attends, on
 * key/value head h / (Hq/Hkv), to ring frames at positions max(0, P+i-W+1)
 * .. P-1 and to new frames P .. P+i.  Reads the rings only.  With n = 1 this
 * is one decode step of the text decoder.  Requires 1 <= n <= W and
 * Hq % Hkv == 0.  Returns 0 or -1. */
int oracle_gqa_stream_step(const double *q_new, const double *k_new, const double *v_new,
                           const double *ring_k, const double *ring_v, const int64_t *pos,
                           double *o, int64_t S, int64_t n, int64_t Hq, int64_t Hkv, int64_t D,
                           int64_t W, double theta, double scale, int bf16, int rope_applied,
                           int nthreads) {
  if (S < 0 || n < 1 || n > W || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 2 || (D & 1) || W < 1)
    return -1;
  if (S == 0) return 0;
  const int64_t G = Hq / Hkv;
  size_t cq = (size_t)(S * n * Hq * D), ck = (size_t)(S * n * Hkv * D);
  double *qr = (double *)malloc(cq * sizeof(double));
  double *kr = (double *)malloc(ck * sizeof(double));
  int64_t *p = (int64_t *)malloc((size_t)(S * n) * sizeof(int64_t));
  if (!qr || !kr || !p) { free(qr); free(kr); free(p); return -1; }
  memcpy(qr, q_new, cq * sizeof(double));
  memcpy(kr, k_new, ck * sizeof(double));
  for (int64_t s = 0; s < S; ++s)
    for (int64_t i = 0; i < n; ++i) p[s * n + i] = pos[s] + i;
  if (!rope_applied) {
    oracle_rope(qr, S, n, Hq, D, p, theta, bf16);
    oracle_rope(kr, S, n, Hkv, D, p, theta, bf16);
  }
  int nt = set_threads(nthreads);
  int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nt) reduction(| : err)
  for (int64_t s = 0; s < S; ++s)
    for (int64_t h = 0; h < Hq; ++h) {
      const int64_t kvh = h / G;
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
          kp[nk] = ring_k + ((s * Hkv + kvh) * W + slot) * D;
          vp[nk] = ring_v + ((s * Hkv + kvh) * W + slot) * D;
        }
        /* new frames P .. P+i: all inside the window because n <= W */
        for (int64_t jj = 0; jj <= i; ++jj, ++nk) {
          kp[nk] = kr + ((s * n + jj) * Hkv + kvh) * D;
          vp[nk] = v_new + ((s * n + jj) * Hkv + kvh) * D;
        }
        attend(qr + ((s * n + i) * Hq + h) * D, kp, vp, nk, D, scale, sc,
               o + ((s * n + i) * Hq + h) * D);
      }
      free(sc); free(kp); free(vp);
    }
  free(qr); free(kr); free(p);
  return err ? -1 : 0;
}

/* Multi-head streaming step: all tensors with H heads; oracle_gqa_stream_step
 * with Hkv = H. */
int oracle_stream_step(const double *q_new, const double *k_new, const double *v_new,
                       const double *ring_k, const double *ring_v, const int64_t *pos,
                       double *o, int64_t S, int64_t n, int64_t H, int64_t D, int64_t W,
                       double theta, double scale, int bf16, int rope_applied, int nthreads) {
  return oracle_gqa_stream_step(q_new, k_new, v_new, ring_k, ring_v, pos, o, S, n, H, H, D, W,
                                theta, scale, bf16, rope_applied, nthreads);
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
