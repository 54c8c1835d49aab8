/*
 * gdn_oracle.c -- fp64 CPU oracle for the gated delta rule and the GDN mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header, table or helper with the HIP path.
 *
 * What it computes (the plain definition, token by token, in fp64):
 *
 *   Gated delta rule -- the recurrent linear-attention computation of the
 *   Gated DeltaNet layers ("open-jev-fast" README, "Phase 3" item 1, which
 *   cites Yang, Kautz & Hatamizadeh, "Gated Delta Networks", ICLR 2025; the
 *   System1-Omni PR #186 page, "Purpose and summary", calls it the model's
 *   recurrent linear-attention computation):
 *
 *       S_t = exp(g_t) * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *       o_t = S_t q_t
 *
 *   S_t is dv x dk.  The decay is applied first, then the delta correction
 *   acts on the decayed state:  S <- e^g S;  S <- S + beta (v - S k) k^T.
 *   This is the same expression multiplied out.
 *
 *   Packed variable-length batches: sequence n owns tokens
 *   [cu[n], cu[n+1]) and has its own initial state h0[n] (prefix
 *   continuation, "open-jev-fast" README, "Phase 2" item 2; PR #186,
 *   "Review scope and map", per-candidate state).  h0 / hT are stored
 *   key-major, H = S^T with shape [dk][dv].  A NULL h0 means a zero state.
 *
 *   Grouped value heads: v-head h reads q/k head h / (Hv/Hk)
 *   ("open-jev-fast" README, "Phase 3" item 3: q/k at 16 heads).
 *
 *   Mixer ("open-jev-fast" README, "Phase 2" item 1: GDN input prep and the
 *   gated RMSNorm):
 *       c[t,ch] = sum_{j=0..3} w[ch,j] x[t-3+j,ch]   (zero before a sequence start)
 *       a = c * sigmoid(c)
 *       q,k per head:  x / sqrt(sum x^2 + eps_l2)
 *       o = gated delta rule(q, k, v, g, beta)
 *       y = o / sqrt(mean(o^2) + eps_norm) * w_norm * z * sigmoid(z)
 *
 *   Gate parameters (the last step the "open-jev-fast" README, "Phase 2" item 1, lists for the
 *   GDN input prep; the pages give no formula, so this follows the gating of the Gated DeltaNet
 *   paper the README cites, a Mamba2-style decay): per token t and v-head h, from the layer's
 *   projections a, b and the per-head parameters A_log, dt_bias,
 *       g    = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])     (log-decay, <= 0)
 *       beta = sigmoid(b[t,h])
 *
 *   The model is bf16 and its fused prep / norm kernels keep the reference's bf16 rounding
 *   points ("open-jev-fast" README, "Phase 2" item 1).  With bf16_points != 0 the mixer rounds
 *   the prepped q, k, v and the rule's output o to bf16 (round to nearest, ties to even) at
 *   exactly those points; every other value stays fp64.
 *
 * Precision: every value is fp64; inputs arrive already upcast to fp64.
 * Threads: OpenMP over independent (sequence, v-head) pairs only; the
 * arithmetic inside a pair is in token order, so results do not depend on
 * the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* One (sequence, v-head) pair: the token recurrence written out. */
static void recur_one(int64_t t_begin, int64_t t_end, int32_t Hk, int32_t Hv, int32_t dk,
                      int32_t dv, int32_t h, const double *q, const double *k,
                      const double *v, const double *g, const double *beta,
                      const double *h0_nh, /* [dk][dv] or NULL */
                      double *o, double *hT_nh /* [dk][dv] or NULL */, double *S,
                      double *u) {
  const int32_t group = Hv / Hk;
  const int32_t hk = h / group;
  /* S is dv x dk; h0 is stored key-major (H = S^T). */
  for (int32_t i = 0; i < dv; ++i)
    for (int32_t j = 0; j < dk; ++j)
      S[(int64_t)i * dk + j] = h0_nh ? h0_nh[(int64_t)j * dv + i] : 0.0;

  for (int64_t t = t_begin; t < t_end; ++t) {
    const double *kt = k + (t * Hk + hk) * dk;
    const double *qt = q + (t * Hk + hk) * dk;
    const double *vt = v + (t * Hv + h) * dv;
    const double gt = g[t * Hv + h];
    const double bt = beta[t * Hv + h];
    const double decay = exp(gt);
    /* S <- exp(g_t) S */
    for (int64_t e = 0; e < (int64_t)dv * dk; ++e) S[e] *= decay;
    /* u = beta_t (v_t - S k_t) */
    for (int32_t i = 0; i < dv; ++i) {
      double sk = 0.0;
      for (int32_t j = 0; j < dk; ++j) sk += S[(int64_t)i * dk + j] * kt[j];
      u[i] = bt * (vt[i] - sk);
    }
    /* S <- S + u k_t^T */
    for (int32_t i = 0; i < dv; ++i)
      for (int32_t j = 0; j < dk; ++j) S[(int64_t)i * dk + j] += u[i] * kt[j];
    /* o_t = S q_t */
    double *ot = o + (t * Hv + h) * dv;
    for (int32_t i = 0; i < dv; ++i) {
      double acc = 0.0;
      for (int32_t j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * qt[j];
      ot[i] = acc;
    }
  }
  if (hT_nh)
    for (int32_t i = 0; i < dv; ++i)
      for (int32_t j = 0; j < dk; ++j) hT_nh[(int64_t)j * dv + i] = S[(int64_t)i * dk + j];
}

/*
 * Gated delta rule over a packed batch, with the initial states drawn from a pool by index.
 *   q, k  : [T, Hk, dk]     v : [T, Hv, dv]     g, beta : [T, Hv]
 *   cu    : [N+1], cu[0] = 0, non-decreasing, cu[N] = T
 *   h0    : [num_h0, Hv, dk, dv] or NULL (zero states)
 *   h0_index : [N] or NULL.  Sequence n starts from h0[h0_index[n]] when that index lies in
 *           [0, num_h0), and from a zero state otherwise.  NULL means sequence n starts from
 *           h0[n] (then num_h0 must be N).  One prefix's final state handed to several
 *           candidates is this with repeated indices ("open-jev-fast" README, "Phase 2" item 2;
 *           PR #186, "Review scope and map").
 *   hT    : [N, Hv, dk, dv] or NULL;  o : [T, Hv, dv]
 * Returns 0, or -1 on bad arguments.
 */
int oracle_gdn_fwd_indexed(int64_t T, int32_t N, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv,
                           const double *q, const double *k, const double *v, const double *g,
                           const double *beta, const int64_t *cu, const double *h0,
                           int32_t num_h0, const int64_t *h0_index, double *o, double *hT,
                           int32_t nthreads) {
  if (N < 1 || Hk < 1 || Hv < 1 || Hv % Hk != 0 || dk < 1 || dv < 1 || T < 0) return -1;
  if (cu[0] != 0 || cu[N] != T) return -1;
  if (!h0_index && h0 && num_h0 != N) return -1;
  for (int32_t n = 0; n < N; ++n)
    if (cu[n + 1] < cu[n]) return -1;
  const int64_t pairs = (int64_t)N * Hv;
  const int64_t state = (int64_t)dk * dv;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double *S = (double *)malloc(sizeof(double) * state);
    double *u = (double *)malloc(sizeof(double) * dv);
    if (!S || !u) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      bad = 1;
    } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
      for (int64_t p = 0; p < pairs; ++p) {
        const int32_t n = (int32_t)(p / Hv), h = (int32_t)(p % Hv);
        const int64_t r = h0_index ? h0_index[n] : n;
        const double *h0_nh = (h0 && r >= 0 && r < num_h0) ? h0 + (r * Hv + h) * state : NULL;
        double *hT_nh = hT ? hT + ((int64_t)n * Hv + h) * state : NULL;
        recur_one(cu[n], cu[n + 1], Hk, Hv, dk, dv, h, q, k, v, g, beta, h0_nh, o, hT_nh, S,
                  u);
      }
    }
    free(S);
    free(u);
  }
  (void)nthreads;
  return bad ? -2 : 0;
}

/* The same with h0 : [N, Hv, dk, dv] or NULL, sequence n starting from h0[n]. */
int oracle_gdn_fwd(int64_t T, int32_t N, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv,
                   const double *q, const double *k, const double *v, const double *g,
                   const double *beta, const int64_t *cu, const double *h0, double *o,
                   double *hT, int32_t nthreads) {
  return oracle_gdn_fwd_indexed(T, N, Hk, Hv, dk, dv, q, k, v, g, beta, cu, h0, N, NULL, o, hT,
                                nthreads);
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Round to the nearest value with 8 significant bits (bf16), ties to even.  Finite inputs in
 * bf16's normal range (|x| >= 2^-126); zero stays zero. */
double oracle_round_bf16(double x) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  const double m = frexp(x, &e);           /* x = m 2^e, 0.5 <= |m| < 1 */
  const double scaled = ldexp(m, 8);       /* 8 significant bits above the binary point */
  double r = floor(scaled);
  const double diff = scaled - r;
  if (diff > 0.5 || (diff == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  return ldexp(r, e - 8);
}

void oracle_round_bf16_array(const double *x, double *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_round_bf16(x[i]);
}

/*
 * Causal depthwise conv1d + SiLU over a packed batch (the first part of the GDN input prep),
 * with a carried input window per sequence.
 *   x : [T, C];  w : [C, taps], tap taps-1 multiplies the current token.
 *   win_in : [num_states, taps-1, C] or NULL -- the last taps-1 conv inputs before a sequence
 *            start, oldest first.  Sequence n reads window win_in[state_index[n]] when that index
 *            lies in [0, num_states), else a window of zeros; a NULL state_index means window n
 *            (then num_states must be N).  A NULL win_in means zeros before every sequence start.
 *   out : [T, C].
 *   win_out : [N, taps-1, C] or NULL -- the last taps-1 inputs of sequence n's stream (its
 *            window followed by its tokens), oldest first: the window the next call continues
 *            from.  (The prefix handing its conv window and recurrent state on to a candidate:
 *            "open-jev-fast" README, "Phase 2" item 2.)
 * The window never reaches across a sequence start into another sequence's tokens.
 */
int oracle_conv_silu_cont(int64_t T, int32_t N, int32_t C, int32_t taps, const double *x,
                          const double *w, const int64_t *cu, const double *win_in,
                          int32_t num_states, const int64_t *state_index, double *out,
                          double *win_out, int32_t nthreads) {
  if (cu[0] != 0 || cu[N] != T || taps < 1) return -1;
  if (!state_index && win_in && num_states != N) return -1;
  const int64_t wrows = (int64_t)(taps - 1) * C;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
  for (int32_t ch = 0; ch < C; ++ch) {
    for (int32_t n = 0; n < N; ++n) {
      const int64_t r = state_index ? state_index[n] : n;
      const double *win = (win_in && r >= 0 && r < num_states) ? win_in + r * wrows : NULL;
      for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
        double c = 0.0;
        for (int32_t j = 0; j < taps; ++j) {
          const int64_t src = t - (taps - 1) + j;
          if (src >= cu[n]) c += w[(int64_t)ch * taps + j] * x[src * C + ch];
          else if (win) c += w[(int64_t)ch * taps + j] * win[(src - cu[n] + taps - 1) * C + ch];
        }
        out[t * C + ch] = c * sigmoid(c);
      }
      if (win_out)
        for (int32_t j = 0; j < taps - 1; ++j) {
          const int64_t p = cu[n + 1] - (taps - 1) + j;  /* stream position, >= cu[n] - (taps-1) */
          double val = 0.0;
          if (p >= cu[n]) val = x[p * C + ch];
          else if (win) val = win[(p - cu[n] + taps - 1) * C + ch];
          win_out[(int64_t)n * wrows + (int64_t)j * C + ch] = val;
        }
    }
  }
  (void)nthreads;
  return 0;
}

/* The same with zeros before every sequence start and no window out. */
int oracle_conv_silu(int64_t T, int32_t N, int32_t C, int32_t taps, const double *x,
                     const double *w, const int64_t *cu, double *out, int32_t nthreads) {
  return oracle_conv_silu_cont(T, N, C, taps, x, w, cu, NULL, N, NULL, out, NULL, nthreads);
}

/*
 * Full mixer: conv+SiLU on all 2*Hk*dk + Hv*dv channels (q | k | v, head-major
 * inside each), L2 norm of q and k per head, the gated delta rule, then the
 * SiLU(z)-gated RMSNorm per (token, v-head) with a weight shared by all heads.
 *   qkv [T, 2*Hk*dk + Hv*dv], conv_w [2*Hk*dk + Hv*dv, taps], g/beta [T, Hv],
 *   z [T, Hv, dv], norm_w [dv]
 *   h0 [num_states, Hv, dk, dv] or NULL, conv_in [num_states, taps-1, 2*Hk*dk + Hv*dv] or NULL,
 *   state_index [N] or NULL: sequence n continues from recurrent state and conv window
 *   state_index[n] (zeros when that index is outside [0, num_states)); NULL means state n.
 *   -> y [T, Hv, dv], hT [N, Hv, dk, dv] or NULL, conv_out [N, taps-1, C] or NULL.
 * Intermediates (q, k, v after prep; o) are fp64 throughout.
 */
int oracle_mixer_fwd_cont(int64_t T, int32_t N, int32_t Hk, int32_t Hv, int32_t dk,
                          int32_t dv, int32_t taps, double eps_l2, double eps_norm,
                          int32_t bf16_points, const double *qkv, const double *conv_w,
                          const double *g, const double *beta, const double *z,
                          const double *norm_w, const int64_t *cu, const double *h0,
                          const double *conv_in, int32_t num_states,
                          const int64_t *state_index, double *y, double *hT, double *conv_out,
                          int32_t nthreads) {
  const int32_t Cq = Hk * dk, Cv = Hv * dv, C = 2 * Cq + Cv;
  const int64_t Tn = T > 0 ? T : 1;
  double *a = (double *)malloc(sizeof(double) * Tn * C);
  double *q = (double *)malloc(sizeof(double) * Tn * Cq);
  double *k = (double *)malloc(sizeof(double) * Tn * Cq);
  double *v = (double *)malloc(sizeof(double) * Tn * Cv);
  double *o = (double *)malloc(sizeof(double) * Tn * Cv);
  int rc = -2;
  if (!a || !q || !k || !v || !o) goto done;
  rc = oracle_conv_silu_cont(T, N, C, taps, qkv, conv_w, cu, conv_in, num_states, state_index, a,
                             conv_out, nthreads);
  if (rc) goto done;
  for (int64_t t = 0; t < T; ++t) {
    const double *row = a + t * C;
    for (int32_t hh = 0; hh < Hk; ++hh) {
      const double *qs = row + (int64_t)hh * dk;
      const double *ks = row + Cq + (int64_t)hh * dk;
      double sq = 0.0, sk = 0.0;
      for (int32_t j = 0; j < dk; ++j) {
        sq += qs[j] * qs[j];
        sk += ks[j] * ks[j];
      }
      const double rq = 1.0 / sqrt(sq + eps_l2), rk = 1.0 / sqrt(sk + eps_l2);
      for (int32_t j = 0; j < dk; ++j) {
        q[(t * Hk + hh) * dk + j] = qs[j] * rq;
        k[(t * Hk + hh) * dk + j] = ks[j] * rk;
      }
    }
    memcpy(v + t * Cv, row + 2 * Cq, sizeof(double) * Cv);
  }
  if (bf16_points) {
    for (int64_t e = 0; e < T * Cq; ++e) {
      q[e] = oracle_round_bf16(q[e]);
      k[e] = oracle_round_bf16(k[e]);
    }
    for (int64_t e = 0; e < T * Cv; ++e) v[e] = oracle_round_bf16(v[e]);
  }
  rc = oracle_gdn_fwd_indexed(T, N, Hk, Hv, dk, dv, q, k, v, g, beta, cu, h0, num_states,
                              state_index, o, hT, nthreads);
  if (rc) goto done;
  if (bf16_points)
    for (int64_t e = 0; e < T * Cv; ++e) o[e] = oracle_round_bf16(o[e]);
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t h = 0; h < Hv; ++h) {
      const double *os = o + (t * Hv + h) * dv;
      const double *zs = z + (t * Hv + h) * dv;
      double ms = 0.0;
      for (int32_t j = 0; j < dv; ++j) ms += os[j] * os[j];
      const double r = 1.0 / sqrt(ms / dv + eps_norm);
      for (int32_t j = 0; j < dv; ++j)
        y[(t * Hv + h) * dv + j] = os[j] * r * norm_w[j] * zs[j] * sigmoid(zs[j]);
    }
  }
done:
  free(a);
  free(q);
  free(k);
  free(v);
  free(o);
  return rc;
}

/* The mixer with zero conv history and h0[n] (or zeros) for sequence n, no window out. */
int oracle_mixer_fwd(int64_t T, int32_t N, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv,
                     int32_t taps, double eps_l2, double eps_norm, int32_t bf16_points,
                     const double *qkv, const double *conv_w, const double *g,
                     const double *beta, const double *z, const double *norm_w,
                     const int64_t *cu, const double *h0, double *y, double *hT,
                     int32_t nthreads) {
  return oracle_mixer_fwd_cont(T, N, Hk, Hv, dk, dv, taps, eps_l2, eps_norm, bf16_points, qkv,
                               conv_w, g, beta, z, norm_w, cu, h0, NULL, N, NULL, y, hT, NULL,
                               nthreads);
}

/* softplus(x) = log(1 + e^x), without overflow for large x. */
static double softplus(double x) { return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x)); }

/* Gate parameters of a packed batch (see the header):  a, b : [T, Hv];  A_log, dt_bias : [Hv];
 * g, beta : [T, Hv] out. */
void oracle_gates(int64_t T, int32_t Hv, const double *a, const double *b, const double *A_log,
                  const double *dt_bias, double *g, double *beta) {
  for (int64_t t = 0; t < T; ++t)
    for (int32_t h = 0; h < Hv; ++h) {
      const int64_t i = t * Hv + h;
      g[i] = -exp(A_log[h]) * softplus(a[i] + dt_bias[h]);
      beta[i] = sigmoid(b[i]);
    }
}
