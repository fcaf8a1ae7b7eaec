/*
 * gdr_oracle.c -- plain fp64 CPU oracle of the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the yardstick the HIP library is
 * measured against; it is not part of the product.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * source, header, table or helper with the HIP library.
 *
 * What it computes, and where each step is defined:
 *
 *   - The fused decode step for one token: split of the packed row into
 *     q, k and v, normalisation of q and k, head repeat, the gates, and the
 *     state update
 *       [page "Add fused GatedDeltaNet decode Triton kernel" (executorch
 *        PR #18865), PR summary].
 *   - The per-token state update: decay, predicted value from the decayed
 *     state, rank-one correction, and the output read from the updated state
 *       [page "Two-pass optimization for channelwise gated delta rule kernel"
 *        (executorch PR #21020), Summary: the pass structure names these
 *        steps; the two-pass grouping is an exact regrouping of the plain
 *        four-traversal form written out below].
 *   - Channelwise decay (one log-decay per key channel) and the scalar
 *     GatedDeltaNet decay (one per token and head)
 *       [page "Add parallel chunked prefill for channelwise gated delta rule"
 *        (executorch PR #21061), Summary; and page PR #18865, summary].
 *
 * The oracle is the token recurrence only.  The chunkwise WY/UT form of
 * PR #21061 is an exact reorganisation of it and is NOT implemented here.
 *
 * Readings taken where the pages are silent (the pages print no formula):
 *   - decay a = exp(g) with g <= 0 the log-decay; S_t = diag(a) S_{t-1} + ...
 *   - prediction from the decayed state, output from the updated state,
 *     o = scale * S_t^T q;
 *   - L2 normalisation x / sqrt(sum x^2 + 1e-6);
 *   - head repeat is repeat-interleave: value head h uses query/key head
 *     h / (H_v / H_qk);
 *   - packed decode row is [q heads | k heads | v heads], each head-major;
 *   - beta = 1 / (1 + exp(-beta_logit));
 *   - fused scalar gate g = -exp(A_log[h]) * softplus(x + dt_bias[h]) with
 *     softplus(z) = log(1 + exp(z)).
 *
 * Layouts (row-major, last index fastest):
 *   sequence form: q, k [B,T,H_qk,dk]; v [B,T,H_v,dv]; beta_logit [B,T,H_v];
 *                  gate channel g [B,T,H_v,dk] | scalar g [B,T,H_v] |
 *                  fused x [B,T,H_v] with A_log, dt_bias [H_v];
 *                  o [B,T,H_v,dv]
 *   decode form:   qkv [B, 2*H_qk*dk + H_v*dv]; beta_logit [B,H_v];
 *                  gate channel g [B,H_v,dk] | scalar g [B,H_v] | fused x [B,H_v];
 *                  o [B,H_v,dv]
 *   state:         S [B,H_v,dk,dv], updated in place.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -fopenmp (no -ffast-math).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_GATE_CHANNEL = 0, ORC_GATE_SCALAR = 1, ORC_GATE_SCALAR_FUSED = 2 };

#define ORC_L2_EPS 1e-6

double orc_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* softplus(z) = log(1 + e^z), evaluated without overflow for large z. */
double orc_softplus(double z) { return z > 0.0 ? z + log1p(exp(-z)) : log1p(exp(z)); }

/* out = x / sqrt(sum_i x_i^2 + eps). */
void orc_l2norm(const double* x, int n, double* out) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss + ORC_L2_EPS);
  for (int i = 0; i < n; ++i) out[i] = x[i] * inv;
}

/* Log-decay of one (token, head): fills g_out[0..dk).
 * gate_ch points at this token/head's dk channel values (channel kind),
 * gate_sc at its single value (scalar kinds). */
static void orc_log_decay(int kind, int dk, const double* gate_ch, double gate_sc,
                          double A_log_h, double dt_bias_h, double* g_out) {
  if (kind == ORC_GATE_CHANNEL) {
    for (int i = 0; i < dk; ++i) g_out[i] = gate_ch[i];
  } else if (kind == ORC_GATE_SCALAR) {
    for (int i = 0; i < dk; ++i) g_out[i] = gate_sc;
  } else {
    double g = -exp(A_log_h) * orc_softplus(gate_sc + dt_bias_h);
    for (int i = 0; i < dk; ++i) g_out[i] = g;
  }
}

/* One token of the delta rule for one (batch, value head), written out as
 * its plain definition, one traversal of S per step:
 *   1. decay:     S <- diag(a) S,            a = exp(g)
 *   2. predict:   vhat = S^T k               (from the decayed state)
 *   3. write:     S <- S + beta k (v - vhat)^T
 *   4. read:      o = scale * S^T q          (from the updated state)
 * S is dk x dv, row-major.  vhat is caller scratch of length dv. */
static void orc_token(int dk, int dv, const double* q, const double* k, const double* v,
                      const double* g, double beta, double scale, double* S, double* vhat,
                      double* o) {
  for (int i = 0; i < dk; ++i) {
    double a = exp(g[i]);
    for (int j = 0; j < dv; ++j) S[i * dv + j] *= a;
  }
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * k[i];
    vhat[j] = acc;
  }
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[i * dv + j] += beta * k[i] * (v[j] - vhat[j]);
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * q[i];
    o[j] = scale * acc;
  }
}

static int orc_bad_dims(int B, int T, int Hqk, int Hv, int dk, int dv) {
  return B < 0 || T < 0 || Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0 || Hv % Hqk != 0;
}

/* Token recurrence over a whole sequence (sequence layout, see header).
 * Returns 0, or -1 on bad dimensions / missing pointers. */
int gdr_oracle_sequence(int B, int T, int Hqk, int Hv, int dk, int dv, const double* q,
                        const double* k, const double* v, int gate_kind, const double* gate_in,
                        const double* A_log, const double* dt_bias, const double* beta_logit,
                        double* state, double* o, double scale, int l2norm, int threads) {
  if (orc_bad_dims(B, T, Hqk, Hv, dk, dv)) return -1;
  if (gate_kind < 0 || gate_kind > 2) return -1;
  if (gate_kind == ORC_GATE_SCALAR_FUSED && (!A_log || !dt_bias)) return -1;
  if (B * T > 0 && (!q || !k || !v || !gate_in || !beta_logit || !o)) return -1;
  if (B > 0 && !state) return -1;
  const int rep = Hv / Hqk;
  if (threads < 1) threads = 1;
  int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(threads) reduction(| : bad)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < Hv; ++h) {
      double* buf = (double*)malloc(sizeof(double) * (size_t)(2 * dk + dk + dv));
      if (!buf) { bad = 1; continue; }
      double* qn = buf;
      double* kn = buf + dk;
      double* g = buf + 2 * dk;
      double* vhat = buf + 3 * dk;
      const int hq = h / rep; /* head repeat: repeat-interleave */
      double* S = state + ((size_t)b * Hv + h) * (size_t)dk * dv;
      for (int t = 0; t < T; ++t) {
        const size_t bt = (size_t)b * T + t;
        const double* qt = q + (bt * Hqk + hq) * dk;
        const double* kt = k + (bt * Hqk + hq) * dk;
        const double* vt = v + (bt * Hv + h) * dv;
        if (l2norm) {
          orc_l2norm(qt, dk, qn);
          orc_l2norm(kt, dk, kn);
        } else {
          memcpy(qn, qt, sizeof(double) * dk);
          memcpy(kn, kt, sizeof(double) * dk);
        }
        const size_t gh = bt * Hv + h;
        orc_log_decay(gate_kind, dk, gate_kind == ORC_GATE_CHANNEL ? gate_in + gh * dk : NULL,
                      gate_kind == ORC_GATE_CHANNEL ? 0.0 : gate_in[gh],
                      A_log ? A_log[h] : 0.0, dt_bias ? dt_bias[h] : 0.0, g);
        double beta = orc_sigmoid(beta_logit[gh]);
        orc_token(dk, dv, qn, kn, vt, g, beta, scale, S, vhat, o + gh * dv);
      }
      free(buf);
    }
  }
  return bad ? -1 : 0;
}

/* One decode token from the packed q|k|v row (decode layout, see header). */
int gdr_oracle_decode(int B, int Hqk, int Hv, int dk, int dv, const double* qkv, int gate_kind,
                      const double* gate_in, const double* A_log, const double* dt_bias,
                      const double* beta_logit, double* state, double* o, double scale,
                      int l2norm, int threads) {
  if (orc_bad_dims(B, 1, Hqk, Hv, dk, dv)) return -1;
  if (gate_kind < 0 || gate_kind > 2) return -1;
  if (gate_kind == ORC_GATE_SCALAR_FUSED && (!A_log || !dt_bias)) return -1;
  if (B > 0 && (!qkv || !gate_in || !beta_logit || !state || !o)) return -1;
  const int rep = Hv / Hqk;
  const size_t row = (size_t)2 * Hqk * dk + (size_t)Hv * dv;
  if (threads < 1) threads = 1;
  int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(threads) reduction(| : bad)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < Hv; ++h) {
      double* buf = (double*)malloc(sizeof(double) * (size_t)(3 * dk + dv));
      if (!buf) { bad = 1; continue; }
      double* qn = buf;
      double* kn = buf + dk;
      double* g = buf + 2 * dk;
      double* vhat = buf + 3 * dk;
      const int hq = h / rep;
      /* Q/K/V split of the packed row. */
      const double* qt = qkv + b * row + (size_t)hq * dk;
      const double* kt = qkv + b * row + (size_t)Hqk * dk + (size_t)hq * dk;
      const double* vt = qkv + b * row + (size_t)2 * Hqk * dk + (size_t)h * dv;
      if (l2norm) {
        orc_l2norm(qt, dk, qn);
        orc_l2norm(kt, dk, kn);
      } else {
        memcpy(qn, qt, sizeof(double) * dk);
        memcpy(kn, kt, sizeof(double) * dk);
      }
      const size_t gh = (size_t)b * Hv + h;
      orc_log_decay(gate_kind, dk, gate_kind == ORC_GATE_CHANNEL ? gate_in + gh * dk : NULL,
                    gate_kind == ORC_GATE_CHANNEL ? 0.0 : gate_in[gh], A_log ? A_log[h] : 0.0,
                    dt_bias ? dt_bias[h] : 0.0, g);
      double beta = orc_sigmoid(beta_logit[gh]);
      double* S = state + gh * (size_t)dk * dv;
      orc_token(dk, dv, qn, kn, vt, g, beta, scale, S, vhat, o + gh * dv);
      free(buf);
    }
  }
  return bad ? -1 : 0;
}

/* Threads OpenMP would actually use for a request of `threads`. */
int gdr_oracle_threads(int threads) {
#ifdef _OPENMP
  int n = 1;
  if (threads < 1) threads = 1;
#pragma omp parallel num_threads(threads)
  {
#pragma omp single
    n = omp_get_num_threads();
  }
  return n;
#else
  (void)threads;
  return 1;
#endif
}
