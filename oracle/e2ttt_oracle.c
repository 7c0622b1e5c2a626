/*
 * e2ttt_oracle.c -- fp64 CPU oracle for the E2-TTT chunk forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * HIP library is checked against.  It shares no code, header, table or helper
 * with the GPU path and must never be linked into it; only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg load it.
 *
 * What it computes, and where the pages fix it
 * (all citations are to "Rethinking Expressivity and Efficiency in Test-Time
 *  Training", E2-TTT, as served by paperpeel.com, unless noted):
 *
 *   - The state is the fast weight W and a momentum buffer M of the same shape
 *     (§2: for a learner with several weight tensors the state symbol stands
 *     for all of them).
 *   - Within chunk r all per-token gradients are evaluated at the chunk-start
 *     weights W_0 (§1, §3; App. A.5 takes every gradient of a chunk at the frozen
 *     chunk-start weights).
 *   - The token-wise state recurrence (Eq. 7, in the optimisation-style reading of
 *     App. A.5: momentum factor beta_t, L2 decay factor gamma_t) is taken as
 *         M_t = beta_t * M_{t-1} + eta_t * G_t
 *         W_t = gamma_t * W_{t-1} + M_t
 *     with G_t the descent direction -grad_W l_t(W_0).  The display equation is
 *     missing from the page; this is the reading whose closed form yields the
 *     two kernels named in §3.2 (K^M = eta*beta~, K^W = eta*beta~*R).
 *   - gamma_t = 1 - eta_t * alpha_t (Eq. 14, App. A.3 "Coupled
 *     parameterization"); an alternative mode takes alpha_t as gamma_t itself.
 *   - The inner loss is the key-value regression 0.5*||f_W(k_t) - v_t||^2
 *     summed over the d outputs (§2).
 *   - Output: o_t = f_{W_0}(q_t), the chunk-start weights (Eq. 6, §3.2).
 *   - (W_C, M_C) of chunk r is (W_0, M_0) of chunk r+1 (§3 notation, §3.2
 *     where equivalence across chunks follows by induction).
 *   - Inner learners: linear f_W(x) = W x (§2), the three-matrix SwiGLU
 *     f(x) = W2 (silu(W1 x) * (W3 x)) (§5.2, App. B.5 "three-matrix
 *     fast-weight network"), and the MLP learner of E2-TTT_MLP (§5, App.
 *     B.3 Table 11, App. B.5: a smaller fast-weight network than the
 *     SwiGLU's; its activation is not named on the page).  Reading taken:
 *     the two-matrix f(x) = W2 silu(W1 x), the SwiGLU without its gate
 *     branch, state packed [W1 (h x d) | W2 (d x h)].
 *   - Option (qk_norm != 0): the TTT branch's input prologue of §4 ("Overall
 *     Architecture"): SiLU applied to q_t and k_t, then L2 normalisation of
 *     each token's vector, before anything else uses them.  The pages give no
 *     epsilon; this divides by max(||x||, 1e-12).  With qk_norm == 2 every
 *     normalised value is then rounded to bf16 (to nearest, ties to even,
 *     through fp32), the precision a bf16 layer stores its q and k in: read
 *     as the unfused form of the prologue, whose outputs the chunk update
 *     consumes as its bf16 inputs, like the layer's own q and k.
 *   - Variant (averaged != 0): the chunk-averaged ablation of §5.4 (Table 5)
 *     and App. B.3 (Table 8), where the per-token momentum and decay factors
 *     beta_t, gamma_t of a chunk are collapsed to chunk-level scalars.  The
 *     pages do not say which average; this takes the arithmetic mean over the
 *     chunk's tokens (of gamma_t, after Eq. 14), and otherwise the same
 *     recurrence.
 *
 *   - Variant (averaged == 2): the LaCT update rule as §3.2 ("Two scalar
 *     kernels with distinct temporal weighting") sets it against E2-TTT
 *     (Eq. 5, whose display is missing from the page): the gradient term
 *     carries only eta_t, with neither the momentum suffix product nor the
 *     weight-decay ratio sum, and the momentum factor is collapsed to a chunk
 *     average; §1 describes LaCT as one fast-weight update per chunk from the
 *     gradient of a summed loss.  Reading taken: per chunk, with bbar and
 *     gbar the means of beta_t and gamma_t (after Eq. 14) over the chunk's
 *     tokens,
 *         M_C = bbar * M_0 + sum_t eta_t G_t
 *         W_C = gbar * W_0 + M_C
 *     i.e. the recurrence's step taken once, on the eta-weighted sum of the
 *     chunk's descent directions (all evaluated at W_0); readout as above.
 *
 *   - Scalar heads (oracle_scalar_heads): §4 ("Overall Architecture",
 *     "Input-Dependent Dynamics") predicts eta_t, beta_t and alpha_t from the
 *     layer input x_t by lightweight linear heads (Eqs. 12-14, App. B.4), and
 *     App. B.3 says eta_base and alpha_base scale per-token sigmoid gates.
 *     Eq. 13 (the timescale form of beta that App. A.3 mentions) is missing from
 *     the page; the reading taken is a plain sigmoid gate.  Per TTT head h:
 *         eta_t   = eta_base   * sigma(<w_eta_h,   x_t> + b_eta_h)
 *         alpha_t = alpha_base * sigma(<w_alpha_h, x_t> + b_alpha_h)
 *         beta_t  =              sigma(<w_beta_h,  x_t> + b_beta_h)
 *     and gamma_t = 1 - eta_t alpha_t (Eq. 14) downstream.
 *
 *   - Option (row_norm != 0): the stabiliser of App. B.1 ("Training
 *     Details"), L2 normalisation of the fast-weight matrices at each chunk
 *     boundary, following LaCT.  The pages name neither the axis nor an
 *     epsilon; this divides every row of every fast-weight matrix (linear W;
 *     SwiGLU W1, W3 and W2, rows as stored, i.e. one row per output unit) by
 *     max(||row||_2, 1e-12) after each chunk's update, the last chunk
 *     included.  M is left as it is.
 *
 * The recurrence is run literally, token by token, on every state entry.
 * Each entry's recurrence involves only that entry, so the loops are ordered
 * state-row outer, token inner; this performs the identical sequence of fp64
 * operations per entry as a token-outer loop.
 *
 * State packing per (batch, head): linear W is d x d row-major.  SwiGLU is
 * [W1 (h x d) | W3 (h x d) | W2 (d x h)], each row-major.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math, so
 * every operation is an IEEE fp64 operation in program order).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_LINEAR = 0, OR_SWIGLU = 1, OR_MLP = 2 };
enum { OR_GAMMA_1_MINUS_ETA_ALPHA = 0, OR_ALPHA_IS_GAMMA = 1 };

static double sigm(double x) { return 1.0 / (1.0 + exp(-x)); }

/* x rounded to the nearest bf16 value (ties to even) through fp32; inf and
 * NaN pass through. */
static double round_bf16(double x) {
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7f800000u) != 0x7f800000u) {
    u += 0x7fffu + ((u >> 16) & 1u);
    u &= 0xffff0000u;
    memcpy(&f, &u, sizeof f);
  }
  return (double)f;
}

/* x <- silu(x) / max(||silu(x)||_2, 1e-12) for L rows of d (the q/k
 * prologue), each result rounded to bf16 when round16 != 0. */
static void silu_l2_rows(double* x, int64_t L, int64_t d, int round16) {
  for (int64_t t = 0; t < L; ++t) {
    double* r = x + t * d;
    double ss = 0.0;
    for (int64_t i = 0; i < d; ++i) {
      r[i] = r[i] * sigm(r[i]);
      ss += r[i] * r[i];
    }
    double nrm = sqrt(ss);
    if (nrm < 1e-12) nrm = 1e-12;
    for (int64_t i = 0; i < d; ++i) r[i] = round16 ? round_bf16(r[i] / nrm) : r[i] / nrm;
  }
}

/* Reverse mode of silu_l2_rows: g holds, per row, the adjoint of the
 * normalised vector y = s / max(||s||, 1e-12), s = silu(x); it is replaced by
 * the adjoint of the raw x.  With n = ||s|| > 1e-12:
 *   ds = (g - y (y . g)) / n,   dx = ds * silu'(x),  silu'(x) = sigma (1 + x (1 - sigma));
 * below the floor the divisor is the constant 1e-12 and ds = g / 1e-12. */
static void silu_l2_rows_vjp(const double* x, double* g, int64_t L, int64_t d) {
  for (int64_t t = 0; t < L; ++t) {
    const double* xr = x + t * d;
    double* gr = g + t * d;
    double ss = 0.0;
    for (int64_t i = 0; i < d; ++i) {
      const double si = xr[i] * sigm(xr[i]);
      ss += si * si;
    }
    const double n = sqrt(ss);
    const double den = n < 1e-12 ? 1e-12 : n;
    double dot = 0.0;
    if (n >= 1e-12)
      for (int64_t i = 0; i < d; ++i) dot += (xr[i] * sigm(xr[i]) / den) * gr[i];
    for (int64_t i = 0; i < d; ++i) {
      const double sg = sigm(xr[i]);
      const double yi = xr[i] * sg / den;
      const double ds = (gr[i] - (n >= 1e-12 ? yi * dot : 0.0)) / den;
      gr[i] = ds * (sg * (1.0 + xr[i] * (1.0 - sg)));
    }
  }
}

/* gamma_t from the per-token scalars (Eq. 14, or alpha taken as gamma). */
static double decay_factor(int decay_mode, double eta, double alpha) {
  if (decay_mode == OR_ALPHA_IS_GAMMA) return alpha;
  return 1.0 - eta * alpha;
}

static int64_t state_size(int kind, int64_t d, int64_t h) {
  return kind == OR_LINEAR ? d * d : kind == OR_MLP ? 2 * d * h : 3 * d * h;
}

/* Offset of W2 in a unit's packed state (SwiGLU: after W1, W3; MLP: after W1). */
static int64_t w2_offset(int kind, int64_t d, int64_t h) {
  return kind == OR_MLP ? h * d : 2 * h * d;
}

/* y = f_W(x).  For SwiGLU also returns the hidden pre-activations a1 = W1 x,
 * a3 = W3 x and z = silu(a1) * a3 (any of them may be NULL for linear); for
 * the MLP a1 = W1 x, z = silu(a1) and a3 = 1 (no gate branch). */
static void fast_forward(int kind, int64_t d, int64_t h, const double* W,
                         const double* x, double* a1, double* a3, double* z,
                         double* y) {
  if (kind == OR_LINEAR) {
    for (int64_t i = 0; i < d; ++i) {
      double s = 0.0;
      for (int64_t j = 0; j < d; ++j) s += W[i * d + j] * x[j];
      y[i] = s;
    }
    return;
  }
  const double* W1 = W;
  const double* W3 = W + h * d;
  const double* W2 = W + w2_offset(kind, d, h);
  if (kind == OR_MLP) {
    for (int64_t i = 0; i < h; ++i) {
      double s1 = 0.0;
      for (int64_t j = 0; j < d; ++j) s1 += W1[i * d + j] * x[j];
      a1[i] = s1;
      a3[i] = 1.0;
      z[i] = s1 * sigm(s1);
    }
  }
  for (int64_t i = 0; kind == OR_SWIGLU && i < h; ++i) {
    double s1 = 0.0, s3 = 0.0;
    for (int64_t j = 0; j < d; ++j) {
      s1 += W1[i * d + j] * x[j];
      s3 += W3[i * d + j] * x[j];
    }
    a1[i] = s1;
    a3[i] = s3;
    z[i] = s1 * sigm(s1) * s3;
  }
  for (int64_t i = 0; i < d; ++i) {
    double s = 0.0;
    for (int64_t j = 0; j < h; ++j) s += W2[i * h + j] * z[j];
    y[i] = s;
  }
}

/* Rank-one factors of the descent direction G = -grad_W 0.5||f_W(k)-v||^2.
 *   linear : G = e k^T,                e = v - W k                 (d)
 *   SwiGLU : G_W2 = e z^T,             e = v - W2 z                (d)
 *            G_W3 = u3 k^T,            u3 = (W2^T e) * silu(a1)    (h)
 *            G_W1 = u1 k^T,            u1 = (W2^T e) * a3 * silu'(a1)
 *   with silu'(a) = sigma(a) (1 + a (1 - sigma(a))).
 *   MLP    : G_W2 = e z^T, G_W1 = u1 k^T with z = silu(a1), a3 = 1 above.
 * Chain rule of the loss of §2 through the learner; z is also returned. */
static void descent_factors(int kind, int64_t d, int64_t h, const double* W,
                            const double* k, const double* v, double* e,
                            double* u1, double* u3, double* z, double* a1,
                            double* a3, double* y) {
  fast_forward(kind, d, h, W, k, a1, a3, z, y);
  for (int64_t i = 0; i < d; ++i) e[i] = v[i] - y[i];
  if (kind == OR_LINEAR) return;
  const double* W2 = W + w2_offset(kind, d, h);
  for (int64_t j = 0; j < h; ++j) {
    double dz = 0.0;
    for (int64_t i = 0; i < d; ++i) dz += W2[i * h + j] * e[i];
    double sg = sigm(a1[j]);
    u3[j] = dz * (a1[j] * sg);
    u1[j] = dz * a3[j] * (sg * (1.0 + a1[j] * (1.0 - sg)));
  }
}

/* Dense descent direction G for one token at weights W (P entries, packed as
 * the state).  Exposed for the gradient checks of the test suite. */
int oracle_token_descent(int kind, int64_t d, int64_t h, const double* W,
                         const double* k, const double* v, double* G) {
  if (kind != OR_LINEAR && kind != OR_SWIGLU && kind != OR_MLP) return 1;
  int64_t hh = kind == OR_LINEAR ? 1 : h;
  double* buf = (double*)malloc(sizeof(double) * (size_t)(2 * d + 5 * hh));
  if (!buf) return 2;
  double *e = buf, *y = buf + d, *u1 = buf + 2 * d, *u3 = u1 + hh,
         *z = u3 + hh, *a1 = z + hh, *a3 = a1 + hh;
  descent_factors(kind, d, h, W, k, v, e, u1, u3, z, a1, a3, y);
  if (kind == OR_LINEAR) {
    for (int64_t i = 0; i < d; ++i)
      for (int64_t j = 0; j < d; ++j) G[i * d + j] = e[i] * k[j];
  } else {
    double* G1 = G;
    double* G3 = G + h * d;
    double* G2 = G + w2_offset(kind, d, h);
    for (int64_t i = 0; i < h; ++i)
      for (int64_t j = 0; j < d; ++j) {
        G1[i * d + j] = u1[i] * k[j];
        if (kind == OR_SWIGLU) G3[i * d + j] = u3[i] * k[j];
      }
    for (int64_t i = 0; i < d; ++i)
      for (int64_t j = 0; j < h; ++j) G2[i * h + j] = e[i] * z[j];
  }
  free(buf);
  return 0;
}

/* y = f_W(x) for one vector (readout check helper). */
int oracle_fast_forward(int kind, int64_t d, int64_t h, const double* W,
                        const double* x, double* y) {
  if (kind != OR_LINEAR && kind != OR_SWIGLU && kind != OR_MLP) return 1;
  int64_t hh = kind == OR_LINEAR ? 1 : h;
  double* buf = (double*)malloc(sizeof(double) * (size_t)(3 * hh));
  if (!buf) return 2;
  fast_forward(kind, d, h, W, x, buf, buf + hh, buf + 2 * hh, y);
  free(buf);
  return 0;
}

/* Divide each row of each fast-weight matrix of one unit's state by
 * max(||row||_2, 1e-12) (the chunk-boundary normalisation option). */
static void normalise_rows(int kind, int64_t d, int64_t h, double* W) {
  int64_t nrows, len;
  for (int part = 0; part < (kind == OR_LINEAR ? 1 : 2); ++part) {
    double* base;
    if (kind == OR_LINEAR) { base = W; nrows = d; len = d; }
    else if (part == 0) { base = W; nrows = kind == OR_MLP ? h : 2 * h; len = d; } /* W1 (, W3) */
    else { base = W + w2_offset(kind, d, h); nrows = d; len = h; }                 /* W2 */
    for (int64_t r = 0; r < nrows; ++r) {
      double ss = 0.0;
      for (int64_t j = 0; j < len; ++j) ss += base[r * len + j] * base[r * len + j];
      double nrm = sqrt(ss);
      if (nrm < 1e-12) nrm = 1e-12;
      for (int64_t j = 0; j < len; ++j) base[r * len + j] /= nrm;
    }
  }
}

/* Reverse mode of normalise_rows: g holds the adjoint of the normalised W
 * and is replaced by the adjoint of W before normalisation (Wpre).  Per row
 * r with norm n: dr = (g - y (y . g)) / n, y = r / n; below the 1e-12 floor
 * the divisor is constant and dr = g / 1e-12. */
static void normalise_rows_vjp(int kind, int64_t d, int64_t h, const double* Wpre,
                               double* g) {
  int64_t nrows, len;
  for (int part = 0; part < (kind == OR_LINEAR ? 1 : 2); ++part) {
    const double* base;
    double* gb;
    if (kind == OR_LINEAR) { base = Wpre; gb = g; nrows = d; len = d; }
    else if (part == 0) { base = Wpre; gb = g; nrows = kind == OR_MLP ? h : 2 * h; len = d; }
    else {
      base = Wpre + w2_offset(kind, d, h); gb = g + w2_offset(kind, d, h); nrows = d; len = h;
    }
    for (int64_t r = 0; r < nrows; ++r) {
      const double* w = base + r * len;
      double* gr = gb + r * len;
      double ss = 0.0;
      for (int64_t j = 0; j < len; ++j) ss += w[j] * w[j];
      const double n = sqrt(ss);
      if (n < 1e-12) {
        for (int64_t j = 0; j < len; ++j) gr[j] /= 1e-12;
        continue;
      }
      double dot = 0.0;
      for (int64_t j = 0; j < len; ++j) dot += (w[j] / n) * gr[j];
      for (int64_t j = 0; j < len; ++j) gr[j] = (gr[j] - (w[j] / n) * dot) / n;
    }
  }
}

/*
 * The chunk forward over a whole sequence, literal recurrence.
 *   q, k, v, out : [B, H, L, d]      eta, alpha, beta : [B, H, L]
 *   W0, M0, Wend, Mend : [B, H, P]
 * Chunks are consecutive runs of C tokens; a final run shorter than C (when
 * C does not divide L) is a chunk of its own.  L == 0 copies the state.
 * averaged == 1 selects the chunk-averaged variant, averaged == 2 the LaCT
 * rule, qk_norm != 0 the q/k
 * prologue, row_norm != 0 the chunk-boundary normalisation (see the header).
 * Returns 0 on success, nonzero on bad arguments or allocation failure.
 */
int oracle_chunk_forward(int kind, int decay_mode, int64_t B, int64_t H,
                         int64_t L, int64_t d, int64_t h, int64_t C,
                         const double* q, const double* k, const double* v,
                         const double* eta, const double* alpha,
                         const double* beta, const double* W0,
                         const double* M0, double* out, double* Wend,
                         double* Mend, int averaged, int qk_norm, int row_norm) {
  if (kind != OR_LINEAR && kind != OR_SWIGLU && kind != OR_MLP) return 1;
  if (decay_mode != OR_GAMMA_1_MINUS_ETA_ALPHA &&
      decay_mode != OR_ALPHA_IS_GAMMA)
    return 1;
  if (B < 0 || H < 0 || L < 0 || d <= 0 || C <= 0) return 1;
  if (kind == OR_SWIGLU && h <= 0) return 1;
  if (averaged < 0 || averaged > 2) return 1;
  const int64_t P = state_size(kind, d, h);
  const int64_t hh = kind == OR_LINEAR ? 1 : h;
  const int64_t Cmax = C < L ? C : (L > 0 ? L : 1);
  int status = 0;

  for (int64_t u = 0; u < B * H; ++u) {
    double* W = Wend + u * P;
    double* M = Mend + u * P;
    memmove(W, W0 + u * P, sizeof(double) * (size_t)P);
    memmove(M, M0 + u * P, sizeof(double) * (size_t)P);
    const double* qu = q + u * L * d;
    const double* ku = k + u * L * d;
    double* qn = NULL;
    double* kn = NULL;
    if (qk_norm && L > 0) {
      qn = (double*)malloc(sizeof(double) * (size_t)(L * d));
      kn = (double*)malloc(sizeof(double) * (size_t)(L * d));
      if (!qn || !kn) {
        free(qn); free(kn);
        return 2;
      }
      memcpy(qn, qu, sizeof(double) * (size_t)(L * d));
      memcpy(kn, ku, sizeof(double) * (size_t)(L * d));
      silu_l2_rows(qn, L, d, qk_norm == 2);
      silu_l2_rows(kn, L, d, qk_norm == 2);
      qu = qn;
      ku = kn;
    }
    const double* vu = v + u * L * d;
    const double* etu = eta + u * L;
    const double* alu = alpha + u * L;
    const double* beu = beta + u * L;
    double* ou = out + u * L * d;

    /* Per-chunk buffers: frozen chunk-start weights and per-token factors. */
    double* Ws = (double*)malloc(sizeof(double) * (size_t)P);
    double* fe = (double*)malloc(sizeof(double) * (size_t)(Cmax * d));
    double* fu1 = (double*)malloc(sizeof(double) * (size_t)(Cmax * hh));
    double* fu3 = (double*)malloc(sizeof(double) * (size_t)(Cmax * hh));
    double* fz = (double*)malloc(sizeof(double) * (size_t)(Cmax * hh));
    double* gam = (double*)malloc(sizeof(double) * (size_t)Cmax);
    double* bet = (double*)malloc(sizeof(double) * (size_t)Cmax);
    if (!Ws || !fe || !fu1 || !fu3 || !fz || !gam || !bet) {
      status = 2;
    }

    for (int64_t t0 = 0; status == 0 && t0 < L; t0 += C) {
      const int64_t n = (L - t0) < C ? (L - t0) : C;
      memcpy(Ws, W, sizeof(double) * (size_t)P); /* W_0 of this chunk */

      /* Readout o_t = f_{W_0}(q_t) and descent factors at W_0. */
#pragma omp parallel
      {
        double* tmp = (double*)malloc(sizeof(double) * (size_t)(3 * hh + 2 * d));
        double *a1 = tmp, *a3 = tmp + hh, *zz = tmp + 2 * hh, *y = zz + hh,
               *y2 = y + d;
#pragma omp for schedule(static)
        for (int64_t t = 0; t < n; ++t) {
          const int64_t tt = t0 + t;
          fast_forward(kind, d, h, Ws, qu + tt * d, a1, a3, zz, y);
          for (int64_t i = 0; i < d; ++i) ou[tt * d + i] = y[i];
          descent_factors(kind, d, h, Ws, ku + tt * d, vu + tt * d,
                          fe + t * d, fu1 + t * hh, fu3 + t * hh,
                          fz + t * hh, a1, a3, y2);
        }
        free(tmp);
      }
      for (int64_t t = 0; t < n; ++t) {
        gam[t] = decay_factor(decay_mode, etu[t0 + t], alu[t0 + t]);
        bet[t] = beu[t0 + t];
      }
      if (averaged) { /* chunk-level scalars: the means over the chunk (both variants) */
        double sb = 0.0, sgm = 0.0;
        for (int64_t t = 0; t < n; ++t) {
          sb += bet[t];
          sgm += gam[t];
        }
        sb /= (double)n;
        sgm /= (double)n;
        for (int64_t t = 0; t < n; ++t) {
          bet[t] = sb;
          gam[t] = sgm;
        }
      }

      /* Token-wise recurrence on every state entry:
       *   M <- beta_t M + eta_t G_t ;  W <- gamma_t W + M.
       * Row r of the packed state has a fixed left factor index and a right
       * factor vector (k_t or z_t). */
      int64_t nrows, ncols;
      if (kind == OR_LINEAR) {
        nrows = d;
        ncols = d;
      } else {
        nrows = (kind == OR_MLP ? h : 2 * h) + d;
        ncols = 0; /* per row, below */
      }
#pragma omp parallel for schedule(dynamic, 4)
      for (int64_t r = 0; r < nrows; ++r) {
        const double* left;  /* left factor per token, stride lstride */
        int64_t lidx, lstride;
        const double* right; /* right factor per token, stride rstride */
        int64_t rstride, nc;
        double* w;
        double* m;
        if (kind == OR_LINEAR) {
          left = fe; lidx = r; lstride = d;
          right = ku + t0 * d; rstride = d; nc = ncols;
          w = W + r * d; m = M + r * d;
        } else if (r < h) { /* W1 row r */
          left = fu1; lidx = r; lstride = hh;
          right = ku + t0 * d; rstride = d; nc = d;
          w = W + r * d; m = M + r * d;
        } else if (kind == OR_MLP) { /* W2 row r-h */
          left = fe; lidx = r - h; lstride = d;
          right = fz; rstride = hh; nc = h;
          w = W + h * d + (r - h) * h;
          m = M + h * d + (r - h) * h;
        } else if (r < 2 * h) { /* W3 row r-h */
          left = fu3; lidx = r - h; lstride = hh;
          right = ku + t0 * d; rstride = d; nc = d;
          w = W + r * d; m = M + r * d;
        } else { /* W2 row r-2h */
          left = fe; lidx = r - 2 * h; lstride = d;
          right = fz; rstride = hh; nc = h;
          w = W + 2 * h * d + (r - 2 * h) * h;
          m = M + 2 * h * d + (r - 2 * h) * h;
        }
        if (averaged == 2) { /* LaCT rule: one step on the eta-weighted sum */
          for (int64_t j = 0; j < nc; ++j) {
            double gs = 0.0;
            for (int64_t t = 0; t < n; ++t)
              gs += etu[t0 + t] * (left[t * lstride + lidx] * right[t * rstride + j]);
            m[j] = bet[0] * m[j] + gs;          /* bet[], gam[] hold the means */
            w[j] = gam[0] * w[j] + m[j];
          }
          continue;
        }
        for (int64_t t = 0; t < n; ++t) {
          const double bt = bet[t];
          const double et = etu[t0 + t];
          const double gt = gam[t];
          const double lt = left[t * lstride + lidx];
          const double* rt = right + t * rstride;
          for (int64_t j = 0; j < nc; ++j) {
            const double g = lt * rt[j];        /* G_t entry (descent) */
            m[j] = bt * m[j] + et * g;          /* momentum */
            w[j] = gt * w[j] + m[j];            /* weight */
          }
        }
      }
      if (row_norm) normalise_rows(kind, d, h, W);
    }
    free(Ws); free(fe); free(fu1); free(fu3); free(fz); free(gam); free(bet);
    free(qn); free(kn);
    if (status) return status;
  }
  return 0;
}

/*
 * Per-token scalar kernels of one chunk by their definition: the factor with
 * which a unit impulse enters the chunk-end state when the recurrence above is
 * run on scalars.
 *   kw[t] : W_C when G_t = 1 and every other input is 0   (weight kernel)
 *   km[t] : M_C for the same impulse                       (momentum kernel)
 *   coef[0] = cW  : W_C when W_0 = 1 (M_0 = 0, G = 0)
 *   coef[1] = cM  : M_C when M_0 = 1 (W_0 = 0, G = 0)
 *   coef[2] = cWM : W_C when M_0 = 1 (W_0 = 0, G = 0)
 * Arrays are [nseg, n] with nseg segments of n tokens; coef is [nseg, 3].
 * O(n^2) per segment: each impulse is propagated literally to the chunk end.
 * averaged != 0: beta and gamma replaced by their segment means first;
 * averaged == 2: the LaCT rule's single chunk step applied to each impulse.
 */
int oracle_scalar_kernels(int decay_mode, int64_t nseg, int64_t n,
                          const double* eta, const double* alpha,
                          const double* beta, double* kw, double* km,
                          double* coef, int averaged) {
  if (decay_mode != OR_GAMMA_1_MINUS_ETA_ALPHA &&
      decay_mode != OR_ALPHA_IS_GAMMA)
    return 1;
  int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t sg = 0; sg < nseg; ++sg) {
    const double* e = eta + sg * n;
    const double* a = alpha + sg * n;
    const double* b0 = beta + sg * n;
    double* b = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* g = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    if (!b || !g) {
#pragma omp atomic write
      status = 2;
      free(b); free(g);
      continue;
    }
    for (int64_t s = 0; s < n; ++s) {
      b[s] = b0[s];
      g[s] = decay_factor(decay_mode, e[s], a[s]);
    }
    if (averaged && n > 0) {
      double sb = 0.0, sgm = 0.0;
      for (int64_t s = 0; s < n; ++s) {
        sb += b[s];
        sgm += g[s];
      }
      sb /= (double)n;
      sgm /= (double)n;
      for (int64_t s = 0; s < n; ++s) {
        b[s] = sb;
        g[s] = sgm;
      }
    }
    if (averaged == 2) { /* LaCT rule: M_C = bbar M_0 + sum eta G, W_C = gbar W_0 + M_C */
      const double bb = n > 0 ? b[0] : 1.0, gg = n > 0 ? g[0] : 1.0;
      for (int64_t t = 0; t < n; ++t) {
        const double m = bb * 0.0 + e[t] * 1.0;
        kw[sg * n + t] = gg * 0.0 + m;
        km[sg * n + t] = m;
      }
      double m = bb * 0.0 + 0.0; /* W_0 impulse */
      coef[sg * 3 + 0] = gg * 1.0 + m;
      m = bb * 1.0 + 0.0;        /* M_0 impulse */
      coef[sg * 3 + 1] = m;
      coef[sg * 3 + 2] = gg * 0.0 + m;
      free(b); free(g);
      continue;
    }
    for (int64_t t = 0; t < n; ++t) {
      /* token t receives the impulse: M = beta*0 + eta*1, W = gamma*0 + M */
      double m = e[t] * 1.0;
      double w = m;
      for (int64_t s = t + 1; s < n; ++s) {
        m = b[s] * m;
        w = g[s] * w + m;
      }
      kw[sg * n + t] = w;
      km[sg * n + t] = m;
    }
    double w = 1.0, m = 0.0; /* W_0 impulse */
    for (int64_t s = 0; s < n; ++s) {
      m = b[s] * m;
      w = g[s] * w + m;
    }
    coef[sg * 3 + 0] = w;
    w = 0.0; m = 1.0; /* M_0 impulse */
    for (int64_t s = 0; s < n; ++s) {
      m = b[s] * m;
      w = g[s] * w + m;
    }
    coef[sg * 3 + 1] = m;
    coef[sg * 3 + 2] = w;
    free(b); free(g);
  }
  return status;
}

/*
 * Reverse mode of G = descent(Ws; k, v) for one token: given the adjoint dG
 * (P entries, packed as the state), adds the contributions to dk, dv and dWs.
 * It walks the steps of descent_factors backwards:
 *   linear : e = v - Ws k,  G = e k^T
 *            de = dG k,  dk += dG^T e - Ws^T de,  dv += de,  dWs -= de k^T
 *   SwiGLU : a1 = W1 k, a3 = W3 k, z = silu(a1) a3, e = v - W2 z, w = W2^T e,
 *            u1 = w a3 silu'(a1), u3 = w silu(a1),
 *            G1 = u1 k^T, G3 = u3 k^T, G2 = e z^T;
 *            each intermediate's adjoint is the sum over its uses, with
 *            silu''(a) = s (1 - s) (2 + a (1 - 2 s)), s = sigma(a).
 * scratch holds at least 16 h + 4 d doubles.
 */
static void descent_vjp(int kind, int64_t d, int64_t h, const double* Ws,
                        const double* k, const double* v, const double* dG,
                        double* dk, double* dv, double* dWs, double* scratch) {
  if (kind == OR_LINEAR) {
    double* e = scratch;
    double* de = scratch + d;
    for (int64_t i = 0; i < d; ++i) {
      double y = 0.0;
      for (int64_t j = 0; j < d; ++j) y += Ws[i * d + j] * k[j];
      e[i] = v[i] - y;
      double s = 0.0;
      for (int64_t j = 0; j < d; ++j) s += dG[i * d + j] * k[j];
      de[i] = s;
    }
    for (int64_t j = 0; j < d; ++j) {
      double s1 = 0.0, s2 = 0.0;
      for (int64_t i = 0; i < d; ++i) {
        s1 += dG[i * d + j] * e[i];
        s2 += Ws[i * d + j] * de[i];
      }
      dk[j] += s1 - s2;
    }
    for (int64_t i = 0; i < d; ++i) {
      dv[i] += de[i];
      for (int64_t j = 0; j < d; ++j) dWs[i * d + j] -= de[i] * k[j];
    }
    return;
  }
  /* The MLP learner (gated == 0) is the same walk with a3 = 1 held
   * constant: no W3, no u3 (G has no W3 block) and no adjoint of a3. */
  const int gated = kind == OR_SWIGLU;
  const double* W1 = Ws;
  const double* W3 = Ws + h * d;
  const double* W2 = Ws + w2_offset(kind, d, h);
  const double* D1 = dG;
  const double* D3 = dG + h * d;
  const double* D2 = dG + w2_offset(kind, d, h);
  double* dW1 = dWs;
  double* dW3 = dWs + h * d;
  double* dW2 = dWs + w2_offset(kind, d, h);
  double *a1 = scratch, *a3 = a1 + h, *z = a3 + h, *w = z + h, *sl = w + h,
         *sp = sl + h, *spp = sp + h, *u1 = spp + h, *u3 = u1 + h, *du1 = u3 + h,
         *du3 = du1 + h, *dz = du3 + h, *dw = dz + h, *da1 = dw + h, *da3 = da1 + h;
  double *y = scratch + 16 * h, *e = y + d, *de = e + d;
  fast_forward(kind, d, h, Ws, k, a1, a3, z, y);
  for (int64_t o = 0; o < d; ++o) e[o] = v[o] - y[o];
  for (int64_t i = 0; i < h; ++i) {
    double s = 0.0;
    for (int64_t o = 0; o < d; ++o) s += W2[o * h + i] * e[o];
    w[i] = s;
    const double sg = sigm(a1[i]);
    sl[i] = a1[i] * sg;
    sp[i] = sg * (1.0 + a1[i] * (1.0 - sg));
    spp[i] = sg * (1.0 - sg) * (2.0 + a1[i] * (1.0 - 2.0 * sg));
    u1[i] = w[i] * a3[i] * sp[i];
    u3[i] = w[i] * sl[i];
  }
  /* G1 = u1 k^T, G3 = u3 k^T */
  for (int64_t i = 0; i < h; ++i) {
    double s1 = 0.0, s3 = 0.0;
    for (int64_t j = 0; j < d; ++j) {
      s1 += D1[i * d + j] * k[j];
      if (gated) s3 += D3[i * d + j] * k[j];
    }
    du1[i] = s1;
    du3[i] = s3;
  }
  for (int64_t j = 0; j < d; ++j) {
    double s = 0.0;
    for (int64_t i = 0; i < h; ++i)
      s += D1[i * d + j] * u1[i] + (gated ? D3[i * d + j] * u3[i] : 0.0);
    dk[j] += s;
  }
  /* G2 = e z^T */
  for (int64_t o = 0; o < d; ++o) {
    double s = 0.0;
    for (int64_t i = 0; i < h; ++i) s += D2[o * h + i] * z[i];
    de[o] = s;
  }
  for (int64_t i = 0; i < h; ++i) {
    double s = 0.0;
    for (int64_t o = 0; o < d; ++o) s += D2[o * h + i] * e[o];
    dz[i] = s;
  }
  /* u1 = w a3 silu'(a1), u3 = w silu(a1) */
  for (int64_t i = 0; i < h; ++i) {
    dw[i] = du3[i] * sl[i] + du1[i] * a3[i] * sp[i];
    da1[i] = du3[i] * w[i] * sp[i] + du1[i] * w[i] * a3[i] * spp[i];
    da3[i] = du1[i] * w[i] * sp[i];
  }
  /* w = W2^T e */
  for (int64_t o = 0; o < d; ++o) {
    double s = 0.0;
    for (int64_t i = 0; i < h; ++i) {
      s += W2[o * h + i] * dw[i];
      dW2[o * h + i] += e[o] * dw[i];
    }
    de[o] += s;
  }
  /* e = v - y, y = W2 z */
  for (int64_t o = 0; o < d; ++o) {
    dv[o] += de[o];
    for (int64_t i = 0; i < h; ++i) dW2[o * h + i] -= de[o] * z[i];
  }
  for (int64_t i = 0; i < h; ++i) {
    double s = 0.0;
    for (int64_t o = 0; o < d; ++o) s += W2[o * h + i] * de[o];
    dz[i] -= s;
  }
  /* z = silu(a1) a3, a1 = W1 k, a3 = W3 k */
  for (int64_t i = 0; i < h; ++i) {
    da1[i] += dz[i] * a3[i] * sp[i];
    da3[i] += dz[i] * sl[i];
    for (int64_t j = 0; j < d; ++j) {
      dW1[i * d + j] += da1[i] * k[j];
      if (gated) dW3[i * d + j] += da3[i] * k[j];
    }
  }
  for (int64_t j = 0; j < d; ++j) {
    double s = 0.0;
    for (int64_t i = 0; i < h; ++i)
      s += W1[i * d + j] * da1[i] + (gated ? W3[i * d + j] * da3[i] : 0.0);
    dk[j] += s;
  }
}

/* Reverse mode of the readout o = f_Ws(x): adds the contributions of the
 * output adjoint dy to dx and dWs.  scratch holds at least 8 h + d doubles. */
static void readout_vjp(int kind, int64_t d, int64_t h, const double* Ws,
                        const double* x, const double* dy, double* dx, double* dWs,
                        double* scratch) {
  if (kind == OR_LINEAR) {
    for (int64_t j = 0; j < d; ++j) {
      double s = 0.0;
      for (int64_t i = 0; i < d; ++i) s += Ws[i * d + j] * dy[i];
      dx[j] += s;
    }
    for (int64_t i = 0; i < d; ++i)
      for (int64_t j = 0; j < d; ++j) dWs[i * d + j] += dy[i] * x[j];
    return;
  }
  const int gated = kind == OR_SWIGLU; /* the MLP: a3 = 1, no W3 */
  const double* W1 = Ws;
  const double* W3 = Ws + h * d;
  const double* W2 = Ws + w2_offset(kind, d, h);
  double* dW1 = dWs;
  double* dW3 = dWs + h * d;
  double* dW2 = dWs + w2_offset(kind, d, h);
  double *a1 = scratch, *a3 = a1 + h, *z = a3 + h, *dz = z + h, *da1 = dz + h,
         *da3 = da1 + h, *y = scratch + 8 * h;
  fast_forward(kind, d, h, Ws, x, a1, a3, z, y);
  for (int64_t i = 0; i < h; ++i) {
    double s = 0.0;
    for (int64_t o = 0; o < d; ++o) s += W2[o * h + i] * dy[o];
    dz[i] = s;
    const double sg = sigm(a1[i]);
    da1[i] = s * a3[i] * (sg * (1.0 + a1[i] * (1.0 - sg)));
    da3[i] = s * (a1[i] * sg);
  }
  for (int64_t o = 0; o < d; ++o)
    for (int64_t i = 0; i < h; ++i) dW2[o * h + i] += dy[o] * z[i];
  for (int64_t i = 0; i < h; ++i)
    for (int64_t j = 0; j < d; ++j) {
      dW1[i * d + j] += da1[i] * x[j];
      if (gated) dW3[i * d + j] += da3[i] * x[j];
    }
  for (int64_t j = 0; j < d; ++j) {
    double s = 0.0;
    for (int64_t i = 0; i < h; ++i)
      s += W1[i * d + j] * da1[i] + (gated ? W3[i * d + j] * da3[i] : 0.0);
    dx[j] += s;
  }
}

/*
 * Reverse mode of the chunk forward (the outer-loop backward), linear,
 * SwiGLU and MLP learners: the gradient of a scalar loss
 *     l = <dout, out> + <dWend, Wend> + <dMend, Mend>
 * with respect to every input of oracle_chunk_forward.  It differentiates the
 * same literal recurrence, one token at a time in reverse:
 *   - the chunk-start states (W, M) of every chunk are recorded by a forward
 *     pass; each chunk is re-run to record the state before each token;
 *   - token t of a chunk with frozen weights Ws did
 *         G = descent(Ws; k_t, v_t),
 *         M <- beta_t M + eta_t G,  W <- gamma_t W + M,
 *     so with (dW, dM) the adjoint of the state after the token:
 *         dMt    = dM + dW                      (W used the new M)
 *         dgamma = <dW, W_before>,  dbeta = <dMt, M_before>
 *         deta  += <dMt, G>,        dG = eta_t dMt
 *         (dk_t, dv_t, dWs) += reverse mode of descent at dG (descent_vjp)
 *         dW <- gamma_t dW,  dM <- beta_t dMt;
 *   - the readout o_t = f_Ws(q_t) adds its reverse mode to dq_t and dWs;
 *   - Ws is the state at the chunk start, so dW += dWs before the previous
 *     chunk is processed;
 *   - gamma_t = 1 - eta_t alpha_t (Eq. 14): deta_t -= alpha_t dgamma,
 *     dalpha_t = -eta_t dgamma; with alpha taken as gamma, dalpha_t = dgamma.
 * With qk_norm != 0 the q/k prologue (SiLU, then L2 per token) runs first, as
 * in the forward, and dq, dk are mapped back through it (silu_l2_rows_vjp).
 * With averaged != 0 (the chunk-averaged variant) every token of a chunk uses
 * the chunk means of beta and gamma, so the per-token adjoints of the two
 * means are summed over the chunk and each token's beta and gamma receive
 * 1/n of the sums.  With averaged == 2 (the LaCT rule) a chunk is one step,
 * M_C = bbar M_s + sum_t eta_t G_t, W_C = gbar W_s + M_C, walked backwards
 * as a whole (the adjoints of the means again shared out by 1/n).  The MLP
 * learner takes the SwiGLU walk with a3 = 1 held constant (no W3 block).
 * With row_norm != 0 (chunk-boundary normalisation) the
 * forward normalises W after every chunk, the last included, so before a
 * chunk is walked in reverse the adjoint of its normalised end state is taken
 * back through the normalisation (normalise_rows_vjp) at the state before it.  dWend or dMend may be NULL (zero).  h is the SwiGLU hidden
 * width (ignored for linear).  Returns 0 on success, 1 on bad arguments,
 * 2 on allocation failure, 3 for an unknown learner.
 */
int oracle_chunk_backward(int kind, int decay_mode, int64_t B, int64_t H,
                          int64_t L, int64_t d, int64_t h, int64_t C,
                          const double* q, const double* k, const double* v,
                          const double* eta, const double* alpha,
                          const double* beta, const double* W0,
                          const double* M0, const double* dout,
                          const double* dWend, const double* dMend,
                          double* dq, double* dk, double* dv, double* deta,
                          double* dalpha, double* dbeta, double* dW0,
                          double* dM0, int qk_norm, int averaged, int row_norm) {
  if (averaged < 0 || averaged > 2) return 1;
  if (kind != OR_LINEAR && kind != OR_SWIGLU && kind != OR_MLP) return 3;
  if (decay_mode != OR_GAMMA_1_MINUS_ETA_ALPHA &&
      decay_mode != OR_ALPHA_IS_GAMMA)
    return 1;
  if (B < 0 || H < 0 || L < 0 || d <= 0 || C <= 0) return 1;
  if (kind != OR_LINEAR && h <= 0) return 1;
  const int64_t P = state_size(kind, d, h);
  const int64_t nC = (L + C - 1) / C;
  const int64_t Cmax = C < L ? C : (L > 0 ? L : 1);
  const int64_t nscr = 16 * (kind == OR_LINEAR ? 1 : h) + 4 * d;
  /* The momentum and decay factors each token of a chunk uses. */
  double* fb = (double*)malloc(sizeof(double) * (size_t)Cmax);
  double* fg = (double*)malloc(sizeof(double) * (size_t)Cmax);
  if (!fb || !fg) {
    free(fb); free(fg);
    return 2;
  }
#define CHUNK_FACTORS(t0_, n_)                                                     \
  do {                                                                             \
    double sb_ = 0.0, sg_ = 0.0;                                                   \
    for (int64_t t_ = 0; t_ < (n_); ++t_) {                                        \
      fb[t_] = beu[(t0_) + t_];                                                    \
      fg[t_] = decay_factor(decay_mode, etu[(t0_) + t_], alu[(t0_) + t_]);         \
      sb_ += fb[t_];                                                               \
      sg_ += fg[t_];                                                               \
    }                                                                              \
    if (averaged)                                                                  \
      for (int64_t t_ = 0; t_ < (n_); ++t_) {                                      \
        fb[t_] = sb_ / (double)(n_);                                               \
        fg[t_] = sg_ / (double)(n_);                                               \
      }                                                                            \
  } while (0)

  double* qkn = NULL; /* normalised q | k of one unit (q/k prologue) */
  if (qk_norm && L > 0) {
    qkn = (double*)malloc(sizeof(double) * (size_t)(2 * L * d));
    if (!qkn) {
      free(fb); free(fg);
      return 2;
    }
  }
  for (int64_t u = 0; u < B * H; ++u) {
    const double* qu = q + u * L * d;
    const double* ku = k + u * L * d;
    if (qkn) {
      memcpy(qkn, qu, sizeof(double) * (size_t)(L * d));
      memcpy(qkn + L * d, ku, sizeof(double) * (size_t)(L * d));
      silu_l2_rows(qkn, L, d, 0);
      silu_l2_rows(qkn + L * d, L, d, 0);
      qu = qkn;
      ku = qkn + L * d;
    }
    const double* vu = v + u * L * d;
    const double* etu = eta + u * L;
    const double* alu = alpha + u * L;
    const double* beu = beta + u * L;
    const double* dou = dout + u * L * d;
    double* dqu = dq + u * L * d;
    double* dku = dk + u * L * d;
    double* dvu = dv + u * L * d;
    double* detu = deta + u * L;
    double* dalu = dalpha + u * L;
    double* dbeu = dbeta + u * L;
    for (int64_t i = 0; i < L * d; ++i) dqu[i] = dku[i] = dvu[i] = 0.0;
    for (int64_t t = 0; t < L; ++t) detu[t] = dalu[t] = dbeu[t] = 0.0;

    double* Wst = (double*)malloc(sizeof(double) * (size_t)((nC > 0 ? nC : 1) * P));
    double* Mst = (double*)malloc(sizeof(double) * (size_t)((nC > 0 ? nC : 1) * P));
    double* Wb = (double*)malloc(sizeof(double) * (size_t)(Cmax * P));
    double* Mb = (double*)malloc(sizeof(double) * (size_t)(Cmax * P));
    double* Gt = (double*)malloc(sizeof(double) * (size_t)(Cmax * P));
    double* W = (double*)malloc(sizeof(double) * (size_t)P);
    double* M = (double*)malloc(sizeof(double) * (size_t)P);
    double* dW = (double*)malloc(sizeof(double) * (size_t)P);
    double* dM = (double*)malloc(sizeof(double) * (size_t)P);
    double* dMt = (double*)malloc(sizeof(double) * (size_t)P);
    double* dG = (double*)malloc(sizeof(double) * (size_t)P);
    double* dWs = (double*)malloc(sizeof(double) * (size_t)P);
    double* scr = (double*)malloc(sizeof(double) * (size_t)nscr);
    if (!Wst || !Mst || !Wb || !Mb || !Gt || !W || !M || !dW || !dM || !dMt || !dG ||
        !dWs || !scr) {
      free(Wst); free(Mst); free(Wb); free(Mb); free(Gt); free(W); free(M);
      free(dW); free(dM); free(dMt); free(dG); free(dWs); free(scr); free(qkn);
      free(fb); free(fg);
      return 2;
    }

    /* Forward: chunk-start states. */
    memcpy(W, W0 + u * P, sizeof(double) * (size_t)P);
    memcpy(M, M0 + u * P, sizeof(double) * (size_t)P);
    for (int64_t r = 0; r < nC; ++r) {
      const int64_t t0 = r * C, n = (L - t0) < C ? (L - t0) : C;
      memcpy(Wst + r * P, W, sizeof(double) * (size_t)P);
      memcpy(Mst + r * P, M, sizeof(double) * (size_t)P);
      const double* Ws = Wst + r * P;
      CHUNK_FACTORS(t0, n);
      if (averaged == 2) { /* LaCT: M <- bbar M + sum eta G, W <- gbar W + M */
        for (int64_t i = 0; i < P; ++i) M[i] *= fb[0];
        for (int64_t t = 0; t < n; ++t) {
          const int64_t tt = t0 + t;
          oracle_token_descent(kind, d, h, Ws, ku + tt * d, vu + tt * d, Gt);
          for (int64_t i = 0; i < P; ++i) M[i] += etu[tt] * Gt[i];
        }
        for (int64_t i = 0; i < P; ++i) W[i] = fg[0] * W[i] + M[i];
      } else {
        for (int64_t t = 0; t < n; ++t) {
          const int64_t tt = t0 + t;
          oracle_token_descent(kind, d, h, Ws, ku + tt * d, vu + tt * d, Gt);
          for (int64_t i = 0; i < P; ++i) {
            M[i] = fb[t] * M[i] + etu[tt] * Gt[i];
            W[i] = fg[t] * W[i] + M[i];
          }
        }
      }
      if (row_norm) normalise_rows(kind, d, h, W);
    }

    /* Backward. */
    for (int64_t i = 0; i < P; ++i) {
      dW[i] = dWend ? dWend[u * P + i] : 0.0;
      dM[i] = dMend ? dMend[u * P + i] : 0.0;
    }
    for (int64_t r = nC - 1; r >= 0; --r) {
      const int64_t t0 = r * C, n = (L - t0) < C ? (L - t0) : C;
      const double* Ws = Wst + r * P;
      if (averaged == 2) {
        /* LaCT: M_C = bbar M_s + sum_t eta_t G_t, W_C = gbar W_s + M_C with
         * the chunk means bbar, gbar.  With (dW, dM) the adjoint of
         * (W_C, M_C): dMt = dM + dW, dgbar = <dW, W_s>, dbbar = <dMt, M_s>,
         * deta_t += <dMt, G_t>, dG_t = eta_t dMt; dW <- gbar dW,
         * dM <- bbar dMt; each token's beta, gamma gets 1/n of dbbar, dgbar. */
        const double* Msr = Mst + r * P;
        CHUNK_FACTORS(t0, n);
        if (row_norm) { /* the chunk end before its normalisation */
          memcpy(W, Ws, sizeof(double) * (size_t)P);
          memcpy(M, Msr, sizeof(double) * (size_t)P);
          for (int64_t i = 0; i < P; ++i) M[i] *= fb[0];
          for (int64_t t = 0; t < n; ++t) {
            const int64_t tt = t0 + t;
            oracle_token_descent(kind, d, h, Ws, ku + tt * d, vu + tt * d, Gt);
            for (int64_t i = 0; i < P; ++i) M[i] += etu[tt] * Gt[i];
          }
          for (int64_t i = 0; i < P; ++i) W[i] = fg[0] * W[i] + M[i];
          normalise_rows_vjp(kind, d, h, W, dW);
        }
        double dgb = 0.0, dbb = 0.0;
        for (int64_t i = 0; i < P; ++i) {
          dMt[i] = dM[i] + dW[i];
          dgb += dW[i] * Ws[i];
          dbb += dMt[i] * Msr[i];
          dWs[i] = 0.0;
        }
        for (int64_t t = 0; t < n; ++t) {
          const int64_t tt = t0 + t;
          oracle_token_descent(kind, d, h, Ws, ku + tt * d, vu + tt * d, Gt);
          double detd = 0.0;
          for (int64_t i = 0; i < P; ++i) {
            detd += dMt[i] * Gt[i];
            dG[i] = etu[tt] * dMt[i];
          }
          detu[tt] += detd;
          descent_vjp(kind, d, h, Ws, ku + tt * d, vu + tt * d, dG, dku + tt * d,
                      dvu + tt * d, dWs, scr);
        }
        for (int64_t i = 0; i < P; ++i) {
          dW[i] = fg[0] * dW[i];
          dM[i] = fb[0] * dMt[i];
        }
        for (int64_t t = 0; t < n; ++t) {
          const int64_t tt = t0 + t;
          const double dg = dgb / (double)n;
          dbeu[tt] += dbb / (double)n;
          if (decay_mode == OR_GAMMA_1_MINUS_ETA_ALPHA) {
            detu[tt] -= alu[tt] * dg;
            dalu[tt] += -etu[tt] * dg;
          } else {
            dalu[tt] += dg;
          }
        }
        for (int64_t t = 0; t < n; ++t) {
          const int64_t tt = t0 + t;
          readout_vjp(kind, d, h, Ws, qu + tt * d, dou + tt * d, dqu + tt * d, dWs, scr);
        }
        for (int64_t i = 0; i < P; ++i) dW[i] += dWs[i];
        continue;
      }
      /* Re-run the chunk, recording the state before each token and G. */
      memcpy(W, Ws, sizeof(double) * (size_t)P);
      memcpy(M, Mst + r * P, sizeof(double) * (size_t)P);
      CHUNK_FACTORS(t0, n);
      for (int64_t t = 0; t < n; ++t) {
        const int64_t tt = t0 + t;
        memcpy(Wb + t * P, W, sizeof(double) * (size_t)P);
        memcpy(Mb + t * P, M, sizeof(double) * (size_t)P);
        double* G = Gt + t * P;
        oracle_token_descent(kind, d, h, Ws, ku + tt * d, vu + tt * d, G);
        for (int64_t i = 0; i < P; ++i) {
          M[i] = fb[t] * M[i] + etu[tt] * G[i];
          W[i] = fg[t] * W[i] + M[i];
        }
      }
      if (row_norm) normalise_rows_vjp(kind, d, h, W, dW); /* W: the chunk end, before it */
      for (int64_t i = 0; i < P; ++i) dWs[i] = 0.0;
      double sum_dbet = 0.0, sum_dgam = 0.0; /* adjoints of the chunk means */
      for (int64_t t = n - 1; t >= 0; --t) {
        const int64_t tt = t0 + t;
        const double et = etu[tt];
        const double g = fg[t];
        const double* G = Gt + t * P;
        double dgam = 0.0, dbet = 0.0, detd = 0.0;
        for (int64_t i = 0; i < P; ++i) {
          dMt[i] = dM[i] + dW[i];
          dgam += dW[i] * Wb[t * P + i];
          dbet += dMt[i] * Mb[t * P + i];
          detd += dMt[i] * G[i];
          dG[i] = et * dMt[i];
        }
        descent_vjp(kind, d, h, Ws, ku + tt * d, vu + tt * d, dG, dku + tt * d,
                    dvu + tt * d, dWs, scr);
        for (int64_t i = 0; i < P; ++i) {
          dW[i] = g * dW[i];
          dM[i] = fb[t] * dMt[i];
        }
        detu[tt] += detd;
        if (averaged) {
          sum_dbet += dbet;
          sum_dgam += dgam;
          continue;
        }
        dbeu[tt] += dbet;
        if (decay_mode == OR_GAMMA_1_MINUS_ETA_ALPHA) {
          detu[tt] -= alu[tt] * dgam;
          dalu[tt] += -et * dgam;
        } else {
          dalu[tt] += dgam;
        }
      }
      if (averaged) /* each token's beta, gamma enters its chunk mean with weight 1/n */
        for (int64_t t = 0; t < n; ++t) {
          const int64_t tt = t0 + t;
          const double dg = sum_dgam / (double)n;
          dbeu[tt] += sum_dbet / (double)n;
          if (decay_mode == OR_GAMMA_1_MINUS_ETA_ALPHA) {
            detu[tt] -= alu[tt] * dg;
            dalu[tt] += -etu[tt] * dg;
          } else {
            dalu[tt] += dg;
          }
        }
      /* Readout o_t = f_Ws(q_t). */
      for (int64_t t = 0; t < n; ++t) {
        const int64_t tt = t0 + t;
        readout_vjp(kind, d, h, Ws, qu + tt * d, dou + tt * d, dqu + tt * d, dWs, scr);
      }
      for (int64_t i = 0; i < P; ++i) dW[i] += dWs[i];
    }
    memcpy(dW0 + u * P, dW, sizeof(double) * (size_t)P);
    memcpy(dM0 + u * P, dM, sizeof(double) * (size_t)P);
    if (qkn) { /* back through the prologue, from the raw inputs */
      silu_l2_rows_vjp(q + u * L * d, dqu, L, d);
      silu_l2_rows_vjp(k + u * L * d, dku, L, d);
    }
    free(Wst); free(Mst); free(Wb); free(Mb); free(Gt); free(W); free(M);
    free(dW); free(dM); free(dMt); free(dG); free(dWs); free(scr);
  }
  free(qkn);
  free(fb);
  free(fg);
#undef CHUNK_FACTORS
  return 0;
}

/*
 * The per-token scalar heads (see the header): x [B, L, D] is the layer
 * input, w [3H, D] the head weights in the order (eta heads 0..H-1, alpha
 * heads, beta heads), bias [3H].  Writes eta, alpha, beta [B, H, L].
 * Returns 0 on success, 1 on bad arguments.
 */
int oracle_scalar_heads(int64_t B, int64_t L, int64_t D, int64_t H, const double* x,
                        const double* w, const double* bias, double eta_base,
                        double alpha_base, double* eta, double* alpha, double* beta) {
  if (B < 0 || L < 0 || D <= 0 || H <= 0) return 1;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < B * L; ++n) {
    const int64_t b = n / L, t = n % L;
    const double* xt = x + n * D;
    for (int64_t c = 0; c < 3 * H; ++c) {
      double z = 0.0;
      for (int64_t j = 0; j < D; ++j) z += w[c * D + j] * xt[j];
      const double s = sigm(z + bias[c]);
      const int64_t head = c % H;
      const int64_t o = (b * H + head) * L + t;
      if (c < H) eta[o] = eta_base * s;
      else if (c < 2 * H) alpha[o] = alpha_base * s;
      else beta[o] = s;
    }
  }
  return 0;
}
