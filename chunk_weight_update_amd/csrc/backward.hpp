// backward.hpp -- outer-loop backward of the chunk forward for the linear
// learner f_W(x) = W x (fp32 inputs, d <= 64, a multiple of 16).
//
// The chunk forward of "Rethinking Expressivity and Efficiency in Test-Time
// Training" (E2-TTT, §3.2 and App. A) gives, per chunk with chunk-start state
// (Ws, Ms), per-token residuals e_t = v_t - Ws k_t and kernels K^W, K^M:
//   out_t = Ws q_t                                         (Eq. 6)
//   W_C = cW Ws + cWM Ms + sum_t K^W_t e_t k_t^T
//   M_C = cM Ms + sum_t K^M_t e_t k_t^T.
// Given the adjoints (dW_C, dM_C) of the chunk-end state and dout, the
// chunk's reverse step is, with u_t = dW_C k_t and m_t = dM_C k_t:
//   dK^W_t = e_t . u_t,  dK^M_t = e_t . m_t
//   de_t = K^W_t u_t + K^M_t m_t,  dv_t = de_t
//   dq_t = Ws^T dout_t
//   dk_t = K^W_t dW_C^T e_t + K^M_t dM_C^T e_t - Ws^T de_t
//   dWs  = cW dW_C + sum_t (dout_t q_t^T - de_t k_t^T)
//   dMs  = cWM dW_C + cM dM_C
//   dcW = <dW_C, Ws>,  dcM = <dM_C, Ms>,  dcWM = <dW_C, Ms>
// and (dWs, dMs) are the adjoints of the previous chunk's end state.  The
// kernels' adjoints are carried to eta, alpha, beta by the reverse mode of the
// scalar scan (App. A.2's suffix products and the affine reverse scan of P),
// which runs forward in token order (k_lin_bwd_scalars).
//
//   k_lin_bwd_tok     per 16 tokens: e, u, m, de, dK^W, dK^M, dv, dq, dk
//   k_lin_bwd_state   per 16-row block of the state: dWs, dMs and the block's
//                     partial sums of dcW, dcM, dcWM (added later in block
//                     order, so results do not depend on scheduling)
//   k_lin_bwd_scalars per (unit, chunk) segment, one wave: deta, dalpha, dbeta
#pragma once

#include "kernels.hpp"

namespace e2ttt {

// dst[i] = src[i] converted (bf16 <-> fp32; fp32 -> bf16 rounds to nearest even).
template <typename S, typename D>
__global__ __launch_bounds__(256) void k_convert(const S* __restrict__ src, D* __restrict__ dst,
                                                 int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) dst[i] = from_f32<D>(to_f32<S>(src[i]));
}

// Reverse mode of the q/k prologue (SiLU, then L2 per token, §4): dy is the
// adjoint of y = s / max(||s||, 1e-12), s = silu(x); writes the adjoint of x:
//   dx = (dy - y (y . dy)) / ||s|| * silu'(x)   (dy / 1e-12 * silu'(x) below the floor).
// One wave per row, as the forward prologue (rows of up to 1024 features).
__global__ __launch_bounds__(256) void k_qk_norm_bwd(const float* __restrict__ x,
                                                     const float* __restrict__ dy,
                                                     float* __restrict__ dx, int64_t rows,
                                                     int64_t d) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* xr = x + row * d;
  const float* gr = dy + row * d;
  float* outr = dx + row * d;
  float s[16], g[16];
  float ss = 0.0f, sg = 0.0f;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int64_t e = lane + 64 * m;
    const float v = e < d ? xr[e] : 0.0f;
    s[m] = v * sigmoidf_(v);
    g[m] = e < d ? gr[e] : 0.0f;
    ss = fmaf(s[m], s[m], ss);
    sg = fmaf(s[m], g[m], sg);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ss += __shfl_xor(ss, off, 64);
    sg += __shfl_xor(sg, off, 64);
  }
  const float n = sqrtf(ss);
  const bool above = n >= 1e-12f;
  const float inv = 1.0f / (above ? n : 1e-12f);
  const float dot = above ? sg * inv : 0.0f;  // y . dy
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int64_t e = lane + 64 * m;
    if (e >= d) continue;
    const float v = xr[e], sgm = sigmoidf_(v);
    const float ds = (g[m] - s[m] * inv * dot) * inv;
    outr[e] = ds * (sgm * (1.0f + v * (1.0f - sgm)));
  }
}

// Reverse mode of k_row_l2norm: g is the adjoint of the normalised rows,
// Wpre the state before normalisation; writes the adjoint of Wpre:
//   dr = (g - y (y . g)) / n,  y = r / n  (g / 1e-12 below the floor).
// Rows and waves as k_row_l2norm; dW may not alias g.
__global__ __launch_bounds__(256) void k_row_l2norm_bwd(const float* __restrict__ Wpre,
                                                        const float* __restrict__ g,
                                                        float* __restrict__ dW, int64_t BH,
                                                        int64_t d, int64_t h) {
  const int lane = threadIdx.x & 63;
  const int64_t rows_u = h == 0 ? d : 2 * h + d;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= BH * rows_u) return;  // whole waves leave together
  const int64_t u = row / rows_u, r = row % rows_u;
  const int64_t P = h == 0 ? d * d : 3 * d * h;
  int64_t off, len;
  if (h == 0 || r < 2 * h) {
    off = u * P + r * d;
    len = d;
  } else {
    off = u * P + 2 * h * d + (r - 2 * h) * h;
    len = h;
  }
  float ss = 0.0f, wg = 0.0f;
  for (int64_t j = lane; j < len; j += 64) {
    const float w = Wpre[off + j];
    ss = fmaf(w, w, ss);
    wg = fmaf(w, g[off + j], wg);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ss += __shfl_down(ss, o);
    wg += __shfl_down(wg, o);
  }
  ss = __shfl(ss, 0);
  wg = __shfl(wg, 0);
  const float n = sqrtf(ss);
  const bool above = n >= 1e-12f;
  const float inv = 1.0f / (above ? n : 1e-12f);
  const float dot = above ? wg * inv : 0.0f;  // y . g
  for (int64_t j = lane; j < len; j += 64)
    dW[off + j] = (g[off + j] - Wpre[off + j] * inv * dot) * inv;
}

struct LinBwdArgs {
  Shape s;
  int r;     // chunk index
  int mode;  // decay mode: 0 gamma = 1 - eta alpha (Eq. 14), 1 gamma = alpha
  const float* q;
  const float* k;
  const float* v;
  const float* dout;
  const float* Ws;   // chunk-start state of chunk r, [BH][P]
  const float* Ms;
  const float* dWC;  // adjoints of chunk r's end state, [BH][P]
  const float* dMC;
  const float* kw;   // [BH][nC][Cp]
  const float* km;
  const float* coef; // [BH][nC][4]: cW, cM, cWM
  float* dq;         // [BH][L][d]
  float* dk;
  float* dv;
  float* de;         // [BH][Cp][d] (zero on padding tokens)
  float* sw;         // dK^W, [BH][nC][Cp]
  float* sm;         // dK^M
  float* dots;       // [BH][nC][d/16][4]: block partials of dcW, dcM, dcWM
  float* dWp;        // adjoints of chunk r's start state, [BH][P]
  float* dMp;
};

// LDS floats of k_lin_bwd_tok: three d x (d+1) matrices and four
// LIN_BWD_TB x (d+1) token tiles.
constexpr int LIN_BWD_TB = 16;  // tokens per workgroup
__host__ __device__ constexpr int64_t lin_bwd_tok_lds_floats(int64_t d) {
  return (3 * d + 4 * LIN_BWD_TB) * (d + 1);
}

// One workgroup per 16 tokens of a chunk; d = 16 R.  Thread (token pr =
// tid / 16, g = tid % 16) owns rows g, g+16, .. (phase 1) and columns g,
// g+16, .. (phase 2), so each thread runs 3R or 4R independent dot products
// with compile-time trip counts.
template <int R>
__global__ __launch_bounds__(256) void k_lin_bwd_tok(LinBwdArgs a) {
  constexpr int d = 16 * R, D1 = d + 1, TB = LIN_BWD_TB;
  extern __shared__ float lsm[];
  const Shape& s = a.s;
  float* Wl = lsm;             // Ws
  float* dWl = Wl + d * D1;    // dW_C
  float* dMl = dWl + d * D1;   // dM_C
  float* Kt = dMl + d * D1;    // k rows of the tile
  float* Xt = Kt + TB * D1;    // v rows, then dout rows
  float* Et = Xt + TB * D1;    // e
  float* Dt = Et + TB * D1;    // de
  const int64_t ntm = s.Cp / TB;
  const int64_t mt = blockIdx.x % ntm, u = blockIdx.x / ntm;
  const int64_t p0 = mt * TB;
  const int64_t tok0 = static_cast<int64_t>(a.r) * s.C;
  const int64_t nv = n_valid(s, a.r);
  constexpr int64_t P = static_cast<int64_t>(d) * d;
  const int64_t seg = u * s.nC + a.r;
#pragma unroll 8
  for (int idx = threadIdx.x; idx < d * d; idx += 256) {
    const int o = (idx / d) * D1 + idx % d;
    Wl[o] = a.Ws[u * P + idx];
    dWl[o] = a.dWC[u * P + idx];
    dMl[o] = a.dMC[u * P + idx];
  }
#pragma unroll 8
  for (int idx = threadIdx.x; idx < TB * d; idx += 256) {
    const int pr = idx / d, c = idx % d;
    const int64_t p = p0 + pr;
    const bool ok = p < nv;
    const int64_t gi = (u * s.L + tok0 + p) * d + c;
    Kt[pr * D1 + c] = ok ? a.k[gi] : 0.0f;
    Xt[pr * D1 + c] = ok ? a.v[gi] : 0.0f;
  }
  __syncthreads();
  const int pr = threadIdx.x >> 4, g = threadIdx.x & 15;
  const int64_t p = p0 + pr;
  const float kwv = p < nv ? a.kw[seg * s.Cp + p] : 0.0f;
  const float kmv = p < nv ? a.km[seg * s.Cp + p] : 0.0f;
  // Phase 1, rows i = g + 16 r: e, u, m, de and this thread's share of
  // dK^W = e . u and dK^M = e . m.
  {
    float y[R], uu[R], mm[R];
#pragma unroll
    for (int r = 0; r < R; ++r) { y[r] = 0.0f; uu[r] = 0.0f; mm[r] = 0.0f; }
#pragma unroll 8
    for (int j = 0; j < d; ++j) {
      const float kj = Kt[pr * D1 + j];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int i = g + 16 * r;
        y[r] += Wl[i * D1 + j] * kj;
        uu[r] += dWl[i * D1 + j] * kj;
        mm[r] += dMl[i * D1 + j] * kj;
      }
    }
    float pw = 0.0f, pm = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int i = g + 16 * r;
      const float e = Xt[pr * D1 + i] - y[r];
      const float de = kwv * uu[r] + kmv * mm[r];
      Et[pr * D1 + i] = e;
      Dt[pr * D1 + i] = de;
      pw += e * uu[r];
      pm += e * mm[r];
      a.de[(u * s.Cp + p) * d + i] = de;
      if (p < nv) a.dv[(u * s.L + tok0 + p) * d + i] = de;
    }
    // The token's 16 threads are 16 consecutive lanes: a fixed tree into g = 0.
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
      pw += __shfl_down(pw, off, 16);
      pm += __shfl_down(pm, off, 16);
    }
    if (g == 0) {
      a.sw[seg * s.Cp + p] = pw;
      a.sm[seg * s.Cp + p] = pm;
    }
  }
  __syncthreads();
#pragma unroll 8
  for (int idx = threadIdx.x; idx < TB * d; idx += 256) {
    const int rr = idx / d, c = idx % d;
    const int64_t pp = p0 + rr;
    Xt[rr * D1 + c] = pp < nv ? a.dout[(u * s.L + tok0 + pp) * d + c] : 0.0f;
  }
  __syncthreads();
  // Phase 2, columns j = g + 16 c: dq and dk.
  float gq[R], gw[R], gm[R], gd[R];
#pragma unroll
  for (int c = 0; c < R; ++c) { gq[c] = 0.0f; gw[c] = 0.0f; gm[c] = 0.0f; gd[c] = 0.0f; }
#pragma unroll 8
  for (int i = 0; i < d; ++i) {
    const float ei = Et[pr * D1 + i], oi = Xt[pr * D1 + i], di = Dt[pr * D1 + i];
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const int j = g + 16 * c;
      const float wij = Wl[i * D1 + j];
      gq[c] += wij * oi;
      gd[c] += wij * di;
      gw[c] += dWl[i * D1 + j] * ei;
      gm[c] += dMl[i * D1 + j] * ei;
    }
  }
  if (p < nv) {
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const int j = g + 16 * c;
      const int64_t gi = (u * s.L + tok0 + p) * d + j;
      a.dq[gi] = gq[c];
      a.dk[gi] = kwv * gw[c] + kmv * gm[c] - gd[c];
    }
  }
}

// LDS floats of k_lin_bwd_state.
__host__ __device__ constexpr int64_t lin_bwd_state_lds_floats(int64_t d) {
  return 2 * 64 * 16 + 2 * 64 * d + 3 * 256;
}

template <int R>
__global__ __launch_bounds__(256) void k_lin_bwd_state(LinBwdArgs a) {
  constexpr int d = 16 * R;
  extern __shared__ float lsm[];
  const Shape& s = a.s;
  float* so = lsm;              // [64][16] dout, this block's rows
  float* sd = so + 64 * 16;     // [64][16] de, this block's rows
  float* sq = sd + 64 * 16;     // [64][d]
  float* sk = sq + 64 * d;      // [64][d]
  float* red = sk + 64 * d;     // [3][256]
  constexpr int nrb = R;
  const int64_t rb = blockIdx.x % nrb, u = blockIdx.x / nrb;
  const int64_t tok0 = static_cast<int64_t>(a.r) * s.C;
  const int64_t nv = n_valid(s, a.r);
  constexpr int64_t P = static_cast<int64_t>(d) * d;
  constexpr int nper = R;  // state entries per thread (16 d / 256)
  float acc[nper];
#pragma unroll
  for (int e = 0; e < nper; ++e) acc[e] = 0.0f;
  for (int64_t pb = 0; pb < s.Cp; pb += 64) {
    __syncthreads();
#pragma unroll 8
    for (int idx = threadIdx.x; idx < 64 * 16; idx += 256) {
      const int pr = idx / 16, i = idx % 16;
      const int64_t p = pb + pr;
      so[idx] = p < nv ? a.dout[(u * s.L + tok0 + p) * d + rb * 16 + i] : 0.0f;
      sd[idx] = a.de[(u * s.Cp + p) * d + rb * 16 + i];
    }
#pragma unroll 8
    for (int idx = threadIdx.x; idx < 64 * d; idx += 256) {
      const int pr = idx / d, c = idx % d;
      const int64_t p = pb + pr;
      const bool ok = p < nv;
      sq[idx] = ok ? a.q[(u * s.L + tok0 + p) * d + c] : 0.0f;
      sk[idx] = ok ? a.k[(u * s.L + tok0 + p) * d + c] : 0.0f;
    }
    __syncthreads();
    float t[nper];
#pragma unroll
    for (int e = 0; e < nper; ++e) t[e] = 0.0f;
#pragma unroll 16
    for (int pr = 0; pr < 64; ++pr) {
#pragma unroll
      for (int e = 0; e < nper; ++e) {
        const int ent = threadIdx.x + 256 * e;
        const int i = ent / d, j = ent % d;
        t[e] += so[pr * 16 + i] * sq[pr * d + j] - sd[pr * 16 + i] * sk[pr * d + j];
      }
    }
#pragma unroll
    for (int e = 0; e < nper; ++e) acc[e] += t[e];
  }
  const float* cf = a.coef + (u * s.nC + a.r) * 4;
  const float cW = cf[0], cM = cf[1], cWM = cf[2];
  float pw = 0.0f, pm = 0.0f, pwm = 0.0f;
#pragma unroll
  for (int e = 0; e < nper; ++e) {
    const int ent = threadIdx.x + 256 * e;
    const int64_t off = u * P + (rb * 16 + ent / d) * d + ent % d;
    const float gW = a.dWC[off], gM = a.dMC[off], w0 = a.Ws[off], m0 = a.Ms[off];
    a.dWp[off] = cW * gW + acc[e];
    a.dMp[off] = cWM * gW + cM * gM;
    pw += gW * w0;
    pm += gM * m0;
    pwm += gW * m0;
  }
  red[threadIdx.x] = pw;
  red[256 + threadIdx.x] = pm;
  red[512 + threadIdx.x] = pwm;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w)
#pragma unroll
      for (int q = 0; q < 3; ++q) red[q * 256 + threadIdx.x] += red[q * 256 + threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x < 3)
    a.dots[((u * s.nC + a.r) * nrb + rb) * 4 + threadIdx.x] = red[threadIdx.x * 256];
}

// ---------------------------------------------------------------------------
// Reverse mode of the scalar scan for one segment (tokens i = 0 .. n-1 of a
// chunk), one wave.  Forward quantities (App. A.2; K^W_i = eta_i P_i,
// K^M_i = eta_i b_i):
//   b_i = prod_{s>i} beta_s,  c_i = prod_{s>i} gamma_s,
//   P_i = c_i + beta_{i+1} P_{i+1} (P_{n-1} = 1),
//   cW = gamma_0 c_0,  cM = beta_0 b_0,  cWM = beta_0 P_0,
// recomputed here in fp64 as the suffix scan of the linear maps
// T_j: (b, c, P) -> (beta_j b, gamma_j c, gamma_j c + beta_j P).  Their
// adjoints, with seeds Pbar_i = eta_i dK^W_i, bbar_i = eta_i dK^M_i (and the
// chunk coefficients' terms at i = 0), run forward in token order:
//   TP_i = Pbar_i + beta_i TP_{i-1},  Tb_i = bbar_i + beta_i Tb_{i-1},
//   Tc_i = TP_i + gamma_i Tc_{i-1}    (TP_{-1} = Tb_{-1} = Tc_{-1} = 0),
// and give dbeta_i = TP_{i-1} P_i + Tb_{i-1} b_i, dgamma_i = Tc_{i-1} c_i for
// i >= 1, dbeta_0 = dcM b_0 + dcWM P_0, dgamma_0 = dcW c_0.  Each recurrence
// is an affine map per token; lanes take contiguous token runs, compose them,
// and exchange carries by a wave scan.
struct AffD {  // x -> a x + s
  double a, s;
};
__device__ __forceinline__ AffD aff_after(const AffD& f, const AffD& g) {  // g after f
  return AffD{g.a * f.a, g.a * f.s + g.s};
}

__global__ __launch_bounds__(64) void k_lin_bwd_scalars(Shape s, int mode, const float* __restrict__ eta,
                                                        const float* __restrict__ alpha,
                                                        const float* __restrict__ beta,
                                                        const float* __restrict__ sw,
                                                        const float* __restrict__ sm,
                                                        const float* __restrict__ dots,
                                                        int nrb, int averaged, double* bcp,
                                                        float* deta, float* dalpha,
                                                        float* dbeta) {
  const int64_t seg = blockIdx.x;
  const int64_t u = seg / s.nC;
  const int r = static_cast<int>(seg % s.nC);
  const int64_t n = n_valid(s, r);
  const int64_t t0 = u * s.L + static_cast<int64_t>(r) * s.C;
  const int lane = threadIdx.x;
  const int64_t tpl = (n + 63) / 64;
  const int64_t lo = lane * tpl, hi = (lo + tpl < n ? lo + tpl : n);  // [lo, hi)
  double* B3 = bcp + seg * s.Cp * 3;
  if (averaged == 2) {
    // The LaCT rule: K^W = K^M = eta and (cW, cM, cWM) = (mean gamma, mean
    // beta, mean beta), so deta = dK^W + dK^M directly, and every token's
    // beta and gamma get 1/n of the adjoints of the means (gamma through
    // Eq. 14 as below).
    double dcW = 0.0, dcM = 0.0, dcWM = 0.0;
    for (int rb = 0; rb < nrb; ++rb) {
      dcW += dots[(seg * nrb + rb) * 4 + 0];
      dcM += dots[(seg * nrb + rb) * 4 + 1];
      dcWM += dots[(seg * nrb + rb) * 4 + 2];
    }
    const double inv_n = 1.0 / static_cast<double>(n > 0 ? n : 1);
    const double dgb = dcW * inv_n, dbb = (dcM + dcWM) * inv_n;
    for (int64_t i = lo; i < hi; ++i) {
      const double e = eta[t0 + i];
      double det = static_cast<double>(sw[seg * s.Cp + i]) + static_cast<double>(sm[seg * s.Cp + i]);
      double dal;
      if (mode == 0) {
        det -= static_cast<double>(alpha[t0 + i]) * dgb;
        dal = -e * dgb;
      } else {
        dal = dgb;
      }
      deta[t0 + i] = static_cast<float>(det);
      dalpha[t0 + i] = static_cast<float>(dal);
      dbeta[t0 + i] = static_cast<float>(dbb);
    }
    return;
  }
  auto gam_tok = [&](int64_t i) -> double {
    const double e = eta[t0 + i], al = alpha[t0 + i];
    return mode == 0 ? 1.0 - e * al : al;
  };
  // Chunk-averaged variant: every token uses the segment means (summed by the
  // wave in a fixed order).
  double mbeta = 0.0, mgam = 0.0;
  if (averaged) {
    double sb = 0.0, sg = 0.0;
    for (int64_t i = lo; i < hi; ++i) {
      sb += beta[t0 + i];
      sg += gam_tok(i);
    }
    for (int off = 32; off >= 1; off >>= 1) {
      sb += __shfl_xor(sb, off, 64);
      sg += __shfl_xor(sg, off, 64);
    }
    mbeta = sb / static_cast<double>(n);
    mgam = sg / static_cast<double>(n);
  }
  auto bet = [&](int64_t i) -> double {
    return averaged ? mbeta : static_cast<double>(beta[t0 + i]);
  };
  auto gam = [&](int64_t i) -> double { return averaged ? mgam : gam_tok(i); };
  // Suffix scan of the maps T_j, j = 1 .. n-1 (B, G, Z): (b, c, P) ->
  // (B b, G c, Z c + B P); F after E = (B_F B_E, G_F G_E, Z_F G_E + B_F Z_E).
  double mB = 1.0, mG = 1.0, mZ = 0.0;  // this lane's composition, T_lo after ... after T_hi-1
  for (int64_t j = hi - 1; j >= lo; --j) {
    if (j < 1) continue;
    const double bj = bet(j), gj = gam(j);
    // (T_j after current): current applied first
    const double nB = bj * mB, nG = gj * mG, nZ = gj * mG + bj * mZ;
    mB = nB; mG = nG; mZ = nZ;
  }
  // Inclusive suffix over lanes: S_l = A_l after... applied to later lanes
  // first: S_l = A_l o A_{l+1} o ... (A_{l+1} applied first).
  double sB = mB, sG = mG, sZ = mZ;
  for (int off = 1; off < 64; off <<= 1) {
    const double oB = __shfl_down(sB, off), oG = __shfl_down(sG, off), oZ = __shfl_down(sZ, off);
    if (lane + off < 64) {
      // (this after other): other applied first
      const double nB = sB * oB, nG = sG * oG, nZ = sZ * oG + sB * oZ;
      sB = nB; sG = nG; sZ = nZ;
    }
  }
  // Exclusive: the maps of the later lanes, applied to (1, 1, 1).
  double xB = __shfl_down(sB, 1), xG = __shfl_down(sG, 1), xZ = __shfl_down(sZ, 1);
  if (lane == 63) { xB = 1.0; xG = 1.0; xZ = 0.0; }
  double vb = xB, vc = xG, vP = xZ + xB;  // v at index hi-1
  for (int64_t i = hi - 1; i >= lo; --i) {
    B3[3 * i] = vb;
    B3[3 * i + 1] = vc;
    B3[3 * i + 2] = vP;
    if (i >= 1) {  // v_{i-1} = T_i(v_i)
      const double bi = bet(i), gi = gam(i);
      const double nb = bi * vb, nc = gi * vc, nP = gi * vc + bi * vP;
      vb = nb; vc = nc; vP = nP;
    }
  }
  __syncthreads();  // every lane's b, c, P written (read back below across lanes)
  // Chunk-coefficient adjoints: block partials added in block order.
  double dcW = 0.0, dcM = 0.0, dcWM = 0.0;
  for (int rb = 0; rb < nrb; ++rb) {
    dcW += dots[(seg * nrb + rb) * 4 + 0];
    dcM += dots[(seg * nrb + rb) * 4 + 1];
    dcWM += dots[(seg * nrb + rb) * 4 + 2];
  }
  const double b0 = B3[0], c0 = B3[1], P0 = B3[2];
  const double beta0 = bet(0), gamma0 = gam(0);
  auto seedP = [&](int64_t i) -> double {
    double v = static_cast<double>(eta[t0 + i]) * sw[seg * s.Cp + i];
    if (i == 0) v += dcWM * beta0;
    return v;
  };
  auto seedb = [&](int64_t i) -> double {
    double v = static_cast<double>(eta[t0 + i]) * sm[seg * s.Cp + i];
    if (i == 0) v += dcM * beta0;
    return v;
  };
  // Pass 1: prefix carries of TP and Tb (multiplier beta_i).
  AffD fP{1.0, 0.0}, fb{1.0, 0.0};
  for (int64_t i = lo; i < hi; ++i) {
    const double bi = bet(i);
    fP = aff_after(fP, AffD{bi, seedP(i)});
    fb = aff_after(fb, AffD{bi, seedb(i)});
  }
  auto prefix = [&](AffD f) -> double {  // value of the recurrence before this lane's run
    for (int off = 1; off < 64; off <<= 1) {
      const double oa = __shfl_up(f.a, off), os = __shfl_up(f.s, off);
      if (lane >= off) f = aff_after(AffD{oa, os}, f);
    }
    const double carry = __shfl_up(f.s, 1);
    return lane == 0 ? 0.0 : carry;
  };
  const double cP = prefix(fP), cb = prefix(fb);
  // Pass 2: the Tc carries (seed TP_i, plus dcW gamma_0 at i = 0).
  AffD fc{1.0, 0.0};
  {
    double TP = cP;
    for (int64_t i = lo; i < hi; ++i) {
      const double bi = bet(i);
      TP = seedP(i) + bi * TP;
      fc = aff_after(fc, AffD{gam(i), TP + (i == 0 ? dcW * gamma0 : 0.0)});
    }
  }
  const double cc = prefix(fc);
  // Pass 3: outputs.  deta has the kernels' direct term (K^W = eta P, K^M =
  // eta b) and, through Eq. 14, the decay's.
  auto write_tok = [&](int64_t i, double dbe, double dga, double P_i, double b_i) {
    const double e = eta[t0 + i];
    double det = static_cast<double>(sw[seg * s.Cp + i]) * P_i +
                 static_cast<double>(sm[seg * s.Cp + i]) * b_i;
    double dal;
    if (mode == 0) {
      det -= static_cast<double>(alpha[t0 + i]) * dga;
      dal = -e * dga;
    } else {
      dal = dga;
    }
    deta[t0 + i] = static_cast<float>(det);
    dalpha[t0 + i] = static_cast<float>(dal);
    dbeta[t0 + i] = static_cast<float>(dbe);
  };
  double sdbe = 0.0, sdga = 0.0;
  double TP = cP, Tb = cb, Tc = cc;  // values at i-1
  for (int64_t i = lo; i < hi; ++i) {
    const double bi = bet(i), gi = gam(i);
    const double b_i = B3[3 * i], c_i = B3[3 * i + 1], P_i = B3[3 * i + 2];
    double dbe, dga;
    if (i == 0) {
      dbe = dcM * b0 + dcWM * P0;
      dga = dcW * c0;
    } else {
      dbe = TP * P_i + Tb * b_i;
      dga = Tc * c_i;
    }
    if (averaged) {  // the adjoints of the two means; distributed below
      sdbe += dbe;
      sdga += dga;
    } else {
      write_tok(i, dbe, dga, P_i, b_i);
    }
    TP = seedP(i) + bi * TP;
    Tb = seedb(i) + bi * Tb;
    Tc = TP + (i == 0 ? dcW * gamma0 : 0.0) + gi * Tc;
  }
  if (averaged) {  // each token's beta and gamma enter the means with weight 1/n
    for (int off = 32; off >= 1; off >>= 1) {
      sdbe += __shfl_xor(sdbe, off, 64);
      sdga += __shfl_xor(sdga, off, 64);
    }
    const double inv_n = 1.0 / static_cast<double>(n);
    for (int64_t i = lo; i < hi; ++i)
      write_tok(i, sdbe * inv_n, sdga * inv_n, B3[3 * i + 2], B3[3 * i]);
  }
}

// dst = src, or zeros when src is null (an absent state gradient).
__global__ __launch_bounds__(256) void k_copy_or_zero(const float* __restrict__ src, float* dst,
                                                      int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.0f;
}

}  // namespace e2ttt
