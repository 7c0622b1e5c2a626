// kernels.hpp -- HIP kernels of the E2-TTT chunk forward for gfx950.
//
// Method: "Rethinking Expressivity and Efficiency in Test-Time Training"
// (E2-TTT).  Per chunk of C tokens and per (batch, head) unit:
//   scan   : the scalar kernels K^W_t, K^M_t and the carried-state factors
//            (cW, cM, cWM) from eta, alpha, beta (§3.2, App. A.2-A.3);
//   fwd13  : A1 = X W1^T, A3 = X W3^T, Z = silu(A1) * A3 for X = [K; Q]
//            at the chunk-start weights (§3, Eq. 6);
//   fwd2   : Y = Z W2^T; Q rows give the readout o_t (Eq. 6), K rows give
//            the activation gradient g_t = v_t - f(k_t) (§3.2 "one backward
//            pass", App. A.4);
//   bwd    : dZ = g W2, dA3 = dZ * silu(A1), dA1 = dZ * A3 * silu'(A1);
//   agg    : the two scaled aggregations U^T diag(K^W|K^M) X (App. A.4) and
//            the chunk-end state W_C = cW W_0 + cWM M_0 + A^W,
//            M_C = cM M_0 + A^M, which becomes the next chunk's start state.
//
// Internal layouts (per unit u, chunk-local token row p in [0, Cp), Cp = C
// rounded up to 128; rows past the chunk's valid tokens are zero inputs with
// zero kernels, so they add nothing):
//   kw, km   fp32 [BH][nC][Cp]         coef fp32 [BH][nC][4] (cW, cM, cWM, 0)
//   kt       T [BH][nC][d][Cp]         K of every chunk, feature-major
//   w13s     T [BH][2h][krep*d]        bf16/f32 shadow of W1,W3: 32-row blocks
//                                      interleaved W1,W3,W1,W3,...; with
//                                      krep = 2 columns [d, 2d) hold the low
//                                      part W - hi (compensated operands)
//   w2s      T [BH][d][krep*h]         W2 shadow;  w2ts T [BH][h][krep*d] W2^T
//   zrow     T [BH][2Cp][h]            Z of K rows then Q rows
//   a1s, a3s fp32 [BH][Cp][h]          A1, A3 of K rows (backward stash)
//   grow     T [BH][Cp][d]             g of K rows
//   ut       T [BH][4h][Cp]            K^W*dA1, K^M*dA1 (32-row interleave),
//                                      then K^W*dA3, K^M*dA3
//   gt       T [BH][2d][Cp]            K^W*g, K^M*g (32-row interleave)
//   zt       T [BH][h][Cp]             Z of K rows, feature-major
// The 32-row W/M interleave puts the W and M aggregates of one state entry
// in the same lane of the aggregation kernel's accumulators.
#pragma once
#include "common.hpp"

namespace e2ttt {

struct Shape {
  int64_t BH, L, d, h, C, Cp, nC;
  int krep;
};

__device__ __forceinline__ int64_t n_valid(const Shape& s, int r) {
  const int64_t rem = s.L - static_cast<int64_t>(r) * s.C;
  return rem < s.C ? rem : s.C;
}

// ---------------------------------------------------------------------------
// Scalar kernels (§3.2 K^M = eta*beta~, K^W = eta*beta~*R; App. A.2 log-space
// suffix products).  One workgroup of NT threads per (unit, chunk) segment of
// n <= C tokens, walked in rounds of R = NT * TPT tokens from the last round
// to the first.  Each round is staged through LDS (coalesced loads and
// stores), and thread i then takes the TPT consecutive tokens i*TPT ...: each
// token's logarithms are taken once, and the block-wide scans run once per
// TPT tokens.
//   b_t = prod_{s>t} beta_s,  c_t = prod_{s>t} gamma_s   (exclusive suffix
//        products, as exp of suffix sums of log|.| with a sign parity)
//   P_t = c_t + beta_{t+1} P_{t+1},  P_{n-1} = 1   (= beta~_t R_t, bounded)
//   K^W_t = eta_t P_t,  K^M_t = eta_t b_t,  cW = prod gamma, cM = prod beta,
//   cWM = beta_0 P_0.
// P is the suffix composition of the affine maps x -> c_t + beta_{t+1} x
// ((A1,B1) o (A2,B2) = (A1 + B1 A2, B1 B2)); the token past the segment
// has beta = 0, which ends the recursion at P_{n-1} = c_{n-1} = 1.
// Suffix sums and compositions: sequential inside a thread, then across the
// threads of a wave by shuffles, across the 4 waves through LDS (double-
// buffered by round parity), plus the carry of the later rounds (suffix log
// sums, parities, P and beta of the first token of the later round).  No
// subtraction of log sums anywhere, so the -inf of a zero factor never turns
// into NaN.  All scan arithmetic is fp64, with the logarithm and exponential
// below.  Output index of token p of chunk r of unit u is
// u*ustride + r*rstride + p; with pad > n tokens p in [n, pad) are written
// as 0.  coef of (u, r) starts at (u*nC + r)*cstride.

// Natural log of a normal positive fp64 x to about 1 ulp: x = 2^e m with
// m in [sqrt(1/2), sqrt(2)), log m = 2 atanh(s), s = (m - 1) / (m + 1),
// |s| <= 0.1716, by the odd series of atanh to s^21 (the first omitted term
// is below 1e-17 relative).  Zero gives -inf; subnormal, infinite and NaN
// inputs take the library log.
__device__ __forceinline__ double log_fast(double x) {
  if (!(x >= 2.2250738585072014e-308 && x <= 1.7976931348623157e308))
    return x == 0.0 ? -__builtin_huge_val() : log(x);
  const long long bits = __double_as_longlong(x);
  int e = static_cast<int>((bits >> 52) & 0x7ff) - 1023;
  double m = __longlong_as_double((bits & 0x000fffffffffffffLL) | 0x3ff0000000000000LL);
  if (m > 1.4142135623730951) {
    m *= 0.5;
    ++e;
  }
  const double f = m - 1.0;  // exact
  const double den = m + 1.0;
  double rc = __builtin_amdgcn_rcp(den);  // refined twice by Newton's iteration
  rc = rc * fma(-den, rc, 2.0);
  rc = rc * fma(-den, rc, 2.0);
  const double s = f * rc;
  const double z = s * s;
  double p = 1.0 / 21.0;
  p = fma(p, z, 1.0 / 19.0);
  p = fma(p, z, 1.0 / 17.0);
  p = fma(p, z, 1.0 / 15.0);
  p = fma(p, z, 1.0 / 13.0);
  p = fma(p, z, 1.0 / 11.0);
  p = fma(p, z, 1.0 / 9.0);
  p = fma(p, z, 1.0 / 7.0);
  p = fma(p, z, 1.0 / 5.0);
  p = fma(p, z, 1.0 / 3.0);
  p = fma(p, z, 1.0);
  constexpr double LN2_HI = 6.93147180369123816490e-01, LN2_LO = 1.90821492927058770002e-10;
  const double de = static_cast<double>(e);
  return fma(de, LN2_HI, fma(de, LN2_LO, 2.0 * s * p));
}

// exp of fp64 y to about 1 ulp: y = k ln2 + r, |r| <= ln2/2, exp r by its
// Taylor series to r^13 (the first omitted term is below 1e-17 relative),
// times 2^k.  Results below the normal range are returned as 0 (they vanish
// in every fp32 output); -inf gives 0, NaN stays NaN.
__device__ __forceinline__ double exp_fast(double y) {
  if (!(y > -708.0)) return y != y ? y : 0.0;
  if (y > 709.0) return exp(y);
  constexpr double LOG2E = 1.44269504088896338700e+00;
  constexpr double LN2_HI = 6.93147180369123816490e-01, LN2_LO = 1.90821492927058770002e-10;
  const double k = __builtin_rint(y * LOG2E);
  double r = fma(-k, LN2_HI, y);
  r = fma(-k, LN2_LO, r);
  double p = 1.0 / 6227020800.0;  // 1/13!
  p = fma(p, r, 1.0 / 479001600.0);
  p = fma(p, r, 1.0 / 39916800.0);
  p = fma(p, r, 1.0 / 3628800.0);
  p = fma(p, r, 1.0 / 362880.0);
  p = fma(p, r, 1.0 / 40320.0);
  p = fma(p, r, 1.0 / 5040.0);
  p = fma(p, r, 1.0 / 720.0);
  p = fma(p, r, 1.0 / 120.0);
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const long long ki = static_cast<long long>(k);
  return p * __longlong_as_double((ki + 1023) << 52);
}

struct LogSigned {  // log|x| and the sign of x (as a parity bit)
  double l;
  int neg;
};

__device__ __forceinline__ LogSigned log_signed(double x) {
  LogSigned r;
  r.neg = x < 0.0;
  r.l = log_fast(fabs(x));  // -inf for 0
  return r;
}

__device__ __forceinline__ double exp_signed(double l, int neg) {
  const double e = exp_fast(l);
  return neg ? -e : e;
}

// NT threads per workgroup, TPT tokens per thread (the host picks them from
// the chunk length so that short segments keep every thread busy).
template <int NT, int TPT>
__global__ __launch_bounds__(NT) void k_scan(const float* __restrict__ eta,
                                                  const float* __restrict__ alpha,
                                                  const float* __restrict__ beta, int64_t L,
                                                  int64_t C, int64_t nC, int mode, float* kw,
                                                  float* km, int64_t ustride, int64_t rstride,
                                                  int64_t pad, float* coef, int cstride) {
  constexpr int NW = NT / 64, R = NT * TPT;
  // Staged round: eta, alpha, beta (s_b[R] = beta of the next round's first
  // token, 0 past the segment), then K^W, K^M of the round.
  __shared__ float s_e[R], s_a[R], s_b[R + 4], s_kw[R], s_km[R];
  __shared__ double s_lb[2][NW], s_lg[2][NW], s_A[2][NW], s_B[2][NW];
  __shared__ int s_par[2][NW];
  const int64_t seg = blockIdx.x;
  const int64_t u = seg / nC;
  const int r = static_cast<int>(seg % nC);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(r) * C;
  const int64_t n = (L - t0) < C ? (L - t0) : C;
  const float* e_g = eta + u * L + t0;
  const float* a_g = alpha + u * L + t0;
  const float* b_g = beta + u * L + t0;
  float* kw_o = kw + u * ustride + r * rstride;
  float* km_o = km + u * ustride + r * rstride;
  for (int64_t i = n + tid; i < pad; i += NT) {
    kw_o[i] = 0.0f;
    km_o[i] = 0.0f;
  }

  // Carry from the later rounds.
  double cLB = 0.0, cLG = 0.0, cP = 0.0, cBeta = 0.0;
  int cPar = 0;  // bit 0: parity of beta signs, bit 1: of gamma signs
  const int64_t nr = (n + R - 1) / R;
  for (int64_t rd = nr - 1; rd >= 0; --rd) {
    const int pb = static_cast<int>(rd & 1);
    const int64_t base = rd * R;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int idx = k * NT + tid;
      const bool ok = base + idx < n;
      s_e[idx] = ok ? e_g[base + idx] : 0.0f;
      s_a[idx] = ok ? a_g[base + idx] : 0.0f;
      s_b[idx] = ok ? b_g[base + idx] : 0.0f;
    }
    if (tid == 0) s_b[R] = static_cast<float>(cBeta);  // exact: cBeta is a staged fp32
    __syncthreads();

    // This thread's tokens j0 .. j0+TPT-1 of the round.
    const int j0 = tid * TPT;
    double lb[TPT], lg[TPT];
    int par[TPT];
    float bt[TPT + 1];
    double TLB = 0.0, TLG = 0.0;
    int TPAR = 0;
#pragma unroll
    for (int j = 0; j < TPT + 1; ++j) bt[j] = s_b[j0 + j];
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      lb[j] = 0.0;
      lg[j] = 0.0;
      par[j] = 0;
      if (base + j0 + j < n) {
        const LogSigned b = log_signed(static_cast<double>(bt[j]));
        lb[j] = b.l;
        par[j] = b.neg;
        const double al = static_cast<double>(s_a[j0 + j]);
        if (mode == 1) {
          const LogSigned g = log_signed(al);
          lg[j] = g.l;
          par[j] |= g.neg << 1;
        } else {
          const double ea = static_cast<double>(s_e[j0 + j]) * al;  // exact
          lg[j] = log_fast(fabs(1.0 - ea));  // log|1 - eta*alpha|
          par[j] |= (ea > 1.0 ? 1 : 0) << 1;
        }
      }
    }
    for (int j = TPT - 1; j >= 0; --j) {  // (fixed order: same sums in every use)
      TLB += lb[j];
      TLG += lg[j];
      TPAR ^= par[j];
    }
    const double beta_first = static_cast<double>(s_b[0]);  // read before the next round restages

    // Sums over the later threads of the round: wave-level inclusive suffix,
    // then the later waves' totals, then the carry.
    double xb = TLB, xg = TLG;
    int xp = TPAR;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double yb = __shfl_down(xb, off, 64);
      const double yg = __shfl_down(xg, off, 64);
      const int yp = __shfl_down(xp, off, 64);
      if (lane + off < 64) {
        xb += yb;
        xg += yg;
        xp ^= yp;
      }
    }
    if (lane == 0) {
      s_lb[pb][w] = xb;
      s_lg[pb][w] = xg;
      s_par[pb][w] = xp;
    }
    __syncthreads();
    double eb = __shfl_down(xb, 1, 64), eg = __shfl_down(xg, 1, 64);
    int ep = __shfl_down(xp, 1, 64);
    if (lane == 63) {
      eb = 0.0;
      eg = 0.0;
      ep = 0;
    }
    double lbw = cLB, lgw = cLG;
    int pw = cPar;
    for (int v = NW - 1; v > w; --v) {
      lbw += s_lb[pb][v];
      lgw += s_lg[pb][v];
      pw ^= s_par[pb][v];
    }
    eb += lbw;
    eg += lgw;
    ep ^= pw;

    // b, c of this thread's tokens, and the thread's affine map.
    double bj[TPT], cj[TPT];
    double A = 0.0, B = 1.0;
    {
      double sb = eb, sg = eg;
      int sp = ep;
#pragma unroll
      for (int j = TPT - 1; j >= 0; --j) {
        bj[j] = exp_signed(sb, sp & 1);
        cj[j] = exp_signed(sg, (sp >> 1) & 1);
        sb += lb[j];
        sg += lg[j];
        sp ^= par[j];
        if (base + j0 + j < n) {
          const double bn = static_cast<double>(bt[j + 1]);
          A = cj[j] + bn * A;
          B = bn * B;
        }
      }
    }
    // Compositions over the later threads of the wave, then the later waves.
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double oA = __shfl_down(A, off, 64);
      const double oB = __shfl_down(B, off, 64);
      if (lane + off < 64) {
        A = A + B * oA;
        B = B * oB;
      }
    }
    if (lane == 0) {
      s_A[pb][w] = A;
      s_B[pb][w] = B;
    }
    __syncthreads();
    double x = cP, x_after_w = cP;
    for (int v = NW - 1; v >= 0; --v) {
      if (v == w) x_after_w = x;
      x = s_A[pb][v] + s_B[pb][v] * x;
    }
    double nA = __shfl_down(A, 1, 64), nB = __shfl_down(B, 1, 64);
    if (lane == 63) {
      nA = 0.0;
      nB = 1.0;
    }
    double P = nA + nB * x_after_w;  // P at the first token after this thread's
#pragma unroll
    for (int j = TPT - 1; j >= 0; --j) {
      if (base + j0 + j < n) {
        P = cj[j] + static_cast<double>(bt[j + 1]) * P;
        const double e = static_cast<double>(s_e[j0 + j]);
        s_kw[j0 + j] = static_cast<float>(e * P);
        s_km[j0 + j] = static_cast<float>(e * bj[j]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int idx = k * NT + tid;
      if (base + idx < n) {
        kw_o[base + idx] = s_kw[idx];
        km_o[base + idx] = s_km[idx];
      }
    }
    // Carry into the earlier round (every thread adds the same totals in the
    // same order).
    for (int v = w; v >= 0; --v) {  // the later waves were added above
      lbw += s_lb[pb][v];
      lgw += s_lg[pb][v];
      pw ^= s_par[pb][v];
    }
    cLB = lbw;
    cLG = lgw;
    cPar = pw;
    cP = x;
    cBeta = beta_first;
  }
  if (tid == 0 && n > 0) {
    float* cf = coef + (u * nC + r) * cstride;
    cf[0] = static_cast<float>(exp_signed(cLG, (cPar >> 1) & 1));
    cf[1] = static_cast<float>(exp_signed(cLB, cPar & 1));
    cf[2] = static_cast<float>(cBeta * cP);
  }
}

// ---------------------------------------------------------------------------
// K of every chunk, feature-major: kt[u][r][c][p'] = k[u][r*C + p][c] (zero
// for rows past the chunk's valid tokens).  With PERM, the token position p'
// is permuted inside each group of 32 tokens so that the 8 tokens one lane
// feeds to a 16x16x32 MFMA (tokens 4g..4g+3 and 16+4g..16+4g+3 of the group)
// are contiguous: p' = 8*((p%16)/4) + 4*((p%32)/16) + p%4.  64x64 tiles
// through LDS, all global accesses 16-byte vectors.
__host__ __device__ constexpr int tok_perm32(int p) {
  return (p & ~31) + 8 * ((p & 15) >> 2) + 4 * ((p & 31) >> 4) + (p & 3);
}

template <typename T, bool PERM>
__global__ __launch_bounds__(256) void k_prep_kt(Shape s, const T* __restrict__ k,
                                                 T* __restrict__ kt) {
  constexpr int VE = 16 / sizeof(T);            // elements per 16-byte vector
  constexpr int NV = 64 * 64 / VE;              // vectors per 64x64 tile
  constexpr int PER = NV / 256;
  __shared__ T tile[64][64 + 1];
  const int64_t ptiles = s.Cp / 64, ctiles = s.d / 64;
  int64_t bid = blockIdx.x;
  const int64_t ct = bid % ctiles; bid /= ctiles;
  const int64_t pt = bid % ptiles; bid /= ptiles;
  const int r = static_cast<int>(bid % s.nC);
  const int64_t u = bid / s.nC;
  const int64_t nv = n_valid(s, r);
  const T* ks = k + (u * s.L + static_cast<int64_t>(r) * s.C) * s.d + ct * 64;
  uint4 reg[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {  // 64 token rows x (64 / VE) vectors
    const int idx = threadIdx.x + 256 * i;
    const int pr = idx / (64 / VE), cv = idx % (64 / VE);
    const int64_t p = pt * 64 + pr;
    const uint4 val = *reinterpret_cast<const uint4*>(ks + (p < nv ? p : 0) * s.d + cv * VE);
    reg[i] = p < nv ? val : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = threadIdx.x + 256 * i;
    const int pr = idx / (64 / VE), cv = idx % (64 / VE);
    const int pos = PERM ? tok_perm32(pr) : pr;
    const T* e = reinterpret_cast<const T*>(&reg[i]);
#pragma unroll
    for (int x = 0; x < VE; ++x) tile[cv * VE + x][pos] = e[x];
  }
  __syncthreads();
  T* dst = kt + ((u * s.nC + r) * s.d + ct * 64) * s.Cp + pt * 64;
#pragma unroll
  for (int i = 0; i < PER; ++i) {  // 64 feature rows x (64 / VE) vectors
    const int idx = threadIdx.x + 256 * i;
    const int cr = idx / (64 / VE), pv = idx % (64 / VE);
    T vals[VE];
#pragma unroll
    for (int x = 0; x < VE; ++x) vals[x] = tile[cr][pv * VE + x];
    *reinterpret_cast<uint4*>(dst + cr * s.Cp + pv * VE) = *reinterpret_cast<const uint4*>(vals);
  }
}

// Hi/lo split of a state value into the operand type.
template <typename T>
__device__ __forceinline__ void split_store(float w, T* hi, T* lo) {
  const T h = from_f32<T>(w);
  *hi = h;
  if (lo) *lo = from_f32<T>(w - to_f32<T>(h));
}

// Operand shadows of one state entry (unit u, packed offset o).
template <typename T>
__device__ __forceinline__ void write_shadow(const Shape& s, int64_t u, int64_t o, float w,
                                             T* w13s, T* w2s, T* w2ts) {
  const int64_t d = s.d, h = s.h, kr = s.krep;
  const int64_t hd = h * d;
  if (o < 2 * hd) {
    const int isW3 = o >= hd;
    const int64_t oo = isW3 ? o - hd : o;
    const int64_t sr = oo / d, c = oo % d;
    const int64_t srow = 64 * (sr / 32) + (isW3 ? 32 : 0) + sr % 32;
    T* base = w13s + (u * 2 * h + srow) * (kr * d);
    split_store<T>(w, base + c, kr == 2 ? base + d + c : nullptr);
  } else {
    const int64_t oo = o - 2 * hd;
    const int64_t i = oo / h, j = oo % h;
    T* b2 = w2s + (u * d + i) * (kr * h);
    split_store<T>(w, b2 + j, kr == 2 ? b2 + h + j : nullptr);
    T* bt = w2ts + (u * h + j) * (kr * d);
    split_store<T>(w, bt + i, kr == 2 ? bt + d + i : nullptr);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_prep_shadow(Shape s, const float* __restrict__ W,
                                                     T* w13s, T* w2s, T* w2ts) {
  const int64_t P = 3 * s.d * s.h;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= s.BH * P) return;
  const int64_t u = idx / P, o = idx % P;
  write_shadow<T>(s, u, o, W[idx], w13s, w2s, w2ts);
}

// ---------------------------------------------------------------------------
// fwd13: [K;Q] rows x shadow W13 -> A1, A3 -> Z.
template <typename T>
__global__ __launch_bounds__(256) void k_fwd13(Shape s, int r, const T* __restrict__ q,
                                               const T* __restrict__ k, const T* __restrict__ w13s,
                                               T* zrow, float* a1s, float* a3s, T* zt) {
  __shared__ __attribute__((aligned(16))) T lds[Tile<T>::LDS_BYTES / sizeof(T)];
  const int64_t ntn = 2 * s.h / 128, ntm = 2 * s.Cp / 128, mtK = s.Cp / 128;
  int64_t bid = blockIdx.x;
  const int64_t nt = bid % ntn; bid /= ntn;
  const int64_t mt = bid % ntm;
  const int64_t u = bid / ntm;
  const bool isQ = mt >= mtK;
  const int64_t p0 = (mt - (isQ ? mtK : 0)) * 128;
  const int64_t tok0 = static_cast<int64_t>(r) * s.C;
  const int64_t nv = n_valid(s, r);
  const T* X = (isQ ? q : k) + (u * s.L + tok0) * s.d;
  RowLoader<T> la, lb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t p = p0 + loader_row(i);
    la.rowp[i] = p < nv ? X + p * s.d : nullptr;
    lb.rowp[i] = w13s + (u * 2 * s.h + nt * 128 + loader_row(i)) * (s.krep * s.d);
  }
  f32x16_t acc[2][2];
  gemm_tile<T>(acc, la, lb, s.krep * s.d, s.d, lds);

  const AccPos ps;
  const int64_t j = nt * 64 + ps.wn * 32 + ps.r32;  // hidden unit of this lane
  float zv[2][2][16];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t p = p0 + ps.row(mi, v);
      const float a1 = acc[mi][0][v], a3 = acc[mi][1][v];
      const float z = a1 * sigmoidf_(a1) * a3;
      zv[mi][0][v] = z;
      zrow[(u * 2 * s.Cp + (isQ ? s.Cp : 0) + p) * s.h + j] = from_f32<T>(z);
      if (!isQ) {
        a1s[(u * s.Cp + p) * s.h + j] = a1;
        a3s[(u * s.Cp + p) * s.h + j] = a3;
      }
    }
  if (!isQ) {
    // Z^T tile (64 hidden rows x 128 tokens) through LDS.
    constexpr int VE = Tile<T>::VE, W = 128 + VE;
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        lds[(ps.wn * 32 + ps.r32) * W + ps.row(mi, v)] = from_f32<T>(zv[mi][0][v]);
    __syncthreads();
    T* dst = zt + (u * s.h + nt * 64) * s.Cp + p0;
    constexpr int VPR = 128 / VE;
    for (int idx = threadIdx.x; idx < 64 * VPR; idx += 256) {
      const int rr = idx / VPR, c = idx % VPR;
      *reinterpret_cast<uint4*>(dst + rr * s.Cp + c * VE) =
          *reinterpret_cast<const uint4*>(lds + rr * W + c * VE);
    }
  }
}

// Transposed store of a 128x128 accumulator-layout tile whose column c goes
// to destination row dst_row(c) (row-contiguous along the tile's rows).
template <typename T, typename RowFn>
__device__ __forceinline__ void store_T(const float (&val)[2][2][16], T* lds, RowFn dst_row) {
  constexpr int VE = Tile<T>::VE, W = 128 + VE, VPR = 128 / VE;
  const AccPos ps;
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        lds[ps.col(ni) * W + ps.row(mi, v)] = from_f32<T>(val[mi][ni][v]);
  __syncthreads();
  for (int idx = threadIdx.x; idx < 128 * VPR; idx += 256) {
    const int rr = idx / VPR, c = idx % VPR;
    *reinterpret_cast<uint4*>(dst_row(rr) + c * VE) =
        *reinterpret_cast<const uint4*>(lds + rr * W + c * VE);
  }
}

// fwd2: Z x W2^T -> Y; readout for Q rows, g = v - Y for K rows.
template <typename T>
__global__ __launch_bounds__(256) void k_fwd2(Shape s, int r, const T* __restrict__ v,
                                              T* out, const T* __restrict__ zrow,
                                              const T* __restrict__ w2s,
                                              const float* __restrict__ kw,
                                              const float* __restrict__ km, T* grow, T* gt) {
  __shared__ __attribute__((aligned(16))) T lds[Tile<T>::LDS_BYTES / sizeof(T)];
  const int64_t ntn = s.d / 128, ntm = 2 * s.Cp / 128, mtK = s.Cp / 128;
  int64_t bid = blockIdx.x;
  const int64_t nt = bid % ntn; bid /= ntn;
  const int64_t mt = bid % ntm;
  const int64_t u = bid / ntm;
  const bool isQ = mt >= mtK;
  const int64_t p0 = (mt - (isQ ? mtK : 0)) * 128;
  const int64_t tok0 = static_cast<int64_t>(r) * s.C;
  const int64_t nv = n_valid(s, r);
  RowLoader<T> la, lb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    la.rowp[i] = zrow + (u * 2 * s.Cp + mt * 128 + loader_row(i)) * s.h;
    lb.rowp[i] = w2s + (u * s.d + nt * 128 + loader_row(i)) * (s.krep * s.h);
  }
  f32x16_t acc[2][2];
  gemm_tile<T>(acc, la, lb, s.krep * s.h, s.h, lds);

  const AccPos ps;
  if (isQ) {
    T* o = out + (u * s.L + tok0) * s.d;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
          const int64_t p = p0 + ps.row(mi, vv);
          if (p < nv) o[p * s.d + nt * 128 + ps.col(ni)] = from_f32<T>(acc[mi][ni][vv]);
        }
    return;
  }
  const T* vs = v + (u * s.L + tok0) * s.d;
  const float* kwr = kw + (u * s.nC + r) * s.Cp;
  const float* kmr = km + (u * s.nC + r) * s.Cp;
  // Loads first (v, kernels), then the stores: grow may alias v as far as the
  // compiler knows, so interleaving would serialise every element.
  float gW[2][2][16], gM[2][2][16];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int64_t p = p0 + ps.row(mi, vv);
        const int64_t i = nt * 128 + ps.col(ni);
        gW[mi][ni][vv] = p < nv ? to_f32<T>(vs[p * s.d + i]) : 0.0f;
      }
  float kwv[2][16], kmv[2][16];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) {
      kwv[mi][vv] = kwr[p0 + ps.row(mi, vv)];
      kmv[mi][vv] = kmr[p0 + ps.row(mi, vv)];
    }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int64_t p = p0 + ps.row(mi, vv);
        const int64_t i = nt * 128 + ps.col(ni);
        const float g = gW[mi][ni][vv] - acc[mi][ni][vv];
        grow[(u * s.Cp + p) * s.d + i] = from_f32<T>(g);
        gW[mi][ni][vv] = kwv[mi][vv] * g;
        gM[mi][ni][vv] = kmv[mi][vv] * g;
      }
  // gt row of d-index i: 64*(i/32) + i%32 (+32 for the momentum copy)
  T* gbase = gt + u * 2 * s.d * s.Cp + p0;
  store_T<T>(gW, lds, [&](int c) {
    const int64_t i = nt * 128 + c;
    return gbase + (64 * (i / 32) + i % 32) * s.Cp;
  });
  store_T<T>(gM, lds, [&](int c) {
    const int64_t i = nt * 128 + c;
    return gbase + (64 * (i / 32) + 32 + i % 32) * s.Cp;
  });
}

// bwd: g x W2 -> dZ -> dA1, dA3, scaled by both kernels, feature-major.
template <typename T>
__global__ __launch_bounds__(256) void k_bwd(Shape s, int r, const T* __restrict__ grow,
                                             const T* __restrict__ w2ts,
                                             const float* __restrict__ a1s,
                                             const float* __restrict__ a3s,
                                             const float* __restrict__ kw,
                                             const float* __restrict__ km, T* ut) {
  __shared__ __attribute__((aligned(16))) T lds[Tile<T>::LDS_BYTES / sizeof(T)];
  const int64_t ntn = s.h / 128, ntm = s.Cp / 128;
  int64_t bid = blockIdx.x;
  const int64_t nt = bid % ntn; bid /= ntn;
  const int64_t mt = bid % ntm;
  const int64_t u = bid / ntm;
  const int64_t p0 = mt * 128;
  RowLoader<T> la, lb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    la.rowp[i] = grow + (u * s.Cp + p0 + loader_row(i)) * s.d;
    lb.rowp[i] = w2ts + (u * s.h + nt * 128 + loader_row(i)) * (s.krep * s.d);
  }
  f32x16_t acc[2][2];
  gemm_tile<T>(acc, la, lb, s.krep * s.d, s.d, lds);

  const AccPos ps;
  const float* kwr = kw + (u * s.nC + r) * s.Cp;
  const float* kmr = km + (u * s.nC + r) * s.Cp;
  float d1[2][2][16], d3[2][2][16];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int64_t p = p0 + ps.row(mi, vv);
        const int64_t j = nt * 128 + ps.col(ni);
        const float a1 = a1s[(u * s.Cp + p) * s.h + j];
        const float a3 = a3s[(u * s.Cp + p) * s.h + j];
        const float sg = sigmoidf_(a1);
        const float dz = acc[mi][ni][vv];
        d3[mi][ni][vv] = dz * (a1 * sg);
        d1[mi][ni][vv] = dz * a3 * (sg * (1.0f + a1 * (1.0f - sg)));
      }
  T* ubase = ut + u * 4 * s.h * s.Cp + p0;
  float sc[2][2][16];
  for (int which = 0; which < 4; ++which) {
    const bool isM = which & 1;
    const bool isA3 = which >= 2;
    const float* kr = isM ? kmr : kwr;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv)
          sc[mi][ni][vv] = kr[p0 + ps.row(mi, vv)] * (isA3 ? d3[mi][ni][vv] : d1[mi][ni][vv]);
    store_T<T>(sc, lds, [&](int c) {
      const int64_t j = nt * 128 + c;
      return ubase + ((isA3 ? 2 * s.h : 0) + 64 * (j / 32) + (isM ? 32 : 0) + j % 32) * s.Cp;
    });
  }
}

// agg: both scaled aggregations over the chunk's tokens + chunk-end state.
template <typename T>
__global__ __launch_bounds__(256) void k_agg(Shape s, int r, int last, const T* __restrict__ ut,
                                             const T* __restrict__ kt, const T* __restrict__ gt,
                                             const T* __restrict__ zt,
                                             const float* __restrict__ coef, const float* Win,
                                             const float* Min, float* Wout, float* Mout, T* w13s,
                                             T* w2s, T* w2ts) {
  __shared__ __attribute__((aligned(16))) T lds[Tile<T>::LDS_BYTES / sizeof(T)];
  const int64_t d = s.d, h = s.h;
  const int64_t na = (4 * h / 128) * (d / 128), nb = (2 * d / 128) * (h / 128);
  const int64_t u = blockIdx.x / (na + nb);
  const int64_t t = blockIdx.x % (na + nb);
  const bool famA = t < na;
  int64_t mt, nt;
  RowLoader<T> la, lb;
  if (famA) {
    mt = t / (d / 128); nt = t % (d / 128);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      la.rowp[i] = ut + (u * 4 * h + mt * 128 + loader_row(i)) * s.Cp;
      lb.rowp[i] = kt + ((u * s.nC + r) * d + nt * 128 + loader_row(i)) * s.Cp;
    }
  } else {
    const int64_t tb = t - na;
    mt = tb / (h / 128); nt = tb % (h / 128);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      la.rowp[i] = gt + (u * 2 * d + mt * 128 + loader_row(i)) * s.Cp;
      lb.rowp[i] = zt + (u * h + nt * 128 + loader_row(i)) * s.Cp;
    }
  }
  f32x16_t acc[2][2];
  gemm_tile<T>(acc, la, lb, s.Cp, s.Cp, lds);

  const float* cf = coef + (u * s.nC + r) * 4;
  const float cW = cf[0], cM = cf[1], cWM = cf[2];
  const int64_t P = 3 * d * h;
  const float* wi = Win + u * P;
  const float* mi_ = Min + u * P;
  float* wo = Wout + u * P;
  float* mo = Mout + u * P;
  const AccPos ps;
  const int64_t blk64 = mt * 2 + ps.wm;  // 64-row block: rows 0-31 W part, 32-63 M part
  // Offsets and start values first, then the stores (W_end may be W_0).
  int64_t offs[2][16];
  float w0v[2][16], m0v[2][16];
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) {
      const int64_t idx32 = 8 * (vv >> 2) + 4 * ps.hf + (vv & 3);
      int64_t off;
      if (famA) {
        const int64_t c = nt * 128 + ps.col(ni);
        if (blk64 < h / 32) off = (blk64 * 32 + idx32) * d + c;
        else off = h * d + ((blk64 - h / 32) * 32 + idx32) * d + c;
      } else {
        const int64_t i = blk64 * 32 + idx32;
        const int64_t j = nt * 128 + ps.col(ni);
        off = 2 * h * d + i * h + j;
      }
      offs[ni][vv] = off;
      w0v[ni][vv] = wi[off];
      m0v[ni][vv] = mi_[off];
    }
#pragma unroll
  for (int ni = 0; ni < 2; ++ni)
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) {
      const int64_t off = offs[ni][vv];
      const float wn = cW * w0v[ni][vv] + cWM * m0v[ni][vv] + acc[0][ni][vv];
      const float mn = cM * m0v[ni][vv] + acc[1][ni][vv];
      wo[off] = wn;
      mo[off] = mn;
      if (!last) write_shadow<T>(s, u, off, wn, w13s, w2s, w2ts);
    }
}

// ---------------------------------------------------------------------------
// Linear learner f_W(x) = W x (fp32 arithmetic; io fp32 or bf16).
// fwd: Y = X W^T for X = [K; Q] rows of chunk r; readout or scaled residuals
// gw = K^W g, gm = K^M g with g = v - W k (fp32, [BH][Cp][d]).
template <typename IO>
__global__ __launch_bounds__(256) void k_lin_fwd(Shape s, int r, const IO* __restrict__ q,
                                                 const IO* __restrict__ k,
                                                 const IO* __restrict__ v,
                                                 const float* __restrict__ Wst,
                                                 const float* __restrict__ kw,
                                                 const float* __restrict__ km, IO* out,
                                                 float* gw, float* gm) {
  extern __shared__ float lsm[];
  const int64_t d = s.d;
  float* Ws = lsm;                 // [d][d+1]
  float* Xs = lsm + d * (d + 1);   // [64][d+1]
  const int64_t ntm = 2 * s.Cp / 64, mtK = s.Cp / 64;
  const int64_t mt = blockIdx.x % ntm, u = blockIdx.x / ntm;
  const bool isQ = mt >= mtK;
  const int64_t p0 = (mt - (isQ ? mtK : 0)) * 64;
  const int64_t tok0 = static_cast<int64_t>(r) * s.C;
  const int64_t nv = n_valid(s, r);
  const IO* X = (isQ ? q : k) + (u * s.L + tok0) * d;
  for (int64_t idx = threadIdx.x; idx < d * d; idx += 256)
    Ws[(idx / d) * (d + 1) + idx % d] = Wst[u * d * d + idx];
  for (int64_t idx = threadIdx.x; idx < 64 * d; idx += 256) {
    const int64_t pr = idx / d, c = idx % d, p = p0 + pr;
    Xs[pr * (d + 1) + c] = p < nv ? to_f32<IO>(X[p * d + c]) : 0.0f;
  }
  __syncthreads();
  const float* kwr = kw + (u * s.nC + r) * s.Cp;
  const float* kmr = km + (u * s.nC + r) * s.Cp;
  for (int64_t idx = threadIdx.x; idx < 64 * d; idx += 256) {
    const int64_t pr = idx / d, c = idx % d, p = p0 + pr;
    float y = 0.0f;
    for (int64_t kk = 0; kk < d; ++kk) y += Xs[pr * (d + 1) + kk] * Ws[c * (d + 1) + kk];
    if (isQ) {
      if (p < nv) out[(u * s.L + tok0 + p) * d + c] = from_f32<IO>(y);
    } else {
      const float vin = p < nv ? to_f32<IO>(v[(u * s.L + tok0 + p) * d + c]) : 0.0f;
      const float g = vin - y;
      gw[(u * s.Cp + p) * d + c] = kwr[p] * g;
      gm[(u * s.Cp + p) * d + c] = kmr[p] * g;
    }
  }
}

// agg: A^W = gw^T K, A^M = gm^T K over the chunk; chunk-end state.
template <typename IO>
__global__ __launch_bounds__(256) void k_lin_agg(Shape s, int r, const IO* __restrict__ k,
                                                 const float* __restrict__ gw,
                                                 const float* __restrict__ gm,
                                                 const float* __restrict__ coef,
                                                 const float* Win, const float* Min, float* Wout,
                                                 float* Mout) {
  extern __shared__ float lsm[];
  const int64_t d = s.d;
  float* sw = lsm;              // [64][16]
  float* smm = lsm + 64 * 16;   // [64][16]
  float* sk = lsm + 2 * 64 * 16;  // [64][d]
  const int64_t nrb = d / 16;
  const int64_t rb = blockIdx.x % nrb, u = blockIdx.x / nrb;
  const int64_t tok0 = static_cast<int64_t>(r) * s.C;
  const int64_t nv = n_valid(s, r);
  const int nper = static_cast<int>(d / 16);  // entries per thread (16*d / 256)
  float aw[8], am[8];
  for (int e = 0; e < 8; ++e) { aw[e] = 0.0f; am[e] = 0.0f; }
  for (int64_t pb = 0; pb < s.Cp; pb += 64) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < 64 * 16; idx += 256) {
      const int64_t pr = idx / 16, i = idx % 16;
      sw[idx] = gw[(u * s.Cp + pb + pr) * d + rb * 16 + i];
      smm[idx] = gm[(u * s.Cp + pb + pr) * d + rb * 16 + i];
    }
    for (int64_t idx = threadIdx.x; idx < 64 * d; idx += 256) {
      const int64_t pr = idx / d, c = idx % d, p = pb + pr;
      sk[idx] = p < nv ? to_f32<IO>(k[(u * s.L + tok0 + p) * d + c]) : 0.0f;
    }
    __syncthreads();
    for (int e = 0; e < nper; ++e) {
      const int64_t ent = threadIdx.x + 256 * e;
      const int64_t i = ent / d, j = ent % d;
      float sW = 0.0f, sM = 0.0f;
      for (int pr = 0; pr < 64; ++pr) {
        const float kv = sk[pr * d + j];
        sW += sw[pr * 16 + i] * kv;
        sM += smm[pr * 16 + i] * kv;
      }
      aw[e] += sW;
      am[e] += sM;
    }
  }
  const float* cf = coef + (u * s.nC + r) * 4;
  const float cW = cf[0], cM = cf[1], cWM = cf[2];
  for (int e = 0; e < nper; ++e) {
    const int64_t ent = threadIdx.x + 256 * e;
    const int64_t off = u * d * d + (rb * 16 + ent / d) * d + ent % d;
    const float w0 = Win[off], m0 = Min[off];
    Wout[off] = cW * w0 + cWM * m0 + aw[e];
    Mout[off] = cM * m0 + am[e];
  }
}

__global__ __launch_bounds__(256) void k_copy2(const float* __restrict__ a,
                                               const float* __restrict__ b, float* ao, float* bo,
                                               int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) {
    ao[i] = a[i];
    bo[i] = b[i];
  }
}

}  // namespace e2ttt
