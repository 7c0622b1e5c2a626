// decode.hpp -- one token of the fast-weight recurrence for every (b, h)
// unit: the streaming / decode use of the method of "Rethinking
// Expressivity and Efficiency in Test-Time Training" (E2-TTT).
//
// Within a chunk the readout uses the chunk-start weights W_0 (Eq. 6, §3.2),
// the token's descent direction G_t = -grad_W 0.5||f_W(k_t) - v_t||^2 is
// taken at W_0 as well (§1, §3), and the state follows the token-wise
// recurrence whose chunk-end values the closed form reproduces (§3.2,
// App. A.5):
//   M <- beta_t M + eta_t G_t,   W <- gamma_t W + M,
// with gamma_t = 1 - eta_t alpha_t (Eq. 14) or alpha_t itself.  After the
// last token of a chunk the running W becomes the next chunk's W_0 (§3.2,
// induction over chunks).  Running the step over a sequence therefore gives
// the same outputs and chunk-end states as the chunk forward.
//
// Per token and unit (SwiGLU, f(x) = W2 (silu(W1 x) * W3 x)):
//   k_dec_fwd13 : a1 = W1 x, a3 = W3 x, z = silu(a1) a3 for x = q and x = k
//   k_dec_fwd2  : y = W2 z; out = y(q); g = v - y(k)
//   k_dec_bwd   : partial dz = W2^T g per block of 64 rows of W2
//   k_dec_dact  : dz (partials added in block order); dA3 = dz silu(a1),
//                 dA1 = dz a3 silu'(a1)
//   k_dec_update: G_W1 = dA1 k^T, G_W3 = dA3 k^T, G_W2 = g z(k)^T and the
//                 recurrence on every state entry (16-byte vectors)
// Linear learner (f(x) = W x): k_dec_lin_fwd (y, out, g) and k_dec_update
// with G = g k^T.  All arithmetic is fp32 on the fp32 state; the per-token
// dot products reduce over lanes (fixed shuffle order), so results do not
// depend on scheduling.
#pragma once
#include "common.hpp"

namespace e2ttt {

struct DecodeArgs {
  int64_t BH, d, h;   // h = 0 for the linear learner
  int mode;           // decay_mode
  int chunk_end;      // nonzero: W_0 <- W after the update
  const float* eta;   // [BH]
  const float* alpha;
  const float* beta;
  float* W0;          // [BH][P] chunk-start weights
  float* W;           // [BH][P] running weights
  float* M;           // [BH][P] running momentum
  float* zq;          // workspace [BH][h]: z of the query
  float* zk;          // [BH][h]: z of the key
  float* a1k;         // [BH][h]
  float* a3k;         // [BH][h]
  float* dA1;         // [BH][h]
  float* dA3;         // [BH][h]
  float* g;           // [BH][d]: v - f_{W_0}(k)
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Rows of a [rows][n] fp32 matrix dotted with lane-strided vectors: lane l
// holds x[l + 64 m] (m < n/64, n % 64 == 0).  R rows per wave, all loads of
// the wave issued before any reduction.
template <int R, int NX, int MAXM>
__device__ __forceinline__ void wave_dots(const float* const (&rows)[R], int64_t n,
                                          const float (&x)[NX][MAXM], float (&out)[R][NX]) {
  const int lane = threadIdx.x & 63;
  const int nm = static_cast<int>(n / 64);
  float acc[R][NX];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < NX; ++c) acc[r][c] = 0.0f;
#pragma unroll
  for (int m = 0; m < MAXM; ++m) {
    if (m < nm) {
      float w[R];
#pragma unroll
      for (int r = 0; r < R; ++r) w[r] = rows[r][lane + 64 * m];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NX; ++c) acc[r][c] = fmaf(w[r], x[c][m], acc[r][c]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < NX; ++c) out[r][c] = wave_sum(acc[r][c]);
}

// W1 and W3 rows of 4 hidden units per wave (16 per workgroup) dotted with q
// and k.  Grid BH * (h / 16); d <= 1024.
template <typename T>
__global__ __launch_bounds__(256) void k_dec_fwd13(DecodeArgs a, const T* __restrict__ q,
                                                   const T* __restrict__ k) {
  const int64_t nb = a.h / 16, u = blockIdx.x / nb, ib = blockIdx.x % nb;
  const int64_t d = a.d, h = a.h;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float x[2][16];
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int64_t e = lane + 64 * m;
    x[0][m] = e < d ? to_f32<T>(q[u * d + e]) : 0.0f;
    x[1][m] = e < d ? to_f32<T>(k[u * d + e]) : 0.0f;
  }
  const float* Wu = a.W0 + u * 3 * d * h;
  const int64_t i0 = ib * 16 + wave * 4;
  const float* rows[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    rows[r] = Wu + (i0 + r) * d;              // W1
    rows[4 + r] = Wu + h * d + (i0 + r) * d;  // W3
  }
  float s[8][2];
  wave_dots<8, 2, 16>(rows, d, x, s);
  if (lane < 4) {
    const int r = lane;
    float s1q = s[0][0], s3q = s[4][0], s1k = s[0][1], s3k = s[4][1];
#pragma unroll
    for (int rr = 1; rr < 4; ++rr)
      if (r == rr) {
        s1q = s[rr][0]; s3q = s[4 + rr][0]; s1k = s[rr][1]; s3k = s[4 + rr][1];
      }
    const int64_t i = u * h + i0 + r;
    a.zq[i] = s1q * sigmoidf_(s1q) * s3q;
    a.zk[i] = s1k * sigmoidf_(s1k) * s3k;
    a.a1k[i] = s1k;
    a.a3k[i] = s3k;
  }
}

// W2 rows of 4 outputs per wave (16 per workgroup): y = W2 z for both z; the
// readout and the residual g.  Grid BH * (d / 16); h <= 4096.
template <typename T>
__global__ __launch_bounds__(256) void k_dec_fwd2(DecodeArgs a, const T* __restrict__ v,
                                                  T* __restrict__ out) {
  const int64_t nb = a.d / 16, u = blockIdx.x / nb, jb = blockIdx.x % nb;
  const int64_t d = a.d, h = a.h;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float z[2][64];
#pragma unroll
  for (int m = 0; m < 64; ++m) {
    const int64_t e = lane + 64 * m;
    z[0][m] = e < h ? a.zq[u * h + e] : 0.0f;
    z[1][m] = e < h ? a.zk[u * h + e] : 0.0f;
  }
  const float* W2 = a.W0 + u * 3 * d * h + 2 * h * d;
  const int64_t j0 = jb * 16 + wave * 4;
  const float* rows[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) rows[r] = W2 + (j0 + r) * h;
  float y[4][2];
  wave_dots<4, 2, 64>(rows, h, z, y);
  if (lane < 4) {
    float yq = y[0][0], yk = y[0][1];
#pragma unroll
    for (int rr = 1; rr < 4; ++rr)
      if (lane == rr) {
        yq = y[rr][0];
        yk = y[rr][1];
      }
    const int64_t j = u * d + j0 + lane;
    out[j] = from_f32<T>(yq);
    a.g[j] = to_f32<T>(v[j]) - yk;
  }
}

// Partial dz = W2^T g over one block of 64 rows j for 64 hidden units per
// workgroup (lane = hidden unit, the 4 waves take 16 rows each, added in
// wave order): part[jb][u][i].  Grid BH * (h / 64) * (d / 64).
__global__ __launch_bounds__(256) void k_dec_bwd(DecodeArgs a, float* __restrict__ part) {
  __shared__ float red[4][64];
  const int64_t nib = a.h / 64, njb = a.d / 64;
  const int64_t jb = blockIdx.x % njb, rest = blockIdx.x / njb;
  const int64_t ib = rest % nib, u = rest / nib;
  const int64_t d = a.d, h = a.h;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* W2 = a.W0 + u * 3 * d * h + 2 * h * d + ib * 64 + lane;
  const int64_t j0 = jb * 64 + wave * 16;
  float w[16], gv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    w[r] = W2[(j0 + r) * h];
    gv[r] = a.g[u * d + j0 + r];
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s = fmaf(w[r], gv[r], s);
  red[wave][lane] = s;
  __syncthreads();
  if (wave == 0)
    part[(jb * a.BH + u) * h + ib * 64 + lane] =
        ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

// dz from the d/64 partials (in block order), then dA1, dA3.  Grid
// ceil(BH * h / 256).
__global__ __launch_bounds__(256) void k_dec_dact(DecodeArgs a, const float* __restrict__ part) {
  const int64_t n = a.BH * a.h;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float dz = part[i];
  for (int64_t jb = 1; jb < a.d / 64; ++jb) dz += part[jb * n + i];
  const float a1 = a.a1k[i], a3 = a.a3k[i];
  const float sg = sigmoidf_(a1);
  a.dA3[i] = dz * (a1 * sg);
  a.dA1[i] = dz * a3 * (sg * (1.0f + a1 * (1.0f - sg)));
}

// Linear learner: y = W x for q and k, 4 waves over the d rows of one unit.
// Grid BH.
template <typename T>
__global__ __launch_bounds__(256) void k_dec_lin_fwd(DecodeArgs a, const T* __restrict__ q,
                                                     const T* __restrict__ k,
                                                     const T* __restrict__ v,
                                                     T* __restrict__ out) {
  __shared__ float xs[2][128];
  const int64_t u = blockIdx.x, d = a.d;
  for (int64_t e = threadIdx.x; e < d; e += 256) {
    xs[0][e] = to_f32<T>(q[u * d + e]);
    xs[1][e] = to_f32<T>(k[u * d + e]);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* Wu = a.W0 + u * d * d;
  for (int64_t i = wave; i < d; i += 4) {
    float yq = 0.0f, yk = 0.0f;
    for (int64_t e = lane; e < d; e += 64) {
      const float x = Wu[i * d + e];
      yq = fmaf(x, xs[0][e], yq);
      yk = fmaf(x, xs[1][e], yk);
    }
    yq = wave_sum(yq);
    yk = wave_sum(yk);
    if (lane == 0) {
      out[u * d + i] = from_f32<T>(yq);
      a.g[u * d + i] = to_f32<T>(v[u * d + i]) - yk;
    }
  }
}

// The recurrence on every state entry, four consecutive entries per thread:
// M <- beta M + eta G, W <- gamma W + M (and W_0 <- W at a chunk end).
// Grid ceil(BH * P / 4 / 256); P % 4 == 0 and every row is a multiple of 4.
template <typename T>
__global__ __launch_bounds__(256) void k_dec_update(DecodeArgs a, const T* __restrict__ k) {
  const int64_t d = a.d, h = a.h;
  const int64_t P = h == 0 ? d * d : 3 * d * h;
  const int64_t e4 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (e4 >= a.BH * P) return;
  const int64_t u = e4 / P, o = e4 % P;
  const float et = a.eta[u], al = a.alpha[u], bt = a.beta[u];
  // gamma in fp64 from the fp32 inputs (the product is exact), one rounding.
  const float gt = a.mode == 1 ? al
                   : static_cast<float>(1.0 - static_cast<double>(et) * static_cast<double>(al));
  float left;        // the left factor of this row of G
  float right[4];    // the right factors of the four entries
  // Four consecutive entries of k (vector load; their index is a multiple
  // of 4 and rows of k are multiples of 16 elements).
  auto k4 = [&](int64_t idx) {
    if constexpr (sizeof(T) == 2) {
      const uint2 p = *reinterpret_cast<const uint2*>(k + idx);
      right[0] = bf2f(static_cast<bf16_t>(p.x & 0xffffu));
      right[1] = bf2f(static_cast<bf16_t>(p.x >> 16));
      right[2] = bf2f(static_cast<bf16_t>(p.y & 0xffffu));
      right[3] = bf2f(static_cast<bf16_t>(p.y >> 16));
    } else {
      const f32x4_t p = *reinterpret_cast<const f32x4_t*>(k + idx);
#pragma unroll
      for (int x = 0; x < 4; ++x) right[x] = p[x];
    }
  };
  if (h == 0) {      // linear: G = g k^T
    const int64_t i = o / d, j = o % d;
    left = a.g[u * d + i];
    k4(u * d + j);
  } else if (o < 2 * h * d) {  // W1 or W3 row i: G = dA k^T
    const bool w3 = o >= h * d;
    const int64_t oo = w3 ? o - h * d : o;
    const int64_t i = oo / d, j = oo % d;
    left = (w3 ? a.dA3 : a.dA1)[u * h + i];
    k4(u * d + j);
  } else {           // W2 row j: G = g z(k)^T
    const int64_t oo = o - 2 * h * d;
    const int64_t j = oo / h, i = oo % h;
    left = a.g[u * d + j];
    const f32x4_t z = *reinterpret_cast<const f32x4_t*>(a.zk + u * h + i);
#pragma unroll
    for (int x = 0; x < 4; ++x) right[x] = z[x];
  }
  const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(a.W + e4);
  const f32x4_t m0 = *reinterpret_cast<const f32x4_t*>(a.M + e4);
  f32x4_t wn, mn;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    mn[x] = fmaf(bt, m0[x], et * (left * right[x]));
    wn[x] = fmaf(gt, w0[x], mn[x]);
  }
  *reinterpret_cast<f32x4_t*>(a.M + e4) = mn;
  *reinterpret_cast<f32x4_t*>(a.W + e4) = wn;
  if (a.chunk_end) *reinterpret_cast<f32x4_t*>(a.W0 + e4) = wn;
}

}  // namespace e2ttt
