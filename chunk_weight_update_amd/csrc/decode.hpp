// decode.hpp -- streaming / decode use of the chunk update of "Rethinking
// Expressivity and Efficiency in Test-Time Training" (E2-TTT): one token of
// every (b, h) unit per call, with the state update amortised over the chunk.
//
// Within a chunk the readout uses the chunk-start weights W_0 (Eq. 6, §3.2)
// and the token's descent direction G_t is taken at W_0 as well (§1, §3), so
// a token needs only W_0: its output and the rank-one factors of G_t are
// computed at once, and the factors (with the token's key and scalars) go
// into the chunk's slot of a buffer.  At the chunk's last token the chunk-end
// pair (W_C, M_C) is formed from the buffered tokens exactly as the chunk
// forward forms it (§3.2, App. A: the scalar kernels by the suffix scan, then
// the two weighted aggregations), and it becomes the next chunk's start (App.
// B.5 notes that this per-chunk bookkeeping is amortised over the chunk's
// tokens).
//
// Per token and unit (SwiGLU, f(x) = W2 (silu(W1 x) * W3 x); the MLP learner
// f(x) = W2 silu(W1 x) on the same kernels with a3 = 1 and dA3 = 0, its
// [W1 | W2] state read in place and, at a chunk end, updated through the
// [W1 | W3 = 0 | W2] layout of the aggregation):
//   k_dec_fwd13 : a1 = W1 x, a3 = W3 x, z = silu(a1) a3 for x = q and x = k
//   k_dec_fwd2  : y = W2 z; out = y(q); g = v - y(k)
//   k_dec_bwd   : partial dz = W2^T g per block of 64 rows of W2
//   k_dec_stash : dz (partials added in block order); dA3 = dz silu(a1),
//                 dA1 = dz a3 silu'(a1); k, z(k), dA1, dA3, g and the
//                 scalars into the chunk slot
// Linear learner (f(x) = W x): k_dec_lin_fwd (y, out, g) and k_dec_stash.
// At the chunk end: the scan over the buffered scalars, k_dec_pack (the
// scaled aggregation operands, feature-major) and the chunk forward's fp32
// aggregation kernel.  All arithmetic is fp32 on the fp32 state; per-token
// dot products reduce over lanes in a fixed shuffle order.
#pragma once
#include "common.hpp"

namespace e2ttt {

struct DecodeArgs {
  int64_t BH, d, h;   // h = 0 for the linear learner
  int64_t P;          // state entries per unit: [W1 | W3 | W2] 3dh, the MLP's [W1 | W2] 2dh
  int gated;          // 0 for the MLP learner: no W3, a3 = 1, dA3 = 0
  const float* W0;    // [BH][P] chunk-start weights
  float* zq;          // workspace [BH][h]: z of the query
  float* zk;          // [BH][h]: z of the key
  float* a1k;         // [BH][h]: the key's pre-activations
  float* a3k;         // [BH][h]
  float* g;           // [BH][d]: v - f_{W_0}(k)
};

// The chunk buffer of the decode workspace (fp32).  Slot t of a chunk holds
// token t.  SwiGLU: feature-major rows of cb slots, as the aggregation
// reads them; linear: token-major.
struct DecodeBuf {
  int64_t cb;          // slots (the chunk length rounded up to the tile)
  float* eb;           // [BH][cb] eta, alpha, beta of the buffered tokens
  float* ab;
  float* bb;
  float* kt;           // SwiGLU [BH][d][cb]: keys
  float* zt;           // [BH][h][cb]: z(k)
  float* d1;           // [BH][h][cb]: dA1
  float* d3;           // [BH][h][cb]: dA3
  float* gb;           // [BH][d][cb]: g
  float* kb;           // linear [BH][cb][d]: keys
  float* gl;           // [BH][cb][d]: g
  // chunk-end operands
  float* kw;           // [BH][cb] K^W, K^M (zero past the chunk's tokens)
  float* km;
  float* coef;         // [BH][4] cW, cM, cWM
  float* ut;           // SwiGLU [BH][4h][cb]: K^W dA1, K^M dA1 | K^W dA3, K^M dA3 (32-row interleave)
  float* gt;           // [BH][2d][cb]: K^W g, K^M g (32-row interleave)
  float* gw;           // linear [BH][cb][d]: K^W g
  float* gm;           // [BH][cb][d]: K^M g
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Rows of a [rows][n] fp32 matrix dotted with lane-strided vectors: lane l
// holds x[4 l + 256 m .. +3] (m < M4; zero past n, n % 4 == 0, n <= 256 M4),
// so a wave reads a 1 KB piece of each row per 16-byte load instruction.
// Every load of the wave is issued before any product, unconditionally:
// pieces past n read the row's last (in-range) 16 bytes, which meet x = 0.
// (A load under a runtime condition makes the compiler wait for each one in
// turn; the first version's 4-byte loads took four times the instructions,
// more than the 63 a wave can have in flight at d = 768.)
template <int R, int NX, int M4>
__device__ __forceinline__ void wave_dots4(const float* const (&rows)[R], int64_t n,
                                           const f32x4_t (&x)[NX][M4], float (&out)[R][NX]) {
  const int lane = threadIdx.x & 63;
  f32x4_t w[M4][R];
#pragma unroll
  for (int m = 0; m < M4; ++m) {
    const int64_t e0 = 4 * lane + 256 * m;
    const int64_t e = e0 < n ? e0 : n - 4;
#pragma unroll
    for (int r = 0; r < R; ++r) w[m][r] = *reinterpret_cast<const f32x4_t*>(rows[r] + e);
  }
  float acc[R][NX];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < NX; ++c) acc[r][c] = 0.0f;
#pragma unroll
  for (int m = 0; m < M4; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NX; ++c) acc[r][c] = fmaf(w[m][r][j], x[c][m][j], acc[r][c]);
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < NX; ++c) out[r][c] = wave_sum(acc[r][c]);
}

// Piece count of wave_dots4 for a vector of n: the smallest of 1, 2, 3, 4, 6,
// 8, 12, 16 with 256 times it >= n.
__host__ __device__ inline int dot_pieces(int64_t n) {
  const int need = static_cast<int>((n + 255) / 256);
  const int set[] = {1, 2, 3, 4, 6, 8, 12, 16};
  for (int v : set)
    if (v >= need) return v;
  return 16;
}


// W1 and W3 rows of 2 hidden units per wave (8 per workgroup) dotted with q
// and k (the MLP learner: W1 only, a3 = 1).  Grid BH * (h / 8); d <= 256 M4.
template <typename T, int M4>
__global__ __launch_bounds__(256) void k_dec_fwd13(DecodeArgs a, const T* __restrict__ q,
                                                   const T* __restrict__ k) {
  const int64_t nb = a.h / 8, u = blockIdx.x / nb, ib = blockIdx.x % nb;
  const int64_t d = a.d, h = a.h;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x4_t x[2][M4];
#pragma unroll
  for (int m = 0; m < M4; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t e = 4 * lane + 256 * m + j;
      x[0][m][j] = e < d ? to_f32<T>(q[u * d + e]) : 0.0f;
      x[1][m][j] = e < d ? to_f32<T>(k[u * d + e]) : 0.0f;
    }
  const float* Wu = a.W0 + u * a.P;
  const int64_t i0 = ib * 8 + wave * 2;
  const float* rows[4];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    rows[r] = Wu + (i0 + r) * d;                                // W1
    rows[2 + r] = a.gated ? Wu + h * d + (i0 + r) * d : rows[r];  // W3 (MLP: unused)
  }
  float s[4][2];
  wave_dots4<4, 2, M4>(rows, d, x, s);
  if (lane < 2) {
    const float s1q = lane ? s[1][0] : s[0][0], s1k = lane ? s[1][1] : s[0][1];
    const float s3q = a.gated ? (lane ? s[3][0] : s[2][0]) : 1.0f;
    const float s3k = a.gated ? (lane ? s[3][1] : s[2][1]) : 1.0f;
    const int64_t i = u * h + i0 + lane;
    a.zq[i] = s1q * sigmoidf_(s1q) * s3q;
    a.zk[i] = s1k * sigmoidf_(s1k) * s3k;
    a.a1k[i] = s1k;
    a.a3k[i] = s3k;
  }
}

// One W2 row per wave (4 per workgroup): y = W2 z for both z; the readout
// and the residual g.  Grid BH * (d / 4); h <= 256 M4.
template <typename T, int M4>
__global__ __launch_bounds__(256) void k_dec_fwd2(DecodeArgs a, const T* __restrict__ v,
                                                  T* __restrict__ out) {
  const int64_t nb = a.d / 4, u = blockIdx.x / nb, jb = blockIdx.x % nb;
  const int64_t d = a.d, h = a.h;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x4_t z[2][M4];
#pragma unroll
  for (int m = 0; m < M4; ++m) {
    const int64_t e0 = 4 * lane + 256 * m;
    const int64_t e = e0 < h ? e0 : h - 4;
    const f32x4_t zq = *reinterpret_cast<const f32x4_t*>(a.zq + u * h + e);
    const f32x4_t zk = *reinterpret_cast<const f32x4_t*>(a.zk + u * h + e);
    const f32x4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
    z[0][m] = e0 < h ? zq : zero;
    z[1][m] = e0 < h ? zk : zero;
  }
  const int64_t j = jb * 4 + wave;
  const float* rows[1] = {a.W0 + u * a.P + (a.P - h * d) + j * h};  // W2 row j
  float y[1][2];
  wave_dots4<1, 2, M4>(rows, h, z, y);
  if (lane == 0) {
    out[u * d + j] = from_f32<T>(y[0][0]);
    a.g[u * d + j] = to_f32<T>(v[u * d + j]) - y[0][1];
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
  const float* W2 = a.W0 + u * a.P + (a.P - h * d) + ib * 64 + lane;
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

// Token `pos` of the chunk into the buffer: the scalars, and (SwiGLU) k,
// z(k), dA1, dA3, g feature-major, or (linear) k, g token-major.  dA1, dA3
// come from dz, the d/64 partials of k_dec_bwd added in block order, and the
// key's pre-activations: dA3 = dz silu(a1), dA1 = dz a3 silu'(a1).  One
// block per (unit, group of 256 entries); grid BH * ceil((3 + 3h + 2d) / 256).
template <typename T>
__global__ __launch_bounds__(256) void k_dec_stash(DecodeArgs a, DecodeBuf b, int64_t pos,
                                                   const T* __restrict__ k,
                                                   const float* __restrict__ eta,
                                                   const float* __restrict__ alpha,
                                                   const float* __restrict__ beta,
                                                   const float* __restrict__ part) {
  const int64_t d = a.d, h = a.h, cb = b.cb;
  const int64_t per = 3 + 3 * h + 2 * d;
  const int64_t nblk = (per + 255) / 256;
  const int64_t u = blockIdx.x / nblk;
  const int64_t e = (blockIdx.x % nblk) * 256 + threadIdx.x;
  if (e >= per) return;
  if (e < 3) {
    const float* src = e == 0 ? eta : e == 1 ? alpha : beta;
    float* dst = e == 0 ? b.eb : e == 1 ? b.ab : b.bb;
    dst[u * cb + pos] = src[u];
    return;
  }
  int64_t x = e - 3;
  if (h == 0) {  // linear: k then g, token-major
    if (x < d) b.kb[(u * cb + pos) * d + x] = to_f32<T>(k[u * d + x]);
    else if (x < 2 * d) b.gl[(u * cb + pos) * d + (x - d)] = a.g[u * d + (x - d)];
    return;
  }
  if (x < d) { b.kt[(u * d + x) * cb + pos] = to_f32<T>(k[u * d + x]); return; }
  x -= d;
  if (x < d) { b.gb[(u * d + x) * cb + pos] = a.g[u * d + x]; return; }
  x -= d;
  const int64_t which = x / h, j = x % h;  // 0: z, 1: dA1, 2: dA3
  const int64_t i = u * h + j;
  if (which == 0) {
    b.zt[i * cb + pos] = a.zk[i];
    return;
  }
  // dz: the partials in block order, loaded four at a time.
  const int64_t n = a.BH * h, nj = d / 64;
  float dz = part[i];
  int64_t jb = 1;
  for (; jb + 4 <= nj; jb += 4) {
    const float p0 = part[jb * n + i], p1 = part[(jb + 1) * n + i];
    const float p2 = part[(jb + 2) * n + i], p3 = part[(jb + 3) * n + i];
    dz = (((dz + p0) + p1) + p2) + p3;
  }
  for (; jb < nj; ++jb) dz += part[jb * n + i];
  const float a1 = a.a1k[i], a3 = a.a3k[i];
  const float sg = sigmoidf_(a1);
  if (which == 1) b.d1[i * cb + pos] = dz * a3 * (sg * (1.0f + a1 * (1.0f - sg)));
  else b.d3[i * cb + pos] = a.gated ? dz * (a1 * sg) : 0.0f;
}

// Chunk end, SwiGLU: the scaled aggregation operands of the n buffered tokens
// (zero in the slots past them), and the key and z rows' slots past them
// zeroed (stale or unset slots must not reach the products).  One block per
// (unit, operand row), threads along the slots; grid BH * (5h + 3d).
__global__ __launch_bounds__(256) void k_dec_pack(DecodeArgs a, DecodeBuf b, int64_t n) {
  const int64_t d = a.d, h = a.h, cb = b.cb;
  const int64_t rows = 5 * h + 3 * d;
  const int64_t u = blockIdx.x / rows;
  int64_t R = blockIdx.x % rows;
  const float* kwu = b.kw + u * cb;
  const float* kmu = b.km + u * cb;
  if (R < 4 * h) {  // ut row R
    const bool a3 = R >= 2 * h;
    const int64_t Rp = a3 ? R - 2 * h : R;
    const bool isM = (Rp % 64) >= 32;
    const int64_t j = 64 * (Rp / 64) / 2 + Rp % 32;
    const float* src = (a3 ? b.d3 : b.d1) + (u * h + j) * cb;
    const float* ks = isM ? kmu : kwu;
    float* dst = b.ut + (u * 4 * h + R) * cb;
    for (int64_t t = threadIdx.x; t < cb; t += 256) dst[t] = t < n ? ks[t] * src[t] : 0.0f;
    return;
  }
  R -= 4 * h;
  if (R < 2 * d) {  // gt row R
    const bool isM = (R % 64) >= 32;
    const int64_t i = 64 * (R / 64) / 2 + R % 32;
    const float* src = b.gb + (u * d + i) * cb;
    const float* ks = isM ? kmu : kwu;
    float* dst = b.gt + (u * 2 * d + R) * cb;
    for (int64_t t = threadIdx.x; t < cb; t += 256) dst[t] = t < n ? ks[t] * src[t] : 0.0f;
    return;
  }
  R -= 2 * d;
  float* row = R < d ? b.kt + (u * d + R) * cb : b.zt + (u * h + (R - d)) * cb;
  for (int64_t t = n + threadIdx.x; t < cb; t += 256) row[t] = 0.0f;
}

// Chunk end, linear learner: K^W g and K^M g of the buffered tokens, zero
// past them.  Grid ceil(BH * cb * d / 256).
__global__ __launch_bounds__(256) void k_dec_pack_lin(DecodeArgs a, DecodeBuf b, int64_t n) {
  const int64_t d = a.d, cb = b.cb;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= a.BH * cb * d) return;
  const int64_t u = e / (cb * d), t = (e / d) % cb;
  const float g = t < n ? b.gl[e] : 0.0f;
  b.gw[e] = t < n ? b.kw[u * cb + t] * g : 0.0f;
  b.gm[e] = t < n ? b.km[u * cb + t] * g : 0.0f;
}

}  // namespace e2ttt
