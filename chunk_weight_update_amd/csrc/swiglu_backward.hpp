// Outer-loop backward of the chunk update for the three-matrix SwiGLU learner
// f(x) = W2 (silu(W1 x) * (W3 x)) ("Rethinking Expressivity and Efficiency in
// Test-Time Training", §5.2 and App. B.5 for the learner; §3.2 and Appendix A
// for the chunk closed form), fp32.
//
// Chunk r with start state (Ws, Ms) produces (§3.2)
//   W_C = cW Ws + cWM Ms + sum_t K^W_t G_t,   M_C = cM Ms + sum_t K^M_t G_t,
//   out_t = f_Ws(q_t),
// with G_t the descent direction at the frozen Ws: for
//   a1 = W1 k, a3 = W3 k, z = silu(a1) a3, e = v - W2 z, w = W2^T e,
//   G_W1 = u1 k^T (u1 = w a3 silu'(a1)), G_W3 = u3 k^T (u3 = w silu(a1)),
//   G_W2 = e z^T.
// Given the adjoints dW_C, dM_C of the chunk-end state, the adjoint of G_t is
// the per-token matrix A_t = K^W_t dW_C + K^M_t dM_C, never formed: every
// product with it is a product with dW_C and dM_C, combined per token.
//   dK^W_t = <dW_C, G_t> = u1.(dW1_C k) + u3.(dW3_C k) + e.(dW2_C z)
//   du1 = A1 k, du3 = A3 k, de = A2 z + W2 dw, dz = A2^T e - W2^T de,
//   dw = du3 silu(a1) + du1 a3 silu'(a1),
//   da1 = du3 w silu' + du1 w a3 silu'' + dz a3 silu',  da3 = du1 w silu' + dz silu,
//   dk = W1^T da1 + W3^T da3 + A1^T u1 + A3^T u3,  dv = de,
//   dWs += [da1; da3] k^T (W1, W3) and e dw^T - de z^T (W2), summed over tokens,
// plus the readout's reverse mode (dq, dWs) and the state terms
//   dW_prev = cW dW_C + dWs,  dM_prev = cWM dW_C + cM dM_C,
//   dcW = <dW_C, Ws>, dcM = <dM_C, Ms>, dcWM = <dW_C, Ms>.
// The scalar adjoints (deta, dalpha, dbeta) follow from dK^W, dK^M and the
// three dots exactly as for the linear learner.
//
// Every product over tokens or features is a call of one batched, strided
// fp32 GEMM (64 x 64 tiles through LDS, fp32 MFMA; products with few tiles
// and a long K on 32 x 32 tiles with K split inside the workgroup); the
// per-token steps are small elementwise kernels.  Only the chunk's n valid
// tokens enter any product.
#pragma once

#include "kernels.hpp"

namespace e2ttt {

// C[b](m, n) = D[b](m, n) + alpha * sum_k A[b](m, k) B[b](k, n), m < M, n < N,
// with A(m, k) at A + b*sAb + m*sAm + k*sAk, B(k, n) at B + b*sBb + k*sBk +
// n*sBn, C and D row-major with leading dimensions ldc, ldd.  D may be null
// (zero) or equal to C.
struct GemmF32 {
  int64_t M, N, K;
  const float* A;
  int64_t sAb, sAm, sAk;
  const float* B;
  int64_t sBb, sBk, sBn;
  const float* D;
  int64_t sDb, ldd;
  float* C;
  int64_t sCb, ldc;
  float alpha;
};

constexpr int GF_T = 64, GF_K = 16;

// 64 x 64 output tile, 256 threads = 4 waves in a 2 x 2 grid, each wave one
// 32 x 32 block on v_mfma_f32_32x32x2f32.  K advances in slabs of 16 staged
// through LDS (k-major, so both operands are read as 32 consecutive floats per
// lane half); the next slab's global loads are in flight during the current
// slab's MFMAs.  Loads run along whichever of an operand's two strides is 1,
// so row- and column-major operands are both read in full cache lines.
__global__ __launch_bounds__(256) void k_gemm_f32(GemmF32 g) {
  __shared__ float As[GF_K][GF_T + 4], Bs[GF_K][GF_T + 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, hf = lane >> 5;
  const int64_t b = blockIdx.z;
  const int64_t kb = 0, ke = g.K;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * GF_T;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * GF_T;
  const float* A = g.A + b * g.sAb;
  const float* B = g.B + b * g.sBb;
  const bool aK = g.sAk == 1;  // k contiguous in A: threads run along k
  const bool bN = g.sBn == 1;  // n contiguous in B: threads run along n
  float ra[4], rb[4];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const int e = tid + 256 * l;
      const int mm = aK ? e / GF_K : e % GF_T, kk = aK ? e % GF_K : e / GF_T;
      const int64_t m = m0 + mm, k = k0 + kk;
      ra[l] = (m < g.M && k < ke) ? A[m * g.sAm + k * g.sAk] : 0.0f;
      const int nn = bN ? e % GF_T : e / GF_K, kb = bN ? e / GF_T : e % GF_K;
      const int64_t n = n0 + nn, kq = k0 + kb;
      rb[l] = (n < g.N && kq < ke) ? B[kq * g.sBk + n * g.sBn] : 0.0f;
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const int e = tid + 256 * l;
      As[aK ? e % GF_K : e / GF_T][aK ? e / GF_K : e % GF_T] = ra[l];
      Bs[bN ? e / GF_T : e % GF_K][bN ? e % GF_T : e / GF_K] = rb[l];
    }
  };
  f32x16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  fetch(kb);
  stash();
  __syncthreads();
  for (int64_t k0 = kb; k0 < ke; k0 += GF_K) {
    const bool more = k0 + GF_K < ke;
    if (more) fetch(k0 + GF_K);
#pragma unroll
    for (int ks = 0; ks < GF_K / 2; ++ks) {
      const int k = 2 * ks + hf;
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(As[k][32 * wm + l32], Bs[k][32 * wn + l32], acc,
                                                 0, 0, 0);
    }
    __syncthreads();
    if (more) {
      stash();
      __syncthreads();
    }
  }
  // Lane l, register v holds row 8 (v / 4) + 4 hf + v % 4, column l % 32 of
  // the wave's block.
  const int64_t n = n0 + 32 * wn + l32;
  if (n >= g.N) return;
  float* C = g.C + b * g.sCb;
  const float* D = g.D ? g.D + b * g.sDb : nullptr;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t m = m0 + 32 * wm + 8 * (v / 4) + 4 * hf + (v % 4);
    if (m >= g.M) continue;
    const float base = D ? D[m * g.ldd + n] : 0.0f;
    C[m * g.ldc + n] = base + g.alpha * acc[v];
  }
}

constexpr int GQ_T = 32;

// K split four ways inside the workgroup: each wave computes the whole
// TxT output tile (T = 32: one 32 x 32 MFMA block; T = 64: four) over its
// quarter of the 16-deep slabs, staged through its own double-buffered LDS
// (so the waves never wait for each other in the loop, and four slabs per
// workgroup are in flight instead of one) and accumulated on
// v_mfma_f32_32x32x2f32; the four partial tiles then meet in LDS and are
// added in wave order, so the result does not depend on scheduling, and
// C = D + alpha * sum is written directly: no partial buffer and no second
// launch.  Loads run along whichever of an operand's strides is 1, as above.
template <int T>
struct GemmK4 {
  static constexpr int LD = T + 4;                            // staged row, floats
  static constexpr int STAGE = 2 * 2 * GF_K * LD;             // [buffer][A, B][k][m or n]
  static constexpr int RED = T * (T + 1);                     // one wave's partial tile
  static constexpr size_t LDS_BYTES =
      4 * static_cast<size_t>(STAGE > RED ? STAGE : RED) * sizeof(float);
  static constexpr int PER = T * GF_K / 64;                   // elements per lane per operand slab
};

template <int T>
__global__ __launch_bounds__(256) void k_gemm_f32_k4(GemmF32 g) {
  using Q = GemmK4<T>;
  constexpr int LD = Q::LD, NB = T / 32;
  extern __shared__ float smem_f[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hf = lane >> 5;
  float* St = smem_f + wave * (Q::STAGE > Q::RED ? Q::STAGE : Q::RED);
  auto sa = [&](int buf, int k, int m) -> float& { return St[((buf * 2 + 0) * GF_K + k) * LD + m]; };
  auto sb = [&](int buf, int k, int n) -> float& { return St[((buf * 2 + 1) * GF_K + k) * LD + n]; };
  const int64_t b = blockIdx.z;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * T;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * T;
  const float* A = g.A + b * g.sAb;
  const float* B = g.B + b * g.sBb;
  const bool aK = g.sAk == 1;
  const bool bN = g.sBn == 1;
  // This wave's slabs: [s0, s1) of the ceil(K / 16) slabs.
  const int64_t ns = (g.K + GF_K - 1) / GF_K;
  const int64_t s0 = ns * wave / 4, s1 = ns * (wave + 1) / 4;
  float ra[Q::PER], rb[Q::PER];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int l = 0; l < Q::PER; ++l) {
      const int e = lane + 64 * l;
      const int mm = aK ? e / GF_K : e % T, kk = aK ? e % GF_K : e / T;
      const int64_t m = m0 + mm, k = k0 + kk;
      ra[l] = (m < g.M && k < g.K) ? A[m * g.sAm + k * g.sAk] : 0.0f;
      const int nn = bN ? e % T : e / GF_K, kq = bN ? e / T : e % GF_K;
      const int64_t n = n0 + nn, kb = k0 + kq;
      rb[l] = (n < g.N && kb < g.K) ? B[kb * g.sBk + n * g.sBn] : 0.0f;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int l = 0; l < Q::PER; ++l) {
      const int e = lane + 64 * l;
      sa(buf, aK ? e % GF_K : e / T, aK ? e / GF_K : e % T) = ra[l];
      sb(buf, bN ? e / T : e % GF_K, bN ? e % T : e / GF_K) = rb[l];
    }
  };
  f32x16_t acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  if (s0 < s1) {
    fetch(s0 * GF_K);
    stash(0);
  }
  int buf = 0;
  for (int64_t sl = s0; sl < s1; ++sl) {
    const bool more = sl + 1 < s1;
    if (more) fetch((sl + 1) * GF_K);
#pragma unroll
    for (int ks = 0; ks < GF_K / 2; ++ks) {
      const int k = 2 * ks + hf;
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(sa(buf, k, 32 * i + l32),
                                                           sb(buf, k, 32 * j + l32), acc[i][j],
                                                           0, 0, 0);
    }
    if (more) stash(buf ^ 1);
    buf ^= 1;
  }
  // Partial tile of this wave into its own area (the staging area is this
  // wave's alone); lane l, register v of block (i, j) holds row
  // 32 i + 8 (v / 4) + 4 hf + v % 4, column 32 j + l % 32.
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        St[(32 * i + 8 * (v / 4) + 4 * hf + (v % 4)) * (T + 1) + 32 * j + l32] = acc[i][j][v];
  __syncthreads();
  const int WS = Q::STAGE > Q::RED ? Q::STAGE : Q::RED;
  float* C = g.C + b * g.sCb;
  const float* D = g.D ? g.D + b * g.sDb : nullptr;
#pragma unroll
  for (int l = 0; l < T * T / 256; ++l) {
    const int e = tid + 256 * l, mm = e / T, nn = e % T;
    const int64_t m = m0 + mm, n = n0 + nn;
    if (m >= g.M || n >= g.N) continue;
    const int o = mm * (T + 1) + nn;
    const float sum = ((smem_f[o] + smem_f[WS + o]) + smem_f[2 * WS + o]) + smem_f[3 * WS + o];
    const float base = D ? D[m * g.ldd + n] : 0.0f;
    C[m * g.ldc + n] = base + g.alpha * sum;
  }
}


__device__ __forceinline__ float sig_acc(float x) { return 1.0f / (1.0f + expf(-x)); }

// The two-matrix MLP learner f(x) = W2 silu(W1 x) (§5.2) runs through the same
// steps on the state laid out as [W1 | W3 = 0 | W2] with gated = 0: the gate
// a3 is held at one, so u3, du3 and da3 are zero and the W3 block of every
// state adjoint stays zero.

// Z = silu(a1) * a3 for n rows of H = [a1 | a3] (row length 2h), per unit
// (a3 = 1 when gated = 0).
__global__ __launch_bounds__(256) void k_swb_act(int64_t BH, int64_t n, int64_t h,
                                                 int64_t ustride, int gated,
                                                 const float* __restrict__ H,
                                                 float* __restrict__ Z) {
  const int64_t per = n * h;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= BH * per) return;
  const int64_t u = i / per, rem = i % per, t = rem / h, j = rem % h;
  const float* hr = H + u * ustride * 2 * h + t * 2 * h;
  const float a1 = hr[j], a3 = gated ? hr[h + j] : 1.0f;
  Z[u * ustride * h + t * h + j] = a1 * sig_acc(a1) * a3;
}

struct SwbTokArgs {
  int64_t n, d, h, Cp, nC;
  int r, gated;
  const float *HK, *WV, *E, *TW, *TM, *SW, *SM, *RW, *RM, *kw, *km;
  float *sw, *sm, *DU, *DW, *DEA, *DZA, *UW, *UM;
};

// One workgroup per (unit, token): dK^W, dK^M and the token's adjoint vectors.
__global__ __launch_bounds__(256) void k_swb_tok(SwbTokArgs a) {
  __shared__ float red[2][256];
  const int64_t u = blockIdx.x / a.n, t = blockIdx.x % a.n;
  const int tid = threadIdx.x;
  const int64_t h = a.h, d = a.d;
  const int64_t rh = (u * a.Cp + t) * h, r2 = 2 * rh, rd = (u * a.Cp + t) * d;
  const int64_t seg = u * a.nC + a.r;
  const float kwt = a.kw[seg * a.Cp + t], kmt = a.km[seg * a.Cp + t];
  float pW = 0.0f, pM = 0.0f;
  for (int64_t i = tid; i < h; i += 256) {
    const float a1 = a.HK[r2 + i], a3 = a.gated ? a.HK[r2 + h + i] : 1.0f, w = a.WV[rh + i];
    const float sg = sig_acc(a1), sl = a1 * sg, sp = sg * (1.0f + a1 * (1.0f - sg));
    const float u1 = w * a3 * sp, u3 = a.gated ? w * sl : 0.0f;
    const float tw1 = a.TW[r2 + i], tw3 = a.TW[r2 + h + i];
    const float tm1 = a.TM[r2 + i], tm3 = a.TM[r2 + h + i];
    pW += u1 * tw1 + u3 * tw3;
    pM += u1 * tm1 + u3 * tm3;
    const float du1 = kwt * tw1 + kmt * tm1;
    const float du3 = a.gated ? kwt * tw3 + kmt * tm3 : 0.0f;
    a.DU[r2 + i] = du1;
    a.DU[r2 + h + i] = du3;
    a.DW[rh + i] = du3 * sl + du1 * a3 * sp;
    a.UW[r2 + i] = kwt * u1;
    a.UW[r2 + h + i] = kwt * u3;
    a.UM[r2 + i] = kmt * u1;
    a.UM[r2 + h + i] = kmt * u3;
    a.DZA[rh + i] = kwt * a.RW[rh + i] + kmt * a.RM[rh + i];
  }
  for (int64_t o = tid; o < d; o += 256) {
    const float e = a.E[rd + o], sw = a.SW[rd + o], sm = a.SM[rd + o];
    pW += e * sw;
    pM += e * sm;
    a.DEA[rd + o] = kwt * sw + kmt * sm;
  }
  red[0][tid] = pW;
  red[1][tid] = pM;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) {
      red[0][tid] += red[0][tid + off];
      red[1][tid] += red[1][tid + off];
    }
    __syncthreads();
  }
  if (tid == 0) {
    a.sw[seg * a.Cp + t] = red[0][0];
    a.sm[seg * a.Cp + t] = red[1][0];
  }
}

// [da1 | da3] of the key rows (from a1, a3, w, du1, du3, dz) and of the query
// rows (readout: from a1, a3 and dz = W2^T dout); da3 = 0 when gated = 0.
__global__ __launch_bounds__(256) void k_swb_da(int64_t BH, int64_t n, int64_t h, int64_t Cp,
                                                int gated,
                                                const float* __restrict__ HK,
                                                const float* __restrict__ WV,
                                                const float* __restrict__ DU,
                                                const float* __restrict__ DZ,
                                                const float* __restrict__ HQ,
                                                const float* __restrict__ DZQ,
                                                float* __restrict__ DA, float* __restrict__ DAQ) {
  const int64_t per = n * h;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= BH * per) return;
  const int64_t u = i / per, rem = i % per, t = rem / h, j = rem % h;
  const int64_t rh = (u * Cp + t) * h, r2 = 2 * rh;
  {
    const float a1 = HK[r2 + j], a3 = gated ? HK[r2 + h + j] : 1.0f, w = WV[rh + j];
    const float du1 = DU[r2 + j], du3 = DU[r2 + h + j], dz = DZ[rh + j];
    const float sg = sig_acc(a1), sl = a1 * sg, sp = sg * (1.0f + a1 * (1.0f - sg));
    const float spp = sg * (1.0f - sg) * (2.0f + a1 * (1.0f - 2.0f * sg));
    DA[r2 + j] = du3 * w * sp + du1 * w * a3 * spp + dz * a3 * sp;
    DA[r2 + h + j] = gated ? du1 * w * sp + dz * sl : 0.0f;
  }
  {
    const float a1 = HQ[r2 + j], a3 = gated ? HQ[r2 + h + j] : 1.0f, dz = DZQ[rh + j];
    const float sg = sig_acc(a1), sl = a1 * sg, sp = sg * (1.0f + a1 * (1.0f - sg));
    DAQ[r2 + j] = dz * a3 * sp;
    DAQ[r2 + h + j] = gated ? dz * sl : 0.0f;
  }
}

constexpr int SWB_STATE_ELEMS = 1024;  // state entries per workgroup of k_swb_state

// dW_prev = cW dW_C, dM_prev = cWM dW_C + cM dM_C (the token sums are added
// afterwards), and this block's partial sums of <dW_C, Ws>, <dM_C, Ms>,
// <dW_C, Ms> (added in block order later, so results do not depend on
// scheduling).  Grid: BH * nrb workgroups, nrb = ceil(P / 1024).
__global__ __launch_bounds__(256) void k_swb_state(int64_t P, int64_t nrb, int64_t nC, int r,
                                                   const float* __restrict__ coef,
                                                   const float* __restrict__ Ws,
                                                   const float* __restrict__ Ms,
                                                   const float* __restrict__ dWC,
                                                   const float* __restrict__ dMC, float* dWp,
                                                   float* dMp, float* __restrict__ dots) {
  __shared__ float red[3][256];
  const int64_t u = blockIdx.x / nrb, rb = blockIdx.x % nrb;
  const int tid = threadIdx.x;
  const float* cf = coef + (u * nC + r) * 4;
  const float cW = cf[0], cM = cf[1], cWM = cf[2];
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f;
  for (int l = 0; l < SWB_STATE_ELEMS / 256; ++l) {
    const int64_t p = rb * SWB_STATE_ELEMS + l * 256 + tid;
    if (p >= P) break;
    const int64_t x = u * P + p;
    const float dw = dWC[x], dm = dMC[x], ws = Ws[x], ms = Ms[x];
    s0 += dw * ws;
    s1 += dm * ms;
    s2 += dw * ms;
    dWp[x] = cW * dw;
    dMp[x] = cWM * dw + cM * dm;
  }
  red[0][tid] = s0;
  red[1][tid] = s1;
  red[2][tid] = s2;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off)
      for (int c = 0; c < 3; ++c) red[c][tid] += red[c][tid + off];
    __syncthreads();
  }
  if (tid < 3) dots[((u * nC + r) * nrb + rb) * 4 + tid] = red[tid][0];
}

}  // namespace e2ttt
