// fused.hpp -- two-kernel chunk step of the SwiGLU learner for head dim 128,
// bf16 operands (gfx950 MFMA 32x32x16).
//
// "Rethinking Expressivity and Efficiency in Test-Time Training" (E2-TTT):
// every per-token gradient of a chunk is taken at the chunk-start weights
// (§3), so each token's forward and backward are independent, and the two
// weighted aggregations of §3.2 / App. A.4 sum rank-one terms over tokens.
//
// Phase A (k_phaseA): one workgroup per block of RB rows of [K; Q] of one
//   (batch, head) unit.  It streams the hidden units in blocks: A1, A3 of the
//   block (MFMA against the W1/W3 shadow), Z = silu(A1) * A3 kept in LDS, and
//   Y += Z W2[:, block]^T.  Q rows: the readout o = Y (Eq. 6).  K rows: the
//   activation gradient g = v - Y (fp32, token-major) for phase B.
// Phase B (k_phaseB): one workgroup per block of 32 hidden units i of one
//   unit.  Hidden unit i owns row i of W1 and W3 and column i of W2, so the
//   state is partitioned with no overlap.  For tiles of 32 tokens it
//   recomputes A1, A3 (K W1[I]^T, K W3[I]^T) and dZ = g W2[:, I], forms
//   dA1 = dZ A3 silu'(A1), dA3 = dZ silu(A1), Z = silu(A1) A3, and feeds them
//   straight into the aggregations over the tile's tokens:
//     A^W_{W1}[I,:] += (K^W dA1)^T K,  A^M_{W1}[I,:] += (K^M dA1)^T K
//     A^W_{W3}[I,:], A^M_{W3}[I,:] likewise with dA3
//     A^W_{W2}[:,I] += (K^W g)^T Z,   A^M_{W2}[:,I] += (K^M g)^T Z
//   and ends with the chunk-end state W_C = cW W_0 + cWM M_0 + A^W,
//   M_C = cM M_0 + A^M and the next chunk's operand shadows.
// The per-token scale multiplies the fp32 factor (dA1, dA3, g) before its
// single rounding to bf16; K enters exactly (it is bf16 already).
#pragma once
#include "common.hpp"

namespace e2ttt {

constexpr int FD = 128;  // head dim of the fused path

struct FusedArgs {
  int64_t BH, L, h, C, Cp, nC;
  int krep;   // 1, or 2 for hi/lo weight operands
  int r;      // chunk index
  int last;   // 1 on the last chunk (no shadow update)
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* out;
  const float* kw;    // [BH][nC][Cp]
  const float* km;
  const float* coef;  // [BH][nC][4]
  const float* Win;
  const float* Min;
  float* Wout;
  float* Mout;
  bf16_t* w13s;  // [BH][2h][krep*FD]
  bf16_t* w2s;   // [BH][FD][krep*h]
  bf16_t* w2ts;  // [BH][h][krep*FD]
  float* gf;     // [BH][Cp][FD] fp32 residuals of the chunk's K rows
};

__device__ __forceinline__ int64_t fused_nvalid(const FusedArgs& a) {
  const int64_t rem = a.L - static_cast<int64_t>(a.r) * a.C;
  return rem < a.C ? rem : a.C;
}

// Copy `rows` rows of `cols` bf16 (cols % 8 == 0) from global (row stride gs,
// null row pointer -> zeros) into LDS (row stride ls) with 16-byte vectors.
template <typename RowPtr>
__device__ __forceinline__ void copy_rows_bf16(bf16_t* lds, int ls, int rows, int cols,
                                               RowPtr rowp) {
  const int vpr = cols / 8;
  for (int idx = threadIdx.x; idx < rows * vpr; idx += blockDim.x) {
    const int rr = idx / vpr, c = idx % vpr;
    const bf16_t* src = rowp(rr);
    uint4 val = src ? *reinterpret_cast<const uint4*>(src + c * 8) : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(lds + rr * ls + c * 8) = val;
  }
}

// One 32x32 MFMA block: acc += A[32 x K] * B[32 x K]^T, both row-major in LDS
// (row strides la, lb elements), K a multiple of 16.
__device__ __forceinline__ void mma_32x32(f32x16_t& acc, const bf16_t* A, int la,
                                          const bf16_t* B, int lb, int K) {
  const int lane = threadIdx.x & 63;
  const int r32 = lane & 31, hf = lane >> 5;
  const bf16_t* pa = A + r32 * la + hf * 8;
  const bf16_t* pb = B + r32 * lb + hf * 8;
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(pa + k0),
                                                  *reinterpret_cast<const bf16x8_t*>(pb + k0),
                                                  acc, 0, 0, 0);
  }
}

// Same with the A operand's k index wrapping at ka (hi/lo split B operand).
__device__ __forceinline__ void mma_32x32_wrapA(f32x16_t& acc, const bf16_t* A, int la, int ka,
                                                const bf16_t* B, int lb, int K) {
  const int lane = threadIdx.x & 63;
  const int r32 = lane & 31, hf = lane >> 5;
  const bf16_t* pa = A + r32 * la + hf * 8;
  const bf16_t* pb = B + r32 * lb + hf * 8;
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int ka0 = k0 < ka ? k0 : k0 - ka;
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(pa + ka0),
                                                  *reinterpret_cast<const bf16x8_t*>(pb + k0),
                                                  acc, 0, 0, 0);
  }
}

__device__ __forceinline__ void zero16(f32x16_t& a) {
#pragma unroll
  for (int v = 0; v < 16; ++v) a[v] = 0.0f;
}

// Row of a 32x32 accumulator held by this lane for register v.
__device__ __forceinline__ int acc_row(int v) {
  const int hf = (threadIdx.x & 63) >> 5;
  return 8 * (v >> 2) + 4 * hf + (v & 3);
}
__device__ __forceinline__ int acc_col() { return threadIdx.x & 31; }

// ---------------------------------------------------------------------------
// Phase A.  RB = 64: waves 2 (rows) x 2 (cols); a hidden block is 64 units
// (128 shadow columns).  RB = 32: waves 1 x 4; a hidden block is 128 units.
template <int RB>
__global__ __launch_bounds__(256) void k_phaseA(FusedArgs a) {
  constexpr int WM = RB / 32;           // waves along rows
  constexpr int WN = 4 / WM;            // waves along columns
  constexpr int HBK = WN * 32;          // hidden units per block
  constexpr int NS = 2 * HBK;           // shadow rows (W1/W3 interleaved) per block
  constexpr int XW = FD + 8;            // X tile row stride
  constexpr int ZW = HBK + 8;           // Z tile row stride
  constexpr int YN = FD / WN;           // Y columns per wave (64 or 32)
  const int kd = a.krep * FD;           // contraction length of GEMM1 (with hi/lo)
  const int W13W = kd + 8;              // W13 block row stride
  const int kh = a.krep * HBK;          // contraction length of GEMM2 per block
  const int W2W = kh + 8;

  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  bf16_t* Xs = reinterpret_cast<bf16_t*>(smem_raw);
  bf16_t* W13b = Xs + RB * XW;
  bf16_t* Zs = W13b + NS * W13W;
  bf16_t* W2b = Zs + RB * ZW;

  const int64_t nrb = 2 * a.Cp / RB, krb = a.Cp / RB;
  const int64_t u = blockIdx.x / nrb;
  const int64_t mb = blockIdx.x % nrb;
  const bool isQ = mb >= krb;
  const int64_t p0 = (mb - (isQ ? krb : 0)) * RB;
  const int64_t tok0 = static_cast<int64_t>(a.r) * a.C;
  const int64_t nv = fused_nvalid(a);
  const bf16_t* X = (isQ ? a.q : a.k) + (u * a.L + tok0) * FD;
  const bf16_t* W13 = a.w13s + u * 2 * a.h * kd;
  const bf16_t* W2 = a.w2s + u * FD * (a.krep * a.h);
  const int64_t w2ld = a.krep * a.h;

  const int wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;

  copy_rows_bf16(Xs, XW, RB, FD, [&](int rr) -> const bf16_t* {
    return p0 + rr < nv ? X + (p0 + rr) * FD : nullptr;
  });

  f32x16_t yacc[YN / 32];
#pragma unroll
  for (int i = 0; i < YN / 32; ++i) zero16(yacc[i]);

  const int nhb = static_cast<int>(a.h / HBK);
  for (int hb = 0; hb < nhb; ++hb) {
    // Stage this block's W13 rows (NS x kd) and W2 columns (FD x kh).
    __syncthreads();  // previous block's GEMM2 is done with Zs/W2b/W13b
    copy_rows_bf16(W13b, W13W, NS, kd, [&](int rr) -> const bf16_t* {
      return W13 + (static_cast<int64_t>(hb) * NS + rr) * kd;
    });
    // W2 block: row j holds [hi cols hb*HBK.. +HBK | lo cols h + hb*HBK .. +HBK]
    {
      const int vpr = HBK / 8;
      for (int idx = threadIdx.x; idx < FD * a.krep * vpr; idx += blockDim.x) {
        const int rr = idx / (a.krep * vpr), rem = idx % (a.krep * vpr);
        const int part = rem / vpr, c = rem % vpr;
        const bf16_t* src = W2 + rr * w2ld + part * a.h + hb * HBK + c * 8;
        *reinterpret_cast<uint4*>(W2b + rr * W2W + part * HBK + c * 8) =
            *reinterpret_cast<const uint4*>(src);
      }
    }
    __syncthreads();
    // GEMM1: this wave's 32 rows x (32 A1 + 32 A3) columns.
    f32x16_t a1, a3;
    zero16(a1);
    zero16(a3);
    const bf16_t* Ar = Xs + wm * 32 * XW;
    const bf16_t* B1 = W13b + (wn * 64) * W13W;
    mma_32x32_wrapA(a1, Ar, XW, FD, B1, W13W, kd);
    mma_32x32_wrapA(a3, Ar, XW, FD, B1 + 32 * W13W, W13W, kd);
    // Z = silu(A1) * A3 -> Zs[row][hidden in block]
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float x1 = a1[v];
      const float z = x1 * sigmoidf_(x1) * a3[v];
      Zs[(wm * 32 + acc_row(v)) * ZW + wn * 32 + acc_col()] = f2bf(z);
    }
    __syncthreads();
    // GEMM2: Y[32 rows of wm][YN cols of wn] += Z[rows][HBK] W2b[cols][HBK]^T
#pragma unroll
    for (int i = 0; i < YN / 32; ++i)
      mma_32x32_wrapA(yacc[i], Zs + wm * 32 * ZW, ZW, HBK, W2b + (wn * YN + i * 32) * W2W, W2W,
                      kh);
  }

  // Epilogue.
#pragma unroll
  for (int i = 0; i < YN / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t p = p0 + wm * 32 + acc_row(v);
      const int64_t j = wn * YN + i * 32 + acc_col();
      const float y = yacc[i][v];
      if (isQ) {
        if (p < nv) a.out[(u * a.L + tok0 + p) * FD + j] = f2bf(y);
      } else {
        const float vin = p < nv ? bf2f(a.v[(u * a.L + tok0 + p) * FD + j]) : 0.0f;
        a.gf[(u * a.Cp + p) * FD + j] = vin - y;
      }
    }
}

template <int RB>
size_t phaseA_lds_bytes(int krep) {
  constexpr int WM = RB / 32, WN = 4 / WM, HBK = WN * 32, NS = 2 * HBK;
  const size_t e = static_cast<size_t>(RB) * (FD + 8) + static_cast<size_t>(NS) * (krep * FD + 8) +
                   static_cast<size_t>(RB) * (HBK + 8) +
                   static_cast<size_t>(FD) * (krep * HBK + 8);
  return e * sizeof(bf16_t);
}

// ---------------------------------------------------------------------------
// Phase B.  One workgroup per (unit, block I of 32 hidden units); wave w owns
// output columns j in [32w, 32w+32) of the W1/W3 aggregates and rows j of the
// W2 aggregate.  Token tiles of TB = 32.
struct PhaseBLds {
  static constexpr int TB = 32;
  static constexpr int KW_ = FD + 8;   // token-major K / g tiles
  static constexpr int TW = TB + 8;    // feature-major tiles (row = feature)
};

__device__ __forceinline__ void state_update_store(const FusedArgs& a, int64_t u, int64_t off,
                                                   float aw, float am, float cW, float cM,
                                                   float cWM, int shadow_kind, int64_t srow,
                                                   int64_t scol) {
  const int64_t P = 3 * FD * a.h;
  const float w0 = a.Win[u * P + off], m0 = a.Min[u * P + off];
  const float wn = cW * w0 + cWM * m0 + aw;
  const float mn = cM * m0 + am;
  a.Wout[u * P + off] = wn;
  a.Mout[u * P + off] = mn;
  if (a.last) return;
  const bf16_t hi = f2bf(wn);
  const bf16_t lo = a.krep == 2 ? f2bf(wn - bf2f(hi)) : bf16_t(0);
  if (shadow_kind == 0) {  // W1 or W3 entry: shadow row srow, column scol (d index)
    bf16_t* b = a.w13s + (u * 2 * a.h + srow) * (a.krep * FD);
    b[scol] = hi;
    if (a.krep == 2) b[FD + scol] = lo;
  } else {  // W2 entry (j = srow, i = scol)
    bf16_t* b2 = a.w2s + (u * FD + srow) * (a.krep * a.h);
    b2[scol] = hi;
    if (a.krep == 2) b2[a.h + scol] = lo;
    bf16_t* bt = a.w2ts + (u * a.h + scol) * (a.krep * FD);
    bt[srow] = hi;
    if (a.krep == 2) bt[FD + srow] = lo;
  }
}

__global__ __launch_bounds__(256) void k_phaseB(FusedArgs a) {
  typedef PhaseBLds S;
  constexpr int TB = S::TB, KW_ = S::KW_, TW = S::TW;
  const int kd = a.krep * FD;
  const int WW = kd + 8;  // weight slice row stride

  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  bf16_t* W1I = reinterpret_cast<bf16_t*>(smem_raw);  // [32][WW]
  bf16_t* W3I = W1I + 32 * WW;
  bf16_t* W2I = W3I + 32 * WW;                         // W2^T rows of I
  bf16_t* Ks = W2I + 32 * WW;                          // [TB][KW_] token-major K
  bf16_t* KT = Ks + TB * KW_;                          // [FD][TW] feature-major K
  bf16_t* Gs = KT + FD * TW;                           // [TB][KW_] bf16(g)
  bf16_t* GTW = Gs + TB * KW_;                         // [FD][TW] bf16(K^W g)
  bf16_t* GTM = GTW + FD * TW;                         // [FD][TW] bf16(K^M g)
  bf16_t* DA = GTM + FD * TW;                          // 4 x [32][TW]: dA1 W,M, dA3 W,M
  bf16_t* ZT = DA + 4 * 32 * TW;                       // [32][TW] Z^T
  float* R = reinterpret_cast<float*>(ZT + 32 * TW);   // 3 x [TB][33]: A1, A3, dZ
  float* ksc = R + 3 * TB * 33;                        // [2][TB] K^W, K^M of the tile

  const int64_t nib = a.h / 32;
  const int64_t u = blockIdx.x / nib;
  const int64_t ib = blockIdx.x % nib;
  const int64_t tok0 = static_cast<int64_t>(a.r) * a.C;
  const int64_t nv = fused_nvalid(a);
  const int wave = threadIdx.x >> 6;
  const int tid = threadIdx.x;

  // Weight slices of this hidden block (rows of the operand shadows).
  {
    const bf16_t* w13 = a.w13s + u * 2 * a.h * kd;
    copy_rows_bf16(W1I, WW, 32, kd, [&](int rr) -> const bf16_t* {
      return w13 + (64 * ib + rr) * kd;
    });
    copy_rows_bf16(W3I, WW, 32, kd, [&](int rr) -> const bf16_t* {
      return w13 + (64 * ib + 32 + rr) * kd;
    });
    const bf16_t* w2t = a.w2ts + u * a.h * kd;
    copy_rows_bf16(W2I, WW, 32, kd, [&](int rr) -> const bf16_t* {
      return w2t + (32 * ib + rr) * kd;
    });
  }

  f32x16_t acc[6];  // W1^W, W1^M, W3^W, W3^M (rows i, cols j of wave), W2^W, W2^M (rows j, cols i)
#pragma unroll
  for (int q = 0; q < 6; ++q) zero16(acc[q]);

  const bf16_t* Kg = a.k + (u * a.L + tok0) * FD;
  const float* gfu = a.gf + u * a.Cp * FD;
  const float* kwr = a.kw + (u * a.nC + a.r) * a.Cp;
  const float* kmr = a.km + (u * a.nC + a.r) * a.Cp;

  for (int64_t t0 = 0; t0 < a.Cp; t0 += TB) {
    __syncthreads();  // previous tile fully consumed
    // K tile: token-major (recompute operand) and feature-major (aggregation operand).
    for (int idx = tid; idx < TB * (FD / 8); idx += 256) {
      const int tr = idx / (FD / 8), c = idx % (FD / 8);
      const int64_t p = t0 + tr;
      uint4 val = p < nv ? *reinterpret_cast<const uint4*>(Kg + p * FD + c * 8)
                         : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(Ks + tr * KW_ + c * 8) = val;
      const bf16_t* e = reinterpret_cast<const bf16_t*>(&val);
#pragma unroll
      for (int x = 0; x < 8; ++x) KT[(c * 8 + x) * TW + tr] = e[x];
    }
    if (tid < TB) {
      ksc[tid] = kwr[t0 + tid];
      ksc[TB + tid] = kmr[t0 + tid];
    }
    __syncthreads();
    // g tile (fp32): bf16 token-major, and K^W / K^M scaled feature-major.
    for (int idx = tid; idx < TB * (FD / 4); idx += 256) {
      const int tr = idx / (FD / 4), c = idx % (FD / 4);
      const float4 g4 = *reinterpret_cast<const float4*>(gfu + (t0 + tr) * FD + c * 4);
      const float gv[4] = {g4.x, g4.y, g4.z, g4.w};
      const float sw = ksc[tr], sm = ksc[TB + tr];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int j = c * 4 + x;
        Gs[tr * KW_ + j] = f2bf(gv[x]);
        GTW[j * TW + tr] = f2bf(sw * gv[x]);
        GTM[j * TW + tr] = f2bf(sm * gv[x]);
      }
    }
    __syncthreads();
    // Recompute A1, A3 (waves 0, 1) and dZ (wave 2) for the tile: [TB x 32 hidden].
    if (wave < 3) {
      f32x16_t racc;
      zero16(racc);
      const bf16_t* Aop = wave == 2 ? Gs : Ks;
      const bf16_t* Bop = wave == 0 ? W1I : (wave == 1 ? W3I : W2I);
      mma_32x32_wrapA(racc, Aop, KW_, FD, Bop, WW, kd);
      float* Rq = R + wave * TB * 33;
#pragma unroll
      for (int v = 0; v < 16; ++v) Rq[acc_row(v) * 33 + acc_col()] = racc[v];
    }
    __syncthreads();
    // Elementwise: dA1, dA3 scaled by both kernels, and Z, written feature-major.
    for (int idx = tid; idx < TB * 32; idx += 256) {
      const int tr = idx / 32, i = idx % 32;
      const float x1 = R[tr * 33 + i], x3 = R[TB * 33 + tr * 33 + i];
      const float dz = R[2 * TB * 33 + tr * 33 + i];
      const float sg = sigmoidf_(x1);
      const float d3 = dz * (x1 * sg);
      const float d1 = dz * x3 * (sg * (1.0f + x1 * (1.0f - sg)));
      const float sw = ksc[tr], sm = ksc[TB + tr];
      DA[0 * 32 * TW + i * TW + tr] = f2bf(sw * d1);
      DA[1 * 32 * TW + i * TW + tr] = f2bf(sm * d1);
      DA[2 * 32 * TW + i * TW + tr] = f2bf(sw * d3);
      DA[3 * 32 * TW + i * TW + tr] = f2bf(sm * d3);
      ZT[i * TW + tr] = f2bf(x1 * sg * x3);
    }
    __syncthreads();
    // Aggregations over the tile's tokens.
    const bf16_t* KTw = KT + (wave * 32) * TW;  // B rows j of this wave
#pragma unroll
    for (int q = 0; q < 4; ++q) mma_32x32(acc[q], DA + q * 32 * TW, TW, KTw, TW, TB);
    mma_32x32(acc[4], GTW + (wave * 32) * TW, TW, ZT, TW, TB);
    mma_32x32(acc[5], GTM + (wave * 32) * TW, TW, ZT, TW, TB);
  }

  // Chunk-end state and operand shadows of this hidden block.
  const float* cf = a.coef + (u * a.nC + a.r) * 4;
  const float cW = cf[0], cM = cf[1], cWM = cf[2];
  const int64_t jc = wave * 32 + acc_col();
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t i = 32 * ib + acc_row(v);  // hidden unit (rows of acc 0..3)
    // W1[i][jc], W3[i][jc]
    state_update_store(a, u, i * FD + jc, acc[0][v], acc[1][v], cW, cM, cWM, 0,
                       64 * ib + acc_row(v), jc);
    state_update_store(a, u, a.h * FD + i * FD + jc, acc[2][v], acc[3][v], cW, cM, cWM, 0,
                       64 * ib + 32 + acc_row(v), jc);
    // W2[j][i]: acc 4/5 rows are j (wave*32 + acc_row), cols i (acc_col)
    const int64_t j2 = wave * 32 + acc_row(v);
    const int64_t i2 = 32 * ib + acc_col();
    state_update_store(a, u, 2 * a.h * FD + j2 * a.h + i2, acc[4][v], acc[5][v], cW, cM, cWM, 1,
                       j2, i2);
  }
}

inline size_t phaseB_lds_bytes(int krep) {
  typedef PhaseBLds S;
  const size_t ww = static_cast<size_t>(krep) * FD + 8;
  const size_t bf = 3 * 32 * ww + 2 * S::TB * S::KW_ + 3 * FD * S::TW + 5 * 32 * S::TW;
  return bf * sizeof(bf16_t) + (3 * S::TB * 33 + 2 * S::TB) * sizeof(float);
}

}  // namespace e2ttt
