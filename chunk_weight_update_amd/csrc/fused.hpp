// fused.hpp -- two-kernel chunk step of the SwiGLU learner for head dim 128,
// bf16 operands (gfx950 MFMA).
//
// "Rethinking Expressivity and Efficiency in Test-Time Training" (E2-TTT):
// every per-token gradient of a chunk is taken at the chunk-start weights
// (§3), so each token's forward and backward are independent, and the two
// weighted aggregations of §3.2 / App. A.4 sum rank-one terms over tokens.
//
// Phase A (k_phaseA): one workgroup per block of RB rows of [K; Q] of one
//   (batch, head) unit.  It streams the hidden units in blocks: A1, A3 of the
//   block (MFMA against the W1/W3 operand shadow), Z = silu(A1) * A3 in LDS,
//   Y += Z W2[:, block]^T.  Q rows: the readout o = Y (Eq. 6).  K rows: the
//   activation gradient g = v - Y, rounded once to bf16 and written
//   token-major (operand of the backward) and feature-major (operand of the
//   W2 aggregation).  Feature-major buffers keep the token order of
//   tok_perm32 inside each group of 32 tokens.
// Phase B (k_phaseB): one workgroup per block of 64 hidden units of one unit;
//   wave w owns 16 hidden units i.  Hidden unit i owns row i of W1 and W3 and
//   column i of W2, so waves and workgroups write disjoint state.  Per tile
//   of 32 tokens a wave recomputes A1, A3 = K W1[i]^T, K W3[i]^T and
//   dZ = g W2[:, i] (16x16x32 MFMAs), forms dA1 = dZ A3 silu'(A1),
//   dA3 = dZ silu(A1), Z = silu(A1) A3 in registers, and feeds them without
//   leaving registers into the aggregations over the tile's tokens, the
//   per-token kernels folded into the register-side operand:
//     A^W_{W1}[i,:] += (K^W dA1)^T K,  A^M_{W1}[i,:] += (K^M dA1)^T K
//     A^W_{W3}[i,:], A^M_{W3}[i,:] likewise with dA3
//     A^W_{W2}[:,i] += g^T (K^W Z),    A^M_{W2}[:,i] += g^T (K^M Z)
//   This works because a 16x16 accumulator gives lane l the column l%16 and
//   rows 4*(l/16)+v: a lane holds one hidden unit for 8 tokens of the tile,
//   which is exactly an operand fragment of a 16x16x32 MFMA that contracts
//   over tokens, once the partner operand (K or g, feature-major in LDS) is
//   read with the same token order.  The chunk-end state
//   W_C = cW W_0 + cWM M_0 + A^W, M_C = cM M_0 + A^M and the next chunk's
//   operand shadows are written at the end.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace e2ttt {

constexpr int FD = 128;  // head dim of the fused path

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct FusedArgs {
  int64_t BH, L, h, C, Cp, nC;
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
  bf16_t* w13s;       // [BH][2h][KREP*FD]
  bf16_t* w2s;        // [BH][FD][KREP*h]
  bf16_t* w2ts;       // [BH][h][KREP*FD]
  const bf16_t* kt;   // [BH][nC][FD][Cp]  K feature-major
  bf16_t* gbf;        // [BH][Cp][FD]      bf16(g), token-major
  bf16_t* gft;        // [BH][FD][Cp]      bf16(g), feature-major
  int nsplit;         // phase B token split (1: fused state epilogue)
  int krep;           // 2 with hi/lo operand shadows
  float* part;        // [BH*h/64][nsplit][48][256] x 4 floats: phase B partial sums
};

__device__ __forceinline__ int64_t fused_nvalid(const FusedArgs& a) {
  const int64_t rem = a.L - static_cast<int64_t>(a.r) * a.C;
  return rem < a.C ? rem : a.C;
}

// Tile copy global -> registers -> LDS with compile-time counts, so that all
// of a thread's global loads are in flight together.  ROWS x COLS bf16
// (COLS % 8 == 0); row rr comes from rowp(rr) (nullptr -> zeros) and lands at
// lds + rr * LS.
template <int ROWS, int COLS, int NT>
struct TileCopy {
  static constexpr int VPR = COLS / 8;
  static constexpr int TOTAL = ROWS * VPR;
  static constexpr int PER = (TOTAL + NT - 1) / NT;
  // One wide vector value rather than an array, so the compiler keeps the
  // prefetched data in registers across loop iterations (an array of uint4
  // held across the loop was demoted to scratch memory).
  typedef uint32_t regs_t __attribute__((ext_vector_type(4 * PER)));
  regs_t reg;
  __device__ __forceinline__ void put(int i, uint4 v) {
    reg[4 * i + 0] = v.x; reg[4 * i + 1] = v.y; reg[4 * i + 2] = v.z; reg[4 * i + 3] = v.w;
  }
  __device__ __forceinline__ uint4 get(int i) const {
    return make_uint4(reg[4 * i + 0], reg[4 * i + 1], reg[4 * i + 2], reg[4 * i + 3]);
  }
  // Branch-free: a null row loads from `dummy` (any valid address) and the
  // value is replaced by zeros, so all loads issue back to back.
  template <typename RowPtr>
  __device__ __forceinline__ void load(RowPtr rowp, const bf16_t* dummy) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = threadIdx.x + i * NT;
      if (TOTAL % NT == 0 || idx < TOTAL) {
        const bf16_t* src = rowp(idx / VPR);
        const bool ok = src != nullptr;
        const uint4 val = *reinterpret_cast<const uint4*>(ok ? src + (idx % VPR) * 8 : dummy);
        put(i, ok ? val : make_uint4(0u, 0u, 0u, 0u));
      }
    }
  }
  template <typename RowPtr>
  __device__ __forceinline__ void load(RowPtr rowp) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = threadIdx.x + i * NT;
      if (TOTAL % NT == 0 || idx < TOTAL)
        put(i, *reinterpret_cast<const uint4*>(rowp(idx / VPR) + (idx % VPR) * 8));
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds, int LS) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = threadIdx.x + i * NT;
      if (TOTAL % NT == 0 || idx < TOTAL)
        *reinterpret_cast<uint4*>(lds + (idx / VPR) * LS + (idx % VPR) * 8) = get(i);
    }
  }
};

__device__ __forceinline__ void zero16(f32x16_t& a) {
#pragma unroll
  for (int v = 0; v < 16; ++v) a[v] = 0.0f;
}
__device__ __forceinline__ void zero4(f32x4_t& a) {
#pragma unroll
  for (int v = 0; v < 4; ++v) a[v] = 0.0f;
}

// acc += A[32 x K] * B[32 x K]^T from LDS (row strides la, lb); A's k index
// wraps at ka (hi/lo split B operand repeats the same A).
template <int K, int KA>
__device__ __forceinline__ void mma32_lds(f32x16_t& acc, const bf16_t* A, int la,
                                          const bf16_t* B, int lb) {
  const int lane = threadIdx.x & 63;
  const bf16_t* pa = A + (lane & 31) * la + (lane >> 5) * 8;
  const bf16_t* pb = B + (lane & 31) * lb + (lane >> 5) * 8;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        *reinterpret_cast<const bf16x8_t*>(pa + (k0 % KA)),
        *reinterpret_cast<const bf16x8_t*>(pb + k0), acc, 0, 0, 0);
  }
}

// Row of a 32x32 accumulator held by this lane for register v; column = lane%32.
__device__ __forceinline__ int acc32_row(int v) {
  return 8 * (v >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (v & 3);
}

// ---------------------------------------------------------------------------
// Phase A.  RB = 64: waves 2 (rows) x 2 (cols), hidden block of 64 units.
// RB = 32: waves 1 x 4, hidden block of 128 units.
template <int RB, int KREP> struct PhaseACfg {
  static constexpr int WM = RB / 32, WN = 4 / WM;
  static constexpr int HBK = WN * 32;       // hidden units per block
  static constexpr int NS = 2 * HBK;        // shadow rows per block (W1/W3 interleaved)
  static constexpr int KD = KREP * FD;      // GEMM1 contraction (with hi/lo)
  static constexpr int KH = KREP * HBK;     // GEMM2 contraction per block
  static constexpr int XW = FD + 8, W13W = KD + 8, ZW = HBK + 8, W2W = KH + 8;
  static constexpr int YN = FD / WN;        // Y columns per wave
  static constexpr int GW = RB + 8;         // transposed g staging row stride
  static constexpr size_t LDS_ELEMS = static_cast<size_t>(RB) * XW + static_cast<size_t>(NS) * W13W +
                                      static_cast<size_t>(RB) * ZW + static_cast<size_t>(FD) * W2W;
  static constexpr size_t LDS_BYTES = LDS_ELEMS * sizeof(bf16_t);
};

// One or two workgroups fit a CU (dynamic LDS), so let the compiler use up to
// 256 VGPRs instead of spilling the prefetch registers for an occupancy the
// LDS budget rules out anyway.
template <int RB, int KREP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_phaseA(
    FusedArgs a) {
  typedef PhaseACfg<RB, KREP> P;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  bf16_t* Xs = reinterpret_cast<bf16_t*>(smem_raw);
  bf16_t* W13b = Xs + RB * P::XW;
  bf16_t* Zs = W13b + P::NS * P::W13W;
  bf16_t* W2b = Zs + RB * P::ZW;

  const int64_t nrb = 2 * a.Cp / RB, krb = a.Cp / RB;
  const int64_t bid = xcd_logical_block();  // a unit's row blocks share one XCD's L2
  const int64_t u = bid / nrb;
  const int64_t mb = bid % nrb;
  const bool isQ = mb >= krb;
  const int64_t p0 = (mb - (isQ ? krb : 0)) * RB;
  const int64_t tok0 = static_cast<int64_t>(a.r) * a.C;
  const int64_t nv = fused_nvalid(a);
  const bf16_t* X = (isQ ? a.q : a.k) + (u * a.L + tok0) * FD;
  // Shadow row strides follow the layout (a.krep); with KREP = 1 and a
  // hi/lo layout only the hi halves are read.
  const int64_t ld13 = a.krep * FD;
  const bf16_t* W13 = a.w13s + u * 2 * a.h * ld13;
  const bf16_t* W2 = a.w2s + u * FD * (a.krep * a.h);
  const int64_t w2ld = a.krep * a.h;
  const int nhb = static_cast<int>(a.h / P::HBK);

  const int wave = threadIdx.x >> 6;
  const int wm = wave / P::WN, wn = wave % P::WN;

  TileCopy<RB, FD, 256> cx;
  TileCopy<P::NS, P::KD, 256> c13;
  auto w13_rows = [&](int hb) {
    return [=](int rr) -> const bf16_t* { return W13 + (static_cast<int64_t>(hb) * P::NS + rr) * ld13; };
  };

  cx.load([&](int rr) -> const bf16_t* { return p0 + rr < nv ? X + (p0 + rr) * FD : nullptr; }, X);
  c13.load(w13_rows(0));
  // W2 block: row j holds [hi: hidden hb*HBK .. +HBK | lo: same at offset h],
  // copied as FD*KREP rows of HBK.
  TileCopy<FD * KREP, P::HBK, 256> c2s;
  auto w2_rows = [&](int hb) {
    return [=](int rr) -> const bf16_t* {
      const int j = rr / KREP, part = rr % KREP;
      return W2 + j * w2ld + part * a.h + static_cast<int64_t>(hb) * P::HBK;
    };
  };
  c2s.load(w2_rows(0));
  cx.store(Xs, P::XW);
  c13.store(W13b, P::W13W);
  // row rr of c2s -> W2b row rr/KREP, column offset (rr%KREP)*HBK
#pragma unroll
  for (int i = 0; i < decltype(c2s)::PER; ++i) {
    const int idx = threadIdx.x + i * 256;
    if (decltype(c2s)::TOTAL % 256 == 0 || idx < decltype(c2s)::TOTAL) {
      const int rr = idx / decltype(c2s)::VPR, c = idx % decltype(c2s)::VPR;
      *reinterpret_cast<uint4*>(W2b + (rr / KREP) * P::W2W + (rr % KREP) * P::HBK + c * 8) =
          c2s.get(i);
    }
  }
  __syncthreads();

  f32x16_t yacc[P::YN / 32];
#pragma unroll
  for (int i = 0; i < P::YN / 32; ++i) zero16(yacc[i]);

  for (int hb = 0; hb < nhb; ++hb) {
    const bool more = hb + 1 < nhb;
    if (more) {  // prefetch the next block's weights; they land after this block
      c13.load(w13_rows(hb + 1));
      c2s.load(w2_rows(hb + 1));
    }
    // GEMM1: this wave's 32 rows x (32 A1 + 32 A3) columns.
    f32x16_t a1, a3;
    zero16(a1);
    zero16(a3);
    const bf16_t* Ar = Xs + wm * 32 * P::XW;
    const bf16_t* B1 = W13b + (wn * 64) * P::W13W;
    mma32_lds<P::KD, FD>(a1, Ar, P::XW, B1, P::W13W);
    mma32_lds<P::KD, FD>(a3, Ar, P::XW, B1 + 32 * P::W13W, P::W13W);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float x1 = a1[v];
      const float z = x1 * sigmoidf_(x1) * a3[v];
      Zs[(wm * 32 + acc32_row(v)) * P::ZW + wn * 32 + (threadIdx.x & 31)] = f2bf(z);
    }
    __syncthreads();
    // GEMM2: Y[32 rows of wm][YN cols of wn] += Z[rows][HBK] W2b[cols][KH]^T
#pragma unroll
    for (int i = 0; i < P::YN / 32; ++i)
      mma32_lds<P::KH, P::HBK>(yacc[i], Zs + wm * 32 * P::ZW, P::ZW,
                               W2b + (wn * P::YN + i * 32) * P::W2W, P::W2W);
    __syncthreads();
    if (more) {
      c13.store(W13b, P::W13W);
#pragma unroll
      for (int i = 0; i < decltype(c2s)::PER; ++i) {
        const int idx = threadIdx.x + i * 256;
        if (decltype(c2s)::TOTAL % 256 == 0 || idx < decltype(c2s)::TOTAL) {
          const int rr = idx / decltype(c2s)::VPR, c = idx % decltype(c2s)::VPR;
          *reinterpret_cast<uint4*>(W2b + (rr / KREP) * P::W2W + (rr % KREP) * P::HBK + c * 8) =
              c2s.get(i);
        }
      }
      __syncthreads();
    }
  }

  // Epilogue: Y through LDS in fp32 (all of LDS is free after the last
  // block's barrier), then every global access is a coalesced 16-byte
  // vector.  Q rows: o = bf16(Y).  K rows: g = bf16(v - Y), rounded once,
  // written token-major and, through a transposed LDS copy in tok_perm32
  // order, feature-major.  Rows past the valid tokens have X = 0, so Y = 0
  // and g = 0 there.
  constexpr int YW = FD + 4;  // fp32 row stride of the Y staging
  static_assert(static_cast<size_t>(RB) * YW * 4 + static_cast<size_t>(FD) * P::GW * 2 <=
                    P::LDS_BYTES, "epilogue staging fits the workgroup's LDS");
  float* Ys = reinterpret_cast<float*>(smem_raw);
#pragma unroll
  for (int i = 0; i < P::YN / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      Ys[(wm * 32 + acc32_row(v)) * YW + wn * P::YN + i * 32 + (threadIdx.x & 31)] = yacc[i][v];
  __syncthreads();
  constexpr int VPR = FD / 8;  // 8-element vectors per row
  if (isQ) {
    for (int idx = threadIdx.x; idx < RB * VPR; idx += 256) {
      const int pr = idx / VPR, c = idx % VPR;
      const int64_t p = p0 + pr;
      if (p < nv) {
        const float* y = Ys + pr * YW + c * 8;
        uint4 o;
        o.x = pack_bf16x2(y[0], y[1]);
        o.y = pack_bf16x2(y[2], y[3]);
        o.z = pack_bf16x2(y[4], y[5]);
        o.w = pack_bf16x2(y[6], y[7]);
        *reinterpret_cast<uint4*>(a.out + (u * a.L + tok0 + p) * FD + c * 8) = o;
      }
    }
    return;
  }
  bf16_t* Tg = reinterpret_cast<bf16_t*>(smem_raw + static_cast<size_t>(RB) * YW * 4);  // [FD][GW]
  // v is an input and gbf workspace: they never overlap (checked on the
  // host), which the restrict qualifiers pass on to the compiler.
  const bf16_t* __restrict__ vsrc = a.v + (u * a.L + tok0) * FD;
  bf16_t* __restrict__ gdst = a.gbf + u * a.Cp * FD;
  for (int idx = threadIdx.x; idx < RB * VPR; idx += 256) {
    const int pr = idx / VPR, c = idx % VPR;
    const int64_t p = p0 + pr;
    uint4 vin = make_uint4(0u, 0u, 0u, 0u);
    if (p < nv) vin = *reinterpret_cast<const uint4*>(vsrc + p * FD + c * 8);
    const float* y = Ys + pr * YW + c * 8;
    const uint32_t vw[4] = {vin.x, vin.y, vin.z, vin.w};
    uint32_t gw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v0 = __uint_as_float(vw[e] << 16), v1 = __uint_as_float(vw[e] & 0xffff0000u);
      gw[e] = pack_bf16x2(v0 - y[2 * e], v1 - y[2 * e + 1]);
      const int col = tok_perm32(pr);
      Tg[(c * 8 + 2 * e) * P::GW + col] = static_cast<bf16_t>(gw[e] & 0xffffu);
      Tg[(c * 8 + 2 * e + 1) * P::GW + col] = static_cast<bf16_t>(gw[e] >> 16);
    }
    *reinterpret_cast<uint4*>(gdst + p * FD + c * 8) = make_uint4(gw[0], gw[1], gw[2], gw[3]);
  }
  __syncthreads();
  constexpr int VPT = RB / 8;
  for (int idx = threadIdx.x; idx < FD * VPT; idx += 256) {
    const int j = idx / VPT, c = idx % VPT;
    *reinterpret_cast<uint4*>(a.gft + (u * FD + j) * a.Cp + p0 + c * 8) =
        *reinterpret_cast<const uint4*>(Tg + j * P::GW + c * 8);
  }
}

// ---------------------------------------------------------------------------
// Phase A, register-resident variant (bf16 operands without hi/lo, h = 4*HW,
// HW in {32, 64}).  Wave w keeps the weights of its HW hidden units in
// registers for the whole launch (W1, W3 rows and W2 columns of units
// w*HW .. w*HW+HW-1, as 32x32x16 MFMA A-fragments), so no weight passes
// through LDS.  A workgroup takes the rows of one (batch, head) unit in
// tiles of 32 ([K; Q] rows of the chunk; a tile is all K or all Q rows):
//   GEMM1 (transposed): A1^T, A3^T [hidden x token] = W1, W3 [hidden x d] X^T;
//   Z^T = silu(A1^T) * A3^T, rounded to bf16 in registers: a 32x32
//     accumulator gives lane l token l%32 and hidden rows 8*(v/4) + 4*(l/32)
//     + v%4, so registers 8*(kb%2) .. +7 of m-block kb/2 are exactly the
//     B-fragment of hidden k-block kb, taken in the order
//     {4*(l/32) + 0..3, 8 + 4*(l/32) + 0..3}; the W2 A-fragments are loaded in
//     that same order;
//   GEMM2 (transposed): the wave's partial Y^T [d x token] = W2[:, its units]
//     Z^T over its HW units.
// The four partials meet in LDS (fp32) and the epilogue adds them in wave
// order and writes out = bf16(Y) (Q rows) or g = bf16(v - Y) token-major and
// feature-major (K rows), all as 16-byte vectors.  The next tile's X rows
// are loaded while the current tile computes.
struct PhaseA2Cfg {
  static constexpr int TR = 32;      // rows per tile
  static constexpr int YW = FD + 4;  // fp32 row stride of one wave's Y partial
  static constexpr int GW = TR + 8;  // g^T staging row stride (bf16)
  static constexpr size_t Y_BYTES = static_cast<size_t>(4) * TR * YW * 4;
  static constexpr size_t LDS_BYTES = Y_BYTES + static_cast<size_t>(FD) * GW * 2;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int HW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_phaseA2(
    FusedArgs a, int wpu) {
  typedef PhaseA2Cfg P;
  constexpr int TR = P::TR;
  constexpr int MB = HW / 32;  // 32-unit m-blocks of GEMM1 per wave
  constexpr int KB2 = HW / 16; // 16-unit k-blocks of GEMM2 per wave
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  float* Yp = reinterpret_cast<float*>(smem_raw);                 // [4][TR][YW]
  bf16_t* Tg = reinterpret_cast<bf16_t*>(smem_raw + P::Y_BYTES);  // [FD][GW]

  const int64_t bid = xcd_logical_block();  // a unit's workgroups share one XCD's L2
  const int64_t u = bid / wpu;
  const int g = static_cast<int>(bid % wpu);
  const int ntile = static_cast<int>(2 * a.Cp / TR);  // tiles of the unit: K rows, then Q rows
  const int per = (ntile + wpu - 1) / wpu;
  const int tb = g * per;
  const int te = tb + per < ntile ? tb + per : ntile;
  const int64_t tok0 = static_cast<int64_t>(a.r) * a.C;
  const int64_t nv = fused_nvalid(a);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l32 = lane & 31, hf = lane >> 5;

  // X rows of a tile as GEMM1 B-fragments: lane l holds row l%32, d 16*kb + 8*hf .. +8.
  // Rows past the valid tokens are zero.  The loads are predicated rather than
  // selected afterwards: a select right after a load would make the wave
  // wait for the prefetch at once.
  auto load_x = [&](int t, bf16x8_t (&x)[8]) {
    const bool isQ = t * TR >= a.Cp;
    const int64_t p = t * TR - (isQ ? a.Cp : 0) + l32;
    const bf16_t* src = (isQ ? a.q : a.k) + (u * a.L + tok0 + p) * FD + 8 * hf;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) x[kb] = bf16x8_t{};
    if (p < nv) {
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) x[kb] = *reinterpret_cast<const bf16x8_t*>(src + 16 * kb);
    }
  };
  // v of a K tile for the epilogue: thread slot e takes (row, 8-column chunk)
  // idx = threadIdx.x + 256*e of the tile's TR x FD/8 chunks.
  constexpr int VPR = FD / 8;
  constexpr int EPT = TR * VPR / 256;  // epilogue chunks per thread
  const bf16_t* vsrc = a.v + (u * a.L + tok0) * FD;
  auto load_v = [&](int t, uint4 (&vv)[EPT]) {
    const bool isQ = t * TR >= a.Cp;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int idx = threadIdx.x + 256 * e;
      const int64_t p = t * TR + idx / VPR;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (!isQ && p < nv) x = *reinterpret_cast<const uint4*>(vsrc + p * FD + (idx % VPR) * 8);
      vv[e] = x;
    }
  };

  // First tile's inputs, then the weights: GEMM1 waits for X and W1/W3 only
  // while W2 is still in flight (loads complete in issue order).
  bf16x8_t xc[8], xn[8];
  uint4 vc[EPT], vn[EPT];
  if (tb < te) {
    load_v(tb, vc);
    load_x(tb, xc);
  }
  bf16x8_t w13[MB][2][8];  // [m-block][W1, W3][d k-block]
  bf16x8_t w2[4][KB2];     // [d m-block of 32][hidden k-block of 16]
  {
    // Shadow rows hold [hi | lo] when the layout carries pairs (a.krep = 2);
    // this kernel multiplies the hi halves only.
    const int64_t ld13 = a.krep * FD, ld2 = a.krep * a.h;
    const bf16_t* W13 = a.w13s + u * 2 * a.h * ld13;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int64_t i = wave * HW + 32 * mb + l32;  // hidden unit of this lane
      const bf16_t* r1 = W13 + (64 * (i / 32) + i % 32) * ld13 + 8 * hf;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        w13[mb][0][kb] = *reinterpret_cast<const bf16x8_t*>(r1 + 16 * kb);
        w13[mb][1][kb] = *reinterpret_cast<const bf16x8_t*>(r1 + 32 * ld13 + 16 * kb);
      }
    }
    const bf16_t* W2 = a.w2s + u * FD * ld2;
#pragma unroll
    for (int jm = 0; jm < 4; ++jm) {
      const bf16_t* rj = W2 + (32 * jm + l32) * ld2 + wave * HW;
#pragma unroll
      for (int kb = 0; kb < KB2; ++kb) {
        const bf16x4_t lo = *reinterpret_cast<const bf16x4_t*>(rj + 16 * kb + 4 * hf);
        const bf16x4_t hi = *reinterpret_cast<const bf16x4_t*>(rj + 16 * kb + 8 + 4 * hf);
        bf16x8_t f;
        f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
        f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
        w2[jm][kb] = f;
      }
    }
  }

  for (int t = tb; t < te; ++t) {
    if (t + 1 < te) {  // next tile's inputs, in flight during this tile
      load_v(t + 1, vn);
      load_x(t + 1, xn);
    }
    f32x16_t y[4];
#pragma unroll
    for (int jm = 0; jm < 4; ++jm) zero16(y[jm]);
    bf16x8_t zf[KB2];
    // z of accumulator registers r, r+1, rounded and packed; the empty asm
    // pins the arithmetic here, inside the MFMA shadow it is interleaved with
    // (pure arithmetic would otherwise be sunk to its first use).
    auto zpair = [](const f32x16_t& a1, const f32x16_t& a3, int r) -> uint32_t {
      const float x0 = a1[r], x1 = a1[r + 1];
      uint32_t w = pack_bf16x2(x0 * sigmoidf_(x0) * a3[r], x1 * sigmoidf_(x1) * a3[r + 1]);
      asm volatile("" : "+v"(w));
      return w;
    };
    if constexpr (MB == 2) {
      // GEMM1 of m-block 0; GEMM1 of m-block 1 interleaved with Z of m-block
      // 0; GEMM2 over k-blocks 0, 1 interleaved with Z of m-block 1; GEMM2
      // over k-blocks 2, 3.
      f32x16_t a1[2], a3[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        zero16(a1[mb]);
        zero16(a3[mb]);
      }
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        a1[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w13[0][0][kb], xc[kb], a1[0], 0, 0, 0);
        a3[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w13[0][1][kb], xc[kb], a3[0], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      u32x4_t zp[4];
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        a1[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w13[1][0][kb], xc[kb], a1[1], 0, 0, 0);
        a3[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w13[1][1][kb], xc[kb], a3[1], 0, 0, 0);
        zp[kb >> 2][kb & 3] = zpair(a1[0], a3[0], 2 * kb);
        __builtin_amdgcn_sched_barrier(0);
      }
      zf[0] = __builtin_bit_cast(bf16x8_t, zp[0]);
      zf[1] = __builtin_bit_cast(bf16x8_t, zp[1]);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int jm = st >> 1, kb = st & 1;
        y[jm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w2[jm][kb], zf[kb], y[jm], 0, 0, 0);
        zp[2 + (st >> 2)][st & 3] = zpair(a1[1], a3[1], 2 * st);
        __builtin_amdgcn_sched_barrier(0);
      }
      zf[2] = __builtin_bit_cast(bf16x8_t, zp[2]);
      zf[3] = __builtin_bit_cast(bf16x8_t, zp[3]);
#pragma unroll
      for (int jm = 0; jm < 4; ++jm)
#pragma unroll
        for (int kb = 2; kb < 4; ++kb)
          y[jm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w2[jm][kb], zf[kb], y[jm], 0, 0, 0);
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x16_t a1, a3;
        zero16(a1);
        zero16(a3);
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
          a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w13[mb][0][kb], xc[kb], a1, 0, 0, 0);
          a3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w13[mb][1][kb], xc[kb], a3, 0, 0, 0);
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          u32x4_t zq;
#pragma unroll
          for (int q = 0; q < 4; ++q) zq[q] = zpair(a1, a3, 8 * h2 + 2 * q);
          zf[2 * mb + h2] = __builtin_bit_cast(bf16x8_t, zq);
        }
      }
#pragma unroll
      for (int jm = 0; jm < 4; ++jm)
#pragma unroll
        for (int kb = 0; kb < KB2; ++kb)
          y[jm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w2[jm][kb], zf[kb], y[jm], 0, 0, 0);
    }
    // Partial to LDS as [wave][token][j]: registers 4q .. 4q+3 are four
    // consecutive j of one token.
    float* yw = Yp + (wave * TR + l32) * P::YW;
#pragma unroll
    for (int jm = 0; jm < 4; ++jm)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4_t v4;
        v4[0] = y[jm][4 * q]; v4[1] = y[jm][4 * q + 1]; v4[2] = y[jm][4 * q + 2]; v4[3] = y[jm][4 * q + 3];
        *reinterpret_cast<f32x4_t*>(yw + 32 * jm + 8 * q + 4 * hf) = v4;
      }
    __syncthreads();
    // Epilogue of the tile.
    const bool isQ = t * TR >= a.Cp;
    const int64_t p0 = t * TR - (isQ ? a.Cp : 0);
    bf16_t* gdst = a.gbf + u * a.Cp * FD;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int idx = threadIdx.x + 256 * e;
      const int pr = idx / VPR, c = idx % VPR;
      const int64_t p = p0 + pr;
      const uint4 vin = vc[e];
      float yv[8];
      {
        const float* s0 = Yp + pr * P::YW + c * 8;
        f32x4_t lo = *reinterpret_cast<const f32x4_t*>(s0);
        f32x4_t hi = *reinterpret_cast<const f32x4_t*>(s0 + 4);
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          lo += *reinterpret_cast<const f32x4_t*>(s0 + w * TR * P::YW);
          hi += *reinterpret_cast<const f32x4_t*>(s0 + w * TR * P::YW + 4);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          yv[e] = lo[e];
          yv[4 + e] = hi[e];
        }
      }
      if (isQ) {
        if (p < nv) {
          uint4 o;
          o.x = pack_bf16x2(yv[0], yv[1]);
          o.y = pack_bf16x2(yv[2], yv[3]);
          o.z = pack_bf16x2(yv[4], yv[5]);
          o.w = pack_bf16x2(yv[6], yv[7]);
          *reinterpret_cast<uint4*>(a.out + (u * a.L + tok0 + p) * FD + c * 8) = o;
        }
      } else {
        const uint32_t vw[4] = {vin.x, vin.y, vin.z, vin.w};
        uint32_t gw[4];
        const int col = tok_perm32(pr);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v0 = __uint_as_float(vw[e] << 16), v1 = __uint_as_float(vw[e] & 0xffff0000u);
          gw[e] = pack_bf16x2(v0 - yv[2 * e], v1 - yv[2 * e + 1]);
          Tg[(c * 8 + 2 * e) * P::GW + col] = static_cast<bf16_t>(gw[e] & 0xffffu);
          Tg[(c * 8 + 2 * e + 1) * P::GW + col] = static_cast<bf16_t>(gw[e] >> 16);
        }
        *reinterpret_cast<uint4*>(gdst + p * FD + c * 8) = make_uint4(gw[0], gw[1], gw[2], gw[3]);
      }
    }
    __syncthreads();
    if (!isQ) {
      constexpr int VPT = TR / 8;
      for (int idx = threadIdx.x; idx < FD * VPT; idx += 256) {
        const int j = idx / VPT, c = idx % VPT;
        *reinterpret_cast<uint4*>(a.gft + (u * FD + j) * a.Cp + p0 + c * 8) =
            *reinterpret_cast<const uint4*>(Tg + j * P::GW + c * 8);
      }
    }
    if (t + 1 < te) {
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) xc[kb] = xn[kb];
#pragma unroll
      for (int e = 0; e < EPT; ++e) vc[e] = vn[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Phase B.  LDS: three token-tile buffers (the recompute weights of the
// wave's hidden units live in registers, hi and lo parts alike).
template <int KREP> struct PhaseBCfg {
  static constexpr int TB = 32;               // tokens per tile
  static constexpr int KS = FD + 8;           // token-major tile row stride
  static constexpr int TS = TB + 8;           // feature-major tile row stride
  static constexpr int NBUF = 3;
  static constexpr int BUF_ELEMS = 2 * TB * KS + 2 * FD * TS;  // K, g | K^T, g^T
  static constexpr size_t BUF_BYTES = BUF_ELEMS * sizeof(bf16_t) + 2 * TB * sizeof(float);
  static constexpr size_t LDS_BYTES = NBUF * BUF_BYTES;
  static_assert((BUF_ELEMS * sizeof(bf16_t)) % 16 == 0, "buffer alignment");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b,
                                          const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two 8-byte pieces -> one 8 x bf16 fragment.
__device__ __forceinline__ bf16x8_t frag_2x4(const bf16_t* p0, const bf16_t* p1) {
  const bf16x4_t lo = *reinterpret_cast<const bf16x4_t*>(p0);
  const bf16x4_t hi = *reinterpret_cast<const bf16x4_t*>(p1);
  bf16x8_t r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Chunk-end state of one entry from its preloaded start values, plus the
// next chunk's operand shadow.  Loads are done by the caller in batches: the
// outputs may alias the inputs (in-place state advance), so a load placed
// after a store could not be hoisted by the compiler and every entry would
// cost a full memory round trip.
__device__ __forceinline__ void state_store(const FusedArgs& a, int krep, int64_t u, int64_t off,
                                            float w0, float m0, float aw, float am, float cW,
                                            float cM, float cWM, int shadow_kind, int64_t srow,
                                            int64_t scol) {
  const int64_t P = 3 * FD * a.h;
  const float wn = cW * w0 + cWM * m0 + aw;
  const float mn = cM * m0 + am;
  a.Wout[u * P + off] = wn;
  a.Mout[u * P + off] = mn;
  if (a.last) return;
  const bf16_t hi = f2bf(wn);
  const bf16_t lo = krep == 2 ? f2bf(wn - bf2f(hi)) : bf16_t(0);
  if (shadow_kind == 0) {  // W1 / W3 entry: shadow row srow, column scol (d index)
    bf16_t* b = a.w13s + (u * 2 * a.h + srow) * (krep * FD);
    b[scol] = hi;
    if (krep == 2) b[FD + scol] = lo;
  } else {  // W2 entry (j = srow, i = scol)
    bf16_t* b2 = a.w2s + (u * FD + srow) * (krep * a.h);
    b2[scol] = hi;
    if (krep == 2) b2[a.h + scol] = lo;
    bf16_t* bt = a.w2ts + (u * a.h + scol) * (krep * FD);
    bt[srow] = hi;
    if (krep == 2) bt[FD + srow] = lo;
  }
}

// State entry behind phase B accumulator value v of thread tid for column
// block jb of weight t (0: W1, 1: W3, 2: W2) in hidden block ib: its offset
// in the packed state and its position in the operand shadow (the layout
// k_state_epi's block transpose follows as well).
struct StateSlot {
  int off, srow, scol;  // within one unit's state (< 3*128*4096 entries)
  int kind;             // 0: W1/W3 entry, 1: W2 entry
};
__device__ __forceinline__ StateSlot phaseB_slot(int h, int ib, int tid, int t, int jb, int v) {
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
  StateSlot r;
  if (t < 2) {  // row i = hidden unit (16*wave + 4*g4 + v), column j = 16*jb + l16
    const int i = 64 * ib + 16 * wave + 4 * g4 + v;
    const int j = 16 * jb + l16;
    r.off = t * h * FD + i * FD + j;
    r.srow = 64 * (i / 32) + i % 32 + 32 * t;
    r.scol = j;
    r.kind = 0;
  } else {      // row j2 = 16*jb + 4*g4 + v, column = hidden unit 16*wave + l16
    const int i = 64 * ib + 16 * wave + l16;
    const int j2 = 16 * jb + 4 * g4 + v;
    r.off = 2 * h * FD + j2 * h + i;
    r.srow = j2;
    r.scol = i;
    r.kind = 1;
  }
  return r;
}

// Phase B: 4 waves (one per SIMD), wave w owns hidden units
// 64*ib + 16*w .. +15 for all FD output columns.  The recompute weights of
// the wave's hidden units stay in registers for the whole launch (KREP = 2:
// hi and lo parts, 96 VGPRs; reading them from LDS per tile, as a first
// version of the hi/lo variant did, cost about 48 KB of LDS reads per wave
// and tile and measured 343 against about 290 us per launch on the 128-unit
// workload).  Fragments of the next step are read from LDS before the MFMAs
// of the current step are issued.
template <int KREP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_phaseB(
    FusedArgs a) {
  typedef PhaseBCfg<KREP> S;
  constexpr int TB = S::TB, KS = S::KS, TS = S::TS;
  constexpr int NT = 256;
  constexpr int KSTEPS = KREP * FD / 32;  // recompute k-steps (16x16x32)
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  auto bufp = [&](int b) -> bf16_t* {
    return reinterpret_cast<bf16_t*>(smem_raw + b * S::BUF_BYTES);
  };
  auto kscp = [&](int b) -> float* {
    return reinterpret_cast<float*>(smem_raw + b * S::BUF_BYTES + S::BUF_ELEMS * sizeof(bf16_t));
  };

  const int64_t nib = a.h / 64;
  // A unit's hidden blocks read the same token tiles: XCD-aware numbering
  // keeps them on one L2.  Measured: it helps the unsplit kernel, and the
  // token-split one (fewer, shorter workgroups) runs faster without it.
  const int64_t bid = a.nsplit == 1 ? xcd_logical_block() : static_cast<int64_t>(blockIdx.x);
  const int64_t grp = bid / a.nsplit;  // (unit, hidden block)
  const int sp = static_cast<int>(bid % a.nsplit);
  const int64_t u = grp / nib;
  const int64_t ib = grp % nib;
  const int64_t tok0 = static_cast<int64_t>(a.r) * a.C;
  const int64_t nv = fused_nvalid(a);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int64_t i_glob = 64 * ib + 16 * wave + l16;  // this lane's hidden unit (B column)

  // Recompute B operands: row = hidden unit, k = d (hi | lo when KREP = 2).
  bf16x8_t wreg[3][KSTEPS];
  {
    const bf16_t* w13 = a.w13s + u * 2 * a.h * (KREP * FD);
    const bf16_t* w1r = w13 + (64 * (i_glob / 32) + i_glob % 32) * (KREP * FD);
    const bf16_t* w2r = a.w2ts + (u * a.h + i_glob) * (KREP * FD);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      wreg[0][ks] = *reinterpret_cast<const bf16x8_t*>(w1r + ks * 32 + g4 * 8);
      wreg[1][ks] = *reinterpret_cast<const bf16x8_t*>(w1r + 32 * (KREP * FD) + ks * 32 + g4 * 8);
      wreg[2][ks] = *reinterpret_cast<const bf16x8_t*>(w2r + ks * 32 + g4 * 8);
    }
  }
  auto wfrag = [&](int q, int ks) -> bf16x8_t { return wreg[q][ks]; };

  // Accumulators (16x16 blocks): [0..7] A^W_W1 (rows i of this wave, cols j
  // block jb), [8..15] A^M_W1, [16..23] A^W_W3, [24..31] A^M_W3,
  // [32..39] A^W_W2 (rows j block jb, cols i), [40..47] A^M_W2.
  f32x4_t acc[48];
#pragma unroll
  for (int q = 0; q < 48; ++q) zero4(acc[q]);

  const bf16_t* Kg = a.k + (u * a.L + tok0) * FD;
  const bf16_t* Gg = a.gbf + u * a.Cp * FD;
  const bf16_t* KTg = a.kt + (u * a.nC + a.r) * FD * a.Cp;
  const bf16_t* GTg = a.gft + u * FD * a.Cp;
  const float* kwr = a.kw + (u * a.nC + a.r) * a.Cp;
  const float* kmr = a.km + (u * a.nC + a.r) * a.Cp;

  // Registers of one tile in flight from global memory.
  struct TileRegs {
    TileCopy<TB, FD, NT> k, g;    // token-major K, bf16(g)
    TileCopy<FD, TB, NT> kt, gt;  // feature-major (permuted tokens) K^T, g^T
    float sk;                     // K^W (first TB) and K^M (next TB) of the tile
  };
  auto load_tile = [&](TileRegs& R, int64_t t0) {
    R.k.load([&](int rr) -> const bf16_t* { return t0 + rr < nv ? Kg + (t0 + rr) * FD : nullptr; },
             Kg);
    R.g.load([&](int rr) -> const bf16_t* { return Gg + (t0 + rr) * FD; });
    R.kt.load([&](int rr) -> const bf16_t* { return KTg + rr * a.Cp + t0; });
    R.gt.load([&](int rr) -> const bf16_t* { return GTg + rr * a.Cp + t0; });
    // Every wave loads (and stores) the same 2*TB kernel values, so no lane
    // mask splits the loop body into several scheduling regions.
    const int ks_i = threadIdx.x & (2 * TB - 1);
    R.sk = (ks_i < TB ? kwr : kmr - TB)[t0 + ks_i];
  };
  auto store_tile = [&](const TileRegs& R, int b) {
    bf16_t* B = bufp(b);
    R.k.store(B, KS);
    R.g.store(B + TB * KS, KS);
    R.kt.store(B + 2 * TB * KS, TS);
    R.gt.store(B + 2 * TB * KS + FD * TS, TS);
    kscp(b)[threadIdx.x & (2 * TB - 1)] = R.sk;
  };
  TileRegs tr;

  // This workgroup's token tiles: split sp of nsplit (the host picks nsplit
  // dividing Cp / TB).
  const int ntiles = static_cast<int>(a.Cp / TB) / a.nsplit;
  const int64_t tbase = static_cast<int64_t>(sp) * ntiles * TB;

  // Recompute of one tile: rows = tokens (2 blocks of 16), cols = this
  // wave's 16 hidden units; A1, A3 from K, dZ from g.
  struct Rec {
    f32x4_t a1[2], a3[2], dz[2];
  };
  auto recompute = [&](const bf16_t* Ks) -> Rec {
    const bf16_t* Gs = Ks + TB * KS;
    Rec rc;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      zero4(rc.a1[tb]);
      zero4(rc.a3[tb]);
      zero4(rc.dz[tb]);
    }
    constexpr int NSTEP = 2 * KSTEPS;
    auto kfrag = [&](const bf16_t* base, int n) {
      const int tb = n / KSTEPS, ks = n % KSTEPS;
      return *reinterpret_cast<const bf16x8_t*>(base + (tb * 16 + l16) * KS + g4 * 8 +
                                                (ks * 32) % FD);
    };
    bf16x8_t fk = kfrag(Ks, 0), fg = kfrag(Gs, 0);
#pragma unroll
    for (int n = 0; n < NSTEP; ++n) {
      const int tb = n / KSTEPS, ks = n % KSTEPS;
      bf16x8_t fk_n = fk, fg_n = fg;
      if (n + 1 < NSTEP) {
        fk_n = kfrag(Ks, n + 1);
        fg_n = kfrag(Gs, n + 1);
      }
      rc.a1[tb] = mfma16(fk, wfrag(0, ks), rc.a1[tb]);
      rc.a3[tb] = mfma16(fk, wfrag(1, ks), rc.a3[tb]);
      rc.dz[tb] = mfma16(fg, wfrag(2, ks), rc.dz[tb]);
      fk = fk_n;
      fg = fg_n;
    }
    return rc;
  };
  // Elementwise; fragment slot s <-> token 16*(s/4) + 4*g4 + s%4.
  struct Frags {
    bf16x8_t w1, m1, w3, m3, zw, zm;
  };
  auto elementwise = [&](const Rec& rc, const float* kws) -> Frags {
    Frags f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int tb = s >> 2, v = s & 3;
      const int t = 16 * tb + 4 * g4 + v;
      const float x1 = rc.a1[tb][v], x3 = rc.a3[tb][v], dz = rc.dz[tb][v];
      const float sg = sigmoidf_(x1);
      const float d3 = dz * (x1 * sg);
      const float d1 = dz * x3 * (sg * (1.0f + x1 * (1.0f - sg)));
      const float sw = kws[t], sm = kws[TB + t];
      const float z = x1 * sg * x3;
      f.w1[s] = static_cast<__bf16>(sw * d1);
      f.m1[s] = static_cast<__bf16>(sm * d1);
      f.w3[s] = static_cast<__bf16>(sw * d3);
      f.m3[s] = static_cast<__bf16>(sm * d3);
      f.zw[s] = static_cast<__bf16>(sw * z);
      f.zm[s] = static_cast<__bf16>(sm * z);
    }
    return f;
  };
  // Aggregations over a tile's 32 tokens: partner fragments (one 16-byte
  // read each thanks to the permuted token order) of block jb+1 are read
  // while block jb's six MFMAs issue.
  auto pfrag = [&](const bf16_t* base, int jb) {
    return *reinterpret_cast<const bf16x8_t*>(base + (jb * 16 + l16) * TS + 8 * g4);
  };
  auto mma_block = [&](const Frags& f, int jb, const bf16x8_t& fk, const bf16x8_t& fg) {
    acc[jb] = mfma16(f.w1, fk, acc[jb]);
    acc[8 + jb] = mfma16(f.m1, fk, acc[8 + jb]);
    acc[16 + jb] = mfma16(f.w3, fk, acc[16 + jb]);
    acc[24 + jb] = mfma16(f.m3, fk, acc[24 + jb]);
    acc[32 + jb] = mfma16(fg, f.zw, acc[32 + jb]);
    acc[40 + jb] = mfma16(fg, f.zm, acc[40 + jb]);
  };
  // The aggregation of tile it fused with elementwise() of tile it+1: step jb
  // issues the six MFMAs of column block jb alternating with the VALU work
  // of fragment slot jb of the next tile (8 slots, 8 blocks), and a
  // scheduling fence after each step keeps the compiler from clustering the
  // MFMAs, so the VALU work runs while the matrix core is busy.
  auto aggregate_next = [&](const Frags& f, const bf16_t* Ks, const Rec& rc,
                            const float* kws) -> Frags {
    const bf16_t* KTs = Ks + 2 * TB * KS;
    const bf16_t* GTs = KTs + FD * TS;
    float sw[8], sm[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int t = 16 * (s >> 2) + 4 * g4 + (s & 3);
      sw[s] = kws[t];
      sm[s] = kws[TB + t];
    }
    // Packed bf16 pairs of the next tile's fragments: [output][slot pair].
    u32x4_t pk[6];
    float ev[6];  // even slot's values, packed with the odd slot after it
    bf16x8_t fk = pfrag(KTs, 0), fg = pfrag(GTs, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jb = 0; jb < FD / 16; ++jb) {
      bf16x8_t fk_n = fk, fg_n = fg;
      if (jb + 1 < FD / 16) {
        fk_n = pfrag(KTs, jb + 1);
        fg_n = pfrag(GTs, jb + 1);
      }
      mma_block(f, jb, fk, fg);
      {
        const int s = jb, tb = s >> 2, v = s & 3;
        const float x1 = rc.a1[tb][v], x3 = rc.a3[tb][v], dz = rc.dz[tb][v];
        const float sg = sigmoidf_(x1);
        const float d3 = dz * (x1 * sg);
        const float d1 = dz * x3 * (sg * (1.0f + x1 * (1.0f - sg)));
        const float z = x1 * sg * x3;
        float o[6] = {sw[s] * d1, sm[s] * d1, sw[s] * d3, sm[s] * d3, sw[s] * z, sm[s] * z};
        if ((s & 1) == 0) {
#pragma unroll
          for (int q = 0; q < 6; ++q) {
            ev[q] = o[q];
            // Pin the value here: pure arithmetic would otherwise be sunk
            // to its use after the last block, out of the MFMA shadow.
            asm volatile("" : "+v"(ev[q]));
          }
        } else {
#pragma unroll
          for (int q = 0; q < 6; ++q) {
            uint32_t w = pack_bf16x2(ev[q], o[q]);
            asm volatile("" : "+v"(w));
            pk[q][s >> 1] = w;
          }
        }
      }
#pragma unroll
      for (int m = 0; m < 6; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_barrier(0);
      fk = fk_n;
      fg = fg_n;
    }
    Frags fn;
    fn.w1 = __builtin_bit_cast(bf16x8_t, pk[0]);
    fn.m1 = __builtin_bit_cast(bf16x8_t, pk[1]);
    fn.w3 = __builtin_bit_cast(bf16x8_t, pk[2]);
    fn.m3 = __builtin_bit_cast(bf16x8_t, pk[3]);
    fn.zw = __builtin_bit_cast(bf16x8_t, pk[4]);
    fn.zm = __builtin_bit_cast(bf16x8_t, pk[5]);
    return fn;
  };

  // Software pipeline over three buffers: iteration it aggregates tile it
  // (fragments formed in the previous iteration) while it recomputes tile
  // it+1 and forms its fragments, so the elementwise VALU work of one tile
  // overlaps the MFMAs of the other; tile it+2 is in flight from global
  // memory meanwhile and lands in the buffer tile it-1 used.  The recompute
  // past the last tile reads a stale (in-bounds) buffer and is discarded.
  {  // the first two tiles' loads in flight together
    TileRegs tr1;
    load_tile(tr, tbase);
    if (ntiles > 1) load_tile(tr1, tbase + TB);
    store_tile(tr, 0);
    if (ntiles > 1) store_tile(tr1, 1);
  }
  __syncthreads();
  Frags f = elementwise(recompute(bufp(0)), kscp(0));
  // No conditional loads or stores in the body: past the end the last
  // tile is fetched again and stored into the free buffer.
  int bc = 0;  // buffer of tile it
  for (int it = 0; it < ntiles; ++it) {
    const int bn = bc == 2 ? 0 : bc + 1;  // tile it+1
    const int bnn = bn == 2 ? 0 : bn + 1; // tile it+2 (= tile it-1's)
    const int tl = it + 2 < ntiles ? it + 2 : ntiles - 1;
    load_tile(tr, tbase + static_cast<int64_t>(tl) * TB);
    const Rec rn = recompute(bufp(bn));
    f = aggregate_next(f, bufp(bc), rn, kscp(bn));
    store_tile(tr, bnn);
    __syncthreads();
    bc = bn;
  }

  if (a.nsplit > 1) {
    // Token-split: this workgroup's partial sums as [q][tid] 16-byte vectors
    // (coalesced); k_state_epi adds the splits in a fixed order and writes
    // the state.
    f32x4_t* __restrict__ dst =
        reinterpret_cast<f32x4_t*>(a.part) + (grp * a.nsplit + sp) * (48 * NT);
#pragma unroll
    for (int q = 0; q < 48; ++q) dst[q * NT + threadIdx.x] = acc[q];
    return;
  }
  // Chunk-end state and operand shadows of this wave's hidden units, one
  // 16-column block jb at a time, software-pipelined: the start values of
  // block jb+1 are loaded before block jb is stored.  (The
  // outputs may alias the inputs, so the compiler keeps loads placed after
  // a store behind it; issuing them early in program order is what lets
  // them overlap.)
  const float* cf = a.coef + (u * a.nC + a.r) * 4;
  const float cW = cf[0], cM = cf[1], cWM = cf[2];
  const int64_t P = 3 * FD * a.h;
  const float* __restrict__ Wi = a.Win + u * P;
  const float* __restrict__ Mi = a.Min + u * P;
  constexpr int NJB = FD / 16;
  float w0[NJB][3][4], m0[NJB][3][4];
  auto load_jb = [&](int jb) {
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int off = phaseB_slot(static_cast<int>(a.h), static_cast<int>(ib), threadIdx.x, t, jb, v).off;
        w0[jb][t][v] = Wi[off];
        m0[jb][t][v] = Mi[off];
      }
  };
  auto store_jb = [&](int jb) {
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const StateSlot sl = phaseB_slot(static_cast<int>(a.h), static_cast<int>(ib), threadIdx.x, t, jb, v);
        state_store(a, KREP, u, sl.off, w0[jb][t][v], m0[jb][t][v], acc[16 * t + jb][v],
                    acc[16 * t + 8 + jb][v], cW, cM, cWM, sl.kind, sl.srow, sl.scol);
      }
  };
  load_jb(0);
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) {
    if (jb + 1 < NJB) load_jb(jb + 1);
    store_jb(jb);
  }
}

// State epilogue of a token-split phase B: W_C = cW W_0 + cWM M_0 + sum of
// the splits' A^W, M_C = cM M_0 + sum of A^M (splits added in index order,
// so the result does not depend on scheduling), plus the operand shadows.
// Workgroup (unit, hidden block, t, jb) of 256 threads takes the 1024 state
// entries of one (W, M) accumulator pair of all phase B threads: a 64 x 16
// block of W1 or W3 (t = 0, 1) or a 16 x 64 block of W2 (t = 2).  Thread tid
// sums the splits of phase B thread tid's four entries, the block is
// transposed through LDS, and each thread then owns four consecutive
// columns of one row: 16-byte loads and stores of W_0, M_0, W_C, M_C and
// 8-byte stores of the row-major shadows.
__global__ __launch_bounds__(256) void k_state_epi(FusedArgs a) {
  __shared__ float sW[64 * 17], sM[64 * 17], sT[64 * 17];
  const int64_t grp = blockIdx.x / 24;
  const int pr = static_cast<int>(blockIdx.x % 24);  // (t, jb) pair
  const int t = pr >> 3, jb = pr & 7;
  const int tid = threadIdx.x;
  const int64_t nib = a.h / 64;
  const int64_t u = grp / nib, ib = grp % nib;
  const int64_t P = 3 * FD * a.h;
  const int64_t h = a.h;
  // After the transpose this thread owns columns c0 .. c0+3 of block row r;
  // their start values are loaded first, in flight with the partial sums.
  const int CC = t < 2 ? 16 : 64;  // columns of the block
  const int r = tid / (CC / 4), c0 = 4 * (tid % (CC / 4));
  int64_t off;  // of the first of the four entries, inside the unit's state
  if (t < 2) off = t * h * FD + (64 * ib + r) * FD + 16 * jb + c0;
  else off = 2 * h * FD + (16 * jb + r) * h + 64 * ib + c0;
  const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(a.Win + u * P + off);
  const f32x4_t m0 = *reinterpret_cast<const f32x4_t*>(a.Min + u * P + off);
  const int qW = 16 * t + jb, qM = qW + 8;
  const f32x4_t* src = reinterpret_cast<const f32x4_t*>(a.part) + grp * a.nsplit * (48 * 256);
  f32x4_t sw = src[qW * 256 + tid], sm = src[qM * 256 + tid];
  for (int sp = 1; sp < a.nsplit; ++sp) {
    sw += src[sp * (48 * 256) + qW * 256 + tid];
    sm += src[sp * (48 * 256) + qM * 256 + tid];
  }
  // Block-local coordinates (row, column) of phase B register v.
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int rr = t < 2 ? 16 * wave + 4 * g4 + v : 4 * g4 + v;
    const int cc = t < 2 ? l16 : 16 * wave + l16;
    sW[rr * (CC + 1) + cc] = sw[v];
    sM[rr * (CC + 1) + cc] = sm[v];
  }
  __syncthreads();
  f32x4_t aw, am;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    aw[e] = sW[r * (CC + 1) + c0 + e];
    am[e] = sM[r * (CC + 1) + c0 + e];
  }
  const float* cf = a.coef + (u * a.nC + a.r) * 4;
  const float cW = cf[0], cM = cf[1], cWM = cf[2];
  f32x4_t wn, mn;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    wn[e] = cW * w0[e] + cWM * m0[e] + aw[e];
    mn[e] = cM * m0[e] + am[e];
  }
  *reinterpret_cast<f32x4_t*>(a.Wout + u * P + off) = wn;
  *reinterpret_cast<f32x4_t*>(a.Mout + u * P + off) = mn;
  if (a.last) return;
  const int kr = a.krep;
  bf16_t hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = f2bf(wn[e]);
    lo[e] = kr == 2 ? f2bf(wn[e] - bf2f(hi[e])) : bf16_t(0);
  }
  auto put4 = [](bf16_t* dst, const bf16_t (&x)[4]) {
    *reinterpret_cast<uint2*>(dst) =
        make_uint2(x[0] | (static_cast<uint32_t>(x[1]) << 16), x[2] | (static_cast<uint32_t>(x[3]) << 16));
  };
  if (t < 2) {  // W1 / W3 row i -> shadow row 64*(i/32) + i%32 (+32 for W3)
    const int64_t i = 64 * ib + r, j = 16 * jb + c0;
    bf16_t* b = a.w13s + (u * 2 * h + 64 * (i / 32) + i % 32 + 32 * t) * (kr * FD);
    put4(b + j, hi);
    if (kr == 2) put4(b + FD + j, lo);
  } else {      // W2 row j2, hidden columns i .. i+3
    const int64_t j2 = 16 * jb + r, i = 64 * ib + c0;
    bf16_t* b2 = a.w2s + (u * FD + j2) * (kr * h);
    put4(b2 + i, hi);
    if (kr == 2) put4(b2 + h + i, lo);
    // W2^T through LDS: thread (il, jq) writes hidden row 64*ib + il, entries
    // 16*jb + jq .. +3 (coalesced 8-byte stores instead of scattered halves).
#pragma unroll
    for (int e = 0; e < 4; ++e) sT[(c0 + e) * 17 + r] = wn[e];
    __syncthreads();
    const int il = tid >> 2, jq = 4 * (tid & 3);
    bf16_t th[4], tlo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = sT[il * 17 + jq + e];
      th[e] = f2bf(x);
      tlo[e] = kr == 2 ? f2bf(x - bf2f(th[e])) : bf16_t(0);
    }
    bf16_t* bt = a.w2ts + (u * h + 64 * ib + il) * (kr * FD) + 16 * jb + jq;
    put4(bt, th);
    if (kr == 2) put4(bt + FD, tlo);
  }
}

}  // namespace e2ttt
