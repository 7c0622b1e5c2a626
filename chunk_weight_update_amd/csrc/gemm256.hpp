// gemm256.hpp -- 256x256-tile bf16 MFMA GEMM for the generic (d != 128)
// aggregation of the SwiGLU learner, with a token split and a streaming
// state epilogue.
//
// The aggregations of §3.2 / App. A.4 of "Rethinking Expressivity and
// Efficiency in Test-Time Training" contract over the chunk's tokens:
//   family A: [K^W dA1 | K^M dA1 | K^W dA3 | K^M dA3]^T K   (4h x d)
//   family B: [K^W g | K^M g]^T Z                          (2d x h)
// with operands already scaled and rounded once (k_bwd, k_fwd2) and stored
// feature-major (rows = output rows, contiguous along tokens).
//
// Tile: 256 x 256 per workgroup, 4 waves in a 2 x 2 grid, 128 x 128 per wave
// (4 x 4 blocks of 32x32x16 MFMA, 256 accumulator registers), k-slabs of 32
// tokens double-buffered in LDS with rows padded to 40 elements (80 bytes:
// eight consecutive rows of a 16-byte fragment read hit distinct banks).  Per
// slab a wave reads 16 KB of fragments for 32 MFMAs (1024 cycles), about 64
// B/clk per CU of LDS: well under what four waves sustain (~86 B/clk), where
// the 128 x 128 tile with 64 x 64 per wave needs 128 B/clk.
//
// Token split: the tile count of one unit can be small (108 at d = 768,
// h = 1536), so the chunk's token slabs are split over S workgroups.  Each
// writes its fp32 partial aggregates in the packed state layout, and
// k_agg_reduce adds the S partials in split order (deterministic) and applies
// W_C = cW W_0 + cWM M_0 + A^W, M_C = cM M_0 + A^M plus the operand shadows.
#pragma once
#include "kernels.hpp"

namespace e2ttt {

struct Tile256 {
  static constexpr int BM = 256, BN = 256, BK = 32;
  static constexpr int LS = BK + 8;                   // LDS row stride (elements)
  static constexpr int SLAB = BM * LS;                // elements per operand slab
  static constexpr size_t LDS_BYTES = 4 * SLAB * 2;  // A, B x double buffer, bf16
};

// Per-thread loader of one 256-row operand: thread t loads rows t/4 + 64*i,
// 16-byte vector t%4 of each 32-element slab.  The four vectors travel as one
// wide value (an array held across the k loop was demoted to scratch).
typedef uint32_t u32x16_t __attribute__((ext_vector_type(16)));
struct Loader256 {
  const bf16_t* rowp[4];
  __device__ __forceinline__ u32x16_t load(int64_t k0) const {
    const int vec = threadIdx.x & 3;
    u32x16_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(rowp[i] + k0 + vec * 8);
      r[4 * i] = v.x; r[4 * i + 1] = v.y; r[4 * i + 2] = v.z; r[4 * i + 3] = v.w;
    }
    return r;
  }
};

__device__ __forceinline__ void stage256(bf16_t* slab, const u32x16_t& r) {
  const int row0 = threadIdx.x >> 2, vec = threadIdx.x & 3;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint4*>(slab + (row0 + 64 * i) * Tile256::LS + vec * 8) =
        make_uint4(r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]);
}

__device__ __forceinline__ int loader256_row(int i) { return (threadIdx.x >> 2) + 64 * i; }

// acc[mi][ni] (rows wm*128 + 32*mi, cols wn*128 + 32*ni) += A B^T over k
// [k0, k1) (multiples of 32).
__device__ __forceinline__ void gemm_tile256(f32x16_t (&acc)[4][4], const Loader256& la,
                                             const Loader256& lb, int64_t k0, int64_t k1,
                                             bf16_t* lds) {
  constexpr int SLAB = Tile256::SLAB, LS = Tile256::LS;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, hf = lane >> 5;
  // One slab in flight from global memory while the current one is computed
  // from LDS.  (A second register set for a deeper prefetch does not fit
  // beside the 256 accumulators: measured, it spills.)
  u32x16_t ra = la.load(k0), rb = lb.load(k0);
  stage256(lds, ra);
  stage256(lds + SLAB, rb);
  __syncthreads();
  const int64_t ns = (k1 - k0) / Tile256::BK;
  for (int64_t s = 0; s < ns; ++s) {
    const int cur = static_cast<int>(s & 1);
    const bool more = s + 1 < ns;
    if (more) {
      ra = la.load(k0 + (s + 1) * Tile256::BK);
      rb = lb.load(k0 + (s + 1) * Tile256::BK);
    }
    const bf16_t* As = lds + 2 * cur * SLAB + (wm * 128 + r32) * LS + 8 * hf;
    const bf16_t* Bs = lds + (2 * cur + 1) * SLAB + (wn * 128 + r32) * LS + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[i] = *reinterpret_cast<const bf16x8_t*>(As + i * 32 * LS + 16 * ks);
        fb[i] = *reinterpret_cast<const bf16x8_t*>(Bs + i * 32 * LS + 16 * ks);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      bf16_t* An = lds + 2 * (cur ^ 1) * SLAB;
      stage256(An, ra);
      stage256(An + SLAB, rb);
    }
    __syncthreads();
  }
}

// Partial aggregates of split sp over token slabs [k0, k1): workgroup
// (unit, split, tile); tiles 0 .. na-1 are family A (4h/256 x d/256), then
// family B (2d/256 x h/256).  The partial of state entry e goes to
// part[((sp * 2 + wm) * BH + u) * P + e], wm = 0 for A^W, 1 for A^M.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_agg256(
    Shape s, int nsplit, const bf16_t* __restrict__ ut, const bf16_t* __restrict__ kt,
    const bf16_t* __restrict__ gt, const bf16_t* __restrict__ zt, int r, float* part) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  bf16_t* lds = reinterpret_cast<bf16_t*>(smem_raw);
  const int64_t d = s.d, h = s.h;
  const int64_t na = (4 * h / 256) * (d / 256), nb = (2 * d / 256) * (h / 256);
  const int64_t per_unit = (na + nb) * nsplit;
  const int64_t bid = xcd_logical_block();  // a unit's tiles share one XCD's L2
  const int64_t u = bid / per_unit;
  const int64_t rest = bid % per_unit;
  const int sp = static_cast<int>(rest / (na + nb));
  const int64_t t = rest % (na + nb);
  const bool famA = t < na;
  int64_t mt, nt;
  Loader256 la, lb;
  if (famA) {
    mt = t / (d / 256); nt = t % (d / 256);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      la.rowp[i] = ut + (u * 4 * h + mt * 256 + loader256_row(i)) * s.Cp;
      lb.rowp[i] = kt + ((u * s.nC + r) * d + nt * 256 + loader256_row(i)) * s.Cp;
    }
  } else {
    const int64_t tb = t - na;
    mt = tb / (h / 256); nt = tb % (h / 256);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      la.rowp[i] = gt + (u * 2 * d + mt * 256 + loader256_row(i)) * s.Cp;
      lb.rowp[i] = zt + (u * h + nt * 256 + loader256_row(i)) * s.Cp;
    }
  }
  const int64_t nslab = s.Cp / Tile256::BK;
  const int64_t per = (nslab + nsplit - 1) / nsplit;
  const int64_t k0 = sp * per * Tile256::BK;
  const int64_t k1 = (sp * per + per < nslab ? sp * per + per : nslab) * Tile256::BK;
  f32x16_t acc[4][4];
  gemm_tile256(acc, la, lb, k0, k1, lds);

  // Output row R (tile row): 64-row block R/64 holds 32 W rows then 32 M rows
  // of the same 32 state rows, so accumulator block mi is W (mi even) or M.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, hf = lane >> 5;
  const int64_t P = 3 * d * h;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    // State rows of block mi: row base and stride in the packed state.
    const int64_t blk64 = (mt * 256 + wm * 128) / 64 + mi / 2;
    int64_t base, stride;
    if (famA) {
      const bool w3 = blk64 >= h / 32;
      base = (w3 ? h * d : 0) + (blk64 - (w3 ? h / 32 : 0)) * 32 * d;
      stride = d;
    } else {
      base = 2 * h * d + blk64 * 32 * h;
      stride = h;
    }
    float* dst = part + ((static_cast<int64_t>(sp) * 2 + (mi & 1)) * s.BH + u) * P + base;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int64_t c = nt * 256 + wn * 128 + ni * 32 + r32;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        dst[(8 * (v >> 2) + 4 * hf + (v & 3)) * stride + c] = acc[mi][ni][v];
    }
  }
}

// Chunk-end state from the split partials: 4 entries per thread (16-byte
// vectors), grid (BH * P / 4 + 255) / 256.
template <typename T>
__global__ __launch_bounds__(256) void k_agg_reduce(Shape s, int nsplit, int r, int last,
                                                    const float* __restrict__ part,
                                                    const float* __restrict__ coef,
                                                    const float* Win, const float* Min,
                                                    float* Wout, float* Mout, T* w13s, T* w2s,
                                                    T* w2ts) {
  const int64_t P = 3 * s.d * s.h;
  const int64_t q4 = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (q4 * 4 >= s.BH * P) return;
  const int64_t u = (q4 * 4) / P, e = (q4 * 4) % P;
  const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(Win + u * P + e);
  const f32x4_t m0 = *reinterpret_cast<const f32x4_t*>(Min + u * P + e);
  f32x4_t aw = *reinterpret_cast<const f32x4_t*>(part + u * P + e);
  f32x4_t am = *reinterpret_cast<const f32x4_t*>(part + (s.BH + u) * P + e);
  for (int sp = 1; sp < nsplit; ++sp) {
    aw += *reinterpret_cast<const f32x4_t*>(part + ((sp * 2) * s.BH + u) * P + e);
    am += *reinterpret_cast<const f32x4_t*>(part + ((sp * 2 + 1) * s.BH + u) * P + e);
  }
  const float* cf = coef + (u * s.nC + r) * 4;
  const float cW = cf[0], cM = cf[1], cWM = cf[2];
  f32x4_t wn, mn;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    wn[i] = cW * w0[i] + cWM * m0[i] + aw[i];
    mn[i] = cM * m0[i] + am[i];
  }
  *reinterpret_cast<f32x4_t*>(Wout + u * P + e) = wn;
  *reinterpret_cast<f32x4_t*>(Mout + u * P + e) = mn;
  if (!last) {
#pragma unroll
    for (int i = 0; i < 4; ++i) write_shadow<T>(s, u, e + i, wn[i], w13s, w2s, w2ts);
  }
}

}  // namespace e2ttt
