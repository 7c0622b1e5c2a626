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
// tokens.  Slabs go from global memory straight into LDS (global_load_lds,
// no registers), four stages deep, so three slabs are in flight while one is
// computed: the memory latency is covered by three slabs of MFMA work rather
// than one.  LDS rows are 64 bytes, unpadded; the four 16-byte pieces of row
// r are stored in the order kc ^ swz256(r), so the 8 or 16 rows that one
// fragment read serves together hit distinct bank groups.  Per slab a wave
// reads 16 KB of fragments for 32 MFMAs.

// Token split: the tile count of one unit can be small (108 at d = 768,
// h = 1536), so the chunk's token slabs are split over S workgroups.  Each
// writes its fp32 partial aggregates in the packed state layout, and
// k_agg_reduce adds the S partials in split order (deterministic) and applies
// W_C = cW W_0 + cWM M_0 + A^W, M_C = cM M_0 + A^M plus the operand shadows.
#pragma once
#include <type_traits>

#include "kernels.hpp"

namespace e2ttt {

struct Tile256 {
  static constexpr int BM = 256, BN = 256, BK = 32;
  static constexpr int NST = 4;                             // LDS stages
  static constexpr int SLAB_BYTES = BM * BK * 2;            // one operand slab (bf16)
  static constexpr size_t LDS_BYTES = NST * 2 * SLAB_BYTES;  // A and B per stage: 128 KB
};

// Source of one 256-row operand for the direct LDS loads.  Load i (0..3) of
// wave w fills the 1 KB of LDS that holds slab rows 16*(4w+i) .. +15: lane l
// brings row 16*(4w+i) + l/4, physical piece l%4, which holds logical k-chunk
// loader256_chunk(i).  rowp[i] points at that row's chunk (k offset 0).
struct Loader256 {
  const bf16_t* rowp[4];
  // Load i of this wave for the slab starting at token k0 into `slab`.
  __device__ __forceinline__ void issue1(int i, int64_t k0, char* slab) const {
    const int wave = threadIdx.x >> 6;
    __builtin_amdgcn_global_load_lds(
        static_cast<const void*>(rowp[i] + k0),
        (__attribute__((address_space(3))) void*)(slab + (4 * wave + i) * 1024), 16, 0, 0);
  }
};

// Physical 16-byte piece of logical k-chunk kc in slab row r: kc ^ swz(r),
// with swz chosen so that 8 or 16 consecutive rows read at one chunk hit
// distinct 16-byte bank groups.
__device__ __forceinline__ int swz256(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

__device__ __forceinline__ int loader256_row(int i) {
  return 16 * (4 * (threadIdx.x >> 6) + i) + ((threadIdx.x & 63) >> 2);
}
__device__ __forceinline__ int loader256_chunk(int i) {
  return (threadIdx.x & 3) ^ swz256(loader256_row(i));
}

// Workgroup barrier without the memory fence of __syncthreads (whose
// release would wait for every load in flight, the prefetched slabs
// included).  LDS visibility is ordered by hand: the slab a barrier
// publishes was waited for with wait_vmcnt before it, and every LDS read of
// a stage is consumed (its MFMAs issued) before the barrier after which the
// stage is refilled.  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most 8n of this wave's slab loads are in flight (n slabs).
__device__ __forceinline__ void wait_slabs(int n);

// Wait until at most N vector memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

__device__ __forceinline__ void wait_slabs(int n) {
  if (n >= 3) wait_vmcnt<24>();
  else if (n == 2) wait_vmcnt<16>();
  else if (n == 1) wait_vmcnt<8>();
  else wait_vmcnt<0>();
}

// acc[mi][ni] (rows wm*128 + 32*mi, cols wn*128 + 32*ni) += A B^T over k
// [k0, k1) (multiples of 32).  Each slab costs a wave 8 loads (4 per
// operand); NST-1 slabs are in flight from global memory while one is
// computed.
//
// Order of one slab's instructions (fixed with scheduling fences): the
// fragments of the first MFMA group, then eight groups of four MFMAs, each
// followed by one of the slab's eight direct LDS loads and by the fragment
// reads of a later group.  A wave with all eight loads up front stalls on
// their issue (the load queue drains at the memory rate) before its first
// MFMA, so the loads and the matrix core took turns instead of overlapping
// (measured: about 1.25x more cycles per slab).  The loop over the slabs that
// issue a refill is kept free of conditions so that each slab body is one
// scheduling region; the last NST-1 slabs run in a second loop.
__device__ __forceinline__ void gemm_tile256(f32x16_t (&acc)[4][4], const Loader256& la,
                                             const Loader256& lb, int64_t k0, int64_t k1,
                                             char* lds) {
  constexpr int NST = Tile256::NST, SB = Tile256::SLAB_BYTES, BK = Tile256::BK;
  static_assert(NST == 4, "wait counts below assume four stages");
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, hf = lane >> 5, sw = swz256(r32);
  // Byte offset of this lane's fragment piece in k-step ks, inside a
  // 32-row block (the block bases are multiples of 32 rows, so the swizzle
  // only depends on r32).
  const int off0 = r32 * 64 + ((hf ^ sw) << 4), off1 = r32 * 64 + (((2 + hf) ^ sw) << 4);
  const int ns = static_cast<int>((k1 - k0) / BK);
  // Load q (0..7) of a slab: operand q / 4, piece q % 4 of the wave's rows.
  auto load = [&](int slab, int q) {
    char* st = lds + (slab % NST) * 2 * SB;
    (q < 4 ? la : lb).issue1(q & 3, k0 + static_cast<int64_t>(slab) * BK, st + (q < 4 ? 0 : SB));
  };
  auto body = [&](int s, bool refill) {
    const char* As = lds + (s % NST) * 2 * SB + wm * 128 * 64;
    const char* Bs = lds + (s % NST) * 2 * SB + SB + wn * 128 * 64;
    bf16x8_t fa[2][4], fb[2][4];
    auto rda = [&](int ks, int i) {
      fa[ks][i] = *reinterpret_cast<const bf16x8_t*>(As + i * 32 * 64 + (ks ? off1 : off0));
    };
    auto rdb = [&](int ks, int j) {
      fb[ks][j] = *reinterpret_cast<const bf16x8_t*>(Bs + j * 32 * 64 + (ks ? off1 : off0));
    };
    // Fragments read after group g (= 4 ks + i), one group ahead of their use.
    auto reads_after = [&](int g) {
      if (g == 0) rda(0, 2);
      else if (g == 1) rda(0, 3);
      else if (g == 2) { rdb(1, 0); rdb(1, 1); rdb(1, 2); rdb(1, 3); rda(1, 0); }
      else if (g == 3) rda(1, 1);
      else if (g == 4) rda(1, 2);
      else if (g == 5) rda(1, 3);
    };
    rdb(0, 0); rdb(0, 1); rdb(0, 2); rdb(0, 3); rda(0, 0); rda(0, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int ks = g >> 2, i = g & 3;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks][i], fb[ks][j], acc[i][j], 0, 0, 0);
      if (refill) load(s + NST - 1, g);
      reads_after(g);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Iteration s: wait for slab s (at most NST-2 later slabs in flight),
  // barrier (every wave has it, and every wave has read slab s-1, whose stage
  // takes slab s+NST-1), then slab s's MFMAs with that refill spread among
  // them.
#pragma unroll
  for (int p = 0; p < NST - 1; ++p)
    if (p < ns)
#pragma unroll
      for (int q = 0; q < 8; ++q) load(p, q);
  int s = 0;
  for (; s < ns - (NST - 1); ++s) {
    wait_vmcnt<8 * (NST - 2)>();
    barrier_nofence();
    body(s, true);
  }
  for (; s < ns; ++s) {
    const int later = ns - 1 - s;
    wait_slabs(later < NST - 2 ? later : NST - 2);
    barrier_nofence();
    body(s, false);
  }
  barrier_nofence();  // every wave's last reads are done before LDS is reused
}

// Partial aggregates of split sp over token slabs [k0, k1): workgroup
// (unit, split, tile); tiles 0 .. na-1 are family A (4h/256 x d/256), then
// family B (2d/256 x h/256).  The partial of state entry e goes to
// part[((sp * 2 + wm) * BH + u) * P + e], wm = 0 for A^W, 1 for A^M.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_agg256(
    Shape s, int nsplit, const bf16_t* __restrict__ ut, const bf16_t* __restrict__ kt,
    const bf16_t* __restrict__ gt, const bf16_t* __restrict__ zt, int r, float* part) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
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
      const int c8 = 8 * loader256_chunk(i);
      la.rowp[i] = ut + (u * 4 * h + mt * 256 + loader256_row(i)) * s.Cp + c8;
      lb.rowp[i] = kt + ((u * s.nC + r) * d + nt * 256 + loader256_row(i)) * s.Cp + c8;
    }
  } else {
    const int64_t tb = t - na;
    mt = tb / (h / 256); nt = tb % (h / 256);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c8 = 8 * loader256_chunk(i);
      la.rowp[i] = gt + (u * 2 * d + mt * 256 + loader256_row(i)) * s.Cp + c8;
      lb.rowp[i] = zt + (u * h + nt * 256 + loader256_row(i)) * s.Cp + c8;
    }
  }
  const int64_t nslab = s.Cp / Tile256::BK;
  const int64_t per = (nslab + nsplit - 1) / nsplit;
  const int64_t k0 = sp * per * Tile256::BK;
  const int64_t k1 = (sp * per + per < nslab ? sp * per + per : nslab) * Tile256::BK;
  f32x16_t acc[4][4];
  gemm_tile256(acc, la, lb, k0, k1, smem_raw);

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


// ---------------------------------------------------------------------------
// Forward of the generic path on the same 256 x 256 tiles (plain bf16
// operands, d, h and the padded chunk multiples of 256).  Same products and
// epilogues as k_fwd13 / k_fwd2; feature-major outputs go through
// LDS one accumulator band at a time: band mi holds tile rows 32*mi + [0,32)
// of both wave rows, i.e. tokens p0 + 32*mi + [0,32) and p0 + 128 + 32*mi +
// [0,32), as a [column][72] bf16 array (64 tokens + 8 pad).

// Operand rows past a chunk's valid tokens load from here (d <= 1024).
__device__ const bf16_t kZeroRow256[1024] = {};

struct Acc256Pos {
  int lane, wave, wm, wn, r32, hf;
  __device__ Acc256Pos() {
    lane = threadIdx.x & 63;
    wave = threadIdx.x >> 6;
    wm = wave >> 1;
    wn = wave & 1;
    r32 = lane & 31;
    hf = lane >> 5;
  }
  // Tile row of accumulator block (mi, *) register v.
  __device__ int row(int mi, int v) const { return 128 * wm + 32 * mi + 8 * (v >> 2) + 4 * hf + (v & 3); }
  // Tile column of accumulator block (*, ni).
  __device__ int col(int ni) const { return 128 * wn + 32 * ni + r32; }
};

// This lane's four consecutive band tokens 8*vq + 4*hf .. +3 of column c.
__device__ __forceinline__ void band_put(bf16_t* lds, int c, const Acc256Pos& ps, int vq,
                                         float x0, float x1, float x2, float x3) {
  *reinterpret_cast<uint2*>(lds + c * 72 + 32 * ps.wm + 8 * vq + 4 * ps.hf) =
      make_uint2(f2bf(x0) | (static_cast<uint32_t>(f2bf(x1)) << 16),
                 f2bf(x2) | (static_cast<uint32_t>(f2bf(x3)) << 16));
}

// Copy ncol band columns out: column c's 64 tokens go to dst_row(c)[0 .. 31]
// and dst_row(c)[128 .. 159] (16-byte vectors).
template <typename RowFn>
__device__ __forceinline__ void band_copy(const bf16_t* lds, int ncol, RowFn dst_row) {
  for (int idx = threadIdx.x; idx < ncol * 8; idx += 256) {
    const int c = idx >> 3, q = idx & 7, half = q >> 2, tok = 8 * (q & 3);
    *reinterpret_cast<uint4*>(dst_row(c) + 128 * half + tok) =
        *reinterpret_cast<const uint4*>(lds + c * 72 + 32 * half + tok);
  }
}

// Compile-time band index (the accumulator array must only be indexed by
// constants, or it is moved to scratch memory).
template <int N>
using Band = std::integral_constant<int, N>;

template <bool B>
using Flag = std::integral_constant<bool, B>;

// Keeps an accumulator block in AGPRs up to this point: without it the
// compiler moves all 256 accumulators to VGPRs right after the k loop, which
// do not fit next to the epilogue's own values.
__device__ __forceinline__ void pin_acc(f32x16_t& x) { asm volatile("" : "+a"(x)); }

template <typename F>
__device__ __forceinline__ void for_bands(F&& f) {
  f(Band<0>{});
  f(Band<1>{});
  f(Band<2>{});
  f(Band<3>{});
}

// fwd13: [K; Q] rows x [W1; W3]^T (w13s rows interleaved in blocks of 32, so
// accumulator blocks 2*pr and 2*pr+1 are A1 and A3 of the same 32 hidden
// units) -> Z = silu(A1) A3 row-major, A1 and A3 (fp32) and Z^T for K rows.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_fwd13_256(
    Shape s, int r, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ w13s, bf16_t* zrow, float* a1s, float* a3s, bf16_t* zt) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  const int64_t ntn = 2 * s.h / 256, ntm = 2 * s.Cp / 256, mtK = s.Cp / 256;
  int64_t bid = xcd_logical_block();
  const int64_t nt = bid % ntn; bid /= ntn;
  const int64_t mt = bid % ntm;
  const int64_t u = bid / ntm;
  const bool isQ = mt >= mtK;
  const int64_t p0 = (mt - (isQ ? mtK : 0)) * 256;
  const int64_t tok0 = static_cast<int64_t>(r) * s.C;
  const int64_t nv = n_valid(s, r);
  const bf16_t* X = (isQ ? q : k) + (u * s.L + tok0) * s.d;
  Loader256 la, lb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c8 = 8 * loader256_chunk(i);
    const int64_t p = p0 + loader256_row(i);
    la.rowp[i] = (p < nv ? X + p * s.d : kZeroRow256) + c8;
    lb.rowp[i] = w13s + (u * 2 * s.h + nt * 256 + loader256_row(i)) * s.d + c8;
  }
  f32x16_t acc[4][4];
  gemm_tile256(acc, la, lb, 0, s.d, smem_raw);

  const Acc256Pos ps;
  bf16_t* lds = reinterpret_cast<bf16_t*>(smem_raw);
  const int h = static_cast<int>(s.h);
  // Row p0 of this tile in each output; offsets below are 32-bit.
  bf16_t* zq = zrow + (u * 2 * s.Cp + (isQ ? s.Cp : 0) + p0) * s.h + nt * 128;
  float* a1u = a1s + (u * s.Cp + p0) * s.h + nt * 128;
  float* a3u = a3s + (u * s.Cp + p0) * s.h + nt * 128;
  // Each band in two pieces (one per 32 hidden units), kept apart by
  // scheduling barriers so that only one piece's values are live at a time.
  auto band = [&](auto MI, auto KROWS) {
    constexpr int mi = decltype(MI)::value;
    constexpr bool krows = decltype(KROWS)::value;
    if constexpr (krows) __syncthreads();  // the previous Z^T band has been copied out
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const int j = ps.wn * 64 + pr * 32 + ps.r32;  // hidden unit - nt*128
      pin_acc(acc[mi][2 * pr]);
      pin_acc(acc[mi][2 * pr + 1]);
      float zv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int off = ps.row(mi, v) * h + j;
        const float a1 = acc[mi][2 * pr][v], a3 = acc[mi][2 * pr + 1][v];
        const float z = a1 * sigmoidf_(a1) * a3;
        zv[v] = z;
        zq[off] = f2bf(z);
        if constexpr (krows) {
          a1u[off] = a1;
          a3u[off] = a3;
        }
      }
      if constexpr (krows) {
#pragma unroll
        for (int vq = 0; vq < 4; ++vq)
          band_put(lds, j, ps, vq, zv[4 * vq], zv[4 * vq + 1], zv[4 * vq + 2], zv[4 * vq + 3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (krows) {  // Z^T band: 128 hidden rows x 64 tokens
      __syncthreads();
      band_copy(lds, 128, [&](int c) { return zt + (u * s.h + nt * 128 + c) * s.Cp + p0 + 32 * mi; });
    }
  };
  if (isQ) for_bands([&](auto MI) { band(MI, Flag<false>{}); });
  else for_bands([&](auto MI) { band(MI, Flag<true>{}); });
}

// fwd2: Z rows x W2^T -> Y; the readout for Q rows, g = v - Y for K rows
// (row-major) and K^W g, K^M g feature-major (rows 64*(i/32) + i%32, +32 for
// the momentum copy).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_fwd2_256(
    Shape s, int r, const bf16_t* __restrict__ v, bf16_t* out, const bf16_t* __restrict__ zrow,
    const bf16_t* __restrict__ w2s, const float* __restrict__ kw, const float* __restrict__ km,
    bf16_t* grow, bf16_t* gt) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  const int64_t ntn = s.d / 256, ntm = 2 * s.Cp / 256, mtK = s.Cp / 256;
  int64_t bid = xcd_logical_block();
  const int64_t nt = bid % ntn; bid /= ntn;
  const int64_t mt = bid % ntm;
  const int64_t u = bid / ntm;
  const bool isQ = mt >= mtK;
  const int64_t p0 = (mt - (isQ ? mtK : 0)) * 256;
  const int64_t tok0 = static_cast<int64_t>(r) * s.C;
  const int64_t nv = n_valid(s, r);
  Loader256 la, lb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c8 = 8 * loader256_chunk(i);
    la.rowp[i] = zrow + (u * 2 * s.Cp + mt * 256 + loader256_row(i)) * s.h + c8;
    lb.rowp[i] = w2s + (u * s.d + nt * 256 + loader256_row(i)) * s.h + c8;
  }
  f32x16_t acc[4][4];
  gemm_tile256(acc, la, lb, 0, s.h, smem_raw);

  const Acc256Pos ps;
  const int d = static_cast<int>(s.d);
  const int nvt = static_cast<int>(nv - p0 < 256 ? nv - p0 : 256);  // valid rows of the tile
  if (isQ) {
    bf16_t* o = out + (u * s.L + tok0) * s.d + nt * 256;
    auto band = [&](auto MI, auto FULL) {
      constexpr int mi = decltype(MI)::value;
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        pin_acc(acc[mi][ni]);
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
          const int pr = ps.row(mi, vv);
          if (decltype(FULL)::value || pr < nvt)
            o[(p0 + pr) * s.d + ps.col(ni)] = f2bf(acc[mi][ni][vv]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (nvt == 256) for_bands([&](auto MI) { band(MI, Flag<true>{}); });
    else for_bands([&](auto MI) { band(MI, Flag<false>{}); });
    return;
  }
  bf16_t* lds = reinterpret_cast<bf16_t*>(smem_raw);
  bf16_t* ldsM = lds + 256 * 72;
  const bf16_t* vs = v + (u * s.L + tok0 + p0) * s.d + nt * 256;
  bf16_t* gr = grow + (u * s.Cp + p0) * s.d + nt * 256;
  const float* kwr = kw + (u * s.nC + r) * s.Cp + p0;
  const float* kmr = km + (u * s.nC + r) * s.Cp + p0;
  bf16_t* gbase = gt + u * 2 * s.d * s.Cp + p0;
  auto band = [&](auto MI, auto FULL) {
    constexpr int mi = decltype(MI)::value;
    constexpr bool full = decltype(FULL)::value;
    // All loads of the band first (v as bf16, the kernels): grow may alias v
    // as far as the compiler knows.  Rows past the valid tokens read row 0
    // and use 0.  Then one piece per accumulator column block, kept apart by
    // scheduling barriers.
    bf16_t vb[4][16];
    float kwv[16], kmv[16];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int pr = ps.row(mi, vv);
        vb[ni][vv] = vs[(full || pr < nvt ? pr : 0) * d + ps.col(ni)];
      }
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) {
      kwv[vv] = kwr[ps.row(mi, vv)];
      kmv[vv] = kmr[ps.row(mi, vv)];
    }
    __syncthreads();  // the previous band has been copied out
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      pin_acc(acc[mi][ni]);
      float g[16];
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        const int pr = ps.row(mi, vv);
        g[vv] = (full || pr < nvt ? bf2f(vb[ni][vv]) : 0.0f) - acc[mi][ni][vv];
        gr[pr * d + ps.col(ni)] = f2bf(g[vv]);
      }
      const int c = ps.col(ni);
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        band_put(lds, c, ps, vq, kwv[4 * vq] * g[4 * vq], kwv[4 * vq + 1] * g[4 * vq + 1],
                 kwv[4 * vq + 2] * g[4 * vq + 2], kwv[4 * vq + 3] * g[4 * vq + 3]);
        band_put(ldsM, c, ps, vq, kmv[4 * vq] * g[4 * vq], kmv[4 * vq + 1] * g[4 * vq + 1],
                 kmv[4 * vq + 2] * g[4 * vq + 2], kmv[4 * vq + 3] * g[4 * vq + 3]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    band_copy(lds, 256, [&](int c) {
      const int64_t i = nt * 256 + c;
      return gbase + (64 * (i / 32) + i % 32) * s.Cp + 32 * mi;
    });
    band_copy(ldsM, 256, [&](int c) {
      const int64_t i = nt * 256 + c;
      return gbase + (64 * (i / 32) + 32 + i % 32) * s.Cp + 32 * mi;
    });
  };
  if (nvt == 256) for_bands([&](auto MI) { band(MI, Flag<true>{}); });
  else for_bands([&](auto MI) { band(MI, Flag<false>{}); });
}

}  // namespace e2ttt
