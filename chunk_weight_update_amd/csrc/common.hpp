// common.hpp -- device-side building blocks shared by the E2-TTT kernels
// (gfx950 / CDNA4: wave64, MFMA 32x32 tiles, LDS staging).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace e2ttt {

typedef uint16_t bf16_t;  // bf16 storage (upper half of an fp32)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even, by gfx950's conversion instruction
// (v_cvt_pk_bf16_f32, one per two values).  It equals rounding the fp32 bit
// pattern to its upper half with ties to even for every non-NaN input,
// denormals included (compared on the device over all 2^32 patterns); a NaN
// stays a NaN.  A software rounding costs about six VALU instructions per
// value, and the wave64 VALU issues at a quarter of the lane rate, which made
// it a visible part of the GEMM epilogues.
__device__ __forceinline__ bf16_t f2bf(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two fp32 -> one dword of two bf16 (same rounding), lo = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) { return bf2f(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f2bf(x); }

// Logistic function with the hardware reciprocal (about 1 ulp), which keeps
// the epilogues free of the multi-instruction IEEE divide sequence.
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// Logical workgroup index for an XCD-aware layout.  gfx950 hands consecutive
// workgroups of a grid to its 8 XCDs in turn, and each XCD has its own L2, so
// workgroups that read the same data (the hidden blocks of one unit, the
// row tiles of one unit's weights) are numbered so that each XCD receives a
// contiguous logical range: physical b -> (b % 8) * (G / 8) + b / 8.  A
// bijection on [0, G) when G is a multiple of 8; otherwise the identity.
__device__ __forceinline__ int64_t xcd_logical_block() {
  const int64_t b = blockIdx.x, G = gridDim.x;
  if (G % 8 != 0) return b;
  return (b % 8) * (G / 8) + b / 8;
}

// ---------------------------------------------------------------------------
// MFMA 32x32 wrappers.  Output layout (both types): lane l, register v holds
// D[row = 8*(v/4) + 4*(l/32) + v%4][col = l%32].  Operand fragments: lane l
// holds A[row = l%32][KPL consecutive k] and B^T[col = l%32][same k].  Which
// k each lane half covers only has to agree between A and B; the tile code
// gives lane half hf = l/32 the contiguous half [hf*BK/2, (hf+1)*BK/2) of a
// k-slab, so fragment reads are wide and contiguous.
template <typename T> struct Mfma;

template <> struct Mfma<bf16_t> {
  static constexpr int KPL = 8;  // k elements per lane per instruction
  typedef bf16x8_t frag;
  static __device__ __forceinline__ frag load(const bf16_t* p) {
    return *reinterpret_cast<const bf16x8_t*>(p);
  }
  static __device__ __forceinline__ f32x16_t mma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  typedef float frag;
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  static __device__ __forceinline__ f32x16_t mma(frag a, frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// 128x128 output tile, 256 threads = 4 waves in a 2x2 grid, each wave 64x64
// (2x2 MFMA blocks).  A slab is BK elements of K = 128 bytes per row.
template <typename T> struct Tile {
  static constexpr int BM = 128, BN = 128;
  static constexpr int VE = 16 / sizeof(T);        // elements per 16-byte vector
  static constexpr int BK = 128 / sizeof(T);       // 64 (bf16) or 32 (f32)
  static constexpr int LDSW = BK + VE;             // padded LDS row (elements)
  static constexpr int SLAB = BM * LDSW;           // elements per operand slab
  static constexpr int LDS_BYTES = 4 * SLAB * sizeof(T);  // A,B x double buffer
  static constexpr int KSTEPS = (BK / 2) / Mfma<T>::KPL;
};

// Per-thread loader state for one 128-row operand: thread tid loads rows
// (tid>>3) + 32*i, vector (tid&7) of every slab.
template <typename T> struct RowLoader {
  const T* rowp[4];
  __device__ __forceinline__ void load(uint4 (&r)[4], int64_t k0) const {
    const int vec = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (rowp[i]) r[i] = *reinterpret_cast<const uint4*>(rowp[i] + k0 + vec * Tile<T>::VE);
      else r[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
};

template <typename T>
__device__ __forceinline__ void stage_lds(T* slab, const uint4 (&r)[4]) {
  const int row0 = threadIdx.x >> 3, vec = threadIdx.x & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint4*>(slab + (row0 + 32 * i) * Tile<T>::LDSW + vec * Tile<T>::VE) = r[i];
}

__device__ __forceinline__ int loader_row(int i) { return (threadIdx.x >> 3) + 32 * i; }

// acc[mi][ni] += A[wm*64+mi*32.., :] * B[wn*64+ni*32.., :]^T over one slab.
template <typename T>
__device__ __forceinline__ void mma_slab(const T* As, const T* Bs, f32x16_t (&acc)[2][2]) {
  typedef Mfma<T> M;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, hf = lane >> 5;
  const T* a0 = As + (wm * 64 + r32) * Tile<T>::LDSW + hf * (Tile<T>::BK / 2);
  const T* b0 = Bs + (wn * 64 + r32) * Tile<T>::LDSW + hf * (Tile<T>::BK / 2);
#pragma unroll
  for (int s = 0; s < Tile<T>::KSTEPS; ++s) {
    const int ko = s * M::KPL;
    typename M::frag fa0 = M::load(a0 + ko);
    typename M::frag fa1 = M::load(a0 + 32 * Tile<T>::LDSW + ko);
    typename M::frag fb0 = M::load(b0 + ko);
    typename M::frag fb1 = M::load(b0 + 32 * Tile<T>::LDSW + ko);
    acc[0][0] = M::mma(fa0, fb0, acc[0][0]);
    acc[0][1] = M::mma(fa0, fb1, acc[0][1]);
    acc[1][0] = M::mma(fa1, fb0, acc[1][0]);
    acc[1][1] = M::mma(fa1, fb1, acc[1][1]);
  }
}

// C_tile = A_tile[128 x K] * B_tile[128 x K]^T with double-buffered LDS.
// A's k index wraps at `ka` (ka == K unless the A operand is repeated along K
// against a hi/lo split B operand); ka and K are multiples of BK.
template <typename T>
__device__ __forceinline__ void gemm_tile(f32x16_t (&acc)[2][2], const RowLoader<T>& la,
                                          const RowLoader<T>& lb, int64_t K, int64_t ka,
                                          T* lds) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  constexpr int BK = Tile<T>::BK, SLAB = Tile<T>::SLAB;
  // Buffer b of A is lds + 2*b*SLAB, of B lds + (2*b+1)*SLAB.  Selected by
  // arithmetic on the LDS pointer (not through an array of pointers) so the
  // compiler keeps LDS address space and emits ds_* instead of flat_* ops,
  // which would otherwise wait on the in-flight global prefetch.
  uint4 ra[4], rb[4];
  const int64_t nk = K / BK;
  la.load(ra, 0);
  lb.load(rb, 0);
  stage_lds(lds, ra);
  stage_lds(lds + SLAB, rb);
  __syncthreads();
  for (int64_t ks = 0; ks < nk; ++ks) {
    const int cur = static_cast<int>(ks & 1);
    const bool more = ks + 1 < nk;
    if (more) {
      const int64_t k1 = (ks + 1) * BK;
      la.load(ra, k1 % ka);
      lb.load(rb, k1);
    }
    T* Ac = lds + 2 * cur * SLAB;
    mma_slab<T>(Ac, Ac + SLAB, acc);
    if (more) {
      T* An = lds + 2 * (cur ^ 1) * SLAB;
      stage_lds(An, ra);
      stage_lds(An + SLAB, rb);
    }
    __syncthreads();
  }
}

// Accumulator coordinates inside the 128x128 tile.
struct AccPos {
  int wm, wn, r32, hf;
  __device__ __forceinline__ AccPos() {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    wm = wave >> 1; wn = wave & 1; r32 = lane & 31; hf = lane >> 5;
  }
  __device__ __forceinline__ int row(int mi, int v) const {
    return wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
  }
  __device__ __forceinline__ int col(int ni) const { return wn * 64 + ni * 32 + r32; }
};

// Store a 128x128 fp32 tile (in accumulator layout) transposed:
// dst[(col) * ldd + row] = T(val[row][col]), through LDS so that global
// writes are 16-byte vectors along `row`.  `lds` must hold 128*(128+VE) T.
// Synchronises the block before and after using LDS.
template <typename T>
__device__ __forceinline__ void store_tile_transposed(const float (&val)[2][2][16], T* lds,
                                                      T* dst, int64_t ldd) {
  constexpr int VE = Tile<T>::VE;
  constexpr int W = 128 + VE;
  const AccPos p;
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        lds[p.col(ni) * W + p.row(mi, v)] = from_f32<T>(val[mi][ni][v]);
  __syncthreads();
  constexpr int VPR = 128 / VE;  // vectors per transposed row
  for (int idx = threadIdx.x; idx < 128 * VPR; idx += 256) {
    const int r = idx / VPR, c = idx % VPR;
    *reinterpret_cast<uint4*>(dst + r * ldd + c * VE) =
        *reinterpret_cast<const uint4*>(lds + r * W + c * VE);
  }
  __syncthreads();
}

}  // namespace e2ttt
