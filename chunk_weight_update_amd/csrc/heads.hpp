// heads.hpp -- the per-token scalar heads of the TTT branch.
//
// "Rethinking Expressivity and Efficiency in Test-Time Training", §4
// (Overall Architecture, Input-Dependent Dynamics), App. B.3 and B.4: linear
// heads on the layer input x_t predict eta_t, alpha_t and beta_t for every
// TTT head; eta_base and alpha_base scale sigmoid gates.  Per head h:
//   eta   = eta_base   * sigma(<w_eta_h,   x_t> + b_eta_h)
//   alpha = alpha_base * sigma(<w_alpha_h, x_t> + b_alpha_h)
//   beta  =              sigma(<w_beta_h,  x_t> + b_beta_h)
// (Eq. 13, beta's timescale form, is missing from the page: a plain sigmoid
// gate is taken).  As a product: Z = X W^T, X [B*L, D], W [3H, D], then the
// gates.  x is read once for all 3H heads (each token's x feeds every head,
// so a per-(unit, chunk) fusion into the scan would read it H times).
//
// One workgroup = 4 waves x 2 row blocks of 16 tokens = 128 tokens, all 3H
// head columns (3, 6 or 12 column blocks of 16, a compile-time count).  W goes through LDS in
// slabs of 64 k (double-buffered; each slab's global loads issued two slabs
// ahead into registers); each lane streams its rows of x straight from
// global memory into a ring of registers PX slabs deep.  The MFMA work per
// slab is small, so the rate is set by the bytes in flight: one slab ahead
// (16 KB of x per CU) ran at 2.2 TB/s.  Barriers wait for the LDS stores
// only, never for the prefetches.  MFMA 16x16x32 bf16 or 16x16x4 fp32:
// lane l feeds row / column l%16 and the k group l/16 of a 16-byte vector
// (8 bf16 or 4 fp32 consecutive k; the fp32 case splits the vector over
// four instructions, A and B with the same k order).
#pragma once

#include "common.hpp"

namespace e2ttt {

struct HeadsArgs {
  const void* x;       // [N][D] io type, N = B * L
  const void* w;       // [3H][D] io type: eta heads, alpha heads, beta heads
  const float* bias;   // [3H]
  int64_t N, L, D;
  int H;
  float eta_base, alpha_base;
  float* eta;          // [B][H][L]
  float* alpha;
  float* beta;
};

// NBT: column blocks of 16 computed (3, 6 or 12: 3H <= 48, 96, 192); the
// columns past 3H read a clamped row of W and are never stored.
template <typename T, int NBT> struct HeadsCfg {
  static constexpr int KS = 64;                         // k per slab
  static constexpr int VE = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte vector
  static constexpr int KSTEP = 4 * VE;                  // k per step (4 lane groups)
  static constexpr int NSTEP = KS / KSTEP;              // steps per slab
  static constexpr int VPR = KS / VE;                   // vectors per W row of a slab
  static constexpr int WVEC = (NBT * 16 * VPR + 255) / 256;  // W vectors per thread per slab
  static constexpr int MAXC = WVEC * 256 / VPR;         // W rows one slab's stores cover
  static constexpr int ROW = KS + 16 / static_cast<int>(sizeof(T));  // LDS row, +16 bytes
  static constexpr int RB = 2;                          // row blocks of 16 per wave
  static constexpr int ROWS = 4 * RB * 16;              // tokens per workgroup
  static constexpr size_t LDS_BYTES = static_cast<size_t>(2) * MAXC * ROW * sizeof(T);
  static constexpr int PX = sizeof(T) == 2 ? 4 : 2;     // slabs of x in flight
  static constexpr int PW = 2;                          // slabs of W in flight (PW divides PX)
  static_assert(MAXC >= NBT * 16, "the stores cover the computed columns");
};
constexpr int kHeadsRows = 128;  // tokens per workgroup (every configuration)

template <typename T> struct HeadsVec;
template <> struct HeadsVec<bf16_t> { typedef bf16x8_t type; };
template <> struct HeadsVec<float> { typedef f32x4_t type; };

template <typename T>
__device__ __forceinline__ f32x4_t heads_mma(const typename HeadsVec<T>::type& a,
                                             const typename HeadsVec<T>::type& b, f32x4_t c);
template <>
__device__ __forceinline__ f32x4_t heads_mma<bf16_t>(const bf16x8_t& a, const bf16x8_t& b,
                                                     f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4_t heads_mma<float>(const f32x4_t& a, const f32x4_t& b,
                                                    f32x4_t c) {
#pragma unroll
  for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
  return c;
}

template <typename T, int NBT>
__global__ __launch_bounds__(256) void k_heads(HeadsArgs a) {
  typedef HeadsCfg<T, NBT> S;
  static_assert(S::ROWS == kHeadsRows, "rows per workgroup");
  typedef typename HeadsVec<T>::type V;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  T* Wl = reinterpret_cast<T*>(smem_raw);  // [2][MAXC][ROW]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int NC = 3 * a.H;
  const int64_t nslab = a.D / S::KS;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * S::ROWS + wave * (S::RB * 16);
  const T* X = static_cast<const T*>(a.x);
  const T* Wg = static_cast<const T*>(a.w);

  // W slab s -> registers (rows past 3H are zero).
  V wr[S::PW][S::WVEC];
  // Loads are unconditional (clamped rows and slabs): a predicated load makes
  // the compiler's wait counts fall back to waiting for every load in flight.
  // Columns past 3H and rows past N only feed accumulators that are never
  // stored; slabs past the last are loaded and not used.
  auto load_w = [&](int64_t s, V (&wv)[S::WVEC]) {
    const int64_t sc = s < nslab ? s : nslab - 1;
#pragma unroll
    for (int i = 0; i < S::WVEC; ++i) {
      const int idx = tid + 256 * i;
      const int c0 = idx / S::VPR, kv = idx % S::VPR;
      const int c = c0 < NC ? c0 : NC - 1;
      wv[i] = *reinterpret_cast<const V*>(Wg + c * a.D + sc * S::KS + kv * S::VE);
    }
  };
  // (every thread stores: rows past the 3H columns are in the buffer, unread)
  auto store_w = [&](int buf, const V (&wv)[S::WVEC]) {
#pragma unroll
    for (int i = 0; i < S::WVEC; ++i) {
      const int idx = tid + 256 * i;
      const int c = idx / S::VPR, kv = idx % S::VPR;
      *reinterpret_cast<V*>(Wl + (buf * S::MAXC + c) * S::ROW + kv * S::VE) = wv[i];
    }
  };
  // This lane's x vectors of slab s: row block rb, step st (rows past N are zero).
  V xr[S::PX][S::RB][S::NSTEP];
  auto load_x = [&](int64_t s, V (&dst)[S::RB][S::NSTEP]) {
    const int64_t sc = s < nslab ? s : nslab - 1;
#pragma unroll
    for (int rb = 0; rb < S::RB; ++rb) {
      const int64_t r = row0 + rb * 16 + l16;
      const int64_t row = r < a.N ? r : a.N - 1;
#pragma unroll
      for (int st = 0; st < S::NSTEP; ++st)
        dst[rb][st] = *reinterpret_cast<const V*>(X + row * a.D + sc * S::KS + st * S::KSTEP +
                                                  g * S::VE);
    }
  };
  // Workgroup barrier that waits for this wave's LDS stores but not for its
  // global loads in flight (__syncthreads would drain those as well).
  auto barrier_lds = [] {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x4_t acc[S::RB][NBT];
#pragma unroll
  for (int rb = 0; rb < S::RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < NBT; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Prologue: W slabs 0, 1 and x slabs 0 .. PX-1 in flight; W slab 0 into
  // LDS buffer 0, then W slab PW into the freed register slot.
  static_assert(S::PW == 2 && S::PX % S::PW == 0, "ring periods");
  load_w(0, wr[0]);
  load_w(1, wr[1]);
#pragma unroll
  for (int p = 0; p < S::PX; ++p) load_x(p, xr[p]);
  store_w(0, wr[0]);
  load_w(2, wr[0]);
  barrier_lds();
  // Slab s: x in xr[s % PX], W in LDS buffer s % 2; then W slab s+1 into the
  // other buffer (read by every wave during slab s-1, before the last
  // barrier), W slab s+3 into the register slot just stored, x slab s+PX
  // into the slot just used.
  for (int64_t s0 = 0; s0 < nslab; s0 += S::PX) {
#pragma unroll
    for (int j = 0; j < S::PX; ++j) {
      const int64_t s = s0 + j;
      if (s < nslab) {
        const T* Wb = Wl + (j & 1) * S::MAXC * S::ROW;
#pragma unroll
        for (int st = 0; st < S::NSTEP; ++st) {
#pragma unroll
          for (int cb = 0; cb < NBT; ++cb) {
            const V b = *reinterpret_cast<const V*>(Wb + (cb * 16 + l16) * S::ROW +
                                                    st * S::KSTEP + g * S::VE);
#pragma unroll
            for (int rb = 0; rb < S::RB; ++rb)
              acc[rb][cb] = heads_mma<T>(xr[j][rb][st], b, acc[rb][cb]);
          }
        }
        store_w((j + 1) & 1, wr[(j + 1) & 1]);
        load_w(s + 3, wr[(j + 1) & 1]);
        load_x(s + S::PX, xr[j]);
        barrier_lds();
      }
    }
  }

  // Gates: lane holds column cb*16 + l16, rows 4g .. 4g+3 of each block.
#pragma unroll
  for (int cb = 0; cb < NBT; ++cb) {
    const int c = cb * 16 + l16;
    if (c >= NC) continue;
    const int grp = c / a.H, head = c % a.H;
    float* dst = grp == 0 ? a.eta : grp == 1 ? a.alpha : a.beta;
    const float scale = grp == 0 ? a.eta_base : grp == 1 ? a.alpha_base : 1.0f;
    const float bc = a.bias[c];
#pragma unroll
    for (int rb = 0; rb < S::RB; ++rb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = row0 + rb * 16 + 4 * g + j;
        if (n < a.N) {
          const int64_t b = n / a.L, t = n % a.L;
          const float z = acc[rb][cb][j] + bc;
          dst[(b * a.H + head) * a.L + t] = scale / (1.0f + __expf(-z));
        }
      }
    }
  }
}

}  // namespace e2ttt
