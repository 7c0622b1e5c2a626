// gemm256.hpp -- the bf16 MFMA GEMMs of the generic SwiGLU path when d, h
// and the padded chunk are multiples of 256 (the large-state layer): the
// forward products, the backward's dZ and the aggregation, with their fused
// epilogues, and the streaming state epilogue.
//
// The aggregations of §3.2 / App. A.4 of "Rethinking Expressivity and
// Efficiency in Test-Time Training" contract over the chunk's tokens:
//   family A: [K^W dA1 | K^M dA1 | K^W dA3 | K^M dA3]^T K   (4h x d)
//   family B: [K^W g | K^M g]^T Z                          (2d x h)
// with operands already scaled and rounded once (the backward, the readout)
// and stored feature-major (rows = output rows, contiguous along tokens).
//
// Two engines share one slab format: k-slabs of 32 (tokens or features)
// go from global memory straight into LDS (global_load_lds, no registers),
// several stages deep, so later slabs are in flight while one is computed.
// LDS rows are 64 bytes, unpadded; the four 16-byte pieces of row r are
// stored in the order kc ^ swz256(r), so the 8 or 16 rows that one fragment
// read serves together hit distinct bank groups.
//   gemm_tile256w8: 256 x 256 tile, 8 waves of 128 x 64 (4 x 2 blocks of
//                   32x32x16 MFMA, 128 accumulator registers, two waves per
//                   SIMD) -- k_fwd13_256 and k_agg256.
//   gemm_rows256:   256 x 32*NB tile, 4 waves of 64 x 32*NB -- the readout
//                   (k_fwd2r) and the backward (k_bwd256), where 192-wide
//                   tiles give one workgroup per CU.
//
// Token split: the tile count of one unit can be small (108 at d = 768,
// h = 1536), so the chunk's token slabs are split over S workgroups.  Each
// writes its fp32 partial aggregates in the packed state layout, and
// k_agg_reduce adds the S partials in split order (deterministic) and applies
// W_C = cW W_0 + cWM M_0 + A^W, M_C = cM M_0 + A^M plus the operand shadows.
#pragma once
#include <type_traits>

#include "kernels.hpp"

namespace e2ttt {

// Physical 16-byte piece of logical k-chunk kc in slab row r: kc ^ swz(r),
// with swz chosen so that 8 or 16 consecutive rows read at one chunk hit
// distinct 16-byte bank groups.
__device__ __forceinline__ int swz256(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

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

// LDS writes visible to the workgroup; vector memory left in flight.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  barrier_nofence();
}

// Wait until at most N vector memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// 256 x 256 tile with 8 waves, two per SIMD: wave w takes rows
// 128*(w/4) + [0,128) (blocks mi = 0..3) and columns 64*(w%4) + [0,64)
// (blocks ni = 0, 1), 128 accumulator registers.  A stage holds the slab's
// 256 A rows then 256 B rows (64 bytes each, the engine's swizzle); each wave
// issues 4 of the slab's 32 direct loads, one every 4 of its 16 MFMAs.  With
// two waves per SIMD one wave's MFMAs run while the other is held by its
// load issue or its fragment reads, which with one wave per SIMD (4 waves of
// 128 x 128) took turns.  A wave with all of a slab's loads up front stalls
// on their issue (the load queue drains at the memory rate) before its first
// MFMA, so the loads are spread among the MFMA groups (measured on the
// 4-wave form: about 1.25x more cycles per slab otherwise).
struct Tile256w8 {
  static constexpr int BK = 32, NST = 4;
  static constexpr int STAGE = 512 * 64;                      // 32 KB
  static constexpr size_t LDS_BYTES = static_cast<size_t>(NST) * STAGE;  // 128 KB
};

// acc[mi][ni] += A B^T over k [k0, k0 + 32*ns), ns >= 1; arow(R), brow(R)
// point at row R of A, B (R < 256, k contiguous, at k = 0).
template <typename ARow, typename BRow>
__device__ __forceinline__ void gemm_tile256w8(f32x16_t (&acc)[4][2], ARow arow, BRow brow,
                                               int64_t k0, int ns, char* lds) {
  constexpr int NST = Tile256w8::NST, SB = Tile256w8::STAGE, BK = Tile256w8::BK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const bf16_t* src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int R = 16 * (8 * i + wave) + (lane >> 2);
    const int c8 = 8 * ((lane & 3) ^ swz256(R));
    src[i] = (R < 256 ? arow(R) : brow(R - 256)) + k0 + c8;
  }
  auto load = [&](int slab, int i) {
    char* st = lds + (slab % NST) * SB;
    __builtin_amdgcn_global_load_lds(
        static_cast<const void*>(src[i] + static_cast<int64_t>(slab) * BK),
        (__attribute__((address_space(3))) void*)(st + (8 * i + wave) * 1024), 16, 0, 0);
  };
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  const int r32 = lane & 31, hf = lane >> 5, sw = swz256(r32);
  const int off0 = r32 * 64 + ((hf ^ sw) << 4), off1 = r32 * 64 + (((2 + hf) ^ sw) << 4);
  struct Frags { bf16x8_t a[4], b[2]; };
  auto read_frags = [&](Frags& f, const char* st, int ks) {
    const int off = ks ? off1 : off0;
    const char* As = st + wm * 128 * 64 + off;
    const char* Bs = st + (256 + wn * 64) * 64 + off;
    f.b[0] = *reinterpret_cast<const bf16x8_t*>(Bs);
    f.a[0] = *reinterpret_cast<const bf16x8_t*>(As);
    f.b[1] = *reinterpret_cast<const bf16x8_t*>(Bs + 32 * 64);
#pragma unroll
    for (int mi = 1; mi < 4; ++mi) f.a[mi] = *reinterpret_cast<const bf16x8_t*>(As + mi * 32 * 64);
  };
  auto step = [&](const Frags& f, auto&& between) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int mi = m >> 1, ni = m & 1;
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mi], f.b[ni], acc[mi][ni], 0, 0, 0);
      between(m);
    }
  };
  auto body = [&](int sl, bool refill) {
    const char* st = lds + (sl % NST) * SB;
    Frags f0, f1;
    read_frags(f0, st, 0);
    __builtin_amdgcn_sched_barrier(0);
    step(f0, [&](int m) {
      if (m == 1) read_frags(f1, st, 1);
      if (refill && (m & 3) == 1) load(sl + NST - 1, m >> 2);
      __builtin_amdgcn_sched_barrier(0);
    });
    step(f1, [&](int m) {
      if (refill && (m & 3) == 1) load(sl + NST - 1, 2 + (m >> 2));
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  static_assert(NST == 4, "wait counts below assume four stages");
#pragma unroll
  for (int p = 0; p < NST - 1; ++p)
    if (p < ns)
#pragma unroll
      for (int i = 0; i < 4; ++i) load(p, i);
  // Iteration sl: wait for slab sl (at most NST-2 later slabs in flight),
  // barrier (every wave has it, and every wave has read slab sl-1, whose
  // stage takes slab sl+NST-1), then slab sl's MFMAs with that refill.
  int sl = 0;
  for (; sl < ns - (NST - 1); ++sl) {
    wait_vmcnt<4 * (NST - 2)>();
    barrier_nofence();
    body(sl, true);
  }
  for (; sl < ns; ++sl) {
    const int later = ns - 1 - sl;  // slabs loaded after this one
    if (later >= 2) wait_vmcnt<8>();
    else if (later == 1) wait_vmcnt<4>();
    else wait_vmcnt<0>();
    barrier_nofence();
    body(sl, false);
  }
  barrier_nofence();  // every wave's last reads are done before LDS is reused
}

// Partial aggregates of split sp over token slabs [k0, k1): workgroup
// (unit, split, tile); tiles 0 .. na-1 are family A, then family B (2d/256 x
// h/256).  Family A is either (s.sk = 0) the scaled backward operands
// [K^W dA1 | K^M dA1 | K^W dA3 | K^M dA3]^T against K (4h/256 x d/256 tiles,
// W and M rows interleaved in 32-row groups) or (s.sk = 1) the unscaled
// [dA1 | dA3]^T against the scaled keys [K^W K | K^M K] (2h/256 x 2d/256
// tiles; column block nt < d/256 is A^W, the rest A^M).  The partial of
// state entry e goes to part[((sp * 2 + wm) * BH + u) * P + e], wm = 0 for
// A^W, 1 for A^M.  8 waves on the 256 x 256 tile (gemm_tile256w8).
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_agg256(
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
  const bf16_t* abase;
  const bf16_t* bbase;
  if (famA && s.sk) {
    mt = t / (2 * d / 256); nt = t % (2 * d / 256);
    abase = ut + (u * 2 * h + mt * 256) * s.Cp;
    bbase = kt + ((u * s.nC + r) * 2 * d + nt * 256) * s.Cp;
  } else if (famA) {
    mt = t / (d / 256); nt = t % (d / 256);
    abase = ut + (u * 4 * h + mt * 256) * s.Cp;
    bbase = kt + ((u * s.nC + r) * d + nt * 256) * s.Cp;
  } else {
    const int64_t tb = t - na;
    mt = tb / (h / 256); nt = tb % (h / 256);
    abase = gt + (u * 2 * d + mt * 256) * s.Cp;
    bbase = zt + (u * h + nt * 256) * s.Cp;
  }
  const int64_t nslab = s.Cp / Tile256w8::BK;
  const int64_t per = (nslab + nsplit - 1) / nsplit;
  const int64_t sl0 = sp * per;
  const int64_t sl1 = sl0 + per < nslab ? sl0 + per : nslab;
  f32x16_t acc[4][2];
  gemm_tile256w8(acc, [&](int R) { return abase + R * s.Cp; }, [&](int R) { return bbase + R * s.Cp; },
                 sl0 * Tile256w8::BK, static_cast<int>(sl1 - sl0), smem_raw);

  // Output row R (tile row): 64-row block R/64 holds 32 W rows then 32 M rows
  // of the same 32 state rows, so accumulator block mi is W (mi even) or M.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int r32 = lane & 31, hf = lane >> 5;
  const int64_t P = 3 * d * h;
  if (famA && s.sk) {
    // Tile rows: state rows of W1 (R < h) or W3 (R >= h, which follow W1 in
    // the packed state); columns: A^W (c < d) or A^M (c - d).
    const int mflag = nt * 256 >= d ? 1 : 0;
    float* dst = part + ((static_cast<int64_t>(sp) * 2 + mflag) * s.BH + u) * P +
                 (mt * 256 + wm * 128) * d + nt * 256 - mflag * d;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int64_t c = wn * 64 + ni * 32 + r32;
#pragma unroll
        for (int v = 0; v < 16; ++v)
          dst[(32 * mi + 8 * (v >> 2) + 4 * hf + (v & 3)) * d + c] = acc[mi][ni][v];
      }
    return;
  }
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
    for (int ni = 0; ni < 2; ++ni) {
      const int64_t c = nt * 256 + wn * 64 + ni * 32 + r32;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        dst[(8 * (v >> 2) + 4 * hf + (v & 3)) * stride + c] = acc[mi][ni][v];
    }
  }
}

// Chunk-end state from the split partials (the S partials added in split
// order), plus the operand shadows of the next chunk's weights.  Blocks
// [0, nA) take the W1/W3 entries of all units, 4 consecutive entries per
// thread (16-byte state accesses, 8-byte shadow stores of one shadow row);
// the other blocks take one 64 x 64 tile of a unit's W2 each, so that the
// transposed shadow W2^T is written in rows through LDS.
__host__ __device__ inline int64_t agg_reduce_blocks_a(const Shape& s) { return (s.BH * 2 * s.h * s.d / 4 + 255) / 256; }
__host__ __device__ inline int64_t agg_reduce_blocks(const Shape& s) {
  return agg_reduce_blocks_a(s) + s.BH * (s.d / 64) * (s.h / 64);
}

template <typename T>
__device__ __forceinline__ void put4_shadow(T* hi, int kr, int64_t lo_off, const f32x4_t& w) {
  const float x[4] = {w[0], w[1], w[2], w[3]};
  split_store4<T>(x, hi, kr == 2 ? hi + lo_off : nullptr);
}

template <typename T>
__global__ __launch_bounds__(256) void k_agg_reduce(Shape s, int nsplit, int r, int last,
                                                    const float* __restrict__ part,
                                                    const float* __restrict__ coef,
                                                    const float* Win, const float* Min,
                                                    float* Wout, float* Mout, T* w13s, T* w2s,
                                                    T* w2ts) {
  __shared__ float tT[64 * 65];
  const int64_t d = s.d, h = s.h, hd = h * d, P = 3 * hd;
  const int kr = s.krep;
  const int64_t nA = agg_reduce_blocks_a(s);
  const int64_t blk = blockIdx.x;
  // Four entries e .. e+3 of unit u: partial sums, chunk-end values.
  auto entry4 = [&](int64_t u, int64_t e, f32x4_t& wn) {
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
    f32x4_t mn;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wn[i] = cW * w0[i] + cWM * m0[i] + aw[i];
      mn[i] = cM * m0[i] + am[i];
    }
    *reinterpret_cast<f32x4_t*>(Wout + u * P + e) = wn;
    *reinterpret_cast<f32x4_t*>(Mout + u * P + e) = mn;
  };
  if (blk < nA) {  // W1 / W3
    const int64_t q4 = blk * 256 + threadIdx.x;
    if (q4 * 4 >= s.BH * 2 * hd) return;
    const int64_t u = (q4 * 4) / (2 * hd), e = (q4 * 4) % (2 * hd);
    f32x4_t wn;
    entry4(u, e, wn);
    if (last) return;
    const int isW3 = e >= hd;
    const int64_t oo = isW3 ? e - hd : e;
    const int64_t sr = oo / d, c = oo % d;
    const int64_t srow = 64 * (sr / 32) + 32 * isW3 + sr % 32;
    put4_shadow<T>(w13s + (u * 2 * h + srow) * (kr * d) + c, kr, d, wn);
    return;
  }
  // W2: tile (J0 .. J0+63 rows = output units, I0 .. I0+63 cols = hidden units)
  const int64_t tb = blk - nA;
  const int64_t tpu = (d / 64) * (h / 64);
  const int64_t u = tb / tpu, t = tb % tpu;
  const int64_t J0 = 64 * (t / (h / 64)), I0 = 64 * (t % (h / 64));
  const int tid = threadIdx.x, rr = tid >> 4, c0 = 4 * (tid & 15);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int jr = rr + 16 * k;
    f32x4_t wn;
    entry4(u, 2 * hd + (J0 + jr) * h + I0 + c0, wn);
    if (!last) {
      put4_shadow<T>(w2s + (u * d + J0 + jr) * (kr * h) + I0 + c0, kr, h, wn);
#pragma unroll
      for (int e = 0; e < 4; ++e) tT[(c0 + e) * 65 + jr] = wn[e];
    }
  }
  if (last) return;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // W2^T row I0 + ir, columns J0 + c0 ..
    const int ir = rr + 16 * k;
    f32x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = tT[ir * 65 + c0 + e];
    put4_shadow<T>(w2ts + (u * h + I0 + ir) * (kr * d) + J0 + c0, kr, d, w);
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
      make_uint2(pack_bf16x2(x0, x1),
                 pack_bf16x2(x2, x3));
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

// The SiLU factors of the backward, f1 = A3 silu'(A1) and f3 = silu(A1), of
// K row t and hidden unit j, as one 32-bit word (bf16 f1 in the low half, f3
// in the high half), stored in the accumulator layout of 32 x 32 blocks: the
// block of tokens 32*tb .. +31 and units 32*hb .. +31 of unit u is 1024
// consecutive words, word 256*(v/4) + 4*lane + v%4 for the lane and register
// v that hold (t, j) in a 32x32 MFMA output.  The forward writes and the
// backward reads each block with the same lanes, in 1 KB vectors.
__device__ __forceinline__ int64_t fac_block(const Shape& s, int64_t u, int64_t tb, int64_t hb) {
  return ((u * (s.Cp / 32) + tb) * (s.h / 32) + hb) * 1024;
}

// fwd13: [K; Q] rows x [W1; W3]^T -> Z = silu(A1) A3 row-major, and for K
// rows Z^T and the SiLU factors of the backward, on the 8-wave engine
// (gemm_tile256w8, two waves per SIMD).  w13s rows are interleaved in blocks
// of 32, so wave w, which holds tile rows 128*(w/4) + [0,128) and columns
// 64*(w%4) + [0,64), has A1 (block ni = 0) and A3 (ni = 1) of the 32 hidden
// units 32*(w%4) + [0,32) of the tile's 128.  The epilogue runs band by band
// (a band: tile rows 32*mi + [0,32) of both wave rows), each wave taking its
// A1/A3 pair and 512 threads sharing the copies out; with two waves per SIMD
// one wave's epilogue arithmetic and LDS traffic run while the other waits
// (a 4-wave version, 128x128 per wave with 256 accumulators, took 103.5
// against 98.0 us per launch at d = 768, h = 1536, C = 8192, same box).
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_fwd13_256(
    Shape s, int r, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
    const bf16_t* __restrict__ w13s, bf16_t* zrow, bf16_t* zt, uint32_t* fac) {
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  const int64_t ntn = 2 * s.h / 256, ntm = 2 * s.Cp / 256;
  int64_t bid = xcd_logical_block();
  const int64_t nt = bid % ntn; bid /= ntn;
  // K and Q row blocks alternate in the numbering, so that every XCD gets
  // as many of the K blocks (whose epilogue writes more) as of the Q blocks.
  const int64_t tq = bid % ntm;
  const int64_t u = bid / ntm;
  const bool isQ = tq & 1;
  const int64_t p0 = (tq >> 1) * 256;
  const int64_t tok0 = static_cast<int64_t>(r) * s.C;
  const int64_t nv = n_valid(s, r);
  const bf16_t* X = (isQ ? q : k) + (u * s.L + tok0) * s.d;
  const bf16_t* W = w13s + (u * 2 * s.h + nt * 256) * s.d;
  f32x16_t acc[4][2];
  gemm_tile256w8(
      acc, [&](int R) { return p0 + R < nv ? X + (p0 + R) * s.d : kZeroRow256; },
      [&](int R) { return W + R * s.d; }, 0, static_cast<int>(s.d / 32), smem_raw);

  Acc256Pos ps;
  ps.wm = ps.wave >> 2;
  ps.wn = ps.wave & 3;
  bf16_t* lds = reinterpret_cast<bf16_t*>(smem_raw);
  constexpr int ZRW = 136;
  bf16_t* zr = lds + 128 * 72;
  const int h = static_cast<int>(s.h);
  bf16_t* zq = zrow + (u * 2 * s.Cp + (isQ ? s.Cp : 0) + p0) * s.h + nt * 128;
  const int j = ps.wn * 32 + ps.r32;  // this lane's hidden unit - nt*128
  auto band = [&](auto MI, auto KROWS) {
    constexpr int mi = decltype(MI)::value;
    constexpr bool krows = decltype(KROWS)::value;
    barrier_lds();  // the previous band's staged rows have been copied out
    {
      pin_acc(acc[mi][0]);
      pin_acc(acc[mi][1]);
      float zv[16];
      uint32_t fw[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float a1 = acc[mi][0][v], a3 = s.gated ? acc[mi][1][v] : 1.0f;
        const float sg = sigmoidf_(a1), sl = a1 * sg;
        const float z = sl * a3;
        zv[v] = z;
        zr[(32 * ps.wm + 8 * (v >> 2) + 4 * ps.hf + (v & 3)) * ZRW + j] = f2bf(z);
        if constexpr (krows)
          fw[v] = pack_bf16x2(a3 * (sg * (1.0f + a1 * (1.0f - sg))), sl);
      }
      if constexpr (krows) {
#pragma unroll
        for (int vq = 0; vq < 4; ++vq)
          band_put(lds, j, ps, vq, zv[4 * vq], zv[4 * vq + 1], zv[4 * vq + 2], zv[4 * vq + 3]);
        const int64_t tb = (p0 + 128 * ps.wm + 32 * mi) / 32;
        const int64_t hb = nt * 4 + ps.wn;
        uint32_t* fb = fac + fac_block(s, u, tb, hb) + 4 * ps.lane;
#pragma unroll
        for (int vq = 0; vq < 4; ++vq)
          *reinterpret_cast<uint4*>(fb + 256 * vq) =
              make_uint4(fw[4 * vq], fw[4 * vq + 1], fw[4 * vq + 2], fw[4 * vq + 3]);
      }
    }
    barrier_lds();
    // Band row br is tile row 128*(br/32) + 32*mi + br%32: 64 rows x 16
    // pieces of 16 bytes, two per thread.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = threadIdx.x + 512 * i, br = idx >> 4, c = idx & 15;
      const int tr = 128 * (br >> 5) + 32 * mi + (br & 31);
      *reinterpret_cast<uint4*>(zq + tr * h + 8 * c) =
          *reinterpret_cast<const uint4*>(zr + br * ZRW + 8 * c);
    }
    if constexpr (krows) {  // Z^T band: 128 hidden rows x 64 tokens, two pieces per thread
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int idx = threadIdx.x + 512 * i;
        const int c = idx >> 3, qq = idx & 7, half = qq >> 2, tok = 8 * (qq & 3);
        *reinterpret_cast<uint4*>(zt + (u * s.h + nt * 128 + c) * s.Cp + p0 + 32 * mi + 128 * half + tok) =
            *reinterpret_cast<const uint4*>(lds + c * 72 + 32 * half + tok);
      }
    }
  };
  if (isQ) for_bands([&](auto MI) { band(MI, Flag<false>{}); });
  else for_bands([&](auto MI) { band(MI, Flag<true>{}); });
}

// ---------------------------------------------------------------------------
// Row engine: a 256 x 32*NB output tile, each of the 4 waves taking 64 rows
// (accumulator blocks mi = 0, 1) and all 32*NB columns (jb = 0 .. NB-1):
// 2*NB blocks, 32*NB accumulator registers.  A stage holds one 32-deep slab
// of 256 + 32*NB rows of 64 bytes (the A rows, then the B rows), stored with
// the swizzle of the 256 engine; loads go straight to LDS, NST stages deep,
// spread one every few MFMAs over the slab.  Used where a 256 x 256 tile
// would leave CUs idle: 256 x 192 tiles put one workgroup on every CU at
// d = 768 (the readout GEMM) and h = 1536 (the backward's dZ).
template <int NB>
struct Rows256 {
  static_assert(NB % 2 == 0 && NB >= 2 && NB <= 6, "columns per tile");
  static constexpr int BM = 256, BN = 32 * NB, BK = 32, NST = 4;
  static constexpr int ROWS = BM + BN;
  static constexpr int STAGE = ROWS * 64;
  static constexpr int LOADS = ROWS / 64;  // direct loads per wave per slab
  static constexpr int STAGES_BYTES = NST * STAGE;
};

// acc[mi][jb] = sum over k < 32*ns of A(64*wave + 32*mi + i, k) B(32*jb + j, k)
// with A row R at arow(R) and B row R at brow(R) (k contiguous).  before_last()
// runs after the last slab's wait and barrier, before its MFMAs (an
// epilogue's first loads overlap them).  ns >= NST - 1.
template <int NB, typename ARow, typename BRow, typename Hook>
__device__ __forceinline__ void gemm_rows256(f32x16_t (&acc)[2][NB], ARow arow, BRow brow, int ns,
                                             char* smem, Hook&& before_last) {
  using G = Rows256<NB>;
  constexpr int NST = G::NST, SB = G::STAGE, NL = G::LOADS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Source of this lane's piece for load i: stage row R = 16*(4i + wave) +
  // lane/4, physical piece lane%4 = logical k-chunk (lane%4) ^ swz256(R).
  const bf16_t* src[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int R = 16 * (4 * i + wave) + (lane >> 2);
    const int c8 = 8 * ((lane & 3) ^ swz256(R));
    src[i] = (R < G::BM ? arow(R) : brow(R - G::BM)) + c8;
  }
  auto load = [&](int slab, int i) {
    char* st = smem + (slab % NST) * SB;
    __builtin_amdgcn_global_load_lds(
        static_cast<const void*>(src[i] + static_cast<int64_t>(slab) * G::BK),
        (__attribute__((address_space(3))) void*)(st + (4 * i + wave) * 1024), 16, 0, 0);
  };
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  const int r32 = lane & 31, hf = lane >> 5, sw = swz256(r32);
  const int off0 = r32 * 64 + ((hf ^ sw) << 4), off1 = r32 * 64 + (((2 + hf) ^ sw) << 4);
  // Fragment set of one 16-deep step: the A blocks of this wave's rows, then
  // the B blocks of the tile's columns.
  struct Frags { bf16x8_t a[2], b[NB]; };
  auto rd = [&](const char* st, int off, int rowbase) {
    return *reinterpret_cast<const bf16x8_t*>(st + rowbase * 64 + off);
  };
  auto read_frags = [&](Frags& f, const char* st, int ks) {
    const int off = ks ? off1 : off0;
    f.a[0] = rd(st, off, 64 * wave);
    f.b[0] = rd(st, off, G::BM);
    f.a[1] = rd(st, off, 64 * wave + 32);
#pragma unroll
    for (int jb = 1; jb < NB; ++jb) f.b[jb] = rd(st, off, G::BM + 32 * jb);
  };
  // The 2*NB MFMAs of one step; the slab's refill loads go one every LSTEP
  // MFMAs from the third of the slab's 4*NB on.
  constexpr int LSTEP = (4 * NB - 2) / NL;
  static_assert(LSTEP >= 1 && 2 + LSTEP * (NL - 1) < 4 * NB, "load slots");
  auto step = [&](const Frags& f, auto&& between) {
#pragma unroll
    for (int m = 0; m < 2 * NB; ++m) {
      const int mi = m & 1, jb = m >> 1;
      acc[mi][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mi], f.b[jb], acc[mi][jb], 0, 0, 0);
      between(m);
    }
  };
  auto body = [&](int sl, bool refill) {
    const char* st = smem + (sl % NST) * SB;
    Frags f0, f1;
    read_frags(f0, st, 0);
    __builtin_amdgcn_sched_barrier(0);
    auto slot = [&](int g) {  // global MFMA index g of the slab
      if (refill && g >= 2 && (g - 2) % LSTEP == 0 && (g - 2) / LSTEP < NL)
        load(sl + NST - 1, (g - 2) / LSTEP);
      __builtin_amdgcn_sched_barrier(0);
    };
    step(f0, [&](int m) {
      if (m == 1) read_frags(f1, st, 1);
      slot(m);
    });
    step(f1, [&](int m) { slot(2 * NB + m); });
  };
#pragma unroll
  for (int p = 0; p < NST - 1; ++p)
#pragma unroll
    for (int i = 0; i < NL; ++i) load(p, i);
  int sl = 0;
  for (; sl < ns - (NST - 1); ++sl) {
    wait_vmcnt<NL * (NST - 2)>();
    barrier_nofence();
    body(sl, true);
  }
  for (; sl < ns - 1; ++sl) {
    if (sl == ns - 3) wait_vmcnt<2 * NL>();
    else wait_vmcnt<NL>();
    barrier_nofence();
    body(sl, false);
  }
  wait_vmcnt<0>();
  barrier_nofence();
  before_last();
  body(sl, false);
}

// ---------------------------------------------------------------------------
// Backward of the 256 path: dZ = g W2 on the tile's tokens and hidden units,
// then dA1 = dZ f1 and dA3 = dZ f3 with the SiLU factors that k_fwd13_256
// stored for the same K rows (bf16), written once each, unscaled and
// feature-major: the aggregation's first family contracts them against the
// scaled keys K^W K, K^M K (k_prep_kts), since (K^W dA1)^T K = dA1^T (K^W K).
// Writing the four scaled products here instead moved twice the bytes.
// Storing the factors costs 4 bytes per token and hidden unit written and
// read; recomputing A1 and A3 here instead cost twice the products of dZ
// (4dh flop per token) on top.
//
// Tile: 256 tokens x 32*NB hidden units of one unit on the row engine (A = g
// rows, B = W2^T rows of the units).
template <int NB>
struct Bwd256 {
  using G = Rows256<NB>;
  static constexpr int BM = G::BM;
  static constexpr int SW = BM + 8;              // staged output row, bf16
  static constexpr int STG = 2 * 64 * SW * 2;    // one epilogue pass: 2 outputs x 64 units
  static constexpr size_t LDS_BYTES = G::STAGES_BYTES > STG ? G::STAGES_BYTES : STG;
};

template <int NB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_bwd256(
    Shape s, int r, const bf16_t* __restrict__ grow, const bf16_t* __restrict__ w2ts,
    const uint32_t* __restrict__ fac, bf16_t* ut) {
  using B = Bwd256<NB>;
  constexpr int BN = 32 * NB;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  const int64_t ntn = s.h / BN, ntm = s.Cp / B::BM;
  // XCD-aware numbering, then groups of 4 token blocks x all hidden tiles
  // with the token block fastest, so that the workgroups an XCD runs at a
  // time share a few token and weight panels in its L2.
  int64_t bid = xcd_logical_block();
  const int64_t GT = ntm % 4 == 0 ? 4 : 1;
  const int64_t u = bid / (ntm * ntn);
  bid %= ntm * ntn;
  const int64_t wi = bid % (GT * ntn);
  const int64_t nt = wi / GT;
  const int64_t mt = bid / (GT * ntn) * GT + wi % GT;
  const int64_t p0 = mt * B::BM, j0 = nt * BN;
  const int64_t d = s.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hf = lane >> 5;
  (void)r;

  using Fac = uint4[2][2][4];
  auto fac_load = [&](Fac& f, int p) __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        const int64_t tb = (p0 + 64 * wave + 32 * mi) / 32, hb = (j0 + 64 * p + 32 * j2) / 32;
        const uint32_t* fb = fac + fac_block(s, u, tb, hb) + 4 * lane;
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) f[mi][j2][vq] = *reinterpret_cast<const uint4*>(fb + 256 * vq);
      }
  };
  Fac fa, fb;
  f32x16_t dz[2][NB];
  // d is a multiple of 256 on this path, so ns >= 8 > NST - 1.  The first
  // epilogue pass's factors are loaded during the last slab.
  gemm_rows256<NB>(
      dz, [&](int R) { return grow + (u * s.Cp + p0 + R) * d; },
      [&](int R) { return w2ts + (u * s.h + j0 + R) * d; }, static_cast<int>(d / 32), smem_raw,
      [&]() __attribute__((always_inline)) { fac_load(fa, 0); });

  // Epilogue, in NB/2 passes of 64 units (blocks jb = 2p, 2p+1).  Lane values
  // of block (mi, jb), register v: token p0 + 64*wave + 32*mi + 8*(v/4) +
  // 4*hf + v%4, unit j0 + 32*jb + r32; the factors of the same token and unit
  // are word v of the lane's quarter of the factor block.  A pass stages its
  // two outputs (o = dA1, dA3) in LDS as [o][unit][256 tokens + 8] bf16 (the
  // stages are free: every wave has passed the last slab's barrier and read
  // its fragments), then copies them out in whole 512-byte rows: ut row
  // (0 | h) + j, tokens p0 .. p0+255.  The next pass's factors are loaded
  // before this pass's stores, so that waiting for them does not wait for
  // the stores.
  constexpr int SW = B::SW;
  bf16_t* stg = reinterpret_cast<bf16_t*>(smem_raw);
  auto pass = [&](auto P, const Fac& f) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) pin_acc(dz[mi][2 * p + j2]);
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const int tk = 64 * wave + 32 * mi + 8 * vq + 4 * hf;
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
          const uint4 fv = f[mi][j2][vq];
          const uint32_t fw[4] = {fv.x, fv.y, fv.z, fv.w};
          float x1[4], x3[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float dzv = dz[mi][2 * p + j2][4 * vq + e];
            x1[e] = dzv * __uint_as_float(fw[e] << 16);
            x3[e] = s.gated ? dzv * __uint_as_float(fw[e] & 0xffff0000u) : 0.0f;
          }
          const int jj = 32 * j2 + r32;
          auto put = [&](int o, const float (&x)[4]) {
            *reinterpret_cast<uint2*>(stg + (o * 64 + jj) * SW + tk) =
                make_uint2(pack_bf16x2(x[0], x[1]),
                           pack_bf16x2(x[2], x[3]));
          };
          put(0, x1);
          put(1, x3);
        }
      }
    }
  };
  bf16_t* ub = ut + u * 2 * s.h * s.Cp + p0;
  auto copy_out = [&](int p) __attribute__((always_inline)) {
    constexpr int VPR = B::BM / 8;  // 16-byte pieces per row
#pragma unroll
    for (int i = 0; i < 2 * 64 * VPR / 256; ++i) {
      const int idx = threadIdx.x + 256 * i;
      const int row = idx / VPR, c = idx % VPR;
      const int o = row / 64, jj = row % 64;
      const int64_t dst = (o ? s.h : 0) + j0 + 64 * p + jj;
      *reinterpret_cast<uint4*>(ub + dst * s.Cp + 8 * c) =
          *reinterpret_cast<const uint4*>(stg + row * SW + 8 * c);
    }
  };
  barrier_lds();  // every wave's last fragment reads are done
  auto run = [&](auto P, const Fac& cur, Fac& nxt) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    pass(P, cur);
    barrier_lds();
    if constexpr (p + 1 < NB / 2) fac_load(nxt, p + 1);
    copy_out(p);
    if constexpr (p + 1 < NB / 2) barrier_lds();  // the stores have read the staging area
  };
  run(Band<0>{}, fa, fb);
  if constexpr (NB >= 4) run(Band<1>{}, fb, fa);
  if constexpr (NB >= 6) run(Band<2>{}, fa, fb);
}

// Family A's token operand on the 256 path: the chunk's keys scaled by both
// kernels, feature-major, [BH][nC][2d][Cp]: rows 0 .. d-1 hold K^W k, rows
// d .. 2d-1 hold K^M k (padded tokens have k = 0 and K = 0), each value
// rounded once to bf16 from the fp32 product.  One block per 64 tokens x 64
// features of one (unit, chunk): the tile goes through LDS transposed, then
// both scaled copies leave in 16-byte pieces of whole rows.
__global__ __launch_bounds__(256) void k_prep_kts(Shape s, const bf16_t* __restrict__ k,
                                                  const float* __restrict__ kw,
                                                  const float* __restrict__ km,
                                                  bf16_t* __restrict__ kts) {
  __shared__ float tile[64][64 + 1];
  __shared__ float ksc[2][64];
  int64_t bid = blockIdx.x;
  const int64_t ptiles = s.Cp / 64, ctiles = s.d / 64;
  const int64_t ct = bid % ctiles; bid /= ctiles;
  const int64_t pt = bid % ptiles; bid /= ptiles;
  const int r = static_cast<int>(bid % s.nC);
  const int64_t u = bid / s.nC;
  const int64_t nv = n_valid(s, r);
  const int tid = threadIdx.x;
  const bf16_t* ks = k + (u * s.L + static_cast<int64_t>(r) * s.C) * s.d + ct * 64;
  uint4 reg[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // 64 token rows x 8 pieces of 8 values
    const int idx = tid + 256 * i;
    const int pr = idx / 8, cv = idx % 8;
    const int64_t p = pt * 64 + pr;
    const uint4 val = *reinterpret_cast<const uint4*>(ks + (p < nv ? p : 0) * s.d + cv * 8);
    reg[i] = p < nv ? val : make_uint4(0u, 0u, 0u, 0u);
  }
  if (tid < 128) {
    const float* kk = tid < 64 ? kw : km;
    ksc[tid / 64][tid % 64] = kk[(u * s.nC + r) * s.Cp + pt * 64 + tid % 64];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid + 256 * i;
    const int pr = idx / 8, cv = idx % 8;
    const uint32_t w[4] = {reg[i].x, reg[i].y, reg[i].z, reg[i].w};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      tile[cv * 8 + 2 * x][pr] = __uint_as_float(w[x] << 16);
      tile[cv * 8 + 2 * x + 1][pr] = __uint_as_float(w[x] & 0xffff0000u);
    }
  }
  __syncthreads();
  bf16_t* dst = kts + ((u * s.nC + r) * 2 * s.d + ct * 64) * s.Cp + pt * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // 2 x 64 feature rows x 8 pieces of 8 tokens
    const int idx = tid + 256 * i;
    const int o = idx / 512, cr = (idx / 8) % 64, pv = idx % 8;
    uint32_t pk[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int t0 = pv * 8 + 2 * x;
      pk[x] = pack_bf16x2(tile[cr][t0] * ksc[o][t0], tile[cr][t0 + 1] * ksc[o][t0 + 1]);
    }
    *reinterpret_cast<uint4*>(dst + (o * s.d + cr) * s.Cp + pv * 8) =
        make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
}

// ---------------------------------------------------------------------------
// fwd2 on the row engine: Z rows x W2^T -> Y for 256 tokens x 32*NB output
// features (NB = 6: 256 workgroups at d = 768, one per CU, where 256 x 256
// tiles gave 192).  The readout for Q rows; g = v - Y for K rows (row-major)
// and K^W g, K^M g feature-major (rows 64*(i/32) + i%32, +32 for the
// momentum copy): the operands of the backward and of the aggregation's
// second family.
//
// Epilogue in NB/2 passes of 64 features (blocks jb = 2p, 2p+1).  A pass
// stages the tile's 256 x 64 values row-major in LDS ([256][64 + 8] bf16:
// the two lane halves, 4 rows apart, hit distinct banks), for K rows first
// filled with v (loaded into registers during the previous pass, or during
// the last slab for pass 0, 16-byte pieces of whole 128-byte row segments),
// which each lane reads and overwrites with g; K^W g and K^M g go through
// two transposed buffers ([64 features][256 + 8] bf16); then everything
// leaves in 16-byte pieces of whole rows.  Rows past the chunk's valid
// tokens read v from a device zero row; the readout writes only valid rows.
template <int NB>
struct Fwd2R {
  using G = Rows256<NB>;
  static constexpr int BM = G::BM;
  static constexpr int VW = 64 + 8;                 // staged row, bf16
  static constexpr int TWW = BM + 8;                // transposed row, bf16
  static constexpr int VR = 0;                      // [256][VW]
  static constexpr int TW = VR + BM * VW * 2;       // [64][TWW]
  static constexpr int TM = TW + 64 * TWW * 2;
  static constexpr int END = TM + 64 * TWW * 2;
  static constexpr int KS = G::STAGES_BYTES > END ? G::STAGES_BYTES : END;  // K^W, K^M
  static constexpr size_t LDS_BYTES = static_cast<size_t>(KS) + 2 * BM * 4;
};

template <int NB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_fwd2r(
    Shape s, int r, const bf16_t* __restrict__ v, bf16_t* out, const bf16_t* __restrict__ zrow,
    const bf16_t* __restrict__ w2s, const float* __restrict__ kw, const float* __restrict__ km,
    bf16_t* grow, bf16_t* gt) {
  using E = Fwd2R<NB>;
  constexpr int BN = 32 * NB, VW = E::VW, TWW = E::TWW;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  const int64_t ntn = s.d / BN, ntm = 2 * s.Cp / 256, mtK = s.Cp / 256;
  int64_t bid = xcd_logical_block();
  const int64_t nt = bid % ntn; bid /= ntn;
  // K and Q row blocks alternate in the numbering, so that every XCD gets
  // as many of the K blocks (whose epilogue writes more) as of the Q blocks.
  const int64_t tq = bid % ntm;
  const int64_t u = bid / ntm;
  const bool isQ = tq & 1;
  const int64_t mt = (tq >> 1) + (isQ ? mtK : 0);  // row block of [K; Q]
  const int64_t p0 = (tq >> 1) * 256, n0 = nt * BN;
  const int64_t tok0 = static_cast<int64_t>(r) * s.C;
  const int64_t nv = n_valid(s, r);
  const int nvt = static_cast<int>(nv - p0 < 256 ? nv - p0 : 256);  // valid rows of the tile
  const int64_t d = s.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hf = lane >> 5;
  float kwt = 0.0f, kmt = 0.0f;
  if (!isQ) {
    kwt = kw[(u * s.nC + r) * s.Cp + p0 + threadIdx.x];
    kmt = km[(u * s.nC + r) * s.Cp + p0 + threadIdx.x];
  }
  // v of pass p: thread piece i (0..7) is row (tid + 256 i) / 8, 16-byte
  // piece (tid + 256 i) % 8 of the pass's 128-byte row segment.
  const bf16_t* vs = v + (u * s.L + tok0 + p0) * d + n0;
  // (One wide vector value: an array of uint4 here was placed in scratch.)
  typedef uint32_t VReg __attribute__((ext_vector_type(32)));
  auto v_load = [&](VReg& x, int p) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = threadIdx.x + 256 * i, row = idx >> 3, c = idx & 7;
      const bf16_t* src = row < nvt ? vs + row * d + 64 * p + 8 * c : kZeroRow256;
      const uint4 y = *reinterpret_cast<const uint4*>(src);
      x[4 * i] = y.x;
      x[4 * i + 1] = y.y;
      x[4 * i + 2] = y.z;
      x[4 * i + 3] = y.w;
    }
  };
  VReg va, vb;
  f32x16_t acc[2][NB];
  gemm_rows256<NB>(
      acc, [&](int R) { return zrow + (u * 2 * s.Cp + mt * 256 + R) * s.h; },
      [&](int R) { return w2s + (u * d + n0 + R) * s.h; }, static_cast<int>(s.h / 32), smem_raw,
      [&]() __attribute__((always_inline)) {
        if (!isQ) v_load(va, 0);
      });

  bf16_t* vr = reinterpret_cast<bf16_t*>(smem_raw + E::VR);
  bf16_t* tW = reinterpret_cast<bf16_t*>(smem_raw + E::TW);
  bf16_t* tM = reinterpret_cast<bf16_t*>(smem_raw + E::TM);
  float* ksh = reinterpret_cast<float*>(smem_raw + E::KS);
  // Staged row of this lane's register v in block mi.
  auto srow = [&](int mi, int vv) { return 64 * wave + 32 * mi + 8 * (vv >> 2) + 4 * hf + (vv & 3); };
  // The staged rows out: row t's 64 features to dst + t*d (rows below
  // `valid`), 16 bytes per thread and step.
  auto rows_out = [&](bf16_t* dst, int valid) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = threadIdx.x + 256 * i, row = idx >> 3, c = idx & 7;
      const uint4 x = *reinterpret_cast<const uint4*>(vr + row * VW + 8 * c);
      if (row < valid) *reinterpret_cast<uint4*>(dst + row * d + 8 * c) = x;
    }
  };
  if (isQ) {
    bf16_t* o = out + (u * s.L + tok0 + p0) * d + n0;
    auto qpass = [&](auto P) __attribute__((always_inline)) {
      constexpr int p = decltype(P)::value;
      barrier_lds();  // the stages, or the previous pass's rows, are free
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int j2 = 0; j2 < 2; ++j2) {
          pin_acc(acc[mi][2 * p + j2]);
#pragma unroll
          for (int vv = 0; vv < 16; ++vv)
            vr[srow(mi, vv) * VW + 32 * j2 + r32] = f2bf(acc[mi][2 * p + j2][vv]);
          __builtin_amdgcn_sched_barrier(0);
        }
      barrier_lds();
      rows_out(o + 64 * p, nvt);
    };
    qpass(Band<0>{});
    if constexpr (NB >= 4) qpass(Band<1>{});
    if constexpr (NB >= 6) qpass(Band<2>{});
    return;
  }
  bf16_t* gr = grow + (u * s.Cp + p0) * d + n0;
  bf16_t* gbase = gt + u * 2 * d * s.Cp + p0;
  auto kpass = [&](auto P, const VReg& cur, VReg& nxt) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    barrier_lds();  // the stages, or the previous pass's buffers, are free
    if constexpr (p == 0) {
      ksh[threadIdx.x] = kwt;
      ksh[256 + threadIdx.x] = kmt;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = threadIdx.x + 256 * i, row = idx >> 3, c = idx & 7;
      *reinterpret_cast<uint4*>(vr + row * VW + 8 * c) =
          make_uint4(cur[4 * i], cur[4 * i + 1], cur[4 * i + 2], cur[4 * i + 3]);
    }
    barrier_lds();
    if constexpr (p + 1 < NB / 2) v_load(nxt, p + 1);  // before this pass's stores
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        pin_acc(acc[mi][2 * p + j2]);
        const int f = 32 * j2 + r32;
        float g[16];
#pragma unroll
        for (int vv = 0; vv < 16; ++vv) {
          bf16_t* e = vr + srow(mi, vv) * VW + f;
          g[vv] = bf2f(*e) - acc[mi][2 * p + j2][vv];
          *e = f2bf(g[vv]);
        }
#pragma unroll
        for (int vq = 0; vq < 4; ++vq) {
          const int t0 = 64 * wave + 32 * mi + 8 * vq + 4 * hf;
          const f32x4_t w4 = *reinterpret_cast<const f32x4_t*>(ksh + t0);
          const f32x4_t m4 = *reinterpret_cast<const f32x4_t*>(ksh + 256 + t0);
          *reinterpret_cast<uint2*>(tW + f * TWW + t0) =
              make_uint2(pack_bf16x2(w4[0] * g[4 * vq], w4[1] * g[4 * vq + 1]),
                         pack_bf16x2(w4[2] * g[4 * vq + 2], w4[3] * g[4 * vq + 3]));
          *reinterpret_cast<uint2*>(tM + f * TWW + t0) =
              make_uint2(pack_bf16x2(m4[0] * g[4 * vq], m4[1] * g[4 * vq + 1]),
                         pack_bf16x2(m4[2] * g[4 * vq + 2], m4[3] * g[4 * vq + 3]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    barrier_lds();
    rows_out(gr + 64 * p, 256);
    // Transposed rows: 2 x 64 rows of 256 tokens, 32 pieces each.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int idx = threadIdx.x + 256 * i, row = idx >> 5, c = idx & 31;
      const int fr = row & 63;
      const int64_t fi = n0 + 64 * p + fr;
      const int64_t dst = 64 * (fi / 32) + (row >= 64 ? 32 : 0) + fi % 32;
      const bf16_t* srcb = (row >= 64 ? tM : tW) + fr * TWW + 8 * c;
      *reinterpret_cast<uint4*>(gbase + dst * s.Cp + 8 * c) = *reinterpret_cast<const uint4*>(srcb);
    }
  };
  kpass(Band<0>{}, va, vb);
  if constexpr (NB >= 4) kpass(Band<1>{}, vb, va);
  if constexpr (NB >= 6) kpass(Band<2>{}, va, vb);
}

}  // namespace e2ttt
