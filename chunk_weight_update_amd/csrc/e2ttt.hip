// e2ttt.hip -- C ABI of the E2-TTT chunk forward (host side + launches).
//
// Call sequence of e2ttt_chunk_forward (all on the caller's stream):
//   scan (all chunks, one launch) -> K^T staging (all chunks) -> operand
//   shadow of W0 -> per chunk r:
//     SwiGLU, d = 128, bf16: phase A, phase B (+ split-sum state epilogue
//       when phase B is token-split);
//     other SwiGLU shapes: fwd13, fwd2, bwd, agg;
//     linear: linear_fwd, linear_agg.
//   The chunk loop is serial because chunk r+1 starts from chunk r's end
//   state (§3.2 of "Rethinking Expressivity and Efficiency in Test-Time
//   Training").
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "e2ttt.h"
#include "kernels.hpp"
#include "gemm256.hpp"
#include "fused.hpp"
#include "decode.hpp"
#include "backward.hpp"
#include "swiglu_backward.hpp"
#include "heads.hpp"

using namespace e2ttt;

namespace {

constexpr int64_t kMaxChunk = 12288;
// Phase B token split: target grid of one workgroup per compute unit of a
// gfx950 (MI355X: 256 CUs), at most 4 splits (measured: more splits cost
// more in the split-sum epilogue than they save).  A plan constant, so that the
// workspace size stays a pure function of the problem.
constexpr int64_t kCUs = 256;
constexpr int kMaxSplitB = 4;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

struct Plan {
  int64_t B, H, BH, L, d, h, C, Cp, nC, P;
  int kind, io, mode;
  int krep;   // operand shadow layout: 1 = bf16 weights, 2 = bf16 hi/lo pairs
  int krepA;  // fused path: phase A products on hi only (1) or on hi/lo (2)
  int averaged = 0;  // chunk-averaged beta, gamma (E2TTT_FLAG_CHUNK_AVERAGED_DECAY)
  int lact = 0;      // the LaCT rule's kernels (E2TTT_FLAG_LACT_RULE)
  int qknorm = 0;    // SiLU + L2 prologue on q, k (E2TTT_FLAG_QK_SILU_L2)
  int rownorm = 0;   // chunk-boundary row normalisation (E2TTT_FLAG_POST_CHUNK_ROW_L2)
  bool fused;   // two-kernel chunk step (SwiGLU, d = 128, bf16 io)
  int rbA;      // phase A rows per workgroup (32 or 64; LDS-streamed variant)
  int wpuA;     // register-resident phase A: workgroups per unit (0: not used)
  int nsplitAgg;  // generic bf16 path: token split of the 256x256-tile aggregation (0: 128x128 tiles)
  bool tile256 = false;  // generic path: forward GEMMs on 256x256 tiles
  int nsplitB;  // phase B token split (1: fused state epilogue)
  size_t opsz;  // bytes per GEMM operand element (2 for bf16, 4 for fp32)
  // Optional output: the states at the starts of chunks 1 .. nC-1, [nC-1][BH][P] each.
  float* saveW;
  float* saveM;
  // workspace offsets (bytes)
  size_t kw, km, coef, kt, w13s, w2s, w2ts, zrow, a1s, a3s, fac, grow, ut, gt, zt, gw, gm, gbf, gft,
      part, part256, qn, kn, wx, mx, total;
};

e2ttt_status check_problem(const e2ttt_problem* p) {
  if (!p || p->struct_size != sizeof(e2ttt_problem)) return E2TTT_EINVAL;
  if (p->kind != E2TTT_LINEAR && p->kind != E2TTT_SWIGLU && p->kind != E2TTT_MLP)
    return E2TTT_EINVAL;
  if (p->io_dtype != E2TTT_F32 && p->io_dtype != E2TTT_BF16) return E2TTT_EINVAL;
  if (p->decay_mode != E2TTT_GAMMA_1_MINUS_ETA_ALPHA && p->decay_mode != E2TTT_ALPHA_IS_GAMMA)
    return E2TTT_EINVAL;
  if ((p->flags & ~static_cast<uint32_t>(E2TTT_FLAG_COMPENSATED_WEIGHTS |
                                         E2TTT_FLAG_CHUNK_AVERAGED_DECAY |
                                         E2TTT_FLAG_QK_SILU_L2 |
                                         E2TTT_FLAG_POST_CHUNK_ROW_L2 |
                                         E2TTT_FLAG_PLAIN_BF16_WEIGHTS |
                                         E2TTT_FLAG_LACT_RULE)) != 0u)
    return E2TTT_EINVAL;
  if ((p->flags & E2TTT_FLAG_LACT_RULE) && (p->flags & E2TTT_FLAG_CHUNK_AVERAGED_DECAY))
    return E2TTT_EINVAL;
  if ((p->flags & E2TTT_FLAG_COMPENSATED_WEIGHTS) && (p->flags & E2TTT_FLAG_PLAIN_BF16_WEIGHTS))
    return E2TTT_EINVAL;
  if (p->reserved != 0u) return E2TTT_EINVAL;
  if (p->batch < 1 || p->heads < 1 || p->seq_len < 0 || p->dim < 1 || p->chunk < 1)
    return E2TTT_EINVAL;
  if (p->kind == E2TTT_LINEAR) {
    if (p->hidden != 0) return E2TTT_EINVAL;
    if (p->dim % 16 != 0 || p->dim > 128) return E2TTT_EUNSUPPORTED;
  } else {
    if (p->hidden < 1) return E2TTT_EINVAL;
    if (p->dim % 128 != 0 || p->hidden % 128 != 0 || p->dim > 1024 || p->hidden > 4096)
      return E2TTT_EUNSUPPORTED;
  }
  if (p->chunk > kMaxChunk) return E2TTT_EUNSUPPORTED;
  // Every element count must fit comfortably in int64 (the grids are checked
  // against the dispatch limit in make_plan).
  int64_t bh, bhl, tot;
  if (!mul_ok(p->batch, p->heads, &bh) || !mul_ok(bh, p->seq_len + kMaxChunk, &bhl) ||
      !mul_ok(bhl, 4 * p->dim, &tot))
    return E2TTT_EUNSUPPORTED;
  if (p->kind != E2TTT_LINEAR) {
    int64_t a, b;
    if (!mul_ok(bh, 12 * p->dim, &a) || !mul_ok(a, p->hidden, &b)) return E2TTT_EUNSUPPORTED;
    if (!mul_ok(bhl, 4 * p->hidden, &a)) return E2TTT_EUNSUPPORTED;
  }
  if (tot > (int64_t(1) << 46)) return E2TTT_EUNSUPPORTED;
  return E2TTT_OK;
}

e2ttt_status make_plan(const e2ttt_problem* p, Plan* pl) {
  const e2ttt_status st = check_problem(p);
  if (st != E2TTT_OK) return st;
  Plan& q = *pl;
  std::memset(&q, 0, sizeof(q));
  q.B = p->batch; q.H = p->heads; q.BH = q.B * q.H; q.L = p->seq_len;
  q.d = p->dim; q.h = p->hidden; q.C = p->chunk;
  q.kind = p->kind; q.io = p->io_dtype; q.mode = p->decay_mode;
  q.averaged = (p->flags & E2TTT_FLAG_CHUNK_AVERAGED_DECAY) ? 1 : 0;
  q.lact = (p->flags & E2TTT_FLAG_LACT_RULE) ? 1 : 0;
  q.qknorm = (p->flags & E2TTT_FLAG_QK_SILU_L2) ? 1 : 0;
  q.rownorm = (p->flags & E2TTT_FLAG_POST_CHUNK_ROW_L2) ? 1 : 0;
  q.nC = q.L > 0 ? (q.L + q.C - 1) / q.C : 0;
  q.P = q.kind == E2TTT_LINEAR ? q.d * q.d : (q.kind == E2TTT_MLP ? 2 : 3) * q.d * q.h;
  const size_t f4 = 4;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align256(o + bytes); return at; };
  if (q.kind == E2TTT_LINEAR) {
    q.Cp = (q.C + 63) / 64 * 64;
    q.krep = 1;
    q.opsz = 4;
    q.kw = take(f4 * q.BH * q.nC * q.Cp);
    q.km = take(f4 * q.BH * q.nC * q.Cp);
    q.coef = take(f4 * q.BH * q.nC * 4);
    q.gw = take(f4 * q.BH * q.Cp * q.d);
    q.gm = take(f4 * q.BH * q.Cp * q.d);
  } else if (q.kind == E2TTT_SWIGLU && q.io == E2TTT_BF16 && q.d == FD) {
    q.fused = true;
    q.Cp = (q.C + 127) / 128 * 128;
    q.opsz = 2;
    // Weight operands: hi/lo shadows and phase B (the products that feed the
    // chunk-end state) on the pair, unless plain bf16 is asked for; phase A
    // (readout and residuals) on the pair only with compensated weights.
    q.krep = (p->flags & E2TTT_FLAG_PLAIN_BF16_WEIGHTS) ? 1 : 2;
    q.krepA = (p->flags & E2TTT_FLAG_COMPENSATED_WEIGHTS) ? 2 : 1;
    q.rbA = (q.krepA == 2 || q.BH * (2 * q.Cp / 64) >= 512) ? 64 : 32;
    // Register-resident phase A (plain bf16 operands, h = 128 or 256): about
    // one workgroup per CU, each taking a contiguous run of one unit's 32-row
    // tiles (the count divides the unit's tiles so none is left empty).  Used
    // when a workgroup gets at least two tiles; with one tile each the load of
    // every wave's weights is not amortised and the LDS-streamed variant, which
    // overlaps the second hidden block's weights with the first block's
    // compute, is faster (measured).
    q.wpuA = 0;
    if (q.krepA == 1 && (q.h == 128 || q.h == 256)) {
      const int64_t ntA = 2 * q.Cp / 32;
      int64_t w = (kCUs + q.BH - 1) / q.BH;
      if (w > ntA) w = ntA;
      while (ntA % w != 0) --w;
      if (ntA / w >= 2) q.wpuA = static_cast<int>(w);
    }
    const size_t T = q.opsz;
    q.kw = take(f4 * q.BH * q.nC * q.Cp);
    q.km = take(f4 * q.BH * q.nC * q.Cp);
    q.coef = take(f4 * q.BH * q.nC * 4);
    q.w13s = take(T * q.BH * 2 * q.h * q.krep * q.d);
    q.w2s = take(T * q.BH * q.d * q.krep * q.h);
    q.w2ts = take(T * q.BH * q.h * q.krep * q.d);
    q.kt = take(T * q.BH * q.nC * q.d * q.Cp);
    q.gbf = take(T * q.BH * q.Cp * q.d);
    q.gft = take(T * q.BH * q.d * q.Cp);
    // Phase B has BH * h/64 workgroups of one CU each; when that leaves most
    // of the chip idle, split the chunk's token tiles over up to kMaxSplitB
    // workgroups per hidden block (a divisor of the tile count) and add the
    // splits in a separate state epilogue.
    const int64_t wgB = q.BH * (q.h / 64), ntile = q.Cp / 32;
    q.nsplitB = 1;
    while (q.nsplitB < kMaxSplitB && wgB * q.nsplitB * 2 <= kCUs && ntile % (q.nsplitB * 2) == 0)
      q.nsplitB *= 2;
    if (q.nsplitB > 1) q.part = take(f4 * static_cast<size_t>(q.nsplitB) * q.BH * 2 * q.P);
  } else {
    q.Cp = (q.C + 127) / 128 * 128;
    q.opsz = q.io == E2TTT_BF16 ? 2 : 4;
    q.krep = (q.io == E2TTT_BF16 && (p->flags & E2TTT_FLAG_COMPENSATED_WEIGHTS)) ? 2 : 1;
    q.krepA = q.krep;
    const size_t T = q.opsz;
    q.kw = take(f4 * q.BH * q.nC * q.Cp);
    q.km = take(f4 * q.BH * q.nC * q.Cp);
    q.coef = take(f4 * q.BH * q.nC * 4);
    // Plain bf16 operands with d, h and the padded chunk multiples of 256:
    // the forward GEMMs (fwd13, fwd2) run on 256x256 tiles, the backward
    // takes the SiLU factors as bf16 pairs instead of an fp32 copy of A1, A3
    // and writes dA1, dA3 unscaled; the aggregation contracts them against
    // the keys scaled by K^W and K^M (two feature-major copies per chunk).
    q.tile256 = q.io == E2TTT_BF16 && q.krep == 1 && q.d % 256 == 0 && q.h % 256 == 0 &&
                q.Cp % 256 == 0;
    q.kt = take(T * q.BH * q.nC * (q.tile256 ? 2 : 1) * q.d * q.Cp);
    q.w13s = take(T * q.BH * 2 * q.h * q.krep * q.d);
    q.w2s = take(T * q.BH * q.d * q.krep * q.h);
    q.w2ts = take(T * q.BH * q.h * q.krep * q.d);
    q.zrow = take(T * q.BH * 2 * q.Cp * q.h);
    q.a1s = q.a3s = q.fac = 0;
    if (q.tile256) {
      q.fac = take(f4 * q.BH * q.Cp * q.h);
    } else {
      q.a1s = take(f4 * q.BH * q.Cp * q.h);
      q.a3s = take(f4 * q.BH * q.Cp * q.h);
    }
    q.grow = take(T * q.BH * q.Cp * q.d);
    q.ut = take(T * q.BH * (q.tile256 ? 2 : 4) * q.h * q.Cp);
    q.gt = take(T * q.BH * 2 * q.d * q.Cp);
    q.zt = take(T * q.BH * q.h * q.Cp);
    // bf16 operands with d, h multiples of 256: the aggregation runs on
    // 256x256 tiles; the chunk's token slabs are split so that the grid comes
    // close to one workgroup per CU, and k_agg_reduce adds the splits.
    q.nsplitAgg = 0;
    if (q.io == E2TTT_BF16 && q.d % 256 == 0 && q.h % 256 == 0) {
      const int64_t tiles = q.BH * ((4 * q.h / 256) * (q.d / 256) + (2 * q.d / 256) * (q.h / 256));
      int S = 1;
      // (S divides the slab count, so every split has at least one slab)
      while (S < 8 && tiles * S * 2 <= kCUs && (q.Cp / 32) % (S * 2) == 0) S *= 2;
      q.nsplitAgg = S;
      q.part256 = take(f4 * static_cast<size_t>(S) * 2 * q.BH * 3 * q.d * q.h);
    }
    if (q.kind == E2TTT_MLP) {  // the state in the SwiGLU layout, W3 = 0
      q.wx = take(f4 * q.BH * 3 * q.d * q.h);
      q.mx = take(f4 * q.BH * 3 * q.d * q.h);
    }
  }
  if (q.qknorm) {  // normalised copies of q and k
    const size_t nx = static_cast<size_t>(q.BH * q.L * q.d) * (q.io == E2TTT_BF16 ? 2 : 4);
    q.qn = take(nx);
    q.kn = take(nx);
  }
  q.total = q.L == 0 ? 0 : o;  // an empty sequence only copies the state
  // Every 1-D launch of the plan must fit one dispatch: blocks * 256
  // work-items below 2^32.  The largest grids of each path:
  int64_t worst = q.BH * q.nC;                          // scan
  auto upd = [&](int64_t blocks) { worst = blocks > worst ? blocks : worst; };
  upd(q.BH * q.P / 256 + 1);                            // state copies
  if (q.qknorm) upd(q.BH * q.L / 4 + 1);                // q/k prologue, 4 rows per block
  if (q.kind == E2TTT_LINEAR) {
    upd(q.BH * (2 * q.Cp / 16));                        // linear forward
    upd(q.BH * q.d / 4 + 1);                            // row normalisation
  } else {
    upd(q.BH * q.nC * (q.Cp / 64) * (q.d / 64));        // K^T staging
    upd(q.BH * 3 * (q.d / 64) * (q.h / 64));            // operand shadows
    upd(q.BH * (2 * q.Cp / 32));                        // phase A (32-row tiles)
    upd(q.BH * (q.h / 64) * 24);                        // split-sum state epilogue
    upd(q.BH * (2 * q.Cp / 128) * (2 * q.h / 128));     // fwd13 (128-row tiles)
    upd(q.BH * 3 * q.d * q.h / 1024 + 1);               // agg reduce, MLP state copies
    upd(q.BH * (2 * q.h + q.d) / 4 + 1);                // row normalisation
  }
  if (worst > static_cast<int64_t>(UINT32_MAX / 256u)) return E2TTT_EUNSUPPORTED;
  return E2TTT_OK;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

Range rng(const void* p, size_t bytes) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(p);
  return Range{b, b + bytes};
}

// gfx950 check, cached per device (a property of the device, not of a call).
std::atomic<int> g_arch_ok[64];

e2ttt_status device_ok() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return E2TTT_EHIP;
  if (dev < 0 || dev >= 64) return E2TTT_EUNSUPPORTED;
  int v = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return E2TTT_EHIP;
    v = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? E2TTT_OK : E2TTT_EUNSUPPORTED;
}

std::atomic<int> g_attr_done{0};

void set_lds_attributes() {
  if (g_attr_done.load(std::memory_order_acquire)) return;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_lin_fwd<float>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_lin_fwd<bf16_t>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  const void* fused_kernels[] = {
      reinterpret_cast<const void*>(&k_phaseA<32, 1>), reinterpret_cast<const void*>(&k_phaseA<64, 1>),
      reinterpret_cast<const void*>(&k_phaseA<64, 2>), reinterpret_cast<const void*>(&k_phaseB<1>),
      reinterpret_cast<const void*>(&k_phaseB<2>), reinterpret_cast<const void*>(&k_phaseA2<32>),
      reinterpret_cast<const void*>(&k_phaseA2<64>), reinterpret_cast<const void*>(&k_agg256),
      reinterpret_cast<const void*>(&k_fwd13_256),
      reinterpret_cast<const void*>(&k_bwd256<4>), reinterpret_cast<const void*>(&k_bwd256<6>),
      reinterpret_cast<const void*>(&k_fwd2r<4>), reinterpret_cast<const void*>(&k_fwd2r<6>),
      reinterpret_cast<const void*>(&k_lin_bwd_tok<1>), reinterpret_cast<const void*>(&k_lin_bwd_tok<2>),
      reinterpret_cast<const void*>(&k_lin_bwd_tok<3>), reinterpret_cast<const void*>(&k_lin_bwd_tok<4>)};
  for (const void* f : fused_kernels)
    (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  const void* heads_kernels[] = {
      reinterpret_cast<const void*>(&k_heads<float, 3>), reinterpret_cast<const void*>(&k_heads<float, 6>),
      reinterpret_cast<const void*>(&k_heads<float, 12>), reinterpret_cast<const void*>(&k_heads<bf16_t, 3>),
      reinterpret_cast<const void*>(&k_heads<bf16_t, 6>), reinterpret_cast<const void*>(&k_heads<bf16_t, 12>)};
  for (const void* f : heads_kernels)
    (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  g_attr_done.store(1, std::memory_order_release);
}

unsigned grid1(int64_t n) { return static_cast<unsigned>(n); }

// Chunk-boundary normalisation of the chunk-end weights, then (SwiGLU, when a
// chunk follows) the next chunk's operand shadows rebuilt from them.
template <typename T>
void launch_rownorm(const Plan& q, const Shape& s, float* Wend, bool more, T* w13s, T* w2s,
                    T* w2ts, hipStream_t st) {
  const int64_t rows = q.BH * (q.h == 0 ? q.d : 2 * q.h + q.d);
  hipLaunchKernelGGL(k_row_l2norm, dim3(grid1((rows + 3) / 4)), dim3(256), 0, st, Wend, q.BH,
                     q.d, q.h);
  if (q.h != 0 && more)
    hipLaunchKernelGGL(k_prep_shadow<T>, dim3(grid1(shadow_blocks(s))), dim3(256), 0, st, s,
                       static_cast<const float*>(Wend), w13s, w2s, w2ts);
}

// Optional event bracketing of one kernel class (benchmark instrumentation).
struct Instr {
  int kclass = -1;
  void* const* ev = nullptr;
  int n_pairs = 0;
  int used = 0;
  // Events of the next launch of class c (null when c is not the timed class
  // or the caller's events are used up).
  void events(int c, hipEvent_t* start, hipEvent_t* stop) {
    *start = nullptr;
    *stop = nullptr;
    if (c == kclass && used < n_pairs) {
      *start = static_cast<hipEvent_t>(ev[2 * used]);
      *stop = static_cast<hipEvent_t>(ev[2 * used + 1]);
      ++used;
    }
  }
};

// Every launch goes through hipExtLaunchKernelGGL, which records the timed
// class's events at the kernel's own start and end (not around the launch,
// which would add the dispatch latency to the measured duration).
#define E2TTT_LAUNCH(I, cls, kern, grid, block, shmem, stream, ...)                          \
  do {                                                                                     \
    hipEvent_t e2_start_, e2_stop_;                                                        \
    (I).events((cls), &e2_start_, &e2_stop_);                                              \
    hipExtLaunchKernelGGL(kern, grid, block, static_cast<uint32_t>(shmem), stream, e2_start_, \
                          e2_stop_, 0u, __VA_ARGS__);                                      \
  } while (0)

// Tokens per scan thread: every thread busy on short segments, up to 8 on
// long ones (fewer block-wide steps per token).
int scan_tpt(int64_t C) { return C <= 256 ? 1 : C <= 512 ? 2 : C <= 1024 ? 4 : 8; }

// Vector accesses of min(tpt, 4) floats need every segment start (u*L + r*C),
// every output row start and every segment length to be multiples of it
// (the base pointers are 16-byte aligned).
bool scan_vec_ok(const Plan& q, int tpt, int64_t ustride, int64_t rstride) {
  const int64_t vw = tpt < 4 ? tpt : 4;
  return q.L % vw == 0 && q.C % vw == 0 && ustride % vw == 0 && rstride % vw == 0;
}

ScanArgs scan_args(const Plan& q, const float* eta, const float* alpha, const float* beta,
                   float* kw, float* km, int64_t ustride, int64_t rstride, int64_t pad,
                   float* coef, int cstride) {
  ScanArgs sa;
  sa.eta = eta; sa.alpha = alpha; sa.beta = beta;
  sa.L = q.L; sa.C = q.C; sa.nC = q.nC; sa.mode = q.mode; sa.averaged = q.averaged;
  sa.lact = q.lact;
  sa.kw = kw; sa.km = km;
  sa.ustride = ustride; sa.rstride = rstride; sa.pad = pad;
  sa.coef = coef; sa.cstride = cstride;
  sa.istride = q.L;
  return sa;
}

// After chunk r: keep a copy of the state that chunk r+1 starts from (the
// MLP learner's from the kernels' [W1 | W3 | W2] layout back to [W1 | W2]).
void save_state(const Plan& q, int64_t r, const float* Wend, const float* Mend, hipStream_t st) {
  if (!q.saveW || r + 1 >= q.nC) return;
  const int64_t n = q.BH * q.P;
  if (q.kind == E2TTT_MLP) {
    const unsigned gx = grid1((q.BH * 3 * q.d * q.h / 4 + 255) / 256);
    hipLaunchKernelGGL(k_mlp_state, dim3(gx), dim3(256), 0, st, Wend, q.saveW + r * n, q.BH,
                       q.d, q.h, 0);
    hipLaunchKernelGGL(k_mlp_state, dim3(gx), dim3(256), 0, st, Mend, q.saveM + r * n, q.BH,
                       q.d, q.h, 0);
    return;
  }
  hipLaunchKernelGGL(k_copy2, dim3(grid1((n + 255) / 256)), dim3(256), 0, st, Wend, Mend,
                     q.saveW + r * n, q.saveM + r * n, n);
}

void launch_scan(const Plan& q, const float* eta, const float* alpha, const float* beta,
                 float* kw, float* km, int64_t ustride, int64_t rstride, int64_t pad,
                 float* coef, int cstride, hipStream_t st, Instr& I) {
  // Tokens per thread: every thread busy on short segments, up to 8 on long
  // ones (fewer block-wide scan steps per token).
  const ScanArgs sa = scan_args(q, eta, alpha, beta, kw, km, ustride, rstride, pad, coef,
                                cstride);
  const int tpt = scan_tpt(q.C);
  const bool vec = scan_vec_ok(q, tpt, ustride, rstride);
  void (*f)(ScanArgs) = tpt == 1 ? k_scan<256, 1, 1>
                      : tpt == 2 ? (vec ? k_scan<256, 2, 2> : k_scan<256, 2, 1>)
                      : tpt == 4 ? (vec ? k_scan<256, 4, 4> : k_scan<256, 4, 1>)
                                 : (vec ? k_scan<256, 8, 4> : k_scan<256, 8, 1>);
  E2TTT_LAUNCH(I, E2TTT_KERNEL_SCAN, f, dim3(grid1(q.BH * q.nC)), dim3(256), 0, st, sa);
}

// 256x256-tile aggregation with a token split, then the split-sum state
// epilogue (bf16 operands only).
template <typename T>
void launch_agg256(const Plan& q, const Shape& s, int r, int last, const T* ut, const T* kt,
                   const T* gt, const T* zt, const float* coef, const float* Win,
                   const float* Min, float* Wend, float* Mend, T* w13s, T* w2s, T* w2ts,
                   float* part, hipStream_t st, Instr& I) {
  static_assert(sizeof(T) == 2 || sizeof(T) == 4, "operand type");
  if constexpr (sizeof(T) == 2) {
    const int64_t tiles = (4 * q.h / 256) * (q.d / 256) + (2 * q.d / 256) * (q.h / 256);
    E2TTT_LAUNCH(I, E2TTT_KERNEL_AGG, k_agg256, dim3(grid1(q.BH * tiles * q.nsplitAgg)),
                 dim3(512), Tile256w8::LDS_BYTES, st, s, q.nsplitAgg, ut, kt, gt, zt, r, part);
    void (*kred)(Shape, int, int, int, const float*, const float*, const float*, const float*,
                 float*, float*, T*, T*, T*) = k_agg_reduce<T>;
    // (the kernels' state layout [W1 | W3 | W2]: 3dh per unit, also for the MLP)
    E2TTT_LAUNCH(I, E2TTT_KERNEL_STATE, kred, dim3(grid1(agg_reduce_blocks(s))),
                 dim3(256), 0, st, s, q.nsplitAgg, r, last, part, coef, Win, Min, Wend, Mend,
                 w13s, w2s, w2ts);
  }
}

// Forward GEMMs of one chunk on 256x256 tiles (plain bf16), then the backward.
template <typename T>
void launch_fwd_bwd256(const Plan& q, const Shape& s, int r, const T* Q, const T* K, const T* V,
                       T* O, const T* w13s, const T* w2s, const T* w2ts, T* zrow, T* zt,
                       const float* kw, const float* km, T* grow, T* gt, T* ut, uint32_t* fac,
                       hipStream_t st, Instr& I) {
  static_assert(sizeof(T) == 2 || sizeof(T) == 4, "operand type");
  if constexpr (sizeof(T) == 2) {
    E2TTT_LAUNCH(I, E2TTT_KERNEL_FWD13, k_fwd13_256,
                 dim3(grid1(q.BH * (2 * q.Cp / 256) * (2 * q.h / 256))), dim3(512),
                 Tile256w8::LDS_BYTES, st, s, r, Q, K, w13s, zrow, zt, fac);
    // 192 output features per readout tile where d allows (one workgroup per
    // CU at d = 768), else 128.
    if (q.d % 192 == 0) {
      E2TTT_LAUNCH(I, E2TTT_KERNEL_FWD2, k_fwd2r<6>,
                   dim3(grid1(q.BH * (2 * q.Cp / 256) * (q.d / 192))), dim3(256),
                   Fwd2R<6>::LDS_BYTES, st, s, r, V, O, zrow, w2s, kw, km, grow, gt);
    } else {
      E2TTT_LAUNCH(I, E2TTT_KERNEL_FWD2, k_fwd2r<4>,
                   dim3(grid1(q.BH * (2 * q.Cp / 256) * (q.d / 128))), dim3(256),
                   Fwd2R<4>::LDS_BYTES, st, s, r, V, O, zrow, w2s, kw, km, grow, gt);
    }
    // 192 hidden units per backward tile where h allows (one workgroup per
    // CU at d = 768, h = 1536), else 128.
    if (q.h % 192 == 0) {
      E2TTT_LAUNCH(I, E2TTT_KERNEL_BWD, k_bwd256<6>,
                   dim3(grid1(q.BH * (q.Cp / 256) * (q.h / 192))), dim3(256),
                   Bwd256<6>::LDS_BYTES, st, s, r, grow, w2ts, fac, ut);
    } else {
      E2TTT_LAUNCH(I, E2TTT_KERNEL_BWD, k_bwd256<4>,
                   dim3(grid1(q.BH * (q.Cp / 256) * (q.h / 128))), dim3(256),
                   Bwd256<4>::LDS_BYTES, st, s, r, grow, w2ts, fac, ut);
    }
  }
}

template <typename T>
void launch_swiglu(const Plan& q, const void* qv, const void* kv, const void* vv,
                   const float* eta, const float* alpha, const float* beta, const float* W0,
                   const float* M0, void* outv, float* Wend, float* Mend, char* ws,
                   hipStream_t st, Instr& I) {
  const T* Q = static_cast<const T*>(qv);
  const T* K = static_cast<const T*>(kv);
  const T* V = static_cast<const T*>(vv);
  T* O = static_cast<T*>(outv);
  Shape s{q.BH, q.L, q.d, q.h, q.C, q.Cp, q.nC, q.krep};
  s.gated = q.kind == E2TTT_MLP ? 0 : 1;
  s.sk = q.tile256 ? 1 : 0;
  float* kw = reinterpret_cast<float*>(ws + q.kw);
  float* km = reinterpret_cast<float*>(ws + q.km);
  float* coef = reinterpret_cast<float*>(ws + q.coef);
  T* kt = reinterpret_cast<T*>(ws + q.kt);
  T* w13s = reinterpret_cast<T*>(ws + q.w13s);
  T* w2s = reinterpret_cast<T*>(ws + q.w2s);
  T* w2ts = reinterpret_cast<T*>(ws + q.w2ts);
  T* zrow = reinterpret_cast<T*>(ws + q.zrow);
  float* a1s = reinterpret_cast<float*>(ws + q.a1s);
  float* a3s = reinterpret_cast<float*>(ws + q.a3s);
  T* grow = reinterpret_cast<T*>(ws + q.grow);
  T* ut = reinterpret_cast<T*>(ws + q.ut);
  T* gt = reinterpret_cast<T*>(ws + q.gt);
  T* zt = reinterpret_cast<T*>(ws + q.zt);

  launch_scan(q, eta, alpha, beta, kw, km, q.nC * q.Cp, q.Cp, q.Cp, coef, 4, st, I);
  if (q.tile256) {
    if constexpr (sizeof(T) == 2)
      E2TTT_LAUNCH(I, E2TTT_KERNEL_PREP, k_prep_kts,
                   dim3(grid1(q.BH * q.nC * (q.Cp / 64) * (q.d / 64))), dim3(256), 0, st, s, K,
                   kw, km, kt);
  } else {
    void (*kprep)(Shape, const T*, T*) = k_prep_kt<T, false>;
    E2TTT_LAUNCH(I, E2TTT_KERNEL_PREP, kprep,
                 dim3(grid1(q.BH * q.nC * (q.Cp / 64) * (q.d / 64))), dim3(256), 0, st, s, K, kt);
  }
  E2TTT_LAUNCH(I, E2TTT_KERNEL_PREP, k_prep_shadow<T>, dim3(grid1(shadow_blocks(s))),
               dim3(256), 0, st, s, W0, w13s, w2s, w2ts);
  const int64_t na = (4 * q.h / 128) * (q.d / 128), nb = (2 * q.d / 128) * (q.h / 128);
  for (int64_t r = 0; r < q.nC; ++r) {
    const float* Win = r == 0 ? W0 : Wend;
    const float* Min = r == 0 ? M0 : Mend;
    const int ri = static_cast<int>(r);
    if (q.tile256) {
      launch_fwd_bwd256(q, s, ri, Q, K, V, O, w13s, w2s, w2ts, zrow, zt, kw, km, grow, gt, ut,
                        reinterpret_cast<uint32_t*>(ws + q.fac), st, I);
    } else {
      E2TTT_LAUNCH(I, E2TTT_KERNEL_FWD13, k_fwd13<T>,
                   dim3(grid1(q.BH * (2 * q.Cp / 128) * (2 * q.h / 128))), dim3(256), 0, st, s,
                   ri, Q, K, w13s, zrow, a1s, a3s, zt);
      E2TTT_LAUNCH(I, E2TTT_KERNEL_FWD2, k_fwd2<T>,
                   dim3(grid1(q.BH * (2 * q.Cp / 128) * (q.d / 128))), dim3(256), 0, st, s, ri, V,
                   O, zrow, w2s, kw, km, grow, gt);
      E2TTT_LAUNCH(I, E2TTT_KERNEL_BWD, k_bwd<T>,
                   dim3(grid1(q.BH * (q.Cp / 128) * (q.h / 128))), dim3(256), 0, st, s, ri, grow,
                   w2ts, a1s, a3s, kw, km, ut);
    }
    if (q.nsplitAgg > 0) {  // the plan sets nsplitAgg for bf16 operands only
      launch_agg256(q, s, ri, static_cast<int>(r == q.nC - 1), ut, kt, gt, zt, coef, Win, Min,
                    Wend, Mend, w13s, w2s, w2ts, reinterpret_cast<float*>(ws + q.part256), st, I);
    } else {
      E2TTT_LAUNCH(I, E2TTT_KERNEL_AGG, k_agg<T>, dim3(grid1(q.BH * (na + nb))), dim3(256), 0,
                   st, s, ri, static_cast<int>(r == q.nC - 1), ut, kt, gt, zt, coef, Win, Min,
                   Wend, Mend, w13s, w2s, w2ts);
    }
    if (q.rownorm) launch_rownorm<T>(q, s, Wend, r + 1 < q.nC, w13s, w2s, w2ts, st);
    save_state(q, r, Wend, Mend, st);
  }
}

void launch_fused(const Plan& q, const void* qv, const void* kv, const void* vv,
                  const float* eta, const float* alpha, const float* beta, const float* W0,
                  const float* M0, void* outv, float* Wend, float* Mend, char* ws,
                  hipStream_t st, Instr& I) {
  FusedArgs a;
  a.BH = q.BH; a.L = q.L; a.h = q.h; a.C = q.C; a.Cp = q.Cp; a.nC = q.nC;
  a.q = static_cast<const bf16_t*>(qv);
  a.k = static_cast<const bf16_t*>(kv);
  a.v = static_cast<const bf16_t*>(vv);
  a.out = static_cast<bf16_t*>(outv);
  a.kw = reinterpret_cast<const float*>(ws + q.kw);
  a.km = reinterpret_cast<const float*>(ws + q.km);
  a.coef = reinterpret_cast<const float*>(ws + q.coef);
  a.w13s = reinterpret_cast<bf16_t*>(ws + q.w13s);
  a.w2s = reinterpret_cast<bf16_t*>(ws + q.w2s);
  a.w2ts = reinterpret_cast<bf16_t*>(ws + q.w2ts);
  a.kt = reinterpret_cast<const bf16_t*>(ws + q.kt);
  a.gbf = reinterpret_cast<bf16_t*>(ws + q.gbf);
  a.gft = reinterpret_cast<bf16_t*>(ws + q.gft);
  a.Wout = Wend;
  a.Mout = Mend;
  a.nsplit = q.nsplitB;
  a.krep = q.krep;
  a.part = q.nsplitB > 1 ? reinterpret_cast<float*>(ws + q.part) : nullptr;
  Shape s{q.BH, q.L, q.d, q.h, q.C, q.Cp, q.nC, q.krep};
  // Scalar kernels, K^T staging and the W0 shadow: independent, one launch.
  const ScanArgs sa = scan_args(q, eta, alpha, beta, reinterpret_cast<float*>(ws + q.kw),
                                reinterpret_cast<float*>(ws + q.km), q.nC * q.Cp, q.Cp, q.Cp,
                                reinterpret_cast<float*>(ws + q.coef), 4);
  const int64_t nscan = q.BH * q.nC, nkt = q.BH * q.nC * (q.Cp / 64) * (q.d / 64);
  const int64_t nshadow = shadow_blocks(s);
  const int tpt = scan_tpt(q.C);
  const bool vec = scan_vec_ok(q, tpt, q.nC * q.Cp, q.Cp);
  void (*kpro)(ScanArgs, Shape, const bf16_t*, bf16_t*, const float*, bf16_t*, bf16_t*,
               bf16_t*, int64_t, int64_t) =
      tpt == 1 ? k_prologue<1, 1>
      : tpt == 2 ? (vec ? k_prologue<2, 2> : k_prologue<2, 1>)
      : tpt == 4 ? (vec ? k_prologue<4, 4> : k_prologue<4, 1>)
                 : (vec ? k_prologue<8, 4> : k_prologue<8, 1>);
  E2TTT_LAUNCH(I, E2TTT_KERNEL_PROLOGUE, kpro, dim3(grid1(nscan + nkt + nshadow)), dim3(256),
               0, st, sa, s, a.k, reinterpret_cast<bf16_t*>(ws + q.kt), W0, a.w13s, a.w2s,
               a.w2ts, nscan, nkt);
  const unsigned gA = grid1(q.BH * (2 * q.Cp / q.rbA));
  const unsigned gB = grid1(q.BH * (q.h / 64) * q.nsplitB);
  for (int64_t r = 0; r < q.nC; ++r) {
    a.r = static_cast<int>(r);
    a.last = static_cast<int>(r == q.nC - 1);
    a.Win = r == 0 ? W0 : Wend;
    a.Min = r == 0 ? M0 : Mend;
    void (*kA)(FusedArgs) = q.krepA == 2 ? k_phaseA<64, 2>
                           : (q.rbA == 64 ? k_phaseA<64, 1> : k_phaseA<32, 1>);
    const size_t ldsA = q.krepA == 2 ? PhaseACfg<64, 2>::LDS_BYTES
                        : (q.rbA == 64 ? PhaseACfg<64, 1>::LDS_BYTES : PhaseACfg<32, 1>::LDS_BYTES);
    void (*kB)(FusedArgs) = q.krep == 2 ? k_phaseB<2> : k_phaseB<1>;
    if (q.wpuA > 0) {
      void (*kA2)(FusedArgs, int) = q.h == 256 ? k_phaseA2<64> : k_phaseA2<32>;
      E2TTT_LAUNCH(I, E2TTT_KERNEL_PHASE_A, kA2, dim3(grid1(q.BH * q.wpuA)), dim3(256),
                   PhaseA2Cfg::LDS_BYTES, st, a, q.wpuA);
    } else {
      E2TTT_LAUNCH(I, E2TTT_KERNEL_PHASE_A, kA, dim3(gA), dim3(256), ldsA, st, a);
    }
    const size_t ldsB = q.krep == 2 ? PhaseBCfg<2>::LDS_BYTES : PhaseBCfg<1>::LDS_BYTES;
    E2TTT_LAUNCH(I, E2TTT_KERNEL_PHASE_B, kB, dim3(gB), dim3(256), ldsB, st, a);
    if (q.nsplitB > 1)
      E2TTT_LAUNCH(I, E2TTT_KERNEL_STATE, k_state_epi, dim3(grid1(q.BH * (q.h / 64) * 24)),
                   dim3(256), 0, st, a);
    if (q.rownorm)
      launch_rownorm<bf16_t>(q, s, Wend, r + 1 < q.nC, a.w13s, a.w2s, a.w2ts, st);
    save_state(q, r, Wend, Mend, st);
  }
}

template <typename IO>
void launch_linear(const Plan& q, const void* qv, const void* kv, const void* vv,
                   const float* eta, const float* alpha, const float* beta, const float* W0,
                   const float* M0, void* outv, float* Wend, float* Mend, char* ws,
                   hipStream_t st, Instr& I) {
  const IO* Q = static_cast<const IO*>(qv);
  const IO* K = static_cast<const IO*>(kv);
  const IO* V = static_cast<const IO*>(vv);
  IO* O = static_cast<IO*>(outv);
  Shape s{q.BH, q.L, q.d, 0, q.C, q.Cp, q.nC, 1};
  float* kw = reinterpret_cast<float*>(ws + q.kw);
  float* km = reinterpret_cast<float*>(ws + q.km);
  float* coef = reinterpret_cast<float*>(ws + q.coef);
  float* gw = reinterpret_cast<float*>(ws + q.gw);
  float* gm = reinterpret_cast<float*>(ws + q.gm);
  launch_scan(q, eta, alpha, beta, kw, km, q.nC * q.Cp, q.Cp, q.Cp, coef, 4, st, I);
  const size_t lds_f = static_cast<size_t>(q.d * (q.d + 1) + LIN_FWD_TB * (q.d + 1)) * sizeof(float);
  const size_t lds_a = static_cast<size_t>(2 * 64 * 16 + 64 * q.d) * sizeof(float);
  for (int64_t r = 0; r < q.nC; ++r) {
    const float* Win = r == 0 ? W0 : Wend;
    const float* Min = r == 0 ? M0 : Mend;
    const int ri = static_cast<int>(r);
    E2TTT_LAUNCH(I, E2TTT_KERNEL_LINEAR_FWD, k_lin_fwd<IO>,
                 dim3(grid1(q.BH * (2 * q.Cp / LIN_FWD_TB))),
                 dim3(256), lds_f, st, s, ri, Q, K, V, Win, kw, km, O, gw, gm);
    E2TTT_LAUNCH(I, E2TTT_KERNEL_LINEAR_AGG, k_lin_agg<IO>, dim3(grid1(q.BH * (q.d / 16))),
                 dim3(256), lds_a, st, s, ri, K, gw, gm, coef, Win, Min, Wend, Mend);
    if (q.rownorm)
      launch_rownorm<float>(q, s, Wend, false, nullptr, nullptr, nullptr, st);
    save_state(q, r, Wend, Mend, st);
  }
}

}  // namespace

extern "C" {

const char* e2ttt_status_string(e2ttt_status s) {
  // A C caller may pass any int; read the bits as one (an out-of-range value
  // of the C++ enum type would be undefined).
  int v = 0;
  std::memcpy(&v, &s, sizeof(v));
  switch (v) {
    case E2TTT_OK: return "E2TTT_OK";
    case E2TTT_EINVAL: return "E2TTT_EINVAL: invalid argument";
    case E2TTT_EWORKSPACE: return "E2TTT_EWORKSPACE: workspace too small";
    case E2TTT_EUNSUPPORTED: return "E2TTT_EUNSUPPORTED: shape, dtype or device not supported";
    case E2TTT_EHIP: return "E2TTT_EHIP: HIP runtime error";
  }
  return "E2TTT: unknown status";
}

e2ttt_status e2ttt_validate(const e2ttt_problem* prob) { return check_problem(prob); }

e2ttt_status e2ttt_workspace_bytes(const e2ttt_problem* prob, size_t* bytes) {
  if (!bytes) return E2TTT_EINVAL;
  Plan q;
  const e2ttt_status st = make_plan(prob, &q);
  if (st != E2TTT_OK) return st;
  *bytes = q.total;
  return E2TTT_OK;
}

}  // extern "C"

namespace {

e2ttt_status forward_impl(const e2ttt_problem* prob, const void* q, const void* k, const void* v,
                          const float* eta, const float* alpha, const float* beta,
                          const float* W0, const float* M0, void* out, float* W_end,
                          float* M_end, void* workspace, size_t workspace_bytes, void* stream,
                          Instr& I, float* W_starts = nullptr, float* M_starts = nullptr,
                          bool want_starts = false) {
  Plan pl;
  e2ttt_status status = make_plan(prob, &pl);
  if (status != E2TTT_OK) return status;
  const bool keep = want_starts && pl.nC > 1;
  if (keep && (!W_starts || !M_starts || !aligned(W_starts, 16) || !aligned(M_starts, 16)))
    return E2TTT_EINVAL;
  if (!W0 || !M0 || !W_end || !M_end) return E2TTT_EINVAL;
  const bool empty = pl.L == 0;
  if (!empty && (!q || !k || !v || !eta || !alpha || !beta || !out)) return E2TTT_EINVAL;
  if (!empty && pl.total > 0 && !workspace) return E2TTT_EINVAL;
  const void* ptrs16[] = {q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end};
  for (const void* p : ptrs16)
    if (p && !aligned(p, 16)) return E2TTT_EINVAL;
  if (workspace && !aligned(workspace, 256)) return E2TTT_EINVAL;
  if (!empty && workspace_bytes < pl.total) return E2TTT_EWORKSPACE;

  const size_t iosz = pl.io == E2TTT_BF16 ? 2 : 4;
  const size_t nx = static_cast<size_t>(pl.BH * pl.L * pl.d) * iosz;
  const size_t ns = static_cast<size_t>(pl.BH * pl.L) * 4;
  const size_t np = static_cast<size_t>(pl.BH * pl.P) * 4;
  const Range in[] = {rng(q, nx), rng(k, nx), rng(v, nx), rng(eta, ns), rng(alpha, ns),
                      rng(beta, ns), rng(W0, np), rng(M0, np)};
  const Range o_out = rng(out, nx), o_w = rng(W_end, np), o_m = rng(M_end, np),
              o_ws = rng(workspace, empty ? 0 : pl.total);
  const size_t nst = keep ? np * static_cast<size_t>(pl.nC - 1) : 0;
  const Range outs[] = {o_out, o_w, o_m, o_ws, rng(keep ? W_starts : nullptr, nst),
                        rng(keep ? M_starts : nullptr, nst)};
  for (int a = 0; a < 6; ++a) {
    for (int b = a + 1; b < 6; ++b)
      if (overlap(outs[a], outs[b])) return E2TTT_EINVAL;
    for (int i = 0; i < 8; ++i) {
      if (!overlap(outs[a], in[i])) continue;
      const bool exact_w = a == 1 && i == 6 && o_w.lo == in[6].lo;
      const bool exact_m = a == 2 && i == 7 && o_m.lo == in[7].lo;
      if (!exact_w && !exact_m) return E2TTT_EINVAL;
    }
  }

  status = device_ok();
  if (status != E2TTT_OK) return status;
  set_lds_attributes();
  (void)hipGetLastError();  // clear a stale error so only our launches are reported
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (keep) {
    pl.saveW = W_starts;
    pl.saveM = M_starts;
  }
  if (empty) {
    if (W_end != W0 || M_end != M0) {
      const int64_t n = pl.BH * pl.P;
      hipLaunchKernelGGL(k_copy2, dim3(grid1((n + 255) / 256)), dim3(256), 0, st, W0, M0, W_end,
                         M_end, n);
    }
  } else {
    char* ws = static_cast<char*>(workspace);
    if (pl.qknorm) {  // q, k -> silu, L2-normalised copies in the workspace
      const int64_t rows = pl.BH * pl.L;
      const unsigned gq = grid1((rows + 3) / 4);
      if (pl.io == E2TTT_BF16) {
        E2TTT_LAUNCH(I, E2TTT_KERNEL_PREP, k_qk_norm<bf16_t>, dim3(gq), dim3(256), 0, st,
                     static_cast<const bf16_t*>(q), reinterpret_cast<bf16_t*>(ws + pl.qn), rows,
                     pl.d);
        E2TTT_LAUNCH(I, E2TTT_KERNEL_PREP, k_qk_norm<bf16_t>, dim3(gq), dim3(256), 0, st,
                     static_cast<const bf16_t*>(k), reinterpret_cast<bf16_t*>(ws + pl.kn), rows,
                     pl.d);
      } else {
        E2TTT_LAUNCH(I, E2TTT_KERNEL_PREP, k_qk_norm<float>, dim3(gq), dim3(256), 0, st,
                     static_cast<const float*>(q), reinterpret_cast<float*>(ws + pl.qn), rows,
                     pl.d);
        E2TTT_LAUNCH(I, E2TTT_KERNEL_PREP, k_qk_norm<float>, dim3(gq), dim3(256), 0, st,
                     static_cast<const float*>(k), reinterpret_cast<float*>(ws + pl.kn), rows,
                     pl.d);
      }
      q = ws + pl.qn;
      k = ws + pl.kn;
    }
    if (pl.kind == E2TTT_LINEAR) {
      if (pl.io == E2TTT_BF16)
        launch_linear<bf16_t>(pl, q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end, ws, st, I);
      else
        launch_linear<float>(pl, q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end, ws, st, I);
    } else if (pl.fused) {
      launch_fused(pl, q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end, ws, st, I);
    } else if (pl.kind == E2TTT_MLP) {
      // The SwiGLU kernels on the state in their layout with W3 = 0 (the
      // gate held at one), advanced in place, then copied back.
      float* Wx = reinterpret_cast<float*>(ws + pl.wx);
      float* Mx = reinterpret_cast<float*>(ws + pl.mx);
      const int64_t n4 = pl.BH * 3 * pl.d * pl.h / 4;
      const unsigned gx = grid1((n4 + 255) / 256);
      hipLaunchKernelGGL(k_mlp_state, dim3(gx), dim3(256), 0, st, W0, Wx, pl.BH, pl.d, pl.h, 1);
      hipLaunchKernelGGL(k_mlp_state, dim3(gx), dim3(256), 0, st, M0, Mx, pl.BH, pl.d, pl.h, 1);
      if (pl.io == E2TTT_BF16)
        launch_swiglu<bf16_t>(pl, q, k, v, eta, alpha, beta, Wx, Mx, out, Wx, Mx, ws, st, I);
      else
        launch_swiglu<float>(pl, q, k, v, eta, alpha, beta, Wx, Mx, out, Wx, Mx, ws, st, I);
      hipLaunchKernelGGL(k_mlp_state, dim3(gx), dim3(256), 0, st, Wx, W_end, pl.BH, pl.d, pl.h,
                         0);
      hipLaunchKernelGGL(k_mlp_state, dim3(gx), dim3(256), 0, st, Mx, M_end, pl.BH, pl.d, pl.h,
                         0);
    } else {
      if (pl.io == E2TTT_BF16)
        launch_swiglu<bf16_t>(pl, q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end, ws, st, I);
      else
        launch_swiglu<float>(pl, q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end, ws, st, I);
    }
  }
  return hipGetLastError() == hipSuccess ? E2TTT_OK : E2TTT_EHIP;
}

}  // namespace

// Scratch of e2ttt_chunk_forward_noalloc: one array per GPU, in the code
// object, so that the entry point needs no allocation.  Host code never uses
// the array's name as an address (that is a host-side stand-in): the device
// address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress and kept.
static_assert(E2TTT_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[E2TTT_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // per device; guarded by g_scratch_mu

// Device address of the current device's scratch array (looked up on the
// first call on that device, with that device current).
e2ttt_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return E2TTT_EHIP;
  if (dev < 0 || dev >= 64) return E2TTT_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return E2TTT_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return E2TTT_OK;
}

}  // namespace

extern "C" {

e2ttt_status e2ttt_chunk_forward(const e2ttt_problem* prob, const void* q, const void* k,
                                 const void* v, const float* eta, const float* alpha,
                                 const float* beta, const float* W0, const float* M0, void* out,
                                 float* W_end, float* M_end, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  Instr none;
  return forward_impl(prob, q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end, workspace,
                      workspace_bytes, stream, none);
}

e2ttt_status e2ttt_chunk_forward_states(const e2ttt_problem* prob, const void* q,
                                        const void* k, const void* v, const float* eta,
                                        const float* alpha, const float* beta, const float* W0,
                                        const float* M0, void* out, float* W_end, float* M_end,
                                        float* W_starts, float* M_starts, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  Instr none;
  return forward_impl(prob, q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end, workspace,
                      workspace_bytes, stream, none, W_starts, M_starts, true);
}

e2ttt_status e2ttt_chunk_forward_noalloc(const e2ttt_problem* prob, const void* q,
                                         const void* k, const void* v, const float* eta,
                                         const float* alpha, const float* beta,
                                         const float* W0, const float* M0, void* out,
                                         float* W_end, float* M_end, void* stream) {
  Plan pl;
  const e2ttt_status st = make_plan(prob, &pl);
  if (st != E2TTT_OK) return st;
  if (pl.total > E2TTT_NOALLOC_SCRATCH_BYTES) return E2TTT_EWORKSPACE;
  void* ws = nullptr;
  if (pl.total > 0) {
    const e2ttt_status sa = scratch_address(&ws);
    if (sa != E2TTT_OK) return sa;
  }
  Instr none;
  return forward_impl(prob, q, k, v, eta, alpha, beta, W0, M0, out, W_end, M_end, ws,
                      pl.total > 0 ? static_cast<size_t>(E2TTT_NOALLOC_SCRATCH_BYTES) : 0,
                      stream, none);
}

e2ttt_status e2ttt_scalar_heads(const e2ttt_problem* prob, const void* x, int64_t model_dim,
                                const void* w_heads, const float* b_heads, float eta_base,
                                float alpha_base, float* eta, float* alpha, float* beta,
                                void* stream) {
  const e2ttt_status st = check_problem(prob);
  if (st != E2TTT_OK) return st;
  const int64_t B = prob->batch, H = prob->heads, L = prob->seq_len, D = model_dim;
  if (D < 64 || D % 64 != 0 || D > 65536 || H > 64) return E2TTT_EUNSUPPORTED;
  int64_t N;
  if (!mul_ok(B, L, &N) || N / kHeadsRows >= (int64_t(1) << 31))
    return E2TTT_EUNSUPPORTED;
  if (L == 0) return E2TTT_OK;
  if (!x || !w_heads || !b_heads || !eta || !alpha || !beta) return E2TTT_EINVAL;
  if (!aligned(x, 16) || !aligned(w_heads, 16) || !aligned(b_heads, 4) || !aligned(eta, 4) ||
      !aligned(alpha, 4) || !aligned(beta, 4))
    return E2TTT_EINVAL;
  const size_t el = prob->io_dtype == E2TTT_BF16 ? 2 : 4;
  const size_t ns = static_cast<size_t>(B * H * L) * 4;
  const Range in[] = {rng(x, static_cast<size_t>(N * D) * el),
                      rng(w_heads, static_cast<size_t>(3 * H * D) * el),
                      rng(b_heads, static_cast<size_t>(3 * H) * 4)};
  const Range outs[] = {rng(eta, ns), rng(alpha, ns), rng(beta, ns)};
  for (int i = 0; i < 3; ++i) {
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return E2TTT_EINVAL;
    for (int j = 0; j < 3; ++j)
      if (overlap(outs[i], in[j])) return E2TTT_EINVAL;
  }
  const e2ttt_status ds = device_ok();
  if (ds != E2TTT_OK) return ds;
  set_lds_attributes();
  (void)hipGetLastError();
  HeadsArgs ha;
  ha.x = x; ha.w = w_heads; ha.bias = b_heads;
  ha.N = N; ha.L = L; ha.D = D; ha.H = static_cast<int>(H);
  ha.eta_base = eta_base; ha.alpha_base = alpha_base;
  ha.eta = eta; ha.alpha = alpha; ha.beta = beta;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const unsigned grid = grid1((N + kHeadsRows - 1) / kHeadsRows);
  const int nb = static_cast<int>((3 * H + 15) / 16);
  auto launch = [&](auto tag, auto nbt) {
    typedef decltype(tag) T;
    constexpr int NBT = decltype(nbt)::value;
    void (*f)(HeadsArgs) = k_heads<T, NBT>;
    constexpr size_t lds = HeadsCfg<T, NBT>::LDS_BYTES;
    hipLaunchKernelGGL(f, dim3(grid), dim3(256), lds, hs, ha);
  };
  using I3 = std::integral_constant<int, 3>;
  using I6 = std::integral_constant<int, 6>;
  using I12 = std::integral_constant<int, 12>;
  if (prob->io_dtype == E2TTT_BF16) {
    if (nb <= 3) launch(bf16_t{}, I3{});
    else if (nb <= 6) launch(bf16_t{}, I6{});
    else launch(bf16_t{}, I12{});
  } else {
    if (nb <= 3) launch(float{}, I3{});
    else if (nb <= 6) launch(float{}, I6{});
    else launch(float{}, I12{});
  }
  return hipGetLastError() == hipSuccess ? E2TTT_OK : E2TTT_EHIP;
}

e2ttt_status e2ttt_chunk_forward_timed(const e2ttt_problem* prob, const void* q, const void* k,
                                       const void* v, const float* eta, const float* alpha,
                                       const float* beta, const float* W0, const float* M0,
                                       void* out, float* W_end, float* M_end, void* workspace,
                                       size_t workspace_bytes, void* stream, int kernel_class,
                                       void* const* events, int n_events, int* n_recorded) {
  if (kernel_class < 0 || kernel_class >= E2TTT_KERNEL_NUM_CLASSES || n_events < 0)
    return E2TTT_EINVAL;
  if (n_events > 0 && !events) return E2TTT_EINVAL;
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return E2TTT_EINVAL;
  Instr I;
  I.kclass = kernel_class;
  I.ev = events;
  I.n_pairs = n_events / 2;
  const e2ttt_status st = forward_impl(prob, q, k, v, eta, alpha, beta, W0, M0, out, W_end,
                                       M_end, workspace, workspace_bytes, stream, I);
  if (n_recorded) *n_recorded = st == E2TTT_OK ? I.used : 0;
  return st;
}

e2ttt_status e2ttt_scalar_kernels(const e2ttt_problem* prob, const float* eta,
                                  const float* alpha, const float* beta, float* k_w, float* k_m,
                                  float* chunk_coef, void* stream) {
  Plan pl;
  e2ttt_status st = make_plan(prob, &pl);
  if (st != E2TTT_OK) return st;
  if (pl.L == 0) return E2TTT_OK;
  if (!eta || !alpha || !beta || !k_w || !k_m || !chunk_coef) return E2TTT_EINVAL;
  const void* p16[] = {eta, alpha, beta, k_w, k_m};
  for (const void* p : p16)
    if (!aligned(p, 16)) return E2TTT_EINVAL;
  if (!aligned(chunk_coef, 4)) return E2TTT_EINVAL;
  const size_t ns = static_cast<size_t>(pl.BH * pl.L) * 4;
  const Range in[] = {rng(eta, ns), rng(alpha, ns), rng(beta, ns)};
  const Range outs[] = {rng(k_w, ns), rng(k_m, ns),
                        rng(chunk_coef, static_cast<size_t>(pl.BH * pl.nC * 3) * 4)};
  for (int a = 0; a < 3; ++a) {
    for (int b = a + 1; b < 3; ++b)
      if (overlap(outs[a], outs[b])) return E2TTT_EINVAL;
    for (int i = 0; i < 3; ++i)
      if (overlap(outs[a], in[i])) return E2TTT_EINVAL;
  }
  st = device_ok();
  if (st != E2TTT_OK) return st;
  set_lds_attributes();
  (void)hipGetLastError();
  Instr none;
  launch_scan(pl, eta, alpha, beta, k_w, k_m, pl.L, pl.C, 0, chunk_coef, 3,
              static_cast<hipStream_t>(stream), none);
  return hipGetLastError() == hipSuccess ? E2TTT_OK : E2TTT_EHIP;
}

}  // extern "C"

namespace {

// Decode workspace: the per-token scratch (z of q and k, a1, a3 of k
// [BH][h]; g [BH][d]; the W2^T g partials [d/64][BH][h]), then the chunk
// buffer of the buffered tokens and the chunk-end operands (DecodeBuf), then,
// with the q/k prologue, the normalised q and k of the token.  All fp32
// except those two (io dtype); sub-buffers 256-byte aligned.
struct DecodeLayout {
  int64_t BH, d, h, C, cb;
  size_t eb, ab, bb, kt, zt, d1, d3, gb, kb, gl, kw, km, coef, ut, gt, gw, gm, wx, mx, qn, kn,
      total;
};

DecodeLayout decode_layout(const e2ttt_problem* p) {
  DecodeLayout L;
  std::memset(&L, 0, sizeof(L));
  L.BH = p->batch * p->heads;
  L.d = p->dim;
  L.h = p->kind == E2TTT_LINEAR ? 0 : p->hidden;
  L.C = p->chunk;
  L.cb = L.h == 0 ? (L.C + 63) / 64 * 64 : (L.C + 127) / 128 * 128;
  const size_t BH = static_cast<size_t>(L.BH), d = static_cast<size_t>(L.d),
               h = static_cast<size_t>(L.h), cb = static_cast<size_t>(L.cb);
  size_t o = align256(4 * BH * (4 * h + d + (d / 64) * h));  // zq, zk, a1k, a3k, g, dz partials
  auto take = [&](size_t bytes) { const size_t at = o; o = align256(o + bytes); return at; };
  L.eb = take(4 * BH * cb);
  L.ab = take(4 * BH * cb);
  L.bb = take(4 * BH * cb);
  if (h != 0) {
    L.kt = take(4 * BH * d * cb);
    L.gb = take(4 * BH * d * cb);
    L.zt = take(4 * BH * h * cb);
    L.d1 = take(4 * BH * h * cb);
    L.d3 = take(4 * BH * h * cb);
    L.ut = take(4 * BH * 4 * h * cb);
    L.gt = take(4 * BH * 2 * d * cb);
  } else {
    L.kb = take(4 * BH * cb * d);
    L.gl = take(4 * BH * cb * d);
    L.gw = take(4 * BH * cb * d);
    L.gm = take(4 * BH * cb * d);
  }
  L.kw = take(4 * BH * cb);
  L.km = take(4 * BH * cb);
  L.coef = take(4 * BH * 4);
  if (p->kind == E2TTT_MLP) {  // the state in the aggregation's layout at a chunk end
    L.wx = take(4 * BH * 3 * d * h);
    L.mx = take(4 * BH * 3 * d * h);
  }
  if (p->flags & E2TTT_FLAG_QK_SILU_L2) {
    const size_t nx = BH * d * (p->io_dtype == E2TTT_BF16 ? 2 : 4);
    L.qn = take(nx);
    L.kn = take(nx);
  }
  L.total = o;
  return L;
}

e2ttt_status decode_check(const e2ttt_problem* prob) {
  const e2ttt_status st = check_problem(prob);
  if (st != E2TTT_OK) return st;
  if (prob->kind == E2TTT_LINEAR && prob->dim > 128) return E2TTT_EUNSUPPORTED;
  return E2TTT_OK;
}

}  // namespace

extern "C" {

e2ttt_status e2ttt_decode_workspace_bytes(const e2ttt_problem* prob, size_t* bytes) {
  if (!bytes) return E2TTT_EINVAL;
  const e2ttt_status st = decode_check(prob);
  if (st != E2TTT_OK) return st;
  *bytes = decode_layout(prob).total;
  return E2TTT_OK;
}

e2ttt_status e2ttt_decode_step(const e2ttt_problem* prob, const void* q, const void* k,
                               const void* v, const float* eta, const float* alpha,
                               const float* beta, float* W, float* M, void* out, int64_t pos,
                               int chunk_end, void* workspace, size_t workspace_bytes,
                               void* stream) {
  e2ttt_status st = decode_check(prob);
  if (st != E2TTT_OK) return st;
  const DecodeLayout Lw = decode_layout(prob);
  const int64_t BH = Lw.BH, d = Lw.d, h = Lw.h, cb = Lw.cb;
  const int64_t P = h == 0 ? d * d : (prob->kind == E2TTT_MLP ? 2 : 3) * d * h;
  if (pos < 0 || pos >= prob->chunk) return E2TTT_EINVAL;
  if (pos == prob->chunk - 1 && !chunk_end) return E2TTT_EINVAL;  // the last slot ends the chunk
  if (!q || !k || !v || !eta || !alpha || !beta || !W || !M || !out || !workspace)
    return E2TTT_EINVAL;
  const void* p16[] = {q, k, v, eta, alpha, beta, W, M, out};
  for (const void* p : p16)
    if (!aligned(p, 16)) return E2TTT_EINVAL;
  if (!aligned(workspace, 256)) return E2TTT_EINVAL;
  if (workspace_bytes < Lw.total) return E2TTT_EWORKSPACE;
  const size_t iosz = prob->io_dtype == E2TTT_BF16 ? 2 : 4;
  const size_t nx = static_cast<size_t>(BH * d) * iosz, ns = static_cast<size_t>(BH) * 4,
               np = static_cast<size_t>(BH * P) * 4;
  const Range in[] = {rng(q, nx), rng(k, nx), rng(v, nx), rng(eta, ns), rng(alpha, ns),
                      rng(beta, ns)};
  const Range outs[] = {rng(W, np), rng(M, np), rng(out, nx), rng(workspace, Lw.total)};
  for (int a = 0; a < 4; ++a) {
    for (int b = a + 1; b < 4; ++b)
      if (overlap(outs[a], outs[b])) return E2TTT_EINVAL;
    for (int i = 0; i < 6; ++i)
      if (overlap(outs[a], in[i])) return E2TTT_EINVAL;
  }
  st = device_ok();
  if (st != E2TTT_OK) return st;
  set_lds_attributes();
  (void)hipGetLastError();
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* wb = static_cast<char*>(workspace);
  float* ws = static_cast<float*>(workspace);
  auto F = [&](size_t off) { return off ? reinterpret_cast<float*>(wb + off) : nullptr; };
  DecodeArgs a;
  a.BH = BH; a.d = d; a.h = h;
  a.P = P;
  a.gated = prob->kind == E2TTT_MLP ? 0 : 1;
  a.W0 = W;
  a.zq = ws; a.zk = ws + BH * h; a.a1k = ws + 2 * BH * h; a.a3k = ws + 3 * BH * h;
  a.g = ws + 4 * BH * h;
  DecodeBuf b;
  b.cb = cb;
  b.eb = F(Lw.eb); b.ab = F(Lw.ab); b.bb = F(Lw.bb);
  b.kt = F(Lw.kt); b.zt = F(Lw.zt); b.d1 = F(Lw.d1); b.d3 = F(Lw.d3); b.gb = F(Lw.gb);
  b.kb = F(Lw.kb); b.gl = F(Lw.gl);
  b.kw = F(Lw.kw); b.km = F(Lw.km); b.coef = F(Lw.coef);
  b.ut = F(Lw.ut); b.gt = F(Lw.gt); b.gw = F(Lw.gw); b.gm = F(Lw.gm);
  auto run = [&](auto tag) {
    typedef decltype(tag) T;
    const T* Q = static_cast<const T*>(q);
    const T* K = static_cast<const T*>(k);
    if (prob->flags & E2TTT_FLAG_QK_SILU_L2) {
      T* qn = reinterpret_cast<T*>(wb + Lw.qn);
      T* kn = reinterpret_cast<T*>(wb + Lw.kn);
      hipLaunchKernelGGL(k_qk_norm<T>, dim3(grid1((BH + 3) / 4)), dim3(256), 0, s, Q, qn, BH, d);
      hipLaunchKernelGGL(k_qk_norm<T>, dim3(grid1((BH + 3) / 4)), dim3(256), 0, s, K, kn, BH, d);
      Q = qn;
      K = kn;
    }
    const T* V = static_cast<const T*>(v);
    T* O = static_cast<T*>(out);
    // The token: readout and descent factors at the chunk-start weights.
    float* part = ws + 4 * BH * h + BH * d;  // k_dec_bwd's partials of dz
    if (h == 0) {
      hipLaunchKernelGGL(k_dec_lin_fwd<T>, dim3(grid1(BH)), dim3(256), 0, s, a, Q, K, V, O);
    } else {
      // (d <= 1024, h <= 4096: the dot products take 1 .. 4 and 1 .. 16
      // pieces of 256 floats, 16 bytes per lane each)
      const int md = dot_pieces(d), mh = dot_pieces(h);
      void (*f13)(DecodeArgs, const T*, const T*) =
          md <= 1 ? k_dec_fwd13<T, 1> : md <= 2 ? k_dec_fwd13<T, 2>
          : md <= 3 ? k_dec_fwd13<T, 3> : k_dec_fwd13<T, 4>;
      void (*f2)(DecodeArgs, const T*, T*) =
          mh <= 1 ? k_dec_fwd2<T, 1> : mh <= 2 ? k_dec_fwd2<T, 2> : mh <= 3 ? k_dec_fwd2<T, 3>
          : mh <= 4 ? k_dec_fwd2<T, 4> : mh <= 6 ? k_dec_fwd2<T, 6> : mh <= 8 ? k_dec_fwd2<T, 8>
          : mh <= 12 ? k_dec_fwd2<T, 12> : k_dec_fwd2<T, 16>;
      hipLaunchKernelGGL(f13, dim3(grid1(BH * (h / 8))), dim3(256), 0, s, a, Q, K);
      hipLaunchKernelGGL(f2, dim3(grid1(BH * (d / 4))), dim3(256), 0, s, a, V, O);
      hipLaunchKernelGGL(k_dec_bwd, dim3(grid1(BH * (h / 64) * (d / 64))), dim3(256), 0, s, a,
                         part);
    }
    const int64_t nblk = (3 + 3 * h + 2 * d + 255) / 256;
    hipLaunchKernelGGL(k_dec_stash<T>, dim3(grid1(BH * nblk)), dim3(256), 0, s, a, b, pos, K,
                       eta, alpha, beta, static_cast<const float*>(part));
    if (!chunk_end) return;
    // Chunk end: the scalar kernels of the buffered tokens, the weighted
    // aggregations, (W, M) <- (W_C, M_C).
    const int64_t n = pos + 1;
    ScanArgs sa;
    sa.eta = b.eb; sa.alpha = b.ab; sa.beta = b.bb;
    // (the chunk-averaged variant and the LaCT rule differ from the default
    // rule only in these kernels and coefficients: the buffered tokens' means)
    sa.L = n; sa.C = n; sa.nC = 1; sa.mode = prob->decay_mode;
    sa.averaged = (prob->flags & E2TTT_FLAG_CHUNK_AVERAGED_DECAY) ? 1 : 0;
    sa.lact = (prob->flags & E2TTT_FLAG_LACT_RULE) ? 1 : 0;
    sa.kw = b.kw; sa.km = b.km; sa.ustride = cb; sa.rstride = 0; sa.pad = cb;
    sa.coef = b.coef; sa.cstride = 4; sa.istride = cb;
    const int tpt = scan_tpt(n);
    void (*fs)(ScanArgs) = tpt == 1 ? k_scan<256, 1, 1> : tpt == 2 ? k_scan<256, 2, 1>
                           : tpt == 4 ? k_scan<256, 4, 1> : k_scan<256, 8, 1>;
    hipLaunchKernelGGL(fs, dim3(grid1(BH)), dim3(256), 0, s, sa);
    if (h == 0) {
      hipLaunchKernelGGL(k_dec_pack_lin, dim3(grid1((BH * cb * d + 255) / 256)), dim3(256), 0, s,
                         a, b, n);
      Shape sh{BH, cb, d, 0, n, cb, 1, 1};
      const size_t lds = static_cast<size_t>(2 * 64 * 16 + 64 * d) * sizeof(float);
      hipLaunchKernelGGL(k_lin_agg<float>, dim3(grid1(BH * (d / 16))), dim3(256), lds, s, sh, 0,
                         static_cast<const float*>(b.kb), static_cast<const float*>(b.gw),
                         static_cast<const float*>(b.gm), static_cast<const float*>(b.coef),
                         static_cast<const float*>(W), static_cast<const float*>(M), W, M);
    } else {
      hipLaunchKernelGGL(k_dec_pack, dim3(grid1(BH * (5 * h + 3 * d))), dim3(256), 0, s, a, b,
                         n);
      // The MLP's [W1 | W2] state goes through the [W1 | W3 = 0 | W2] layout
      // of the aggregation (its W3 aggregates are zero: dA3 = 0).
      const bool mlp = prob->kind == E2TTT_MLP;
      float* Ws = mlp ? F(Lw.wx) : W;
      float* Ms = mlp ? F(Lw.mx) : M;
      const unsigned gx = grid1((BH * 3 * d * h / 4 + 255) / 256);
      if (mlp) {
        hipLaunchKernelGGL(k_mlp_state, dim3(gx), dim3(256), 0, s, W, Ws, BH, d, h, 1);
        hipLaunchKernelGGL(k_mlp_state, dim3(gx), dim3(256), 0, s, M, Ms, BH, d, h, 1);
      }
      Shape sh{BH, cb, d, h, cb, cb, 1, 1};
      const int64_t na = (4 * h / 128) * (d / 128), nbk = (2 * d / 128) * (h / 128);
      hipLaunchKernelGGL(k_agg<float>, dim3(grid1(BH * (na + nbk))), dim3(256), 0, s, sh, 0, 1,
                         static_cast<const float*>(b.ut), static_cast<const float*>(b.kt),
                         static_cast<const float*>(b.gt), static_cast<const float*>(b.zt),
                         static_cast<const float*>(b.coef), static_cast<const float*>(Ws),
                         static_cast<const float*>(Ms), Ws, Ms, static_cast<float*>(nullptr),
                         static_cast<float*>(nullptr), static_cast<float*>(nullptr));
      if (prob->flags & E2TTT_FLAG_POST_CHUNK_ROW_L2) {
        const int64_t rows = BH * (2 * h + d);
        hipLaunchKernelGGL(k_row_l2norm, dim3(grid1((rows + 3) / 4)), dim3(256), 0, s, Ws, BH, d,
                           h);
      }
      if (mlp) {
        hipLaunchKernelGGL(k_mlp_state, dim3(gx), dim3(256), 0, s, Ws, W, BH, d, h, 0);
        hipLaunchKernelGGL(k_mlp_state, dim3(gx), dim3(256), 0, s, Ms, M, BH, d, h, 0);
      }
      return;
    }
    if (prob->flags & E2TTT_FLAG_POST_CHUNK_ROW_L2) {
      const int64_t rows = BH * d;
      hipLaunchKernelGGL(k_row_l2norm, dim3(grid1((rows + 3) / 4)), dim3(256), 0, s, W, BH, d, h);
    }
  };
  if (prob->io_dtype == E2TTT_BF16) run(bf16_t{});
  else run(float{});
  return hipGetLastError() == hipSuccess ? E2TTT_OK : E2TTT_EHIP;
}

}  // extern "C"

namespace {

// Workspace of the linear learner's backward: the forward's scan and
// residual buffers, then the chunk-start states, the state adjoints and the
// per-token adjoint terms (byte offsets, 256-aligned).
struct BwdPlan {
  Plan f;
  // State length per unit inside the backward: the caller's P, except for the
  // MLP learner, whose states and adjoints are carried in the SwiGLU layout
  // [W1 | W3 = 0 | W2] (3dh) and expanded / compacted at the boundary.
  int64_t P;
  bool mlp;
  size_t w0x, m0x, dw0x, dm0x;  // MLP: expanded W0, M0 and the adjoints of them, [BH][3dh]
  size_t wst, mst;            // chunk-start states of chunks 1 .. nC-1 (slot r), [nC][BH][P]
  size_t dwa, dwb, dma, dmb;  // state adjoints, two of each in turn, [BH][P]
  size_t de;                  // linear: [BH][Cp][d]
  size_t sw, sm;              // dK^W, dK^M, [BH][nC][Cp]
  size_t dots;                // [BH][nC][nrb][4]
  size_t bcp;                 // fp64 b, c, P, [BH][nC][Cp][3]
  int64_t nrb;                // partial-sum blocks of the chunk-coefficient dots
  // SwiGLU, one chunk at a time, token-major [BH][Cp][width]:
  size_t hk, hq, tw, tm, du, uw, um, da, daq;  // width 2h
  size_t zk, zq, wv, dzq, r2w, r2m, dwv, dza;  // width h
  size_t e, s2w, s2m, dea;                     // width d
  // bf16 io: fp32 copies of q, k, v, dout and fp32 dq, dk, dv, [BH][L][d]
  bool bf16io;
  size_t xq, xk, xv, xdo, xdq, xdk, xdv;
  // q/k prologue: normalised q, k and their adjoints, fp32 [BH][L][d]
  bool qknorm;
  size_t nq, nk, dnq, dnk;
  // chunk-boundary row normalisation: each chunk's end state before it,
  // [nC][BH][P], and the adjoint taken back through it, [BH][P]
  bool rownorm;
  size_t wpre, dwn;
  size_t total;
};

e2ttt_status make_bwd_plan(const e2ttt_problem* p, BwdPlan* bp) {
  // The backward computes in fp32; bf16 io is converted at the boundary, so
  // the inner plan (and the forward re-run) is the fp32 one.
  e2ttt_problem pf;
  if (p && p->struct_size == sizeof(e2ttt_problem)) {
    pf = *p;
    pf.io_dtype = E2TTT_F32;
  }
  const e2ttt_status st = make_plan(p && p->struct_size == sizeof(e2ttt_problem) ? &pf : p,
                                    &bp->f);
  if (st != E2TTT_OK) return st;
  if (p->io_dtype != E2TTT_F32 && p->io_dtype != E2TTT_BF16) return E2TTT_EINVAL;
  bp->bf16io = p->io_dtype == E2TTT_BF16;
  const Plan& q = bp->f;
  // Every flag of the forward is supported (the compensated-weights option
  // only concerns bf16 matrix operands; the backward computes in fp32).
  bp->mlp = q.kind == E2TTT_MLP;
  bp->P = bp->mlp ? 3 * q.d * q.h : q.P;
  bp->qknorm = q.qknorm != 0;
  bp->rownorm = q.rownorm != 0;
  if (q.kind == E2TTT_LINEAR && q.d > 64) return E2TTT_EUNSUPPORTED;
  if (q.kind == E2TTT_SWIGLU && q.BH > 65535) return E2TTT_EUNSUPPORTED;  // grid z
  size_t o = align256(q.total);
  auto take = [&](size_t bytes) { const size_t at = o; o = align256(o + bytes); return at; };
  const size_t np = 4 * static_cast<size_t>(q.BH * bp->P);
  bp->nrb = q.kind == E2TTT_LINEAR ? q.d / 16 : (bp->P + SWB_STATE_ELEMS - 1) / SWB_STATE_ELEMS;
  bp->wst = take(np * q.nC);
  bp->mst = take(np * q.nC);
  bp->dwa = take(np);
  bp->dwb = take(np);
  bp->dma = take(np);
  bp->dmb = take(np);
  bp->sw = take(4 * static_cast<size_t>(q.BH * q.nC * q.Cp));
  bp->sm = take(4 * static_cast<size_t>(q.BH * q.nC * q.Cp));
  bp->dots = take(4 * static_cast<size_t>(q.BH * q.nC * bp->nrb * 4));
  bp->bcp = take(8 * static_cast<size_t>(q.BH * q.nC * q.Cp * 3));
  const size_t rows = 4 * static_cast<size_t>(q.BH * q.Cp);
  if (q.kind == E2TTT_LINEAR) {
    bp->de = take(rows * q.d);
  } else {
    for (size_t* b : {&bp->hk, &bp->hq, &bp->tw, &bp->tm, &bp->du, &bp->uw, &bp->um, &bp->da,
                      &bp->daq})
      *b = take(rows * 2 * q.h);
    for (size_t* b : {&bp->zk, &bp->zq, &bp->wv, &bp->dzq, &bp->r2w, &bp->r2m, &bp->dwv,
                      &bp->dza})
      *b = take(rows * q.h);
    for (size_t* b : {&bp->e, &bp->s2w, &bp->s2m, &bp->dea}) *b = take(rows * q.d);
  }
  if (bp->bf16io)
    for (size_t* b : {&bp->xq, &bp->xk, &bp->xv, &bp->xdo, &bp->xdq, &bp->xdk, &bp->xdv})
      *b = take(4 * static_cast<size_t>(q.BH * q.L * q.d));
  if (bp->qknorm)
    for (size_t* b : {&bp->nq, &bp->nk, &bp->dnq, &bp->dnk})
      *b = take(4 * static_cast<size_t>(q.BH * q.L * q.d));
  if (bp->rownorm) {
    bp->wpre = take(np * q.nC);
    bp->dwn = take(np);
  }
  if (bp->mlp)
    for (size_t* b : {&bp->w0x, &bp->m0x, &bp->dw0x, &bp->dm0x}) *b = take(np);
  bp->total = q.L == 0 ? 0 : o;
  return E2TTT_OK;
}

// Batched fp32 GEMM over the BH units (grid z).  Products with few 64 x 64
// output tiles and a long K (where the grid would leave most CUs idle) run
// on 32 x 32 tiles with K split four ways inside each workgroup.
void gemm_f32(GemmF32 g, int64_t BH, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return;
  const int64_t tiles = ((g.N + GF_T - 1) / GF_T) * ((g.M + GF_T - 1) / GF_T) * BH;
  if (tiles <= kCUs && g.K >= 2 * 4 * GF_K) {
    const dim3 grid(static_cast<unsigned>((g.N + GQ_T - 1) / GQ_T),
                    static_cast<unsigned>((g.M + GQ_T - 1) / GQ_T), static_cast<unsigned>(BH));
    hipLaunchKernelGGL(k_gemm_f32_k4<32>, grid, dim3(256), GemmK4<32>::LDS_BYTES, s, g);
    return;
  }
  const dim3 grid(static_cast<unsigned>((g.N + GF_T - 1) / GF_T),
                  static_cast<unsigned>((g.M + GF_T - 1) / GF_T), static_cast<unsigned>(BH));
  hipLaunchKernelGGL(k_gemm_f32, grid, dim3(256), 0, s, g);
}

GemmF32 gf(int64_t M, int64_t N, int64_t K, const float* A, int64_t sAb, int64_t sAm,
           int64_t sAk, const float* B, int64_t sBb, int64_t sBk, int64_t sBn, const float* D,
           int64_t sDb, int64_t ldd, float* C, int64_t sCb, int64_t ldc, float alpha = 1.0f) {
  return GemmF32{M, N, K, A, sAb, sAm, sAk, B, sBb, sBk, sBn, D, sDb, ldd, C, sCb, ldc, alpha};
}

// The SwiGLU learner's backward (fp32): forward re-run for the chunk-start
// states, then the chunks in reverse, each as the GEMMs and per-token steps
// listed in swiglu_backward.hpp.  The scalar kernels, the chunk
// coefficients and the adjoint buffers are set up by the caller.
void swiglu_backward(const BwdPlan& bp, char* ws, const float* Q, const float* K,
                     const float* V, const float* W0, const float* M0, const float* DO,
                     const float* dWC, const float* dMC, float* dq, float* dk, float* dv,
                     float* dW0, float* dM0, const float* Wsv, const float* Msv,
                     hipStream_t s) {
  const Plan& q = bp.f;
  auto wsf = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  Shape sh{q.BH, q.L, q.d, q.h, q.C, q.Cp, q.nC, q.krep};
  sh.gated = bp.mlp ? 0 : 1;
  const int64_t BH = q.BH, L = q.L, d = q.d, h = q.h, Cp = q.Cp, P = bp.P, nP = BH * P;
  const int64_t Ld = L * d;
  float* kw = wsf(q.kw);
  float* km = wsf(q.km);
  float* coef = wsf(q.coef);
  auto Wst = [&](int64_t r) -> float* { return wsf(bp.wst) + r * nP; };
  auto Mst = [&](int64_t r) -> float* { return wsf(bp.mst) + r * nP; };
  // Chunk-start states: the caller's (from e2ttt_chunk_forward_states) or re-run.
  auto Win = [&](int64_t r) -> const float* {
    return r == 0 ? W0 : Wsv ? Wsv + (r - 1) * nP : Wst(r);
  };
  auto Min = [&](int64_t r) -> const float* {
    return r == 0 ? M0 : Msv ? Msv + (r - 1) * nP : Mst(r);
  };
  // Forward re-run (the generic chunk kernels; the readout goes to dq, which
  // the backward overwrites for every token), unless the states were given.
  if (!Wsv) {
    float* kt = wsf(q.kt);
    float* w13s = wsf(q.w13s);
    float* w2s = wsf(q.w2s);
    float* w2ts = wsf(q.w2ts);
    float* zrow = wsf(q.zrow);
    float* a1s = wsf(q.a1s);
    float* a3s = wsf(q.a3s);
    float* grow = wsf(q.grow);
    float* ut = wsf(q.ut);
    float* gt = wsf(q.gt);
    float* zt = wsf(q.zt);
    // With row normalisation every chunk is re-run (the last one's end state
    // before normalisation is needed too); each end state is kept before it
    // is normalised into the next chunk's start (and its operand shadows).
    const bool rn = bp.rownorm;
    if (q.nC > 1 || rn) {
      hipLaunchKernelGGL((k_prep_kt<float, false>),
                         dim3(grid1(BH * q.nC * (Cp / 64) * (d / 64))), dim3(256), 0, s, sh, K, kt);
      hipLaunchKernelGGL(k_prep_shadow<float>, dim3(grid1(shadow_blocks(sh))), dim3(256), 0, s,
                         sh, W0, w13s, w2s, w2ts);
    }
    const int64_t na = (4 * h / 128) * (d / 128), nb = (2 * d / 128) * (h / 128);
    for (int64_t r = 0; r + (rn ? 0 : 1) < q.nC; ++r) {
      const int ri = static_cast<int>(r);
      const bool more = r + 1 < q.nC;
      float* Wout = rn ? wsf(bp.wpre) + r * nP : Wst(r + 1);
      float* Mout = more ? Mst(r + 1) : wsf(bp.dwn);  // the last M is not needed
      hipLaunchKernelGGL(k_fwd13<float>, dim3(grid1(BH * (2 * Cp / 128) * (2 * h / 128))),
                         dim3(256), 0, s, sh, ri, Q, K, w13s, zrow, a1s, a3s, zt);
      hipLaunchKernelGGL(k_fwd2<float>, dim3(grid1(BH * (2 * Cp / 128) * (d / 128))), dim3(256),
                         0, s, sh, ri, V, dq, zrow, w2s, kw, km, grow, gt);
      hipLaunchKernelGGL(k_bwd<float>, dim3(grid1(BH * (Cp / 128) * (h / 128))), dim3(256), 0,
                         s, sh, ri, grow, w2ts, a1s, a3s, kw, km, ut);
      hipLaunchKernelGGL(k_agg<float>, dim3(grid1(BH * (na + nb))), dim3(256), 0, s, sh, ri,
                         rn ? 1 : 0, ut, kt, gt, zt, coef, Win(r), Min(r), Wout, Mout, w13s, w2s,
                         w2ts);
      if (rn && more) {
        hipLaunchKernelGGL(k_copy_or_zero, dim3(grid1((nP + 255) / 256)), dim3(256), 0, s,
                           static_cast<const float*>(Wout), Wst(r + 1), nP);
        launch_rownorm<float>(q, sh, Wst(r + 1), true, w13s, w2s, w2ts, s);
      }
    }
  }
  float *HK = wsf(bp.hk), *HQ = wsf(bp.hq), *TW = wsf(bp.tw), *TM = wsf(bp.tm),
        *DU = wsf(bp.du), *UW = wsf(bp.uw), *UM = wsf(bp.um), *DA = wsf(bp.da),
        *DAQ = wsf(bp.daq), *ZK = wsf(bp.zk), *ZQ = wsf(bp.zq), *WV = wsf(bp.wv),
        *DZQ = wsf(bp.dzq), *R2W = wsf(bp.r2w), *R2M = wsf(bp.r2m), *DW = wsf(bp.dwv),
        *DZA = wsf(bp.dza), *E = wsf(bp.e), *S2W = wsf(bp.s2w), *S2M = wsf(bp.s2m),
        *DEA = wsf(bp.dea);
  const int64_t b2 = Cp * 2 * h, b1 = Cp * h, bd = Cp * d;  // unit strides of the buffers
  const int64_t o2 = 2 * h * d;                              // offset of W2 in a state
  const int64_t nrows = BH * (2 * h + d);
  for (int64_t r = q.nC - 1; r >= 0; --r) {
    const int ri = static_cast<int>(r);
    const int64_t t0 = r * q.C, n = (L - t0) < q.C ? (L - t0) : q.C;
    if (bp.rownorm) {  // back through this chunk's normalisation
      hipLaunchKernelGGL(k_row_l2norm_bwd, dim3(grid1((nrows + 3) / 4)), dim3(256), 0, s,
                         static_cast<const float*>(wsf(bp.wpre) + r * nP), dWC, wsf(bp.dwn), BH,
                         d, h);
      dWC = wsf(bp.dwn);
    }
    const float *Kr = K + t0 * d, *Qr = Q + t0 * d, *Vr = V + t0 * d, *DOr = DO + t0 * d;
    float *dqr = dq + t0 * d, *dkr = dk + t0 * d, *dvr = dv + t0 * d;
    const float* Ws = Win(r);
    const float* Ms = Min(r);
    float* dWp;
    float* dMp;
    if (r == 0) {
      dWp = dW0;
      dMp = dM0;
    } else {
      dWp = dWC == wsf(bp.dwa) ? wsf(bp.dwb) : wsf(bp.dwa);
      dMp = dMC == wsf(bp.dma) ? wsf(bp.dmb) : wsf(bp.dma);
    }
    // Forward quantities at Ws.
    gemm_f32(gf(n, 2 * h, d, Kr, Ld, d, 1, Ws, P, 1, d, nullptr, 0, 0, HK, b2, 2 * h), BH, s);
    gemm_f32(gf(n, 2 * h, d, Qr, Ld, d, 1, Ws, P, 1, d, nullptr, 0, 0, HQ, b2, 2 * h), BH, s);
    const unsigned gact = grid1((BH * n * h + 255) / 256);
    hipLaunchKernelGGL(k_swb_act, dim3(gact), dim3(256), 0, s, BH, n, h, Cp, sh.gated, HK, ZK);
    hipLaunchKernelGGL(k_swb_act, dim3(gact), dim3(256), 0, s, BH, n, h, Cp, sh.gated, HQ, ZQ);
    gemm_f32(gf(n, d, h, ZK, b1, h, 1, Ws + o2, P, 1, h, Vr, Ld, d, E, bd, d, -1.0f), BH, s);
    gemm_f32(gf(n, h, d, E, bd, d, 1, Ws + o2, P, h, 1, nullptr, 0, 0, WV, b1, h), BH, s);
    gemm_f32(gf(n, h, d, DOr, Ld, d, 1, Ws + o2, P, h, 1, nullptr, 0, 0, DZQ, b1, h), BH, s);
    // Products with the chunk-end adjoints.
    gemm_f32(gf(n, 2 * h, d, Kr, Ld, d, 1, dWC, P, 1, d, nullptr, 0, 0, TW, b2, 2 * h), BH, s);
    gemm_f32(gf(n, 2 * h, d, Kr, Ld, d, 1, dMC, P, 1, d, nullptr, 0, 0, TM, b2, 2 * h), BH, s);
    gemm_f32(gf(n, d, h, ZK, b1, h, 1, dWC + o2, P, 1, h, nullptr, 0, 0, S2W, bd, d), BH, s);
    gemm_f32(gf(n, d, h, ZK, b1, h, 1, dMC + o2, P, 1, h, nullptr, 0, 0, S2M, bd, d), BH, s);
    gemm_f32(gf(n, h, d, E, bd, d, 1, dWC + o2, P, h, 1, nullptr, 0, 0, R2W, b1, h), BH, s);
    gemm_f32(gf(n, h, d, E, bd, d, 1, dMC + o2, P, h, 1, nullptr, 0, 0, R2M, b1, h), BH, s);
    if (n > 0) {
      SwbTokArgs ta;
      ta.n = n; ta.d = d; ta.h = h; ta.Cp = Cp; ta.nC = q.nC; ta.r = ri; ta.gated = sh.gated;
      ta.HK = HK; ta.WV = WV; ta.E = E; ta.TW = TW; ta.TM = TM; ta.SW = S2W; ta.SM = S2M;
      ta.RW = R2W; ta.RM = R2M; ta.kw = kw; ta.km = km;
      ta.sw = wsf(bp.sw); ta.sm = wsf(bp.sm); ta.DU = DU; ta.DW = DW; ta.DEA = DEA;
      ta.DZA = DZA; ta.UW = UW; ta.UM = UM;
      hipLaunchKernelGGL(k_swb_tok, dim3(grid1(BH * n)), dim3(256), 0, s, ta);
    }
    // de (= dv) and dz.
    gemm_f32(gf(n, d, h, DW, b1, h, 1, Ws + o2, P, 1, h, DEA, bd, d, dvr, Ld, d), BH, s);
    gemm_f32(gf(n, h, d, dvr, Ld, d, 1, Ws + o2, P, h, 1, DZA, b1, h, DZA, b1, h, -1.0f), BH, s);
    hipLaunchKernelGGL(k_swb_da, dim3(gact), dim3(256), 0, s, BH, n, h, Cp, sh.gated, HK, WV,
                       DU, DZA, HQ, DZQ, DA, DAQ);
    // dk, dq.
    gemm_f32(gf(n, d, 2 * h, DA, b2, 2 * h, 1, Ws, P, d, 1, nullptr, 0, 0, dkr, Ld, d), BH, s);
    gemm_f32(gf(n, d, 2 * h, UW, b2, 2 * h, 1, dWC, P, d, 1, dkr, Ld, d, dkr, Ld, d), BH, s);
    gemm_f32(gf(n, d, 2 * h, UM, b2, 2 * h, 1, dMC, P, d, 1, dkr, Ld, d, dkr, Ld, d), BH, s);
    gemm_f32(gf(n, d, 2 * h, DAQ, b2, 2 * h, 1, Ws, P, d, 1, nullptr, 0, 0, dqr, Ld, d), BH, s);
    // Previous chunk's state adjoints: state terms, then the token sums.
    hipLaunchKernelGGL(k_swb_state, dim3(grid1(BH * bp.nrb)), dim3(256), 0, s, P, bp.nrb, q.nC,
                       ri, coef, Ws, Ms, dWC, dMC, dWp, dMp, wsf(bp.dots));
    gemm_f32(gf(2 * h, d, n, DA, b2, 1, 2 * h, Kr, Ld, d, 1, dWp, P, d, dWp, P, d), BH, s);
    gemm_f32(gf(2 * h, d, n, DAQ, b2, 1, 2 * h, Qr, Ld, d, 1, dWp, P, d, dWp, P, d), BH, s);
    gemm_f32(gf(d, h, n, E, bd, 1, d, DW, b1, h, 1, dWp + o2, P, h, dWp + o2, P, h), BH, s);
    gemm_f32(gf(d, h, n, dvr, Ld, 1, d, ZK, b1, h, 1, dWp + o2, P, h, dWp + o2, P, h, -1.0f),
             BH, s);
    gemm_f32(gf(d, h, n, DOr, Ld, 1, d, ZQ, b1, h, 1, dWp + o2, P, h, dWp + o2, P, h), BH, s);
    dWC = dWp;
    dMC = dMp;
  }
}

// The linear learner's backward (fp32): forward re-run for the chunk-start
// states, then the chunks in reverse (backward.hpp).
void linear_backward(const BwdPlan& bp, char* ws, const float* Q, const float* K,
                     const float* V, const float* W0, const float* M0, const float* DO,
                     const float* dWC, const float* dMC, float* dq, float* dk, float* dv,
                     float* dW0, float* dM0, const float* Wsv, const float* Msv,
                     hipStream_t s) {
  const Plan& pl = bp.f;
  auto wsf = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  const Shape sh{pl.BH, pl.L, pl.d, 0, pl.C, pl.Cp, pl.nC, 1};
  const int64_t nP = pl.BH * pl.P;
  float* kw = wsf(pl.kw);
  float* km = wsf(pl.km);
  float* coef = wsf(pl.coef);
  // Forward re-run for the chunk-start states (the readout goes to dq, which
  // the backward overwrites for every token).
  auto Wst = [&](int64_t r) -> float* { return wsf(bp.wst) + r * nP; };
  auto Mst = [&](int64_t r) -> float* { return wsf(bp.mst) + r * nP; };
  // Chunk-start states: the caller's (from e2ttt_chunk_forward_states) or re-run.
  auto Win = [&](int64_t r) -> const float* {
    return r == 0 ? W0 : Wsv ? Wsv + (r - 1) * nP : Wst(r);
  };
  auto Min = [&](int64_t r) -> const float* {
    return r == 0 ? M0 : Msv ? Msv + (r - 1) * nP : Mst(r);
  };
  const size_t lds_f = static_cast<size_t>(pl.d * (pl.d + 1) + LIN_FWD_TB * (pl.d + 1)) * sizeof(float);
  const size_t lds_a = static_cast<size_t>(2 * 64 * 16 + 64 * pl.d) * sizeof(float);
  // With row normalisation every chunk is re-run (the last one's end state
  // before normalisation is needed too) and each end state is kept before
  // being normalised into the next chunk's start.
  const bool rn = bp.rownorm;
  const int64_t rows = pl.BH * pl.d;
  for (int64_t r = 0; !Wsv && r + (rn ? 0 : 1) < pl.nC; ++r) {
    const int ri = static_cast<int>(r);
    const bool more = r + 1 < pl.nC;
    float* Wout = rn ? wsf(bp.wpre) + r * nP : Wst(r + 1);
    float* Mout = more ? Mst(r + 1) : wsf(bp.dwn);  // the last M is not needed
    hipLaunchKernelGGL(k_lin_fwd<float>, dim3(grid1(pl.BH * (2 * pl.Cp / LIN_FWD_TB))), dim3(256), lds_f,
                       s, sh, ri, Q, K, V, Win(r), kw, km, dq, wsf(pl.gw), wsf(pl.gm));
    hipLaunchKernelGGL(k_lin_agg<float>, dim3(grid1(pl.BH * (pl.d / 16))), dim3(256), lds_a, s,
                       sh, ri, K, wsf(pl.gw), wsf(pl.gm), coef, Win(r), Min(r), Wout, Mout);
    if (rn && more) {
      hipLaunchKernelGGL(k_copy_or_zero, dim3(grid1((nP + 255) / 256)), dim3(256), 0, s,
                         static_cast<const float*>(Wout), Wst(r + 1), nP);
      hipLaunchKernelGGL(k_row_l2norm, dim3(grid1((rows + 3) / 4)), dim3(256), 0, s, Wst(r + 1),
                         pl.BH, pl.d, int64_t(0));
    }
  }
  // Reverse chunk loop.
  const size_t lds_t = static_cast<size_t>(lin_bwd_tok_lds_floats(pl.d)) * sizeof(float);
  const size_t lds_s = static_cast<size_t>(lin_bwd_state_lds_floats(pl.d)) * sizeof(float);
  for (int64_t r = pl.nC - 1; r >= 0; --r) {
    if (rn) {  // back through this chunk's normalisation
      hipLaunchKernelGGL(k_row_l2norm_bwd, dim3(grid1((rows + 3) / 4)), dim3(256), 0, s,
                         static_cast<const float*>(wsf(bp.wpre) + r * nP), dWC, wsf(bp.dwn),
                         pl.BH, pl.d, int64_t(0));
      dWC = wsf(bp.dwn);
    }
    LinBwdArgs a;
    a.s = sh;
    a.r = static_cast<int>(r);
    a.mode = pl.mode;
    a.q = Q; a.k = K; a.v = V; a.dout = DO;
    a.Ws = Win(r); a.Ms = Min(r);
    a.dWC = dWC; a.dMC = dMC;
    a.kw = kw; a.km = km; a.coef = coef;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.de = wsf(bp.de); a.sw = wsf(bp.sw); a.sm = wsf(bp.sm); a.dots = wsf(bp.dots);
    if (r == 0) {
      a.dWp = dW0;
      a.dMp = dM0;
    } else {
      a.dWp = dWC == wsf(bp.dwa) ? wsf(bp.dwb) : wsf(bp.dwa);
      a.dMp = dMC == wsf(bp.dma) ? wsf(bp.dmb) : wsf(bp.dma);
    }
    const int R = static_cast<int>(pl.d / 16);
    void (*ktok)(LinBwdArgs) = R == 1 ? k_lin_bwd_tok<1> : R == 2 ? k_lin_bwd_tok<2>
                               : R == 3 ? k_lin_bwd_tok<3> : k_lin_bwd_tok<4>;
    void (*kst)(LinBwdArgs) = R == 1 ? k_lin_bwd_state<1> : R == 2 ? k_lin_bwd_state<2>
                              : R == 3 ? k_lin_bwd_state<3> : k_lin_bwd_state<4>;
    hipLaunchKernelGGL(ktok, dim3(grid1(pl.BH * (pl.Cp / LIN_BWD_TB))), dim3(256), lds_t, s, a);
    hipLaunchKernelGGL(kst, dim3(grid1(pl.BH * R)), dim3(256), lds_s, s, a);
    dWC = a.dWp;
    dMC = a.dMp;
  }
}

}  // namespace

extern "C" {

e2ttt_status e2ttt_backward_workspace_bytes(const e2ttt_problem* prob, size_t* bytes) {
  if (!bytes) return E2TTT_EINVAL;
  BwdPlan bp;
  const e2ttt_status st = make_bwd_plan(prob, &bp);
  if (st != E2TTT_OK) return st;
  *bytes = bp.total;
  return E2TTT_OK;
}

namespace {

e2ttt_status backward_impl(const e2ttt_problem* prob, const void* q, const void* k,
                           const void* v, const float* eta, const float* alpha,
                           const float* beta, const float* W0, const float* M0,
                           const void* dout, const float* dW_end, const float* dM_end,
                           const float* W_starts, const float* M_starts, void* dq, void* dk,
                           void* dv, float* deta, float* dalpha, float* dbeta, float* dW0,
                           float* dM0, void* workspace, size_t workspace_bytes, void* stream) {
  BwdPlan bp;
  e2ttt_status st = make_bwd_plan(prob, &bp);
  if (st != E2TTT_OK) return st;
  const Plan& pl = bp.f;
  const bool empty = pl.L == 0;
  if ((W_starts == nullptr) != (M_starts == nullptr)) return E2TTT_EINVAL;
  const bool keep = W_starts && pl.nC > 1;  // caller-kept chunk-start states
  if (keep && (!aligned(W_starts, 16) || !aligned(M_starts, 16))) return E2TTT_EINVAL;
  // The reverse of the row normalisation needs each chunk's end state before
  // it, which the kept (normalised) states do not carry.
  if (keep && bp.rownorm) return E2TTT_EUNSUPPORTED;
  if (!W0 || !M0 || !dW0 || !dM0) return E2TTT_EINVAL;
  if (!empty && (!q || !k || !v || !eta || !alpha || !beta || !dout || !dq || !dk || !dv ||
                 !deta || !dalpha || !dbeta || !workspace))
    return E2TTT_EINVAL;
  const void* p16[] = {q, k, v, eta, alpha, beta, W0, M0, dout, dW_end, dM_end,
                       dq, dk, dv, deta, dalpha, dbeta, dW0, dM0};
  for (const void* p : p16)
    if (p && !aligned(p, 16)) return E2TTT_EINVAL;
  if (workspace && !aligned(workspace, 256)) return E2TTT_EINVAL;
  if (!empty && workspace_bytes < bp.total) return E2TTT_EWORKSPACE;
  const size_t nx = static_cast<size_t>(pl.BH * pl.L * pl.d) * (bp.bf16io ? 2 : 4);
  const size_t ns = static_cast<size_t>(pl.BH * pl.L) * 4;
  const size_t np = static_cast<size_t>(pl.BH * pl.P) * 4;
  const size_t nst = keep ? np * static_cast<size_t>(pl.nC - 1) : 0;
  const Range in[] = {rng(q, nx), rng(k, nx), rng(v, nx), rng(eta, ns), rng(alpha, ns),
                      rng(beta, ns), rng(W0, np), rng(M0, np), rng(dout, nx),
                      rng(dW_end, np), rng(dM_end, np), rng(keep ? W_starts : nullptr, nst),
                      rng(keep ? M_starts : nullptr, nst)};
  const Range outs[] = {rng(dq, nx), rng(dk, nx), rng(dv, nx), rng(deta, ns),
                        rng(dalpha, ns), rng(dbeta, ns), rng(dW0, np), rng(dM0, np),
                        rng(workspace, empty ? 0 : bp.total)};
  constexpr int NO = 9, NI = 13;
  for (int a = 0; a < NO; ++a) {
    for (int b = a + 1; b < NO; ++b)
      if (overlap(outs[a], outs[b])) return E2TTT_EINVAL;
    for (int i = 0; i < NI; ++i)
      if (overlap(outs[a], in[i])) return E2TTT_EINVAL;
  }
  st = device_ok();
  if (st != E2TTT_OK) return st;
  set_lds_attributes();
  (void)hipGetLastError();
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nP = pl.BH * pl.P;
  const unsigned gP = grid1((nP + 255) / 256);
  if (empty) {  // Wend = W0, Mend = M0: the state gradients pass through
    hipLaunchKernelGGL(k_copy_or_zero, dim3(gP), dim3(256), 0, s, dW_end, dW0, nP);
    hipLaunchKernelGGL(k_copy_or_zero, dim3(gP), dim3(256), 0, s, dM_end, dM0, nP);
    return hipGetLastError() == hipSuccess ? E2TTT_OK : E2TTT_EHIP;
  }
  char* ws = static_cast<char*>(workspace);
  auto wsf = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  const Shape sh{pl.BH, pl.L, pl.d, 0, pl.C, pl.Cp, pl.nC, 1};
  const float* Q = static_cast<const float*>(q);
  const float* K = static_cast<const float*>(k);
  const float* V = static_cast<const float*>(v);
  const float* DO = static_cast<const float*>(dout);
  float* dQ = static_cast<float*>(dq);
  float* dK = static_cast<float*>(dk);
  float* dV = static_cast<float*>(dv);
  const int64_t nxe = pl.BH * pl.L * pl.d;
  const unsigned gx = grid1((nxe + 255) / 256);
  if (bp.bf16io) {  // widen the bf16 inputs; the outputs are rounded back at the end
    const bf16_t* src[] = {static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                           static_cast<const bf16_t*>(v), static_cast<const bf16_t*>(dout)};
    const size_t dst[] = {bp.xq, bp.xk, bp.xv, bp.xdo};
    for (int i = 0; i < 4; ++i)
      hipLaunchKernelGGL((k_convert<bf16_t, float>), dim3(gx), dim3(256), 0, s, src[i],
                         wsf(dst[i]), nxe);
    Q = wsf(bp.xq); K = wsf(bp.xk); V = wsf(bp.xv); DO = wsf(bp.xdo);
    dQ = wsf(bp.xdq); dK = wsf(bp.xdk); dV = wsf(bp.xdv);
  }
  float* kw = wsf(pl.kw);
  float* km = wsf(pl.km);
  float* coef = wsf(pl.coef);
  Instr none;
  launch_scan(pl, eta, alpha, beta, kw, km, pl.nC * pl.Cp, pl.Cp, pl.Cp, coef, 4, s, none);
  const float* dWC = dW_end;
  const float* dMC = dM_end;
  const float* W0r = W0;
  const float* M0r = M0;
  float* dW0r = dW0;
  float* dM0r = dM0;
  const float* Wkeep = keep ? W_starts : nullptr;
  const float* Mkeep = keep ? M_starts : nullptr;
  if (bp.mlp) {
    // The MLP learner's states, their adjoints and any kept chunk-start
    // states in the SwiGLU layout with W3 = 0 (absent adjoints as zeros); the
    // kept state of chunk r + 1 goes to slot r + 1 of the re-run's buffers.
    const int64_t nP3 = pl.BH * bp.P;
    const unsigned gx3 = grid1((nP3 / 4 + 255) / 256);
    auto expand = [&](const float* src, float* dst) {
      if (src)
        hipLaunchKernelGGL(k_mlp_state, dim3(gx3), dim3(256), 0, s, src, dst, pl.BH, pl.d, pl.h,
                           1);
      else
        hipLaunchKernelGGL(k_copy_or_zero, dim3(grid1((nP3 + 255) / 256)), dim3(256), 0, s,
                           static_cast<const float*>(nullptr), dst, nP3);
    };
    expand(W0, wsf(bp.w0x));
    expand(M0, wsf(bp.m0x));
    expand(dW_end, wsf(bp.dwb));
    expand(dM_end, wsf(bp.dmb));
    W0r = wsf(bp.w0x);
    M0r = wsf(bp.m0x);
    dWC = wsf(bp.dwb);
    dMC = wsf(bp.dmb);
    dW0r = wsf(bp.dw0x);
    dM0r = wsf(bp.dm0x);
    if (keep) {
      for (int64_t r = 0; r + 1 < pl.nC; ++r) {
        expand(W_starts + r * nP, wsf(bp.wst) + (r + 1) * nP3);
        expand(M_starts + r * nP, wsf(bp.mst) + (r + 1) * nP3);
      }
      Wkeep = wsf(bp.wst) + nP3;
      Mkeep = wsf(bp.mst) + nP3;
    }
  } else if (!dWC || !dMC) {  // absent state gradients: zeros in the first adjoint pair
    hipLaunchKernelGGL(k_copy_or_zero, dim3(gP), dim3(256), 0, s, dW_end, wsf(bp.dwb), nP);
    hipLaunchKernelGGL(k_copy_or_zero, dim3(gP), dim3(256), 0, s, dM_end, wsf(bp.dmb), nP);
    dWC = wsf(bp.dwb);
    dMC = wsf(bp.dmb);
  }
  void (*run)(const BwdPlan&, char*, const float*, const float*, const float*, const float*,
              const float*, const float*, const float*, const float*, float*, float*, float*,
              float*, float*, const float*, const float*, hipStream_t) =
      pl.kind == E2TTT_LINEAR ? linear_backward : swiglu_backward;
  const float* Qraw = Q;
  const float* Kraw = K;
  float* dQout = dQ;
  float* dKout = dK;
  const unsigned gqk = grid1((pl.BH * pl.L + 3) / 4);
  if (bp.qknorm) {  // the prologue as in the forward; its reverse mode after the run
    hipLaunchKernelGGL(k_qk_norm<float>, dim3(gqk), dim3(256), 0, s, Qraw, wsf(bp.nq),
                       pl.BH * pl.L, pl.d);
    hipLaunchKernelGGL(k_qk_norm<float>, dim3(gqk), dim3(256), 0, s, Kraw, wsf(bp.nk),
                       pl.BH * pl.L, pl.d);
    Q = wsf(bp.nq);
    K = wsf(bp.nk);
    dQ = wsf(bp.dnq);
    dK = wsf(bp.dnk);
  }
  run(bp, ws, Q, K, V, W0r, M0r, DO, dWC, dMC, dQ, dK, dV, dW0r, dM0r, Wkeep, Mkeep, s);
  if (bp.mlp) {  // the adjoints of W0, M0 back in the caller's [W1 | W2] layout
    const unsigned gx3 = grid1((pl.BH * bp.P / 4 + 255) / 256);
    hipLaunchKernelGGL(k_mlp_state, dim3(gx3), dim3(256), 0, s,
                       static_cast<const float*>(dW0r), dW0, pl.BH, pl.d, pl.h, 0);
    hipLaunchKernelGGL(k_mlp_state, dim3(gx3), dim3(256), 0, s,
                       static_cast<const float*>(dM0r), dM0, pl.BH, pl.d, pl.h, 0);
  }
  if (bp.qknorm) {
    hipLaunchKernelGGL(k_qk_norm_bwd, dim3(gqk), dim3(256), 0, s, Qraw, dQ, dQout,
                       pl.BH * pl.L, pl.d);
    hipLaunchKernelGGL(k_qk_norm_bwd, dim3(gqk), dim3(256), 0, s, Kraw, dK, dKout,
                       pl.BH * pl.L, pl.d);
    dQ = dQout;
    dK = dKout;
  }
  if (bp.bf16io) {
    bf16_t* dst[] = {static_cast<bf16_t*>(dq), static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv)};
    const float* src[] = {dQ, dK, dV};
    for (int i = 0; i < 3; ++i)
      hipLaunchKernelGGL((k_convert<float, bf16_t>), dim3(gx), dim3(256), 0, s, src[i], dst[i],
                         nxe);
  }
  hipLaunchKernelGGL(k_lin_bwd_scalars, dim3(grid1(pl.BH * pl.nC)), dim3(64), 0, s, sh, pl.mode,
                     eta, alpha, beta, static_cast<const float*>(wsf(bp.sw)),
                     static_cast<const float*>(wsf(bp.sm)), static_cast<const float*>(wsf(bp.dots)),
                     static_cast<int>(bp.nrb), pl.lact ? 2 : pl.averaged,
                     reinterpret_cast<double*>(ws + bp.bcp), deta, dalpha, dbeta);
  return hipGetLastError() == hipSuccess ? E2TTT_OK : E2TTT_EHIP;
}

}  // namespace

e2ttt_status e2ttt_chunk_backward(const e2ttt_problem* prob, const void* q, const void* k,
                                  const void* v, const float* eta, const float* alpha,
                                  const float* beta, const float* W0, const float* M0,
                                  const void* dout, const float* dW_end, const float* dM_end,
                                  void* dq, void* dk, void* dv, float* deta, float* dalpha,
                                  float* dbeta, float* dW0, float* dM0, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return backward_impl(prob, q, k, v, eta, alpha, beta, W0, M0, dout, dW_end, dM_end, nullptr,
                       nullptr, dq, dk, dv, deta, dalpha, dbeta, dW0, dM0, workspace,
                       workspace_bytes, stream);
}

e2ttt_status e2ttt_chunk_backward_states(const e2ttt_problem* prob, const void* q,
                                         const void* k, const void* v, const float* eta,
                                         const float* alpha, const float* beta, const float* W0,
                                         const float* M0, const float* W_starts,
                                         const float* M_starts, const void* dout,
                                         const float* dW_end, const float* dM_end, void* dq,
                                         void* dk, void* dv, float* deta, float* dalpha,
                                         float* dbeta, float* dW0, float* dM0, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  return backward_impl(prob, q, k, v, eta, alpha, beta, W0, M0, dout, dW_end, dM_end, W_starts,
                       M_starts, dq, dk, dv, deta, dalpha, dbeta, dW0, dM0, workspace,
                       workspace_bytes, stream);
}

}  // extern "C"
