// fused_ln_impl.hpp -- residual add + LayerNorm + tanh-GeLU in one pass over
// each row ("算子融合与 Kernel 优化：从 CUDA Graph 到 FlashAttention 的极致性能",
// section 2.3; LayerNorm as in "4、算子融合（Kernel Fusion）", section 4.3):
//
//   v = x + residual;  mean = sum(v) / cols;  var = sum((v - mean)^2) / cols
//   u = (v - mean) / sqrt(var + eps) * gamma + beta;  y = gelu_tanh(u)
//
// The row is loaded once into registers, reduced twice (the mean, then the sum
// of squared deviations from it: the pages' one-pass E[v^2] - mean^2 loses the
// variance when |mean| >> std), normalised and stored once.  Only the inputs
// and the output touch HBM; LDS holds only the per-wave partial sums.
//
// Number types: bf16 I/O computes in fp32 (the statistics included); fp32 I/O
// computes the statistics and the normalisation in binary64 and rounds once to
// fp32 at the store.
//
// Two kernels, chosen by the host from pointer alignment and row length:
//  * ln_vec_kernel: rows start on 16-byte boundaries (x, residual, y, gamma,
//    beta 16-byte aligned and cols a whole number of 16-byte vectors).  gamma
//    and beta are loaded once per block into registers.
//  * ln_shift_kernel: anything else (rows off 16-byte boundaries such as
//    bf16 rows of 4095 elements, any pointer misalignment): the same register
//    layout, filled from and drained to aligned 16-byte windows with lane
//    shifts (details at the kernel).
#pragma once

#include <type_traits>

#include "mbp_internal.hpp"
#include "row_common.hpp"

namespace mbp {
namespace ln {

using namespace rows;

// acc: statistics and normalisation; val: the row values held in registers
// (the exact x + residual: binary64 for fp32 I/O with a residual).
template <class IO, bool RES>
struct Types {
  typedef float acc;
  typedef float val;
};
template <bool RES>
struct Types<F32IO, RES> {
  typedef double acc;
  typedef typename std::conditional<RES, double, float>::type val;
};

template <class IO>
__device__ __forceinline__ u32x4 load_vec(const typename IO::elem* base, int64_t vi) {
  return reinterpret_cast<const u32x4*>(base)[vi];
}
template <class IO>
__device__ __forceinline__ u32x4 stream_vec(const typename IO::elem* base, int64_t vi) {
  return load_nt(reinterpret_cast<const u32x4*>(base) + vi);
}

template <class IO>
__device__ __forceinline__ u32x4 pack_vec(const float* o) {
  u32x4 r;
  if constexpr (IO::kVec == 8) {
#pragma unroll
    for (int w = 0; w < 4; ++w) r.w[w] = pack_bf16x2(o[2 * w], o[2 * w + 1]);
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) r.w[w] = __float_as_uint(o[w]);
  }
  return r;
}

// Place element e of a vector from a scalar (element-wise loads at the edges).
template <class IO>
__device__ __forceinline__ void set_elem(u32x4& v, int e, typename IO::elem val) {
  if constexpr (IO::kVec == 8) {
    const uint32_t h = (uint32_t)val;
    v.w[e >> 1] = (e & 1) ? ((v.w[e >> 1] & 0x0000ffffu) | (h << 16)) : ((v.w[e >> 1] & 0xffff0000u) | h);
  } else {
    v.w[e] = __float_as_uint(val);
  }
}

// Element e of a vector, as stored bits.
template <class IO>
__device__ __forceinline__ typename IO::elem elem_bits(const u32x4& v, int e) {
  if constexpr (IO::kVec == 8) return (typename IO::elem)(v.w[e >> 1] >> (16 * (e & 1)));
  else return __uint_as_float(v.w[e]);
}

// Elements c0 .. c0 + V - 1 of a vector of n elements, zero past n (c0 < n):
// clamped loads that do not depend on each other, so they issue together.
template <class IO>
__device__ __forceinline__ u32x4 partial_vec(const typename IO::elem* p, int c0, int n) {
  typename IO::elem t[IO::kVec];
#pragma unroll
  for (int e = 0; e < IO::kVec; ++e) t[e] = p[min(c0 + e, n - 1)];
  u32x4 r = {{0u, 0u, 0u, 0u}};
#pragma unroll
  for (int e = 0; e < IO::kVec; ++e)
    if (c0 + e < n) set_elem<IO>(r, e, t[e]);
  return r;
}

// normalise, affine, then the epilogue: tanh-GeLU (relu and dropout follow
// at the store, where the element's index is known)
template <class Acc, int EPI>
__device__ __forceinline__ float finish(Acc d, Acc rstd, Acc g, Acc b) {
  const float u = (float)fma_t(d * rstd, g, b);
  if constexpr (EPI == kEpiGelu) return gelu_tanh_f32(u);
  return u;
}

// relu, then dropout, of N outputs with flat indices i0 .. i0 + N - 1, as one
// select: an element survives if it is kept and not below 0 (relu maps u < 0
// to 0, and 0 * scale is 0; -0 and NaN pass through relu unchanged and are
// scaled when kept)
template <int N, bool ALIGNED>
__device__ __forceinline__ void relu_dropout(float* o, uint64_t i0, const Drop& drop) {
  uint32_t h[N];
  dropout_bits<N, ALIGNED>(i0, drop.seed, drop.offset, h);
#pragma unroll
  for (int e = 0; e < N; ++e) o[e] = (h[e] >= drop.thr && !(o[e] < 0.0f)) ? o[e] * drop.scale : 0.0f;
}

// The 16-bit halves o .. o + 7 of the two generator blocks w0 || w1 (o in
// 0 .. 7, uniform over the wave: a scalar branch, then one v_alignbyte_b32
// per output word).
__device__ __forceinline__ void halves_at(const u32x4& w0, const u32x4& w1, int o, uint32_t* h) {
  uint32_t w[8];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    w[t] = w0.w[t];
    w[4 + t] = w1.w[t];
  }
  const int bb = (o & 1) * 2;
  uint32_t r[4];
  switch (o >> 1) {
    case 0:
#pragma unroll
      for (int t = 0; t < 4; ++t) r[t] = __builtin_amdgcn_alignbyte(w[t + 1], w[t], bb);
      break;
    case 1:
#pragma unroll
      for (int t = 0; t < 4; ++t) r[t] = __builtin_amdgcn_alignbyte(w[t + 2], w[t + 1], bb);
      break;
    case 2:
#pragma unroll
      for (int t = 0; t < 4; ++t) r[t] = __builtin_amdgcn_alignbyte(w[t + 3], w[t + 2], bb);
      break;
    default:
#pragma unroll
      for (int t = 0; t < 4; ++t) r[t] = __builtin_amdgcn_alignbyte(w[t + 4], w[t + 3], bb);
      break;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (e & 1) ? (r[e >> 1] >> 16) : (r[e >> 1] & 0xFFFFu);
}

// ------------------------------------------------------------ wide rows

// fp32 rows of more than kRegCols columns: one 1024-lane block per row, three
// passes over it -- the sum, the squared deviations about the mean, the
// output -- the second and third rereading x (and the residual) from the
// caches.  Column c is lane c mod 1024's; any width, alignment and row
// strides.  The statistics are those of the register-resident kernels.
template <class IO, bool RES, int EPI>
__global__ __launch_bounds__(1024) void ln_wide_kernel(
    const typename IO::elem* x, const typename IO::elem* res,
    const typename IO::elem* __restrict__ gamma, const typename IO::elem* __restrict__ beta,
    typename IO::elem* y, int64_t rows, int cols, int64_t ldx, int64_t ldr, int64_t ldy, double eps_d,
    Drop drop) {
  typedef typename Types<IO, RES>::acc Acc;
  typedef typename Types<IO, RES>::val Val;
  constexpr int LANES = 1024;
  __shared__ Acc red[2][LANES / 64];
  const int lane = threadIdx.x;
  const Acc eps = (Acc)eps_d;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const typename IO::elem* xr = x + row * ldx;
    const typename IO::elem* rr = RES ? res + row * ldr : nullptr;
    typename IO::elem* yr = y + row * ldy;
    Acc sum = 0;
#pragma unroll 4
    for (int c = lane; c < cols; c += LANES) {
      Val t = (Val)IO::load1(xr, c);
      if constexpr (RES) t += (Val)IO::load1(rr, c);
      sum += (Acc)t;
    }
    const Acc mean = mean_cols(group_sum<LANES, LANES>(sum, red[0]), cols);
    Acc m2 = 0;
#pragma unroll 4
    for (int c = lane; c < cols; c += LANES) {
      Val t = (Val)IO::load1(xr, c);
      if constexpr (RES) t += (Val)IO::load1(rr, c);
      const Acc d = (Acc)t - mean;
      m2 = fma_t(d, d, m2);
    }
    const Acc rstd = inv_sqrt(div_cols(group_sum<LANES, LANES>(m2, red[1]), cols) + eps);
#pragma unroll 4
    for (int c = lane; c < cols; c += LANES) {
      Val t = (Val)IO::load1(xr, c);
      if constexpr (RES) t += (Val)IO::load1(rr, c);
      float o = finish<Acc, EPI>((Acc)t - mean, rstd, (Acc)IO::load1(gamma, c), (Acc)IO::load1(beta, c));
      if constexpr (EPI == kEpiReluDrop) relu_dropout<1, true>(&o, (uint64_t)row * (uint64_t)cols + (uint64_t)c, drop);
      IO::store1(yr, c, o);
    }
  }
}

// ------------------------------------------------------------ aligned rows

template <class IO, int LANES, int VPL, bool RES, int EPI>
__global__ __launch_bounds__(block_for(LANES)) void ln_vec_kernel(
    const typename IO::elem* x, const typename IO::elem* res,
    const typename IO::elem* __restrict__ gamma, const typename IO::elem* __restrict__ beta,
    typename IO::elem* y, int64_t rows, int cols, int64_t ldx, int64_t ldr, int64_t ldy, double eps_d,
    Drop drop) {
  typedef typename Types<IO, RES>::acc Acc;
  typedef typename Types<IO, RES>::val Val;
  constexpr int V = IO::kVec;
  constexpr int BLOCK = block_for(LANES);
  constexpr int RPB = BLOCK / LANES;
  constexpr bool kInPlace = std::is_same<Acc, Val>::value;
  __shared__ Acc red[2][BLOCK / 64];

  const int lane = threadIdx.x % LANES;
  const int sub = threadIdx.x / LANES;
  const int nvec = cols / V;
  const Acc eps = (Acc)eps_d;

  // gamma / beta of this lane's columns.  Wide bf16 rows keep them packed
  // (widened at each use, one shift or mask per element): measured faster on
  // the 8192- and 12288-wide rows than holding 2 * VPL * 8 fp32 registers.
  constexpr bool kPacked = sizeof(typename IO::elem) == 2 && LANES >= 128 && VPL >= 3;
  float g[VPL][V], b[VPL][V];
  u32x4 gp[VPL], bp[VPL];
  // Loads of slots past the row: zero-filled behind a branch, or (kClamp) a
  // branch-free reread of the last vector (never used).  The two compile to
  // differently scheduled code: the branch-free form measured 2.8-3.7% faster
  // on 256-lane rows with the GeLU epilogue (16384 x 8192), and 1-2.5% slower
  // on 512-lane rows and 4-5% slower with the dropout epilogue, so each
  // layout keeps its faster form.
  constexpr bool kClamp = LANES == 256 && EPI == kEpiGelu;
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int vi = lane + k * LANES;
    u32x4 gv = {{0u, 0u, 0u, 0u}}, bv = {{0u, 0u, 0u, 0u}};
    if constexpr (kClamp) {
      gv = load_vec<IO>(gamma, min(vi, nvec - 1));
      bv = load_vec<IO>(beta, min(vi, nvec - 1));
    } else if (vi < nvec) {
      gv = load_vec<IO>(gamma, vi);
      bv = load_vec<IO>(beta, vi);
    }
    gp[k] = gv;
    bp[k] = bv;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      g[k][e] = IO::get(gv, e);
      b[k][e] = IO::get(bv, e);
    }
  }

  const int64_t groups = (rows + RPB - 1) / RPB;
  // The loads of a row group: a group past the last row reads the last row
  // (and stores nothing); a slot past the row's last vector reads that vector
  // and is left out of the sums.  Every load is in bounds and none needs a
  // branch or a zero fill.
  auto issue_loads = [&](int64_t gi, u32x4* xo, u32x4* ro) {
    const int64_t r = gi * RPB + sub;
    const int64_t lr = r < rows ? r : rows - 1;
    const typename IO::elem* xr = x + lr * ldx;
    const typename IO::elem* rr = RES ? res + lr * ldr : nullptr;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int vi = min(lane + k * LANES, nvec - 1);
      xo[k] = stream_vec<IO>(xr, vi);
      if constexpr (RES) ro[k] = stream_vec<IO>(rr, vi);
    }
  };
  // 16-bit rows in groups of up to 256 lanes: the first row group's loads
  // are issued before the wait for gamma/beta, and each next group's before
  // the current one is computed; so do plain fp32 LayerNorm rows in 256 x 4,
  // which the host runs as a persistent loop (below: 100 -> 114 registers,
  // still four waves per SIMD).  Other fp32 rows issue a group's loads at the
  // top of its iteration: holding a second fp32 row cost an occupancy step
  // (8192 x 8192 fp32 + residual + GeLU: 104 -> 136 registers, 135 -> 164 us);
  // so did 512-lane 16-bit groups (16384 x 12288 + GeLU: 193.3 -> 199.1 us).
  constexpr bool kAhead = (sizeof(typename IO::elem) == 2 && LANES <= 256) ||
                          (sizeof(typename IO::elem) == 4 && !RES && EPI == kEpiNone && LANES == 256 && VPL == 4);
  u32x4 xv[VPL], rv[VPL];
  if constexpr (kAhead) {
    if ((int64_t)blockIdx.x < groups) issue_loads(blockIdx.x, xv, rv);
  }
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
    u32x4 xn[VPL], rn[VPL];
    const bool more = kAhead && grp + gridDim.x < groups;
    if (more) issue_loads(grp + gridDim.x, xn, rn);
    if constexpr (kPacked) {
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        opaque(gp[k]);
        opaque(bp[k]);
      }
    }
    if constexpr (sizeof(Acc) == 8) {
      // fp32 gamma/beta are widened to binary64 at each use; without this the
      // compiler would widen them once and hold twice the registers.
#pragma unroll
      for (int k = 0; k < VPL; ++k)
#pragma unroll
        for (int e = 0; e < V; ++e) {
          opaque(g[k][e]);
          opaque(b[k][e]);
        }
    }
    const int64_t row = grp * RPB + sub;
    const bool live = row < rows;
    typename IO::elem* yr = y + row * ldy;
    if constexpr (!kAhead) issue_loads(grp, xv, rv);
    Val v[VPL][V];
    Acc sum = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      Acc part = 0;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        Val t = (Val)IO::get(xv[k], e);
        if constexpr (RES) t += (Val)IO::get(rv[k], e);
        v[k][e] = t;
        part += (Acc)t;
      }
      if (lane + k * LANES < nvec) sum += part;
    }
    const Acc mean = mean_cols(group_sum<LANES, BLOCK>(sum, red[0]), cols);

    Acc m2 = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      Acc part = 0;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const Acc d = (Acc)v[k][e] - mean;
        if constexpr (kInPlace) v[k][e] = d;
        part = fma_t(d, d, part);
      }
      if (lane + k * LANES < nvec) m2 += part;
    }
    const Acc rstd = inv_sqrt(div_cols(group_sum<LANES, BLOCK>(m2, red[1]), cols) + eps);

#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int vi = lane + k * LANES;
      if (!(live && vi < nvec)) continue;
      float o[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const Acc d = kInPlace ? (Acc)v[k][e] : (Acc)v[k][e] - mean;
        if constexpr (kPacked)
          o[e] = finish<Acc, EPI>(d, rstd, (Acc)IO::get(gp[k], e), (Acc)IO::get(bp[k], e));
        else
          o[e] = finish<Acc, EPI>(d, rstd, (Acc)g[k][e], (Acc)b[k][e]);
      }
      if constexpr (EPI == kEpiReluDrop)  // rows start on multiples of V: one aligned group
        relu_dropout<V, true>(o, (uint64_t)row * (uint64_t)cols + (uint64_t)(vi * V), drop);
      store_nt(reinterpret_cast<u32x4*>(yr) + vi, pack_vec<IO>(o));
    }
    if (more) {
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        xv[k] = xn[k];
        if constexpr (RES) rv[k] = rn[k];
      }
    }
  }
}

// ------------------------------------------------------------ 16-byte windows

// Geometry of one tensor's window space.  The base is derived from the
// tensor pointer by pointer arithmetic (never through an integer), so the
// compiler keeps it in the global address space and emits global (not flat)
// memory instructions, whose completion does not hold up LDS waits.
struct Win {
  const char* base;  // 16-byte boundary at or below the tensor pointer
  int mb;            // tensor pointer - base (bytes)
  int64_t end;       // one past the tensor's last byte, relative to base
};

template <class IO>
__device__ __forceinline__ Win make_win(const void* p, int64_t total) {
  Win w;
  w.mb = (int)(reinterpret_cast<uintptr_t>(p) & 15);
  w.base = static_cast<const char*>(p) - w.mb;
  w.end = w.mb + (int64_t)sizeof(typename IO::elem) * total;
  return w;
}

// DPP lane moves inside a wave (lane l of the result):
//   shl1: lane l+1 of v (lane 63 keeps old);  rol1: lane (l+1) mod 64 of v;
//   shr1: lane l-1 of v (lane 0 keeps old);   ror1: lane (l-1) mod 64 of v.
__device__ __forceinline__ uint32_t dpp_shl1(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, 0x130, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t dpp_rol1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x134, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t dpp_shr1(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, 0x138, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t dpp_ror1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x13C, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t lane_read(uint32_t v, int src_lane) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane << 2, (int)v);
}

// Word t of the slot after this one (next) or before it (prev), given the
// slot's round-k value c and the value a of the adjacent round (k+1 for next,
// k-1 for prev).
template <int LANES>
__device__ __forceinline__ uint32_t next_word(uint32_t c, uint32_t a) {
  if constexpr (LANES >= 64) {
    return dpp_shl1(dpp_rol1(a), c);
  } else {
    const int wl = threadIdx.x & 63;
    const uint32_t far = lane_read(a, wl & ~(LANES - 1));  // the group's lane 0
    const uint32_t near = dpp_shl1(0u, c);
    return ((wl & (LANES - 1)) == LANES - 1) ? far : near;
  }
}
template <int LANES>
__device__ __forceinline__ uint32_t prev_word(uint32_t c, uint32_t a) {
  if constexpr (LANES >= 64) {
    return dpp_shr1(dpp_ror1(a), c);
  } else {
    const int wl = threadIdx.x & 63;
    const uint32_t far = lane_read(a, wl | (LANES - 1));  // the group's last lane
    const uint32_t near = dpp_shr1(0u, c);
    return ((wl & (LANES - 1)) == 0) ? far : near;
  }
}

// Bytes [4Q + bb, 4Q + bb + 16) of the 32 bytes lo || hi (bb = 0 or 2).
template <int ES, int Q>
__device__ __forceinline__ u32x4 funnel(const u32x4& lo, const uint32_t* hi, int bb) {
  uint32_t w[8];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    w[t] = lo.w[t];
    w[4 + t] = hi[t];
  }
  u32x4 r;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if constexpr (ES == 4) r.w[t] = w[Q + t];
    else r.w[t] = __builtin_amdgcn_alignbyte(w[Q + t + 1], w[Q + t], bb);
  }
  return r;
}

// ------------------------------------------------------------ rows congruent modulo 16 bytes

// Rows off 16-byte boundaries whose x, residual and y share one alignment
// (the usual case: e.g. bf16 rows of 4095 elements in freshly allocated
// tensors, or rows of one padded buffer: the three share one row stride).
// The byte offset of row r in its line, (base + r * pitch) mod line (pitch:
// the row stride in bytes), with line = 128 bytes when the three tensors agree
// modulo 128 (else 16), repeats with period P = line / gcd(line, pitch) rows;
// the rows with one offset form a class.  A block serves one class, so the offset is
// uniform over the block: d whole windows and s elements past the line.  The
// row is processed directly in window space: relative slot j holds window j of
// the row, element e of it being column V*j + e - s, and relative slot j sits
// at slot (j + d) mod nvec of the ln_vec_kernel layout, so every load and
// store instruction covers whole 128-byte lines (runs that straddle lines cost
// 10% of the bandwidth).  gamma and beta are laid out once per block to
// match (an LDS ring for layouts up to 2048 slots, registers beyond).
//
// A row spans nvec = ceil(cols / V) windows, or one more when its offset
// pushes its tail into window nvec.  In that case the tail (fewer than s
// elements) is moved into the unused head of relative slot 0 (whose first s
// elements belong to the previous row), so VPL is the same as for aligned
// rows.  Only relative slots 0 and nvec - 1 hold elements outside the row:
// they are zeroed in the packed inputs, their deviations are set to 0 before
// the variance sum, and their windows (and the folded one) are stored element
// by element.
//
// The host passes [r_lo, r_hi), the rows whose windows lie inside the
// tensors; the rest (at most the first and last few rows: rows starting
// within 16 bytes of a tensor's unaligned start or end) take the last
// `edge_blocks` blocks of the grid, which handle them element by element.
// Layouts of up to 2048 slots keep gamma / beta in LDS (at most 64 KB per
// block), which leaves the 16-bit row loop of up to 4 vectors per lane within
// 128 registers: four waves per SIMD (not with the dropout epilogue, whose
// generator blocks take more LDS).
constexpr bool class_raw_gb(int lanes, int vpl) { return lanes * vpl <= 2048; }
constexpr int class_min_waves(int lanes, int vpl, int es, int epi) {
  return es == 2 && vpl <= 4 && epi != kEpiReluDrop && class_raw_gb(lanes, vpl) ? 4 : 1;
}

template <class IO, int LANES, int VPL, bool RES, int EPI>
__global__ __launch_bounds__(block_for(LANES)) __attribute__((amdgpu_waves_per_eu(class_min_waves(LANES, VPL, (int)sizeof(typename IO::elem), EPI)))) void ln_class_kernel(
    const typename IO::elem* x, const typename IO::elem* res,
    const typename IO::elem* __restrict__ gamma, const typename IO::elem* __restrict__ beta,
    typename IO::elem* y, int64_t rows, int cols, int64_t ld, double eps_d, int period, int line,
    int64_t r_lo, int64_t r_hi, int edge_blocks, Drop drop) {
  typedef typename IO::elem E;
  typedef typename Types<IO, RES>::acc Acc;
  typedef typename Types<IO, RES>::val Val;
  constexpr int ES = (int)sizeof(E);
  constexpr int V = IO::kVec;
  constexpr int BLOCK = block_for(LANES);
  constexpr int RPB = BLOCK / LANES;
  constexpr bool kInPlace = std::is_same<Acc, Val>::value;
  constexpr bool kRaw = class_raw_gb(LANES, VPL);
  // Dropout: a row's elements lie off the generator's 8-element blocks, so
  // each slot straddles two blocks.  Where LDS allows, every block of the row
  // is computed once, by one lane, into LDS (two buffers, alternating by row
  // group, so a wave may run ahead by one row; one buffer and a barrier before
  // each refill where two do not fit) and each slot reads its two; otherwise
  // each slot computes both.
  constexpr int kPB = (LANES * VPL * V) / 8 + 2;  // blocks of a row, at most
  constexpr bool kDrop = EPI == kEpiReluDrop;
  constexpr int kRingB = kRaw ? 2 * LANES * VPL * 16 : 0;
  // two buffers where they fit, else one (and a barrier before each refill)
  constexpr int kPhBuf = !kDrop ? 0 : 2 * RPB * kPB * 16 + kRingB <= 60 * 1024 ? 2
                                    : RPB * kPB * 16 + kRingB <= 60 * 1024       ? 1
                                                                                 : 0;
  constexpr bool kPhLds = kPhBuf > 0;
  __shared__ Acc red[2][BLOCK / 64];

  const int lane = threadIdx.x % LANES;
  const int sub = threadIdx.x / LANES;
  const Acc eps = (Acc)eps_d;

  const int nb = (int)gridDim.x - edge_blocks;  // class blocks
  if ((int)blockIdx.x >= nb) {
    // edge rows: lane l takes columns l, l + LANES, ...; three passes over
    // the row (sum, squared deviations, output), the later ones from cache
    const int64_t i = (int64_t)((int)blockIdx.x - nb) * RPB + sub;
    const int64_t n_edge = r_lo + (rows - r_hi);
    const bool live = i < n_edge;
    const int64_t row = !live ? 0 : (i < r_lo ? i : r_hi + (i - r_lo));
    const int64_t e0 = row * ld;  // the row in memory (x, residual and y share the row stride)
    auto val = [&](int c) -> Val {
      Val t = (Val)IO::load1(x, e0 + c);
      if constexpr (RES) t += (Val)IO::load1(res, e0 + c);
      return t;
    };
    Acc sum = 0;
    for (int c = lane; c < cols; c += LANES) sum += (Acc)val(c);
    const Acc mean = mean_cols(group_sum<LANES, BLOCK>(sum, red[0]), cols);
    Acc m2 = 0;
    for (int c = lane; c < cols; c += LANES) {
      const Acc d = (Acc)val(c) - mean;
      m2 = fma_t(d, d, m2);
    }
    const Acc rstd = inv_sqrt(div_cols(group_sum<LANES, BLOCK>(m2, red[1]), cols) + eps);
    if (live)
      for (int c = lane; c < cols; c += LANES) {
        float o = finish<Acc, EPI>((Acc)val(c) - mean, rstd, (Acc)IO::load1(gamma, c), (Acc)IO::load1(beta, c));
        if constexpr (EPI == kEpiReluDrop) relu_dropout<1, true>(&o, (uint64_t)(row * cols + c), drop);
        IO::store1(y, e0 + c, o);
      }
    return;
  }

  // period: a power of two (1 .. 16)
  const int lp = __builtin_ctz((unsigned)period);
  // Consecutive blocks take the classes of consecutive rows, so the whole
  // grid sweeps the tensors front to back together (measured faster than
  // giving each XCD a contiguous run of rows).
  const int bid = (int)blockIdx.x;
  const int cls = bid & (period - 1);
  const int64_t blk = bid >> lp;
  const int64_t nblk = nb >> lp;
  const int64_t first = r_lo + cls;  // first row of the class
  if (first >= r_hi) return;         // an empty class: the whole block leaves
  const int64_t crows = ((r_hi - 1 - first) >> lp) + 1;
  const int64_t cgroups = (crows + RPB - 1) / RPB;
  const int64_t last_row = first + ((crows - 1) << lp);

  const int mb = (int)(reinterpret_cast<uintptr_t>(x) & 15);
  // the class's byte offset in its line (line = 128 or 16 bytes): window
  // offset d, byte offset sb in that window
  const int sl = (int)((reinterpret_cast<uintptr_t>(x) + (uint64_t)((int64_t)ES * first * ld)) & (unsigned)(line - 1));
  const int d = sl >> 4;
  const int sb = sl & 15;
  const int s = sb / ES;
  const int nvec = (cols + V - 1) / V;
  // Slot p = lane + k*LANES holds window rel(p) = (p - d) mod nvec of the
  // row, so the run of slots a load or store instruction covers starts on a
  // line: relative slot 0 sits at slot d and the last d windows wrap round to
  // slots 0 .. d-1 (the host ensures d < min(nvec, LANES)).  Slots p >= nvec
  // are unused and clamped.
  auto rel = [&](int k) -> int {
    const int p = min(lane + k * LANES, nvec - 1);
    return p < d ? p - d + nvec : p - d;
  };
  const int nv = (sb + ES * cols + 15) >> 4;
  const bool fold = nv > nvec;
  const int klast = (nvec - 1) / LANES;

  // column of element e of slot j (-1: outside the row)
  auto col_of = [&](int j, int e) -> int {
    if (j == 0 && e < s) return fold ? V * nvec + e - s : -1;
    return V * j + e - s;
  };
  // Elements of slot 0 and slot nvec - 1 inside the row (bit e): slot 0
  // holds columns e - s for e in [s, min(V, s + cols)) and, folded, the tail
  // columns for e < cols - (V*nvec - s); slot nvec - 1 (when not slot 0)
  // columns up to cols - 1, i.e. e < cols - V*(nvec - 1) + s.
  auto low = [](int n) -> uint32_t { return n <= 0 ? 0u : (1u << n) - 1u; };
  const uint32_t in0 = (low(min(V, s + cols)) & ~low(s)) | (fold ? low(cols - (V * nvec - s)) : 0u);
  const uint32_t inl = nvec == 1 ? in0 : low(min(V, cols - V * (nvec - 1) + s));
  // the same as masks of the packed words (all ones: inside)
  uint32_t mk0[4], mkl[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if constexpr (ES == 2) {
      mk0[t] = (((in0 >> (2 * t)) & 1u) ? 0xffffu : 0u) | (((in0 >> (2 * t + 1)) & 1u) ? 0xffff0000u : 0u);
      mkl[t] = (((inl >> (2 * t)) & 1u) ? 0xffffu : 0u) | (((inl >> (2 * t + 1)) & 1u) ? 0xffff0000u : 0u);
    } else {
      mk0[t] = ((in0 >> t) & 1u) ? 0xffffffffu : 0u;
      mkl[t] = ((inl >> t) & 1u) ? 0xffffffffu : 0u;
    }
  }

  // gamma / beta in the class's window layout: relative slot j holds columns
  // V*j - s + e, i.e. bytes [16 - sb, 32 - sb) of vectors j-1 || j; slot 0
  // takes vector nvec - 1 as its "j-1", which yields exactly the folded tail
  // columns V*nvec - s + e, e < s.  A partial last vector is read element by
  // element (zero past the end, no byte past gamma or beta).
  //
  // Layouts of up to 2048 slots (kRaw) keep gamma and beta in an LDS ring of
  // nvec vectors: ring vector j is relative slot j's vector, funnelled from
  // vectors j-1 and j, so each slot reads its gamma / beta aligned in the row
  // loop.  One thread builds each ring vector (consecutive lanes, consecutive
  // 16 bytes: no bank conflicts), then one barrier.  Wider layouts funnel
  // once per block into registers.
  const bool gb_aligned = ((reinterpret_cast<uintptr_t>(gamma) | reinterpret_cast<uintptr_t>(beta)) & 15) == 0;
  const bool partial = (cols % V) != 0;
  const int jfull = partial ? nvec - 2 : nvec - 1;  // last whole vector (-1: none)
  const int q = ((16 - sb) & 15) >> 2, bb = (16 - sb) & 3;
  __shared__ u32x4 ringg[kRaw ? LANES * VPL : 1], ringb[kRaw ? LANES * VPL : 1];
  u32x4 gp[kRaw ? 1 : VPL], bp[kRaw ? 1 : VPL];
  if constexpr (kRaw) {
    constexpr int kIt = (LANES * VPL + BLOCK - 1) / BLOCK;
    auto fetch = [&](int vi, u32x4& g, u32x4& b) {
      if (gb_aligned && vi <= jfull) {
        g = load_vec<IO>(gamma, vi);
        b = load_vec<IO>(beta, vi);
      } else {  // the partial last vector, or gamma / beta off 16-byte boundaries
        g = partial_vec<IO>(gamma, V * vi, cols);
        b = partial_vec<IO>(beta, V * vi, cols);
      }
    };
    // every gamma / beta vector is read from global memory once: the raw
    // vectors go to the ring first, each slot takes its predecessor from
    // there, and the funnelled vectors replace them
    u32x4 tg[kIt], tb[kIt];
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int jc = min((int)threadIdx.x + i * BLOCK, nvec - 1);
      fetch(jc, tg[i], tb[i]);
    }
    if (sb != 0) {
#pragma unroll
      for (int i = 0; i < kIt; ++i) {
        const int v = (int)threadIdx.x + i * BLOCK;
        if (v < nvec) {
          ringg[v] = tg[i];
          ringb[v] = tb[i];
        }
      }
      lds_barrier();
      u32x4 ga[kIt], ba[kIt];
#pragma unroll
      for (int i = 0; i < kIt; ++i) {
        const int jc = min((int)threadIdx.x + i * BLOCK, nvec - 1);
        const int jp = jc == 0 ? nvec - 1 : jc - 1;
        ga[i] = ringg[jp];
        ba[i] = ringb[jp];
      }
      lds_barrier();
#pragma unroll
      for (int i = 0; i < kIt; ++i) {
        const u32x4 gc = tg[i], bc = tb[i];
        switch (q) {
          case 0: tg[i] = funnel<ES, 0>(ga[i], gc.w, bb); tb[i] = funnel<ES, 0>(ba[i], bc.w, bb); break;
          case 1: tg[i] = funnel<ES, 1>(ga[i], gc.w, bb); tb[i] = funnel<ES, 1>(ba[i], bc.w, bb); break;
          case 2: tg[i] = funnel<ES, 2>(ga[i], gc.w, bb); tb[i] = funnel<ES, 2>(ba[i], bc.w, bb); break;
          default: tg[i] = funnel<ES, 3>(ga[i], gc.w, bb); tb[i] = funnel<ES, 3>(ba[i], bc.w, bb); break;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int v = (int)threadIdx.x + i * BLOCK;
      if (v < nvec) {
        ringg[v] = tg[i];
        ringb[v] = tb[i];
      }
    }
    lds_barrier();
  } else if (gb_aligned) {
    u32x4 pg = {{0u, 0u, 0u, 0u}}, pb = {{0u, 0u, 0u, 0u}};
    if (partial) {
      pg = partial_vec<IO>(gamma, V * (nvec - 1), cols);
      pb = partial_vec<IO>(beta, V * (nvec - 1), cols);
    }
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int jc = rel(k);
      const int jp = jc == 0 ? nvec - 1 : jc - 1;
      u32x4 ga = pg, gb = pg, ba = pb, bv = pb;
      if (jfull >= 0) {
        ga = load_vec<IO>(gamma, min(jp, jfull));
        gb = load_vec<IO>(gamma, min(jc, jfull));
        ba = load_vec<IO>(beta, min(jp, jfull));
        bv = load_vec<IO>(beta, min(jc, jfull));
        if (k == 0 || k == klast) {  // the partial vector appears only in these rounds
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if (jp > jfull) { ga.w[t] = pg.w[t]; ba.w[t] = pb.w[t]; }
            if (jc > jfull) { gb.w[t] = pg.w[t]; bv.w[t] = pb.w[t]; }
          }
        }
      }
      switch (sb == 0 ? -1 : q) {
        case -1: gp[k] = gb; bp[k] = bv; break;
        case 0: gp[k] = funnel<ES, 0>(ga, gb.w, bb); bp[k] = funnel<ES, 0>(ba, bv.w, bb); break;
        case 1: gp[k] = funnel<ES, 1>(ga, gb.w, bb); bp[k] = funnel<ES, 1>(ba, bv.w, bb); break;
        case 2: gp[k] = funnel<ES, 2>(ga, gb.w, bb); bp[k] = funnel<ES, 2>(ba, bv.w, bb); break;
        default: gp[k] = funnel<ES, 3>(ga, gb.w, bb); bp[k] = funnel<ES, 3>(ba, bv.w, bb); break;
      }
    }
  } else {
    // element gather; clamped unconditional loads, so they issue together
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int j = rel(k);
      u32x4 gv = {{0u, 0u, 0u, 0u}}, bv = {{0u, 0u, 0u, 0u}};
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int c = col_of(j, e);
        const int cc = min(max(c, 0), cols - 1);
        const E ge = gamma[cc], be = beta[cc];
        if (c >= 0 && c < cols) {
          set_elem<IO>(gv, e, ge);
          set_elem<IO>(bv, e, be);
        }
      }
      gp[k] = gv;
      bp[k] = bv;
    }
  }

  int jr[VPL];
  bool used[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    jr[k] = rel(k);
    used[k] = lane + k * LANES < nvec;
  }

  __shared__ u32x4 pblk[kPhLds ? kPhBuf * RPB * kPB : 1];
  int parity = 0;
  for (int64_t grp = blk; grp < cgroups; grp += nblk, parity ^= 1) {
    if constexpr (!kRaw) {
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        opaque(gp[k]);
        opaque(bp[k]);
      }
    }
    const int64_t row = first + (int64_t)period * (grp * RPB + sub);
    const bool live = row <= last_row;
    const int64_t e0 = (live ? row : last_row) * ld;  // memory offset of the row
    const int64_t q0 = (mb + (int64_t)ES * e0) >> 4;

    // every window of the row lies inside the tensors (rows in [r_lo, r_hi))
    const u32x4* sx = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(x) - mb) + q0;
    const u32x4* sr = RES ? reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(res) - mb) + q0
                          : nullptr;
    u32x4 xw[VPL], rw[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      xw[k] = load_nt(sx + jr[k]);
      if constexpr (RES) rw[k] = load_nt(sr + jr[k]);
    }
    if (fold && lane == d) {  // relative slot 0 takes the row's last window into its bytes [0, sb)
      int sbv = sb;
      opaque(sbv);
      const u32x4 xf = load_nt(sx + nvec);
      u32x4 rf = {{0u, 0u, 0u, 0u}};
      if constexpr (RES) rf = load_nt(sr + nvec);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int sh = min(max(sbv - 4 * t, 0), 4);  // bytes of word t taken from the tail
        const uint32_t keep = sh == 4 ? 0u : 0xffffffffu << (8 * sh);
        xw[0].w[t] = (xw[0].w[t] & keep) | (xf.w[t] & ~keep);
        if constexpr (RES) rw[0].w[t] = (rw[0].w[t] & keep) | (rf.w[t] & ~keep);
      }
    }
    // dropout: the row's generator blocks bfirst .. bfirst + nb_row - 1,
    // each computed once into this group's buffer (while the loads are in
    // flight)
    uint64_t rc = 0, bfirst = 0;
    int nb_row = 0;
    if constexpr (kDrop) {
      rc = (uint64_t)(live ? row : last_row) * (uint64_t)cols;
      bfirst = rc >> 3;
      nb_row = (int)(((rc + (uint64_t)cols - 1) >> 3) - bfirst) + 1;
      if constexpr (kPhLds) {
        if constexpr (kPhBuf == 1) {
          if (grp != blk) lds_barrier();  // every lane has read the previous row's blocks
        }
        u32x4* pb = pblk + ((kPhBuf == 2 ? parity : 0) * RPB + sub) * kPB;
        for (int i = lane; i < nb_row; i += LANES) {
          uint32_t w[4];
          philox4x32_10(bfirst + (uint64_t)i, drop.seed, drop.offset, w);
          pb[i] = u32x4{{w[0], w[1], w[2], w[3]}};
        }
      }
    }
    // zero the elements outside the row (slot 0 and slot nvec - 1 only)
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      if (k != 0 && k != klast) continue;  // relative slots 0 and nvec - 1 sit in these rounds
      const int j = jr[k];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t m = (j == 0 ? mk0[t] : 0xffffffffu) & (j == nvec - 1 ? mkl[t] : 0xffffffffu);
        xw[k].w[t] &= m;
        if constexpr (RES) rw[k].w[t] &= m;
      }
    }

    Val v[VPL][V];
    Acc sum = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      Acc part = 0;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        Val t = (Val)IO::get(xw[k], e);
        if constexpr (RES) t += (Val)IO::get(rw[k], e);
        v[k][e] = t;
        part += (Acc)t;
      }
      if (used[k]) sum += part;
    }
    const Acc mean = mean_cols(group_sum<LANES, BLOCK>(sum, red[0]), cols);

    Acc m2 = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int j = jr[k];
      Acc dv[V];
#pragma unroll
      for (int e = 0; e < V; ++e) dv[e] = (Acc)v[k][e] - mean;
      // elements outside the row (relative slots 0 and nvec - 1, which sit in
      // rounds 0 and klast) add nothing to the centred sum of squares: their
      // deviation is set to 0 rather than (0 - mean)^2 taken out again, which
      // in fp32 would cancel badly for rows far from 0.  Only the one or two
      // lanes holding those slots need it: with fp32 statistics a wave-uniform
      // branch skips the selects in every other wave (16384 x 4095 bf16: -0.9%,
      // with dropout at 8191: -5.2%); with binary64 statistics the selects cost
      // nothing measurable and the branch cost 17% (8192 x 4093 fp32).
      if (k == 0 || k == klast) {
        const uint32_t inb = (j == 0 ? in0 : ~0u) & (j == nvec - 1 ? inl : ~0u);
        if (sizeof(Acc) == 8 || __builtin_amdgcn_ballot_w64(inb != ~0u) != 0) {
#pragma unroll
          for (int e = 0; e < V; ++e) dv[e] = ((inb >> e) & 1u) ? dv[e] : (Acc)0;
        }
      }
      Acc part = 0;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if constexpr (kInPlace) v[k][e] = dv[e];
        part = fma_t(dv[e], dv[e], part);
      }
      if (used[k]) m2 += part;
    }
    const Acc rstd = inv_sqrt(div_cols(group_sum<LANES, BLOCK>(m2, red[1]), cols) + eps);
    if constexpr (kPhLds) lds_barrier();  // the generator blocks are in LDS

    if (!live) continue;
    u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<char*>(y) - mb) + q0;
    E* yrow = y + row * ld;
    // fp32: element stores of the windows shared with a neighbouring row go
    // through a volatile pointer; otherwise the compiler sinks the last one
    // into a common tail with the whole-window store, which then splits into
    // dwordx3 + dword (8192 x 4093: 72.0 against 58.9 us).  The 16-bit forms
    // keep plain stores (volatile ones cost them 12-36%).
    typedef typename std::conditional<ES == 4, volatile E, E>::type VE;
    VE* vrow = yrow;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int j = jr[k];
      if (!used[k]) continue;
      float o[V];
      u32x4 gk, bk;
      if constexpr (kRaw) {
        gk = ringg[j];
        bk = ringb[j];
      } else {
        gk = gp[k];
        bk = bp[k];
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const Acc dv = kInPlace ? (Acc)v[k][e] : (Acc)v[k][e] - mean;
        o[e] = finish<Acc, EPI>(dv, rstd, (Acc)IO::get(gk, e), (Acc)IO::get(bk, e));
      }
      if constexpr (kDrop) {
        // element e of relative slot j has flat index rc + V*j - s + e; the
        // folded tail of relative slot 0 (e < s) has rc + V*nvec - s + e
        uint32_t h[8];
        auto bits = [&](uint64_t i0, uint32_t* hh) {
          if constexpr (kPhLds) {
            const u32x4* pb = pblk + ((kPhBuf == 2 ? parity : 0) * RPB + sub) * kPB;
            const int64_t b = (int64_t)((i0 >> 3) - bfirst);  // -1: the previous row's block
            const u32x4 w0 = pb[min(max(b, (int64_t)0), (int64_t)nb_row - 1)];
            const u32x4 w1 = pb[min(max(b + 1, (int64_t)0), (int64_t)nb_row - 1)];
            int o8 = (int)(i0 & 7);
            // one row per wave and V*j a multiple of 8: the same for the whole wave
            if constexpr (LANES >= 64 && V == 8) o8 = __builtin_amdgcn_readfirstlane(o8);
            halves_at(w0, w1, o8, hh);
          } else {
            dropout_bits<V, false>(i0, drop.seed, drop.offset, hh);
          }
        };
        bits(rc + (uint64_t)(V * j) - (uint64_t)s, h);
        if (fold && j == 0) {
          uint32_t ht[8];
          bits(rc + (uint64_t)(V * nvec) - (uint64_t)s, ht);
#pragma unroll
          for (int e = 0; e < V; ++e)
            if (e < s) h[e] = ht[e];
        }
#pragma unroll
        for (int e = 0; e < V; ++e) o[e] = (h[e] >= drop.thr && !(o[e] < 0.0f)) ? o[e] * drop.scale : 0.0f;
      }
      const u32x4 ov = pack_vec<IO>(o);
      // window j holds columns V*j - s + e; slot 0 and slot nvec - 1 may
      // share their window with a neighbouring row: store only [ea, eb)
      int ea = j == 0 ? s : 0;
      int eb = min(V, cols - (V * j - s));
      if (ea == 0 && eb == V) {
        store_nt(dst + j, ov);
      } else {
        opaque(ea);  // keep the per-element tests in this branch
        opaque(eb);
#pragma unroll
        for (int e = 0; e < V; ++e)
          if (e >= ea && e < eb) vrow[V * j - s + e] = elem_bits<IO>(ov, e);
        if (fold && j == 0) {  // the folded tail: columns V*nvec - s + e
          int fb = cols - (V * nvec - s);
          opaque(fb);
#pragma unroll
          for (int e = 0; e < V; ++e)
            if (e < fb) vrow[V * nvec - s + e] = elem_bits<IO>(ov, e);
        }
      }
    }
  }
}

// ------------------------------------------------------------ rows off 16-byte boundaries

// Rows that do not start on 16-byte boundaries (e.g. bf16 rows of 4095
// elements, 8190 bytes), with any misalignment of x, residual, y, gamma and
// beta.  The register layout and the arithmetic are those of ln_vec_kernel;
// only the way vectors reach and leave the registers differs.
//
// Window space: window q of a tensor is bytes [16q, 16q + 16) above the
// 16-byte boundary at or below its base pointer.  Loads: the row vector in
// slot j (row bytes [16j, 16j + 16)) is the byte funnel of windows j and j+1
// of the row at the row's byte offset in its first window.  Every slot loads
// its window j; window j+1 is the window of the neighbouring slot, fetched
// with a DPP lane shift, except for the one slot per wave (or row group)
// whose neighbour sits in another wave, which loads it itself.  Stores: output
// window j is the funnel of output vectors j-1 and j at the output row's
// offset; vector j-1 comes from the neighbouring lane the same way, and the
// two windows per wave whose halves sit in different waves are written half
// by half with element stores.  Windows shared with the neighbouring rows (the
// first and last of a row) are written element by element, so no byte of
// another row is written.  A row whose first or last window reaches outside a
// tensor (only the tensor's first and last row can) is read element by
// element, so no byte outside the tensors is read.
//
// Slots: for groups of at least a wave, wave w of the group holds the slots
// w*64*VPL + k*64 + l (round k, wave lane l), so each wave covers one
// contiguous stretch of the row and a load instruction 64 consecutive
// windows.  Narrower groups use slot k*LANES + lane as ln_vec_kernel does.

// Row vectors of all rounds from windows c[0..VPL] (c[VPL]: the slot after
// the last round, needed only where next_word reads it) at byte offset sb.
// The word shift is uniform over the row; for groups of at least a wave it is
// made wave-uniform so the switch is a scalar branch and each case moves only
// the words it needs.
template <class IO, int LANES, int VPL>
__device__ __forceinline__ void realign_in(const u32x4 (&c)[VPL + 1], int sb, u32x4 (&out)[VPL]) {
  constexpr int ES = (int)sizeof(typename IO::elem);
  constexpr int XW = ES == 2 ? 1 : 0;  // bf16 shifts by half-words need one more word
  int q = sb >> 2;
  const int bb = sb & 3;
  if constexpr (LANES >= 64) q = __builtin_amdgcn_readfirstlane(q);
  uint32_t n[VPL][4];
  if constexpr (LANES < 64) {
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
      for (int t = 0; t < 4; ++t) n[k][t] = next_word<LANES>(c[k].w[t], c[k + 1].w[t]);
  }
#define MBP_REALIGN_CASE(Q)                                                            \
  case Q:                                                                              \
    _Pragma("unroll") for (int k = 0; k < VPL; ++k) {                                  \
      if constexpr (LANES >= 64) {                                                     \
        _Pragma("unroll") for (int t = 0; t < 4; ++t) n[k][t] =                        \
            (t < Q + XW) ? next_word<LANES>(c[k].w[t], c[k + 1].w[t]) : 0u;           \
      }                                                                                \
      out[k] = funnel<ES, Q>(c[k], n[k], bb);                                          \
    }                                                                                  \
    break;
  switch (q) {
    MBP_REALIGN_CASE(0)
    MBP_REALIGN_CASE(1)
    MBP_REALIGN_CASE(2)
    default: MBP_REALIGN_CASE(3)
  }
#undef MBP_REALIGN_CASE
}

template <class IO, int LANES, int VPL, bool RES, int EPI>
__global__ __launch_bounds__(block_for(LANES)) void ln_shift_kernel(
    const typename IO::elem* x, const typename IO::elem* res,
    const typename IO::elem* __restrict__ gamma, const typename IO::elem* __restrict__ beta,
    typename IO::elem* y, int64_t rows, int cols, int64_t ldx, int64_t ldr, int64_t ldy, double eps_d,
    Drop drop) {
  typedef typename IO::elem E;
  typedef typename Types<IO, RES>::acc Acc;
  typedef typename Types<IO, RES>::val Val;
  constexpr int ES = (int)sizeof(E);
  constexpr int V = IO::kVec;
  constexpr int BLOCK = block_for(LANES);
  constexpr int RPB = BLOCK / LANES;
  constexpr int WL = LANES < 64 ? LANES : 64;  // lanes of a group inside one wave
  constexpr bool kInPlace = std::is_same<Acc, Val>::value;
  __shared__ Acc red[2][BLOCK / 64];

  const int lane = threadIdx.x % LANES;
  const int sub = threadIdx.x / LANES;
  const int wl = lane % WL;
  const int nvec = (cols + V - 1) / V;  // the last vector may be partial
  const int rem = cols - V * (nvec - 1);  // its elements inside the row (1 .. V)
  const Acc eps = (Acc)eps_d;
  // each tensor's extent: its last row ends (rows - 1) * ld + cols elements in
  const Win wx = make_win<IO>(x, (rows - 1) * ldx + cols);
  const Win wr = RES ? make_win<IO>(res, (rows - 1) * ldr + cols) : wx;
  const Win wy = make_win<IO>(y, (rows - 1) * ldy + cols);
  auto slot = [&](int k) -> int {
    return LANES >= 64 ? (lane / 64) * 64 * VPL + k * 64 + wl : k * LANES + lane;
  };

  // gamma / beta of this lane's slots, packed
  const bool gvec = (((uintptr_t)gamma | (uintptr_t)beta) & 15) == 0;
  u32x4 gp[VPL], bp[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int j = slot(k);
    u32x4 gv = {{0u, 0u, 0u, 0u}}, bv = {{0u, 0u, 0u, 0u}};
    if (gvec && V * j + V <= cols) {
      gv = load_vec<IO>(gamma, j);
      bv = load_vec<IO>(beta, j);
    } else if (j < nvec) {
      gv = partial_vec<IO>(gamma, V * j, cols);
      bv = partial_vec<IO>(beta, V * j, cols);
    }
    gp[k] = gv;
    bp[k] = bv;
  }

  const int64_t groups = (rows + RPB - 1) / RPB;
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      opaque(gp[k]);
      opaque(bp[k]);
    }
    const int64_t row = grp * RPB + sub;
    const bool live = row < rows;
    const int64_t lrow = live ? row : rows - 1;
    const int64_t ex = lrow * ldx, er = lrow * ldr;  // the row in x and in the residual

    // row vectors of x and residual
    u32x4 xa[VPL], ra[VPL];
    {
      const int64_t offx = wx.mb + (int64_t)ES * ex, offr = wr.mb + (int64_t)ES * er;
      const int64_t qx = offx >> 4, qr = offr >> 4;
      const int nvx = (int)(((offx & 15) + (int64_t)ES * cols + 15) >> 4);
      const int nvr = (int)(((offr & 15) + (int64_t)ES * cols + 15) >> 4);
      bool inside = 16 * qx >= wx.mb && 16 * (qx + nvx) <= wx.end;
      if constexpr (RES) inside = inside && 16 * qr >= wr.mb && 16 * (qr + nvr) <= wr.end;
      if (inside) {
        const u32x4* sx = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(x) - wx.mb) + qx;
        const u32x4* sr = RES ? reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(res) - wr.mb) + qr
                              : nullptr;
        u32x4 cx[VPL + 1], cr[VPL + 1];
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
          cx[k] = load_nt(sx + min(slot(k), nvx - 1));
          if constexpr (RES) cr[k] = load_nt(sr + min(slot(k), nvr - 1));
        }
        cx[VPL] = cr[VPL] = u32x4{{0u, 0u, 0u, 0u}};
        if (wl == 0) {  // the slot after this wave's (group's) last one
          cx[VPL] = load_nt(sx + min(slot(VPL), nvx - 1));
          if constexpr (RES) cr[VPL] = load_nt(sr + min(slot(VPL), nvr - 1));
        }
        realign_in<IO, LANES, VPL>(cx, (int)(offx & 15), xa);
        if constexpr (RES) realign_in<IO, LANES, VPL>(cr, (int)(offr & 15), ra);
      } else {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
          // elements of the slot inside the row; opaque so the per-element
          // tests stay in this rarely taken branch instead of being hoisted
          int lim = cols - V * slot(k);
          opaque(lim);
          xa[k] = ra[k] = u32x4{{0u, 0u, 0u, 0u}};
#pragma unroll
          for (int e = 0; e < V; ++e)
            if (e < lim) {
              set_elem<IO>(xa[k], e, x[ex + V * slot(k) + e]);
              if constexpr (RES) set_elem<IO>(ra[k], e, res[er + V * slot(k) + e]);
            }
        }
      }
    }

    Val v[VPL][V];
    Acc sum = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int j = slot(k);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        Val t = (Val)IO::get(xa[k], e);
        if constexpr (RES) t += (Val)IO::get(ra[k], e);
        v[k][e] = t;
      }
      if (j == nvec - 1) {  // the last vector: elements from rem on lie past the row
#pragma unroll
        for (int e = 0; e < V; ++e)
          if (e >= rem) v[k][e] = 0;
      }
      Acc part = 0;
#pragma unroll
      for (int e = 0; e < V; ++e) part += (Acc)v[k][e];
      if (j < nvec) sum += part;
    }
    const Acc mean = mean_cols(group_sum<LANES, BLOCK>(sum, red[0]), cols);

    Acc m2 = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int j = slot(k);
      Acc dd[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        dd[e] = (Acc)v[k][e] - mean;
        if constexpr (kInPlace) v[k][e] = dd[e];
      }
      if (j == nvec - 1) {
#pragma unroll
        for (int e = 0; e < V; ++e)
          if (e >= rem) dd[e] = 0;
      }
      Acc part = 0;
#pragma unroll
      for (int e = 0; e < V; ++e) part = fma_t(dd[e], dd[e], part);
      if (j < nvec) m2 += part;
    }
    const Acc rstd = inv_sqrt(div_cols(group_sum<LANES, BLOCK>(m2, red[1]), cols) + eps);

    u32x4 ov[VPL + 1];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      float o[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const Acc d = kInPlace ? (Acc)v[k][e] : (Acc)v[k][e] - mean;
        o[e] = finish<Acc, EPI>(d, rstd, (Acc)IO::get(gp[k], e), (Acc)IO::get(bp[k], e));
      }
      if constexpr (EPI == kEpiReluDrop)  // slot j holds columns V*j .. V*j + V - 1 of the row
        relu_dropout<V, false>(o, (uint64_t)(live ? row : 0) * (uint64_t)cols + (uint64_t)(V * slot(k)), drop);
      ov[k] = pack_vec<IO>(o);
    }
    ov[VPL] = ov[VPL - 1];

    // Output window j = bytes [16 - sb, 32 - sb) of vectors j-1 || j (sb > 0),
    // or vector j (sb == 0).  Slot j writes window j; its bytes from vector
    // j-1 only where that vector is known here (not in the first slot of a
    // wave or group), and the slot after the last one (k == VPL, lane 0 of
    // the wave or group) writes the bytes of the last slot's vector.
    const int64_t offy = wy.mb + (int64_t)ES * (row * ldy);
    const int sb = (int)(offy & 15);
    const int nvy = (int)((sb + (int64_t)ES * cols + 15) >> 4);
    u32x4* dy = reinterpret_cast<u32x4*>(reinterpret_cast<char*>(y) - wy.mb) + (offy >> 4);
    E* yrow = y + row * ldy;
    const int rbytes = ES * cols;
    // window of each round (k == VPL: the slot after the last)
    u32x4 win[VPL + 1];
    {
      int q = ((16 - sb) & 15) >> 2;
      const int bb = (16 - sb) & 3;
      if constexpr (LANES >= 64) q = __builtin_amdgcn_readfirstlane(q);
      if (sb == 0) {
#pragma unroll
        for (int k = 0; k <= VPL; ++k) win[k] = ov[k];
      } else {
        // prev[k]: vector of slot j-1 (round k); its word t from the lane before
        uint32_t pw[VPL + 1][4];
#pragma unroll
        for (int k = 0; k <= VPL; ++k)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            pw[k][t] = prev_word<LANES>(ov[k].w[t], ov[k > 0 ? k - 1 : 0].w[t]);
#define MBP_OUT_CASE(Q)                                                          \
  case Q:                                                                        \
    _Pragma("unroll") for (int k = 0; k <= VPL; ++k) {                           \
      u32x4 p;                                                                   \
      _Pragma("unroll") for (int t = 0; t < 4; ++t) p.w[t] = pw[k][t];           \
      win[k] = funnel<ES, Q>(p, ov[k].w, bb);                                    \
    }                                                                            \
    break;
        switch (q) {
          MBP_OUT_CASE(0)
          MBP_OUT_CASE(1)
          MBP_OUT_CASE(2)
          default: MBP_OUT_CASE(3)
        }
#undef MBP_OUT_CASE
      }
    }
    if (live) {
#pragma unroll
      for (int k = 0; k <= VPL; ++k) {
        if (k == VPL && wl != 0) continue;
        const int j = slot(k);
        if (j >= nvy) continue;
        const int a = 16 * j - sb;  // row byte of the window's first byte
        const bool prev_ok = sb != 0 && !(k == 0 && wl == 0);
        const bool cur_ok = k < VPL;
        const int lo = max(prev_ok ? a : 16 * j, 0);
        const int hi = min(cur_ok ? a + 16 : 16 * j, rbytes);
        if (lo == a && hi == a + 16) {
          store_nt(dy + j, win[k]);
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const int rb = a + ES * e;
            if (rb >= lo && rb < hi) {
              if constexpr (ES == 2)
                yrow[rb / ES] = (E)(win[k].w[e >> 1] >> (16 * (e & 1)));
              else
                yrow[rb / ES] = __uint_as_float(win[k].w[e]);
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------ dispatch

template <class IO, bool RES, int EPI>
struct VecSel {
  template <int L, int P>
  struct K {
    static const void* ptr() { return reinterpret_cast<const void*>(&ln_vec_kernel<IO, L, P, RES, EPI>); }
  };
};
// fp32 rows of up to 2048 vectors take the shift kernel unless the epilogue
// is dropout (launch_flags), so those class layouts are not instantiated
template <class IO, bool RES, int EPI>
struct ClassSel {
  template <int L, int P>
  struct K {
    static const void* ptr() {
      if constexpr (sizeof(typename IO::elem) == 4 && EPI != kEpiReluDrop && L * P <= 2048) return nullptr;
      else return reinterpret_cast<const void*>(&ln_class_kernel<IO, L, P, RES, EPI>);
    }
  };
};
template <class IO, bool RES, int EPI>
struct ShiftSel {
  template <int L, int P>
  struct K {
    static const void* ptr() { return reinterpret_cast<const void*>(&ln_shift_kernel<IO, L, P, RES, EPI>); }
  };
};
constexpr int64_t kMaxGrid = 1 << 30;
constexpr int64_t kShiftGroups = 4;
constexpr int64_t kClassGroups = 4;

template <class IO, bool RES, int EPI>
hipError_t launch_flags(const void* x, int64_t ldx, const void* res, int64_t ldr, const void* gamma,
                        const void* beta, void* y, int64_t ldy, int64_t rows, int64_t cols, double eps,
                        const Drop& drop_in, hipStream_t s) {
  constexpr int V = IO::kVec;
  constexpr int64_t ES = (int64_t)sizeof(typename IO::elem);
  // rows on 16-byte boundaries: aligned bases and row strides of whole 16-byte vectors
  const bool aligned = aligned16(x) && aligned16(y) && (!res || aligned16(res)) && aligned16(gamma) &&
                       aligned16(beta) && cols % V == 0 && (ES * ldx) % 16 == 0 && (ES * ldy) % 16 == 0 &&
                       (!res || (ES * ldr) % 16 == 0);
  // fp32 rows past kRegCols columns take the multi-pass kernel; 16-bit rows
  // (at most 4096 vectors of 8 at the 32768-column maximum) all stay in
  // registers (512-lane layouts, below)
  if constexpr (ES == 4) {
    if (cols > kRegCols) {
      const int wgrid = (int)(rows < 4096 ? rows : 4096);
      int wcols = (int)cols;
      Drop wdrop = drop_in;
      void* wargs[] = {&x, &res, &gamma, &beta, &y, &rows, &wcols, &ldx, &ldr, &ldy, &eps, &wdrop};
      return hipLaunchKernel(reinterpret_cast<const void*>(&ln_wide_kernel<IO, RES, EPI>), dim3(wgrid),
                             dim3(1024), wargs, 0, s);
    }
  }
  const int i = pick_shape((cols + V - 1) / V);
  if (i < 0) return hipErrorInvalidValue;
  // Rows of 2049-4096 vectors: 512-lane groups of 6 or 8 vectors a lane
  // instead of 1024 x 3 / 1024 x 4, for plain fp32 LayerNorm (8192 rows of
  // 10000, 12287, 12288, 16384 columns: 4-6% faster; not with a residual:
  // 12288 + GeLU 1.7% slower; not measured with the other epilogues) and for
  // every 16-bit form (16385-32768 columns, where the multi-pass kernel
  // took 1.4-3.8 times as long: 16384 x 24576 + residual + GeLU 786.5 ->
  // 499.0 us, LayerNorm -> ReLU -> dropout 1367.3 -> 361.0 us)
  constexpr bool kAlt = (ES == 4 && !RES && EPI == kEpiNone) || ES == 2;
  const bool w512 = kAlt && i >= 10;
  // the families with the 512-lane alternatives never take the 1024-lane layouts
  constexpr int kLast = kAlt ? 9 : 11;
  const int lanes = w512 ? 512 : kShapes[i].lanes;
  const int block_v = block_for(lanes);
  const int rpb_v = block_v / lanes;
  const int64_t groups = (rows + rpb_v - 1) / rpb_v;
  // one block per row group, within what a dispatch can address (the row
  // kernels loop over the rest)
  const int64_t gmax = dispatch_blocks(block_v) < kMaxGrid ? dispatch_blocks(block_v) : kMaxGrid;
  const int grid = (int)(groups < gmax ? groups : gmax);
  int icols = (int)cols;
  Drop drop = drop_in;
  void* args[] = {&x, &res, &gamma, &beta, &y, &rows, &icols, &ldx, &ldr, &ldy, &eps, &drop};
  if (aligned) {
    const void* k = shape_kernel_alt<VecSel<IO, RES, EPI>::template K, kAlt, true, kLast>(i, w512);
    // two row groups per block, when there are thousands: fp32 rows
    // (measured at 8192 x 4096: 46.2 us against 47.5 for one; 4 or 8 per
    // block no better) and 16-bit rows in 256-lane groups other than the
    // dropout epilogue, whose second group's loads are then issued while the
    // first is computed (16384 x 8192 + residual + GeLU: 134.7 -> 130.7 us,
    // plain LayerNorm 96.7 -> 90.0; one group a block: 132.5 and 91.5).
    // The dropout epilogue and the other 16-bit layouts take one (dropout
    // 16384 x 8192: 92.5 us for two groups a block without the early loads,
    // 91.3 for one with them, 92.4 for two with them; 32768 x 4096 + GeLU:
    // 128.0, 125.9 with them, 128.8 for two)
    int64_t vgrid = grid;
    if (groups >= 4096 && (ES == 4 || (lanes == 256 && EPI != kEpiReluDrop))) vgrid = (groups + 1) / 2;
    // plain fp32 LayerNorm in 256 x 4 (3073-4096 columns): a persistent loop
    // of two blocks per compute unit, each loading gamma/beta (32 KB) once
    // for its many rows and issuing the next row's loads ahead (same process,
    // us: 8192 x 4096 45.8 -> 45.0, 16384 x 4096 88.8 -> 87.9, 12000 x 4096
    // 66.0 -> 64.7, 4096 x 4096 25.0 -> 24.8; three blocks per unit 45.1, four
    // 47.1; the same for 16-bit rows was slower, 2-18%)
    if constexpr (ES == 4 && !RES && EPI == kEpiNone) {
      if (i == 7 && !w512) {
        const int64_t pg = 2 * (int64_t)compute_units();
        if (pg > 0) vgrid = groups < pg ? groups : pg;
      }
    }
    if (vgrid > grid) vgrid = grid;
    return hipLaunchKernel(k, dim3((unsigned)vgrid), dim3(block_v), args, 0, s);
  }
  const uintptr_t ax = reinterpret_cast<uintptr_t>(x);
  // x, residual and y agree modulo 16 bytes in every row: congruent bases and
  // one row stride
  const bool congruent = ((ax ^ reinterpret_cast<uintptr_t>(y)) & 15) == 0 &&
                         (!res || ((ax ^ reinterpret_cast<uintptr_t>(res)) & 15) == 0) && ldx > 0 &&
                         ldy == ldx && (!res || ldr == ldx);
  // fp32 rows of up to 2048 vectors (LayerNorm, + residual, + GeLU) take the
  // shift kernel even when congruent:
  // measured faster than the class kernel there (8192 x 4093: 55.0 -> 53.2 us;
  // 8192 x 1001: 21.4 -> 17.9; with residual and GeLU 76.7 -> 75.3 and
  // 26.1 -> 23.4), slower at 12287 columns (186 -> 192 us, 239 -> 263 with
  // residual and GeLU); the dropout epilogue stays on the class kernel (its
  // shift form 25-47% slower), and so do bf16 rows (32768 x 4095 + GeLU:
  // 144.1 us in the class kernel, 161.6 in the shift kernel with y one
  // element off)
  const bool shift_f32 = ES == 4 && EPI != kEpiReluDrop && (cols + V - 1) / V <= 2048;
  // 16-bit dropout rows of 3073-4096 vectors: the class kernel would need more
  // than the 256 registers of 512-thread blocks (140 bytes a lane of spill;
  // measured 797 us against 861 for the shift kernel on 16384 x 32767), so
  // they take the spill-free shift kernel
  const bool shift_drop8 = ES == 2 && EPI == kEpiReluDrop && i == 11;
  if (congruent && !shift_f32 && !shift_drop8) {
    // 16-bit rows without dropout in two vectors a lane, one row group a
    // block: 385-512 vectors in 256 lanes rather than the table's 128 x 4
    // (32768 x 4095 + residual + GeLU: 145.4 -> 143.3 us, 74 registers
    // against 117 and no scalar spills; with eight row groups a block 149.7,
    // 512 x 1 143.5 / 149.2; 32768 x 3501: 129.5 -> 128.2), 769-1024 vectors
    // in 512 lanes rather than 256 x 4, eight row groups a block (16384 x 8191
    // + residual + GeLU: 146.2 -> 141.7 us, without the residual 108.9 ->
    // 102.7, 16384 x 6999: 130.1 -> 128.0; four groups a block 144.8, twelve
    // or sixteen 152).  Shorter rows keep the table's layout (32768 x 2101 in
    // 256 x 2: 95.7 against 100.9 us, the second vector of most lanes unused)
    const int nv2 = (int)((cols + V - 1) / V);
    const bool c256 = ES == 2 && EPI != kEpiReluDrop && i == 5 && nv2 > 384;
    const bool c512 = ES == 2 && EPI != kEpiReluDrop && i == 7 && nv2 > 768;
    const int rpb = (c256 || c512) ? 1 : rpb_v;
    const int block = c256 ? 256 : c512 ? 512 : block_v;
    // Rows whose windows lie inside the tensors: [r_lo, r_hi).  With the row
    // pitch pb (bytes), a row starting fewer than 16 - (x mod 16) bytes past an
    // unaligned start, or ending fewer than (end mod 16) bytes before an
    // unaligned end, has a window that reaches outside; that is the first
    // ceil((16 - x mod 16) / pb) and the last ceil((end mod 16) / pb) rows.
    const int64_t pb = ES * ldx;
    const int64_t mb = (int64_t)(ax & 15);
    const int64_t me = (int64_t)((ax + (uintptr_t)(ES * ((rows - 1) * ldx + cols))) & 15);
    int64_t r_lo = mb == 0 ? 0 : (16 - mb + pb - 1) / pb;
    int64_t r_hi = me == 0 ? rows : rows - (me + pb - 1) / pb;
    if (r_lo > rows) r_lo = rows;
    if (r_hi < r_lo) r_hi = r_lo;
    const int64_t n_edge = r_lo + (rows - r_hi);
    const int edge_blocks = (int)((n_edge + rpb - 1) / rpb);
    // Classes are taken modulo a 128-byte line when x, residual and y agree
    // modulo 128 and a row spans at least a wave of windows: the kernel then
    // starts every wave's loads and stores on a line (a 4095-wide bf16 row
    // stream measured 150 us with runs straddling lines, 136 us with runs on
    // lines, 136 us for 4096-wide rows).  Otherwise modulo 16 bytes.
    const int nvec = (int)((cols + V - 1) / V);
    const bool same_line = ((ax ^ reinterpret_cast<uintptr_t>(y)) & 127) == 0 &&
                           (!res || ((ax ^ reinterpret_cast<uintptr_t>(res)) & 127) == 0);
    int line = same_line && nvec >= 64 ? 128 : 16;
    // P classes of rows with one offset in the line; each block takes up to
    // kClassGroups row groups of its class, twice that for fp32 rows and the
    // dropout epilogue where a block holds one row group (groups of 256 lanes
    // or more), whose per-block set-up (the gamma/beta ring, the generator's
    // blocks) then weighs more: 8192 x 4093 fp32 58.5 -> 55.1 us, 16384 x 8191
    // bf16 dropout 149.8 -> 142.5 us.  Four stay best for two row groups a
    // block (16384 x 4095 dropout: eight +9.6%) and for bf16 + GeLU (32768 x
    // 4095: eight +0.6%; 16384 x 8191: +0.8%); two and sixteen are slower
    // everywhere.
    int period = line;
    while (period > 1 && (pb * (period / 2)) % line == 0) period /= 2;
    const int64_t cgroups = ((r_hi - r_lo + period - 1) / period + rpb - 1) / rpb;
    const int64_t per_block =
        (c512 || (rpb == 1 && (ES == 4 || EPI == kEpiReluDrop))) ? 2 * kClassGroups : kClassGroups;
    int64_t nblk = (cgroups + per_block - 1) / per_block;
    if (nblk > kMaxGrid / 128) nblk = kMaxGrid / 128;
    // the blocks of a class loop over its row groups; keep the launch within
    // what a dispatch can address
    const int64_t nmax = (dispatch_blocks(block) - edge_blocks) / period;
    if (nblk > nmax) nblk = nmax;
    const void* k =
        c512   ? reinterpret_cast<const void*>(&ln_class_kernel<IO, 512, 2, RES, EPI>)
        : c256 ? reinterpret_cast<const void*>(&ln_class_kernel<IO, 256, 2, RES, EPI>)
             : shape_kernel_alt<ClassSel<IO, RES, EPI>::template K, kAlt, !(ES == 2 && EPI == kEpiReluDrop), kLast>(i, w512);
    void* cargs[] = {&x,   &res,    &gamma, &beta, &y,    &rows, &icols, &ldx,
                     &eps, &period, &line,  &r_lo, &r_hi, (void*)&edge_blocks, &drop};
    return hipLaunchKernel(k, dim3((unsigned)(edge_blocks + period * nblk)), dim3(block), cargs, 0, s);
  }
  // kShiftGroups row groups per block amortise the per-block gamma/beta set-up
  const void* k = shape_kernel_alt<ShiftSel<IO, RES, EPI>::template K, kAlt, true, kLast>(i, w512);
  const int64_t sg = (groups + kShiftGroups - 1) / kShiftGroups;
  const int sgrid = (int)(sg < grid ? sg : grid);  // the shift kernel loops over the rest
  return hipLaunchKernel(k, dim3(sgrid), dim3(block_v), args, 0, s);
}

// act: kEpiNone, kEpiGelu, kEpiReluDrop (no residual; `drop` describes it).
// Row strides in elements: row i of x, residual and y starts at i * ld.
template <class IO>
hipError_t launch(const void* x, int64_t ldx, const void* res, int64_t ldr, const void* gamma,
                  const void* beta, void* y, int64_t ldy, int64_t rows, int64_t cols, double eps, int act,
                  const Drop* drop, hipStream_t s) {
  const Drop none{0, 0, 0, 1.0f};
  if (rows == 1) ldx = ldr = ldy = cols;  // one row: its stride is never used
  if (act == kEpiReluDrop) {
    if (res || !drop) return hipErrorInvalidValue;
    return launch_flags<IO, false, kEpiReluDrop>(x, ldx, res, ldr, gamma, beta, y, ldy, rows, cols, eps, *drop, s);
  }
  const bool gelu = act == kEpiGelu;
  if (res)
    return gelu ? launch_flags<IO, true, kEpiGelu>(x, ldx, res, ldr, gamma, beta, y, ldy, rows, cols, eps, none, s)
                : launch_flags<IO, true, kEpiNone>(x, ldx, res, ldr, gamma, beta, y, ldy, rows, cols, eps, none, s);
  return gelu ? launch_flags<IO, false, kEpiGelu>(x, ldx, res, ldr, gamma, beta, y, ldy, rows, cols, eps, none, s)
              : launch_flags<IO, false, kEpiNone>(x, ldx, res, ldr, gamma, beta, y, ldy, rows, cols, eps, none, s);
}

}  // namespace ln
}  // namespace mbp
