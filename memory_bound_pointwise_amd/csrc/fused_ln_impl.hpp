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
// Three kernels, chosen by the host from pointer alignment and row length:
//  * ln_vec_kernel: rows start on 16-byte boundaries (x, residual, y, gamma,
//    beta 16-byte aligned and cols a whole number of 16-byte vectors).  gamma
//    and beta stay in registers for all rows a block processes.
//  * ln_win_kernel: x, residual and y share one misalignment mod 16 (e.g. bf16
//    rows of 4095 elements, 8190 bytes): each row is covered by the 16-byte
//    aligned windows that overlap it, so the loads and the interior stores are
//    128-bit accesses (details at the kernel).
//  * ln_scalar_kernel: anything else (pointers with different misalignments);
//    one element per lane and load.
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

template <class Acc, bool GELU>
__device__ __forceinline__ float finish(Acc d, Acc rstd, Acc g, Acc b) {
  const float u = (float)fma_t(d * rstd, g, b);
  if constexpr (GELU) return gelu_tanh_f32(u);
  return u;
}

// ------------------------------------------------------------ aligned rows

template <class IO, int LANES, int VPL, bool RES, bool GELU>
__global__ __launch_bounds__(block_for(LANES)) void ln_vec_kernel(
    const typename IO::elem* x, const typename IO::elem* res,
    const typename IO::elem* __restrict__ gamma, const typename IO::elem* __restrict__ beta,
    typename IO::elem* y, int64_t rows, int cols, double eps_d) {
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

  // gamma / beta of this lane's columns, as fp32 for all rows of the block
  float g[VPL][V], b[VPL][V];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int vi = lane + k * LANES;
    u32x4 gv = {{0u, 0u, 0u, 0u}}, bv = {{0u, 0u, 0u, 0u}};
    if (vi < nvec) {
      gv = load_vec<IO>(gamma, vi);
      bv = load_vec<IO>(beta, vi);
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
      g[k][e] = IO::get(gv, e);
      b[k][e] = IO::get(bv, e);
    }
  }

  const int64_t groups = (rows + RPB - 1) / RPB;
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
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
    // A group past the last row reads the last row (and stores nothing); a slot
    // past the row's last vector reads that vector and is left out of the
    // sums.  Every load is in bounds and none needs a branch or a zero fill.
    const int64_t lrow = live ? row : rows - 1;
    const typename IO::elem* xr = x + lrow * (int64_t)cols;
    const typename IO::elem* rr = RES ? res + lrow * (int64_t)cols : nullptr;
    typename IO::elem* yr = y + row * (int64_t)cols;

    // issue every load of the row first
    u32x4 xv[VPL], rv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int vi = min(lane + k * LANES, nvec - 1);
      xv[k] = stream_vec<IO>(xr, vi);
      if constexpr (RES) rv[k] = stream_vec<IO>(rr, vi);
    }
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
    const Acc mean = group_sum<LANES, BLOCK>(sum, red[0]) / (Acc)cols;

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
    const Acc rstd = inv_sqrt(group_sum<LANES, BLOCK>(m2, red[1]) / (Acc)cols + eps);

#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int vi = lane + k * LANES;
      if (!(live && vi < nvec)) continue;
      float o[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const Acc d = kInPlace ? (Acc)v[k][e] : (Acc)v[k][e] - mean;
        o[e] = finish<Acc, GELU>(d, rstd, (Acc)g[k][e], (Acc)b[k][e]);
      }
      store_nt(reinterpret_cast<u32x4*>(yr) + vi, pack_vec<IO>(o));
    }
  }
}

// ------------------------------------------------------------ windowed rows

// Rows that do not start on 16-byte boundaries, with x, residual and y sharing
// one misalignment mb.  Each row is covered by the aligned 16-byte windows that
// overlap it (window q = bytes [16q, 16q + 16) above the boundary below the
// base pointer); slot j of a row holds window q0 + j, whose element e is column
// V*j + e - s, where s is the row's start inside its first window.  s repeats
// with period P = 16 / gcd(16, cols * sizeof(E)) over the rows, so each block
// serves one residue class of rows (row = r0 + cls + P*t) in which s, the
// number of windows nv and the element masks of the first and last window are
// constants; gamma/beta are gathered once per block into that shifted layout.
// The rows handled here are the interior rows [r0, r1) whose windows lie inside
// the tensor; the few rows at either end whose windows would reach outside it
// are done element by element by the blocks past the last residue block.  So
// the hot loop differs from the aligned kernel only in its addressing and in
// the two partial windows per row (masked out of the sums, stored element by
// element).  Slots past a row's last window are skipped.  The block is
// persistent, so the next row's windows are loaded while the current row is
// reduced and written.
template <class IO, int LANES, int VPL, bool RES, bool GELU>
__global__ __launch_bounds__(block_for(LANES)) void ln_win_kernel(
    const typename IO::elem* x, const typename IO::elem* res,
    const typename IO::elem* __restrict__ gamma, const typename IO::elem* __restrict__ beta,
    typename IO::elem* y, int64_t rows, int cols, double eps_d, int period, int64_t r0,
    int64_t r1, int main_blocks) {
  typedef typename IO::elem E;
  typedef typename Types<IO, RES>::acc Acc;
  typedef typename Types<IO, RES>::val Val;
  constexpr int V = IO::kVec;
  constexpr int ES = (int)sizeof(E);
  constexpr int BLOCK = block_for(LANES);
  constexpr int RPB = BLOCK / LANES;
  constexpr bool kInPlace = std::is_same<Acc, Val>::value;
  constexpr unsigned kFull = (1u << V) - 1;
  __shared__ Acc red[2][BLOCK / 64];
  const Acc eps = (Acc)eps_d;

  if ((int)blockIdx.x >= main_blocks) {
    // an edge row: the whole block, one element per lane and load
    const int64_t i = (int64_t)blockIdx.x - main_blocks;
    const int64_t row = i < r0 ? i : r1 + (i - r0);
    const int64_t e0 = row * (int64_t)cols;
    Acc sum = 0;
    for (int c = threadIdx.x; c < cols; c += BLOCK) {
      Val t = (Val)IO::load1(x, e0 + c);
      if constexpr (RES) t += (Val)IO::load1(res, e0 + c);
      sum += (Acc)t;
    }
    const Acc mean = group_sum<BLOCK, BLOCK>(sum, red[0]) / (Acc)cols;
    Acc m2 = 0;
    for (int c = threadIdx.x; c < cols; c += BLOCK) {
      Val t = (Val)IO::load1(x, e0 + c);
      if constexpr (RES) t += (Val)IO::load1(res, e0 + c);
      const Acc d = (Acc)t - mean;
      m2 = fma_t(d, d, m2);
    }
    const Acc rstd = inv_sqrt(group_sum<BLOCK, BLOCK>(m2, red[1]) / (Acc)cols + eps);
    for (int c = threadIdx.x; c < cols; c += BLOCK) {
      Val t = (Val)IO::load1(x, e0 + c);
      if constexpr (RES) t += (Val)IO::load1(res, e0 + c);
      IO::store1(y, e0 + c, finish<Acc, GELU>((Acc)t - mean, rstd, (Acc)IO::load1(gamma, c),
                                             (Acc)IO::load1(beta, c)));
    }
    return;
  }

  const int lane = threadIdx.x % LANES;
  const int sub = threadIdx.x / LANES;
  const int mb = (int)(reinterpret_cast<uintptr_t>(x) & 15);
  const u32x4* xw = reinterpret_cast<const u32x4*>(reinterpret_cast<uintptr_t>(x) - mb);
  const u32x4* rw = RES ? reinterpret_cast<const u32x4*>(reinterpret_cast<uintptr_t>(res) - mb) : nullptr;
  u32x4* yw = reinterpret_cast<u32x4*>(reinterpret_cast<uintptr_t>(y) - mb);
  const int64_t row_bytes = (int64_t)ES * cols;

  // this block's residue class: rows r0 + cls + P*t, t < cls_rows
  const int cls = blockIdx.x % period;
  const int per_cls = main_blocks / period;
  const int64_t span = r1 - r0 - cls;
  const int64_t cls_rows = span > 0 ? (span + period - 1) / period : 0;
  const int64_t groups = (cls_rows + RPB - 1) / RPB;
  const int s = (int)((mb + row_bytes * (r0 + cls)) & 15) / ES;
  const int nv = (s * ES + (int)row_bytes + 15) >> 4;  // windows per row

  // per slot: which elements belong to the row (only the first and last
  // window are partial), and gamma/beta gathered into the shifted layout
  unsigned emask[VPL];
  u32x4 graw[VPL], braw[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int j = lane + k * LANES;
    emask[k] = 0;
    graw[k] = braw[k] = u32x4{{0u, 0u, 0u, 0u}};
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int c = V * j + e - s;
      if (j < nv && c >= 0 && c < cols) {
        emask[k] |= 1u << e;
        set_elem<IO>(graw[k], e, gamma[c]);
        set_elem<IO>(braw[k], e, beta[c]);
      }
    }
  }

  // row of group grp for this lane group (past the class's end: its last row)
  auto row_of = [&](int64_t grp, bool& live) {
    const int64_t t = grp * RPB + sub;
    live = t < cls_rows;
    return r0 + cls + (int64_t)period * (live ? t : cls_rows - 1);
  };
  // the windows of a row; slots without row elements load nothing
  auto load_row = [&](int64_t row, u32x4* xv, u32x4* rv) {
    const int64_t q0 = (mb + row_bytes * row) >> 4;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      if (emask[k] == 0) continue;
      xv[k] = load_nt(xw + q0 + lane + k * LANES);
      if constexpr (RES) rv[k] = load_nt(rw + q0 + lane + k * LANES);
    }
  };

  // the next row's windows are loaded while the current row is reduced
  u32x4 nx[VPL], nr[VPL];
  if (blockIdx.x / period < groups) {
    bool live;
    load_row(row_of(blockIdx.x / period, live), nx, nr);
  }
  for (int64_t grp = blockIdx.x / period; grp < groups; grp += per_cls) {
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      opaque(graw[k]);
      opaque(braw[k]);
    }
    bool live;
    const int64_t row = row_of(grp, live);
    const int64_t q0 = (mb + row_bytes * row) >> 4;
    u32x4 xv[VPL], rv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      xv[k] = nx[k];
      if constexpr (RES) rv[k] = nr[k];
    }
    if (grp + per_cls < groups) {
      bool nlive;
      load_row(row_of(grp + per_cls, nlive), nx, nr);
    }

    Val v[VPL][V];
    Acc sum = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      if (emask[k] == 0) continue;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        Val tv = (Val)IO::get(xv[k], e);
        if constexpr (RES) tv += (Val)IO::get(rv[k], e);
        v[k][e] = tv;
      }
      if (emask[k] != kFull) {
#pragma unroll
        for (int e = 0; e < V; ++e)
          if (!((emask[k] >> e) & 1u)) v[k][e] = 0;
      }
      Acc part = 0;
#pragma unroll
      for (int e = 0; e < V; ++e) part += (Acc)v[k][e];
      sum += part;
    }
    const Acc mean = group_sum<LANES, BLOCK>(sum, red[0]) / (Acc)cols;

    Acc m2 = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      if (emask[k] == 0) continue;
      Acc dd[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        dd[e] = (Acc)v[k][e] - mean;
        if constexpr (kInPlace) v[k][e] = dd[e];
      }
      if (emask[k] != kFull) {
#pragma unroll
        for (int e = 0; e < V; ++e)
          if (!((emask[k] >> e) & 1u)) dd[e] = 0;
      }
      Acc part = 0;
#pragma unroll
      for (int e = 0; e < V; ++e) part = fma_t(dd[e], dd[e], part);
      m2 += part;
    }
    const Acc rstd = inv_sqrt(group_sum<LANES, BLOCK>(m2, red[1]) / (Acc)cols + eps);

    if (!live) continue;
    const int64_t e0 = row * (int64_t)cols;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      if (emask[k] == 0) continue;
      float o[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const Acc d = kInPlace ? (Acc)v[k][e] : (Acc)v[k][e] - mean;
        o[e] = finish<Acc, GELU>(d, rstd, (Acc)IO::get(graw[k], e), (Acc)IO::get(braw[k], e));
      }
      const int j = lane + k * LANES;
      if (emask[k] == kFull) {
        store_nt(yw + q0 + j, pack_vec<IO>(o));
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e)
          if ((emask[k] >> e) & 1u) IO::store1(y, e0 + V * j + e - s, o[e]);
      }
    }
  }
}

// ------------------------------------------------------------ any pointers

template <class IO, int LANES, int EPL, bool RES, bool GELU>
__global__ __launch_bounds__(block_for(LANES)) void ln_scalar_kernel(
    const typename IO::elem* x, const typename IO::elem* res,
    const typename IO::elem* __restrict__ gamma, const typename IO::elem* __restrict__ beta,
    typename IO::elem* y, int64_t rows, int cols, double eps_d) {
  typedef typename Types<IO, RES>::acc Acc;
  typedef typename Types<IO, RES>::val Val;
  constexpr int BLOCK = block_for(LANES);
  constexpr int RPB = BLOCK / LANES;
  __shared__ Acc red[2][BLOCK / 64];
  const int lane = threadIdx.x % LANES;
  const int sub = threadIdx.x / LANES;
  const Acc eps = (Acc)eps_d;
  const int64_t groups = (rows + RPB - 1) / RPB;
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
    const int64_t row = grp * RPB + sub;
    const bool live = row < rows;
    const int64_t e0 = row * (int64_t)cols;
    Val v[EPL];
    Acc sum = 0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const int c = lane + k * LANES;
      Val t = 0;
      if (live && c < cols) {
        t = (Val)IO::load1(x, e0 + c);
        if constexpr (RES) t += (Val)IO::load1(res, e0 + c);
      }
      v[k] = t;
      sum += (Acc)t;
    }
    const Acc mean = group_sum<LANES, BLOCK>(sum, red[0]) / (Acc)cols;
    Acc m2 = 0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const Acc d = (Acc)v[k] - mean;
      if (lane + k * LANES < cols) m2 = fma_t(d, d, m2);
    }
    const Acc rstd = inv_sqrt(group_sum<LANES, BLOCK>(m2, red[1]) / (Acc)cols + eps);
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      const int c = lane + k * LANES;
      if (!(live && c < cols)) continue;
      const Acc d = (Acc)v[k] - mean;
      IO::store1(y, e0 + c,
                 finish<Acc, GELU>(d, rstd, (Acc)IO::load1(gamma, c), (Acc)IO::load1(beta, c)));
    }
  }
}

// ------------------------------------------------------------ dispatch

template <class IO, bool RES, bool GELU>
struct VecSel {
  template <int L, int P>
  struct K {
    static const void* ptr() { return reinterpret_cast<const void*>(&ln_vec_kernel<IO, L, P, RES, GELU>); }
  };
};
// Window layouts: at most 3 windows per lane (the gathered gamma/beta take as
// many registers as the data); the last slot is only partly used.
constexpr Shape kWinShapes[] = {{16, 2},  {32, 2},  {32, 3},  {64, 3},   {128, 3},
                                {256, 3}, {512, 3}, {1024, 3}};
constexpr int kNumWin = sizeof(kWinShapes) / sizeof(Shape);

inline int pick_win_shape(int64_t nvec) {
  for (int i = 0; i < kNumWin; ++i)
    if ((int64_t)kWinShapes[i].lanes * kWinShapes[i].vpl >= nvec) return i;
  return -1;
}

template <template <int, int> class K>
const void* win_kernel(int i) {
  switch (i) {
    case 0: return K<16, 2>::ptr();
    case 1: return K<32, 2>::ptr();
    case 2: return K<32, 3>::ptr();
    case 3: return K<64, 3>::ptr();
    case 4: return K<128, 3>::ptr();
    case 5: return K<256, 3>::ptr();
    case 6: return K<512, 3>::ptr();
    default: return K<1024, 3>::ptr();
  }
}

template <class IO, bool RES, bool GELU>
struct WinSel {
  template <int L, int P>
  struct K {
    static const void* ptr() { return reinterpret_cast<const void*>(&ln_win_kernel<IO, L, P, RES, GELU>); }
  };
};

constexpr int64_t kMaxGrid = 1 << 30;

template <class IO, bool RES, bool GELU>
hipError_t launch_flags(const void* x, const void* res, const void* gamma, const void* beta,
                        void* y, int64_t rows, int64_t cols, double eps, hipStream_t s) {
  constexpr int V = IO::kVec;
  const uintptr_t mb = reinterpret_cast<uintptr_t>(x) & 15;
  const bool congruent = ((reinterpret_cast<uintptr_t>(y) & 15) == mb) &&
                         (!res || (reinterpret_cast<uintptr_t>(res) & 15) == mb);
  const bool aligned = congruent && mb == 0 && cols % V == 0 && aligned16(gamma) && aligned16(beta);
  const void* k;
  int lanes;
  size_t lds = 0;
  if (aligned) {
    const int i = pick_shape(cols / V);
    if (i < 0) return hipErrorInvalidValue;
    k = shape_kernel<VecSel<IO, RES, GELU>::template K>(i);
    lanes = kShapes[i].lanes;
  } else if (congruent) {
    const int i = pick_win_shape(cols / V + 2);
    if (i < 0) return hipErrorInvalidValue;
    k = win_kernel<WinSel<IO, RES, GELU>::template K>(i);
    lanes = kWinShapes[i].lanes;
  } else if (cols <= 64 * 16) {
    k = reinterpret_cast<const void*>(&ln_scalar_kernel<IO, 64, 16, RES, GELU>);
    lanes = 64;
  } else {
    k = reinterpret_cast<const void*>(&ln_scalar_kernel<IO, 1024, 16, RES, GELU>);
    lanes = 1024;
  }
  const int block = block_for(lanes);
  const int rpb = block / lanes;
  const int64_t groups = (rows + rpb - 1) / rpb;
  int icols = (int)cols;
  if (aligned || !congruent) {
    // One block per row group: new blocks start as old ones finish, which keeps
    // more loads in flight than a persistent loop.
    const int grid = (int)(groups < kMaxGrid ? groups : kMaxGrid);
    void* args[] = {&x, &res, &gamma, &beta, &y, &rows, &icols, &eps};
    return hipLaunchKernel(k, dim3(grid), dim3(block), args, lds, s);
  }
  // Windowed rows: interior rows [r0, r1) (their windows lie inside the
  // tensor) in persistent blocks, a whole number per residue class of the row
  // shift; then one block per edge row.
  const int es = (int)sizeof(typename IO::elem);
  const int64_t row_bytes = (int64_t)es * cols;
  const int64_t mbi = (int64_t)mb, end_byte = mbi + row_bytes * rows;
  auto inside = [&](int64_t r) {
    const int64_t off = mbi + row_bytes * r;
    const int64_t q0 = off >> 4, nv = ((off & 15) + row_bytes + 15) >> 4;
    return 16 * q0 >= mbi && 16 * (q0 + nv) <= end_byte;
  };
  int64_t r0 = 0, r1 = rows;
  while (r0 < rows && !inside(r0)) ++r0;
  while (r1 > r0 && !inside(r1 - 1)) --r1;
  const int64_t edge_rows = rows - (r1 - r0);
  int period = 1;
  while (period < 16 && (row_bytes * period) % 16 != 0) period *= 2;
  const int64_t cls_groups = ((r1 - r0 + period - 1) / period + rpb - 1) / rpb;
  const int resident = persistent_grid(k, block, (int64_t)1 << 30, lds);
  int64_t per_cls = resident / period;
  if (per_cls < 1) per_cls = 1;
  if (per_cls > cls_groups) per_cls = cls_groups;
  int main_blocks = (int)(per_cls * period);
  if (r1 == r0) main_blocks = 0;
  const int grid = (int)(main_blocks + edge_rows);
  void* args[] = {&x, &res, &gamma, &beta, &y, &rows, &icols, &eps, &period, &r0, &r1, &main_blocks};
  return hipLaunchKernel(k, dim3(grid), dim3(block), args, lds, s);
}

template <class IO>
hipError_t launch(const void* x, const void* res, const void* gamma, const void* beta, void* y,
                  int64_t rows, int64_t cols, double eps, int act, hipStream_t s) {
  const bool gelu = act == 1;
  if (res)
    return gelu ? launch_flags<IO, true, true>(x, res, gamma, beta, y, rows, cols, eps, s)
                : launch_flags<IO, true, false>(x, res, gamma, beta, y, rows, cols, eps, s);
  return gelu ? launch_flags<IO, false, true>(x, res, gamma, beta, y, rows, cols, eps, s)
              : launch_flags<IO, false, false>(x, res, gamma, beta, y, rows, cols, eps, s);
}

}  // namespace ln
}  // namespace mbp
