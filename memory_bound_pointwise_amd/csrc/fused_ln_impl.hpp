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
// and the output touch HBM; LDS holds the per-wave partial sums (and, on the
// window path, gamma/beta).
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
//    aligned windows that overlap it, so every load and store is a 128-bit
//    access; elements of a window outside the row are masked out, and windows
//    that stick out of the row are stored element by element.  A window that
//    reaches outside the tensor itself is loaded element by element, so no
//    byte outside the tensor is touched.  The column of a register slot moves
//    with the row's offset, so gamma/beta are read from LDS.
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

// Dynamic LDS: (gamma, beta) of column c at index c + V, zero-padded by V
// entries on both sides, so a window's slot e of row-relative vector j reads
// index V*j + e - s + V >= 0 for every row offset s in [0, V).
template <class IO, int LANES, int VPL, bool RES, bool GELU>
__global__ __launch_bounds__(block_for(LANES)) void ln_win_kernel(
    const typename IO::elem* x, const typename IO::elem* res,
    const typename IO::elem* __restrict__ gamma, const typename IO::elem* __restrict__ beta,
    typename IO::elem* y, int64_t rows, int cols, double eps_d) {
  typedef typename IO::elem E;
  typedef typename Types<IO, RES>::acc Acc;
  typedef typename Types<IO, RES>::val Val;
  constexpr int V = IO::kVec;
  constexpr int ES = (int)sizeof(E);
  constexpr int BLOCK = block_for(LANES);
  constexpr int RPB = BLOCK / LANES;
  constexpr bool kInPlace = std::is_same<Acc, Val>::value;
  __shared__ Acc red[2][BLOCK / 64];
  extern __shared__ float2 gb[];

  for (int i = threadIdx.x; i < cols + 2 * V; i += BLOCK) {
    const int c = i - V;
    float2 p = make_float2(0.0f, 0.0f);
    if (c >= 0 && c < cols) p = make_float2(IO::load1(gamma, c), IO::load1(beta, c));
    gb[i] = p;
  }
  __syncthreads();

  const int lane = threadIdx.x % LANES;
  const int sub = threadIdx.x / LANES;
  const Acc eps = (Acc)eps_d;
  // x, residual and y share the misalignment mb; windows are indexed from the
  // 16-byte boundary just below each base pointer.
  const int mb = (int)(reinterpret_cast<uintptr_t>(x) & 15);
  const u32x4* xw = reinterpret_cast<const u32x4*>(reinterpret_cast<uintptr_t>(x) - mb);
  const u32x4* rw = RES ? reinterpret_cast<const u32x4*>(reinterpret_cast<uintptr_t>(res) - mb) : nullptr;
  u32x4* yw = reinterpret_cast<u32x4*>(reinterpret_cast<uintptr_t>(y) - mb);
  const int64_t total = rows * (int64_t)cols;
  const int64_t end_byte = mb + (int64_t)ES * total;  // tensor = bytes [mb, end_byte) of the windows

  const int64_t groups = (rows + RPB - 1) / RPB;
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
    const int64_t row = grp * RPB + sub;
    const bool live = row < rows;
    const int64_t e0 = (live ? row : rows - 1) * (int64_t)cols;  // past the end: reread the last row
    const int64_t off = mb + (int64_t)ES * e0;
    const int64_t q0 = off >> 4;
    const int s = (int)(off & 15) / ES;                              // row start within window q0
    const int nv = (int)(((off + (int64_t)ES * cols + 15) >> 4) - q0);  // windows overlapping the row

    u32x4 xv[VPL], rv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int j = lane + k * LANES;
      xv[k] = rv[k] = u32x4{{0u, 0u, 0u, 0u}};
      if (j < nv) {
        const int64_t q = q0 + j;
        if (16 * q >= mb && 16 * q + 16 <= end_byte) {
          xv[k] = load_nt(xw + q);
          if constexpr (RES) rv[k] = load_nt(rw + q);
        } else {
          // the first window of the tensor or its last: only elements inside
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const int64_t f = (16 * q + ES * e - mb) / ES;
            if (f >= 0 && f < total) {
              set_elem<IO>(xv[k], e, x[f]);
              if constexpr (RES) set_elem<IO>(rv[k], e, res[f]);
            }
          }
        }
      }
    }

    Val v[VPL][V];
    Acc sum = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int j = lane + k * LANES;
      const bool inrow = V * j - s >= 0 && V * j + V - s <= cols;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        Val t = (Val)IO::get(xv[k], e);
        if constexpr (RES) t += (Val)IO::get(rv[k], e);
        v[k][e] = t;
      }
      if (!inrow) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const int c = V * j + e - s;
          if (c < 0 || c >= cols) v[k][e] = 0;
        }
      }
#pragma unroll
      for (int e = 0; e < V; ++e) sum += (Acc)v[k][e];
    }
    const Acc mean = group_sum<LANES, BLOCK>(sum, red[0]) / (Acc)cols;

    Acc m2 = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int j = lane + k * LANES;
      const bool inrow = V * j - s >= 0 && V * j + V - s <= cols;
      Acc dd[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        dd[e] = (Acc)v[k][e] - mean;
        if constexpr (kInPlace) v[k][e] = dd[e];
      }
      if (!inrow) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const int c = V * j + e - s;
          if (c < 0 || c >= cols) dd[e] = 0;
        }
      }
      Acc part = 0;
#pragma unroll
      for (int e = 0; e < V; ++e) part = fma_t(dd[e], dd[e], part);
      m2 += part;
    }
    const Acc rstd = inv_sqrt(group_sum<LANES, BLOCK>(m2, red[1]) / (Acc)cols + eps);

#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int j = lane + k * LANES;
      if (!(live && j < nv)) continue;
      const float2* gbj = gb + (V * j - s + V);
      float o[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float2 p = gbj[e];
        const Acc d = kInPlace ? (Acc)v[k][e] : (Acc)v[k][e] - mean;
        o[e] = finish<Acc, GELU>(d, rstd, (Acc)p.x, (Acc)p.y);
      }
      if (V * j - s >= 0 && V * j + V - s <= cols) {
        store_nt(yw + q0 + j, pack_vec<IO>(o));
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const int c = V * j + e - s;
          if (c >= 0 && c < cols) IO::store1(y, e0 + c, o[e]);
        }
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
    const int i = pick_shape(cols / V + 2);
    if (i < 0) return hipErrorInvalidValue;
    k = shape_kernel<WinSel<IO, RES, GELU>::template K>(i);
    lanes = kShapes[i].lanes;
    lds = (size_t)(cols + 2 * V) * sizeof(float2);
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
  // Aligned rows: one block per row group (new blocks start as old ones finish,
  // which keeps more loads in flight than a persistent loop).  Windowed rows
  // stage gamma/beta in LDS per block, so a block takes several row groups.
  const int grid = aligned ? (int)(groups < kMaxGrid ? groups : kMaxGrid)
                           : persistent_grid(k, block, groups, lds);
  int icols = (int)cols;
  void* args[] = {&x, &res, &gamma, &beta, &y, &rows, &icols, &eps};
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
