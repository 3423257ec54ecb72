// fused_softmax.hip -- row softmax as one pass over each row: the "Reduce +
// Element-wise" pattern of "4、算子融合（Kernel Fusion）", section 4.2, with the
// online statistics of the PyTorch operator-fusion practice post, section 4.2
// (and "算子融合与 Kernel 优化", section 3.2, step 3):
//
//   m = max_j x_j;   l = sum_j exp(x_j - m);   y_j = exp(x_j - m) / l
//
// The row is loaded once into the registers of a lane group (the layouts of
// row_common.hpp).  Each lane reduces its own elements to a (max, sum) pair
// relative to its own maximum; the pairs are merged across the group with the
// pages' running-max rule -- a larger maximum rescales the other sum by
// exp(m_old - m_new) -- so the two statistics cost one group reduction, not
// two.  The merge is symmetric and IEEE addition commutes, so both partners
// of every butterfly exchange get the same pair and the result does not depend
// on timing.  The output is exp(x_j - m_lane) * (exp(m_lane - m) / l): one
// exponential per element.  Arithmetic in fp32 (fp32, bf16 or fp16 storage;
// one rounding at the store).  -inf entries (masks) give exactly 0; a row of
// -inf only gives NaN (0 / 0, as the definition); a NaN makes its row NaN.
#include "mbp_internal.hpp"
#include "row_common.hpp"

namespace mbp {
namespace {

using namespace rows;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp_f(float v) { return __builtin_amdgcn_exp2f(v * kLog2e); }

// Merge of two (max, sum) pairs, each sum relative to its own max.
__device__ __forceinline__ void ms_merge(float& m, float& l, float om, float ol) {
  const float M = __builtin_fmaxf(m, om);
  const float a = (m == M) ? l : l * exp_f(m - M);
  const float b = (om == M) ? ol : ol * exp_f(om - M);
  m = M;
  l = a + b;
}

template <int LANES, int BLOCK>
__device__ __forceinline__ void group_merge(float& m, float& l, float* lds_m, float* lds_l) {
  constexpr int kIn = LANES < 64 ? LANES : 64;
#pragma unroll
  for (int k = 1; k < kIn; k <<= 1) {
    const float om = __shfl_xor(m, k), ol = __shfl_xor(l, k);
    ms_merge(m, l, om, ol);
  }
  if constexpr (LANES > 64) {
    constexpr int kWaves = LANES / 64;
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      lds_m[wave] = m;
      lds_l[wave] = l;
    }
    lds_barrier();
    const int first = (threadIdx.x / LANES) * kWaves;
    m = lds_m[first];
    l = lds_l[first];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) ms_merge(m, l, lds_m[first + w], lds_l[first + w]);
  }
}

// VW: elements per access (IO::kVec: 16-byte vectors, rows on 16-byte
// boundaries; 1: one element).  VPL accesses per lane.  One block per row group.
template <class IO, int LANES, int VPL, int VW>
__global__ __launch_bounds__(block_for(LANES)) void softmax_kernel(const typename IO::elem* x,
                                                                   typename IO::elem* y, int64_t rows,
                                                                   int cols) {
  typedef typename IO::elem E;
  constexpr int BLOCK = block_for(LANES);
  constexpr int RPB = BLOCK / LANES;
  __shared__ float lds_m[BLOCK / 64 > 0 ? BLOCK / 64 : 1], lds_l[BLOCK / 64 > 0 ? BLOCK / 64 : 1];

  const int lane = threadIdx.x % LANES;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LANES;
  const bool live = row < rows;
  const int nvec = (cols + VW - 1) / VW;
  // past the last row: reread the last row, store nothing
  const E* xr = x + (live ? row : rows - 1) * (int64_t)cols;
  E* yr = y + row * (int64_t)cols;

  float v[VPL][VW];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int vi = min(lane + k * LANES, nvec - 1);
    if constexpr (VW == 1) {
      v[k][0] = IO::load1(xr, vi);
    } else {
      const u32x4 t = load_nt(reinterpret_cast<const u32x4*>(xr) + vi);
#pragma unroll
      for (int e = 0; e < VW; ++e) v[k][e] = IO::get(t, e);
    }
    if (lane + k * LANES >= nvec) {  // slot past the row: no contribution
#pragma unroll
      for (int e = 0; e < VW; ++e) v[k][e] = -__builtin_inff();
    }
  }

  // this lane's (max, sum); a lane with only -inf has (-inf, 0)
  float m = -__builtin_inff();
#pragma unroll
  for (int k = 0; k < VPL; ++k)
#pragma unroll
    for (int e = 0; e < VW; ++e) m = __builtin_fmaxf(m, v[k][e]);
  const float mm = (m == -__builtin_inff()) ? 0.0f : m;
  float l = 0.0f;
#pragma unroll
  for (int k = 0; k < VPL; ++k)
#pragma unroll
    for (int e = 0; e < VW; ++e) {
      v[k][e] = exp_f(v[k][e] - mm);
      l += v[k][e];
    }
  const float m_lane = m;
  group_merge<LANES, BLOCK>(m, l, lds_m, lds_l);
  // per-lane factor exp(m_lane - M) / L; 0 for a lane of masked entries;
  // NaN for a row of -inf only (0 / 0)
  float f;
  if (m == -__builtin_inff()) f = __builtin_nanf("");
  else if (m_lane == -__builtin_inff()) f = 0.0f;
  else f = exp_f(m_lane - m) / l;
  if (!live) return;

#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int vi = lane + k * LANES;
    if (vi >= nvec) continue;
    if constexpr (VW == 1) {
      IO::store1(yr, vi, v[k][0] * f);
    } else {
      u32x4 ov;
      if constexpr (sizeof(E) == 4) {
#pragma unroll
        for (int w = 0; w < 4; ++w) ov.w[w] = __float_as_uint(v[k][w] * f);
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (IO::kVec == 8 && __is_same(IO, BF16IO))
            ov.w[w] = pack_bf16x2(v[k][2 * w] * f, v[k][2 * w + 1] * f);
          else
            ov.w[w] = (uint32_t)f32_to_f16(v[k][2 * w] * f) | ((uint32_t)f32_to_f16(v[k][2 * w + 1] * f) << 16);
        }
      }
      store_nt(reinterpret_cast<u32x4*>(yr) + vi, ov);
    }
  }
}

template <class IO, bool VEC>
struct SoftmaxSel {
  template <int L, int V>
  struct K {
    static const void* ptr() {
      return VEC ? reinterpret_cast<const void*>(&softmax_kernel<IO, L, V, IO::kVec>)
                 : reinterpret_cast<const void*>(&softmax_kernel<IO, L, IO::kVec * V, 1>);
    }
  };
};

template <class IO>
hipError_t launch_softmax_io(const void* x, void* y, int64_t rows, int64_t cols, hipStream_t s) {
  typedef typename IO::elem E;
  constexpr int V = IO::kVec;
  const bool vec = cols % V == 0 && aligned16(x) && aligned16(y);
  const int shape = pick_shape((cols + V - 1) / V);
  if (shape < 0) return hipErrorInvalidValue;
  const void* k = vec ? shape_kernel<SoftmaxSel<IO, true>::template K>(shape)
                      : shape_kernel<SoftmaxSel<IO, false>::template K>(shape);
  const int block = block_for(kShapes[shape].lanes);
  const int rpb = block / kShapes[shape].lanes;
  const int64_t groups = (rows + rpb - 1) / rpb;
  const int grid = (int)(groups < (1 << 30) ? groups : (1 << 30));
  if (groups > grid) return hipErrorInvalidValue;  // one block per row group
  const E* xe = static_cast<const E*>(x);
  E* ye = static_cast<E*>(y);
  int icols = (int)cols;
  void* args[] = {&xe, &ye, &rows, &icols};
  return hipLaunchKernel(k, dim3(grid), dim3(block), args, 0, s);
}

}  // namespace

hipError_t launch_softmax(int dtype, const void* x, void* y, int64_t rows, int64_t cols, hipStream_t s) {
  if (dtype == 0) return launch_softmax_io<F32IO>(x, y, rows, cols, s);
  if (dtype == 1) return launch_softmax_io<BF16IO>(x, y, rows, cols, s);
  return launch_softmax_io<F16IO>(x, y, rows, cols, s);
}

}  // namespace mbp
