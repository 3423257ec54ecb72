// fused_tenop.hip -- the 10-op graph of "TorchInductor Pipeline 与算子融合" (the
// model at the top of the post) as one persistent row kernel:
//
//   t = x*alpha + bias;  a = relu(t);  s = a*a + a*c;
//   m = (row sum of s) / cols   (section 6.4: a sum, then the division);
//   y = (s - m)*gamma + beta
//
// Section 8 of that post describes the fused kernel Inductor generates: one
// program per row, the row in registers, the row sums never written (section
// 02, Table 2: ~8 MiB of traffic instead of ~80 MiB).  Here a row lives in the
// registers of a lane group (row_common.hpp), s is computed once per element
// (the three copies of a in the lowered graph share one value), the row sum is
// reduced across the group, and the epilogue writes y.  Arithmetic is binary64
// (fp32 in and out), so the result is the exactly rounded value up to a few
// binary64 roundings.  Rows that do not start on 16-byte boundaries take the
// same kernel with one element per load.
#include "mbp_internal.hpp"
#include "row_common.hpp"

namespace mbp {
namespace {

using namespace rows;

// ---------------------------------------------------------------- 10-op graph

template <int LANES, int VPL, int VW>
__global__ __launch_bounds__(block_for(LANES)) void tenop_kernel(
    const float* x, const float* __restrict__ bias, const float* __restrict__ gamma,
    const float* __restrict__ beta, float* y, int64_t rows, int cols, double alpha, double c) {
  constexpr int BLOCK = block_for(LANES);
  constexpr int RPB = BLOCK / LANES;
  __shared__ double red[2][BLOCK / 64];

  const int lane = threadIdx.x % LANES;
  const int sub = threadIdx.x / LANES;
  const int nvec = (cols + VW - 1) / VW;

  float bi[VPL][VW], g[VPL][VW], be[VPL][VW];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int vi = lane + k * LANES;
#pragma unroll
    for (int e = 0; e < VW; ++e) {
      const int j = vi * VW + e;
      const bool ok = vi < nvec;
      bi[k][e] = ok ? bias[j] : 0.0f;
      g[k][e] = ok ? gamma[j] : 0.0f;
      be[k][e] = ok ? beta[j] : 0.0f;
    }
  }

  const int64_t groups = (rows + RPB - 1) / RPB;
  int parity = 0;
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x, parity ^= 1) {
    // the parameters stay fp32 across rows (see ln_kernel)
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        opaque(bi[k][e]);
        opaque(g[k][e]);
        opaque(be[k][e]);
      }
    const int64_t row = grp * RPB + sub;
    const bool live = row < rows;
    // past the last row: reread the last row, store nothing; slots past the
    // row's end reread its last vector and stay out of the sum (no branches)
    const float* xr = x + (live ? row : rows - 1) * (int64_t)cols;
    float* yr = y + row * (int64_t)cols;

    float xv[VPL][VW];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int vi = min(lane + k * LANES, nvec - 1);
      if constexpr (VW == 1) {
        xv[k][0] = xr[vi];
      } else {
        const float4 t = load_nt(reinterpret_cast<const float4*>(xr) + vi);
        xv[k][0] = t.x; xv[k][1] = t.y; xv[k][2] = t.z; xv[k][3] = t.w;
      }
    }
    double s[VPL][VW];
    double sum = 0.0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      double part = 0.0;
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        const double t = __builtin_fma((double)xv[k][e], alpha, (double)bi[k][e]);
        const double a = (t < 0.0) ? 0.0 : t;  // relu; NaN passes through
        s[k][e] = __builtin_fma(a, a, a * c);
        part += s[k][e];
      }
      if (lane + k * LANES < nvec) sum += part;
    }
    const double m = group_sum<LANES, BLOCK>(sum, red[parity]) / (double)cols;

#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int vi = lane + k * LANES;
      if (!(live && vi < nvec)) continue;
      float o[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e)
        o[e] = (float)__builtin_fma(s[k][e] - m, (double)g[k][e], (double)be[k][e]);
      if constexpr (VW == 1) {
        yr[vi] = o[0];
      } else {
        store_nt(reinterpret_cast<float4*>(yr) + vi, make_float4(o[0], o[1], o[2], o[3]));
      }
    }
  }
}


template <int VW>
struct TenopSel {
  template <int L, int V>
  struct K {
    static const void* ptr() { return reinterpret_cast<const void*>(&tenop_kernel<L, (VW == 1 ? 4 * V : V), VW>); }
  };
};

}  // namespace

hipError_t launch_row_mean(const float* x, const float* bias, const float* gamma,
                           const float* beta, float* y, int64_t rows, int64_t cols, double alpha,
                           double c, hipStream_t s) {
  const bool vector_ok = (cols % 4) == 0 && aligned16(x) && aligned16(bias) && aligned16(gamma) &&
                         aligned16(beta) && aligned16(y);
  // the scalar path holds 4x the vectors of a layout, one element each
  const int shape = pick_shape(vector_ok ? cols / 4 : (cols + 3) / 4);
  if (shape < 0) return hipErrorInvalidValue;
  const void* k = vector_ok ? shape_kernel<TenopSel<4>::K>(shape) : shape_kernel<TenopSel<1>::K>(shape);
  const int block = block_for(kShapes[shape].lanes);
  const int rpb = block / kShapes[shape].lanes;
  const int64_t groups = (rows + rpb - 1) / rpb;
  const int grid = (int)(groups < (1 << 30) ? groups : (1 << 30));  // one block per row group
  int icols = (int)cols;
  void* args[] = {&x, &bias, &gamma, &beta, &y, &rows, &icols, &alpha, &c};
  return hipLaunchKernel(k, dim3(grid), dim3(block), args, 0, s);
}

}  // namespace mbp
