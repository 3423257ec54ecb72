// fused_rows.hip -- one-pass row kernels: a reduction fused with its pointwise
// prologue and epilogue, so that a row is read from HBM once, lives in
// registers while its statistics are reduced, and is written once.
//
//  * tenop_kernel: the 10-op graph of "TorchInductor Pipeline 与算子融合" (the
//    model at the top of the post): t = x*alpha + bias, a = relu(t),
//    s = a*a + a*c, m = row sum of s / cols (section 6.4), y = (s - m)*gamma +
//    beta.  Section 8 of that post describes the persistent reduction that keeps
//    a row in registers and never writes the row sums (section 02, Table 2:
//    ~8 MiB instead of ~80 MiB of traffic).  Arithmetic: binary64.
//  * ln_kernel: residual add + LayerNorm + tanh-GeLU ("算子融合与 Kernel 优化",
//    section 2.3; LayerNorm as in "4、算子融合（Kernel Fusion）", section 4.3).
//    Two-pass statistics over the register-resident row: the mean first, then
//    the sum of squared deviations from it (the pages' one-pass E[x^2] - mean^2
//    loses the variance when |mean| >> std).  fp32 I/O computes in binary64;
//    bf16 I/O computes in fp32.
//
// Layout.  A row is served by a group of LANES consecutive lanes (16 ... 1024).
// Lane l of the group holds the vectors l, l + LANES, l + 2*LANES, ... of the
// row (VPL of them), so each load instruction of the group covers a contiguous
// stretch of the row (coalesced).  A vector is 16 bytes (4 fp32 / 8 bf16) on the
// 128-bit path or one element on the scalar path (rows whose start is not
// 16-byte aligned).  A block holds block / LANES rows;
// blocks are persistent (no more than can be resident) and stride over the row
// groups, so gamma, beta and bias are loaded into registers once per block.
// Groups of up to 256 lanes run in 256-lane blocks; wider groups are one block.
// Row sums: xor butterfly inside a wave (identical in every lane), LDS only
// across the waves of a group wider than 64 lanes (mbp::group_sum).
#include "mbp_device.hpp"
#include "mbp_internal.hpp"

#include <type_traits>

namespace mbp {
namespace {

constexpr int kMinBlock = 256;

// Block size for a group of LANES lanes: at least kMinBlock, one group if wider.
constexpr int block_for(int lanes) { return lanes > kMinBlock ? lanes : kMinBlock; }

// An empty asm that claims to rewrite its operand: the value is unchanged, but
// the compiler must treat it as new at this point of the program.
__device__ __forceinline__ void opaque(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(uint16_t& v) {
  uint32_t t = v;
  asm volatile("" : "+v"(t));
  v = (uint16_t)t;
}
__device__ __forceinline__ void opaque(u32x4& v) {
#pragma unroll
  for (int w = 0; w < 4; ++w) opaque(v.w[w]);
}

template <typename T>
__device__ __forceinline__ T div_by(T a, int cols) {
  return a / (T)cols;
}

__device__ __forceinline__ float inv_sqrt(float a) { return 1.0f / __builtin_sqrtf(a); }
__device__ __forceinline__ double inv_sqrt(double a) { return 1.0 / __builtin_sqrt(a); }

// ---------------------------------------------------------------- LayerNorm

// Row values are held as V: fp32 for bf16 I/O and for fp32 I/O without a
// residual (v = x exactly), binary64 for fp32 I/O with a residual (the exact
// sum x + r).  Statistics accumulate in Acc: fp32 for bf16 I/O, binary64 for
// fp32 I/O.
template <class IO, bool WIDE>
struct LnTypes {
  typedef float acc;
  typedef float val;
};
template <bool WIDE>
struct LnTypes<F32IO, WIDE> {
  typedef double acc;
  typedef typename std::conditional<WIDE, double, float>::type val;
};

// x and res may alias y (in place): every element of a row is loaded before
// the row's reductions complete, and the stores depend on those reductions.
template <class IO, int LANES, int VPL, int VW, bool WIDE>
__global__ __launch_bounds__(block_for(LANES)) void ln_kernel(
    const typename IO::elem* x, const typename IO::elem* res,
    const typename IO::elem* __restrict__ gamma, const typename IO::elem* __restrict__ beta,
    typename IO::elem* y, int64_t rows, int cols, double eps_d, int gelu) {
  typedef typename IO::elem E;
  typedef typename LnTypes<IO, WIDE>::acc Acc;
  typedef typename LnTypes<IO, WIDE>::val Val;
  typedef typename std::conditional<VW == 1, E, u32x4>::type Raw;
  constexpr int BLOCK = block_for(LANES);
  constexpr int RPB = BLOCK / LANES;
  __shared__ Acc red[2][BLOCK / 64];

  const int lane = threadIdx.x % LANES;
  const int sub = threadIdx.x / LANES;
  const int nvec = (cols + VW - 1) / VW;  // VW divides cols on the vector path
  const Acc eps = (Acc)eps_d;

  auto get = [](const Raw& r, int e) -> float {
    if constexpr (VW == 1) {
      if constexpr (sizeof(E) == 2) return bf16_to_f32(r);
      else return r;
    } else {
      return IO::get(r, e);
    }
  };

  // gamma / beta of this lane's columns, kept in their storage form for the
  // whole block (widened at use: one shift or mask per bf16 element)
  Raw graw[VPL], braw[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int vi = lane + k * LANES;
    if (vi < nvec) {
      graw[k] = reinterpret_cast<const Raw*>(gamma)[vi];
      braw[k] = reinterpret_cast<const Raw*>(beta)[vi];
    } else {
      graw[k] = braw[k] = Raw{};
    }
  }

  const int64_t groups = (rows + RPB - 1) / RPB;
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
    // Keep gamma/beta in storage form across rows: opaque() hides their value
    // from the optimiser once per iteration, so their widening (to fp32, or to
    // binary64) cannot be hoisted out of the row loop, which would double or
    // quadruple the registers they occupy.
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      opaque(graw[k]);
      opaque(braw[k]);
    }
    const int64_t row = grp * RPB + sub;
    const bool live = row < rows;
    const Raw* xr = reinterpret_cast<const Raw*>(x + row * (int64_t)cols);
    const Raw* rr = res ? reinterpret_cast<const Raw*>(res + row * (int64_t)cols) : nullptr;
    Raw* yr = reinterpret_cast<Raw*>(y + row * (int64_t)cols);

    // load (+ residual) and row sum
    Val v[VPL][VW];
    Acc sum = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int vi = lane + k * LANES;
      Raw xv{}, rv{};
      if (live && vi < nvec) {
        xv = xr[vi];
        if (rr) rv = rr[vi];
      }
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        Val t = (Val)get(xv, e);
        if (rr) t += (Val)get(rv, e);
        v[k][e] = t;
        sum += (Acc)t;
      }
    }
    const Acc mean = div_by(group_sum<LANES, BLOCK>(sum, red[0]), cols);

    // sum of squared deviations over the row's own elements
    Acc m2 = 0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int vi = lane + k * LANES;
      Acc part = 0;
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        const Acc d = (Acc)v[k][e] - mean;
        part = __builtin_fma(d, d, part);
      }
      if (live && vi < nvec) m2 += part;
    }
    const Acc var = div_by(group_sum<LANES, BLOCK>(m2, red[1]), cols);
    const Acc rstd = inv_sqrt(var + eps);

    // normalise, affine, optional GeLU, store
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int vi = lane + k * LANES;
      if (!(live && vi < nvec)) continue;
      float o[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        const Acc d = (Acc)v[k][e] - mean;
        const float u = (float)__builtin_fma(d * rstd, (Acc)get(graw[k], e), (Acc)get(braw[k], e));
        o[e] = gelu ? gelu_tanh_f32(u) : u;
      }
      if constexpr (VW == 1) {
        IO::store1(reinterpret_cast<E*>(yr), vi, o[0]);
      } else {
        u32x4 ov;
        if constexpr (sizeof(E) == 2) {
#pragma unroll
          for (int w = 0; w < 4; ++w) ov.w[w] = pack_bf16x2(o[2 * w], o[2 * w + 1]);
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) ov.w[w] = __float_as_uint(o[w]);
        }
        yr[vi] = ov;
      }
    }
  }
}

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
    const float* xr = x + row * (int64_t)cols;
    float* yr = y + row * (int64_t)cols;

    double s[VPL][VW];
    double sum = 0.0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int vi = lane + k * LANES;
      float xv[VW] = {};
      const bool ok = live && vi < nvec;
      if (ok) {
        if constexpr (VW == 1) {
          xv[0] = xr[vi];
        } else {
          const float4 t = reinterpret_cast<const float4*>(xr)[vi];
          xv[0] = t.x; xv[1] = t.y; xv[2] = t.z; xv[3] = t.w;
        }
      }
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        const double t = __builtin_fma((double)xv[e], alpha, (double)bi[k][e]);
        const double a = (t < 0.0) ? 0.0 : t;  // relu; NaN passes through
        const double sv = __builtin_fma(a, a, a * c);
        s[k][e] = ok ? sv : 0.0;
        sum += s[k][e];
      }
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
        reinterpret_cast<float4*>(yr)[vi] = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

// ---------------------------------------------------------------- dispatch

// (LANES, VPL) candidates in order of preference; the first whose LANES * VPL
// vectors cover the row is used.  Vector paths hold at most 4 vectors (16 fp32
// or 32 bf16 values) per lane, the scalar path at most 16 values, which keeps
// every kernel free of register spills; wider rows take wider groups.
struct Shape {
  int lanes, vpl;
};
constexpr Shape kVecShapes[] = {{16, 2},  {32, 2},  {32, 3},  {32, 4},  {64, 4},   {128, 4},
                                {256, 3}, {256, 4}, {512, 3}, {512, 4}, {1024, 3}, {1024, 4}};
constexpr Shape kScalarShapes[] = {{16, 8},   {32, 8},   {64, 8},    {128, 8},
                                   {256, 8},  {256, 12}, {256, 16},  {512, 12},
                                   {512, 16}, {1024, 12}, {1024, 16}};
constexpr int kNumVec = sizeof(kVecShapes) / sizeof(Shape);
constexpr int kNumScalar = sizeof(kScalarShapes) / sizeof(Shape);

int pick_shape(const Shape* table, int n, int64_t nvec) {
  for (int i = 0; i < n; ++i)
    if ((int64_t)table[i].lanes * table[i].vpl >= nvec) return i;
  return -1;
}

// Kernel pointer for shape i of the vector (VW > 1) or scalar table.
template <template <int, int> class K, bool VEC>
const void* shape_kernel(int i) {
  if constexpr (VEC) {
    switch (i) {
      case 0: return K<16, 2>::ptr();
      case 1: return K<32, 2>::ptr();
      case 2: return K<32, 3>::ptr();
      case 3: return K<32, 4>::ptr();
      case 4: return K<64, 4>::ptr();
      case 5: return K<128, 4>::ptr();
      case 6: return K<256, 3>::ptr();
      case 7: return K<256, 4>::ptr();
      case 8: return K<512, 3>::ptr();
      case 9: return K<512, 4>::ptr();
      case 10: return K<1024, 3>::ptr();
      default: return K<1024, 4>::ptr();
    }
  } else {
    switch (i) {
      case 0: return K<16, 8>::ptr();
      case 1: return K<32, 8>::ptr();
      case 2: return K<64, 8>::ptr();
      case 3: return K<128, 8>::ptr();
      case 4: return K<256, 8>::ptr();
      case 5: return K<256, 12>::ptr();
      case 6: return K<256, 16>::ptr();
      case 7: return K<512, 12>::ptr();
      case 8: return K<512, 16>::ptr();
      case 9: return K<1024, 12>::ptr();
      default: return K<1024, 16>::ptr();
    }
  }
}

template <class IO, int VW, bool WIDE>
struct LnSel {
  template <int L, int V>
  struct K {
    static const void* ptr() { return reinterpret_cast<const void*>(&ln_kernel<IO, L, V, VW, WIDE>); }
  };
};

template <int VW>
struct TenopSel {
  template <int L, int V>
  struct K {
    static const void* ptr() { return reinterpret_cast<const void*>(&tenop_kernel<L, V, VW>); }
  };
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_layernorm(int dtype, const void* x, const void* residual, const void* gamma,
                            const void* beta, void* y, int64_t rows, int64_t cols, double eps,
                            int act, hipStream_t s) {
  const int es = dtype == 1 ? 2 : 4;
  const int vec = 16 / es;
  const bool vector_ok = (cols % vec) == 0 && aligned16(x) && aligned16(gamma) &&
                         aligned16(beta) && aligned16(y) && (!residual || aligned16(residual));
  const Shape* table = vector_ok ? kVecShapes : kScalarShapes;
  const int shape = pick_shape(table, vector_ok ? kNumVec : kNumScalar, vector_ok ? cols / vec : cols);
  if (shape < 0) return hipErrorInvalidValue;
  const bool wide = residual != nullptr;
  const void* k;
  if (dtype == 1)
    k = vector_ok ? shape_kernel<LnSel<BF16IO, 8, false>::K, true>(shape)
                  : shape_kernel<LnSel<BF16IO, 1, false>::K, false>(shape);
  else if (wide)
    k = vector_ok ? shape_kernel<LnSel<F32IO, 4, true>::K, true>(shape)
                  : shape_kernel<LnSel<F32IO, 1, true>::K, false>(shape);
  else
    k = vector_ok ? shape_kernel<LnSel<F32IO, 4, false>::K, true>(shape)
                  : shape_kernel<LnSel<F32IO, 1, false>::K, false>(shape);
  const int block = block_for(table[shape].lanes);
  const int rpb = block / table[shape].lanes;
  const int grid = persistent_grid(k, block, (rows + rpb - 1) / rpb);
  int icols = (int)cols;
  int gelu = act == 1 ? 1 : 0;
  void* args[] = {&x, &residual, &gamma, &beta, &y, &rows, &icols, &eps, &gelu};
  return hipLaunchKernel(k, dim3(grid), dim3(block), args, 0, s);
}

hipError_t launch_row_mean(const float* x, const float* bias, const float* gamma,
                           const float* beta, float* y, int64_t rows, int64_t cols, double alpha,
                           double c, hipStream_t s) {
  const bool vector_ok = (cols % 4) == 0 && aligned16(x) && aligned16(bias) && aligned16(gamma) &&
                         aligned16(beta) && aligned16(y);
  const Shape* table = vector_ok ? kVecShapes : kScalarShapes;
  const int shape = pick_shape(table, vector_ok ? kNumVec : kNumScalar, vector_ok ? cols / 4 : cols);
  if (shape < 0) return hipErrorInvalidValue;
  const void* k = vector_ok ? shape_kernel<TenopSel<4>::K, true>(shape)
                            : shape_kernel<TenopSel<1>::K, false>(shape);
  const int block = block_for(table[shape].lanes);
  const int rpb = block / table[shape].lanes;
  const int grid = persistent_grid(k, block, (rows + rpb - 1) / rpb);
  int icols = (int)cols;
  void* args[] = {&x, &bias, &gamma, &beta, &y, &rows, &icols, &alpha, &c};
  return hipLaunchKernel(k, dim3(grid), dim3(block), args, 0, s);
}

}  // namespace mbp
