// unfused.hip -- the deliberately unfused "before" variants: one launch per op,
// every intermediate stored to HBM in the I/O type and read back by the next
// launch, as eager execution does ("PyTorch operator-fusion practice post",
// section 1.1; "TorchInductor Pipeline 与算子融合", section 02 Table 2;
// "4、算子融合（Kernel Fusion）", section 4.3).
//
// Every element-wise op computes one correctly rounded fp32 operation on values
// widened exactly from the storage type and rounds the result once to the
// storage type (fp32, or bf16 round-to-nearest-even).  The explicit _rn
// intrinsics keep the compiler from contracting a multiply and an add.  Row
// reductions (mean, variance) accumulate in binary64 and store fp32.  The
// kernels stream with 128-bit loads/stores where every full-tensor operand is
// 16-byte aligned and the row length is a whole number of vectors, so the
// comparison with the fused kernels is one of bytes and launches, not of load
// width.
#include "mbp_device.hpp"
#include "mbp_internal.hpp"

namespace mbp {
namespace {

constexpr int kBlock = 256;
constexpr int64_t kMaxGrid = 1 << 30;

template <int OP>
__device__ __forceinline__ float ew_apply(float a, float b, float c, float scalar) {
  if constexpr (OP == EW_ADD) return __fadd_rn(a, b);
  if constexpr (OP == EW_SUB) return __fsub_rn(a, b);
  if constexpr (OP == EW_MUL) return __fmul_rn(a, b);
  if constexpr (OP == EW_RELU) return (a < 0.0f) ? 0.0f : a;
  if constexpr (OP == EW_MULS) return __fmul_rn(a, scalar);
  if constexpr (OP == EW_DIVSD) return __fdiv_rn(a, __fsqrt_rn(__fadd_rn(b, scalar)));
  if constexpr (OP == EW_MULADD) return __fadd_rn(__fmul_rn(a, b), c);
  if constexpr (OP == EW_GELU) return gelu_tanh_f32(a);
  return 0.0f;
}

// Operand of an element-wise op at flat index i (row = i / cols, col = i % cols).
template <class IO>
__device__ __forceinline__ float operand(const void* p, int ix, int64_t i, int64_t cols) {
  if (p == nullptr) return 0.0f;
  if (ix == IX_FULL) return IO::load1(static_cast<const typename IO::elem*>(p), i);
  if (ix == IX_COL) return IO::load1(static_cast<const typename IO::elem*>(p), i % cols);
  return static_cast<const float*>(p)[i / cols];
}

// One element per work item (VW == 1) or one 16-byte vector (VW == IO::kVec).
template <class IO, int OP, int VW>
__global__ __launch_bounds__(kBlock) void ew_kernel(const typename IO::elem* a, const void* b,
                                                    int b_ix, const void* c, int c_ix,
                                                    typename IO::elem* out, int64_t n,
                                                    int64_t cols, float scalar) {
  const int64_t items = n / VW;
  for (int64_t it = (int64_t)blockIdx.x * kBlock + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * kBlock) {
    if constexpr (VW == 1) {
      const float r = ew_apply<OP>(IO::load1(a, it), operand<IO>(b, b_ix, it, cols),
                                   operand<IO>(c, c_ix, it, cols), scalar);
      IO::store1(out, it, r);
    } else {
      const int64_t i0 = it * VW;
      const u32x4 av = reinterpret_cast<const u32x4*>(a)[it];
      u32x4 bv = {{0u, 0u, 0u, 0u}}, cv = {{0u, 0u, 0u, 0u}};
      if (b && b_ix == IX_FULL) bv = reinterpret_cast<const u32x4*>(b)[it];
      if (b && b_ix == IX_COL) bv = reinterpret_cast<const u32x4*>(b)[(i0 % cols) / VW];
      if (c && c_ix == IX_COL) cv = reinterpret_cast<const u32x4*>(c)[(i0 % cols) / VW];
      const float brow = (b && b_ix == IX_ROW) ? static_cast<const float*>(b)[i0 / cols] : 0.0f;
      float r[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        const float bb = (b_ix == IX_ROW) ? brow : IO::get(bv, e);
        r[e] = ew_apply<OP>(IO::get(av, e), bb, IO::get(cv, e), scalar);
      }
      u32x4 ov;
      if constexpr (VW == 8) {
#pragma unroll
        for (int w = 0; w < 4; ++w) ov.w[w] = pack_bf16x2(r[2 * w], r[2 * w + 1]);
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) ov.w[w] = __float_as_uint(r[w]);
      }
      reinterpret_cast<u32x4*>(out)[it] = ov;
    }
  }
}

// Row statistics: one 256-lane block per row (blocks stride over rows); each
// lane sums its columns j = lane, lane + 256, ... in binary64, then a fixed-order
// block reduction.  MODE 0: mean; MODE 1: biased variance about `mean`.
template <class IO, int MODE>
__global__ __launch_bounds__(kBlock) void row_stat_kernel(const typename IO::elem* a,
                                                          const float* mean, float* out,
                                                          int64_t rows, int64_t cols) {
  __shared__ double red[2][kBlock / 64];
  int parity = 0;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x, parity ^= 1) {
    const typename IO::elem* ar = a + row * cols;
    const double mu = MODE == 1 ? (double)mean[row] : 0.0;
    double acc = 0.0;
    for (int64_t j = threadIdx.x; j < cols; j += kBlock) {
      const double v = (double)IO::load1(ar, j);
      if constexpr (MODE == 0) {
        acc += v;
      } else {
        const double d = v - mu;
        acc += d * d;
      }
    }
    const double tot = group_sum<kBlock, kBlock>(acc, red[parity]);
    if (threadIdx.x == 0) out[row] = (float)(tot / (double)cols);
  }
}

template <class IO, int VW>
const void* ew_ptr(int op) {
  switch (op) {
    case EW_ADD: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_ADD, VW>);
    case EW_SUB: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_SUB, VW>);
    case EW_MUL: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_MUL, VW>);
    case EW_RELU: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_RELU, VW>);
    case EW_MULS: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_MULS, VW>);
    case EW_DIVSD: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_DIVSD, VW>);
    case EW_MULADD: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_MULADD, VW>);
    case EW_GELU: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_GELU, VW>);
    default: return nullptr;
  }
}

bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_ew(int op, int dtype, const void* a, const void* b, int b_ix, const void* c,
                     int c_ix, void* out, int64_t rows, int64_t cols, float scalar,
                     hipStream_t s) {
  const int64_t n = rows * cols;
  const int vec = dtype == 1 ? 8 : 4;
  bool vector_ok = (cols % vec) == 0 && a16(a) && a16(out);
  if (b && b_ix != IX_ROW) vector_ok = vector_ok && a16(b);
  if (c) vector_ok = vector_ok && a16(c);
  const int vw = vector_ok ? vec : 1;
  const void* k = dtype == 1 ? (vector_ok ? ew_ptr<BF16IO, 8>(op) : ew_ptr<BF16IO, 1>(op))
                             : (vector_ok ? ew_ptr<F32IO, 4>(op) : ew_ptr<F32IO, 1>(op));
  if (!k) return hipErrorInvalidValue;
  int64_t grid = (n / vw + kBlock - 1) / kBlock;
  if (grid > kMaxGrid) grid = kMaxGrid;
  if (grid < 1) grid = 1;
  void* args[] = {&a, &b, &b_ix, &c, &c_ix, &out, (void*)&n, &cols, &scalar};
  return hipLaunchKernel(k, dim3((unsigned)grid), dim3(kBlock), args, 0, s);
}

hipError_t launch_row_mean_only(int dtype, const void* a, float* mean, int64_t rows,
                                int64_t cols, hipStream_t s) {
  const void* k = dtype == 1 ? reinterpret_cast<const void*>(&row_stat_kernel<BF16IO, 0>)
                             : reinterpret_cast<const void*>(&row_stat_kernel<F32IO, 0>);
  const float* none = nullptr;
  const int grid = persistent_grid(k, kBlock, rows, 0);
  void* args[] = {&a, &none, &mean, &rows, &cols};
  return hipLaunchKernel(k, dim3(grid), dim3(kBlock), args, 0, s);
}

hipError_t launch_row_var(int dtype, const void* a, const float* mean, float* var, int64_t rows,
                          int64_t cols, hipStream_t s) {
  const void* k = dtype == 1 ? reinterpret_cast<const void*>(&row_stat_kernel<BF16IO, 1>)
                             : reinterpret_cast<const void*>(&row_stat_kernel<F32IO, 1>);
  const int grid = persistent_grid(k, kBlock, rows, 0);
  void* args[] = {&a, &mean, &var, &rows, &cols};
  return hipLaunchKernel(k, dim3(grid), dim3(kBlock), args, 0, s);
}

}  // namespace mbp
