// fused_pointwise.hip -- the fused pointwise chain y = relu(x + b1) * scale + b2
// and the plain streaming copy used for bandwidth calibration.
//
// The chain is the example of the PyTorch operator-fusion practice post
// (0539edu.com), section 1.1 (four eager kernels add -> relu -> mul -> add, each
// a full HBM round trip) and section 3.2 (one fused kernel with 16-byte loads).
// Here one launch reads x, b1, b2 once and writes y once (16 bytes per element),
// with 128-bit nontemporal loads/stores on the aligned body and scalar handling
// of the unaligned head and the n % 4 tail.  The arithmetic is binary64: the exact sum
// x + b1 (rounded once to binary64), the relu select, one fused multiply-add with
// b2, and one rounding to fp32 at the store.  On gfx950 binary64 FMA runs at the
// same lane rate as fp32, and this kernel needs about 8 VALU ops per 16 bytes.
#include "mbp_device.hpp"
#include "mbp_internal.hpp"

namespace mbp {
namespace {

constexpr int kBlock = 256;
constexpr int kChainUnroll = 1;
constexpr int64_t kMaxGrid = dispatch_blocks(kBlock);  // every kernel here loops over its items

__device__ __forceinline__ float chain_op(float x, float b1, float b2, double scale) {
  const double t = (double)x + (double)b1;
  const double r = (t < 0.0) ? 0.0 : t;  // relu; a NaN passes through
  return (float)__builtin_fma(r, scale, (double)b2);
}

// Work items of one launch: [0, n4) are float4 vectors of the aligned body
// (elements h .. h + 4*n4), [n4, n4 + nscal) are single elements: the head
// [0, h) and the tail [h + 4*n4, n).  A block covers kBlock * U consecutive
// items; blocks stride over the item range so any n fits the grid.
template <int U>
__global__ __launch_bounds__(kBlock) void chain_kernel(const float* x, const float* b1,
                                                       const float* b2, float* y, int64_t h,
                                                       int64_t n4, int64_t nscal, double scale) {
  const float4* X = reinterpret_cast<const float4*>(x + h);
  const float4* A = reinterpret_cast<const float4*>(b1 + h);
  const float4* B = reinterpret_cast<const float4*>(b2 + h);
  float4* Y = reinterpret_cast<float4*>(y + h);
  const int64_t items = n4 + nscal;
  const int64_t nblk = (items + kBlock * U - 1) / (kBlock * U);
  for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int64_t base = blk * (kBlock * U) + threadIdx.x;
    float4 xv[U], av[U], bv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * kBlock;
      if (i < n4) {
        xv[u] = load_nt(X + i);
        av[u] = load_nt(A + i);
        bv[u] = load_nt(B + i);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * kBlock;
      if (i < n4) {
        float4 o;
        o.x = chain_op(xv[u].x, av[u].x, bv[u].x, scale);
        o.y = chain_op(xv[u].y, av[u].y, bv[u].y, scale);
        o.z = chain_op(xv[u].z, av[u].z, bv[u].z, scale);
        o.w = chain_op(xv[u].w, av[u].w, bv[u].w, scale);
        store_nt(Y + i, o);
      } else if (i < items) {
        const int64_t k = i - n4;
        const int64_t e = (k < h) ? k : 4 * n4 + k;
        y[e] = chain_op(x[e], b1[e], b2[e], scale);
      }
    }
  }
}

// Two-dimensional form: rows x cols, a row stride per operand (0: one row
// used for every row), fp32 / bf16 / fp16 storage.  An item is one 16-byte
// vector of a row (VW = IO::kVec; every operand row starts on a 16-byte
// boundary and cols is a whole number of vectors) or one element (VW = 1).
// Binary64 arithmetic as above, one rounding to the storage type at the store.
template <class IO>
__device__ __forceinline__ double chain_op_d(float x, float b1, float b2, double scale) {
  const double t = (double)x + (double)b1;
  const double r = (t < 0.0) ? 0.0 : t;
  return __builtin_fma(r, scale, (double)b2);
}

template <class IO, int VW>
__global__ __launch_bounds__(kBlock) void chain2d_kernel(
    const typename IO::elem* x, int64_t ldx, const typename IO::elem* b1, int64_t ldb1,
    const typename IO::elem* b2, int64_t ldb2, typename IO::elem* y, int64_t ldy, int64_t rows,
    int64_t cols, double scale) {
  typedef typename IO::elem E;
  const int64_t per_row = cols / VW;
  const int64_t items = rows * per_row;
  for (int64_t it = (int64_t)blockIdx.x * kBlock + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * kBlock) {
    const int64_t row = it / per_row;
    const int64_t c0 = (it - row * per_row) * VW;
    if constexpr (VW == 1) {
      const double r = chain_op_d<IO>(IO::load1(x, row * ldx + c0), IO::load1(b1, row * ldb1 + c0),
                                      IO::load1(b2, row * ldb2 + c0), scale);
      const uint32_t bits = narrow_bits<IO>(r);
      if constexpr (sizeof(E) == 4) y[row * ldy + c0] = __uint_as_float(bits);
      else y[row * ldy + c0] = (uint16_t)bits;
    } else {
      const u32x4 xv = load_nt(reinterpret_cast<const u32x4*>(x + row * ldx + c0));
      const u32x4 av = *reinterpret_cast<const u32x4*>(b1 + row * ldb1 + c0);
      const u32x4 bv = *reinterpret_cast<const u32x4*>(b2 + row * ldb2 + c0);
      u32x4 ov = {{0u, 0u, 0u, 0u}};
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        const uint32_t bits =
            narrow_bits<IO>(chain_op_d<IO>(IO::get(xv, e), IO::get(av, e), IO::get(bv, e), scale));
        if constexpr (sizeof(E) == 4) ov.w[e] = bits;
        else ov.w[e >> 1] |= bits << (16 * (e & 1));
      }
      store_nt(reinterpret_cast<u32x4*>(y + row * ldy + c0), ov);
    }
  }
}

// Element path for rows of at least kRowBlockCols elements: a block takes a
// whole row (blocks stride over rows).  Its threads start at the row's first
// 128-byte line boundary of x (the head before it taken by the first
// threads), so each block-wide access covers whole lines of x: with the flat
// mapping above a block's 256-element run starts wherever the row does, and
// the line it shares with the next block -- which runs on another XCD, with
// another L2 -- was fetched twice (12% more reads measured on [8192, 4095]
// fp32 rows one element off 16-byte boundaries).  No per-element division.
constexpr int64_t kRowBlockCols = 1024;

template <class IO>
__device__ __forceinline__ void chain_elem(const typename IO::elem* xr, const typename IO::elem* ar,
                                           const typename IO::elem* br, typename IO::elem* yr, int64_t c,
                                           double scale) {
  const uint32_t bits = narrow_bits<IO>(chain_op_d<IO>(IO::load1(xr, c), IO::load1(ar, c), IO::load1(br, c), scale));
  if constexpr (sizeof(typename IO::elem) == 4) yr[c] = __uint_as_float(bits);
  else yr[c] = (uint16_t)bits;
}

template <class IO>
__global__ __launch_bounds__(kBlock) void chain2d_rows_kernel(
    const typename IO::elem* x, int64_t ldx, const typename IO::elem* b1, int64_t ldb1,
    const typename IO::elem* b2, int64_t ldb2, typename IO::elem* y, int64_t ldy, int64_t rows,
    int64_t cols, double scale) {
  typedef typename IO::elem E;
  constexpr int ES = (int)sizeof(E);
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const E* xr = x + row * ldx;
    const E* ar = b1 + row * ldb1;
    const E* br = b2 + row * ldb2;
    E* yr = y + row * ldy;
    // elements before x's first line boundary in this row
    const int64_t head = min(cols, (int64_t)(((128 - (reinterpret_cast<uintptr_t>(xr) & 127)) & 127) / ES));
    if (threadIdx.x < head) chain_elem<IO>(xr, ar, br, yr, threadIdx.x, scale);
#pragma unroll 4
    for (int64_t c = head + threadIdx.x; c < cols; c += kBlock) chain_elem<IO>(xr, ar, br, yr, c, scale);
  }
}

template <class IO>
hipError_t launch_chain2d_io(const void* x, int64_t ldx, const void* b1, int64_t ldb1, const void* b2,
                             int64_t ldb2, void* y, int64_t ldy, int64_t rows, int64_t cols, double scale,
                             hipStream_t s) {
  typedef typename IO::elem E;
  constexpr int V = IO::kVec;
  auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  auto row16 = [](int64_t ld) { return (ld * (int64_t)sizeof(E)) % 16 == 0; };
  const bool vec = cols % V == 0 && a16(x) && a16(b1) && a16(b2) && a16(y) && row16(ldx) && row16(ldb1) &&
                   row16(ldb2) && row16(ldy);
  const int vw = vec ? V : 1;
  int64_t grid = (rows * (cols / vw) + kBlock - 1) / kBlock;
  if (grid > kMaxGrid) grid = kMaxGrid;
  const void* k = vec ? reinterpret_cast<const void*>(&chain2d_kernel<IO, V>)
                      : reinterpret_cast<const void*>(&chain2d_kernel<IO, 1>);
  if (!vec && cols >= kRowBlockCols) {
    k = reinterpret_cast<const void*>(&chain2d_rows_kernel<IO>);
    grid = rows < 8192 ? rows : 8192;
  }
  const E *xe = static_cast<const E*>(x), *ae = static_cast<const E*>(b1), *be = static_cast<const E*>(b2);
  E* ye = static_cast<E*>(y);
  void* args[] = {&xe, &ldx, &ae, &ldb1, &be, &ldb2, &ye, &ldy, &rows, &cols, &scale};
  return hipLaunchKernel(k, dim3((unsigned)grid), dim3(kBlock), args, 0, s);
}

__global__ __launch_bounds__(kBlock) void copy_kernel(const u32x4* src, u32x4* dst, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kBlock)
    store_nt(dst + i, load_nt(src + i));
}

// The copy's access pattern with NSRC inputs: dst = src0 ^ src1 ^ ..., so
// every load is used -- the bare stream of a kernel that reads NSRC tensors
// and writes one, with no arithmetic.
struct Srcs {
  const u32x4* p[4];
};
template <int NSRC>
__global__ __launch_bounds__(kBlock) void stream_kernel(Srcs src, u32x4* dst, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * kBlock) {
    u32x4 v[NSRC];
#pragma unroll
    for (int k = 0; k < NSRC; ++k) v[k] = load_nt(src.p[k] + i);
    u32x4 o = v[0];
#pragma unroll
    for (int k = 1; k < NSRC; ++k)
#pragma unroll
      for (int w = 0; w < 4; ++w) o.w[w] ^= v[k].w[w];
    store_nt(dst + i, o);
  }
}


// binary32 -> bfloat16 with the conversion every bf16-storing kernel uses
// (pack_bf16x2 / f32_to_bf16: v_cvt_pk_bf16_f32, round to nearest even), for
// checking it over every binary32 bit pattern.  Eight values per item when x
// and y are 16-byte aligned, then the n % 8 tail one at a time.
__global__ __launch_bounds__(kBlock) void to_bf16_kernel(const float* x, uint16_t* y, int64_t n,
                                                       int vec) {
  const int64_t n8 = vec ? n / 8 : 0;
  const int64_t items = n8 + (n - 8 * n8);
  for (int64_t it = (int64_t)blockIdx.x * kBlock + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * kBlock) {
    if (it < n8) {
      const u32x4 a = load_nt(reinterpret_cast<const u32x4*>(x) + 2 * it);
      const u32x4 b = load_nt(reinterpret_cast<const u32x4*>(x) + 2 * it + 1);
      u32x4 o;
      o.w[0] = pack_bf16x2(__uint_as_float(a.w[0]), __uint_as_float(a.w[1]));
      o.w[1] = pack_bf16x2(__uint_as_float(a.w[2]), __uint_as_float(a.w[3]));
      o.w[2] = pack_bf16x2(__uint_as_float(b.w[0]), __uint_as_float(b.w[1]));
      o.w[3] = pack_bf16x2(__uint_as_float(b.w[2]), __uint_as_float(b.w[3]));
      store_nt(reinterpret_cast<u32x4*>(y) + it, o);
    } else {
      const int64_t i = 8 * n8 + (it - n8);
      y[i] = f32_to_bf16(x[i]);
    }
  }
}

}  // namespace

hipError_t launch_to_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t s) {
  const int vec = ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15) == 0;
  const int64_t items = vec ? n / 8 + n % 8 : n;
  int64_t grid = (items + kBlock - 1) / kBlock;
  if (grid > kMaxGrid) grid = kMaxGrid;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)grid), dim3(kBlock), 0, s, x, y, n, vec);
  return hipGetLastError();
}

hipError_t launch_chain(const float* x, const float* b1, const float* b2, float* y, int64_t n,
                        double scale, hipStream_t s) {
  // The 128-bit body needs all four pointers congruent mod 16 bytes; the head
  // brings them to a 16-byte boundary.  Otherwise every element is a scalar item.
  const uintptr_t mis = reinterpret_cast<uintptr_t>(x) & 15;
  const bool congruent = ((reinterpret_cast<uintptr_t>(b1) & 15) == mis) &&
                         ((reinterpret_cast<uintptr_t>(b2) & 15) == mis) &&
                         ((reinterpret_cast<uintptr_t>(y) & 15) == mis);
  int64_t h = n, n4 = 0;
  if (congruent) {
    h = (int64_t)(((16 - mis) & 15) / 4);
    if (h > n) h = n;
    n4 = (n - h) / 4;
  }
  const int64_t nscal = n - 4 * n4;
  const int64_t items = n4 + nscal;
  int64_t grid = (items + kBlock * kChainUnroll - 1) / (kBlock * kChainUnroll);
  if (grid > kMaxGrid) grid = kMaxGrid;
  hipLaunchKernelGGL(chain_kernel<kChainUnroll>, dim3((unsigned)grid), dim3(kBlock), 0, s, x, b1,
                     b2, y, h, n4, nscal, scale);
  return hipGetLastError();
}

hipError_t launch_chain_2d(int dtype, const void* x, int64_t ldx, const void* b1, int64_t ldb1,
                          const void* b2, int64_t ldb2, void* y, int64_t ldy, int64_t rows, int64_t cols,
                          double scale, hipStream_t s) {
  // dense fp32 (every stride == cols, or one row): the one-dimensional kernel
  const bool dense = rows == 1 || (ldx == cols && ldb1 == cols && ldb2 == cols && ldy == cols);
  if (dtype == 0 && dense)
    return launch_chain(static_cast<const float*>(x), static_cast<const float*>(b1),
                        static_cast<const float*>(b2), static_cast<float*>(y), rows * cols, scale, s);
  if (dtype == 0) return launch_chain2d_io<F32IO>(x, ldx, b1, ldb1, b2, ldb2, y, ldy, rows, cols, scale, s);
  if (dtype == 1) return launch_chain2d_io<BF16IO>(x, ldx, b1, ldb1, b2, ldb2, y, ldy, rows, cols, scale, s);
  return launch_chain2d_io<F16IO>(x, ldx, b1, ldb1, b2, ldb2, y, ldy, rows, cols, scale, s);
}

hipError_t launch_stream(const void* const* srcs, int nsrc, void* dst, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t grid = (n16 + kBlock - 1) / kBlock;
  if (grid > kMaxGrid) grid = kMaxGrid;
  Srcs p = {{nullptr, nullptr, nullptr, nullptr}};
  for (int k = 0; k < nsrc; ++k) p.p[k] = static_cast<const u32x4*>(srcs[k]);
  u32x4* d = static_cast<u32x4*>(dst);
  const dim3 g((unsigned)grid), b(kBlock);
  switch (nsrc) {
    case 1: hipLaunchKernelGGL(stream_kernel<1>, g, b, 0, s, p, d, n16); break;
    case 2: hipLaunchKernelGGL(stream_kernel<2>, g, b, 0, s, p, d, n16); break;
    case 3: hipLaunchKernelGGL(stream_kernel<3>, g, b, 0, s, p, d, n16); break;
    case 4: hipLaunchKernelGGL(stream_kernel<4>, g, b, 0, s, p, d, n16); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t grid = (n16 + kBlock - 1) / kBlock;
  if (grid > kMaxGrid) grid = kMaxGrid;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(kBlock), 0, s,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace mbp
