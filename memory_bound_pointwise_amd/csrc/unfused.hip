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
// element-wise kernels use 128-bit loads/stores wherever every full-size
// operand is 16-byte aligned (any row length: broadcast operands are indexed
// per element), and the row reductions read aligned 16-byte windows, so the
// comparison with the fused kernels is one of bytes and launches, not of load
// width.
#include <atomic>
#include <mutex>

#include "mbp.h"
#include "mbp_device.hpp"
#include "mbp_internal.hpp"

// Scratch memory for the entry point that allocates nothing
// (grouped_row_mean_epilogue_noalloc): one copy of this array per GPU, in that
// GPU's memory from the first use until the process ends.  In host code the
// name `scratch` is only a host-side stand-in, not a device address: host code
// reaches the array through the pointer static_scratch() looks up for the
// current device, never through the name.
static __device__ __align__(256) unsigned char scratch[MBP_STATIC_SCRATCH_BYTES];

namespace mbp {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::atomic<int> g_cu_count[kMaxDevices];
std::mutex g_scratch_mu;

constexpr int kBlock = 256;
constexpr int64_t kMaxGrid = dispatch_blocks(kBlock);  // every kernel here loops over its items

template <int OP>
__device__ __forceinline__ float ew_apply(float a, float b, float c, float d, float scalar,
                                          float scalar2) {
  if constexpr (OP == EW_ADD) return __fadd_rn(a, b);
  if constexpr (OP == EW_SUB) return __fsub_rn(a, b);
  if constexpr (OP == EW_MUL) return __fmul_rn(a, b);
  if constexpr (OP == EW_RELU) return (a < 0.0f) ? 0.0f : a;
  if constexpr (OP == EW_MULS) return __fmul_rn(a, scalar);
  // __builtin_sqrtf is the correctly rounded square root here; __fsqrt_rn is
  // not on gfx950 with this toolchain (about 15% of random inputs come back
  // 1 ulp off, measured against a binary64 root rounded once)
  if constexpr (OP == EW_DIVSD) return __fdiv_rn(a, __builtin_sqrtf(__fadd_rn(b, scalar)));
  if constexpr (OP == EW_MULADD) return __fadd_rn(__fmul_rn(a, b), c);
  if constexpr (OP == EW_GELU) return gelu_tanh_f32(a);
  if constexpr (OP == EW_DROPOUT) return a;  // the mask and the scale are applied by the caller
  if constexpr (OP == EW_PROLOGUE) {
    // the element-wise group of the 10-op graph, each op rounded as its own
    // eager kernel would round it
    const float t = __fadd_rn(__fmul_rn(a, scalar), b);
    const float r = t < 0.0f ? 0.0f : t;
    return __fadd_rn(__fmul_rn(r, r), __fmul_rn(r, scalar2));
  }
  if constexpr (OP == EW_CENTER_AFFINE) return __fadd_rn(__fmul_rn(__fsub_rn(a, b), c), d);
  if constexpr (OP == EW_EXP) return expf(a);
  if constexpr (OP == EW_DIV) return __fdiv_rn(a, b);
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

// Operand element e of the vector starting at flat index i0 = row0 * cols +
// col0 (col0 < cols, cols >= VW: the vector wraps into the next row at most once).
template <class IO, int VW>
__device__ __forceinline__ float vec_operand(const void* p, int ix, const u32x4& full, int e, int64_t row0,
                                             int64_t col0, int64_t cols) {
  if (p == nullptr) return 0.0f;
  if (ix == IX_FULL) return IO::get(full, e);
  const bool wrap = col0 + e >= cols;
  if (ix == IX_COL) return IO::load1(static_cast<const typename IO::elem*>(p), wrap ? col0 + e - cols : col0 + e);
  return static_cast<const float*>(p)[wrap ? row0 + 1 : row0];
}

// One element per work item (VW == 1), or one 16-byte vector (VW == IO::kVec)
// for items below n / VW and single elements for the n % VW tail.  The vector
// form needs every full-size operand 16-byte aligned and, when an operand is
// broadcast, cols >= VW.
template <class IO, int OP, int VW>
__global__ __launch_bounds__(kBlock) void ew_kernel(const typename IO::elem* a, const void* b,
                                                    int b_ix, const void* c, int c_ix,
                                                    const void* d, int d_ix,
                                                    typename IO::elem* out, int64_t n,
                                                    int64_t cols, float scalar, float scalar2,
                                                    Drop drop) {
  // the fourth operand exists for EW_CENTER_AFFINE only
  constexpr bool kD = OP == EW_CENTER_AFFINE;
  const int64_t nv = n / VW;
  const int64_t items = nv + (n - nv * VW);
  const bool bcast = (b && b_ix != IX_FULL) || (c && c_ix != IX_FULL) || (kD && d && d_ix != IX_FULL);
  const bool col_vec = VW > 1 && cols % VW == 0 && (!b || b_ix != IX_COL || ((uintptr_t)b & 15) == 0) &&
                       (!c || c_ix != IX_COL || ((uintptr_t)c & 15) == 0) &&
                       (!kD || !d || d_ix != IX_COL || ((uintptr_t)d & 15) == 0);
  for (int64_t it = (int64_t)blockIdx.x * kBlock + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * kBlock) {
    if (VW == 1 || it >= nv) {
      const int64_t i = VW == 1 ? it : nv * VW + (it - nv);
      const float dv = kD ? operand<IO>(d, d_ix, i, cols) : 0.0f;
      float r = ew_apply<OP>(IO::load1(a, i), operand<IO>(b, b_ix, i, cols),
                             operand<IO>(c, c_ix, i, cols), dv, scalar, scalar2);
      if constexpr (OP == EW_DROPOUT) {
        uint32_t h;
        dropout_bits<1, true>((uint64_t)i, drop.seed, drop.offset, &h);
        r = (h >= drop.thr) ? __fmul_rn(r, drop.scale) : 0.0f;
      }
      IO::store1(out, i, r);
    } else {
      const int64_t i0 = it * VW;
      int64_t row0 = 0, col0 = 0;
      if (bcast) {
        row0 = i0 / cols;
        col0 = i0 - row0 * cols;
      }
      const u32x4 av = reinterpret_cast<const u32x4*>(a)[it];
      // a column-broadcast operand whose vectors line up with the row (cols a
      // multiple of VW, 16-byte aligned) is read as one vector, as if full
      int bx = b_ix, cx = c_ix, dx = d_ix;
      if (bx == IX_COL && col_vec) bx = IX_FULL;
      if (cx == IX_COL && col_vec) cx = IX_FULL;
      if (dx == IX_COL && col_vec) dx = IX_FULL;
      u32x4 bv = {{0u, 0u, 0u, 0u}}, cv = {{0u, 0u, 0u, 0u}}, dv = {{0u, 0u, 0u, 0u}};
      if (b && b_ix == IX_FULL) bv = reinterpret_cast<const u32x4*>(b)[it];
      if (b && b_ix == IX_COL && col_vec) bv = reinterpret_cast<const u32x4*>(b)[col0 / VW];
      if (c && c_ix == IX_FULL) cv = reinterpret_cast<const u32x4*>(c)[it];
      if (c && c_ix == IX_COL && col_vec) cv = reinterpret_cast<const u32x4*>(c)[col0 / VW];
      if constexpr (kD) {
        if (d && d_ix == IX_FULL) dv = reinterpret_cast<const u32x4*>(d)[it];
        if (d && d_ix == IX_COL && col_vec) dv = reinterpret_cast<const u32x4*>(d)[col0 / VW];
      }
      float r[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e)
        r[e] = ew_apply<OP>(IO::get(av, e), vec_operand<IO, VW>(b, bx, bv, e, row0, col0, cols),
                            vec_operand<IO, VW>(c, cx, cv, e, row0, col0, cols),
                            kD ? vec_operand<IO, VW>(d, dx, dv, e, row0, col0, cols) : 0.0f, scalar,
                            scalar2);
      if constexpr (OP == EW_DROPOUT) {
        uint32_t h[VW];
        dropout_bits<VW, true>((uint64_t)i0, drop.seed, drop.offset, h);
#pragma unroll
        for (int e = 0; e < VW; ++e) r[e] = (h[e] >= drop.thr) ? __fmul_rn(r[e], drop.scale) : 0.0f;
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

// Row statistics: a lane group per row (one wave for rows of up to 4 KiB,
// the 256-lane block otherwise), binary64 accumulation, then a fixed-order
// group reduction.  MODE 0: mean; MODE 1: biased variance about
// `mean`; MODE 2: maximum (NaN elements skipped; -inf for a row without a
// larger value); MODE 3: sum.  The row is read in aligned 16-byte windows
// (window q: bytes [16q, 16q + 16) above the 16-byte boundary at or below
// `a`), kU windows per lane in flight; elements of a window outside the row
// are skipped, and a window reaching outside the tensor (at its first or last
// row only) is read element by element.
constexpr int kU = 4;

template <class IO>
__device__ __forceinline__ u32x4 stat_window(const typename IO::elem* a, const u32x4* win, int mb, int64_t end,
                                             int64_t q) {
  typedef typename IO::elem E;
  constexpr int ES = (int)sizeof(E);
  const int64_t wb = 16 * q;
  if (wb >= mb && wb + 16 <= end) return win[q];
  u32x4 w = {{0u, 0u, 0u, 0u}};
#pragma unroll
  for (int e = 0; e < IO::kVec; ++e) {
    const int64_t bb = wb + ES * e;
    if (bb >= mb && bb < end) {
      const E v = a[(bb - mb) / ES];
      if constexpr (IO::kVec == 8) {
        const uint32_t h = (uint32_t)v;
        w.w[e >> 1] |= (e & 1) ? (h << 16) : h;
      } else {
        w.w[e] = __float_as_uint(v);
      }
    }
  }
  return w;
}

template <class IO, int MODE, int LANES>
__global__ __launch_bounds__(kBlock) void row_stat_kernel(const typename IO::elem* a,
                                                          const float* mean, float* out,
                                                          int64_t rows, int64_t cols) {
  constexpr int ES = (int)sizeof(typename IO::elem);
  constexpr int V = IO::kVec;
  constexpr int RPB = kBlock / LANES;  // rows per block, one group of LANES lanes each
  __shared__ double red[2][kBlock / 64];
  const int mb = (int)(reinterpret_cast<uintptr_t>(a) & 15);
  const u32x4* win = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a) - mb);
  const int64_t end = mb + (int64_t)ES * rows * cols;  // tensor bytes, relative to the window base
  const int lane = threadIdx.x % LANES;
  int parity = 0;
  for (int64_t grp = blockIdx.x; grp * RPB < rows; grp += gridDim.x, parity ^= 1) {
    const int64_t row = grp * RPB + threadIdx.x / LANES;
    const bool live = row < rows;
    const int64_t lo = mb + (int64_t)ES * (live ? row : 0) * cols, hi = live ? lo + (int64_t)ES * cols : lo;
    const int64_t q_end = (hi + 15) >> 4;
    const double mu = MODE == 1 && live ? (double)mean[row] : 0.0;
    double acc = MODE == 2 ? -__builtin_inf() : 0.0;
    for (int64_t q0 = (lo >> 4) + lane; q0 < q_end; q0 += kU * LANES) {
      u32x4 w[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t q = q0 + u * LANES;
        w[u] = q < q_end ? stat_window<IO>(a, win, mb, end, q) : u32x4{{0u, 0u, 0u, 0u}};
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t wb = 16 * (q0 + u * LANES);
        const bool inner = wb >= lo && wb + 16 <= hi;
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const int64_t bb = wb + ES * e;
          if (inner || (bb >= lo && bb < hi)) {
            const double v = (double)IO::get(w[u], e);
            if constexpr (MODE == 0 || MODE == 3) {
              acc += v;
            } else if constexpr (MODE == 2) {
              acc = v > acc ? v : acc;
            } else {
              const double d = v - mu;
              acc += d * d;
            }
          }
        }
      }
    }
    double tot;
    if constexpr (MODE == 2) tot = group_max<LANES, kBlock>(acc, red[parity]);
    else tot = group_sum<LANES, kBlock>(acc, red[parity]);
    if (live && lane == 0) out[row] = (float)(MODE >= 2 ? tot : tot / (double)cols);
  }
}

// Only the (type, op, access width) forms a caller can reach are
// instantiated: the bf16 calls never multiply, scale or take the 10-op
// groups (the unfused chain and 10-op graph are fp32), and relu and exp only
// ever read and write the 256-byte aligned workspace, so never one element
// at a time.
template <class IO, int VW>
const void* ew_ptr(int op) {
  constexpr bool kBf16 = sizeof(typename IO::elem) == 2;
  switch (op) {
    case EW_ADD: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_ADD, VW>);
    case EW_SUB: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_SUB, VW>);
    case EW_MUL:
      if constexpr (!kBf16) return reinterpret_cast<const void*>(&ew_kernel<IO, EW_MUL, VW>);
      return nullptr;
    case EW_RELU:
      if constexpr (VW != 1) return reinterpret_cast<const void*>(&ew_kernel<IO, EW_RELU, VW>);
      return nullptr;
    case EW_MULS:
      if constexpr (!kBf16) return reinterpret_cast<const void*>(&ew_kernel<IO, EW_MULS, VW>);
      return nullptr;
    case EW_DIVSD: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_DIVSD, VW>);
    case EW_MULADD: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_MULADD, VW>);
    case EW_GELU: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_GELU, VW>);
    case EW_DROPOUT: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_DROPOUT, VW>);
    case EW_PROLOGUE:
      if constexpr (!kBf16) return reinterpret_cast<const void*>(&ew_kernel<IO, EW_PROLOGUE, VW>);
      return nullptr;
    case EW_CENTER_AFFINE:
      if constexpr (!kBf16) return reinterpret_cast<const void*>(&ew_kernel<IO, EW_CENTER_AFFINE, VW>);
      return nullptr;
    case EW_EXP:
      if constexpr (VW != 1) return reinterpret_cast<const void*>(&ew_kernel<IO, EW_EXP, VW>);
      return nullptr;
    case EW_DIV: return reinterpret_cast<const void*>(&ew_kernel<IO, EW_DIV, VW>);
    default: return nullptr;
  }
}

bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Rows of up to 4 KiB: one wave per row (4 rows per block); longer rows: the
// whole 256-lane block.
template <class IO, int MODE>
const void* stat_ptr(int64_t cols) {
  return cols * (int64_t)sizeof(typename IO::elem) <= 4096
             ? reinterpret_cast<const void*>(&row_stat_kernel<IO, MODE, 64>)
             : reinterpret_cast<const void*>(&row_stat_kernel<IO, MODE, kBlock>);
}

int64_t stat_grid(int64_t rows, int64_t cols, int es) {
  const int64_t rpb = cols * es <= 4096 ? kBlock / 64 : 1;
  const int64_t g = (rows + rpb - 1) / rpb;  // one block per row group
  return g < kMaxGrid ? g : kMaxGrid;
}

}  // namespace

int compute_units() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    g_cu_count[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t static_scratch(void** ptr, size_t* bytes) {
  *ptr = nullptr;
  *bytes = 0;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      // with `dev` current: this GPU's copy of the array
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  *bytes = sizeof scratch;
  return hipSuccess;
}

hipError_t launch_ew(int op, int dtype, const void* a, const void* b, int b_ix, const void* c,
                     int c_ix, void* out, int64_t rows, int64_t cols, float scalar,
                     hipStream_t s, const Drop* drop) {
  return launch_ew4(op, dtype, a, b, b_ix, c, c_ix, nullptr, IX_FULL, out, rows, cols, scalar, 0.0f, s,
                    drop);
}

hipError_t launch_ew4(int op, int dtype, const void* a, const void* b, int b_ix, const void* c,
                      int c_ix, const void* d, int d_ix, void* out, int64_t rows, int64_t cols,
                      float scalar, float scalar2, hipStream_t s, const Drop* drop) {
  const int64_t n = rows * cols;
  const int vec = dtype == 1 ? 8 : 4;
  if (op != EW_CENTER_AFFINE) d = nullptr;
  // 128-bit form: every full-size operand 16-byte aligned; a broadcast
  // operand needs cols >= vec (a vector then wraps into the next row at most once)
  const bool bcast = (b && b_ix != IX_FULL) || (c && c_ix != IX_FULL) || (d && d_ix != IX_FULL);
  bool vector_ok = a16(a) && a16(out) && (!bcast || cols >= vec);
  if (b && b_ix == IX_FULL) vector_ok = vector_ok && a16(b);
  if (c && c_ix == IX_FULL) vector_ok = vector_ok && a16(c);
  if (d && d_ix == IX_FULL) vector_ok = vector_ok && a16(d);
  const int vw = vector_ok ? vec : 1;
  const void* k = dtype == 1 ? (vector_ok ? ew_ptr<BF16IO, 8>(op) : ew_ptr<BF16IO, 1>(op))
                             : (vector_ok ? ew_ptr<F32IO, 4>(op) : ew_ptr<F32IO, 1>(op));
  if (!k) return hipErrorInvalidValue;
  int64_t grid = (n / vw + n % vw + kBlock - 1) / kBlock;
  if (grid > kMaxGrid) grid = kMaxGrid;
  if (grid < 1) grid = 1;
  Drop dv = drop ? *drop : Drop{0, 0, 0, 1.0f};
  if (op == EW_DROPOUT && !drop) return hipErrorInvalidValue;
  void* args[] = {&a, &b, &b_ix, &c, &c_ix, &d, &d_ix, &out, (void*)&n, &cols, &scalar, &scalar2, &dv};
  return hipLaunchKernel(k, dim3((unsigned)grid), dim3(kBlock), args, 0, s);
}

hipError_t launch_row_mean_only(int dtype, const void* a, float* mean, int64_t rows,
                                int64_t cols, hipStream_t s) {
  const void* k = dtype == 1 ? stat_ptr<BF16IO, 0>(cols) : stat_ptr<F32IO, 0>(cols);
  const float* none = nullptr;
  const int grid = (int)stat_grid(rows, cols, dtype == 1 ? 2 : 4);
  void* args[] = {&a, &none, &mean, &rows, &cols};
  return hipLaunchKernel(k, dim3(grid), dim3(kBlock), args, 0, s);
}

hipError_t launch_row_max(int dtype, const void* a, float* out, int64_t rows, int64_t cols, hipStream_t s) {
  const void* k = dtype == 1 ? stat_ptr<BF16IO, 2>(cols) : stat_ptr<F32IO, 2>(cols);
  const float* none = nullptr;
  const int grid = (int)stat_grid(rows, cols, dtype == 1 ? 2 : 4);
  void* args[] = {&a, &none, &out, &rows, &cols};
  return hipLaunchKernel(k, dim3(grid), dim3(kBlock), args, 0, s);
}

hipError_t launch_row_sum(int dtype, const void* a, float* out, int64_t rows, int64_t cols, hipStream_t s) {
  const void* k = dtype == 1 ? stat_ptr<BF16IO, 3>(cols) : stat_ptr<F32IO, 3>(cols);
  const float* none = nullptr;
  const int grid = (int)stat_grid(rows, cols, dtype == 1 ? 2 : 4);
  void* args[] = {&a, &none, &out, &rows, &cols};
  return hipLaunchKernel(k, dim3(grid), dim3(kBlock), args, 0, s);
}

hipError_t launch_row_var(int dtype, const void* a, const float* mean, float* var, int64_t rows,
                          int64_t cols, hipStream_t s) {
  const void* k = dtype == 1 ? stat_ptr<BF16IO, 1>(cols) : stat_ptr<F32IO, 1>(cols);
  const int grid = (int)stat_grid(rows, cols, dtype == 1 ? 2 : 4);
  void* args[] = {&a, &mean, &var, &rows, &cols};
  return hipLaunchKernel(k, dim3(grid), dim3(kBlock), args, 0, s);
}

}  // namespace mbp
