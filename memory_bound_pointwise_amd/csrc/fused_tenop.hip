// fused_tenop.hip -- the 10-op graph of "TorchInductor Pipeline 与算子融合" (the
// model at the top of the post) as one row kernel:
//
//   t = x*alpha + bias;  a = relu(t);  s = a*a + a*c;
//   m = (row sum of s) / cols   (section 6.4: a sum, then the division; here
//                                the sum times 1/cols, within a binary64 ulp);
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
// same kernel with one element per load.  The same kernel serves bf16 and fp16
// storage and row-strided x / y (each result rounded once to the storage type);
// 16-bit rows on 16-byte boundaries take tenop8_kernel (16-byte accesses).
#include "mbp_internal.hpp"
#include "row_common.hpp"

namespace mbp {
namespace {

using namespace rows;

// ---------------------------------------------------------------- 10-op graph

// Four consecutive elements: one 16-byte access for fp32, one 8-byte access
// for the 16-bit types (nontemporal: x is read once, y written once).
template <class IO>
__device__ __forceinline__ void load4_nt(const typename IO::elem* p, float* v) {
  if constexpr (sizeof(typename IO::elem) == 4) {
    const u32x4 t = load_nt(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(t.w[e]);
  } else {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    const uint32_t w0 = __builtin_nontemporal_load(q), w1 = __builtin_nontemporal_load(q + 1);
    u32x4 t = {{w0, w1, 0u, 0u}};
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = IO::get(t, e);
  }
}
template <class IO>
__device__ __forceinline__ void load4(const typename IO::elem* p, float* v) {
  if constexpr (sizeof(typename IO::elem) == 4) {
    const u32x4 t = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(t.w[e]);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    u32x4 t = {{w.x, w.y, 0u, 0u}};
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = IO::get(t, e);
  }
}
template <class IO>
__device__ __forceinline__ void store4_nt(typename IO::elem* p, const uint32_t* bits) {
  if constexpr (sizeof(typename IO::elem) == 4) {
    store_nt(reinterpret_cast<u32x4*>(p), u32x4{{bits[0], bits[1], bits[2], bits[3]}});
  } else {
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
    __builtin_nontemporal_store(bits[0] | (bits[1] << 16), q);
    __builtin_nontemporal_store(bits[2] | (bits[3] << 16), q + 1);
  }
}

// IO: storage type of every operand (fp32, bf16, fp16).  VW: elements per
// access (4: rows aligned to 4 elements; 1: one element).  x and y rows are
// ldx and ldy elements apart.  Every type holds the same number of elements
// per lane for a layout, so the 16-bit kernels use the fp32 kernel's registers.
template <class IO, int LANES, int VPL, int VW>
__global__ __launch_bounds__(block_for(LANES)) void tenop_kernel(
    const typename IO::elem* x, int64_t ldx, const typename IO::elem* __restrict__ bias,
    const typename IO::elem* __restrict__ gamma, const typename IO::elem* __restrict__ beta,
    typename IO::elem* y, int64_t ldy, int64_t rows, int cols, double alpha, double c, double inv_cols) {
  typedef typename IO::elem E;
  constexpr int BLOCK = block_for(LANES);
  constexpr int RPB = BLOCK / LANES;
  __shared__ double red[2][BLOCK / 64];

  const int lane = threadIdx.x % LANES;
  const int sub = threadIdx.x / LANES;
  const int nvec = (cols + VW - 1) / VW;

  float bi[VPL][VW], g[VPL][VW], be[VPL][VW];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    // 4-element accesses (the host requires bias, gamma, beta aligned for
    // them); a slot past the row rereads the last group and stays unused
    const int vi = min(lane + k * LANES, nvec - 1);
    if constexpr (VW == 4) {
      load4<IO>(bias + 4 * vi, bi[k]);
      load4<IO>(gamma + 4 * vi, g[k]);
      load4<IO>(beta + 4 * vi, be[k]);
    } else {
      bi[k][0] = IO::load1(bias, vi);
      g[k][0] = IO::load1(gamma, vi);
      be[k][0] = IO::load1(beta, vi);
    }
  }

  const int64_t groups = (rows + RPB - 1) / RPB;
  int parity = 0;
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x, parity ^= 1) {
    const int64_t row = grp * RPB + sub;
    const bool live = row < rows;
    // past the last row: reread the last row, store nothing; slots past the
    // row's end reread its last vector and stay out of the sum (no branches)
    const E* xr = x + (live ? row : rows - 1) * ldx;
    E* yr = y + row * ldy;

    float xv[VPL][VW];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int vi = min(lane + k * LANES, nvec - 1);
      if constexpr (VW == 1) xv[k][0] = IO::load1(xr, vi);
      else load4_nt<IO>(xr + 4 * vi, xv[k]);
    }
    // the parameters stay fp32 across rows (an empty asm keeps the compiler
    // from widening them to binary64 once and holding the wide copies); it
    // comes after the row's loads are issued, so that on the first row the
    // parameter loads and the row loads are in flight together
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        opaque(bi[k][e]);
        opaque(g[k][e]);
        opaque(be[k][e]);
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
    // gamma and beta widened while the reduction's exchanges are in flight
    // (one vector a lane; with more, the wide copies would cost registers)
    constexpr bool kEarly = VPL * VW <= 4;
    double gd[VPL][VW], bd[VPL][VW];
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        gd[k][e] = (double)g[k][e];
        bd[k][e] = (double)be[k][e];
        if constexpr (kEarly) {
          opaque(gd[k][e]);
          opaque(bd[k][e]);
        }
      }
    const double m = group_sum<LANES, BLOCK>(sum, red[parity]) * inv_cols;

#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int vi = lane + k * LANES;
      if (!(live && vi < nvec)) continue;
      double yv[VW];
#pragma unroll
      for (int e = 0; e < VW; ++e) yv[e] = __builtin_fma(s[k][e] - m, gd[k][e], bd[k][e]);
      uint32_t o[VW];
      narrow_n<IO, VW>(yv, o);
      if constexpr (VW == 1) {
        if constexpr (sizeof(E) == 4) yr[vi] = __uint_as_float(o[0]);
        else yr[vi] = (uint16_t)o[0];
      } else {
        store4_nt<IO>(yr + 4 * vi, o);
      }
    }
  }
}

// fp32 rows of at most 256 vectors (4-element accesses): one vector a lane,
// one row group per block and no loop over row groups, every load issued up
// front -- bias first (its widening overlaps the wait for the row), then the
// row, then gamma and beta, which are needed only after the reduction.
// Measured at 1024 x 1024 (graph-replayed calls, inputs out of the caches)
// against tenop_kernel<F32IO, 256, 1, 4>, whose grid-stride loop holds the
// parameters in storage form across rows: 3.41 -> 3.25 us; giving each block
// 2, 4 or 8 rows with all their loads issued first: 3.57, 3.80, 5.06 us;
// 128 x 2, 64 x 4 and 32 x 8 lanes x vectors: slower still.
template <int LANES>
__global__ __launch_bounds__(block_for(LANES)) void tenop1_kernel(
    const float* x, int64_t ldx, const float* __restrict__ bias, const float* __restrict__ gamma,
    const float* __restrict__ beta, float* y, int64_t ldy, int64_t rows, int cols, double alpha, double c,
    double inv_cols) {
  constexpr int BLOCK = block_for(LANES);
  constexpr int RPB = BLOCK / LANES;
  __shared__ double red[BLOCK / 64];
  const int lane = threadIdx.x % LANES;
  const int nvec = cols / 4;
  const int vi = min(lane, nvec - 1);  // lanes past the row reread its last vector
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LANES;
  const int64_t rowc = row < rows ? row : rows - 1;  // rows past the end reread the last row
  float bi[4], g[4], be[4], xv[4];
  load4<F32IO>(bias + 4 * vi, bi);
  load4_nt<F32IO>(x + rowc * ldx + 4 * vi, xv);
  load4<F32IO>(gamma + 4 * vi, g);
  load4<F32IO>(beta + 4 * vi, be);
  double bd[4], gd[4], ed[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bd[e] = bi[e];
    gd[e] = g[e];
    ed[e] = be[e];
  }
  double s[4], part = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double t = __builtin_fma((double)xv[e], alpha, bd[e]);
    const double a = (t < 0.0) ? 0.0 : t;  // relu; NaN passes through
    s[e] = __builtin_fma(a, a, a * c);
    part += s[e];
  }
  const double m = group_sum<LANES, BLOCK>(lane < nvec ? part : 0.0, red) * inv_cols;
  if (row < rows && lane < nvec) {
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = narrow_bits<F32IO>(__builtin_fma(s[e] - m, gd[e], ed[e]));
    store4_nt<F32IO>(y + row * ldy + 4 * lane, o);
  }
}

// s = relu(x * alpha + bias) * (relu(...) + c) as the 10-op kernels form it
__device__ __forceinline__ double tenop_s(float xv, float bv, double alpha, double c) {
  const double t = __builtin_fma((double)xv, alpha, (double)bv);
  const double a = (t < 0.0) ? 0.0 : t;  // relu; NaN passes through
  return __builtin_fma(a, a, a * c);
}

// Rows of more than kRegCols columns: one 1024-lane block per row, two
// passes -- s and its row sum, then s again (the same binary64 operations)
// and the output -- the second rereading x from the caches; any width,
// alignment and row strides.
template <class IO>
__global__ __launch_bounds__(1024) void tenop_wide_kernel(
    const typename IO::elem* x, int64_t ldx, const typename IO::elem* __restrict__ bias,
    const typename IO::elem* __restrict__ gamma, const typename IO::elem* __restrict__ beta,
    typename IO::elem* y, int64_t ldy, int64_t rows, int cols, double alpha, double c, double inv_cols) {
  constexpr int LANES = 1024;
  __shared__ double red[2][LANES / 64];  // alternating by row
  const int lane = threadIdx.x;
  int parity = 0;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x, parity ^= 1) {
    const typename IO::elem* xr = x + row * ldx;
    typename IO::elem* yr = y + row * ldy;
    double sum = 0.0;
#pragma unroll 4
    for (int j = lane; j < cols; j += LANES) sum += tenop_s(IO::load1(xr, j), IO::load1(bias, j), alpha, c);
    const double m = group_sum<LANES, LANES>(sum, red[parity]) * inv_cols;
#pragma unroll 4
    for (int j = lane; j < cols; j += LANES) {
      const double sv = tenop_s(IO::load1(xr, j), IO::load1(bias, j), alpha, c);
      const uint32_t o =
          narrow_bits<IO>(__builtin_fma(sv - m, (double)IO::load1(gamma, j), (double)IO::load1(beta, j)));
      if constexpr (sizeof(typename IO::elem) == 4) yr[j] = __uint_as_float(o);
      else yr[j] = (uint16_t)o;
    }
  }
}

// 16-bit storage on 16-byte boundaries: 8 elements per access (one 16-byte
// load or store per vector).  The row and the parameters stay in storage form;
// s is held in binary64 registers from the row sum to the epilogue (two
// registers per element; measured 10% faster than computing it twice at
// 8192 x 1024 fp16).
template <class IO, int LANES, int VPL>
__global__ __launch_bounds__(block_for(LANES)) void tenop8_kernel(
    const typename IO::elem* x, int64_t ldx, const typename IO::elem* __restrict__ bias,
    const typename IO::elem* __restrict__ gamma, const typename IO::elem* __restrict__ beta,
    typename IO::elem* y, int64_t ldy, int64_t rows, int cols, double alpha, double c, double inv_cols) {
  typedef typename IO::elem E;
  static_assert(sizeof(E) == 2, "16-bit storage only");
  constexpr int BLOCK = block_for(LANES);
  constexpr int RPB = BLOCK / LANES;
  __shared__ double red[2][BLOCK / 64];

  const int lane = threadIdx.x % LANES;
  const int sub = threadIdx.x / LANES;
  const int nvec = cols / 8;  // the host requires cols % 8 == 0

  u32x4 pb[VPL], pg[VPL], pe[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int vi = min(lane + k * LANES, nvec - 1);
    pb[k] = reinterpret_cast<const u32x4*>(bias)[vi];
    pg[k] = reinterpret_cast<const u32x4*>(gamma)[vi];
    pe[k] = reinterpret_cast<const u32x4*>(beta)[vi];
  }

  const int64_t groups = (rows + RPB - 1) / RPB;
  int parity = 0;
  for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x, parity ^= 1) {
    const int64_t row = grp * RPB + sub;
    const bool live = row < rows;
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + (live ? row : rows - 1) * ldx);
    u32x4* yr = reinterpret_cast<u32x4*>(y + row * ldy);

    u32x4 xv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) xv[k] = load_nt(xr + min(lane + k * LANES, nvec - 1));
#pragma unroll
    for (int k = 0; k < VPL; ++k) opaque(pb[k]);

    double sk[VPL][8];
    double sum = 0.0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      double part = 0.0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double t = __builtin_fma((double)IO::get(xv[k], e), alpha, (double)IO::get(pb[k], e));
        const double a = (t < 0.0) ? 0.0 : t;  // relu; NaN passes through
        const double sv = __builtin_fma(a, a, a * c);
        sk[k][e] = sv;
        part += sv;
      }
      if (lane + k * LANES < nvec) sum += part;
    }
    const double m = group_sum<LANES, BLOCK>(sum, red[parity]) * inv_cols;

#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      opaque(pg[k]);
      opaque(pe[k]);
    }
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int vi = lane + k * LANES;
      if (!(live && vi < nvec)) continue;
      double yv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) yv[e] = __builtin_fma(sk[k][e] - m, (double)IO::get(pg[k], e), (double)IO::get(pe[k], e));
      uint32_t o[8];
      narrow_n<IO, 8>(yv, o);
      store_nt(yr + vi, u32x4{{o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16),
                               o[6] | (o[7] << 16)}});
    }
  }
}

// 16-bit rows of 65-512 vectors: a wave per row (64 lanes x VPL vectors: 2
// up to 128 vectors, 4 up to 256, 8 up to 512), RPB rows a block (16; 8 for
// 8 vectors, whose 512-thread blocks leave 256 registers a lane: 164-168
// used, LDS 96 KB).  Measured (same process, inputs out of the caches, us)
// against tenop8_kernel's table layouts: 4 vectors 8192 x 2048 fp16 18.02 ->
// 16.09, 8192 x 1536 bf16 15.24 -> 13.25, 4096 x 1032 fp16 8.70 -> 7.49; 8
// vectors 4096 x 2056 fp16 15.38 -> 14.20, 4096 x 4096 bf16 18.12 -> 17.59.
// bias, gamma and beta are widened to binary64
// once per block into LDS (24 KB) instead of twice per use in every wave --
// the kernel is bound by its vector instructions, and the widenings were six
// of its ~30 a element: 8192 x 1024 fp16 10.42 -> 9.40 us, bf16 10.26 ->
// 9.54, 32768 x 1024 fp16 33.7 -> 31.9 (4 rows a block: 11.2; 8: 9.6).  With
// each vector's eight values side by side, a wave's 16-byte reads were 64
// bytes apart and stalled on LDS bank conflicts (2.65 M conflict cycles a
// launch at 8192 x 1024); pairs interleaved by vector are read conflict-free:
// 9.71 -> 8.85 us (bf16 9.73 -> 8.72, 8192 x 600 fp16 8.83 -> 8.52).  The
// arithmetic and the reduction order are tenop8_kernel's, so are the results.
template <class IO, int VPL, int RPB = 16>
__global__ __launch_bounds__(64 * RPB) void tenop8_wave_kernel(
    const typename IO::elem* x, int64_t ldx, const typename IO::elem* __restrict__ bias,
    const typename IO::elem* __restrict__ gamma, const typename IO::elem* __restrict__ beta,
    typename IO::elem* y, int64_t ldy, int64_t rows, int cols, double alpha, double c, double inv_cols) {
  constexpr int LANES = 64, BLOCK = LANES * RPB;
  static_assert(sizeof(typename IO::elem) == 2, "16-bit storage only");
  // bias, gamma, beta of the row's columns; element e of vector v at
  // pidx(v, e): pairs of elements interleaved by vector, so that the lanes of
  // a wave read consecutive 16-byte pairs
  constexpr int NV = LANES * VPL;
  __shared__ double pw[3][8 * NV];
  auto pidx = [](int v, int e) { return ((e >> 1) * NV + v) * 2 + (e & 1); };
  const int lane = threadIdx.x % LANES;
  const int nvec = cols / 8;  // (LANES VPL / 2, LANES VPL] (the host checks)
  for (int v = threadIdx.x; v < nvec; v += BLOCK) {
    const u32x4 b = reinterpret_cast<const u32x4*>(bias)[v];
    const u32x4 g = reinterpret_cast<const u32x4*>(gamma)[v];
    const u32x4 e = reinterpret_cast<const u32x4*>(beta)[v];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      pw[0][pidx(v, k)] = (double)IO::get(b, k);
      pw[1][pidx(v, k)] = (double)IO::get(g, k);
      pw[2][pidx(v, k)] = (double)IO::get(e, k);
    }
  }
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LANES;
  const bool live = row < rows;
  // past the last row: reread the last row, store nothing; slots past the
  // row's end reread its last vector and stay out of the sum
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + (live ? row : rows - 1) * ldx);
  u32x4 xv[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) xv[k] = load_nt(xr + min(lane + k * LANES, nvec - 1));
  __syncthreads();  // the widened parameters are in LDS
  double sk[VPL][8];
  double sum = 0.0;
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int vi = min(lane + k * LANES, nvec - 1);
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double t = __builtin_fma((double)IO::get(xv[k], e), alpha, pw[0][pidx(vi, e)]);
      const double a = (t < 0.0) ? 0.0 : t;  // relu; NaN passes through
      sk[k][e] = __builtin_fma(a, a, a * c);
      part += sk[k][e];
    }
    if (lane + k * LANES < nvec) sum += part;
  }
  const double m = wave_reduce<LANES>(sum, SumOp()) * inv_cols;
  if (!live) return;
  u32x4* yr = reinterpret_cast<u32x4*>(y + row * ldy);
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int vi = lane + k * LANES;
    if (vi >= nvec) continue;
    double yv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) yv[e] = __builtin_fma(sk[k][e] - m, pw[1][pidx(vi, e)], pw[2][pidx(vi, e)]);
    uint32_t o[8];
    narrow_n<IO, 8>(yv, o);
    store_nt(yr + vi, u32x4{{o[0] | (o[1] << 16), o[2] | (o[3] << 16), o[4] | (o[5] << 16), o[6] | (o[7] << 16)}});
  }
}

// Rows of 65-512 vectors (32 x 3 up to 128 x 4) take tenop8_wave_kernel and
// rows past 16384 columns the two-pass kernel, so those layouts are not
// instantiated here.
template <class IO>
struct Tenop8Sel {
  template <int L, int V>
  struct K {
    static const void* ptr() {
      if constexpr ((L == 32 && V >= 3) || (L == 64 && V == 4) || (L == 128 && V == 4) || L == 1024) return nullptr;
      else return reinterpret_cast<const void*>(&tenop8_kernel<IO, L, V>);
    }
  };
};

// Kernel of layout (L, V) of the row tables: V groups of 4 elements per lane,
// or, on the element path, the same elements one at a time.  fp32 rows of
// 4-element accesses take tenop1_kernel up to 256 vectors, 512 x 6 past 2048
// and the two-pass kernel past 3072, so those layouts are not instantiated.
template <class IO, bool VEC>
struct TenopSel {
  template <int L, int V>
  struct K {
    static const void* ptr() {
      if constexpr (VEC && sizeof(typename IO::elem) == 4 && (L * V <= 256 || L == 1024)) return nullptr;
      else if constexpr (VEC) return reinterpret_cast<const void*>(&tenop_kernel<IO, L, V, 4>);
      else return reinterpret_cast<const void*>(&tenop_kernel<IO, L, 4 * V, 1>);
    }
  };
};

template <class IO>
hipError_t launch_tenop(const void* x, int64_t ldx, const void* bias, const void* gamma, const void* beta,
                        void* y, int64_t ldy, int64_t rows, int64_t cols, double alpha, double c,
                        hipStream_t s) {
  typedef typename IO::elem E;
  // tenop1_kernel and tenop8_wave_kernel take one block per row group and no
  // loop: rows past what one dispatch can address go in chunks (rows are
  // independent; a stride of 0 keeps its one row)
  if (rows > kRowsPerDispatch) {
    for (int64_t r0 = 0; r0 < rows; r0 += kRowsPerDispatch) {
      const int64_t n = rows - r0 < kRowsPerDispatch ? rows - r0 : kRowsPerDispatch;
      const hipError_t e = launch_tenop<IO>(static_cast<const E*>(x) + r0 * ldx, ldx, bias, gamma, beta,
                                            static_cast<E*>(y) + r0 * ldy, ldy, n, cols, alpha, c, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // 4-element accesses: every row start on a 4-element boundary
  constexpr uintptr_t A4 = 4 * sizeof(E);
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) % A4) == 0; };
  const bool vector_ok = (cols % 4) == 0 && al(x) && al(y) && al(bias) && al(gamma) && al(beta) &&
                         ldx % 4 == 0 && ldy % 4 == 0;
  // 16-bit storage with every row start on a 16-byte boundary: 8 elements per access
  const bool vector8_ok = sizeof(E) == 2 && (cols % 8) == 0 && aligned16(x) && aligned16(y) &&
                          aligned16(bias) && aligned16(gamma) && aligned16(beta) && ldx % 8 == 0 &&
                          ldy % 8 == 0;
  // fp32 rows of 4-element accesses past 3072 vectors take the two-pass
  // kernel too: 1024 x 4 held s for 16 elements a lane in binary64 within the
  // 128 registers of 1024-thread blocks (1024 x 16384: 110.2 against 43.4 us)
  const bool wide_f32 = sizeof(E) == 4 && vector_ok && (cols + 3) / 4 > 3072;
  // so do element-path rows past 12288 columns, whose 1024 x 16 elements a
  // lane spill (68-76 bytes a lane)
  const bool wide_elem = !vector_ok && !vector8_ok && cols > 12288;
  if (cols > kRegCols || wide_f32 || wide_elem) {  // rows wider than the register-resident layouts
    const int wgrid = (int)(rows < 4096 ? rows : 4096);
    hipLaunchKernelGGL(tenop_wide_kernel<IO>, dim3(wgrid), dim3(1024), 0, s, static_cast<const E*>(x), ldx,
                       static_cast<const E*>(bias), static_cast<const E*>(gamma), static_cast<const E*>(beta),
                       static_cast<E*>(y), ldy, rows, (int)cols, alpha, c, 1.0 / (double)cols);
    return hipGetLastError();
  }
  const int shape = vector8_ok ? pick_shape(cols / 8) : pick_shape((cols + 3) / 4);
  if (shape < 0) return hipErrorInvalidValue;
  // the element path never takes 1024 x 4 (its rows past 12288 columns took
  // the two-pass kernel above)
  const void* k = vector_ok ? shape_kernel<TenopSel<IO, true>::template K>(shape)
                            : shape_kernel<TenopSel<IO, false>::template K, 10>(shape);
  bool one_pass = false;  // tenop1_kernel: one row group a block, no loop
  int lanes = kShapes[shape].lanes;
  if constexpr (sizeof(E) == 2) {
    if (vector8_ok) k = shape_kernel<Tenop8Sel<IO>::template K>(shape);
    // rows of 65-512 vectors: a wave per row with the parameters widened
    // once per block (above; rows of 65-128 vectors: 64 lanes x 2 rather than
    // the table's 32 x 4, 8192 x 1024 fp16 in rows of 1056: 10.26 against
    // 10.57 us; 128 x 1: 10.63)
    if (vector8_ok && cols / 8 > 64 && cols / 8 <= 512) {
      const bool w8 = cols / 8 > 256;
      const int rpbw = w8 ? 8 : 16;
      const int64_t g16 = (rows + rpbw - 1) / rpbw;
      // one block per 16 rows, no loop (at most kRowsPerDispatch rows here)
      if (g16 > dispatch_blocks(64 * rpbw)) return hipErrorInvalidValue;
      {
        int icols8 = (int)cols;
        const E *xe = static_cast<const E*>(x), *bie = static_cast<const E*>(bias);
        const E *ge = static_cast<const E*>(gamma), *bee = static_cast<const E*>(beta);
        E* ye = static_cast<E*>(y);
        double inv8 = 1.0 / (double)cols;
        void* args8[] = {&xe, &ldx, &bie, &ge, &bee, &ye, &ldy, &rows, &icols8, &alpha, &c, &inv8};
        const void* kw = cols / 8 <= 128 ? reinterpret_cast<const void*>(&tenop8_wave_kernel<IO, 2>)
                         : !w8            ? reinterpret_cast<const void*>(&tenop8_wave_kernel<IO, 4>)
                                          : reinterpret_cast<const void*>(&tenop8_wave_kernel<IO, 8, 8>);
        return hipLaunchKernel(kw, dim3((unsigned)g16), dim3(64 * rpbw), args8, 0, s);
      }
    }
  } else {
    // fp32 rows of at most 256 vectors: one vector per lane (measured at
    // 1024 x 1024: 3.67 us against 3.80 for 64 lanes x 4; 8192 x 1024: 14.1
    // against 14.6)
    const int nvec = (int)((cols + 3) / 4);
    // rows of 2049-3072 vectors: 512 lanes x 6 rather than 1024 x 3
    // (1024 x 12288: 31.9 -> 26.8 us)
    if (vector_ok && nvec > 2048) {
      lanes = 512;
      k = reinterpret_cast<const void*>(&tenop_kernel<IO, 512, 6, 4>);
    }
    if (vector_ok && nvec <= 256) {
      lanes = nvec <= 16 ? 16 : nvec <= 32 ? 32 : nvec <= 64 ? 64 : nvec <= 128 ? 128 : 256;
      // one block per row group, no loop (at most kRowsPerDispatch rows here)
      const int64_t g1 = (rows + 256 / lanes - 1) / (256 / lanes);
      if (g1 > dispatch_blocks(256)) return hipErrorInvalidValue;
      one_pass = true;
      k = lanes == 16    ? reinterpret_cast<const void*>(&tenop1_kernel<16>)
          : lanes == 32  ? reinterpret_cast<const void*>(&tenop1_kernel<32>)
          : lanes == 64  ? reinterpret_cast<const void*>(&tenop1_kernel<64>)
          : lanes == 128 ? reinterpret_cast<const void*>(&tenop1_kernel<128>)
                         : reinterpret_cast<const void*>(&tenop1_kernel<256>);
    }
  }
  if (!k) return hipErrorInvalidValue;  // no layout instantiated for this case (not reached)
  const int block = block_for(lanes);
  const int rpb = block / lanes;
  const int64_t groups = (rows + rpb - 1) / rpb;
  // one block per row group (tenop_kernel and tenop8_kernel loop over the rest)
  int grid = (int)(groups < dispatch_blocks(block) ? groups : dispatch_blocks(block));
  // The looping kernels load bias, gamma and beta once per block: a grid of a
  // few blocks per compute unit, each looping over many row groups, moves
  // them from L2 a few hundred times instead of once per row (8192 x 4096
  // fp32: 48 KB a block, 400 MB at one block a row against 268 MB from HBM).
  // Same process, inputs out of the caches, us (one block a row -> this):
  // fp32 two a unit, 8192 x 4096 54.9 -> 44.8, 16384 x 2048 51.4 -> 44.6,
  // 8192 x 8192 107.2 -> 92.0, 4096 x 12288 79.1 -> 69.7; 16-bit four a unit,
  // 4096 x 8192 bf16 35.9 -> 31.2 (two 34.1, three 30.9, eight 30.7).
  if (!one_pass) {
    const int64_t cap = (sizeof(E) == 4 ? 2 : 4) * (int64_t)compute_units();
    if (cap > 0 && grid > cap) grid = (int)cap;
  }
  int icols = (int)cols;
  const E *xe = static_cast<const E*>(x), *bie = static_cast<const E*>(bias);
  const E *ge = static_cast<const E*>(gamma), *bee = static_cast<const E*>(beta);
  E* ye = static_cast<E*>(y);
  double inv_cols = 1.0 / (double)cols;  // the mean is the row sum times this
  void* args[] = {&xe, &ldx, &bie, &ge, &bee, &ye, &ldy, &rows, &icols, &alpha, &c, &inv_cols};
  return hipLaunchKernel(k, dim3(grid), dim3(block), args, 0, s);
}

}  // namespace

hipError_t launch_row_mean_2d(int dtype, const void* x, int64_t ldx, const void* bias, const void* gamma,
                              const void* beta, void* y, int64_t ldy, int64_t rows, int64_t cols,
                              double alpha, double c, hipStream_t s) {
  if (dtype == 0) return launch_tenop<F32IO>(x, ldx, bias, gamma, beta, y, ldy, rows, cols, alpha, c, s);
  if (dtype == 1) return launch_tenop<BF16IO>(x, ldx, bias, gamma, beta, y, ldy, rows, cols, alpha, c, s);
  return launch_tenop<F16IO>(x, ldx, bias, gamma, beta, y, ldy, rows, cols, alpha, c, s);
}

hipError_t launch_row_mean(const float* x, const float* bias, const float* gamma,
                           const float* beta, float* y, int64_t rows, int64_t cols, double alpha,
                           double c, hipStream_t s) {
  return launch_row_mean_2d(0, x, cols, bias, gamma, beta, y, cols, rows, cols, alpha, c, s);
}

}  // namespace mbp
