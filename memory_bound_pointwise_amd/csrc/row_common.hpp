// row_common.hpp -- pieces shared by the one-pass row kernels (LayerNorm family
// and the 10-op graph): block sizing, the (lanes, vectors-per-lane) layout
// tables, and small arithmetic helpers.
//
// Layout.  A row is served by a group of LANES consecutive lanes (16 ... 1024).
// Lane l of the group holds the vectors l, l + LANES, l + 2*LANES, ... of the
// row (VPL of them), so each load instruction of the group covers a contiguous
// stretch of the row (coalesced).  A vector is 16 bytes (4 fp32 / 8 bf16).
// Groups of up to 256 lanes run in 256-lane blocks (several rows per block);
// wider groups are one block.  The kernels loop over row groups with a grid
// stride, loading the per-column vectors (gamma, beta, bias) once per block;
// the launchers mostly give each block one row group (the hardware dispatcher
// then keeps the most loads in flight).
#pragma once

#include "mbp_device.hpp"

namespace mbp {
namespace rows {

constexpr int kMinBlock = 256;

// Block size for a group of LANES lanes: at least kMinBlock, one group if wider.
constexpr int block_for(int lanes) { return lanes > kMinBlock ? lanes : kMinBlock; }

// An empty asm that claims to rewrite its operand: the value is unchanged, but
// the compiler must treat it as new at this point of the program (used to keep
// a loop-invariant value from being widened once and held wide across a loop).
__device__ __forceinline__ void opaque(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(double& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(int& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(u32x4& v) {
#pragma unroll
  for (int w = 0; w < 4; ++w) opaque(v.w[w]);
}

// fused multiply-add in the type of the operands (__builtin_fma is binary64)
__device__ __forceinline__ float fma_t(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_t(double a, double b, double c) { return __builtin_fma(a, b, c); }

// 1 / sqrt(a).  fp32 statistics (16-bit I/O): v_rsq_f32, within about an
// ulp, where a correctly rounded square root and an IEEE division would cost
// some twenty instructions per row in every wave; binary64 statistics keep
// the correctly rounded root and division.
__device__ __forceinline__ float inv_sqrt(float a) { return __builtin_amdgcn_rsqf(a); }
__device__ __forceinline__ double inv_sqrt(double a) { return 1.0 / __builtin_sqrt(a); }

// v / n for a row length n: fp32 statistics multiply by v_rcp_f32(n) (within
// about an ulp of the quotient, exact for powers of two) instead of an IEEE
// division sequence; binary64 statistics divide.
__device__ __forceinline__ float div_cols(float v, int n) { return v * __builtin_amdgcn_rcpf((float)n); }
__device__ __forceinline__ double div_cols(double v, int n) { return v / (double)n; }

// The row mean s / n.  fp32: the quotient q = s * rcp(n) corrected once with
// its residual s - q n (exact in an fma), which lands within half an ulp but
// for rare ties and returns c exactly when s = n c exactly (a row of equal
// values), where q alone can be an ulp off, and that ulp, divided by the
// row's zero spread, would be scaled up by 1 / sqrt(eps); the mean's error
// counts |mean| / sigma times in the output, so it gets the two extra
// instructions the spread's quotient does not need.  binary64: division.
__device__ __forceinline__ float mean_cols(float s, int n) {
  const float nf = (float)n, r = __builtin_amdgcn_rcpf(nf);
  const float q = s * r;
  return __builtin_fmaf(__builtin_fmaf(-q, nf, s), r, q);
}
__device__ __forceinline__ double mean_cols(double s, int n) { return s / (double)n; }

// fp32 rows of more than kRegCols columns are not held in registers: they
// take the multi-pass row kernels (one 1024-lane block per row, the later
// passes rereading the row from the caches), which hold nothing per element.
// 16-bit LayerNorm and softmax rows stay in registers up to the 32768-column
// maximum (4096 vectors: 512 x 8); the 10-op graph's 16-bit rows past
// kRegCols take its multi-pass kernel.
constexpr int64_t kRegCols = 16384;

// (LANES, VPL) layouts.  The first layout whose LANES * VPL vectors cover the
// row is used.  At most 5 vectors (40 bf16 / 20 fp32 values) per lane keeps the
// kernels free of register spills; wider rows take wider groups.
struct Shape {
  int lanes, vpl;
};
constexpr Shape kShapes[] = {{16, 2},  {32, 2},  {32, 3},  {32, 4},   {64, 4},   {128, 4},
                             {128, 5}, {256, 4}, {512, 3}, {512, 4},  {1024, 3}, {1024, 4}};
constexpr int kNumShapes = sizeof(kShapes) / sizeof(Shape);

inline int pick_shape(int64_t nvec) {
  for (int i = 0; i < kNumShapes; ++i)
    if ((int64_t)kShapes[i].lanes * kShapes[i].vpl >= nvec) return i;
  return -1;
}

// Kernel pointer of layout i: K<LANES, VPL>::ptr().  LAST: the last layout
// the caller's family can be asked for (later ones are not instantiated; a
// larger i gives nullptr, which the callers never pass on).
template <template <int, int> class K, int LAST = 11>
const void* shape_kernel(int i) {
  switch (i) {
    case 0: return K<16, 2>::ptr();
    case 1: return K<32, 2>::ptr();
    case 2: return K<32, 3>::ptr();
    case 3: return K<32, 4>::ptr();
    case 4: return K<64, 4>::ptr();
    case 5: return K<128, 4>::ptr();
    case 6: return K<128, 5>::ptr();
    case 7: return K<256, 4>::ptr();
    case 8: return K<512, 3>::ptr();
    case 9: return K<512, 4>::ptr();
    case 10:
      if constexpr (LAST >= 10) return K<1024, 3>::ptr();
      else return nullptr;
    default:
      if constexpr (LAST >= 11) return K<1024, 4>::ptr();
      else return nullptr;
  }
}

// The 512-lane alternatives of the two 1024-lane layouts (index 10: 1024 x 3
// -> 512 x 6; 11: 1024 x 4 -> 512 x 8), for the kernels whose fp32 rows of
// 2049-4096 vectors measured faster in them (the caller says which).
// EIGHT false: the family has no 512 x 8 instance (the caller never asks for
// index 11 there).
template <template <int, int> class K, bool EIGHT = true>
const void* shape_kernel_512(int i) {
  if constexpr (EIGHT) return i == 10 ? K<512, 6>::ptr() : K<512, 8>::ptr();
  else return K<512, 6>::ptr();
}
// Layout i, or its 512-lane alternative where `alt` (instantiated only when
// the caller's kernel family can take it: ALT).
template <template <int, int> class K, bool ALT, bool EIGHT = true, int LAST = 11>
const void* shape_kernel_alt(int i, bool alt) {
  if constexpr (ALT) {
    if (alt) return shape_kernel_512<K, EIGHT>(i);
  }
  return shape_kernel<K, LAST>(i);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace rows
}  // namespace mbp
