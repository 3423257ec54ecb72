// mbp_device.hpp -- device-side building blocks shared by the HIP kernels of
// libmbp: 128-bit vector types, bfloat16 unpack/pack, and the deterministic
// lane-group reductions used by every row reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mbp {

// 16 bytes = one global_load_dwordx4 / global_store_dwordx4 per lane.
struct alignas(16) u32x4 {
  uint32_t w[4];
};

// Streaming (nontemporal) 128-bit access: global_load/store_dwordx4 with the
// nt bit.  Data read once or written once should not displace reused lines
// (gamma, beta, bias) from the caches; on MI355X this raises the sustained
// bandwidth of a 2-read/1-write row stream from ~5.7 to ~6.4 TB/s.
__device__ __forceinline__ u32x4 load_nt(const u32x4* p) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) r.w[w] = __builtin_nontemporal_load(&p->w[w]);
  return r;
}
__device__ __forceinline__ void store_nt(u32x4* p, const u32x4& v) {
#pragma unroll
  for (int w = 0; w < 4; ++w) __builtin_nontemporal_store(v.w[w], &p->w[w]);
}
__device__ __forceinline__ float4 load_nt(const float4* p) {
  return make_float4(__builtin_nontemporal_load(&p->x), __builtin_nontemporal_load(&p->y),
                     __builtin_nontemporal_load(&p->z), __builtin_nontemporal_load(&p->w));
}
__device__ __forceinline__ void store_nt(float4* p, const float4& v) {
  __builtin_nontemporal_store(v.x, &p->x);
  __builtin_nontemporal_store(v.y, &p->y);
  __builtin_nontemporal_store(v.z, &p->z);
  __builtin_nontemporal_store(v.w, &p->w);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// bfloat16 is the upper half of a binary32; widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two fp32 values -> one word of two bf16, round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Element type traits for the I/O types.
struct F32IO {
  typedef float elem;
  static constexpr int kVec = 4;  // elements per 16-byte vector
  __device__ __forceinline__ static float load1(const elem* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store1(elem* p, int64_t i, float v) { p[i] = v; }
  __device__ __forceinline__ static float get(const u32x4& v, int e) { return __uint_as_float(v.w[e]); }
};

struct BF16IO {
  typedef uint16_t elem;
  static constexpr int kVec = 8;
  __device__ __forceinline__ static float load1(const elem* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store1(elem* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
  __device__ __forceinline__ static float get(const u32x4& v, int e) {
    return (e & 1) ? bf16_hi(v.w[e >> 1]) : bf16_lo(v.w[e >> 1]);
  }
};

// IEEE binary16; widening to fp32 is exact, narrowing (v_cvt_f16_f32) rounds
// to nearest even.
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

struct F16IO {
  typedef uint16_t elem;
  static constexpr int kVec = 8;
  __device__ __forceinline__ static float load1(const elem* p, int64_t i) { return f16_to_f32(p[i]); }
  __device__ __forceinline__ static void store1(elem* p, int64_t i, float v) { p[i] = f32_to_f16(v); }
  __device__ __forceinline__ static float get(const u32x4& v, int e) {
    return f16_to_f32((uint16_t)(v.w[e >> 1] >> (16 * (e & 1))));
  }
};

// binary64 -> binary32 rounded to odd: truncate toward zero, then set the
// last significand bit if anything was dropped.  Rounding that value to
// nearest even into a format with at most 22 significand bits (binary16,
// bfloat16) equals rounding the binary64 value directly (round-to-odd as the
// intermediate of a double rounding: S. Boldo and G. Melquiond, "Emulation of
// FMA and correctly rounded sums: proved algorithms using rounding to odd",
// IEEE Trans. Computers 57(4), 2008).
__device__ __forceinline__ float round_odd_f32(double d) {
  float r = (float)d;  // nearest even
  const double back = (double)r;
  if (back != d && d == d) {
    uint32_t u = __float_as_uint(r);
    if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1;  // rounded away from zero: step back
    u |= 1u;                                                // sticky bit
    r = __uint_as_float(u);
  }
  return r;
}

// The stored bits of a binary64 value, rounded once to nearest even.
template <class IO>
__device__ __forceinline__ uint32_t narrow_bits(double d) {
  if constexpr (sizeof(typename IO::elem) == 4) return __float_as_uint((float)d);
  else if constexpr (IO::kVec == 8 && __is_same(IO, BF16IO)) return f32_to_bf16(round_odd_f32(d));
  else return f32_to_f16(round_odd_f32(d));
}

// N binary64 values -> their stored bits, each rounded once to nearest even,
// as narrow_bits gives them.  For the 16-bit types: rounding to nearest
// binary32 first and then to 16 bits gives the same result unless the binary32
// value is itself a halfway point of the 16-bit format -- every such halfway
// point is a binary32 value and both roundings are monotone, so a value that
// does not land on one stays on its side of every halfway point.  Halfway
// points have the bits below the 16-bit significand equal to 100...0 (bf16:
// the low 16 bits, at every exponent; binary16: the low 13 bits in its normal
// range, including the boundary to infinity, 65520); binary16's subnormal
// range, whose halfway points sit at other positions, is sent the same way.
// Those values -- about one in 8192 -- take round_odd_f32, once per N values
// when any lane has one.
template <class IO, int N>
__device__ __forceinline__ void narrow_n(const double* d, uint32_t* o) {
  if constexpr (sizeof(typename IO::elem) == 4) {
#pragma unroll
    for (int e = 0; e < N; ++e) o[e] = __float_as_uint((float)d[e]);
  } else {
    constexpr bool kBf16 = __is_same(IO, BF16IO);
    float r[N];
    bool tie = false;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      r[e] = (float)d[e];
      const uint32_t u = __float_as_uint(r[e]);
      if constexpr (kBf16) tie |= (u & 0xffffu) == 0x8000u;
      else tie |= ((u & 0x1fffu) == 0x1000u) | (__builtin_fabsf(r[e]) < 0x1p-14f);
    }
    if (__builtin_expect(tie, 0)) {
#pragma unroll
      for (int e = 0; e < N; ++e) r[e] = round_odd_f32(d[e]);
    }
#pragma unroll
    for (int e = 0; e < N; ++e) o[e] = kBf16 ? f32_to_bf16(r[e]) : f32_to_f16(r[e]);
  }
}

// tanh-approximated GeLU, 0.5 u (1 + tanh(k0 (u + k1 u^3))) with k0 = 0.7978845608,
// k1 = 0.044715 ("算子融合与 Kernel 优化", section 2.3), evaluated through the exact
// identity 0.5 (1 + tanh z) = 1 / (1 + exp(-2 z)) and exp(w) = exp2(w log2 e):
// one v_exp_f32 and one v_rcp_f32.  For u << 0, exp2 overflows to +inf and the
// result is -0, the limit of the formula.
__device__ __forceinline__ float gelu_tanh_f32(float u) {
  constexpr float kA = (float)(-2.0 * 0.7978845608 * 1.4426950408889634);
  constexpr float kB = (float)(-2.0 * 0.7978845608 * 0.044715 * 1.4426950408889634);
  const float u2 = u * u;
  const float w = u * __builtin_fmaf(u2, kB, kA);
  const float e = __builtin_amdgcn_exp2f(w);
  return u * __builtin_amdgcn_rcpf(1.0f + e);
}

// Workgroup barrier for LDS traffic only: wait for this wave's LDS operations,
// then s_barrier.  Unlike __syncthreads() it does not wait for outstanding
// global stores (a workgroup release fence would add s_waitcnt vmcnt(0)),
// which lets the streaming stores of one row overlap the next row's work.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// a ^ b ^ c in one instruction: v_bitop3_b32 with the truth table of a
// three-way XOR (0x96); gfx950 has no v_xor3_b32 and the compiler does not
// form this from two XORs.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Philox4x32-10 (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC'11): counter
// (q lo, q hi, offset lo, offset hi), key (seed lo, seed hi); each round
// multiplies counter words 0 and 2 by 0xD2511F53 and 0xCD9E8D57 into 64-bit
// products and mixes in words 1 and 3 and the key, which advances by the Weyl
// constants 0x9E3779B9 and 0xBB67AE85.
__device__ __forceinline__ void philox4x32_10(uint64_t q, uint64_t seed, uint64_t offset, uint32_t out[4]) {
  uint32_t c0 = (uint32_t)q, c1 = (uint32_t)(q >> 32), c2 = (uint32_t)offset, c3 = (uint32_t)(offset >> 32);
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
    const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// The 16 random bits of elements i0 .. i0 + N - 1 (N = 1, 4 or 8) of a
// dropout with (seed, offset): half i mod 8 of block i div 8.  ALIGNED: i0 is
// a multiple of N, so the elements lie in one block; otherwise they may span two.
template <int N, bool ALIGNED>
__device__ __forceinline__ void dropout_bits(uint64_t i0, uint64_t seed, uint64_t offset, uint32_t* h) {
  uint32_t b0[4];
  philox4x32_10(i0 >> 3, seed, offset, b0);
  if constexpr (ALIGNED) {
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const int t = N == 8 ? e : (int)(i0 & 7) + e;  // half index within the block
      const int wi = t >> 1;
      const uint32_t w = N == 8 ? b0[e >> 1] : (wi == 0 ? b0[0] : wi == 1 ? b0[1] : wi == 2 ? b0[2] : b0[3]);
      h[e] = (t & 1) ? (w >> 16) : (w & 0xFFFFu);
    }
  } else {
    uint32_t b1[4];
    philox4x32_10((i0 >> 3) + 1, seed, offset, b1);
    const int o = (int)(i0 & 7);
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const int t = o + e;  // half index within the two blocks (0 .. 14)
      const int wi = (t & 7) >> 1;
      const uint32_t w0v = wi == 0 ? b0[0] : wi == 1 ? b0[1] : wi == 2 ? b0[2] : b0[3];
      const uint32_t w1v = wi == 0 ? b1[0] : wi == 1 ? b1[1] : wi == 2 ? b1[2] : b1[3];
      const uint32_t w = t < 8 ? w0v : w1v;
      h[e] = (t & 1) ? (w >> 16) : (w & 0xFFFFu);
    }
  }
}

// Butterfly exchange within a wave, without LDS traffic.  lane_pair<S>(v, a, b)
// (S = 1, 2, 4, 8, 16, 32) hands each lane the values {a, b} of itself and of
// its partner at stage S of an all-reduce; both lanes of a pair get the same
// two values, so a symmetric combine (a + b, max) leaves them bitwise equal.
// Stages 1 and 2 pair lane i with i ^ 1 and i ^ 2 (DPP quad permutations).
// Stages 4 and 8 pair it with 7 - i and 15 - i within its 8 and 16 lanes (DPP
// row_half_mirror, row_mirror): like i ^ 4 and i ^ 8 these pair whole blocks of
// 4 and 8 lanes, and once each block holds a single value, as it does after the
// earlier stages, they combine the same values.  Stages 16 and 32 swap rows of
// 16 lanes and the halves of the wave (gfx950's v_permlane16_swap and
// v_permlane32_swap), which give both lanes {lower one's value, upper one's}.
template <int S>
__device__ __forceinline__ void lane_pair(uint32_t v, uint32_t& a, uint32_t& b) {
  if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  } else if constexpr (S == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  } else {
    static_assert(S == 1 || S == 2 || S == 4 || S == 8, "stage");
    constexpr int kCtrl = S == 1 ? 0xB1 : S == 2 ? 0x4E : S == 4 ? 0x141 : 0x140;
    a = v;
    b = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xf, 0xf, false);
  }
}
template <int S>
__device__ __forceinline__ void lane_pair(float v, float& a, float& b) {
  uint32_t ua, ub;
  lane_pair<S>(__builtin_bit_cast(uint32_t, v), ua, ub);
  a = __builtin_bit_cast(float, ua);
  b = __builtin_bit_cast(float, ub);
}
template <int S>
__device__ __forceinline__ void lane_pair(double v, double& a, double& b) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  uint32_t la, lb, ha, hb;
  lane_pair<S>((uint32_t)u, la, lb);
  lane_pair<S>((uint32_t)(u >> 32), ha, hb);
  a = __builtin_bit_cast(double, ((uint64_t)ha << 32) | la);
  b = __builtin_bit_cast(double, ((uint64_t)hb << 32) | lb);
}

struct SumOp {
  template <typename T>
  __device__ __forceinline__ T operator()(T a, T b) const { return a + b; }
};
// `>` never selects a NaN: callers keep NaN out of the operands.
struct MaxOp {
  template <typename T>
  __device__ __forceinline__ T operator()(T a, T b) const { return b > a ? b : a; }
};

// All-reduce of v with op over groups of N consecutive lanes (N a power of
// two, at most 64) inside a wave; every lane of a group ends with bitwise the
// same value.
template <int N, typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  T a, b;
  if constexpr (N > 1) { lane_pair<1>(v, a, b); v = op(a, b); }
  if constexpr (N > 2) { lane_pair<2>(v, a, b); v = op(a, b); }
  if constexpr (N > 4) { lane_pair<4>(v, a, b); v = op(a, b); }
  if constexpr (N > 8) { lane_pair<8>(v, a, b); v = op(a, b); }
  if constexpr (N > 16) { lane_pair<16>(v, a, b); v = op(a, b); }
  if constexpr (N > 32) { lane_pair<32>(v, a, b); v = op(a, b); }
  return v;
}

// op over a group of LANES consecutive lanes (LANES a power of two), every
// lane of the group ending with bitwise the same value, independent of timing.
// Within a wave: wave_reduce.  Groups wider than a wave: each wave writes its
// result to LDS, one barrier, and every lane combines the group's partials in
// wave order.  `lds` must hold one slot per wave of the block and must not be
// rewritten by any lane before all lanes have read it (callers alternate
// between slots).
template <int LANES, int BLOCK, typename T, typename Op>
__device__ __forceinline__ T group_reduce(T v, T* lds, Op op) {
  v = wave_reduce<(LANES < 64 ? LANES : 64)>(v, op);
  if constexpr (LANES <= 64) {
    return v;
  } else {
    static_assert(LANES % 64 == 0 && BLOCK % LANES == 0, "wave-multiple groups");
    constexpr int kWaves = LANES / 64;
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[wave] = v;
    lds_barrier();
    const int first = (threadIdx.x / LANES) * kWaves;
    T s = lds[first];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s = op(s, lds[first + w]);
    return s;
  }
}

// Sum of v over a group of LANES consecutive lanes, as group_reduce.
template <int LANES, int BLOCK, typename T>
__device__ __forceinline__ T group_sum(T v, T* lds) {
  return group_reduce<LANES, BLOCK>(v, lds, SumOp());
}

// Maximum of v over a group of LANES consecutive lanes, as group_reduce.  The
// maximum is exact and independent of the combine order.  Callers keep NaN out
// of v (a NaN element propagates later, as in the sum of exponentials).
template <int LANES, int BLOCK, typename T>
__device__ __forceinline__ T group_max(T v, T* lds) {
  return group_reduce<LANES, BLOCK>(v, lds, MaxOp());
}

}  // namespace mbp
