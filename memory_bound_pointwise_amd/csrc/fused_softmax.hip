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
// Rows on 128-byte lines take 16-byte accesses (softmax_kernel); other rows
// whose x and y agree modulo 16 bytes take 16-byte windows rotated onto lines
// (softmax_win_kernel); anything else one element per access.
#include "mbp_internal.hpp"
#include "row_common.hpp"

#include <type_traits>

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

template <int S>
__device__ __forceinline__ void merge_stage(float& m, float& l) {
  float ma, mb, la, lb;
  lane_pair<S>(m, ma, mb);
  lane_pair<S>(l, la, lb);
  m = ma;
  l = la;
  ms_merge(m, l, mb, lb);
}

template <int LANES, int BLOCK>
__device__ __forceinline__ void group_merge(float& m, float& l, float* lds_m, float* lds_l) {
  constexpr int kIn = LANES < 64 ? LANES : 64;
  // butterfly stages as in wave_reduce; ms_merge is symmetric in its two pairs
  if constexpr (kIn > 1) merge_stage<1>(m, l);
  if constexpr (kIn > 2) merge_stage<2>(m, l);
  if constexpr (kIn > 4) merge_stage<4>(m, l);
  if constexpr (kIn > 8) merge_stage<8>(m, l);
  if constexpr (kIn > 16) merge_stage<16>(m, l);
  if constexpr (kIn > 32) merge_stage<32>(m, l);
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
                                                                   int cols, int64_t ldx, int64_t ldy) {
  typedef typename IO::elem E;
  constexpr int BLOCK = block_for(LANES);
  constexpr int RPB = BLOCK / LANES;
  __shared__ float lds_m[BLOCK / 64 > 0 ? BLOCK / 64 : 1], lds_l[BLOCK / 64 > 0 ? BLOCK / 64 : 1];

  const int lane = threadIdx.x % LANES;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LANES;
  const bool live = row < rows;
  const int nvec = (cols + VW - 1) / VW;
  // past the last row: reread the last row, store nothing
  const E* xr = x + (live ? row : rows - 1) * ldx;
  E* yr = y + row * ldy;

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

// fp32 rows of more than kRegCols columns: one 1024-lane block per row, three
// passes -- the row maximum M, then L = sum of exp(x - M), then the output
// exp(x - M) / L -- the later two rereading x from the caches; any width,
// alignment and row strides.  -inf entries give exactly 0, a row of -inf
// only gives NaN (0 / 0) and a NaN makes its row NaN, as in softmax_kernel.
template <class IO>
__global__ __launch_bounds__(1024) void softmax_wide_kernel(const typename IO::elem* x, typename IO::elem* y,
                                                            int64_t rows, int cols, int64_t ldx, int64_t ldy) {
  constexpr int LANES = 1024;
  __shared__ float red[2][LANES / 64];
  const int lane = threadIdx.x;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const typename IO::elem* xr = x + row * ldx;
    typename IO::elem* yr = y + row * ldy;
    float m = -__builtin_inff();
#pragma unroll 4
    for (int c = lane; c < cols; c += LANES) m = __builtin_fmaxf(m, IO::load1(xr, c));
    m = group_max<LANES, LANES>(m, red[0]);
    const float mm = (m == -__builtin_inff()) ? 0.0f : m;
    float l = 0.0f;
#pragma unroll 4
    for (int c = lane; c < cols; c += LANES) l += exp_f(IO::load1(xr, c) - mm);
    l = group_sum<LANES, LANES>(l, red[1]);
    const float inv_l = 1.0f / l;
#pragma unroll 4
    for (int c = lane; c < cols; c += LANES) IO::store1(yr, c, exp_f(IO::load1(xr, c) - mm) * inv_l);
    // red[0] is written again by the next row's maximum only after every lane
    // has passed this row's second barrier (red[1])
  }
}

// Element e of a packed output vector, as stored bits.
template <class IO>
__device__ __forceinline__ typename IO::elem stored_elem(const u32x4& v, int e) {
  if constexpr (IO::kVec == 8) return (typename IO::elem)(v.w[e >> 1] >> (16 * (e & 1)));
  else return __uint_as_float(v.w[e]);
}

// Rows off 16-byte boundaries (or on them, but not on 128-byte lines) whose x
// and y share one alignment modulo 16: the row is read and written in 16-byte
// windows of the tensors.  Row r starts s elements (sb bytes) into its first
// window and d windows into its 128-byte line (d = 0 when x and y do not agree
// modulo 128, or the row is shorter than 64 windows).  Relative slot j holds
// window j of the row, element e being column V*j + e - s; it sits at slot
// (j + d) mod nvec of the ln layouts, so every load and store instruction
// covers whole lines.  A row spanning nvec + 1 windows has its tail (fewer
// than s elements) folded into the head of relative slot 0, whose first s
// elements belong to the previous row.  Elements outside the row (in relative
// slots 0 and nvec - 1 only) become -inf, so they add nothing; the windows
// they share with a neighbouring row are stored element by element.  The host
// passes [r_lo, r_hi), the rows whose windows lie inside both tensors; the
// rest (at most a few rows at an unaligned start or end) take the last
// edge_blocks blocks, element by element.
template <class IO, int LANES, int VPL>
__global__ __launch_bounds__(block_for(LANES)) void softmax_win_kernel(const typename IO::elem* x,
                                                                       typename IO::elem* y, int64_t rows,
                                                                       int cols, int64_t ldx, int64_t ldy,
                                                                       int line, int64_t r_lo,
                                                                       int64_t r_hi, int edge_blocks) {
  typedef typename IO::elem E;
  constexpr int ES = (int)sizeof(E);
  constexpr int V = IO::kVec;
  constexpr int BLOCK = block_for(LANES);
  constexpr int RPB = BLOCK / LANES;
  constexpr float kNegInf = -__builtin_inff();
  __shared__ float lds_m[BLOCK / 64 > 0 ? BLOCK / 64 : 1], lds_l[BLOCK / 64 > 0 ? BLOCK / 64 : 1];

  const int lane = threadIdx.x % LANES;
  const int sub = threadIdx.x / LANES;
  const int nb = (int)gridDim.x - edge_blocks;

  if ((int)blockIdx.x >= nb) {
    // edge rows: lane l takes columns l, l + LANES, ...; three passes over the
    // row (max, sum, output), the later ones from cache
    const int64_t i = (int64_t)((int)blockIdx.x - nb) * RPB + sub;
    const int64_t n_edge = r_lo + (rows - r_hi);
    const bool live = i < n_edge;
    const int64_t row = !live ? 0 : (i < r_lo ? i : r_hi + (i - r_lo));
    const E* xr = x + row * ldx;
    float m = kNegInf;
    for (int c = lane; c < cols; c += LANES) m = __builtin_fmaxf(m, IO::load1(xr, c));
    const float mm = (m == kNegInf) ? 0.0f : m;
    float l = 0.0f;
    for (int c = lane; c < cols; c += LANES) l += exp_f(IO::load1(xr, c) - mm);
    const float m_lane = m;
    group_merge<LANES, BLOCK>(m, l, lds_m, lds_l);
    float f;
    if (m == kNegInf) f = __builtin_nanf("");
    else if (m_lane == kNegInf) f = 0.0f;
    else f = exp_f(m_lane - m) / l;
    if (live)
      for (int c = lane; c < cols; c += LANES) IO::store1(y + row * ldy, c, exp_f(IO::load1(xr, c) - mm) * f);
    return;
  }

  const int64_t row = r_lo + (int64_t)blockIdx.x * RPB + sub;
  const bool live = row < r_hi;
  const int64_t lrow = live ? row : r_hi - 1;  // past the last row: reread it, store nothing
  const char* xb = reinterpret_cast<const char*>(x) + (int64_t)ES * lrow * ldx;
  const int sl = (int)(reinterpret_cast<uintptr_t>(xb) & (unsigned)(line - 1));
  const int d = sl >> 4, sb = sl & 15, s = sb / ES;
  const int nvec = (cols + V - 1) / V;
  const bool fold = ((sb + ES * cols + 15) >> 4) > nvec;
  const int klast = (nvec - 1) / LANES;
  const u32x4* sx = reinterpret_cast<const u32x4*>(xb - sb);

  // relative slot of round k (clamped for slots past the row) and whether the
  // slot is used
  int jr[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int p = min(lane + k * LANES, nvec - 1);
    jr[k] = p < d ? p - d + nvec : p - d;
  }
  u32x4 xw[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) xw[k] = load_nt(sx + jr[k]);
  if (fold && lane == d) {  // relative slot 0 takes the row's last window into its bytes [0, sb)
    const u32x4 xf = load_nt(sx + nvec);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int sh = min(max(sb - 4 * t, 0), 4);  // bytes of word t taken from the tail
      const uint32_t keep = sh == 4 ? 0u : 0xffffffffu << (8 * sh);
      xw[0].w[t] = (xw[0].w[t] & keep) | (xf.w[t] & ~keep);
    }
  }
  // column of element e of relative slot j (-1: outside the row)
  auto col_of = [&](int j, int e) -> int {
    if (j == 0 && e < s) return fold ? V * nvec + e - s : -1;
    return V * j + e - s;
  };
  float v[VPL][V];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const bool used = lane + k * LANES < nvec;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      float t = IO::get(xw[k], e);
      if (!used) t = kNegInf;
      if (k == 0 || k == klast) {  // relative slots 0 and nvec - 1 sit in these rounds
        const int c = col_of(jr[k], e);
        if (c < 0 || c >= cols) t = kNegInf;
      }
      v[k][e] = t;
    }
  }

  float m = kNegInf;
#pragma unroll
  for (int k = 0; k < VPL; ++k)
#pragma unroll
    for (int e = 0; e < V; ++e) m = __builtin_fmaxf(m, v[k][e]);
  const float mm = (m == kNegInf) ? 0.0f : m;
  float l = 0.0f;
#pragma unroll
  for (int k = 0; k < VPL; ++k)
#pragma unroll
    for (int e = 0; e < V; ++e) {
      v[k][e] = exp_f(v[k][e] - mm);
      l += v[k][e];
    }
  const float m_lane = m;
  group_merge<LANES, BLOCK>(m, l, lds_m, lds_l);
  float f;
  if (m == kNegInf) f = __builtin_nanf("");
  else if (m_lane == kNegInf) f = 0.0f;
  else f = exp_f(m_lane - m) / l;
  if (!live) return;

  char* yb = reinterpret_cast<char*>(y) + (int64_t)ES * row * ldy;
  u32x4* dst = reinterpret_cast<u32x4*>(yb - sb);  // the row of y agrees with the row of x modulo 16
  // fp32: element stores through a volatile pointer, so that the compiler
  // keeps the whole-window store one dwordx4 instead of sinking its last dword
  // into a tail shared with the element stores; 16-bit: plain stores
  typedef typename std::conditional<ES == 4, volatile E, E>::type VE;
  VE* vrow = reinterpret_cast<E*>(yb);
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    if (lane + k * LANES >= nvec) continue;
    const int j = jr[k];
    float o[V];
#pragma unroll
    for (int e = 0; e < V; ++e) o[e] = v[k][e] * f;
    u32x4 ov;
    if constexpr (ES == 4) {
#pragma unroll
      for (int w = 0; w < 4; ++w) ov.w[w] = __float_as_uint(o[w]);
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (__is_same(IO, BF16IO))
          ov.w[w] = pack_bf16x2(o[2 * w], o[2 * w + 1]);
        else
          ov.w[w] = (uint32_t)f32_to_f16(o[2 * w]) | ((uint32_t)f32_to_f16(o[2 * w + 1]) << 16);
      }
    }
    // window j holds columns V*j - s + e; relative slots 0 and nvec - 1 may
    // share their window with a neighbouring row: store only [ea, eb)
    int ea = j == 0 ? s : 0;
    int eb = min(V, cols - (V * j - s));
    if (ea == 0 && eb == V) {
      store_nt(dst + j, ov);
    } else {
      opaque(ea);  // keep the per-element tests in this branch
      opaque(eb);
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (e >= ea && e < eb) vrow[V * j - s + e] = stored_elem<IO>(ov, e);
      if (fold && j == 0) {  // the folded tail: columns V*nvec - s + e
        int fb = cols - (V * nvec - s);
        opaque(fb);
#pragma unroll
        for (int e = 0; e < V; ++e)
          if (e < fb) vrow[V * nvec - s + e] = stored_elem<IO>(ov, e);
      }
    }
  }
}

template <class IO>
struct SoftmaxWinSel {
  template <int L, int V>
  struct K {
    static const void* ptr() { return reinterpret_cast<const void*>(&softmax_win_kernel<IO, L, V>); }
  };
};

template <class IO, bool VEC>
struct SoftmaxSel {
  template <int L, int V>
  struct K {
    static const void* ptr() {
      if constexpr (VEC) return reinterpret_cast<const void*>(&softmax_kernel<IO, L, V, IO::kVec>);
      else return reinterpret_cast<const void*>(&softmax_kernel<IO, L, IO::kVec * V, 1>);
    }
  };
};

template <class IO>
hipError_t launch_softmax_io(const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows, int64_t cols,
                             hipStream_t s) {
  typedef typename IO::elem E;
  constexpr int V = IO::kVec;
  constexpr int64_t ES = (int64_t)sizeof(E);
  // softmax_kernel and softmax_win_kernel take one block per row group and no
  // loop: rows past what one dispatch can address go in chunks (rows are
  // independent; a stride of 0 keeps its one row)
  if (rows > kRowsPerDispatch) {
    for (int64_t r0 = 0; r0 < rows; r0 += kRowsPerDispatch) {
      const int64_t n = rows - r0 < kRowsPerDispatch ? rows - r0 : kRowsPerDispatch;
      const hipError_t e = launch_softmax_io<IO>(static_cast<const E*>(x) + r0 * ldx, ldx,
                                                 static_cast<E*>(y) + r0 * ldy, ldy, n, cols, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (rows == 1) ldx = ldy = cols;  // one row: its stride is never used
  const int64_t nvec = (cols + V - 1) / V;
  // fp32 rows past kRegCols columns take the multi-pass kernel; 16-bit rows
  // (at most 4096 vectors of 8 at the 32768-column maximum) all stay in
  // registers (512-lane layouts, below: 16384 rows of 24576 bf16 606.1 ->
  // 259.9 us, 32768 columns 815.1 -> 376.9 us)
  if constexpr (ES == 4) {
    if (cols > kRegCols) {
      const int wgrid = (int)(rows < 4096 ? rows : 4096);
      hipLaunchKernelGGL(softmax_wide_kernel<IO>, dim3(wgrid), dim3(1024), 0, s, static_cast<const E*>(x),
                         static_cast<E*>(y), rows, (int)cols, ldx, ldy);
      return hipGetLastError();
    }
  }
  const int shape = pick_shape(nvec);
  if (shape < 0) return hipErrorInvalidValue;
  // 16-bit rows of 2049-4096 vectors: 512 x 6 / 512 x 8 (the 1024-lane
  // layouts are not instantiated for them)
  constexpr bool kAlt16 = ES == 2;
  const bool a16 = kAlt16 && shape >= 10;
  const int block = a16 ? 512 : block_for(kShapes[shape].lanes);
  const int rpb = a16 ? 1 : block / kShapes[shape].lanes;
  const E* xe = static_cast<const E*>(x);
  E* ye = static_cast<E*>(y);
  int icols = (int)cols;
  const uintptr_t ax = reinterpret_cast<uintptr_t>(x), ay = reinterpret_cast<uintptr_t>(y);
  const int64_t px = ES * ldx, py = ES * ldy;  // row pitches (bytes)
  // rows on 16-byte boundaries: aligned bases, pitches of whole vectors
  const bool vec = cols % V == 0 && aligned16(x) && aligned16(y) && px % 16 == 0 && py % 16 == 0;
  // windows on 128-byte lines need every row of x and y to agree modulo 128
  // and rows of a wave's worth of windows; rows on 16-byte boundaries whose
  // pitches are multiples of 128 bytes are on lines already (a 4088-wide bf16
  // row stream measured 386 us against 342 for 4096 before the windows were
  // rotated onto lines)
  const bool line_ok = ((ax ^ ay) & 127) == 0 && (px - py) % 128 == 0 && nvec >= 64;
  const bool win_ok = ((ax ^ ay) & 15) == 0 && (px - py) % 16 == 0 && ldx > 0;
  if (win_ok && !(vec && ((px % 128 == 0 && py % 128 == 0) || !line_ok))) {
    // Rows whose windows lie inside both tensors: [r_lo, r_hi).  A row
    // starting fewer than 16 - (x mod 16) bytes past an unaligned start, or
    // ending fewer than (end mod 16) bytes before an unaligned end, has a
    // window that reaches outside: the first ceil((16 - x mod 16) / pitch)
    // and the last ceil((end mod 16) / pitch) rows (x and y end alike modulo
    // 16; the smaller pitch counts).
    // Rows of 2049-4096 vectors: 512-lane groups of 6 or 8 vectors a lane
    // instead of 1024 x 3 / 1024 x 4 (fp32, 8192 rows of 12287: 2816 ->
    // 2239 us; fp32 rows on 16-byte boundaries, which the vector kernel
    // takes, measured 1.5-8.5% slower in them and keep the 1024-lane ones)
    const bool w512 = shape >= 10;
    const int wblock = w512 ? 512 : block, wrpb = w512 ? 1 : rpb;
    const int64_t pmin = px < py ? px : py;
    const int64_t mb = (int64_t)(ax & 15);
    const int64_t me = (int64_t)((ax + (uintptr_t)(ES * ((rows - 1) * ldx + cols))) & 15);
    int64_t r_lo = mb == 0 ? 0 : (16 - mb + pmin - 1) / pmin;
    int64_t r_hi = me == 0 ? rows : rows - (me + pmin - 1) / pmin;
    if (r_lo > rows) r_lo = rows;
    if (r_hi < r_lo) r_hi = r_lo;
    const int64_t n_edge = r_lo + (rows - r_hi);
    const int64_t main_blocks = (r_hi - r_lo + wrpb - 1) / wrpb;
    const int64_t edge_blocks = (n_edge + wrpb - 1) / wrpb;
    // one block per row group (at most kRowsPerDispatch rows here)
    if (main_blocks + edge_blocks > dispatch_blocks(wblock)) return hipErrorInvalidValue;
    int line = line_ok ? 128 : 16;
    int eb = (int)edge_blocks;
    const void* k = shape_kernel_alt<SoftmaxWinSel<IO>::template K, true, true, 9>(shape, w512);
    void* args[] = {&xe, &ye, &rows, &icols, &ldx, &ldy, &line, &r_lo, &r_hi, &eb};
    return hipLaunchKernel(k, dim3((unsigned)(main_blocks + edge_blocks)), dim3(wblock), args, 0, s);
  }
  const void* k = vec ? shape_kernel_alt<SoftmaxSel<IO, true>::template K, kAlt16, true, kAlt16 ? 9 : 11>(shape, a16)
                      : shape_kernel_alt<SoftmaxSel<IO, false>::template K, kAlt16, true, kAlt16 ? 9 : 11>(shape, a16);
  const int64_t groups = (rows + rpb - 1) / rpb;
  const int grid = (int)(groups < dispatch_blocks(block) ? groups : dispatch_blocks(block));
  if (groups > grid) return hipErrorInvalidValue;  // one block per row group (at most kRowsPerDispatch rows here)
  void* args[] = {&xe, &ye, &rows, &icols, &ldx, &ldy};
  return hipLaunchKernel(k, dim3(grid), dim3(block), args, 0, s);
}

}  // namespace

hipError_t launch_softmax(int dtype, const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows,
                          int64_t cols, hipStream_t s) {
  if (dtype == 0) return launch_softmax_io<F32IO>(x, ldx, y, ldy, rows, cols, s);
  if (dtype == 1) return launch_softmax_io<BF16IO>(x, ldx, y, ldy, rows, cols, s);
  return launch_softmax_io<F16IO>(x, ldx, y, ldy, rows, cols, s);
}

}  // namespace mbp
