// abi.cpp -- the C ABI of libmbp (declared in include/mbp.h): host-side
// argument validation, workspace carving for the unfused variants, and the
// per-thread error message.  Nothing here touches the device until every
// argument has been checked; then the launchers in fused_*.hip / unfused.hip
// enqueue the work on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <initializer_list>
#include <new>
#include <cstdio>
#include <string>
#include <tuple>
#include <utility>

#include "mbp.h"
#include "mbp_internal.hpp"

namespace {

thread_local std::string g_last_error;

mbp_status fail(mbp_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mbp_status fail(mbp_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

mbp_status ok() {
  g_last_error.clear();
  return MBP_OK;
}

mbp_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MBP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A byte range [p, p + bytes).
struct Span {
  const void* p;
  size_t bytes;
};

bool overlaps(Span a, Span b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// The output may be exactly one of the inputs (same base, same extent) when
// in-place use is allowed; any other intersection is an error.
bool bad_overlap(Span out, Span in, bool exact_ok) {
  if (!overlaps(out, in)) return false;
  return !(exact_ok && out.p == in.p && out.bytes == in.bytes);
}

bool misaligned(const void* p, size_t a) { return p && (reinterpret_cast<uintptr_t>(p) % a) != 0; }

constexpr int64_t kMaxElems = INT64_MAX / 64;

// rows x cols with 0 <= rows, 1 <= cols <= MBP_MAX_COLS, product within range.
mbp_status check_rows_cols(int64_t rows, int64_t cols) {
  if (rows < 0) return fail(MBP_ERR_SHAPE, "rows must be >= 0 (got %lld)", (long long)rows);
  if (cols <= 0 || cols > MBP_MAX_COLS)
    return fail(MBP_ERR_SHAPE, "cols must be in [1, %d] (got %lld)", MBP_MAX_COLS, (long long)cols);
  if (rows > kMaxElems / cols) return fail(MBP_ERR_SHAPE, "rows * cols overflows");
  return MBP_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// ---------------------------------------------------------------- workspace

constexpr size_t kWsAlign = 256;
size_t round_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

struct Carver {
  char* base;
  size_t used = 0;
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used += round_up(bytes);
    return p;
  }
};

// Buffers of the unfused variants, carved in a fixed order from the workspace.
struct ChainWs {
  float *a, *b;
};
struct RowMeanWs {
  float *a, *b, *c, *m;
};
struct GroupedWs {
  float *s, *m;
};
struct LnWs {
  void *r, *a, *b;
  float *m, *v;
};

size_t chain_ws(char* base, int64_t n, ChainWs* w) {
  Carver c{base};
  ChainWs t;
  t.a = (float*)c.take(n * 4);
  t.b = (float*)c.take(n * 4);
  if (w) *w = t;
  return c.used;
}

size_t row_mean_ws(char* base, int64_t rows, int64_t cols, RowMeanWs* w) {
  Carver c{base};
  RowMeanWs t;
  t.a = (float*)c.take(rows * cols * 4);
  t.b = (float*)c.take(rows * cols * 4);
  t.c = (float*)c.take(rows * cols * 4);
  t.m = (float*)c.take(rows * 4);
  if (w) *w = t;
  return c.used;
}

// softmax as eager ops: m [rows], d = x - m, e = exp(d) [rows, cols] in the
// I/O type, l [rows]
struct SoftmaxWs {
  float* m;
  void *d, *e;
  float* l;
};

size_t softmax_ws(char* base, int dtype, int64_t rows, int64_t cols, SoftmaxWs* w) {
  Carver c{base};
  const size_t full = (size_t)rows * cols * (dtype == MBP_BF16 ? 2 : 4);
  SoftmaxWs t;
  t.m = (float*)c.take(rows * 4);
  t.d = c.take(full);
  t.e = c.take(full);
  t.l = (float*)c.take(rows * 4);
  if (w) *w = t;
  return c.used;
}

size_t grouped_ws(char* base, int64_t rows, int64_t cols, GroupedWs* w) {
  Carver c{base};
  GroupedWs t;
  t.s = (float*)c.take(rows * cols * 4);
  t.m = (float*)c.take(rows * 4);
  if (w) *w = t;
  return c.used;
}

size_t ln_ws(char* base, int dtype, int64_t rows, int64_t cols, bool res, bool gelu, int gran,
             LnWs* w) {
  Carver c{base};
  const size_t es = dtype == MBP_BF16 ? 2 : 4;
  const size_t full = (size_t)rows * cols * es;
  LnWs t{nullptr, nullptr, nullptr, nullptr, nullptr};
  if (res) t.r = c.take(full);
  if (gran == MBP_UNFUSED_PRIMITIVE) {
    t.a = c.take(full);
    t.b = c.take(full);
    t.m = (float*)c.take(rows * 4);
    t.v = (float*)c.take(rows * 4);
  } else if (gelu) {
    t.a = c.take(full);
  }
  if (w) *w = t;
  return c.used;
}

mbp_status check_workspace(void* ws, size_t have, size_t need, std::initializer_list<Span> args) {
  if (need == 0) return MBP_OK;
  if (!ws) return fail(MBP_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (misaligned(ws, kWsAlign)) return fail(MBP_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(MBP_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
  for (const Span& a : args)
    if (overlaps(Span{ws, need}, a)) return fail(MBP_ERR_OVERLAP, "workspace overlaps an argument");
  return MBP_OK;
}

// ---------------------------------------------------------------- common checks

mbp_status check_chain(const float* x, const float* b1, const float* b2, float* y, int64_t n,
                       double scale, bool in_place_ok) {
  if (n < 0 || n > kMaxElems) return fail(MBP_ERR_SHAPE, "n must be in [0, 2^57) (got %lld)", (long long)n);
  if (n == 0) return MBP_OK;
  if (!x || !b1 || !b2 || !y) return fail(MBP_ERR_NULL, "x, b1, b2 and y must be non-NULL");
  if (misaligned(x, 4) || misaligned(b1, 4) || misaligned(b2, 4) || misaligned(y, 4))
    return fail(MBP_ERR_ALIGN, "fp32 pointers must be 4-byte aligned");
  if (!std::isfinite(scale)) return fail(MBP_ERR_ARG, "scale must be finite");
  const size_t B = (size_t)n * 4;
  const Span ys{y, B};
  for (const void* in : {(const void*)x, (const void*)b1, (const void*)b2})
    if (bad_overlap(ys, Span{in, B}, in_place_ok)) return fail(MBP_ERR_OVERLAP, "y overlaps an input");
  return MBP_OK;
}

mbp_status check_row_mean(const float* x, const float* bias, const float* gamma,
                          const float* beta, float* y, int64_t rows, int64_t cols, double alpha,
                          double c, bool in_place_ok) {
  mbp_status st = check_rows_cols(rows, cols);
  if (st != MBP_OK) return st;
  if (rows == 0) return MBP_OK;
  if (!x || !bias || !gamma || !beta || !y) return fail(MBP_ERR_NULL, "a required pointer is NULL");
  for (const void* p : {(const void*)x, (const void*)bias, (const void*)gamma, (const void*)beta, (const void*)y})
    if (misaligned(p, 4)) return fail(MBP_ERR_ALIGN, "fp32 pointers must be 4-byte aligned");
  if (!std::isfinite(alpha) || !std::isfinite(c)) return fail(MBP_ERR_ARG, "alpha and c must be finite");
  const size_t full = (size_t)rows * cols * 4, vec = (size_t)cols * 4;
  const Span ys{y, full};
  if (bad_overlap(ys, Span{x, full}, in_place_ok)) return fail(MBP_ERR_OVERLAP, "y overlaps x");
  for (const void* p : {(const void*)bias, (const void*)gamma, (const void*)beta})
    if (overlaps(ys, Span{p, vec})) return fail(MBP_ERR_OVERLAP, "y overlaps bias, gamma or beta");
  return MBP_OK;
}

mbp_status check_ln(mbp_dtype dtype, const void* x, const void* residual, const void* gamma,
                    const void* beta, void* y, int64_t rows, int64_t cols, double eps, mbp_act act,
                    bool in_place_ok) {
  if (dtype != MBP_F32 && dtype != MBP_BF16) return fail(MBP_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  if (act != MBP_ACT_NONE && act != MBP_ACT_GELU_TANH) return fail(MBP_ERR_DTYPE, "unknown act %d", (int)act);
  mbp_status st = check_rows_cols(rows, cols);
  if (st != MBP_OK) return st;
  if (rows == 0) return MBP_OK;
  if (!x || !gamma || !beta || !y) return fail(MBP_ERR_NULL, "x, gamma, beta and y must be non-NULL");
  const size_t es = dtype == MBP_BF16 ? 2 : 4;
  for (const void* p : {x, residual, gamma, beta, (const void*)y})
    if (misaligned(p, es)) return fail(MBP_ERR_ALIGN, "pointers must be aligned to the element size");
  if (!std::isfinite(eps) || eps < 0) return fail(MBP_ERR_ARG, "eps must be finite and >= 0");
  const size_t full = (size_t)rows * cols * es, vec = (size_t)cols * es;
  const Span ys{y, full};
  if (bad_overlap(ys, Span{x, full}, in_place_ok)) return fail(MBP_ERR_OVERLAP, "y overlaps x");
  if (residual && bad_overlap(ys, Span{residual, full}, in_place_ok))
    return fail(MBP_ERR_OVERLAP, "y overlaps residual");
  if (overlaps(ys, Span{gamma, vec}) || overlaps(ys, Span{beta, vec}))
    return fail(MBP_ERR_OVERLAP, "y overlaps gamma or beta");
  return MBP_OK;
}

size_t dtype_size(mbp_dtype d) { return d == MBP_F32 ? 4 : 2; }

// Bytes spanned by a [rows, cols] operand with row stride ld (0: one row).
size_t extent(int64_t rows, int64_t cols, int64_t ld, size_t es) {
  return es * (size_t)((rows - 1) * ld + cols);
}

// Shared checks of the *_2d entry points.  `ins` are the [rows, cols] inputs
// with their strides; the output may be exactly the input `inplace` (same
// pointer and stride), if given.
struct Operand2d {
  const void* p;
  int64_t ld;
};

mbp_status check_2d(mbp_dtype dtype, std::initializer_list<Operand2d> ins, void* y, int64_t ldy,
                    int64_t rows, int64_t cols, int64_t max_cols, const void* inplace) {
  if (dtype != MBP_F32 && dtype != MBP_BF16 && dtype != MBP_F16)
    return fail(MBP_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  if (rows < 0) return fail(MBP_ERR_SHAPE, "rows must be >= 0 (got %lld)", (long long)rows);
  if (cols <= 0 || cols > max_cols)
    return fail(MBP_ERR_SHAPE, "cols must be in [1, %lld] (got %lld)", (long long)max_cols, (long long)cols);
  if (rows == 0) return MBP_OK;
  const size_t es = dtype_size(dtype);
  if (!y) return fail(MBP_ERR_NULL, "y must be non-NULL");
  if (misaligned(y, es)) return fail(MBP_ERR_ALIGN, "pointers must be aligned to the element size");
  if (rows > 1 && ldy < cols) return fail(MBP_ERR_SHAPE, "ldy must be >= cols (got %lld)", (long long)ldy);
  if (ldy < 0) return fail(MBP_ERR_SHAPE, "ldy must be >= 0");
  const int64_t lim = kMaxElems / 2;
  if (rows > lim / (ldy > cols ? ldy : cols)) return fail(MBP_ERR_SHAPE, "rows * ldy overflows");
  const Span ys{y, extent(rows, cols, rows > 1 ? ldy : 0, es)};
  for (const Operand2d& in : ins) {
    if (!in.p) return fail(MBP_ERR_NULL, "a required pointer is NULL");
    if (misaligned(in.p, es)) return fail(MBP_ERR_ALIGN, "pointers must be aligned to the element size");
    if (in.ld != 0 && in.ld < cols)
      return fail(MBP_ERR_SHAPE, "an input stride must be 0 or >= cols (got %lld)", (long long)in.ld);
    if (in.ld < 0) return fail(MBP_ERR_SHAPE, "strides must be >= 0");
    if (in.ld > 0 && rows > lim / in.ld) return fail(MBP_ERR_SHAPE, "rows * ld overflows");
    const Span is{in.p, extent(rows, cols, in.ld, es)};
    const bool same = in.p == inplace && in.p == y && (in.ld == ldy || rows == 1);
    if (overlaps(ys, is) && !same) return fail(MBP_ERR_OVERLAP, "y overlaps an input");
  }
  return MBP_OK;
}

// Dropout description of drop probability p: threshold round(p * 2^16) on
// 16 random bits, scale 1 / (1 - p) (p == 1 drops everything).
mbp::Drop make_drop(double p, uint64_t seed, uint64_t offset) {
  mbp::Drop d;
  d.seed = seed;
  d.offset = offset;
  d.thr = (uint32_t)std::llround(p * 65536.0);
  d.scale = p >= 1.0 ? 0.0f : (float)(1.0 / (1.0 - p));
  return d;
}

mbp_status check_dropout_p(double p) {
  if (!(p >= 0.0 && p <= 1.0)) return fail(MBP_ERR_ARG, "p must be in [0, 1]");
  return MBP_OK;
}

// The 10-op graph as TVM's three groups, s and m in the buffers `w`.
hipError_t launch_grouped(const float* x, const float* bias, const float* gamma, const float* beta,
                          float* y, int64_t rows, int64_t cols, double alpha, double c,
                          const GroupedWs& w, hipStream_t s) {
  const float a32 = (float)alpha, c32 = (float)c;
  using namespace mbp;
  const int F = MBP_F32;
  // group 1: x*alpha + bias, relu, a*a, a*c, p + q  ->  s
  hipError_t e = launch_ew4(EW_PROLOGUE, F, x, bias, IX_COL, nullptr, 0, nullptr, 0, w.s, rows, cols,
                            a32, c32, s);
  // group 2: the row mean of s
  if (e == hipSuccess) e = launch_row_mean_only(F, w.s, w.m, rows, cols, s);
  // group 3: (s - m) * gamma + beta
  if (e == hipSuccess)
    e = launch_ew4(EW_CENTER_AFFINE, F, w.s, w.m, IX_ROW, gamma, IX_COL, beta, IX_COL, y, rows, cols,
                   0.0f, 0.0f, s);
  return e;
}

}  // namespace


// ---------------------------------------------------------------- C ABI

extern "C" {

mbp_status fused_pointwise_chain(const float* x, const float* b1, const float* b2, float* y,
                                 int64_t n, double scale, void* stream) {
  mbp_status st = check_chain(x, b1, b2, y, n, scale, true);
  if (st != MBP_OK) return st;
  if (n == 0) return ok();
  return from_hip(mbp::launch_chain(x, b1, b2, y, n, scale, as_stream(stream)), "fused_pointwise_chain");
}

mbp_status fused_row_mean_epilogue(const float* x, const float* bias, const float* gamma,
                                   const float* beta, float* y, int64_t rows, int64_t cols,
                                   double alpha, double c, void* stream) {
  mbp_status st = check_row_mean(x, bias, gamma, beta, y, rows, cols, alpha, c, true);
  if (st != MBP_OK) return st;
  if (rows == 0) return ok();
  return from_hip(mbp::launch_row_mean(x, bias, gamma, beta, y, rows, cols, alpha, c, as_stream(stream)),
                  "fused_row_mean_epilogue");
}

mbp_status fused_add_layernorm_gelu(mbp_dtype dtype, const void* x, const void* residual,
                                    const void* gamma, const void* beta, void* y, int64_t rows,
                                    int64_t cols, double eps, mbp_act act, void* stream) {
  mbp_status st = check_ln(dtype, x, residual, gamma, beta, y, rows, cols, eps, act, true);
  if (st != MBP_OK) return st;
  if (rows == 0) return ok();
  return from_hip(mbp::launch_layernorm(dtype, x, residual, gamma, beta, y, rows, cols, eps, act, nullptr,
                                        as_stream(stream)),
                  "fused_add_layernorm_gelu");
}

mbp_status fused_pointwise_chain_2d(mbp_dtype dtype, const void* x, int64_t ldx, const void* b1,
                                    int64_t ldb1, const void* b2, int64_t ldb2, void* y,
                                    int64_t ldy, int64_t rows, int64_t cols, double scale,
                                    void* stream) {
  if (!std::isfinite(scale)) return fail(MBP_ERR_ARG, "scale must be finite");
  // element-wise: y may be exactly any one of the inputs (the first that equals it)
  const void* inplace = y == x ? x : (y == b1 ? b1 : (y == b2 ? b2 : nullptr));
  mbp_status st = check_2d(dtype, {{x, ldx}, {b1, ldb1}, {b2, ldb2}}, y, ldy, rows, cols, kMaxElems, inplace);
  if (st != MBP_OK) return st;
  if (rows == 0) return ok();
  return from_hip(mbp::launch_chain_2d(dtype, x, ldx, b1, ldb1, b2, ldb2, y, ldy, rows, cols, scale,
                                       as_stream(stream)),
                  "fused_pointwise_chain_2d");
}

mbp_status fused_row_mean_epilogue_2d(mbp_dtype dtype, const void* x, int64_t ldx,
                                      const void* bias, const void* gamma, const void* beta,
                                      void* y, int64_t ldy, int64_t rows, int64_t cols,
                                      double alpha, double c, void* stream) {
  if (!std::isfinite(alpha) || !std::isfinite(c)) return fail(MBP_ERR_ARG, "alpha and c must be finite");
  // bias, gamma and beta are one row each (stride 0); y may be exactly x
  mbp_status st = check_2d(dtype, {{x, ldx}, {bias, 0}, {gamma, 0}, {beta, 0}}, y, ldy, rows, cols,
                           MBP_MAX_COLS, x);
  if (st != MBP_OK) return st;
  if (rows == 0) return ok();
  return from_hip(mbp::launch_row_mean_2d(dtype, x, ldx, bias, gamma, beta, y, ldy, rows, cols, alpha, c,
                                          as_stream(stream)),
                  "fused_row_mean_epilogue_2d");
}

mbp_status fused_softmax(mbp_dtype dtype, const void* x, void* y, int64_t rows, int64_t cols,
                         void* stream) {
  mbp_status st = check_2d(dtype, {{x, cols}}, y, cols, rows, cols, MBP_MAX_COLS, x);
  if (st != MBP_OK) return st;
  if (rows == 0) return ok();
  return from_hip(mbp::launch_softmax(dtype, x, cols, y, cols, rows, cols, as_stream(stream)), "fused_softmax");
}

mbp_status fused_softmax_2d(mbp_dtype dtype, const void* x, int64_t ldx, void* y, int64_t ldy,
                            int64_t rows, int64_t cols, void* stream) {
  mbp_status st = check_2d(dtype, {{x, ldx}}, y, ldy, rows, cols, MBP_MAX_COLS, x);
  if (st != MBP_OK) return st;
  if (rows == 0) return ok();
  return from_hip(mbp::launch_softmax(dtype, x, ldx, y, ldy, rows, cols, as_stream(stream)), "fused_softmax_2d");
}

mbp_status fused_add_layernorm_gelu_2d(mbp_dtype dtype, const void* x, int64_t ldx, const void* residual,
                                       int64_t ldr, const void* gamma, const void* beta, void* y,
                                       int64_t ldy, int64_t rows, int64_t cols, double eps, mbp_act act,
                                       void* stream) {
  if (dtype != MBP_F32 && dtype != MBP_BF16) return fail(MBP_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  if (act != MBP_ACT_NONE && act != MBP_ACT_GELU_TANH) return fail(MBP_ERR_DTYPE, "unknown act %d", (int)act);
  if (!std::isfinite(eps) || eps < 0) return fail(MBP_ERR_ARG, "eps must be finite and >= 0");
  // y may be exactly x or exactly the residual (same pointer, same stride)
  const void* inplace = y == x ? x : (residual && y == residual ? residual : nullptr);
  mbp_status st = residual ? check_2d(dtype, {{x, ldx}, {residual, ldr}, {gamma, 0}, {beta, 0}}, y, ldy, rows,
                                      cols, MBP_MAX_COLS, inplace)
                           : check_2d(dtype, {{x, ldx}, {gamma, 0}, {beta, 0}}, y, ldy, rows, cols,
                                      MBP_MAX_COLS, inplace);
  if (st != MBP_OK) return st;
  if (rows == 0) return ok();
  return from_hip(mbp::launch_layernorm_2d(dtype, x, ldx, residual, ldr, gamma, beta, y, ldy, rows, cols, eps,
                                           act, nullptr, as_stream(stream)),
                  "fused_add_layernorm_gelu_2d");
}

mbp_status fused_layernorm_relu_dropout_2d(mbp_dtype dtype, const void* x, int64_t ldx, const void* gamma,
                                           const void* beta, void* y, int64_t ldy, int64_t rows, int64_t cols,
                                           double eps, double p, uint64_t seed, uint64_t offset,
                                           void* stream) {
  if (dtype != MBP_F32 && dtype != MBP_BF16) return fail(MBP_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  if (!std::isfinite(eps) || eps < 0) return fail(MBP_ERR_ARG, "eps must be finite and >= 0");
  mbp_status st = check_dropout_p(p);
  if (st != MBP_OK) return st;
  st = check_2d(dtype, {{x, ldx}, {gamma, 0}, {beta, 0}}, y, ldy, rows, cols, MBP_MAX_COLS, x);
  if (st != MBP_OK) return st;
  if (rows == 0) return ok();
  const mbp::Drop d = make_drop(p, seed, offset);
  return from_hip(mbp::launch_layernorm_2d(dtype, x, ldx, nullptr, 0, gamma, beta, y, ldy, rows, cols, eps,
                                           mbp::kEpiReluDrop, &d, as_stream(stream)),
                  "fused_layernorm_relu_dropout_2d");
}

mbp_status fused_layernorm_relu_dropout(mbp_dtype dtype, const void* x, const void* gamma,
                                        const void* beta, void* y, int64_t rows, int64_t cols,
                                        double eps, double p, uint64_t seed, uint64_t offset,
                                        void* stream) {
  mbp_status st = check_ln(dtype, x, nullptr, gamma, beta, y, rows, cols, eps, MBP_ACT_NONE, true);
  if (st != MBP_OK) return st;
  st = check_dropout_p(p);
  if (st != MBP_OK) return st;
  if (rows == 0) return ok();
  const mbp::Drop d = make_drop(p, seed, offset);
  return from_hip(mbp::launch_layernorm(dtype, x, nullptr, gamma, beta, y, rows, cols, eps, mbp::kEpiReluDrop,
                                        &d, as_stream(stream)),
                  "fused_layernorm_relu_dropout");
}

mbp_status unfused_softmax(mbp_dtype dtype, const void* x, void* y, int64_t rows, int64_t cols,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != MBP_F32 && dtype != MBP_BF16) return fail(MBP_ERR_DTYPE, "unfused_softmax takes fp32 or bf16");
  mbp_status st = check_2d(dtype, {{x, cols}}, y, cols, rows, cols, MBP_MAX_COLS, nullptr);
  if (st != MBP_OK) return st;
  if (rows == 0) return ok();
  const size_t need = softmax_ws(nullptr, dtype, rows, cols, nullptr);
  const size_t full = (size_t)rows * cols * dtype_size(dtype);
  st = check_workspace(workspace, workspace_bytes, need, {{x, full}, {y, full}});
  if (st != MBP_OK) return st;
  SoftmaxWs w;
  softmax_ws((char*)workspace, dtype, rows, cols, &w);
  hipStream_t s = as_stream(stream);
  using namespace mbp;
  const int D = dtype;
  // the eager sequence: row max, x - m, exp, row sum, divide
  hipError_t e = launch_row_max(D, x, w.m, rows, cols, s);
  if (e == hipSuccess) e = launch_ew(EW_SUB, D, x, w.m, IX_ROW, nullptr, 0, w.d, rows, cols, 0.f, s);
  if (e == hipSuccess) e = launch_ew(EW_EXP, D, w.d, nullptr, 0, nullptr, 0, w.e, rows, cols, 0.f, s);
  if (e == hipSuccess) e = launch_row_sum(D, w.e, w.l, rows, cols, s);
  if (e == hipSuccess) e = launch_ew(EW_DIV, D, w.e, w.l, IX_ROW, nullptr, 0, y, rows, cols, 0.f, s);
  return from_hip(e, "unfused_softmax");
}

mbp_status unfused_layernorm_relu_dropout(mbp_dtype dtype, const void* x, const void* gamma,
                                          const void* beta, void* y, int64_t rows, int64_t cols,
                                          double eps, double p, uint64_t seed, uint64_t offset,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  mbp_status st = check_ln(dtype, x, nullptr, gamma, beta, y, rows, cols, eps, MBP_ACT_NONE, false);
  if (st != MBP_OK) return st;
  st = check_dropout_p(p);
  if (st != MBP_OK) return st;
  if (rows == 0) return ok();
  const size_t es = dtype == MBP_BF16 ? 2 : 4;
  const size_t full = (size_t)rows * cols * es, vec = (size_t)cols * es;
  Carver c{(char*)workspace};
  void* ln_out = c.take(full);
  void* relu_out = c.take(full);
  st = check_workspace(workspace, workspace_bytes, c.used, {{x, full}, {y, full}, {gamma, vec}, {beta, vec}});
  if (st != MBP_OK) return st;
  const mbp::Drop d = make_drop(p, seed, offset);
  hipStream_t s = as_stream(stream);
  using namespace mbp;
  // the three eager launches of [P2] section 2.1: layer_norm, relu, dropout
  hipError_t e = launch_layernorm(dtype, x, nullptr, gamma, beta, ln_out, rows, cols, eps, kEpiNone, nullptr, s);
  if (e == hipSuccess) e = launch_ew(EW_RELU, dtype, ln_out, nullptr, 0, nullptr, 0, relu_out, rows, cols, 0.f, s);
  if (e == hipSuccess)
    e = launch_ew(EW_DROPOUT, dtype, relu_out, nullptr, 0, nullptr, 0, y, rows, cols, 0.f, s, &d);
  return from_hip(e, "unfused_layernorm_relu_dropout");
}

mbp_status unfused_pointwise_chain(const float* x, const float* b1, const float* b2, float* y,
                                   int64_t n, double scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  mbp_status st = check_chain(x, b1, b2, y, n, scale, false);
  if (st != MBP_OK) return st;
  if (n == 0) return ok();
  const size_t need = chain_ws(nullptr, n, nullptr);
  const size_t B = (size_t)n * 4;
  st = check_workspace(workspace, workspace_bytes, need, {{x, B}, {b1, B}, {b2, B}, {y, B}});
  if (st != MBP_OK) return st;
  ChainWs w;
  chain_ws((char*)workspace, n, &w);
  const float s32 = (float)scale;
  hipStream_t s = as_stream(stream);
  using namespace mbp;
  hipError_t e = launch_ew(EW_ADD, MBP_F32, x, b1, IX_FULL, nullptr, 0, w.a, 1, n, 0.f, s);
  if (e == hipSuccess) e = launch_ew(EW_RELU, MBP_F32, w.a, nullptr, 0, nullptr, 0, w.b, 1, n, 0.f, s);
  if (e == hipSuccess) e = launch_ew(EW_MULS, MBP_F32, w.b, nullptr, 0, nullptr, 0, w.a, 1, n, s32, s);
  if (e == hipSuccess) e = launch_ew(EW_ADD, MBP_F32, w.a, b2, IX_FULL, nullptr, 0, y, 1, n, 0.f, s);
  return from_hip(e, "unfused_pointwise_chain");
}

mbp_status unfused_row_mean_epilogue(const float* x, const float* bias, const float* gamma,
                                     const float* beta, float* y, int64_t rows, int64_t cols,
                                     double alpha, double c, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  mbp_status st = check_row_mean(x, bias, gamma, beta, y, rows, cols, alpha, c, false);
  if (st != MBP_OK) return st;
  if (rows == 0) return ok();
  const size_t need = row_mean_ws(nullptr, rows, cols, nullptr);
  const size_t full = (size_t)rows * cols * 4, vec = (size_t)cols * 4;
  st = check_workspace(workspace, workspace_bytes, need,
                       {{x, full}, {y, full}, {bias, vec}, {gamma, vec}, {beta, vec}});
  if (st != MBP_OK) return st;
  RowMeanWs w;
  row_mean_ws((char*)workspace, rows, cols, &w);
  const float a32 = (float)alpha, c32 = (float)c;
  hipStream_t s = as_stream(stream);
  using namespace mbp;
  const int F = MBP_F32;
  hipError_t e = launch_ew(EW_MULS, F, x, nullptr, 0, nullptr, 0, w.a, rows, cols, a32, s);     // x*alpha
  if (e == hipSuccess) e = launch_ew(EW_ADD, F, w.a, bias, IX_COL, nullptr, 0, w.b, rows, cols, 0.f, s);  // t
  if (e == hipSuccess) e = launch_ew(EW_RELU, F, w.b, nullptr, 0, nullptr, 0, w.a, rows, cols, 0.f, s);  // a
  if (e == hipSuccess) e = launch_ew(EW_MUL, F, w.a, w.a, IX_FULL, nullptr, 0, w.b, rows, cols, 0.f, s);  // p
  if (e == hipSuccess) e = launch_ew(EW_MULS, F, w.a, nullptr, 0, nullptr, 0, w.c, rows, cols, c32, s);   // q
  if (e == hipSuccess) e = launch_ew(EW_ADD, F, w.b, w.c, IX_FULL, nullptr, 0, w.a, rows, cols, 0.f, s);  // s
  if (e == hipSuccess) e = launch_row_mean_only(F, w.a, w.m, rows, cols, s);                            // m
  if (e == hipSuccess) e = launch_ew(EW_SUB, F, w.a, w.m, IX_ROW, nullptr, 0, w.b, rows, cols, 0.f, s);  // s-m
  if (e == hipSuccess) e = launch_ew(EW_MUL, F, w.b, gamma, IX_COL, nullptr, 0, w.c, rows, cols, 0.f, s); // *g
  if (e == hipSuccess) e = launch_ew(EW_ADD, F, w.c, beta, IX_COL, nullptr, 0, y, rows, cols, 0.f, s);   // +b
  return from_hip(e, "unfused_row_mean_epilogue");
}

mbp_status grouped_row_mean_epilogue(const float* x, const float* bias, const float* gamma,
                                     const float* beta, float* y, int64_t rows, int64_t cols,
                                     double alpha, double c, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  mbp_status st = check_row_mean(x, bias, gamma, beta, y, rows, cols, alpha, c, false);
  if (st != MBP_OK) return st;
  if (rows == 0) return ok();
  const size_t need = grouped_ws(nullptr, rows, cols, nullptr);
  const size_t full = (size_t)rows * cols * 4, vec = (size_t)cols * 4;
  st = check_workspace(workspace, workspace_bytes, need,
                       {{x, full}, {y, full}, {bias, vec}, {gamma, vec}, {beta, vec}});
  if (st != MBP_OK) return st;
  GroupedWs w;
  grouped_ws((char*)workspace, rows, cols, &w);
  return from_hip(launch_grouped(x, bias, gamma, beta, y, rows, cols, alpha, c, w, as_stream(stream)),
                  "grouped_row_mean_epilogue");
}

mbp_status grouped_row_mean_epilogue_noalloc(const float* x, const float* bias, const float* gamma,
                                             const float* beta, float* y, int64_t rows, int64_t cols,
                                             double alpha, double c, void* stream) {
  mbp_status st = check_row_mean(x, bias, gamma, beta, y, rows, cols, alpha, c, false);
  if (st != MBP_OK) return st;
  if (rows == 0) return ok();
  const size_t need = grouped_ws(nullptr, rows, cols, nullptr);
  if (need > (size_t)MBP_STATIC_SCRATCH_BYTES)
    return fail(MBP_ERR_WORKSPACE,
                "%lld x %lld needs %zu bytes of scratch; the static scratch holds %zu (rows * cols "
                "must stay below about %zu elements)",
                (long long)rows, (long long)cols, need, (size_t)MBP_STATIC_SCRATCH_BYTES,
                (size_t)MBP_STATIC_SCRATCH_BYTES / 4);
  hipStream_t s = as_stream(stream);
  // the scratch looked up below is the current GPU's copy: the work must run there
  int cur = -1, sdev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess && s) e = hipStreamGetDevice(s, &sdev);
  if (e != hipSuccess) return from_hip(e, "grouped_row_mean_epilogue_noalloc");
  if (s && sdev != cur)
    return fail(MBP_ERR_ARG, "the stream belongs to device %d but device %d is current", sdev, cur);
  void* base = nullptr;
  size_t have = 0;
  e = mbp::static_scratch(&base, &have);
  if (e != hipSuccess) return from_hip(e, "grouped_row_mean_epilogue_noalloc: scratch lookup");
  if (have < need) return fail(MBP_ERR_WORKSPACE, "static scratch is smaller than %zu bytes", need);
  GroupedWs w;
  grouped_ws((char*)base, rows, cols, &w);
  return from_hip(launch_grouped(x, bias, gamma, beta, y, rows, cols, alpha, c, w, s),
                  "grouped_row_mean_epilogue_noalloc");
}

mbp_status unfused_add_layernorm_gelu(mbp_dtype dtype, const void* x, const void* residual,
                                      const void* gamma, const void* beta, void* y, int64_t rows,
                                      int64_t cols, double eps, mbp_act act, int granularity,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  mbp_status st = check_ln(dtype, x, residual, gamma, beta, y, rows, cols, eps, act, false);
  if (st != MBP_OK) return st;
  if (granularity != MBP_UNFUSED_PRIMITIVE && granularity != MBP_UNFUSED_EAGER)
    return fail(MBP_ERR_ARG, "unknown granularity %d", granularity);
  if (rows == 0) return ok();
  const bool res = residual != nullptr, gelu = act == MBP_ACT_GELU_TANH;
  const size_t need = ln_ws(nullptr, dtype, rows, cols, res, gelu, granularity, nullptr);
  const size_t es = dtype == MBP_BF16 ? 2 : 4;
  const size_t full = (size_t)rows * cols * es, vec = (size_t)cols * es;
  st = check_workspace(workspace, workspace_bytes, need,
                       {{x, full}, {residual, full}, {y, full}, {gamma, vec}, {beta, vec}});
  if (st != MBP_OK) return st;
  LnWs w;
  ln_ws((char*)workspace, dtype, rows, cols, res, gelu, granularity, &w);
  hipStream_t s = as_stream(stream);
  using namespace mbp;
  const int D = dtype;
  hipError_t e = hipSuccess;
  const void* src = x;
  if (res) {
    e = launch_ew(EW_ADD, D, x, residual, IX_FULL, nullptr, 0, w.r, rows, cols, 0.f, s);
    src = w.r;
  }
  void* ln_out = gelu ? w.a : y;
  if (granularity == MBP_UNFUSED_PRIMITIVE) {
    const float eps32 = (float)eps;
    if (e == hipSuccess) e = launch_row_mean_only(D, src, w.m, rows, cols, s);
    if (e == hipSuccess) e = launch_row_var(D, src, w.m, w.v, rows, cols, s);
    if (e == hipSuccess) e = launch_ew(EW_SUB, D, src, w.m, IX_ROW, nullptr, 0, w.a, rows, cols, 0.f, s);
    if (e == hipSuccess) e = launch_ew(EW_DIVSD, D, w.a, w.v, IX_ROW, nullptr, 0, w.b, rows, cols, eps32, s);
    if (e == hipSuccess)
      e = launch_ew(EW_MULADD, D, w.b, gamma, IX_COL, beta, IX_COL, ln_out, rows, cols, 0.f, s);
  } else {
    if (e == hipSuccess)
      e = launch_layernorm(D, src, nullptr, gamma, beta, ln_out, rows, cols, eps, MBP_ACT_NONE, nullptr, s);
  }
  if (gelu && e == hipSuccess)
    e = launch_ew(EW_GELU, D, w.a, nullptr, 0, nullptr, 0, y, rows, cols, 0.f, s);
  return from_hip(e, "unfused_add_layernorm_gelu");
}

// ---------------------------------------------------------------- graphs

struct mbp_graph_s {
  hipGraphExec_t exec;
  size_t nodes;
};

mbp_status mbp_graph_capture_begin(void* stream) {
  if (!stream) return fail(MBP_ERR_ARG, "capture needs a created stream, not the NULL stream");
  return from_hip(hipStreamBeginCapture(as_stream(stream), hipStreamCaptureModeThreadLocal),
                  "hipStreamBeginCapture");
}

mbp_status mbp_graph_capture_end(void* stream, mbp_graph** graph) {
  if (!graph) return fail(MBP_ERR_NULL, "graph must be non-NULL");
  *graph = nullptr;
  if (!stream) return fail(MBP_ERR_ARG, "capture needs a created stream, not the NULL stream");
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(as_stream(stream), &g);
  if (e != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return from_hip(e, "hipStreamEndCapture");
  }
  size_t nodes = 0;
  e = hipGraphGetNodes(g, nullptr, &nodes);
  if (e != hipSuccess || nodes == 0) {
    (void)hipGraphDestroy(g);
    return e != hipSuccess ? from_hip(e, "hipGraphGetNodes") : fail(MBP_ERR_ARG, "nothing was captured");
  }
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);  // the executable graph does not need its template
  if (e != hipSuccess) return from_hip(e, "hipGraphInstantiate");
  mbp_graph* h = new (std::nothrow) mbp_graph{exec, nodes};
  if (!h) {
    (void)hipGraphExecDestroy(exec);
    return fail(MBP_ERR_ARG, "out of host memory");
  }
  *graph = h;
  return ok();
}

mbp_status mbp_graph_launch(const mbp_graph* graph, void* stream) {
  if (!graph) return fail(MBP_ERR_NULL, "graph must be non-NULL");
  return from_hip(hipGraphLaunch(graph->exec, as_stream(stream)), "hipGraphLaunch");
}

int64_t mbp_graph_nodes(const mbp_graph* graph) { return graph ? (int64_t)graph->nodes : -1; }

mbp_status mbp_graph_destroy(mbp_graph* graph) {
  if (!graph) return ok();
  const hipError_t e = hipGraphExecDestroy(graph->exec);
  delete graph;
  return from_hip(e, "hipGraphExecDestroy");
}

size_t mbp_unfused_workspace_bytes(mbp_op op, mbp_dtype dtype, int64_t rows, int64_t cols,
                                   int has_residual, mbp_act act, int granularity) {
  if (rows < 0 || cols < 0) return (size_t)-1;
  if (rows == 0 || cols == 0) return 0;
  if (rows > kMaxElems / cols) return (size_t)-1;
  switch (op) {
    case MBP_OP_CHAIN: return chain_ws(nullptr, rows * cols, nullptr);
    case MBP_OP_ROW_MEAN:
      if (granularity == MBP_UNFUSED_GROUPED) return grouped_ws(nullptr, rows, cols, nullptr);
      return row_mean_ws(nullptr, rows, cols, nullptr);
    case MBP_OP_SOFTMAX:
      if (dtype != MBP_F32 && dtype != MBP_BF16) return (size_t)-1;
      return softmax_ws(nullptr, dtype, rows, cols, nullptr);
    case MBP_OP_LN_RELU_DROPOUT: {
      if (dtype != MBP_F32 && dtype != MBP_BF16) return (size_t)-1;
      Carver c{nullptr};
      c.take((size_t)rows * cols * (dtype == MBP_BF16 ? 2 : 4));
      c.take((size_t)rows * cols * (dtype == MBP_BF16 ? 2 : 4));
      return c.used;
    }
    case MBP_OP_LAYERNORM:
      if (dtype != MBP_F32 && dtype != MBP_BF16) return (size_t)-1;
      if (granularity != MBP_UNFUSED_PRIMITIVE && granularity != MBP_UNFUSED_EAGER) return (size_t)-1;
      return ln_ws(nullptr, dtype, rows, cols, has_residual != 0, act == MBP_ACT_GELU_TANH,
                   granularity, nullptr);
    default: return (size_t)-1;
  }
}

int mbp_launches_per_call(mbp_op op, int fused, int granularity, int has_residual, mbp_act act) {
  if (fused) return (op >= MBP_OP_CHAIN && op <= MBP_OP_SOFTMAX) ? 1 : -1;
  switch (op) {
    case MBP_OP_SOFTMAX: return 5;
    case MBP_OP_LN_RELU_DROPOUT: return 3;
    case MBP_OP_CHAIN: return 4;
    case MBP_OP_ROW_MEAN: return granularity == MBP_UNFUSED_GROUPED ? 3 : 10;
    case MBP_OP_LAYERNORM: {
      const int extra = (has_residual ? 1 : 0) + (act == MBP_ACT_GELU_TANH ? 1 : 0);
      if (granularity == MBP_UNFUSED_PRIMITIVE) return 5 + extra;
      if (granularity == MBP_UNFUSED_EAGER) return 1 + extra;
      return -1;
    }
    default: return -1;
  }
}

mbp_status mbp_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return ok();
  if (!src || !dst) return fail(MBP_ERR_NULL, "src and dst must be non-NULL");
  if (misaligned(src, 16) || misaligned(dst, 16) || bytes % 16)
    return fail(MBP_ERR_ALIGN, "src, dst and bytes must be multiples of 16");
  if (overlaps(Span{src, bytes}, Span{dst, bytes})) return fail(MBP_ERR_OVERLAP, "src and dst overlap");
  return from_hip(mbp::launch_copy(src, dst, bytes, as_stream(stream)), "mbp_stream_copy");
}

mbp_status mbp_stream_rw(const void* const* srcs, int nsrc, void* dst, size_t bytes, void* stream) {
  if (nsrc < 1 || nsrc > 4) return fail(MBP_ERR_ARG, "nsrc must be 1 .. 4 (got %d)", nsrc);
  if (bytes == 0) return ok();
  if (!srcs || !dst) return fail(MBP_ERR_NULL, "srcs and dst must be non-NULL");
  if (misaligned(dst, 16) || bytes % 16) return fail(MBP_ERR_ALIGN, "dst and bytes must be multiples of 16");
  for (int k = 0; k < nsrc; ++k) {
    if (!srcs[k]) return fail(MBP_ERR_NULL, "srcs[%d] is NULL", k);
    if (misaligned(srcs[k], 16)) return fail(MBP_ERR_ALIGN, "srcs[%d] must be 16-byte aligned", k);
    if (overlaps(Span{srcs[k], bytes}, Span{dst, bytes})) return fail(MBP_ERR_OVERLAP, "dst overlaps srcs[%d]", k);
  }
  return from_hip(mbp::launch_stream(srcs, nsrc, dst, bytes, as_stream(stream)), "mbp_stream_rw");
}

mbp_status mbp_convert_f32_to_bf16(const float* x, uint16_t* y, int64_t n, void* stream) {
  if (n < 0) return fail(MBP_ERR_SHAPE, "n must be >= 0 (got %lld)", (long long)n);
  if (n == 0) return ok();
  if (n > kMaxElems) return fail(MBP_ERR_SHAPE, "n is too large");
  if (!x || !y) return fail(MBP_ERR_NULL, "x and y must be non-NULL");
  if (misaligned(x, 4) || misaligned(y, 2)) return fail(MBP_ERR_ALIGN, "x must be 4-byte and y 2-byte aligned");
  if (overlaps(Span{x, (size_t)n * 4}, Span{y, (size_t)n * 2})) return fail(MBP_ERR_OVERLAP, "y overlaps x");
  return from_hip(mbp::launch_to_bf16(x, y, n, as_stream(stream)), "mbp_convert_f32_to_bf16");
}

const char* mbp_status_string(mbp_status s) {
  switch (s) {
    case MBP_OK: return "ok";
    case MBP_ERR_NULL: return "a required pointer is NULL";
    case MBP_ERR_SHAPE: return "invalid shape";
    case MBP_ERR_DTYPE: return "unknown dtype or activation";
    case MBP_ERR_ALIGN: return "misaligned pointer";
    case MBP_ERR_OVERLAP: return "output overlaps an input";
    case MBP_ERR_WORKSPACE: return "invalid workspace";
    case MBP_ERR_HIP: return "HIP runtime error";
    case MBP_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

const char* mbp_last_error(void) { return g_last_error.c_str(); }

int mbp_abi_version(void) { return MBP_ABI_VERSION; }

}  // extern "C"
