/*
 * oracle.c -- the plain, slow CPU reference for the fused memory-bound chains.
 *
 * TEST INFRASTRUCTURE ONLY.  The product path (the HIP library libmbp.so and its
 * Python binding) never includes, links, imports or calls anything in oracle/.
 * Only the tests, the smoke check and the bench's cpu_baseline leg use it.  It
 * shares no header, helper, table or constant with the HIP sources.
 *
 * Form.  Every function runs the UNFUSED op sequence literally: one loop per op,
 * in the order the pages write the ops, with every intermediate materialised as
 * a full array.  Inputs are the stored binary32 / bfloat16 values widened
 * exactly to binary64.  Built with -O2 -fno-fast-math -ffp-contract=off, so no
 * multiply-add is contracted and nothing is reassociated.
 *
 * Modes.
 *   ORACLE_EXACT (0): every intermediate is binary64; constants are the decimal
 *     literals parsed to binary64.  This is the reference the fused kernels are
 *     gated against.
 *   ORACLE_SEQ (1): emulates one-op-per-launch execution.  After each op the
 *     value is rounded to the unfused variant's storage type (binary32 for the
 *     fp32 chains; bfloat16 for bf16 I/O, reached as binary32 then bfloat16,
 *     because such a kernel computes in fp32 and stores bf16).  Row statistics
 *     are stored as binary32.  Constants are rounded to binary32 first, as an
 *     fp32 kernel multiplying by a Python float does.  For + - * / sqrt on
 *     binary32 operands, computing in binary64 and rounding once to binary32 is
 *     the correctly rounded binary32 result (53 >= 2*24 + 2; S. A. Figueroa,
 *     "When is double rounding innocuous?", SIGNUM Newsletter 1995), so SEQ is
 *     bit-exact for element-wise ops.  Reductions depend on summation order;
 *     SEQ sums in binary64, so for them it is a tolerance reference only.
 *   ORACLE_SEQ3 (2): residual add + LayerNorm + GeLU as three eager launches
 *     (add, a LayerNorm kernel, gelu), each stored in the I/O type.
 *
 * All outputs are written as binary64 (the stored value, widened, in SEQ modes).
 * Return value: 0 on success, negative on a bad argument or allocation failure.
 *
 * Storage formats.  oracle_round_to_f16 / oracle_round_to_bf16 round binary64
 * values once, to nearest even, to binary16 / bfloat16 bit patterns: the
 * expected stored result of a kernel that computes in binary64 and stores a
 * 16-bit type (binary16 and bfloat16 inputs widen exactly to binary32, so the
 * chain and the 10-op graph take them through their binary32 interfaces).
 *
 * Sources (the four pages on operator fusion):
 *   [P1] PyTorch operator-fusion practice post, 0539edu.com/news/5489619
 *        section 1.1 (the add/relu/mul/add step table), section 3.1 (baseline
 *        chain, randn inputs, scale 0.5).
 *   [P2] "算子融合与 Kernel 优化：从 CUDA Graph 到 FlashAttention 的极致性能"
 *        (plumephp.com), section 2.3 (residual + LayerNorm + GeLU kernel).
 *   [P3] "4、算子融合（Kernel Fusion）" (5688vip.com course chapter), section 4.3
 *        (LayerNorm definition and its five unfused kernels).
 *   [P4] "TorchInductor Pipeline 与算子融合" (blog.kkkzoz.top), the 10-op model at
 *        the top of the post, section 6.4 (mean = row sum, then divide), section
 *        02 Table 2 (the ten eager kernels).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_EXACT = 0, ORACLE_SEQ = 1, ORACLE_SEQ3 = 2 };
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };
enum { ORACLE_ACT_NONE = 0, ORACLE_ACT_GELU_TANH = 1 };

/* ---- storage formats ------------------------------------------------------ */

/* bfloat16 is the upper half of a binary32 bit pattern. */
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* binary32 -> bfloat16, round to nearest even on the dropped 16 bits; a NaN
 * stays a (quiet) NaN. */
static uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* round a binary64 value to binary32 (x86-64 SSE conversion, round-to-nearest-even) */
static double r32(double v) { return (double)(float)v; }

/* round to bfloat16 the way a kernel that computes in fp32 and stores bf16 does */
static double rbf16(double v) { return bf16_bits_to_double(float_to_bf16_rne((float)v)); }

/* round to the storage type of the I/O (SEQ modes) */
static double rstore(int dtype, double v) { return dtype == ORACLE_BF16 ? rbf16(v) : r32(v); }

static double load_elem(int dtype, const void* p, int64_t i) {
  if (dtype == ORACLE_BF16) return bf16_bits_to_double(((const uint16_t*)p)[i]);
  return (double)((const float*)p)[i];
}

static double* alloc_d(int64_t n) { return (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double)); }

/* ---- tanh-approximated GeLU ----------------------------------------------
 * [P2] section 2.3: g(u) = 0.5 u (1 + tanh(0.7978845608 (u + 0.044715 u^3))),
 * constants exactly as the page writes them. */
static double gelu_tanh(double u) {
  double u3 = u * u * u;
  double inner = u + 0.044715 * u3;
  double z = 0.7978845608 * inner;
  return 0.5 * u * (1.0 + tanh(z));
}

void oracle_gelu_tanh(const double* u, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = gelu_tanh(u[i]);
}

/* bfloat16 encode/decode, exported so that the tests can pin them against an
 * independent library conversion. */
void oracle_to_bf16(const float* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = float_to_bf16_rne(in[i]);
}

/* ---- binary64 -> a narrower binary format, one rounding -------------------
 * IEEE 754 binary formats with p significand bits (the leading one counted),
 * smallest normal exponent emin and largest exponent emax: binary16 (p = 11,
 * emin = -14, emax = 15) and bfloat16 (p = 8, emin = -126, emax = 127).  Round
 * to nearest, ties to even, directly from the binary64 value: scale by a power
 * of two so that the last significand bit of the result has weight 1 (below
 * the normal range that weight is fixed at 2^(emin - p + 1)), round to an
 * integer with rint() (ties to even in the default rounding mode), scale back.
 * Both scalings are exact.  A result above the largest finite value becomes
 * infinity; zeros, infinities and NaN pass through. */
static double round_binary(double v, int p, int emin, int emax) {
  if (v != v || v == 0.0 || isinf(v)) return v;
  double a = fabs(v);
  int e;
  frexp(a, &e); /* a = f * 2^e with f in [0.5, 1): the leading bit has weight 2^(e - 1) */
  int lead = e - 1;
  if (lead < emin) lead = emin;
  int q = lead - (p - 1); /* weight of the last significand bit: 2^q */
  double r = ldexp(rint(ldexp(a, -q)), q);
  double maxf = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
  if (r > maxf) r = INFINITY;
  return v < 0 ? -r : r;
}

/* bit pattern of a value representable in binary16 */
static uint16_t encode_binary16(double r) {
  uint16_t s = signbit(r) ? 0x8000u : 0u;
  if (r != r) return 0x7e00u;
  double a = fabs(r);
  if (isinf(a)) return (uint16_t)(s | 0x7c00u);
  if (a < ldexp(1.0, -14)) return (uint16_t)(s | (uint16_t)ldexp(a, 24)); /* zero or subnormal */
  int e;
  double f = frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  uint16_t frac = (uint16_t)(ldexp(f, 11) - 1024.0);
  return (uint16_t)(s | (uint16_t)((e - 1 + 15) << 10) | frac);
}

/* bit pattern of a value representable in bfloat16: the upper half of its
 * (exact) binary32 pattern */
static uint16_t encode_bfloat16(double r) {
  if (r != r) return 0x7fc0u;
  float f = (float)r;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

void oracle_round_to_f16(const double* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = encode_binary16(round_binary(in[i], 11, -14, 15));
}

void oracle_round_to_bf16(const double* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = encode_bfloat16(round_binary(in[i], 8, -126, 127));
}

/* ---- (a) pointwise chain --------------------------------------------------
 * [P1] section 1.1 and 3.1: y = relu(x + b1) * scale + b2, run as four eager
 * ops: t = x + b1; r = relu(t); u = r * scale; y = u + b2.  b1 and b2 are full
 * tensors of x's shape (randn_like).  relu keeps NaN (eager semantics: t < 0
 * selects 0, everything else passes through). */
int oracle_pointwise_chain(const float* x, const float* b1, const float* b2, int64_t n,
                           double scale, int mode, double* y) {
  if (n < 0) return -1;
  if (mode != ORACLE_EXACT && mode != ORACLE_SEQ) return -2;
  if (n == 0) return 0;
  if (!x || !b1 || !b2 || !y) return -1;
  const int seq = (mode == ORACLE_SEQ);
  const double s = seq ? r32(scale) : scale;
  double* t = alloc_d(n);
  double* r = alloc_d(n);
  double* u = alloc_d(n);
  if (!t || !r || !u) { free(t); free(r); free(u); return -3; }

  for (int64_t i = 0; i < n; ++i) {           /* op 1: add */
    t[i] = (double)x[i] + (double)b1[i];
    if (seq) t[i] = r32(t[i]);
  }
  for (int64_t i = 0; i < n; ++i)             /* op 2: relu */
    r[i] = (t[i] < 0.0) ? 0.0 : t[i];
  for (int64_t i = 0; i < n; ++i) {           /* op 3: mul by the scalar */
    u[i] = r[i] * s;
    if (seq) u[i] = r32(u[i]);
  }
  for (int64_t i = 0; i < n; ++i) {           /* op 4: add */
    y[i] = u[i] + (double)b2[i];
    if (seq) y[i] = r32(y[i]);
  }
  free(t); free(r); free(u);
  return 0;
}

/* ---- (b1) the 10-op graph: prologue, row mean, epilogue --------------------
 * [P4] the model at the top of the post, x [rows, cols], bias/gamma/beta [cols]
 * broadcast over rows (section 1.1: stride 0 along the row dimension):
 *   t = x * alpha + bias        (two ops: mul, add)        alpha = 1.1
 *   a = relu(t)
 *   p = a * a ; q = a * c ; s = p + q                      c = 0.1
 *   m = s.mean(dim=1)           (section 6.4: a row SUM, then divide by cols)
 *   y = (s - m) * gamma + beta  (three ops: sub, mul, add)
 * Ten eager kernels in all (section 02, Table 2). */
int oracle_row_mean_epilogue(const float* x, const float* bias, const float* gamma,
                             const float* beta, int64_t rows, int64_t cols, double alpha,
                             double c, int mode, double* y) {
  if (rows < 0 || cols <= 0) return -1;
  if (mode != ORACLE_EXACT && mode != ORACLE_SEQ) return -2;
  if (rows == 0) return 0;
  if (!x || !bias || !gamma || !beta || !y) return -1;
  const int seq = (mode == ORACLE_SEQ);
  const double al = seq ? r32(alpha) : alpha;
  const double cc = seq ? r32(c) : c;
  const int64_t n = rows * cols;
  double* t1 = alloc_d(n);
  double* t = alloc_d(n);
  double* a = alloc_d(n);
  double* p = alloc_d(n);
  double* q = alloc_d(n);
  double* s = alloc_d(n);
  double* m = alloc_d(rows);
  double* d = alloc_d(n);
  double* e = alloc_d(n);
  int rc = 0;
  if (!t1 || !t || !a || !p || !q || !s || !m || !d || !e) { rc = -3; goto done; }
#define RS(v) (seq ? r32(v) : (v))
  for (int64_t i = 0; i < rows; ++i)          /* op 1: mul by alpha */
    for (int64_t j = 0; j < cols; ++j) t1[i * cols + j] = RS((double)x[i * cols + j] * al);
  for (int64_t i = 0; i < rows; ++i)          /* op 2: add bias[j] */
    for (int64_t j = 0; j < cols; ++j) t[i * cols + j] = RS(t1[i * cols + j] + (double)bias[j]);
  for (int64_t k = 0; k < n; ++k)             /* op 3: relu */
    a[k] = (t[k] < 0.0) ? 0.0 : t[k];
  for (int64_t k = 0; k < n; ++k)             /* op 4: a * a */
    p[k] = RS(a[k] * a[k]);
  for (int64_t k = 0; k < n; ++k)             /* op 5: a * c */
    q[k] = RS(a[k] * cc);
  for (int64_t k = 0; k < n; ++k)             /* op 6: p + q */
    s[k] = RS(p[k] + q[k]);
  for (int64_t i = 0; i < rows; ++i) {        /* op 7: row mean = row sum / cols */
    double acc = 0.0;
    for (int64_t j = 0; j < cols; ++j) acc += s[i * cols + j];
    m[i] = RS(acc / (double)cols);
  }
  for (int64_t i = 0; i < rows; ++i)          /* op 8: s - m (m broadcast over the row) */
    for (int64_t j = 0; j < cols; ++j) d[i * cols + j] = RS(s[i * cols + j] - m[i]);
  for (int64_t i = 0; i < rows; ++i)          /* op 9: * gamma[j] */
    for (int64_t j = 0; j < cols; ++j) e[i * cols + j] = RS(d[i * cols + j] * (double)gamma[j]);
  for (int64_t i = 0; i < rows; ++i)          /* op 10: + beta[j] */
    for (int64_t j = 0; j < cols; ++j) y[i * cols + j] = RS(e[i * cols + j] + (double)beta[j]);
#undef RS
done:
  free(t1); free(t); free(a); free(p); free(q); free(s); free(m); free(d); free(e);
  return rc;
}

/* ---- (b2) residual add + LayerNorm + tanh-GeLU -----------------------------
 * [P3] section 4.3: mean = mean(x); var = var(x); y = (x - mean)/sqrt(var + eps)
 * * gamma + beta, as five unfused kernels (mean, var, subtract, divide,
 * multiply-add).  The variance is the biased one (divide by cols), computed
 * about the finished mean (the chapter's second pass).  [P2] section 2.3 puts a
 * residual add in front (v = x + residual) and the tanh-GeLU behind:
 * out = gelu(LN(x + residual) * gamma + beta).  residual == NULL skips the add;
 * act == ORACLE_ACT_NONE skips the GeLU (plain LayerNorm).
 * dtype ORACLE_F32: x, residual, gamma, beta are binary32; ORACLE_BF16: all four
 * are bfloat16 bit patterns (uint16). */
int oracle_add_layernorm_gelu(int dtype, const void* x, const void* residual, const void* gamma,
                              const void* beta, int64_t rows, int64_t cols, double eps, int act,
                              int mode, double* y) {
  if (rows < 0 || cols <= 0) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -2;
  if (act != ORACLE_ACT_NONE && act != ORACLE_ACT_GELU_TANH) return -2;
  if (mode != ORACLE_EXACT && mode != ORACLE_SEQ && mode != ORACLE_SEQ3) return -2;
  if (rows == 0) return 0;
  if (!x || !gamma || !beta || !y) return -1;
  const int seq = (mode == ORACLE_SEQ);
  const int seq3 = (mode == ORACLE_SEQ3);
  const int64_t n = rows * cols;
  double* v = alloc_d(n);
  double* mean = alloc_d(rows);
  double* var = alloc_d(rows);
  double* cen = alloc_d(n);
  double* nrm = alloc_d(n);
  double* u = alloc_d(n);
  if (!v || !mean || !var || !cen || !nrm || !u) {
    free(v); free(mean); free(var); free(cen); free(nrm); free(u);
    return -3;
  }
  const double eps_used = seq ? r32(eps) : eps;

  /* op 0 (only with a residual): v = x + residual */
  for (int64_t k = 0; k < n; ++k) {
    double xv = load_elem(dtype, x, k);
    if (residual) {
      xv = xv + load_elem(dtype, residual, k);
      if (seq || seq3) xv = rstore(dtype, xv);
    }
    v[k] = xv;
  }
  /* op 1: mean over the row */
  for (int64_t i = 0; i < rows; ++i) {
    double acc = 0.0;
    for (int64_t j = 0; j < cols; ++j) acc += v[i * cols + j];
    mean[i] = acc / (double)cols;
    if (seq) mean[i] = r32(mean[i]);
  }
  /* op 2: biased variance about that mean */
  for (int64_t i = 0; i < rows; ++i) {
    double acc = 0.0;
    for (int64_t j = 0; j < cols; ++j) {
      double dlt = v[i * cols + j] - mean[i];
      acc += dlt * dlt;
    }
    var[i] = acc / (double)cols;
    if (seq) var[i] = r32(var[i]);
  }
  /* op 3: subtract the mean */
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t j = 0; j < cols; ++j) {
      double cv = v[i * cols + j] - mean[i];
      cen[i * cols + j] = seq ? rstore(dtype, cv) : cv;
    }
  /* op 4: divide by sqrt(var + eps) (eps inside the root) */
  for (int64_t i = 0; i < rows; ++i) {
    double sd = seq ? r32(sqrt(r32(var[i] + eps_used))) : sqrt(var[i] + eps_used);
    for (int64_t j = 0; j < cols; ++j) {
      double nv = cen[i * cols + j] / sd;
      nrm[i * cols + j] = seq ? rstore(dtype, nv) : nv;
    }
  }
  /* op 5: multiply-add with gamma[j], beta[j] */
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t j = 0; j < cols; ++j) {
      double g = load_elem(dtype, gamma, j), b = load_elem(dtype, beta, j);
      double uv;
      if (seq) uv = rstore(dtype, r32(r32(nrm[i * cols + j] * g) + b));
      else uv = nrm[i * cols + j] * g + b;
      if (seq3) uv = rstore(dtype, uv);
      u[i * cols + j] = uv;
    }
  /* op 6 (only with act): tanh-GeLU */
  for (int64_t k = 0; k < n; ++k) {
    double o = u[k];
    if (act == ORACLE_ACT_GELU_TANH) {
      o = gelu_tanh(o);
      if (seq || seq3) o = rstore(dtype, o);
    }
    y[k] = o;
  }
  free(v); free(mean); free(var); free(cen); free(nrm); free(u);
  return 0;
}

/* ---- row softmax ------------------------------------------------------------
 * [P1] section 4.2 and [P2] section 3.2 (step 3): softmax over the last
 * dimension, normalised relative to the row maximum so that no exponential
 * overflows:
 *   m_i = max_j x_ij;   e_ij = exp(x_ij - m_i);   l_i = sum_j e_ij;   y_ij = e_ij / l_i.
 * The ops run in that order, each intermediate materialised, in binary64 on
 * the stored values (widened exactly; 16-bit inputs arrive as binary32).  The
 * pages' running-max update (a new maximum rescales the partial sum by
 * exp(m_old - m_new)) reaches the same values in exact arithmetic; this is
 * the plain definition.  A NaN anywhere in a row makes its sum NaN, so the row
 * is NaN; a row of -inf only is 0/0 = NaN (both as torch.softmax).
 * ORACLE_SEQ: the same four ops as eager one-op kernels evaluate them ([P3]
 * section 4.2 names softmax as the reduce + element-wise pattern that fusion
 * targets): the difference x - m, the exponential and the quotient are each
 * rounded as such a kernel stores its result -- to binary32, then to the I/O
 * type (dtype ORACLE_BF16: bfloat16, nearest even) -- and the row sum is
 * accumulated in binary64 and stored as binary32.  ORACLE_EXACT ignores
 * dtype. */
int oracle_softmax_mode(int dtype, const float* x, int64_t rows, int64_t cols, int mode, double* y) {
  if (mode != ORACLE_EXACT && mode != ORACLE_SEQ) return -2;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -3;
  if (rows < 0 || (rows > 0 && cols <= 0)) return -1;
  if (rows == 0) return 0;
  const int seq = mode == ORACLE_SEQ;
  const int64_t n = rows * cols;
  double* m = alloc_d(rows);
  double* e = alloc_d(n);
  double* l = alloc_d(rows);
  if (!m || !e || !l) { free(m); free(e); free(l); return -2; }
  /* op 1: row maximum (NaN is skipped here and propagates through op 3) */
  for (int64_t i = 0; i < rows; ++i) {
    double mi = -INFINITY;
    for (int64_t j = 0; j < cols; ++j) {
      double v = (double)x[i * cols + j];
      if (v > mi) mi = v;
    }
    m[i] = mi;
  }
  /* op 2: shifted exponentials (SEQ: the difference and the exponential are
   * two eager ops, each result stored in the I/O type) */
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t j = 0; j < cols; ++j) {
      double d = (double)x[i * cols + j] - m[i];
      if (seq) d = rstore(dtype, d);
      const double ev = exp(d);
      e[i * cols + j] = seq ? rstore(dtype, ev) : ev;
    }
  /* op 3: row sum (SEQ: accumulated in binary64, stored as binary32) */
  for (int64_t i = 0; i < rows; ++i) {
    double acc = 0.0;
    for (int64_t j = 0; j < cols; ++j) acc += e[i * cols + j];
    l[i] = seq ? r32(acc) : acc;
  }
  /* op 4: divide */
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t j = 0; j < cols; ++j) {
      const double q = e[i * cols + j] / l[i];
      y[i * cols + j] = seq ? rstore(dtype, q) : q;
    }
  free(m); free(e); free(l);
  return 0;
}

int oracle_softmax(const float* x, int64_t rows, int64_t cols, double* y) {
  return oracle_softmax_mode(ORACLE_F32, x, rows, cols, ORACLE_EXACT, y);
}

/* ---- counter-based random numbers: Philox4x32-10 ---------------------------
 * J. K. Salmon, M. A. Moraes, R. O. Dror and D. E. Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3" (SC'11), the Philox-4x32 generator with 10
 * rounds: a 128-bit counter (c0..c3) and a 64-bit key (k0, k1).  One round
 * multiplies c0 and c2 by the constants 0xD2511F53 and 0xCD9E8D57 into 64-bit
 * products (hi, lo) and forms the new counter
 *   (hi(c2 * M1) ^ c1 ^ k0,  lo(c2 * M1),  hi(c0 * M0) ^ c3 ^ k1,  lo(c0 * M0));
 * between rounds the key is bumped by the Weyl constants 0x9E3779B9 and
 * 0xBB67AE85.  The output of 10 rounds is four 32-bit words. */
static void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    uint32_t n1 = (uint32_t)p1;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    uint32_t n3 = (uint32_t)p0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
  }
  out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

/* exported for the known-answer pins: n blocks, counters and keys interleaved
 * (ctr: 4 words per block, key: 2 words per block) */
void oracle_philox4x32_10(const uint32_t* ctr, const uint32_t* key, int64_t n, uint32_t* out) {
  for (int64_t i = 0; i < n; ++i) philox4x32_10(ctr + 4 * i, key + 2 * i, out + 4 * i);
}

/* The 16 random bits of element i of a call with (seed, offset): half i mod 8
 * of Philox4x32-10 with key = (seed low, seed high) and counter =
 * (q low, q high, offset low, offset high), q = i div 8 -- word (i mod 8) div 2,
 * its low half for even i, its high half for odd i. */
static uint32_t dropout_bits(uint64_t seed, uint64_t offset, uint64_t i) {
  const uint64_t q = i >> 3;
  const uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  philox4x32_10(ctr, key, out);
  const uint32_t w = out[(i & 7) >> 1];
  return (i & 1) ? (w >> 16) : (w & 0xFFFFu);
}

/* ---- LayerNorm -> ReLU -> Dropout ------------------------------------------
 * [P2] section 2.1: y = dropout(relu(layer_norm(x, weight, bias)), p), three
 * element-wise stages after the row statistics, fused there into one kernel.
 * Ops in order:
 *   u = LayerNorm(x) * gamma + beta      (biased variance, eps inside the root,
 *                                          as oracle_add_layernorm_gelu)
 *   r = max(u, 0)                         (relu; NaN passes through)
 *   y = keep_i ? r * scale : 0            (dropout; training semantics)
 * keep_i: element i = row * cols + col is kept iff its 16 random bits (above)
 * are >= threshold; threshold = round(p * 2^16) in [0, 65536], so an element
 * is dropped with probability threshold / 2^16 = p to within 2^-17 (65536
 * drops everything); scale = 1 / (1 - p).  The caller passes threshold and
 * scale.  x holds rows [first_row, first_row + rows) of a larger [*, cols]
 * tensor (first_row 0: the whole tensor): element (i, j) of x has the index
 * (first_row + i) * cols + j there, which picks its random bits, so a tensor
 * can be evaluated in row chunks with the same result.
 * Modes: ORACLE_EXACT, binary64 throughout; ORACLE_SEQ3 stores u, r
 * and y in the I/O type (three eager launches), the dropout launch being an
 * fp32 kernel: its scale is rounded to binary32 first, like every constant in
 * the SEQ modes, and the product is rounded as it is stored.  dtype
 * ORACLE_F32 / ORACLE_BF16 as for the LayerNorm oracle. */
int oracle_ln_relu_dropout(int dtype, const void* x, const void* gamma, const void* beta, int64_t rows,
                           int64_t cols, double eps, uint32_t threshold, double scale, uint64_t seed,
                           uint64_t offset, int64_t first_row, int mode, double* y) {
  if (mode != ORACLE_EXACT && mode != ORACLE_SEQ3) return -1;
  if (first_row < 0) return -1;
  const int seq3 = mode == ORACLE_SEQ3;
  const double sc = seq3 ? r32(scale) : scale;
  int rc = oracle_add_layernorm_gelu(dtype, x, NULL, gamma, beta, rows, cols, eps, ORACLE_ACT_NONE,
                                     mode, y);
  if (rc != 0) return rc;
  const int64_t n = rows * cols;
  /* op: relu */
  for (int64_t k = 0; k < n; ++k) y[k] = (y[k] < 0.0) ? 0.0 : y[k];
  /* op: dropout */
  for (int64_t k = 0; k < n; ++k) {
    const uint32_t w = dropout_bits(seed, offset, (uint64_t)(first_row * cols + k));
    const int keep = w >= threshold;
    double v = keep ? y[k] * sc : 0.0;
    if (seq3) v = rstore(dtype, v);
    y[k] = v;
  }
  return 0;
}
