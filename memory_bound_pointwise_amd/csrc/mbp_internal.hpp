// mbp_internal.hpp -- host-side launchers behind the C ABI.  Arguments reach
// these functions already validated by abi.cpp; each launcher only picks a
// launch configuration, enqueues its kernel(s) and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mbp {

// Dropout of one call: element i (flat index) is kept iff its 16 random bits
// are >= thr; kept values are multiplied by scale.  The bits of element i are
// half i mod 8 of Philox4x32-10 with key (seed) and counter (i div 8, offset).
struct Drop {
  uint64_t seed;
  uint64_t offset;
  uint32_t thr;  // round(p * 2^16), 0 .. 65536
  float scale;   // 1 / (1 - p)
};

// epilogues of the LayerNorm kernels
constexpr int kEpiNone = 0, kEpiGelu = 1, kEpiReluDrop = 2;

// A dispatch addresses at most 2^32 - 1 work-items along x, so a launch of
// `block`-thread blocks takes at most this many blocks.  Kernels that loop
// over their work cap their grids at it; kernels with one block per row group
// and no loop are launched on row chunks of at most kRowsPerDispatch rows
// (2^21 rows make at most 2^21 row groups: with the few edge blocks of the
// window kernels, under 2^22 blocks of up to 1024 threads).
constexpr int64_t dispatch_blocks(int block) { return (int64_t)0xFFFFFFFFu / block; }
constexpr int64_t kRowsPerDispatch = int64_t(1) << 21;

hipError_t launch_chain(const float* x, const float* b1, const float* b2, float* y, int64_t n,
                        double scale, hipStream_t s);
// dtype: 0 fp32, 1 bf16, 2 fp16; row strides in elements (0: broadcast row)
hipError_t launch_chain_2d(int dtype, const void* x, int64_t ldx, const void* b1, int64_t ldb1,
                          const void* b2, int64_t ldb2, void* y, int64_t ldy, int64_t rows, int64_t cols,
                          double scale, hipStream_t s);
// row softmax over the last dimension (dtype 0 fp32, 1 bf16, 2 fp16); row i
// of x at i * ldx, of y at i * ldy (elements)
hipError_t launch_softmax(int dtype, const void* x, int64_t ldx, void* y, int64_t ldy, int64_t rows,
                          int64_t cols, hipStream_t s);
hipError_t launch_row_mean_2d(int dtype, const void* x, int64_t ldx, const void* bias, const void* gamma,
                              const void* beta, void* y, int64_t ldy, int64_t rows, int64_t cols,
                              double alpha, double c, hipStream_t s);
hipError_t launch_row_mean(const float* x, const float* bias, const float* gamma,
                           const float* beta, float* y, int64_t rows, int64_t cols, double alpha,
                           double c, hipStream_t s);
// act: kEpiNone, kEpiGelu or kEpiReluDrop (then `drop` describes the dropout)
hipError_t launch_layernorm(int dtype, const void* x, const void* residual, const void* gamma,
                            const void* beta, void* y, int64_t rows, int64_t cols, double eps,
                            int act, const Drop* drop, hipStream_t s);
// the same with row strides (elements): row i of x, residual and y at i * ld
// (an input stride of 0: one row used for every row)
hipError_t launch_layernorm_2d(int dtype, const void* x, int64_t ldx, const void* residual, int64_t ldr,
                               const void* gamma, const void* beta, void* y, int64_t ldy, int64_t rows,
                               int64_t cols, double eps, int act, const Drop* drop, hipStream_t s);
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
// dst = srcs[0] ^ ... ^ srcs[nsrc - 1] (nsrc 1 .. 4), 16-byte accesses
hipError_t launch_stream(const void* const* srcs, int nsrc, void* dst, size_t bytes, hipStream_t s);
hipError_t launch_to_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t s);

// Unfused primitives (one launch each).
enum EwOp {
  EW_ADD = 0,      // a + b
  EW_SUB = 1,      // a - b
  EW_MUL = 2,      // a * b
  EW_RELU = 3,     // a < 0 ? 0 : a
  EW_MULS = 4,     // a * scalar
  EW_DIVSD = 5,    // a / sqrt(b + scalar)     (b: per-row variance)
  EW_MULADD = 6,   // a * b + c   (two roundings)
  EW_GELU = 7,     // tanh-GeLU of a
  EW_DROPOUT = 8,  // keep(i) ? a * drop.scale : 0   (the element's index i picks its random bits)
  EW_PROLOGUE = 9,       // r = relu(a * scalar + b); r * r + r * scalar2   (five roundings)
  EW_CENTER_AFFINE = 10, // (a - b) * c + d   (three roundings)
  EW_EXP = 11,           // exp(a)   (fp32 expf)
  EW_DIV = 12,           // a / b
};
// How operand b (and c) is indexed: full tensor, per column (vector of cols),
// or per row (vector of rows, fp32).
enum EwIndex { IX_FULL = 0, IX_COL = 1, IX_ROW = 2 };

hipError_t launch_ew(int op, int dtype, const void* a, const void* b, int b_ix, const void* c,
                     int c_ix, void* out, int64_t rows, int64_t cols, float scalar,
                     hipStream_t s, const Drop* drop = nullptr);
// launch_ew with a fourth operand d (read by EW_CENTER_AFFINE only) and a
// second scalar (read by EW_PROLOGUE only).
hipError_t launch_ew4(int op, int dtype, const void* a, const void* b, int b_ix, const void* c,
                      int c_ix, const void* d, int d_ix, void* out, int64_t rows, int64_t cols,
                      float scalar, float scalar2, hipStream_t s, const Drop* drop = nullptr);
// Row maximum (NaN skipped) and row sum (binary64 accumulation) of a
// [rows, cols] tensor, stored as fp32 [rows].
hipError_t launch_row_max(int dtype, const void* a, float* out, int64_t rows, int64_t cols, hipStream_t s);
hipError_t launch_row_sum(int dtype, const void* a, float* out, int64_t rows, int64_t cols, hipStream_t s);
// Row mean (fp32 out) and biased variance about a given mean (fp32 out) of a
// [rows, cols] tensor; binary64 accumulation.
hipError_t launch_row_mean_only(int dtype, const void* a, float* mean, int64_t rows,
                                int64_t cols, hipStream_t s);
hipError_t launch_row_var(int dtype, const void* a, const float* mean, float* var, int64_t rows,
                          int64_t cols, hipStream_t s);

// The current GPU's copy of the library's static scratch array (its device
// address, found once per GPU with hipGetSymbolAddress and kept) and its size
// in bytes.  Allocates nothing.
hipError_t static_scratch(void** ptr, size_t* bytes);

// Compute units of the current GPU (looked up once per GPU and kept); 0 when
// the runtime does not say.
int compute_units();

}  // namespace mbp
