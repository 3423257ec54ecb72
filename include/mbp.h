/*
 * mbp.h -- C ABI of libmbp: vertically fused memory-bound chains on gfx950.
 *
 * Every entry point takes plain device pointers and sizes, enqueues its work on
 * the given HIP stream and returns at once (asynchronous, like a kernel launch).
 * The caller owns every buffer: the library never allocates or frees device
 * memory and keeps no mutable global state beyond a per-thread error message.
 * (An instantiated graph, below, holds the HIP runtime's own resources until
 * the caller destroys it; grouped_row_mean_epilogue_noalloc keeps its
 * intermediates in a static device array compiled into the library.)
 *
 * Conventions shared by all entry points
 *   - Tensors are dense and row-major (contiguous).  A [rows, cols] tensor has
 *     element (i, j) at offset i*cols + j.  Vectors of length cols (bias, gamma,
 *     beta) are broadcast over the rows (stride 0 along the row dimension), as
 *     the TorchInductor post describes for bias in "TorchInductor Pipeline 与算子
 *     融合", section 1.1.
 *   - fp32 pointers must be 4-byte aligned and bf16 pointers 2-byte aligned;
 *     16-byte alignment (with row lengths whose bytes are a multiple of 16)
 *     selects the 128-bit load/store path, anything else a narrower path that
 *     gives identical results.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *   - Arguments are validated on the host before anything is launched.  A bad
 *     argument returns an error status and launches nothing.  A launch failure
 *     reported by the HIP runtime returns MBP_ERR_HIP; faults inside a kernel
 *     surface, as always with HIP, at the caller's next synchronisation.
 *   - n == 0 or rows == 0 is a no-op that returns MBP_OK (pointers may be NULL).
 *   - Fused entry points allow exact in-place use (y == x); any other overlap
 *     between the output and an input returns MBP_ERR_OVERLAP.
 *   - Results do not depend on the launch configuration or on the run: every
 *     reduction uses a fixed lane-to-element map and a fixed combine order.
 *
 * Sources (the four pages on operator fusion):
 *   [P1] PyTorch operator-fusion practice post (http://www.0539edu.com/news/5489619/)
 *   [P2] "算子融合与 Kernel 优化：从 CUDA Graph 到 FlashAttention 的极致性能" (plumephp.com)
 *   [P3] "4、算子融合（Kernel Fusion）：将多个小算子合并为一个，减少Kernel Launch开销" (5688vip.com)
 *   [P4] "TorchInductor Pipeline 与算子融合" (blog.kkkzoz.top)
 */
#ifndef MBP_H
#define MBP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MBP_ABI_VERSION 7

/* Largest row length (cols) the row kernels accept.  Rows of up to 16384
 * columns, and bf16 / fp16 LayerNorm and softmax rows of up to 32768, live in
 * the registers of one lane group (read once, written once); other wider rows
 * take one 1024-lane block each and two or three passes over the row, the
 * later ones rereading it from the caches. */
#define MBP_MAX_COLS 32768

typedef enum {
  MBP_OK = 0,
  MBP_ERR_NULL = 1,      /* a required pointer is NULL */
  MBP_ERR_SHAPE = 2,     /* negative size, cols <= 0, cols > MBP_MAX_COLS, or size overflow */
  MBP_ERR_DTYPE = 3,     /* unknown dtype or activation code */
  MBP_ERR_ALIGN = 4,     /* pointer not aligned to its element size */
  MBP_ERR_OVERLAP = 5,   /* output overlaps an input other than exactly (y == x) */
  MBP_ERR_WORKSPACE = 6, /* workspace NULL, misaligned (256 B) or smaller than required */
  MBP_ERR_HIP = 7,       /* the HIP runtime reported an error (see mbp_last_error) */
  MBP_ERR_ARG = 8        /* other invalid argument: non-finite constant, eps < 0, bad op code */
} mbp_status;

/* Storage types.  MBP_F16 (IEEE binary16) is accepted by the *_2d entry points
 * and by fused_softmax. */
typedef enum { MBP_F32 = 0, MBP_BF16 = 1, MBP_F16 = 2 } mbp_dtype;

typedef enum { MBP_ACT_NONE = 0, MBP_ACT_GELU_TANH = 1 } mbp_act;

typedef enum {
  MBP_OP_CHAIN = 0,
  MBP_OP_ROW_MEAN = 1,
  MBP_OP_LAYERNORM = 2,
  MBP_OP_LN_RELU_DROPOUT = 3,
  MBP_OP_SOFTMAX = 4
} mbp_op;

/* Granularity of the unfused variants. */
#define MBP_UNFUSED_PRIMITIVE 0 /* one launch per primitive op (4 / 10 / 5 / 7 launches) */
#define MBP_UNFUSED_EAGER 1     /* LayerNorm as one launch: add, layernorm, gelu (<= 3) */
#define MBP_UNFUSED_GROUPED 2   /* the 10-op graph in TVM's three groups (MBP_OP_ROW_MEAN only) */

/* ------------------------------------------------------------------------- */
/* Fused entry points: one launch; only the inputs are read and the output is
 * written in HBM, every intermediate stays in registers (LDS holds only the
 * per-wave partial sums of a row reduction).                                */

/*
 * y[i] = relu(x[i] + b1[i]) * scale + b2[i],  i < n.
 * [P1] section 1.1 (the four eager steps add, relu, mul, add) and section 3.1
 * (x, b1, b2 full fp32 tensors of one shape; scale 0.5 in the pages' example);
 * section 3.2 is the fused float4 kernel this replaces, which dropped the n % 4
 * tail -- here every n is handled.
 * x, b1, b2: device fp32 [n], read only.  y: device fp32 [n], written; y == x,
 * y == b1 or y == b2 is allowed.  scale: any finite double.  Arithmetic is
 * binary64 inside the kernel with one rounding to fp32 at the store, so y is
 * within 1 ulp of the exactly rounded result.  relu passes NaN through.
 */
mbp_status fused_pointwise_chain(const float* x, const float* b1, const float* b2, float* y,
                                 int64_t n, double scale, void* stream);

/*
 * The 10-op graph of [P4] (the model at the top of the post; section 02,
 * Table 2 lists its ten eager kernels), for every row i < rows:
 *   t = x[i,:] * alpha + bias;  a = relu(t);  s = a*a + a*c;
 *   m_i = (sum_j s[i,j]) / cols            (row sum, then divide: section 6.4)
 *   y[i,:] = (s - m_i) * gamma + beta
 * x, y: device fp32 [rows, cols]; bias, gamma, beta: device fp32 [cols].
 * y == x is allowed.  alpha, c: finite doubles (1.1 and 0.1 in the pages).
 * Arithmetic is binary64 inside the kernel; the row sum never leaves the chip.
 */
mbp_status fused_row_mean_epilogue(const float* x, const float* bias, const float* gamma,
                                   const float* beta, float* y, int64_t rows, int64_t cols,
                                   double alpha, double c, void* stream);

/*
 * Residual add + LayerNorm + tanh-GeLU, one row per lane group, for i < rows:
 *   v = x[i,:] + residual[i,:]              (residual == NULL: v = x[i,:])
 *   mu = mean(v);  var = mean((v - mu)^2)    (biased; [P3] section 4.3)
 *   u = (v - mu) / sqrt(var + eps) * gamma + beta
 *   y[i,:] = act == MBP_ACT_GELU_TANH ? 0.5 u (1 + tanh(0.7978845608 (u + 0.044715 u^3))) : u
 * [P2] section 2.3 gives the fused residual + LayerNorm + GeLU kernel and its
 * constants; [P3] section 4.3 the LayerNorm and its five unfused kernels.
 * dtype MBP_F32: x, residual, gamma, beta, y are fp32; the statistics and the
 * normalisation are computed in binary64.  dtype MBP_BF16: all five are bf16;
 * arithmetic is fp32, the output is rounded to nearest even.  The statistics are
 * two-pass over the row (mean first, then the centred sum of squares), held in
 * registers up to 16384 columns (bf16: up to MBP_MAX_COLS).  GeLU uses the identity 0.5 (1 + tanh z) = 1 / (1 + exp(-2 z)).
 * x, residual: [rows, cols]; gamma, beta: [cols]; y: [rows, cols]; y == x or
 * y == residual is allowed.  eps: finite, >= 0.  1 <= cols <= MBP_MAX_COLS.
 */
mbp_status fused_add_layernorm_gelu(mbp_dtype dtype, const void* x, const void* residual,
                                    const void* gamma, const void* beta, void* y, int64_t rows,
                                    int64_t cols, double eps, mbp_act act, void* stream);

/*
 * LayerNorm -> ReLU -> Dropout ([P2] section 2.1: layer_norm, relu, dropout
 * with p = 0.1 there, three memory round trips fused into one kernel), for
 * every row i < rows and column j < cols:
 *   u = (x[i,:] - mean) / sqrt(var + eps) * gamma + beta   (as the LayerNorm above)
 *   r = max(u, 0);   y[i,j] = keep(k) ? r / (1 - p) : 0,   k = i*cols + j
 * Dropout in training semantics.  keep(k): the 16 random bits of element k
 * -- half k mod 8 of the Philox4x32-10 block (counter = (k div 8, offset),
 * key = seed; J. K. Salmon et al., "Parallel random numbers: as easy as 1, 2,
 * 3", SC'11) -- are >= round(p * 2^16); p is realised to within 2^-17.  The
 * mask depends only on (seed, offset, k): the same call gives the same mask,
 * a caller advances `offset` to draw a new one.  x, y: device [rows, cols] in
 * `dtype` (MBP_F32 or MBP_BF16); gamma, beta: [cols]; y == x allowed.
 * p in [0, 1] (p == 1: y = 0).  Arithmetic as fused_add_layernorm_gelu.
 */
mbp_status fused_layernorm_relu_dropout(mbp_dtype dtype, const void* x, const void* gamma,
                                        const void* beta, void* y, int64_t rows, int64_t cols,
                                        double eps, double p, uint64_t seed, uint64_t offset,
                                        void* stream);

/*
 * Row softmax over the last dimension, for every row i < rows:
 *   m_i = max_j x[i,j];  l_i = sum_j exp(x[i,j] - m_i);  y[i,j] = exp(x[i,j] - m_i) / l_i
 * ([P1] section 4.2: normalised by the row maximum, with the running
 * max / sum statistics; [P3] section 4.2 lists softmax as the "Reduce +
 * Element-wise" fusion pattern).  One launch; up to 16384 columns (bf16 and
 * fp16: up to MBP_MAX_COLS) the row is read once and written once.  x, y: device [rows, cols], dense, in `dtype` (MBP_F32,
 * MBP_BF16 or MBP_F16); y == x is allowed.  cols <= MBP_MAX_COLS.
 * Arithmetic in fp32 with one rounding to `dtype` at the store; -inf entries
 * (masks) give exactly 0, a row of -inf only gives NaN (0/0), a NaN makes its
 * row NaN.  Results are deterministic (fixed reduction order).
 */
mbp_status fused_softmax(mbp_dtype dtype, const void* x, void* y, int64_t rows, int64_t cols,
                         void* stream);

/* ------------------------------------------------------------------------- */
/* Two-dimensional forms with row strides and 16-bit storage.  The pages'
 * chain and 10-op graph written for any storage type of one tensor family
 * (MBP_F32, MBP_BF16, MBP_F16: every operand in `dtype`) and for operands
 * that are not dense: element (i, j) of an operand with row stride ld is at
 * offset i*ld + j (unit stride along a row).  An input with ld == 0 is one
 * row used for every row (a broadcast bias, stride 0 as in [P4] section 1.1);
 * [P1] section 6.2 warns that a non-contiguous input otherwise costs a hidden
 * .contiguous() copy.  Arithmetic is binary64; each result is rounded once, to
 * nearest even, to `dtype` at the store (through a round-to-odd binary32 for
 * the 16-bit types, which equals one rounding from binary64).
 * Strides: an input's ld is 0 or >= cols; the output's ldy >= cols (any ldy
 * when rows == 1).  Pointers aligned to the element size.  In-place use needs
 * y == x and ldy == ldx; any other overlap of the output's extent with an
 * input's extent returns MBP_ERR_OVERLAP.  rows == 0 is a no-op.
 */

/*
 * y[i,j] = relu(x[i,j] + b1[i,j]) * scale + b2[i,j] for i < rows, j < cols,
 * with row strides ldx, ldb1, ldb2, ldy.  [P1] sections 1.1 and 3.1 (the
 * chain; b1 and b2 full tensors there, broadcast rows here when ld == 0).
 * cols: any positive length (no MBP_MAX_COLS bound: nothing is held per row).
 */
mbp_status fused_pointwise_chain_2d(mbp_dtype dtype, const void* x, int64_t ldx, const void* b1,
                                    int64_t ldb1, const void* b2, int64_t ldb2, void* y,
                                    int64_t ldy, int64_t rows, int64_t cols, double scale,
                                    void* stream);

/*
 * The 10-op graph of [P4] (as fused_row_mean_epilogue) with x and y of row
 * strides ldx and ldy and every operand in `dtype`; bias, gamma, beta: dense
 * [cols] vectors in `dtype`.  cols <= MBP_MAX_COLS.
 */
mbp_status fused_row_mean_epilogue_2d(mbp_dtype dtype, const void* x, int64_t ldx,
                                      const void* bias, const void* gamma, const void* beta,
                                      void* y, int64_t ldy, int64_t rows, int64_t cols,
                                      double alpha, double c, void* stream);

/*
 * fused_add_layernorm_gelu with row strides: row i of x starts at element
 * i*ldx, of the residual at i*ldr, of y at i*ldy (unit stride along a row),
 * so padded or sliced activations (x[:, :cols] of a wider buffer) are read
 * and written in place, without the hidden .contiguous() copy [P1] section
 * 6.2 warns about.  dtype MBP_F32 or MBP_BF16; gamma, beta: dense [cols].
 * residual may be NULL (ldr ignored).  ldx and ldr: 0 (one row used for
 * every row) or >= cols; ldy >= cols (any value when rows == 1).  y may be
 * exactly x (y == x, ldy == ldx) or exactly the residual; any other overlap
 * of y's extent with an input's returns MBP_ERR_OVERLAP.  Results equal
 * those of fused_add_layernorm_gelu on the same rows bit for bit.  The
 * fastest paths need rows on 16-byte boundaries (16-byte aligned bases and
 * strides of whole 16-byte vectors), or x, residual and y sharing one stride
 * and one alignment modulo 16 bytes.
 */
mbp_status fused_add_layernorm_gelu_2d(mbp_dtype dtype, const void* x, int64_t ldx, const void* residual,
                                       int64_t ldr, const void* gamma, const void* beta, void* y,
                                       int64_t ldy, int64_t rows, int64_t cols, double eps, mbp_act act,
                                       void* stream);

/*
 * fused_layernorm_relu_dropout with row strides ldx and ldy (as above; y may
 * be exactly x).  The dropout mask still follows the element's position in
 * the [rows, cols] result, k = i*cols + j, not its address, so it is the
 * dense call's mask.
 */
mbp_status fused_layernorm_relu_dropout_2d(mbp_dtype dtype, const void* x, int64_t ldx, const void* gamma,
                                           const void* beta, void* y, int64_t ldy, int64_t rows, int64_t cols,
                                           double eps, double p, uint64_t seed, uint64_t offset,
                                           void* stream);

/*
 * fused_softmax with row strides ldx (0 or >= cols) and ldy (>= cols);
 * fp32, bf16 or fp16; y may be exactly x.  Rows of x and y that agree
 * modulo 16 bytes (equal alignment and strides that differ by a multiple of
 * 16 bytes) keep the 16-byte window path.
 */
mbp_status fused_softmax_2d(mbp_dtype dtype, const void* x, int64_t ldx, void* y, int64_t ldy,
                            int64_t rows, int64_t cols, void* stream);

/* ------------------------------------------------------------------------- */
/* Unfused "before" variants: one launch per op, every intermediate written to
 * and read back from the caller's workspace in the I/O type (row statistics in
 * fp32), as eager execution does.  They exist for the before/after comparison.
 * Each op rounds its result to the storage type; row reductions accumulate in
 * binary64 and store fp32.  Workspace: device memory of at least
 * mbp_unfused_workspace_bytes(...) bytes, 256-byte aligned, not overlapping any
 * argument; its contents on entry do not matter.  The output may not alias an
 * input.                                                                    */

/* [P1] section 1.1: four launches add, relu, mul, add (fp32 intermediates). */
mbp_status unfused_pointwise_chain(const float* x, const float* b1, const float* b2, float* y,
                                   int64_t n, double scale, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* [P4] section 02, Table 2: ten launches mul, add, relu, mul, mul, add, mean,
 * sub, mul, add (alpha and c rounded to fp32, as eager fp32 kernels do). */
mbp_status unfused_row_mean_epilogue(const float* x, const float* bias, const float* gamma,
                                     const float* beta, float* y, int64_t rows, int64_t cols,
                                     double alpha, double c, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* The 10-op graph partitioned as TVM's FuseOps rules partition it ([P4]
 * section 09, Figure 17): three launches, each one kernel of its own group --
 *   1. s = relu(x*alpha + bias)^2 + relu(x*alpha + bias)*c  (written to the workspace),
 *   2. m = row mean of s,
 *   3. y = (s - m)*gamma + beta.
 * s is written once and read twice.  Every op rounds to fp32 as its eager
 * kernel does (alpha and c rounded to fp32, no contraction), so y equals the
 * output of unfused_row_mean_epilogue bit for bit.  Workspace:
 * mbp_unfused_workspace_bytes(MBP_OP_ROW_MEAN, MBP_F32, rows, cols, 0, 0,
 * MBP_UNFUSED_GROUPED). */
mbp_status grouped_row_mean_epilogue(const float* x, const float* bias, const float* gamma,
                                     const float* beta, float* y, int64_t rows, int64_t cols,
                                     double alpha, double c, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Bytes of the library's static scratch array (one per GPU). */
#define MBP_STATIC_SCRATCH_BYTES (16u << 20)

/*
 * grouped_row_mean_epilogue for callers that cannot allocate device memory
 * (code recorded by graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same three launches and the same result bit for bit, with s
 * and m kept in a static array of MBP_STATIC_SCRATCH_BYTES compiled into the
 * library instead of a caller's workspace.  No workspace argument; the call
 * allocates nothing and issues no memset (every byte of s and m it reads it
 * has written first).  Limit: rows * cols * 4 plus rows * 4 (each rounded up
 * to 256 bytes) must fit the array -- about 4 M elements, e.g. 1024 x 1024 --
 * else MBP_ERR_WORKSPACE.  Each GPU has its own copy of the array, held from
 * the first call on that GPU until the process ends; the first call on a GPU
 * looks the copy up (make it outside a capture).  `stream` must belong to the
 * current device (else MBP_ERR_ARG).  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (different streams, or threads
 * without ordering) race on it and must not be made; calls in one stream are
 * ordered and safe.  Arguments and errors otherwise as
 * grouped_row_mean_epilogue.
 */
mbp_status grouped_row_mean_epilogue_noalloc(const float* x, const float* bias, const float* gamma,
                                             const float* beta, float* y, int64_t rows, int64_t cols,
                                             double alpha, double c, void* stream);

/* [P3] section 4.3 and [P2] section 2.3.  granularity MBP_UNFUSED_PRIMITIVE:
 * [add,] mean, var, sub, div, mul-add[, gelu]  (5 launches for plain
 * LayerNorm, 7 with residual and GeLU).  granularity MBP_UNFUSED_EAGER:
 * [add,] layernorm[, gelu] (the fused LayerNorm kernel as the middle launch). */
mbp_status unfused_add_layernorm_gelu(mbp_dtype dtype, const void* x, const void* residual,
                                      const void* gamma, const void* beta, void* y, int64_t rows,
                                      int64_t cols, double eps, mbp_act act, int granularity,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * LayerNorm -> ReLU -> Dropout as the three eager launches of [P2] section
 * 2.1 (layer_norm, relu, dropout), each result stored in `dtype` in the
 * workspace (two [rows, cols] buffers; mbp_unfused_workspace_bytes with
 * MBP_OP_LN_RELU_DROPOUT).  Same mask as the fused entry point.
 */
mbp_status unfused_layernorm_relu_dropout(mbp_dtype dtype, const void* x, const void* gamma,
                                          const void* beta, void* y, int64_t rows, int64_t cols,
                                          double eps, double p, uint64_t seed, uint64_t offset,
                                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * The row softmax of fused_softmax as the eager sequence of five launches
 * ([P3] section 4.2 names softmax as the reduce + element-wise pattern that
 * fusion collapses): row max m; d = x - m; e = exp(d); row sum l; y = e / l.
 * d and e are stored in `dtype` (MBP_F32 or MBP_BF16) in the workspace, m and
 * l as fp32; each element-wise op computes in fp32 (expf for the exponential)
 * and rounds once to `dtype`; the row sum accumulates in binary64.
 * Workspace: mbp_unfused_workspace_bytes(MBP_OP_SOFTMAX, dtype, rows, cols,
 * 0, 0, 0).  y may not alias x.
 */
mbp_status unfused_softmax(mbp_dtype dtype, const void* x, void* y, int64_t rows, int64_t cols,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace the unfused variant of `op` needs (bytes; 0 for a no-op shape).
 * For MBP_OP_CHAIN pass rows = 1, cols = n.  has_residual and act matter only
 * for MBP_OP_LAYERNORM; granularity for MBP_OP_LAYERNORM and (GROUPED or not)
 * MBP_OP_ROW_MEAN.  Returns (size_t)-1 for invalid arguments. */
size_t mbp_unfused_workspace_bytes(mbp_op op, mbp_dtype dtype, int64_t rows, int64_t cols,
                                   int has_residual, mbp_act act, int granularity);

/* Kernel launches one call makes (fused = 1: the fused entry point; fused = 0:
 * the unfused one at `granularity`).  -1 for invalid arguments. */
int mbp_launches_per_call(mbp_op op, int fused, int granularity, int has_residual, mbp_act act);

/* ------------------------------------------------------------------------- */
/* Graph capture ([P2] section 4: capture a fixed sequence of launches once,
 * instantiate it, then submit it with one call; shapes and addresses are fixed
 * at capture).  Between mbp_graph_capture_begin and mbp_graph_capture_end,
 * every launch this thread enqueues on `stream` -- any of the entry points
 * above -- is recorded, not executed.  The entry points validate their
 * arguments as usual while recording: one that returns an error records
 * nothing.  The entry points make no allocation and no memset, so a graph holds
 * kernel nodes only.
 *   - stream: a created hipStream_t (the NULL stream cannot be captured).
 *   - The capture is thread-local (hipStreamCaptureModeThreadLocal): this
 *     thread may not call hipMalloc or synchronise while it records.
 *   - mbp_graph_capture_end ends the capture in every case; it instantiates
 *     the graph and returns a handle the caller owns (MBP_ERR_ARG if nothing
 *     was captured; MBP_ERR_HIP if the capture was invalidated).
 *   - mbp_graph_launch enqueues one replay on any stream (NULL allowed); the
 *     buffers named at capture must still be alive.  Replays of one graph on
 *     different streams must not overlap in time (they write the same memory).
 *   - mbp_graph_destroy releases the handle (NULL is a no-op); no replay may
 *     still be pending. */
typedef struct mbp_graph_s mbp_graph;

mbp_status mbp_graph_capture_begin(void* stream);
mbp_status mbp_graph_capture_end(void* stream, mbp_graph** graph);
mbp_status mbp_graph_launch(const mbp_graph* graph, void* stream);
/* Number of nodes in the captured graph (-1 for NULL). */
int64_t mbp_graph_nodes(const mbp_graph* graph);
mbp_status mbp_graph_destroy(mbp_graph* graph);

/* ------------------------------------------------------------------------- */
/* Calibration and diagnostics.                                              */

/* Plain device-to-device copy of `bytes` bytes with 128-bit loads and stores
 * (the same streaming pattern as the fused kernels, no arithmetic).  Used to
 * measure attainable HBM bandwidth and to scale rocprofv3 byte counters.
 * src and dst: device pointers, 16-byte aligned, not overlapping; bytes a
 * multiple of 16. */
mbp_status mbp_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

/* The same streaming pattern with nsrc (1 .. 4) inputs of `bytes` bytes each:
 * dst = srcs[0] ^ srcs[1] ^ ... (bitwise), so every load is used.  The bare
 * stream of a kernel that reads nsrc tensors and writes one, with no
 * arithmetic: the like-for-like floor of each fused kernel ([P1] section 6.3:
 * confirm a gain with the profiler and the bandwidth arithmetic).  srcs: host
 * array of nsrc device pointers, each 16-byte aligned and not overlapping
 * dst; dst 16-byte aligned; bytes a multiple of 16 (0: no-op). */
mbp_status mbp_stream_rw(const void* const* srcs, int nsrc, void* dst, size_t bytes, void* stream);

/* y[i] = x[i] rounded to bfloat16 (nearest even; NaN stays NaN with its sign),
 * with the binary32 -> bfloat16 conversion that every kernel storing bf16 uses
 * (v_cvt_pk_bf16_f32), exposed so that it can be checked over every binary32
 * bit pattern.  x: device fp32 [n], 4-byte aligned; y: device [n] bf16 bit
 * patterns, 2-byte aligned, not overlapping x.  n == 0 is a no-op. */
mbp_status mbp_convert_f32_to_bf16(const float* x, uint16_t* y, int64_t n, void* stream);

/* Static description of a status code. */
const char* mbp_status_string(mbp_status s);

/* Detail of the last failing call on this thread ("" if none). */
const char* mbp_last_error(void);

/* MBP_ABI_VERSION of the built library. */
int mbp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MBP_H */
