// fused_ln_f32.hip -- the fp32 instantiation of the residual + LayerNorm +
// tanh-GeLU kernels (fused_ln_impl.hpp), plus the dtype dispatch.
#include "fused_ln_impl.hpp"

namespace mbp {

hipError_t launch_layernorm_bf16(const void* x, int64_t ldx, const void* residual, int64_t ldr,
                                 const void* gamma, const void* beta, void* y, int64_t ldy, int64_t rows,
                                 int64_t cols, double eps, int act, const Drop* drop, hipStream_t s);

hipError_t launch_layernorm_2d(int dtype, const void* x, int64_t ldx, const void* residual, int64_t ldr,
                               const void* gamma, const void* beta, void* y, int64_t ldy, int64_t rows,
                               int64_t cols, double eps, int act, const Drop* drop, hipStream_t s) {
  if (dtype == 1)
    return launch_layernorm_bf16(x, ldx, residual, ldr, gamma, beta, y, ldy, rows, cols, eps, act, drop, s);
  return ln::launch<F32IO>(x, ldx, residual, ldr, gamma, beta, y, ldy, rows, cols, eps, act, drop, s);
}

hipError_t launch_layernorm(int dtype, const void* x, const void* residual, const void* gamma,
                            const void* beta, void* y, int64_t rows, int64_t cols, double eps,
                            int act, const Drop* drop, hipStream_t s) {
  return launch_layernorm_2d(dtype, x, cols, residual, cols, gamma, beta, y, cols, rows, cols, eps, act, drop, s);
}

}  // namespace mbp
