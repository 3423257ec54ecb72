// fused_ln_f32.hip -- the fp32 instantiation of the residual + LayerNorm +
// tanh-GeLU kernels (fused_ln_impl.hpp), plus the dtype dispatch.
#include "fused_ln_impl.hpp"

namespace mbp {

hipError_t launch_layernorm_bf16(const void* x, const void* residual, const void* gamma,
                                 const void* beta, void* y, int64_t rows, int64_t cols, double eps,
                                 int act, const Drop* drop, hipStream_t s);

hipError_t launch_layernorm(int dtype, const void* x, const void* residual, const void* gamma,
                            const void* beta, void* y, int64_t rows, int64_t cols, double eps,
                            int act, const Drop* drop, hipStream_t s) {
  if (dtype == 1) return launch_layernorm_bf16(x, residual, gamma, beta, y, rows, cols, eps, act, drop, s);
  return ln::launch<F32IO>(x, residual, gamma, beta, y, rows, cols, eps, act, drop, s);
}

}  // namespace mbp
