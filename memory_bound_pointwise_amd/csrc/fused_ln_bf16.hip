// fused_ln_bf16.hip -- the bf16 instantiation of the residual + LayerNorm +
// tanh-GeLU kernels (fused_ln_impl.hpp); its own translation unit so that the
// two element types compile in parallel.
#include "fused_ln_impl.hpp"

namespace mbp {

hipError_t launch_layernorm_bf16(const void* x, int64_t ldx, const void* residual, int64_t ldr,
                                 const void* gamma, const void* beta, void* y, int64_t ldy, int64_t rows,
                                 int64_t cols, double eps, int act, const Drop* drop, hipStream_t s) {
  return ln::launch<BF16IO>(x, ldx, residual, ldr, gamma, beta, y, ldy, rows, cols, eps, act, drop, s);
}

}  // namespace mbp
