// The d_k 128 dK / dV kernel of the attention backward (attn_bwd_kernels.hpp:
// split by gradient over two waves per SIMD), in a translation unit of its own so
// that it is compiled without the setting that keeps matrix-core results in VGPRs.
#include "attn_bwd_kernels.hpp"

namespace bpt {

int launch_bwd_dkv128(const BwdArgs& g, int grid, bool general, hipStream_t s) {
  auto k = general ? bwd_dkv_split_kernel<128, 64, true> : bwd_dkv_split_kernel<128, 64, false>;
  hipLaunchKernelGGL(k, dim3(grid), dim3(512), 0, s, g);
  return 0;
}

}  // namespace bpt
