// The per-layer launch sequence on one stream: the six weight matrices repacked
// into matrix-core fragment order, LN1 into the packed activation operand, the
// QKV projection, attention, and the fused FFN epilogue. Optional events
// between the stages are for measurement only.
#include "bpt_launch.hpp"

namespace bpt {

namespace {
int mark(const LayerLaunch& L, int i, hipStream_t s, char* err, size_t n) {
  if (!L.events) return 0;
  hipError_t e = hipEventRecord(reinterpret_cast<hipEvent_t>(L.events[i]), s);
  if (e != hipSuccess) {
    set_err(err, n, "hipEventRecord: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}
}  // namespace

int launch_layer(const LayerLaunch& L, void* stream, char* err, size_t n) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return mark(L, 0, s, err, n) || launch_pack(L, s, err, n) || launch_ln_qkv(L, s, err, n, 0) ||
         mark(L, 1, s, err, n) || launch_ln_qkv(L, s, err, n, 1) || mark(L, 2, s, err, n) ||
         launch_attention(L, s, err, n) || mark(L, 3, s, err, n) || launch_ffn(L, s, err, n) ||
         mark(L, 4, s, err, n);
}

}  // namespace bpt
