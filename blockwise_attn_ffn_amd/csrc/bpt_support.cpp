// Which kernel instances exist: the host-side support table, kept beside the
// dispatch in k_*.hip (every combination accepted here has an instance).
#include <stdio.h>

#include "bpt_internal.h"

namespace bpt {
namespace {
void set_err(char* err, size_t n, const char* fmt, const char* a = "", int b = 0) {
  if (err && n) snprintf(err, n, fmt, a, b);
}
}  // namespace

int kernels_support(int d_model, int d_head, int block_q, int block_kv, int compute_f32,
                    int x_f32, int z_f32, int d_ff, int split, char* err, size_t errlen) {
  (void)x_f32;
  (void)z_f32;
  const bool bf = !compute_f32;
  bool d_ok = false;
  if (bf) {
    d_ok = d_model == 256 || d_model == 512 || d_model == 768 || d_model == 1024 ||
           d_model == 2048 || d_model == 4096;
  } else {
    d_ok = d_model == 128 || d_model == 256;
  }
  if (!d_ok) {
    set_err(err, errlen, "d_model %s%d has no kernel instance for this dtype", "", d_model);
    return 0;
  }
  if (d_head != 64 && d_head != 128) {
    set_err(err, errlen, "head size %s%d unsupported (64 or 128)", "", d_head);
    return 0;
  }
  if ((block_q != 64 && block_q != 128) || (block_kv != 64 && block_kv != 128)) {
    set_err(err, errlen, "block sizes must be 64 or 128%s", "");
    return 0;
  }
  if (!bf && d_head == 128 && block_kv == 128) {
    set_err(err, errlen, "fp32 with head size 128 needs block_kv 64%s", "");
    return 0;
  }
  if (split && !bf) {
    set_err(err, errlen, "precision 1 (bf16 pairs) needs dtype BPT_BF16%s", "");
    return 0;
  }
  if (d_ff % 256 != 0 || d_ff <= 0) {
    set_err(err, errlen, "d_ff %s%d must be a positive multiple of 256", "", d_ff);
    return 0;
  }
  return 1;
}

int operands_fit(int d_model, int d_ff, int kv_pad, size_t rows_pad, size_t es, int split,
                 char* err, size_t errlen) {
  const unsigned long long lim = 1ull << 32;
  const unsigned long long d = (unsigned long long)d_model, f = (unsigned long long)d_ff;
  // the QKV projection: the packed W_Q | W_K | W_V block and LN1(X)
  unsigned long long big = (d + 2ull * (unsigned long long)kv_pad) * d * es;
  unsigned long long act = (unsigned long long)rows_pad * d * es;
  if (staged_epilogue(d_model, split, d_ff)) {
    // staged epilogue: W_1, W_2 and one hidden block [h, d_ff] as operands
    const unsigned long long h = hidden_block_rows(d_model, rows_pad);
    if (f * d * es > big) big = f * d * es;
    if (h * f * es > act) act = h * f * es;
  }
  if (big >= lim || act >= lim) {
    if (err && errlen)
      snprintf(err, errlen, "a matrix-product operand of %llu bytes: 4 GiB or more is not supported",
               big > act ? big : act);
    return 0;
  }
  return 1;
}

}  // namespace bpt
