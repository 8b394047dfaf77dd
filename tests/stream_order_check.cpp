// Host check of the epilogue weight-stream order (ffn_stream.hpp), built with g++
// by tests/test_stream_order.py. The consumption order is re-derived here from the
// epilogue's loop structure (W_O by k-block then Z tile; per hidden chunk W_1 by
// k-block then hidden tile, then W_2 by k-block then Z tile) and every fragment of
// W_O, W_1 and W_2 must land exactly on the slot where its wave reads it.
#include <stdio.h>
#include <vector>

#include "../blockwise_attn_ffn_amd/csrc/ffn_stream.hpp"

using bpt::FfnStream;
using bpt::kFfnChunk;
using bpt::kFfnWaves;

static int check(int d, int dff) {
  const FfnStream fs{d, dff};
  const int nt = d / 32 / kFfnWaves, ft = kFfnChunk / 32 / kFfnWaves;
  const size_t total = (size_t)(d * d + 2 * d * dff) / 512;   // fragments in the stream
  std::vector<int> hits(total, 0);
  size_t bad = 0;
  for (int w = 0; w < kFfnWaves; ++w) {
    size_t slot = (size_t)w * fs.stages() * 4;
    auto expect = [&](size_t got) {
      if (got >= total) { ++bad; return; }
      if (got != slot) ++bad;
      ++hits[got];
      ++slot;
    };
    for (int kb = 0; kb < d / 64; ++kb)
      for (int a = 0; a < nt; ++a)
        for (int j = 0; j < 4; ++j) expect(fs.slot_wo(w * nt + a, kb * 4 + j));
    for (int c = 0; c < dff / kFfnChunk; ++c) {
      for (int kb = 0; kb < d / 64; ++kb)
        for (int f = 0; f < ft; ++f)
          for (int j = 0; j < 4; ++j)
            expect(fs.slot_w1(c * (kFfnChunk / 32) + w * ft + f, kb * 4 + j));
      for (int kb = 0; kb < kFfnChunk / 64; ++kb)
        for (int a = 0; a < nt; ++a)
          for (int j = 0; j < 4; ++j)
            expect(fs.slot_w2(w * nt + a, c * (kFfnChunk / 16) + kb * 4 + j));
    }
    if (slot != (size_t)(w + 1) * fs.stages() * 4) ++bad;
  }
  for (size_t i = 0; i < total; ++i)
    if (hits[i] != 1) ++bad;
  if (bad) printf("d=%d dff=%d: %zu mismatches\n", d, dff, bad);
  return bad != 0;
}

int main() {
  int fail = 0;
  const int dims[][2] = {{128, 512}, {256, 1024}, {512, 2048}, {768, 3072}, {1024, 4096},
                         {2048, 8192}, {1024, 256}, {256, 768}};
  for (const auto& p : dims) fail |= check(p[0], p[1]);
  if (!fail) printf("ALL OK\n");
  return fail;
}
