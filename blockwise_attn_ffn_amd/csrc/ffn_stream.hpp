// Order of the fused epilogue's weight stream (shared by the packing kernel and
// the epilogue so that both agree on it).
//
// The epilogue runs 4 waves per workgroup. Wave w owns the Z features
// [w d/4, (w+1) d/4) (NT tiles of 32) and, inside every hidden chunk of HC units,
// the units [w HC/4, (w+1) HC/4) (FT tiles of 32). It consumes its share of
// W_O, W_1 and W_2 as a sequence of stages; a stage is one 32-row tile of a
// weight over 4 consecutive k-steps of 16, i.e. 4 packed fragments (bpt_device.hpp).
// The sequence for one wave is
//   W_O:                 k-block kb (64 wide) major, Z tile a minor      (N_WO stages)
//   for every chunk c:   W_1[c]: k-block major, hidden tile f minor      (N_W1 stages)
//                        W_2[c]: k-block (64 units) major, Z tile minor  (N_W2 stages)
// and is stored contiguously, wave after wave, so the epilogue reads stage t of
// wave w at fragment 4 (w * stages + t): one linear stream per wave.
#pragma once

#include <stddef.h>

#if defined(__HIPCC__)
#define BPT_HD __host__ __device__
#else
#define BPT_HD
#endif

namespace bpt {

constexpr int kFfnWaves = 4;
constexpr int kFfnChunk = 256;      // hidden units per chunk (HC)

struct FfnStream {
  int d, dff;
  BPT_HD constexpr int nt() const { return d / (32 * kFfnWaves); }
  BPT_HD constexpr int ft() const { return kFfnChunk / (32 * kFfnWaves); }
  BPT_HD constexpr int n_wo() const { return d / 64 * nt(); }
  BPT_HD constexpr int n_w1() const { return d / 64 * ft(); }
  BPT_HD constexpr int n_w2() const { return kFfnChunk / 64 * nt(); }
  BPT_HD constexpr int per_chunk() const { return n_w1() + n_w2(); }
  BPT_HD constexpr int stages() const { return n_wo() + dff / kFfnChunk * per_chunk(); }

  BPT_HD size_t slot(int wave, int t, int j) const {
    return ((size_t)wave * stages() + t) * 4 + j;
  }
  // Stream slot of fragment (32-row tile r, k-step ks) of W_O [d, d].
  BPT_HD size_t slot_wo(int r, int ks) const {
    const int w = r / nt(), a = r % nt();
    return slot(w, (ks / 4) * nt() + a, ks % 4);
  }
  // ... of W_1 [dff, d] (rows are hidden units).
  BPT_HD size_t slot_w1(int r, int ks) const {
    const int tpc = kFfnChunk / 32;               // hidden tiles per chunk
    const int c = r / tpc, rr = r % tpc, w = rr / ft(), f = rr % ft();
    return slot(w, n_wo() + c * per_chunk() + (ks / 4) * ft() + f, ks % 4);
  }
  // ... of W_2 [d, dff] (k runs over hidden units).
  BPT_HD size_t slot_w2(int r, int ks) const {
    const int kpc = kFfnChunk / 16;               // k-steps per chunk
    const int w = r / nt(), a = r % nt(), c = ks / kpc, kk = ks % kpc;
    return slot(w, n_wo() + c * per_chunk() + n_w1() + (kk / 4) * nt() + a, kk % 4);
  }
};

}  // namespace bpt
