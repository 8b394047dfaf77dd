// Host-only driver for the C ABI's validation layer, built with ASan + UBSan by
// tests/test_abi.py. The kernel launcher is replaced by a stub that records what
// it was asked to do, so valid calls can be exercised without a GPU.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../blockwise_attn_ffn_amd/csrc/bpt_internal.h"
#include "bpt.h"

namespace bpt {
static int g_launches = 0;
static LayerLaunch g_last[8];
int launch_layer(const LayerLaunch& L, void*, char*, size_t) {
  if (g_launches < 8) g_last[g_launches] = L;
  ++g_launches;
  return 0;
}
static int g_bwd_launches = 0;
static AttnBwdLaunch g_bwd;
int launch_attention_bwd(const AttnBwdLaunch& L, void*, char*, size_t) {
  g_bwd = L;
  ++g_bwd_launches;
  return 0;
}
static int g_fwd_launches = 0, g_merge_launches = 0;
static AttnFwdLaunch g_fwd;
int launch_attention_fwd(const AttnFwdLaunch& L, void*, char*, size_t) {
  g_fwd = L;
  ++g_fwd_launches;
  return 0;
}
int launch_attention_merge(int, int, int, int, float*, float*, const void*, const float*, void*, char*,
                           size_t) {
  ++g_merge_launches;
  return 0;
}
static int g_layer_bwd_launches = 0;
static LayerBwdLaunch g_layer_bwd;
int launch_layer_bwd(const LayerBwdLaunch& L, void*, char*, size_t) {
  g_layer_bwd = L;
  ++g_layer_bwd_launches;
  return 0;
}
static int g_ring_pack = 0, g_ring_share = 0;
static RingShareLaunch g_ring;
int launch_ring_pack_kv(const RingKvLaunch&, void*, char*, size_t) {
  ++g_ring_pack;
  return 0;
}
int launch_ring_share(const RingShareLaunch& L, void*, char*, size_t) {
  g_ring = L;
  ++g_ring_share;
  return 0;
}
// the no-allocation entry point's fixed scratch: a fake device address
static int g_scratch_queries = 0;
int noalloc_scratch(void** ptr, char*, size_t) {
  ++g_scratch_queries;
  *ptr = reinterpret_cast<void*>(uintptr_t(0x7f0000000000ull + (5ull << 36)));
  return 0;
}
}  // namespace bpt

static int g_fail = 0;
#define EXPECT(c)                                               \
  do {                                                          \
    if (!(c)) {                                                 \
      printf("FAILED line %d: %s (%s)\n", __LINE__, #c, bpt_last_error()); \
      g_fail = 1;                                               \
    }                                                           \
  } while (0)

static char* fake(uint64_t off) { return reinterpret_cast<char*>(uintptr_t(0x7f0000000000ull + off)); }

int main() {
  bpt_layer_desc_t d;
  memset(&d, 0, sizeof(d));
  d.batch = 2; d.seq_len = 200; d.d_model = 256; d.n_heads = 4; d.d_ff = 1024;
  d.block_q = 128; d.block_kv = 64; d.causal = 1; d.ln_eps = 1e-5f;
  d.dtype = BPT_BF16; d.out_dtype = BPT_BF16;
  bpt_layer_weights_t w[3];
  for (int l = 0; l < 3; ++l) {
    const void** p = reinterpret_cast<const void**>(&w[l]);
    for (int i = 0; i < 10; ++i) p[i] = fake((3ull << 36) + (uint64_t)(l * 10 + i) * (1ull << 30));
  }
  const size_t need = bpt_layer_workspace_bytes(&d);
  EXPECT(need > 0);
  // a valid layer call reaches the launcher once, with the carved workspace
  EXPECT(bpt_layer_fwd(&d, fake(0), &w[0], fake(1ull << 36), fake(2ull << 36), need, nullptr) == BPT_OK);
  EXPECT(bpt::g_launches == 1);
  EXPECT(bpt::g_last[0].seq_pad == 256 && bpt::g_last[0].d_head == 64);
  EXPECT(bpt::g_last[0].xpack == fake(2ull << 36) && bpt::g_last[0].rows_pad == 512);
  EXPECT((char*)bpt::g_last[0].vt > (char*)bpt::g_last[0].k && (char*)bpt::g_last[0].k > (char*)bpt::g_last[0].q);
  EXPECT(bpt::g_last[0].lse == nullptr);
  // the no-allocation entry point carves the same layout from its fixed scratch
  bpt::g_launches = 0;
  EXPECT(bpt_layer_fwd_noalloc(&d, fake(0), &w[0], fake(1ull << 36), nullptr) == BPT_OK);
  EXPECT(bpt::g_launches == 1 && bpt::g_scratch_queries == 1);
  EXPECT(bpt::g_last[0].xpack == fake(5ull << 36) && bpt::g_last[0].rows_pad == 512);
  {  // too large for the scratch: rejected before the scratch is looked up
    bpt_layer_desc_t big = d;
    big.batch = 64; big.seq_len = 1024; big.d_model = 1024; big.n_heads = 16; big.d_ff = 4096;
    EXPECT(bpt_layer_workspace_bytes(&big) > BPT_NOALLOC_SCRATCH_BYTES);
    EXPECT(bpt_layer_fwd_noalloc(&big, fake(0), &w[0], fake(1ull << 36), nullptr) == BPT_ERR_WORKSPACE);
    EXPECT(bpt::g_scratch_queries == 1 && bpt::g_launches == 1);
    EXPECT(bpt_layer_fwd_noalloc(&d, nullptr, &w[0], fake(1ull << 36), nullptr) == BPT_ERR_NULL);
    EXPECT(bpt_layer_fwd_noalloc(&d, fake(4), &w[0], fake(1ull << 36), nullptr) == BPT_ERR_ALIGN);
    EXPECT(bpt::g_scratch_queries == 1);
  }
  // the statistics entry passes its lse buffer to the launcher
  float* lse = reinterpret_cast<float*>(fake(3ull << 35));
  bpt::g_launches = 0;
  EXPECT(bpt_layer_fwd_lse(&d, fake(0), &w[0], fake(1ull << 36), lse, fake(2ull << 36), need, nullptr) == BPT_OK);
  EXPECT(bpt::g_launches == 1 && bpt::g_last[0].lse == lse);
  // a 3-layer stack with a bf16 Z uses the workspace residual buffer between layers
  const size_t need3 = bpt_stack_workspace_bytes(&d, 3);
  EXPECT(need3 > need);
  bpt::g_launches = 0;
  EXPECT(bpt_stack_fwd(&d, 3, fake(0), w, fake(1ull << 36), fake(2ull << 36), need3, nullptr) == BPT_OK);
  EXPECT(bpt::g_launches == 3);
  EXPECT(bpt::g_last[0].x == fake(0) && bpt::g_last[0].x_f32 == 0 && bpt::g_last[0].z_f32 == 1);
  EXPECT(bpt::g_last[1].x == bpt::g_last[0].z && bpt::g_last[1].z == bpt::g_last[0].z);
  EXPECT(bpt::g_last[2].z == fake(1ull << 36) && bpt::g_last[2].z_f32 == 0);
  EXPECT(bpt_stack_fwd(&d, 3, fake(0), w, fake(1ull << 36), fake(2ull << 36), need3 - 1, nullptr) == BPT_ERR_WORKSPACE);
  // with an fp32 Z the residual stream lives in Z
  d.out_dtype = BPT_F32;
  EXPECT(bpt_stack_workspace_bytes(&d, 3) == need);
  bpt::g_launches = 0;
  EXPECT(bpt_stack_fwd(&d, 3, fake(0), w, fake(1ull << 36), fake(2ull << 36), need, nullptr) == BPT_OK);
  EXPECT(bpt::g_last[0].z == fake(1ull << 36) && bpt::g_last[1].x == fake(1ull << 36));
  // invalid inputs never reach the launcher
  bpt::g_launches = 0;
  bpt_layer_desc_t bad = d;
  bad.ln_eps = NAN;
  EXPECT(bpt_layer_fwd(&bad, fake(0), &w[0], fake(1ull << 36), fake(2ull << 36), need, nullptr) == BPT_ERR_SHAPE);
  bad = d; bad.n_heads = 3;
  EXPECT(bpt_layer_fwd(&bad, fake(0), &w[0], fake(1ull << 36), fake(2ull << 36), need, nullptr) == BPT_ERR_SHAPE);
  bad = d; bad.block_kv = 32;
  EXPECT(bpt_layer_fwd(&bad, fake(0), &w[0], fake(1ull << 36), fake(2ull << 36), need, nullptr) == BPT_ERR_UNSUPPORTED);
  EXPECT(bpt_layer_fwd(&d, fake(0), &w[0], fake(64), fake(2ull << 36), need, nullptr) == BPT_ERR_ALIAS);
  EXPECT(bpt_layer_fwd(&d, fake(0), nullptr, fake(1ull << 36), fake(2ull << 36), need, nullptr) == BPT_ERR_NULL);
  EXPECT(bpt_layer_fwd(nullptr, fake(0), &w[0], fake(1ull << 36), fake(2ull << 36), need, nullptr) == BPT_ERR_NULL);
  EXPECT(bpt_layer_fwd_lse(&d, fake(0), &w[0], fake(1ull << 36), nullptr, fake(2ull << 36), need, nullptr) == BPT_ERR_NULL);
  EXPECT(bpt_layer_fwd_lse(&d, fake(0), &w[0], fake(1ull << 36), lse + 1, fake(2ull << 36), need, nullptr) == BPT_ERR_ALIGN);
  EXPECT(bpt_layer_fwd_lse(&d, fake(0), &w[0], fake(1ull << 36), reinterpret_cast<float*>(fake(64)), fake(2ull << 36), need, nullptr) == BPT_ERR_ALIAS);
  EXPECT(bpt_layer_fwd_lse(&d, fake(0), &w[0], fake(1ull << 36), reinterpret_cast<float*>(fake((1ull << 36) + 64)), fake(2ull << 36), need, nullptr) == BPT_ERR_ALIAS);
  EXPECT(bpt_layer_fwd_lse(&d, fake(0), &w[0], fake(1ull << 36), reinterpret_cast<float*>(fake((2ull << 36) + 4096)), fake(2ull << 36), need, nullptr) == BPT_ERR_ALIAS);
  EXPECT(bpt::g_launches == 0);
  EXPECT(strlen(bpt_last_error()) > 0);
  EXPECT(strcmp(bpt_status_str(BPT_ERR_ALIAS), "overlapping buffers") == 0);
  // empty calls
  bad = d; bad.batch = 0;
  EXPECT(bpt_layer_fwd(&bad, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == BPT_OK);
  EXPECT(bpt_layer_fwd_lse(&bad, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == BPT_OK);
  EXPECT(bpt::g_launches == 0);

  // attention backward: sizing, carving, validation
  bpt_attn_desc_t a = {2, 200, 256, 2, 1, BPT_BF16};      // d_head 128, Np 256
  const size_t anp = 256, sbytes = (size_t)2 * 2 * anp * 4;
  const size_t pbytes = (size_t)2 * anp * 256 * 2;
  const size_t aneed = bpt_attention_bwd_workspace_bytes(&a);
  EXPECT(aneed == 2 * sbytes + 3 * pbytes);
  const size_t in_b = (size_t)400 * 256 * 2;
  char* base = fake(4ull << 36);
  const void* in[5];
  for (int i = 0; i < 5; ++i) in[i] = base + (size_t)i * in_b;      // Q K V O dO back to back
  const float* alse = reinterpret_cast<const float*>(fake(5ull << 36));
  float* outs[3];
  for (int i = 0; i < 3; ++i) outs[i] = reinterpret_cast<float*>(fake((6ull + i) << 36));
  char* aws = fake(9ull << 36);
  EXPECT(bpt_attention_bwd(&a, in[0], in[1], in[2], in[3], in[4], alse, outs[0], outs[1], outs[2], aws,
                           aneed, nullptr) == BPT_OK);
  EXPECT(bpt::g_bwd_launches == 1 && bpt::g_bwd.d_head == 128 && bpt::g_bwd.seq_pad == 256);
  EXPECT(bpt::g_bwd.stat_d == reinterpret_cast<float*>(aws));
  EXPECT(bpt::g_bwd.stat_l2 == reinterpret_cast<float*>(aws + sbytes));
  EXPECT((char*)bpt::g_bwd.packed[0] == aws + 2 * sbytes);
  EXPECT((char*)bpt::g_bwd.packed[2] == aws + 2 * sbytes + 2 * pbytes);
  EXPECT(bpt::g_bwd.q == in[0] && bpt::g_bwd.dout == in[4] && bpt::g_bwd.dv == outs[2]);
  void* bev[5] = {fake(1), fake(2), fake(3), fake(4), fake(5)};
  EXPECT(bpt_attention_bwd_profiled(&a, in[0], in[1], in[2], in[3], in[4], alse, outs[0], outs[1], outs[2],
                                    aws, aneed, nullptr, bev) == BPT_OK);
  EXPECT(bpt::g_bwd.events == bev);
  bev[3] = nullptr;
  EXPECT(bpt_attention_bwd_profiled(&a, in[0], in[1], in[2], in[3], in[4], alse, outs[0], outs[1], outs[2],
                                    aws, aneed, nullptr, bev) == BPT_ERR_NULL);
  // inputs may coincide (Q = K, say)
  EXPECT(bpt_attention_bwd(&a, in[0], in[0], in[0], in[3], in[4], alse, outs[0], outs[1], outs[2], aws,
                           aneed, nullptr) == BPT_OK);
  bpt::g_bwd_launches = 0;
  EXPECT(bpt_attention_bwd(&a, in[0], in[1], in[2], in[3], in[4], alse, outs[0], outs[1], outs[2], aws,
                           aneed - 1, nullptr) == BPT_ERR_WORKSPACE);
  EXPECT(bpt_attention_bwd(&a, nullptr, in[1], in[2], in[3], in[4], alse, outs[0], outs[1], outs[2], aws,
                           aneed, nullptr) == BPT_ERR_NULL);
  EXPECT(bpt_attention_bwd(&a, in[0], in[1], in[2], in[3], in[4], nullptr, outs[0], outs[1], outs[2], aws,
                           aneed, nullptr) == BPT_ERR_NULL);
  EXPECT(bpt_attention_bwd(&a, in[0], in[1], in[2], in[3], in[4], alse, outs[0], outs[1], outs[2], nullptr,
                           aneed, nullptr) == BPT_ERR_NULL);
  EXPECT(bpt_attention_bwd(&a, in[0], in[1], in[2], in[3], in[4], alse + 1, outs[0], outs[1], outs[2], aws,
                           aneed, nullptr) == BPT_ERR_ALIGN);
  EXPECT(bpt_attention_bwd(&a, in[0], in[1], in[2], in[3], in[4], alse, outs[0] + 2, outs[1], outs[2], aws,
                           aneed, nullptr) == BPT_ERR_ALIGN);
  // dQ over the end of V; dK = dV; the workspace over dQ; lse inside dK
  EXPECT(bpt_attention_bwd(&a, in[0], in[1], in[2], in[3], in[4], alse,
                           reinterpret_cast<float*>(base + 2 * in_b + 4096), outs[1], outs[2], aws, aneed,
                           nullptr) == BPT_ERR_ALIAS);
  EXPECT(bpt_attention_bwd(&a, in[0], in[1], in[2], in[3], in[4], alse, outs[0], outs[1], outs[1], aws,
                           aneed, nullptr) == BPT_ERR_ALIAS);
  EXPECT(bpt_attention_bwd(&a, in[0], in[1], in[2], in[3], in[4], alse, outs[0], outs[1], outs[2],
                           reinterpret_cast<char*>(outs[0]) + 256, aneed, nullptr) == BPT_ERR_ALIAS);
  EXPECT(bpt_attention_bwd(&a, in[0], in[1], in[2], in[3], in[4], outs[1] + 64, outs[0], outs[1], outs[2],
                           aws, aneed, nullptr) == BPT_ERR_ALIAS);
  bpt_attn_desc_t ab = a;
  ab.dtype = BPT_F32;
  EXPECT(bpt_attention_bwd_workspace_bytes(&ab) == 0);
  EXPECT(bpt_attention_bwd(&ab, in[0], in[1], in[2], in[3], in[4], alse, outs[0], outs[1], outs[2], aws,
                           aneed, nullptr) == BPT_ERR_UNSUPPORTED);
  ab = a; ab.n_heads = 8;                                    // d_head 32
  EXPECT(bpt_attention_bwd(&ab, in[0], in[1], in[2], in[3], in[4], alse, outs[0], outs[1], outs[2], aws,
                           aneed, nullptr) == BPT_ERR_UNSUPPORTED);
  ab = a; ab.n_heads = 3;
  EXPECT(bpt_attention_bwd(&ab, in[0], in[1], in[2], in[3], in[4], alse, outs[0], outs[1], outs[2], aws,
                           aneed, nullptr) == BPT_ERR_SHAPE);
  ab = a; ab.causal = 2;
  EXPECT(bpt_attention_bwd(&ab, in[0], in[1], in[2], in[3], in[4], alse, outs[0], outs[1], outs[2], aws,
                           aneed, nullptr) == BPT_ERR_SHAPE);
  ab = a; ab.seq_len = -1;
  EXPECT(bpt_attention_bwd(&ab, in[0], in[1], in[2], in[3], in[4], alse, outs[0], outs[1], outs[2], aws,
                           aneed, nullptr) == BPT_ERR_SHAPE);
  EXPECT(bpt_attention_bwd(nullptr, in[0], in[1], in[2], in[3], in[4], alse, outs[0], outs[1], outs[2], aws,
                           aneed, nullptr) == BPT_ERR_NULL);
  ab = a; ab.batch = 1 << 20;                                 // 2^20 * 256 * 256 elements
  EXPECT(bpt_attention_bwd_workspace_bytes(&ab) == 0);
  EXPECT(bpt::g_bwd_launches == 0);
  ab = a; ab.seq_len = 0;
  EXPECT(bpt_attention_bwd_workspace_bytes(&ab) == 0);
  EXPECT(bpt_attention_bwd(&ab, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, nullptr, 0, nullptr) == BPT_OK);
  EXPECT(bpt::g_bwd_launches == 0);
  // ring attention step and merge: carving and validation
  {
    bpt_attn_desc_t r = {2, 200, 256, 2, 1, BPT_BF16};
    const size_t need = bpt_attention_fwd_workspace_bytes(&r);
    EXPECT(need == 3 * (size_t)2 * 256 * 256 * 2);
    char* fb = fake(10ull << 36);
    const size_t io = (size_t)400 * 256 * 2;
    float* lse_r = reinterpret_cast<float*>(fake(11ull << 36));
    char* wsr = fake(12ull << 36);
    EXPECT(bpt_attention_fwd(&r, fb, fb + io, fb + 2 * io, fb + 3 * io, lse_r, wsr, need, nullptr) == BPT_OK);
    EXPECT(bpt::g_fwd_launches == 1 && bpt::g_fwd.seq_pad == 256 && bpt::g_fwd.d_head == 128);
    EXPECT((char*)bpt::g_fwd.packed[2] == wsr + 2 * (need / 3) && bpt::g_fwd.o == fb + 3 * io);
    EXPECT(bpt_attention_fwd(&r, fb, fb + io, fb + 2 * io, fb + 3 * io, lse_r, wsr, need - 1, nullptr) ==
           BPT_ERR_WORKSPACE);
    EXPECT(bpt_attention_fwd(&r, fb, fb + io, fb + 2 * io, fb + 2 * io + 512, lse_r, wsr, need, nullptr) ==
           BPT_ERR_ALIAS);
    EXPECT(bpt_attention_fwd(&r, fb, fb + io, fb + 2 * io, fb + 3 * io, lse_r + 1, wsr, need, nullptr) ==
           BPT_ERR_ALIGN);
    EXPECT(bpt_attention_fwd(&r, nullptr, fb + io, fb + 2 * io, fb + 3 * io, lse_r, wsr, need, nullptr) ==
           BPT_ERR_NULL);
    float* oacc = reinterpret_cast<float*>(fake(13ull << 36));
    float* lacc = reinterpret_cast<float*>(fake(14ull << 36));
    EXPECT(bpt_attention_merge(&r, oacc, lacc, fb + 3 * io, lse_r, nullptr) == BPT_OK);
    EXPECT(bpt_attention_merge(&r, oacc, lse_r, fb + 3 * io, lse_r, nullptr) == BPT_ERR_ALIAS);
    EXPECT(bpt_attention_merge(&r, nullptr, lacc, fb + 3 * io, lse_r, nullptr) == BPT_ERR_NULL);
    EXPECT(bpt::g_merge_launches == 1);
  }
  // the host layer runs for real here: small fp32 layer, window mask, grouped heads
  {
    bpt_layer_desc_t hd{};
    hd.batch = 2; hd.seq_len = 37; hd.d_model = 32; hd.n_heads = 4; hd.d_ff = 64;
    hd.block_q = 16; hd.block_kv = 64; hd.causal = 1; hd.ln_eps = 1e-5f;
    hd.dtype = BPT_F32; hd.out_dtype = BPT_F32; hd.window = 9; hd.n_kv_heads = 2;
    const int rows = 2 * 37, dm = 32, dkv = 16, ff = 64;
    std::vector<float> x(rows * dm), z(rows * dm, -1.f), g(dm, 1.f), bz(dm, 0.f);
    std::vector<float> wq(dm * dm), wk(dkv * dm), wv(dkv * dm), wo(dm * dm), w1(ff * dm), w2(dm * ff);
    unsigned seed = 1;
    auto rnd = [&]() { seed = seed * 1664525u + 1013904223u; return ((seed >> 8) & 0xFFFF) / 65536.f - 0.5f; };
    for (auto* v : {&x, &wq, &wk, &wv, &wo, &w1, &w2})
      for (auto& e : *v) e = rnd();
    bpt_layer_weights_t hw = {g.data(), bz.data(), wq.data(), wk.data(), wv.data(), wo.data(),
                              g.data(), bz.data(), w1.data(), w2.data()};
    const size_t nb = bpt_layer_host_workspace_bytes(&hd, 3);
    EXPECT(nb > 0);
    std::vector<float> ws(nb / 4 + 1);
    EXPECT(bpt_layer_fwd_host(&hd, x.data(), &hw, z.data(), ws.data(), nb, 3) == BPT_OK);
    bool finite = true;
    for (float e : z) finite = finite && isfinite(e) && e != -1.f;
    EXPECT(finite);
    EXPECT(bpt_layer_fwd_host(&hd, x.data(), &hw, z.data(), ws.data(), nb - 4, 3) == BPT_ERR_WORKSPACE);
    EXPECT(bpt_layer_fwd_host(&hd, x.data(), &hw, x.data(), ws.data(), nb, 3) == BPT_ERR_ALIAS);
    EXPECT(bpt_layer_fwd_host(&hd, x.data(), nullptr, z.data(), ws.data(), nb, 3) == BPT_ERR_NULL);
    EXPECT(bpt_layer_host_workspace_bytes(&hd, 0) == 0);
  }
  // the layer backward: a valid call reaches its launcher with the carved workspace
  {
    bpt_layer_desc_t bd = d;
    bpt_layer_grads_t g;
    float** gp = reinterpret_cast<float**>(&g);
    for (int i = 0; i < 10; ++i) gp[i] = reinterpret_cast<float*>(fake((7ull << 36) + (uint64_t)i * (1ull << 30)));
    float* blse = reinterpret_cast<float*>(fake(3ull << 35));
    const float* dz = reinterpret_cast<const float*>(fake(9ull << 36));
    float* dx = reinterpret_cast<float*>(fake(10ull << 36));
    const size_t nb = bpt_layer_bwd_workspace_bytes(&bd);
    EXPECT(nb > 0);
    char* bws = fake(11ull << 36);
    EXPECT(bpt_layer_bwd(&bd, fake(0), &w[0], blse, dz, dx, &g, bws, nb, nullptr) == BPT_OK);
    EXPECT(bpt::g_layer_bwd_launches == 1);
    const bpt::LayerBwdLaunch& L = bpt::g_layer_bwd;
    EXPECT(L.rows == 400 && L.seq_pad == 256 && L.block_rows == 400 && L.wgrad_splits == 1);
    EXPECT(L.x1 == bws && L.lse == blse && L.dz == dz && L.dx == dx && L.g.w_2 == g.w_2);
    EXPECT((char*)L.ln_part + (size_t)L.ln_parts * 2 * 256 * 4 <= bws + nb);
    EXPECT(L.dq == L.y && L.dx1 == L.dy2 && L.da == L.dzb && L.dqkvb == L.q);
    EXPECT((char*)L.k == (char*)L.q + (size_t)400 * 256 * 2 && (char*)L.v == (char*)L.k + (size_t)400 * 256 * 2);
    EXPECT(L.dyt == L.dzt && L.dqt == L.y2t && L.dkt == L.attnt && L.rows_t == 400 && L.blk_ld == 400);
    EXPECT(bpt_layer_bwd(&bd, fake(0), &w[0], blse, dz, dx, &g, bws, nb - 1, nullptr) == BPT_ERR_WORKSPACE);
    EXPECT(bpt_layer_bwd(&bd, fake(0), &w[0], blse, dz, dx, nullptr, bws, nb, nullptr) == BPT_ERR_NULL);
    EXPECT(bpt_layer_bwd(&bd, fake(0), &w[0], blse, dz, reinterpret_cast<float*>(fake(9ull << 36) + 64), &g,
                         bws, nb, nullptr) == BPT_ERR_ALIAS);
    g.w_o = reinterpret_cast<float*>(fake(3ull << 36));   // over the forward's w_q
    EXPECT(bpt_layer_bwd(&bd, fake(0), &w[0], blse, dz, dx, &g, bws, nb, nullptr) == BPT_ERR_ALIAS);
    bd.precision = 1;
    EXPECT(bpt_layer_bwd_workspace_bytes(&bd) == 0);
    EXPECT(bpt::g_layer_bwd_launches == 1);
  }
  // the ring share: packing and the share reach their launchers with the carve-up
  {
    bpt_attn_desc_t ad{};
    ad.batch = 1; ad.seq_len = 300; ad.d_model = 256; ad.n_heads = 2; ad.causal = 1; ad.dtype = BPT_BF16;
    const size_t kvb = bpt_ring_kv_bytes(&ad);
    EXPECT(kvb == 2 * (size_t)384 * 256 * 2);
    EXPECT(bpt_ring_pack_kv(&ad, fake(0), fake(1ull << 30), fake(2ull << 30), kvb, nullptr) == BPT_OK);
    EXPECT(bpt_ring_pack_kv(&ad, fake(0), fake(1ull << 30), fake(2ull << 30), kvb - 1, nullptr) == BPT_ERR_WORKSPACE);
    EXPECT(bpt_ring_pack_kv(&ad, fake(0), fake(1ull << 30), fake(64), kvb, nullptr) == BPT_ERR_ALIAS);
    const void* shards[4] = {fake(3ull << 30), fake(4ull << 30), fake(5ull << 30), nullptr};
    const size_t wsb = bpt_ring_share_workspace_bytes(&ad);
    EXPECT(wsb > 0);
    float* rl = reinterpret_cast<float*>(fake(7ull << 30));
    EXPECT(bpt_ring_share_fwd(&ad, 4, 2, fake(0), shards, fake(6ull << 30), rl, fake(8ull << 30), wsb, nullptr) == BPT_OK);
    EXPECT(bpt::g_ring_share == 1 && bpt::g_ring.own == 2 && bpt::g_ring.n_shards == 4 && bpt::g_ring.seq_pad == 384);
    EXPECT((char*)bpt::g_ring.o_acc == fake(8ull << 30) + (size_t)384 * 256 * 2);
    // a shard the causal share reads may not be NULL; without the mask every one is read
    EXPECT(bpt_ring_share_fwd(&ad, 4, 3, fake(0), shards, fake(6ull << 30), rl, fake(8ull << 30), wsb, nullptr) == BPT_ERR_NULL);
    ad.causal = 0;
    EXPECT(bpt_ring_share_fwd(&ad, 4, 2, fake(0), shards, fake(6ull << 30), rl, fake(8ull << 30), wsb, nullptr) == BPT_ERR_NULL);
    ad.causal = 1;
    EXPECT(bpt_ring_share_fwd(&ad, 4, 4, fake(0), shards, fake(6ull << 30), rl, fake(8ull << 30), wsb, nullptr) == BPT_ERR_SHAPE);
    EXPECT(bpt_ring_share_fwd(&ad, 4, 2, fake(0), shards, fake(3ull << 30), rl, fake(8ull << 30), wsb, nullptr) == BPT_ERR_ALIAS);
    EXPECT(bpt_ring_share_fwd(&ad, 4, 2, fake(0), shards, fake(6ull << 30), rl, fake(8ull << 30), wsb - 1, nullptr) == BPT_ERR_WORKSPACE);
    ad.window = 8;
    EXPECT(bpt_ring_kv_bytes(&ad) == 0 && bpt_ring_share_workspace_bytes(&ad) == 0);
    EXPECT(bpt::g_ring_share == 1 && bpt::g_ring_pack == 1);
  }
  if (!g_fail) printf("ALL OK\n");
  return g_fail;
}
