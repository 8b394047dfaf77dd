// Device-side building blocks shared by the BPT kernels (gfx950 / CDNA4).
//
// Matrix-core convention used everywhere: one 32x32 output tile per
// v_mfma_f32_32x32x16_bf16 (bf16 operands) or per eight v_mfma_f32_32x32x2_f32
// (fp32 operands), for a k-step of 16.
//   * A operand ("rows"), B operand ("cols"): lane l serves row/col (l % 32) and
//     holds eight consecutive k values k = 8 * (l / 32) + [0, 8) of the k-step.
//     (Only the agreement of A and B matters for the product; both use this map.)
//   * C/D: lane l holds column (l % 32); register i holds row
//     8 * (i / 4) + 4 * (l / 32) + (i % 4).
// Row permutation pi: when the A operand's row rho is fed from source row
// pi(rho) (pi swaps bits 2 and 3 of rho), lane half hf holds, in registers
// 0..7, source rows 8*hf + 0..7 and in registers 8..15 source rows 16 + 8*hf + 0..7.
// Every kernel uses this so that each lane owns 8 consecutive output features:
// 16-byte stores, and C fragments that feed the next product's B operand
// without a shuffle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bpt {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// pi: swap bits 2 and 3 of a row index inside its 32-row group.
__device__ __host__ constexpr int pi_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Source row held by register i (0..15) of a C fragment in lane half hf when
// the A operand rows were fed through pi: 8*hf + i for i < 8, 16 + 8*hf + (i-8).
__device__ constexpr int c_row_pi(int i, int hf) { return (i & 8) * 2 + 8 * hf + (i & 7); }

// LDS swizzle of 8-element chunks: keeps any 8 consecutive rows, in natural or
// pi order, on distinct 16-byte bank groups.
__device__ constexpr int swz(int row) {
  return (row & 3) | ((((row >> 2) ^ (row >> 3)) & 1) << 2);
}

// ---------------------------------------------------------------------------
// Compute-type traits: a fragment is 8 k-consecutive operand values.
// ---------------------------------------------------------------------------
template <typename T> struct Op;

template <> struct Op<bf16> {
  typedef bf16x8 frag;
  static constexpr int kBytes = 2;
  __device__ static inline void mma(f32x16& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
  __device__ static inline frag from_f32(const float* v) {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (bf16)v[i];
    return f;
  }
};

template <> struct Op<float> {
  typedef f32x8 frag;
  static constexpr int kBytes = 4;
  __device__ static inline void mma(f32x16& acc, const frag& a, const frag& b) {
#pragma unroll
    for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], b[t], acc, 0, 0, 0);
  }
  __device__ static inline frag from_f32(const float* v) {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = v[i];
    return f;
  }
};

// ---------------------------------------------------------------------------
// 8-element vector loads/stores of any element type, converting to/from fp32.
// ---------------------------------------------------------------------------
__device__ inline void load8_f32(const bf16* p, float* v) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ inline void load8_f32(const float* p, float* v) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ inline void store8_f32(bf16* p, const float* v) {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (bf16)v[i];
  *reinterpret_cast<bf16x8*>(p) = f;
}
__device__ inline void store8_f32(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Raw 8-element chunk copy (global or LDS), for staging operands unchanged.
template <typename T> struct Chunk;
template <> struct Chunk<bf16> {
  typedef uint4 type;
};
template <> struct Chunk<float> {
  struct type { uint4 a, b; };
};
template <typename T>
__device__ inline typename Chunk<T>::type ld_chunk(const T* p) {
  return *reinterpret_cast<const typename Chunk<T>::type*>(p);
}
template <typename T>
__device__ inline void st_chunk(T* p, const typename Chunk<T>::type& c) {
  *reinterpret_cast<typename Chunk<T>::type*>(p) = c;
}
template <typename T>
__device__ inline typename Chunk<T>::type zero_chunk() {
  typename Chunk<T>::type c;
  __builtin_memset(&c, 0, sizeof(c));
  return c;
}
template <typename T>
__device__ inline typename Op<T>::frag ld_frag(const T* p) {
  return *reinterpret_cast<const typename Op<T>::frag*>(p);
}

// ---------------------------------------------------------------------------
// Packed fragments. A matrix-core operand fragment (a 32-row tile x one 16-wide
// k-step, 8 values per lane) stored as PCS = sizeof(T)/2 pieces of 64 lanes x
// 16 bytes: element e of lane l sits at piece e / EPP, position l * EPP + e % EPP
// (EPP = 16 / sizeof(T) elements per piece). One piece is 1 KB of contiguous
// memory, so a 64-lane load of it touches 8 whole cache lines.
// ---------------------------------------------------------------------------
constexpr int kFragElems = 512;

template <typename T>
__device__ __host__ constexpr int frag_pieces() { return (int)sizeof(T) / 2; }

template <typename T>
__device__ __host__ constexpr int packed_index(int lane, int e) {
  return (e / (16 / (int)sizeof(T))) * 64 * (16 / (int)sizeof(T)) + lane * (16 / (int)sizeof(T)) +
         e % (16 / (int)sizeof(T));
}

// Load lane's fragment from a packed fragment at p (global or LDS).
__device__ inline bf16x8 ld_packed(const bf16* p, int lane) {
  return *reinterpret_cast<const bf16x8*>(p + lane * 8);
}
__device__ inline f32x8 ld_packed(const float* p, int lane) {
  const float4 a = *reinterpret_cast<const float4*>(p + lane * 4);
  const float4 b = *reinterpret_cast<const float4*>(p + 256 + lane * 4);
  return f32x8{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}
// Store 8 values of lane's slot in a packed fragment at p.
__device__ inline void st_packed(bf16* p, int lane, const float* v) { store8_f32(p + lane * 8, v); }
__device__ inline void st_packed(float* p, int lane, const float* v) {
  *reinterpret_cast<float4*>(p + lane * 4) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 256 + lane * 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ inline void st_packed_chunk(bf16* p, int lane, const Chunk<bf16>::type& c) {
  st_chunk(p + lane * 8, c);
}
__device__ inline void st_packed_chunk(float* p, int lane, const Chunk<float>::type& c) {
  *reinterpret_cast<uint4*>(p + lane * 4) = c.a;
  *reinterpret_cast<uint4*>(p + 256 + lane * 4) = c.b;
}

// LDS pointer for the direct global -> LDS copy instruction.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
// Copy 16 bytes per lane from global memory (per-lane address src) into LDS at
// dst + 16 * lane (dst wave-uniform). Completion is tracked by the vector memory
// counter of the issuing wave.
__device__ inline void dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 16, 0, 0);
}
// Wait until all of this wave's vector-memory operations (including LDS copies) are done.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ inline float bf16_round(float x) { return (float)(bf16)x; }

// exp2 on the hardware transcendental unit (v_exp_f32).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// GELU, tanh form: 0.5 u (1 + tanh(z)) = u / (1 + exp(-2 z)),
// z = sqrt(2/pi) (u + 0.044715 u^3). exp(-2z) = 2^(-2 z log2 e).
__device__ inline float gelu_tanh(float u) {
  const float k = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float z = u * (1.0f + 0.044715f * u * u);
  const float e = fast_exp2(k * z);
  return u * __builtin_amdgcn_rcpf(1.0f + e);   // e = inf gives rcp = 0 and h = -0
}

}  // namespace bpt
