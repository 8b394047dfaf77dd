// Host-side launch helpers shared by the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdio.h>

#include "bpt_internal.h"

namespace bpt {

inline void set_err(char* err, size_t n, const char* fmt, const char* a = "", int b = 0) {
  if (err && n) snprintf(err, n, fmt, a, b);
}

// Opt a kernel into more than 64 KB of dynamic LDS (gfx950 has 160 KB per CU).
template <typename K>
int set_smem(K kernel, size_t bytes, char* err, size_t errlen) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) {
    set_err(err, errlen, "hipFuncSetAttribute: %s", hipGetErrorString(e));
    return 1;
  }
  return 0;
}

inline int check_launch(const char* what, char* err, size_t errlen) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    if (err && errlen) snprintf(err, errlen, "%s launch: %s", what, hipGetErrorString(e));
    return 1;
  }
  return 0;
}

// Per-kernel launchers (one translation unit each).
int launch_ln_qkv(const LayerLaunch& L, hipStream_t s, char* err, size_t n, int phase);
int launch_attention(const LayerLaunch& L, hipStream_t s, char* err, size_t n);
int launch_ffn(const LayerLaunch& L, hipStream_t s, char* err, size_t n);
int launch_pack(const LayerLaunch& L, hipStream_t s, char* err, size_t n);
int launch_qkv(const LayerLaunch& L, hipStream_t s, char* err, size_t n);
int launch_ffn_staged(const LayerLaunch& L, hipStream_t s, char* err, size_t n);
int launch_ffn_coop(const LayerLaunch& L, hipStream_t s, char* err, size_t n);
int launch_ln_rows(const LayerLaunch& L, const void* y, int rows, hipStream_t s, char* err, size_t n);

}  // namespace bpt
