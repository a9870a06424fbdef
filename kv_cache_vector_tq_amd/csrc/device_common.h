// Small device helpers shared by the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/tq.h"

namespace tq {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline float half_bits_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ inline float bf16_bits_to_float(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Element idx of a buffer holding F16 (0), BF16 (1) or F32 (2) values.
__device__ inline float load_any(const void* p, int64_t idx, int dtype) {
  if (dtype == TQ_DTYPE_F32) return static_cast<const float*>(p)[idx];
  const uint16_t v = static_cast<const uint16_t*>(p)[idx];
  return dtype == TQ_DTYPE_F16 ? half_bits_to_float(v) : bf16_bits_to_float(v);
}

// Work-group barrier for data exchanged through LDS only.  __syncthreads is
// a release/acquire fence on all memory and waits for every global load in
// flight; this one orders LDS alone, so loads issued early keep flying across
// it.  Only for phases that share no global memory between threads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Bits [pos, pos+n) of a little-endian bit string held in 32-bit words
// (n <= 8; pos and n are compile-time after unrolling).
template <int N>
__device__ inline uint32_t bits_at(const uint32_t* w, int pos) {
  const int wi = pos >> 5, bi = pos & 31;
  uint32_t v = w[wi] >> bi;
  if (bi + N > 32) v |= w[wi + 1] << (32 - bi);
  return v & ((1u << N) - 1u);
}

}  // namespace tq
