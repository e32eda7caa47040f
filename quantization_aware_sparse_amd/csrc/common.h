// Shared device helpers for the WHA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qwha {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 I/O
// bf16 values travel as raw uint16 bit patterns; math is fp32.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest, ties to even (inputs are finite by precondition).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t lsb = (u >> 16) & 1u;
  return static_cast<uint16_t>((u + 0x7FFFu + lsb) >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
  }
  static __device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) {
    p[i] = f32_to_bf16(v);
  }
};

// Load 16 consecutive elements (16-byte aligned) into fp32/fp64 registers.
template <typename Acc>
__device__ __forceinline__ void load16(const float* p, Acc* v) {
  const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float4 f = q[i];
    v[4 * i + 0] = static_cast<Acc>(f.x);
    v[4 * i + 1] = static_cast<Acc>(f.y);
    v[4 * i + 2] = static_cast<Acc>(f.z);
    v[4 * i + 3] = static_cast<Acc>(f.w);
  }
}
template <typename Acc>
__device__ __forceinline__ void load16(const uint16_t* p, Acc* v) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint4 u = q[i];
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * i + 2 * k + 0] = static_cast<Acc>(__uint_as_float(w[k] << 16));
      v[8 * i + 2 * k + 1] = static_cast<Acc>(__uint_as_float(w[k] & 0xFFFF0000u));
    }
  }
}

// ------------------------------------------------------- wave reductions
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Inclusive prefix sum across the wave (lane order).
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ------------------------------------------------------- random draws
// Output n (n = 0, 1, ...) of the SplitMix64 generator seeded with `seed`
// (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
// OOPSLA 2014): the state after n+1 steps is seed + (n+1) * 0x9E3779B97F4A7C15
// (mod 2^64), passed through the generator's 64-bit mix. Counter-based: any
// draw is computed directly from n.
__device__ __forceinline__ unsigned long long splitmix64(unsigned long long seed,
                                                         unsigned long long n) {
  unsigned long long z = seed + (n + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace qwha
