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
// Scans and sums go through DPP (register moves between lanes of a row of
// 16, or from the last lane of a row to the rows after it), not through
// LDS permutes: row_shr 1, 2, 4, 8 scan each row; row_bcast:15 into rows 1
// and 3 and row_bcast:31 into rows 2 and 3 carry the rows' totals. Lanes a
// shift moves in from outside their row read 0. The active lanes must be a
// prefix of the wave (a whole wave, or the first k lanes of a workgroup's
// last wave); sums are read from the last active lane.
__device__ __forceinline__ int last_active_lane() {
  return 63 - __builtin_clzll(__builtin_amdgcn_read_exec());
}
template <int CTRL, int ROW_MASK = 0xF, bool BOUND = true>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, BOUND);
}
template <int CTRL, int ROW_MASK = 0xF, bool BOUND = true>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = dpp_i32<CTRL, ROW_MASK, BOUND>(static_cast<int>(b));
  const int hi = dpp_i32<CTRL, ROW_MASK, BOUND>(static_cast<int>(b >> 32));
  return __longlong_as_double((static_cast<long long>(hi) << 32) |
                              static_cast<unsigned int>(lo));
}

// Inclusive prefix sum across the wave (lane order).
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  v += dpp_i32<0x111>(v);
  v += dpp_i32<0x112>(v);
  v += dpp_i32<0x114>(v);
  v += dpp_i32<0x118>(v);
  v += dpp_i32<0x142, 0xA, false>(v);
  v += dpp_i32<0x143, 0xC, false>(v);
  return v;
}

// Sum over the wave, the same value in every lane.
__device__ __forceinline__ int wave_sum_i32(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan_i32(v), last_active_lane());
}

// fp64 sum over the wave (the scan's order: within rows of 16, then rows),
// the same value in every lane.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0x111>(v);
  v += dpp_f64<0x112>(v);
  v += dpp_f64<0x114>(v);
  v += dpp_f64<0x118>(v);
  v += dpp_f64<0x142, 0xA, false>(v);
  v += dpp_f64<0x143, 0xC, false>(v);
  const long long b = __double_as_longlong(v);
  const int last = last_active_lane();
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), last);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), last);
  return __longlong_as_double((static_cast<long long>(hi) << 32) |
                              static_cast<unsigned int>(lo));
}

// int64 sum over the wave, the same value in every lane.
template <int CTRL, int ROW_MASK = 0xF, bool BOUND = true>
__device__ __forceinline__ long long dpp_i64(long long v) {
  const int lo = dpp_i32<CTRL, ROW_MASK, BOUND>(static_cast<int>(v));
  const int hi = dpp_i32<CTRL, ROW_MASK, BOUND>(static_cast<int>(v >> 32));
  return (static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo);
}
__device__ __forceinline__ long long wave_sum_i64(long long v) {
  v += dpp_i64<0x111>(v);
  v += dpp_i64<0x112>(v);
  v += dpp_i64<0x114>(v);
  v += dpp_i64<0x118>(v);
  v += dpp_i64<0x142, 0xA, false>(v);
  v += dpp_i64<0x143, 0xC, false>(v);
  const int last = last_active_lane();
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(v), last);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(v >> 32), last);
  return (static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo);
}

// Largest unsigned 32-bit value over the wave, the same in every lane.
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
  auto mx = [](unsigned a, int b) { return a > static_cast<unsigned>(b) ? a : static_cast<unsigned>(b); };
  v = mx(v, dpp_i32<0x111>(static_cast<int>(v)));
  v = mx(v, dpp_i32<0x112>(static_cast<int>(v)));
  v = mx(v, dpp_i32<0x114>(static_cast<int>(v)));
  v = mx(v, dpp_i32<0x118>(static_cast<int>(v)));
  v = mx(v, dpp_i32<0x142, 0xA, false>(static_cast<int>(v)));
  v = mx(v, dpp_i32<0x143, 0xC, false>(static_cast<int>(v)));
  return static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(v), last_active_lane()));
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
