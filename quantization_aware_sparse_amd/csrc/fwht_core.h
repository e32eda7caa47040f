// Fast Walsh-Hadamard transform of one row, Sylvester (natural) order:
//   out[j] = sum_m in[m] * (-1)^popcount(m & j),  n = 2^LOG_N <= 16384.
// The transform kernel H of the WHA adapter (QWHA notes, papernotes.org,
// 方法详解 › 关键设计 1; gist.science summary §2.1): a +-1 matrix applied with
// additions and subtractions only.
//
// Layout: each thread holds EPT = 16 elements in registers (EPT = n when
// n < 16). The LOG_N index bits are processed in passes of 4: in pass p the
// 4 register bits are index bits [lo(p), lo(p)+4) and the radix-2 stages on
// those bits run in registers; between passes the row goes through LDS
// (padded by one word every 16 to spread banks). Pass p < last covers bits
// [4p, 4p+4); the last pass takes the top 4 bits [LOG_N-4, LOG_N) and only
// runs the stages not done before, so that thread u holds elements
// u + r*(n/16): consecutive lanes touch consecutive addresses on the final
// store. H is a Kronecker product of 2x2 factors, one per index bit, so the
// order of the stages does not change the result.
#pragma once

#include "common.h"

namespace qwha {

template <int LOG_N>
struct Fwht {
  static constexpr int N = 1 << LOG_N;
  static constexpr int EPT = LOG_N >= 4 ? 16 : N;        // elements per thread
  static constexpr int TPR = N / EPT;                    // threads per row
  static constexpr int NP = LOG_N >= 4 ? (LOG_N + 3) / 4 : 1;   // passes
  static constexpr int LDS = N + (N >> 4);               // padded row length

  static __host__ __device__ constexpr int lo(int p) {
    return LOG_N < 4 ? 0 : (p == NP - 1 ? LOG_N - 4 : 4 * p);
  }
  // first register bit whose stage runs in pass p
  static __host__ __device__ constexpr int first_stage(int p) {
    return LOG_N < 4 ? 0 : 4 * p - lo(p);
  }
  static __host__ __device__ constexpr int nstage_bits() { return LOG_N < 4 ? LOG_N : 4; }

  // index of register r of thread u in pass p
  static __device__ __forceinline__ int thread_part(int p, int u) {
    if (LOG_N < 4) return 0;
    const int l = lo(p);
    return (u & ((1 << l) - 1)) | ((u >> l) << (l + 4));
  }
  static __host__ __device__ constexpr int reg_part(int p, int r) { return r << lo(p); }
  static __device__ __forceinline__ int pad(int j) { return j + (j >> 4); }

  template <typename Acc>
  static __device__ __forceinline__ void stages(Acc* v, int p) {
#pragma unroll
    for (int b = 0; b < nstage_bits(); ++b) {
      if (b < first_stage(p)) continue;
      const int h = 1 << b;
#pragma unroll
      for (int r = 0; r < EPT; ++r) {
        if (r & h) continue;
        Acc a = v[r], c = v[r + h];
        v[r] = a + c;
        v[r + h] = a - c;
      }
    }
  }

  template <typename Acc>
  static __device__ __forceinline__ void to_lds(Acc* lds, const Acc* v, int p, int u) {
    const int tp = thread_part(p, u);
#pragma unroll
    for (int r = 0; r < EPT; ++r) lds[pad(tp + reg_part(p, r))] = v[r];
  }
  template <typename Acc>
  static __device__ __forceinline__ void from_lds(const Acc* lds, Acc* v, int p, int u) {
    const int tp = thread_part(p, u);
#pragma unroll
    for (int r = 0; r < EPT; ++r) v[r] = lds[pad(tp + reg_part(p, r))];
  }

  // Runs all passes. On entry v holds the pass-0 layout (thread u owns the
  // EPT consecutive elements starting at u*EPT); on exit the last-pass
  // layout (element u + r*TPR... i.e. thread_part(NP-1,u) + reg_part(NP-1,r)).
  // All threads of the block must call this (it contains __syncthreads()).
  // Threads with active == false only take part in the barriers.
  template <typename Acc>
  static __device__ __forceinline__ void run(Acc* v, Acc* lds, int u, bool active = true) {
    stages(v, 0);
#pragma unroll
    for (int p = 1; p < NP; ++p) {
      __syncthreads();          // earlier readers of lds are done
      if (active) to_lds(lds, v, p - 1, u);
      __syncthreads();
      if (active) from_lds(lds, v, p, u);
      stages(v, p);
    }
  }

  // Element index held in register r by thread u after run().
  static __device__ __forceinline__ int out_index(int u, int r) {
    return thread_part(NP - 1, u) + reg_part(NP - 1, r);
  }
};

}  // namespace qwha
