// Materialisation of the adapter weight: dW = alpha * F H^-1 = (alpha/n) F H
// with F = Scatter(c, E) (QWHA notes, papernotes.org, 方法详解 › 整体框架;
// gist.science summary §2.1). Row i of F is scattered into an LDS row and
// transformed in place; F is never dense in HBM. Under the block-diagonal
// transform (nblk Sylvester blocks per row) each block of a row is its own
// LDS row, filled with the row's nonzeros in that block. HBM traffic per row: the
// row's nonzeros in, n outputs out (plus n in when accumulating).
#include "fwht_core.h"
#include "launch.h"

namespace qwha {

template <int LOG_N>
struct MatCfg {
  using F = Fwht<LOG_N>;
  static constexpr int BLOCK = F::TPR > 256 ? F::TPR : 256;
  static constexpr int RPW = BLOCK / F::TPR;
};

template <int LOG_N, typename TOut>
__global__ __launch_bounds__(MatCfg<LOG_N>::BLOCK) void materialize_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ E,
    const float* __restrict__ c, int d_out, int nblk, float scale, TOut* __restrict__ dW,
    int accumulate) {
  using F = Fwht<LOG_N>;
  constexpr int RPW = MatCfg<LOG_N>::RPW;
  __shared__ __align__(16) float lds_all[RPW * F::LDS];
  const int slot = threadIdx.x / F::TPR;
  const int u = threadIdx.x % F::TPR;
  // virtual row r of the [d_out * nblk][N] view: block blk of row i
  const int vrow = blockIdx.x * RPW + slot;
  const bool live = vrow < d_out * nblk;
  const int row = vrow / nblk, blk = vrow - row * nblk;
  float* lds = lds_all + slot * F::LDS;

  if constexpr (F::LDS % 4 == 0) {   // 16-byte stores (the row offset is a multiple of 16 B)
    float4* z4 = reinterpret_cast<float4*>(lds);
    for (int j = u; j < F::LDS / 4; j += F::TPR) z4[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
    for (int j = u; j < F::LDS; j += F::TPR) lds[j] = 0.f;
  }
  __syncthreads();
  if (live) {
    const int k1 = row_ptr[row + 1];
    for (int k = row_ptr[row] + u; k < k1; k += F::TPR) {
      const int j = E[2 * static_cast<int64_t>(k) + 1];
      if ((j >> LOG_N) == blk) lds[F::pad(j & (F::N - 1))] = c[k];
    }
  }
  __syncthreads();
  float v[F::EPT];
#pragma unroll
  for (int r = 0; r < F::EPT; ++r) v[r] = lds[F::pad(u * F::EPT + r)];
  F::run(v, lds, u);
  if (live) {
    TOut* dst = dW + static_cast<int64_t>(vrow) * F::N;
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) {
      const int j = F::out_index(u, r);
      float val = v[r] * scale;
      if (accumulate) val += Elem<TOut>::ld(dst, j);
      Elem<TOut>::st(dst, j, val);
    }
  }
}

template <int LOG_N, typename TOut>
static hipError_t mat_t(const int32_t* row_ptr, const int32_t* E, const float* c, int d_out,
                        int nblk, float scale, void* dW, int acc, hipStream_t s) {
  constexpr int RPW = MatCfg<LOG_N>::RPW;
  const int blocks = (d_out * nblk + RPW - 1) / RPW;
  hipLaunchKernelGGL((materialize_kernel<LOG_N, TOut>), dim3(blocks), dim3(MatCfg<LOG_N>::BLOCK), 0,
                     s, row_ptr, E, c, d_out, nblk, scale, static_cast<TOut*>(dW), acc);
  return hipGetLastError();
}

hipError_t launch_materialize(const int32_t* row_ptr, const int32_t* E, const float* c, int d_out,
                              int log_n, float alpha, Dt out_dt, void* dW, int accumulate,
                              hipStream_t s, int nblk) {
  const float scale = alpha / static_cast<float>(1 << log_n);
  switch (log_n) {
#define QWHA_CASE(L)                                                             \
  case L:                                                                        \
    return out_dt == Dt::F32                                                     \
               ? mat_t<L, float>(row_ptr, E, c, d_out, nblk, scale, dW, accumulate, s) \
               : mat_t<L, uint16_t>(row_ptr, E, c, d_out, nblk, scale, dW, accumulate, s);
    QWHA_CASE(1) QWHA_CASE(2) QWHA_CASE(3) QWHA_CASE(4) QWHA_CASE(5) QWHA_CASE(6) QWHA_CASE(7)
    QWHA_CASE(8) QWHA_CASE(9) QWHA_CASE(10) QWHA_CASE(11) QWHA_CASE(12) QWHA_CASE(13)
    QWHA_CASE(14)
#undef QWHA_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace qwha
