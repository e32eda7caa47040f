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

// Rows of 1024 or more columns: a workgroup of TPR threads takes rows
// blockIdx.x, blockIdx.x + gridDim.x, ... The scatter row S stays zero between
// rows (each thread clears the positions it wrote once every thread has read
// S), the passes go through a second LDS row, and the next row's first
// 2 * TPR nonzeros are loaded while the current row is transformed and stored.
// Same arithmetic as materialize_kernel, in the same order.
template <int LOG_N, typename TOut>
__global__ __launch_bounds__(Fwht<LOG_N>::TPR) void materialize_rows_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ E,
    const float* __restrict__ c, int d_out, int nblk, float scale, TOut* __restrict__ dW,
    int accumulate) {
  using F = Fwht<LOG_N>;
  constexpr int TPR = F::TPR;
  __shared__ __align__(16) float S[F::LDS];
  __shared__ __align__(16) float Tb[F::LDS];
  const int u = threadIdx.x;
  for (int j = u; j < F::LDS / 4; j += TPR)
    reinterpret_cast<float4*>(S)[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  const int nv = d_out * nblk;
  int ja = -1, jb = -1, k0 = 0, k1 = 0;
  float ca = 0.f, cb = 0.f;
  auto fetch = [&](int vr) {
    const int row = vr / nblk;
    k0 = row_ptr[row];
    k1 = row_ptr[row + 1];
    const int ka = k0 + u, kb = ka + TPR;
    ja = ka < k1 ? E[2 * static_cast<int64_t>(ka) + 1] : -1;
    ca = ka < k1 ? c[ka] : 0.f;
    jb = kb < k1 ? E[2 * static_cast<int64_t>(kb) + 1] : -1;
    cb = kb < k1 ? c[kb] : 0.f;
  };
  // the nonzeros of block blk of the row (value v, or 0 to clear)
  auto put = [&](int blk, bool clear) {
    if (ja >= 0 && (ja >> LOG_N) == blk) S[F::pad(ja & (F::N - 1))] = clear ? 0.f : ca;
    if (jb >= 0 && (jb >> LOG_N) == blk) S[F::pad(jb & (F::N - 1))] = clear ? 0.f : cb;
    for (int k = k0 + u + 2 * TPR; k < k1; k += TPR) {
      const int j = E[2 * static_cast<int64_t>(k) + 1];
      if ((j >> LOG_N) == blk) S[F::pad(j & (F::N - 1))] = clear ? 0.f : c[k];
    }
  };
  int vrow = blockIdx.x;
  if (vrow < nv) fetch(vrow);
  __syncthreads();
  for (; vrow < nv; vrow += gridDim.x) {
    const int blk = vrow % nblk;
    put(blk, false);
    __syncthreads();   // S holds the row; the last row's reads of Tb are done
    float v[F::EPT];
    F::from_lds(S, v, 0, u);
    F::stages(v, 0);
#pragma unroll
    for (int p = 1; p < F::NP; ++p) {
      if (p > 1) __syncthreads();
      F::to_lds(Tb, v, p - 1, u);
      __syncthreads();
      if (p == 1) put(blk, true);   // every read of S is done
      F::from_lds(Tb, v, p, u);
      F::stages(v, p);
    }
    const int nx = vrow + gridDim.x;
    if (nx < nv) fetch(nx);
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
  if constexpr (LOG_N >= 10) {
    // up to 16 waves per CU on each of the 256 CUs, as far as LDS allows;
    // each workgroup takes every gridDim.x-th row
    constexpr int kLds = 2 * Fwht<LOG_N>::LDS * static_cast<int>(sizeof(float));
    constexpr int kByLds = 160 * 1024 / kLds;
    constexpr int kByWaves = 1024 / Fwht<LOG_N>::TPR;
    constexpr int kPerCu = kByLds < kByWaves ? (kByLds < 1 ? 1 : kByLds) : kByWaves;
    const int nv = d_out * nblk;
    const int grid = nv < 256 * kPerCu ? nv : 256 * kPerCu;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((materialize_rows_kernel<LOG_N, TOut>), dim3(grid),
                       dim3(Fwht<LOG_N>::TPR), 0, s, row_ptr, E, c, d_out, nblk, scale,
                       static_cast<TOut*>(dW), acc);
    return hipGetLastError();
  }
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
