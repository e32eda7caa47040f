// Row-wise fast Walsh-Hadamard transform over HBM (the standalone FWHT):
// out[r][:] = scale * in[r][:] H  (+ out[r][:] when accumulating).
// Used for z = FWHT(x)/n in the forward pass and dx = alpha FWHT(dz)/n in
// the backward pass; H is the +-1 Sylvester kernel of the WHA adapter
// (QWHA notes, papernotes.org, 关键设计 1).
//
// Traffic per row: n*(in bytes + out bytes), streamed once; the transform
// itself is log2(n) add/sub per element in registers plus ceil(log2 n / 4)-1
// LDS round trips, so the kernel is HBM-bound.
#include "fwht_core.h"
#include "launch.h"

namespace qwha {

template <int LOG_N>
struct FwhtLaunch {
  using F = Fwht<LOG_N>;
  static constexpr int BLOCK = F::TPR > 256 ? F::TPR : 256;
  static constexpr int RPW = BLOCK / F::TPR;     // rows per workgroup
};

template <int LOG_N, typename TIn, typename TOut>
__global__ __launch_bounds__(FwhtLaunch<LOG_N>::BLOCK) void fwht_rows_kernel(
    const TIn* __restrict__ in, TOut* __restrict__ out, int64_t rows, float scale,
    int accumulate) {
  using F = Fwht<LOG_N>;
  constexpr int RPW = FwhtLaunch<LOG_N>::RPW;
  __shared__ float lds_all[RPW * F::LDS];
  const int slot = threadIdx.x / F::TPR;
  const int u = threadIdx.x % F::TPR;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPW + slot;
  const bool live = row < rows;
  float* lds = lds_all + slot * F::LDS;

  float v[F::EPT];
  if (live) {
    const TIn* src = in + row * F::N + static_cast<int64_t>(u) * F::EPT;
    if constexpr (F::EPT == 16) {
      load16(src, v);
    } else {
#pragma unroll
      for (int r = 0; r < F::EPT; ++r) v[r] = Elem<TIn>::ld(src, r);
    }
  } else {
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) v[r] = 0.f;
  }
  F::run(v, lds, u);
  if (live) {
    TOut* dst = out + row * F::N;
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) {
      const int j = F::out_index(u, r);
      float val = v[r] * scale;
      if (accumulate) val += Elem<TOut>::ld(dst, j);
      Elem<TOut>::st(dst, j, val);
    }
  }
}

template <int LOG_N, typename TIn, typename TOut>
static hipError_t launch_t(const void* in, void* out, int64_t rows, float scale, int acc,
                           hipStream_t s) {
  constexpr int RPW = FwhtLaunch<LOG_N>::RPW;
  const int64_t blocks = (rows + RPW - 1) / RPW;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((fwht_rows_kernel<LOG_N, TIn, TOut>), dim3(static_cast<unsigned>(blocks)),
                     dim3(FwhtLaunch<LOG_N>::BLOCK), 0, s, static_cast<const TIn*>(in),
                     static_cast<TOut*>(out), rows, scale, acc);
  return hipGetLastError();
}

template <int LOG_N>
static hipError_t launch_n(const void* in, Dt idt, void* out, Dt odt, int64_t rows, float scale,
                           int acc, hipStream_t s) {
  if (idt == Dt::F32 && odt == Dt::F32)
    return launch_t<LOG_N, float, float>(in, out, rows, scale, acc, s);
  if (idt == Dt::F32 && odt == Dt::BF16)
    return launch_t<LOG_N, float, uint16_t>(in, out, rows, scale, acc, s);
  if (idt == Dt::BF16 && odt == Dt::F32)
    return launch_t<LOG_N, uint16_t, float>(in, out, rows, scale, acc, s);
  return launch_t<LOG_N, uint16_t, uint16_t>(in, out, rows, scale, acc, s);
}

hipError_t launch_fwht(const void* in, Dt in_dt, void* out, Dt out_dt, int64_t rows, int log_n,
                       float scale, int accumulate, hipStream_t s) {
  switch (log_n) {
#define QWHA_CASE(L) \
  case L:            \
    return launch_n<L>(in, in_dt, out, out_dt, rows, scale, accumulate, s);
    QWHA_CASE(1) QWHA_CASE(2) QWHA_CASE(3) QWHA_CASE(4) QWHA_CASE(5) QWHA_CASE(6) QWHA_CASE(7)
    QWHA_CASE(8) QWHA_CASE(9) QWHA_CASE(10) QWHA_CASE(11) QWHA_CASE(12) QWHA_CASE(13)
    QWHA_CASE(14)
#undef QWHA_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace qwha
