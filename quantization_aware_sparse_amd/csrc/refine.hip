// Value Refinement with a calibration Hessian (QWHA notes, papernotes.org,
// 关键设计 3 and 损失函数 / 训练策略; gist.science summary §2.2).
//
// Per output channel i the refined values on the chosen columns S = E_i
// solve min_x ||v - x B'||^2 with v = dW_Q[i,:] R, B = H^-1 R and
// R R^T = Hs = XX^T (activations X; here token-major, so Hs = X^T X). Its
// normal equations are
//   x G[S,S] = Q[i,S],   G = H Hs H / n^2,   Q = dW_Q Hs H / n,
// and AdaAlloc allocates by the activation error magnitude
// ||dW_Q[i,:] R|| = sqrt(dW_Q[i,:] Hs dW_Q[i,:]^T).
//
// Kernels (all fp64):
//   gemm64_kernel      dense products on the fp64 matrix cores
//                      (v_mfma_f64_16x16x4): Hs = X^T X (symmetric: 64x64
//                      tiles on and below the diagonal, mirrored) and
//                      M = dW_Q Hs (128x128 tiles);
//   calib_rows_kernel  per row of M: w_i and Q[i,:] = (M + delta dW_Q)[i,:] H/n;
//   fwht64_rows_kernel + transpose64_kernel: G = H (H Hs)^T / n^2 (Hs is
//                      symmetric), plus delta/n on the diagonal;
//   refine_kernel      per row: gather G[S,S] with the right-hand side as an
//                      extra last row, blocked Cholesky of that augmented
//                      matrix (its last row becomes L^-1 rhs), then the
//                      back substitution; c = fp32(x).
#include "fwht_core.h"
#include "launch.h"

namespace qwha {

namespace {

typedef double v4d __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ GEMM
constexpr int kGK = 16;    // K per staged chunk

__device__ __forceinline__ double to_f64(float v) { return static_cast<double>(v); }
__device__ __forceinline__ double to_f64(uint16_t v) { return static_cast<double>(bf16_to_f32(v)); }
__device__ __forceinline__ double to_f64(double v) { return v; }

// EPT (4 or 8) consecutive elements at p, 16-byte vector loads (p aligned
// to EPT elements), times `mask` (0 or 1).
template <typename T, int EPT>
__device__ __forceinline__ void load_vec(const T* p, double mask, double* v) {
  if constexpr (sizeof(T) == 4) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < EPT / 4; ++i) {
      const float4 f = q[i];
      v[4 * i] = f.x * mask;
      v[4 * i + 1] = f.y * mask;
      v[4 * i + 2] = f.z * mask;
      v[4 * i + 3] = f.w * mask;
    }
  } else if constexpr (sizeof(T) == 2) {
    uint32_t w[EPT / 2];
    if constexpr (EPT == 8) {
      const uint4 u = *reinterpret_cast<const uint4*>(p);
      w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      w[0] = u.x; w[1] = u.y;
    }
#pragma unroll
    for (int i = 0; i < EPT / 2; ++i) {
      v[2 * i] = static_cast<double>(__uint_as_float(w[i] << 16)) * mask;
      v[2 * i + 1] = static_cast<double>(__uint_as_float(w[i] & 0xFFFF0000u)) * mask;
    }
  } else {
    const double2* q = reinterpret_cast<const double2*>(p);
#pragma unroll
    for (int i = 0; i < EPT / 2; ++i) {
      const double2 d = q[i];
      v[2 * i] = d.x * mask;
      v[2 * i + 1] = d.y * mask;
    }
  }
}

// EPT consecutive elements at p, `valid` of them in range (<= 0: none).
template <typename T, int EPT>
__device__ __forceinline__ void load_guarded(const T* p, int valid, double* v) {
#pragma unroll
  for (int r = 0; r < EPT; ++r) v[r] = r < valid ? to_f64(p[r]) : 0.0;
}

// C[m][n] = (accumulate ? C[m][n] : 0) + sum_k A(m,k) B(k,n), fp64, with
//   A(m,k) = A_KM ? a[k*lda + m] : a[m*lda + k],   B(k,n) = b[k*ldb + n].
// 256 threads; a TT x TT tile per workgroup (TT = 32 WB), a quarter of it per
// wave as WB x WB blocks of v_mfma_f64_16x16x4 (operand lane l: row/column
// l%16, k l/16; result lane l register r: row l/16 + 4r, column l%16). K is
// staged 16 at a time through LDS, the next chunk's global loads in flight
// during the current MFMAs.
// VEC: 16-byte loads with no per-element tests: requires N % TT == 0,
// M % TT == 0 when A is k-major, lda % 8 == 0 and K % 16 == 0 when A is
// m-major, ldb % 8 == 0 and 16-byte aligned a, b; rows past M or K are read
// at a clamped row and multiplied by 0. Otherwise every element is tested.
// SYM (A and B the same matrix, M == N): only tiles on or below the
// diagonal are computed, each stored at (m,n) and (n,m); with accumulate the
// old C must be symmetric.
template <typename TA, bool A_KM, typename TB, bool VEC, bool SYM, int WB>
__global__ __launch_bounds__(256, 2) void gemm64_kernel(const TA* __restrict__ a, int64_t lda,
                                                     const TB* __restrict__ b, int64_t ldb,
                                                     double* __restrict__ c, int64_t ldc, int M,
                                                     int N, int64_t K, int accumulate) {
  constexpr int TT = 32 * WB;          // workgroup tile
  constexpr int EPT = TT / 16;         // staged elements per thread and operand
  constexpr int LDW = TT + 4;          // LDS row stride (doubles)
  __shared__ double As[kGK][LDW];
  __shared__ double Bs[kGK][LDW];
  int tm, tn;
  if (SYM) {
    const int q = blockIdx.x;
    int t = static_cast<int>((sqrt(8.0 * q + 1.0) - 1.0) * 0.5);
    while ((t + 1) * (t + 2) / 2 <= q) ++t;
    while (t * (t + 1) / 2 > q) --t;
    tm = t;
    tn = q - t * (t + 1) / 2;
  } else {
    tm = blockIdx.y;
    tn = blockIdx.x;
  }
  const int m0 = tm * TT, n0 = tn * TT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = (w >> 1) * (TT / 2), wn = (w & 1) * (TT / 2);

  v4d acc[WB][WB];
#pragma unroll
  for (int i = 0; i < WB; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j) acc[i][j] = v4d{0.0, 0.0, 0.0, 0.0};

  // staging coordinates: k-major operands take row kk = tid / 16 and
  // columns (tid % 16) * EPT; the m-major A takes row tid / (16 / EPT)
  // and k offset (tid % (16 / EPT)) * EPT
  const int kk_km = tid >> 4, col_km = (tid & 15) * EPT;
  constexpr int TPR = 16 / EPT;
  const int mm_mk = tid / TPR, kk_mk = (tid % TPR) * EPT;
  double ra[EPT], rb[EPT];
  auto fetch = [&](int64_t k0) {
    if (A_KM) {
      const int64_t k = k0 + kk_km;
      if (VEC) {
        const int64_t kc = k < K ? k : K - 1;
        load_vec<TA, EPT>(a + kc * lda + m0 + col_km, k < K ? 1.0 : 0.0, ra);
      } else {
        load_guarded<TA, EPT>(a + k * lda + m0 + col_km, k < K ? M - (m0 + col_km) : 0, ra);
      }
    } else {
      const int m = m0 + mm_mk;
      if (VEC) {
        const int mc = m < M ? m : M - 1;
        load_vec<TA, EPT>(a + static_cast<int64_t>(mc) * lda + k0 + kk_mk, m < M ? 1.0 : 0.0,
                          ra);
      } else {
        const int64_t left = K - (k0 + kk_mk);
        const int valid = m < M ? static_cast<int>(left < EPT ? left : EPT) : 0;
        load_guarded<TA, EPT>(a + static_cast<int64_t>(m) * lda + k0 + kk_mk, valid, ra);
      }
    }
    const int64_t k = k0 + kk_km;
    if (VEC) {
      const int64_t kc = k < K ? k : K - 1;
      load_vec<TB, EPT>(b + kc * ldb + n0 + col_km, k < K ? 1.0 : 0.0, rb);
    } else {
      load_guarded<TB, EPT>(b + k * ldb + n0 + col_km, k < K ? N - (n0 + col_km) : 0, rb);
    }
  };
  auto stage = [&]() {
    if (A_KM) {
#pragma unroll
      for (int r = 0; r < EPT; ++r) As[kk_km][col_km + r] = ra[r];
    } else {
#pragma unroll
      for (int r = 0; r < EPT; ++r) As[kk_mk + r][mm_mk] = ra[r];
    }
#pragma unroll
    for (int r = 0; r < EPT; ++r) Bs[kk_km][col_km + r] = rb[r];
  };

  if (K > 0) fetch(0);
  for (int64_t k0 = 0; k0 < K; k0 += kGK) {
    __syncthreads();
    stage();
    __syncthreads();
    if (k0 + kGK < K) fetch(k0 + kGK);
#pragma unroll
    for (int ks = 0; ks < kGK; ks += 4) {
      const int kr = ks + (lane >> 4);
      double af[WB], bf[WB];
#pragma unroll
      for (int i = 0; i < WB; ++i) af[i] = As[kr][wm + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < WB; ++j) bf[j] = Bs[kr][wn + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < WB; ++i)
#pragma unroll
        for (int j = 0; j < WB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }

#pragma unroll
  for (int i = 0; i < WB; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + i * 16 + (lane >> 4) + 4 * r;
        const int n = n0 + wn + j * 16 + (lane & 15);
        if (m < M && n < N) {
          double v = acc[i][j][r];
          const int64_t at = static_cast<int64_t>(m) * ldc + n;
          if (accumulate) v += c[at];
          c[at] = v;
          if (SYM && tm != tn) c[static_cast<int64_t>(n) * ldc + m] = v;
        }
      }
}

template <typename TA, bool A_KM, typename TB, bool SYM, int WB>
hipError_t gemm64_t(const TA* a, int64_t lda, const TB* b, int64_t ldb, double* c, int64_t ldc,
                    int M, int N, int64_t K, int accumulate, hipStream_t s) {
  constexpr int TT = 32 * WB;
  const bool vec = (lda % 8 == 0) && (ldb % 8 == 0) && (N % TT == 0) &&
                   (!A_KM || M % TT == 0) && (A_KM || K % kGK == 0) &&
                   (reinterpret_cast<uintptr_t>(a) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(b) % 16 == 0);
  const int tm = (M + TT - 1) / TT, tn = (N + TT - 1) / TT;
  const dim3 grid = SYM ? dim3(tm * (tm + 1) / 2) : dim3(tn, tm);
  if (vec)
    hipLaunchKernelGGL((gemm64_kernel<TA, A_KM, TB, true, SYM, WB>), grid, dim3(256), 0, s, a,
                       lda, b, ldb, c, ldc, M, N, K, accumulate);
  else
    hipLaunchKernelGGL((gemm64_kernel<TA, A_KM, TB, false, SYM, WB>), grid, dim3(256), 0, s, a,
                       lda, b, ldb, c, ldc, M, N, K, accumulate);
  return hipGetLastError();
}

// ------------------------------------------------------------------ rows
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  v = wave_sum_f64(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  double t = 0.0;
  for (int k = 0; k < nw; ++k) t += red[k];
  return t;
}

// Row i of M = dW_Q Hs: v = M[i,:] + delta dW_Q[i,:]; w_i = sqrt(max(v.dW_Q[i,:], 0));
// Q[i,:] = v H / n (natural column order). Q may alias M.
// BLOCKED: rows of nblk blocks of N columns under the block-diagonal
// transform; thread t = blk * TPR + u transforms its part of block blk in
// that block's slice of the dynamic LDS; the dot spans the whole row.
template <int LOG_N, bool BLOCKED>
__global__ __launch_bounds__(BLOCKED ? 1024 : (Fwht<LOG_N>::TPR < 64 ? 64 : Fwht<LOG_N>::TPR))
void calib_rows_kernel(const double* M, const float* __restrict__ dWq,
                       const double* __restrict__ delta, double* Q, double* __restrict__ w,
                       int nblk) {
  using F = Fwht<LOG_N>;
  extern __shared__ double lds_blocks[];
  __shared__ double lds_row[BLOCKED ? 1 : F::LDS];
  __shared__ double red[16];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int u = BLOCKED ? t % F::TPR : t;
  const int64_t d_in = BLOCKED ? static_cast<int64_t>(nblk) * F::N : F::N;
  const bool active = BLOCKED ? t < nblk * F::TPR : t < F::TPR;
  double* lds = BLOCKED ? lds_blocks + (t / F::TPR) * F::LDS : lds_row;
  const double dl = *delta;
  double v[F::EPT];
  double dot = 0.0;
  if (active) {
    const double* src = M + row * d_in + t * F::EPT;
    const float* dq = dWq + row * d_in + t * F::EPT;
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) {
      const double d = static_cast<double>(dq[r]);
      v[r] = src[r] + dl * d;
      dot += v[r] * d;
    }
  } else {
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) v[r] = 0.0;
  }
  dot = block_sum_f64(dot, red);      // every thread has read its part of M
  if (threadIdx.x == 0) w[row] = sqrt(dot > 0.0 ? dot : 0.0);
  F::run(v, lds, u, active);
  if (active) {
    double* dst = Q + row * d_in + (t / F::TPR) * F::N;
    const double inv_n = 1.0 / static_cast<double>(F::N);
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) dst[F::out_index(u, r)] = v[r] * inv_n;
  }
}

// out[r][:] = scale * in[r][:] H (fp64); with diag_num, *diag_num * diag_mul
// is added on the diagonal of the square matrix whose rows are nblk of these
// rows each (row r is block r % nblk of matrix row r / nblk). in may alias
// out.
template <int LOG_N>
__global__ __launch_bounds__(Fwht<LOG_N>::TPR < 64 ? 64 : Fwht<LOG_N>::TPR) void fwht64_rows_kernel(
    const double* in, double* out, double scale, const double* __restrict__ diag_num,
    double diag_mul, int nblk) {
  using F = Fwht<LOG_N>;
  __shared__ double lds[F::LDS];
  const int64_t row = blockIdx.x;
  const int u = threadIdx.x;
  const bool active = u < F::TPR;
  double v[F::EPT];
  if (active) {
    const double* src = in + row * F::N + u * F::EPT;
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) v[r] = src[r];
  } else {
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) v[r] = 0.0;
  }
  __syncthreads();
  F::run(v, lds, u, active);
  const double dadd = diag_num ? *diag_num * diag_mul : 0.0;
  const int64_t mrow = row / nblk;                         // matrix row
  const int64_t mcol0 = (row - mrow * nblk) * F::N;        // first matrix column
  if (active) {
    double* dst = out + row * F::N;
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) {
      const int j = F::out_index(u, r);
      double o = v[r] * scale;
      if (mcol0 + j == mrow) o += dadd;
      dst[j] = o;
    }
  }
}

// out = in^T for an n x n fp64 matrix, 32x32 tiles through LDS.
__global__ __launch_bounds__(256) void transpose64_kernel(const double* __restrict__ in,
                                                          double* __restrict__ out, int n) {
  __shared__ double t[32][33];
  const int bx = blockIdx.x * 32, by = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int r = ty; r < 32; r += 8) {
    const int y = by + r, x = bx + tx;
    if (y < n && x < n) t[r][tx] = in[static_cast<int64_t>(y) * n + x];
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int y = bx + r, x = by + tx;
    if (y < n && x < n) out[static_cast<int64_t>(y) * n + x] = t[tx][r];
  }
}

// delta = damp * mean(diag Hs) (exactly 0 for damp == 0)
__global__ __launch_bounds__(256) void delta_kernel(const double* __restrict__ Hs, int n,
                                                    double damp, double* __restrict__ delta) {
  __shared__ double red[4];
  double s = 0.0;
  for (int j = threadIdx.x; j < n; j += 256) s += Hs[static_cast<int64_t>(j) * n + j];
  s = block_sum_f64(s, red);
  if (threadIdx.x == 0) *delta = damp == 0.0 ? 0.0 : damp * (s / n);
}

__global__ __launch_bounds__(256) void rhs_gather_kernel(const double* __restrict__ Q, int d_in,
                                                         const int32_t* __restrict__ E,
                                                         int64_t p, double* __restrict__ rhs) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (k < p) rhs[k] = Q[static_cast<int64_t>(E[2 * k]) * d_in + E[2 * k + 1]];
}

// ------------------------------------------------------------------ refine
constexpr int kNB = 32;   // Cholesky panel width
constexpr int kST = 64;   // trailing-update tile

__device__ __forceinline__ int64_t tri(int64_t a) { return a * (a + 1) / 2; }

// v (fp64) of lane `lane` (wave-uniform index), broadcast to the wave
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane);
  return __longlong_as_double((static_cast<long long>(hi) << 32) |
                              static_cast<unsigned int>(lo));
}

// off[i] = sum over rows i' < i of tri(p_i' + 1): start (in doubles) of row
// i's packed augmented triangle; off[d_out] = total. One workgroup.
__global__ __launch_bounds__(1024) void refine_offsets_kernel(const int32_t* __restrict__ row_ptr,
                                                              int d_out,
                                                              int64_t* __restrict__ off) {
  __shared__ long long wsum[16];
  __shared__ long long carry;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int i0 = 0; i0 < d_out; i0 += 1024) {
    const int i = i0 + threadIdx.x;
    const long long v = i < d_out ? tri(static_cast<int64_t>(row_ptr[i + 1] - row_ptr[i]) + 1) : 0;
    long long incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    long long before = 0, all = 0;
    for (int k = 0; k < 16; ++k) {
      if (k < wid) before += wsum[k];
      all += wsum[k];
    }
    if (i < d_out) off[i] = carry + before + incl - v;
    __syncthreads();
    if (threadIdx.x == 0) carry += all;
    __syncthreads();
  }
  if (threadIdx.x == 0) off[d_out] = carry;
}

// One row per workgroup (256 threads). Its region of `work` holds the
// packed lower triangle (row a at tri(a)) of the (p+1)x(p+1) matrix
// [[G[S,S], .], [rhs^T, .]]. Blocked right-looking Cholesky, panels of 32
// columns: factor the diagonal block in LDS (a pivot at or below
// pivot_tol * G[S_k][S_k] stops the row: status[0] += 1, c untouched),
// solve the rows below against it, subtract their outer product from the
// trailing matrix (the rows below are solved through the inverse of the
// 32x32 diagonal block). The last row ends as y = L^-1 rhs; back substitution
// L^T x = y overwrites it; c = fp32(x). Rows whose region would pass
// `cap` doubles are skipped (status[1] += 1).
__global__ __launch_bounds__(256) void refine_kernel(const int32_t* __restrict__ row_ptr,
                                                     const int32_t* __restrict__ E,
                                                     const double* __restrict__ G, int ld,
                                                     const double* __restrict__ rhs,
                                                     const int64_t* __restrict__ off,
                                                     double* __restrict__ work, int64_t cap,
                                                     float* __restrict__ c,
                                                     int32_t* __restrict__ status,
                                                     double pivot_tol) {
  __shared__ double Ld[kNB][kNB + 1];
  __shared__ double Li[kNB][kNB + 1];
  __shared__ double Sa[kST][kNB + 1];
  __shared__ double Sb[kST][kNB + 1];
  __shared__ double red[8][kNB + 1];
  __shared__ int bad;
  const int row = blockIdx.x;
  const int kb = row_ptr[row];
  const int p = row_ptr[row + 1] - kb;
  if (p <= 0) return;
  const int tid = threadIdx.x;
  const int64_t base = off[row];
  if (base + tri(static_cast<int64_t>(p) + 1) > cap) {
    if (tid == 0) atomicAdd(&status[1], 1);
    return;
  }
  double* T = work + base;
  const int32_t* S = E + 2 * static_cast<int64_t>(kb) + 1;   // column of position a: S[2a]

  // 1. gather the augmented lower triangle
  {
    const int64_t total = tri(static_cast<int64_t>(p) + 1);
    int a = 0;
    int64_t bcol = tid;
    for (int64_t q = tid; q < total; q += 256) {
      while (bcol > a) {
        bcol -= a + 1;
        ++a;
      }
      double val;
      if (a < p)
        val = G[static_cast<int64_t>(S[2 * a]) * ld + S[2 * bcol]];
      else
        val = bcol < p ? rhs[kb + bcol] : 0.0;
      T[q] = val;
      bcol += 256;
    }
  }
  __syncthreads();

  // 2. blocked Cholesky of rows 0..p (row p only as a row)
  for (int k0 = 0; k0 < p; k0 += kNB) {
    const int nb = min(kNB, p - k0);
    for (int e = tid; e < kNB * kNB; e += 256) {
      const int r = e / kNB, cc = e % kNB;
      Ld[r][cc] = (r < nb && cc <= r) ? T[tri(k0 + r) + k0 + cc] : 0.0;
    }
    __syncthreads();
    // factor the diagonal block in wave 0, lane r holding row r in
    // registers; pivots and column entries are broadcast by readlane. A
    // pivot at or below pivot_tol times the entry's original value
    // G[S_k][S_k] stops the row.
    if (tid < 64) {
      const int r = tid;
      double arow[kNB];
#pragma unroll
      for (int cc = 0; cc < kNB; ++cc) arow[cc] = (r < nb && cc <= r) ? Ld[r][cc] : 0.0;
      double dg = 0.0;
      if (r < nb) {
        const int sr = S[2 * (k0 + r)];
        dg = G[static_cast<int64_t>(sr) * ld + sr];
      }
      int ok = 1;
#pragma unroll
      for (int k = 0; k < kNB; ++k) {
        if (k < nb && ok) {
          const double piv = readlane_f64(arow[k], k);
          if (!(piv > pivot_tol * readlane_f64(dg, k))) {
            ok = 0;
          } else {
            const double dk = sqrt(piv);
            if (r == k) arow[k] = dk;
            else if (r > k) arow[k] = arow[k] / dk;
#pragma unroll
            for (int cc = k + 1; cc < kNB; ++cc) {
              if (cc < nb) {
                const double lck = readlane_f64(arow[k], cc);
                if (r >= cc) arow[cc] -= arow[k] * lck;
              }
            }
          }
        }
      }
#pragma unroll
      for (int cc = 0; cc < kNB; ++cc)
        if (r < nb && cc <= r) Ld[r][cc] = arow[cc];
      if (tid == 0) bad = ok ? 0 : 1;
    }
    __syncthreads();
    if (bad) {
      if (tid == 0) atomicAdd(&status[0], 1);
      return;
    }
    for (int e = tid; e < kNB * kNB; e += 256) {
      const int r = e / kNB, cc = e % kNB;
      if (r < nb && cc <= r) T[tri(k0 + r) + k0 + cc] = Ld[r][cc];
    }
    // rows below the block, the right-hand side row included:
    // L21 = A21 L11^-T, with L11^-1 formed in wave 0: lane cc solves for
    // column cc, reading L11 uniformly and its own earlier entries from LDS
    if (tid < kNB) {
      const int cc = tid;
      for (int r = 0; r < nb; ++r) {
        double s = r == cc ? 1.0 : 0.0;
        int c2 = 0;
        for (; c2 + 4 <= r; c2 += 4) {
          const double l0 = Ld[r][c2], l1 = Ld[r][c2 + 1], l2 = Ld[r][c2 + 2], l3 = Ld[r][c2 + 3];
          const double x0 = Li[c2][cc], x1 = Li[c2 + 1][cc], x2 = Li[c2 + 2][cc],
                       x3 = Li[c2 + 3][cc];
          s -= l0 * x0;
          s -= l1 * x1;
          s -= l2 * x2;
          s -= l3 * x3;
        }
        for (; c2 < r; ++c2) s -= Ld[r][c2] * Li[c2][cc];
        Li[r][cc] = cc < nb ? s / Ld[r][r] : 0.0;
      }
      for (int r = nb; r < kNB; ++r) Li[r][cc] = 0.0;
    }
    __syncthreads();
    for (int a0 = k0 + nb; a0 <= p; a0 += kST) {
      for (int e = tid; e < kST * kNB; e += 256) {
        const int r = e / kNB, cc = e % kNB;
        const int a = a0 + r;
        Sa[r][cc] = (a <= p && cc < nb) ? T[tri(a) + k0 + cc] : 0.0;
      }
      __syncthreads();
      const int r = tid >> 2, c0 = (tid & 3) * 8;
      double o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = 0.0;
      for (int c2 = 0; c2 < nb; ++c2) {
        const double av = Sa[r][c2];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] += av * Li[c0 + j][c2];
      }
      if (a0 + r <= p) {
        double* Ta = T + tri(a0 + r) + k0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (c0 + j < nb) Ta[c0 + j] = o[j];
      }
      __syncthreads();
    }
    // trailing update: T[a][b] -= sum_c L21[a][c] L21[b][c], r0 <= b <= a <= p, b < p
    const int r0 = k0 + nb;
    const int rn = p + 1 - r0;
    const int nt = (rn + kST - 1) / kST;
    for (int ta = 0; ta < nt; ++ta) {
      for (int e = tid; e < kST * kNB; e += 256) {
        const int r = e / kNB, cc = e % kNB;
        const int a = r0 + ta * kST + r;
        Sa[r][cc] = (a <= p && cc < nb) ? T[tri(a) + k0 + cc] : 0.0;
      }
      for (int tb = 0; tb <= ta; ++tb) {
        for (int e = tid; e < kST * kNB; e += 256) {
          const int r = e / kNB, cc = e % kNB;
          const int bb = r0 + tb * kST + r;
          Sb[r][cc] = (bb < p && cc < nb) ? T[tri(bb) + k0 + cc] : 0.0;
        }
        __syncthreads();
        const int ia = (tid >> 4) * 4, ib = (tid & 15) * 4;
        double acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
        for (int cc = 0; cc < nb; ++cc) {
          double av[4], bv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) av[i] = Sa[ia + i][cc];
#pragma unroll
          for (int j = 0; j < 4; ++j) bv[j] = Sb[ib + j][cc];
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * bv[j];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int a = r0 + ta * kST + ia + i;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int bb = r0 + tb * kST + ib + j;
            if (a <= p && bb < p && bb <= a) T[tri(a) + bb] -= acc[i][j];
          }
        }
        __syncthreads();
      }
    }
  }

  // 3. back substitution L^T x = y, y = the last row; x replaces it
  double* Y = T + tri(p);
  for (int blk = (p - 1) / kNB; blk >= 0; --blk) {
    const int k1 = blk * kNB, nb = min(kNB, p - k1);
    {
      const int cc = tid & 31, g = tid >> 5;
      double s = 0.0;
      if (cc < nb)
        for (int bb = k1 + nb + g; bb < p; bb += 8) s += T[tri(bb) + k1 + cc] * Y[bb];
      red[g][cc] = s;
    }
    for (int e = tid; e < kNB * kNB; e += 256) {
      const int r = e / kNB, cc = e % kNB;
      Ld[r][cc] = (r < nb && cc <= r) ? T[tri(k1 + r) + k1 + cc] : 0.0;
    }
    __syncthreads();
    if (tid < 64) {
      const int cc = tid;
      double s = 0.0;
      if (cc < nb) {
        s = Y[k1 + cc];
#pragma unroll
        for (int g = 0; g < 8; ++g) s -= red[g][cc];
      }
      for (int k = nb - 1; k >= 0; --k) {
        double xk = cc == k ? s / Ld[k][k] : 0.0;
        xk = __shfl(xk, k, 64);
        if (cc < k) s -= Ld[k][cc] * xk;
        if (cc == k) s = xk;
      }
      if (cc < nb) Y[k1 + cc] = s;
    }
    __syncthreads();
  }

  // 4. values
  for (int a = tid; a < p; a += 256) c[kb + a] = __double2float_rn(Y[a]);
}

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// scratch: delta, w [d_out], Q [d_out][d_in], T1 [d_in][d_in] (all fp64)
struct CalWs {
  size_t delta, w, q, t1, total;
};

size_t al256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

CalWs cal_ws(int d_out, int d_in) {
  CalWs l;
  l.delta = 0;
  l.w = 256;
  l.q = l.w + al256(static_cast<size_t>(d_out) * 8);
  l.t1 = l.q + al256(static_cast<size_t>(d_out) * d_in * 8);
  l.total = l.t1 + al256(static_cast<size_t>(d_in) * d_in * 8);
  return l;
}

template <int L>
hipError_t fwht64_t(const double* in, double* out, int64_t rows, double scale,
                    const double* diag_num, double diag_mul, int nblk, hipStream_t s) {
  hipLaunchKernelGGL(fwht64_rows_kernel<L>, dim3(static_cast<unsigned>(rows)),
                     dim3(Fwht<L>::TPR < 64 ? 64 : Fwht<L>::TPR), 0, s, in, out, scale, diag_num,
                     diag_mul, nblk);
  return hipGetLastError();
}

template <int L>
hipError_t calib_rows_t(const double* M, const float* dWq, const double* delta, double* Q,
                        double* w, int d_out, int nblk, hipStream_t s) {
  using F = Fwht<L>;
  if (nblk == 1) {
    hipLaunchKernelGGL((calib_rows_kernel<L, false>), dim3(d_out),
                       dim3(F::TPR < 64 ? 64 : F::TPR), 0, s, M, dWq, delta, Q, w, 1);
    return hipGetLastError();
  }
  if constexpr (L >= 6 && L <= 12) {
    // whole waves (the wave sums take every lane of a wave; threads past
    // nblk * TPR hold no columns)
    const int threads = (nblk * F::TPR + 63) / 64 * 64;
    const size_t lds = static_cast<size_t>(nblk) * F::LDS * sizeof(double);
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&calib_rows_kernel<L, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((calib_rows_kernel<L, true>), dim3(d_out), dim3(threads), lds, s, M, dWq,
                       delta, Q, w, nblk);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace

// ------------------------------------------------------------------ launchers
hipError_t launch_hessian(const void* X, Dt x_dt, int64_t N, int d_in, double* Hs,
                          int accumulate, hipStream_t s) {
  if (x_dt == Dt::F32)
    return gemm64_t<float, true, float, true, 2>(static_cast<const float*>(X), d_in,
                                                 static_cast<const float*>(X), d_in, Hs, d_in,
                                                 d_in, d_in, N, accumulate, s);
  return gemm64_t<uint16_t, true, uint16_t, true, 2>(static_cast<const uint16_t*>(X), d_in,
                                                     static_cast<const uint16_t*>(X), d_in, Hs,
                                                     d_in, d_in, d_in, N, accumulate, s);
}

size_t calibrated_scratch_bytes(int d_out, int d_in) { return cal_ws(d_out, d_in).total; }

hipError_t launch_calib_prepare(const float* dWq, int d_out, int log_n, const double* Hs,
                                double damp, void* scratch, double** w_out, hipStream_t s,
                                int nblk) {
  const int d_in = nblk << log_n;
  const CalWs l = cal_ws(d_out, d_in);
  char* base = static_cast<char*>(scratch);
  double* delta = reinterpret_cast<double*>(base + l.delta);
  double* w = reinterpret_cast<double*>(base + l.w);
  double* Q = reinterpret_cast<double*>(base + l.q);
  hipLaunchKernelGGL(delta_kernel, dim3(1), dim3(256), 0, s, Hs, d_in, damp, delta);
  hipError_t e = gemm64_t<float, false, double, false, 4>(dWq, d_in, Hs, d_in, Q, d_in, d_out,
                                                          d_in, d_in, 0, s);
  if (e != hipSuccess) return e;
  switch (log_n) {
#define QWHA_CASE(L) \
  case L: e = calib_rows_t<L>(Q, dWq, delta, Q, w, d_out, nblk, s); break;
    QWHA_CASE(1) QWHA_CASE(2) QWHA_CASE(3) QWHA_CASE(4) QWHA_CASE(5) QWHA_CASE(6) QWHA_CASE(7)
    QWHA_CASE(8) QWHA_CASE(9) QWHA_CASE(10) QWHA_CASE(11) QWHA_CASE(12) QWHA_CASE(13)
    QWHA_CASE(14)
#undef QWHA_CASE
    default:
      return hipErrorInvalidValue;
  }
  *w_out = w;
  return e;
}

hipError_t launch_calib_finish(const int32_t* E, int64_t p, int d_out, int log_n, const double* Hs,
                               void* scratch, double* G, double* rhs, hipStream_t s, int nblk) {
  const int d_in = nblk << log_n;
  const CalWs l = cal_ws(d_out, d_in);
  char* base = static_cast<char*>(scratch);
  const double* delta = reinterpret_cast<const double*>(base + l.delta);
  const double* Q = reinterpret_cast<const double*>(base + l.q);
  double* T1 = reinterpret_cast<double*>(base + l.t1);
  if (p > 0)
    hipLaunchKernelGGL(rhs_gather_kernel, dim3(static_cast<unsigned>((p + 255) / 256)), dim3(256),
                       0, s, Q, d_in, E, p, rhs);
  const double b = static_cast<double>(1 << log_n);
  const double inv_b2 = 1.0 / (b * b);
  const int64_t vrows = static_cast<int64_t>(d_in) * nblk;   // [d_in * nblk][b] views
  hipError_t e = hipSuccess;
  switch (log_n) {
#define QWHA_CASE(L)                                                                     \
  case L:                                                                                \
    e = fwht64_t<L>(Hs, G, vrows, 1.0, nullptr, 0.0, nblk, s);                         \
    if (e != hipSuccess) return e;                                                       \
    hipLaunchKernelGGL(transpose64_kernel, dim3((d_in + 31) / 32, (d_in + 31) / 32),      \
                       dim3(256), 0, s, G, T1, d_in);                                    \
    e = fwht64_t<L>(T1, G, vrows, inv_b2, delta, 1.0 / b, nblk, s);                      \
    break;
    QWHA_CASE(1) QWHA_CASE(2) QWHA_CASE(3) QWHA_CASE(4) QWHA_CASE(5) QWHA_CASE(6) QWHA_CASE(7)
    QWHA_CASE(8) QWHA_CASE(9) QWHA_CASE(10) QWHA_CASE(11) QWHA_CASE(12) QWHA_CASE(13)
    QWHA_CASE(14)
#undef QWHA_CASE
    default:
      return hipErrorInvalidValue;
  }
  return e;
}

size_t refine_header_bytes(int d_out) { return al256(static_cast<size_t>(d_out + 1) * 8); }

hipError_t launch_refine(const int32_t* row_ptr, const int32_t* E, const double* G, int d_in,
                         const double* rhs, int d_out, float* c, int32_t* status, void* ws,
                         size_t ws_bytes, double pivot_tol, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  int64_t* off = reinterpret_cast<int64_t*>(base);
  const size_t hb = refine_header_bytes(d_out);
  double* work = reinterpret_cast<double*>(base + hb);
  const int64_t cap = static_cast<int64_t>((ws_bytes - hb) / 8);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(64), 0, s, status, 2, 0);
  hipLaunchKernelGGL(refine_offsets_kernel, dim3(1), dim3(1024), 0, s, row_ptr, d_out, off);
  hipLaunchKernelGGL(refine_kernel, dim3(d_out), dim3(256), 0, s, row_ptr, E, G, d_in, rhs, off,
                     work, cap, c, status, pivot_tol);
  return hipGetLastError();
}

}  // namespace qwha
