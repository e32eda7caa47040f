// Adapter forward / backward through the sparse coefficient matrix F.
//
// With dW = alpha F H / n (QWHA notes, papernotes.org, 方法详解 › 整体框架) and
// z = x H / n (H symmetric), the adapter branch is
//   forward   y  = x dW^T  = alpha * z F^T            (gather-SpMM, CSR)
//   backward  dx = dy dW   = alpha * FWHT(dy F) / n   (gather-SpMM, CSC)
//             dc_k = alpha * sum_t dy[t, i_k] z[t, j_k] (sampled dense-dense
//                    product at E: only c is trainable, W_Q and H frozen,
//                    papernotes.org, 损失函数 / 训练策略).
//
// Kernel shape (gfx950, wave64): one workgroup = 8 waves = a tile of TT = 128
// tokens x (8 * 64) output rows (8 * 32 with dc partials); every output row's
// accumulators for the tile's tokens live in registers. The source matrix (z
// for the forward, dy for the backward) is staged through LDS in blocks of
// JB = 128 source columns, token-minor, double buffered: the next block's
// global loads are in flight while the current block is consumed. The
// nonzeros of every (output row, source block) pair are contiguous in a
// packed stream (LDS byte offset of the column, value) prepared per call.
#include "common.h"
#include "launch.h"

namespace qwha {

constexpr int kTT = 128;          // tokens per tile
constexpr int kJB = 128;          // source columns per staged block
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kSfwd = 12;         // rows per 16-lane group, plain SpMM (48 per wave)
constexpr int kSdc = 8;           // rows per group when dc partials are also produced

SpmmPlan spmm_plan_impl(int64_t T, int n_src, int n_out, bool dc) {
  SpmmPlan pl;
  pl.tt = kTT;
  pl.jb = kJB;
  pl.rows_wg = kWaves * 4 * (dc ? kSdc : kSfwd);
  pl.nblk = (n_src + kJB - 1) / kJB;
  pl.ntiles = (T + kTT - 1) / kTT;
  (void)n_out;
  return pl;
}

SpmmPlan spmm_plan(int64_t T, int n_src, int n_out) { return spmm_plan_impl(T, n_src, n_out, false); }

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

size_t spmm_prep_bytes(int64_t nnz, int n_out, const SpmmPlan& pl) {
  return align256(static_cast<size_t>(nnz) * 8) +
         align256(static_cast<size_t>(n_out) * (pl.nblk + 1) * 4);
}

static int2* prep_packed(void* prep) { return static_cast<int2*>(prep); }
static int32_t* prep_bptr(void* prep, int64_t nnz) {
  return reinterpret_cast<int32_t*>(static_cast<char*>(prep) + align256(static_cast<size_t>(nnz) * 8));
}

// ------------------------------------------------------------ prep
__global__ void pack_csr_kernel(const int32_t* __restrict__ E, const float* __restrict__ c,
                                int64_t nnz, int2* __restrict__ packed) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k >= nnz) return;
  const int col = E[2 * k + 1];
  const int jj = col % kJB;
  packed[k] = make_int2(jj * kTT * 4, __float_as_int(c[k]));
}

__global__ void pack_csc_kernel(const int32_t* __restrict__ perm, const int32_t* __restrict__ E,
                                const float* __restrict__ c, int64_t nnz, int2* __restrict__ packed) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= nnz) return;
  const int k = perm[q];
  const int row = E[2 * static_cast<int64_t>(k)];
  const int ii = row % kJB;
  packed[q] = make_int2(ii * kTT * 4, __float_as_int(c[k]));
}

// bptr[o][b] = first position in segment o whose source column is >= b*JB.
// key(pos) = E[2*pos + 1] (CSR) or E[2*perm[pos]] (CSC).
__global__ void bptr_kernel(const int32_t* __restrict__ seg_ptr, const int32_t* __restrict__ E,
                            const int32_t* __restrict__ perm, int n_out, int nblk,
                            int32_t* __restrict__ bptr) {
  const int64_t id = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(n_out) * (nblk + 1);
  if (id >= total) return;
  const int o = static_cast<int>(id / (nblk + 1));
  const int b = static_cast<int>(id % (nblk + 1));
  int lo = seg_ptr[o], hi = seg_ptr[o + 1];
  const int target = b * kJB;
  while (lo < hi) {
    const int mid = lo + ((hi - lo) >> 1);
    const int key = perm ? E[2 * static_cast<int64_t>(perm[mid])] : E[2 * static_cast<int64_t>(mid) + 1];
    if (key < target) lo = mid + 1; else hi = mid;
  }
  bptr[id] = lo;
}

hipError_t launch_prep_csr(const int32_t* row_ptr, const int32_t* E, const float* c, int d_out,
                           int64_t nnz, const SpmmPlan& pl, void* prep, hipStream_t s) {
  if (nnz > 0)
    hipLaunchKernelGGL(pack_csr_kernel, dim3(static_cast<unsigned>((nnz + 255) / 256)), dim3(256), 0,
                       s, E, c, nnz, prep_packed(prep));
  const int64_t total = static_cast<int64_t>(d_out) * (pl.nblk + 1);
  hipLaunchKernelGGL(bptr_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s,
                     row_ptr, E, nullptr, d_out, pl.nblk, prep_bptr(prep, nnz));
  return hipGetLastError();
}

hipError_t launch_prep_csc(const int32_t* col_ptr, const int32_t* perm, const int32_t* E,
                           const float* c, int d_in, int64_t nnz, const SpmmPlan& pl, void* prep,
                           hipStream_t s) {
  if (nnz > 0)
    hipLaunchKernelGGL(pack_csc_kernel, dim3(static_cast<unsigned>((nnz + 255) / 256)), dim3(256), 0,
                       s, perm, E, c, nnz, prep_packed(prep));
  const int64_t total = static_cast<int64_t>(d_in) * (pl.nblk + 1);
  hipLaunchKernelGGL(bptr_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s,
                     col_ptr, E, perm, d_in, pl.nblk, prep_bptr(prep, nnz));
  return hipGetLastError();
}

// ------------------------------------------------------------ staging
template <typename SrcT>
struct Stage {
  static constexpr int VEC = 16 / static_cast<int>(sizeof(SrcT));   // elements per 16-byte load
  static constexpr int NL = kJB / (4 * VEC);                         // loads per thread per block
  uint4 raw[NL];

  // thread -> token tt = tid % 128, column group g = tid / 128 (0..3);
  // load q covers local columns (q*4 + g)*VEC .. +VEC-1.
  __device__ __forceinline__ void load(const SrcT* __restrict__ src, int64_t T, int n_src,
                                       int64_t t0, int b, bool vec_ok) {
    const int tt = threadIdx.x & (kTT - 1);
    const int g = threadIdx.x >> 7;
    const int64_t t = t0 + tt;
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      const int col = b * kJB + (q * 4 + g) * VEC;
      if (t < T && vec_ok && col + VEC <= n_src) {
        raw[q] = *reinterpret_cast<const uint4*>(src + t * n_src + col);
      } else {
        uint32_t w[4] = {0, 0, 0, 0};
        if (t < T) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            if (col + e < n_src) {
              uint32_t bits;
              if constexpr (sizeof(SrcT) == 4) bits = __float_as_uint(static_cast<float>(src[t * n_src + col + e]));
              else bits = static_cast<uint32_t>(src[t * n_src + col + e]);
              if constexpr (sizeof(SrcT) == 4) w[e] = bits;
              else w[e >> 1] |= bits << (16 * (e & 1));
            }
          }
        }
        raw[q] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }

  __device__ __forceinline__ void store(float* __restrict__ st) const {
    const int tt = threadIdx.x & (kTT - 1);
    const int g = threadIdx.x >> 7;
#pragma unroll
    for (int q = 0; q < NL; ++q) {
      const int cl = (q * 4 + g) * VEC;
      const uint32_t w[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float f;
        if constexpr (sizeof(SrcT) == 4) f = __uint_as_float(w[e]);
        else f = (e & 1) ? __uint_as_float(w[e >> 1] & 0xFFFF0000u) : __uint_as_float(w[e >> 1] << 16);
        st[(cl + e) * kTT + tt] = f;
      }
    }
  }
};

// ------------------------------------------------------------ main kernel
// Wave layout: 4 groups of 16 lanes. Group g owns the rows o0 + g*S + s
// (s < S); lane gl of the group owns tokens t0 + 8*gl .. +7 of the tile, so
// the 16 lanes of a group cover all 128 tokens. A nonzero of the group's
// current row is read by the group's 16 lanes as two ds_read_b128 each (512
// contiguous bytes of the staged block: conflict-free) and costs 8 FMAs per
// lane. Nonzeros are fetched per lane with vector loads, a batch of 4 at a
// time, and the first batch of the next row is in flight while the current
// row is processed. With zsrc (backward), each nonzero also yields
// sum_{t in lane} src[t][col] * zsrc[t][o], reduced over the group's 16 lanes
// with four DPP row shifts into lane 15, which stores the tile's partial.
constexpr int kGroups = 4;
constexpr int kTPL = 8;          // tokens per lane
constexpr int kBatch = 4;        // nonzeros fetched per vector load batch

__device__ __forceinline__ float dpp_row_shr(float v, int n) {
  int r;
  switch (n) {
    case 1: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, true); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, true); break;
    case 4: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, true); break;
    default: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, true); break;
  }
  return __int_as_float(r);
}

// Inclusive prefix over each row of 16 lanes: lane 15 of a row ends with the
// row's total.
__device__ __forceinline__ float row16_total(float v) {
  v += dpp_row_shr(v, 1);
  v += dpp_row_shr(v, 2);
  v += dpp_row_shr(v, 4);
  v += dpp_row_shr(v, 8);
  return v;
}

struct Batch {
  int2 e[kBatch];
};

__device__ __forceinline__ Batch load_batch(const int2* __restrict__ nz, int k, int k1) {
  Batch b;
#pragma unroll
  for (int u = 0; u < kBatch; ++u) b.e[u] = (k + u < k1) ? nz[k + u] : make_int2(0, 0);
  return b;
}

template <int S, typename SrcT, typename OutT, bool DC>
__global__ __launch_bounds__(kThreads) void spmm_kernel(
    const SrcT* __restrict__ src, int64_t T, int n_src, const int2* __restrict__ nz,
    const int32_t* __restrict__ bptr, int64_t nnz, int n_out, int nblk, float alpha,
    OutT* __restrict__ out, int accumulate, const float* __restrict__ zsrc,
    float* __restrict__ partial) {
  __shared__ float stage[2][kJB * kTT];
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int gl = lane & 15;
  const int w = uniform(threadIdx.x >> 6);
  const int64_t tile = blockIdx.x;
  const int64_t t0 = tile * kTT;
  const int rows_wg = kWaves * kGroups * S;
  const int orow = static_cast<int>(blockIdx.y) * rows_wg + w * (kGroups * S) + g * S;
  const bool vec_ok = (n_src % Stage<SrcT>::VEC) == 0;
  const int lds_lane = gl * (kTPL * 4);      // byte offset of the lane's 8 tokens

  float acc[S][kTPL];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int q = 0; q < kTPL; ++q) acc[s][q] = 0.f;

  float zr[DC ? S : 1][kTPL];
  if constexpr (DC) {
#pragma unroll
    for (int q = 0; q < kTPL; ++q) {
      const int64_t t = t0 + kTPL * gl + q;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int o = orow + s;
        zr[s][q] = (t < T && o < n_out) ? zsrc[t * n_out + o] : 0.f;
      }
    }
  }

  // per-slot cursor into the packed stream: start of the current block
  int kcur[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int o = orow + s;
    kcur[s] = (o < n_out) ? bptr[static_cast<int64_t>(o) * (nblk + 1)] : 0;
  }

  Stage<SrcT> pf;
  pf.load(src, T, n_src, t0, 0, vec_ok);
  for (int b = 0; b < nblk; ++b) {
    float* st = stage[b & 1];
    pf.store(st);
    __syncthreads();
    if (b + 1 < nblk) pf.load(src, T, n_src, t0, b + 1, vec_ok);
    int kend[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int o = orow + s;
      kend[s] = (o < n_out) ? bptr[static_cast<int64_t>(o) * (nblk + 1) + b + 1] : 0;
    }
    const char* sb = reinterpret_cast<const char*>(st) + lds_lane;
    Batch next = load_batch(nz, kcur[0], kend[0]);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      Batch cur = next;
      if (s + 1 < S) next = load_batch(nz, kcur[s + 1], kend[s + 1]);
      const int k1 = kend[s];
      for (int kb = kcur[s]; kb < k1; kb += kBatch) {
        if (kb != kcur[s]) cur = load_batch(nz, kb, k1);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (kb + u < k1) {
            const int2 e = cur.e[u];
            const float4 v0 = *reinterpret_cast<const float4*>(sb + e.x);
            const float4 v1 = *reinterpret_cast<const float4*>(sb + e.x + 16);
            const float cv = __int_as_float(e.y);
            const float v[kTPL] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
            for (int q = 0; q < kTPL; ++q) acc[s][q] = fmaf(cv, v[q], acc[s][q]);
            if constexpr (DC) {
              float d = v[0] * zr[s][0];
#pragma unroll
              for (int q = 1; q < kTPL; ++q) d = fmaf(v[q], zr[s][q], d);
              d = row16_total(d);
              if (gl == 15) partial[tile * nnz + kb + u] = d;
            }
          }
        }
      }
      kcur[s] = k1;
    }
  }

  // epilogue: lane writes rows orow .. orow+S-1 (contiguous) of its 8 tokens
#pragma unroll
  for (int q = 0; q < kTPL; ++q) {
    const int64_t t = t0 + kTPL * gl + q;
    if (t >= T) continue;
    OutT* dst = out + t * n_out;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int o = orow + s;
      if (o < n_out) {
        float val = alpha * acc[s][q];
        if (accumulate) val += Elem<OutT>::ld(dst, o);
        Elem<OutT>::st(dst, o, val);
      }
    }
  }
}

template <int S, typename SrcT, typename OutT, bool DC>
static hipError_t spmm_t(const void* src, int64_t T, int n_src, const void* prep, int64_t nnz,
                         int n_out, const SpmmPlan& pl, float alpha, void* out, int acc,
                         const float* zsrc, float* partial, hipStream_t s) {
  constexpr int rows_wg = kWaves * kGroups * S;
  const int gy = (n_out + rows_wg - 1) / rows_wg;
  void* pp = const_cast<void*>(prep);
  hipLaunchKernelGGL((spmm_kernel<S, SrcT, OutT, DC>), dim3(static_cast<unsigned>(pl.ntiles), gy),
                     dim3(kThreads), 0, s, static_cast<const SrcT*>(src), T, n_src,
                     prep_packed(pp), prep_bptr(pp, nnz), nnz, n_out, pl.nblk, alpha,
                     static_cast<OutT*>(out), acc, zsrc, partial);
  return hipGetLastError();
}

hipError_t launch_spmm(const void* src, Dt src_dt, int64_t T, int n_src, const void* prep,
                       int64_t nnz, int n_out, const SpmmPlan& pl, float alpha, void* out,
                       Dt out_dt, int accumulate, const float* zsrc, float* partial,
                       hipStream_t s) {
  if (pl.ntiles == 0) return hipSuccess;
  const bool dc = partial != nullptr;
  if (dc) {
    if (src_dt == Dt::F32 && out_dt == Dt::F32)
      return spmm_t<kSdc, float, float, true>(src, T, n_src, prep, nnz, n_out, pl, alpha, out,
                                              accumulate, zsrc, partial, s);
    if (src_dt == Dt::BF16 && out_dt == Dt::F32)
      return spmm_t<kSdc, uint16_t, float, true>(src, T, n_src, prep, nnz, n_out, pl, alpha, out,
                                                 accumulate, zsrc, partial, s);
    return hipErrorInvalidValue;
  }
  if (src_dt == Dt::F32 && out_dt == Dt::F32)
    return spmm_t<kSfwd, float, float, false>(src, T, n_src, prep, nnz, n_out, pl, alpha, out,
                                              accumulate, nullptr, nullptr, s);
  if (src_dt == Dt::F32 && out_dt == Dt::BF16)
    return spmm_t<kSfwd, float, uint16_t, false>(src, T, n_src, prep, nnz, n_out, pl, alpha, out,
                                                 accumulate, nullptr, nullptr, s);
  if (src_dt == Dt::BF16 && out_dt == Dt::F32)
    return spmm_t<kSfwd, uint16_t, float, false>(src, T, n_src, prep, nnz, n_out, pl, alpha, out,
                                                 accumulate, nullptr, nullptr, s);
  return spmm_t<kSfwd, uint16_t, uint16_t, false>(src, T, n_src, prep, nnz, n_out, pl, alpha, out,
                                                  accumulate, nullptr, nullptr, s);
}

// ------------------------------------------------------------ dc reduction
__global__ void dc_reduce_kernel(const float* __restrict__ partial, int64_t ntiles, int64_t nnz,
                                 const int32_t* __restrict__ perm, float alpha,
                                 float* __restrict__ dc) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= nnz) return;
  float s = 0.f;
  for (int64_t t = 0; t < ntiles; ++t) s += partial[t * nnz + q];
  dc[perm[q]] = alpha * s;
}

hipError_t launch_dc_reduce(const float* partial, int64_t ntiles, int64_t nnz,
                            const int32_t* csc_perm, float alpha, float* dc, hipStream_t s) {
  if (nnz == 0) return hipSuccess;
  hipLaunchKernelGGL(dc_reduce_kernel, dim3(static_cast<unsigned>((nnz + 255) / 256)), dim3(256), 0,
                     s, partial, ntiles, nnz, csc_perm, alpha, dc);
  return hipGetLastError();
}

// ------------------------------------------------------------ update
__global__ void sign_update_kernel(float* __restrict__ c, const float* __restrict__ dc, int64_t p,
                                   float step) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k >= p) return;
  const float g = dc[k];
  const float sg = g > 0.f ? 1.f : (g < 0.f ? -1.f : 0.f);
  c[k] = c[k] + step * sg;
}

hipError_t launch_sign_update(float* c, const float* dc, int64_t p, float step, hipStream_t s) {
  if (p == 0) return hipSuccess;
  hipLaunchKernelGGL(sign_update_kernel, dim3(static_cast<unsigned>((p + 255) / 256)), dim3(256), 0, s,
                     c, dc, p, step);
  return hipGetLastError();
}

}  // namespace qwha
