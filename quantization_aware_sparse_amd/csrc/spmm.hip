// Adapter forward / backward through the sparse coefficient matrix F.
//
// With dW = alpha F H / n (QWHA notes, papernotes.org, 方法详解 › 整体框架) and
// z = x H / n (H symmetric), the adapter branch is
//   forward   y  = x dW^T  = alpha * z F^T            (gather-SpMM over rows of F)
//   backward  dx = dy dW   = alpha * FWHT(dy F) / n   (gather-SpMM over columns of F)
//             dc_k = alpha * sum_t dy[t, i_k] z[t, j_k] (sampled dense-dense
//                    product at E: only c is trainable, W_Q and H frozen,
//                    papernotes.org, 损失函数 / 训练策略).
//
// Both directions compute out[t][o] = alpha * sum over the nonzeros
// (o, col, val) of segment o of val * src[t][col], where the segments are the
// rows of F (forward; src = z) or its columns (backward; src = dy); the
// backward kernel also forms the dc partials.
//
// Work decomposition (gfx950, wave64). A workgroup of 16 waves owns a tile of
// 256 tokens and a group of output rows (16 per wave, or 8 with dc
// partials); lane l owns tokens 4l .. 4l+3, so a row's accumulators for the
// tile live in 4 registers per lane and every row is processed by the whole
// wave: no divergence between rows. The source is staged through LDS in
// blocks of 64 columns, token-minor (row jj of the staged block holds the
// 256 tokens of source column jj), double buffered; a nonzero costs the wave
// one conflict-free ds_read_b128 (1 KiB) and four FMAs per lane.
//
// The nonzeros are re-laid out per call "column-block major": for block b,
// the segments of all output rows in row order, so a workgroup's share of a
// block is one contiguous run of the stream. It is staged in LDS with the
// block, and waves read their entries from there (in-order LDS counters let
// the next entry's read overlap the current one's).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace qwha {

// Compile-time loop: f(std::integral_constant<int, I>) for I in [I0, N).
template <int I0, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < N) {
    f(std::integral_constant<int, I0>{});
    static_for<I0 + 1, N>(f);
  }
}

constexpr int kPad = 16;          // padding entries after the stream

// wave-uniform rows (plain SpMM)
constexpr int kRT = 256;          // tokens per tile: 64 lanes x 4
constexpr int kRJB = 64;          // source columns per staged block (64 KiB fp32)
constexpr int kRJB16 = 128;       // the same for a bf16 source kept as bf16 (64 KiB)
constexpr int kRW = 16;           // waves per workgroup
constexpr int kRR = 16;           // output rows per wave
constexpr int kRRdc = 8;          // output rows per wave with dc partials
// The row after which a wave stores the first half of the next block and
// issues the loads of its second half (forward, backward; measured at the
// 4096x4096 layer). The first half's loads go out before the block's opening
// barrier, so they have the barrier wait and the first rows to land.
constexpr int kMidF = 8;
constexpr int kMidB = 2;
constexpr int kEntCap = 1536;     // stream entries staged in LDS per block
constexpr int kMaxBlk = 256;      // blocks held in a workgroup's run table

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

SpmmPlan spmm_plan(int64_t T, int n_src, int n_out, int64_t nnz, bool dc, bool stage16) {
  (void)nnz;
  SpmmPlan pl;
  // wave-uniform rows: 256-token tiles, 64-column blocks; the plain product
  // walks entry pairs (segments padded to even lengths), the one with dc
  // partials single entries (one partial per real entry)
  pl.kind = dc ? 2 : 1;
  pl.tt = kRT;
  pl.jb = dc && stage16 ? kRJB16 : kRJB;
  pl.esz = dc && stage16 ? 2 : 4;
  pl.rows_wg = dc ? kRW * kRRdc : kRW * kRR;
  pl.seg_mult = dc ? 1 : 2;
  pl.nblk = (n_src + pl.jb - 1) / pl.jb;
  pl.ntiles = (T + pl.tt - 1) / pl.tt;
  const int n_out_pad = (n_out + pl.rows_wg - 1) / pl.rows_wg * pl.rows_wg;
  pl.ptr_stride = n_out_pad + 1;
  return pl;
}

// prep layout: [stream int2 x (cap+pad)] [korig int32 x cap]
//              [bptr int32 x n_out*(nblk+1)] [ptr int32 x nblk*ptr_stride] [base int32 x nblk+1]
struct PrepLayout {
  size_t stream, korig, bptr, ptr, base, total;
  int64_t cap;   // stream entries (padding included)
};

// Every (row, block) segment is padded with zero entries (LDS offset 0,
// value 0) to a multiple of seg_mult: at most seg_mult - 1 per nonempty
// segment, so at most (seg_mult - 1) * min(segments, nnz) in all.
static int64_t stream_cap(int64_t nnz, int n_out, const SpmmPlan& pl) {
  const int64_t segs = static_cast<int64_t>(n_out) * pl.nblk;
  return nnz + static_cast<int64_t>(pl.seg_mult - 1) * (segs < nnz ? segs : nnz);
}
static PrepLayout prep_layout(int64_t nnz, int n_out, const SpmmPlan& pl) {
  PrepLayout l;
  l.stream = 0;
  l.cap = stream_cap(nnz, n_out, pl);
  l.korig = align256(static_cast<size_t>(l.cap + kPad) * 8);
  l.bptr = l.korig + align256(static_cast<size_t>(l.cap) * 4);
  l.ptr = l.bptr + align256(static_cast<size_t>(n_out) * (pl.nblk + 1) * 4);
  l.base = l.ptr + align256(static_cast<size_t>(pl.nblk) * pl.ptr_stride * 4);
  l.total = l.base + align256(static_cast<size_t>(pl.nblk + 1) * 4);
  return l;
}

size_t spmm_prep_bytes(int64_t nnz, int n_out, const SpmmPlan& pl) {
  return prep_layout(nnz, n_out, pl).total;
}

const int32_t* spmm_prep_korig(const void* prep, int64_t nnz, int n_out, const SpmmPlan& pl) {
  return reinterpret_cast<const int32_t*>(static_cast<const char*>(prep) +
                                          prep_layout(nnz, n_out, pl).korig);
}

template <typename T>
static T* at(void* prep, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(prep) + off);
}

// ------------------------------------------------------------ prep
// Segment o of the source structure: positions [seg_ptr[o], seg_ptr[o+1]);
// the source column of position q is E[2q+1] (rows of F) or E[2 perm[q]]
// (columns of F, perm = csc_perm); columns ascend within a segment.
__device__ __forceinline__ int seg_key(const int32_t* E, const int32_t* perm, int64_t q) {
  return perm ? E[2 * static_cast<int64_t>(perm[q])] : E[2 * q + 1];
}

// bptr[o][b] = first position of segment o whose column is >= b*JB
// (b = 0 .. nblk; bptr[o][nblk] is the segment's end)
__global__ void bptr_kernel(const int32_t* __restrict__ seg_ptr, const int32_t* __restrict__ E,
                            const int32_t* __restrict__ perm, int n_out, int nblk, int jb,
                            int32_t* __restrict__ bptr) {
  const int64_t id = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(n_out) * (nblk + 1);
  if (id >= total) return;
  const int o = static_cast<int>(id / (nblk + 1));
  const int b = static_cast<int>(id % (nblk + 1));
  int lo = seg_ptr[o], hi = seg_ptr[o + 1];
  const int target = b * jb;
  while (lo < hi) {
    const int mid = lo + ((hi - lo) >> 1);
    if (seg_key(E, perm, mid) < target) lo = mid + 1; else hi = mid;
  }
  bptr[id] = lo;
}

// Per block b: ptr[b][o] = entries of block b in rows before o (exclusive
// scan over rows of the counts padded to a multiple of mult), ptr[b][n_rows]
// and base[b] = the block's total. Rows n_out .. stride-2 (padding up to a
// whole workgroup of rows) are empty.
__global__ __launch_bounds__(1024) void blk_scan_kernel(const int32_t* __restrict__ bptr,
                                                        int n_out, int stride, int nblk, int mult,
                                                        int32_t* __restrict__ ptr,
                                                        int32_t* __restrict__ base) {
  __shared__ int wsum[16];
  __shared__ int carry;
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  int32_t* pb = ptr + static_cast<int64_t>(b) * stride;
  const int n_rows = stride - 1;
  for (int o0 = 0; o0 < n_rows; o0 += 1024) {
    const int o = o0 + threadIdx.x;
    int cnt = 0;
    if (o < n_out) {
      const int64_t r = static_cast<int64_t>(o) * (nblk + 1) + b;
      cnt = bptr[r + 1] - bptr[r];
      cnt = (cnt + mult - 1) / mult * mult;
    }
    const int incl = wave_incl_scan_i32(cnt);
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    int before = 0, all = 0;
    for (int i = 0; i < 16; ++i) {
      const int v = wsum[i];
      if (i < wid) before += v;
      all += v;
    }
    if (o < n_rows) pb[o] = carry + before + incl - cnt;
    __syncthreads();
    if (threadIdx.x == 0) carry += all;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    pb[n_rows] = carry;
    base[b] = carry;
  }
}

// base[b] <- exclusive scan of the block totals (base[nblk] = stream length)
__global__ __launch_bounds__(1024) void blk_base_kernel(int32_t* __restrict__ base, int nblk) {
  __shared__ int wsum[16];
  __shared__ int carry;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int b0 = 0; b0 < nblk; b0 += 1024) {
    const int b = b0 + threadIdx.x;
    const int v = (b < nblk) ? base[b] : 0;
    const int incl = wave_incl_scan_i32(v);
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    int before = 0, all = 0;
    for (int i = 0; i < 16; ++i) {
      const int x = wsum[i];
      if (i < wid) before += x;
      all += x;
    }
    __syncthreads();
    if (b < nblk) base[b] = carry + before + incl - v;
    __syncthreads();
    if (threadIdx.x == 0) carry += all;
    __syncthreads();
  }
  if (threadIdx.x == 0) base[nblk] = carry;
}

// Scatter every nonzero into the column-block-major stream.
// Rows of F: position q = k, row o = E[2k], column E[2k+1], value c[k].
// Columns of F: position q, row o = E[2 perm[q] + 1] (a column of F),
// column E[2 perm[q]] (a row of F), value c[perm[q]].
// korig[pos] (if given) keeps the nonzero's index k in E. The last entry of
// a segment whose padded length exceeds its count writes the zero padding
// entries (offset 0, value 0, korig -1); thread 0 zeroes the kPad entries
// past the stream's end.
__global__ void scatter_kernel(const int32_t* __restrict__ E, const float* __restrict__ c,
                               const int32_t* __restrict__ perm, int64_t nnz, int stride,
                               int nblk, int jb, int tt, int esz, int mult,
                               const int32_t* __restrict__ bptr,
                               const int32_t* __restrict__ ptr, const int32_t* __restrict__ base,
                               int2* __restrict__ stream, int32_t* __restrict__ korig) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q == 0) {
    const int64_t end = base[nblk];
    for (int i = 0; i < kPad; ++i) stream[end + i] = make_int2(0, 0);
  }
  if (q >= nnz) return;
  const int64_t k = perm ? perm[q] : q;
  const int o = perm ? E[2 * k + 1] : E[2 * k];
  const int col = perm ? E[2 * k] : E[2 * k + 1];
  const int b = col / jb;
  const int64_t r = static_cast<int64_t>(o) * (nblk + 1) + b;
  const int first = bptr[r];
  const int64_t pos = static_cast<int64_t>(base[b]) +
                      ptr[static_cast<int64_t>(b) * stride + o] + (q - first);
  stream[pos] = make_int2((col - b * jb) * tt * esz, c ? __float_as_int(c[k]) : 0);
  if (korig) korig[pos] = static_cast<int32_t>(k);
  if (mult > 1) {
    const int last = bptr[r + 1] - 1;
    if (q == last) {
      const int cnt = last + 1 - first;
      const int pad = (cnt + mult - 1) / mult * mult - cnt;
      for (int i = 1; i <= pad; ++i) {
        stream[pos + i] = make_int2(0, 0);
        if (korig) korig[pos + i] = -1;
      }
    }
  }
}

static hipError_t prep_common(const int32_t* seg_ptr, const int32_t* E, const float* c,
                              const int32_t* perm, int n_out, int64_t nnz, const SpmmPlan& pl,
                              bool with_korig, void* prep, hipStream_t s) {
  const PrepLayout l = prep_layout(nnz, n_out, pl);
  int32_t* bptr = at<int32_t>(prep, l.bptr);
  int32_t* ptr = at<int32_t>(prep, l.ptr);
  int32_t* base = at<int32_t>(prep, l.base);
  const int64_t nb = static_cast<int64_t>(n_out) * (pl.nblk + 1);
  hipLaunchKernelGGL(bptr_kernel, dim3(static_cast<unsigned>((nb + 255) / 256)), dim3(256), 0, s,
                     seg_ptr, E, perm, n_out, pl.nblk, pl.jb, bptr);
  hipLaunchKernelGGL(blk_scan_kernel, dim3(pl.nblk), dim3(1024), 0, s, bptr, n_out,
                     pl.ptr_stride, pl.nblk, pl.seg_mult, ptr, base);
  hipLaunchKernelGGL(blk_base_kernel, dim3(1), dim3(1024), 0, s, base, pl.nblk);
  const int64_t nthreads = nnz > 0 ? nnz : 1;
  hipLaunchKernelGGL(scatter_kernel, dim3(static_cast<unsigned>((nthreads + 255) / 256)), dim3(256),
                     0, s, E, c, perm, nnz, pl.ptr_stride, pl.nblk, pl.jb, pl.tt, pl.esz,
                     pl.seg_mult, bptr, ptr, base, at<int2>(prep, l.stream),
                     with_korig ? at<int32_t>(prep, l.korig) : nullptr);
  return hipGetLastError();
}

hipError_t launch_prep_csr(const int32_t* row_ptr, const int32_t* E, const float* c, int d_out,
                           int64_t nnz, const SpmmPlan& pl, void* prep, hipStream_t s) {
  return prep_common(row_ptr, E, c, nullptr, d_out, nnz, pl, false, prep, s);
}

hipError_t launch_prep_csc(const int32_t* col_ptr, const int32_t* perm, const int32_t* E,
                           const float* c, int d_in, int64_t nnz, const SpmmPlan& pl, void* prep,
                           hipStream_t s) {
  return prep_common(col_ptr, E, c, perm, d_in, nnz, pl, true, prep, s);
}

// ------------------------------------------------------------ cached structure
// A prepared stream whose positions depend only on E (frozen after the init):
// the structure is built once, with korig kept in both directions, and each
// call only gathers the current values, stream[q].value = c[korig[q]] (0 for
// the padding entries). The stream's length is base[nblk], read on the device.
hipError_t launch_prep_structure(const int32_t* seg_ptr, const int32_t* E, const int32_t* perm,
                                 int n_out, int64_t nnz, const SpmmPlan& pl, void* prep,
                                 hipStream_t s) {
  return prep_common(seg_ptr, E, nullptr, perm, n_out, nnz, pl, true, prep, s);
}

__global__ void refresh_values_kernel(int2* __restrict__ stream, const int32_t* __restrict__ korig,
                                      const float* __restrict__ c,
                                      const int32_t* __restrict__ end, int64_t cap) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= cap || q >= static_cast<int64_t>(*end)) return;
  const int k = korig[q];
  stream[q].y = k >= 0 ? __float_as_int(c[k]) : 0;
}

hipError_t launch_prep_refresh(const float* c, int64_t nnz, int n_out, const SpmmPlan& pl,
                               void* prep, hipStream_t s) {
  const PrepLayout l = prep_layout(nnz, n_out, pl);
  if (l.cap == 0) return hipSuccess;
  hipLaunchKernelGGL(refresh_values_kernel, dim3(static_cast<unsigned>((l.cap + 255) / 256)),
                     dim3(256), 0, s, at<int2>(prep, l.stream), at<int32_t>(prep, l.korig), c,
                     at<int32_t>(prep, l.base) + pl.nblk, l.cap);
  return hipGetLastError();
}

// ------------------------------------------------------------ helpers
template <int N>
__device__ __forceinline__ float dpp_row_shr(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + N, 0xF, 0xF, true));
}

// ------------------------------------------------------------ wave-uniform rows
// Plain SpMM (no dc partials). A workgroup of 16 waves owns a tile of 256
// tokens and 256 output rows; wave w owns rows row0 .. row0+15 and lane l
// owns tokens 4l .. 4l+3 of the tile, so a row's segment is the same for the
// whole wave: its entries are read from the run staged in LDS (one broadcast
// read per pair of entries, issued a pair ahead) and each costs one
// conflict-free ds_read_b128 (1 KiB per wave), one address add and four FMAs.
// No entry is masked; segments are padded with zero entries to even lengths.
//
// Staging: block b of 64 source columns is held token-minor (row jj of the
// block is the 256 tokens of column jj), double buffered; thread tid loads
// 16 columns of token tid % 256 (16-byte loads), the next block's loads are
// in flight while the current block is consumed.
template <typename SrcT, bool VEC_OK>
struct StageRows {
  static constexpr int VEC = 16 / static_cast<int>(sizeof(SrcT));  // elements per 16 bytes
  static constexpr int NL = 16 / VEC;                                // 16-byte loads per thread
  static constexpr int NH = NL / 2;                                  // loads per half
  uint4 raw[NH];

  // Block b lies wholly inside the source and the tile wholly inside T:
  // no clamping and no zeroing (uniform).
  static __device__ __forceinline__ bool whole(int64_t T, int n_src, int64_t t0, int b) {
    return VEC_OK && t0 + kRT <= T && (b + 1) * kRJB <= n_src;
  }

  // half h covers the thread's columns g*16 + h*8 .. +7
  __device__ __forceinline__ void load(const SrcT* __restrict__ src, int64_t T, int n_src,
                                       int64_t t0, int b, int h) {
    const int tt = threadIdx.x & (kRT - 1);
    const int g = threadIdx.x / kRT;
    if (whole(T, n_src, t0, b)) {
      const SrcT* row = src + (t0 + tt) * n_src + b * kRJB + g * 16 + h * 8;
#pragma unroll
      for (int q = 0; q < NH; ++q) raw[q] = *reinterpret_cast<const uint4*>(row + q * VEC);
      return;
    }
    const int64_t t = t0 + tt < T ? t0 + tt : T - 1;
    const SrcT* row = src + t * n_src;
#pragma unroll
    for (int q = 0; q < NH; ++q) {
      const int col = b * kRJB + g * 16 + h * 8 + q * VEC;
      if constexpr (VEC_OK) {
        const int cc = col + VEC <= n_src ? col : n_src - VEC;
        raw[q] = *reinterpret_cast<const uint4*>(row + cc);
      } else {
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int cc = col + e < n_src ? col + e : n_src - 1;
          if constexpr (sizeof(SrcT) == 4) {
            w[e] = __float_as_uint(reinterpret_cast<const float*>(row)[cc]);
          } else {
            const uint32_t bits = reinterpret_cast<const uint16_t*>(row)[cc];
            w[e >> 1] |= bits << (16 * (e & 1));
          }
        }
        raw[q] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }

  static __device__ __forceinline__ float elem(const uint32_t (&w)[4], int e) {
    if constexpr (sizeof(SrcT) == 4) return __uint_as_float(w[e]);
    else return (e & 1) ? __uint_as_float(w[e >> 1] & 0xFFFF0000u) : __uint_as_float(w[e >> 1] << 16);
  }

  __device__ __forceinline__ void store(float* __restrict__ st, int64_t T, int n_src, int64_t t0,
                                        int b, int h) const {
    const int tt = threadIdx.x & (kRT - 1);
    const int g = threadIdx.x / kRT;
    if (whole(T, n_src, t0, b)) {
#pragma unroll
      for (int q = 0; q < NH; ++q) {
        const int cl = g * 16 + h * 8 + q * VEC;
        const uint32_t w[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
        for (int e = 0; e < VEC; ++e) st[(cl + e) * kRT + tt] = elem(w, e);
      }
      return;
    }
    const bool tok_ok = t0 + tt < T;
#pragma unroll
    for (int q = 0; q < NH; ++q) {
      const int cl = g * 16 + h * 8 + q * VEC;
      const int col = b * kRJB + cl;
      const uint32_t w[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const bool ok = tok_ok && (VEC_OK ? (col + VEC <= n_src) : (col + e < n_src));
        st[(cl + e) * kRT + tt] = ok ? elem(w, e) : 0.f;
      }
    }
  }
};

// 16 consecutive outputs at a 16-byte aligned address (+= when accumulate)
__device__ __forceinline__ void store_row16(float* dst, const float (&v)[16], int accumulate) {
  float4* d = reinterpret_cast<float4*>(dst);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float4 o = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    if (accumulate) {
      const float4 a = d[j];
      o.x += a.x; o.y += a.y; o.z += a.z; o.w += a.w;
    }
    d[j] = o;
  }
}

__device__ __forceinline__ void store_row16(uint16_t* dst, const float (&v)[16], int accumulate) {
  uint4* d = reinterpret_cast<uint4*>(dst);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = v[8 * j + e];
    if (accumulate) {
      const uint4 a = d[j];
      const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        f[e] += bf16_to_f32(static_cast<uint16_t>((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu)));
    }
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = static_cast<uint32_t>(f32_to_bf16(f[2 * e])) |
             (static_cast<uint32_t>(f32_to_bf16(f[2 * e + 1])) << 16);
    d[j] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__device__ __forceinline__ void fma4(float (&a)[4], float v, const float4& z) {
  a[0] = fmaf(v, z.x, a[0]);
  a[1] = fmaf(v, z.y, a[1]);
  a[2] = fmaf(v, z.z, a[2]);
  a[3] = fmaf(v, z.w, a[3]);
}

// A group of up to four consecutive entries: ea = entries 0, 1 and eb =
// entries 2, 3 as (LDS byte offset, value bits) pairs.
__device__ __forceinline__ float4 lds4(const char* sb, int off) {
  return *reinterpret_cast<const float4*>(sb + off);
}

// The wave's rows in one block: row r owns pairs [sg[r], sg[r+1]) of the
// workgroup's run (segments are padded to even lengths), of which pairs
// [c0, c0 + kEntCap / 2) are staged in pp as (offset0, offset1, value0,
// value1). The wave walks its pairs in order across its rows, reading the
// next pair while the current pair's z reads are in flight, so a row's first
// pair is already in registers when the row starts. mid() runs once, after
// half the rows.
template <typename Mid>
__device__ __forceinline__ void rows_pairs(float (&acc)[kRR][4], const int (&sg)[kRR + 1],
                                           int c0, const char* sb, const int4* pp, Mid mid) {
  const int c1 = c0 + kEntCap / 2;
  const int4* pc = pp - c0;
  auto clampc = [&](int v) { return v < c0 ? c0 : (v > c1 ? c1 : v); };
  int4 cur = pc[clampc(sg[0])];
#pragma unroll
  for (int r = 0; r < kRR; ++r) {
    const int hi = clampc(sg[r + 1]);
    for (int i = clampc(sg[r]); i < hi; ++i) {
      const int4 nx = pc[i + 1];
      const float4 z0 = lds4(sb, cur.x);
      const float4 z1 = lds4(sb, cur.y);
      fma4(acc[r], __int_as_float(cur.z), z0);
      fma4(acc[r], __int_as_float(cur.w), z1);
      cur = nx;
    }
    if (r == kMidF - 1) mid();
  }
}

// Per-block metadata of a workgroup of ROWS rows: the rows' segment bounds
// relative to the start k0 of the workgroup's run of the stream, and the
// run's first kEntCap entries. SPLIT = false: staged as pairs (offset0,
// offset1, value0, value1); SPLIT = true: as an array of offsets followed by
// an array of values (kEntCap + 2 each). Longer runs are restaged in chunks.
template <int ROWS, bool SPLIT>
struct RowsMeta {
  int seg;     // thread tid <= ROWS: bound of row tid, before subtracting p0
  int p0;      // the run's block-local start
  int4 pair;   // thread tid <= kEntCap / 2: pair tid of the run
  int k0;      // uniform
  // Run table of a workgroup, one int4 per block: (k0, the block-local
  // start p0, the run length). Built once per workgroup so that a block's
  // staging waits for one table read, not a chain of scalar loads.
  static __device__ __forceinline__ void build_runs(int4* runs, const int32_t* __restrict__ ptr,
                                                    const int32_t* __restrict__ base,
                                                    int ptr_stride, int rg0, int nblk) {
    for (int b = threadIdx.x; b < nblk; b += blockDim.x) {
      const int32_t* pb = ptr + static_cast<int64_t>(b) * ptr_stride + rg0;
      const int p0 = pb[0];
      runs[b] = make_int4(base[b] + p0, p0, pb[ROWS] - p0, 0);
    }
  }
  // with_table: the run table holds every block (nblk <= kMaxBlk); else the
  // run is read from ptr / base directly.
  __device__ __forceinline__ void load(const int2* __restrict__ stream,
                                       const int32_t* __restrict__ ptr,
                                       const int32_t* __restrict__ base, const int4* runs,
                                       bool with_table, int ptr_stride, int rg0, int b) {
    const int32_t* pb = ptr + static_cast<int64_t>(b) * ptr_stride + rg0;
    int cnt;
    if (with_table) {
      const int4 rb = runs[b];
      k0 = uniform(rb.x);
      p0 = rb.y;
      cnt = rb.z;
    } else {
      p0 = pb[0];
      k0 = base[b] + p0;
      cnt = pb[ROWS] - p0;
    }
    const int tid = threadIdx.x;
    // raw: subtracting p0 here would make the compiler wait for this load
    // (and every load issued before it) at once; store() does it instead
    seg = tid <= ROWS ? pb[tid] : 0;
    // the stream is padded past its end, so a pair may straddle the run's
    // end; pair kEntCap / 2 (read past the staged run, never used) is zero
    pair = 2 * tid < cnt && tid < kEntCap / 2
               ? *reinterpret_cast<const int4*>(stream + k0 + 2 * tid)
               : make_int4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void store(int* segs, int4* pairs) const {
    const int tid = threadIdx.x;
    if (tid <= ROWS) segs[tid] = seg - p0;
    if (tid < kEntCap / 2 + 1) store_pair(pairs, tid, pair);
  }
  static __device__ __forceinline__ void store_pair(int4* pairs, int t, const int4& e) {
    if constexpr (SPLIT) {
      int* offs = reinterpret_cast<int*>(pairs);
      int* vals = offs + kEntCap + 2;
      *reinterpret_cast<int2*>(offs + 2 * t) = make_int2(e.x, e.z);
      *reinterpret_cast<int2*>(vals + 2 * t) = make_int2(e.y, e.w);
    } else {
      pairs[t] = make_int4(e.x, e.z, e.y, e.w);
    }
  }
};

template <typename SrcT, typename OutT, bool VEC_OK>
__global__ __launch_bounds__(kRW * 64) void rows_kernel(
    const SrcT* __restrict__ src, int64_t T, int n_src, const int2* __restrict__ stream,
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ base, int n_out, int ptr_stride,
    int nblk, float alpha, OutT* __restrict__ out, int accumulate) {
  __shared__ float stage[2][kRJB * kRT];
  __shared__ int4 pairs[2][kEntCap / 2 + 1];   // + entries read past the end
  __shared__ int segs[2][kRW * kRR + 1];
  __shared__ int4 runs[kMaxBlk];
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRT;
  const int rg0 = static_cast<int>(blockIdx.y) * (kRW * kRR);
  const int row0 = rg0 + w * kRR;

  float acc[kRR][4];
#pragma unroll
  for (int r = 0; r < kRR; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[r][q] = 0.f;

  StageRows<SrcT, VEC_OK> pf;
  RowsMeta<kRW * kRR, false> meta;
  const bool tab = nblk <= kMaxBlk;
  if (tab) RowsMeta<kRW * kRR, false>::build_runs(runs, ptr, base, ptr_stride, rg0, nblk);
  __syncthreads();
  meta.load(stream, ptr, base, runs, tab, ptr_stride, rg0, 0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    pf.load(src, T, n_src, t0, 0, h);
    pf.store(stage[0], T, n_src, t0, 0, h);
  }
  meta.store(segs[0], pairs[0]);
  int k0n = meta.k0;   // k0 of the block staged next
  if (nblk > 1) {
    pf.load(src, T, n_src, t0, 1, 0);
    meta.load(stream, ptr, base, runs, tab, ptr_stride, rg0, 1);
  }
  for (int b = 0; b < nblk; ++b) {
    __syncthreads();
    const int k0 = k0n;
    const bool more = b + 1 < nblk;
    const int nb = b + 1;
    float* nst = stage[nb & 1];
    const int buf = b & 1;
    int sg[kRR + 1];
#pragma unroll
    for (int r = 0; r <= kRR; ++r) sg[r] = uniform(segs[buf][w * kRR + r]) >> 1;
    const char* sb = reinterpret_cast<const char*>(stage[buf]) + lane * 16;
    auto mid = [&]() {
      if (more) {
        pf.store(nst, T, n_src, t0, nb, 0);
        pf.load(src, T, n_src, t0, nb, 1);
      }
    };
    // Runs longer than the staged cap go in chunks of kEntCap / 2 pairs,
    // restaged from the stream between barriers (all waves take part).
    const int run = uniform(segs[buf][kRW * kRR]) >> 1;
    rows_pairs(acc, sg, 0, sb, pairs[buf], mid);
    for (int c0 = kEntCap / 2; c0 < run; c0 += kEntCap / 2) {
      __syncthreads();
      const int t = threadIdx.x;
      if (t < kEntCap / 2) {
        const int4 e = c0 + t < run ? *reinterpret_cast<const int4*>(stream + k0 + 2 * (c0 + t))
                                    : make_int4(0, 0, 0, 0);
        RowsMeta<kRW * kRR, false>::store_pair(pairs[buf], t, e);
      }
      __syncthreads();
      rows_pairs(acc, sg, c0, sb, pairs[buf], [] {});
    }
    if (more) {
      pf.store(nst, T, n_src, t0, nb, 1);
      meta.store(segs[nb & 1], pairs[nb & 1]);
      k0n = meta.k0;
      if (nb + 1 < nblk) {   // registers only: nothing in LDS is touched
        pf.load(src, T, n_src, t0, nb + 1, 0);
        meta.load(stream, ptr, base, runs, tab, ptr_stride, rg0, nb + 1);
      }
    }
  }

  // epilogue: lane writes rows row0 .. row0+15 (contiguous) of its 4 tokens,
  // as 16-byte stores when the rows are whole and aligned
  constexpr int kVec = 16 / static_cast<int>(sizeof(OutT));
  const bool vec = row0 + kRR <= n_out && n_out % kVec == 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = t0 + 4 * lane + q;
    if (t >= T) continue;
    OutT* dst = out + t * n_out;
    if (vec) {
      float v[kRR];
#pragma unroll
      for (int r = 0; r < kRR; ++r) v[r] = alpha * acc[r][q];
      store_row16(dst + row0, v, accumulate);
    } else {
#pragma unroll
      for (int r = 0; r < kRR; ++r) {
        const int o = row0 + r;
        if (o < n_out) {
          float val = alpha * acc[r][q];
          if (accumulate) val += Elem<OutT>::ld(dst, o);
          Elem<OutT>::st(dst, o, val);
        }
      }
    }
  }
}

// ------------------------------------------------------------ rows with dc
// Backward through the columns of F with the dc partials. Rows are the
// columns j of F (outputs dz[:, j]), the source is dy; a wave owns 8 rows and
// also holds z[t, j] of its rows for its 4 tokens. Per entry (row i of F,
// value c, column j): dz[t, j] += c * dy[t, i] (4 FMAs) and the entry's
// partial of dc over the tile's 256 tokens, sum_t dy[t, i] z[t, j]: a 4-term
// dot per lane, summed across the wave by DPP into lane 63, which stores it
// at the entry's stream position. Entries go one at a time (no padding); the
// next entry's offset is read while this entry's LDS read is in flight and
// its value after this entry's FMAs.

__device__ __forceinline__ float wave_total_lane63(float v) {
  v += dpp_row_shr<1>(v);
  v += dpp_row_shr<2>(v);
  v += dpp_row_shr<4>(v);
  v += dpp_row_shr<8>(v);   // lane 15 of each row of 16: the row's sum
  // row_bcast:15 then row_bcast:31 on every row: lane 63 gathers rows 0-2
  // (the other lanes end with partial sums that are not used)
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xF, 0xF, true));
  return v;   // lane 63: the sum over all 64 lanes
}

// The 4 tokens of a lane from a staged row: fp32 (16 bytes) or bf16 kept as
// bf16 (8 bytes, widened exactly: a bf16 is the top half of its fp32).
template <bool B16>
__device__ __forceinline__ float4 lds_tok4(const char* sb, int off) {
  if constexpr (B16) {
    const uint2 q = *reinterpret_cast<const uint2*>(sb + off);
    return make_float4(__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xFFFF0000u),
                       __uint_as_float(q.y << 16), __uint_as_float(q.y & 0xFFFF0000u));
  } else {
    return *reinterpret_cast<const float4*>(sb + off);
  }
}

// Entries are taken two at a time in stream order: a pair inside row RA, or
// straddling from RA into the next row RB (RA's last entry and RB's first).
// (off, val) hold the pair's offsets and values; the next pair's offsets are
// read while this pair's LDS reads are in flight and its values after the
// FMAs. Lane 63 stores the two dc partials.
template <int RA, int RB, bool B16>
__device__ __forceinline__ void dc_pair(float (&acc)[kRRdc][4], const float (&zr)[kRRdc][4],
                                        const char* sb, const int* offs, const int* vals, int j,
                                        int2& off, int2& val, float* __restrict__ prow, int i,
                                        int lane) {
  const float4 z0 = lds_tok4<B16>(sb, off.x);
  const float4 z1 = lds_tok4<B16>(sb, off.y);
  off = make_int2(offs[j + 2], offs[j + 3]);
  asm volatile("" ::: "memory");
  fma4(acc[RA], __int_as_float(val.x), z0);
  fma4(acc[RB], __int_as_float(val.y), z1);
  val = make_int2(vals[j + 2], vals[j + 3]);
  asm volatile("" ::: "memory");
  float d0 = z0.x * zr[RA][0], d1 = z1.x * zr[RB][0];
  d0 = fmaf(z0.y, zr[RA][1], d0);
  d1 = fmaf(z1.y, zr[RB][1], d1);
  d0 = fmaf(z0.z, zr[RA][2], d0);
  d1 = fmaf(z1.z, zr[RB][2], d1);
  d0 = fmaf(z0.w, zr[RA][3], d0);
  d1 = fmaf(z1.w, zr[RB][3], d1);
  d0 = wave_total_lane63(d0);
  d1 = wave_total_lane63(d1);
  if (lane == 63) {
    prow[i] = d0;
    prow[i + 1] = d1;
  }
}

// One entry of row RA (its row's last, with no next row to pair with).
template <int RA, bool B16>
__device__ __forceinline__ void dc_single(float (&acc)[kRRdc][4], const float (&zr)[kRRdc][4],
                                          const char* sb, const int* offs, const int* vals, int j,
                                          int2& off, int2& val, float* __restrict__ prow, int i,
                                          int lane) {
  const float4 z0 = lds_tok4<B16>(sb, off.x);
  off = make_int2(offs[j + 1], offs[j + 2]);
  asm volatile("" ::: "memory");
  fma4(acc[RA], __int_as_float(val.x), z0);
  val = make_int2(vals[j + 1], vals[j + 2]);
  asm volatile("" ::: "memory");
  float d0 = z0.x * zr[RA][0];
  d0 = fmaf(z0.y, zr[RA][1], d0);
  d0 = fmaf(z0.z, zr[RA][2], d0);
  d0 = fmaf(z0.w, zr[RA][3], d0);
  d0 = wave_total_lane63(d0);
  if (lane == 63) prow[i] = d0;
}

// The wave's rows in one block: row r owns entries [sg[r], sg[r+1]) of the
// workgroup's run, of which [c0, c0 + kEntCap) are staged (offs, vals).
template <bool B16, typename Mid>
__device__ __forceinline__ void rows_entries_dc(float (&acc)[kRRdc][4],
                                                const float (&zr)[kRRdc][4],
                                                const int (&sg)[kRRdc + 1], int c0,
                                                const char* sb, const int4* staged,
                                                float* __restrict__ prow, int lane, Mid mid) {
  const int c1 = c0 + kEntCap;
  const int* offs = reinterpret_cast<const int*>(staged) - c0;
  const int* vals = reinterpret_cast<const int*>(staged) + kEntCap + 2 - c0;
  auto clampc = [&](int v) { return v < c0 ? c0 : (v > c1 ? c1 : v); };
  int i = clampc(sg[0]);
  int2 off = make_int2(offs[i], offs[i + 1]);
  int2 val = make_int2(vals[i], vals[i + 1]);
  asm volatile("" ::: "memory");
  static_for<0, kRRdc>([&](auto rc) {
    constexpr int r = decltype(rc)::value;
    const int hi = clampc(sg[r + 1]);
    for (; i + 1 < hi; i += 2)
      dc_pair<r, r, B16>(acc, zr, sb, offs, vals, i, off, val, prow, i, lane);
    if (i < hi) {
      bool paired = false;
      if constexpr (r + 1 < kRRdc) {
        if (i + 1 < clampc(sg[r + 2])) {   // row r+1 is not empty: pair across
          dc_pair<r, r + 1, B16>(acc, zr, sb, offs, vals, i, off, val, prow, i, lane);
          i += 2;
          paired = true;
        }
      }
      if (!paired) {
        dc_single<r, B16>(acc, zr, sb, offs, vals, i, off, val, prow, i, lane);
        i += 1;
      }
    }
    if (r == kMidB - 1) mid();
  });
}

template <typename SrcT, bool VEC_OK>
__global__ __launch_bounds__(kRW * 64) void rows_dc_kernel(
    const SrcT* __restrict__ src, int64_t T, int n_src, const int2* __restrict__ stream,
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ base, int64_t nnz, int n_out,
    int ptr_stride, int nblk, float* __restrict__ out, const float* __restrict__ zsrc,
    float* __restrict__ partial, float alpha, int accumulate) {
  __shared__ float stage[2][kRJB * kRT];
  __shared__ int4 pairs[2][kEntCap / 2 + 1];   // + the entries read past the end
  __shared__ int segs[2][kRW * kRRdc + 1];
  __shared__ int4 runs[kMaxBlk];
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int64_t tile = blockIdx.x;
  const int64_t t0 = tile * kRT;
  const int rg0 = static_cast<int>(blockIdx.y) * (kRW * kRRdc);
  const int row0 = rg0 + w * kRRdc;

  float acc[kRRdc][4], zr[kRRdc][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = t0 + 4 * lane + q;
#pragma unroll
    for (int r = 0; r < kRRdc; ++r) {
      acc[r][q] = 0.f;
      zr[r][q] = (t < T && row0 + r < n_out) ? zsrc[t * n_out + row0 + r] : 0.f;
    }
  }

  StageRows<SrcT, VEC_OK> pf;
  RowsMeta<kRW * kRRdc, true> meta;
  const bool tab = nblk <= kMaxBlk;
  if (tab) RowsMeta<kRW * kRRdc, true>::build_runs(runs, ptr, base, ptr_stride, rg0, nblk);
  __syncthreads();
  meta.load(stream, ptr, base, runs, tab, ptr_stride, rg0, 0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    pf.load(src, T, n_src, t0, 0, h);
    pf.store(stage[0], T, n_src, t0, 0, h);
  }
  meta.store(segs[0], pairs[0]);
  int k0n = meta.k0;   // k0 of the block staged next
  if (nblk > 1) {
    pf.load(src, T, n_src, t0, 1, 0);
    meta.load(stream, ptr, base, runs, tab, ptr_stride, rg0, 1);
  }
  for (int b = 0; b < nblk; ++b) {
    __syncthreads();
    const int k0 = k0n;
    const bool more = b + 1 < nblk;
    const int nb = b + 1;
    float* nst = stage[nb & 1];
    const int buf = b & 1;
    int sg[kRRdc + 1];
#pragma unroll
    for (int r = 0; r <= kRRdc; ++r) sg[r] = uniform(segs[buf][w * kRRdc + r]);
    const char* sb = reinterpret_cast<const char*>(stage[buf]) + lane * 16;
    float* prow = partial + tile * nnz + k0;
    auto mid = [&]() {
      if (more) {
        pf.store(nst, T, n_src, t0, nb, 0);
        pf.load(src, T, n_src, t0, nb, 1);
      }
    };
    const int run = uniform(segs[buf][kRW * kRRdc]);
    rows_entries_dc<false>(acc, zr, sg, 0, sb, pairs[buf], prow, lane, mid);
    for (int c0 = kEntCap; c0 < run; c0 += kEntCap) {
      __syncthreads();
      const int t = threadIdx.x;
      if (t < kEntCap / 2 + 1) {
        const int4 e = t < kEntCap / 2 && c0 + 2 * t < run
                           ? *reinterpret_cast<const int4*>(stream + k0 + c0 + 2 * t)
                           : make_int4(0, 0, 0, 0);
        RowsMeta<kRW * kRRdc, true>::store_pair(pairs[buf], t, e);
      }
      __syncthreads();
      rows_entries_dc<false>(acc, zr, sg, c0, sb, pairs[buf], prow, lane, [] {});
    }
    if (more) {
      pf.store(nst, T, n_src, t0, nb, 1);
      meta.store(segs[nb & 1], pairs[nb & 1]);
      k0n = meta.k0;
      if (nb + 1 < nblk) {   // registers only: nothing in LDS is touched
        pf.load(src, T, n_src, t0, nb + 1, 0);
        meta.load(stream, ptr, base, runs, tab, ptr_stride, rg0, nb + 1);
      }
    }
  }

  // epilogue. A whole tile goes through LDS, 128 tokens at a time, laid out
  // [token][row] (stride 129 floats), so that each token's 128 outputs leave
  // as 512 contiguous bytes; otherwise each lane writes its own 8 rows.
  if (t0 + kRT <= T && rg0 + kRW * kRRdc <= n_out && n_out % 4 == 0) {
    constexpr int kEp = kRW * kRRdc + 1;
    float* ep = &stage[0][0];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __syncthreads();   // the staging buffers (or the previous half) are free
      if ((lane >> 5) == h) {
        const int lt = 4 * (lane & 31);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int r = 0; r < kRRdc; ++r) ep[(lt + q) * kEp + w * kRRdc + r] = acc[r][q];
      }
      __syncthreads();
      for (int task = threadIdx.x; task < (kRT / 2) * (kRW * kRRdc / 4); task += kRW * 64) {
        const int tt = task / (kRW * kRRdc / 4);
        const int c4 = task % (kRW * kRRdc / 4);
        const float* e = ep + tt * kEp + 4 * c4;
        float4* d = reinterpret_cast<float4*>(out + (t0 + (kRT / 2) * h + tt) * n_out + rg0 +
                                              4 * c4);
        float4 v = make_float4(alpha * e[0], alpha * e[1], alpha * e[2], alpha * e[3]);
        if (accumulate) {
          const float4 a = *d;
          v.x += a.x; v.y += a.y; v.z += a.z; v.w += a.w;
        }
        *d = v;
      }
    }
    return;
  }
  const bool vec = row0 + kRRdc <= n_out && n_out % 4 == 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = t0 + 4 * lane + q;
    if (t >= T) continue;
    float* dst = out + t * n_out;
    if (vec) {
      float4* d = reinterpret_cast<float4*>(dst + row0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float4 v = make_float4(alpha * acc[4 * h][q], alpha * acc[4 * h + 1][q],
                               alpha * acc[4 * h + 2][q], alpha * acc[4 * h + 3][q]);
        if (accumulate) {
          const float4 a = d[h];
          v.x += a.x; v.y += a.y; v.z += a.z; v.w += a.w;
        }
        d[h] = v;
      }
    } else {
#pragma unroll
      for (int r = 0; r < kRRdc; ++r)
        if (row0 + r < n_out)
          dst[row0 + r] = alpha * acc[r][q] + (accumulate ? dst[row0 + r] : 0.f);
    }
  }
}

// Staging of a 128-column block of a bf16 source kept as bf16: row jj of the
// block holds the 256 tokens of column jj as 128 dwords (tokens 2i and 2i+1
// in dword i), 512 bytes. Thread tid takes the token pair tp = tid % 128 and
// columns 16g .. 16g+15 (g = tid / 128) in two parts of 8: per part one
// 16-byte load per token and one dword store per column (a wave writes 256
// contiguous bytes of a row).
template <bool VEC_OK>
struct StageB16 {
  uint4 ra, rb;   // the part's 8 columns of tokens 2tp and 2tp+1

  static __device__ __forceinline__ bool whole(int64_t T, int n_src, int64_t t0, int b) {
    return VEC_OK && t0 + kRT <= T && (b + 1) * kRJB16 <= n_src;
  }

  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int64_t T, int n_src,
                                       int64_t t0, int b, int h) {
    const int tp = threadIdx.x & 127, g = threadIdx.x >> 7;
    const int col = b * kRJB16 + g * 16 + h * 8;
    const int64_t ta = t0 + 2 * tp;
    if (whole(T, n_src, t0, b)) {
      ra = *reinterpret_cast<const uint4*>(src + ta * n_src + col);
      rb = *reinterpret_cast<const uint4*>(src + (ta + 1) * n_src + col);
      return;
    }
    const int64_t tA = ta < T ? ta : T - 1, tB = ta + 1 < T ? ta + 1 : T - 1;
    if constexpr (VEC_OK) {
      // n_src is a multiple of 8: the part is wholly inside or wholly past it
      const int cc = col + 8 <= n_src ? col : n_src - 8;
      ra = *reinterpret_cast<const uint4*>(src + tA * n_src + cc);
      rb = *reinterpret_cast<const uint4*>(src + tB * n_src + cc);
    } else {
      uint32_t wa[4] = {0, 0, 0, 0}, wb[4] = {0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int cc = col + e < n_src ? col + e : n_src - 1;
        wa[e >> 1] |= static_cast<uint32_t>(src[tA * n_src + cc]) << (16 * (e & 1));
        wb[e >> 1] |= static_cast<uint32_t>(src[tB * n_src + cc]) << (16 * (e & 1));
      }
      ra = make_uint4(wa[0], wa[1], wa[2], wa[3]);
      rb = make_uint4(wb[0], wb[1], wb[2], wb[3]);
    }
  }

  __device__ __forceinline__ void store(uint32_t* __restrict__ st, int64_t T, int n_src, int64_t t0,
                                        int b, int h) const {
    const int tp = threadIdx.x & 127, g = threadIdx.x >> 7;
    const int cl = g * 16 + h * 8;
    const uint32_t a[4] = {ra.x, ra.y, ra.z, ra.w};
    const uint32_t c[4] = {rb.x, rb.y, rb.z, rb.w};
    if (whole(T, n_src, t0, b)) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        st[(cl + 2 * k) * (kRT / 2) + tp] = (a[k] & 0xFFFFu) | (c[k] << 16);
        st[(cl + 2 * k + 1) * (kRT / 2) + tp] = (a[k] >> 16) | (c[k] & 0xFFFF0000u);
      }
      return;
    }
    const uint32_t mA = t0 + 2 * tp < T ? 0xFFFFu : 0u;
    const uint32_t mB = t0 + 2 * tp + 1 < T ? 0xFFFF0000u : 0u;
    const int col = b * kRJB16 + cl;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bool ok = VEC_OK ? (col + 8 <= n_src) : (col + 2 * k + e < n_src);
        const uint32_t lo = e ? (a[k] >> 16) : (a[k] & 0xFFFFu);
        const uint32_t hi = e ? (c[k] & 0xFFFF0000u) : (c[k] << 16);
        st[(cl + 2 * k + e) * (kRT / 2) + tp] = ok ? ((lo & mA) | (hi & mB)) : 0u;
      }
    }
  }
};

// The backward with dc partials on a bf16 source, staged as bf16 in blocks
// of 128 columns (the same LDS bytes as 64 fp32 columns, twice the entries
// per row and block to walk between barriers); dy widens to fp32 exactly, so
// every product and sum is the same as rows_dc_kernel's.
template <bool VEC_OK>
__global__ __launch_bounds__(kRW * 64) void rows_dc16_kernel(
    const uint16_t* __restrict__ src, int64_t T, int n_src, const int2* __restrict__ stream,
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ base, int64_t nnz, int n_out,
    int ptr_stride, int nblk, float* __restrict__ out, const float* __restrict__ zsrc,
    float* __restrict__ partial, float alpha, int accumulate) {
  __shared__ __align__(16) uint32_t stage[2][kRJB16 * kRT / 2];
  __shared__ int4 pairs[2][kEntCap / 2 + 1];   // + the entries read past the end
  __shared__ int segs[2][kRW * kRRdc + 1];
  __shared__ int4 runs[kMaxBlk];
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int64_t tile = blockIdx.x;
  const int64_t t0 = tile * kRT;
  const int rg0 = static_cast<int>(blockIdx.y) * (kRW * kRRdc);
  const int row0 = rg0 + w * kRRdc;

  float acc[kRRdc][4], zr[kRRdc][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = t0 + 4 * lane + q;
#pragma unroll
    for (int r = 0; r < kRRdc; ++r) {
      acc[r][q] = 0.f;
      zr[r][q] = (t < T && row0 + r < n_out) ? zsrc[t * n_out + row0 + r] : 0.f;
    }
  }

  StageB16<VEC_OK> pf;
  RowsMeta<kRW * kRRdc, true> meta;
  const bool tab = nblk <= kMaxBlk;
  if (tab) RowsMeta<kRW * kRRdc, true>::build_runs(runs, ptr, base, ptr_stride, rg0, nblk);
  __syncthreads();
  meta.load(stream, ptr, base, runs, tab, ptr_stride, rg0, 0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    pf.load(src, T, n_src, t0, 0, h);
    pf.store(stage[0], T, n_src, t0, 0, h);
  }
  meta.store(segs[0], pairs[0]);
  int k0n = meta.k0;   // k0 of the block staged next
  if (nblk > 1) {
    pf.load(src, T, n_src, t0, 1, 0);
    meta.load(stream, ptr, base, runs, tab, ptr_stride, rg0, 1);
  }
  for (int b = 0; b < nblk; ++b) {
    __syncthreads();
    const int k0 = k0n;
    const bool more = b + 1 < nblk;
    const int nb = b + 1;
    uint32_t* nst = stage[nb & 1];
    const int buf = b & 1;
    int sg[kRRdc + 1];
#pragma unroll
    for (int r = 0; r <= kRRdc; ++r) sg[r] = uniform(segs[buf][w * kRRdc + r]);
    const char* sb = reinterpret_cast<const char*>(stage[buf]) + lane * 8;
    float* prow = partial + tile * nnz + k0;
    auto mid = [&]() {
      if (more) {
        pf.store(nst, T, n_src, t0, nb, 0);
        pf.load(src, T, n_src, t0, nb, 1);
      }
    };
    const int run = uniform(segs[buf][kRW * kRRdc]);
    rows_entries_dc<true>(acc, zr, sg, 0, sb, pairs[buf], prow, lane, mid);
    for (int c0 = kEntCap; c0 < run; c0 += kEntCap) {
      __syncthreads();
      const int t = threadIdx.x;
      if (t < kEntCap / 2 + 1) {
        const int4 e = t < kEntCap / 2 && c0 + 2 * t < run
                           ? *reinterpret_cast<const int4*>(stream + k0 + c0 + 2 * t)
                           : make_int4(0, 0, 0, 0);
        RowsMeta<kRW * kRRdc, true>::store_pair(pairs[buf], t, e);
      }
      __syncthreads();
      rows_entries_dc<true>(acc, zr, sg, c0, sb, pairs[buf], prow, lane, [] {});
    }
    if (more) {
      pf.store(nst, T, n_src, t0, nb, 1);
      meta.store(segs[nb & 1], pairs[nb & 1]);
      k0n = meta.k0;
      if (nb + 1 < nblk) {   // registers only: nothing in LDS is touched
        pf.load(src, T, n_src, t0, nb + 1, 0);
        meta.load(stream, ptr, base, runs, tab, ptr_stride, rg0, nb + 1);
      }
    }
  }

  // epilogue. A whole tile goes through LDS, 128 tokens at a time, laid out
  // [token][row] (stride 129 floats), so that each token's 128 outputs leave
  // as 512 contiguous bytes; otherwise each lane writes its own 8 rows.
  if (t0 + kRT <= T && rg0 + kRW * kRRdc <= n_out && n_out % 4 == 0) {
    constexpr int kEp = kRW * kRRdc + 1;
    float* ep = reinterpret_cast<float*>(&stage[0][0]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __syncthreads();   // the staging buffers (or the previous half) are free
      if ((lane >> 5) == h) {
        const int lt = 4 * (lane & 31);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int r = 0; r < kRRdc; ++r) ep[(lt + q) * kEp + w * kRRdc + r] = acc[r][q];
      }
      __syncthreads();
      for (int task = threadIdx.x; task < (kRT / 2) * (kRW * kRRdc / 4); task += kRW * 64) {
        const int tt = task / (kRW * kRRdc / 4);
        const int c4 = task % (kRW * kRRdc / 4);
        const float* e = ep + tt * kEp + 4 * c4;
        float4* d = reinterpret_cast<float4*>(out + (t0 + (kRT / 2) * h + tt) * n_out + rg0 +
                                              4 * c4);
        float4 v = make_float4(alpha * e[0], alpha * e[1], alpha * e[2], alpha * e[3]);
        if (accumulate) {
          const float4 a = *d;
          v.x += a.x; v.y += a.y; v.z += a.z; v.w += a.w;
        }
        *d = v;
      }
    }
    return;
  }
  const bool vec = row0 + kRRdc <= n_out && n_out % 4 == 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = t0 + 4 * lane + q;
    if (t >= T) continue;
    float* dst = out + t * n_out;
    if (vec) {
      float4* d = reinterpret_cast<float4*>(dst + row0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float4 v = make_float4(alpha * acc[4 * h][q], alpha * acc[4 * h + 1][q],
                               alpha * acc[4 * h + 2][q], alpha * acc[4 * h + 3][q]);
        if (accumulate) {
          const float4 a = d[h];
          v.x += a.x; v.y += a.y; v.z += a.z; v.w += a.w;
        }
        d[h] = v;
      }
    } else {
#pragma unroll
      for (int r = 0; r < kRRdc; ++r)
        if (row0 + r < n_out)
          dst[row0 + r] = alpha * acc[r][q] + (accumulate ? dst[row0 + r] : 0.f);
    }
  }
}

template <typename SrcT>
static hipError_t rows_dc_t(const void* src, int64_t T, int n_src, const void* prep, int64_t nnz,
                            int n_out, const SpmmPlan& pl, void* out, const float* zsrc,
                            float* partial, float alpha, int accumulate, hipStream_t s) {
  const int gy = (n_out + pl.rows_wg - 1) / pl.rows_wg;
  void* pp = const_cast<void*>(prep);
  const PrepLayout l = prep_layout(nnz, n_out, pl);
  const dim3 grid(static_cast<unsigned>(pl.ntiles), gy);
  constexpr int VEC = 16 / static_cast<int>(sizeof(SrcT));
  const bool vec_ok = (n_src % VEC) == 0 && n_src >= VEC;
  if constexpr (sizeof(SrcT) == 2) {
    if (pl.jb == kRJB16) {
      if (vec_ok)
        hipLaunchKernelGGL((rows_dc16_kernel<true>), grid, dim3(kRW * 64), 0, s,
                           static_cast<const uint16_t*>(src), T, n_src, at<int2>(pp, l.stream),
                           at<int32_t>(pp, l.ptr), at<int32_t>(pp, l.base), nnz, n_out,
                           pl.ptr_stride, pl.nblk, static_cast<float*>(out), zsrc, partial,
                           alpha, accumulate);
      else
        hipLaunchKernelGGL((rows_dc16_kernel<false>), grid, dim3(kRW * 64), 0, s,
                           static_cast<const uint16_t*>(src), T, n_src, at<int2>(pp, l.stream),
                           at<int32_t>(pp, l.ptr), at<int32_t>(pp, l.base), nnz, n_out,
                           pl.ptr_stride, pl.nblk, static_cast<float*>(out), zsrc, partial,
                           alpha, accumulate);
      return hipGetLastError();
    }
  }
  if (pl.jb != kRJB || pl.esz != 4) return hipErrorInvalidValue;
  if (vec_ok)
    hipLaunchKernelGGL((rows_dc_kernel<SrcT, true>), grid, dim3(kRW * 64), 0, s,
                       static_cast<const SrcT*>(src), T, n_src, at<int2>(pp, l.stream),
                       at<int32_t>(pp, l.ptr), at<int32_t>(pp, l.base), nnz, n_out,
                       pl.ptr_stride, pl.nblk, static_cast<float*>(out), zsrc, partial, alpha,
                       accumulate);
  else
    hipLaunchKernelGGL((rows_dc_kernel<SrcT, false>), grid, dim3(kRW * 64), 0, s,
                       static_cast<const SrcT*>(src), T, n_src, at<int2>(pp, l.stream),
                       at<int32_t>(pp, l.ptr), at<int32_t>(pp, l.base), nnz, n_out,
                       pl.ptr_stride, pl.nblk, static_cast<float*>(out), zsrc, partial, alpha,
                       accumulate);
  return hipGetLastError();
}

template <typename SrcT, typename OutT>
static hipError_t rows_t(const void* src, int64_t T, int n_src, const void* prep, int64_t nnz,
                         int n_out, const SpmmPlan& pl, float alpha, void* out, int acc,
                         hipStream_t s) {
  const int gy = (n_out + pl.rows_wg - 1) / pl.rows_wg;
  void* pp = const_cast<void*>(prep);
  const PrepLayout l = prep_layout(nnz, n_out, pl);
  const dim3 grid(static_cast<unsigned>(pl.ntiles), gy);
  constexpr int VEC = 16 / static_cast<int>(sizeof(SrcT));
  const bool vec_ok = (n_src % VEC) == 0 && n_src >= VEC;
  if (vec_ok)
    hipLaunchKernelGGL((rows_kernel<SrcT, OutT, true>), grid, dim3(kRW * 64), 0, s,
                       static_cast<const SrcT*>(src), T, n_src, at<int2>(pp, l.stream),
                       at<int32_t>(pp, l.ptr), at<int32_t>(pp, l.base), n_out, pl.ptr_stride,
                       pl.nblk, alpha, static_cast<OutT*>(out), acc);
  else
    hipLaunchKernelGGL((rows_kernel<SrcT, OutT, false>), grid, dim3(kRW * 64), 0, s,
                       static_cast<const SrcT*>(src), T, n_src, at<int2>(pp, l.stream),
                       at<int32_t>(pp, l.ptr), at<int32_t>(pp, l.base), n_out, pl.ptr_stride,
                       pl.nblk, alpha, static_cast<OutT*>(out), acc);
  return hipGetLastError();
}

hipError_t launch_spmm(const void* src, Dt src_dt, int64_t T, int n_src, const void* prep,
                       int64_t nnz, int n_out, const SpmmPlan& pl, float alpha, void* out,
                       Dt out_dt, int accumulate, const float* zsrc, float* partial,
                       hipStream_t s) {
  if (pl.ntiles == 0) return hipSuccess;
  if (pl.kind == 2) {
    // dz = alpha dy F (+ dz when accumulate, fp32) and the dc partials
    if (partial == nullptr || zsrc == nullptr || out_dt != Dt::F32) return hipErrorInvalidValue;
    return src_dt == Dt::F32
               ? rows_dc_t<float>(src, T, n_src, prep, nnz, n_out, pl, out, zsrc, partial, alpha,
                                  accumulate, s)
               : rows_dc_t<uint16_t>(src, T, n_src, prep, nnz, n_out, pl, out, zsrc, partial,
                                     alpha, accumulate, s);
  }
  if (partial != nullptr) return hipErrorInvalidValue;
  if (src_dt == Dt::F32 && out_dt == Dt::F32)
    return rows_t<float, float>(src, T, n_src, prep, nnz, n_out, pl, alpha, out, accumulate, s);
  if (src_dt == Dt::F32 && out_dt == Dt::BF16)
    return rows_t<float, uint16_t>(src, T, n_src, prep, nnz, n_out, pl, alpha, out, accumulate, s);
  if (src_dt == Dt::BF16 && out_dt == Dt::F32)
    return rows_t<uint16_t, float>(src, T, n_src, prep, nnz, n_out, pl, alpha, out, accumulate, s);
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------ dc reduction
// dc[korig[q]] = alpha * sum over tiles of partial[tile][q], tiles in order
// (the same order in both forms). VEC4: four consecutive q per thread with
// 16-byte loads (nnz % 4 == 0), eight tiles' loads in flight.
template <bool VEC4>
__global__ __launch_bounds__(256) void dc_reduce_kernel(const float* __restrict__ partial,
                                                        int64_t ntiles, int64_t nnz,
                                                        const int32_t* __restrict__ korig,
                                                        float alpha, float* __restrict__ dc) {
  const int64_t id = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (!VEC4) {
    if (id >= nnz) return;
    float s = 0.f;
    for (int64_t t = 0; t < ntiles; ++t) s += partial[t * nnz + id];
    const int k = korig[id];
    if (k >= 0) dc[k] = alpha * s;
    return;
  }
  const int64_t q = id * 4;
  if (q >= nnz) return;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t t0 = 0; t0 < ntiles; t0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (t0 + u < ntiles) v[u] = *reinterpret_cast<const float4*>(partial + (t0 + u) * nnz + q);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (t0 + u < ntiles) {
        s.x += v[u].x;
        s.y += v[u].y;
        s.z += v[u].z;
        s.w += v[u].w;
      }
    }
  }
  const int4 k = *reinterpret_cast<const int4*>(korig + q);
  if (k.x >= 0) dc[k.x] = alpha * s.x;
  if (k.y >= 0) dc[k.y] = alpha * s.y;
  if (k.z >= 0) dc[k.z] = alpha * s.z;
  if (k.w >= 0) dc[k.w] = alpha * s.w;
}

hipError_t launch_dc_reduce(const float* partial, int64_t ntiles, int64_t nnz,
                            const int32_t* korig, float alpha, float* dc, hipStream_t s) {
  if (nnz == 0) return hipSuccess;
  const bool vec = nnz % 4 == 0 && reinterpret_cast<uintptr_t>(partial) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(korig) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL((dc_reduce_kernel<true>), dim3(static_cast<unsigned>((nnz / 4 + 255) / 256)),
                       dim3(256), 0, s, partial, ntiles, nnz, korig, alpha, dc);
  else
    hipLaunchKernelGGL((dc_reduce_kernel<false>), dim3(static_cast<unsigned>((nnz + 255) / 256)),
                       dim3(256), 0, s, partial, ntiles, nnz, korig, alpha, dc);
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
