// Global selection variants of the init, the alternatives AdaAlloc is
// compared with in the ablation (QWHA notes, papernotes.org, 关键设计 2 (the
// global top-p of the dense solution) and 实验关键数据 › 消融实验, Table 4;
// gist.science summary §2.2): the p positions of the whole matrix with the
// largest keys, where a key is |C| = |dW_Q H| (magnitude) or the complement
// of the position's SplitMix64 draw (random: the p smallest draws). Equal
// keys are taken in row-major order. Values are c = fp32(C[E]) as for
// AdaAlloc (refinement with an identity Hessian).
//
// Steps: (magnitude) the keys of all d_out*d_in positions, fp64 FWHT per row;
// the exact p-th largest key tau by an MSB-first radix select, 8 bits per
// pass, counts in device memory (no host round trip); per row the counts of
// keys above and equal to tau; the rows' budgets (keys above tau plus the
// ties the earlier rows left over, in row order) and row_ptr. The per-row
// selection itself is the AdaAlloc kernel given tau.
#include "fwht_core.h"
#include "launch.h"

namespace qwha {

namespace {

// select state: prefix and mask of the key bits fixed so far, how many keys
// equal to the prefix are still to be taken
struct SelState {
  unsigned long long prefix;
  unsigned long long mask;
  long long krem;
  long long pad;
};

constexpr int kHistThreads = 256;
constexpr int kHistBlocks = 2048;

struct GsLayout {
  size_t state, hist, gt, eq, keys, total;
};

static size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

GsLayout gs_layout(int d_out, int d_in, int mode) {
  GsLayout l;
  l.state = 0;
  l.hist = 256;
  l.gt = l.hist + align256(256 * 8);
  l.eq = l.gt + align256(static_cast<size_t>(d_out) * 4);
  l.keys = l.eq + align256(static_cast<size_t>(d_out) * 4);
  l.total = l.keys + (mode == 1 ? align256(static_cast<size_t>(d_out) * d_in * 8) : 0);
  return l;
}

__device__ __forceinline__ unsigned long long key_at(const unsigned long long* __restrict__ keys,
                                                     unsigned long long seed, long long q) {
  return keys ? keys[q] : ~splitmix64(seed, static_cast<unsigned long long>(q));
}

}  // namespace

size_t global_select_scratch_bytes(int d_out, int d_in, int mode) {
  return gs_layout(d_out, d_in, mode).total;
}

// |C| keys of one row of N columns (fp64 FWHT, natural column order); under
// the block-diagonal transform a row of nblk blocks is nblk such rows.
template <int LOG_N>
__global__ __launch_bounds__(Fwht<LOG_N>::TPR < 64 ? 64 : Fwht<LOG_N>::TPR) void mag_keys_kernel(
    const float* __restrict__ dWq, unsigned long long* __restrict__ keys) {
  using F = Fwht<LOG_N>;
  __shared__ double lds[F::LDS];
  const int64_t row = blockIdx.x;
  const int u = threadIdx.x;
  const bool active = u < F::TPR;
  double v[F::EPT];
  if (active) {
    const float* src = dWq + row * F::N + u * F::EPT;
    if constexpr (F::EPT == 16) {
      load16(src, v);
    } else {
#pragma unroll
      for (int r = 0; r < F::EPT; ++r) v[r] = static_cast<double>(src[r]);
    }
  } else {
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) v[r] = 0.0;
  }
  F::run(v, lds, u, active);
  if (active) {
    unsigned long long* dst = keys + row * F::N;
#pragma unroll
    for (int r = 0; r < F::EPT; ++r)
      dst[F::out_index(u, r)] =
          static_cast<unsigned long long>(__double_as_longlong(v[r])) & 0x7FFFFFFFFFFFFFFFull;
  }
}

__global__ void gsel_init_kernel(SelState* st, unsigned long long* hist, long long p) {
  const int t = threadIdx.x;
  if (t < 256) hist[t] = 0;
  if (t == 0) {
    if (p == 0) {
      // nothing to take: a threshold no key exceeds, no ties taken
      st->prefix = ~0ull;
      st->mask = ~0ull;
    } else {
      st->prefix = 0;
      st->mask = 0;
    }
    st->krem = p;
  }
}

// Histogram of bits [shift, shift+8) of the keys that match the prefix.
__global__ __launch_bounds__(kHistThreads) void radix_hist_kernel(
    const unsigned long long* __restrict__ keys, unsigned long long seed, long long n,
    const SelState* __restrict__ st, int shift, unsigned long long* __restrict__ hist) {
  __shared__ unsigned h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const unsigned long long prefix = st->prefix, mask = st->mask;
  if (mask != ~0ull) {
    const long long stride = static_cast<long long>(gridDim.x) * kHistThreads;
    for (long long q = static_cast<long long>(blockIdx.x) * kHistThreads + threadIdx.x; q < n;
         q += stride) {
      const unsigned long long k = key_at(keys, seed, q);
      if ((k & mask) == prefix) atomicAdd(&h[(k >> shift) & 255u], 1u);
    }
  }
  __syncthreads();
  if (h[threadIdx.x]) atomicAdd(&hist[threadIdx.x], static_cast<unsigned long long>(h[threadIdx.x]));
}

// Fix the next 8 bits: the digit d whose keys contain the krem-th largest,
// counting from the top digit; krem drops by the keys above d. Clears the
// histogram for the next pass.
__global__ __launch_bounds__(256) void radix_pick_kernel(SelState* st,
                                                         unsigned long long* hist, int shift) {
  __shared__ unsigned long long suf[256];
  const int d = threadIdx.x;
  const unsigned long long hd = hist[d];
  suf[d] = hd;
  __syncthreads();
  // suffix sums: suf[d] = sum of hist[d'] for d' >= d
  for (int off = 1; off < 256; off <<= 1) {
    const unsigned long long add = d + off < 256 ? suf[d + off] : 0ull;
    __syncthreads();
    suf[d] += add;
    __syncthreads();
  }
  const unsigned long long incl = suf[d];
  const unsigned long long above = incl - hd;
  const SelState s = *st;
  __syncthreads();
  if (s.mask != ~0ull) {
    const unsigned long long kr = static_cast<unsigned long long>(s.krem);
    if (above < kr && kr <= incl) {
      st->prefix = s.prefix | (static_cast<unsigned long long>(d) << shift);
      st->mask = s.mask | (255ull << shift);
      st->krem = s.krem - static_cast<long long>(above);
    }
  }
  hist[d] = 0;
}

// Per row (one wave): keys above the threshold and keys equal to it.
__global__ __launch_bounds__(256) void row_ties_kernel(const unsigned long long* __restrict__ keys,
                                                       unsigned long long seed, int d_out,
                                                       int d_in, const SelState* __restrict__ st,
                                                       int32_t* __restrict__ gt,
                                                       int32_t* __restrict__ eq) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= d_out) return;
  const unsigned long long tau = st->prefix;
  int g = 0, e = 0;
  for (int j = lane; j < d_in; j += 64) {
    const unsigned long long k = key_at(keys, seed, static_cast<long long>(row) * d_in + j);
    g += k > tau ? 1 : 0;
    e += k == tau ? 1 : 0;
  }
  g = wave_sum_i32(g);
  e = wave_sum_i32(e);
  if (lane == 0) {
    gt[row] = g;
    eq[row] = e;
  }
}

// Budgets: row i takes its keys above tau and min(eq_i, ties left) of its
// ties, the ties going to rows in order (krem of them in all); row_ptr is the
// exclusive scan of the budgets. One workgroup, rows in chunks of 1024.
__global__ __launch_bounds__(1024) void global_budget_kernel(const int32_t* __restrict__ gt,
                                                             const int32_t* __restrict__ eq,
                                                             int d_out,
                                                             const SelState* __restrict__ st,
                                                             int32_t* __restrict__ row_ptr) {
  __shared__ int wsum[16];
  __shared__ long long ties_left;
  __shared__ int carry;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (threadIdx.x == 0) {
    ties_left = st->krem;
    carry = 0;
  }
  __syncthreads();
  for (int i0 = 0; i0 < d_out; i0 += 1024) {
    const int i = i0 + threadIdx.x;
    const int e = i < d_out ? eq[i] : 0;
    // exclusive prefix of eq within the chunk
    int incl = wave_incl_scan_i32(e);
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    int before = 0, all = 0;
    for (int k = 0; k < 16; ++k) {
      if (k < wid) before += wsum[k];
      all += wsum[k];
    }
    const long long left = ties_left - (before + incl - e);
    const int take = left <= 0 ? 0 : (left >= e ? e : static_cast<int>(left));
    const int b = i < d_out ? gt[i] + take : 0;
    __syncthreads();
    // exclusive prefix of the budgets -> row_ptr
    incl = wave_incl_scan_i32(b);
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    int bb = 0, ball = 0;
    for (int k = 0; k < 16; ++k) {
      if (k < wid) bb += wsum[k];
      ball += wsum[k];
    }
    if (i < d_out) row_ptr[i] = carry + bb + incl - b;
    __syncthreads();
    if (threadIdx.x == 0) {
      carry += ball;
      ties_left -= all;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) row_ptr[d_out] = carry;
}

hipError_t launch_global_budgets(const float* dWq, int d_out, int log_n, int64_t p, int mode,
                                 unsigned long long seed, int32_t* row_ptr, void* scratch,
                                 const unsigned long long** gtau, hipStream_t s, int nblk) {
  const int d_in = nblk << log_n;
  const GsLayout l = gs_layout(d_out, d_in, mode);
  char* base = static_cast<char*>(scratch);
  SelState* st = reinterpret_cast<SelState*>(base + l.state);
  unsigned long long* hist = reinterpret_cast<unsigned long long*>(base + l.hist);
  int32_t* gt = reinterpret_cast<int32_t*>(base + l.gt);
  int32_t* eq = reinterpret_cast<int32_t*>(base + l.eq);
  unsigned long long* keys =
      mode == 1 ? reinterpret_cast<unsigned long long*>(base + l.keys) : nullptr;
  if (mode == 1) {
    switch (log_n) {
#define QWHA_CASE(L)                                                                           \
  case L:                                                                                      \
    hipLaunchKernelGGL(mag_keys_kernel<L>, dim3(d_out * nblk),                                 \
                       dim3(Fwht<L>::TPR < 64 ? 64 : Fwht<L>::TPR), 0, s, dWq, keys);           \
    break;
      QWHA_CASE(1) QWHA_CASE(2) QWHA_CASE(3) QWHA_CASE(4) QWHA_CASE(5) QWHA_CASE(6) QWHA_CASE(7)
      QWHA_CASE(8) QWHA_CASE(9) QWHA_CASE(10) QWHA_CASE(11) QWHA_CASE(12) QWHA_CASE(13)
      QWHA_CASE(14)
#undef QWHA_CASE
      default:
        return hipErrorInvalidValue;
    }
  }
  const long long n = static_cast<long long>(d_out) * d_in;
  hipLaunchKernelGGL(gsel_init_kernel, dim3(1), dim3(256), 0, s, st, hist,
                     static_cast<long long>(p));
  const long long want = (n + kHistThreads - 1) / kHistThreads;
  const unsigned hb = static_cast<unsigned>(want < kHistBlocks ? want : kHistBlocks);
  for (int shift = 56; shift >= 0; shift -= 8) {
    hipLaunchKernelGGL(radix_hist_kernel, dim3(hb), dim3(kHistThreads), 0, s, keys, seed, n, st,
                       shift, hist);
    hipLaunchKernelGGL(radix_pick_kernel, dim3(1), dim3(256), 0, s, st, hist, shift);
  }
  hipLaunchKernelGGL(row_ties_kernel, dim3((d_out + 3) / 4), dim3(256), 0, s, keys, seed, d_out,
                     d_in, st, gt, eq);
  hipLaunchKernelGGL(global_budget_kernel, dim3(1), dim3(1024), 0, s, gt, eq, d_out, st,
                     row_ptr);
  *gtau = &st->prefix;
  return hipGetLastError();
}

}  // namespace qwha
