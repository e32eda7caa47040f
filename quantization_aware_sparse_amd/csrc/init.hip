// Quantization-aware init of the WHA adapter: per-row error norms, AdaAlloc
// budgets, in-row top-magnitude selection of E and the values c, and the
// column index of F.
//   QWHA notes (papernotes.org), 方法详解 › 关键设计 2 (AdaAlloc) and 3 (Value
//   Refinement: x0 = (dW_Q H)_i is the dense solution); gist.science summary
//   §2.2 (budget proportional to the channel's error magnitude, a per-channel
//   lower bound, top-magnitude coefficients within each channel).
// With an identity Hessian the refined values equal the dense solution at
// the chosen positions, so c = fp32_RNE(C[i, E_i]).
#include "fwht_core.h"
#include "launch.h"

namespace qwha {

// ------------------------------------------------------------ block helpers
// Sum over the block of a wave-uniform value (lane 0 of each wave posts it).
__device__ __forceinline__ int block_total_i32(int v, int* red, int parity) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = (blockDim.x + 63) >> 6;
  if (lane == 0) red[parity * 16 + wid] = v;
  __syncthreads();
  int t = 0;
  for (int i = 0; i < nw; ++i) t += red[parity * 16 + i];
  return t;
}

// Exclusive prefix over threads in threadIdx order; *total gets the sum.
__device__ __forceinline__ int block_excl_scan_i32(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = (blockDim.x + 63) >> 6;
  const int incl = wave_incl_scan_i32(v);
  __syncthreads();                       // tmp free from any earlier use
  if (lane == 63) tmp[wid] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int i = 0; i < nw; ++i) {
    const int x = tmp[i];
    if (i < wid) before += x;
    all += x;
  }
  *total = all;
  return before + incl - v;
}

// ------------------------------------------------------------ row norms
// w_i = sqrt(sum_j dWq[i][j]^2) in fp64; one wave per row.
__global__ __launch_bounds__(256) void row_norms_kernel(const float* __restrict__ dWq, int d_out,
                                                        int d_in, double* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= d_out) return;
  const float* src = dWq + static_cast<int64_t>(row) * d_in;
  double acc = 0.0;
  if (d_in >= 4) {
    // eight 16-byte loads in flight per lane before they are summed
    for (int j0 = lane * 4; j0 < d_in; j0 += 256 * 8) {
      float4 f[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        f[u] = j0 + 256 * u < d_in ? *reinterpret_cast<const float4*>(src + j0 + 256 * u)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc += static_cast<double>(f[u].x) * f[u].x;
        acc += static_cast<double>(f[u].y) * f[u].y;
        acc += static_cast<double>(f[u].z) * f[u].z;
        acc += static_cast<double>(f[u].w) * f[u].w;
      }
    }
  } else {
    for (int j = lane; j < d_in; j += 64) acc += static_cast<double>(src[j]) * src[j];
  }
  acc = wave_sum_f64(acc);
  if (lane == 0) w[row] = sqrt(acc);
}

hipError_t launch_row_norms(const float* dWq, int d_out, int d_in, double* w, hipStream_t s) {
  hipLaunchKernelGGL(row_norms_kernel, dim3((d_out + 3) / 4), dim3(256), 0, s, dWq, d_out, d_in, w);
  return hipGetLastError();
}

// ------------------------------------------------------------ AdaAlloc
// One workgroup. Proportional passes over the rows not yet fixed: share
// q_i = P s_i / S (s_i = w_i^(1/t)), p_i = floor(q_i). Rows with q_i < m are
// held at m; if there are none, rows with q_i > d_in are held at d_in and the
// rows held at the floor are released (capping raises the others' share);
// repeat until a pass holds nothing. This is the clamped proportional split
// clamp(lambda s_i, m, d_in) before rounding. The leftover r = p - sum p_i (< d_out) goes one unit
// each to the rows with the smallest budget, lower row index first, rows at
// d_in skipped (in further rounds if r exceeds the eligible rows).
// Finally row_ptr = exclusive scan of the budgets.
constexpr int kAllocThreads = 1024;

size_t adaalloc_scratch_bytes(int d_out) {
  // s (double), budget (int64), fixed (int32)
  return static_cast<size_t>(d_out) * (8 + 8 + 4) + 256;
}

__global__ __launch_bounds__(kAllocThreads) void adaalloc_kernel(
    const double* __restrict__ w, int d_out, int d_in, int64_t p, int m, double t,
    int32_t* __restrict__ row_ptr, double* __restrict__ s, int64_t* __restrict__ budget,
    int32_t* __restrict__ fixed) {
  __shared__ double red_d[16];
  __shared__ long long red_l[2][16];
  __shared__ int red_i[2][16];
  __shared__ int flags[4];
  __shared__ int hist[16385 + 1];
  __shared__ int scan_tmp[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  constexpr int NW = kAllocThreads / 64;

  for (int i = tid; i < d_out; i += kAllocThreads) {
    s[i] = (t == 1.0) ? w[i] : pow(w[i], 1.0 / t);
    budget[i] = 0;
    fixed[i] = 0;
  }
  __syncthreads();

  int parity = 0;
  for (;;) {
    // S over unfixed rows (fp64, fixed order), budget sum over fixed rows,
    // count of unfixed rows.
    double ps = 0.0;
    long long pf = 0;
    int nu = 0;
    for (int i = tid; i < d_out; i += kAllocThreads) {
      if (fixed[i]) pf += budget[i];
      else { ps += s[i]; ++nu; }
    }
    ps = wave_sum_f64(ps);
    pf = wave_sum_i64(pf);
    nu = wave_sum_i32(nu);
    if (lane == 0) { red_d[wid] = ps; red_l[parity][wid] = pf; red_i[parity][wid] = nu; }
    if (tid < 4) flags[tid] = 0;
    __syncthreads();
    double S = 0.0;
    long long F = 0;
    int NU = 0;
    for (int i = 0; i < NW; ++i) { S += red_d[i]; F += red_l[parity][i]; NU += red_i[parity][i]; }
    parity ^= 1;
    if (NU == 0) break;
    const long long P = p - F;
    // share q_i = P s_i / S (unfloored), budget = floor(q_i); fixed: 0 free,
    // 1 held at the floor m, 2 held at the cap d_in
    int low = 0, high = 0;
    for (int i = tid; i < d_out; i += kAllocThreads) {
      if (fixed[i]) continue;
      const double qi = (S > 0.0) ? (static_cast<double>(P) * s[i]) / S
                                  : static_cast<double>(P / NU);
      budget[i] = static_cast<long long>(floor(qi));
      if (qi < static_cast<double>(m)) { low = 1; fixed[i] = -1; }           // tentative
      else if (qi > static_cast<double>(d_in)) { high = 1; fixed[i] = -2; }  // tentative
    }
    if (low) flags[0] = 1;
    if (high) flags[1] = 1;
    __syncthreads();
    if (flags[0]) {
      // rows below the floor are held at m; tentative caps are dropped
      for (int i = tid; i < d_out; i += kAllocThreads) {
        if (fixed[i] == -1) { budget[i] = m; fixed[i] = 1; }
        else if (fixed[i] == -2) fixed[i] = 0;
      }
      __syncthreads();
      continue;
    }
    if (flags[1]) {
      // rows above the cap are held at d_in and rows at the floor released
      for (int i = tid; i < d_out; i += kAllocThreads) {
        if (fixed[i] == -2) { budget[i] = d_in; fixed[i] = 2; }
        else if (fixed[i] == 1) fixed[i] = 0;
      }
      __syncthreads();
      continue;
    }
    break;
  }
  __syncthreads();

  // leftover. Thread tid owns the contiguous rows [tid * rpt, (tid+1) * rpt)
  // and the budget values [tid * vpt, (tid+1) * vpt), so that one block scan
  // orders a pass (row order and value order are thread order).
  const int rpt = (d_out + kAllocThreads - 1) / kAllocThreads;
  const int vpt = (d_in + 1 + kAllocThreads - 1) / kAllocThreads;
  const int r0 = tid * rpt, r1 = min(r0 + rpt, d_out);
  const int v0 = tid * vpt, v1 = min(v0 + vpt, d_in + 1);
  __shared__ int vstar;
  __shared__ int below_star;
  for (;;) {
    long long tot = 0;
    for (int i = tid; i < d_out; i += kAllocThreads) tot += budget[i];
    tot = wave_sum_i64(tot);
    if (lane == 0) red_l[parity][wid] = tot;
    for (int v = tid; v <= d_in; v += kAllocThreads) hist[v] = 0;
    if (tid == 0) vstar = -1;
    __syncthreads();
    long long TOT = 0;
    for (int i = 0; i < NW; ++i) TOT += red_l[parity][i];
    parity ^= 1;
    const long long r = p - TOT;
    if (r <= 0) break;
    for (int i = tid; i < d_out; i += kAllocThreads)
      if (budget[i] < d_in) atomicAdd(&hist[budget[i]], 1);
    __syncthreads();
    // v* = the budget value at which the eligible rows, counted from the
    // smallest budget up, reach r: before(v*) < r <= before(v*) + hist[v*]
    {
      int h = 0;
      for (int v = v0; v < v1; ++v) h += hist[v];
      int all_h;
      int before = block_excl_scan_i32(h, scan_tmp, &all_h);
      for (int v = v0; v < v1; ++v) {
        const int hv = hist[v];
        if (hv > 0 && before < r && before + hv >= r) { vstar = v; below_star = before; }
        before += hv;
      }
    }
    __syncthreads();
    const int vs = vstar;
    if (vs < 0) {
      // fewer eligible rows than the leftover: every eligible row gets one
      for (int i = tid; i < d_out; i += kAllocThreads)
        if (budget[i] < d_in) budget[i] += 1;
      __syncthreads();
      continue;
    }
    const long long need = r - below_star;       // rows at vs that get a unit
    // rows below vs get one; rows at vs get one in row order while need lasts
    int eq = 0;
    for (int i = r0; i < r1; ++i) eq += budget[i] == vs ? 1 : 0;
    int all_eq;
    int rank = block_excl_scan_i32(eq, scan_tmp, &all_eq);
    for (int i = r0; i < r1; ++i) {
      const long long bi = budget[i];
      if (bi < vs) {
        budget[i] = bi + 1;
      } else if (bi == vs) {
        if (rank < need) budget[i] = bi + 1;
        ++rank;
      }
    }
    __syncthreads();
  }
  __syncthreads();

  // row_ptr = exclusive scan of budgets
  {
    int sum = 0;
    for (int i = r0; i < r1; ++i) sum += static_cast<int>(budget[i]);
    int total;
    int pos = block_excl_scan_i32(sum, scan_tmp, &total);
    for (int i = r0; i < r1; ++i) {
      row_ptr[i] = pos;
      pos += static_cast<int>(budget[i]);
    }
    if (tid == 0) row_ptr[d_out] = total;
  }
}

// The same passes with every row's state in registers: thread tid owns the
// contiguous rows [tid * rpt, (tid+1) * rpt) (rpt <= kAllocRegRows), so a
// pass is register work plus one block reduction, with no global memory
// between passes. The sums over rows are taken in this order (per thread,
// then across threads); the leftover and the row_ptr scan are as above.
constexpr int kAllocRegRows = 16;

__global__ __launch_bounds__(kAllocThreads) void adaalloc_reg_kernel(
    const double* __restrict__ w, int d_out, int d_in, int64_t p, int m, double t,
    int32_t* __restrict__ row_ptr) {
  __shared__ double red_d[2][16];
  __shared__ long long red_l[2][16];
  __shared__ int red_i[2][16];
  __shared__ int red_f[2][16];
  __shared__ int hist[16385 + 1];
  __shared__ int scan_tmp[16];
  __shared__ int vstar;
  __shared__ int below_star;
  constexpr int R = kAllocRegRows;
  constexpr int NW = kAllocThreads / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int rpt = (d_out + kAllocThreads - 1) / kAllocThreads;
  const int r0 = tid * rpt;

  double s[R];
  int bud[R];
  int fx[R];   // 0 free, 1 held at the floor m, 2 held at the cap d_in, -1 / -2 tentative
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = r0 + r;
    const bool own = r < rpt && i < d_out;
    s[r] = own ? ((t == 1.0) ? w[i] : pow(w[i], 1.0 / t)) : 0.0;
    bud[r] = 0;
    fx[r] = own ? 0 : 3;   // 3: not a row
  }

  int parity = 0;
  for (;;) {
    double ps = 0.0;
    long long pf = 0;
    int nu = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (fx[r] == 0) { ps += s[r]; ++nu; }
      else if (fx[r] == 1 || fx[r] == 2) pf += bud[r];
    }
    ps = wave_sum_f64(ps);
    pf = wave_sum_i64(pf);
    nu = wave_sum_i32(nu);
    if (lane == 0) { red_d[parity][wid] = ps; red_l[parity][wid] = pf; red_i[parity][wid] = nu; }
    __syncthreads();
    double S = 0.0;
    long long F = 0;
    int NU = 0;
    for (int i = 0; i < NW; ++i) { S += red_d[parity][i]; F += red_l[parity][i]; NU += red_i[parity][i]; }
    const int pp = parity;   // the next pass (or the leftover) posts to the other slots
    parity ^= 1;
    if (NU == 0) break;
    const long long P = p - F;
    int low = 0, high = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (fx[r] != 0) continue;
      const double qi = (S > 0.0) ? (static_cast<double>(P) * s[r]) / S
                                  : static_cast<double>(P / NU);
      bud[r] = static_cast<int>(floor(qi));
      if (qi < static_cast<double>(m)) { low = 1; fx[r] = -1; }
      else if (qi > static_cast<double>(d_in)) { high = 1; fx[r] = -2; }
    }
    low = __any(low);
    high = __any(high);
    if (lane == 0) red_f[pp][wid] = (low ? 1 : 0) | (high ? 2 : 0);
    __syncthreads();
    int fl = 0;
    for (int i = 0; i < NW; ++i) fl |= red_f[pp][i];
    if (fl & 1) {
      // rows below the floor are held at m; tentative caps are dropped
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (fx[r] == -1) { bud[r] = m; fx[r] = 1; }
        else if (fx[r] == -2) fx[r] = 0;
      }
      continue;
    }
    if (fl & 2) {
      // rows above the cap are held at d_in and rows at the floor released
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (fx[r] == -2) { bud[r] = d_in; fx[r] = 2; }
        else if (fx[r] == 1) fx[r] = 0;
      }
      continue;
    }
    break;
  }

  // leftover: as adaalloc_kernel, with budget values [tid * vpt, (tid+1) * vpt)
  const int vpt = (d_in + 1 + kAllocThreads - 1) / kAllocThreads;
  const int v0 = tid * vpt, v1 = min(v0 + vpt, d_in + 1);
  for (;;) {
    long long tot = 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (fx[r] != 3) tot += bud[r];
    tot = wave_sum_i64(tot);
    if (lane == 0) red_l[parity][wid] = tot;
    for (int v = tid; v <= d_in; v += kAllocThreads) hist[v] = 0;
    if (tid == 0) vstar = -1;
    __syncthreads();
    long long TOT = 0;
    for (int i = 0; i < NW; ++i) TOT += red_l[parity][i];
    parity ^= 1;
    const long long rem = p - TOT;
    if (rem <= 0) break;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (fx[r] != 3 && bud[r] < d_in) atomicAdd(&hist[bud[r]], 1);
    __syncthreads();
    {
      int h = 0;
      for (int v = v0; v < v1; ++v) h += hist[v];
      int all_h;
      int before = block_excl_scan_i32(h, scan_tmp, &all_h);
      for (int v = v0; v < v1; ++v) {
        const int hv = hist[v];
        if (hv > 0 && before < rem && before + hv >= rem) { vstar = v; below_star = before; }
        before += hv;
      }
    }
    __syncthreads();
    const int vs = vstar;
    if (vs < 0) {
      // fewer eligible rows than the leftover: every eligible row gets one
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (fx[r] != 3 && bud[r] < d_in) bud[r] += 1;
      __syncthreads();   // hist and vstar are read before the next pass resets them
      continue;
    }
    const long long need = rem - below_star;   // rows at vs that get a unit
    int eq = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) eq += (fx[r] != 3 && bud[r] == vs) ? 1 : 0;
    int all_eq;
    int rank = block_excl_scan_i32(eq, scan_tmp, &all_eq);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (fx[r] == 3) continue;
      if (bud[r] < vs) {
        bud[r] += 1;
      } else if (bud[r] == vs) {
        if (rank < need) bud[r] += 1;
        ++rank;
      }
    }
    __syncthreads();   // vstar / below_star are read before the next pass resets them
  }

  // row_ptr = exclusive scan of budgets
  int sum = 0;
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (fx[r] != 3) sum += bud[r];
  int total;
  int pos = block_excl_scan_i32(sum, scan_tmp, &total);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (fx[r] == 3) continue;
    row_ptr[r0 + r] = pos;
    pos += bud[r];
  }
  if (tid == 0) row_ptr[d_out] = total;
}

hipError_t launch_adaalloc(const double* w, int d_out, int d_in, int64_t p, int m, double t,
                           int32_t* row_ptr, void* scratch, hipStream_t st) {
  char* base = static_cast<char*>(scratch);
  double* s = reinterpret_cast<double*>(base);
  int64_t* budget = reinterpret_cast<int64_t*>(base + static_cast<size_t>(d_out) * 8);
  int32_t* fixed = reinterpret_cast<int32_t*>(base + static_cast<size_t>(d_out) * 16);
  if (d_out <= kAllocThreads * kAllocRegRows) {
    hipLaunchKernelGGL(adaalloc_reg_kernel, dim3(1), dim3(kAllocThreads), 0, st, w, d_out, d_in,
                       p, m, t, row_ptr);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(adaalloc_kernel, dim3(1), dim3(kAllocThreads), 0, st, w, d_out, d_in, p, m, t,
                     row_ptr, s, budget, fixed);
  return hipGetLastError();
}

// ------------------------------------------------------------ radix select
// Needs a block of whole waves: every wave scans the whole histogram with
// its 64 lanes (4 bins each) and takes the same decisions.
// The k-th largest of the block's keys (non-negative IEEE doubles as bit
// patterns, so integer order is value order), MSB first:
//  level 0: a 256-bin histogram of bins relative to the largest key, 16
//           per octave: bin = 16 (e_max - e) + 15 - m4 (e the exponent, m4
//           the top four mantissa bits), bin 0 holding the largest keys;
//  levels 1..6: 8-bit digits of the remaining 48 mantissa bits, counted
//           only for the keys in the bucket found so far.
// Each level finds the bin where the count from the top reaches k, keeps
// the keys above it and narrows to it; it stops when the bucket holds
// exactly the keys still needed or the bits run out (a tie). Returns false
// (tau unset) when the k-th key lies 16 octaves or more below the largest.
// On success tau is the smallest key the bucket can hold: every key above
// the bucket exceeds it, every key below is smaller, and the keys equal to
// it are all in the bucket.
__device__ __forceinline__ int wave_first_ge(int incl, int k) {
  const unsigned long long b = __ballot(incl >= k);
  return b == 0 ? 64 : __ffsll(static_cast<long long>(b)) - 1;
}

// Every wave reads the whole histogram h[256] (the top of the order at
// bin 0) and finds, uniformly, the bin b where the running count reaches k
// (k >= 1 and the total >= k), the count above it and the count in it.
__device__ __forceinline__ void hist_cross(const int* h, int k, int& b, int& above, int& in) {
  const int lane = threadIdx.x & 63;
  const int4 c = reinterpret_cast<const int4*>(h)[lane];
  const int s4 = c.x + c.y + c.z + c.w;
  const int incl = wave_incl_scan_i32(s4);
  const int L = wave_first_ge(incl, k);
  const int before = __builtin_amdgcn_readlane(incl - s4, L);
  const int x = __builtin_amdgcn_readlane(c.x, L), y = __builtin_amdgcn_readlane(c.y, L);
  const int z = __builtin_amdgcn_readlane(c.z, L), w = __builtin_amdgcn_readlane(c.w, L);
  int q, cnt;
  if (before + x >= k) { q = 0; cnt = x; }
  else if (before + x + y >= k) { q = 1; cnt = y; }
  else if (before + x + y + z >= k) { q = 2; cnt = z; }
  else { q = 3; cnt = w; }
  b = uniform(4 * L + q);
  above = uniform(before + (q > 0 ? x : 0) + (q > 1 ? y : 0) + (q > 2 ? z : 0));
  in = uniform(cnt);
}

template <int EPT>
__device__ __forceinline__ bool radix_kth_largest(const unsigned long long (&key)[EPT],
                                                  bool active, int k, int* hist,
                                                  unsigned long long* red64,
                                                  unsigned long long* tau) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = (blockDim.x + 63) >> 6;
  const int tid = threadIdx.x, nth = blockDim.x;
  // the largest exponent: the high 32 bits of the keys carry it (bits 20..30)
  unsigned m = 0;
  if (active) {
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const unsigned h = static_cast<unsigned>(key[r] >> 32);
      m = h > m ? h : m;
    }
  }
  m = wave_max_u32(m);
  if (lane == 0) red64[wid] = m;
  for (int i = tid; i < 512; i += nth) hist[i] = 0;    // levels 0 and 1
  __syncthreads();
  unsigned long long kmax = 0;
  for (int i = 0; i < nw; ++i) kmax = red64[i] > kmax ? red64[i] : kmax;
  const int emax = static_cast<int>(kmax >> 20);
  if (active) {
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const int e = static_cast<int>(key[r] >> 52);
      const int d = (emax - e) * 16 + 15 - static_cast<int>((key[r] >> 48) & 15);
      atomicAdd(&hist[d > 255 ? 255 : d], 1);
    }
  }
  __syncthreads();
  int b, above, in;
  hist_cross(hist, k, b, above, in);
  if (b == 255) return false;
  int need = k - above;
  unsigned long long P = (static_cast<unsigned long long>(emax - b / 16) << 4) |
                         static_cast<unsigned long long>(15 - b % 16);     // bits 48..62
  int sh = 48;
  int lev = 1;
  while (sh > 0 && in != need) {
    int* h = hist + 256 * (lev % 3);
    int* hz = hist + 256 * ((lev + 1) % 3);   // the next level's, read two levels ago
    if (active) {
#pragma unroll
      for (int r = 0; r < EPT; ++r)
        if ((key[r] >> sh) == P) atomicAdd(&h[255 - static_cast<int>((key[r] >> (sh - 8)) & 255)], 1);
    }
    for (int i = tid; i < 256; i += nth) hz[i] = 0;
    __syncthreads();
    hist_cross(h, need, b, above, in);
    need -= above;
    P = (P << 8) | static_cast<unsigned long long>(255 - b);
    sh -= 8;
    ++lev;
  }
  *tau = P << sh;
  return true;
}

// ------------------------------------------------------------ selection
// One workgroup per row i: C = dWq[i] H in fp64 (LDS-staged FWHT), then the
// k = p_i columns first in the order (-|C_j|, j) are emitted ascending as
// E rows (i, j) with c = fp32_RNE(C_j). The k-th largest magnitude tau is
// found by bisection on the IEEE bit pattern of |C| (monotone for
// non-negative doubles; +0 and -0 share the pattern 0); every |C| > tau is
// taken and the lowest-index columns with |C| == tau fill the rest.
template <int LOG_N>
struct SelCfg {
  using F = Fwht<LOG_N>;
  static constexpr int BLOCK = F::TPR < 64 ? 64 : F::TPR;
};

// MODE 0 (AdaAlloc): the row's budget picks its own threshold by bisection
// on the |C| keys. Modes 1 / 2 (global selection): the threshold *gtau over
// the whole matrix is given and the row takes its keys above it plus, of the
// keys equal to it, as many as its budget leaves (lowest column first); the
// keys are |C| (mode 1) or the complement of the position's SplitMix64 draw
// (mode 2, output row*N + col of the generator seeded with `seed`).
//
// BLOCKED: a row of nblk * N columns under the block-diagonal transform (nblk
// Sylvester blocks of order N): thread t = blk * TPR + u transforms its part
// of block blk in that block's slice of the dynamic LDS; the selection runs
// over the whole row, and thread t holds columns t*EPT .. t*EPT + EPT - 1 in
// both cases.
template <int LOG_N, int MODE, bool BLOCKED>
__global__ __launch_bounds__(BLOCKED ? 1024 : SelCfg<LOG_N>::BLOCK) void init_select_kernel(
    const float* __restrict__ dWq, const int32_t* __restrict__ row_ptr, int32_t* __restrict__ E,
    float* __restrict__ c, const unsigned long long* __restrict__ gtau,
    unsigned long long seed, int nblk) {
  using F = Fwht<LOG_N>;
  extern __shared__ double lds_blocks[];
  __shared__ double lds_row[BLOCKED ? 1 : F::LDS];
  __shared__ int red[32];
  __shared__ int scan_tmp[16];
  __shared__ int hist[3 * 256];
  __shared__ unsigned long long red64[16];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int u = BLOCKED ? t % F::TPR : t;
  const int d_in = BLOCKED ? nblk * F::N : F::N;
  const bool active = BLOCKED ? t < nblk * F::TPR : t < F::TPR;
  double* lds = BLOCKED ? lds_blocks + (t / F::TPR) * F::LDS : lds_row;
  const int col0 = t * F::EPT;     // first column this thread holds
  const int base = row_ptr[row];
  const int k = row_ptr[row + 1] - base;

  double v[F::EPT];
  if (active) {
    const float* src = dWq + static_cast<int64_t>(row) * d_in + col0;
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
  // back to natural order, then to "EPT consecutive columns per thread"
  __syncthreads();
  if (active) {
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) lds[F::pad(F::out_index(u, r))] = v[r];
  }
  __syncthreads();
  unsigned long long key[F::EPT];
  if (active) {
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) {
      v[r] = lds[F::pad(u * F::EPT + r)];
      key[r] = MODE == 2
                   ? ~splitmix64(seed, static_cast<unsigned long long>(row) * d_in + col0 + r)
                   : static_cast<unsigned long long>(__double_as_longlong(v[r])) &
                         0x7FFFFFFFFFFFFFFFull;
    }
  } else {
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) key[r] = 0;
  }

  // tau = the k-th largest key: the largest t with count(key >= t) >= k,
  // found by bisection, first on the top 32 bits of the keys (32-bit
  // compares), then, only if the top bits leave more than k keys at the
  // threshold, on the full keys within that 2^32-wide range. Counts go by
  // wave ballots (one barrier per step); the search stops as soon as the
  // keys >= lo are exactly k.
  unsigned long long tau = 0;
  int need = 0;      // how many |C| == tau are taken (lowest index first)
  bool all = (k >= d_in), none = (k <= 0);
  int parity = 0;
  if (!all && !none && MODE != 0) {
    tau = *gtau;
    int gt = 0;
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) gt += __popcll(__ballot(active && key[r] > tau));
    gt = block_total_i32(gt, red, parity);
    parity ^= 1;
    need = k - gt;
  } else if (!all && !none &&
             radix_kth_largest<F::EPT>(key, active, k, hist, red64, &tau)) {
    const int gt = [&] {
      int cnt = 0;
#pragma unroll
      for (int r = 0; r < F::EPT; ++r) cnt += __popcll(__ballot(active && key[r] > tau));
      return block_total_i32(cnt, red, parity);
    }();
    parity ^= 1;
    need = k - gt;
  } else if (!all && !none) {
    auto count_ge32 = [&](unsigned m) {
      int cnt = 0;
#pragma unroll
      for (int r = 0; r < F::EPT; ++r)
        cnt += __popcll(__ballot(static_cast<unsigned>(key[r] >> 32) >= m));
      return block_total_i32(cnt, red, parity);
    };
    auto count_ge64 = [&](unsigned long long m) {
      int cnt = 0;
#pragma unroll
      for (int r = 0; r < F::EPT; ++r) cnt += __popcll(__ballot(key[r] >= m));
      return block_total_i32(cnt, red, parity);
    };
    // count(top32 >= lo32) >= k > count(top32 >= hi32); keys are < 2^63
    unsigned lo32 = 0, hi32 = 1u << 31;
    int cnt_lo = d_in;
    while (hi32 - lo32 > 1 && cnt_lo != k) {
      const unsigned mid = lo32 + ((hi32 - lo32) >> 1);
      const int cnt = count_ge32(mid);
      parity ^= 1;
      if (cnt >= k) { lo32 = mid; cnt_lo = cnt; } else { hi32 = mid; }
    }
    unsigned long long lo = static_cast<unsigned long long>(lo32) << 32;
    unsigned long long hi = static_cast<unsigned long long>(hi32) << 32;
    while (hi - lo > 1 && cnt_lo != k) {
      const unsigned long long mid = lo + ((hi - lo) >> 1);
      const int cnt = count_ge64(mid);
      parity ^= 1;
      if (cnt >= k) { lo = mid; cnt_lo = cnt; } else { hi = mid; }
    }
    tau = lo;
    const int gt = count_ge64(tau + 1);
    parity ^= 1;
    need = k - gt;
  }

  // selection flags in column order
  unsigned sel = 0;
  int nsel = 0;
  {
    int neq = 0;
    if (active && !all && !none) {
#pragma unroll
      for (int r = 0; r < F::EPT; ++r) neq += (key[r] == tau) ? 1 : 0;
    }
    int tot;
    const int eq_before = block_excl_scan_i32(neq, scan_tmp, &tot);
    if (active) {
      int e = eq_before;
#pragma unroll
      for (int r = 0; r < F::EPT; ++r) {
        bool take;
        if (all) take = true;
        else if (none) take = false;
        else if (key[r] > tau) take = true;
        else if (key[r] == tau) { take = e < need; ++e; }
        else take = false;
        if (take) { sel |= 1u << r; ++nsel; }
      }
    }
  }
  int tot;
  const int pos0 = block_excl_scan_i32(nsel, scan_tmp, &tot);
  if (active) {
    int pos = base + pos0;
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) {
      if (sel & (1u << r)) {
        E[2 * static_cast<int64_t>(pos)] = row;
        E[2 * static_cast<int64_t>(pos) + 1] = col0 + r;
        c[pos] = __double2float_rn(v[r]);
        ++pos;
      }
    }
  }
}

template <int L, bool BLOCKED>
hipError_t launch_select_mode(const float* dWq, int d_out, const int32_t* row_ptr, int32_t* E,
                              float* c, int mode, const unsigned long long* gtau,
                              unsigned long long seed, int nblk, hipStream_t s) {
  using F = Fwht<L>;
  const dim3 grid(d_out);
  int threads = SelCfg<L>::BLOCK;
  size_t lds = 0;
  if (BLOCKED) {
    // whole waves: the radix select scans its histogram with every lane of
    // every wave (threads past nblk * TPR hold no columns)
    threads = (nblk * F::TPR + 63) / 64 * 64;
    lds = static_cast<size_t>(nblk) * F::LDS * sizeof(double);
  }
  const dim3 block(threads);
  auto go = [&](auto kernel) {
    if (BLOCKED) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kernel, grid, block, lds, s, dWq, row_ptr, E, c, gtau, seed, nblk);
    return hipGetLastError();
  };
  if (mode == 0) return go(init_select_kernel<L, 0, BLOCKED>);
  if (mode == 1) return go(init_select_kernel<L, 1, BLOCKED>);
  return go(init_select_kernel<L, 2, BLOCKED>);
}

hipError_t launch_init_select(const float* dWq, int d_out, int log_n, const int32_t* row_ptr,
                              int32_t* E, float* c, int mode, const unsigned long long* gtau,
                              unsigned long long seed, hipStream_t s, int nblk) {
  if (mode < 0 || mode > 2 || nblk < 1) return hipErrorInvalidValue;
  if (nblk == 1) {
    switch (log_n) {
#define QWHA_CASE(L)                                                                       \
  case L:                                                                                  \
    return launch_select_mode<L, false>(dWq, d_out, row_ptr, E, c, mode, gtau, seed, 1, s);
      QWHA_CASE(1) QWHA_CASE(2) QWHA_CASE(3) QWHA_CASE(4) QWHA_CASE(5) QWHA_CASE(6)
      QWHA_CASE(7) QWHA_CASE(8) QWHA_CASE(9) QWHA_CASE(10) QWHA_CASE(11) QWHA_CASE(12)
      QWHA_CASE(13) QWHA_CASE(14)
#undef QWHA_CASE
      default:
        return hipErrorInvalidValue;
    }
  }
  // block widths: blocks of 64 .. 4096 columns, at most 1024 threads a row
  switch (log_n) {
#define QWHA_CASE(L)                                                                      \
  case L:                                                                                 \
    return launch_select_mode<L, true>(dWq, d_out, row_ptr, E, c, mode, gtau, seed, nblk, s);
    QWHA_CASE(6) QWHA_CASE(7) QWHA_CASE(8) QWHA_CASE(9) QWHA_CASE(10) QWHA_CASE(11)
    QWHA_CASE(12)
#undef QWHA_CASE
    default:
      return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------ CSC index
// Stable counting sort of E by column: csc_perm lists k column by column,
// ascending k (hence ascending row) within a column. Rows are cut into
// chunks; per-chunk column histograms give each chunk its slot range per
// column, and each chunk then places its rows in order (the columns within
// one row are distinct, so a row's entries are placed in parallel).
constexpr int kCscThreads = 256;

static int csc_chunks(int d_out) { return d_out < 256 ? d_out : 256; }

size_t csc_scratch_bytes(int d_out, int d_in) {
  return static_cast<size_t>(csc_chunks(d_out)) * d_in * 4 + 256;
}

__global__ __launch_bounds__(kCscThreads) void csc_hist_kernel(const int32_t* __restrict__ row_ptr,
                                                               const int32_t* __restrict__ E,
                                                               int d_out, int d_in, int nchunks,
                                                               int32_t* __restrict__ hist) {
  extern __shared__ int h[];
  const int ch = blockIdx.x;
  const int r0 = static_cast<int>(static_cast<int64_t>(d_out) * ch / nchunks);
  const int r1 = static_cast<int>(static_cast<int64_t>(d_out) * (ch + 1) / nchunks);
  for (int j = threadIdx.x; j < d_in; j += kCscThreads) h[j] = 0;
  __syncthreads();
  for (int k = row_ptr[r0] + threadIdx.x; k < row_ptr[r1]; k += kCscThreads)
    atomicAdd(&h[E[2 * static_cast<int64_t>(k) + 1]], 1);
  __syncthreads();
  for (int j = threadIdx.x; j < d_in; j += kCscThreads)
    hist[static_cast<int64_t>(ch) * d_in + j] = h[j];
}

// hist[ch][j] -> number of entries of column j in chunks before ch; the
// column's total goes to cnt[j]. A workgroup takes 16 columns; thread
// (g, jj) sums chunks g*cpg .. g*cpg + cpg - 1 of column j0 + jj (all loads
// issued before the sum), the 16 group sums are scanned in LDS, and each
// thread then writes its chunks' running counts.
constexpr int kColsumCols = 16;
constexpr int kColsumGroups = 16;

__global__ __launch_bounds__(kColsumCols * kColsumGroups) void csc_colsum_kernel(
    int32_t* __restrict__ hist, int d_in, int nchunks, int32_t* __restrict__ cnt) {
  __shared__ int gsum[kColsumGroups][kColsumCols];
  const int jj = threadIdx.x % kColsumCols;
  const int g = threadIdx.x / kColsumCols;
  const int j = blockIdx.x * kColsumCols + jj;
  const int cpg = (nchunks + kColsumGroups - 1) / kColsumGroups;   // <= 16
  const int c0 = g * cpg;
  int hv[16];
  int mine = 0;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    hv[u] = (u < cpg && c0 + u < nchunks && j < d_in)
                ? hist[static_cast<int64_t>(c0 + u) * d_in + j] : 0;
    mine += hv[u];
  }
  gsum[g][jj] = mine;
  __syncthreads();
  int run = 0, total = 0;
  for (int q = 0; q < kColsumGroups; ++q) {
    const int v = gsum[q][jj];
    if (q < g) run += v;
    total += v;
  }
  if (j >= d_in) return;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    if (u < cpg && c0 + u < nchunks) hist[static_cast<int64_t>(c0 + u) * d_in + j] = run;
    run += hv[u];
  }
  if (g == 0) cnt[j] = total;
}

// col_ptr = exclusive scan of the column counts (cnt may alias col_ptr).
// Thread t owns the contiguous columns [t * cpt, (t+1) * cpt): one block scan.
__global__ __launch_bounds__(1024) void csc_scan_kernel(int32_t* __restrict__ col_ptr, int d_in) {
  __shared__ int scan_tmp[16];
  const int cpt = (d_in + 1023) / 1024;
  const int j0 = threadIdx.x * cpt, j1 = min(j0 + cpt, d_in);
  int sum = 0;
  for (int j = j0; j < j1; ++j) sum += col_ptr[j];
  int total;
  int pos = block_excl_scan_i32(sum, scan_tmp, &total);
  for (int j = j0; j < j1; ++j) {
    const int c = col_ptr[j];
    col_ptr[j] = pos;
    pos += c;
  }
  if (threadIdx.x == 0) col_ptr[d_in] = total;
}

__global__ __launch_bounds__(kCscThreads) void csc_place_kernel(const int32_t* __restrict__ row_ptr,
                                                                const int32_t* __restrict__ E,
                                                                int d_out, int d_in, int nchunks,
                                                                const int32_t* __restrict__ col_ptr,
                                                                const int32_t* __restrict__ before,
                                                                int32_t* __restrict__ perm) {
  extern __shared__ int run[];
  const int ch = blockIdx.x;
  const int r0 = static_cast<int>(static_cast<int64_t>(d_out) * ch / nchunks);
  const int r1 = static_cast<int>(static_cast<int64_t>(d_out) * (ch + 1) / nchunks);
  for (int j = threadIdx.x; j < d_in; j += kCscThreads) run[j] = 0;
  __syncthreads();
  for (int r = r0; r < r1; ++r) {
    for (int k = row_ptr[r] + threadIdx.x; k < row_ptr[r + 1]; k += kCscThreads) {
      const int j = E[2 * static_cast<int64_t>(k) + 1];
      const int slot = col_ptr[j] + before[static_cast<int64_t>(ch) * d_in + j] + run[j];
      run[j] += 1;
      perm[slot] = k;
    }
    __syncthreads();
  }
}

// The same placement with every row of the chunk at once, for chunks of at
// most 64 rows: bit r of mask[j] marks that row r0 + r holds column j (a
// row's columns are distinct), so an entry's rank among its column's entries
// in earlier rows of the chunk is a popcount, whatever the order the bits
// were set in.
constexpr int kCscMaskRows = 64;

__global__ __launch_bounds__(kCscThreads) void csc_place_mask_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ E, int d_out, int d_in,
    int nchunks, const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ before,
    int32_t* __restrict__ perm) {
  extern __shared__ unsigned long long mask[];
  const int ch = blockIdx.x;
  const int r0 = static_cast<int>(static_cast<int64_t>(d_out) * ch / nchunks);
  const int r1 = static_cast<int>(static_cast<int64_t>(d_out) * (ch + 1) / nchunks);
  for (int j = threadIdx.x; j < d_in; j += kCscThreads) mask[j] = 0;
  __syncthreads();
  const int k0 = row_ptr[r0], k1 = row_ptr[r1];
  for (int k = k0 + threadIdx.x; k < k1; k += kCscThreads) {
    const int r = E[2 * static_cast<int64_t>(k)] - r0;
    const int j = E[2 * static_cast<int64_t>(k) + 1];
    atomicOr(&mask[j], 1ull << r);
  }
  __syncthreads();
  for (int k = k0 + threadIdx.x; k < k1; k += kCscThreads) {
    const int r = E[2 * static_cast<int64_t>(k)] - r0;
    const int j = E[2 * static_cast<int64_t>(k) + 1];
    const int rank = __popcll(mask[j] & ((1ull << r) - 1ull));
    perm[col_ptr[j] + before[static_cast<int64_t>(ch) * d_in + j] + rank] = k;
  }
}

hipError_t launch_csc_build(const int32_t* row_ptr, const int32_t* E, int d_out, int d_in,
                            int32_t* col_ptr, int32_t* csc_perm, void* scratch, hipStream_t s) {
  const int nchunks = csc_chunks(d_out);
  int32_t* hist = static_cast<int32_t*>(scratch);
  const size_t sh = static_cast<size_t>(d_in) * 4;
  hipLaunchKernelGGL(csc_hist_kernel, dim3(nchunks), dim3(kCscThreads), sh, s, row_ptr, E, d_out,
                     d_in, nchunks, hist);
  hipLaunchKernelGGL(csc_colsum_kernel, dim3((d_in + kColsumCols - 1) / kColsumCols),
                     dim3(kColsumCols * kColsumGroups), 0, s, hist, d_in, nchunks, col_ptr);
  hipLaunchKernelGGL(csc_scan_kernel, dim3(1), dim3(1024), 0, s, col_ptr, d_in);
  // rows per chunk <= 64 and the masks fit in LDS: all rows of a chunk at once
  const int rows_per_chunk = (d_out + nchunks - 1) / nchunks;
  const size_t shm = static_cast<size_t>(d_in) * 8;
  if (rows_per_chunk <= kCscMaskRows && shm <= 160 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(csc_place_mask_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(shm));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(csc_place_mask_kernel, dim3(nchunks), dim3(kCscThreads), shm, s, row_ptr,
                       E, d_out, d_in, nchunks, col_ptr, hist, csc_perm);
  } else {
    hipLaunchKernelGGL(csc_place_kernel, dim3(nchunks), dim3(kCscThreads), sh, s, row_ptr, E,
                       d_out, d_in, nchunks, col_ptr, hist, csc_perm);
  }
  return hipGetLastError();
}

}  // namespace qwha
