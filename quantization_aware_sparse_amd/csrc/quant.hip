// The quantized base layer with the adapter (the inference path; QWHA notes,
// papernotes.org, 损失函数 / 训练策略: the adapter is merged into the
// group-quantized model; gist.science summary §4 for its inference cost).
//
// Weights are b-bit codes q with a scale s and zero z per group of `group`
// input columns: W_Q = (q - z) * s. Codes are stored floor(32/b) to a uint32
// word, code j of a row in word j / cpw at bit (j % cpw) * b.
//
//   merge_kernel  W = W_Q + alpha F H^-1 per row: the materialisation of
//                 the adapter (scatter c into LDS, FWHT) with the
//                 dequantized row added before the single store;
//   qgemm_kernel  y = x W_Q^T + add on the bf16 matrix cores
//                 (v_mfma_f32_16x16x32_bf16): the weight operand is q - z,
//                 an integer that bf16 holds exactly; each group's partial
//                 sums are scaled by s in fp32 and accumulated, so the only
//                 roundings are those of the fp32 sums. `add` carries the
//                 adapter's alpha z F^T (fp32) into the single bf16 store.
//                 2-, 3- and 8-bit codes;
//   qgemm4_ring_kernel  the same product for 4-bit codes, its operands
//                 loaded straight into LDS two steps ahead.
#include <type_traits>

#include "fwht_core.h"
#include "launch.h"

namespace qwha {

namespace {

__device__ __forceinline__ float dequant(const QuantW& qw, int64_t row, int j) {
  const uint32_t wi = __umulhi(static_cast<uint32_t>(j), qw.cpw_magic);   // j / cpw
  const int sh = (j - static_cast<int>(wi) * qw.cpw) * qw.bits;
  const uint32_t w = qw.codes[row * qw.wpr + wi];
  const float q = static_cast<float>((w >> sh) & ((1u << qw.bits) - 1u));
  const int64_t g = row * qw.gpr + (j >> qw.lg_group);
  return (q - qw.zeros[g]) * qw.scales[g];
}

template <int LOG_N>
struct MergeCfg {
  using F = Fwht<LOG_N>;
  static constexpr int BLOCK = F::TPR > 256 ? F::TPR : 256;
  static constexpr int RPW = BLOCK / F::TPR;
};

template <int LOG_N, typename TOut>
__global__ __launch_bounds__(MergeCfg<LOG_N>::BLOCK) void merge_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ E,
    const float* __restrict__ c, int d_out, int nblk, float scale, QuantW qw,
    TOut* __restrict__ W) {
  using F = Fwht<LOG_N>;
  constexpr int RPW = MergeCfg<LOG_N>::RPW;
  __shared__ float lds_all[RPW * F::LDS];
  const int slot = threadIdx.x / F::TPR;
  const int u = threadIdx.x % F::TPR;
  // virtual row r of the [d_out * nblk][N] view: block blk of row i
  const int vrow = blockIdx.x * RPW + slot;
  const bool live = vrow < d_out * nblk;
  const int row = vrow / nblk, blk = vrow - row * nblk;
  float* lds = lds_all + slot * F::LDS;

  for (int j = u; j < F::LDS; j += F::TPR) lds[j] = 0.f;
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
    TOut* dst = W + static_cast<int64_t>(vrow) * F::N;
#pragma unroll
    for (int r = 0; r < F::EPT; ++r) {
      const int j = F::out_index(u, r);
      Elem<TOut>::st(dst, j, dequant(qw, row, blk * F::N + j) + v[r] * scale);
    }
  }
}

template <int LOG_N, typename TOut>
hipError_t merge_t(const int32_t* row_ptr, const int32_t* E, const float* c, int d_out,
                   int nblk, float scale, const QuantW& qw, void* W, hipStream_t s) {
  constexpr int RPW = MergeCfg<LOG_N>::RPW;
  const int blocks = (d_out * nblk + RPW - 1) / RPW;
  hipLaunchKernelGGL((merge_kernel<LOG_N, TOut>), dim3(blocks), dim3(MergeCfg<LOG_N>::BLOCK), 0,
                     s, row_ptr, E, c, d_out, nblk, scale, qw, static_cast<TOut*>(W));
  return hipGetLastError();
}

// ------------------------------------------------------------------ GEMM
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQT = 128;       // tile: tokens and output rows
constexpr int kQK = 64;        // K per step (two MFMAs deep)
constexpr int kQLd = kQK + 8;  // LDS row stride, bf16
constexpr int kXcd = 8;        // XCDs (workgroups go round-robin over them)

__device__ __forceinline__ uint16_t bf16_bits_exact(float v) {
  return static_cast<uint16_t>(__float_as_uint(v) >> 16);   // v is a small integer
}

// Code words covering 16 consecutive columns of a row: 16 / CPW whole words
// when CPW divides 16, else up to 3 words from the one holding the first.
template <int BITS>
struct Codes16 {
  static constexpr int CPW = 32 / BITS;
  static constexpr bool ALIGNED = (16 % CPW) == 0;
  static constexpr int NW = ALIGNED ? 16 / CPW : 3;
};

// words for columns k0..k0+15 of the row (wpr words long)
template <int BITS>
__device__ __forceinline__ void load_codes16(const uint32_t* __restrict__ row_words, int k0,
                                             int wpr, uint32_t* w) {
  using C = Codes16<BITS>;
  const int base = k0 / C::CPW;
#pragma unroll
  for (int i = 0; i < C::NW; ++i) w[i] = row_words[min(base + i, wpr - 1)];
}

// those 16 codes as q - z in bf16 (exact for |q - z| <= 256), two to a word
template <int BITS>
__device__ __forceinline__ void unpack16(const uint32_t* w, int k0, float z, uint32_t* out) {
  using C = Codes16<BITS>;
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  const int base = k0 / C::CPW;
  uint16_t h[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    uint32_t q;
    if constexpr (C::ALIGNED) {
      q = (w[e / C::CPW] >> ((e % C::CPW) * BITS)) & MASK;
    } else {
      const int j = k0 + e;
      q = (w[j / C::CPW - base] >> ((j % C::CPW) * BITS)) & MASK;
    }
    h[e] = bf16_bits_exact(static_cast<float>(q) - z);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    out[i] = static_cast<uint32_t>(h[2 * i]) | (static_cast<uint32_t>(h[2 * i + 1]) << 16);
}

// y[t][n] = bf16(sum_g s[n][g] * sum_{k in g} x[t][k] (q[n][k] - z[n][g]) + add[t][n]).
// 256 threads, a 128 (tokens) x 128 (output rows) tile, 64x64 per wave as
// 4x4 blocks of 16x16; K in steps of 64 through double-buffered LDS (one
// barrier per step), the next step's loads in flight during the MFMAs.
// Tile order: workgroup b runs on XCD b % 8; when the output-row tiles
// split evenly over the XCDs, each XCD keeps its own 1/8 of them (their
// codes stay in its L2) and walks the token tiles, so a token tile is read
// by its XCD's workgroups at about the same time.
// MFMA operands: lane l holds row / column l%16 and k 8(l/16)..+8; result
// register r of lane l is row 4(l/16)+r, column l%16, so a lane's results
// share one output row n and one group scale.
template <int BITS>
__global__ __launch_bounds__(256, 2) void qgemm_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                       int K, int N, QuantW qw,
                                                       const float* __restrict__ add,
                                                       uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kQT][kQLd];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kQT][kQLd];
  const int ntn = (N + kQT - 1) / kQT;
  int tm, tn;
  {
    const int b = blockIdx.x;
    if (ntn % kXcd == 0) {
      const int per = ntn / kXcd, slot = b / kXcd;
      tm = slot / per;
      tn = (b % kXcd) * per + slot % per;
    } else {
      tm = b / ntn;
      tn = b % ntn;
    }
  }
  const int64_t m0 = static_cast<int64_t>(tm) * kQT;
  const int n0 = tn * kQT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;

  f32x4 acc[4][4], gacc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      gacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // staging: thread -> row tid/2, 32 columns at (tid&1)*32 (two 16-column halves)
  const int sr = tid >> 1, sk = (tid & 1) * 32;
  const int64_t xrow = m0 + sr;
  const bool xlive = xrow < T;
  const uint16_t* xp = x + (xlive ? xrow : 0) * K + sk;
  const int wrow = n0 + sr;
  const bool wlive = wrow < N;
  const uint32_t* wp = qw.codes + static_cast<int64_t>(wlive ? wrow : 0) * qw.wpr;
  const float* zp = qw.zeros + static_cast<int64_t>(wlive ? wrow : 0) * qw.gpr;

  uint4 xa[4];
  uint32_t cw[2][Codes16<BITS>::NW];
  float zc = 0.f;
  int kf = 0;
  // global loads of a step (raw code words; unpacked when staged); the 32
  // columns of a thread lie in one group (groups are >= 32 columns, aligned)
  auto fetch = [&](int k0) {
    kf = k0 + sk;
    if (xlive) {
      const uint4* q = reinterpret_cast<const uint4*>(xp + k0);
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = q[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = uint4{0u, 0u, 0u, 0u};
    }
    if (wlive) {
      load_codes16<BITS>(wp, kf, qw.wpr, cw[0]);
      load_codes16<BITS>(wp, kf + 16, qw.wpr, cw[1]);
      zc = zp[kf >> qw.lg_group];
    }
  };
  auto stage = [&](int buf) {
    uint4* da = reinterpret_cast<uint4*>(&As[buf][sr][sk]);
#pragma unroll
    for (int i = 0; i < 4; ++i) da[i] = xa[i];
    uint4* db = reinterpret_cast<uint4*>(&Bs[buf][sr][sk]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t wb[8];
      if (wlive) {
        unpack16<BITS>(cw[h], kf + 16 * h, zc, wb);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) wb[i] = 0u;
      }
      db[2 * h] = uint4{wb[0], wb[1], wb[2], wb[3]};
      db[2 * h + 1] = uint4{wb[4], wb[5], wb[6], wb[7]};
    }
  };

  // group >= 64: whole steps per group; group 32: two groups per step
  const int steps_per_group = (1 << qw.lg_group) >= kQK ? (1 << qw.lg_group) / kQK : 1;
  fetch(0);
  stage(0);
  __syncthreads();
  int buf = 0;
  const int nsteps = K / kQK;
  for (int st = 0; st < nsteps; ++st) {
    const int k0 = st * kQK;
    if (st + 1 < nsteps) fetch(k0 + kQK);
#pragma unroll
    for (int kh = 0; kh < kQK / 32; ++kh) {
      const int kc = kh * 32 + 8 * (lane >> 4);
      bf16x8 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&As[buf][wm + i * 16 + (lane & 15)][kc]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][wn + j * 16 + (lane & 15)][kc]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          gacc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], gacc[i][j], 0, 0, 0);
      // a group ends after this half-step: with 32-column groups every half,
      // else at the end of the group's last step
      const bool ends = (1 << qw.lg_group) < kQK ? true
                                                 : (kh == kQK / 32 - 1 && (st + 1) % steps_per_group == 0);
      if (ends) {
        const int g = (k0 + kh * 32) >> qw.lg_group;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn + j * 16 + (lane & 15);
          const float sc = n < N ? qw.scales[static_cast<int64_t>(n) * qw.gpr + g] : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[i][j] += sc * gacc[i][j];
            gacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
    }
    if (st + 1 < nsteps) stage(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = m0 + wm + i * 16 + 4 * (lane >> 4) + r;
        if (t < T && n < N) {
          const int64_t at = t * N + n;
          y[at] = f32_to_bf16(add ? acc[i][j][r] + add[at] : acc[i][j][r]);
        }
      }
    }
}

// ---- 4-bit codes: a three-step ring of direct-to-LDS loads
// Same tile, wave split and MFMA layout as qgemm_kernel, with two changes:
// - x, the code words and the step's scales and zeros go global -> LDS by
//   global_load_lds (no staging registers), two steps ahead of use, so their
//   latency hides behind two steps of MFMA;
// - the weight operand is 128 + q, whose bf16 bits are 0x4300 | q (a byte
//   permute and an and-or per pair of codes), and the zero point comes back
//   per group:
//   sum_k x (q - z) = sum_k x (128 + q) - (128 + z) sum_k x, with sum_k x
//   from one more MFMA per 16 tokens against a ones operand. Products and
//   sums stay exact in fp32 up to the order of the fp32 additions.
constexpr int kRing = 3;

// 16-byte chunk slot of k-chunk c (0..7) in row r of a 128-byte LDS row:
// conflict-free ds_read_b128 over 16 consecutive rows
__device__ __forceinline__ int qswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Direct-to-LDS loads: lane l's bytes go from sbase + voff to LDS at m0 +
// size * l (m0 wave-uniform). Issued in asm so that the compiler adds no
// waits of its own before later LDS reads; every wait on them is explicit
// (wait_vm). An LDS address is the low half of the generic address. M0 is
// a reserved register the compiler sets itself before each of its own uses
// (on gfx950 LDS instructions need none; this kernel has no other use), so
// it is not listed as clobbered.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff),
               "s"(sbase), "s"(m0)
               : "memory");
}
__device__ __forceinline__ void dma4(uint32_t voff, const void* sbase, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff),
               "s"(sbase), "s"(m0)
               : "memory");
}

// bf16x8 of 128 + q for the 8 codes of a word (bf16(128 + q) = 0x4300 | q):
// dword i takes byte i of w (low nibble q_2i) and byte i of w >> 4 (low
// nibble q_2i+1) into its bytes 0 and 2, then keeps those nibbles
__device__ __forceinline__ bf16x8 unpack_off128(uint32_t w, uint32_t mask) {
  const uint32_t u = w >> 4;
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = __builtin_amdgcn_perm(u, w, 0x0C040C00u + 0x00010001u * i);
    // (x & mask) | 0x43004300 in one instruction (mask 0x000F000F in a VGPR:
    // one scalar operand per VALU instruction on this target)
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d[i]) : "v"(x), "v"(mask), "s"(0x43004300u));
  }
  bf16x8 r;
  __builtin_memcpy(&r, d, 16);
  return r;
}

// ring slot S: its own LDS arrays, so that every LDS address of a step is a
// compile-time constant (the step loop is unrolled over the three slots)
template <int S>
struct RingSlot {
  static __device__ __forceinline__ uint16_t* A() {
    __shared__ __attribute__((aligned(16))) uint16_t a[kQT * kQK];   // 16 KiB
    return a;
  }
  static __device__ __forceinline__ uint32_t* C() {
    __shared__ __attribute__((aligned(16))) uint32_t c[kQT * 8];     // 4 KiB
    return c;
  }
  static __device__ __forceinline__ float* SZ() {
    __shared__ __attribute__((aligned(16))) float sz[512];            // scales | zeros, 2 halves
    return sz;
  }
};

template <bool G32>
__global__ __launch_bounds__(256, 2) void qgemm4_ring_kernel(const uint16_t* __restrict__ x,
                                                             int64_t T, int K, int N, QuantW qw,
                                                             const float* __restrict__ add,
                                                             uint16_t* __restrict__ y) {
  const int ntn = (N + kQT - 1) / kQT;
  int tm, tn;
  {
    const int b = blockIdx.x;
    if (ntn % kXcd == 0) {
      const int per = ntn / kXcd, slot = b / kXcd;
      tm = slot / per;
      tn = (b % kXcd) * per + slot % per;
    } else {
      tm = b / ntn;
      tn = b % ntn;
    }
  }
  const int64_t m0 = static_cast<int64_t>(tm) * kQT;
  const int n0 = tn * kQT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
  // the arrays are written only by the loads into LDS; this store (never
  // taken) keeps the compiler from treating their contents as undefined
  if (K < 0) {
    RingSlot<0>::A()[tid] = 0; RingSlot<1>::A()[tid] = 0; RingSlot<2>::A()[tid] = 0;
    RingSlot<0>::C()[tid] = 0; RingSlot<1>::C()[tid] = 0; RingSlot<2>::C()[tid] = 0;
    RingSlot<0>::SZ()[tid] = 0; RingSlot<1>::SZ()[tid] = 0; RingSlot<2>::SZ()[tid] = 0;
  }

  // ring loads: per-thread byte offsets from wave-uniform bases; rows past
  // T or N repeat the last row (their results are never stored). Code rows
  // are stored with half h of row n at 16-byte position 2n + (h ^ bit 3 of
  // n), so that the 16 rows a read covers hit distinct banks.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint16_t* xtile = x + m0 * K;
  uint32_t xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = i * 32 + w * 8 + (lane >> 3);
    const int c = (lane & 7) ^ qswz(r);
    const int64_t rr = (m0 + r < T ? m0 + r : T - 1) - m0;
    xoff[i] = static_cast<uint32_t>((rr * K + 8 * c) * 2);
  }
  const int cp = w * 64 + lane;                        // 16-byte position in the code slot
  const int cn = cp >> 1;                              // its code row
  const int chalf = (cp & 1) ^ ((cn >> 3) & 1);
  const uint32_t* ctile = qw.codes + static_cast<int64_t>(n0) * qw.wpr;
  const uint32_t coff = static_cast<uint32_t>(
      ((static_cast<int64_t>(n0 + cn < N ? n0 + cn : N - 1) - n0) * qw.wpr + 4 * chalf) * 4);
  const int szr = cp & 127;
  const float* sztile = (wu < 2 ? qw.scales : qw.zeros) + static_cast<int64_t>(n0) * qw.gpr;
  const uint32_t szoff =
      static_cast<uint32_t>((static_cast<int64_t>(n0 + szr < N ? n0 + szr : N - 1) - n0) * qw.gpr * 4);
  constexpr int kLoadsPerStep = 7;

  f32x4 acc[4][4], gacc[4][4], xsum[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xsum[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      gacc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  bf16x8 ones;
  {
    const uint32_t o[4] = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    __builtin_memcpy(&ones, o, 16);
  }
  const int gmask = (1 << qw.lg_group) - 1;
  uint32_t nib_mask = 0x000F000Fu;
  asm volatile("" : "+v"(nib_mask));   // kept in a VGPR
  const int lr = lane & 15, lq = lane >> 4;
  const int aswz = qswz(lr);
  const int nsteps = K / kQK;

  // exactly kLoadsPerStep loads per thread, always in this order: the
  // explicit vmcnt waits count on it
  auto issue = [&](auto slot_c, int st) {
    using RS = RingSlot<decltype(slot_c)::value>;
    const int k0 = st * kQK;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16(xoff[i], xtile + k0, lds_addr(RS::A()) + (i * 256 + wu * 64) * 16);
    dma16(coff, ctile + k0 / 8, lds_addr(RS::C()) + wu * 64 * 16);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      dma4(szoff, sztile + ((k0 + 32 * h) >> qw.lg_group), lds_addr(RS::SZ()) + (h * 256 + wu * 64) * 4);
  };

  // one step on ring slot S (its loads are in), issuing step st + 2's loads
  // into slot (S + 2) % 3 first. Both half-steps' operands are read up
  // front. A group's first half-step starts its sums from zero (no clears):
  // with 32-column groups every half-step, else the first half of a step
  // that starts a group.
  const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
  auto step = [&](auto slot_c, int st) {
    constexpr int S = decltype(slot_c)::value;
    using RS = RingSlot<S>;
    if (st + 2 < nsteps) issue(std::integral_constant<int, (S + 2) % kRing>{}, st + 2);
    const char* abase = reinterpret_cast<const char*>(RS::A());
    const uint32_t* cbase = RS::C();
    const float* szb = RS::SZ();
    bf16x8 af[2][4];
    uint32_t cw[2][4];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int kc = kh * 4 + lq;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[kh][i] = *reinterpret_cast<const bf16x8*>(abase + (wm + i * 16 + lr) * 128 +
                                                     16 * (kc ^ aswz));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        cw[kh][j] = cbase[(2 * (wn + j * 16 + lr) + (kh ^ (lr >> 3))) * 4 + lq];
    }
    const int k0 = st * kQK;
    const bool gstart = (k0 & gmask) == 0;
    auto half = [&](int kh, bool fresh) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xsum[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kh][i], ones, fresh ? zero4 : xsum[i],
                                                          0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 bf = unpack_off128(cw[kh][j], nib_mask);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          gacc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kh][i], bf,
                                                               fresh ? zero4 : gacc[i][j], 0, 0, 0);
      }
    };
    // y += s (sum x (128 + q) - (128 + z) sum x) for the group of half kh
    auto close = [&](int kh) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float sc = szb[kh * 256 + wn + j * 16 + lr];
        const float zo = 128.f + szb[kh * 256 + 128 + wn + j * 16 + lr];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i][j][r] = fmaf(sc, fmaf(-zo, xsum[i][r], gacc[i][j][r]), acc[i][j][r]);
      }
    };
    if (G32) {
      half(0, true);
      close(0);
      half(1, true);
      close(1);
    } else {
      if (gstart) half(0, true); else half(0, false);
      half(1, false);
      if (((k0 + kQK) & gmask) == 0) close(1);
    }
    if (st + 1 < nsteps) {
      // this wave's loads of step st + 1 are in (those of st + 2 may still
      // fly) and its LDS reads of this step are done; then every wave's
      if (st + 2 < nsteps) wait_vm<kLoadsPerStep>(); else wait_vm<0>();
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      lds_barrier();
    }
  };

  issue(std::integral_constant<int, 0>{}, 0);
  if (nsteps > 1) issue(std::integral_constant<int, 1>{}, 1);
  if (nsteps > 1) wait_vm<kLoadsPerStep>(); else wait_vm<0>();
  lds_barrier();
  for (int st = 0; st < nsteps; st += kRing) {
    step(std::integral_constant<int, 0>{}, st);
    if (st + 1 < nsteps) step(std::integral_constant<int, 1>{}, st + 1);
    if (st + 2 < nsteps) step(std::integral_constant<int, 2>{}, st + 2);
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn + j * 16 + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = m0 + wm + i * 16 + 4 * lq + r;
        if (t < T && n < N) {
          const int64_t at = t * N + n;
          y[at] = f32_to_bf16(add ? acc[i][j][r] + add[at] : acc[i][j][r]);
        }
      }
    }
}

}  // namespace

QuantW make_quant(const uint32_t* codes, const float* scales, const float* zeros, int bits,
                  int group, int d_in) {
  QuantW qw;
  qw.codes = codes;
  qw.scales = scales;
  qw.zeros = zeros;
  qw.bits = bits;
  qw.cpw = 32 / bits;
  qw.cpw_magic = static_cast<uint32_t>((0x100000000ull + qw.cpw - 1) / qw.cpw);
  qw.wpr = (d_in + qw.cpw - 1) / qw.cpw;
  int lg = 0;
  while ((1 << lg) < group) ++lg;
  qw.lg_group = lg;
  qw.gpr = d_in / group;
  return qw;
}

hipError_t launch_merge(const int32_t* row_ptr, const int32_t* E, const float* c, int d_out,
                        int log_n, float alpha, const QuantW& qw, Dt out_dt, void* W,
                        hipStream_t s, int nblk) {
  const float scale = alpha / static_cast<float>(1 << log_n);
  switch (log_n) {
#define QWHA_CASE(L)                                                        \
  case L:                                                                   \
    return out_dt == Dt::F32                                                \
               ? merge_t<L, float>(row_ptr, E, c, d_out, nblk, scale, qw, W, s)   \
               : merge_t<L, uint16_t>(row_ptr, E, c, d_out, nblk, scale, qw, W, s);
    QWHA_CASE(1) QWHA_CASE(2) QWHA_CASE(3) QWHA_CASE(4) QWHA_CASE(5) QWHA_CASE(6) QWHA_CASE(7)
    QWHA_CASE(8) QWHA_CASE(9) QWHA_CASE(10) QWHA_CASE(11) QWHA_CASE(12) QWHA_CASE(13)
    QWHA_CASE(14)
#undef QWHA_CASE
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_qgemm(const uint16_t* x, int64_t T, int K, int N, const QuantW& qw,
                        const float* add, uint16_t* y, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(((N + kQT - 1) / kQT) * ((T + kQT - 1) / kQT)));
  switch (qw.bits) {
    case 2:
      hipLaunchKernelGGL(qgemm_kernel<2>, grid, dim3(256), 0, s, x, T, K, N, qw, add, y);
      break;
    case 3:
      hipLaunchKernelGGL(qgemm_kernel<3>, grid, dim3(256), 0, s, x, T, K, N, qw, add, y);
      break;
    case 4:
      if (qw.lg_group == 5)
        hipLaunchKernelGGL(qgemm4_ring_kernel<true>, grid, dim3(256), 0, s, x, T, K, N, qw, add, y);
      else
        hipLaunchKernelGGL(qgemm4_ring_kernel<false>, grid, dim3(256), 0, s, x, T, K, N, qw, add, y);
      break;
    case 8:
      hipLaunchKernelGGL(qgemm_kernel<8>, grid, dim3(256), 0, s, x, T, K, N, qw, add, y);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qwha
