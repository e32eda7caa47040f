// Internal launchers (C++), called by the C-ABI layer in api.hip after it
// has validated every argument. Each returns the HIP error of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qwha {

enum class Dt : int { F32 = 0, BF16 = 1 };

// out[r][:] = scale * FWHT(in[r][:]) (+ out[r][:] if accumulate)
hipError_t launch_fwht(const void* in, Dt in_dt, void* out, Dt out_dt, int64_t rows,
                       int log_n, float scale, int accumulate, hipStream_t s);

// ---- init
hipError_t launch_row_norms(const float* dWq, int d_out, int d_in, double* w, hipStream_t s);
hipError_t launch_adaalloc(const double* w, int d_out, int d_in, int64_t p, int m, double t,
                           int32_t* row_ptr, void* scratch, hipStream_t s);
size_t adaalloc_scratch_bytes(int d_out);
// mode 0: AdaAlloc budgets in row_ptr, per-row threshold; mode 1 / 2: the
// global threshold *gtau on |C| / random keys (see select_global.hip)
// nblk > 1: rows of nblk blocks of 2^log_n columns under the block-diagonal
// transform (2^log_n in [64, 4096])
hipError_t launch_init_select(const float* dWq, int d_out, int log_n, const int32_t* row_ptr,
                              int32_t* E, float* c, int mode, const unsigned long long* gtau,
                              unsigned long long seed, hipStream_t s, int nblk = 1);

// ---- global selection variants (magnitude / random)
size_t global_select_scratch_bytes(int d_out, int d_in, int mode);
// keys (mode 1), the global threshold by radix select and the row budgets:
// writes row_ptr and the threshold at *gtau (inside the scratch)
hipError_t launch_global_budgets(const float* dWq, int d_out, int log_n, int64_t p, int mode,
                                 unsigned long long seed, int32_t* row_ptr, void* scratch,
                                 const unsigned long long** gtau, hipStream_t s, int nblk = 1);
size_t csc_scratch_bytes(int d_out, int d_in);
hipError_t launch_csc_build(const int32_t* row_ptr, const int32_t* E, int d_out, int d_in,
                            int32_t* col_ptr, int32_t* csc_perm, void* scratch, hipStream_t s);

// ---- refinement with a calibration Hessian (refine.hip)
// Hs (+)= X^T X, fp64 [d_in][d_in], X [N][d_in] in x_dt
hipError_t launch_hessian(const void* X, Dt x_dt, int64_t N, int d_in, double* Hs,
                          int accumulate, hipStream_t s);
size_t calibrated_scratch_bytes(int d_out, int d_in);
// delta = damp * mean(diag Hs); M = dW_Q Hs; per row w_i (activation error
// norm, returned in *w_out, inside the scratch) and Q = (M + delta dW_Q) H / n
hipError_t launch_calib_prepare(const float* dWq, int d_out, int log_n, const double* Hs,
                                double damp, void* scratch, double** w_out, hipStream_t s,
                                int nblk = 1);
// rhs[k] = Q[E_k]; G = H Hs H / n^2 + (delta / n) I
hipError_t launch_calib_finish(const int32_t* E, int64_t p, int d_out, int log_n,
                               const double* Hs, void* scratch, double* G, double* rhs,
                               hipStream_t s, int nblk = 1);
size_t refine_header_bytes(int d_out);
hipError_t launch_refine(const int32_t* row_ptr, const int32_t* E, const double* G, int d_in,
                         const double* rhs, int d_out, float* c, int32_t* status, void* ws,
                         size_t ws_bytes, double pivot_tol, hipStream_t s);

// ---- quantized base layer (quant.hip)
// b-bit codes, floor(32/b) per uint32 word (code j in word j / cpw at bit
// (j % cpw) * b), scale and zero per group of 2^lg_group columns
struct QuantW {
  const uint32_t* codes;
  const float* scales;
  const float* zeros;
  int bits, cpw;
  uint32_t cpw_magic;   // ceil(2^32 / cpw): j / cpw = umulhi(j, cpw_magic) for j < 2^16
  int wpr;              // words per row
  int lg_group;
  int gpr;              // groups per row
};
QuantW make_quant(const uint32_t* codes, const float* scales, const float* zeros, int bits,
                  int group, int d_in);
// W = W_Q + alpha F H^-1
hipError_t launch_merge(const int32_t* row_ptr, const int32_t* E, const float* c, int d_out,
                        int log_n, float alpha, const QuantW& qw, Dt out_dt, void* W,
                        hipStream_t s, int nblk = 1);
// y = bf16(x W_Q^T + add), x bf16 [T][K], add fp32 [T][N], y bf16 [T][N]
hipError_t launch_qgemm(const uint16_t* x, int64_t T, int K, int N, const QuantW& qw,
                        const float* add, uint16_t* y, hipStream_t s);

// ---- materialize
// nblk > 1: rows of nblk blocks of 2^log_n columns (block-diagonal transform)
hipError_t launch_materialize(const int32_t* row_ptr, const int32_t* E, const float* c, int d_out,
                              int log_n, float alpha, Dt out_dt, void* dW, int accumulate,
                              hipStream_t s, int nblk = 1);

// ---- adapter forward / backward (gather SpMM / SDDMM)
struct SpmmPlan {
  int kind;      // 1: plain gather (entry pairs), 2: with dc partials (single entries)
  int tt;        // tokens per tile
  int jb;        // source columns per staged block
  int rows_wg;   // output rows per workgroup
  int nblk;      // source blocks
  int64_t ntiles;
  int seg_mult;  // (row, block) segments padded with zero entries to a multiple of this
  int ptr_stride;  // per-block segment table stride (>= n_out + 1)
  int esz;       // bytes per staged source element (4: fp32, 2: bf16 kept as bf16)
};
// stage16: the product with dc partials on a bf16 source, staged as bf16 in
// blocks of 128 columns (same LDS bytes as 64 fp32 columns)
SpmmPlan spmm_plan(int64_t T, int n_src, int n_out, int64_t nnz, bool dc, bool stage16 = false);
size_t spmm_prep_bytes(int64_t nnz, int n_out, const SpmmPlan& pl);
// index k in E of each entry of the prepared stream (stream order)
const int32_t* spmm_prep_korig(const void* prep, int64_t nnz, int n_out, const SpmmPlan& pl);

// Rows of F (forward): the column-block-major stream of (LDS byte offset of
// the column within its block, value) from row_ptr / E / c.
hipError_t launch_prep_csr(const int32_t* row_ptr, const int32_t* E, const float* c, int d_out,
                           int64_t nnz, const SpmmPlan& pl, void* prep, hipStream_t s);
// Columns of F (backward): the same from col_ptr / csc_perm / E / c.
hipError_t launch_prep_csc(const int32_t* col_ptr, const int32_t* csc_perm, const int32_t* E,
                           const float* c, int d_in, int64_t nnz, const SpmmPlan& pl, void* prep,
                           hipStream_t s);

// The same streams built from E alone (values 0, korig kept in both
// directions), and the per-call gather of the values from c.
hipError_t launch_prep_structure(const int32_t* seg_ptr, const int32_t* E, const int32_t* perm,
                                 int n_out, int64_t nnz, const SpmmPlan& pl, void* prep,
                                 hipStream_t s);
hipError_t launch_prep_refresh(const float* c, int64_t nnz, int n_out, const SpmmPlan& pl,
                               void* prep, hipStream_t s);

// out[t][o] (+)= alpha * sum_k val_k * src[t][col_k]; with zsrc, also
// partial[tile][q] = sum_{t in tile} src[t][col_q] * zsrc[t][o] per stream entry q.
hipError_t launch_spmm(const void* src, Dt src_dt, int64_t T, int n_src, const void* prep,
                       int64_t nnz, int n_out, const SpmmPlan& pl, float alpha, void* out,
                       Dt out_dt, int accumulate, const float* zsrc, float* partial,
                       hipStream_t s);

// dc[korig[q]] = alpha * sum_tile partial[tile][q]   (fixed tile order)
hipError_t launch_dc_reduce(const float* partial, int64_t ntiles, int64_t nnz,
                            const int32_t* korig, float alpha, float* dc, hipStream_t s);

hipError_t launch_sign_update(float* c, const float* dc, int64_t p, float step, hipStream_t s);

}  // namespace qwha
