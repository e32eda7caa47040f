/*
 * qwha.h -- C-ABI of the MI355X (gfx950) Walsh-Hadamard adapter (WHA) library.
 *
 * The adapter of QWHA writes the weight update as dW = alpha * F H^-1 where
 * H is the frozen Sylvester Walsh-Hadamard matrix (entries +-1, applied along
 * the input dimension only, H^-1 = H / d_in) and F = Scatter(c, E) is a
 * sparse d_out x d_in coefficient matrix with p nonzeros: positions E
 * (p x 2) and values c (p). Only c is trained; W_Q and H stay frozen.
 *   Sources: QWHA notes, papernotes.org (ICLR 2026), 方法详解 › 整体框架 and
 *   关键设计 1-3, 损失函数 / 训练策略; QWHA technical summary, gist.science
 *   (arXiv 2509.17428), §2.1 Adapter Design, §2.2 Quantization-Aware
 *   Initialization.
 *
 * Conventions for every entry point:
 *  - Ownership: all array arguments are DEVICE pointers owned by the caller;
 *    the library never allocates, frees or keeps a pointer past the work it
 *    enqueues. Buffers must stay alive until that work has run.
 *  - Asynchrony: work is enqueued on `stream` and the call returns at once.
 *  - Validation: arguments are checked on the host before anything is
 *    enqueued; a non-OK status means nothing was enqueued.
 *    qwha_last_error() (thread-local) then says why.
 *  - Layout: dense matrices are row-major and contiguous. E is int32 [p][2]
 *    holding (row i, column j), sorted by (i, j). row_ptr is int32
 *    [d_out + 1] (exclusive scan of the per-row budgets). col_ptr is int32
 *    [d_in + 1] and csc_perm int32 [p] lists positions k of E column by
 *    column, ascending k within a column.
 *  - Alignment: dense activation / weight arrays and workspaces must be
 *    16-byte aligned, index and value arrays 4-byte aligned
 *    (QWHA_ERR_ALIGN otherwise).
 *  - Shapes: 2 <= d_in <= 16384, 1 <= d_out <= 1048576, T >= 0 (T == 0
 *    is a no-op), p <= 2^31 - 1 (QWHA_ERR_SHAPE otherwise). The calls that
 *    run the gather-SpMM (qwha_fwd, qwha_fwd_save, qwha_bwd, qwha_bwd_saved,
 *    qwha_layer_fwd) take p <= (2^31 - 65) / 2 = 1073741791, since their
 *    prepared stream of at most 2p + 16 entries is indexed in int32
 *    (QWHA_ERR_BUDGET otherwise; their workspace queries return 0). The transform
 *    H is the Sylvester matrix of order d_in when d_in is a power of two.
 *    Otherwise d_in = m * b, with b the largest power of two dividing it
 *    (m odd), and H is block-diagonal with m Sylvester blocks of order b,
 *    H^-1 = H / b, so every "/ n" below reads "/ b". The pages only use
 *    power-of-two widths; this reading keeps the +-1 entries, orthogonality
 *    and the fast transform. It requires b >= 64 (d_in = 14336 = 7 * 2048
 *    qualifies, 96 = 3 * 32 does not). qwha_fwht takes powers of two only.
 *  - Aliasing: inputs and outputs must not overlap, except that an output is
 *    read back when its `accumulate` flag is set.
 *  - Preconditions not checked (they would need device reads): inputs are
 *    finite; row_ptr[d_out] == p; E / row_ptr / col_ptr / csc_perm are the
 *    consistent output of qwha_init_select (or equivalent).
 *  - Calls are reentrant; there is no global state apart from the
 *    thread-local error string and the thread-local profiling request of
 *    qwha_profile_next().
 */
#ifndef QWHA_H
#define QWHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t; /* HIP's opaque stream handle; NULL = default stream */
typedef struct ihipEvent_t* hipEvent_t;   /* HIP's opaque event handle */

typedef enum qwha_status {
  QWHA_OK = 0,
  QWHA_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad flag or scalar */
  QWHA_ERR_SHAPE = 2,       /* d_in not a supported width (see Shapes), d_out or T out of range */
  QWHA_ERR_BUDGET = 3,      /* p outside its allowed range */
  QWHA_ERR_DTYPE = 4,       /* unknown qwha_dtype */
  QWHA_ERR_ALIGN = 5,       /* pointer not aligned as required */
  QWHA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than the *_workspace_bytes query */
  QWHA_ERR_HIP = 7          /* a HIP launch failed; qwha_last_error() has the HIP message */
} qwha_status;

typedef enum qwha_dtype { QWHA_F32 = 0, QWHA_BF16 = 1 } qwha_dtype;

/* Static strings; never NULL. */
const char* qwha_status_string(qwha_status s);
/* Message of the last failed call on this thread ("" if none). */
const char* qwha_last_error(void);
/* Library ABI version (major * 100 + minor). */
int32_t qwha_version(void);

/* ---------------------------------------------------------------------------
 * Quantization-aware initialisation (papernotes.org, 关键设计 2 AdaAlloc and
 * 3 Value Refinement; gist.science §2.2).
 *
 * From the quantization error dWq = W0 - W_Q (fp32 [d_out][d_in]):
 *   1. w_i = ||dWq[i,:]||_2 (fp64): each output channel's error magnitude
 *      (identity Hessian: no calibration activations).
 *   2. AdaAlloc budgets p_i with sum p_i = p, by passes over the rows not
 *      yet held: each such row gets the share q_i = P s_i / S, with
 *      s_i = w_i^(1/temperature), P = p minus the budgets of the held rows
 *      and S the sum of s_i over the free rows, and p_i = floor(q_i). If any
 *      free row has q_i < min_per_row, those rows are held at min_per_row.
 *      Otherwise, if any free row has q_i > d_in, those rows are held at
 *      d_in and every row held at the floor is released again (capping a
 *      row raises the others' shares). The passes repeat until one holds
 *      nothing; this reaches the clamped proportional split
 *      clamp(lambda s_i, min_per_row, d_in). The leftover (< d_out) then
 *      goes one unit each to the rows with the smallest budget (lower row
 *      first, rows at d_in skipped). The exact formula is missing from the
 *      pages (papernotes.org, 关键设计 2 keeps only "proportional to each
 *      channel's error magnitude" with a temperature); this is that
 *      proportional reading (temperature 1 = linear).
 *   3. Dense solution C = dWq H (fp64 fast WHT per row).
 *   4. Row i keeps the p_i columns with the largest |C[i,j]|, ties to the
 *      lower column; they are written to E ascending, and
 *      c = fp32_RNE(C[i,j]) (value refinement with an identity Hessian
 *      returns the dense solution at the chosen positions).
 *   5. col_ptr / csc_perm: the column index of F (stable in k).
 * Outputs: row_ptr [d_out+1], E [p][2], c [p], col_ptr [d_in+1], csc_perm [p].
 * Requires min_per_row >= 0, min_per_row * d_out <= p <= d_in * d_out
 * (QWHA_ERR_BUDGET), temperature > 0 and finite, and a workspace of at least
 * qwha_init_workspace_bytes(d_out, d_in) bytes.
 * --------------------------------------------------------------------------- */
size_t qwha_init_workspace_bytes(int32_t d_out, int32_t d_in);
qwha_status qwha_init_select(const float* dWq, int32_t d_out, int32_t d_in, int64_t p,
                             int32_t min_per_row, double temperature, int32_t* row_ptr,
                             int32_t* E, float* c, int32_t* col_ptr, int32_t* csc_perm,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Materialisation (papernotes.org, 方法详解 › 整体框架; gist.science §2.1):
 *   dW = alpha * F H^-1 = (alpha / d_in) * Scatter(c, E) H
 * written to dW [d_out][d_in] in out_dtype (QWHA_F32 or QWHA_BF16, rounded
 * to nearest even); accumulate != 0 adds into the existing dW instead
 * (dW += alpha F H^-1, e.g. merging into a dequantized weight).
 * --------------------------------------------------------------------------- */
qwha_status qwha_materialize(const int32_t* row_ptr, const int32_t* E, const float* c,
                             int32_t d_out, int32_t d_in, int64_t p, float alpha,
                             qwha_dtype out_dtype, void* dW, int32_t accumulate,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Forward through the adapter branch (papernotes.org, 方法详解 › 整体框架):
 *   y = x dW^T = alpha * (FWHT(x) / d_in) F^T
 * x [T][d_in] and y [T][d_out] share the activation dtype `act`; math is fp32.
 * accumulate != 0 adds into y (the caller's base output x W_Q^T).
 * Workspace: qwha_fwd_workspace_bytes(T, d_in, d_out, p) bytes.
 * --------------------------------------------------------------------------- */
size_t qwha_fwd_workspace_bytes(int64_t T, int32_t d_in, int32_t d_out, int64_t p);
qwha_status qwha_fwd(const void* x, qwha_dtype act, int64_t T, int32_t d_in, int32_t d_out,
                     int64_t p, const int32_t* row_ptr, const int32_t* E, const float* c,
                     float alpha, void* y, int32_t accumulate, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Backward through the adapter branch, W_Q and H frozen, only c trainable
 * (papernotes.org, 损失函数 / 训练策略):
 *   dx   = dy dW = alpha * FWHT(dy F) / d_in               [T][d_in], dtype act
 *   dc_k = alpha * sum_t dy[t, i_k] * (FWHT(x)/d_in)[t, j_k]  [p], fp32
 * dx or dc may be NULL to skip that output; accumulate_dx != 0 adds into dx.
 * dc is reduced in a fixed order (deterministic).
 * Workspace: qwha_bwd_workspace_bytes(T, d_in, d_out, p) bytes.
 * --------------------------------------------------------------------------- */
size_t qwha_bwd_workspace_bytes(int64_t T, int32_t d_in, int32_t d_out, int64_t p);
qwha_status qwha_bwd(const void* x, const void* dy, qwha_dtype act, int64_t T, int32_t d_in,
                     int32_t d_out, int64_t p, const int32_t* row_ptr, const int32_t* E,
                     const float* c, const int32_t* col_ptr, const int32_t* csc_perm,
                     float alpha, void* dx, int32_t accumulate_dx, float* dc, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * qwha_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and kernels as qwha_fwd, with the workspace taken from a
 * static device array of 64 MiB (64 << 20 bytes) that the library holds on
 * each GPU it runs on until the process ends. The call itself allocates
 * nothing. A call whose qwha_fwd_workspace_bytes(T, d_in, d_out, p) exceeds
 * 64 MiB is rejected with QWHA_ERR_WORKSPACE (e.g. d_in = d_out = 4096,
 * p = 524288 takes T up to about 3300 tokens). The stream must belong to
 * the current device (QWHA_ERR_INVALID_ARG otherwise); the first call on a
 * device looks up the array's address there. Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (two streams, two host
 * threads) race and must be serialised by the caller. Nothing in the array
 * needs clearing between calls: each call writes all it reads.
 * --------------------------------------------------------------------------- */
qwha_status qwha_fwd_noalloc(const void* x, qwha_dtype act, int64_t T, int32_t d_in,
                             int32_t d_out, int64_t p, const int32_t* row_ptr, const int32_t* E,
                             const float* c, float alpha, void* y, int32_t accumulate,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * The same forward and backward with the forward's transform kept, as
 * autograd keeps a saved activation: qwha_fwd_save also writes
 * z = FWHT(x)/d_in to z (fp32 [T][d_in], caller-owned, 16-byte aligned),
 * and qwha_bwd_saved takes that z in place of x (dc uses it; x is neither
 * read nor transformed again). Workspaces as qwha_fwd / qwha_bwd. z must
 * hold the transform of the x the forward saw.
 * --------------------------------------------------------------------------- */
qwha_status qwha_fwd_save(const void* x, qwha_dtype act, int64_t T, int32_t d_in,
                          int32_t d_out, int64_t p, const int32_t* row_ptr, const int32_t* E,
                          const float* c, float alpha, void* y, int32_t accumulate, float* z,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);
qwha_status qwha_bwd_saved(const float* z, const void* dy, qwha_dtype act, int64_t T,
                           int32_t d_in, int32_t d_out, int64_t p, const int32_t* row_ptr,
                           const int32_t* E, const float* c, const int32_t* col_ptr,
                           const int32_t* csc_perm, float alpha, void* dx,
                           int32_t accumulate_dx, float* dc, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Adapters that read the same input (the q, k and v projections of an
 * attention block read the same x): the transform is linear and acts along
 * d_in only (papernotes.org, 方法详解 › 整体框架; gist.science §2.1), so
 * one z = FWHT(x)/d_in serves every adapter's forward and dc, and one
 * transform of the summed dz gives the summed dx:
 *   dx_q + dx_k + dx_v = FWHT(alpha_q dy_q F_q + alpha_k dy_k F_k
 *                             + alpha_v dy_v F_v) / d_in.
 * qwha_fwd_z:  y (+)= alpha z F^T from a z kept by qwha_fwd_save (fp32
 *   [T][d_in]); y in `act`. Workspace: qwha_fwd_workspace_bytes(...) bytes
 *   suffice (only the prepared stream is used).
 * qwha_bwd_dz: dz (+)= alpha dy F into the caller's fp32 dz [T][d_in]
 *   (accumulate_dz = 1 adds to it), and, when dc is not NULL, dc as in
 *   qwha_bwd from the kept z. No transform runs: dx = FWHT(dz)/d_in is then
 *   one qwha_fwht call with scale 1/d_in (rows T*m and n = b for a
 *   block-diagonal width). Workspace: qwha_bwd_workspace_bytes(...) bytes
 *   suffice (the prepared stream and the dc partials only are used).
 * --------------------------------------------------------------------------- */
qwha_status qwha_fwd_z(const float* z, qwha_dtype act, int64_t T, int32_t d_in, int32_t d_out,
                       int64_t p, const int32_t* row_ptr, const int32_t* E, const float* c,
                       float alpha, void* y, int32_t accumulate, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);
qwha_status qwha_bwd_dz(const float* z, const void* dy, qwha_dtype act, int64_t T,
                        int32_t d_in, int32_t d_out, int64_t p, const int32_t* E, const float* c,
                        const int32_t* col_ptr, const int32_t* csc_perm, float alpha, float* dz,
                        int32_t accumulate_dz, float* dc, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Plans: the structure of F that the gather-SpMMs walk, built once. E is
 * frozen after the init and only c trains (papernotes.org, 损失函数 / 训练策略),
 * so the streams qwha_fwd / qwha_bwd prepare on every call (the nonzeros in
 * column-block order, for the rows of F and for its columns) depend on E
 * alone; a plan keeps them, and each planned call only gathers the current
 * c into them (one small kernel per direction).
 *
 * qwha_plan_bytes: the plan's size for (d_in, d_out, p); 0 when out of range.
 * qwha_plan_build: builds the plan from row_ptr, E, col_ptr, csc_perm into
 *   `plan` (device, 256-byte aligned, at least qwha_plan_bytes) for
 *   activations of type `act` (the backward stages bf16 dy as bf16, in its
 *   own layout): the planned calls must pass the same act. Rebuild it
 *   whenever E changes.
 * qwha_fwd_plan: qwha_fwd on a plan: y (+)= alpha z F^T with z = FWHT(x)/d_in
 *   computed from x, or taken from z_in (a kept transform; x is then not
 *   read); z_out (optional, exclusive with z_in) keeps the transform as
 *   qwha_fwd_save does. Workspace: T * d_in * 4 bytes rounded up to 256 when
 *   neither z_in nor z_out is given, else none (qwha_fwd_workspace_bytes
 *   suffices).
 * qwha_bwd_plan: qwha_bwd_saved on a plan, from the kept z: dc as qwha_bwd
 *   (required), and either dx (+)= alpha FWHT(dy F)/d_in (dx not NULL) or,
 *   with dz not NULL, dz (+)= alpha dy F without the transform, as
 *   qwha_bwd_dz (dx and dz are exclusive; both NULL forms dc only).
 *   Workspace: qwha_bwd_workspace_bytes suffices.
 * The plan's values are rewritten by every planned call: calls that share a
 * plan must not overlap. The shapes, p and c must be those of the plan's
 * adapter (not checked: the plan lives on the device).
 * --------------------------------------------------------------------------- */
size_t qwha_plan_bytes(int32_t d_in, int32_t d_out, int64_t p);
qwha_status qwha_plan_build(const int32_t* row_ptr, const int32_t* E, const int32_t* col_ptr,
                            const int32_t* csc_perm, int32_t d_in, int32_t d_out, int64_t p,
                            qwha_dtype act, void* plan, size_t plan_bytes, hipStream_t stream);
qwha_status qwha_fwd_plan(const void* x, const float* z_in, qwha_dtype act, int64_t T,
                          int32_t d_in, int32_t d_out, int64_t p, void* plan, const float* c,
                          float alpha, void* y, int32_t accumulate, float* z_out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);
qwha_status qwha_bwd_plan(const float* z, const void* dy, qwha_dtype act, int64_t T,
                          int32_t d_in, int32_t d_out, int64_t p, void* plan, const float* c,
                          float alpha, void* dx, int32_t accumulate_dx, float* dz,
                          int32_t accumulate_dz, float* dc, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Coefficient update of the attention-block training step:
 *   c[k] += step * sign(dc[k])   (sign(0) = 0), fp32, in place.
 * --------------------------------------------------------------------------- */
qwha_status qwha_sign_update(float* c, const float* dc, int64_t p, float step,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Global selection variants of the init: the baselines AdaAlloc is compared
 * with (papernotes.org, 关键设计 2 (global top-p of the dense solution) and
 * 实验关键数据 › 消融实验, Table 4; gist.science §2.2).
 *   QWHA_SELECT_MAGNITUDE: the p positions of the whole matrix with the
 *     largest |C| (C = dWq H, fp64 as in qwha_init_select).
 *   QWHA_SELECT_RANDOM: p positions uniformly at random without
 *     replacement: the p smallest draws u[i][j] = SplitMix64 output
 *     i*d_in + j of the generator seeded with `seed` (Steele, Lea & Flood,
 *     OOPSLA 2014; output n is mix64(seed + (n+1) * 0x9E3779B97F4A7C15)).
 * Equal keys are taken in row-major order (lower row, then lower column).
 * The budgets p_i follow from the selection; E ascending per row and
 * c = fp32_RNE(C[i,j]) as in qwha_init_select (the values are the dense
 * solution for both strategies). Outputs as qwha_init_select. Requires
 * 0 <= p <= d_in * d_out (QWHA_ERR_BUDGET), a known strategy
 * (QWHA_ERR_INVALID_ARG) and a workspace of at least
 * qwha_init_global_workspace_bytes(d_out, d_in, strategy) bytes (0 for an
 * unknown strategy); the magnitude strategy keeps one 64-bit key per
 * position there (8 * d_out * d_in bytes).
 * --------------------------------------------------------------------------- */
enum { QWHA_SELECT_MAGNITUDE = 1, QWHA_SELECT_RANDOM = 2 };
size_t qwha_init_global_workspace_bytes(int32_t d_out, int32_t d_in, int32_t strategy);
qwha_status qwha_init_select_global(const float* dWq, int32_t d_out, int32_t d_in, int64_t p,
                                    int32_t strategy, uint64_t seed, int32_t* row_ptr,
                                    int32_t* E, float* c, int32_t* col_ptr, int32_t* csc_perm,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Value Refinement with calibration data (papernotes.org, 关键设计 2 and 3,
 * 损失函数 / 训练策略; gist.science §2.2).
 *
 * The init's objective is the layer-output error ||dW_Q X - F H^-1 X||_F^2
 * on calibration activations; with the Hessian Hs = XX^T it splits into
 * channels. Activations are token-major here ([N][d_in]), so Hs = X^T X.
 *
 * qwha_hessian: Hs (+)= X^T X in fp64 (X [N][d_in] fp32 or bf16, Hs
 *   [d_in][d_in] fp64, both triangles written). accumulate = 1 adds to Hs,
 *   which must then be symmetric (as this call leaves it): calibration
 *   batches can be summed call by call. N = 0 leaves Hs (or zeros it).
 *
 * qwha_init_select_calibrated: the init of qwha_init_select with
 *   Hs' = Hs + damp * mean(diag Hs) * I in place of the identity:
 *   w_i = sqrt(dW_Q[i] Hs' dW_Q[i]^T) (the activation error magnitude) for
 *   AdaAlloc; positions by the in-row top |C| (C = dW_Q H does not depend
 *   on Hs); c = fp32(C[E]) (the dense solution, refined by the next call);
 *   and the refinement system
 *     G   [d_in][d_in] fp64 = H Hs' H / d_in^2,
 *     rhs [p] fp64,  rhs_k = (dW_Q Hs' H / d_in)[i_k, j_k].
 *   damp >= 0 (0 = no damping, the plain reading). Other requirements as
 *   qwha_init_select, with a workspace of at least
 *   qwha_init_calibrated_workspace_bytes(d_out, d_in) bytes (it holds
 *   dW_Q Hs' and one d_in x d_in temporary, fp64).
 *
 * qwha_refine_values: for each row i with positions S = E_i, solves
 *   x G[S,S] = rhs[S] (the normal equations of min_x ||v - x B'||^2,
 *   v = dW_Q[i] R, B' the rows of H^-1 R at S) by Cholesky in fp64 and
 *   writes c[S] = fp32(x). A row whose pivot falls to or below 1e-10 times
 *   its diagonal entry of G (G[S,S] not positive definite) keeps its c
 *   and counts in status[0]; a row whose system does not fit the workspace
 *   keeps its c and counts in status[1] (status: device int32 [2], set by
 *   the call). Needs qwha_refine_workspace_bytes(row_ptr_host, d_out)
 *   bytes for every row to be solved, where row_ptr_host is a host copy of
 *   row_ptr (0 when it is not a valid row_ptr); at least
 *   8 * (d_out + 1) rounded up to 256 (QWHA_ERR_WORKSPACE otherwise).
 * --------------------------------------------------------------------------- */
qwha_status qwha_hessian(const void* X, qwha_dtype x_dtype, int64_t N, int32_t d_in,
                         double* Hs, int32_t accumulate, hipStream_t stream);
size_t qwha_init_calibrated_workspace_bytes(int32_t d_out, int32_t d_in);
qwha_status qwha_init_select_calibrated(const float* dWq, int32_t d_out, int32_t d_in,
                                        const double* Hs, double damp, int64_t p,
                                        int32_t min_per_row, double temperature,
                                        int32_t* row_ptr, int32_t* E, float* c,
                                        int32_t* col_ptr, int32_t* csc_perm, double* G,
                                        double* rhs, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);
size_t qwha_refine_workspace_bytes(const int32_t* row_ptr_host, int32_t d_out);
qwha_status qwha_refine_values(const int32_t* row_ptr, const int32_t* E, const double* G,
                               const double* rhs, int32_t d_out, int32_t d_in, int64_t p,
                               float* c, int32_t* status, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * The quantized base layer with its adapter: the inference path
 * (papernotes.org, 损失函数 / 训练策略: the adapter is merged into the
 * group-quantized model; gist.science §4 for its inference cost).
 *
 * Base weights W_Q [d_out][d_in] are b-bit codes (b in {2, 3, 4, 8}) with
 * an fp32 scale s and an fp32 integer-valued zero z per group of `group`
 * consecutive input columns (group a power of two dividing d_in):
 *   W_Q[i][j] = (q[i][j] - z[i][j/group]) * s[i][j/group]   (fp32).
 * codes: uint32 [d_out][ceil(d_in / cpw)], cpw = floor(32 / b) codes per
 * word, code j of a row in word j / cpw at bit (j % cpw) * b (least
 * significant first; the last word of a row padded with zero codes).
 * scales, zeros: fp32 [d_out][d_in / group].
 *
 * qwha_merge: W = W_Q + alpha F H^-1 (the adapter merged into dense
 *   weights), written in out_dtype [d_out][d_in]; fp32 math, one rounding
 *   for bf16 output.
 *
 * qwha_layer_fwd: y = x W_Q^T + alpha z F^T, z = FWHT(x)/d_in, for bf16
 *   activations x [T][d_in] (QWHA_ERR_DTYPE otherwise), y bf16 [T][d_out].
 *   The base product runs on the bf16 matrix cores with the weight operand
 *   q - z (exact in bf16 when |q - z| <= 256, always so for a min/max
 *   quantizer whose groups span zero), each group's fp32 partial sums
 *   scaled by s; the adapter's fp32 output is added before the single
 *   rounding to bf16. Requires d_in >= 64, group >= 32, and a workspace of
 *   qwha_layer_fwd_workspace_bytes(T, d_in, d_out, p) bytes.
 * --------------------------------------------------------------------------- */
qwha_status qwha_merge(const uint32_t* codes, const float* scales, const float* zeros,
                       int32_t bits, int32_t group, int32_t d_out, int32_t d_in, int64_t p,
                       const int32_t* row_ptr, const int32_t* E, const float* c, float alpha,
                       qwha_dtype out_dtype, void* W, hipStream_t stream);
size_t qwha_layer_fwd_workspace_bytes(int64_t T, int32_t d_in, int32_t d_out, int64_t p);
qwha_status qwha_layer_fwd(const void* x, qwha_dtype act, int64_t T, int32_t d_in,
                           int32_t d_out, const uint32_t* codes, const float* scales,
                           const float* zeros, int32_t bits, int32_t group, int64_t p,
                           const int32_t* row_ptr, const int32_t* E, const float* c, float alpha,
                           void* y, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Profiling aid: the next launch of kernel `kernel` made by this thread
 * (inside any entry point above) is bracketed by hipEventRecord(start) and
 * hipEventRecord(stop) on that launch's stream; the request is then
 * consumed. Requests for different kernel ids are independent (one pending
 * request per id). kernel = QWHA_KERNEL_NONE cancels every pending request.
 * Thread-local state; the events must outlive the launch they bracket.
 * --------------------------------------------------------------------------- */
typedef enum qwha_kernel {
  QWHA_KERNEL_NONE = 0,
  QWHA_KERNEL_FWD_FWHT = 1,     /* z = FWHT(x)/n inside qwha_fwd */
  QWHA_KERNEL_FWD_SPMM = 2,     /* y = alpha z F^T inside qwha_fwd */
  QWHA_KERNEL_BWD_FWHT_X = 3,   /* z recomputed inside qwha_bwd (not qwha_bwd_saved) */
  QWHA_KERNEL_BWD_SPMM = 4,     /* dz = dy F and the dc partials inside qwha_bwd */
  QWHA_KERNEL_BWD_FWHT_DX = 5,  /* dx = alpha FWHT(dz)/n inside qwha_bwd */
  QWHA_KERNEL_BWD_DC_REDUCE = 6,
  QWHA_KERNEL_INIT_SELECT = 7,  /* fp64 transform + top-k inside qwha_init_select */
  QWHA_KERNEL_MATERIALIZE = 8,
  QWHA_KERNEL_FWHT = 9,         /* qwha_fwht */
  QWHA_KERNEL_GLOBAL_THRESHOLD = 10, /* keys, radix select and budgets in qwha_init_select_global */
  QWHA_KERNEL_HESSIAN = 11,     /* qwha_hessian */
  QWHA_KERNEL_CALIB_PREPARE = 12, /* dW_Q Hs, norms and Q inside qwha_init_select_calibrated */
  QWHA_KERNEL_CALIB_SYSTEM = 13,  /* rhs gather and G inside qwha_init_select_calibrated */
  QWHA_KERNEL_REFINE = 14,      /* the per-row solves of qwha_refine_values */
  QWHA_KERNEL_MERGE = 15,       /* qwha_merge */
  QWHA_KERNEL_QGEMM = 16        /* the base GEMM inside qwha_layer_fwd */
} qwha_kernel;
qwha_status qwha_profile_next(int32_t kernel, hipEvent_t start, hipEvent_t stop);

/* ---------------------------------------------------------------------------
 * Standalone row-wise fast Walsh-Hadamard transform (the +-1 kernel H,
 * papernotes.org 关键设计 1):
 *   out[r][:] = scale * in[r][:] H   for r < rows, n a power of two <= 16384.
 * in / out dtypes independent (QWHA_F32 / QWHA_BF16); math is fp32.
 * --------------------------------------------------------------------------- */
qwha_status qwha_fwht(const void* in, qwha_dtype in_dtype, void* out, qwha_dtype out_dtype,
                      int64_t rows, int32_t n, float scale, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QWHA_H */
