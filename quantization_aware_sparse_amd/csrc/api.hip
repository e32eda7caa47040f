// C-ABI entry points: host-side validation, workspace carving, launches.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/qwha.h"
#include "launch.h"

using namespace qwha;

// Device memory of qwha_fwd_noalloc, for callers that cannot allocate: the
// forward's workspace (z and the prepared stream) lives here instead of in a
// caller buffer. Each GPU the library runs on holds its own copy until the
// process ends. In host code `scratch` is only a stand-in for the symbol;
// its device address comes from hipGetSymbolAddress (scratch_address).
constexpr size_t kScratchBytes = static_cast<size_t>(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local char g_err[512] = {0};

qwha_status fail(qwha_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

qwha_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(QWHA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return QWHA_OK;
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// one-shot profiling requests (qwha_profile_next), one slot per kernel id
struct Hook {
  hipEvent_t start, stop;
};
constexpr int kNumKernelIds = 17;
thread_local Hook g_hook[kNumKernelIds] = {};

// Runs `launch` (a callable returning hipError_t) for kernel id `k`, with the
// pending profiling events recorded around it when requested.
template <typename Fn>
hipError_t timed(int k, hipStream_t s, Fn&& launch) {
  if (g_hook[k].start == nullptr) return launch();
  const Hook h = g_hook[k];
  g_hook[k] = Hook{nullptr, nullptr};
  hipError_t e = hipEventRecord(h.start, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  return hipEventRecord(h.stop, s);
}

int log2_pow2(int32_t n) {
  if (n < 2 || n > 16384 || (n & (n - 1)) != 0) return -1;
  int l = 0;
  while ((1 << l) < n) ++l;
  return l;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// d_in = nblk * 2^log_b with 2^log_b the largest power of two dividing it:
// the transform is one Sylvester matrix (nblk = 1) or nblk Sylvester blocks
// on the diagonal, which needs blocks of at least 64 columns.
qwha_status check_width(int32_t d_out, int32_t d_in, int* log_b, int* nblk) {
  if (d_in < 2 || d_in > 16384)
    return fail(QWHA_ERR_SHAPE, "d_in=%d outside [2, 16384]", d_in);
  const int32_t b = d_in & -d_in;
  *nblk = d_in / b;
  *log_b = log2_pow2(b);
  if (*nblk > 1 && b < 64)
    return fail(QWHA_ERR_SHAPE,
                "d_in=%d: a width that is not a power of two needs a power-of-two factor of at "
                "least 64 (block-diagonal transform)", d_in);
  if (d_out < 1 || d_out > (1 << 20)) return fail(QWHA_ERR_SHAPE, "d_out=%d out of [1, 2^20]", d_out);
  return QWHA_OK;
}


qwha_status check_p(int64_t p, int32_t d_out, int32_t d_in) {
  if (p < 0 || p > INT32_MAX || p > static_cast<int64_t>(d_out) * d_in)
    return fail(QWHA_ERR_BUDGET, "p=%lld outside [0, min(2^31-1, d_out*d_in)]",
                static_cast<long long>(p));
  return QWHA_OK;
}

// The SpMMs' prepared stream addresses its entries with int32 positions;
// padded to whole pairs it holds at most 2p + 16 entries.
constexpr int64_t kMaxStreamP = (static_cast<int64_t>(INT32_MAX) - 64) / 2;
qwha_status check_stream_p(int64_t p) {
  if (p > kMaxStreamP)
    return fail(QWHA_ERR_BUDGET, "p=%lld exceeds %lld, the most the SpMM stream addresses",
                static_cast<long long>(p), static_cast<long long>(kMaxStreamP));
  return QWHA_OK;
}

qwha_status check_quant(int32_t bits, int32_t group, int32_t d_in, int32_t min_group) {
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(QWHA_ERR_INVALID_ARG, "bits=%d is not one of 2, 3, 4, 8", bits);
  if (group < min_group || group > d_in || (group & (group - 1)) != 0)
    return fail(QWHA_ERR_INVALID_ARG, "group=%d is not a power of two in [%d, d_in]", group,
                min_group);
  // every group holds whole columns: a partial last group would have no
  // scale and zero of its own (the kernels index groups as j / group)
  if (d_in % group != 0)
    return fail(QWHA_ERR_INVALID_ARG, "group=%d does not divide d_in=%d", group, d_in);
  return QWHA_OK;
}

qwha_status check_dt(int d, const char* name) {
  if (d != QWHA_F32 && d != QWHA_BF16) return fail(QWHA_ERR_DTYPE, "%s: unknown dtype %d", name, d);
  return QWHA_OK;
}

#define QWHA_TRY(expr)            \
  do {                            \
    qwha_status _s = (expr);      \
    if (_s != QWHA_OK) return _s; \
  } while (0)

#define QWHA_NEED(ptr, align)                                                          \
  do {                                                                                 \
    if ((ptr) == nullptr) return fail(QWHA_ERR_INVALID_ARG, "%s is NULL", #ptr);       \
    if (!aligned((ptr), (align)))                                                      \
      return fail(QWHA_ERR_ALIGN, "%s is not %d-byte aligned", #ptr, (int)(align));    \
  } while (0)

// ---- workspace layouts
struct InitWs {
  size_t w, alloc, csc, total;
};
InitWs init_ws(int32_t d_out, int32_t d_in) {
  InitWs l;
  l.w = 0;
  l.alloc = align256(static_cast<size_t>(d_out) * 8);
  l.csc = l.alloc + align256(adaalloc_scratch_bytes(d_out));
  l.total = l.csc + align256(csc_scratch_bytes(d_out, d_in));
  return l;
}

struct FwdWs {
  size_t z, prep, total;
  SpmmPlan plan;
};
FwdWs fwd_ws(int64_t T, int32_t d_in, int32_t d_out, int64_t p) {
  FwdWs l;
  l.plan = spmm_plan(T, d_in, d_out, p, false);
  l.z = 0;
  l.prep = align256(static_cast<size_t>(T) * d_in * 4);
  l.total = l.prep + align256(spmm_prep_bytes(p, d_out, l.plan));
  return l;
}

struct BwdWs {
  size_t z, dz, prep, partial, total;
  SpmmPlan plan;
};
// with_dc: the dz pass also forms the dc partials (one fp32 per nonzero and
// token tile); without, it is the plain gather over entry pairs.
// stage16: dy is bf16 and the dc pass keeps it as bf16 in LDS (blocks of 128
// columns); its prepared stream is no larger than the fp32 layout's, which
// the size queries use.
BwdWs bwd_ws(int64_t T, int32_t d_in, int32_t d_out, int64_t p, bool with_dc,
             bool stage16 = false) {
  BwdWs l;
  l.plan = spmm_plan(T, d_out, d_in, p, with_dc, with_dc && stage16);
  const size_t zb = align256(static_cast<size_t>(T) * d_in * 4);
  l.z = 0;
  l.dz = zb;
  l.prep = 2 * zb;
  l.partial = l.prep + align256(spmm_prep_bytes(p, d_in, l.plan));
  l.total = l.partial;
  if (with_dc)
    l.total += align256(static_cast<size_t>(l.plan.ntiles) * static_cast<size_t>(p) * 4);
  return l;
}

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// A plan: the forward's stream (rows of F, entry pairs) and the backward's
// (columns of F, single entries with the dc partials), both with korig.
struct PlanLayout {
  size_t fwd, bwd, total;
  SpmmPlan pf, pb;   // ntiles is per call
};
PlanLayout plan_layout(int32_t d_in, int32_t d_out, int64_t p) {
  PlanLayout l;
  l.pf = spmm_plan(0, d_in, d_out, p, false);
  l.pb = spmm_plan(0, d_out, d_in, p, true);
  l.fwd = 0;
  l.bwd = align256(spmm_prep_bytes(p, d_out, l.pf));
  l.total = l.bwd + align256(spmm_prep_bytes(p, d_in, l.pb));
  return l;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

qwha_status scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QWHA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(QWHA_ERR_HIP, "device %d outside the %d the static scratch serves", dev,
                kMaxDevices);
  if (stream != nullptr) {
    int sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess)
      return fail(QWHA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(QWHA_ERR_INVALID_ARG,
                  "the stream belongs to device %d but device %d is current", sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(QWHA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QWHA_OK;
}

}  // namespace

extern "C" {

const char* qwha_status_string(qwha_status s) {
  switch (s) {
    case QWHA_OK: return "ok";
    case QWHA_ERR_INVALID_ARG: return "invalid argument";
    case QWHA_ERR_SHAPE: return "unsupported shape";
    case QWHA_ERR_BUDGET: return "budget out of range";
    case QWHA_ERR_DTYPE: return "unknown dtype";
    case QWHA_ERR_ALIGN: return "misaligned pointer";
    case QWHA_ERR_WORKSPACE: return "workspace too small";
    case QWHA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* qwha_last_error(void) { return g_err; }

int32_t qwha_version(void) { return 100; }

// ------------------------------------------------------------------ init
size_t qwha_init_workspace_bytes(int32_t d_out, int32_t d_in) {
  if (d_out < 1 || d_in < 1) return 0;
  return init_ws(d_out, d_in).total;
}

qwha_status qwha_init_select(const float* dWq, int32_t d_out, int32_t d_in, int64_t p,
                             int32_t min_per_row, double temperature, int32_t* row_ptr,
                             int32_t* E, float* c, int32_t* col_ptr, int32_t* csc_perm,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  int log_n;
  int nblk;
  QWHA_TRY(check_width(d_out, d_in, &log_n, &nblk));
  if (min_per_row < 0 || min_per_row > d_in)
    return fail(QWHA_ERR_INVALID_ARG, "min_per_row=%d outside [0, d_in]", min_per_row);
  if (!(temperature > 0.0) || !isfinite(temperature))
    return fail(QWHA_ERR_INVALID_ARG, "temperature must be finite and > 0");
  QWHA_TRY(check_p(p, d_out, d_in));
  if (p < static_cast<int64_t>(min_per_row) * d_out)
    return fail(QWHA_ERR_BUDGET, "p=%lld < min_per_row*d_out=%lld", static_cast<long long>(p),
                static_cast<long long>(min_per_row) * d_out);
  QWHA_NEED(dWq, 16);
  QWHA_NEED(row_ptr, 4);
  QWHA_NEED(col_ptr, 4);
  if (p > 0) {
    QWHA_NEED(E, 4);
    QWHA_NEED(c, 4);
    QWHA_NEED(csc_perm, 4);
  }
  const InitWs l = init_ws(d_out, d_in);
  if (workspace == nullptr || workspace_bytes < l.total)
    return fail(QWHA_ERR_WORKSPACE, "init workspace needs %zu bytes", l.total);
  QWHA_NEED(workspace, 256);

  double* w = reinterpret_cast<double*>(at(workspace, l.w));
  QWHA_TRY(hip_check(launch_row_norms(dWq, d_out, d_in, w, stream), "row_norms"));
  QWHA_TRY(hip_check(launch_adaalloc(w, d_out, d_in, p, min_per_row, temperature, row_ptr,
                                     at(workspace, l.alloc), stream),
                     "adaalloc"));
  QWHA_TRY(hip_check(timed(QWHA_KERNEL_INIT_SELECT, stream,
                           [&] {
                             return launch_init_select(dWq, d_out, log_n, row_ptr, E, c, 0,
                                                       nullptr, 0, stream, nblk);
                           }),
                     "init_select"));
  QWHA_TRY(hip_check(launch_csc_build(row_ptr, E, d_out, d_in, col_ptr, csc_perm,
                                      at(workspace, l.csc), stream),
                     "csc_build"));
  return QWHA_OK;
}

size_t qwha_init_global_workspace_bytes(int32_t d_out, int32_t d_in, int32_t strategy) {
  if (d_out < 1 || d_in < 1) return 0;
  if (strategy != QWHA_SELECT_MAGNITUDE && strategy != QWHA_SELECT_RANDOM) return 0;
  return align256(global_select_scratch_bytes(d_out, d_in, strategy)) +
         align256(csc_scratch_bytes(d_out, d_in));
}

qwha_status qwha_init_select_global(const float* dWq, int32_t d_out, int32_t d_in, int64_t p,
                                    int32_t strategy, uint64_t seed, int32_t* row_ptr,
                                    int32_t* E, float* c, int32_t* col_ptr, int32_t* csc_perm,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  g_err[0] = 0;
  int log_n;
  int nblk;
  QWHA_TRY(check_width(d_out, d_in, &log_n, &nblk));
  if (strategy != QWHA_SELECT_MAGNITUDE && strategy != QWHA_SELECT_RANDOM)
    return fail(QWHA_ERR_INVALID_ARG, "strategy=%d is neither QWHA_SELECT_MAGNITUDE nor "
                "QWHA_SELECT_RANDOM", strategy);
  QWHA_TRY(check_p(p, d_out, d_in));
  QWHA_NEED(dWq, 16);
  QWHA_NEED(row_ptr, 4);
  QWHA_NEED(col_ptr, 4);
  if (p > 0) {
    QWHA_NEED(E, 4);
    QWHA_NEED(c, 4);
    QWHA_NEED(csc_perm, 4);
  }
  const size_t sel_bytes = align256(global_select_scratch_bytes(d_out, d_in, strategy));
  const size_t total = sel_bytes + align256(csc_scratch_bytes(d_out, d_in));
  if (workspace == nullptr || workspace_bytes < total)
    return fail(QWHA_ERR_WORKSPACE, "global init workspace needs %zu bytes", total);
  QWHA_NEED(workspace, 256);

  const unsigned long long* gtau = nullptr;
  QWHA_TRY(hip_check(timed(QWHA_KERNEL_GLOBAL_THRESHOLD, stream,
                           [&] {
                             return launch_global_budgets(dWq, d_out, log_n, p, strategy, seed,
                                                          row_ptr, workspace, &gtau, stream,
                                                          nblk);
                           }),
                     "global_threshold"));
  QWHA_TRY(hip_check(timed(QWHA_KERNEL_INIT_SELECT, stream,
                           [&] {
                             return launch_init_select(dWq, d_out, log_n, row_ptr, E, c,
                                                       strategy, gtau, seed, stream, nblk);
                           }),
                     "init_select"));
  QWHA_TRY(hip_check(launch_csc_build(row_ptr, E, d_out, d_in, col_ptr, csc_perm,
                                      at(workspace, sel_bytes), stream),
                     "csc_build"));
  return QWHA_OK;
}

// ------------------------------------------------------------------ calibration
qwha_status qwha_hessian(const void* X, qwha_dtype x_dtype, int64_t N, int32_t d_in, double* Hs,
                         int32_t accumulate, hipStream_t stream) {
  g_err[0] = 0;
  {
    int log_b, nblk;
    QWHA_TRY(check_width(1, d_in, &log_b, &nblk));
  }
  if (N < 0 || N > (static_cast<int64_t>(1) << 40))
    return fail(QWHA_ERR_SHAPE, "N=%lld out of [0, 2^40]", static_cast<long long>(N));
  QWHA_TRY(check_dt(x_dtype, "x_dtype"));
  if (accumulate != 0 && accumulate != 1)
    return fail(QWHA_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  QWHA_NEED(Hs, 16);
  if (N > 0) QWHA_NEED(X, 16);
  return hip_check(timed(QWHA_KERNEL_HESSIAN, stream,
                         [&] {
                           return launch_hessian(X, static_cast<Dt>(x_dtype), N, d_in, Hs,
                                                 accumulate, stream);
                         }),
                   "hessian");
}

size_t qwha_init_calibrated_workspace_bytes(int32_t d_out, int32_t d_in) {
  if (d_out < 1 || d_in < 1) return 0;
  return align256(calibrated_scratch_bytes(d_out, d_in)) +
         align256(adaalloc_scratch_bytes(d_out)) + align256(csc_scratch_bytes(d_out, d_in));
}

qwha_status qwha_init_select_calibrated(const float* dWq, int32_t d_out, int32_t d_in,
                                        const double* Hs, double damp, int64_t p,
                                        int32_t min_per_row, double temperature,
                                        int32_t* row_ptr, int32_t* E, float* c,
                                        int32_t* col_ptr, int32_t* csc_perm, double* G,
                                        double* rhs, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  g_err[0] = 0;
  int log_n;
  int nblk;
  QWHA_TRY(check_width(d_out, d_in, &log_n, &nblk));
  if (min_per_row < 0 || min_per_row > d_in)
    return fail(QWHA_ERR_INVALID_ARG, "min_per_row=%d outside [0, d_in]", min_per_row);
  if (!(temperature > 0.0) || !isfinite(temperature))
    return fail(QWHA_ERR_INVALID_ARG, "temperature must be finite and > 0");
  if (!(damp >= 0.0) || !isfinite(damp))
    return fail(QWHA_ERR_INVALID_ARG, "damp must be finite and >= 0");
  QWHA_TRY(check_p(p, d_out, d_in));
  if (p < static_cast<int64_t>(min_per_row) * d_out)
    return fail(QWHA_ERR_BUDGET, "p=%lld < min_per_row*d_out=%lld", static_cast<long long>(p),
                static_cast<long long>(min_per_row) * d_out);
  QWHA_NEED(dWq, 16);
  QWHA_NEED(Hs, 16);
  QWHA_NEED(G, 16);
  QWHA_NEED(row_ptr, 4);
  QWHA_NEED(col_ptr, 4);
  if (p > 0) {
    QWHA_NEED(E, 4);
    QWHA_NEED(c, 4);
    QWHA_NEED(csc_perm, 4);
    QWHA_NEED(rhs, 8);
  }
  const size_t cal = align256(calibrated_scratch_bytes(d_out, d_in));
  const size_t alloc = align256(adaalloc_scratch_bytes(d_out));
  const size_t total = cal + alloc + align256(csc_scratch_bytes(d_out, d_in));
  if (workspace == nullptr || workspace_bytes < total)
    return fail(QWHA_ERR_WORKSPACE, "calibrated init workspace needs %zu bytes", total);
  QWHA_NEED(workspace, 256);

  double* w = nullptr;
  QWHA_TRY(hip_check(timed(QWHA_KERNEL_CALIB_PREPARE, stream,
                           [&] {
                             return launch_calib_prepare(dWq, d_out, log_n, Hs, damp, workspace,
                                                         &w, stream, nblk);
                           }),
                     "calib_prepare"));
  QWHA_TRY(hip_check(launch_adaalloc(w, d_out, d_in, p, min_per_row, temperature, row_ptr,
                                     at(workspace, cal), stream),
                     "adaalloc"));
  QWHA_TRY(hip_check(launch_init_select(dWq, d_out, log_n, row_ptr, E, c, 0, nullptr, 0, stream,
                                        nblk),
                     "init_select"));
  QWHA_TRY(hip_check(launch_csc_build(row_ptr, E, d_out, d_in, col_ptr, csc_perm,
                                      at(workspace, cal + alloc), stream),
                     "csc_build"));
  QWHA_TRY(hip_check(timed(QWHA_KERNEL_CALIB_SYSTEM, stream,
                           [&] {
                             return launch_calib_finish(E, p, d_out, log_n, Hs, workspace, G, rhs,
                                                        stream, nblk);
                           }),
                     "calib_system"));
  return QWHA_OK;
}

size_t qwha_refine_workspace_bytes(const int32_t* row_ptr_host, int32_t d_out) {
  if (row_ptr_host == nullptr || d_out < 1 || row_ptr_host[0] != 0) return 0;
  size_t n = 0;
  for (int32_t i = 0; i < d_out; ++i) {
    const int64_t pi = static_cast<int64_t>(row_ptr_host[i + 1]) - row_ptr_host[i];
    if (pi < 0) return 0;
    n += static_cast<size_t>((pi + 1) * (pi + 2) / 2);
  }
  return refine_header_bytes(d_out) + 8 * n;
}

qwha_status qwha_refine_values(const int32_t* row_ptr, const int32_t* E, const double* G,
                               const double* rhs, int32_t d_out, int32_t d_in, int64_t p,
                               float* c, int32_t* status, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  int log_n;
  int nblk;
  QWHA_TRY(check_width(d_out, d_in, &log_n, &nblk));
  QWHA_TRY(check_p(p, d_out, d_in));
  QWHA_NEED(row_ptr, 4);
  QWHA_NEED(G, 8);
  QWHA_NEED(status, 4);
  if (p > 0) {
    QWHA_NEED(E, 4);
    QWHA_NEED(rhs, 8);
    QWHA_NEED(c, 4);
  }
  const size_t hb = refine_header_bytes(d_out);
  if (workspace == nullptr || workspace_bytes < hb)
    return fail(QWHA_ERR_WORKSPACE, "refine workspace needs at least %zu bytes", hb);
  QWHA_NEED(workspace, 256);
  return hip_check(timed(QWHA_KERNEL_REFINE, stream,
                         [&] {
                           return launch_refine(row_ptr, E, G, d_in, rhs, d_out, c, status,
                                                workspace, workspace_bytes, 1e-10, stream);
                         }),
                   "refine");
}

// ------------------------------------------------------------------ quantized base
qwha_status qwha_merge(const uint32_t* codes, const float* scales, const float* zeros,
                       int32_t bits, int32_t group, int32_t d_out, int32_t d_in, int64_t p,
                       const int32_t* row_ptr, const int32_t* E, const float* c, float alpha,
                       qwha_dtype out_dtype, void* W, hipStream_t stream) {
  g_err[0] = 0;
  int log_n;
  int nblk;
  QWHA_TRY(check_width(d_out, d_in, &log_n, &nblk));
  QWHA_TRY(check_p(p, d_out, d_in));
  QWHA_TRY(check_quant(bits, group, d_in, 1));
  QWHA_TRY(check_dt(out_dtype, "out_dtype"));
  if (!isfinite(alpha)) return fail(QWHA_ERR_INVALID_ARG, "alpha must be finite");
  QWHA_NEED(codes, 4);
  QWHA_NEED(scales, 4);
  QWHA_NEED(zeros, 4);
  QWHA_NEED(row_ptr, 4);
  QWHA_NEED(W, 16);
  if (p > 0) {
    QWHA_NEED(E, 4);
    QWHA_NEED(c, 4);
  }
  const QuantW qw = make_quant(codes, scales, zeros, bits, group, d_in);
  return hip_check(timed(QWHA_KERNEL_MERGE, stream,
                         [&] {
                           return launch_merge(row_ptr, E, c, d_out, log_n, alpha, qw,
                                               static_cast<Dt>(out_dtype), W, stream, nblk);
                         }),
                   "merge");
}

size_t qwha_layer_fwd_workspace_bytes(int64_t T, int32_t d_in, int32_t d_out, int64_t p) {
  if (T < 0 || d_in < 1 || d_out < 1 || p < 0 || p > kMaxStreamP) return 0;
  return fwd_ws(T, d_in, d_out, p).total + align256(static_cast<size_t>(T) * d_out * 4);
}

qwha_status qwha_layer_fwd(const void* x, qwha_dtype act, int64_t T, int32_t d_in,
                           int32_t d_out, const uint32_t* codes, const float* scales,
                           const float* zeros, int32_t bits, int32_t group, int64_t p,
                           const int32_t* row_ptr, const int32_t* E, const float* c, float alpha,
                           void* y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  int log_n;
  int nblk;
  QWHA_TRY(check_width(d_out, d_in, &log_n, &nblk));
  if (d_in < 64) return fail(QWHA_ERR_SHAPE, "d_in=%d below 64", d_in);
  QWHA_TRY(check_p(p, d_out, d_in));
  QWHA_TRY(check_stream_p(p));
  QWHA_TRY(check_dt(act, "act"));
  if (act != QWHA_BF16)
    return fail(QWHA_ERR_DTYPE, "the base GEMM runs on bf16 activations");
  QWHA_TRY(check_quant(bits, group, d_in, 32));
  if (T < 0 || T > (static_cast<int64_t>(1) << 31)) return fail(QWHA_ERR_SHAPE, "T out of range");
  if (!isfinite(alpha)) return fail(QWHA_ERR_INVALID_ARG, "alpha must be finite");
  QWHA_NEED(codes, 4);
  QWHA_NEED(scales, 4);
  QWHA_NEED(zeros, 4);
  QWHA_NEED(row_ptr, 4);
  if (p > 0) {
    QWHA_NEED(E, 4);
    QWHA_NEED(c, 4);
  }
  if (T == 0) return QWHA_OK;
  QWHA_NEED(x, 16);
  QWHA_NEED(y, 16);
  const FwdWs l = fwd_ws(T, d_in, d_out, p);
  const size_t total = l.total + align256(static_cast<size_t>(T) * d_out * 4);
  if (workspace == nullptr || workspace_bytes < total)
    return fail(QWHA_ERR_WORKSPACE, "layer fwd workspace needs %zu bytes", total);
  QWHA_NEED(workspace, 256);

  float* y32 = nullptr;
  if (p > 0) {
    float* z = reinterpret_cast<float*>(at(workspace, l.z));
    void* prep = at(workspace, l.prep);
    y32 = reinterpret_cast<float*>(at(workspace, l.total));
    QWHA_TRY(hip_check(launch_fwht(x, Dt::BF16, z, Dt::F32, T * nblk, log_n,
                                   1.0f / static_cast<float>(1 << log_n), 0, stream),
                       "layer fwht"));
    QWHA_TRY(hip_check(launch_prep_csr(row_ptr, E, c, d_out, p, l.plan, prep, stream),
                       "layer prep"));
    QWHA_TRY(hip_check(launch_spmm(z, Dt::F32, T, d_in, prep, p, d_out, l.plan, alpha, y32,
                                   Dt::F32, 0, nullptr, nullptr, stream),
                       "layer spmm"));
  }
  const QuantW qw = make_quant(codes, scales, zeros, bits, group, d_in);
  return hip_check(timed(QWHA_KERNEL_QGEMM, stream,
                         [&] {
                           return launch_qgemm(static_cast<const uint16_t*>(x), T, d_in, d_out,
                                               qw, y32, static_cast<uint16_t*>(y), stream);
                         }),
                   "base gemm");
}

// ------------------------------------------------------------------ materialize
qwha_status qwha_materialize(const int32_t* row_ptr, const int32_t* E, const float* c,
                             int32_t d_out, int32_t d_in, int64_t p, float alpha,
                             qwha_dtype out_dtype, void* dW, int32_t accumulate,
                             hipStream_t stream) {
  g_err[0] = 0;
  int log_n;
  int nblk;
  QWHA_TRY(check_width(d_out, d_in, &log_n, &nblk));
  QWHA_TRY(check_p(p, d_out, d_in));
  QWHA_TRY(check_dt(out_dtype, "out_dtype"));
  if (!isfinite(alpha)) return fail(QWHA_ERR_INVALID_ARG, "alpha must be finite");
  if (accumulate != 0 && accumulate != 1) return fail(QWHA_ERR_INVALID_ARG, "accumulate must be 0/1");
  QWHA_NEED(row_ptr, 4);
  if (p > 0) {
    QWHA_NEED(E, 4);
    QWHA_NEED(c, 4);
  }
  QWHA_NEED(dW, 16);
  return hip_check(timed(QWHA_KERNEL_MATERIALIZE, stream,
                         [&] {
                           return launch_materialize(row_ptr, E, c, d_out, log_n, alpha,
                                                     static_cast<Dt>(out_dtype), dW, accumulate,
                                                     stream, nblk);
                         }),
                   "materialize");
}

// ------------------------------------------------------------------ forward
size_t qwha_fwd_workspace_bytes(int64_t T, int32_t d_in, int32_t d_out, int64_t p) {
  if (T < 0 || d_in < 1 || d_out < 1 || p < 0 || p > kMaxStreamP) return 0;
  return fwd_ws(T, d_in, d_out, p).total;
}

}  // extern "C"

namespace {

// qwha_fwd; with z_out, z = FWHT(x)/n goes there (kept for the backward)
// instead of into the workspace. With use_scratch, the workspace is the
// static `scratch` array (workspace and workspace_bytes are ignored).
// With z_in (a transform kept by an earlier forward), x is not read and no
// transform runs.
qwha_status fwd_impl(const void* x, qwha_dtype act, int64_t T, int32_t d_in, int32_t d_out,
                     int64_t p, const int32_t* row_ptr, const int32_t* E, const float* c,
                     float alpha, void* y, int32_t accumulate, float* z_out, void* workspace,
                     size_t workspace_bytes, hipStream_t stream, bool use_scratch = false,
                     const float* z_in = nullptr) {
  g_err[0] = 0;
  int log_n;
  int nblk;
  QWHA_TRY(check_width(d_out, d_in, &log_n, &nblk));
  QWHA_TRY(check_p(p, d_out, d_in));
  QWHA_TRY(check_stream_p(p));
  QWHA_TRY(check_dt(act, "act"));
  if (T < 0 || T > (static_cast<int64_t>(1) << 31)) return fail(QWHA_ERR_SHAPE, "T out of range");
  if (!isfinite(alpha)) return fail(QWHA_ERR_INVALID_ARG, "alpha must be finite");
  if (accumulate != 0 && accumulate != 1) return fail(QWHA_ERR_INVALID_ARG, "accumulate must be 0/1");
  QWHA_NEED(row_ptr, 4);
  if (p > 0) {
    QWHA_NEED(E, 4);
    QWHA_NEED(c, 4);
  }
  if (T == 0) return QWHA_OK;
  if (z_in != nullptr)
    QWHA_NEED(z_in, 16);
  else
    QWHA_NEED(x, 16);
  QWHA_NEED(y, 16);
  FwdWs l = fwd_ws(T, d_in, d_out, p);
  if (z_in != nullptr) {   // no transform: the workspace holds the prepared stream only
    l.total -= l.prep;
    l.prep = 0;
  }
  if (use_scratch) {
    if (l.total > kScratchBytes)
      return fail(QWHA_ERR_WORKSPACE,
                  "this forward needs %zu bytes of workspace; the static scratch of "
                  "qwha_fwd_noalloc holds %zu (use qwha_fwd with a caller workspace)",
                  l.total, kScratchBytes);
    QWHA_TRY(scratch_address(stream, &workspace));
    workspace_bytes = kScratchBytes;
  }
  if (workspace == nullptr || workspace_bytes < l.total)
    return fail(QWHA_ERR_WORKSPACE, "fwd workspace needs %zu bytes", l.total);
  QWHA_NEED(workspace, 256);

  if (z_out != nullptr) QWHA_NEED(z_out, 16);
  const float* z = z_in;
  void* prep = at(workspace, l.prep);
  const Dt adt = static_cast<Dt>(act);
  if (z_in == nullptr) {
    float* zw = z_out ? z_out : reinterpret_cast<float*>(at(workspace, l.z));
    z = zw;
    QWHA_TRY(hip_check(timed(QWHA_KERNEL_FWD_FWHT, stream,
                             [&] {
                               return launch_fwht(x, adt, zw, Dt::F32, T * nblk, log_n,
                                                  1.0f / static_cast<float>(1 << log_n), 0,
                                                  stream);
                             }),
                       "fwd fwht"));
  }
  QWHA_TRY(hip_check(launch_prep_csr(row_ptr, E, c, d_out, p, l.plan, prep, stream), "fwd prep"));
  QWHA_TRY(hip_check(timed(QWHA_KERNEL_FWD_SPMM, stream,
                           [&] {
                             return launch_spmm(z, Dt::F32, T, d_in, prep, p, d_out, l.plan, alpha,
                                                y, adt, accumulate, nullptr, nullptr, stream);
                           }),
                     "fwd spmm"));
  return QWHA_OK;
}

}  // namespace

extern "C" {

qwha_status qwha_fwd(const void* x, qwha_dtype act, int64_t T, int32_t d_in, int32_t d_out,
                     int64_t p, const int32_t* row_ptr, const int32_t* E, const float* c,
                     float alpha, void* y, int32_t accumulate, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  return fwd_impl(x, act, T, d_in, d_out, p, row_ptr, E, c, alpha, y, accumulate, nullptr,
                  workspace, workspace_bytes, stream);
}

qwha_status qwha_fwd_noalloc(const void* x, qwha_dtype act, int64_t T, int32_t d_in,
                             int32_t d_out, int64_t p, const int32_t* row_ptr, const int32_t* E,
                             const float* c, float alpha, void* y, int32_t accumulate,
                             hipStream_t stream) {
  return fwd_impl(x, act, T, d_in, d_out, p, row_ptr, E, c, alpha, y, accumulate, nullptr,
                  nullptr, 0, stream, true);
}

qwha_status qwha_fwd_z(const float* z, qwha_dtype act, int64_t T, int32_t d_in, int32_t d_out,
                       int64_t p, const int32_t* row_ptr, const int32_t* E, const float* c,
                       float alpha, void* y, int32_t accumulate, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (z == nullptr && T > 0) return fail(QWHA_ERR_INVALID_ARG, "z is NULL");
  return fwd_impl(nullptr, act, T, d_in, d_out, p, row_ptr, E, c, alpha, y, accumulate, nullptr,
                  workspace, workspace_bytes, stream, false, z);
}

qwha_status qwha_fwd_save(const void* x, qwha_dtype act, int64_t T, int32_t d_in,
                          int32_t d_out, int64_t p, const int32_t* row_ptr, const int32_t* E,
                          const float* c, float alpha, void* y, int32_t accumulate, float* z,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (z == nullptr && T > 0) return fail(QWHA_ERR_INVALID_ARG, "z is NULL");
  return fwd_impl(x, act, T, d_in, d_out, p, row_ptr, E, c, alpha, y, accumulate, z, workspace,
                  workspace_bytes, stream);
}

// ------------------------------------------------------------------ backward
size_t qwha_bwd_workspace_bytes(int64_t T, int32_t d_in, int32_t d_out, int64_t p) {
  if (T < 0 || d_in < 1 || d_out < 1 || p < 0 || p > kMaxStreamP) return 0;
  const size_t a = bwd_ws(T, d_in, d_out, p, true).total;
  const size_t b = bwd_ws(T, d_in, d_out, p, false).total;
  return a > b ? a : b;
}

}  // extern "C"

namespace {

// qwha_bwd; with z_in (the forward's z = FWHT(x)/n), x is not read and z is
// not recomputed.
qwha_status bwd_impl(const void* x, const float* z_in, const void* dy, qwha_dtype act,
                     int64_t T, int32_t d_in, int32_t d_out, int64_t p, const int32_t* row_ptr,
                     const int32_t* E, const float* c, const int32_t* col_ptr,
                     const int32_t* csc_perm, float alpha, void* dx, int32_t accumulate_dx,
                     float* dc, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  int log_n;
  int nblk;
  QWHA_TRY(check_width(d_out, d_in, &log_n, &nblk));
  QWHA_TRY(check_p(p, d_out, d_in));
  QWHA_TRY(check_stream_p(p));
  QWHA_TRY(check_dt(act, "act"));
  if (T < 0 || T > (static_cast<int64_t>(1) << 31)) return fail(QWHA_ERR_SHAPE, "T out of range");
  if (!isfinite(alpha)) return fail(QWHA_ERR_INVALID_ARG, "alpha must be finite");
  if (accumulate_dx != 0 && accumulate_dx != 1)
    return fail(QWHA_ERR_INVALID_ARG, "accumulate_dx must be 0/1");
  (void)row_ptr;
  if (p > 0) {
    QWHA_NEED(E, 4);
    QWHA_NEED(c, 4);
    QWHA_NEED(csc_perm, 4);
  }
  QWHA_NEED(col_ptr, 4);
  if (dx == nullptr && dc == nullptr) return QWHA_OK;
  if (dc != nullptr && !aligned(dc, 4)) return fail(QWHA_ERR_ALIGN, "dc is not 4-byte aligned");
  if (dx != nullptr && !aligned(dx, 16)) return fail(QWHA_ERR_ALIGN, "dx is not 16-byte aligned");
  if (T == 0) {
    // no tokens: dc is all zeros (a reduction over zero partials; no memset,
    // so the call stays safe under stream capture)
    if (dc != nullptr && p > 0)
      return hip_check(launch_dc_reduce(nullptr, 0, p, csc_perm, alpha, dc, stream), "dc zero");
    return QWHA_OK;
  }
  QWHA_NEED(dy, 16);
  if (dc != nullptr) {
    if (z_in != nullptr)
      QWHA_NEED(z_in, 16);
    else
      QWHA_NEED(x, 16);
  }
  const BwdWs l = bwd_ws(T, d_in, d_out, p, dc != nullptr, act == QWHA_BF16);
  if (workspace == nullptr || workspace_bytes < l.total)
    return fail(QWHA_ERR_WORKSPACE, "bwd workspace needs %zu bytes", l.total);
  QWHA_NEED(workspace, 256);

  const float* z = z_in ? z_in : reinterpret_cast<float*>(at(workspace, l.z));
  float* dz = reinterpret_cast<float*>(at(workspace, l.dz));
  void* prep = at(workspace, l.prep);
  float* partial = dc ? reinterpret_cast<float*>(at(workspace, l.partial)) : nullptr;
  const Dt adt = static_cast<Dt>(act);
  if (dc && z_in == nullptr)
    QWHA_TRY(hip_check(timed(QWHA_KERNEL_BWD_FWHT_X, stream,
                             [&] {
                               return launch_fwht(x, adt, at(workspace, l.z), Dt::F32,
                                                  T * nblk, log_n,
                                                  1.0f / static_cast<float>(1 << log_n), 0,
                                                  stream);
                             }),
                       "bwd fwht(x)"));
  QWHA_TRY(hip_check(launch_prep_csc(col_ptr, csc_perm, E, c, d_in, p, l.plan, prep, stream),
                     "bwd prep"));
  QWHA_TRY(hip_check(timed(QWHA_KERNEL_BWD_SPMM, stream,
                           [&] {
                             return launch_spmm(dy, adt, T, d_out, prep, p, d_in, l.plan, 1.0f, dz,
                                                Dt::F32, 0, dc ? z : nullptr, partial, stream);
                           }),
                     "bwd spmm"));
  if (dx)
    QWHA_TRY(hip_check(timed(QWHA_KERNEL_BWD_FWHT_DX, stream,
                             [&] {
                               return launch_fwht(dz, Dt::F32, dx, adt, T * nblk, log_n,
                                                  alpha / static_cast<float>(1 << log_n),
                                                  accumulate_dx,
                                                  stream);
                             }),
                       "bwd fwht(dz)"));
  if (dc)
    QWHA_TRY(hip_check(timed(QWHA_KERNEL_BWD_DC_REDUCE, stream,
                             [&] {
                               return launch_dc_reduce(partial, l.plan.ntiles, p,
                                                       spmm_prep_korig(prep, p, d_in, l.plan),
                                                       alpha, dc, stream);
                             }),
                       "dc reduce"));
  return QWHA_OK;
}

}  // namespace

extern "C" {

qwha_status qwha_bwd(const void* x, const void* dy, qwha_dtype act, int64_t T, int32_t d_in,
                     int32_t d_out, int64_t p, const int32_t* row_ptr, const int32_t* E,
                     const float* c, const int32_t* col_ptr, const int32_t* csc_perm,
                     float alpha, void* dx, int32_t accumulate_dx, float* dc, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(x, nullptr, dy, act, T, d_in, d_out, p, row_ptr, E, c, col_ptr, csc_perm,
                  alpha, dx, accumulate_dx, dc, workspace, workspace_bytes, stream);
}

qwha_status qwha_bwd_saved(const float* z, const void* dy, qwha_dtype act, int64_t T,
                           int32_t d_in, int32_t d_out, int64_t p, const int32_t* row_ptr,
                           const int32_t* E, const float* c, const int32_t* col_ptr,
                           const int32_t* csc_perm, float alpha, void* dx,
                           int32_t accumulate_dx, float* dc, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (z == nullptr && T > 0 && dc != nullptr) return fail(QWHA_ERR_INVALID_ARG, "z is NULL");
  return bwd_impl(nullptr, z, dy, act, T, d_in, d_out, p, row_ptr, E, c, col_ptr, csc_perm,
                  alpha, dx, accumulate_dx, dc, workspace, workspace_bytes, stream);
}

qwha_status qwha_bwd_dz(const float* z, const void* dy, qwha_dtype act, int64_t T,
                        int32_t d_in, int32_t d_out, int64_t p, const int32_t* E, const float* c,
                        const int32_t* col_ptr, const int32_t* csc_perm, float alpha, float* dz,
                        int32_t accumulate_dz, float* dc, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  int log_n;
  int nblk;
  QWHA_TRY(check_width(d_out, d_in, &log_n, &nblk));
  QWHA_TRY(check_p(p, d_out, d_in));
  QWHA_TRY(check_stream_p(p));
  QWHA_TRY(check_dt(act, "act"));
  if (T < 0 || T > (static_cast<int64_t>(1) << 31)) return fail(QWHA_ERR_SHAPE, "T out of range");
  if (!isfinite(alpha)) return fail(QWHA_ERR_INVALID_ARG, "alpha must be finite");
  if (accumulate_dz != 0 && accumulate_dz != 1)
    return fail(QWHA_ERR_INVALID_ARG, "accumulate_dz must be 0/1");
  if (p > 0) {
    QWHA_NEED(E, 4);
    QWHA_NEED(c, 4);
    QWHA_NEED(csc_perm, 4);
  }
  QWHA_NEED(col_ptr, 4);
  if (dz == nullptr) return fail(QWHA_ERR_INVALID_ARG, "dz is NULL");
  if (dc != nullptr && !aligned(dc, 4)) return fail(QWHA_ERR_ALIGN, "dc is not 4-byte aligned");
  if (T == 0) {
    if (dc != nullptr && p > 0)
      return hip_check(launch_dc_reduce(nullptr, 0, p, csc_perm, alpha, dc, stream), "dc zero");
    return QWHA_OK;
  }
  QWHA_NEED(dz, 16);
  QWHA_NEED(dy, 16);
  if (dc != nullptr) QWHA_NEED(z, 16);
  // z and dz belong to the caller: the workspace holds the prepared stream
  // and the dc partials only
  BwdWs l = bwd_ws(T, d_in, d_out, p, dc != nullptr, act == QWHA_BF16);
  l.total -= l.prep;
  l.partial -= l.prep;
  l.prep = 0;
  if (workspace == nullptr || workspace_bytes < l.total)
    return fail(QWHA_ERR_WORKSPACE, "bwd workspace needs %zu bytes", l.total);
  QWHA_NEED(workspace, 256);

  void* prep = at(workspace, l.prep);
  float* partial = dc ? reinterpret_cast<float*>(at(workspace, l.partial)) : nullptr;
  const Dt adt = static_cast<Dt>(act);
  QWHA_TRY(hip_check(launch_prep_csc(col_ptr, csc_perm, E, c, d_in, p, l.plan, prep, stream),
                     "bwd prep"));
  QWHA_TRY(hip_check(timed(QWHA_KERNEL_BWD_SPMM, stream,
                           [&] {
                             return launch_spmm(dy, adt, T, d_out, prep, p, d_in, l.plan, alpha,
                                                dz, Dt::F32, accumulate_dz, dc ? z : nullptr,
                                                partial, stream);
                           }),
                     "bwd spmm"));
  if (dc)
    QWHA_TRY(hip_check(timed(QWHA_KERNEL_BWD_DC_REDUCE, stream,
                             [&] {
                               return launch_dc_reduce(partial, l.plan.ntiles, p,
                                                       spmm_prep_korig(prep, p, d_in, l.plan),
                                                       alpha, dc, stream);
                             }),
                       "dc reduce"));
  return QWHA_OK;
}

// ------------------------------------------------------------------ plans
size_t qwha_plan_bytes(int32_t d_in, int32_t d_out, int64_t p) {
  if (d_in < 1 || d_out < 1 || p < 0 || p > kMaxStreamP) return 0;
  return plan_layout(d_in, d_out, p).total;
}

qwha_status qwha_plan_build(const int32_t* row_ptr, const int32_t* E, const int32_t* col_ptr,
                            const int32_t* csc_perm, int32_t d_in, int32_t d_out, int64_t p,
                            qwha_dtype act, void* plan, size_t plan_bytes, hipStream_t stream) {
  g_err[0] = 0;
  int log_n;
  int nblk;
  QWHA_TRY(check_width(d_out, d_in, &log_n, &nblk));
  QWHA_TRY(check_p(p, d_out, d_in));
  QWHA_TRY(check_stream_p(p));
  QWHA_TRY(check_dt(act, "act"));
  QWHA_NEED(row_ptr, 4);
  QWHA_NEED(col_ptr, 4);
  if (p > 0) {
    QWHA_NEED(E, 4);
    QWHA_NEED(csc_perm, 4);
  }
  const PlanLayout l = plan_layout(d_in, d_out, p);
  if (plan == nullptr || plan_bytes < l.total)
    return fail(QWHA_ERR_WORKSPACE, "the plan needs %zu bytes", l.total);
  QWHA_NEED(plan, 256);
  QWHA_TRY(hip_check(launch_prep_structure(row_ptr, E, nullptr, d_out, p, l.pf,
                                           at(plan, l.fwd), stream),
                     "plan (rows of F)"));
  // the backward's layout follows the activations' type (bf16 dy staged as bf16)
  const SpmmPlan pb = spmm_plan(0, d_out, d_in, p, true, act == QWHA_BF16);
  return hip_check(launch_prep_structure(col_ptr, E, csc_perm, d_in, p, pb, at(plan, l.bwd),
                                         stream),
                   "plan (columns of F)");
}

qwha_status qwha_fwd_plan(const void* x, const float* z_in, qwha_dtype act, int64_t T,
                          int32_t d_in, int32_t d_out, int64_t p, void* plan, const float* c,
                          float alpha, void* y, int32_t accumulate, float* z_out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  int log_n;
  int nblk;
  QWHA_TRY(check_width(d_out, d_in, &log_n, &nblk));
  QWHA_TRY(check_p(p, d_out, d_in));
  QWHA_TRY(check_stream_p(p));
  QWHA_TRY(check_dt(act, "act"));
  if (T < 0 || T > (static_cast<int64_t>(1) << 31)) return fail(QWHA_ERR_SHAPE, "T out of range");
  if (!isfinite(alpha)) return fail(QWHA_ERR_INVALID_ARG, "alpha must be finite");
  if (accumulate != 0 && accumulate != 1) return fail(QWHA_ERR_INVALID_ARG, "accumulate must be 0/1");
  if (z_in != nullptr && z_out != nullptr)
    return fail(QWHA_ERR_INVALID_ARG, "z_in and z_out are exclusive");
  QWHA_NEED(plan, 256);
  if (p > 0) QWHA_NEED(c, 4);
  if (T == 0) return QWHA_OK;
  if (z_in != nullptr)
    QWHA_NEED(z_in, 16);
  else
    QWHA_NEED(x, 16);
  if (z_out != nullptr) QWHA_NEED(z_out, 16);
  QWHA_NEED(y, 16);
  const bool own_z = z_in == nullptr && z_out == nullptr;
  const size_t need = own_z ? align256(static_cast<size_t>(T) * d_in * 4) : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(QWHA_ERR_WORKSPACE, "fwd workspace needs %zu bytes", need);
  if (need > 0) QWHA_NEED(workspace, 256);

  PlanLayout l = plan_layout(d_in, d_out, p);
  l.pf = spmm_plan(T, d_in, d_out, p, false);
  void* prep = at(plan, l.fwd);
  const Dt adt = static_cast<Dt>(act);
  QWHA_TRY(hip_check(launch_prep_refresh(c, p, d_out, l.pf, prep, stream), "fwd values"));
  const float* z = z_in;
  if (z_in == nullptr) {
    float* zw = z_out ? z_out : reinterpret_cast<float*>(workspace);
    z = zw;
    QWHA_TRY(hip_check(timed(QWHA_KERNEL_FWD_FWHT, stream,
                             [&] {
                               return launch_fwht(x, adt, zw, Dt::F32, T * nblk, log_n,
                                                  1.0f / static_cast<float>(1 << log_n), 0,
                                                  stream);
                             }),
                       "fwd fwht"));
  }
  return hip_check(timed(QWHA_KERNEL_FWD_SPMM, stream,
                         [&] {
                           return launch_spmm(z, Dt::F32, T, d_in, prep, p, d_out, l.pf, alpha,
                                              y, adt, accumulate, nullptr, nullptr, stream);
                         }),
                   "fwd spmm");
}

qwha_status qwha_bwd_plan(const float* z, const void* dy, qwha_dtype act, int64_t T,
                          int32_t d_in, int32_t d_out, int64_t p, void* plan, const float* c,
                          float alpha, void* dx, int32_t accumulate_dx, float* dz,
                          int32_t accumulate_dz, float* dc, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  int log_n;
  int nblk;
  QWHA_TRY(check_width(d_out, d_in, &log_n, &nblk));
  QWHA_TRY(check_p(p, d_out, d_in));
  QWHA_TRY(check_stream_p(p));
  QWHA_TRY(check_dt(act, "act"));
  if (T < 0 || T > (static_cast<int64_t>(1) << 31)) return fail(QWHA_ERR_SHAPE, "T out of range");
  if (!isfinite(alpha)) return fail(QWHA_ERR_INVALID_ARG, "alpha must be finite");
  if (accumulate_dx != 0 && accumulate_dx != 1)
    return fail(QWHA_ERR_INVALID_ARG, "accumulate_dx must be 0/1");
  if (accumulate_dz != 0 && accumulate_dz != 1)
    return fail(QWHA_ERR_INVALID_ARG, "accumulate_dz must be 0/1");
  if (dz != nullptr && dx != nullptr)
    return fail(QWHA_ERR_INVALID_ARG, "dx and dz are exclusive (dz skips the transform)");
  if (dc == nullptr)
    return fail(QWHA_ERR_INVALID_ARG, "dc is NULL (the plan's backward forms dc)");
  if (!aligned(dc, 4)) return fail(QWHA_ERR_ALIGN, "dc is not 4-byte aligned");
  QWHA_NEED(plan, 256);
  if (p > 0) QWHA_NEED(c, 4);
  const PlanLayout l0 = plan_layout(d_in, d_out, p);
  const void* prep_b = at(plan, l0.bwd);
  const bool b16 = act == QWHA_BF16;
  if (T == 0) {
    if (p > 0)
      return hip_check(launch_dc_reduce(nullptr, 0, p,
                                        spmm_prep_korig(prep_b, p, d_in,
                                                        spmm_plan(0, d_out, d_in, p, true, b16)),
                                        alpha, dc, stream),
                       "dc zero");
    return QWHA_OK;
  }
  QWHA_NEED(z, 16);
  QWHA_NEED(dy, 16);
  if (dx != nullptr) QWHA_NEED(dx, 16);
  if (dz != nullptr) QWHA_NEED(dz, 16);
  const SpmmPlan pb = spmm_plan(T, d_out, d_in, p, true, b16);
  const size_t zb = dz ? 0 : align256(static_cast<size_t>(T) * d_in * 4);
  const size_t total = zb + align256(static_cast<size_t>(pb.ntiles) * static_cast<size_t>(p) * 4);
  if (workspace == nullptr || workspace_bytes < total)
    return fail(QWHA_ERR_WORKSPACE, "bwd workspace needs %zu bytes", total);
  QWHA_NEED(workspace, 256);

  void* prep = at(plan, l0.bwd);
  float* dzw = dz ? dz : reinterpret_cast<float*>(workspace);
  float* partial = reinterpret_cast<float*>(at(workspace, zb));
  const Dt adt = static_cast<Dt>(act);
  // with a caller dz the SpMM applies alpha; otherwise the transform does
  const float a_spmm = dz ? alpha : 1.0f;
  QWHA_TRY(hip_check(launch_prep_refresh(c, p, d_in, pb, prep, stream), "bwd values"));
  QWHA_TRY(hip_check(timed(QWHA_KERNEL_BWD_SPMM, stream,
                           [&] {
                             return launch_spmm(dy, adt, T, d_out, prep, p, d_in, pb, a_spmm,
                                                dzw, Dt::F32, dz ? accumulate_dz : 0, z,
                                                partial, stream);
                           }),
                     "bwd spmm"));
  if (dx != nullptr)
    QWHA_TRY(hip_check(timed(QWHA_KERNEL_BWD_FWHT_DX, stream,
                             [&] {
                               return launch_fwht(dzw, Dt::F32, dx, adt, T * nblk, log_n,
                                                  alpha / static_cast<float>(1 << log_n),
                                                  accumulate_dx, stream);
                             }),
                       "bwd fwht(dz)"));
  return hip_check(timed(QWHA_KERNEL_BWD_DC_REDUCE, stream,
                         [&] {
                           return launch_dc_reduce(partial, pb.ntiles, p,
                                                   spmm_prep_korig(prep, p, d_in, pb), alpha, dc,
                                                   stream);
                         }),
                   "dc reduce");
}

// ------------------------------------------------------------------ update
qwha_status qwha_sign_update(float* c, const float* dc, int64_t p, float step,
                             hipStream_t stream) {
  g_err[0] = 0;
  if (p < 0 || p > INT32_MAX) return fail(QWHA_ERR_BUDGET, "p out of range");
  if (!isfinite(step)) return fail(QWHA_ERR_INVALID_ARG, "step must be finite");
  if (p == 0) return QWHA_OK;
  QWHA_NEED(c, 4);
  QWHA_NEED(dc, 4);
  return hip_check(launch_sign_update(c, dc, p, step, stream), "sign_update");
}

// ------------------------------------------------------------------ fwht
qwha_status qwha_fwht(const void* in, qwha_dtype in_dtype, void* out, qwha_dtype out_dtype,
                      int64_t rows, int32_t n, float scale, hipStream_t stream) {
  g_err[0] = 0;
  const int log_n = log2_pow2(n);
  if (log_n < 0) return fail(QWHA_ERR_SHAPE, "n=%d is not a power of two in [2, 16384]", n);
  QWHA_TRY(check_dt(in_dtype, "in_dtype"));
  QWHA_TRY(check_dt(out_dtype, "out_dtype"));
  if (rows < 0 || rows > (static_cast<int64_t>(1) << 31))
    return fail(QWHA_ERR_SHAPE, "rows out of range");
  if (!isfinite(scale)) return fail(QWHA_ERR_INVALID_ARG, "scale must be finite");
  if (rows == 0) return QWHA_OK;
  QWHA_NEED(in, 16);
  QWHA_NEED(out, 16);
  return hip_check(timed(QWHA_KERNEL_FWHT, stream,
                         [&] {
                           return launch_fwht(in, static_cast<Dt>(in_dtype), out,
                                              static_cast<Dt>(out_dtype), rows, log_n, scale, 0,
                                              stream);
                         }),
                   "fwht");
}

qwha_status qwha_profile_next(int32_t kernel, hipEvent_t start, hipEvent_t stop) {
  g_err[0] = 0;
  if (kernel < QWHA_KERNEL_NONE || kernel > QWHA_KERNEL_QGEMM ||
      kernel >= kNumKernelIds)
    return fail(QWHA_ERR_INVALID_ARG, "unknown kernel id %d", kernel);
  if (kernel == QWHA_KERNEL_NONE) {
    for (int i = 0; i < kNumKernelIds; ++i) g_hook[i] = Hook{nullptr, nullptr};
    return QWHA_OK;
  }
  if (start == nullptr || stop == nullptr)
    return fail(QWHA_ERR_INVALID_ARG, "start/stop events are NULL");
  g_hook[kernel] = Hook{start, stop};
  return QWHA_OK;
}

}  // extern "C"
