// api.cpp -- the C ABI (include/norm_bwd.h): argument checks, planning, and
// the launches on the caller's stream (kernel A then kernel B; for rows too
// wide for them the row-loop kernel then the column walk; the forward).
// Every check happens before the first launch. Nothing here allocates memory.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nb_api.hpp"
#include "nb_launch.hpp"
#include "norm_bwd.h"
#include "plan.hpp"

namespace {

thread_local char g_last_error[256] = "";

// NORM_BWD_LOG set to a non-empty value other than "0": each failing call
// also writes its message to stderr. Read once, on the first failure.
bool log_errors() {
  static const bool on = [] {
    const char* v = getenv("NORM_BWD_LOG");
    return v && v[0] && strcmp(v, "0") != 0;
  }();
  return on;
}

int set_error(int status, const char* what) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", norm_bwd_status_string(status),
           what ? what : "");
  if (log_errors()) fprintf(stderr, "norm_bwd: %s\n", g_last_error);
  return status;
}

int hip_error(hipError_t e, const char* where) {
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s: %s",
           norm_bwd_status_string(NORM_BWD_ERR_HIP), where, hipGetErrorString(e));
  if (log_errors()) fprintf(stderr, "norm_bwd: %s\n", g_last_error);
  return NORM_BWD_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Buffers {
  const void* x;
  const void* dy;
  const void* gamma;
  const float* mean;
  const float* rstd;
  void* dx;
  void* dgamma;
  void* dbeta;
  void* ws;
  size_t ws_bytes;
  int64_t ldx = 0, ldy = 0, ldo = 0;  // row strides in elements; 0 = N
};

// Bytes spanned by M rows of N elements with row stride ld (elements).
size_t extent(int64_t M, int64_t N, int64_t ld, int eb) {
  if (M <= 0 || N <= 0) return 0;
  return (size_t)((M - 1) * ld + N) * (size_t)eb;
}

// Row strides valid for (M, N)? Fills in 0 -> N. Returns a status.
int check_strides(int64_t M, int64_t N, Buffers& b) {
  for (int64_t* ld : {&b.ldx, &b.ldy, &b.ldo}) {
    if (*ld == 0) *ld = N;
    if (*ld < N) return set_error(NORM_BWD_ERR_INVALID_ARG, "row stride smaller than N");
    if (M > 1 && *ld > (int64_t)(((uint64_t)1 << 62) / (uint64_t)M / 4u))
      return set_error(NORM_BWD_ERR_INVALID_ARG, "M * row stride too large");
  }
  return NORM_BWD_OK;
}

// Checks shared by every entry point that runs kernel A and/or kernel B.
// `recompute`: kernel A computes the statistics from x (mean/rstd are NULL).
int check_buffers(int kind, int64_t M, int64_t N, int io_dtype, int wgrad_dtype, bool run_a,
                  bool run_b, size_t ws_needed, const Buffers& b, bool recompute = false) {
  const int eb = nb::dtype_bytes(io_dtype);
  const int wb = nb::dtype_bytes(wgrad_dtype);
  if (run_b) {
    if (wb == 0) return set_error(NORM_BWD_ERR_UNSUPPORTED, "unknown wgrad_dtype");
    // with kernel A in the same call, dgamma/dbeta are fp32 or the I/O type
    if (run_a && wgrad_dtype != NORM_BWD_F32 && wgrad_dtype != io_dtype)
      return set_error(NORM_BWD_ERR_UNSUPPORTED, "wgrad_dtype must be NORM_BWD_F32 or io_dtype");
  }
  if (M < 0 || N < 0) return set_error(NORM_BWD_ERR_INVALID_ARG, "M and N must be >= 0");
  if (N > 0 && M > (int64_t)(((uint64_t)1 << 62) / (uint64_t)N / 4u))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "M * N too large");
  if (N == 0) return NORM_BWD_OK;
  const bool rows = run_a && M > 0;
  if (rows) {
    if (!b.x || !b.dy || !b.gamma || !b.dx)
      return set_error(NORM_BWD_ERR_INVALID_ARG, "x, dy, gamma and dx must be non-NULL");
    if (!recompute && !b.rstd)
      return set_error(NORM_BWD_ERR_INVALID_ARG, "rstd must be non-NULL");
    if (!recompute && kind == NORM_BWD_LAYERNORM && !b.mean)
      return set_error(NORM_BWD_ERR_INVALID_ARG, "LayerNorm needs mean");
  }
  if (run_b && !b.dgamma) return set_error(NORM_BWD_ERR_INVALID_ARG, "dgamma must be non-NULL");
  if (ws_needed > 0) {
    if (!b.ws) return set_error(NORM_BWD_ERR_WORKSPACE, "workspace is NULL");
    if (b.ws_bytes < ws_needed) return set_error(NORM_BWD_ERR_WORKSPACE, "workspace too small");
    if (!aligned16(b.ws)) return set_error(NORM_BWD_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  // No output may overlap an input, another output or the workspace (for a
  // strided matrix: anything within its first row's start and its last
  // row's end).
  const int64_t N_ = N;
  auto mat = [&](int64_t ld) { return extent(M, N_, ld ? ld : N_, eb); };
  const size_t vec_in = (size_t)N * (size_t)eb;
  const size_t vec_out = (size_t)N * (size_t)(wb ? wb : 4);
  const size_t stat = (size_t)M * 4u;
  struct R { const void* p; size_t n; };
  const R inputs[] = {{rows ? b.x : nullptr, mat(b.ldx)},
                      {rows ? b.dy : nullptr, mat(b.ldy)},
                      {rows ? b.gamma : nullptr, vec_in},
                      {rows && !recompute && kind == NORM_BWD_LAYERNORM ? b.mean : nullptr, stat},
                      {rows && !recompute ? b.rstd : nullptr, stat}};
  const R outputs[] = {{rows ? b.dx : nullptr, mat(b.ldo)},
                       {run_b ? b.dgamma : nullptr, vec_out},
                       {run_b ? b.dbeta : nullptr, vec_out},
                       {b.ws, ws_needed}};
  const int nout = sizeof(outputs) / sizeof(outputs[0]);
  for (int i = 0; i < nout; ++i) {
    for (const R& in : inputs)
      if (nb::ranges_overlap(outputs[i].p, outputs[i].n, in.p, in.n))
        return set_error(NORM_BWD_ERR_INVALID_ARG, "an output overlaps an input");
    for (int j = i + 1; j < nout; ++j)
      if (nb::ranges_overlap(outputs[i].p, outputs[i].n, outputs[j].p, outputs[j].n))
        return set_error(NORM_BWD_ERR_INVALID_ARG, "outputs/workspace overlap each other");
  }
  return NORM_BWD_OK;
}

int launch_partials(const norm_bwd_plan_t& p, const Buffers& b, hipStream_t stream,
                    bool recompute = false, float eps = 0.0f) {
  if (p.M == 0 || p.N == 0) return NORM_BWD_OK;
  nb::LaunchA a;
  a.kind = p.kind;
  a.nacc = p.with_dbeta ? 2 : 1;
  a.vec_full = p.vec > 1 ? 1 : 0;
  a.chunks = p.chunks;
  a.x = b.x;
  a.dy = b.dy;
  a.gamma = b.gamma;
  a.mean = b.mean;
  a.rstd = b.rstd;
  a.dx = b.dx;
  a.ws = static_cast<float*>(b.ws);
  a.M = p.M;
  a.N = (int)p.N;
  a.ldx = b.ldx ? b.ldx : p.N;
  a.ldy = b.ldy ? b.ldy : p.N;
  a.ldo = b.ldo ? b.ldo : p.N;
  a.G = p.groups;
  a.R = p.rows_per_group;
  a.S = p.waves_per_row;
  a.P = p.rows_in_flight;
  a.threads = p.threads;
  a.grid = p.grid;
  a.lds = p.lds_bytes;
  a.recompute = recompute ? 1 : 0;
  a.eps = eps;
  a.ws_stream = nb::stream_workspace(p.workspace_bytes) ? 1 : 0;
  a.rows_per_wave = p.rows_per_wave;
  a.stream = stream;
  (void)hipGetLastError();  // clear a stale error so a launch failure is ours
  hipError_t e;
  switch (p.io_dtype) {
    case NORM_BWD_F32: e = nb::launch_a_f32(a); break;
    case NORM_BWD_F16: e = nb::launch_a_f16(a); break;
    default: e = nb::launch_a_bf16(a); break;
  }
  if (e != hipSuccess) return hip_error(e, "kernel A launch");
  return NORM_BWD_OK;
}

int launch_reduce(int64_t groups, int64_t N, int wgrad_dtype, const void* ws, void* dgamma,
                  void* dbeta, hipStream_t stream, bool accumulate = false) {
  if (N == 0) return NORM_BWD_OK;
  if (accumulate && groups == 0) return NORM_BWD_OK;  // adds the empty sum: nothing
  const size_t bytes = (size_t)(dbeta ? 2 : 1) * (size_t)groups * (size_t)N * 4u;
  (void)hipGetLastError();
  hipError_t e = nb::launch_reduce(wgrad_dtype, static_cast<const float*>(ws), groups, (int)N,
                                   dgamma, dbeta, accumulate ? 1 : 0,
                                   nb::stream_workspace(bytes) ? 1 : 0, stream);
  if (e != hipSuccess) return hip_error(e, "kernel B launch");
  return NORM_BWD_OK;
}

// Pointer alignment the plan's vector width needs (x, dy, gamma, dx).
int check_vec_alignment(const norm_bwd_plan_t& p, const Buffers& b) {
  if (p.vec > 1 && p.M > 0 && p.N > 0) {
    if (!aligned16(b.x) || !aligned16(b.dy) || !aligned16(b.gamma) || !aligned16(b.dx))
      return set_error(NORM_BWD_ERR_INVALID_ARG,
                       "plan.vec > 1 needs 16-byte aligned x, dy, gamma and dx");
  }
  return NORM_BWD_OK;
}

// Launch the column walk (arguments already checked). M = 0 writes zeros, or
// with `accumulate` launches nothing.
int launch_colwalk(int kind, const void* x, const void* dy, const float* mean, const float* rstd,
                   int64_t M, int64_t N, int64_t ldx, int64_t ldy, int io_dtype, int wgrad_dtype,
                   void* dgamma, void* dbeta, bool accumulate, hipStream_t stream) {
  if (N == 0 || (accumulate && M == 0)) return NORM_BWD_OK;
  const int eb = nb::dtype_bytes(io_dtype);
  const bool vec_ok = M == 0 || (aligned16(x) && aligned16(dy) && ((size_t)N * eb) % 16 == 0 &&
                                 ((size_t)ldx * eb) % 16 == 0 && ((size_t)ldy * eb) % 16 == 0);
  const int vec = vec_ok ? 16 / eb : 1;
  nb::LaunchW w;
  w.kind = kind;
  w.nacc = dbeta ? 2 : 1;
  w.vec_full = vec_ok ? 1 : 0;
  w.lpr = nb::wgrad_lanes_per_row(N, vec);
  w.x = x;
  w.dy = dy;
  w.mean = kind == NORM_BWD_LAYERNORM ? mean : nullptr;
  w.rstd = rstd;
  w.M = M;
  w.N = N;
  w.ldx = ldx;
  w.ldy = ldy;
  w.dgamma = dgamma;
  w.dbeta = dbeta;
  w.out_dtype = wgrad_dtype;
  w.accumulate = accumulate ? 1 : 0;
  w.grid = (N + (int64_t)w.lpr * vec - 1) / ((int64_t)w.lpr * vec);
  w.stream = stream;
  (void)hipGetLastError();  // clear a stale error so a launch failure is ours
  hipError_t e;
  switch (io_dtype) {
    case NORM_BWD_F32: e = nb::launch_w_f32(w); break;
    case NORM_BWD_F16: e = nb::launch_w_f16(w); break;
    default: e = nb::launch_w_bf16(w); break;
  }
  if (e != hipSuccess) return hip_error(e, "column-walk launch");
  return NORM_BWD_OK;
}

// Workspace of the wide-row path: the recomputed statistics (LayerNorm mean
// and rstd, RMSNorm rstd) in recompute mode, nothing otherwise.
size_t rowloop_workspace(int kind, int64_t M, bool recompute) {
  return recompute ? (size_t)M * 4u * (kind == NORM_BWD_LAYERNORM ? 2u : 1u) : 0;
}

// Rows too wide for the fused kernels: dx by the row-loop kernel (which also
// stores the statistics in recompute mode), then the weight gradients by the
// column walk.
int run_wide(int kind, Buffers b, int64_t M, int64_t N, int io_dtype, int wgrad_dtype,
             float eps, bool recompute, bool accumulate, hipStream_t stream,
             nb::WorkspaceProvider provider) {
  if (N > INT32_MAX) return set_error(NORM_BWD_ERR_UNSUPPORTED, "N too large");
  const size_t need = rowloop_workspace(kind, M, recompute);
  if (provider) {
    const int ps = provider(need, &b.ws, &b.ws_bytes, stream);
    if (ps != NORM_BWD_OK) return ps;
  }
  int st = check_buffers(kind, M, N, io_dtype, wgrad_dtype, true, true, need, b, recompute);
  if (st != NORM_BWD_OK) return st;
  if (N == 0) return NORM_BWD_OK;
  float* stats = static_cast<float*>(b.ws);
  float* mean_out = recompute && kind == NORM_BWD_LAYERNORM ? stats : nullptr;
  float* rstd_out = recompute ? (kind == NORM_BWD_LAYERNORM ? stats + M : stats) : nullptr;
  if (M > 0) {
    const int eb = nb::dtype_bytes(io_dtype);
    nb::LaunchL l;
    l.kind = kind;
    l.recompute = recompute ? 1 : 0;
    l.vec_full = (aligned16(b.x) && aligned16(b.dy) && aligned16(b.gamma) && aligned16(b.dx) &&
                  (N * eb) % 16 == 0 && (b.ldx * eb) % 16 == 0 && (b.ldy * eb) % 16 == 0 &&
                  (b.ldo * eb) % 16 == 0)
                     ? 1
                     : 0;
    l.x = b.x;
    l.dy = b.dy;
    l.gamma = b.gamma;
    l.mean = b.mean;
    l.rstd = b.rstd;
    l.dx = b.dx;
    l.mean_out = mean_out;
    l.rstd_out = rstd_out;
    l.M = M;
    l.N = N;
    l.ldx = b.ldx;
    l.ldy = b.ldy;
    l.ldo = b.ldo;
    l.eps = eps;
    l.chunks = l.vec_full ? nb::rowreg_chunks(N, io_dtype, true,
                                              recompute && kind == NORM_BWD_LAYERNORM)
                          : 0;
    l.grid = l.chunks ? nb::rowreg_grid(M) : nb::rowloop_grid(M);
    l.stream = stream;
    (void)hipGetLastError();  // clear a stale error so a launch failure is ours
    hipError_t e;
    switch (io_dtype) {
      case NORM_BWD_F32: e = nb::launch_l_f32(l); break;
      case NORM_BWD_F16: e = nb::launch_l_f16(l); break;
      default: e = nb::launch_l_bf16(l); break;
    }
    if (e != hipSuccess) return hip_error(e, "row-loop launch");
  }
  return launch_colwalk(kind, b.x, b.dy, recompute ? mean_out : b.mean,
                        recompute ? rstd_out : b.rstd, M, N, b.ldx, b.ldy, io_dtype, wgrad_dtype,
                        b.dgamma, b.dbeta, accumulate, stream);
}

// The whole backward with an automatic or explicit group count: the named
// entry points and norm_bwd_ex. Row strides of b must be filled in (>= N).
int run_backward(int kind, Buffers b, int64_t M, int64_t N, int io_dtype, int wgrad_dtype,
                 float eps, int64_t groups, bool accumulate, void* stream,
                 nb::WorkspaceProvider provider = nullptr) {
  if (!(eps >= 0.0f) || isinf(eps))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "eps must be finite and >= 0");
  // NULL statistics (LayerNorm: both) select the recompute mode
  if (kind == NORM_BWD_LAYERNORM && (b.mean == nullptr) != (b.rstd == nullptr))
    return set_error(NORM_BWD_ERR_INVALID_ARG,
                     "LayerNorm takes both mean and rstd, or neither (recompute)");
  const bool recompute = b.rstd == nullptr;
  const int eb = nb::dtype_bytes(io_dtype);
  // 16-byte vectors need every row of x, dy and dx to start 16-byte aligned
  const bool rows16 = eb > 0 && (b.ldx * eb) % 16 == 0 && (b.ldy * eb) % 16 == 0 &&
                      (b.ldo * eb) % 16 == 0;
  const bool vec_ok = rows16 && aligned16(b.x) && aligned16(b.dy) && aligned16(b.gamma) &&
                      aligned16(b.dx);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (eb > 0 && N > 0 && !nb::fused_fits(N, io_dtype, b.dbeta ? 1 : 0, vec_ok)) {
    if (groups != 0)
      return set_error(NORM_BWD_ERR_UNSUPPORTED, "explicit groups need rows the fused path holds");
    if (wgrad_dtype != NORM_BWD_F32 && wgrad_dtype != io_dtype)
      return set_error(NORM_BWD_ERR_UNSUPPORTED, "wgrad_dtype must be NORM_BWD_F32 or io_dtype");
    return run_wide(kind, b, M, N, io_dtype, wgrad_dtype, eps, recompute, accumulate, s,
                    provider);
  }
  norm_bwd_plan_t p;
  const char* why = nullptr;
  int64_t max_ld = b.ldx > b.ldy ? b.ldx : b.ldy;
  if (b.ldo > max_ld) max_ld = b.ldo;
  int st = nb::make_plan(kind, M, N, io_dtype, b.dbeta ? 1 : 0, groups, vec_ok, &p, &why,
                         recompute, max_ld);
  if (st != NORM_BWD_OK) return set_error(st, why);
  if (provider) {
    st = provider(p.workspace_bytes, &b.ws, &b.ws_bytes, stream);
    if (st != NORM_BWD_OK) return st;
  }
  st = check_buffers(kind, M, N, io_dtype, wgrad_dtype, true, true, p.workspace_bytes, b,
                     recompute);
  if (st != NORM_BWD_OK) return st;
  st = launch_partials(p, b, s, recompute, eps);
  if (st != NORM_BWD_OK) return st;
  return launch_reduce(p.groups, N, wgrad_dtype, b.ws, b.dgamma, b.dbeta, s, accumulate);
}

int run_auto(int kind, const void* x, const void* dy, const void* gamma, const float* mean,
             const float* rstd, int64_t M, int64_t N, int io_dtype, int wgrad_dtype, float eps,
             void* dx, void* dgamma, void* dbeta, void* workspace, size_t workspace_bytes,
             void* stream) {
  Buffers b{x, dy, gamma, mean, rstd, dx, dgamma, dbeta, workspace, workspace_bytes};
  b.ldx = b.ldy = b.ldo = N > 0 ? N : 0;
  return run_backward(kind, b, M, N, io_dtype, wgrad_dtype, eps, 0, false, stream);
}

int run_forward(int kind, const void* x, const void* gamma, const void* beta, int64_t M,
                int64_t N, int io_dtype, float eps, void* y, float* mean, float* rstd,
                void* stream) {
  if (kind != NORM_BWD_LAYERNORM && kind != NORM_BWD_RMSNORM)
    return set_error(NORM_BWD_ERR_INVALID_ARG, "kind invalid");
  const int eb = nb::dtype_bytes(io_dtype);
  if (eb == 0) return set_error(NORM_BWD_ERR_UNSUPPORTED, "unknown io_dtype");
  if (M < 0 || N < 0) return set_error(NORM_BWD_ERR_INVALID_ARG, "M and N must be >= 0");
  if (N > 0 && M > (int64_t)(((uint64_t)1 << 62) / (uint64_t)N / 4u))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "M * N too large");
  if (!(eps >= 0.0f) || isinf(eps))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (M == 0 || N == 0) return NORM_BWD_OK;
  if (!x || !gamma || !y) return set_error(NORM_BWD_ERR_INVALID_ARG, "x, gamma and y must be non-NULL");
  const bool vec_ok = aligned16(x) && aligned16(gamma) && aligned16(y) && (!beta || aligned16(beta));
  norm_bwd_plan_t g;
  const char* why = nullptr;
  // rows the fused forward cannot hold in registers take the row-loop kernel
  const bool wide = nb::make_geometry(kind, N, io_dtype, 0, vec_ok, &g, &why, true) != NORM_BWD_OK;
  if (wide && N > INT32_MAX) return set_error(NORM_BWD_ERR_UNSUPPORTED, "N too large");
  // y and the statistics must not overlap the inputs or each other
  const size_t mat = (size_t)M * (size_t)N * (size_t)eb, vec = (size_t)N * (size_t)eb;
  const size_t stat = (size_t)M * 4u;
  struct R { const void* p; size_t n; };
  const R inputs[] = {{x, mat}, {gamma, vec}, {beta, vec}};
  const R outputs[] = {{y, mat}, {kind == NORM_BWD_LAYERNORM ? mean : nullptr, stat}, {rstd, stat}};
  for (int i = 0; i < 3; ++i) {
    for (const R& in : inputs)
      if (nb::ranges_overlap(outputs[i].p, outputs[i].n, in.p, in.n))
        return set_error(NORM_BWD_ERR_INVALID_ARG, "an output overlaps an input");
    for (int j = i + 1; j < 3; ++j)
      if (nb::ranges_overlap(outputs[i].p, outputs[i].n, outputs[j].p, outputs[j].n))
        return set_error(NORM_BWD_ERR_INVALID_ARG, "outputs overlap each other");
  }
  nb::LaunchF f;
  f.kind = kind;
  f.vec_full = wide ? ((vec_ok && ((size_t)N * eb) % 16 == 0) ? 1 : 0) : (g.vec > 1 ? 1 : 0);
  // wide rows: held in registers (4 or 8 chunks per thread) or streamed (0)
  f.chunks = wide ? (f.vec_full ? nb::rowreg_chunks(N, io_dtype, true,
                                                    kind == NORM_BWD_LAYERNORM && beta)
                                : 0)
                  : g.chunks;
  f.x = x;
  f.gamma = gamma;
  f.beta = beta;
  f.y = y;
  f.mean = kind == NORM_BWD_LAYERNORM ? mean : nullptr;
  f.rstd = rstd;
  f.M = M;
  f.N = (int)N;
  f.eps = eps;
  f.S = wide ? 0 : g.waves_per_row;
  f.rows_per_wave = wide ? 1 : g.rows_per_wave;
  if (f.rows_per_wave == 2) {
    // two rows per wave: P waves of a row pair each, over ceil(M / 2) pairs
    f.P = nb::forward_two_row_waves(M);
    f.threads = 64 * f.P;
    f.grid = (int)nb::forward_two_row_grid(M, f.P);
  } else {
    f.P = wide ? 0 : nb::forward_rows_in_flight(M, g.waves_per_row, g.rows_in_flight,
                                                g.vec * g.chunks);
    f.threads = wide ? 0 : 64 * f.S * f.P;
    f.grid = wide ? (int)(f.chunks ? nb::rowreg_grid(M) : nb::rowloop_grid(M))
                  : (int)nb::forward_grid(M, f.S, f.P);
  }
  f.stream = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so a launch failure is ours
  hipError_t e;
  switch (io_dtype) {
    case NORM_BWD_F32: e = wide ? nb::launch_fl_f32(f) : nb::launch_f_f32(f); break;
    case NORM_BWD_F16: e = wide ? nb::launch_fl_f16(f) : nb::launch_f_f16(f); break;
    default: e = wide ? nb::launch_fl_bf16(f) : nb::launch_f_bf16(f); break;
  }
  if (e != hipSuccess) return hip_error(e, "forward launch");
  return NORM_BWD_OK;
}

}  // namespace

namespace nb {

int report_error(int status, const char* what) { return set_error(status, what); }
int report_hip_error(hipError_t e, const char* where) { return hip_error(e, where); }

int run_ex(const norm_bwd_args_t* a, WorkspaceProvider provider) {
  if (!a) return set_error(NORM_BWD_ERR_INVALID_ARG, "args is NULL");
  if (a->kind != NORM_BWD_LAYERNORM && a->kind != NORM_BWD_RMSNORM)
    return set_error(NORM_BWD_ERR_INVALID_ARG, "kind invalid");
  if (a->flags & ~(uint32_t)NORM_BWD_ACCUMULATE)
    return set_error(NORM_BWD_ERR_INVALID_ARG, "unknown flag bits");
  if (a->M < 0 || a->N < 0) return set_error(NORM_BWD_ERR_INVALID_ARG, "M and N must be >= 0");
  if (a->groups < 0) return set_error(NORM_BWD_ERR_INVALID_ARG, "groups must be >= 0");
  if (a->reserved != 0) return set_error(NORM_BWD_ERR_INVALID_ARG, "reserved must be 0");
  Buffers b{a->x, a->dy, a->gamma, a->mean, a->rstd, a->dx, a->dgamma, a->dbeta,
            a->workspace, a->workspace_bytes};
  b.ldx = a->ldx;
  b.ldy = a->lddy;
  b.ldo = a->lddx;
  if (a->ldx < 0 || a->lddy < 0 || a->lddx < 0)
    return set_error(NORM_BWD_ERR_INVALID_ARG, "row strides must be >= 0");
  int st = check_strides(a->M, a->N, b);
  if (st != NORM_BWD_OK) return st;
  return run_backward(a->kind, b, a->M, a->N, a->io_dtype, a->wgrad_dtype, a->eps, a->groups,
                      (a->flags & NORM_BWD_ACCUMULATE) != 0, a->stream, provider);
}

}  // namespace nb

extern "C" {

int norm_fwd_layernorm(const void* x, const void* gamma, const void* beta, int64_t M, int64_t N,
                       int io_dtype, float eps, void* y, float* mean, float* rstd, void* stream) {
  return run_forward(NORM_BWD_LAYERNORM, x, gamma, beta, M, N, io_dtype, eps, y, mean, rstd,
                     stream);
}

int norm_fwd_rmsnorm(const void* x, const void* gamma, int64_t M, int64_t N, int io_dtype,
                     float eps, void* y, float* rstd, void* stream) {
  return run_forward(NORM_BWD_RMSNORM, x, gamma, nullptr, M, N, io_dtype, eps, y, nullptr, rstd,
                     stream);
}

int norm_bwd_layernorm(const void* x, const void* dy, const void* gamma, const float* mean,
                       const float* rstd, int64_t M, int64_t N, int io_dtype, int wgrad_dtype,
                       float eps, void* dx, void* dgamma, void* dbeta, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return run_auto(NORM_BWD_LAYERNORM, x, dy, gamma, mean, rstd, M, N, io_dtype, wgrad_dtype, eps,
                  dx, dgamma, dbeta, workspace, workspace_bytes, stream);
}

int norm_bwd_rmsnorm(const void* x, const void* dy, const void* gamma, const float* rstd,
                     int64_t M, int64_t N, int io_dtype, int wgrad_dtype, float eps, void* dx,
                     void* dgamma, void* dbeta, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return run_auto(NORM_BWD_RMSNORM, x, dy, gamma, nullptr, rstd, M, N, io_dtype, wgrad_dtype,
                  eps, dx, dgamma, dbeta, workspace, workspace_bytes, stream);
}

size_t norm_bwd_workspace_bytes(int kind, int64_t M, int64_t N, int io_dtype, int with_dbeta) {
  // enough for the automatic plan of either statistics mode, on the fused
  // path or (rows too wide for it, or unaligned) the row-loop path
  if ((kind != NORM_BWD_LAYERNORM && kind != NORM_BWD_RMSNORM) || nb::dtype_bytes(io_dtype) == 0 ||
      M < 0 || N < 0 || N > INT32_MAX ||
      (N > 0 && M > (int64_t)(((uint64_t)1 << 62) / (uint64_t)N / 4u)))
    return (size_t)-1;
  size_t need = rowloop_workspace(kind, M, true);
  if (nb::fused_fits(N, io_dtype, with_dbeta ? 1 : 0, true)) {
    norm_bwd_plan_t p, q;
    if (nb::make_plan(kind, M, N, io_dtype, with_dbeta ? 1 : 0, 0, true, &p, nullptr) !=
            NORM_BWD_OK ||
        nb::make_plan(kind, M, N, io_dtype, with_dbeta ? 1 : 0, 0, true, &q, nullptr, true) !=
            NORM_BWD_OK)
      return (size_t)-1;
    if (p.workspace_bytes > need) need = p.workspace_bytes;
    if (q.workspace_bytes > need) need = q.workspace_bytes;
  }
  return need;
}

int norm_bwd_make_plan(int kind, int64_t M, int64_t N, int io_dtype, int with_dbeta,
                       int64_t groups, norm_bwd_plan_t* plan) {
  const char* why = nullptr;
  int st = nb::make_plan(kind, M, N, io_dtype, with_dbeta, groups, true, plan, &why);
  if (st != NORM_BWD_OK) return set_error(st, why);
  return NORM_BWD_OK;
}

int norm_bwd_ex(const norm_bwd_args_t* a) { return nb::run_ex(a, nullptr); }

int norm_bwd_wgrad(int kind, const void* x, const void* dy, const float* mean, const float* rstd,
                   int64_t M, int64_t N, int io_dtype, int wgrad_dtype, void* dgamma,
                   void* dbeta, unsigned flags, void* stream) {
  if (kind != NORM_BWD_LAYERNORM && kind != NORM_BWD_RMSNORM)
    return set_error(NORM_BWD_ERR_INVALID_ARG, "kind invalid");
  if (flags & ~(unsigned)NORM_BWD_ACCUMULATE)
    return set_error(NORM_BWD_ERR_INVALID_ARG, "unknown flag bits");
  const int eb = nb::dtype_bytes(io_dtype);
  const int wb = nb::dtype_bytes(wgrad_dtype);
  if (eb == 0) return set_error(NORM_BWD_ERR_UNSUPPORTED, "unknown io_dtype");
  if (wb == 0 || (wgrad_dtype != NORM_BWD_F32 && wgrad_dtype != io_dtype))
    return set_error(NORM_BWD_ERR_UNSUPPORTED, "wgrad_dtype must be NORM_BWD_F32 or io_dtype");
  if (M < 0 || N < 0) return set_error(NORM_BWD_ERR_INVALID_ARG, "M and N must be >= 0");
  if (N > INT32_MAX) return set_error(NORM_BWD_ERR_UNSUPPORTED, "N too large");
  if (N > 0 && M > (int64_t)(((uint64_t)1 << 62) / (uint64_t)N / 4u))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "M * N too large");
  if (N == 0) return NORM_BWD_OK;
  if (!dgamma) return set_error(NORM_BWD_ERR_INVALID_ARG, "dgamma must be non-NULL");
  if (M > 0) {
    if (!x || !dy || !rstd)
      return set_error(NORM_BWD_ERR_INVALID_ARG, "x, dy and rstd must be non-NULL");
    if (kind == NORM_BWD_LAYERNORM && !mean)
      return set_error(NORM_BWD_ERR_INVALID_ARG, "LayerNorm needs mean");
  }
  const size_t mat = (size_t)M * (size_t)N * (size_t)eb, stat = (size_t)M * 4u;
  const size_t vec_out = (size_t)N * (size_t)wb;
  struct R { const void* p; size_t n; };
  const R inputs[] = {{x, mat}, {dy, mat}, {kind == NORM_BWD_LAYERNORM ? mean : nullptr, stat},
                      {rstd, stat}};
  const R outputs[] = {{dgamma, vec_out}, {dbeta, vec_out}};
  for (int i = 0; i < 2; ++i)
    for (const R& in : inputs)
      if (nb::ranges_overlap(outputs[i].p, outputs[i].n, in.p, in.n))
        return set_error(NORM_BWD_ERR_INVALID_ARG, "an output overlaps an input");
  if (nb::ranges_overlap(dgamma, vec_out, dbeta, vec_out))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "dgamma and dbeta overlap");
  return launch_colwalk(kind, x, dy, mean, rstd, M, N, N, N, io_dtype, wgrad_dtype, dgamma, dbeta,
                        (flags & NORM_BWD_ACCUMULATE) != 0, static_cast<hipStream_t>(stream));
}

int norm_bwd_execute(const norm_bwd_plan_t* plan, const void* x, const void* dy,
                     const void* gamma, const float* mean, const float* rstd, int wgrad_dtype,
                     void* dx, void* dgamma, void* dbeta, void* workspace, size_t workspace_bytes,
                     void* stream) {
  const char* why = nullptr;
  int st = nb::validate_plan(plan, &why);
  if (st != NORM_BWD_OK) return set_error(st, why);
  if ((dbeta != nullptr) != (plan->with_dbeta != 0))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "dbeta must be non-NULL exactly when plan.with_dbeta");
  Buffers b{x, dy, gamma, mean, rstd, dx, dgamma, dbeta, workspace, workspace_bytes};
  st = check_buffers(plan->kind, plan->M, plan->N, plan->io_dtype, wgrad_dtype, true, true,
                     plan->workspace_bytes, b);
  if (st != NORM_BWD_OK) return st;
  st = check_vec_alignment(*plan, b);
  if (st != NORM_BWD_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_partials(*plan, b, s);
  if (st != NORM_BWD_OK) return st;
  return launch_reduce(plan->groups, plan->N, wgrad_dtype, workspace, dgamma, dbeta, s);
}

int norm_bwd_execute_partials(const norm_bwd_plan_t* plan, const void* x, const void* dy,
                              const void* gamma, const float* mean, const float* rstd, void* dx,
                              void* workspace, size_t workspace_bytes, void* stream) {
  const char* why = nullptr;
  int st = nb::validate_plan(plan, &why);
  if (st != NORM_BWD_OK) return set_error(st, why);
  Buffers b{x, dy, gamma, mean, rstd, dx, nullptr, nullptr, workspace, workspace_bytes};
  st = check_buffers(plan->kind, plan->M, plan->N, plan->io_dtype, NORM_BWD_F32, true, false,
                     plan->workspace_bytes, b);
  if (st != NORM_BWD_OK) return st;
  st = check_vec_alignment(*plan, b);
  if (st != NORM_BWD_OK) return st;
  return launch_partials(*plan, b, static_cast<hipStream_t>(stream));
}

int norm_bwd_reduce_partials(int64_t groups, int64_t N, int wgrad_dtype, const void* workspace,
                             size_t workspace_bytes, void* dgamma, void* dbeta, void* stream) {
  if (groups < 0 || N < 0) return set_error(NORM_BWD_ERR_INVALID_ARG, "groups and N must be >= 0");
  if (N > INT32_MAX) return set_error(NORM_BWD_ERR_UNSUPPORTED, "N too large");
  // the partials' size below must not wrap around
  if (N > 0 && groups > (int64_t)(((uint64_t)1 << 62) / (uint64_t)N / 8u))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "groups * N too large");
  const size_t need = (size_t)(dbeta ? 2 : 1) * (size_t)groups * (size_t)N * 4u;
  Buffers b{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, dgamma, dbeta,
            const_cast<void*>(workspace), workspace_bytes};
  int st = check_buffers(NORM_BWD_RMSNORM, 0, N, NORM_BWD_F32, wgrad_dtype, false, true, need, b);
  if (st != NORM_BWD_OK) return st;
  return launch_reduce(groups, N, wgrad_dtype, workspace, dgamma, dbeta,
                       static_cast<hipStream_t>(stream));
}

const char* norm_bwd_status_string(int status) {
  switch (status) {
    case NORM_BWD_OK: return "NORM_BWD_OK";
    case NORM_BWD_ERR_INVALID_ARG: return "NORM_BWD_ERR_INVALID_ARG";
    case NORM_BWD_ERR_UNSUPPORTED: return "NORM_BWD_ERR_UNSUPPORTED";
    case NORM_BWD_ERR_WORKSPACE: return "NORM_BWD_ERR_WORKSPACE";
    case NORM_BWD_ERR_HIP: return "NORM_BWD_ERR_HIP";
    default: return "NORM_BWD_ERR_UNKNOWN";
  }
}

const char* norm_bwd_last_error(void) { return g_last_error; }

int norm_bwd_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return NORM_BWD_OK;
  if (!src || !dst || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "copy probe needs 16-byte aligned, 16-byte multiple");
  if (nb::ranges_overlap(src, bytes, dst, bytes))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "copy probe buffers overlap");
  (void)hipGetLastError();  // clear a stale error so a launch failure is ours
  hipError_t e = nb::launch_copy(src, dst, bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_error(e, "copy probe launch");
  return NORM_BWD_OK;
}

int norm_bwd_probe_triad(const void* a, const void* b, void* c, size_t bytes, int grid,
                         int unroll, void* stream) {
  if (bytes == 0) return NORM_BWD_OK;
  if (!a || !b || !c || bytes % 16 != 0 || !aligned16(a) || !aligned16(b) || !aligned16(c))
    return set_error(NORM_BWD_ERR_INVALID_ARG,
                     "triad probe needs non-NULL, 16-byte aligned buffers of a 16-byte multiple");
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8)
    return set_error(NORM_BWD_ERR_INVALID_ARG, "triad probe unroll must be 1, 2, 4 or 8");
  if (grid < 0 || grid > (1 << 20))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "triad probe grid must be in [0, 2^20]");
  if (nb::ranges_overlap(c, bytes, a, bytes) || nb::ranges_overlap(c, bytes, b, bytes))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "triad probe output overlaps an input");
  if (grid == 0) {  // one pass: every thread handles `unroll` vectors once
    const uint64_t per_block = 256ull * (uint64_t)unroll;
    const uint64_t g = (bytes / 16 + per_block - 1) / per_block;
    grid = (int)(g > (1u << 20) ? (1u << 20) : g);
  }
  (void)hipGetLastError();  // clear a stale error so a launch failure is ours
  hipError_t e = nb::launch_triad(a, b, c, bytes, grid, unroll, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_error(e, "triad probe launch");
  return NORM_BWD_OK;
}

int norm_bwd_probe_triad_policy(const void* a, const void* b, void* c, size_t bytes, int unroll,
                                int load_policy, int store_policy, void* stream) {
  if (bytes == 0) return NORM_BWD_OK;
  if (!a || !b || !c || !aligned16(a) || !aligned16(b) || !aligned16(c))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "triad policy probe needs non-NULL, 16-byte "
                                               "aligned buffers");
  if (unroll != 1 && unroll != 2 && unroll != 4)
    return set_error(NORM_BWD_ERR_INVALID_ARG, "triad policy probe unroll must be 1, 2 or 4");
  if (bytes % (4096u * (unsigned)unroll) != 0 || bytes > NORM_BWD_PROBE_POLICY_MAX_BYTES)
    return set_error(NORM_BWD_ERR_INVALID_ARG, "triad policy probe bytes must be a multiple of "
                                               "4096 * unroll, at most 2^32 - 4096 * 4");
  const auto valid = [](int p) { return p >= 0 && (p & ~(1 | 2 | 16)) == 0; };
  if (!valid(load_policy) || !valid(store_policy))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "triad policy probe policies must be ORs of "
                                               "1 (sc0), 2 (nt) and 16 (sc1)");
  if (nb::ranges_overlap(c, bytes, a, bytes) || nb::ranges_overlap(c, bytes, b, bytes))
    return set_error(NORM_BWD_ERR_INVALID_ARG, "triad policy probe output overlaps an input");
  (void)hipGetLastError();
  hipError_t e = nb::launch_triad_policy(a, b, c, (uint32_t)bytes, unroll, load_policy,
                                         store_policy, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_error(e, "triad policy probe launch");
  return NORM_BWD_OK;
}

}  // extern "C"
