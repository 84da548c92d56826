/*
 * A plain C99 consumer of the library's C ABI (include/norm_bwd.h): no Python,
 * no torch, only the HIP runtime for device memory. Test infrastructure.
 *
 *   c_abi_consumer host
 *       Host-only calls (no device memory, nothing launched): status strings,
 *       workspace sizes, plans, and argument errors. Exit 0 when all hold.
 *
 *   c_abi_consumer run KIND M N IO_DTYPE WGRAD_DTYPE WITH_DBETA IN OUT
 *       KIND 0 LayerNorm / 1 RMSNorm, dtypes as the header's codes. IN holds,
 *       back to back: x[M*N], dy[M*N], gamma[N] in IO_DTYPE, then (LayerNorm)
 *       mean[M] and rstd[M] as fp32. Runs the backward three ways on the
 *       default stream: the named entry point with norm_bwd_workspace_bytes
 *       of workspace; norm_bwd_make_plan + norm_bwd_execute; and
 *       norm_bwd_execute_partials + norm_bwd_reduce_partials. All three must
 *       give the same bytes (the same automatic plan, no atomics). A call with
 *       one byte too little workspace must fail with NORM_BWD_ERR_WORKSPACE and
 *       leave dx untouched. OUT receives dx[M*N] (IO_DTYPE), dgamma[N] and, with
 *       WITH_DBETA, dbeta[N] (WGRAD_DTYPE) from the named entry point.
 *
 * Exit status: 0 ok, 1 usage or I/O, 2 a library or HIP error, 3 a check failed.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "norm_bwd.h"

static int failures = 0;

#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      fprintf(stderr, "check failed (%s:%d): ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                        \
      fprintf(stderr, "\n");                               \
      ++failures;                                          \
    }                                                      \
  } while (0)

#define HIP(call)                                                          \
  do {                                                                     \
    hipError_t e_ = (call);                                                \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
      exit(2);                                                             \
    }                                                                      \
  } while (0)

#define LIB(call)                                                          \
  do {                                                                     \
    int s_ = (call);                                                       \
    if (s_ != NORM_BWD_OK) {                                               \
      fprintf(stderr, "%s returned %d (%s): %s\n", #call, s_,              \
              norm_bwd_status_string(s_), norm_bwd_last_error());          \
      exit(2);                                                             \
    }                                                                      \
  } while (0)

static size_t elem_bytes(int dtype) {
  return dtype == NORM_BWD_F32 ? 4 : (dtype == NORM_BWD_F16 || dtype == NORM_BWD_BF16) ? 2 : 0;
}

static int host_checks(void) {
  for (int s = 0; s <= 4; ++s)
    CHECK(norm_bwd_status_string(s) != NULL && norm_bwd_status_string(s)[0] != '\0',
          "status string %d", s);
  CHECK(norm_bwd_status_string(99) != NULL, "unknown status string");

  /* workspace sizes: invalid arguments give (size_t)-1 */
  CHECK(norm_bwd_workspace_bytes(7, 16, 16, NORM_BWD_F32, 0) == (size_t)-1, "bad kind");
  CHECK(norm_bwd_workspace_bytes(NORM_BWD_RMSNORM, -1, 16, NORM_BWD_F32, 0) == (size_t)-1,
        "negative M");
  CHECK(norm_bwd_workspace_bytes(NORM_BWD_RMSNORM, 16, 16, 9, 0) == (size_t)-1, "bad dtype");

  /* a plan's workspace is groups * N * 4 bytes per gradient vector, and the
     named entry points' workspace covers it */
  norm_bwd_plan_t p;
  LIB(norm_bwd_make_plan(NORM_BWD_RMSNORM, 16384, 4096, NORM_BWD_BF16, 0, 0, &p));
  CHECK(p.groups >= 1 && p.groups <= p.M, "groups %lld", (long long)p.groups);
  CHECK(p.workspace_bytes == (size_t)p.groups * 4096u * 4u, "plan workspace");
  CHECK(p.rows_per_group == (p.M + p.groups - 1) / p.groups, "rows per group");
  CHECK(p.threads == 64 * p.waves_per_row * p.rows_in_flight, "threads");
  CHECK(norm_bwd_workspace_bytes(NORM_BWD_RMSNORM, 16384, 4096, NORM_BWD_BF16, 0) >=
            p.workspace_bytes, "workspace bytes cover the plan");
  norm_bwd_plan_t q;
  LIB(norm_bwd_make_plan(NORM_BWD_LAYERNORM, 1000, 1024, NORM_BWD_F16, 1, 7, &q));
  CHECK(q.groups == 7 && q.workspace_bytes == 2u * 7u * 1024u * 4u, "explicit groups");
  LIB(norm_bwd_make_plan(NORM_BWD_LAYERNORM, 5, 1024, NORM_BWD_F16, 1, 64, &q));
  CHECK(q.groups == 5, "groups clamped to M: %lld", (long long)q.groups);
  CHECK(norm_bwd_make_plan(NORM_BWD_RMSNORM, 16, 1 << 20, NORM_BWD_BF16, 0, 0, &q) ==
            NORM_BWD_ERR_UNSUPPORTED, "plans cover the fused path only");

  /* argument errors are reported before anything is launched (a NULL
     required pointer: no device pointer is ever dereferenced) */
  int s = norm_bwd_rmsnorm(NULL, NULL, NULL, NULL, 4, 8, NORM_BWD_F32, NORM_BWD_F32, 1e-5f,
                           NULL, NULL, NULL, NULL, 0, NULL);
  CHECK(s == NORM_BWD_ERR_INVALID_ARG, "NULL x gives %d", s);
  CHECK(strlen(norm_bwd_last_error()) > 0, "last error message");
  s = norm_bwd_layernorm(NULL, NULL, NULL, NULL, NULL, 4, 8, 5, NORM_BWD_F32, 1e-5f, NULL, NULL,
                         NULL, NULL, 0, NULL);
  CHECK(s != NORM_BWD_OK, "bad dtype accepted");
  CHECK(norm_bwd_reduce_partials(-1, 8, NORM_BWD_F32, NULL, 0, NULL, NULL, NULL) ==
            NORM_BWD_ERR_INVALID_ARG, "negative groups");
  if (failures) return 3;
  printf("host checks ok\n");
  return 0;
}

static void* read_all(const char* path, size_t want) {
  FILE* f = fopen(path, "rb");
  if (!f) { perror(path); exit(1); }
  void* buf = malloc(want ? want : 1);
  if (!buf || fread(buf, 1, want, f) != want) { fprintf(stderr, "%s: short read\n", path); exit(1); }
  char extra;
  if (fread(&extra, 1, 1, f) != 0) { fprintf(stderr, "%s: longer than expected\n", path); exit(1); }
  fclose(f);
  return buf;
}

static void* dev_copy(const void* host, size_t bytes) {
  void* d = NULL;
  HIP(hipMalloc(&d, bytes ? bytes : 16));
  if (bytes) HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

static void* dev_fill(size_t bytes, int byte) {
  void* d = NULL;
  HIP(hipMalloc(&d, bytes ? bytes : 16));
  HIP(hipMemset(d, byte, bytes ? bytes : 16));
  return d;
}

static void* to_host(const void* d, size_t bytes) {
  void* h = malloc(bytes ? bytes : 1);
  if (!h) exit(1);
  if (bytes) HIP(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
  return h;
}

static int run(int argc, char** argv) {
  if (argc != 10) return 1;
  const int kind = atoi(argv[2]);
  const int64_t M = atoll(argv[3]), N = atoll(argv[4]);
  const int io = atoi(argv[5]), wg = atoi(argv[6]), with_db = atoi(argv[7]);
  const size_t eb = elem_bytes(io), wb = elem_bytes(wg);
  if (!eb || !wb || M < 0 || N < 1 || (kind != 0 && kind != 1)) return 1;
  const size_t mat = (size_t)M * (size_t)N * eb, vec = (size_t)N * eb, wvec = (size_t)N * wb;
  const size_t stats = (size_t)M * 4;
  const size_t in_bytes = 2 * mat + vec + (kind == NORM_BWD_LAYERNORM ? 2 : 1) * stats;
  unsigned char* in = (unsigned char*)read_all(argv[8], in_bytes);

  size_t off = 0;
  void* x = dev_copy(in + off, mat); off += mat;
  void* dy = dev_copy(in + off, mat); off += mat;
  void* gamma = dev_copy(in + off, vec); off += vec;
  float* mean = NULL;
  if (kind == NORM_BWD_LAYERNORM) { mean = (float*)dev_copy(in + off, stats); off += stats; }
  float* rstd = (float*)dev_copy(in + off, stats);

  /* three routes, each with its own outputs, filled with a sentinel first */
  void *dx[3], *dg[3], *db[3];
  for (int r = 0; r < 3; ++r) {
    dx[r] = dev_fill(mat, 0x5a);
    dg[r] = dev_fill(wvec, 0x5a);
    db[r] = with_db ? dev_fill(wvec, 0x5a) : NULL;
  }
  const size_t ws_bytes = norm_bwd_workspace_bytes(kind, M, N, io, with_db);
  if (ws_bytes == (size_t)-1) { fprintf(stderr, "workspace size refused\n"); return 2; }
  void* ws = dev_fill(ws_bytes, 0);

  /* too little workspace: refused, nothing launched */
  if (ws_bytes > 0) {
    int s = kind == NORM_BWD_LAYERNORM
                ? norm_bwd_layernorm(x, dy, gamma, mean, rstd, M, N, io, wg, 1e-5f, dx[0], dg[0],
                                     db[0], ws, ws_bytes - 1, NULL)
                : norm_bwd_rmsnorm(x, dy, gamma, rstd, M, N, io, wg, 1e-5f, dx[0], dg[0], db[0],
                                   ws, ws_bytes - 1, NULL);
    CHECK(s == NORM_BWD_ERR_WORKSPACE, "short workspace gives %d", s);
    HIP(hipDeviceSynchronize());
    unsigned char* h = (unsigned char*)to_host(dx[0], mat);
    size_t bad = 0;
    for (size_t i = 0; i < mat; ++i) bad += h[i] != 0x5a;
    CHECK(bad == 0, "a refused call wrote %zu bytes of dx", bad);
    free(h);
  }

  /* route 0: the named entry point */
  if (kind == NORM_BWD_LAYERNORM)
    LIB(norm_bwd_layernorm(x, dy, gamma, mean, rstd, M, N, io, wg, 1e-5f, dx[0], dg[0], db[0],
                           ws, ws_bytes, NULL));
  else
    LIB(norm_bwd_rmsnorm(x, dy, gamma, rstd, M, N, io, wg, 1e-5f, dx[0], dg[0], db[0], ws,
                         ws_bytes, NULL));

  /* route 1: an explicit automatic plan, executed */
  norm_bwd_plan_t plan;
  LIB(norm_bwd_make_plan(kind, M, N, io, with_db, 0, &plan));
  void* ws1 = dev_fill(plan.workspace_bytes, 0);
  LIB(norm_bwd_execute(&plan, x, dy, gamma, mean, rstd, wg, dx[1], dg[1], db[1], ws1,
                       plan.workspace_bytes, NULL));

  /* route 2: kernel A alone, then kernel B alone */
  void* ws2 = dev_fill(plan.workspace_bytes, 0);
  LIB(norm_bwd_execute_partials(&plan, x, dy, gamma, mean, rstd, dx[2], ws2,
                                plan.workspace_bytes, NULL));
  LIB(norm_bwd_reduce_partials(plan.groups, N, wg, ws2, plan.workspace_bytes, dg[2], db[2],
                               NULL));
  HIP(hipDeviceSynchronize());

  void *hx[3], *hg[3], *hb[3];
  for (int r = 0; r < 3; ++r) {
    hx[r] = to_host(dx[r], mat);
    hg[r] = to_host(dg[r], wvec);
    hb[r] = with_db ? to_host(db[r], wvec) : NULL;
  }
  for (int r = 1; r < 3; ++r) {
    CHECK(memcmp(hx[0], hx[r], mat) == 0, "dx of route %d differs from the named entry point", r);
    CHECK(memcmp(hg[0], hg[r], wvec) == 0, "dgamma of route %d differs", r);
    if (with_db) CHECK(memcmp(hb[0], hb[r], wvec) == 0, "dbeta of route %d differs", r);
  }

  FILE* f = fopen(argv[9], "wb");
  if (!f) { perror(argv[9]); return 1; }
  int ok = fwrite(hx[0], 1, mat, f) == mat && fwrite(hg[0], 1, wvec, f) == wvec &&
           (!with_db || fwrite(hb[0], 1, wvec, f) == wvec);
  if (fclose(f) != 0 || !ok) { fprintf(stderr, "%s: write failed\n", argv[9]); return 1; }

  for (int r = 0; r < 3; ++r) {
    HIP(hipFree(dx[r]));
    HIP(hipFree(dg[r]));
    if (db[r]) HIP(hipFree(db[r]));
    free(hx[r]);
    free(hg[r]);
    free(hb[r]);
  }
  HIP(hipFree(ws));
  HIP(hipFree(ws1));
  HIP(hipFree(ws2));
  HIP(hipFree(x));
  HIP(hipFree(dy));
  HIP(hipFree(gamma));
  if (mean) HIP(hipFree(mean));
  HIP(hipFree(rstd));
  free(in);
  if (failures) return 3;
  printf("run ok: kind %d, %lld x %lld, groups %lld, three routes agree\n", kind, (long long)M,
         (long long)N, (long long)plan.groups);
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "host") == 0) return host_checks();
  if (argc >= 2 && strcmp(argv[1], "run") == 0) {
    int rc = run(argc, argv);
    if (rc == 1) fprintf(stderr, "usage: %s run KIND M N IO WGRAD WITH_DBETA IN OUT\n", argv[0]);
    return rc;
  }
  fprintf(stderr, "usage: %s host | run ...\n", argv[0]);
  return 1;
}
