// plan_driver.cpp -- exercises the host-side planner (csrc/plan.cpp) over a
// grid of valid and invalid arguments, for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py). Every plan the
// planner accepts must pass its own validation and the invariants the
// kernels rely on; every invalid argument must be refused with a status.
// Prints "plan driver: N plans, R refusals" and exits 0, or names the first
// broken case and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "norm_bwd.h"
#include "plan.hpp"

static int fails = 0;

#define EXPECT(cond, ...)                                      \
  do {                                                         \
    if (!(cond)) {                                             \
      if (fails++ < 10) {                                      \
        fprintf(stderr, "FAILED %s: ", #cond);                 \
        fprintf(stderr, __VA_ARGS__);                          \
        fprintf(stderr, "\n");                                 \
      }                                                        \
    }                                                          \
  } while (0)

int main() {
  const int kinds[] = {NORM_BWD_LAYERNORM, NORM_BWD_RMSNORM};
  const int dtypes[] = {NORM_BWD_F32, NORM_BWD_F16, NORM_BWD_BF16};
  const int64_t Ms[] = {0, 1, 2, 3, 4, 5, 7, 63, 64, 255, 256, 257, 1023, 1024, 1151, 4099,
                        16384, 65536, 262144, (int64_t)1 << 31, (int64_t)1 << 40};
  const int64_t Ns[] = {0, 1, 2, 3, 7, 8, 15, 16, 63, 64, 65, 255, 256, 257, 511, 512, 513,
                        768, 1000, 1024, 2048, 4096, 4100, 8191, 8192, 8193, 16383, 16384,
                        16385, 32767, 32768, 32769, 65536};
  const int64_t Gs[] = {0, 1, 2, 7, 16, 255, 256, 257, 512, 1000, (int64_t)1 << 30};
  long plans = 0, refusals = 0;
  for (int kind : kinds)
    for (int dt : dtypes)
      for (int64_t M : Ms)
        for (int64_t N : Ns)
          for (int db = 0; db < 2; ++db)
            for (int64_t G : Gs)
              for (int vec_ok = 0; vec_ok < 2; ++vec_ok)
                for (int rc = 0; rc < 2; ++rc) {
                  norm_bwd_plan_t p;
                  memset(&p, 0xAB, sizeof(p));
                  const char* why = nullptr;
                  const int st = nb::make_plan(kind, M, N, dt, db, G, vec_ok != 0, &p, &why,
                                               rc != 0);
                  if (st != NORM_BWD_OK) {
                    ++refusals;
                    EXPECT(why != nullptr, "refusal without a reason");
                    EXPECT(st == NORM_BWD_ERR_UNSUPPORTED, "M=%lld N=%lld status %d",
                           (long long)M, (long long)N, st);
                    continue;
                  }
                  ++plans;
                  const int vst = nb::validate_plan(&p, &why);
                  EXPECT(vst == NORM_BWD_OK, "kind %d dt %d M %lld N %lld db %d G %lld: %s",
                         kind, dt, (long long)M, (long long)N, db, (long long)G,
                         why ? why : "");
                  if (N == 0) continue;
                  const int eb = nb::dtype_bytes(dt);
                  EXPECT(p.vec == 1 || (N * eb) % 16 == 0, "vector rows");
                  if (p.rows_per_wave == 2) {
                    // two rows per wave: 32 lanes cover the row exactly
                    EXPECT(p.vec == 16 / eb, "two-row layout on 16-byte lanes");
                    EXPECT((int64_t)32 * p.vec * p.chunks == N &&
                               (p.chunks == 1 || p.chunks == 3),
                           "two-row coverage");
                    EXPECT(p.waves_per_row == 1 && p.rows_in_flight % 2 == 0 &&
                               p.threads == 32 * p.rows_in_flight && p.threads <= 512,
                           "two-row threads");
                    if (M > 0) {
                      EXPECT(nb::two_row_span_ok(N, N, dt), "two-row span");
                      EXPECT(p.groups >= 1 && 2 * p.groups <= M + 1, "groups of row pairs");
                      EXPECT(p.rows_per_group == nb::two_row_rows_per_group(M, p.groups),
                             "rows per group of row pairs");
                    }
                  } else {
                    EXPECT(p.rows_per_wave == 1, "rows_per_wave");
                    EXPECT((int64_t)p.waves_per_row * 64 * p.vec * p.chunks >= N, "coverage");
                    EXPECT(p.threads == 64 * p.waves_per_row * p.rows_in_flight, "threads");
                    EXPECT(p.threads <= nb::kernel_a_max_threads(p.vec * p.chunks), "bound");
                  }
                  if (M > 0) {
                    EXPECT(p.groups >= 1 && p.groups <= M, "groups in [1, M]");
                    EXPECT(p.rows_per_group * p.groups >= M, "groups cover M");
                    EXPECT(p.rows_per_wave == 2 || p.rows_per_group == (M + p.groups - 1) / p.groups,
                           "rows per group");
                    EXPECT(p.grid >= 1 && p.grid <= p.groups, "grid");
                    EXPECT(p.workspace_bytes ==
                               (size_t)(db ? 2 : 1) * (size_t)p.groups * (size_t)N * 4u,
                           "workspace");
                    if (G == 0)  // automatic groups never depend on the device
                      EXPECT(p.groups == nb::auto_groups(kind, M, N, dt, rc != 0) ||
                                 p.groups == M || p.groups == (M + 1) / 2,
                             "automatic groups");
                  }
                }
  // the forward's launch: row-statistics geometry, rows in flight and grid
  long forwards = 0;
  for (int kind : kinds)
    for (int dt : dtypes)
      for (int64_t M : Ms)
        for (int64_t N : Ns)
          for (int vec_ok = 0; vec_ok < 2; ++vec_ok) {
            if (M == 0 || N == 0) continue;
            norm_bwd_plan_t g;
            const char* why = nullptr;
            if (nb::make_geometry(kind, N, dt, 0, vec_ok != 0, &g, &why, true) != NORM_BWD_OK)
              continue;
            ++forwards;
            if (g.rows_per_wave == 2) {
              // two rows per wave: waves of a row pair each over ceil(M / 2) pairs
              EXPECT(vec_ok && (int64_t)32 * g.vec * g.chunks == N, "forward two-row coverage");
              const int W = nb::forward_two_row_waves(M);
              EXPECT(W >= 1 && 64 * W <= 512, "forward two-row waves %d", W);
              const int64_t pairs = (M + 1) / 2;
              const int64_t grid = nb::forward_two_row_grid(M, W);
              EXPECT(grid >= 1 && grid <= (pairs + W - 1) / W, "forward two-row grid");
              EXPECT(nb::two_row_span_ok(N, N, dt), "forward two-row span");
              continue;
            }
            const int S = g.waves_per_row, P0 = g.rows_in_flight;
            const int P = nb::forward_rows_in_flight(M, S, P0, g.vec * g.chunks);
            EXPECT(P == P0 || P == 2 * P0, "forward P %d from %d", P, P0);
            EXPECT(S * P <= 16, "forward waves S %d P %d", S, P);
            EXPECT(64 * S * P <= nb::kernel_a_max_threads(g.vec * g.chunks), "forward bound");
            const int64_t grid = nb::forward_grid(M, S, P);
            EXPECT(grid >= 1 && grid <= (M + P - 1) / P, "forward grid %lld", (long long)grid);
            if (P == 2 * P0) EXPECT(M >= 4 * grid * P, "forward rows per lane");
          }
  EXPECT(forwards > 1000, "forward cases %ld", forwards);

  // invalid arguments are refused with a status, and leave no half-filled plan used
  const struct { int kind, dt; int64_t M, N; int db; int64_t G; } bad[] = {
      {7, NORM_BWD_BF16, 8, 8, 0, 0}, {NORM_BWD_RMSNORM, 9, 8, 8, 0, 0},
      {NORM_BWD_RMSNORM, NORM_BWD_BF16, -1, 8, 0, 0}, {NORM_BWD_RMSNORM, NORM_BWD_BF16, 8, -1, 0, 0},
      {NORM_BWD_RMSNORM, NORM_BWD_BF16, 8, 8, 2, 0}, {NORM_BWD_RMSNORM, NORM_BWD_BF16, 8, 8, 0, -3},
      {NORM_BWD_RMSNORM, NORM_BWD_BF16, 8, (int64_t)1 << 40, 0, 0}};
  for (const auto& b : bad) {
    norm_bwd_plan_t p;
    const char* why = nullptr;
    const int st = nb::make_plan(b.kind, b.M, b.N, b.dt, b.db, b.G, true, &p, &why, false);
    EXPECT(st != NORM_BWD_OK && why != nullptr, "bad arguments accepted");
    ++refusals;
  }
  EXPECT(nb::make_plan(NORM_BWD_RMSNORM, 8, 8, NORM_BWD_BF16, 0, 0, true, nullptr, nullptr,
                       false) == NORM_BWD_ERR_INVALID_ARG,
         "NULL plan");
  // validation refuses edited plans that break an invariant
  norm_bwd_plan_t good;
  const char* why = nullptr;
  EXPECT(nb::make_plan(NORM_BWD_LAYERNORM, 4099, 4096, NORM_BWD_BF16, 1, 0, true, &good, &why,
                       false) == NORM_BWD_OK,
         "headline-like plan");
  struct Edit { const char* what; void (*f)(norm_bwd_plan_t&); };
  const Edit edits[] = {
      {"groups 0", [](norm_bwd_plan_t& p) { p.groups = 0; }},
      {"groups > M", [](norm_bwd_plan_t& p) { p.groups = p.M + 1; }},
      {"threads", [](norm_bwd_plan_t& p) { p.threads += 64; }},
      {"coverage", [](norm_bwd_plan_t& p) { p.waves_per_row = 1; p.threads = 64 * p.rows_in_flight; }},
      {"workspace", [](norm_bwd_plan_t& p) { p.workspace_bytes -= 4; }},
      {"vec", [](norm_bwd_plan_t& p) { p.vec = 3; }},
      {"grid", [](norm_bwd_plan_t& p) { p.grid = (int32_t)p.groups + 1; }},
      {"lds", [](norm_bwd_plan_t& p) { p.lds_bytes += 4; }},
      {"kind", [](norm_bwd_plan_t& p) { p.kind = 5; }},
      {"with_dbeta", [](norm_bwd_plan_t& p) { p.with_dbeta = 2; }},
      {"rows_per_wave 3", [](norm_bwd_plan_t& p) { p.rows_per_wave = 3; }},
      {"rows_per_wave 2, N not covered", [](norm_bwd_plan_t& p) { p.rows_per_wave = 2; }},
  };
  for (const Edit& e : edits) {
    norm_bwd_plan_t p = good;
    e.f(p);
    EXPECT(nb::validate_plan(&p, &why) != NORM_BWD_OK, "edit '%s' accepted", e.what);
    ++refusals;
  }
  EXPECT(nb::validate_plan(nullptr, &why) == NORM_BWD_ERR_INVALID_ARG, "NULL plan validated");
  // overlap helper: adjacent ranges do not overlap, shared bytes do
  char buf[64];
  EXPECT(!nb::ranges_overlap(buf, 32, buf + 32, 32), "adjacent");
  EXPECT(nb::ranges_overlap(buf, 33, buf + 32, 32), "one shared byte");
  EXPECT(!nb::ranges_overlap(nullptr, 8, buf, 8), "NULL never overlaps");
  if (fails) {
    fprintf(stderr, "plan driver: %d failures\n", fails);
    return 1;
  }
  printf("plan driver: %ld plans, %ld refusals\n", plans, refusals);
  return 0;
}
