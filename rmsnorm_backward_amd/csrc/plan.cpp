// plan.cpp -- host-side planning and validation (no HIP calls).
//
// The group count G is what fixes the summation order of dgamma/dbeta, so it
// is a function of (kind, M, N, io_dtype, statistics mode) alone and never of
// the device's compute-unit count: results are the same on any partitioning
// of the GPU.
#include "plan.hpp"

#include <string.h>

namespace nb {

namespace {
// Kernel A with saved statistics (and in RMSNorm recompute mode): one
// workgroup per compute unit on a 256-CU part (4096 x 16384 bf16 RMSNorm step: 72.6 us at 256 groups, 89.5 us
// at the 128 that 2048 waves in flight would give).
constexpr int64_t kSavedStatsGroups = 256;
// Kernel A: rows in flight per workgroup, the fewest (a power of two) whose
// x and dy together reach this many bytes (step times with four rotating
// buffer sets: 65536 x 1024 bf16 RMSNorm 68.5 us at 4 rows, 76.4 us at 8;
// 262144 x 768 218.5 us at 8, 229.6 us at 4; 16384 x 4096 69.2 us at 1,
// 69.9 us at 2).
constexpr int64_t kRowBytesInFlight = 16384;
// The same for RMSNorm rows laid out on 16-byte lanes (one chunk): 65536 x
// 1536 bf16 best at 2 rows (12 KiB; 4 rows 0.714, 2 rows 0.759 of 8 TB/s),
// 32768 x 3584 at 1 row (14 KiB; 114.0 against 119.6 us at 2).
constexpr int64_t kRowBytesInFlight16 = 12288;
// Groups that sweep more than this many bytes of each operand run kernel A's
// general loop rather than its steady-state loop (the kernel holds the same
// bound). There one row in flight leaves HBM idle between rows, and two rows
// in flight were faster on every shape measured (bf16, saved statistics):
// 131072 x 4096 LayerNorm 643 -> 528 us, RMSNorm 580 -> 527 us; 65536 x 8192
// LayerNorm 527 -> 520 us, RMSNorm 527 -> 522 us; 262144 x 4096 RMSNorm
// 1168 -> 1154 us; 65536 x 4096 fp32 even. Inside the bound the steady-state
// loop with one row was faster (65536 x 4096 RMSNorm 268 us against 272 us,
// 32768 x 8192 LayerNorm 264 against 270 us).
constexpr int64_t kSteadyGroupBytes = (int64_t)2 << 20;
// LayerNorm in recompute mode exchanges twice per row; a second workgroup per
// compute unit hides that latency (65536 x 8192 bf16: 570 us at 512 groups
// against 645 us at 256), so it aims at 4096 waves in flight.
constexpr int64_t kRecomputeLnTargetWaves = 4096;
// The forward streams one operand per row where kernel A streams two, so it
// needs twice the waves (16 per compute unit) for as many bytes in flight.
constexpr int64_t kForwardTargetWaves = 4096;
constexpr int64_t kMinRowsPerGroup = 4;
// Group counts above this are rounded down to a multiple of it, so that the
// workgroups (one per group) spread evenly over the 256 compute units. LayerNorm
// recompute of 1151x8192 fp16: 288 groups (the rows-per-group cap) 30.4 us,
// 256 groups 24.2 us; 192, 288 and 384 groups were slower than 256 or 512 on
// every shape measured.
constexpr int64_t kGroupQuantum = 256;
constexpr int64_t kMaxGrid = 1 << 20;
constexpr int kMaxLdsBytes = 65536 - 1024;  // dynamic LDS; the kernel adds 256 B static
// The forward and kernel A in LayerNorm recompute mode fill this many
// threads with rows instead (LayerNorm recompute with the saved-statistics
// rules: 65536 x 8192 bf16 563 -> 655 us, 16384 x 4096 82.4 -> 84.9 us).
// RMSNorm recompute, one exchange per row as with saved statistics, takes
// the saved-statistics rules (16384 x 4096 bf16 70.2 -> 67.9 us, 65536 x
// 1024 75.6 -> 69.3 us, 4096 x 16384 105.7 -> 76.6 us).
constexpr int kRowStatsThreads = 512;
// At most this many bytes of each operand per lane (16 bf16/fp16 or 8 fp32
// elements) before wider lanes are considered: 16384 x 4096 fp32 RMSNorm
// step 129.9 us at 32 bytes (8 waves per row), 149.2 us at 64 (4 waves).
constexpr int kPreferredLaneBytes = 32;
// Column-walk workgroups to aim for: one per compute unit. With the kernel's
// XCD-aware tile order (line neighbours share an L2) narrow tiles cost no
// extra HBM traffic, and the widest tile giving 256 tiles was the fastest on
// every bf16 workload measured (N = 4096: 32-byte rows, 97 us vs 118 us at
// 64 bytes; N = 8192: 64-byte rows, 527 us vs 570 us at 128 bytes).
constexpr int64_t kWgradTargetTiles = 256;
// The two-rows-per-wave kernel's launch bound (nb_tworow.hpp).
constexpr int kTwoRowMaxThreads = 512;
// Its rows in flight per workgroup: the fewest (even, a power of two) whose x
// and dy reach this many bytes. Interleaved on the same buffers, one row per
// wave against two: 262144 x 768 bf16 RMSNorm 219.1 us against 210.7 us at 4
// rows (8: 220.9, 16: 231.1); 1048576 x 256 317.5 against 285.7 at 8 rows
// (4: 411.4, 16: 309.6). Rings deeper than 3 row pairs were slower (LayerNorm
// with saved statistics runs a ring of 2: nb_tworow.hpp).
constexpr int64_t kTwoRowBytesInFlight = 8192;
// LayerNorm, with its second row sum, needs more rows in flight on that
// layout: paired on the same buffers over six placements, A + B, against one
// row per wave (64 lanes with idle lanes): 87381 x 768 bf16 78.7 -> 76.5 us
// at 8 rows (4: 83.8, 16: 81.6), 262144 x 768 224.8 -> 219.0 us (4: 233.6),
// 131072 x 768 fp16 116.1 -> 111.8 us (4: 129.4, 16: 119.1); 262144 x 256
// bf16 88.6 -> 74.2 us at 16 rows (8: 74.6).
constexpr int64_t kTwoRowBytesInFlightLN = 16384;
// Recompute mode (both kinds) takes the LayerNorm target too: A + B on the
// same buffers, RMSNorm 1048576 x 256 bf16 296.5 us at 8 KiB (8 rows) against
// 266.7 at 16 KiB (16 rows), 262144 x 768 214.8 against 217.4, 262144 x 384
// fp32 even; 32 KiB was slower in every case (226.2, 266.7, 224.9).
// LayerNorm recompute at 8 KiB instead: 262144 x 768 bf16 299.9 against
// 221.0 us, 87381 x 768 105.7 against 77.5, 262144 x 256 85.0 against 74.9.
// The two-row forward: 8 waves per workgroup (its launch bound) and about
// this many waves in all (256 workgroups). Forward step times against 4096
// waves (512 workgroups) and against the one-row-per-wave forward: 1048576 x
// 256 bf16 RMSNorm 192.6 us (197.4; 329.0), 262144 x 256 LayerNorm 51.6
// (50.4; 93.1), 262144 x 768 RMSNorm 140.1 (142.9; 140.5), LayerNorm 141.7
// (144.1; 146.0), 131072 x 768 fp16 LayerNorm 70.1 (72.1; 82.6), 262144 x 384
// fp32 RMSNorm 139.2 (144.0; 147.4).
constexpr int64_t kForwardTwoRowTargetWaves = 2048;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int fail(const char** why, const char* msg, int status) {
  if (why) *why = msg;
  return status;
}
}  // namespace

int dtype_bytes(int dtype) {
  switch (dtype) {
    case NORM_BWD_F32: return 4;
    case NORM_BWD_F16: return 2;
    case NORM_BWD_BF16: return 2;
    default: return 0;
  }
}

int max_lane_elems(int io_dtype, int vec_full, int with_dbeta) {
  if (!vec_full) return 8;
  if (dtype_bytes(io_dtype) == 4) return 16;
  return with_dbeta ? 32 : 64;
}

bool kernel_a_exists(int io_dtype, int vec_full, int with_dbeta, int chunks) {
  if (dtype_bytes(io_dtype) == 0) return false;
  if (chunks != 1 && chunks != 2 && chunks != 4 && chunks != 8) return false;
  const int vec = vec_full ? 16 / dtype_bytes(io_dtype) : 1;
  return vec * chunks <= max_lane_elems(io_dtype, vec_full, with_dbeta);
}

int kernel_a_max_threads(int lane_elems) { return lane_elems > 16 ? 512 : 1024; }

int two_row_chunks(int64_t N, int io_dtype) {
  const int eb = dtype_bytes(io_dtype);
  if (eb == 0 || N <= 0) return 0;
  const int64_t vw = 16 / eb;
  if (N % (64 * vw) == 0) return 0;  // 64-lane waves cover it without idle lanes
  const int chunk_counts[] = {1, 3};
  for (int c : chunk_counts)
    if (N == (int64_t)c * 32 * vw) return c;
  return 0;
}

bool two_row_span_ok(int64_t N, int64_t ld, int io_dtype) {
  const int eb = dtype_bytes(io_dtype);
  if (ld < N) ld = N;
  if (eb == 0 || ld > ((int64_t)1 << 32)) return false;
  return (ld + N) * eb < ((int64_t)1 << 32);
}

int64_t two_row_rows_per_group(int64_t M, int64_t G) {
  return G > 0 ? 2 * ceil_div(ceil_div(M, 2), G) : 0;
}

// LDS of kernel A's combine of P > 1 row-lanes: one plane of per-lane
// partials (S waves, C chunks of vec floats), reused for dgamma and dbeta.
static int combine_lds_bytes(int S, int C, int vec) { return S * C * 64 * vec * 4; }

// Lane layout of kernel A for rows of N elements (fills vec, chunks,
// waves_per_row, rows_in_flight, threads, lds_bytes of *p).
int make_geometry(int kind, int64_t N, int io_dtype, int with_dbeta, bool vec_ok16,
                  norm_bwd_plan_t* p, const char** why, bool row_stats, bool saved_stats,
                  bool two_row) {
  const int eb = dtype_bytes(io_dtype);
  const int nacc = with_dbeta ? 2 : 1;
  const int vw = 16 / eb;
  const int full = (vec_ok16 && N % vw == 0) ? 1 : 0;
  p->vec = full ? vw : 1;
  p->rows_per_wave = 1;
  if (N == 0) {  // a minimal valid geometry
    p->chunks = 1;
    p->waves_per_row = 1;
    p->rows_in_flight = 1;
    p->threads = 64;
    p->lds_bytes = 0;
    return NORM_BWD_OK;
  }
  const int64_t max_n = !full ? NORM_BWD_MAX_N_UNALIGNED
                       : eb == 4 ? NORM_BWD_MAX_N_F32
                       : with_dbeta ? NORM_BWD_MAX_N_16BIT_DBETA : NORM_BWD_MAX_N_16BIT;
  if (N > max_n) return fail(why, "N exceeds the fused path's limit", NORM_BWD_ERR_UNSUPPORTED);

  // Prefer at most kPreferredLaneBytes bytes of each operand per lane (the
  // pipelined kernel holds three rows of them in registers), then the
  // smallest S (fewer waves coupled by a barrier per row), then the smallest
  // C. Wider lanes are used only when nothing narrower covers N.
  int S = 0, C = 0;
  for (int pass = 0; pass < 2 && !S; ++pass) {
    for (int s = 1; s <= 16 && !S; s *= 2) {
      for (int c = 1; c <= 8; c *= 2) {
        if (!kernel_a_exists(io_dtype, full, with_dbeta, c)) continue;
        if (pass == 0 && p->vec * c * eb > kPreferredLaneBytes) continue;
        if (s * 64 > kernel_a_max_threads(p->vec * c)) continue;
        if ((int64_t)s * 64 * p->vec * c >= N) { S = s; C = c; break; }
      }
    }
  }
  if (!S) return fail(why, "no kernel geometry covers N", NORM_BWD_ERR_UNSUPPORTED);
  // Widths that waves of kPreferredLaneBytes lanes cover exactly, with a wave
  // count that is not a power of two (5120 16-bit elements: 5 waves of 32
  // bytes a lane), take that count: no idle lanes, and the rows run the
  // steady-state loop. Kernel A, bf16 RMSNorm, fraction of 8 TB/s (power of
  // two with idle lanes -> exact): 16384 x 5120 0.697 -> 0.762 (LayerNorm
  // 0.634 -> 0.723), x 3072 0.695 -> 0.737, x 7168 0.738 -> 0.756, x 6144
  // 0.746 -> 0.753; 8192 x 12288 0.732 -> 0.746.
  if (full && (int64_t)S * 64 * p->vec * C != N) {
    const int c = kPreferredLaneBytes / (p->vec * eb);
    const int64_t per_wave = (int64_t)64 * p->vec * c;
    if (c >= 1 && kernel_a_exists(io_dtype, full, with_dbeta, c) && N % per_wave == 0) {
      const int64_t s = N / per_wave;
      if (s >= 1 && s <= 16 && s * 64 <= kernel_a_max_threads(p->vec * c)) {
        S = (int)s;
        C = c;
      }
    }
  }
  // Widths that 32-byte lanes cannot cover exactly but 16-byte lanes can,
  // with an odd wave count (1536, 2560, 3584 16-bit elements: 3, 5, 7 waves
  // of one chunk), take that layout too. Paired on the same buffers over ten
  // placements, bf16, A + B (power of two with idle lanes -> exact):
  // RMSNorm 65536 x 1536 106.4 -> 102.1 us (2 rows in flight), 32768 x 2560
  // 92.3 -> 88.0 us (2 rows), 32768 x 3584 120.7 -> 114.0 us (1 row; 119.6
  // with 2); LayerNorm 32768 x 2560 99.9 -> 91.1 us, 32768 x 3584 124.7 ->
  // 121.3 us (2 rows each). RMSNorm with saved statistics takes the fewest
  // rows whose x and dy reach kRowBytesInFlight16; LayerNorm keeps
  // kRowBytesInFlight and takes the layout only where that means at most two
  // rows: 65536 x 1536 LayerNorm was slower with it (109.2 -> 114.2 us with 2
  // rows; 1 row far slower still). The forward and recompute mode share the
  // layout (their row sums then run in one order) with their own rows in
  // flight.
  bool exact16 = false;
  if (full && (int64_t)S * 64 * p->vec * C != N && kernel_a_exists(io_dtype, full, with_dbeta, 1)) {
    const int64_t per_wave = (int64_t)64 * p->vec;
    const int64_t s = N % per_wave == 0 ? N / per_wave : 0;
    const bool rows_ok = kind == NORM_BWD_RMSNORM || 2 * (2 * N * eb) >= kRowBytesInFlight;
    if (s >= 1 && s <= 16 && rows_ok) {
      S = (int)s;
      C = 1;
      exact16 = true;
    }
  }
  // Rows in flight: the kernels that compute row statistics fill
  // kRowStatsThreads; kernel A with saved statistics takes the fewest rows
  // whose x and dy reach kRowBytesInFlight (kRowBytesInFlight16 for RMSNorm
  // on 16-byte lanes).
  int P = 1;
  if (row_stats) {
    P = kRowStatsThreads / (64 * S);
    if (P < 1) P = 1;
  } else {
    const int64_t target = exact16 && saved_stats && kind == NORM_BWD_RMSNORM
                               ? kRowBytesInFlight16 : kRowBytesInFlight;
    while (P < 16 && (int64_t)P * 2 * N * eb < target) P *= 2;
    while (P > 1 && S * P > 16) P /= 2;
  }
  while (P > 1 && S * P * 64 > kernel_a_max_threads(p->vec * C)) P /= 2;
  int lds = combine_lds_bytes(S, C, p->vec);
  if (P == 1 || lds > kMaxLdsBytes) { P = 1; lds = 0; }
  p->chunks = C;
  p->waves_per_row = S;
  p->rows_in_flight = P;
  p->threads = 64 * S * P;
  p->lds_bytes = lds;
  // Two rows per wave where 32 lanes cover the row exactly, for every kernel
  // that has the layout (kernel A in both statistics modes, the forward), so
  // that the forward and recompute mode form a row's statistics in one order.
  const int c2 = (two_row && full) ? two_row_chunks(N, io_dtype) : 0;
  if (c2) {
    const int64_t target = (kind == NORM_BWD_LAYERNORM || !saved_stats)
                               ? kTwoRowBytesInFlightLN : kTwoRowBytesInFlight;
    int P2 = 2;
    while (P2 * 32 < kTwoRowMaxThreads && (int64_t)P2 * 2 * N * eb < target) P2 *= 2;
    p->rows_per_wave = 2;
    p->chunks = c2;
    p->waves_per_row = 1;
    p->rows_in_flight = P2;
    p->threads = 32 * P2;
    p->lds_bytes = P2 > 2 ? nacc * c2 * 32 * p->vec * 4 : 0;
  }
  return NORM_BWD_OK;
}

bool fused_fits(int64_t N, int io_dtype, int with_dbeta, bool vec_ok16) {
  norm_bwd_plan_t g;
  const char* why = nullptr;
  return make_geometry(NORM_BWD_RMSNORM, N, io_dtype, with_dbeta, vec_ok16, &g, &why, false,
                       true) == NORM_BWD_OK;
}

int64_t rowloop_grid(int64_t M) { return M < 512 ? (M < 1 ? 1 : M) : 512; }

// The register-held wide-row kernels run 1024 threads (16 waves) per row;
// with 64 elements of x and dy per thread one workgroup fills a compute
// unit's register file, so the grid is one workgroup per compute unit.
constexpr int64_t kRowThreads = 1024;

// At 8 chunks the row's x and dy take 64 of the 128 registers a thread of a
// 1024-thread workgroup has; LayerNorm recompute (backward) and LayerNorm
// with beta (forward) need more than the rest and would spill, so those rows
// keep the row loop.
int rowreg_chunks(int64_t N, int io_dtype, bool vec_ok16, bool ln_heavy) {
  const int eb = dtype_bytes(io_dtype);
  if (!vec_ok16 || eb == 0 || N <= 0 || ((int64_t)N * eb) % 16 != 0) return 0;
  const int64_t per_chunk = kRowThreads * (16 / eb);
  if (N <= 4 * per_chunk) return 4;
  if (N <= 8 * per_chunk && !ln_heavy) return 8;
  return 0;
}

int64_t rowreg_grid(int64_t M) { return M < 256 ? (M < 1 ? 1 : M) : 256; }

// Partials of 16 MiB (8192 features, both gradients, 256 groups) written
// with cached stores cost up to 5 us more per step than with non-temporal
// stores read back with non-temporal loads (1151x8192 fp16 LayerNorm 25.5 ->
// 20.7 us, 8192x8192 bf16 80.6 -> 77.2 us); 8 MiB showed no difference, and
// at 4 MiB (the 16384x4096 RMSNorm step) the cached form was 0.4 us faster.
constexpr size_t kStreamWorkspaceBytes = (size_t)12 << 20;

bool stream_workspace(size_t bytes) { return bytes >= kStreamWorkspaceBytes; }

int64_t forward_grid(int64_t M, int S, int P) {
  if (M <= 0) return 0;
  int64_t g = kForwardTargetWaves / (S * P);
  // wave counts that are not powers of two would leave a partial second
  // round of workgroups (14 waves: 292): whole multiples of 256 instead
  if (g > kGroupQuantum) g -= g % kGroupQuantum;
  const int64_t sweep = ceil_div(M, P);
  if (g > sweep) g = sweep;
  if (g > kMaxGrid) g = kMaxGrid;
  return g < 1 ? 1 : g;
}

// The forward doubles the row-statistics rows in flight (1024 threads) when
// every row-lane still gets at least this many rows: the second row hides
// the exchange of the first. Step times, 512 -> 1024 threads: 65536 x 8192
// bf16 LayerNorm 401.4 -> 374.7 us, RMSNorm 396.1 -> 360.4 us; 16384 x 4096
// fp32 RMSNorm 90.8 -> 87.5 us, bf16 46.7 -> 46.0 us; 262144 x 768 144.5 ->
// 143.7 us; 65536 x 1024 even. With few rows per lane it lost: 1151 x 8192
// fp16 LayerNorm 11.3 -> 12.5 us (about 2 rows per lane).
constexpr int64_t kForwardRowsPerLaneMin = 4;

int forward_rows_in_flight(int64_t M, int S, int P, int lane_elems) {
  const int P2 = 2 * P;
  if (M <= 0 || S * P2 > 16 || 64 * S * P2 > kernel_a_max_threads(lane_elems)) return P;
  const int64_t lanes = forward_grid(M, S, P2) * P2;
  return M >= kForwardRowsPerLaneMin * lanes ? P2 : P;
}

int forward_two_row_waves(int64_t M) {
  (void)M;
  return kTwoRowMaxThreads / 64;
}

int64_t forward_two_row_grid(int64_t M, int W) {
  if (M <= 0 || W <= 0) return 0;
  int64_t g = kForwardTwoRowTargetWaves / W;
  const int64_t sweep = ceil_div(ceil_div(M, 2), W);  // one sweep of row pairs
  if (g > sweep) g = sweep;
  if (g > kMaxGrid) g = kMaxGrid;
  return g < 1 ? 1 : g;
}

int wgrad_lanes_per_row(int64_t N, int vec) {
  int lpr = 64 / vec;  // the 64-column tile
  while (lpr > 1 && ceil_div(N, (int64_t)lpr * vec) < kWgradTargetTiles) lpr >>= 1;
  return lpr;
}

int64_t auto_groups(int kind, int64_t M, int64_t N, int io_dtype, bool recompute) {
  if (M <= 0) return 0;
  // kSavedStatsGroups, except in LayerNorm recompute mode on one row per
  // wave: enough workgroups for about kRecomputeLnTargetWaves waves in
  // flight (16 per compute unit on a 256-CU part). Never fewer than kMinRowsPerGroup rows
  // per group, above kGroupQuantum a multiple of it. The geometry is itself
  // a function of (kind, N, io_dtype), so the group count depends on the
  // problem only, never on the device.
  int64_t G = kSavedStatsGroups;
  if (recompute && kind == NORM_BWD_LAYERNORM) {
    norm_bwd_plan_t g;
    const char* why = nullptr;
    int waves = 8;
    bool two_row = false;
    if (N > 0 && make_geometry(kind, N, io_dtype, 0, true, &g, &why, true, false) == NORM_BWD_OK) {
      waves = g.threads / 64;
      two_row = g.rows_per_wave == 2;
    }
    // (the two-row layout has no barrier per row: the saved-statistics count)
    if (!two_row) G = kRecomputeLnTargetWaves / waves;
  }
  const int64_t cap = ceil_div(M, kMinRowsPerGroup);
  if (G > cap) G = cap;
  if (G > kGroupQuantum) G -= G % kGroupQuantum;
  return G < 1 ? 1 : G;
}

int make_plan(int kind, int64_t M, int64_t N, int io_dtype, int with_dbeta,
              int64_t groups, bool vec_ok16, norm_bwd_plan_t* plan, const char** why,
              bool recompute, int64_t max_ld) {
  if (!plan) return fail(why, "plan is NULL", NORM_BWD_ERR_INVALID_ARG);
  if (kind != NORM_BWD_LAYERNORM && kind != NORM_BWD_RMSNORM)
    return fail(why, "kind must be NORM_BWD_LAYERNORM or NORM_BWD_RMSNORM", NORM_BWD_ERR_INVALID_ARG);
  const int eb = dtype_bytes(io_dtype);
  if (eb == 0) return fail(why, "unknown io_dtype", NORM_BWD_ERR_UNSUPPORTED);
  if (M < 0 || N < 0) return fail(why, "M and N must be >= 0", NORM_BWD_ERR_INVALID_ARG);
  if (groups < 0) return fail(why, "groups must be >= 0", NORM_BWD_ERR_INVALID_ARG);
  if (with_dbeta != 0 && with_dbeta != 1)
    return fail(why, "with_dbeta must be 0 or 1", NORM_BWD_ERR_INVALID_ARG);

  norm_bwd_plan_t p;
  memset(&p, 0, sizeof(p));
  p.kind = kind;
  p.io_dtype = io_dtype;
  p.with_dbeta = with_dbeta;
  p.M = M;
  p.N = N;
  const int nacc = with_dbeta ? 2 : 1;

  const char* gwhy = nullptr;
  const int st = make_geometry(kind, N, io_dtype, with_dbeta, vec_ok16, &p, &gwhy,
                               recompute && kind == NORM_BWD_LAYERNORM, !recompute, true);
  if (st != NORM_BWD_OK) return fail(why, gwhy, st);
  if (N == 0) {  // nothing to compute
    *plan = p;
    return NORM_BWD_OK;
  }

  if (M > 0) {
    // a row pair whose stride needs offsets beyond 32 bits keeps one row per wave
    if (p.rows_per_wave == 2 && !two_row_span_ok(N, max_ld ? max_ld : N, io_dtype))
      make_geometry(kind, N, io_dtype, with_dbeta, vec_ok16, &p, &gwhy,
                    recompute && kind == NORM_BWD_LAYERNORM, !recompute, false);
    int64_t G = groups ? groups : auto_groups(kind, M, N, io_dtype, recompute);
    // every group holds at least one row (two-row plans: one row pair)
    const int64_t units = p.rows_per_wave == 2 ? ceil_div(M, 2) : M;
    if (G > units) G = units;
    p.groups = G;
    p.rows_per_group = p.rows_per_wave == 2 ? two_row_rows_per_group(M, G) : ceil_div(M, G);
    p.grid = (int32_t)(G < kMaxGrid ? G : kMaxGrid);
    // groups on the general loop: two rows in flight (the rows-in-flight
    // rules of saved statistics, which RMSNorm recompute shares)
    const int S = p.waves_per_row, C = p.chunks;
    if (!(recompute && kind == NORM_BWD_LAYERNORM) && p.rows_per_wave == 1 &&
        p.rows_in_flight == 1 &&
        p.rows_per_group * N * dtype_bytes(io_dtype) > kSteadyGroupBytes && 2 * S <= 16 &&
        2 * S * 64 <= kernel_a_max_threads(p.vec * C) &&
        combine_lds_bytes(S, C, p.vec) <= kMaxLdsBytes) {
      p.rows_in_flight = 2;
      p.threads = 2 * S * 64;
      p.lds_bytes = combine_lds_bytes(S, C, p.vec);
    }
  } else {
    p.rows_per_group = 1;
    p.groups = 0;
    p.grid = 0;
  }
  p.workspace_bytes = (size_t)nacc * (size_t)p.groups * (size_t)N * 4u;
  *plan = p;
  return NORM_BWD_OK;
}

// The remaining checks of a two-rows-per-wave plan (fields up to vec done).
static int validate_two_row(const norm_bwd_plan_t* p, const char** why) {
  const int nacc = p->with_dbeta ? 2 : 1;
  if (p->vec != 16 / dtype_bytes(p->io_dtype))
    return fail(why, "plan.rows_per_wave = 2 needs 16-byte vectors", NORM_BWD_ERR_INVALID_ARG);
  if ((p->chunks != 1 && p->chunks != 3) || p->N != (int64_t)p->chunks * 32 * p->vec)
    return fail(why, "plan.rows_per_wave = 2 needs chunks 1 or 3 and N = 32 * vec * chunks",
                NORM_BWD_ERR_UNSUPPORTED);
  if (p->waves_per_row != 1)
    return fail(why, "plan.rows_per_wave = 2 needs waves_per_row = 1", NORM_BWD_ERR_INVALID_ARG);
  const int P = p->rows_in_flight;
  if (P < 2 || P % 2 != 0 || 32 * P > kTwoRowMaxThreads)
    return fail(why, "plan.rows_in_flight must be even, in [2, 16], with rows_per_wave = 2",
                NORM_BWD_ERR_INVALID_ARG);
  if (p->threads != 32 * P)
    return fail(why, "plan.threads must be 32 * rows_in_flight with rows_per_wave = 2",
                NORM_BWD_ERR_INVALID_ARG);
  const int want_lds = P > 2 ? nacc * p->chunks * 32 * p->vec * 4 : 0;
  if (p->lds_bytes != want_lds)
    return fail(why, "plan.lds_bytes inconsistent", NORM_BWD_ERR_INVALID_ARG);
  if (p->M == 0) {
    if (p->groups != 0) return fail(why, "plan.groups must be 0 when M = 0", NORM_BWD_ERR_INVALID_ARG);
    return NORM_BWD_OK;
  }
  if (p->groups < 1 || p->groups > ceil_div(p->M, 2))
    return fail(why, "plan.groups must be in [1, ceil(M / 2)] with rows_per_wave = 2",
                NORM_BWD_ERR_INVALID_ARG);
  if (p->rows_per_group != two_row_rows_per_group(p->M, p->groups))
    return fail(why, "plan.rows_per_group must be 2 * ceil(ceil(M / 2) / groups)",
                NORM_BWD_ERR_INVALID_ARG);
  if (p->grid < 1 || p->grid > p->groups || p->grid > kMaxGrid)
    return fail(why, "plan.grid must be in [1, groups]", NORM_BWD_ERR_INVALID_ARG);
  if (!two_row_span_ok(p->N, p->N, p->io_dtype))
    return fail(why, "plan.rows_per_wave = 2: a row pair too long for 32-bit offsets",
                NORM_BWD_ERR_INVALID_ARG);
  return NORM_BWD_OK;
}

int validate_plan(const norm_bwd_plan_t* p, const char** why) {
  if (!p) return fail(why, "plan is NULL", NORM_BWD_ERR_INVALID_ARG);
  if (p->kind != NORM_BWD_LAYERNORM && p->kind != NORM_BWD_RMSNORM)
    return fail(why, "plan.kind invalid", NORM_BWD_ERR_INVALID_ARG);
  const int eb = dtype_bytes(p->io_dtype);
  if (eb == 0) return fail(why, "plan.io_dtype unknown", NORM_BWD_ERR_UNSUPPORTED);
  if (p->with_dbeta != 0 && p->with_dbeta != 1)
    return fail(why, "plan.with_dbeta must be 0 or 1", NORM_BWD_ERR_INVALID_ARG);
  if (p->M < 0 || p->N < 0) return fail(why, "plan.M/N negative", NORM_BWD_ERR_INVALID_ARG);
  const int nacc = p->with_dbeta ? 2 : 1;
  if (p->workspace_bytes != (size_t)nacc * (size_t)p->groups * (size_t)p->N * 4u)
    return fail(why, "plan.workspace_bytes inconsistent with groups and N", NORM_BWD_ERR_INVALID_ARG);
  if (p->N == 0) return NORM_BWD_OK;
  const int vw = 16 / eb;
  int full;
  if (p->vec == vw && p->N % vw == 0) full = 1;
  else if (p->vec == 1) full = 0;
  else return fail(why, "plan.vec must be 16/elem_size (with N a multiple of it) or 1",
                   NORM_BWD_ERR_INVALID_ARG);
  if (p->rows_per_wave == 2) return validate_two_row(p, why);
  if (p->rows_per_wave != 1)
    return fail(why, "plan.rows_per_wave must be 1 or 2", NORM_BWD_ERR_INVALID_ARG);
  if (!kernel_a_exists(p->io_dtype, full, p->with_dbeta, p->chunks))
    return fail(why, "plan.chunks: no kernel for this vec*chunks", NORM_BWD_ERR_UNSUPPORTED);
  const int S = p->waves_per_row, P = p->rows_in_flight;
  if (S < 1 || P < 1 || S * P > 16)
    return fail(why, "plan.waves_per_row * rows_in_flight must be in [1, 16]", NORM_BWD_ERR_INVALID_ARG);
  if (p->threads != 64 * S * P)
    return fail(why, "plan.threads must be 64 * waves_per_row * rows_in_flight", NORM_BWD_ERR_INVALID_ARG);
  if (p->threads > kernel_a_max_threads(p->vec * p->chunks))
    return fail(why, "plan.threads above the kernel's launch bound", NORM_BWD_ERR_INVALID_ARG);
  if ((int64_t)S * 64 * p->vec * p->chunks < p->N)
    return fail(why, "plan geometry does not cover N", NORM_BWD_ERR_INVALID_ARG);
  const int want_lds = P > 1 ? combine_lds_bytes(S, p->chunks, p->vec) : 0;
  if (p->lds_bytes != want_lds || want_lds > kMaxLdsBytes)
    return fail(why, "plan.lds_bytes inconsistent (or above 63 KiB)", NORM_BWD_ERR_INVALID_ARG);
  if (p->M == 0) {
    if (p->groups != 0) return fail(why, "plan.groups must be 0 when M = 0", NORM_BWD_ERR_INVALID_ARG);
    return NORM_BWD_OK;
  }
  if (p->groups < 1 || p->groups > p->M)
    return fail(why, "plan.groups must be in [1, M]", NORM_BWD_ERR_INVALID_ARG);
  if (p->rows_per_group != ceil_div(p->M, p->groups))
    return fail(why, "plan.rows_per_group must be ceil(M / groups)", NORM_BWD_ERR_INVALID_ARG);
  if (p->grid < 1 || p->grid > p->groups || p->grid > kMaxGrid)
    return fail(why, "plan.grid must be in [1, groups]", NORM_BWD_ERR_INVALID_ARG);
  return NORM_BWD_OK;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace nb
