// plan.hpp -- host-side planning and validation for the norm-backward
// library. Pure C++ (no HIP headers), so it runs and is tested without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "norm_bwd.h"

namespace nb {

// Element size in bytes of a NORM_BWD_* dtype code, or 0 if unknown.
int dtype_bytes(int dtype);

// Largest elements-per-lane (vec * chunks) kernel A is instantiated for.
int max_lane_elems(int io_dtype, int vec_full, int with_dbeta);

// Whether kernel A is instantiated for these template parameters.
bool kernel_a_exists(int io_dtype, int vec_full, int with_dbeta, int chunks);

// Largest workgroup kernel A accepts for vec * chunks elements per lane.
int kernel_a_max_threads(int lane_elems);

// Lane layout for rows of N elements (vec, chunks, waves_per_row,
// rows_in_flight, threads, lds_bytes, rows_per_wave of *plan), for kernel A
// with saved statistics or, with `row_stats`, for the kernels that compute
// row statistics with a barrier per row (the forward, LayerNorm recompute
// mode): the lane layout is the same, the rows in flight differ. Returns a
// status. `saved_stats`: kernel A with saved statistics, which has its own
// rows-in-flight target for RMSNorm rows on 16-byte lanes. `two_row`: rows
// that 32 lanes cover exactly take the two-rows-per-wave layout (every mode
// has it; its rows in flight are those of kernel A, which the forward
// replaces by its own).
int make_geometry(int kind, int64_t N, int io_dtype, int with_dbeta, bool vec_ok16,
                  norm_bwd_plan_t* plan, const char** why, bool row_stats,
                  bool saved_stats = false, bool two_row = true);

// The two-rows-per-wave layout for rows of N elements: its chunk count (1 or
// 3) when 32 lanes of 16-byte vectors cover N exactly and 64-lane waves would
// not, else 0.
int two_row_chunks(int64_t N, int io_dtype);

// Whether a row pair of the two-row layout (adjacent rows, row stride ld
// elements) spans fewer than 2^32 bytes (its 32-bit buffer offsets).
bool two_row_span_ok(int64_t N, int64_t ld, int io_dtype);

// The most rows a group of the two-row layout holds: groups are sets of row
// pairs, so 2 * ceil(ceil(M / 2) / G).
int64_t two_row_rows_per_group(int64_t M, int64_t G);

// Whether the fused kernels (rows held in registers) cover rows of N elements
// of io_dtype; wider rows take the row-loop path.
bool fused_fits(int64_t N, int io_dtype, int with_dbeta, bool vec_ok16);

// Rows too wide for the fused kernels that one 1024-thread workgroup can hold
// in registers: the number of 16-byte chunks per thread (4 or 8), or 0 when
// the row needs the row loop (also for rows that are not 16-byte aligned).
// `ln_heavy`: LayerNorm recompute (backward) or LayerNorm with beta
// (forward), which do not fit at 8 chunks.
int rowreg_chunks(int64_t N, int io_dtype, bool vec_ok16, bool ln_heavy);
int64_t rowreg_grid(int64_t M);

// Whether kernels A and B move a workspace of `bytes` with non-temporal
// stores and loads rather than cached ones.
bool stream_workspace(size_t bytes);

// Workgroups of the row-loop kernel for M rows: one 16-wave workgroup per row,
// at most two per compute unit.
int64_t rowloop_grid(int64_t M);

// Workgroups of the forward kernel for M rows with S waves per row and P rows
// in flight: enough for about 4096 waves (16 per compute unit), above 256 a
// multiple of 256, at most one sweep of rows.
int64_t forward_grid(int64_t M, int S, int P);

// Rows in flight of the forward for M rows, given the row-statistics
// geometry's S waves per row, P rows in flight and vec * chunks elements per
// lane: 2P (1024 threads) when 16 waves and the launch bound allow it and
// every row-lane of the resulting grid still gets at least 4 rows, else P.
int forward_rows_in_flight(int64_t M, int S, int P, int lane_elems);

// Waves per workgroup of the two-rows-per-wave forward for M rows (each wave
// two rows): the kernel's launch bound, 8.
int forward_two_row_waves(int64_t M);

// Workgroups of the two-rows-per-wave forward for M rows and W waves per
// workgroup: about 2048 waves, at most one sweep of the ceil(M / 2) pairs.
int64_t forward_two_row_grid(int64_t M, int W);

// Lanes per row of the column-walk tile (tile = lpr * vec columns) for N
// columns: the widest tile (up to 64 columns) that still gives at least 256
// tiles, and at least one lane.
int wgrad_lanes_per_row(int64_t N, int vec);

// Automatic group count for (kind, M, N, io_dtype) and the statistics mode:
// 256, except LayerNorm in recompute mode on one row per wave (about 4096
// waves in flight: 512 for its 512-thread workgroups); at least 4 rows per
// group, above 256 a multiple of 256. Independent of the device.
int64_t auto_groups(int kind, int64_t M, int64_t N, int io_dtype, bool recompute = false);

// Fill *plan (see norm_bwd_make_plan). `vec_ok16` says whether the caller's
// pointers are 16-byte aligned. Writes a message into *why on failure.
// `recompute`: the plan is for recompute mode (affects the automatic groups
// and rows in flight). `max_ld`: the largest
// row stride in elements of x, dy and dx (0: N), for the two-row layout's
// span.
int make_plan(int kind, int64_t M, int64_t N, int io_dtype, int with_dbeta,
              int64_t groups, bool vec_ok16, norm_bwd_plan_t* plan, const char** why,
              bool recompute = false, int64_t max_ld = 0);

// Check every field of a (possibly caller-edited) plan. Returns a status.
int validate_plan(const norm_bwd_plan_t* plan, const char** why);

// Byte ranges [p, p+n) overlap?
bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb);

}  // namespace nb
