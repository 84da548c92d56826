// nb_launch.hpp -- internal launch interface between the C ABI and the
// per-dtype kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nb {

struct LaunchA {
  int kind;      // NORM_BWD_LAYERNORM / RMSNORM
  int nacc;      // 1: dgamma partials, 2: dgamma and dbeta partials
  int vec_full;  // 1: 16-byte vectors, 0: one element per lane
  int chunks;
  const void* x;
  const void* dy;
  const void* gamma;
  const float* mean;
  const float* rstd;
  void* dx;
  float* ws;
  int64_t M;
  int N;
  int64_t ldx, ldy, ldo;  // row strides (elements) of x, dy, dx
  int64_t G, R;
  int S, P, threads, grid, lds;
  int recompute;  // 1: mean/rstd are NULL and recomputed from x with eps
  float eps;
  int ws_stream;  // 1: non-temporal stores of the partials (16-byte vector rows)
  int rows_per_wave;  // 2: the two-rows-per-wave kernel (nb_tworow.hpp), P = rows in flight
  hipStream_t stream;
};

struct LaunchF {
  int kind;
  int vec_full;
  int chunks;
  const void* x;
  const void* gamma;
  const void* beta;  // may be NULL
  void* y;
  float* mean;       // may be NULL
  float* rstd;       // may be NULL
  int64_t M;
  int N;
  float eps;
  int S, P, threads, grid;
  int rows_per_wave;  // 2: the two-rows-per-wave forward (nb_tworow.hpp), P = waves
  hipStream_t stream;
};

struct LaunchW {
  int kind;
  int nacc;      // 2 when dbeta is written
  int vec_full;  // 1: 16-byte vectors, 0: one element per lane
  int lpr;       // lanes per row of the column tile (tile = lpr * vec columns)
  const void* x;
  const void* dy;
  const float* mean;
  const float* rstd;
  int64_t M, N, ldx, ldy;
  void* dgamma;
  void* dbeta;
  int out_dtype;
  int accumulate;
  int64_t grid;
  hipStream_t stream;
};

struct LaunchL {  // dx for wide rows
  int kind;
  int recompute;
  int vec_full;
  int chunks;       // 4 or 8: the row held in registers (16-byte chunks per thread); 0: row loop
  const void* x;
  const void* dy;
  const void* gamma;
  const float* mean;
  const float* rstd;
  void* dx;
  float* mean_out;  // recompute mode: the statistics, for the weight-gradient pass
  float* rstd_out;
  int64_t M, N, ldx, ldy, ldo;
  float eps;
  int64_t grid;
  hipStream_t stream;
};

// forward for wide rows: chunks 4 or 8 holds the row in registers, 0 streams it
hipError_t launch_fl_f32(const LaunchF& f);
hipError_t launch_fl_f16(const LaunchF& f);
hipError_t launch_fl_bf16(const LaunchF& f);
hipError_t launch_l_f32(const LaunchL& l);
hipError_t launch_l_f16(const LaunchL& l);
hipError_t launch_l_bf16(const LaunchL& l);

hipError_t launch_w_f32(const LaunchW& w);
hipError_t launch_w_f16(const LaunchW& w);
hipError_t launch_w_bf16(const LaunchW& w);

hipError_t launch_a_f32(const LaunchA& a);
hipError_t launch_a_f16(const LaunchA& a);
hipError_t launch_a_bf16(const LaunchA& a);
hipError_t launch_a_tworow_f32(const LaunchA& a);
hipError_t launch_a_tworow_f16(const LaunchA& a);
hipError_t launch_a_tworow_bf16(const LaunchA& a);
hipError_t launch_a_recompute_f32(const LaunchA& a);
hipError_t launch_a_recompute_f16(const LaunchA& a);
hipError_t launch_a_recompute_bf16(const LaunchA& a);
hipError_t launch_f_f32(const LaunchF& f);
hipError_t launch_f_f16(const LaunchF& f);
hipError_t launch_f_bf16(const LaunchF& f);
hipError_t launch_f_tworow_f32(const LaunchF& f);
hipError_t launch_f_tworow_f16(const LaunchF& f);
hipError_t launch_f_tworow_bf16(const LaunchF& f);
hipError_t launch_reduce(int wgrad_dtype, const float* ws, int64_t G, int N, void* dgamma,
                         void* dbeta, int accumulate, int ws_stream, hipStream_t stream);
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);
hipError_t launch_triad(const void* a, const void* b, void* c, size_t bytes, int grid,
                        int unroll, hipStream_t stream);
hipError_t launch_triad_policy(const void* a, const void* b, void* c, uint32_t bytes, int unroll,
                               int load_policy, int store_policy, hipStream_t stream);

}  // namespace nb
