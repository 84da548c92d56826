// nb_device.hpp -- device code of the norm-backward library (gfx950, wave64).
//
// Kernel A (dx_partials_kernel): one pass over x and dy. For each row it
// recomputes xhat from the saved statistics (or, in recompute mode, first
// recomputes the statistics themselves from the row held in registers),
// takes the in-row sums sum_j(dy*gamma) (LayerNorm only) and
// sum_j(dy*gamma*xhat), writes dx, and adds dy*xhat (and dy) into per-lane
// fp32 accumulators. Rows of x, dy and dx may have their own strides. Workgroup g owns row
// group g -- the rows r with r mod G == g -- processes them in ascending
// order and stores one partial row per group into the workspace. No two
// workgroups ever write the same slot, so there are no atomics: this is the
// register-accumulated disjoint-row partial scheme of "Norm backward in
// Triton -- the dγ/dβ reduction", section "2 · grouped partial buffers + a
// tiny reduce kernel", without its atomics. Interleaving the groups (rather
// than giving each a contiguous block) makes all workgroups sweep one
// address window together, which the HBM sustains measurably better.
//
// Kernel B (reduce_partials_kernel): column tiles of 64 features; 16 waves
// each sum a fixed contiguous slice of the groups in ascending order, then
// one wave adds the 16 slice sums in slice order (and, when accumulating, the
// output's previous value) and rounds to the output type. The order depends
// only on the group count.
//
// Lane ownership inside a row (kernel A). A row of N elements is split into
// C chunks; chunk c is covered by the S waves sharing the row, wave s taking
// 64*VEC consecutive elements, lane l taking VEC consecutive elements:
//     col(c, s, l, v) = ((c*S + s)*64 + l)*VEC + v.
// Every wave load instruction therefore reads 64*VEC*sizeof(T) contiguous
// bytes (1 KiB for 16-byte vectors). VEC > 1 requires N % VEC == 0, so a
// vector is either entirely inside the row or entirely past its end; lanes
// past the end load nothing and contribute exact zeros to every sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace nb {

// ---------------------------------------------------------------- element types
struct TF32 { static constexpr int kBytes = 4; };
struct TF16 { static constexpr int kBytes = 2; };
struct TBF16 { static constexpr int kBytes = 2; };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <class Tg> __device__ __forceinline__ float lo16_to_f32(uint32_t w);
template <class Tg> __device__ __forceinline__ float hi16_to_f32(uint32_t w);
template <> __device__ __forceinline__ float lo16_to_f32<TBF16>(uint32_t w) {
  return __uint_as_float(w << 16);
}
template <> __device__ __forceinline__ float hi16_to_f32<TBF16>(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}
template <> __device__ __forceinline__ float lo16_to_f32<TF16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <> __device__ __forceinline__ float hi16_to_f32<TF16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Two fp32 values to two 16-bit values packed in one word, round to nearest
// even (gfx950 has a packed bf16 convert; fp16 uses the IEEE convert).
template <class Tg> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<TBF16>(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
template <> __device__ __forceinline__ uint32_t pack2<TF16>(float lo, float hi) {
  uint32_t a = __builtin_bit_cast(uint16_t, (_Float16)lo);
  uint32_t b = __builtin_bit_cast(uint16_t, (_Float16)hi);
  return a | (b << 16);
}
template <class Tg> __device__ __forceinline__ uint16_t pack1(float f);
template <> __device__ __forceinline__ uint16_t pack1<TBF16>(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
template <> __device__ __forceinline__ uint16_t pack1<TF16>(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Cache-policy operand of the raw buffer builtins that sets the
// non-temporal bit (the same hint __builtin_nontemporal_load gives).
constexpr int kBufNonTemporal = 2;

// A raw buffer resource over `bytes` bytes starting at p (stride 0; the
// fourth word is the 32-bit data format gfx9-family parts take for raw
// buffers). The kernels address a row through it from a scalar base and a
// 32-bit lane offset, and only where every lane's offset is inside the row
// (the hardware would read zeros and drop stores past `bytes`).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// VEC elements of type Tg held as raw bits: one aligned load / store each.
template <class Tg, int VEC>
struct Pack {
  static constexpr int kBytes = VEC * Tg::kBytes;
  static constexpr int kWords = kBytes >= 4 ? kBytes / 4 : 1;
  uint32_t w[kWords];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = 0u;
  }
  // Plain loads/stores (cached): gamma and anything read again soon.
  __device__ __forceinline__ void load(const void* p) {
    if constexpr (kBytes == 16) {
      const u32x4 t = *reinterpret_cast<const u32x4*>(p);
      w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    } else if constexpr (kBytes == 8) {
      const u32x2 t = *reinterpret_cast<const u32x2*>(p);
      w[0] = t.x; w[1] = t.y;
    } else if constexpr (kBytes == 4) {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
      w[0] = *reinterpret_cast<const uint16_t*>(p);
    }
  }
  // Streaming loads/stores for data touched exactly once (x, dy, dx): the
  // non-temporal hint keeps them from displacing reused lines in the caches.
  __device__ __forceinline__ void load_stream(const void* p) {
    if constexpr (kBytes == 16) {
      const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
      w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    } else if constexpr (kBytes == 8) {
      const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
      w[0] = t.x; w[1] = t.y;
    } else if constexpr (kBytes == 4) {
      w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    } else {
      w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
    }
  }
  __device__ __forceinline__ void store_stream(void* p) const {
    if constexpr (kBytes == 16) {
      const u32x4 t = {w[0], w[1], w[2], w[3]};
      __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(p));
    } else if constexpr (kBytes == 8) {
      const u32x2 t = {w[0], w[1]};
      __builtin_nontemporal_store(t, reinterpret_cast<u32x2*>(p));
    } else if constexpr (kBytes == 4) {
      __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(p));
    } else {
      __builtin_nontemporal_store((uint16_t)w[0], reinterpret_cast<uint16_t*>(p));
    }
  }
  // Streaming loads/stores at byte offset `off` of a row's buffer resource
  // (row_rsrc), with the same non-temporal hint as load_stream/store_stream.
  __device__ __forceinline__ void load_stream_buf(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    if constexpr (kBytes == 16) {
      const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kBufNonTemporal);
      w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    } else if constexpr (kBytes == 8) {
      const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kBufNonTemporal);
      w[0] = t.x; w[1] = t.y;
    } else if constexpr (kBytes == 4) {
      w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, kBufNonTemporal);
    } else {
      w[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, kBufNonTemporal);
    }
  }
  __device__ __forceinline__ void store_stream_buf(__amdgpu_buffer_rsrc_t rs, uint32_t off) const {
    if constexpr (kBytes == 16) {
      const u32x4 t = {w[0], w[1], w[2], w[3]};
      __builtin_amdgcn_raw_buffer_store_b128(t, rs, off, 0, kBufNonTemporal);
    } else if constexpr (kBytes == 8) {
      const u32x2 t = {w[0], w[1]};
      __builtin_amdgcn_raw_buffer_store_b64(t, rs, off, 0, kBufNonTemporal);
    } else if constexpr (kBytes == 4) {
      __builtin_amdgcn_raw_buffer_store_b32(w[0], rs, off, 0, kBufNonTemporal);
    } else {
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)w[0], rs, off, 0, kBufNonTemporal);
    }
  }
  // element v as fp32 (exact widening)
  __device__ __forceinline__ float get(int v) const {
    if constexpr (Tg::kBytes == 4) {
      return __uint_as_float(w[v]);
    } else if constexpr (kBytes == 2) {
      return lo16_to_f32<Tg>(w[0]);
    } else {
      return (v & 1) ? hi16_to_f32<Tg>(w[v >> 1]) : lo16_to_f32<Tg>(w[v >> 1]);
    }
  }
  // set from VEC fp32 values, rounding to nearest even
  __device__ __forceinline__ void set(const float (&f)[VEC]) {
    if constexpr (Tg::kBytes == 4) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) w[v] = __float_as_uint(f[v]);
    } else if constexpr (kBytes == 2) {
      w[0] = pack1<Tg>(f[0]);
    } else {
#pragma unroll
      for (int i = 0; i < kWords; ++i) w[i] = pack2<Tg>(f[2 * i], f[2 * i + 1]);
    }
  }
};

// Tell the compiler the packed words may have changed, so fp32 values it
// unpacked from them earlier cannot be kept live across this point: they are
// recomputed from the packed registers instead (one ALU op per element) and
// the register file holds the packed form only. Emits no instruction.
template <class Tg, int VEC, int C>
__device__ __forceinline__ void keep_packed(Pack<Tg, VEC> (&p)[C]) {
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int i = 0; i < Pack<Tg, VEC>::kWords; ++i) asm volatile("" : "+v"(p[c].w[i]));
}

// Same for fp32 values: they must be materialised here (so work that feeds
// them cannot be deferred past this point, keeping its inputs alive).
template <int NA, int C, int VEC>
__device__ __forceinline__ void pin(float (&a)[NA][C][VEC]) {
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int v = 0; v < VEC; ++v) asm volatile("" : "+v"(a[i][c][v]));
}

// ---------------------------------------------------------------- wave sums
// Butterfly over 16 lanes with DPP (lane^1, lane^2, mirror in 8, mirror in
// 16): afterwards every lane of a 16-lane row holds that row's sum, bitwise
// equal across the row (each step adds the same two values). The four row
// sums are then read into scalars and added as (r0 + r1) + (r2 + r3). The
// order is fixed, so the result is deterministic and uniform over the wave.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

constexpr int kLayerNorm = 0;
constexpr int kRmsNorm = 1;
constexpr int kMaxWaves = 16;

template <int VEC, int C>
constexpr int max_threads_for() { return VEC * C > 16 ? 512 : 1024; }

// Rows of x/dy held in registers per wave (a ring: D - 1 rows in flight
// while one is processed), sized by the bytes each lane holds per operand and
// the register budget the launch bound MAXT leaves (128 VGPRs at 1024
// threads, 256 at 512): up to 32 B -> 3 rows; 64 B -> 2 rows within 256
// VGPRs; otherwise 1 (no prefetch).
template <class Tg, int VEC, int C, int MAXT = max_threads_for<VEC, C>()>
constexpr int prefetch_depth() {
  constexpr int bytes = VEC * C * Tg::kBytes;
  return bytes <= 32 ? 3 : (MAXT <= 512 && bytes <= 64 ? 2 : 1);
}

// Kernel A in recompute mode also exists with a 512-thread launch bound
// (256 VGPRs) where a lane holds 32 bytes of each operand: the recompute
// plans' 512-thread workgroups then take the steady-state loop, which did not
// fit the 128 VGPRs of the 1024-thread bound (16384 x 4096 bf16 RMSNorm
// recompute step 73.8 -> 70.4 us, 65536 x 8192 LayerNorm 565 -> 551 us).
// So does the saved-statistics fp16 kernel with 16 elements per lane and
// both gradients, the one saved-statistics kernel whose steady-state loop
// spilled under the 1024-thread bound.
template <bool RECOMP, class Tg, int VEC, int C, int NACC>
constexpr bool has_narrow_bound() {
  return VEC > 1 && VEC * C * Tg::kBytes == 32 && max_threads_for<VEC, C>() == 1024 &&
         (RECOMP || (std::is_same<Tg, TF16>::value && NACC == 2));
}

// Whether kernel A pipelines the two exchanges of LayerNorm recompute across
// rows. It reads the next row from the ring, so the ring must hold two rows;
// and fp16 rows of 16 elements per lane with both gradients are left out:
// pipelined under the 1024-thread bound that kernel needed 3 registers more
// than the 128 it allows and spilled (bf16 fits, with 123); under the
// 512-thread bound it fits but ran 1% slower on 1151 x 8192.
template <class Tg, int VEC, int C, int NACC, int MAXT = max_threads_for<VEC, C>()>
constexpr bool pipeline_ln_recompute() {
  return prefetch_depth<Tg, VEC, C, MAXT>() >= 2 &&
         !(std::is_same<Tg, TF16>::value && VEC * C == 16 && NACC == 2);
}

// Whether kernel A runs its steady-state loop (every row and every lane
// chunk in bounds, so no per-lane or per-row conditions). Kernels whose row
// sits in 16-byte vectors: with saved statistics up to 32 elements per lane,
// in recompute mode one vector per operand per lane (32 bytes under the
// 512-thread bound). Left out, because the extra loop made them spill under
// their register budget: one element per lane, 64 elements per lane, fp16
// rows of 16 elements per lane with both gradients under the 1024-thread
// bound, and recompute mode with more bytes per operand.
constexpr int64_t kSteadyGroupBytes = (int64_t)2 << 20;

template <bool RECOMP, class Tg, int VEC, int C, int NACC, int MAXT = max_threads_for<VEC, C>()>
constexpr bool steady_loop() {
  return VEC > 1 && VEC * C <= 32 &&
         (!RECOMP || VEC * C * Tg::kBytes <= (MAXT <= 512 ? 32 : 16)) &&
         !(std::is_same<Tg, TF16>::value && VEC * C == 16 && NACC == 2 && MAXT == 1024);
}

// ---------------------------------------------------------------- kernel A
// Turn per-lane partial sums into row sums: the wave butterfly, then, when
// S > 1 waves share the row, an exchange through LDS in which the S wave sums
// are added in slice order 0, 1, ..., S-1 (lane q < S fetches slice q's pair
// in one LDS read; the pairs are added from scalar copies). `a` takes part
// only when USE_A. Every wave of the workgroup must make the same sequence of
// calls (the exchange holds a barrier); `phase` alternates the two LDS
// buffers so that one barrier per call suffices.
template <bool USE_A>
__device__ __forceinline__ void row_sum2(float& a, float& b, float (*red)[kMaxWaves][2],
                                         int& phase, int lane, int wave, int S, int p) {
  b = wave_sum(b);
  if (USE_A) a = wave_sum(a);
  if (S > 1) {
    const int buf = phase & 1;
    if (lane == 0) {
      red[buf][wave][0] = a;
      red[buf][wave][1] = b;
    }
    __syncthreads();
    float2 mine = make_float2(0.0f, 0.0f);
    if (lane < S) mine = *reinterpret_cast<const float2*>(&red[buf][p * S + lane][0]);
    const int ab = __builtin_bit_cast(int, mine.x), bb = __builtin_bit_cast(int, mine.y);
    float ta = 0.0f, tb = 0.0f;
    for (int q = 0; q < S; ++q) {
      ta += __builtin_bit_cast(float, __builtin_amdgcn_readlane(ab, q));
      tb += __builtin_bit_cast(float, __builtin_amdgcn_readlane(bb, q));
    }
    a = ta;
    b = tb;
  }
  ++phase;
}

// Four row sums in one exchange (pipelined LayerNorm recompute: one row's
// second pair of sums travels with the next row's first pair). Each sum is
// formed exactly as row_sum2 forms it: the wave butterfly, then the S slice
// sums added in slice order. Same calling rules as row_sum2, with its own
// double buffer.
__device__ __forceinline__ void row_sum4(float& a, float& b, float& c, float& d,
                                         float (*red4)[kMaxWaves][4], int& phase, int lane,
                                         int wave, int S, int p) {
  a = wave_sum(a);
  b = wave_sum(b);
  c = wave_sum(c);
  d = wave_sum(d);
  if (S > 1) {
    const int buf = phase & 1;
    if (lane == 0) {
      red4[buf][wave][0] = a;
      red4[buf][wave][1] = b;
      red4[buf][wave][2] = c;
      red4[buf][wave][3] = d;
    }
    __syncthreads();
    float4 mine = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (lane < S) mine = *reinterpret_cast<const float4*>(&red4[buf][p * S + lane][0]);
    const int ab = __builtin_bit_cast(int, mine.x), bb = __builtin_bit_cast(int, mine.y);
    const int cb = __builtin_bit_cast(int, mine.z), db = __builtin_bit_cast(int, mine.w);
    float ta = 0.0f, tb = 0.0f, tc = 0.0f, td = 0.0f;
    for (int q = 0; q < S; ++q) {
      ta += __builtin_bit_cast(float, __builtin_amdgcn_readlane(ab, q));
      tb += __builtin_bit_cast(float, __builtin_amdgcn_readlane(bb, q));
      tc += __builtin_bit_cast(float, __builtin_amdgcn_readlane(cb, q));
      td += __builtin_bit_cast(float, __builtin_amdgcn_readlane(db, q));
    }
    a = ta;
    b = tb;
    c = tc;
    d = td;
  }
  ++phase;
}

// A zero the compiler cannot see through (it lives in a vector register).
// Adding it to the index of a per-row statistic keeps that load on the vector
// memory path, in issue order with the row's x/dy loads. A scalar load there
// would be worse: scalar loads return out of order, so every use of one waits
// for all scalar loads in flight -- including those issued for the rows being
// prefetched -- and every LDS wait before a barrier would wait for them too.
__device__ __forceinline__ int opaque_lane_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// One row's operands as they come from memory, plus its saved statistics.
template <class Tg, int VEC, int C>
struct RowBuf {
  Pack<Tg, VEC> x[C], dy[C];
  float mu, rs;
};

// Issue the loads of row r into b. Nothing is loaded for an inactive row
// (RALL: every row is active) or for a lane's chunks past the row's end;
// process_row never reads those registers (it skips exactly the same cases).
// CALL: the lanes cover the row exactly, so no chunk is past the end and the
// loads go through the row's buffer resource (a scalar base and a 32-bit
// lane offset: fewer vector registers and address instructions than 64-bit
// lane addresses; 16384 x 4096 bf16 RMSNorm step 68.8 -> 68.0 us). With
// RECOMP the statistics are not loaded: process_row computes them from x.
template <int KIND, bool RECOMP, bool RALL, bool CALL, class Tg, int VEC, int C>
__device__ __forceinline__ void fetch_row(RowBuf<Tg, VEC, C>& b, const char* __restrict__ x,
                                          const char* __restrict__ dy,
                                          const float* __restrict__ mean,
                                          const float* __restrict__ rstd, int64_t r, bool active,
                                          int N, int64_t ldx, int64_t ldy, int col0,
                                          int cstride) {
  constexpr int EB = Tg::kBytes;
  if (RALL || active) {
    if constexpr (!RECOMP) {
      const int64_t rz = r + opaque_lane_zero();
      b.rs = rstd[rz];
      b.mu = (KIND == kLayerNorm) ? mean[rz] : 0.0f;
    }
    if constexpr (CALL) {
      const uint32_t row_bytes = (uint32_t)N * EB;
      const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + r * ldx * EB, row_bytes);
      const __amdgpu_buffer_rsrc_t ry = row_rsrc(dy + r * ldy * EB, row_bytes);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const uint32_t off = (uint32_t)(col0 + c * cstride) * EB;
        b.x[c].load_stream_buf(rx, off);
        b.dy[c].load_stream_buf(ry, off);
      }
    } else {
      const int64_t xb = r * ldx, yb = r * ldy;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int col = col0 + c * cstride;
        if (col < N) {
          b.x[c].load_stream(x + (xb + col) * EB);
          b.dy[c].load_stream(dy + (yb + col) * EB);
        }
      }
    }
  }
}

// Everything kernel A does with one row once its operands are in registers.
// With xc = x - mean (RMSNorm: xc = x), xhat = xc * rstd and dyhat = dy * gamma:
//   pass 1: s1 = sum_j dyhat (LayerNorm only), s2 = sum_j dyhat * xc, and the
//           row's weight-gradient terms dy * xhat = (dy * xc) * rstd and dy go
//           into the lane's accumulators (an inactive row holds zeros and
//           adds exact zeros);
//   the sums are completed across the wave (butterfly) and across the S
//   waves of the row (LDS), then
//   pass 2: dx = rstd * (dyhat - mean(dyhat) - xhat * mean(dyhat * xhat))
//              = dyhat * rstd + xc * c2 + c1,
//           with the per-row constants mean(dyhat * xhat) = rstd * s2 / N,
//           c2 = -rstd^2 * mean(dyhat * xhat) and c1 = -rstd * s1 / N.
// With RECOMP the statistics are recomputed from the row in registers, as
// the forward computes them: LayerNorm first sums x (with s1 = sum dyhat in
// the same exchange), then with mean = sum(x)/N sums xc^2 and dyhat * xc;
// RMSNorm sums x^2 and dyhat * x in one exchange. rstd = 1/sqrt(sum(xc^2)/N
// + eps). The dgamma terms, which need rstd, are accumulated in pass 2.
// LayerNorm recompute, first pass over a row held in registers: sum(x) and
// sum(dy * gamma), and the row's dbeta terms into the accumulators.
template <bool RALL = false, bool CALL = false, class Tg, int VEC, int C, int NACC>
__device__ __forceinline__ void ln_recompute_sums1(const RowBuf<Tg, VEC, C>& b,
                                                   const float (&gam)[C][VEC],
                                                   float (&acc)[NACC][C][VEC], bool active,
                                                   int N, int col0, int cstride, float& sx,
                                                   float& s1) {
  sx = 0.0f;
  s1 = 0.0f;
  if (RALL || active) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (CALL || col0 + c * cstride < N) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float dyv = b.dy[c].get(v);
          sx += b.x[c].get(v);
          s1 = __builtin_fmaf(dyv, gam[c][v], s1);
          if (NACC == 2) acc[NACC - 1][c][v] += dyv;
        }
      }
    }
  }
}

// Recompute, second pass: sum(xc^2) and sum(dyhat * xc) with xc = x - mean
// (RMSNorm: mean 0, and its dbeta terms here, as it has no first pass).
template <int KIND, bool RALL = false, bool CALL = false, class Tg, int VEC, int C, int NACC>
__device__ __forceinline__ void recompute_sums2(const RowBuf<Tg, VEC, C>& b,
                                                const float (&gam)[C][VEC],
                                                float (&acc)[NACC][C][VEC], bool active, int N,
                                                int col0, int cstride, float mu, float& sxx,
                                                float& s2) {
  sxx = 0.0f;
  s2 = 0.0f;
  if (RALL || active) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (CALL || col0 + c * cstride < N) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float xc = b.x[c].get(v) - mu;
          const float dyv = b.dy[c].get(v);
          sxx = __builtin_fmaf(xc, xc, sxx);
          s2 = __builtin_fmaf(dyv * gam[c][v], xc, s2);
          if (KIND != kLayerNorm && NACC == 2) acc[NACC - 1][c][v] += dyv;
        }
      }
    }
  }
}

// dx of one row from its statistics and row sums:
//   dx = dyhat * rstd + xc * c2 + c1, c2 = -rstd^2 * mean(dyhat * xhat),
//   c1 = -rstd * s1 / N (LayerNorm), and in recompute mode the row's dgamma
// terms, which need rstd.
// CALL: as in fetch_row (the stores go through the row's buffer resource).
template <int KIND, bool RECOMP, bool RALL = false, bool CALL = false, class Tg, int VEC, int C,
          int NACC>
__device__ __forceinline__ void write_dx(const RowBuf<Tg, VEC, C>& b, const float (&gam)[C][VEC],
                                         float (&acc)[NACC][C][VEC], char* __restrict__ dx,
                                         int64_t r, bool active, int N, int64_t ldo, float inv_n,
                                         float mu, float rs, float s1, float s2, int col0,
                                         int cstride) {
  constexpr int EB = Tg::kBytes;
  if (RALL || active) {
    const float m2 = s2 * inv_n * rs;  // mean_j(dyhat * xhat)
    const float c2 = -(rs * rs) * m2;
    const float c1 = (KIND == kLayerNorm) ? -rs * (s1 * inv_n) : 0.0f;
    const int64_t rb = r * ldo;
    const __amdgpu_buffer_rsrc_t ro = row_rsrc(dx + rb * EB, (uint32_t)N * EB);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int col = col0 + c * cstride;
      if (CALL || col < N) {
        float o[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float xc = b.x[c].get(v) - mu;
          const float dyh = b.dy[c].get(v) * gam[c][v];
          o[v] = __builtin_fmaf(dyh, rs, __builtin_fmaf(xc, c2, c1));
          // recompute mode: the dgamma term, now that rstd is known
          if constexpr (RECOMP)
            acc[0][c][v] = __builtin_fmaf(b.dy[c].get(v) * xc, rs, acc[0][c][v]);
        }
        Pack<Tg, VEC> out;
        out.set(o);
        if constexpr (CALL) out.store_stream_buf(ro, (uint32_t)col * EB);
        else out.store_stream(dx + (rb + col) * EB);
      }
    }
  }
}

template <int KIND, bool RECOMP, bool RALL = false, bool CALL = false, class Tg, int VEC, int C,
          int NACC>
__device__ __forceinline__ void process_row(RowBuf<Tg, VEC, C>& b, const float (&gam)[C][VEC],
                                            float (&acc)[NACC][C][VEC], char* __restrict__ dx,
                                            float (*red)[kMaxWaves][2], int& phase, int64_t r,
                                            bool active, int N, int64_t ldo, float inv_n, float eps,
                                            int col0, int cstride, int lane, int wave, int S,
                                            int p) {
  float s1 = 0.0f, s2 = 0.0f;
  float mu, rs;
  if constexpr (!RECOMP) {
    mu = b.mu;
    rs = b.rs;
    if (RALL || active) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if (CALL || col0 + c * cstride < N) {
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            const float xc = b.x[c].get(v) - mu;
            const float dyv = b.dy[c].get(v);
            const float dyh = dyv * gam[c][v];
            if (KIND == kLayerNorm) s1 = __builtin_fmaf(dyv, gam[c][v], s1);
            s2 = __builtin_fmaf(dyh, xc, s2);
            acc[0][c][v] = __builtin_fmaf(dyv * xc, rs, acc[0][c][v]);
            if (NACC == 2) acc[NACC - 1][c][v] += dyv;
          }
        }
      }
    }
    pin(acc);
    keep_packed(b.x);
    keep_packed(b.dy);
    row_sum2<KIND == kLayerNorm>(s1, s2, red, phase, lane, wave, S, p);
  } else {
    mu = 0.0f;
    if constexpr (KIND == kLayerNorm) {
      float sx;
      ln_recompute_sums1<RALL, CALL>(b, gam, acc, active, N, col0, cstride, sx, s1);
      keep_packed(b.x);
      keep_packed(b.dy);
      row_sum2<true>(sx, s1, red, phase, lane, wave, S, p);
      mu = sx * inv_n;
    }
    float sxx;
    recompute_sums2<KIND, RALL, CALL>(b, gam, acc, active, N, col0, cstride, mu, sxx, s2);
    keep_packed(b.x);
    keep_packed(b.dy);
    row_sum2<true>(sxx, s2, red, phase, lane, wave, S, p);
    rs = 1.0f / __builtin_sqrtf(__builtin_fmaf(sxx, inv_n, eps));
  }
  write_dx<KIND, RECOMP, RALL, CALL>(b, gam, acc, dx, r, active, N, ldo, inv_n, mu, rs, s1, s2,
                                     col0, cstride);
}

// WSNT: the partial rows are stored non-temporally (chosen for large
// workspaces by the planner's stream_workspace); the values are the same.
// MAXT: the launch bound (max_threads_for, or 512 where has_narrow_bound).
template <int KIND, bool RECOMP, class Tg, int VEC, int C, int NACC, bool WSNT,
          int MAXT = max_threads_for<VEC, C>()>
__global__ __launch_bounds__(MAXT)
void dx_partials_kernel(const void* __restrict__ xv, const void* __restrict__ dyv,
                        const void* __restrict__ gv, const float* __restrict__ mean,
                        const float* __restrict__ rstd, void* __restrict__ dxv,
                        float* __restrict__ ws, int64_t M, int N, int64_t ldx, int64_t ldy,
                        int64_t ldo, int64_t G, int64_t R, int S, int P, float eps) {
  using PK = Pack<Tg, VEC>;
  using RB = RowBuf<Tg, VEC, C>;
  constexpr int EB = Tg::kBytes;
  const char* __restrict__ x = static_cast<const char*>(xv);
  const char* __restrict__ dy = static_cast<const char*>(dyv);
  const char* __restrict__ gm = static_cast<const char*>(gv);
  char* __restrict__ dx = static_cast<char*>(dxv);

  __shared__ __align__(8) float red[2][kMaxWaves][2];
  extern __shared__ float comb[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = wave % S;         // slice of the row this wave covers
  const int p = wave / S;         // which of the P rows in flight
  const int cstride = S * 64 * VEC;
  const int col0 = (s * 64 + lane) * VEC;
  const float inv_n = 1.0f / (float)N;

  // gamma for this lane's columns, widened to fp32 once and kept in registers
  float gam[C][VEC];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int col = col0 + c * cstride;
    PK t;
    if (col < N) t.load(gm + (int64_t)col * EB);
    else t.zero();
#pragma unroll
    for (int v = 0; v < VEC; ++v) gam[c][v] = t.get(v);
  }

  int phase = 0;  // parity of the row-sum exchange buffer (S > 1)
  for (int64_t g = blockIdx.x; g < G; g += gridDim.x) {
    // group g holds rows g, g + G, g + 2G, ...; row-lane p of the workgroup
    // takes every P-th of them, so iteration k of row-lane p is row
    // g + (k*P + p)*G. Every wave runs the same number of iterations.
    const int64_t rows = (M - g + G - 1) / G;
    const int iters = (int)((rows + P - 1) / P);
    auto row_of = [&](int k) { return g + ((int64_t)k * P + p) * G; };

    float acc[NACC][C][VEC];
#pragma unroll
    for (int a = 0; a < NACC; ++a)
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[a][c][v] = 0.0f;

    // Ring of D row buffers: the loads of row k + D - 1 are issued before
    // row k is processed, so each wave keeps D - 1 rows of x and dy in flight
    // while it computes.
    constexpr int D = prefetch_depth<Tg, VEC, C, MAXT>();
    RB buf[D];
    // Steady state: when the lanes cover the row exactly and the group has
    // enough iterations in which every row-lane has a row, those iterations
    // run through a loop with no per-lane or per-row conditions. Every load
    // and store then issues on every path, so the compiler can wait for
    // exactly the row it needs (vmcnt counts the loads issued since) instead
    // of draining all loads in flight. The general loop below takes the
    // iterations that remain, from the same ring state. (Rows that the lanes
    // do not cover exactly were slower through buffer resources with
    // range-checked lanes: 262144 x 768 bf16 RMSNorm 218.6 -> 231.6 us.)
    const int kfull = (int)(rows / P);  // iterations whose P rows all exist
    int it0 = 0;
    constexpr bool kPipelined =
        RECOMP && KIND == kLayerNorm && pipeline_ln_recompute<Tg, VEC, C, NACC, MAXT>();
    // Groups that sweep more than kSteadyGroupBytes of each operand keep the
    // general loop: there the steady-state loop lost 1.3-2% (65536 x 8192
    // bf16 LayerNorm, 4 MiB per group), while at 2 MiB it was even
    // (32768 x 8192) and up to 1 MiB it gained 2.5-5%. The planner gives
    // such groups two rows in flight (the planner's copy of this bound must
    // stay equal to it).
    const bool steady = steady_loop<RECOMP, Tg, VEC, C, NACC, MAXT>() && N == C * cstride &&
                        kfull >= 2 * D - 1 && rows * (int64_t)N * EB <= kSteadyGroupBytes;
    if (steady) {
#pragma unroll
      for (int k = 0; k < D - 1; ++k)
        fetch_row<KIND, RECOMP, true, true>(buf[k], x, dy, mean, rstd, row_of(k), true, N, ldx,
                                            ldy, col0, cstride);
      // (the pipelined LayerNorm recompute loop runs its own steady state)
      if constexpr (steady_loop<RECOMP, Tg, VEC, C, NACC, MAXT>() && !kPipelined) {
        for (; it0 + 2 * D - 2 < kfull; it0 += D) {
#pragma unroll
          for (int d = 0; d < D; ++d) {
            const int k = it0 + d;
            fetch_row<KIND, RECOMP, true, true>(buf[(d + D - 1) % D], x, dy, mean, rstd,
                                                row_of(k + D - 1), true, N, ldx, ldy, col0,
                                                cstride);
            process_row<KIND, RECOMP, true, true>(buf[d], gam, acc, dx, red, phase, row_of(k),
                                                  true, N, ldo, inv_n, eps, col0, cstride, lane,
                                                  wave, S, p);
          }
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < D - 1; ++k) {
        if (k < iters) {
          const int64_t rk = row_of(k);
          fetch_row<KIND, RECOMP, false, false>(buf[k], x, dy, mean, rstd, rk, rk < M, N, ldx,
                                                ldy, col0, cstride);
        }
      }
    }
    if constexpr (kPipelined) {
      // LayerNorm recompute needs two exchanges per row (sum x, then the
      // squared deviations from the mean). Pipelined across rows, step k
      // exchanges row k's second pair of sums together with row k + 1's
      // first pair (read from the ring, where row k + 1 already is), so a
      // row costs one barrier. Every sum keeps its own order, and each
      // accumulator still takes the rows in ascending order, so the results
      // are those of process_row.
      __shared__ __align__(16) float red4[2][kMaxWaves][4];
      float mu = 0.0f, s1 = 0.0f;
      if (iters > 0) {
        float sx;
        const int64_t r0 = row_of(0);
        ln_recompute_sums1(buf[0], gam, acc, r0 < M, N, col0, cstride, sx, s1);
        keep_packed(buf[0].x);
        keep_packed(buf[0].dy);
        row_sum2<true>(sx, s1, red, phase, lane, wave, S, p);
        mu = sx * inv_n;
      }
      // Step k: row k's second pair of sums and row k + 1's first pair in
      // one exchange, then row k's dx. `rall`, `call`: as in the
      // steady-state loop.
      auto step = [&](auto rall, auto call, int d, int k) {
        constexpr bool RALL = decltype(rall)::value;
        constexpr bool CALL = decltype(call)::value;
        RB& b = buf[d];
        const int64_t rk = row_of(k);
        float sxx, s2, sx_next = 0.0f, s1_next = 0.0f;
        recompute_sums2<KIND, RALL, CALL>(b, gam, acc, rk < M, N, col0, cstride, mu, sxx, s2);
        if (RALL || k + 1 < iters) {
          RB& nx = buf[(d + 1) % D];
          ln_recompute_sums1<RALL, CALL>(nx, gam, acc, row_of(k + 1) < M, N, col0, cstride,
                                         sx_next, s1_next);
          keep_packed(nx.x);
          keep_packed(nx.dy);
        }
        keep_packed(b.x);
        keep_packed(b.dy);
        row_sum4(sxx, s2, sx_next, s1_next, red4, phase, lane, wave, S, p);
        const float rs = 1.0f / __builtin_sqrtf(__builtin_fmaf(sxx, inv_n, eps));
        write_dx<KIND, RECOMP, RALL, CALL>(b, gam, acc, dx, rk, rk < M, N, ldo, inv_n, mu, rs, s1,
                                           s2, col0, cstride);
        mu = sx_next * inv_n;
        s1 = s1_next;
      };
      if constexpr (steady_loop<RECOMP, Tg, VEC, C, NACC, MAXT>()) {
        if (steady) {
          for (; it0 + 2 * D - 2 < kfull; it0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
              const int k = it0 + d;
              fetch_row<KIND, RECOMP, true, true>(buf[(d + D - 1) % D], x, dy, mean, rstd,
                                                  row_of(k + D - 1), true, N, ldx, ldy, col0,
                                                  cstride);
              step(std::true_type(), std::true_type(), d, k);
            }
          }
        }
      }
      for (int it = it0; it < iters; it += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const int k = it + d;
          if (k + D - 1 < iters) {
            const int64_t rf = row_of(k + D - 1);
            fetch_row<KIND, RECOMP, false, false>(buf[(d + D - 1) % D], x, dy, mean, rstd, rf,
                                                  rf < M, N, ldx, ldy, col0, cstride);
          }
          if (k < iters) step(std::false_type(), std::false_type(), d, k);
        }
      }
    } else {
      for (int it = it0; it < iters; it += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const int k = it + d;
          if (k + D - 1 < iters) {
            const int64_t rf = row_of(k + D - 1);
            fetch_row<KIND, RECOMP, false, false>(buf[(d + D - 1) % D], x, dy, mean, rstd, rf,
                                                  rf < M, N, ldx, ldy, col0, cstride);
          }
          if (k < iters) {
            const int64_t rk = row_of(k);
            process_row<KIND, RECOMP>(buf[d], gam, acc, dx, red, phase, rk, rk < M, N, ldo,
                                      inv_n, eps, col0, cstride, lane, wave, S, p);
          }
        }
      }
    }

    // Combine the P row-lanes' partials in the fixed order 0, 1, ..., P-1,
    // one accumulator (dgamma, then dbeta) at a time through one plane of
    // S * C * 64 * VEC floats: half the LDS of exchanging both at once, so
    // LayerNorm rows of 8192 bf16 with both gradients (8 waves a row) can run
    // two rows in flight within 64 KiB.
    if (P > 1) {
#pragma unroll
      for (int a = 0; a < NACC; ++a) {
        for (int q = 1; q < P; ++q) {
          if (p == q) {
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
              for (int v = 0; v < VEC; ++v)
                comb[((c * S + s) * 64 + lane) * VEC + v] = acc[a][c][v];
          }
          __syncthreads();
          if (p == 0) {
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
              for (int v = 0; v < VEC; ++v)
                acc[a][c][v] += comb[((c * S + s) * 64 + lane) * VEC + v];
          }
          __syncthreads();
        }
      }
    }
    if (p == 0) {
#pragma unroll
      for (int a = 0; a < NACC; ++a) {
        float* __restrict__ dst = ws + ((int64_t)a * G + g) * (int64_t)N;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int col = col0 + c * cstride;
          if (col < N) {
            // WSNT: non-temporal stores (large workspaces, see the planner's
            // stream_workspace)
            if constexpr (VEC % 4 == 0) {
#pragma unroll
              for (int v = 0; v < VEC; v += 4) {
                const f32x4 t = {acc[a][c][v], acc[a][c][v + 1], acc[a][c][v + 2],
                                 acc[a][c][v + 3]};
                f32x4* q = reinterpret_cast<f32x4*>(dst + col + v);
                if constexpr (WSNT) __builtin_nontemporal_store(t, q);
                else *q = t;
              }
            } else {
#pragma unroll
              for (int v = 0; v < VEC; ++v) {
                if constexpr (WSNT) __builtin_nontemporal_store(acc[a][c][v], dst + col + v);
                else dst[col + v] = acc[a][c][v];
              }
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- kernel B
constexpr int kReduceWaves = 16;
constexpr int kReduceCols = 64;
constexpr int kReduceUnroll = 8;

template <class OutT> __device__ __forceinline__ void store_out(void* p, int64_t j, float v);
template <> __device__ __forceinline__ void store_out<TF32>(void* p, int64_t j, float v) {
  static_cast<float*>(p)[j] = v;
}
template <> __device__ __forceinline__ void store_out<TF16>(void* p, int64_t j, float v) {
  static_cast<uint16_t*>(p)[j] = pack1<TF16>(v);
}
template <> __device__ __forceinline__ void store_out<TBF16>(void* p, int64_t j, float v) {
  static_cast<uint16_t*>(p)[j] = pack1<TBF16>(v);
}
template <class OutT> __device__ __forceinline__ float load_out(const void* p, int64_t j) {
  if constexpr (OutT::kBytes == 4) {
    return static_cast<const float*>(p)[j];
  } else {
    Pack<OutT, 1> t;
    t.load(static_cast<const char*>(p) + j * 2);
    return t.get(0);
  }
}

// Sum of partial rows [lo, hi) of column `col` in ascending order, NT loads
// in batches of kReduceUnroll (non-temporal loads when NT).
template <bool NT>
__device__ __forceinline__ float sum_groups(const float* __restrict__ src, int64_t lo,
                                            int64_t hi, int N, int col) {
  auto ld = [&](int64_t g) {
    const float* p = src + g * (int64_t)N + col;
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
  };
  float sum = 0.0f;
  int64_t g = lo;
  for (; g + kReduceUnroll <= hi; g += kReduceUnroll) {
    float t[kReduceUnroll];
#pragma unroll
    for (int k = 0; k < kReduceUnroll; ++k) t[k] = ld(g + k);
#pragma unroll
    for (int k = 0; k < kReduceUnroll; ++k) sum += t[k];
  }
  for (; g < hi; ++g) sum += ld(g);
  return sum;
}

// Lane = feature (each wave load reads 256 contiguous bytes of one partial
// row); wave q sums groups [q*G/16, (q+1)*G/16) in ascending order, issuing
// kReduceUnroll loads before adding them in order; wave 0 then adds the 16
// slice sums in slice order. With `accumulate` the output's previous value is
// added to that sum (old + sum, one rounding to the output type). ws_stream
// selects non-temporal loads; the sums are the same either way.
template <class OutT>
__global__ __launch_bounds__(kReduceWaves * 64)
void reduce_partials_kernel(const float* __restrict__ ws, int64_t G, int N,
                            void* __restrict__ dgamma, void* __restrict__ dbeta,
                            int accumulate, int ws_stream) {
  __shared__ float part[kReduceWaves][kReduceCols];
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  const int plane = blockIdx.y;  // 0: dgamma partials, 1: dbeta partials
  const int col = blockIdx.x * kReduceCols + lane;
  const float* __restrict__ src = ws + (int64_t)plane * G * (int64_t)N;
  const int64_t lo = G * q / kReduceWaves;
  const int64_t hi = G * (q + 1) / kReduceWaves;
  float sum = 0.0f;
  if (col < N)
    sum = ws_stream ? sum_groups<true>(src, lo, hi, N, col) : sum_groups<false>(src, lo, hi, N, col);
  part[q][lane] = sum;
  __syncthreads();
  if (q == 0 && col < N) {
    float t = part[0][lane];
#pragma unroll
    for (int k = 1; k < kReduceWaves; ++k) t += part[k][lane];
    void* out = plane == 0 ? dgamma : dbeta;
    if (accumulate) t = load_out<OutT>(out, col) + t;
    store_out<OutT>(out, col, t);
  }
}

}  // namespace nb
