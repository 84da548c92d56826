// nb_device.hpp -- device code of the norm-backward library (gfx950, wave64).
//
// Kernel A (dx_partials_kernel): one pass over x and dy. For each row it
// recomputes xhat from the saved statistics, takes the in-row sums
// sum_j(dy*gamma) (LayerNorm only) and sum_j(dy*gamma*xhat), writes dx, and
// adds dy*xhat (and dy) into per-lane fp32 accumulators. Each workgroup owns
// whole row groups (disjoint contiguous row blocks) and stores one partial
// row per group into the workspace. This is the disjoint-block, register-
// accumulated partial scheme of "Norm backward in Triton -- the dγ/dβ
// reduction", section "2 · grouped partial buffers + a tiny reduce kernel",
// without its atomics.
//
// Kernel B (reduce_partials_kernel): column tiles of 64 features; 16 waves
// each sum a fixed contiguous slice of the groups in ascending order, then
// one wave adds the 16 slice sums in slice order and rounds to the output
// type. The order depends only on the group count.
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

namespace nb {

// ---------------------------------------------------------------- element types
struct TF32 { static constexpr int kBytes = 4; };
struct TF16 { static constexpr int kBytes = 2; };
struct TBF16 { static constexpr int kBytes = 2; };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
  __device__ __forceinline__ void load(const void* p) {
    if constexpr (kBytes == 16) {
      uint4 t = *reinterpret_cast<const uint4*>(p);
      w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
    } else if constexpr (kBytes == 8) {
      uint2 t = *reinterpret_cast<const uint2*>(p);
      w[0] = t.x; w[1] = t.y;
    } else if constexpr (kBytes == 4) {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
      w[0] = *reinterpret_cast<const uint16_t*>(p);
    }
  }
  __device__ __forceinline__ void store(void* p) const {
    if constexpr (kBytes == 16) {
      *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if constexpr (kBytes == 8) {
      *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    } else if constexpr (kBytes == 4) {
      *reinterpret_cast<uint32_t*>(p) = w[0];
    } else {
      *reinterpret_cast<uint16_t*>(p) = (uint16_t)w[0];
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

// ---------------------------------------------------------------- kernel A
template <int KIND, class Tg, int VEC, int C, int NACC>
__global__ __launch_bounds__((max_threads_for<VEC, C>()))
void dx_partials_kernel(const void* __restrict__ xv, const void* __restrict__ dyv,
                        const void* __restrict__ gv, const float* __restrict__ mean,
                        const float* __restrict__ rstd, void* __restrict__ dxv,
                        float* __restrict__ ws, int64_t M, int N, int64_t G, int64_t R,
                        int S, int P) {
  using PK = Pack<Tg, VEC>;
  constexpr int EB = Tg::kBytes;
  const char* __restrict__ x = static_cast<const char*>(xv);
  const char* __restrict__ dy = static_cast<const char*>(dyv);
  const char* __restrict__ gm = static_cast<const char*>(gv);
  char* __restrict__ dx = static_cast<char*>(dxv);

  __shared__ float red[2][kMaxWaves][2];
  extern __shared__ float comb[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = wave % S;         // slice of the row this wave covers
  const int p = wave / S;         // which of the P rows in flight
  const int cstride = S * 64 * VEC;
  const int col0 = (s * 64 + lane) * VEC;
  const float fN = (float)N;

  // gamma for this lane's columns, kept packed in registers for every row
  PK gam[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int col = col0 + c * cstride;
    if (col < N) gam[c].load(gm + (int64_t)col * EB);
    else gam[c].zero();
  }

  int phase = 0;  // parity of the row-sum exchange buffer (S > 1)
  for (int64_t g = blockIdx.x; g < G; g += gridDim.x) {
    const int64_t r0 = g * R;
    const int64_t r1 = (r0 + R < M) ? r0 + R : M;
    const int iters = (int)((r1 - r0 + P - 1) / P);

    float acc[NACC][C][VEC];
#pragma unroll
    for (int a = 0; a < NACC; ++a)
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[a][c][v] = 0.0f;

    for (int it = 0; it < iters; ++it, ++phase) {
      const int64_t r = r0 + (int64_t)it * P + p;
      const bool active = r < r1;  // uniform over the wave
      keep_packed(gam);
      PK xr[C], dr[C];
      float mu = 0.0f, rs = 0.0f;
      if (active) {
        rs = rstd[r];
        if (KIND == kLayerNorm) mu = mean[r];
        const int64_t rb = r * (int64_t)N;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int col = col0 + c * cstride;
          if (col < N) {
            xr[c].load(x + (rb + col) * EB);
            dr[c].load(dy + (rb + col) * EB);
          } else {
            xr[c].zero();
            dr[c].zero();
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < C; ++c) { xr[c].zero(); dr[c].zero(); }
      }

      // in-row sums: s1 = sum(dyhat) (LayerNorm), s2 = sum(dyhat * xhat)
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float xh = (xr[c].get(v) - mu) * rs;
          const float dyh = dr[c].get(v) * gam[c].get(v);
          if (KIND == kLayerNorm) s1 += dyh;
          s2 = __builtin_fmaf(dyh, xh, s2);
        }
      keep_packed(xr);
      keep_packed(dr);
      keep_packed(gam);
      s2 = wave_sum(s2);
      if (KIND == kLayerNorm) s1 = wave_sum(s1);
      if (S > 1) {
        const int buf = phase & 1;
        if (lane == 0) {
          red[buf][wave][0] = s1;
          red[buf][wave][1] = s2;
        }
        __syncthreads();
        float t1 = 0.0f, t2 = 0.0f;
        for (int q = 0; q < S; ++q) {
          t1 += red[buf][p * S + q][0];
          t2 += red[buf][p * S + q][1];
        }
        s1 = t1;
        s2 = t2;
      }

      if (active) {
        const float m2 = s2 / fN;
        const float m1 = (KIND == kLayerNorm) ? s1 / fN : 0.0f;
        const int64_t rb = r * (int64_t)N;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int col = col0 + c * cstride;
          if (col < N) {
            float o[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
              const float dyv_ = dr[c].get(v);
              const float xh = (xr[c].get(v) - mu) * rs;
              const float dyh = dyv_ * gam[c].get(v);
              o[v] = (dyh - m1 - xh * m2) * rs;
              acc[0][c][v] = __builtin_fmaf(dyv_, xh, acc[0][c][v]);
              if (NACC == 2) acc[NACC - 1][c][v] += dyv_;
            }
            PK out;
            out.set(o);
            out.store(dx + (rb + col) * EB);
          }
        }
      }
    }

    // Combine the P row-lanes' partials in the fixed order 0, 1, ..., P-1.
    if (P > 1) {
      for (int q = 1; q < P; ++q) {
        if (p == q) {
#pragma unroll
          for (int a = 0; a < NACC; ++a)
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
              for (int v = 0; v < VEC; ++v)
                comb[(((a * C + c) * S + s) * 64 + lane) * VEC + v] = acc[a][c][v];
        }
        __syncthreads();
        if (p == 0) {
#pragma unroll
          for (int a = 0; a < NACC; ++a)
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
              for (int v = 0; v < VEC; ++v)
                acc[a][c][v] += comb[(((a * C + c) * S + s) * 64 + lane) * VEC + v];
        }
        __syncthreads();
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
            if constexpr (VEC % 4 == 0) {
#pragma unroll
              for (int v = 0; v < VEC; v += 4)
                *reinterpret_cast<float4*>(dst + col + v) =
                    make_float4(acc[a][c][v], acc[a][c][v + 1], acc[a][c][v + 2], acc[a][c][v + 3]);
            } else {
#pragma unroll
              for (int v = 0; v < VEC; ++v) dst[col + v] = acc[a][c][v];
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

template <class OutT> __device__ __forceinline__ void store_out(void* p, int j, float v);
template <> __device__ __forceinline__ void store_out<TF32>(void* p, int j, float v) {
  static_cast<float*>(p)[j] = v;
}
template <> __device__ __forceinline__ void store_out<TF16>(void* p, int j, float v) {
  static_cast<uint16_t*>(p)[j] = pack1<TF16>(v);
}
template <> __device__ __forceinline__ void store_out<TBF16>(void* p, int j, float v) {
  static_cast<uint16_t*>(p)[j] = pack1<TBF16>(v);
}

template <class OutT>
__global__ __launch_bounds__(kReduceWaves * 64)
void reduce_partials_kernel(const float* __restrict__ ws, int64_t G, int N,
                            void* __restrict__ dgamma, void* __restrict__ dbeta) {
  __shared__ float part[kReduceWaves][kReduceCols];
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  const int plane = blockIdx.y;  // 0: dgamma partials, 1: dbeta partials
  const int col = blockIdx.x * kReduceCols + lane;
  const float* __restrict__ src = ws + (int64_t)plane * G * (int64_t)N;
  const int64_t lo = G * q / kReduceWaves;
  const int64_t hi = G * (q + 1) / kReduceWaves;
  float sum = 0.0f;
  if (col < N) {
    int64_t g = lo;
    for (; g + 8 <= hi; g += 8) {
      float t[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) t[k] = src[(g + k) * (int64_t)N + col];
#pragma unroll
      for (int k = 0; k < 8; ++k) sum += t[k];
    }
    for (; g < hi; ++g) sum += src[g * (int64_t)N + col];
  }
  part[q][lane] = sum;
  __syncthreads();
  if (q == 0 && col < N) {
    float t = part[0][lane];
#pragma unroll
    for (int k = 1; k < kReduceWaves; ++k) t += part[k][lane];
    store_out<OutT>(plane == 0 ? dgamma : dbeta, col, t);
  }
}

}  // namespace nb
