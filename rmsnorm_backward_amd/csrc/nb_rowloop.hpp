// nb_rowloop.hpp -- dx for rows too wide to hold in registers (gfx950).
//
// The fused kernel A keeps a whole row of x and dy in registers, which bounds
// N (16384 to 32768 elements). Wider rows take this kernel: one workgroup of
// 16 waves per row (rows strided over the grid) streams the row in chunks of
// 1024 * VEC elements, once to form the row sums and once more to write dx
// ("Norm backward in Triton", "The gradients"):
//   s1 = sum_j dyhat (LayerNorm), s2 = sum_j dyhat * xc,
//   dx = dyhat * rstd + xc * c2 + c1,  c2 = -rstd^3 * s2 / N, c1 = -rstd * s1 / N
// In recompute mode the statistics come first, computed as the forward does
// (LayerNorm: mean, then the sum of squared deviations; RMSNorm: sum x^2 with
// s2 in the same pass), and are stored for the weight-gradient pass. The
// weight gradients come from the column walk, not from this kernel. Sums over
// the 16 waves are added in wave order, so the results are reproducible.
#pragma once

#include "nb_device.hpp"

namespace nb {

constexpr int kRowWaves = 16;
constexpr int kRowUnroll = 4;

// Three sums over the workgroup: wave butterflies, then the 16 wave sums in
// wave order (read by every lane from LDS). Uniform results. Every wave must
// make the same calls; `phase` alternates the two buffers so one barrier per
// call suffices.
__device__ __forceinline__ void block_sum3(float& a, float& b, float& c,
                                           float (*buf)[kRowWaves][4], int& phase, int lane,
                                           int wave) {
  a = wave_sum(a);
  b = wave_sum(b);
  c = wave_sum(c);
  const int k = phase & 1;
  if (lane == 0) {
    buf[k][wave][0] = a;
    buf[k][wave][1] = b;
    buf[k][wave][2] = c;
  }
  __syncthreads();
  float ta = 0.0f, tb = 0.0f, tc = 0.0f;
  for (int w = 0; w < kRowWaves; ++w) {
    ta += buf[k][w][0];
    tb += buf[k][w][1];
    tc += buf[k][w][2];
  }
  a = ta;
  b = tb;
  c = tc;
  ++phase;
}

template <int KIND, bool RECOMP, class Tg, int VEC>
__global__ __launch_bounds__(kRowWaves * 64)
void dx_rowloop_kernel(const void* __restrict__ xv, const void* __restrict__ dyv,
                       const void* __restrict__ gv, const float* __restrict__ mean,
                       const float* __restrict__ rstd, void* __restrict__ dxv,
                       float* __restrict__ mean_out, float* __restrict__ rstd_out, int64_t M,
                       int64_t N, int64_t ldx, int64_t ldy, int64_t ldo, float eps) {
  using PK = Pack<Tg, VEC>;
  constexpr int EB = Tg::kBytes;
  constexpr int64_t kStep = (int64_t)kRowWaves * 64 * VEC;  // elements per sweep
  const char* __restrict__ xs = static_cast<const char*>(xv);
  const char* __restrict__ ys = static_cast<const char*>(dyv);
  const char* __restrict__ gs = static_cast<const char*>(gv);
  char* __restrict__ dxs = static_cast<char*>(dxv);
  __shared__ float buf[2][kRowWaves][4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)threadIdx.x * VEC;
  const float inv_n = 1.0f / (float)N;
  int phase = 0;

  // Visit this thread's chunks of the row, kRowUnroll loads in flight: f gets
  // the chunk's x, dy and gamma packs (chunks past N are skipped).
  auto sweep = [&](int64_t r, auto&& f) {
    const char* xr = xs + r * ldx * EB;
    const char* yr = ys + r * ldy * EB;
    for (int64_t base = c0; base < N; base += kStep * kRowUnroll) {
      PK xb[kRowUnroll], yb[kRowUnroll], gb[kRowUnroll];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int64_t col = base + u * kStep;
        if (col < N) {
          xb[u].load(xr + col * EB);
          yb[u].load(yr + col * EB);
          gb[u].load(gs + col * EB);
        }
      }
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int64_t col = base + u * kStep;
        if (col < N) f(col, xb[u], yb[u], gb[u]);
      }
    }
  };

  for (int64_t r = blockIdx.x; r < M; r += gridDim.x) {
    float mu = 0.0f, rs, s1 = 0.0f, s2 = 0.0f, unused = 0.0f;
    if constexpr (!RECOMP) {
      mu = (KIND == kLayerNorm) ? mean[r] : 0.0f;
      rs = rstd[r];
      sweep(r, [&](int64_t, const PK& x, const PK& y, const PK& g) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float dyh = y.get(v) * g.get(v);
          if (KIND == kLayerNorm) s1 = __builtin_fmaf(y.get(v), g.get(v), s1);
          s2 = __builtin_fmaf(dyh, x.get(v) - mu, s2);
        }
      });
      block_sum3(s1, s2, unused, buf, phase, lane, wave);
    } else {
      if constexpr (KIND == kLayerNorm) {
        float sx = 0.0f, u1 = 0.0f;
        sweep(r, [&](int64_t, const PK& x, const PK&, const PK&) {
#pragma unroll
          for (int v = 0; v < VEC; ++v) sx += x.get(v);
        });
        block_sum3(sx, u1, unused, buf, phase, lane, wave);
        mu = sx * inv_n;
      }
      float sxx = 0.0f;
      sweep(r, [&](int64_t, const PK& x, const PK& y, const PK& g) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float xc = x.get(v) - mu;
          const float dyh = y.get(v) * g.get(v);
          sxx = __builtin_fmaf(xc, xc, sxx);
          if (KIND == kLayerNorm) s1 = __builtin_fmaf(y.get(v), g.get(v), s1);
          s2 = __builtin_fmaf(dyh, xc, s2);
        }
      });
      block_sum3(sxx, s1, s2, buf, phase, lane, wave);
      rs = 1.0f / __builtin_sqrtf(__builtin_fmaf(sxx, inv_n, eps));
      if (threadIdx.x == 0) {
        if (KIND == kLayerNorm) mean_out[r] = mu;
        rstd_out[r] = rs;
      }
    }
    const float m2 = s2 * inv_n * rs;
    const float c2 = -(rs * rs) * m2;
    const float c1 = (KIND == kLayerNorm) ? -rs * (s1 * inv_n) : 0.0f;
    char* dr = dxs + r * ldo * EB;
    sweep(r, [&](int64_t col, const PK& x, const PK& y, const PK& g) {
      float o[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v)
        o[v] = __builtin_fmaf(y.get(v) * g.get(v), rs, __builtin_fmaf(x.get(v) - mu, c2, c1));
      PK out;
      out.set(o);
      out.store_stream(dr + col * EB);
    });
  }
}

// The forward for rows too wide for norm_fwd_kernel: LayerNorm sums x, then
// the squared deviations from the mean, then writes y = gamma * xhat + beta;
// RMSNorm sums x^2, then writes y. Each pass streams the row in chunks; the
// statistics are stored by one thread ("05: Layer norm", the Phobos
// tutorial's forward, which also walks the row in chunks three times).
template <int KIND, class Tg, int VEC, bool BETA>
__global__ __launch_bounds__(kRowWaves * 64)
void fwd_rowloop_kernel(const void* __restrict__ xv, const void* __restrict__ gv,
                        const void* __restrict__ bv, void* __restrict__ yv,
                        float* __restrict__ mean_out, float* __restrict__ rstd_out, int64_t M,
                        int64_t N, float eps) {
  using PK = Pack<Tg, VEC>;
  constexpr int EB = Tg::kBytes;
  constexpr int64_t kStep = (int64_t)kRowWaves * 64 * VEC;
  const char* __restrict__ xs = static_cast<const char*>(xv);
  const char* __restrict__ gs = static_cast<const char*>(gv);
  const char* __restrict__ bs = static_cast<const char*>(bv);
  char* __restrict__ ys = static_cast<char*>(yv);
  __shared__ float buf[2][kRowWaves][4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)threadIdx.x * VEC;
  const float inv_n = 1.0f / (float)N;
  int phase = 0;

  // this thread's chunks of row r, kRowUnroll loads in flight
  auto sweep = [&](int64_t r, auto&& f) {
    const char* xr = xs + r * N * EB;
    for (int64_t base = c0; base < N; base += kStep * kRowUnroll) {
      PK xb[kRowUnroll];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int64_t col = base + u * kStep;
        if (col < N) xb[u].load(xr + col * EB);
      }
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int64_t col = base + u * kStep;
        if (col < N) f(col, xb[u]);
      }
    }
  };

  for (int64_t r = blockIdx.x; r < M; r += gridDim.x) {
    float mu = 0.0f, u1 = 0.0f, u2 = 0.0f;
    if constexpr (KIND == kLayerNorm) {
      float sx = 0.0f;
      sweep(r, [&](int64_t, const PK& x) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) sx += x.get(v);
      });
      block_sum3(sx, u1, u2, buf, phase, lane, wave);
      mu = sx * inv_n;
    }
    float s2 = 0.0f;
    sweep(r, [&](int64_t, const PK& x) {
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const float xc = x.get(v) - mu;
        s2 = __builtin_fmaf(xc, xc, s2);
      }
    });
    block_sum3(s2, u1, u2, buf, phase, lane, wave);
    const float rs = 1.0f / __builtin_sqrtf(__builtin_fmaf(s2, inv_n, eps));
    if (threadIdx.x == 0) {
      if (mean_out && KIND == kLayerNorm) mean_out[r] = mu;
      if (rstd_out) rstd_out[r] = rs;
    }
    char* yr = ys + r * N * EB;
    sweep(r, [&](int64_t col, const PK& x) {
      PK g, b;
      g.load(gs + col * EB);
      if (BETA) b.load(bs + col * EB);
      float o[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v)
        o[v] = __builtin_fmaf((x.get(v) - mu) * rs, g.get(v), BETA ? b.get(v) : 0.0f);
      PK out;
      out.set(o);
      out.store_stream(yr + col * EB);
    });
  }
}

// Wide rows that fit in the registers of one workgroup: up to
// kRowWaves * 64 * VEC * C elements (C = 8: 65536 16-bit or 32768 fp32
// elements). One row per workgroup at a time, rows strided over the grid.
// Thread t holds the VEC-element chunks starting at (c * 1024 + t) * VEC,
// c < C, of x and dy, so each is read once per row for both the row sums and
// dx, where dx_rowloop_kernel streams the row twice. Same formulas
// as dx_rowloop_kernel ("Norm backward in Triton", "The gradients"); the
// weight gradients come from the column walk. Sums over the 16 waves are
// added in wave order, so results are reproducible.
template <int KIND, bool RECOMP, class Tg, int VEC, int C>
__global__ __launch_bounds__(kRowWaves * 64)
void dx_rowreg_kernel(const void* __restrict__ xv, const void* __restrict__ dyv,
                      const void* __restrict__ gv, const float* __restrict__ mean,
                      const float* __restrict__ rstd, void* __restrict__ dxv,
                      float* __restrict__ mean_out, float* __restrict__ rstd_out, int64_t M,
                      int64_t N, int64_t ldx, int64_t ldy, int64_t ldo, float eps) {
  using PK = Pack<Tg, VEC>;
  constexpr int EB = Tg::kBytes;
  constexpr int kStep = kRowWaves * 64 * VEC;  // elements between a thread's chunks
  const char* __restrict__ xs = static_cast<const char*>(xv);
  const char* __restrict__ ys = static_cast<const char*>(dyv);
  const char* __restrict__ gs = static_cast<const char*>(gv);
  char* __restrict__ dxs = static_cast<char*>(dxv);
  __shared__ float buf[2][kRowWaves][4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c0 = threadIdx.x * VEC;
  // Addresses: a uniform base per row and chunk plus this thread's 32-bit
  // byte offset, the same for every chunk (one offset register in all).
  const uint32_t lo = (uint32_t)c0 * EB;
  constexpr int64_t kChunkBytes = (int64_t)kStep * EB;
  const float inv_n = 1.0f / (float)N;
  int phase = 0;

  for (int64_t r = blockIdx.x; r < M; r += gridDim.x) {
    const char* xr = xs + r * ldx * EB;
    const char* yr = ys + r * ldy * EB;
    PK xb[C], yb[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (c0 + c * kStep < N) {
        xb[c].load_stream(xr + c * kChunkBytes + lo);
        yb[c].load_stream(yr + c * kChunkBytes + lo);
      }
    }
    // gamma (the same for every row, so cached) is read where it is used
    // rather than held: the row's x and dy already take 64 registers per
    // thread at C = 8
    auto gam = [&](int c) {
      PK g;
      g.load(gs + c * kChunkBytes + lo);
      return g;
    };
    float mu = 0.0f, rs, s1 = 0.0f, s2 = 0.0f, unused = 0.0f;
    if constexpr (!RECOMP) {
      mu = (KIND == kLayerNorm) ? mean[r] : 0.0f;
      rs = rstd[r];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if (c0 + c * kStep < N) {
          const PK g = gam(c);
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            const float dyh = yb[c].get(v) * g.get(v);
            if (KIND == kLayerNorm) s1 = __builtin_fmaf(yb[c].get(v), g.get(v), s1);
            s2 = __builtin_fmaf(dyh, xb[c].get(v) - mu, s2);
          }
        }
      }
      keep_packed(xb);
      keep_packed(yb);
      block_sum3(s1, s2, unused, buf, phase, lane, wave);
    } else {
      if constexpr (KIND == kLayerNorm) {
        float sx = 0.0f, u1 = 0.0f;
#pragma unroll
        for (int c = 0; c < C; ++c)
          if (c0 + c * kStep < N)
#pragma unroll
            for (int v = 0; v < VEC; ++v) sx += xb[c].get(v);
        keep_packed(xb);
        block_sum3(sx, u1, unused, buf, phase, lane, wave);
        mu = sx * inv_n;
      }
      float sxx = 0.0f;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if (c0 + c * kStep < N) {
          const PK g = gam(c);
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            const float xc = xb[c].get(v) - mu;
            const float dyh = yb[c].get(v) * g.get(v);
            sxx = __builtin_fmaf(xc, xc, sxx);
            if (KIND == kLayerNorm) s1 = __builtin_fmaf(yb[c].get(v), g.get(v), s1);
            s2 = __builtin_fmaf(dyh, xc, s2);
          }
        }
      }
      keep_packed(xb);
      keep_packed(yb);
      block_sum3(sxx, s1, s2, buf, phase, lane, wave);
      rs = 1.0f / __builtin_sqrtf(__builtin_fmaf(sxx, inv_n, eps));
      if (threadIdx.x == 0) {
        if (KIND == kLayerNorm) mean_out[r] = mu;
        rstd_out[r] = rs;
      }
    }
    const float m2 = s2 * inv_n * rs;
    const float c2 = -(rs * rs) * m2;
    const float c1 = (KIND == kLayerNorm) ? -rs * (s1 * inv_n) : 0.0f;
    char* dr = dxs + r * ldo * EB;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (c0 + c * kStep < N) {
        const PK g = gam(c);
        float o[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v)
          o[v] = __builtin_fmaf(yb[c].get(v) * g.get(v), rs,
                                __builtin_fmaf(xb[c].get(v) - mu, c2, c1));
        PK out;
        out.set(o);
        out.store_stream(dr + c * kChunkBytes + lo);
      }
    }
  }
}

// The forward for the same rows: x held in registers (read once), gamma and
// beta read per row as y is written. LayerNorm sums x, then the squared
// deviations from the mean, over the registers; RMSNorm sums x^2.
template <int KIND, class Tg, int VEC, int C, bool BETA>
__global__ __launch_bounds__(kRowWaves * 64)
void fwd_rowreg_kernel(const void* __restrict__ xv, const void* __restrict__ gv,
                       const void* __restrict__ bv, void* __restrict__ yv,
                       float* __restrict__ mean_out, float* __restrict__ rstd_out, int64_t M,
                       int64_t N, float eps) {
  using PK = Pack<Tg, VEC>;
  constexpr int EB = Tg::kBytes;
  constexpr int kStep = kRowWaves * 64 * VEC;
  const char* __restrict__ xs = static_cast<const char*>(xv);
  const char* __restrict__ gs = static_cast<const char*>(gv);
  const char* __restrict__ bs = static_cast<const char*>(bv);
  char* __restrict__ ys = static_cast<char*>(yv);
  __shared__ float buf[2][kRowWaves][4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c0 = threadIdx.x * VEC;
  const uint32_t lo = (uint32_t)c0 * EB;  // as in dx_rowreg_kernel
  constexpr int64_t kChunkBytes = (int64_t)kStep * EB;
  const float inv_n = 1.0f / (float)N;
  int phase = 0;

  for (int64_t r = blockIdx.x; r < M; r += gridDim.x) {
    const char* xr = xs + r * N * EB;
    PK xb[C];
#pragma unroll
    for (int c = 0; c < C; ++c)
      if (c0 + c * kStep < N) xb[c].load_stream(xr + c * kChunkBytes + lo);
    float mu = 0.0f, u1 = 0.0f, u2 = 0.0f;
    if constexpr (KIND == kLayerNorm) {
      float sx = 0.0f;
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (c0 + c * kStep < N)
#pragma unroll
          for (int v = 0; v < VEC; ++v) sx += xb[c].get(v);
      keep_packed(xb);
      block_sum3(sx, u1, u2, buf, phase, lane, wave);
      mu = sx * inv_n;
    }
    float s2 = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (c0 + c * kStep < N) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float xc = xb[c].get(v) - mu;
          s2 = __builtin_fmaf(xc, xc, s2);
        }
      }
    }
    keep_packed(xb);
    block_sum3(s2, u1, u2, buf, phase, lane, wave);
    const float rs = 1.0f / __builtin_sqrtf(__builtin_fmaf(s2, inv_n, eps));
    if (threadIdx.x == 0) {
      if (mean_out && KIND == kLayerNorm) mean_out[r] = mu;
      if (rstd_out) rstd_out[r] = rs;
    }
    char* yr = ys + r * N * EB;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (c0 + c * kStep < N) {
        PK g, b;
        g.load(gs + c * kChunkBytes + lo);
        if (BETA) b.load(bs + c * kChunkBytes + lo);
        float o[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v)
          o[v] = __builtin_fmaf((xb[c].get(v) - mu) * rs, g.get(v), BETA ? b.get(v) : 0.0f);
        PK out;
        out.set(o);
        out.store_stream(yr + c * kChunkBytes + lo);
      }
    }
  }
}

}  // namespace nb
