// nb_forward.hpp -- the forward pass that produces the statistics the
// backward consumes (gfx950, wave64).
//
// Per row x of width N ("05: Layer norm", the Phobos tutorial's ln_fwd;
// "Norm backward in Triton -- the dγ/dβ reduction", "The gradients" for
// RMSNorm):
//   LayerNorm: mean = sum(x)/N, var = sum((x - mean)^2)/N (biased, two passes
//              over the registers, the two exchanges pipelined across rows),
//              rstd = 1/sqrt(var + eps), y = gamma * (x - mean) * rstd + beta
//   RMSNorm:   rstd = 1/sqrt(sum(x^2)/N + eps), y = gamma * x * rstd (+ beta)
// and mean/rstd are stored as fp32 for the backward.
//
// The layout is kernel A's: S waves share a row, each lane holds C chunks of
// VEC contiguous elements, P rows in flight per workgroup, and a ring of
// register buffers keeps the next rows' loads in flight. Rows carry no
// cross-row state, so workgroup b simply takes rows (k*gridDim.x + b)*P + p:
// all workgroups sweep one address window together. As in kernel A, the
// sweeps in which every row exists run through a loop without per-lane or
// per-row conditions when the lanes cover the row exactly (steady state).
#pragma once

#include "nb_device.hpp"

namespace nb {

template <bool B>
using Flag = std::integral_constant<bool, B>;

// Whether the forward runs its steady-state loop (see kernel A's).
template <int KIND, class Tg, int VEC, int C, bool BETA>
constexpr bool fwd_steady_loop() {
  return VEC > 1 && VEC * C <= 32;
}

template <class Tg, int VEC, int C>
struct XBuf {
  Pack<Tg, VEC> x[C];
};

template <int KIND, class Tg, int VEC, int C, bool BETA>
__global__ __launch_bounds__((max_threads_for<VEC, C>()))
void norm_fwd_kernel(const void* __restrict__ xv, const void* __restrict__ gv,
                     const void* __restrict__ bv, void* __restrict__ yv,
                     float* __restrict__ mean_out, float* __restrict__ rstd_out, int64_t M,
                     int N, float eps, int S, int P) {
  using PK = Pack<Tg, VEC>;
  constexpr int EB = Tg::kBytes;
  const char* __restrict__ x = static_cast<const char*>(xv);
  char* __restrict__ y = static_cast<char*>(yv);

  __shared__ __align__(8) float red[2][kMaxWaves][2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int s = wave % S;
  const int p = wave / S;
  const int cstride = S * 64 * VEC;
  const int col0 = (s * 64 + lane) * VEC;
  const float inv_n = 1.0f / (float)N;

  float gam[C][VEC], bet[C][VEC];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int col = col0 + c * cstride;
    PK tg, tb;
    tg.zero();
    tb.zero();
    if (col < N) {
      tg.load(static_cast<const char*>(gv) + (int64_t)col * EB);
      if (BETA) tb.load(static_cast<const char*>(bv) + (int64_t)col * EB);
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      gam[c][v] = tg.get(v);
      bet[c][v] = BETA ? tb.get(v) : 0.0f;
    }
  }

  const int64_t rows_per_sweep = (int64_t)gridDim.x * P;
  const int iters = (int)((M + rows_per_sweep - 1) / rows_per_sweep);
  auto row_of = [&](int k) { return ((int64_t)k * gridDim.x + blockIdx.x) * P + p; };

  // Sweeps in which every row exists, and whether the steady-state loop may
  // run (the lanes cover the row exactly).
  const int kfull = (int)(M / rows_per_sweep);
  const bool cover = N == C * cstride;

  // `all` (Flag<true>): the row exists and every chunk is inside it, so no
  // condition is evaluated, and x and y go through the row's buffer
  // resource (scalar base, 32-bit lane offset).
  auto fetch = [&](auto all, XBuf<Tg, VEC, C>& b, int64_t r) {
    constexpr bool ALL = decltype(all)::value;
    if (ALL || r < M) {
      const int64_t rb = r * (int64_t)N;
      if constexpr (ALL) {
        const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + rb * EB, (uint32_t)N * EB);
#pragma unroll
        for (int c = 0; c < C; ++c)
          b.x[c].load_stream_buf(rx, (uint32_t)(col0 + c * cstride) * EB);
      } else {
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int col = col0 + c * cstride;
          if (col < N) b.x[c].load_stream(x + (rb + col) * EB);
        }
      }
    }
  };
  // store one lane's vector of y at column col (row base rb, in elements)
  auto store_y = [&](auto all, const PK& out, int64_t rb, int col) {
    constexpr bool ALL = decltype(all)::value;
    if constexpr (ALL)
      out.store_stream_buf(row_rsrc(y + rb * EB, (uint32_t)N * EB), (uint32_t)col * EB);
    else
      out.store_stream(y + (rb + col) * EB);
  };

  int phase = 0;
  // RMSNorm: one exchange per row (sum of x^2), then y
  auto process = [&](auto all, XBuf<Tg, VEC, C>& b, int64_t r) {
    constexpr bool ALL = decltype(all)::value;
    const bool active = ALL || r < M;
    float unused = 0.0f;
    const float mu = 0.0f;
    float s2 = 0.0f;  // sum(x^2)
    if (active) {
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (ALL || col0 + c * cstride < N)
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            const float xc = b.x[c].get(v) - mu;
            s2 = __builtin_fmaf(xc, xc, s2);
          }
    }
    keep_packed(b.x);
    row_sum2<false>(unused, s2, red, phase, lane, wave, S, p);
    if (active) {
      const float rs = 1.0f / __builtin_sqrtf(__builtin_fmaf(s2, inv_n, eps));
      const int64_t rb = r * (int64_t)N;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int col = col0 + c * cstride;
        if (ALL || col < N) {
          float o[VEC];
#pragma unroll
          for (int v = 0; v < VEC; ++v)
            o[v] = __builtin_fmaf((b.x[c].get(v) - mu) * rs, gam[c][v], bet[c][v]);
          PK out;
          out.set(o);
          store_y(all, out, rb, col);
        }
      }
      // one lane stores the row's statistic (a predicated vector store)
      if (s == 0 && lane == 0 && rstd_out) rstd_out[r] = rs;
    }
  };

  if constexpr (KIND == kLayerNorm) {
    // LayerNorm: the two exchanges a row needs are pipelined across rows, so
    // a row costs one barrier. Step k exchanges row k's sum of squared
    // deviations together with row k+1's sum of x; the prologue exchanges
    // the first row's sum of x alone. Each sum keeps its own order, so mean
    // and rstd are those of the unpipelined two-pass form. The ring holds one
    // more row, as row k+1 is read one step earlier.
    constexpr int D = prefetch_depth<Tg, VEC, C>() + 1;
    XBuf<Tg, VEC, C> buf[D];
    auto xsum = [&](auto all, XBuf<Tg, VEC, C>& b, bool active) {
      constexpr bool ALL = decltype(all)::value;
      float sx = 0.0f;
      if (ALL || active) {
#pragma unroll
        for (int c = 0; c < C; ++c)
          if (ALL || col0 + c * cstride < N)
#pragma unroll
            for (int v = 0; v < VEC; ++v) sx += b.x[c].get(v);
      }
      return sx;
    };
    // Step k of the pipelined row loop: row k's squared deviations and
    // row k+1's sum of x in one exchange, then row k's y and statistics.
    float mu_next = 0.0f;
    auto ln_step = [&](auto all, int d, int k) {
      constexpr bool ALL = decltype(all)::value;
      XBuf<Tg, VEC, C>& b = buf[d];
      const int64_t r = row_of(k);
      const bool active = ALL || r < M;
      const float mu = mu_next;
      float s2 = 0.0f;
      if (active) {
#pragma unroll
        for (int c = 0; c < C; ++c)
          if (ALL || col0 + c * cstride < N)
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
              const float xc = b.x[c].get(v) - mu;
              s2 = __builtin_fmaf(xc, xc, s2);
            }
      }
      float sx1 = (ALL || k + 1 < iters) ? xsum(all, buf[(d + 1) % D], ALL || row_of(k + 1) < M)
                                         : 0.0f;
      keep_packed(b.x);
      row_sum2<true>(sx1, s2, red, phase, lane, wave, S, p);
      mu_next = sx1 * inv_n;
      if (active) {
        const float rs = 1.0f / __builtin_sqrtf(__builtin_fmaf(s2, inv_n, eps));
        const int64_t rb = r * (int64_t)N;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int col = col0 + c * cstride;
          if (ALL || col < N) {
            float o[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v)
              o[v] = __builtin_fmaf((b.x[c].get(v) - mu) * rs, gam[c][v], bet[c][v]);
            PK out;
            out.set(o);
            store_y(all, out, rb, col);
          }
        }
        if (s == 0 && lane == 0) {
          if (mean_out) mean_out[r] = mu;
          if (rstd_out) rstd_out[r] = rs;
        }
      }
    };
    const bool steady = fwd_steady_loop<KIND, Tg, VEC, C, BETA>() && cover && kfull >= 2 * D - 1;
    int it0 = 0;
    if (steady) {
#pragma unroll
      for (int k = 0; k < D - 1; ++k) fetch(Flag<true>(), buf[k], row_of(k));
    } else {
#pragma unroll
      for (int k = 0; k < D - 1; ++k)
        if (k < iters) fetch(Flag<false>(), buf[k], row_of(k));
    }
    float unused = 0.0f;
    float sx0 = iters > 0 ? xsum(Flag<false>(), buf[0], row_of(0) < M) : 0.0f;
    row_sum2<false>(unused, sx0, red, phase, lane, wave, S, p);
    mu_next = sx0 * inv_n;
    if constexpr (fwd_steady_loop<KIND, Tg, VEC, C, BETA>()) {
      if (steady) {
        for (; it0 + 2 * D - 2 < kfull; it0 += D) {
#pragma unroll
          for (int d = 0; d < D; ++d) {
            const int k = it0 + d;
            fetch(Flag<true>(), buf[(d + D - 1) % D], row_of(k + D - 1));
            ln_step(Flag<true>(), d, k);
          }
        }
      }
    }
    for (int it = it0; it < iters; it += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int k = it + d;
        if (k + D - 1 < iters) fetch(Flag<false>(), buf[(d + D - 1) % D], row_of(k + D - 1));
        if (k < iters) ln_step(Flag<false>(), d, k);
      }
    }
  } else {
    constexpr int D = prefetch_depth<Tg, VEC, C>();
    XBuf<Tg, VEC, C> buf[D];
    const bool steady = fwd_steady_loop<KIND, Tg, VEC, C, BETA>() && cover && kfull >= 2 * D - 1;
    int it0 = 0;
    if (steady) {
#pragma unroll
      for (int k = 0; k < D - 1; ++k) fetch(Flag<true>(), buf[k], row_of(k));
      if constexpr (fwd_steady_loop<KIND, Tg, VEC, C, BETA>()) {
        for (; it0 + 2 * D - 2 < kfull; it0 += D) {
#pragma unroll
          for (int d = 0; d < D; ++d) {
            const int k = it0 + d;
            fetch(Flag<true>(), buf[(d + D - 1) % D], row_of(k + D - 1));
            process(Flag<true>(), buf[d], row_of(k));
          }
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < D - 1; ++k)
        if (k < iters) fetch(Flag<false>(), buf[k], row_of(k));
    }
    for (int it = it0; it < iters; it += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int k = it + d;
        if (k + D - 1 < iters) fetch(Flag<false>(), buf[(d + D - 1) % D], row_of(k + D - 1));
        if (k < iters) process(Flag<false>(), buf[d], row_of(k));
      }
    }
  }
}

}  // namespace nb
