// nb_tworow.hpp -- kernel A and the forward for rows that 32 lanes cover
// exactly with 16-byte vectors (N = 32 * VEC * C, C = 1 or 3; for 16-bit
// elements 256 or 768 features). Such rows leave half the lanes of a 64-lane
// layout idle in their last chunk and keep it out of the branch-free
// steady-state loop; here every wave takes two rows at once, one per 32-lane
// half, so every lane holds data and every load and store instruction moves
// two 512-byte runs. Kernel A takes saved statistics or (RECOMP) recomputes
// them; the forward computes them. Both compute a row's statistics with the
// same helpers (lane sums in chunk order, then the half's butterfly), so
// recompute mode sees the statistics the forward saved, bit for bit.
//
// What is computed is kernel A's (nb_device.hpp), from the same formulas of
// "Norm backward in Triton -- the dγ/dβ reduction", "The gradients": dx per
// row, and per row group g (below) the group's partial dgamma (and dbeta) in
// fp32 registers, stored once into the workspace.
//
// Layout. Rows go in pairs (2q, 2q + 1), and row group g is the pairs with
// q mod G == g (disjoint groups, as kernel A's, with pairs in place of rows).
// Lane l of wave w is in half h = l / 32 and covers the columns
// (l mod 32) * VEC + c * 32 * VEC, c < C, of its row. With P waves per
// workgroup, iteration k of group g gives wave w the group's pair
// q = g + (k * P + w) * G and its half h row 2q + h: the two halves of a load
// instruction read adjacent rows. A half's row sums are complete after a
// 32-lane butterfly (no exchange between waves, no barrier). Each half
// accumulates its rows in ascending order; at the end of the group the two
// halves are added (half 0 + half 1), then the P waves in wave order through
// LDS. The summation order depends on (M, G, P) only.
#pragma once

#include "nb_device.hpp"

namespace nb {

// Sum over each 32-lane half of the wave: the 16-lane DPP butterfly of
// wave_sum, then half 0 takes (lanes 0-15) + (lanes 16-31) and half 1
// (lanes 32-47) + (lanes 48-63), each in that order.
__device__ __forceinline__ float half_sum(float v, bool hi) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  const float lo = r0 + r1, hi_sum = r2 + r3;
  return hi ? hi_sum : lo;
}

// A lane's part of a row's statistics, in the order the forward and
// recompute mode share: sum(x), and sum((x - mu)^2) by fused multiply-adds,
// chunk by chunk, element by element.
template <class Tg, int VEC, int C>
__device__ __forceinline__ float lane_sum_x(const Pack<Tg, VEC> (&x)[C]) {
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int v = 0; v < VEC; ++v) s += x[c].get(v);
  return s;
}

template <class Tg, int VEC, int C>
__device__ __forceinline__ float lane_sum_sq(const Pack<Tg, VEC> (&x)[C], float mu) {
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const float xc = x[c].get(v) - mu;
      s = __builtin_fmaf(xc, xc, s);
    }
  return s;
}

constexpr int kTwoRowDepth = 3;  // ring of row pairs (two ahead; LayerNorm saved: see the kernel)
constexpr int kTwoRowMaxThreads = 512;  // launch bound: 256 VGPRs per lane

// Loads of one row pair. RALL (steady state): both rows exist; the wave
// addresses them through one buffer resource based at its first row, the
// second half adding `hoff` bytes (one row stride). Otherwise each lane loads
// through its own address, and only when its row exists.
template <int KIND, bool RECOMP, bool RALL, class Tg, int VEC, int C>
__device__ __forceinline__ void fetch_pair(RowBuf<Tg, VEC, C>& b, const char* __restrict__ x,
                                           const char* __restrict__ dy,
                                           const float* __restrict__ mean,
                                           const float* __restrict__ rstd, int64_t r0, int64_t r,
                                           bool active, int64_t ldx, int64_t ldy, uint32_t hoff_x,
                                           uint32_t hoff_y, uint32_t span_x, uint32_t span_y,
                                           int col0, int cstride) {
  constexpr int EB = Tg::kBytes;
  if (RALL || active) {
    if constexpr (!RECOMP) {
      const int64_t rz = r + opaque_lane_zero();
      b.rs = rstd[rz];
      b.mu = (KIND == kLayerNorm) ? mean[rz] : 0.0f;
    }
    if constexpr (RALL) {
      const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + r0 * ldx * EB, span_x);
      const __amdgpu_buffer_rsrc_t ry = row_rsrc(dy + r0 * ldy * EB, span_y);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const uint32_t off = (uint32_t)(col0 + c * cstride) * EB;
        b.x[c].load_stream_buf(rx, hoff_x + off);
        b.dy[c].load_stream_buf(ry, hoff_y + off);
      }
    } else {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int64_t col = col0 + c * cstride;
        b.x[c].load_stream(x + (r * ldx + col) * EB);
        b.dy[c].load_stream(dy + (r * ldy + col) * EB);
      }
    }
  }
}

// One row pair once its operands are in registers: the weight-gradient terms
// into the accumulators, the half's row sums, then dx (RALL: through the
// pair's buffer resource, as fetch_pair). RECOMP: the statistics come from
// the row itself, as kernel A's recompute mode forms them (LayerNorm: sum(x)
// with sum(dyhat), then with mean = sum(x)/N sum((x - mean)^2) with
// sum(dyhat * (x - mean)); RMSNorm: sum(x^2) with sum(dyhat * x)), and the
// dgamma terms, which need rstd, join the dx pass. Every lane takes part in
// each butterfly (rows that do not exist add zeros to sums nobody uses).
template <int KIND, bool RECOMP, bool RALL, class Tg, int VEC, int C, int NACC>
__device__ __forceinline__ void process_pair(RowBuf<Tg, VEC, C>& b, const float (&gam)[C][VEC],
                                             float (&acc)[NACC][C][VEC], char* __restrict__ dx,
                                             int64_t r0, int64_t r, bool active, bool hi,
                                             int64_t ldo, uint32_t hoff_o, uint32_t span_o,
                                             float inv_n, float eps, int col0, int cstride) {
  constexpr int EB = Tg::kBytes;
  float mu, rs;
  float s1 = 0.0f, s2 = 0.0f;
  if constexpr (!RECOMP) {
    mu = b.mu;
    rs = b.rs;
    if (RALL || active) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
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
    pin(acc);
    keep_packed(b.x);
    keep_packed(b.dy);
    s2 = half_sum(s2, hi);
    if (KIND == kLayerNorm) s1 = half_sum(s1, hi);
  } else {
    mu = 0.0f;
    if constexpr (KIND == kLayerNorm) {
      float sx = 0.0f;
      if (RALL || active) {
        sx = lane_sum_x(b.x);
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
          for (int v = 0; v < VEC; ++v) {
            const float dyv = b.dy[c].get(v);
            s1 = __builtin_fmaf(dyv, gam[c][v], s1);
            if (NACC == 2) acc[NACC - 1][c][v] += dyv;
          }
      }
      keep_packed(b.x);
      keep_packed(b.dy);
      sx = half_sum(sx, hi);
      s1 = half_sum(s1, hi);
      mu = sx * inv_n;
    }
    float sxx = 0.0f;
    if (RALL || active) {
      sxx = lane_sum_sq(b.x, mu);
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float xc = b.x[c].get(v) - mu;
          const float dyv = b.dy[c].get(v);
          s2 = __builtin_fmaf(dyv * gam[c][v], xc, s2);
          if (KIND != kLayerNorm && NACC == 2) acc[NACC - 1][c][v] += dyv;
        }
    }
    keep_packed(b.x);
    keep_packed(b.dy);
    sxx = half_sum(sxx, hi);
    s2 = half_sum(s2, hi);
    rs = 1.0f / __builtin_sqrtf(__builtin_fmaf(sxx, inv_n, eps));
  }
  if (RALL || active) {
    const float m2 = s2 * inv_n * rs;  // mean_j(dyhat * xhat)
    const float c2 = -(rs * rs) * m2;
    const float c1 = (KIND == kLayerNorm) ? -rs * (s1 * inv_n) : 0.0f;
    __amdgpu_buffer_rsrc_t ro;
    if constexpr (RALL) ro = row_rsrc(dx + r0 * ldo * EB, span_o);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int col = col0 + c * cstride;
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
      if constexpr (RALL) out.store_stream_buf(ro, hoff_o + (uint32_t)col * EB);
      else out.store_stream(dx + (r * ldo + col) * EB);
    }
  }
}

// P = waves per workgroup (2 * P rows in flight). span_* = bytes from a row
// pair's first row to the end of its second row (ld + N elements), which the
// host checked to be below 2^32.
template <int KIND, bool RECOMP, class Tg, int C, int NACC, bool WSNT>
__global__ __launch_bounds__(kTwoRowMaxThreads)
void dx_partials_tworow_kernel(const void* __restrict__ xv, const void* __restrict__ dyv,
                               const void* __restrict__ gv, const float* __restrict__ mean,
                               const float* __restrict__ rstd, void* __restrict__ dxv,
                               float* __restrict__ ws, int64_t M, int N, int64_t ldx,
                               int64_t ldy, int64_t ldo, int64_t G, int P, float eps) {
  constexpr int EB = Tg::kBytes;
  constexpr int VEC = 16 / EB;
  // LayerNorm with saved statistics, and RMSNorm recompute on rows of three
  // chunks, keep one pair less in flight: their workgroups of 4 waves (every
  // SIMD busy with their heavier arithmetic) put twice the bytes in flight
  // with a ring of 3 that the 2-wave RMSNorm workgroups do. Ring of 2
  // against 3, on the same buffers: LayerNorm 87381 x 768 bf16 73.2 against
  // 76.9 us, 262144 x 768 206.8 against 218.7, 262144 x 256 73.9 against
  // 74.4, fp32 x 384 even; RMSNorm recompute 262144 x 768 210.0 against
  // 217.8, fp32 x 384 213.9 against 215.8. Slower with it: LayerNorm
  // recompute (x 768 +2.5 and +4.3%, x 256 +12%), RMSNorm recompute of one
  // chunk (x 256 +7%), RMSNorm with saved statistics (2-wave workgroups:
  // x 768 +25%, x 256 +13%).
  constexpr int D = ((KIND == kLayerNorm && !RECOMP) || (KIND == kRmsNorm && RECOMP && C == 3))
                        ? 2 : kTwoRowDepth;
  using PK = Pack<Tg, VEC>;
  using RB = RowBuf<Tg, VEC, C>;
  const char* __restrict__ x = static_cast<const char*>(xv);
  const char* __restrict__ dy = static_cast<const char*>(dyv);
  const char* __restrict__ gm = static_cast<const char*>(gv);
  char* __restrict__ dx = static_cast<char*>(dxv);
  extern __shared__ float comb[];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const bool hi = h != 0;
  const int col0 = (lane & 31) * VEC;
  constexpr int cstride = 32 * VEC;
  const float inv_n = 1.0f / (float)N;
  // the second half's row is the next row
  const uint32_t hoff_x = (uint32_t)(h * ldx * EB);
  const uint32_t hoff_y = (uint32_t)(h * ldy * EB);
  const uint32_t hoff_o = (uint32_t)(h * ldo * EB);
  const uint32_t span_x = (uint32_t)((ldx + N) * EB);
  const uint32_t span_y = (uint32_t)((ldy + N) * EB);
  const uint32_t span_o = (uint32_t)((ldo + N) * EB);

  float gam[C][VEC];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    PK t;
    t.load(gm + (int64_t)(col0 + c * cstride) * EB);
#pragma unroll
    for (int v = 0; v < VEC; ++v) gam[c][v] = t.get(v);
  }

  for (int64_t g = blockIdx.x; g < G; g += gridDim.x) {
    // group g = the row pairs (2q, 2q + 1) with q mod G == g
    const int64_t npairs = ((M + 1) / 2 - g + G - 1) / G;     // pairs of group g
    const int64_t nfull = (M / 2 > g) ? (M / 2 - g + G - 1) / G : 0;  // complete pairs
    const int64_t rows = 2 * nfull;  // (for the steady-state byte rule)
    const int iters = (int)((npairs + P - 1) / P);
    auto pair0 = [&](int k) { return 2 * (g + (int64_t)(k * P + w) * G); };
    auto row_of = [&](int k) { return pair0(k) + h; };
    auto exists = [&](int k) { return row_of(k) < M; };

    float acc[NACC][C][VEC];
#pragma unroll
    for (int a = 0; a < NACC; ++a)
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[a][c][v] = 0.0f;

    RB buf[D];
    // Steady state (as kernel A's): iterations in which all 2P rows exist run
    // through a loop with no per-lane or per-row conditions; the general loop
    // takes the remaining iterations from the same ring state.
    const int kfull = (int)(nfull / P);
    int it0 = 0;
    const bool steady =
        kfull >= 2 * D - 1 && rows * (int64_t)N * EB <= kSteadyGroupBytes;
    if (steady) {
#pragma unroll
      for (int k = 0; k < D - 1; ++k)
        fetch_pair<KIND, RECOMP, true>(buf[k], x, dy, mean, rstd, pair0(k), row_of(k), true, ldx, ldy,
                               hoff_x, hoff_y, span_x, span_y, col0, cstride);
      for (; it0 + 2 * D - 2 < kfull; it0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const int k = it0 + d;
          fetch_pair<KIND, RECOMP, true>(buf[(d + D - 1) % D], x, dy, mean, rstd, pair0(k + D - 1),
                                 row_of(k + D - 1), true, ldx, ldy, hoff_x, hoff_y, span_x,
                                 span_y, col0, cstride);
          process_pair<KIND, RECOMP, true>(buf[d], gam, acc, dx, pair0(k), row_of(k), true, hi, ldo,
                                   hoff_o, span_o, inv_n, eps, col0, cstride);
          // RMSNorm with saved statistics: keep the next pair's arithmetic
          // below this point. Hoisted above the loop top, it needed the
          // pair loaded last and so a wait for nearly every load in flight
          // (vmcnt counts in order): the ring drained once a loop (waits
          // down to 1 of 18 loads). Fenced, the waits keep 6-16 in flight:
          // 262144 x 768 bf16 202.5 -> 195.1 us, 1048576 x 256 270.9 ->
          // 261.0, fp32 x 384 222.8 -> 212.0, fp32 x 128 135.6 -> 132.1.
          // LayerNorm and recompute mode were even or slower fenced (fp32
          // LayerNorm x 128 +7.8%, RMSNorm recompute x 256 +19.8%).
          if constexpr (!RECOMP && KIND == kRmsNorm) __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < D - 1; ++k)
        if (k < iters)
          fetch_pair<KIND, RECOMP, false>(buf[k], x, dy, mean, rstd, pair0(k), row_of(k), exists(k), ldx,
                                  ldy, hoff_x, hoff_y, span_x, span_y, col0, cstride);
    }
    for (int it = it0; it < iters; it += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int k = it + d;
        if (k + D - 1 < iters)
          fetch_pair<KIND, RECOMP, false>(buf[(d + D - 1) % D], x, dy, mean, rstd, pair0(k + D - 1),
                                  row_of(k + D - 1), exists(k + D - 1), ldx, ldy, hoff_x,
                                  hoff_y, span_x, span_y, col0, cstride);
        if (k < iters)
          process_pair<KIND, RECOMP, false>(buf[d], gam, acc, dx, pair0(k), row_of(k), exists(k), hi,
                                    ldo, hoff_o, span_o, inv_n, eps, col0, cstride);
      }
    }

    // the two halves: half 0 + half 1 (the same sum in both halves)
#pragma unroll
    for (int a = 0; a < NACC; ++a)
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float other = __shfl_xor(acc[a][c][v], 32);
          acc[a][c][v] = hi ? other + acc[a][c][v] : acc[a][c][v] + other;
        }
    // the P waves in wave order 0, 1, ..., P-1 (half 0 of each)
    if (P > 1) {
      for (int q = 1; q < P; ++q) {
        if (w == q && !hi) {
#pragma unroll
          for (int a = 0; a < NACC; ++a)
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
              for (int v = 0; v < VEC; ++v)
                comb[((a * C + c) * 32 + (lane & 31)) * VEC + v] = acc[a][c][v];
        }
        __syncthreads();
        if (w == 0) {
#pragma unroll
          for (int a = 0; a < NACC; ++a)
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
              for (int v = 0; v < VEC; ++v)
                acc[a][c][v] += comb[((a * C + c) * 32 + (lane & 31)) * VEC + v];
        }
        __syncthreads();
      }
    }
    if (w == 0 && !hi) {
#pragma unroll
      for (int a = 0; a < NACC; ++a) {
        float* __restrict__ dst = ws + ((int64_t)a * G + g) * (int64_t)N;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int col = col0 + c * cstride;
#pragma unroll
          for (int v = 0; v < VEC; v += 4) {
            const f32x4 t = {acc[a][c][v], acc[a][c][v + 1], acc[a][c][v + 2], acc[a][c][v + 3]};
            f32x4* q = reinterpret_cast<f32x4*>(dst + col + v);
            if constexpr (WSNT) __builtin_nontemporal_store(t, q);
            else *q = t;
          }
        }
      }
    }
  }
}

// The forward on the same layout: per row, the statistics from lane_sum_x /
// lane_sum_sq and the half's butterfly (as recompute mode forms them), then
// y = gamma * (x - mean) * rstd + beta, and mean/rstd stored as fp32 by the
// first lane of each half. Rows carry no cross-row state, so in sweep k
// wave w of workgroup b takes the pair q = (k * gridDim.x + b) * P + w: all
// workgroups sweep one address window together. Rows are contiguous (row
// stride N), and the launch checks N = 32 * VEC * C, so a pair spans at most
// 2 * 768 * 2 bytes and its 32-bit buffer offsets cannot overflow.
template <int KIND, class Tg, int C, bool BETA>
__global__ __launch_bounds__(kTwoRowMaxThreads)
void norm_fwd_tworow_kernel(const void* __restrict__ xv, const void* __restrict__ gv,
                            const void* __restrict__ bv, void* __restrict__ yv,
                            float* __restrict__ mean_out, float* __restrict__ rstd_out,
                            int64_t M, int N, float eps, int P) {
  constexpr int EB = Tg::kBytes;
  constexpr int VEC = 16 / EB;
  // Rows of three chunks keep one pair less in flight (3 KiB a wave, as rows
  // of one chunk with a ring of three hold 2 KiB). Ring of 2 against 3, on
  // the same buffers: 262144 x 768 bf16 RMSNorm 136.3 against 143.6 us,
  // 262144 x 384 fp32 131.8 against 142.2, LayerNorm x 768 even; rows of one
  // chunk were slower with it (262144 x 256 LayerNorm 62.0 against 52.1,
  // 1048576 x 256 RMSNorm 215.3 against 203.4).
  constexpr int D = C == 3 ? 2 : kTwoRowDepth;
  using PK = Pack<Tg, VEC>;
  const char* __restrict__ x = static_cast<const char*>(xv);
  char* __restrict__ y = static_cast<char*>(yv);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const bool hi = h != 0;
  const int col0 = (lane & 31) * VEC;
  constexpr int cstride = 32 * VEC;
  const float inv_n = 1.0f / (float)N;
  const uint32_t hoff = (uint32_t)(h * N * EB);
  const uint32_t span = (uint32_t)(2 * N * EB);

  float gam[C][VEC], bet[C][VEC];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int64_t col = col0 + c * cstride;
    PK tg, tb;
    tg.load(static_cast<const char*>(gv) + col * EB);
    if (BETA) tb.load(static_cast<const char*>(bv) + col * EB);
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      gam[c][v] = tg.get(v);
      bet[c][v] = BETA ? tb.get(v) : 0.0f;
    }
  }

  const int64_t per_sweep = (int64_t)gridDim.x * P;
  const int iters = (int)(((M + 1) / 2 + per_sweep - 1) / per_sweep);
  const int kfull = (int)((M / 2) / per_sweep);  // sweeps of complete pairs only
  auto pair0 = [&](int k) { return 2 * (((int64_t)k * gridDim.x + blockIdx.x) * P + w); };

  PK buf[D][C];
  // RALL: both rows of the pair exist; they go through one buffer resource
  // based at the pair's first row.
  auto fetch = [&](auto all, PK (&b)[C], int k) {
    constexpr bool RALL = decltype(all)::value;
    const int64_t r0 = pair0(k), r = r0 + h;
    if (RALL || r < M) {
      if constexpr (RALL) {
        const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + r0 * N * EB, span);
#pragma unroll
        for (int c = 0; c < C; ++c)
          b[c].load_stream_buf(rx, hoff + (uint32_t)(col0 + c * cstride) * EB);
      } else {
#pragma unroll
        for (int c = 0; c < C; ++c) b[c].load_stream(x + (r * N + col0 + c * cstride) * EB);
      }
    }
  };
  auto process = [&](auto all, PK (&b)[C], int k) {
    constexpr bool RALL = decltype(all)::value;
    const int64_t r0 = pair0(k), r = r0 + h;
    const bool active = RALL || r < M;
    float mu = 0.0f;
    if constexpr (KIND == kLayerNorm) {
      float sx = active ? lane_sum_x(b) : 0.0f;
      keep_packed(b);
      sx = half_sum(sx, hi);
      mu = sx * inv_n;
    }
    float sxx = active ? lane_sum_sq(b, mu) : 0.0f;
    keep_packed(b);
    sxx = half_sum(sxx, hi);
    if (active) {
      const float rs = 1.0f / __builtin_sqrtf(__builtin_fmaf(sxx, inv_n, eps));
      __amdgpu_buffer_rsrc_t ry;
      if constexpr (RALL) ry = row_rsrc(y + r0 * N * EB, span);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int col = col0 + c * cstride;
        float o[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v)
          o[v] = __builtin_fmaf((b[c].get(v) - mu) * rs, gam[c][v], bet[c][v]);
        PK out;
        out.set(o);
        if constexpr (RALL) out.store_stream_buf(ry, hoff + (uint32_t)col * EB);
        else out.store_stream(y + (r * N + col) * EB);
      }
      // the first lane of each half stores its row's statistics
      if ((lane & 31) == 0) {
        if (KIND == kLayerNorm && mean_out) mean_out[r] = mu;
        if (rstd_out) rstd_out[r] = rs;
      }
    }
  };

  // the steady state and general loop of kernel A's ring
  int it0 = 0;
  if (kfull >= 2 * D - 1) {
#pragma unroll
    for (int k = 0; k < D - 1; ++k) fetch(std::true_type(), buf[k], k);
    for (; it0 + 2 * D - 2 < kfull; it0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int k = it0 + d;
        fetch(std::true_type(), buf[(d + D - 1) % D], k + D - 1);
        // Ring of two: issue the next pair's loads before this pair's
        // arithmetic. Unfenced, the compiler put the first pass over this
        // pair above them, so every pair waited on its own loads with nothing
        // else in flight (waits down to 0 of 6). Fenced: 262144 x 768 bf16
        // LayerNorm 144.2 -> 141.2 us, RMSNorm 135.9 -> 135.2, fp32 x 384
        // even. Kernel A's rings of two ran 3-5% slower so fenced and stay
        // unfenced.
        if constexpr (D == 2) __builtin_amdgcn_sched_barrier(0);
        process(std::true_type(), buf[d], k);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < D - 1; ++k)
      if (k < iters) fetch(std::false_type(), buf[k], k);
  }
  for (int it = it0; it < iters; it += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int k = it + d;
      if (k + D - 1 < iters) fetch(std::false_type(), buf[(d + D - 1) % D], k + D - 1);
      if (k < iters) process(std::false_type(), buf[d], k);
    }
  }
}

}  // namespace nb
