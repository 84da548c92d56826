// nb_wgrad.hpp -- weight gradients alone by a column walk (gfx950, wave64).
//
// dgamma[j] = sum over rows of dy * xhat and dbeta[j] = sum over rows of dy
// ("Norm backward in Triton", "The gradients"), computed without a workspace:
// each workgroup owns a tile of TW = LPR * VEC adjacent columns and walks all
// M rows, as the Phobos tutorial's ln_bwd_dwdb does ("05: Layer norm"), so no
// two workgroups write the same column.
//
// Layout inside a workgroup of 16 waves: lane l of a wave covers the VEC
// columns (l mod LPR) * VEC of the tile in row slot l / LPR; a wave load
// covers RPW = 64 / LPR rows, and wave w takes rows w * RPW + slot + k * 16 *
// RPW for k = 0, 1, ... Each lane sums its own rows in ascending order in fp32
// registers; then the RPW slots of a wave are added by an xor butterfly (the
// same tree for every lane), and the 16 wave sums in wave order through LDS.
// The order depends on (M, LPR, VEC) only, so results are reproducible.
//
// Tiles narrower than a 128-byte line share lines with their neighbours.
// Workgroups are dispatched to the 8 XCDs round-robin (block b to XCD b mod 8)
// and each XCD has its own L2, so neighbouring tiles on different XCDs would
// each fetch the shared lines from HBM. Block b therefore takes tile
// (b mod 8) * (T / 8) + b / 8 when the tile count T is a multiple of 8: each
// XCD walks a contiguous run of tiles, and line neighbours share its L2.
#pragma once

#include "nb_device.hpp"

namespace nb {

constexpr int kWgradWaves = 16;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each
constexpr int kWgradUnroll = 4;
constexpr int kWgradMaxTile = 64;  // columns

template <class OutT>
__device__ __forceinline__ void put_out(void* p, int64_t j, float v, bool accumulate) {
  if (accumulate) v = load_out<OutT>(p, j) + v;
  store_out<OutT>(p, j, v);
}

template <int KIND, class Tg, int VEC, int NACC>
__global__ __launch_bounds__(kWgradWaves * 64)
void wgrad_colwalk_kernel(const void* __restrict__ xv, const void* __restrict__ dyv,
                          const float* __restrict__ mean, const float* __restrict__ rstd,
                          int64_t M, int64_t N, int64_t ldx, int64_t ldy, int LPR,
                          void* __restrict__ dgamma, void* __restrict__ dbeta, int out_dtype,
                          int accumulate) {
  using PK = Pack<Tg, VEC>;
  constexpr int EB = Tg::kBytes;
  const char* __restrict__ x = static_cast<const char*>(xv);
  const char* __restrict__ dy = static_cast<const char*>(dyv);
  __shared__ float part[NACC][kWgradWaves][kWgradMaxTile];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int RPW = 64 / LPR;
  const int c = lane % LPR;
  const int slot = lane / LPR;
  const int TW = LPR * VEC;
  const int64_t T = gridDim.x;
  const int64_t tile = (T % kXcds == 0)
                           ? (int64_t)(blockIdx.x % kXcds) * (T / kXcds) + blockIdx.x / kXcds
                           : (int64_t)blockIdx.x;
  const int64_t col = tile * TW + (int64_t)c * VEC;
  const bool colok = col < N;  // N is a multiple of VEC on this path
  const int64_t rstep = (int64_t)kWgradWaves * RPW;

  float ag[VEC], ab[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    ag[v] = 0.0f;
    ab[v] = 0.0f;
  }

  // rows of this lane: r0, r0 + rstep, ...; kWgradUnroll of them are loaded
  // before they are added, in ascending order
  for (int64_t r0 = (int64_t)wave * RPW + slot; r0 < M; r0 += rstep * kWgradUnroll) {
    PK xb[kWgradUnroll], yb[kWgradUnroll];
    float mu[kWgradUnroll], rs[kWgradUnroll];
#pragma unroll
    for (int u = 0; u < kWgradUnroll; ++u) {
      const int64_t r = r0 + u * rstep;
      if (colok && r < M) {
        xb[u].load(x + (r * ldx + col) * EB);
        yb[u].load(dy + (r * ldy + col) * EB);
        rs[u] = rstd[r];
        mu[u] = (KIND == kLayerNorm) ? mean[r] : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kWgradUnroll; ++u) {
      const int64_t r = r0 + u * rstep;
      if (colok && r < M) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const float dyv = yb[u].get(v);
          ag[v] = __builtin_fmaf(dyv * (xb[u].get(v) - mu[u]), rs[u], ag[v]);
          if (NACC == 2) ab[v] += dyv;
        }
      }
    }
  }

  // add the RPW row slots of the wave (lanes c, c + LPR, c + 2 LPR, ...)
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      ag[v] += __shfl_xor(ag[v], off);
      if (NACC == 2) ab[v] += __shfl_xor(ab[v], off);
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      part[0][wave][c * VEC + v] = ag[v];
      if (NACC == 2) part[NACC - 1][wave][c * VEC + v] = ab[v];
    }
  }
  __syncthreads();
  // thread t < NACC * TW finishes column t % TW of plane t / TW: the wave
  // sums in wave order, then the optional previous value
  const int t = threadIdx.x;
  if (t < NACC * TW) {
    const int plane = t / TW, j = t % TW;
    const int64_t oc = tile * TW + j;
    if (oc < N) {
      float s = part[plane][0][j];
      for (int w = 1; w < kWgradWaves; ++w) s += part[plane][w][j];
      void* out = plane == 0 ? dgamma : dbeta;
      switch (out_dtype) {
        case 0: put_out<TF32>(out, oc, s, accumulate != 0); break;
        case 1: put_out<TF16>(out, oc, s, accumulate != 0); break;
        default: put_out<TBF16>(out, oc, s, accumulate != 0); break;
      }
    }
  }
}

}  // namespace nb
