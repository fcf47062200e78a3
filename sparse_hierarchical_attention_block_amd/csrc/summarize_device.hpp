// summarize_device.hpp -- the block-summary routine of Stage 0 of
// DashAttention ("local chunk summarization", DashAttention explainer,
// Technical summary): s_j = mean(k of block j) . W_s, accumulated in float32.
// Used by the summary kernel of dash_summarize and dash_prefill, and by the
// decode step for the block it completes.
//
// HBM-bound scan: every key of a block is read once with 16-byte loads
// (bs * d * elt bytes per block); the projection reads W_s (d x d float32,
// L2-resident) once for all the blocks a call summarises.
#pragma once

#include "device_common.hpp"

namespace dash {

constexpr int kSumThreads = 256;

// Summaries of nblk <= NB consecutive blocks.  kb points at the first key row
// of the first block (rows of D elements, blocks of bs rows, contiguous), out
// at the first summary (D floats per block, contiguous).  All 256 threads call.
template <typename T, int D, int NB>
__device__ void summarize_blocks(const T* __restrict__ kb, int nblk, int bs,
                                 const float* __restrict__ w_s, float* __restrict__ out) {
  constexpr int EPV = 16 / sizeof(T);       // elements per 16-byte load
  constexpr int CH = D / EPV;               // 16-byte chunks per row
  constexpr int RG = kSumThreads / CH;      // row groups
  __shared__ float part[RG][D];
  __shared__ float mean[NB][D];
  const int ch = threadIdx.x % CH, rg = threadIdx.x / CH;
  // this thread's W_s entries (column c, rows pg + PG i), loaded before the
  // keys so that both arrive in one memory round trip
  constexpr int PG = kSumThreads / D;
  const int c = threadIdx.x % D, pg = threadIdx.x / D;
  float wcol[D / PG];
#pragma unroll
  for (int i = 0; i < D / PG; ++i) wcol[i] = w_s[(pg + PG * i) * D + c];
  for (int bi = 0; bi < nblk; ++bi) {
    const T* blk = kb + (int64_t)bi * bs * D;
    float acc[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] = 0.f;
#pragma unroll 4
    for (int t = rg; t < bs; t += RG) {
      const u32x4 w = *(const u32x4*)(blk + (int64_t)t * D + ch * EPV);
      if constexpr (sizeof(T) == 2) {
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += bf16_lo(ww[e]);
          acc[2 * e + 1] += bf16_hi(ww[e]);
        }
      } else {
        acc[0] += __uint_as_float(w.x);
        acc[1] += __uint_as_float(w.y);
        acc[2] += __uint_as_float(w.z);
        acc[3] += __uint_as_float(w.w);
      }
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e) part[rg][ch * EPV + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < RG; ++r) s += part[r][threadIdx.x];
      mean[bi][threadIdx.x] = s * (1.0f / (float)bs);
    }
    __syncthreads();
  }
  // projection: out[bi][c] = sum_r mean[bi][r] * W_s[r][c], r split over the
  // 256 / D row groups; W_s is read once for all blocks
  float o[NB];
#pragma unroll
  for (int bi = 0; bi < NB; ++bi) o[bi] = 0.f;
#pragma unroll
  for (int i = 0; i < D / PG; ++i) {
    const int r = pg + PG * i;
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) o[bi] = fmaf(mean[bi][r], wcol[i], o[bi]);
  }
  // `part` is reused as [PG][NB][D]
  static_assert(RG >= PG * NB, "LDS scratch too small");
#pragma unroll
  for (int bi = 0; bi < NB; ++bi) (&part[0][0])[(pg * NB + bi) * D + c] = o[bi];
  __syncthreads();
  if (threadIdx.x < D) {
    for (int bi = 0; bi < nblk; ++bi) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < PG; ++q) s += (&part[0][0])[(q * NB + bi) * D + threadIdx.x];
      out[bi * D + threadIdx.x] = s;
    }
  }
  __syncthreads();
}

}  // namespace dash
