// summarize_device.hpp -- the block-summary routine of Stage 0 of
// DashAttention ("local chunk summarization", DashAttention explainer,
// Technical summary): a block's keys are pooled into one vector m_j, and
// s_j = m_j . W_s, accumulated in float32.  Pooling is the uniform mean, or,
// given the KV head's summary query qbar, scaled dot-product attention of
// qbar over the block's keys (the keys are also the values):
// m_j = sum_t softmax_t(qbar . k_t / sqrt(d)) k_t.  A zero query is the mean.
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
// One 16-byte load of key elements as floats.
template <typename T>
__device__ __forceinline__ void load_key_chunk(const T* __restrict__ p,
                                               float (&x)[16 / sizeof(T)]) {
  const u32x4 w = *(const u32x4*)p;
  if constexpr (sizeof(T) == 2) {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_lo(ww[e]);
      x[2 * e + 1] = bf16_hi(ww[e]);
    }
  } else {
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z);
    x[3] = __uint_as_float(w.w);
  }
}

// Summaries of nblk <= NB consecutive blocks.  kb points at the first key row
// of the first block (rows of D elements, blocks of bs rows, contiguous), out
// at the first summary (D floats per block, contiguous).  qbar is nullptr
// (uniform pooling) or the D float32 summary query of the blocks' KV head.
// All 256 threads call.
template <typename T, int D, int NB>
__device__ void summarize_blocks(const T* __restrict__ kb, int nblk, int bs,
                                 const float* __restrict__ w_s, const float* __restrict__ qbar,
                                 float* __restrict__ out) {
  constexpr int EPV = 16 / sizeof(T);       // elements per 16-byte load
  constexpr int CH = D / EPV;               // 16-byte chunks per row
  constexpr int RG = kSumThreads / CH;      // row groups
  __shared__ float part[RG][D];
  __shared__ float mean[NB][D];
  __shared__ float gmax[RG], gsum[RG];
  const int ch = threadIdx.x % CH, rg = threadIdx.x / CH;
  // this thread's W_s entries (column c, rows pg + PG i), loaded before the
  // keys so that both arrive in one memory round trip
  constexpr int PG = kSumThreads / D;
  const int c = threadIdx.x % D, pg = threadIdx.x / D;
  float wcol[D / PG];
#pragma unroll
  for (int i = 0; i < D / PG; ++i) wcol[i] = w_s[(pg + PG * i) * D + c];
  if (qbar == nullptr) {
    for (int bi = 0; bi < nblk; ++bi) {
      const T* blk = kb + (int64_t)bi * bs * D;
      float acc[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[e] = 0.f;
#pragma unroll 4
      for (int t = rg; t < bs; t += RG) {
        float x[EPV];
        load_key_chunk<T>(blk + (int64_t)t * D + ch * EPV, x);
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] += x[e];
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
  } else {
    // Attention pooling.  The CH lanes of a row are consecutive, so a row's
    // score is a CH-lane reduction; each row group keeps an online softmax
    // (running max, running sum, rescaled accumulator) over its rows, in
    // base-2 units (the query is pre-scaled by log2(e) / sqrt(d)); the row
    // groups are merged through LDS.
    float qv[EPV];
    const float qscale = kLog2e * rsqrtf((float)D);
#pragma unroll
    for (int e = 0; e < EPV; ++e) qv[e] = qbar[ch * EPV + e] * qscale;
    for (int bi = 0; bi < nblk; ++bi) {
      const T* blk = kb + (int64_t)bi * bs * D;
      float acc[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[e] = 0.f;
      float mrun = -INFINITY, lrun = 0.f;
#pragma unroll 4
      for (int t = rg; t < bs; t += RG) {
        float x[EPV];
        load_key_chunk<T>(blk + (int64_t)t * D + ch * EPV, x);
        float z = 0.f;
#pragma unroll
        for (int e = 0; e < EPV; ++e) z = fmaf(qv[e], x[e], z);
        z = group_reduce(z, CH, DppAdd{});
        const float mnew = fmaxf(mrun, z);
        const float corr = fast_exp2(mrun - mnew);   // 0 on the first row
        const float pw = fast_exp2(z - mnew);
        lrun = fmaf(lrun, corr, pw);
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] = fmaf(acc[e], corr, pw * x[e]);
        mrun = mnew;
      }
#pragma unroll
      for (int e = 0; e < EPV; ++e) part[rg][ch * EPV + e] = acc[e];
      if (ch == 0) {
        gmax[rg] = mrun;
        gsum[rg] = lrun;
      }
      __syncthreads();
      if (threadIdx.x < D) {
        float m = -INFINITY;
#pragma unroll
        for (int r = 0; r < RG; ++r) m = fmaxf(m, gmax[r]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          const float f = fast_exp2(gmax[r] - m);
          num = fmaf(f, part[r][threadIdx.x], num);
          den = fmaf(f, gsum[r], den);
        }
        mean[bi][threadIdx.x] = num / den;
      }
      __syncthreads();
    }
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
