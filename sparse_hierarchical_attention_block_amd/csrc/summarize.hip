// summarize.hip -- Stage 0 of DashAttention ("local chunk summarization",
// DashAttention explainer, Technical summary): one summary per complete key
// block, s_j = pool(k of block j) . W_s, accumulated in float32, where pool is
// the mean or the summary query's local attention over the block.  A chunk's
// summary is computed once, when the chunk is complete, and cached.
//
// HBM-bound scan: every key of a complete block is read once with 16-byte
// loads (bs * d * elt bytes per block).  A workgroup summarises up to NB
// blocks of one (sequence, KV head) so W_s (64 KB at d = 128, L2-resident) is
// read once per NB blocks.
#include "dash_internal.hpp"
#include "device_common.hpp"
#include "summarize_device.hpp"

namespace dash {

constexpr int kSumNB = 2;   // blocks per workgroup (2 measured best: more workgroups, W_s still shared)

// grid.x = ceil(nblk / NB) * B * Hkv
template <typename T, int D>
__global__ __launch_bounds__(kSumThreads) void summarize_kernel(
    const T* __restrict__ k, int64_t kv_len, int bs, int64_t blk_begin, int64_t nblk,
    const float* __restrict__ w_s, const float* __restrict__ q_bar, int hkv,
    float* __restrict__ summ, int64_t summ_blocks, const int32_t* __restrict__ seq_len) {
  const int64_t ngrp = (nblk + kSumNB - 1) / kSumNB;
  const int64_t u = blockIdx.x;
  const int64_t grp = u % ngrp, bg = u / ngrp;
  const int64_t j = blk_begin + grp * kSumNB;
  // blocks of this group that exist: with per-sequence lengths, only the
  // complete blocks of that sequence
  int64_t end = blk_begin + nblk;
  if (seq_len) {
    const int64_t l = seq_len[bg / hkv];
    end = min(end, (l < 0 ? 0 : min(l, kv_len)) / bs);
  }
  const int here = (int)min((int64_t)kSumNB, end - j);
  if (here <= 0) return;
  const float* qb = q_bar ? q_bar + (bg % hkv) * D : nullptr;
  summarize_blocks<T, D, kSumNB>(k + (bg * kv_len + j * bs) * D, here, bs, w_s, qb,
                                 summ + (bg * summ_blocks + j) * D);
}

template <typename T, int D>
static hipError_t summarize_t(const Shape& s, const void* k, int64_t kv_len, int64_t b0,
                              int64_t b1, const float* w_s, const float* q_bar, float* summ,
                              int64_t sb, hipStream_t st, const int32_t* seq_len) {
  const int64_t nblk = b1 - b0;
  dim3 grid((unsigned)(((nblk + kSumNB - 1) / kSumNB) * s.B * s.Hkv));
  hipLaunchKernelGGL((summarize_kernel<T, D>), grid, dim3(kSumThreads), 0, st,
                     (const T*)k, kv_len, s.bs, b0, nblk, w_s, q_bar, s.Hkv, summ, sb, seq_len);
  return hipGetLastError();
}

hipError_t launch_summarize(const Shape& s, const void* k, int64_t kv_len, int64_t blk_begin,
                            int64_t blk_end, const float* w_s, const float* q_bar, float* summ,
                            int64_t summ_blocks, hipStream_t st, const int32_t* seq_len) {
  if (blk_end <= blk_begin) return hipSuccess;
  if (s.dtype == DASH_BF16)
    return s.d == 64 ? summarize_t<__bf16, 64>(s, k, kv_len, blk_begin, blk_end, w_s, q_bar,
                                               summ, summ_blocks, st, seq_len)
                     : summarize_t<__bf16, 128>(s, k, kv_len, blk_begin, blk_end, w_s, q_bar,
                                                summ, summ_blocks, st, seq_len);
  return s.d == 64 ? summarize_t<float, 64>(s, k, kv_len, blk_begin, blk_end, w_s, q_bar, summ,
                                            summ_blocks, st, seq_len)
                   : summarize_t<float, 128>(s, k, kv_len, blk_begin, blk_end, w_s, q_bar, summ,
                                             summ_blocks, st, seq_len);
}

}  // namespace dash
