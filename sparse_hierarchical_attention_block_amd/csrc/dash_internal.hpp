// dash_internal.hpp -- host-side launchers shared between the C ABI layer
// (api.cpp) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dash.h"

namespace dash {

// Validated problem shape.
struct Shape {
  int B, H, Hkv, G, d, bs;
  float alpha, gamma;
  int dtype;  // dash_dtype
  float sigma;   // prior strength: routed-block bias sigma * log pbar
  int window;    // near-diagonal branch: own block + window - 1 blocks before it
};

// Stage 0: summaries of blocks [blk_begin, blk_end) for every (b, kv head);
// q_bar is nullptr (mean pooling) or [Hkv, d] summary queries.
// seq_len: null, or [B] valid positions per sequence (only its complete
// blocks are summarised); the same for the two prefill launches below.
hipError_t launch_summarize(const Shape& s, const void* k, int64_t kv_len, int64_t blk_begin,
                            int64_t blk_end, const float* w_s, const float* q_bar, float* summ,
                            int64_t summ_blocks, hipStream_t st,
                            const int32_t* seq_len = nullptr);

// Stage 1, causal prefill of positions 0..n-1.
hipError_t launch_route_prefill(const Shape& s, const void* q, int64_t n, const float* summ,
                                int64_t summ_blocks, const dash_route_buf& rb, hipStream_t st,
                                const int32_t* seq_len = nullptr);

// Bit-packed tile masks -> ascending lists (prefill layout).
hipError_t launch_mask_to_list(const Shape& s, int64_t n, const dash_route_buf& rb,
                               hipStream_t st);

// Stage 2, causal prefill.
hipError_t launch_attend_prefill(const Shape& s, const void* q, const void* k, const void* v,
                                 int64_t n, const dash_route_buf& rb, void* o, hipStream_t st,
                                 const int32_t* seq_len = nullptr);

// Decode workspace layout (byte offsets from the workspace base).
struct DecodeLayout {
  int64_t nb;          // ceil(max_len / bs)
  int64_t ncand_max;   // (max_len - 1) / bs
  int64_t n_split;     // splits of the (own + selected) block list
  size_t off_x, off_tau, off_count, off_idx, off_logp, off_part, total;
};
DecodeLayout decode_layout(const Shape& s, int64_t max_len);
// Prefill routing, pass-based path (rows longer than 128 candidates): threads
// per workgroup and the LDS bytes its per-pass score buffer may use.
#ifndef DASH_ROUTE_PASS_THREADS
#define DASH_ROUTE_PASS_THREADS 512
#endif
#ifndef DASH_ROUTE_X_BUDGET
#define DASH_ROUTE_X_BUDGET (80 * 1024)
#endif

constexpr int kDecodeSplit = 32;   // list entries (blocks) per split (8 per wave)
constexpr int kDecodeMaxBg = 8192; // sequences x KV heads of one bf16 decode call
constexpr int kMaxDevices = 64;    // per-device launch-shape caches

// One decode step (route, attend, combine, summary update).  block_table
// null: contiguous caches [B, Hkv, max_len, d]; otherwise paged caches
// [num_pages, Hkv, bs, d] with block j of sequence b in page
// block_table[b * max_blocks + j].
hipError_t launch_decode(const Shape& s, const void* q, const void* kc, const void* vc,
                         const int32_t* cache_len, int64_t max_len, const float* w_s,
                         const float* q_bar, float* summ, int64_t summ_blocks, void* o,
                         const dash_route_buf& rb,
                         const DecodeLayout& L, char* ws, hipStream_t st,
                         const int32_t* block_table = nullptr, int64_t max_blocks = 0,
                         int64_t num_pages = 0);

// Backward pass of the causal prefill (mean-pooled summaries): workspace
// layout and launch.
struct BwdLayout {
  size_t off_lse, off_delta, off_dlogp, off_u, off_ds, off_mean, off_dm, off_dspart, off_wspart,
      total;
  int64_t slab;   // query tiles per slab of the per-tile arrays
};
BwdLayout bwd_layout(const Shape& s, int64_t n);
hipError_t launch_prefill_backward(const Shape& s, const void* q, const void* k, const void* v,
                                   const void* o, const void* dO, int64_t n, const float* w_s,
                                   const float* summ, int64_t summ_blocks,
                                   const dash_route_buf& rb, float* dq, float* dk, float* dv,
                                   float* dw_s, const BwdLayout& L, char* ws, hipStream_t st);

}  // namespace dash
