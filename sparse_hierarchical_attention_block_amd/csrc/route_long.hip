// route_long.hip -- Stage 1 of DashAttention ("entmax chunk routing",
// DashAttention explainer, Technical summary) for query tiles with 129 to 512
// candidate blocks and bf16 queries: coarse scores held in MFMA
// accumulators, the alpha-entmax threshold per (position, head) row, the GQA
// average, the Stage 2 bias and the tile's union, as in route.hip's
// tile-resident kernel but for rows too long for one wave per 64 rows.
#include "dash_internal.hpp"
#include "device_common.hpp"
#include "entmax_device.hpp"
#include "route_common.hpp"

namespace dash {

// ------------------------------------------------------------------------------------------
// Long rows (up to 512 candidates, bf16 queries, G >= 2).  The tile's 64 G
// rows are cut into G / 2 parts of 128 rows (128 / G positions x the G heads
// of a position), one workgroup of 8 waves per part and 16 rows per wave.
// As in the tile-resident kernel, a row's scores stay in MFMA accumulators --
// here for 32 candidate tiles of 16 -- but the summaries stream through LDS
// 64 candidates at a time: each part loads and splits every summary row once
// (the pass-based kernel reloads and resplits them for every pass of a few
// positions).  With one part (G = 2) the workgroup compacts the tile's list
// itself; otherwise each part leaves its union as bit-packed words at the
// front of the tile's sel_idx row and route_merge_kernel ORs the parts and
// compacts.
// ------------------------------------------------------------------------------------------
constexpr int kLongChunk = 64;     // candidates per staged chunk
constexpr int kLongThreads = 512;  // 8 waves x 16 rows
constexpr int kLongRows = 16 * kLongThreads / kWave;   // rows per part

template <int D, int MODE, int G>
__global__ __launch_bounds__(kLongThreads) void route_long_kernel(RouteArgs a) {
  constexpr int SP = D + 8;                                 // plane row pitch (bf16)
  constexpr int KS = D / 32;
  constexpr int CCT = kLongChunk / 16;                      // candidate tiles per chunk
  constexpr int SV = kLongChunk * (D / 4) / kLongThreads;   // float4s per thread per chunk
  static_assert(SV >= 1, "one chunk covers every thread");
  __shared__ __attribute__((aligned(16))) __bf16 planes[3 * kLongChunk * SP];   // hi, mid, lo
  extern __shared__ int lflag[];                            // [pitch] union flags of the part

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int l16 = lane % 16, lg = lane / 16;
  constexpr int parts = kQT * G / kLongRows, ppos = kQT / parts;   // positions per part
  const int64_t nbg = (int64_t)a.B * a.Hkv;
  const int part = (int)(blockIdx.x % parts);
  const int64_t rank = blockIdx.x / parts;
  const int64_t qt = a.n_qt - 1 - rank / nbg;               // heaviest tiles first
  const int64_t bg = rank % nbg;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t p_begin = qt * kQT;
  const int t = max(0, (int)(p_begin / a.bs) - (a.window - 1));   // candidates
  const int64_t tile = bg * a.n_qt + qt;
  a.nv = valid_len(a.seq_len, b, a.n);
  if (p_begin >= a.nv) {
    if (parts == 1) route_tile_past_end(a, tile);
    return;
  }
  const int r = 16 * wave + l16;          // row within the part
  const int m = r / G, h = r % G;
  const int64_t pos = p_begin + part * ppos + m;
  const int64_t rglob = ((int64_t)b * a.H + g * G + h) * a.n + pos;
  if (t == 0) {
    if (lg == 0 && pos < a.nv) {
      a.tau[rglob] = __builtin_nanf("");
      if (a.bits)
        for (int w = 0; w < a.nwords; ++w) a.bits[rglob * a.nwords + w] = 0u;
    }
    if (parts == 1) {
      if (threadIdx.x == 0) a.sel_count[tile] = 0;
      if (a.tile_bits)
        for (int w = threadIdx.x; w < a.nwords; w += kLongThreads) a.tile_bits[tile * a.nwords + w] = 0u;
    }
    return;
  }
  const int CT = (t + 15) / 16;
  for (int j = threadIdx.x; j < a.pitch; j += kLongThreads) lflag[j] = 0;

  // Q^T fragments of the wave's 16 rows: column = row l16, k = d in [32 s + 8 lg, +8)
  bf16x8 qf[KS];
  {
    const __bf16* qrow = (const __bf16*)a.q + rglob * D;
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      u32x4 qv = {0u, 0u, 0u, 0u};
      if (pos < a.nv) qv = *(const u32x4*)(qrow + 32 * s2 + 8 * lg);
      qf[s2] = as_bf16x8(qv);
    }
  }
  // a chunk of summary rows: loaded into registers one chunk ahead, split
  // into the three bf16 planes when stored
  // (a buffer resource over the t candidate rows: loads past them return
  // zeros without a branch, so nothing waits on them before the next store)
  const buf_rsrc srs = make_rsrc(a.summ + bg * a.summ_blocks * D, (uint32_t)t * D * 4);
  f32x4 pre[SV];
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int u = 0; u < SV; ++u) {
      const int e = threadIdx.x + u * kLongThreads;
      const int cand = e / (D / 4), c4 = e % (D / 4);
      pre[u] = __builtin_bit_cast(f32x4, buf_load16(srs, (uint32_t)(((c0 + cand) * D + 4 * c4) * 4)));
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int u = 0; u < SV; ++u) {
      const int e = threadIdx.x + u * kLongThreads;
      const int cand = e / (D / 4), c4 = e % (D / 4);
      const float xs[4] = {pre[u].x, pre[u].y, pre[u].z, pre[u].w};
      // scale folded into the summaries, then split exactly into hi + mid + lo
      uint32_t hw[2], mw[2], lw[2];
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2)
        split3_bf16(xs[2 * p2] * a.scale, xs[2 * p2 + 1] * a.scale, hw[p2], mw[p2], lw[p2]);
      const int off = cand * SP + 4 * c4;
      *(u32x2*)(planes + off) = (u32x2){hw[0], hw[1]};
      *(u32x2*)(planes + kLongChunk * SP + off) = (u32x2){mw[0], mw[1]};
      *(u32x2*)(planes + 2 * kLongChunk * SP + off) = (u32x2){lw[0], lw[1]};
    }
  };

  // ---- scores: X[ct][i] = x(row r, cand 16 ct + 4 lg + i) ----
  f32x4 X[kLongMaxCT];
#pragma unroll
  for (int ct = 0; ct < kLongMaxCT; ++ct) X[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
  load_chunk(0);
#pragma unroll
  for (int c = 0; c < kLongMaxCT / CCT; ++c) {
    if (c * CCT >= CT) break;
    __syncthreads();   // every wave is done with the previous chunk's planes
    store_chunk();
    __syncthreads();
    if ((c + 1) * CCT < CT) load_chunk((c + 1) * kLongChunk);
#pragma unroll
    for (int k = 0; k < CCT; ++k) {
      if (c * CCT + k < CT) {
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
          const int off = (16 * k + l16) * SP + 32 * s2 + 8 * lg;
          const bf16x8 hi = as_bf16x8(*(const u32x4*)(planes + off));
          const bf16x8 mid = as_bf16x8(*(const u32x4*)(planes + kLongChunk * SP + off));
          const bf16x8 lo = as_bf16x8(*(const u32x4*)(planes + 2 * kLongChunk * SP + off));
          X[c * CCT + k] = mfma16(lo, qf[s2], X[c * CCT + k]);
          X[c * CCT + k] = mfma16(mid, qf[s2], X[c * CCT + k]);
          X[c * CCT + k] = mfma16(hi, qf[s2], X[c * CCT + k]);
        }
      }
    }
  }

  // ---- threshold, support bits, pbar and the Stage 2 bias, in the accumulators ----
  // (candidates past t in the last candidate tile become -inf; tiles at or
  // past CT are never read)
  static_for<0, kLongMaxCT>([&](auto CTc) {
    constexpr int ct = decltype(CTc)::value;
    if (ct == CT - 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (16 * ct + 4 * lg + i >= t) X[ct][i] = -INFINITY;
    }
  });
  const float tau = entmax_tau_reg<4 * kLongMaxCT, MODE>(X, Stride16Reduce{}, a.e, CT);
  if (a.bits) {
    // ballots give, for each (ct, i), the bit of every (row, lg) pair
    uint32_t chunk[kLongMaxCT];
#pragma unroll
    for (int ct = 0; ct < kLongMaxCT; ++ct) {
      chunk[ct] = 0u;
      if (ct < CT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint64_t mk = __ballot(X[ct][i] > tau);
#pragma unroll
          for (int l2 = 0; l2 < 4; ++l2)
            chunk[ct] |= (uint32_t)((mk >> (16 * l2 + l16)) & 1ull) << (4 * l2 + i);
        }
      }
    }
    if (lg == 0 && pos < a.nv)
      for (int w = 0; w < a.nwords; ++w) {
        uint32_t word = 0u;
#pragma unroll
        for (int ct = 0; ct < kLongMaxCT; ++ct)
          if (ct / 2 == w) word |= chunk[ct] << (16 * (ct % 2));
        a.bits[rglob * a.nwords + w] = word;
      }
  }
  if (lg == 0 && pos < a.nv) a.tau[rglob] = tau;
  static_for<0, kLongMaxCT>([&](auto CTc) {
    constexpr int ct = decltype(CTc)::value;
    if (ct < CT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) X[ct][i] = entmax_prob<MODE>(X[ct][i] - tau, a.e);
    }
  });
  route_rows_bias<G, kLongMaxCT>(a, X, CT, t, lg, h, pos, p_begin, tile, lflag);
  __syncthreads();
  if (threadIdx.x >= kWave) return;
  if (parts == 1) {
    compact_union(a, lflag, t, tile);
    return;
  }
  // this part's union, bit-packed, at words part * nwords + w (w < ceil(t /
  // 32), so no part writes into the next one's words) of the tile's sel_idx
  // row (parts * nwords <= nb whenever t > 128)
  uint32_t* words = (uint32_t*)(a.sel_idx + tile * a.nb) + part * a.nwords;
  const int nwt = (t + 31) / 32;
  for (int j0 = 0; j0 < t; j0 += kWave) {
    const uint64_t mask = __ballot(j0 + lane < t && lflag[j0 + lane] != 0);
    if (lane < 2 && j0 / 32 + lane < nwt) words[j0 / 32 + lane] = (uint32_t)(mask >> (32 * lane));
  }
}

// The parts' union words of each tile (route_long_kernel) ORed into the
// tile's list: one wave per tile.  Every word is read into a register before
// the list, which overwrites them, is written.
__global__ __launch_bounds__(kWave) void route_merge_kernel(RouteArgs a, int parts) {
  const int64_t tile = blockIdx.x;
  const int64_t qt = tile % a.n_qt, bg = tile / a.n_qt;
  const int b = (int)(bg / a.Hkv);
  const int lane = threadIdx.x;
  const int64_t p_begin = qt * kQT;
  const int t = p_begin < valid_len(a.seq_len, b, a.n)
                    ? max(0, (int)(p_begin / a.bs) - (a.window - 1)) : 0;
  const int nwt = (t + 31) / 32;   // <= 16 words (t <= 512)
  int32_t* row = a.sel_idx + tile * a.nb;
  uint32_t wv = 0u;
  if (lane < nwt)
    for (int p = 0; p < parts; ++p) wv |= ((const uint32_t*)row)[p * a.nwords + lane];
  int base = 0;
  for (int j0 = 0; j0 < t; j0 += kWave) {
    const uint32_t w0 = __shfl(wv, j0 / 32), w1 = __shfl(wv, j0 / 32 + 1);
    const uint64_t mask = ((uint64_t)w1 << 32 | w0) &
                          (t - j0 >= kWave ? ~0ull : ((1ull << (t - j0)) - 1ull));
    if ((mask >> lane) & 1ull) row[base + __popcll(mask & ((1ull << lane) - 1ull))] = j0 + lane;
    base += __popcll(mask);
  }
  if (a.tile_bits)   // nwt <= 16, so a word below nwt is this lane's own
    for (int w = lane; w < a.nwords; w += kWave) a.tile_bits[tile * a.nwords + w] = w < nwt ? wv : 0u;
  if (lane == 0) a.sel_count[tile] = base;
}

hipError_t launch_route_long(RouteArgs a, const Shape& s, int t_max, hipStream_t st) {
  // workgroups of 128 rows, scores in registers
  a.pitch = round_up16(t_max);
  const int parts = kQT * s.G / kLongRows;
  const size_t lds = (size_t)a.pitch * 4;
  dim3 grid_l((unsigned)(a.n_qt * s.B * s.Hkv * parts));
#define DASH_RL(D, M)                                                                        \
  do {                                                                                       \
    if (s.G == 2)                                                                            \
      hipLaunchKernelGGL((route_long_kernel<D, M, 2>), grid_l, dim3(kLongThreads), lds, st, a); \
    else if (s.G == 4)                                                                       \
      hipLaunchKernelGGL((route_long_kernel<D, M, 4>), grid_l, dim3(kLongThreads), lds, st, a); \
    else                                                                                     \
      hipLaunchKernelGGL((route_long_kernel<D, M, 8>), grid_l, dim3(kLongThreads), lds, st, a); \
  } while (0)
#define DASH_RL2(D)                                                \
  do {                                                             \
    if (a.mode == kEntmax15) DASH_RL(D, kEntmax15);                \
    else if (a.mode == kSparsemax) DASH_RL(D, kSparsemax);         \
    else if (a.mode == kEntmaxQuartic) DASH_RL(D, kEntmaxQuartic); \
    else DASH_RL(D, kEntmaxGeneral);                               \
  } while (0)
  if (s.d == 64) DASH_RL2(64); else DASH_RL2(128);
#undef DASH_RL2
#undef DASH_RL
  if (parts > 1)
    hipLaunchKernelGGL(route_merge_kernel, dim3((unsigned)(a.n_qt * s.B * s.Hkv)), dim3(kWave), 0,
                       st, a, parts);
  return hipGetLastError();
}

}  // namespace dash
