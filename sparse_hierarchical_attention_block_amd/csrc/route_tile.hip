// route_tile.hip -- Stage 1 of DashAttention ("entmax chunk routing",
// DashAttention explainer, Technical summary) for query tiles with at most 128
// candidate blocks and bf16 queries.
#include "dash_internal.hpp"
#include "device_common.hpp"
#include "entmax_device.hpp"
#include "route_common.hpp"

namespace dash {

// ------------------------------------------------------------------------------------------
// Tile-resident variant for up to 128 candidates (bf16 queries): the whole
// tile's scores stay in MFMA accumulator registers.  The workgroup splits
// the tile's summaries once into three bf16 planes in LDS; wave w owns RTW
// 16-row tiles (one for G <= 4, so a tile of 64 G rows runs on 4 G waves and
// each SIMD keeps several waves to hide VALU latency) and computes X^T = S Q^T for every
// candidate tile with MFMA 16x16x32.  In the accumulator a row's values sit in
// lanes l16, l16+16, l16+32, l16+48, so the entmax reductions are two lane
// swaps; the G heads of a position are adjacent rows (lanes differing in the
// low bits of l16), so the GQA sum is log2(G) more swaps.
// ------------------------------------------------------------------------------------------

template <int D, int MODE, int G>
__global__ __launch_bounds__(1024) void route_tile_kernel(RouteArgs a) {
  constexpr int RTW = G <= 4 ? 1 : 2;             // row tiles of 16 per wave
  extern __shared__ __attribute__((aligned(16))) char tsm[];
  constexpr int SP = D + 8;                       // plane row pitch (bf16)
  constexpr int KS = D / 32;
  const int TP = a.pitch;                         // candidate rows per plane (x16)
  __bf16* planes = (__bf16*)tsm;                  // [3][TP][SP]: hi, mid, lo
  int* uflag = (int*)(tsm + (size_t)3 * TP * SP * 2);

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int l16 = lane % 16, lg = lane / 16;
  const int nthreads = blockDim.x;
  const int64_t nbg = (int64_t)a.B * a.Hkv;
  const int64_t qt = a.n_qt - 1 - blockIdx.x / nbg;   // heaviest tiles first
  const int64_t bg = blockIdx.x % nbg;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t p_begin = qt * kQT;
  const int t = max(0, (int)(p_begin / a.bs) - (a.window - 1));   // candidates
  const int64_t tile = bg * a.n_qt + qt;
  a.nv = valid_len(a.seq_len, b, a.n);
  if (p_begin >= a.nv) {
    route_tile_past_end(a, tile);
    return;
  }

  if (t == 0) {
    const int npos = (int)min((int64_t)kQT, a.nv - p_begin);
    for (int idx = threadIdx.x; idx < npos * G; idx += nthreads) {
      const int m = idx / G, h = idx % G;
      const int64_t r = ((int64_t)b * a.H + g * G + h) * a.n + p_begin + m;
      a.tau[r] = __builtin_nanf("");
      if (a.bits)
        for (int w = 0; w < a.nwords; ++w) a.bits[r * a.nwords + w] = 0u;
    }
    if (threadIdx.x == 0) a.sel_count[tile] = 0;
    if (a.tile_bits)
      for (int w = threadIdx.x; w < a.nwords; w += blockDim.x) a.tile_bits[tile * a.nwords + w] = 0u;
    return;
  }
  const int CT = (t + 15) / 16;

  // ---- stage the summaries, split into hi + mid + lo bf16 ----
  // (batches of 8 loads per thread are issued before any is consumed)
  const int n4 = CT * 16 * (D / 4);
  for (int e0 = threadIdx.x; e0 < n4; e0 += 8 * nthreads) {
    f32x4 vb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * nthreads;
      const int cand = e / (D / 4), c4 = e % (D / 4);
      vb[u] = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (e < n4 && cand < t) vb[u] = *(const f32x4*)(a.summ + (bg * a.summ_blocks + cand) * D + 4 * c4);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + u * nthreads;
      if (e >= n4) break;
      const int cand = e / (D / 4), c4 = e % (D / 4);
      const float xs[4] = {vb[u].x, vb[u].y, vb[u].z, vb[u].w};
      uint32_t hw[2], mw[2], lw[2];
#pragma unroll
      for (int p2 = 0; p2 < 2; ++p2) {
        float hv[2], mv[2], lv[2];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const float x = xs[2 * p2 + q2] * a.scale;   // scale folded into the summaries
          const float h = (float)(__bf16)x;
          const float r1 = x - h;
          const float m = (float)(__bf16)r1;
          hv[q2] = h;
          mv[q2] = m;
          lv[q2] = r1 - m;
        }
        hw[p2] = pack_bf16(hv[0], hv[1]);
        mw[p2] = pack_bf16(mv[0], mv[1]);
        lw[p2] = pack_bf16(lv[0], lv[1]);
      }
      const int off = cand * SP + 4 * c4;
      *(u32x2*)(planes + off) = (u32x2){hw[0], hw[1]};
      *(u32x2*)(planes + (size_t)TP * SP + off) = (u32x2){mw[0], mw[1]};
      *(u32x2*)(planes + (size_t)2 * TP * SP + off) = (u32x2){lw[0], lw[1]};
    }
  }
  for (int j = threadIdx.x; j < TP; j += nthreads) uflag[j] = 0;

  // ---- Q^T fragments of the wave's RTW row tiles ----
  const __bf16* q = (const __bf16*)a.q;
  bf16x8 qf[RTW][KS];
  int64_t rpos[RTW];
  int rh[RTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const int r = 16 * RTW * wave + 16 * rt + l16;
    const int m = r / G, h = r % G;
    rpos[rt] = p_begin + m;
    rh[rt] = h;
    const __bf16* qrow = q + (((int64_t)b * a.H + g * G + h) * a.n + rpos[rt]) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 qv = {0u, 0u, 0u, 0u};
      if (rpos[rt] < a.nv) qv = *(const u32x4*)(qrow + 32 * s + 8 * lg);
      qf[rt][s] = as_bf16x8(qv);
    }
  }
  __syncthreads();

  // ---- scores: X[rt][ct][i] = x(row 16 rt + l16, cand 16 ct + 4 lg + i) ----
  f32x4 X[RTW][kTileMaxCT];
#pragma unroll
  for (int ct = 0; ct < kTileMaxCT; ++ct) {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) X[rt][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (ct < CT) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int off = (16 * ct + l16) * SP + 32 * s + 8 * lg;
        const bf16x8 hi = as_bf16x8(*(const u32x4*)(planes + off));
        const bf16x8 mid = as_bf16x8(*(const u32x4*)(planes + (size_t)TP * SP + off));
        const bf16x8 lo = as_bf16x8(*(const u32x4*)(planes + (size_t)2 * TP * SP + off));
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
          X[rt][ct] = mfma16(lo, qf[rt][s], X[rt][ct]);
          X[rt][ct] = mfma16(mid, qf[rt][s], X[rt][ct]);
          X[rt][ct] = mfma16(hi, qf[rt][s], X[rt][ct]);
        }
      }
    }
  }

#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    // the row's slots are the accumulators themselves: candidates past t in
    // the last candidate tile become -inf; tiles at or past CT are never read
    f32x4 (&xv)[kTileMaxCT] = X[rt];
    static_for<0, kTileMaxCT>([&](auto CTc) {
      constexpr int ct = decltype(CTc)::value;
      if (ct == CT - 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * ct + 4 * lg + i >= t) xv[ct][i] = -INFINITY;
      }
    });
    const float tau = entmax_tau_reg<4 * kTileMaxCT, MODE>(xv, Stride16Reduce{}, a.e, CT);
    const int64_t pos = rpos[rt];
    const int h = rh[rt];
    const int64_t rglob = ((int64_t)b * a.H + g * G + h) * a.n + pos;
    if (a.bits) {
      // per-head support bits: ballots give, for each (ct, i), the bit of
      // every (row, lg) pair
      uint32_t chunk[kTileMaxCT];
#pragma unroll
      for (int ct = 0; ct < kTileMaxCT; ++ct) {
        chunk[ct] = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint64_t mk = __ballot(ct < CT && xv[ct][i] > tau);
#pragma unroll
          for (int l2 = 0; l2 < 4; ++l2)
            chunk[ct] |= (uint32_t)((mk >> (16 * l2 + l16)) & 1ull) << (4 * l2 + i);
        }
      }
      if (lg == 0 && pos < a.nv)
        for (int w = 0; w < a.nwords; ++w) {
          uint32_t word = 0u;
#pragma unroll
          for (int ct = 0; ct < kTileMaxCT; ++ct)
            if (ct / 2 == w) word |= chunk[ct] << (16 * (ct % 2));
          a.bits[rglob * a.nwords + w] = word;
        }
    }
    if (lg == 0 && pos < a.nv) a.tau[rglob] = tau;
    static_for<0, kTileMaxCT>([&](auto CTc) {
      constexpr int ct = decltype(CTc)::value;
      if (ct < CT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) xv[ct][i] = entmax_prob<MODE>(xv[ct][i] - tau, a.e);
      }
    });
    route_rows_bias<G, kTileMaxCT>(a, xv, CT, t, lg, h, pos, p_begin, tile, uflag);
  }
  __syncthreads();

  // ---- compaction (ascending block ids) ----
  if (threadIdx.x < kWave) compact_union(a, uflag, t, tile);
}

hipError_t launch_route_tile(RouteArgs a, const Shape& s, int t_max, hipStream_t st) {
  // one wave per 16 RTW rows of the tile's 64 G rows
  a.pitch = round_up16(t_max > 0 ? t_max : 1);
  const size_t lds_t = (size_t)3 * a.pitch * (s.d + 8) * 2 + (size_t)a.pitch * 4;
  dim3 grid_t((unsigned)(a.n_qt * s.B * s.Hkv));
  const int rtw = s.G <= 4 ? 1 : 2;
  const int threads = kWave * (4 * s.G / rtw);
#define DASH_RTT3(D, M, GG)                                                                  \
  do {                                                                                       \
    if (lds_t > 64 * 1024)                                                                   \
      (void)hipFuncSetAttribute((const void*)route_tile_kernel<D, M, GG>,                    \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_t);      \
    hipLaunchKernelGGL((route_tile_kernel<D, M, GG>), grid_t, dim3(threads), lds_t, st, a);  \
  } while (0)
#define DASH_RTT(D, M)                       \
  do {                                       \
    if (s.G == 1) DASH_RTT3(D, M, 1);        \
    else if (s.G == 2) DASH_RTT3(D, M, 2);   \
    else if (s.G == 4) DASH_RTT3(D, M, 4);   \
    else DASH_RTT3(D, M, 8);                 \
  } while (0)
#define DASH_RTT2(D)                                                \
  do {                                                              \
    if (a.mode == kEntmax15) DASH_RTT(D, kEntmax15);                \
    else if (a.mode == kSparsemax) DASH_RTT(D, kSparsemax);         \
    else if (a.mode == kEntmaxQuartic) DASH_RTT(D, kEntmaxQuartic); \
    else DASH_RTT(D, kEntmaxGeneral);                               \
  } while (0)
  if (s.d == 64) DASH_RTT2(64); else DASH_RTT2(128);
#undef DASH_RTT2
#undef DASH_RTT
#undef DASH_RTT3
  return hipGetLastError();
}

}  // namespace dash
