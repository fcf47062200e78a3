// route_common.hpp -- what the prefill routing kernels share: their argument
// block, sequence bounds and the compaction of a tile's union flags into its
// ascending block list (Stage 1 output, "entmax chunk routing", DashAttention
// explainer, Technical summary).
#pragma once

#include "dash_internal.hpp"
#include "device_common.hpp"
#include "entmax_device.hpp"

namespace dash {

constexpr int kQT = DASH_QUERY_TILE;

struct RouteArgs {
  const void* q;
  int64_t n;            // positions per sequence in memory (the row stride)
  const int32_t* seq_len;  // [B] valid positions per sequence, or null (all n)
  int64_t nv;           // valid positions of the workgroup's sequence
  const float* summ;
  int64_t summ_blocks;
  float* tau;
  int32_t* sel_count;
  int32_t* sel_idx;
  float* sel_logp;
  uint32_t* bits;
  uint32_t* tile_bits;   // optional bit-packed union per tile
  int64_t n_qt, nb;
  int nwords;
  int H, Hkv, G, bs, B;
  int mode;
  float e, scale;
  float sigma;  // prior strength: sel_logp = sigma * log pbar
  int window;   // near-diagonal branch in blocks
  int PP;      // positions per pass
  int pitch;   // X row pitch in floats (multiple of 4)
};

__host__ __device__ inline int round_up16(int x) { return (x + 15) & ~15; }

// Valid positions of sequence b: seq_len[b] clamped into [0, n], or n.
__device__ __forceinline__ int64_t valid_len(const int32_t* seq_len, int b, int64_t n) {
  if (!seq_len) return n;
  const int64_t l = seq_len[b];
  return l < 0 ? 0 : (l > n ? n : l);
}

// A tile at or past its sequence's end: an empty list (its rows are not written).
__device__ __forceinline__ void route_tile_past_end(const RouteArgs& a, int64_t tile) {
  if (threadIdx.x == 0) a.sel_count[tile] = 0;
  if (a.tile_bits)
    for (int w = threadIdx.x; w < a.nwords; w += blockDim.x) a.tile_bits[tile * a.nwords + w] = 0u;
}

// Compaction of the tile's union flags (blocks j < t) into the ascending list
// sel_idx / sel_count, and the same set as the tile's bit-packed mask when
// asked for (words past the candidates are zero).  One wave calls.
__device__ __forceinline__ void compact_union(const RouteArgs& a, const int* uflag, int t,
                                              int64_t tile) {
  const int lane = threadIdx.x % kWave;
  uint32_t* tb = a.tile_bits ? a.tile_bits + tile * a.nwords : nullptr;
  int base = 0;
  for (int j0 = 0; j0 < t; j0 += kWave) {
    const int j = j0 + lane;
    const bool f = j < t && uflag[j] != 0;
    const uint64_t mask = __ballot(f);
    if (f) a.sel_idx[tile * a.nb + base + __popcll(mask & ((1ull << lane) - 1ull))] = j;
    base += __popcll(mask);
    if (tb && lane < 2 && j0 / 32 + lane < a.nwords)
      tb[j0 / 32 + lane] = (uint32_t)(mask >> (32 * lane));
  }
  if (tb)
    for (int w = 2 * ((t + kWave - 1) / kWave) + lane; w < a.nwords; w += kWave) tb[w] = 0u;
  if (lane == 0) a.sel_count[tile] = base;
}

// Two summary values split into three bf16 parts each, packed in pairs
// (value 0 in the low half): hi is x with the low 16 bits of its pattern
// cleared, mid the same of x - hi (exact: hi holds x's leading bits), lo the
// rest (at most 8 significant bits, so exactly a bf16), hence hi + mid + lo
// = x exactly; the pairs are packed by byte permutes of the upper halves.
__device__ __forceinline__ void split3_bf16(float x0, float x1, uint32_t& hw, uint32_t& mw,
                                            uint32_t& lw) {
  constexpr uint32_t kUpper = 0x07060302u;   // upper halves of (src1, src0) -> (lo, hi)
  constexpr uint32_t kMask = 0xffff0000u;
  const uint32_t b0 = __builtin_bit_cast(uint32_t, x0), b1 = __builtin_bit_cast(uint32_t, x1);
  hw = __builtin_amdgcn_perm(b1, b0, kUpper);
  const float r0 = x0 - __builtin_bit_cast(float, b0 & kMask);
  const float r1 = x1 - __builtin_bit_cast(float, b1 & kMask);
  const uint32_t c0 = __builtin_bit_cast(uint32_t, r0), c1 = __builtin_bit_cast(uint32_t, r1);
  mw = __builtin_amdgcn_perm(c1, c0, kUpper);
  const float l0 = r0 - __builtin_bit_cast(float, c0 & kMask);
  const float l1 = r1 - __builtin_bit_cast(float, c1 & kMask);
  lw = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, l1), __builtin_bit_cast(uint32_t, l0),
                             kUpper);
}

// GQA sum of a row's probabilities and the Stage 2 bias, for rows whose
// scores sit in MFMA 16x16 accumulators (lane l16 + 16 lg of a wave holds
// row l16's candidates 16 ct + 4 lg + i, i < 4, in slot 4 ct + i).  The sum over
// the G rows of a position is a reduce-scatter over the lanes whose l16
// differ in the bits of h = l16 % G: after it, the lane of head h holds the
// sum for the slots s with s % G == h (slot s = 4 ct + i is candidate
// 16 ct + 4 lg + i), which it writes.  xv: the row's slots, a float array or
// the MFMA accumulator fragments themselves (xget / xset).  Slots of candidate tiles at or past
// CT are never written (their j is at least t).
template <int G, int MAXCT, typename XV>
__device__ __forceinline__ void route_rows_bias(const RouteArgs& a, XV& xv, int CT, int t, int lg,
                                                int h, int64_t pos, int64_t p_begin,
                                                int64_t tile, int* lflag) {
  static_for<0, 3>([&](auto BB) {
    constexpr int bit = 1 << decltype(BB)::value;
    if constexpr (bit < G) {
      const bool up = (h & bit) != 0;
      static_for<0, 4 * MAXCT / (2 * bit)>([&](auto K) {
        constexpr int s2 = 2 * bit * decltype(K)::value;
        if ((s2 >> 2) < CT) {
          const float lo = xget(xv, s2), hi = xget(xv, s2 | bit);
          const float send = up ? lo : hi, keep = up ? hi : lo;
          xset(xv, s2, keep + lane_xor<bit>(send));
        }
      });
    }
  });
  if (pos >= a.nv) return;
  constexpr float invG = 1.0f / (float)G;
  const float sl2 = a.sigma * kLn2;
  // the bias rows of the tile's t candidates through a buffer resource of
  // their size (32-bit offsets)
  const buf_rsrc lp = make_rsrc(a.sel_logp + tile * a.nb * kQT, (uint32_t)t * kQT * 4);
  const int jl = 16 * (h >> 2) + (h & 3) + 4 * lg;   // lane part of j
  const uint32_t voff = (uint32_t)(jl * kQT + (pos - p_begin)) * 4;
  static_for<0, 4 * MAXCT / G>([&](auto K) {
    constexpr int s2 = G * decltype(K)::value;
    constexpr int jc = 16 * (s2 >> 2) + (s2 & 3);     // j = jc + jl
    if ((s2 >> 2) < CT && jc + jl < t) {
      const float pb = xget(xv, s2) * invG;
      buf_store4(prior_bias(pb, sl2), lp, voff + (uint32_t)jc * kQT * 4, 0u);
      if (pb > 0.f) lflag[jc + jl] = 1;
    }
  });
}

// Rows of at most 128 candidates (bf16 queries): route_tile.hip.
constexpr int kTileMaxCT = 8;      // candidate tiles of 16 per row (128 candidates)
hipError_t launch_route_tile(RouteArgs a, const Shape& s, int t_max, hipStream_t st);

// Rows of 129 to 512 candidates (bf16 queries, G >= 2): route_long.hip.
constexpr int kLongMaxCT = 32;     // candidate tiles of 16 per row (512 candidates)
hipError_t launch_route_long(RouteArgs a, const Shape& s, int t_max, hipStream_t st);

}  // namespace dash
