// decode.hip -- one incremental decoding step of DashAttention (the pages'
// kernels support "prefill and incremental decoding"; chunk summaries are
// cached once a chunk is complete -- DashAttention explainer, Technical
// summary, Stage 0 and Contributions).
//
// Per sequence b the new query sits at position L = cache_len[b] - 1:
//   1. scores          x[b,h,j] = (alpha-1) gamma q_h . s_j / sqrt(d) for the
//                      cached summaries j < floor(L / bs) - (window - 1) (the
//                      blocks before the near-diagonal branch): a coalesced
//                      scan of the float32 summary cache with MFMA 4x4x1 f32
//   2. route           one wave per query head finds tau; the G heads of a KV
//                      head average p; the union is compacted into an
//                      ascending list with the bias sigma log pbar per block
//      (1 and 2 run as one kernel, decode_select, when there are enough
//      (sequence, KV head) pairs to fill the GPU with one workgroup each;
//      otherwise as decode_scores + decode_route)
//   3. decode_attend   split-K over the list [branch blocks, selected blocks...]
//                      (branch: the own block and the window - 1 before it),
//                      32 entries per work item, a persistent grid walking
//                      the items, 4 waves; MFMA 16x16x32 with the G query
//                      heads as MFMA rows (padded to 16); K and V stream from
//                      HBM straight into registers, V is transposed 8x8 in
//                      registers
//   4. decode_combine  log-sum-exp merge of the splits in a fixed order; one
//                      more workgroup per (sequence, KV head) writes the
//                      summary of the block the step completes, if any
//                      (cache_len[b] % bs == 0), off the critical path
#include <atomic>
#include <type_traits>

#include "dash_internal.hpp"
#include "device_common.hpp"
#include "entmax_device.hpp"
#include "summarize_device.hpp"

namespace dash {

struct DecodeArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* cache_len;
  int64_t max_len;
  const float* summ;
  int64_t summ_blocks;
  void* o;
  float* x;          // [B, H, nb]
  float* tau;        // [B, H]
  int32_t* count;    // [B, Hkv]
  int32_t* idx;      // [B, Hkv, nb]
  float* logp;       // [B, Hkv, nb]  by block id
  uint32_t* bits;    // [B, H, nwords] or null
  uint32_t* tile_bits;  // [B, Hkv, nwords] bit-packed union, or null
  float* part;       // [B, Hkv, n_split, G, D + 2]
  float* summ_w;     // the summary cache, written for a block this step completes
  const float* w_s;
  const float* q_bar;  // [Hkv, D] summary queries, or null (mean pooling)
  // paged caches: kc / vc are [num_pages, Hkv, bs, D] and block j of sequence
  // b lives in page block_table[b * max_blocks + j]; null = contiguous caches
  // [B, Hkv, max_len, D]
  const int32_t* block_table;
  int64_t max_blocks;
  int64_t num_pages;
  int64_t nb;
  int64_t n_split;
  int nwords;
  int H, Hkv, G, bs, B;
  int bs_log;        // log2(bs)
  int xpitch;        // fused score/route kernel: LDS row pitch of the scores
  int mode;
  float e, scale, scale_log2;
  float sigma;       // prior strength: logp = sigma * log pbar
  int window;        // near-diagonal branch in blocks
};

__host__ __device__ inline int64_t min64(int64_t x, int64_t y) { return x < y ? x : y; }

// Element offset of the first key of block j of (sequence b, KV head g) in
// the K or V cache.  Paged: the table entry, with j and the page id clamped
// into range (a bad table gives wrong keys, never an access outside the
// pages).
__device__ __forceinline__ int64_t page_of(const DecodeArgs& a, int b, int64_t j) {
  const int64_t jc = j < 0 ? 0 : (j >= a.max_blocks ? a.max_blocks - 1 : j);
  const int64_t pg = a.block_table[(int64_t)b * a.max_blocks + jc];
  return pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
}
template <int D>
__device__ __forceinline__ int64_t block_offset(const DecodeArgs& a, int b, int g, int64_t j) {
  if (a.block_table) return (page_of(a, b, j) * a.Hkv + g) * a.bs * D;
  return (((int64_t)b * a.Hkv + g) * a.max_len + j * a.bs) * D;
}

__device__ __forceinline__ int64_t clamp_len(int32_t v, int64_t max_len) {
  int64_t l = v;
  return l < 1 ? 1 : (l > max_len ? max_len : l);
}

// Routing candidates of a query at position len - 1: the complete blocks
// before its near-diagonal branch (own block and the window - 1 before it).
__device__ __forceinline__ int decode_ncand(const DecodeArgs& a, int64_t len) {
  return max(0, (int)((len - 1) >> a.bs_log) - (a.window - 1));
}
// Blocks of that branch: min(window, own + 1); the list of a (sequence, KV
// head) is [own, own - 1, ..., own - n_branch + 1, selected blocks...].
__device__ __forceinline__ int decode_nbranch(const DecodeArgs& a, int64_t len) {
  return min(a.window, (int)((len - 1) >> a.bs_log) + 1);
}

// ---- 1. coarse scores ------------------------------------------------------------------------
// x[h][j] = scale * q_h . s_j over the float32 summary rows of one (sequence,
// KV head), in groups of 16 rows.  Lane l = 16 rq + 4 ks + m loads row
// 4 rq + m of a group, floats 16 u + 4 ks + [0, 4) for u < D / 16, so one
// load instruction covers 16 rows x 64 contiguous bytes.  MFMA 4x4x1 f32
// block (rq, ks) multiplies these rows by the heads 4 hs + m of head set hs
// (B operand from the same lane) over that d slice; two row rotations add
// the four ks partial sums, after which lane (rq, 0, m) holds x of rows
// 4 rq + i, head 4 hs + m in element i.  The wave takes groups g_first,
// g_first + g_step, ... < g_end in batches of NG; with PIPE the next batch's
// loads are issued before the current batch is multiplied, so a wave's
// arithmetic overlaps its own loads instead of waiting for all of them.  x of
// row j, head h goes to out[h * pitch + j] (rows < ncand only).
// With XL (the pipelined scan of decode_scores_kernel) the loads are laid out
// for the memory system instead -- lane L reads row 8 sb + L / 8 of a group,
// floats 32 u + 4 (L % 8) + [0, 4), so one instruction covers 8 rows x 128
// contiguous bytes (the MFMA layout puts four consecutive lanes on four
// rows, which reads measurably slower) -- and each wave moves its batch
// through a private LDS region xl (rows kXlPitch floats apart, a pitch at
// which both the row-wise stores and the MFMA-layout reads are free of bank
// conflicts) into the MFMA layout.
constexpr int kXlPitch = 144;
template <typename T, int D, int NG, bool PIPE = false, bool XL = false>
__device__ __forceinline__ void score_groups(const DecodeArgs& a, int64_t bg, int64_t row0,
                                             int ncand, int g_first, int g_step, int g_end,
                                             float* out, int64_t pitch, float* xl = nullptr) {
  constexpr int NU = D / 16;
  constexpr bool kBf16 = sizeof(T) == 2;
  const int lane = threadIdx.x % kWave;
  const int rq = lane >> 4, ks = (lane >> 2) & 3, m = lane & 3;
  const int G = a.G;
  // B operand q[head 4 hs + m][16 u + 4 ks + t]; heads >= G fall outside the
  // resource and read as zeros.  bf16 stays packed until use.
  typedef typename std::conditional<kBf16, u32x2, f32x4>::type QW;
  QW qw[2][NU];
  {
    const buf_rsrc rq_ = make_rsrc((const T*)a.q + row0 * D, (uint32_t)(G * D * sizeof(T)));
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const uint32_t off = (uint32_t)(((4 * hs + m) * D + 16 * u + 4 * ks) * sizeof(T));
        if constexpr (kBf16) qw[hs][u] = buf_load8(rq_, off);
        else qw[hs][u] = __builtin_bit_cast(f32x4, buf_load16(rq_, off));
      }
  }
  const buf_rsrc rs = make_rsrc(a.summ + bg * a.summ_blocks * D, (uint32_t)(ncand * D * 4));
  // rows past ncand read as zeros; their scores are never stored
  auto load_batch = [&](int g0, f32x4 (&sv)[NG][NU]) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      if constexpr (XL) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const uint32_t r = (uint32_t)(16 * (g0 + g_step * gi) + 8 * (u & 1) + (lane >> 3));
          sv[gi][u] = __builtin_bit_cast(
              f32x4, buf_load16_nt(rs, (r * D + 32 * (u >> 1) + 4 * (lane & 7)) * 4));
        }
      } else {
        const uint32_t r = (uint32_t)(16 * (g0 + g_step * gi) + 4 * rq + m);
#pragma unroll
        for (int u = 0; u < NU; ++u)
          sv[gi][u] = __builtin_bit_cast(f32x4, buf_load16_nt(rs, (r * D + 16 * u + 4 * ks) * 4));
      }
    }
  };
  auto mul_batch = [&](int g0, const f32x4 (&lv)[NG][NU]) {
    f32x4 sv[NG][NU];
    if constexpr (XL) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int u = 0; u < NU; ++u)
          *(f32x4*)(xl + (16 * gi + 8 * (u & 1) + (lane >> 3)) * kXlPitch + 32 * (u >> 1) +
                    4 * (lane & 7)) = lv[gi][u];
      // the rows are read back by other lanes of the same wave
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int u = 0; u < NU; ++u)
          sv[gi][u] = *(const f32x4*)(xl + (16 * gi + 4 * rq + m) * kXlPitch + 16 * u + 4 * ks);
    } else {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int u = 0; u < NU; ++u) sv[gi][u] = lv[gi][u];
    }
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      if (hs * 4 >= G) break;
      f32x4 acc[NG];
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) acc[gi] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        float qf[4];
        if constexpr (kBf16) {
          qf[0] = bf16_lo(qw[hs][u].x); qf[1] = bf16_hi(qw[hs][u].x);
          qf[2] = bf16_lo(qw[hs][u].y); qf[3] = bf16_hi(qw[hs][u].y);
        } else {
          qf[0] = qw[hs][u].x; qf[1] = qw[hs][u].y; qf[2] = qw[hs][u].z; qf[3] = qw[hs][u].w;
        }
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          acc[gi] = mfma4x4(sv[gi][u].x, qf[0], acc[gi]);
          acc[gi] = mfma4x4(sv[gi][u].y, qf[1], acc[gi]);
          acc[gi] = mfma4x4(sv[gi][u].z, qf[2], acc[gi]);
          acc[gi] = mfma4x4(sv[gi][u].w, qf[3], acc[gi]);
        }
      }
      const int head = 4 * hs + m;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc[gi][t] += row_ror<8>(acc[gi][t]);
          acc[gi][t] += row_ror<4>(acc[gi][t]);
        }
        const int j0 = 16 * (g0 + g_step * gi) + 4 * rq;
        if (g0 + g_step * gi < g_end && ks == 0 && head < G) {
          float* o = out + head * pitch + j0;
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (j0 + t < ncand) o[t] = acc[gi][t] * a.scale;
        }
      }
    }
  };
  if constexpr (!PIPE) {
    for (int g0 = g_first; g0 < g_end; g0 += g_step * NG) {
      f32x4 sv[NG][NU];
      load_batch(g0, sv);
      __builtin_amdgcn_sched_barrier(0);
      mul_batch(g0, sv);
    }
  } else {
    f32x4 cur[NG][NU];
    if (g_first < g_end) load_batch(g_first, cur);
    for (int g0 = g_first; g0 < g_end; g0 += g_step * NG) {
      const int g1 = g0 + g_step * NG;
      f32x4 nxt[NG][NU];
      if (g1 < g_end) load_batch(g1, nxt);
      __builtin_amdgcn_sched_barrier(0);
      mul_batch(g0, cur);
      __builtin_amdgcn_sched_barrier(0);
      if (g1 < g_end) {
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
          for (int u = 0; u < NU; ++u) cur[gi][u] = nxt[gi][u];
      }
    }
  }
}

// Score kernel for the two-kernel path: grid (ceil(ncand_max / kScoreRows), B Hkv),
// 4 waves x 8 groups = 512 rows per workgroup, in batches of 2 groups per wave.
// (One workgroup per CU at decode_128k: while a wave multiplies one batch,
// the next batch's loads, 16 KB per wave and 64 KB per CU, are in flight.)
constexpr int kScoreThreads = 256;
constexpr int kScoreGroups = 8;
constexpr int kScoreNG = 2;   // groups per batch, pipelined
constexpr int kScoreRows = kScoreThreads / kWave * kScoreGroups * 16;
template <typename T, int D>
__global__ __launch_bounds__(kScoreThreads) void decode_scores_kernel(DecodeArgs a) {
  const int64_t bg = blockIdx.y;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t len = clamp_len(a.cache_len[b], a.max_len);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int ncand = decode_ncand(a, len);
  const int gb = blockIdx.x * (kScoreRows / 16);
  const int ge = min((ncand + 15) >> 4, gb + kScoreRows / 16);
  if (gb >= ge) return;
  const int64_t row0 = (int64_t)b * a.H + g * a.G;
  __shared__ __attribute__((aligned(16))) float xl[kScoreThreads / kWave][kScoreNG * 16 * kXlPitch];
  score_groups<T, D, kScoreNG, true, true>(a, bg, row0, ncand, gb + wave, kScoreThreads / kWave,
                                           ge, a.x + row0 * a.nb, a.nb, xl[wave]);
}

// ---- 2. threshold, GQA average, union, compaction ------------------------------------------
constexpr int kMaxRouteWaves = 8;   // routing workgroups have at most 512 threads

// Row of query head `row` with no candidate: tau is NaN, no support bit set.
__device__ __forceinline__ void route_row_empty(const DecodeArgs& a, int64_t row) {
  const int lane = threadIdx.x % kWave;
  if (lane == 0) a.tau[row] = __builtin_nanf("");
  if (a.bits)
    for (int w = lane; w < a.nwords; w += kWave) a.bits[row * a.nwords + w] = 0u;
}

// One wave: tau of a row whose candidates sit in registers (candidate j in
// lane j % 64, slot j / 64; -inf past ncand), the support bits, and the
// probabilities [x - tau]_+^e into prow[0, ncand).
template <int VPL, int MODE>
__device__ __forceinline__ void route_row_reg(const DecodeArgs& a, int64_t row, int ncand,
                                              float (&xv)[VPL], float* prow) {
  const int lane = threadIdx.x % kWave;
  const int nact4 = (ncand + 4 * kWave - 1) / (4 * kWave);
  const float tau = entmax_tau_reg<VPL, MODE>(xv, WaveReduce{}, a.e, nact4);
  if (lane == 0) a.tau[row] = tau;
  if (a.bits) {
    // candidate j = 64 i + lane sits in bit lane of the ballot of slot i
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const uint64_t m = __ballot(xv[i] > tau);   // -inf slots never pass
      if (lane == 0) {
        if (2 * i < a.nwords) a.bits[row * a.nwords + 2 * i] = (uint32_t)m;
        if (2 * i + 1 < a.nwords) a.bits[row * a.nwords + 2 * i + 1] = (uint32_t)(m >> 32);
      }
    }
    for (int w = 2 * VPL + lane; w < a.nwords; w += kWave) a.bits[row * a.nwords + w] = 0u;
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int j = lane + kWave * i;
    const float y = xv[i] - tau;
    if (j < ncand) prow[j] = y > 0.f ? entmax_pow(y, MODE, a.e) : 0.f;
  }
}

// All threads of the workgroup, after the G rows of probabilities are in
// Ps[h * pitch + j]: pbar = mean over the heads, log pbar per candidate, and
// the ascending list of blocks with pbar > 0.  Wave w owns a contiguous range
// of candidates (a multiple of 64): it counts its blocks, the counts are
// prefixed across waves, and each wave writes its part of the list.
__device__ __forceinline__ void route_union(const DecodeArgs& a, int64_t bg, int ncand, float* Ps,
                                            int pitch) {
  __shared__ int wcount[kMaxRouteWaves];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const int span = (ncand + nw * kWave - 1) / (nw * kWave) * kWave;
  const int jb = wave * span, je = min(ncand, jb + span);
  const float invG = 1.0f / (float)a.G;
  int cnt = 0;
  for (int j0 = jb; j0 < je; j0 += kWave) {
    const int j = j0 + lane;
    float pb = 0.f;
    if (j < je) {
      for (int h = 0; h < a.G; ++h) pb += Ps[h * pitch + j];
      pb *= invG;
      a.logp[bg * a.nb + j] = prior_bias(pb, a.sigma * kLn2);
      Ps[j] = pb;   // column j is only touched by this lane
    }
    cnt += __popcll(__ballot(pb > 0.f));
  }
  if (lane == 0) wcount[wave] = cnt;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < nw; ++w) {
    const int c = wcount[w];
    base += w < wave ? c : 0;
    total += c;
  }
  uint32_t* tb = a.tile_bits ? a.tile_bits + bg * a.nwords : nullptr;
  for (int j0 = jb; j0 < je; j0 += kWave) {
    const int j = j0 + lane;
    const bool f = j < je && Ps[j] > 0.f;
    const uint64_t mask = __ballot(f);
    if (f) a.idx[bg * a.nb + base + __popcll(mask & ((1ull << lane) - 1ull))] = j;
    base += __popcll(mask);
    // the bit-packed union: j0 is a multiple of 64, so this chunk is two words
    if (tb && lane < 2 && j0 / 32 + lane < a.nwords)
      tb[j0 / 32 + lane] = (uint32_t)(mask >> (32 * lane));
  }
  if (tb)
    for (int w = 2 * ((ncand + kWave - 1) / kWave) + (int)threadIdx.x; w < a.nwords;
         w += blockDim.x)
      tb[w] = 0u;
  if (threadIdx.x == 0) a.count[bg] = total;
}

// The routing result of a (sequence, KV head) without candidates.
__device__ __forceinline__ void route_pair_empty(const DecodeArgs& a, int64_t bg) {
  if (threadIdx.x == 0) a.count[bg] = 0;
  if (a.tile_bits)
    for (int w = threadIdx.x; w < a.nwords; w += blockDim.x) a.tile_bits[bg * a.nwords + w] = 0u;
}

// One workgroup per (sequence, KV head), one wave per query head.  With VPL > 0
// the wave keeps its row of scores in registers (VPL per lane) and solves for
// tau there (MODE: entmax_mode of alpha); VPL = 0 walks the row in memory for
// lists longer than 64 * 32.
template <int VPL, int MODE>
__global__ __launch_bounds__(512) void decode_route_kernel(DecodeArgs a) {
  extern __shared__ float Ps[];   // [G][nb]
  const int64_t bg = blockIdx.x;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t len = clamp_len(a.cache_len[b], a.max_len);
  const int ncand = decode_ncand(a, len);
  const int lane = threadIdx.x % kWave;
  // the wave index as a scalar, so that the row's buffer resource is too
  const int hh = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t row = (int64_t)b * a.H + g * a.G + hh;
  const float* xr = a.x + row * a.nb;
  if (ncand == 0) {
    route_row_empty(a, row);
    route_pair_empty(a, bg);
    return;
  }
  if constexpr (VPL > 0) {
    // every load issued before any is used: a buffer resource over the row's
    // ncand scores returns zeros past them, masked to -inf after the loads
    const buf_rsrc rx = make_rsrc(xr, (uint32_t)ncand * 4);
    float xv[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      xv[i] = __builtin_bit_cast(float, buf_load4(rx, (uint32_t)(lane + kWave * i) * 4));
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + kWave * i >= ncand) xv[i] = -INFINITY;
    route_row_reg<VPL, MODE>(a, row, ncand, xv, Ps + hh * a.nb);
  } else {
    const float tau = entmax_tau([&](int j) { return xr[j]; }, ncand, lane, kWave, a.mode, a.e);
    if (lane == 0) a.tau[row] = tau;
    if (a.bits)
      for (int w = lane; w < a.nwords; w += kWave) {
        uint32_t word = 0u;
        for (int i = 0; i < 32; ++i) {
          const int j = w * 32 + i;
          if (j < ncand && xr[j] > tau) word |= 1u << i;
        }
        a.bits[row * a.nwords + w] = word;
      }
    for (int j = lane; j < ncand; j += kWave) {
      const float y = xr[j] - tau;
      Ps[hh * a.nb + j] = y > 0.f ? entmax_pow(y, a.mode, a.e) : 0.f;
    }
  }
  __syncthreads();
  route_union(a, bg, ncand, Ps, (int)a.nb);
}

// ---- 1+2 fused (bf16): scores and routing of one (sequence, KV head) per workgroup ----------
// For many (sequence, KV head) pairs with rows of at most 2048 candidates.
// The scores go to LDS instead of HBM and the routing needs no second launch:
// 8 waves scan the summaries (score_groups), then wave h < G finds tau of
// head h in registers, and the workgroup forms pbar, log pbar and the block
// list.
constexpr int kSelectThreads = 512;
constexpr int kSelectWaves = kSelectThreads / kWave;
constexpr int kSelectGroups = 4;
#ifndef DASH_SELECT_MIN_PAIRS
#define DASH_SELECT_MIN_PAIRS 128
#endif
constexpr int kSelectMinPairs = DASH_SELECT_MIN_PAIRS;

template <int D, int VPL, int MODE>
__global__ __launch_bounds__(kSelectThreads) void decode_select_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) float xs[];   // [G][xpitch] x, then p
  const int pitch = a.xpitch;
  const int64_t bg = blockIdx.x;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int G = a.G;
  const int64_t len = clamp_len(a.cache_len[b], a.max_len);
  const int ncand = decode_ncand(a, len);
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t row0 = (int64_t)b * a.H + g * G;
  if (ncand == 0) {
    if (wave < G) route_row_empty(a, row0 + wave);
    route_pair_empty(a, bg);
    return;
  }
  score_groups<__bf16, D, kSelectGroups>(a, bg, row0, ncand, wave, kSelectWaves,
                                         (ncand + 15) >> 4, xs, pitch);
  __syncthreads();
  if (wave < G) {
    float* prow = xs + wave * pitch;
    float xv[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int j = lane + kWave * i;
      xv[i] = j < ncand ? prow[j] : -INFINITY;
    }
    route_row_reg<VPL, MODE>(a, row0 + wave, ncand, xv, prow);
  }
  __syncthreads();
  route_union(a, bg, ncand, xs, pitch);
}

// ---- 3. split-K attend (bf16, MFMA) ----------------------------------------------------------
// One work item: split s of the list of (sequence, KV head) bgi, i.e. entries
// [s * kDecodeSplit, (s + 1) * kDecodeSplit) of [branch blocks (own block
// first), selected blocks...].
// All 256 threads call; ms / ls / os are the workgroup's merge buffers.
template <int D, bool PAGED>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, int bgi, int s,
                                            float (&ms)[4][16], float (&ls)[4][16],
                                            float (&os)[4][8][D]) {
  constexpr int DPL = D / 16;   // d columns per lane in the PV product
  const int64_t bg = bgi;
  const int b = bgi / a.Hkv, g = bgi % a.Hkv;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int l16 = lane % 16, lg = lane / 16;
  // Everything the K/V addresses depend on arrives with one vector load:
  // lanes 0..kPerWave-1 read this wave's block ids e = s * kDecodeSplit +
  // wave + 4 i (slots clamped into the list buffer; ids past the list's end
  // are never used), lane kPerWave the list length, the other lanes the
  // sequence length.  Biases are read later, behind the K/V loads.
  constexpr int kPerWave = kDecodeSplit / 4;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  int32_t meta;
  {
    // entry e >= n_branch is selected block e - n_branch; when a sequence
    // has selected blocks its branch is full (n_branch = window)
    const int64_t slot =
        min64(max(s * kDecodeSplit + wv + 4 * lane - a.window, 0), a.nb - 1);
    const int32_t* src = lane < kPerWave    ? a.idx + bg * a.nb + slot
                         : lane == kPerWave ? a.count + bg
                                            : a.cache_len + b;
    meta = *src;
  }
  int32_t jraw[kPerWave];
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) jraw[i] = __builtin_amdgcn_readlane(meta, i);
  const int count = __builtin_amdgcn_readlane(meta, kPerWave);
  const int64_t len = clamp_len(__builtin_amdgcn_readlane(meta, kPerWave + 1), a.max_len);
  const int64_t own = (len - 1) >> a.bs_log;
  const int n_branch = decode_nbranch(a, len);
  const int n_entries = n_branch + count;

  // Contiguous caches: K/V of this (sequence, KV head) through buffer
  // resources sized to the current length (keys >= len read as zeros and are
  // masked below).  Paged caches: one more vector load fetches the page of
  // each of this wave's entries; each block gets its own resource.
  buf_rsrc rk, rv;
  int32_t pages[kPerWave];
  if constexpr (PAGED) {
    int32_t pg = 0;
    if (lane < kPerWave) {
      const int e = s * kDecodeSplit + wv + 4 * lane;
      pg = (int32_t)page_of(a, b, e < n_branch ? own - e : (int64_t)meta);
    }
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) pages[i] = __builtin_amdgcn_readlane(pg, i);
  } else {
    const uint32_t len_bytes = (uint32_t)(len * (D * 2));
    rk = make_rsrc((const __bf16*)a.kc + bg * a.max_len * D, len_bytes);
    rv = make_rsrc((const __bf16*)a.vc + bg * a.max_len * D, len_bytes);
  }

  // Q^T operand: column = query head l16 (< G), k = d in [32 s' + 8 lg, +8);
  // columns l16 >= G fall outside the resource and read as zeros
  bf16x8 qf[D / 32];
  {
    const buf_rsrc rq =
        make_rsrc((const __bf16*)a.q + ((int64_t)b * a.H + g * a.G) * D, (uint32_t)(a.G * D * 2));
#pragma unroll
    for (int sp = 0; sp < D / 32; ++sp)
      qf[sp] = as_bf16x8(buf_load16(rq, (uint32_t)(l16 * D + 32 * sp + 8 * lg) * 2));
  }
  f32x4 acc[DPL];
#pragma unroll
  for (int c = 0; c < DPL; ++c) acc[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int e_end = min(n_entries, (s + 1) * kDecodeSplit);
#pragma unroll
  for (int ei = 0; ei < kPerWave; ++ei) {
    const int e = s * kDecodeSplit + wv + 4 * ei;
    if (e >= e_end) break;
    const int64_t j = e < n_branch ? own - e : (int64_t)jraw[ei];
    if constexpr (PAGED) {
      // the block's page, limited to the keys below len
      const int64_t off = ((int64_t)pages[ei] * a.Hkv + g) * a.bs * D;
      const uint32_t nbytes = (uint32_t)(min64(a.bs, len - (j << a.bs_log)) * (D * 2));
      rk = make_rsrc((const __bf16*)a.kc + off, nbytes);
      rv = make_rsrc((const __bf16*)a.vc + off, nbytes);
    }
    for (int c64 = 0; c64 < (a.bs >> 6); ++c64) {
      const int64_t key0 = (j << a.bs_log) + 64 * c64;
      if (key0 >= len) break;
      // Issue every load of the chunk before any use (32-bit byte offsets
      // from the chunk's first key, within the block when paged).
      const uint32_t c0 = PAGED ? (uint32_t)(64 * c64 * (D * 2)) : (uint32_t)(key0 * (D * 2));
      u32x4 kw[4][D / 32];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int sp = 0; sp < D / 32; ++sp)
          kw[kt][sp] = buf_load16_nt(rk, c0 + (16 * kt + l16) * (D * 2) + (32 * sp + 8 * lg) * 2);
      // V rows this lane needs: k = 8 lg + e' <-> key 32 ks + 16 (e'/4) + 4 lg + e'%4,
      // DPL consecutive d starting at DPL * l16
      uint32_t vin[2][8][DPL / 2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ep = 0; ep < 8; ++ep) {
          const uint32_t off =
              c0 + (32 * ks + 16 * (ep / 4) + 4 * lg + (ep % 4)) * (D * 2) + DPL * l16 * 2;
          if constexpr (DPL == 8) {
            const u32x4 t = buf_load16_nt(rv, off);
            vin[ks][ep][0] = t.x; vin[ks][ep][1] = t.y; vin[ks][ep][2] = t.z; vin[ks][ep][3] = t.w;
          } else {
            const u32x2 t = buf_load8_nt(rv, off);
            vin[ks][ep][0] = t.x; vin[ks][ep][1] = t.y;
          }
        }
      const float bias2 = e < n_branch ? 0.f : a.logp[bg * a.nb + j] * kLog2e;
      // keep every load of the chunk ahead of the first use: one HBM latency
      // per chunk instead of one per dependent group of loads
      __builtin_amdgcn_sched_barrier(0);
      // S^T = K Q^T: st[kt][i] = S[query l16][key 16 kt + 4 lg + i]
      f32x4 st[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        st[kt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sp = 0; sp < D / 32; ++sp) st[kt] = mfma16(as_bf16x8(kw[kt][sp]), qf[sp], st[kt]);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sv = fmaf(st[kt][i], a.scale_log2, bias2);
          if (key0 + 16 * kt + 4 * lg + i >= len) sv = -INFINITY;
          st[kt][i] = sv;
          mx = fmaxf(mx, sv);
        }
      mx = xor_reduce<32>(xor_reduce<16>(mx, DppMax{}), DppMax{});
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float corr = fast_exp2(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = fast_exp2(st[kt][i] - m_use);
          st[kt][i] = pv;
          psum += pv;
        }
      psum = xor_reduce<32>(xor_reduce<16>(psum, DppAdd{}), DppAdd{});
      l_run = l_run * corr + psum;
      m_run = m_new;
      // acc rows are queries 4 lg + i: their correction lives in lane 4 lg + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ci = __shfl(corr, 4 * lg + i, kWave);
#pragma unroll
        for (int c = 0; c < DPL; ++c) acc[c][i] *= ci;
      }
      // O += P V over two 32-key steps
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 pw = {pack_bf16(st[2 * ks][0], st[2 * ks][1]), pack_bf16(st[2 * ks][2], st[2 * ks][3]),
                    pack_bf16(st[2 * ks + 1][0], st[2 * ks + 1][1]),
                    pack_bf16(st[2 * ks + 1][2], st[2 * ks + 1][3])};
        const bf16x8 pf = as_bf16x8(pw);
#pragma unroll
        for (int c = 0; c < DPL; ++c) {
          u32x4 vw;
          if (c % 2 == 0) {
            vw.x = pack_lo(vin[ks][0][c / 2], vin[ks][1][c / 2]);
            vw.y = pack_lo(vin[ks][2][c / 2], vin[ks][3][c / 2]);
            vw.z = pack_lo(vin[ks][4][c / 2], vin[ks][5][c / 2]);
            vw.w = pack_lo(vin[ks][6][c / 2], vin[ks][7][c / 2]);
          } else {
            vw.x = pack_hi(vin[ks][0][c / 2], vin[ks][1][c / 2]);
            vw.y = pack_hi(vin[ks][2][c / 2], vin[ks][3][c / 2]);
            vw.z = pack_hi(vin[ks][4][c / 2], vin[ks][5][c / 2]);
            vw.w = pack_hi(vin[ks][6][c / 2], vin[ks][7][c / 2]);
          }
          // C[query 4 lg + i][col l16] with col l16 <-> d = DPL * l16 + c
          acc[c] = mfma16(pf, as_bf16x8(vw), acc[c]);
        }
      }
    }
  }

  // ---- merge the 4 waves in a fixed order (query rows 4 lg + i < 8 hold the G <= 8 heads) ----
  if (lane < 16) {
    ms[wave][lane] = m_run;
    ls[wave][lane] = l_run;
  }
  if (lg < 2) {
#pragma unroll
    for (int c = 0; c < DPL; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) os[wave][4 * lg + i][DPL * l16 + c] = acc[c][i];
  }
  __syncthreads();
  float* part = a.part + ((bg * a.n_split + s) * a.G) * (D + 2);
  for (int e = threadIdx.x; e < a.G * D; e += 256) {
    const int qr = e / D, d = e % D;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, ms[w][qr]);
    float L = 0.f, O = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float f = ms[w][qr] == -INFINITY ? 0.f : fast_exp2(ms[w][qr] - M);
      L += ls[w][qr] * f;
      O += os[w][qr][d] * f;
    }
    float* pr = part + qr * (D + 2);
    if (d == 0) { pr[0] = M; pr[1] = L; }
    pr[2 + d] = O;
  }

  __syncthreads();   // the merge buffers are reused by the next item
}

// Persistent grid (as many workgroups as fit on the GPU at once): every
// workgroup derives the work items from the list lengths -- each list of
// n_branch + count[bg] entries splits into full items of kDecodeSplit
// entries and at most one shorter last item -- and takes items blockIdx.x,
// + gridDim.x, ...  No workgroup is launched for a split past its list, so
// none holds a slot waiting only to find it has nothing to do.
template <int D, bool PAGED>
__global__ __launch_bounds__(256) void decode_attend_bf16_kernel(DecodeArgs a) {
  __shared__ float ms[4][16], ls[4][16];
  __shared__ float os[4][8][D];
  // Items: first every full split (kDecodeSplit entries) of every list, then
  // the partial last splits, so the workgroups that take a second item in
  // the tail mostly get short ones.  Exclusive prefixes over the pairs of the
  // full-split counts (preF) and of the partial-split flags (preP).
  extern __shared__ int pre[];   // [2][B Hkv + 1], sized at launch
  __shared__ int wsum[2][4];
  const int nbg = a.B * a.Hkv;
  int* preF = pre;
  int* preP = pre + nbg + 1;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  // 256 contiguous ranges of pairs, then a scan of the range totals
  const int per = (nbg + 255) / 256;
  const int i0 = min(nbg, (int)threadIdx.x * per), i1 = min(nbg, i0 + per);
  int totF = 0, totP = 0;
  for (int i = i0; i < i1; ++i) {
    const int nbr = a.window == 1 ? 1
                                  : decode_nbranch(a, clamp_len(a.cache_len[i / a.Hkv], a.max_len));
    const int n = a.count[i] + nbr;
    preF[i] = n / kDecodeSplit;
    preP[i] = n % kDecodeSplit != 0;
    totF += preF[i];
    totP += preP[i];
  }
  int inclF = totF, inclP = totP;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int yf = __shfl_up(inclF, o, kWave), yp = __shfl_up(inclP, o, kWave);
    if (lane >= o) {
      inclF += yf;
      inclP += yp;
    }
  }
  if (lane == kWave - 1) {
    wsum[0][wave] = inclF;
    wsum[1][wave] = inclP;
  }
  __syncthreads();
  int runF = inclF - totF, runP = inclP - totP;
  for (int w = 0; w < wave; ++w) {
    runF += wsum[0][w];
    runP += wsum[1][w];
  }
  for (int i = i0; i < i1; ++i) {
    const int f = preF[i], pp = preP[i];
    preF[i] = runF;
    preP[i] = runP;
    runF += f;
    runP += pp;
  }
  const int totalF = wsum[0][0] + wsum[0][1] + wsum[0][2] + wsum[0][3];
  const int totalP = wsum[1][0] + wsum[1][1] + wsum[1][2] + wsum[1][3];
  if (threadIdx.x == 0) {
    preF[nbg] = totalF;
    preP[nbg] = totalP;
  }
  __syncthreads();
  for (int it = blockIdx.x; it < totalF + totalP; it += gridDim.x) {
    const bool full = it < totalF;
    const int* pr = full ? preF : preP;
    const int key = full ? it : it - totalF;
    int lo = 0, hi = nbg;   // pr[lo] <= key < pr[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pr[mid] <= key) lo = mid; else hi = mid;
    }
    // a partial split comes after the pair's full ones
    const int split = full ? key - preF[lo] : preF[lo + 1] - preF[lo];
    decode_item<D, PAGED>(a, lo, split, ms, ls, os);
  }
}

// ---- 3'. split-K attend (float32, plain FMAs; one thread per (query head, d)) --------------
template <int D>
__global__ __launch_bounds__(256) void decode_attend_f32_kernel(DecodeArgs a) {
  __shared__ float qs[8][D];
  __shared__ float sc[8][64];
  const int s = blockIdx.x;
  const int64_t bg = blockIdx.y;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t len = clamp_len(a.cache_len[b], a.max_len);
  const int64_t own = (len - 1) / a.bs;
  const int count = a.count[bg];
  const int n_branch = decode_nbranch(a, len);
  const int n_entries = n_branch + count;
  if (s * kDecodeSplit >= n_entries) return;
  const float* qb = (const float*)a.q + ((int64_t)b * a.H + g * a.G) * D;
  for (int e = threadIdx.x; e < a.G * D; e += 256) qs[e / D][e % D] = qb[e];
  const int qr = threadIdx.x / 32, dl = threadIdx.x % 32;   // 8 heads x 32 lanes
  float m_run = -INFINITY, l_run = 0.f, ov[D / 32];
  for (int c = 0; c < D / 32; ++c) ov[c] = 0.f;
  const int e_end = min(n_entries, (s + 1) * kDecodeSplit);
  for (int e = s * kDecodeSplit; e < e_end; ++e) {
    const int64_t j = e < n_branch ? own - e : (int64_t)a.idx[bg * a.nb + e - n_branch];
    const float bias2 = e < n_branch ? 0.f : a.logp[bg * a.nb + j] * kLog2e;
    // keys and values of block j, indexed by key - j * bs
    const int64_t boff = block_offset<D>(a, b, g, j), kfirst = j * a.bs;
    const float* kb = (const float*)a.kc + boff;
    const float* vb = (const float*)a.vc + boff;
    for (int64_t key0 = j * a.bs; key0 < (j + 1) * a.bs && key0 < len; key0 += 64) {
      __syncthreads();
      for (int p = threadIdx.x; p < a.G * 64; p += 256) {
        const int h = p / 64, kk = p % 64;
        const int64_t key = key0 + kk;
        float sv = -INFINITY;
        if (key < len) {
          float acc = 0.f;
          for (int c = 0; c < D; ++c) acc = fmaf(qs[h][c], kb[(key - kfirst) * D + c], acc);
          sv = fmaf(acc, a.scale_log2, bias2);
        }
        sc[h][kk] = sv;
      }
      __syncthreads();
      if (qr < a.G) {
        for (int kk = 0; kk < 64; ++kk) {
          const float sv = sc[qr][kk];
          if (sv == -INFINITY) continue;
          const float m_new = fmaxf(m_run, sv);
          const float corr = fast_exp2(m_run - m_new), p = fast_exp2(sv - m_new);
          l_run = l_run * corr + p;
          for (int c = 0; c < D / 32; ++c)
            ov[c] = fmaf(p, vb[(key0 + kk - kfirst) * D + dl + 32 * c], ov[c] * corr);
          m_run = m_new;
        }
      }
    }
  }
  if (qr < a.G) {
    float* pr = a.part + ((bg * a.n_split + s) * a.G + qr) * (D + 2);
    if (dl == 0) { pr[0] = m_run; pr[1] = l_run; }
    for (int c = 0; c < D / 32; ++c) pr[2 + dl + 32 * c] = ov[c];
  }
}

// ---- 4. combine ----------------------------------------------------------------------------
// grid (ceil(G D / 256), B Hkv): workgroup x merges outputs [256 x, 256 x + 256)
// of the G heads x D columns of one (sequence, KV head), one output per
// thread.  Each thread reads the maximum, sum and its column of up to
// kCombineChunk splits at once (one memory round trip per chunk; the split
// maxima and sums are the same for the D threads of a head and arrive as one
// request per wave) and merges them in split order, rescaling the running
// column when a later chunk raises the maximum.
constexpr int kCombineThreads = 256;
constexpr int kCombineChunk = 16;
template <typename T, int D>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecodeArgs a) {
  constexpr int HPW = kCombineThreads / D;   // heads per workgroup (D <= 256)
  static_assert(kCombineThreads == kSumThreads, "summary column runs summarize_blocks");
  const int bgi = blockIdx.y;
  const int64_t bg = bgi;
  const int b = bgi / a.Hkv, g = bgi % a.Hkv;
  if (blockIdx.x == gridDim.x - 1) {
    // the step that makes cache_len[b] a multiple of bs completes block
    // cache_len[b] / bs - 1: its summary, for the next steps' routing
    const int64_t len = clamp_len(a.cache_len[b], a.max_len);
    if ((len & (a.bs - 1)) == 0) {
      const int64_t j = (len >> a.bs_log) - 1;
      summarize_blocks<T, D, 1>((const T*)a.kc + block_offset<D>(a, b, g, j), 1, a.bs, a.w_s,
                                a.q_bar ? a.q_bar + g * D : nullptr,
                                a.summ_w + (bg * a.summ_blocks + j) * D);
    }
    return;
  }
  const int n_entries =
      decode_nbranch(a, clamp_len(a.cache_len[b], a.max_len)) + a.count[bg];
  const int ns = (n_entries + kDecodeSplit - 1) / kDecodeSplit;
  const int G = a.G;
  const int hq = threadIdx.x / D, d = threadIdx.x % D;
  const int qr = blockIdx.x * HPW + hq;
  if (qr >= G) return;
  const int stride = G * (D + 2);   // one split: G rows of [m, l, o(D)]
  // the pair's ns splits; offsets past them read as zeros
  const buf_rsrc rp = make_rsrc(a.part + bg * a.n_split * stride, (uint32_t)(ns * stride * 4));
  const uint32_t row = (uint32_t)(qr * (D + 2)) * 4;
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kCombineChunk) {
    float mv[kCombineChunk], lv[kCombineChunk], ov[kCombineChunk];
#pragma unroll
    for (int u = 0; u < kCombineChunk; ++u) {
      const uint32_t off = (uint32_t)((s0 + u) * stride) * 4 + row;
      mv[u] = __builtin_bit_cast(float, buf_load4(rp, off));
      lv[u] = __builtin_bit_cast(float, buf_load4(rp, off + 4));
      ov[u] = __builtin_bit_cast(float, buf_load4(rp, off + 8 + 4 * d));
    }
    float Mc = M;
#pragma unroll
    for (int u = 0; u < kCombineChunk; ++u)
      if (s0 + u < ns) Mc = fmaxf(Mc, mv[u]);
    const float f0 = M == -INFINITY ? 0.f : fast_exp2(M - Mc);
    L *= f0;
    O *= f0;
#pragma unroll
    for (int u = 0; u < kCombineChunk; ++u) {
      const float f = s0 + u >= ns || mv[u] == -INFINITY ? 0.f : fast_exp2(mv[u] - Mc);
      L += lv[u] * f;
      O += ov[u] * f;
    }
    M = Mc;
  }
  ((T*)a.o)[((int64_t)b * a.H + g * G + qr) * D + d] = from_f32<T>(O / L);
}

// Workgroups of decode_attend_bf16_kernel<D> resident on the current device at
// once with `lds` bytes of dynamic LDS (cached per device and 4 KB step of lds).
constexpr int kLdsSteps = 2 * (kDecodeMaxBg + 1) * 4 / 4096 + 1;
template <int D, bool PAGED>
static int persistent_grid(size_t lds) {
  static std::atomic<int> cache[kMaxDevices][kLdsSteps];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  const int step = (int)(lds / 4096);
  lds = (size_t)(step + 1) * 4096;   // occupancy of the step's upper end
  int g = cache[dev][step].load(std::memory_order_relaxed);
  if (g == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, (const void*)decode_attend_bf16_kernel<D, PAGED>, 256, lds) != hipSuccess)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    g = (per_cu < 1 ? 1 : per_cu) * (cus < 1 ? 1 : cus);
    cache[dev][step].store(g, std::memory_order_relaxed);
  }
  return g;
}

DecodeLayout decode_layout(const Shape& s, int64_t max_len) {
  DecodeLayout L;
  L.nb = (max_len + s.bs - 1) / s.bs;
  // list entries per (sequence, KV head): branch blocks + candidates <= own + 1
  const int64_t own_max = (max_len - 1) / s.bs;
  L.ncand_max = own_max - (s.window - 1) > 0 ? own_max - (s.window - 1) : 0;
  L.n_split = (own_max + 1 + kDecodeSplit - 1) / kDecodeSplit;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 0;
  L.off_x = off;     off = al(off + sizeof(float) * s.B * s.H * L.nb);
  L.off_tau = off;   off = al(off + sizeof(float) * s.B * s.H);
  L.off_count = off; off = al(off + sizeof(int32_t) * s.B * s.Hkv);
  L.off_idx = off;   off = al(off + sizeof(int32_t) * s.B * s.Hkv * L.nb);
  L.off_logp = off;  off = al(off + sizeof(float) * s.B * s.Hkv * L.nb);
  L.off_part = off;  off = al(off + sizeof(float) * s.B * s.Hkv * L.n_split * s.G * (s.d + 2));
  L.total = off;
  return L;
}

hipError_t launch_decode(const Shape& s, const void* q, const void* kc, const void* vc,
                         const int32_t* cache_len, int64_t max_len, const float* w_s,
                         const float* q_bar, float* summ, int64_t summ_blocks, void* o,
                         const dash_route_buf& rb, const DecodeLayout& L, char* ws,
                         hipStream_t st, const int32_t* block_table, int64_t max_blocks,
                         int64_t num_pages) {
  DecodeArgs a;
  a.xpitch = 0;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.num_pages = num_pages;
  a.q = q;
  a.kc = kc;
  a.vc = vc;
  a.cache_len = cache_len;
  a.max_len = max_len;
  a.summ = summ;
  a.summ_blocks = summ_blocks;
  a.o = o;
  a.x = (float*)(ws + L.off_x);
  a.tau = rb.tau ? rb.tau : (float*)(ws + L.off_tau);
  a.count = rb.sel_count ? rb.sel_count : (int32_t*)(ws + L.off_count);
  a.idx = rb.sel_idx ? rb.sel_idx : (int32_t*)(ws + L.off_idx);
  a.logp = rb.sel_logp ? rb.sel_logp : (float*)(ws + L.off_logp);
  a.bits = rb.support_bits;
  a.tile_bits = rb.tile_bits;
  a.part = (float*)(ws + L.off_part);
  a.summ_w = summ;
  a.w_s = w_s;
  a.q_bar = q_bar;
  a.nb = L.nb;
  a.n_split = L.n_split;
  a.nwords = (int)((L.nb + 31) / 32);
  a.H = s.H;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.bs = s.bs;
  a.bs_log = s.bs == 128 ? 7 : 6;
  a.B = s.B;
  a.mode = entmax_mode(s.alpha);
  a.e = 1.0f / (s.alpha - 1.0f);
  a.scale = (s.alpha - 1.0f) * s.gamma / sqrtf((float)s.d);
  a.scale_log2 = kLog2e / sqrtf((float)s.d);
  a.sigma = s.sigma;
  a.window = s.window;
  const bool bf16 = s.dtype == DASH_BF16;
  const unsigned nbg = (unsigned)(s.B * s.Hkv);

  // rows of up to 64 * VPL candidates stay in registers
  const int64_t nc = L.ncand_max;
  const int vpl = nc <= 256 ? 4 : nc <= 512 ? 8 : nc <= 1024 ? 16 : nc <= 2048 ? 32 : 0;
  const int mode = entmax_mode(s.alpha);
  // one fused workgroup per (sequence, KV head) only keeps the GPU's memory
  // system busy with enough of them; otherwise the scan is spread over
  // ceil(ncand / 256) workgroups per pair and routed by a second kernel
  const bool fused = bf16 && vpl > 0 && (int64_t)nbg >= kSelectMinPairs;
  if (fused) {
    a.xpitch = (int)((nc + 15) / 16 * 16);
    const size_t lds_sel = sizeof(float) * (size_t)s.G * a.xpitch;
    const void* fn = nullptr;
#define DASH_SK(D, V)                                                                        \
  fn = mode == kSparsemax       ? (const void*)decode_select_kernel<D, V, kSparsemax>        \
       : mode == kEntmax15      ? (const void*)decode_select_kernel<D, V, kEntmax15>         \
       : mode == kEntmaxQuartic ? (const void*)decode_select_kernel<D, V, kEntmaxQuartic>    \
                                : (const void*)decode_select_kernel<D, V, kEntmaxGeneral>
#define DASH_SKD(D)                                                                          \
  do {                                                                                       \
    if (vpl == 4) DASH_SK(D, 4); else if (vpl == 8) DASH_SK(D, 8);                           \
    else if (vpl == 16) DASH_SK(D, 16); else DASH_SK(D, 32);                                 \
  } while (0)
    if (s.d == 64) DASH_SKD(64); else DASH_SKD(128);
#undef DASH_SKD
#undef DASH_SK
    if (lds_sel > 64 * 1024)
      (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_sel);
    void* kargs[] = {&a};
    hipError_t e1 = hipLaunchKernel(fn, dim3(nbg), dim3(kSelectThreads), kargs, lds_sel, st);
    if (e1 != hipSuccess) return e1;
  } else {
    if (L.ncand_max > 0) {
      dim3 g1((unsigned)((L.ncand_max + kScoreRows - 1) / kScoreRows), nbg);
#define DASH_DS(T, D) \
  hipLaunchKernelGGL((decode_scores_kernel<T, D>), g1, dim3(kScoreThreads), 0, st, a)
      if (bf16) { if (s.d == 64) DASH_DS(__bf16, 64); else DASH_DS(__bf16, 128); }
      else { if (s.d == 64) DASH_DS(float, 64); else DASH_DS(float, 128); }
#undef DASH_DS
    }
    const size_t lds = sizeof(float) * s.G * L.nb;
    const void* fn = (const void*)decode_route_kernel<0, kEntmaxGeneral>;
#define DASH_RK(V)                                                                    \
  fn = mode == kSparsemax       ? (const void*)decode_route_kernel<V, kSparsemax>     \
       : mode == kEntmax15      ? (const void*)decode_route_kernel<V, kEntmax15>      \
       : mode == kEntmaxQuartic ? (const void*)decode_route_kernel<V, kEntmaxQuartic> \
                                : (const void*)decode_route_kernel<V, kEntmaxGeneral>
    if (vpl == 4) DASH_RK(4); else if (vpl == 8) DASH_RK(8); else if (vpl == 16) DASH_RK(16);
    else if (vpl == 32) DASH_RK(32);
#undef DASH_RK
    if (lds > 64 * 1024)
      (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    void* kargs[] = {&a};
    hipError_t e2 = hipLaunchKernel(fn, dim3(nbg), dim3(64 * s.G), kargs, lds, st);
    if (e2 != hipSuccess) return e2;
  }

  dim3 g3((unsigned)L.n_split, nbg);
  if (bf16) {
    const int64_t items_max = (int64_t)nbg * L.n_split;
    const size_t lds_pre = 2 * sizeof(int) * ((size_t)nbg + 1);   // the item prefixes
#define DASH_DA(D, PG)                                                                     \
  hipLaunchKernelGGL((decode_attend_bf16_kernel<D, PG>),                                   \
                     dim3((unsigned)min64(items_max, persistent_grid<D, PG>(lds_pre))),    \
                     dim3(256), lds_pre, st, a)
    if (s.d == 64) { if (a.block_table) DASH_DA(64, true); else DASH_DA(64, false); }
    else { if (a.block_table) DASH_DA(128, true); else DASH_DA(128, false); }
#undef DASH_DA
  } else {
    if (s.d == 64) hipLaunchKernelGGL(decode_attend_f32_kernel<64>, g3, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(decode_attend_f32_kernel<128>, g3, dim3(256), 0, st, a);
  }
  const int hpw = kCombineThreads / s.d;
  // one more column of workgroups writes the completed blocks' summaries
  dim3 g4((unsigned)((s.G + hpw - 1) / hpw + 1), nbg);
#define DASH_DC(T, D) \
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), g4, dim3(kCombineThreads), 0, st, a)
  if (bf16) { if (s.d == 64) DASH_DC(__bf16, 64); else DASH_DC(__bf16, 128); }
  else { if (s.d == 64) DASH_DC(float, 64); else DASH_DC(float, 128); }
#undef DASH_DC
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return hipSuccess;
}

}  // namespace dash
