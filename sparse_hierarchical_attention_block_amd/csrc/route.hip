// route.hip -- Stage 1 of DashAttention for causal prefill ("entmax chunk
// routing", DashAttention explainer, Technical summary): coarse scores of
// every query against the block summaries, w = alpha-entmax(gamma * zbar) per
// (query, head), GQA average of the probabilities of the heads sharing a KV
// head, union over a 64-position query tile and compaction into an ascending
// block list.
//
// One workgroup per (sequence, KV head, query tile of 64 positions), heaviest
// tiles (most candidate blocks) first.  Candidates of tile qt are the complete
// blocks before its near-diagonal branch, j < floor(64 qt / bs) - (window - 1).
// Rows are (position, head of the group)
// pairs.  Tiles of at most 128 candidates keep their scores in MFMA
// accumulators (route_tile_kernel); bf16 rows of 129 to 512 candidates with
// G >= 2 go to route_long.hip; the rest (float32 queries, G = 1, longer rows)
// are processed in passes of PP positions, PP as large as an 80 KB LDS score
// buffer allows:
//   1. scores X[row][j] = scale * q_row . s_j into an LDS buffer; bf16 queries
//      use MFMA 16x16x32 with the float32 summaries split into three bf16
//      parts (hi + mid + lo carries 24 mantissa bits), float32 queries use
//      plain FMAs;
//   2. tau per row (entmax_device.hpp), lanes-per-row = threads / rows;
//   3. pbar per (position, block) = mean over the group's heads of
//      [x - tau]_+^e, written as the Stage 2 bias sigma log pbar (-inf for 0)
//      into sel_logp, and the tile-union flags.
// Finally wave 0 compacts the flags into sel_idx / sel_count.
#include "dash_internal.hpp"
#include "device_common.hpp"
#include "entmax_device.hpp"
#include "route_common.hpp"

namespace dash {

constexpr int kRoutePassThreads = DASH_ROUTE_PASS_THREADS;   // pass-based path
constexpr size_t kRouteXBudget = DASH_ROUTE_X_BUDGET;         // its LDS score buffer
constexpr int kRouteMaxRowTiles = 4;   // rows per pass <= 64

// ---- step 1, bf16: MFMA with a 3-way bf16 split of the summaries ----------------
// Wave w computes candidate tiles w, w + NT/64, ... against every row tile of
// the pass; the pass's Q fragments are loaded once up front.  (Prefetching the
// next tile's summaries would cost the registers that keep two waves per SIMD.)
template <int D, int MAXRT, int NT>
__device__ void route_scores_bf16(const RouteArgs& a, float* X, int t, int64_t bg, int b, int g,
                                  int64_t pos0, int R) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int l16 = lane % 16, lg = lane / 16;
  const __bf16* q = (const __bf16*)a.q;
  const int CT = round_up16(t) / 16;
  constexpr int KS = D / 32;
  const int RT = R / 16;
  if (wave >= CT) return;
  // Q^T fragments of every row tile: column = row l16, k = d in [32 s + 8 lg, +8)
  bf16x8 qf[MAXRT][KS];
#pragma unroll
  for (int rt = 0; rt < MAXRT; ++rt) {
    const int row = rt * 16 + l16;
    const int m = row / a.G, h = row % a.G;
    const int64_t pos = pos0 + m;
    const __bf16* qrow = q + (((int64_t)b * a.H + g * a.G + h) * a.n + pos) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 qv = {0u, 0u, 0u, 0u};
      if (rt < RT && pos < a.nv) qv = *(const u32x4*)(qrow + 32 * s + 8 * lg);
      qf[rt][s] = as_bf16x8(qv);
    }
  }
  auto load_s = [&](int ct, f32x4 (&v)[KS][2]) {
    const int cand = ct * 16 + l16;
    const float* srow = a.summ + (bg * a.summ_blocks + (cand < t ? cand : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      v[s][0] = *(const f32x4*)(srow + 32 * s + 8 * lg);
      v[s][1] = *(const f32x4*)(srow + 32 * s + 8 * lg + 4);
      if (cand >= t) v[s][0] = v[s][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  };
  for (int ct = wave; ct < CT; ct += NT / kWave) {
    f32x4 sv[KS][2];
    load_s(ct, sv);
    bf16x8 hi[KS], mid[KS], lo[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float xv[8] = {sv[s][0].x, sv[s][0].y, sv[s][0].z, sv[s][0].w,
                           sv[s][1].x, sv[s][1].y, sv[s][1].z, sv[s][1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const __bf16 h = (__bf16)xv[i];
        const float r1 = xv[i] - (float)h;
        const __bf16 m = (__bf16)r1;
        hi[s][i] = h;
        mid[s][i] = m;
        lo[s][i] = (__bf16)(r1 - (float)m);
      }
    }
#pragma unroll
    for (int rt = 0; rt < MAXRT; ++rt) {
      if (rt < RT) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          acc = mfma16(lo[s], qf[rt][s], acc);
          acc = mfma16(mid[s], qf[rt][s], acc);
          acc = mfma16(hi[s], qf[rt][s], acc);
        }
        // C[cand 4*lg + i][row l16]
        const f32x4 outv = {acc.x * a.scale, acc.y * a.scale, acc.z * a.scale, acc.w * a.scale};
        *(f32x4*)(X + (rt * 16 + l16) * a.pitch + ct * 16 + 4 * lg) = outv;
      }
    }
  }
}

// ---- step 1, float32: plain FMAs -----------------------------------------------------
template <int D, int NT>
__device__ void route_scores_f32(const RouteArgs& a, float* X, int t, int64_t bg, int b, int g,
                                 int64_t pos0, int R) {
  const float* q = (const float*)a.q;
  for (int idx = threadIdx.x; idx < R * t; idx += NT) {
    const int row = idx / t, j = idx % t;
    const int m = row / a.G, h = row % a.G;
    const int64_t pos = pos0 + m;
    float acc = 0.f;
    if (pos < a.nv) {
      const float* qrow = q + (((int64_t)b * a.H + g * a.G + h) * a.n + pos) * D;
      const float* srow = a.summ + (bg * a.summ_blocks + j) * D;
      for (int c = 0; c < D; ++c) acc = fmaf(qrow[c], srow[c], acc);
    }
    X[row * a.pitch + j] = acc * a.scale;
  }
}

template <typename T, int D, int VPL, int MODE, int NT, int RT>
__global__ __launch_bounds__(NT) void route_prefill_kernel(RouteArgs a) {
  extern __shared__ float smem[];
  const int R = a.PP * a.G;
  float* X = smem;
  float* tau_s = X + R * a.pitch;
  int* uflag = (int*)(tau_s + R);

  const int64_t nbg = (int64_t)a.B * a.Hkv;
  const int64_t qt = a.n_qt - 1 - blockIdx.x / nbg;   // heaviest tiles first
  const int64_t bg = blockIdx.x % nbg;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t p_begin = qt * kQT;
  const int64_t tile = bg * a.n_qt + qt;
  a.nv = valid_len(a.seq_len, b, a.n);
  if (p_begin >= a.nv) {
    route_tile_past_end(a, tile);
    return;
  }
  const int npos = (int)min((int64_t)kQT, a.nv - p_begin);
  const int t = max(0, (int)(p_begin / a.bs) - (a.window - 1));   // candidates

  if (t == 0) {
    for (int idx = threadIdx.x; idx < npos * a.G; idx += NT) {
      const int m = idx / a.G, h = idx % a.G;
      const int64_t r = ((int64_t)b * a.H + g * a.G + h) * a.n + p_begin + m;
      a.tau[r] = __builtin_nanf("");
      if (a.bits)
        for (int w = 0; w < a.nwords; ++w) a.bits[r * a.nwords + w] = 0u;
    }
    if (threadIdx.x == 0) a.sel_count[tile] = 0;
    if (a.tile_bits)
      for (int w = threadIdx.x; w < a.nwords; w += blockDim.x) a.tile_bits[tile * a.nwords + w] = 0u;
    return;
  }

  for (int j = threadIdx.x; j < t; j += NT) uflag[j] = 0;
  const int lpr = NT / R;   // lanes per row in step 2
  const float invG = 1.0f / (float)a.G;

  for (int pp = 0; pp < npos; pp += a.PP) {
    const int64_t pos0 = p_begin + pp;
    __syncthreads();
    if constexpr (sizeof(T) == 2) route_scores_bf16<D, RT, NT>(a, X, t, bg, b, g, pos0, R);
    else route_scores_f32<D, NT>(a, X, t, bg, b, g, pos0, R);
    __syncthreads();

    const int np = min(a.PP, npos - pp);
    if constexpr (VPL > 0) {
      constexpr int LPR = NT / (16 * RT);   // lanes per row: NT / rows per pass
      // steps 2-3 with the row in registers: lane `sub` of the row's group
      // holds x_{sub + lpr*i}; the G rows of a position are adjacent groups,
      // so the GQA sum is a shuffle over G * lpr lanes.
      const int row = threadIdx.x / lpr, sub = threadIdx.x % lpr;
      const float* xr = X + row * a.pitch;
      float xv[VPL];
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int j = sub + lpr * i;
        xv[i] = j < t ? xr[j] : -INFINITY;
      }
      // slots 4 k .. 4 k + 3 hold candidates [4 k lpr, 4 (k + 1) lpr): only the
      // groups below t are visited
      const int nact4 = (t + 4 * lpr - 1) / (4 * lpr);
      float tau;
      if constexpr (LPR <= 16) tau = entmax_tau_reg<VPL, MODE>(xv, DppGroupReduce<LPR>{}, a.e, nact4);
      else tau = entmax_tau_reg<VPL, MODE>(xv, GroupReduce{lpr}, a.e, nact4);
      const int m = row / a.G, h = row % a.G;
      const int64_t pos = pos0 + m;
      if (pos < a.nv) {
        const int64_t r = ((int64_t)b * a.H + g * a.G + h) * a.n + pos;
        if (sub == 0) a.tau[r] = tau;
        if (a.bits)
          for (int w = sub; w < a.nwords; w += lpr) {
            uint32_t word = 0u;
            for (int i = 0; i < 32; ++i) {
              const int j = w * 32 + i;
              if (j < t && xr[j] > tau) word |= 1u << i;
            }
            a.bits[r * a.nwords + w] = word;
          }
      }
      float* pv = xv;   // p overwrites x
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const float y = xv[i] - tau;
        pv[i] = y > 0.f ? entmax_pow(y, MODE, a.e) : 0.f;
      }
      // GQA sum as a reduce-scatter over the G rows of a position (lanes
      // lpr apart): at the step over bit `bit` of h a lane keeps the half of
      // its slots whose bit agrees with its own h and sends the other half
      // to its partner.  Afterwards slot s (low log2 G bits clear) holds the
      // sum for slot s | h, which this lane then writes.
#pragma unroll
      for (int bb = 0; bb < 3; ++bb) {
        const int bit = 1 << bb;
        if (bit < a.G) {
          const bool up = (h & bit) != 0;
#pragma unroll
          for (int s2 = 0; s2 < VPL; ++s2) {
            if ((s2 & (2 * bit - 1)) != 0 || (s2 >> 2) >= nact4) continue;
            const float lo = pv[s2], hi = pv[s2 | bit];
            const float send = up ? lo : hi, keep = up ? hi : lo;
            pv[s2] = keep + lane_xor_c(send, LPR * bit);
          }
        }
      }
      if (m < np) {
#pragma unroll
        for (int s2 = 0; s2 < VPL; ++s2) {
          if (s2 % a.G != 0 || (s2 >> 2) >= nact4) continue;
          const int j = sub + lpr * (s2 | h);
          if (j < t) {
            const float pb = pv[s2] * invG;
            a.sel_logp[(tile * a.nb + j) * kQT + pp + m] = prior_bias(pb, a.sigma * kLn2);
            if (pb > 0.f) uflag[j] = 1;
          }
        }
      }
    } else {
      static_assert(VPL > 0 || MODE == kEntmaxGeneral, "the LDS path takes the mode at run time");
      // step 2: threshold per row (row read from LDS on every iteration)
      {
        const int row = threadIdx.x / lpr, sub = threadIdx.x % lpr;
        const float* xr = X + row * a.pitch;
        const float tau = entmax_tau([&](int j) { return xr[j]; }, t, sub, lpr, a.mode, a.e);
        const int m = row / a.G, h = row % a.G;
        const int64_t pos = pos0 + m;
        if (sub == 0) tau_s[row] = tau;
        if (pos < a.nv) {
          const int64_t r = ((int64_t)b * a.H + g * a.G + h) * a.n + pos;
          if (sub == 0) a.tau[r] = tau;
          if (a.bits)
            for (int w = sub; w < a.nwords; w += lpr) {
              uint32_t word = 0u;
              for (int i = 0; i < 32; ++i) {
                const int j = w * 32 + i;
                if (j < t && xr[j] > tau) word |= 1u << i;
              }
              a.bits[r * a.nwords + w] = word;
            }
        }
      }
      __syncthreads();
      // step 3: GQA average, log prior, tile-union flags
      for (int idx = threadIdx.x; idx < t * np; idx += NT) {
        const int j = idx / np, m = idx % np;
        float pb = 0.f;
        for (int h = 0; h < a.G; ++h) {
          const int row = m * a.G + h;
          const float y = X[row * a.pitch + j] - tau_s[row];
          if (y > 0.f) pb += entmax_pow(y, a.mode, a.e);
        }
        pb *= invG;
        a.sel_logp[(tile * a.nb + j) * kQT + pp + m] = prior_bias(pb, a.sigma * kLn2);
        if (pb > 0.f) uflag[j] = 1;
      }
    }
  }
  __syncthreads();

  // step 4: compaction (ascending block ids)
  if (threadIdx.x < kWave) compact_union(a, uflag, t, tile);
}


// positions per pass: largest power of two in [16/G, 64] whose score buffer
// fits the LDS budget
static int route_pp(int G, int pitch, size_t budget) {
  int pp = 64;
  while (pp > 1 && (size_t)pp * G * pitch * 4 > budget) pp >>= 1;
  while (pp * G < 16) pp <<= 1;
  while (pp * G > 16 * kRouteMaxRowTiles) pp >>= 1;
  return pp;
}

// Bit-packed tile masks -> ascending lists: one wave per tile; only bits on
// the tile's routing candidates count.
__global__ __launch_bounds__(kWave) void mask_to_list_kernel(
    const uint32_t* __restrict__ tile_bits, int32_t* __restrict__ sel_count,
    int32_t* __restrict__ sel_idx, int64_t n_qt, int64_t nb, int nwords, int bs, int window) {
  const int64_t tile = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t qt = tile % n_qt;
  const int t = max(0, (int)((qt * kQT) / bs) - (window - 1));
  const uint32_t* tb = tile_bits + tile * nwords;
  int base = 0;
  for (int j0 = 0; j0 < t; j0 += kWave) {
    const int j = j0 + lane;
    const bool f = j < t && ((tb[j >> 5] >> (j & 31)) & 1u) != 0u;
    const uint64_t mask = __ballot(f);
    if (f) sel_idx[tile * nb + base + __popcll(mask & ((1ull << lane) - 1ull))] = j;
    base += __popcll(mask);
  }
  if (lane == 0) sel_count[tile] = base;
}

hipError_t launch_mask_to_list(const Shape& s, int64_t n, const dash_route_buf& rb,
                               hipStream_t st) {
  const int64_t n_qt = (n + kQT - 1) / kQT;
  const int64_t nb = (n + s.bs - 1) / s.bs;
  hipLaunchKernelGGL(mask_to_list_kernel, dim3((unsigned)(n_qt * s.B * s.Hkv)), dim3(kWave), 0,
                     st, (const uint32_t*)rb.tile_bits, rb.sel_count, rb.sel_idx, n_qt, nb,
                     (int)((nb + 31) / 32), s.bs, s.window);
  return hipGetLastError();
}

hipError_t launch_route_prefill(const Shape& s, const void* q, int64_t n, const float* summ,
                                int64_t summ_blocks, const dash_route_buf& rb, hipStream_t st,
                                const int32_t* seq_len) {
  if (n <= 0) return hipSuccess;
  RouteArgs a;
  a.q = q;
  a.n = n;
  a.seq_len = seq_len;
  a.nv = n;
  a.summ = summ;
  a.summ_blocks = summ_blocks;
  a.tau = rb.tau;
  a.sel_count = rb.sel_count;
  a.sel_idx = rb.sel_idx;
  a.sel_logp = rb.sel_logp;
  a.bits = rb.support_bits;
  a.tile_bits = rb.tile_bits;
  a.n_qt = (n + kQT - 1) / kQT;
  a.nb = (n + s.bs - 1) / s.bs;
  a.nwords = (int)((a.nb + 31) / 32);
  a.H = s.H;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.bs = s.bs;
  a.B = s.B;
  a.mode = entmax_mode(s.alpha);
  a.e = 1.0f / (s.alpha - 1.0f);
  a.scale = (s.alpha - 1.0f) * s.gamma / sqrtf((float)s.d);
  a.sigma = s.sigma;
  a.window = s.window;
  const int t_max = max(0, (int)(((a.n_qt - 1) * kQT) / s.bs) - (s.window - 1));
  if (s.dtype == DASH_BF16 && t_max > 16 * kTileMaxCT && t_max <= 16 * kLongMaxCT && s.G >= 2)
    return launch_route_long(a, s, t_max, st);
  if (s.dtype == DASH_BF16 && t_max <= 16 * kTileMaxCT) return launch_route_tile(a, s, t_max, st);
  // pass-based path: NT threads, PP positions per pass with their score rows
  // in an LDS buffer of at most kRouteXBudget bytes
  a.pitch = round_up16(t_max > 0 ? t_max : 1) + 4;
  constexpr int NT = kRoutePassThreads;
  a.PP = route_pp(s.G, a.pitch, kRouteXBudget);
  const size_t lds = ((size_t)a.PP * s.G * a.pitch + (size_t)a.PP * s.G) * 4 +
                     (size_t)round_up16(t_max > 0 ? t_max : 1) * 4;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  dim3 grid((unsigned)(a.n_qt * s.B * s.Hkv));
  // register path: the row's candidates fit VPL per lane and a position's
  // G rows share one wave
  const int lpr = NT / (a.PP * s.G);
  const int need = (t_max + lpr - 1) / lpr;
  int vpl = 0;
  if (lpr * s.G <= kWave)
    vpl = need <= 8 ? 8 : need <= 16 ? 16 : need <= 32 ? 32 : (need <= 64 && NT <= 256) ? 64 : 0;
  const int rt_pass = a.PP * s.G / 16;   // row tiles per pass: 1, 2 or 4
#define DASH_RT4(T, D, V, M, R)                                                                 \
  do {                                                                                          \
    if (lds > 64 * 1024)                                                                        \
      (void)hipFuncSetAttribute((const void*)route_prefill_kernel<T, D, V, M, NT, R>,           \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);           \
    hipLaunchKernelGGL((route_prefill_kernel<T, D, V, M, NT, R>), grid, dim3(NT), lds, st, a);  \
  } while (0)
#define DASH_RT3(T, D, V, M)                                                  \
  do {                                                                        \
    if (rt_pass == 1) DASH_RT4(T, D, V, M, 1);                                \
    else if (rt_pass == 2) DASH_RT4(T, D, V, M, 2);                           \
    else DASH_RT4(T, D, V, M, 4);                                             \
  } while (0)
#define DASH_RT2(T, D, V)                                          \
  do {                                                             \
    if (a.mode == kEntmax15) DASH_RT3(T, D, V, kEntmax15);         \
    else if (a.mode == kSparsemax) DASH_RT3(T, D, V, kSparsemax);  \
    else if (a.mode == kEntmaxQuartic) DASH_RT3(T, D, V, kEntmaxQuartic); \
    else DASH_RT3(T, D, V, kEntmaxGeneral);                        \
  } while (0)
#define DASH_RT(T, D)                                              \
  do {                                                             \
    if (vpl == 8) DASH_RT2(T, D, 8);                               \
    else if (vpl == 16) DASH_RT2(T, D, 16);                        \
    else if (vpl == 32) DASH_RT2(T, D, 32);                        \
    else if (vpl == 64) DASH_RT2(T, D, 64);                        \
    else DASH_RT3(T, D, 0, kEntmaxGeneral);                        \
  } while (0)
  if (s.dtype == DASH_BF16) {
    if (s.d == 64) DASH_RT(__bf16, 64); else DASH_RT(__bf16, 128);
  } else {
    if (s.d == 64) DASH_RT(float, 64); else DASH_RT(float, 128);
  }
#undef DASH_RT
#undef DASH_RT2
#undef DASH_RT3
#undef DASH_RT4
  return hipGetLastError();
}

}  // namespace dash
