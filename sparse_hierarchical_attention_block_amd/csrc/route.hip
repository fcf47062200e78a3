// route.hip -- Stage 1 of DashAttention for causal prefill ("entmax chunk
// routing", DashAttention explainer, Technical summary): coarse scores of
// every query against the block summaries, w = alpha-entmax(gamma * zbar) per
// (query, head), GQA average of the probabilities of the heads sharing a KV
// head, union over a 64-position query tile and compaction into an ascending
// block list.
//
// One workgroup per (sequence, KV head, query tile of 64 positions), heaviest
// tiles (most candidate blocks) first.  Candidates of tile qt are the complete
// blocks j < floor(64 qt / bs).  Rows are (position, head of the group)
// pairs; they are processed in passes of PP positions:
//   1. scores X[row][j] = scale * q_row . s_j into an LDS buffer; bf16 queries
//      use MFMA 16x16x32 with the float32 summaries split into three bf16
//      parts (hi + mid + lo carries 24 mantissa bits), float32 queries use
//      plain FMAs;
//   2. tau per row (entmax_device.hpp), lanes-per-row = 256 / rows;
//   3. pbar per (position, block) = mean over the group's heads of
//      [x - tau]_+^e, written as log pbar (-inf for 0) into sel_logp, and the
//      tile-union flags.
// Finally wave 0 compacts the flags into sel_idx / sel_count.
#include "dash_internal.hpp"
#include "device_common.hpp"
#include "entmax_device.hpp"

namespace dash {

constexpr int kRouteThreads = 256;
constexpr int kQT = DASH_QUERY_TILE;

struct RouteArgs {
  const void* q;
  int64_t n;
  const float* summ;
  int64_t summ_blocks;
  float* tau;
  int32_t* sel_count;
  int32_t* sel_idx;
  float* sel_logp;
  uint32_t* bits;
  int64_t n_qt, nb;
  int nwords;
  int H, Hkv, G, bs, B;
  int mode;
  float e, scale;
  int PP;      // positions per pass
  int pitch;   // X row pitch in floats (multiple of 4)
};

__host__ __device__ inline int round_up16(int x) { return (x + 15) & ~15; }

// ---- step 1, bf16: MFMA with a 3-way bf16 split of the summaries ----------------
template <int D>
__device__ void route_scores_bf16(const RouteArgs& a, float* X, int t, int64_t bg, int b, int g,
                                  int64_t pos0, int R) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int l16 = lane % 16, lg = lane / 16;
  const __bf16* q = (const __bf16*)a.q;
  const int CT = round_up16(t) / 16;
  constexpr int KS = D / 32;
  for (int ct = wave; ct < CT; ct += kRouteThreads / kWave) {
    const int cand = ct * 16 + l16;
    const float* srow = a.summ + (bg * a.summ_blocks + cand) * D;
    bf16x8 hi[KS], mid[KS], lo[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
      if (cand < t) {
        v0 = *(const f32x4*)(srow + 32 * s + 8 * lg);
        v1 = *(const f32x4*)(srow + 32 * s + 8 * lg + 4);
      }
      float xv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __bf16 h = (__bf16)xv[i];
        float r1 = xv[i] - (float)h;
        __bf16 m = (__bf16)r1;
        float r2 = r1 - (float)m;
        hi[s][i] = h;
        mid[s][i] = m;
        lo[s][i] = (__bf16)r2;
      }
    }
    for (int rt = 0; rt < R / 16; ++rt) {
      const int row = rt * 16 + l16;
      const int m = row / a.G, h = row % a.G;
      const int64_t pos = pos0 + m;
      const __bf16* qrow = q + (((int64_t)b * a.H + g * a.G + h) * a.n + pos) * D;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        u32x4 qv = {0u, 0u, 0u, 0u};
        if (pos < a.n) qv = *(const u32x4*)(qrow + 32 * s + 8 * lg);
        bf16x8 qf = as_bf16x8(qv);
        acc = mfma16(lo[s], qf, acc);
        acc = mfma16(mid[s], qf, acc);
        acc = mfma16(hi[s], qf, acc);
      }
      // C[cand 4*lg + i][row l16]
      f32x4 outv = {acc.x * a.scale, acc.y * a.scale, acc.z * a.scale, acc.w * a.scale};
      *(f32x4*)(X + row * a.pitch + ct * 16 + 4 * lg) = outv;
    }
  }
}

// ---- step 1, float32: plain FMAs -----------------------------------------------------
template <int D>
__device__ void route_scores_f32(const RouteArgs& a, float* X, int t, int64_t bg, int b, int g,
                                 int64_t pos0, int R) {
  const float* q = (const float*)a.q;
  for (int idx = threadIdx.x; idx < R * t; idx += kRouteThreads) {
    const int row = idx / t, j = idx % t;
    const int m = row / a.G, h = row % a.G;
    const int64_t pos = pos0 + m;
    float acc = 0.f;
    if (pos < a.n) {
      const float* qrow = q + (((int64_t)b * a.H + g * a.G + h) * a.n + pos) * D;
      const float* srow = a.summ + (bg * a.summ_blocks + j) * D;
      for (int c = 0; c < D; ++c) acc = fmaf(qrow[c], srow[c], acc);
    }
    X[row * a.pitch + j] = acc * a.scale;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kRouteThreads) void route_prefill_kernel(RouteArgs a) {
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
  const int npos = (int)min((int64_t)kQT, a.n - p_begin);
  const int t = (int)(p_begin / a.bs);
  const int64_t tile = bg * a.n_qt + qt;

  if (t == 0) {
    for (int idx = threadIdx.x; idx < npos * a.G; idx += kRouteThreads) {
      const int m = idx / a.G, h = idx % a.G;
      const int64_t r = ((int64_t)b * a.H + g * a.G + h) * a.n + p_begin + m;
      a.tau[r] = __builtin_nanf("");
      if (a.bits)
        for (int w = 0; w < a.nwords; ++w) a.bits[r * a.nwords + w] = 0u;
    }
    if (threadIdx.x == 0) a.sel_count[tile] = 0;
    return;
  }

  for (int j = threadIdx.x; j < t; j += kRouteThreads) uflag[j] = 0;
  const int lpr = kRouteThreads / R;   // lanes per row in step 2
  const float invG = 1.0f / (float)a.G;

  for (int pp = 0; pp < npos; pp += a.PP) {
    const int64_t pos0 = p_begin + pp;
    __syncthreads();
    if constexpr (sizeof(T) == 2) route_scores_bf16<D>(a, X, t, bg, b, g, pos0, R);
    else route_scores_f32<D>(a, X, t, bg, b, g, pos0, R);
    __syncthreads();

    // step 2: threshold per row
    {
      const int row = threadIdx.x / lpr, sub = threadIdx.x % lpr;
      const float* xr = X + row * a.pitch;
      const float tau = entmax_tau([&](int j) { return xr[j]; }, t, sub, lpr, a.mode, a.e);
      const int m = row / a.G, h = row % a.G;
      const int64_t pos = pos0 + m;
      if (sub == 0) tau_s[row] = tau;
      if (pos < a.n) {
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
    const int np = min(a.PP, npos - pp);
    for (int idx = threadIdx.x; idx < t * np; idx += kRouteThreads) {
      const int j = idx / np, m = idx % np;
      float pb = 0.f;
      for (int h = 0; h < a.G; ++h) {
        const int row = m * a.G + h;
        const float y = X[row * a.pitch + j] - tau_s[row];
        if (y > 0.f) pb += entmax_pow(y, a.mode, a.e);
      }
      pb *= invG;
      a.sel_logp[(tile * a.nb + j) * kQT + pp + m] = pb > 0.f ? __logf(pb) : -INFINITY;
      if (pb > 0.f) uflag[j] = 1;
    }
  }
  __syncthreads();

  // step 4: compaction (ascending block ids)
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int base = 0;
    for (int j0 = 0; j0 < t; j0 += kWave) {
      const int j = j0 + lane;
      const bool f = j < t && uflag[j] != 0;
      const uint64_t mask = __ballot(f);
      const int before = __popcll(mask & ((1ull << lane) - 1ull));
      if (f) a.sel_idx[tile * a.nb + base + before] = j;
      base += __popcll(mask);
    }
    if (lane == 0) a.sel_count[tile] = base;
  }
}

// positions per pass: largest power of two in [16/G, 64] whose score buffer
// fits the LDS budget
static int route_pp(int G, int pitch, size_t budget) {
  int pp = 64;
  while (pp > 1 && (size_t)pp * G * pitch * 4 > budget) pp >>= 1;
  while (pp * G < 16) pp <<= 1;
  while (pp * G > kRouteThreads) pp >>= 1;
  return pp;
}

hipError_t launch_route_prefill(const Shape& s, const void* q, int64_t n, const float* summ,
                                int64_t summ_blocks, const dash_route_buf& rb, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  RouteArgs a;
  a.q = q;
  a.n = n;
  a.summ = summ;
  a.summ_blocks = summ_blocks;
  a.tau = rb.tau;
  a.sel_count = rb.sel_count;
  a.sel_idx = rb.sel_idx;
  a.sel_logp = rb.sel_logp;
  a.bits = rb.support_bits;
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
  const int t_max = (int)(((a.n_qt - 1) * kQT) / s.bs);
  a.pitch = round_up16(t_max > 0 ? t_max : 1) + 4;
  a.PP = route_pp(s.G, a.pitch, 64 * 1024);
  const size_t lds = ((size_t)a.PP * s.G * a.pitch + (size_t)a.PP * s.G) * 4 +
                     (size_t)round_up16(t_max > 0 ? t_max : 1) * 4;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  dim3 grid((unsigned)(a.n_qt * s.B * s.Hkv));
#define DASH_RT(T, D)                                                                   \
  do {                                                                                  \
    if (lds > 64 * 1024)                                                                \
      (void)hipFuncSetAttribute((const void*)route_prefill_kernel<T, D>,                \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);   \
    hipLaunchKernelGGL((route_prefill_kernel<T, D>), grid, dim3(kRouteThreads), lds, st, a); \
  } while (0)
  if (s.dtype == DASH_BF16) {
    if (s.d == 64) DASH_RT(__bf16, 64); else DASH_RT(__bf16, 128);
  } else {
    if (s.d == 64) DASH_RT(float, 64); else DASH_RT(float, 128);
  }
#undef DASH_RT
  return hipGetLastError();
}

}  // namespace dash
