// decode.hip -- one incremental decoding step of DashAttention (the pages'
// kernels support "prefill and incremental decoding"; chunk summaries are
// cached once a chunk is complete -- DashAttention explainer, Technical
// summary, Stage 0 and Contributions).
//
// Per sequence b the new query sits at position L = cache_len[b] - 1:
//   1. decode_scores   x[b,h,j] = (alpha-1) gamma q_h . s_j / sqrt(d) for the
//                      cached summaries j < floor(L / bs)  (HBM scan of the
//                      float32 summary cache, 64 blocks per workgroup)
//   2. decode_route    one wave per query head finds tau; the G heads of a KV
//                      head average p; the union is compacted into an
//                      ascending list with log pbar per listed block
//   3. decode_attend   split-K over the list [own block, selected blocks...],
//                      16 entries per workgroup, 4 waves; MFMA 16x16x32 with
//                      the G query heads as MFMA rows (padded to 16); K and V
//                      stream from HBM straight into registers, V is
//                      transposed 8x8 in registers
//   4. decode_combine  log-sum-exp merge of the splits in a fixed order
//   5. when cache_len[b] % bs == 0 the completed block's summary is written.
#include "dash_internal.hpp"
#include "device_common.hpp"
#include "entmax_device.hpp"

namespace dash {

hipError_t launch_summarize_completed(const Shape& s, const void* kc, int64_t max_len,
                                      const int32_t* cache_len, const float* w_s, float* summ,
                                      int64_t summ_blocks, hipStream_t st);

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
  float* part;       // [B, Hkv, n_split, G, D + 2]
  int64_t nb;
  int64_t n_split;
  int nwords;
  int H, Hkv, G, bs, B;
  int mode;
  float e, scale, scale_log2;
};

__device__ __forceinline__ int64_t min64(int64_t x, int64_t y) { return x < y ? x : y; }

__device__ __forceinline__ int64_t clamp_len(int32_t v, int64_t max_len) {
  int64_t l = v;
  return l < 1 ? 1 : (l > max_len ? max_len : l);
}

// ---- 1. coarse scores ------------------------------------------------------------------------
// One thread per cached summary j; the row is read with 16-byte loads (32
// floats in flight per batch) and serves all G heads, whose queries sit in LDS.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_scores_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) float qs[8][D];
  const int64_t bg = blockIdx.y;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t len = clamp_len(a.cache_len[b], a.max_len);
  const int64_t ncand = (len - 1) / a.bs;
  const int64_t j0 = (int64_t)blockIdx.x * 64;
  if (j0 >= ncand) return;
  const T* qb = (const T*)a.q + ((int64_t)b * a.H + g * a.G) * D;
  for (int e = threadIdx.x; e < a.G * D; e += 64) qs[e / D][e % D] = to_f32(qb[e]);
  __syncthreads();
  const int64_t j = j0 + threadIdx.x;
  if (j >= ncand) return;
  const float* srow = a.summ + (bg * a.summ_blocks + j) * D;
  float acc[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) acc[h] = 0.f;
#pragma unroll
  for (int c0 = 0; c0 < D; c0 += 32) {
    f32x4 sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = *(const f32x4*)(srow + c0 + 4 * i);
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      if (h < a.G) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const f32x4 qv = *(const f32x4*)(&qs[h][c0 + 4 * i]);
          acc[h] = fmaf(qv.x, sv[i].x, acc[h]);
          acc[h] = fmaf(qv.y, sv[i].y, acc[h]);
          acc[h] = fmaf(qv.z, sv[i].z, acc[h]);
          acc[h] = fmaf(qv.w, sv[i].w, acc[h]);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 8; ++h)
    if (h < a.G) a.x[((int64_t)b * a.H + g * a.G + h) * a.nb + j] = acc[h] * a.scale;
}

// ---- 2. threshold, GQA average, union, compaction ------------------------------------------
__global__ __launch_bounds__(512) void decode_route_kernel(DecodeArgs a) {
  extern __shared__ float Ps[];   // [G][nb]
  const int64_t bg = blockIdx.x;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t len = clamp_len(a.cache_len[b], a.max_len);
  const int ncand = (int)((len - 1) / a.bs);
  const int lane = threadIdx.x % kWave, hh = threadIdx.x / kWave;
  const int64_t row = (int64_t)b * a.H + g * a.G + hh;
  const float* xr = a.x + row * a.nb;
  if (ncand == 0) {
    if (lane == 0) a.tau[row] = __builtin_nanf("");
    if (a.bits)
      for (int w = lane; w < a.nwords; w += kWave) a.bits[row * a.nwords + w] = 0u;
    if (threadIdx.x == 0) a.count[bg] = 0;
    return;
  }
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
  __syncthreads();
  const float invG = 1.0f / (float)a.G;
  for (int j = threadIdx.x; j < ncand; j += blockDim.x) {
    float pb = 0.f;
    for (int h = 0; h < a.G; ++h) pb += Ps[h * a.nb + j];
    pb *= invG;
    a.logp[bg * a.nb + j] = pb > 0.f ? __logf(pb) : -INFINITY;
    Ps[j] = pb;   // column j is only touched by this thread
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    int base = 0;
    for (int j0 = 0; j0 < ncand; j0 += kWave) {
      const int j = j0 + lane;
      const bool f = j < ncand && Ps[j] > 0.f;
      const uint64_t mask = __ballot(f);
      if (f) a.idx[bg * a.nb + base + __popcll(mask & ((1ull << lane) - 1ull))] = j;
      base += __popcll(mask);
    }
    if (lane == 0) a.count[bg] = base;
  }
}

// ---- 3. split-K attend (bf16, MFMA) ----------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_attend_bf16_kernel(DecodeArgs a) {
  constexpr int DPL = D / 16;   // d columns per lane in the PV product
  __shared__ float ms[4][16], ls[4][16];
  __shared__ float os[4][16][D];
  const int s = blockIdx.x;
  const int64_t bg = blockIdx.y;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t len = clamp_len(a.cache_len[b], a.max_len);
  const int64_t own = (len - 1) / a.bs;
  const int count = a.count[bg];
  const int n_entries = 1 + count;
  if (s * kDecodeSplit >= n_entries) return;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int l16 = lane % 16, lg = lane / 16;

  const __bf16* kb = (const __bf16*)a.kc + bg * a.max_len * D;
  const __bf16* vb = (const __bf16*)a.vc + bg * a.max_len * D;

  // Q^T operand: column = query head l16 (< G), k = d in [32 s' + 8 lg, +8)
  bf16x8 qf[D / 32];
  {
    const __bf16* qrow = (const __bf16*)a.q + ((int64_t)b * a.H + g * a.G + l16) * D;
#pragma unroll
    for (int sp = 0; sp < D / 32; ++sp) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (l16 < a.G) w = *(const u32x4*)(qrow + 32 * sp + 8 * lg);
      qf[sp] = as_bf16x8(w);
    }
  }
  f32x4 acc[DPL];
#pragma unroll
  for (int c = 0; c < DPL; ++c) acc[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int e_end = min(n_entries, (s + 1) * kDecodeSplit);
  for (int e = s * kDecodeSplit + wave; e < e_end; e += 4) {
    const int64_t j = e == 0 ? own : (int64_t)a.idx[bg * a.nb + e - 1];
    const float bias2 = e == 0 ? 0.f : a.logp[bg * a.nb + j] * kLog2e;
    for (int c64 = 0; c64 < a.bs / 64; ++c64) {
      const int64_t key0 = j * a.bs + 64 * c64;
      if (key0 >= len) break;
      // Issue every load of the chunk before any use.  Addresses are clamped
      // to the last valid key, so each load stays in bounds and reads finite
      // data; keys >= len are masked below (score -inf, probability 0).
      u32x4 kw[4][D / 32];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int64_t key = min64(key0 + 16 * kt + l16, len - 1);
#pragma unroll
        for (int sp = 0; sp < D / 32; ++sp)
          kw[kt][sp] = *(const u32x4*)(kb + key * D + 32 * sp + 8 * lg);
      }
      // V rows this lane needs: k = 8 lg + e' <-> key 32 ks + 16 (e'/4) + 4 lg + e'%4,
      // DPL consecutive d starting at DPL * l16
      uint32_t vin[2][8][DPL / 2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ep = 0; ep < 8; ++ep) {
          const int64_t key = min64(key0 + 32 * ks + 16 * (ep / 4) + 4 * lg + (ep % 4), len - 1);
          if constexpr (DPL == 8) {
            const u32x4 t = *(const u32x4*)(vb + key * D + DPL * l16);
            vin[ks][ep][0] = t.x; vin[ks][ep][1] = t.y; vin[ks][ep][2] = t.z; vin[ks][ep][3] = t.w;
          } else {
            const u32x2 t = *(const u32x2*)(vb + key * D + DPL * l16);
            vin[ks][ep][0] = t.x; vin[ks][ep][1] = t.y;
          }
        }
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
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
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
      psum += __shfl_xor(psum, 16, kWave);
      psum += __shfl_xor(psum, 32, kWave);
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

  // ---- merge the 4 waves in a fixed order ----
  if (lane < 16) {
    ms[wave][lane] = m_run;
    ls[wave][lane] = l_run;
  }
#pragma unroll
  for (int c = 0; c < DPL; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) os[wave][4 * lg + i][DPL * l16 + c] = acc[c][i];
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
  const int n_entries = 1 + count;
  if (s * kDecodeSplit >= n_entries) return;
  const float* kb = (const float*)a.kc + bg * a.max_len * D;
  const float* vb = (const float*)a.vc + bg * a.max_len * D;
  const float* qb = (const float*)a.q + ((int64_t)b * a.H + g * a.G) * D;
  for (int e = threadIdx.x; e < a.G * D; e += 256) qs[e / D][e % D] = qb[e];
  const int qr = threadIdx.x / 32, dl = threadIdx.x % 32;   // 8 heads x 32 lanes
  float m_run = -INFINITY, l_run = 0.f, ov[D / 32];
  for (int c = 0; c < D / 32; ++c) ov[c] = 0.f;
  const int e_end = min(n_entries, (s + 1) * kDecodeSplit);
  for (int e = s * kDecodeSplit; e < e_end; ++e) {
    const int64_t j = e == 0 ? own : (int64_t)a.idx[bg * a.nb + e - 1];
    const float bias2 = e == 0 ? 0.f : a.logp[bg * a.nb + j] * kLog2e;
    for (int64_t key0 = j * a.bs; key0 < (j + 1) * a.bs && key0 < len; key0 += 64) {
      __syncthreads();
      for (int p = threadIdx.x; p < a.G * 64; p += 256) {
        const int h = p / 64, kk = p % 64;
        const int64_t key = key0 + kk;
        float sv = -INFINITY;
        if (key < len) {
          float acc = 0.f;
          for (int c = 0; c < D; ++c) acc = fmaf(qs[h][c], kb[key * D + c], acc);
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
          for (int c = 0; c < D / 32; ++c) ov[c] = fmaf(p, vb[(key0 + kk) * D + dl + 32 * c], ov[c] * corr);
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

// ---- 4. combine --------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int64_t bh = blockIdx.x;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int g = h / a.G, qr = h % a.G;
  const int64_t bg = (int64_t)b * a.Hkv + g;
  const int n_entries = 1 + a.count[bg];
  const int ns = (n_entries + kDecodeSplit - 1) / kDecodeSplit;
  const float* part = a.part + (bg * a.n_split * a.G + qr) * (D + 2);
  const int64_t stride = (int64_t)a.G * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, part[s * stride]);
  float L = 0.f, O = 0.f;
  const int d = threadIdx.x;
  for (int s = 0; s < ns; ++s) {
    const float ms = part[s * stride];
    const float f = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
    L += part[s * stride + 1] * f;
    O += part[s * stride + 2 + d] * f;
  }
  ((T*)a.o)[bh * D + d] = from_f32<T>(O / L);
}

DecodeLayout decode_layout(const Shape& s, int64_t max_len) {
  DecodeLayout L;
  L.nb = (max_len + s.bs - 1) / s.bs;
  L.ncand_max = (max_len - 1) / s.bs;
  L.n_split = (L.ncand_max + 1 + kDecodeSplit - 1) / kDecodeSplit;
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
                         const int32_t* cache_len, int64_t max_len, const float* w_s, float* summ,
                         int64_t summ_blocks, void* o, const dash_route_buf& rb,
                         const DecodeLayout& L, char* ws, hipStream_t st) {
  DecodeArgs a;
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
  a.part = (float*)(ws + L.off_part);
  a.nb = L.nb;
  a.n_split = L.n_split;
  a.nwords = (int)((L.nb + 31) / 32);
  a.H = s.H;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.bs = s.bs;
  a.B = s.B;
  a.mode = entmax_mode(s.alpha);
  a.e = 1.0f / (s.alpha - 1.0f);
  a.scale = (s.alpha - 1.0f) * s.gamma / sqrtf((float)s.d);
  a.scale_log2 = kLog2e / sqrtf((float)s.d);
  const bool bf16 = s.dtype == DASH_BF16;
  const unsigned nbg = (unsigned)(s.B * s.Hkv);

  if (L.ncand_max > 0) {
    dim3 g1((unsigned)((L.ncand_max + 63) / 64), nbg);
#define DASH_DS(T, D) hipLaunchKernelGGL((decode_scores_kernel<T, D>), g1, dim3(64), 0, st, a)
    if (bf16) { if (s.d == 64) DASH_DS(__bf16, 64); else DASH_DS(__bf16, 128); }
    else { if (s.d == 64) DASH_DS(float, 64); else DASH_DS(float, 128); }
#undef DASH_DS
  }
  const size_t lds = sizeof(float) * s.G * L.nb;
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute((const void*)decode_route_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(decode_route_kernel, dim3(nbg), dim3(64 * s.G), lds, st, a);

  dim3 g3((unsigned)L.n_split, nbg);
  if (bf16) {
    if (s.d == 64) hipLaunchKernelGGL(decode_attend_bf16_kernel<64>, g3, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(decode_attend_bf16_kernel<128>, g3, dim3(256), 0, st, a);
  } else {
    if (s.d == 64) hipLaunchKernelGGL(decode_attend_f32_kernel<64>, g3, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(decode_attend_f32_kernel<128>, g3, dim3(256), 0, st, a);
  }
  dim3 g4((unsigned)(s.B * s.H));
#define DASH_DC(T, D) hipLaunchKernelGGL((decode_combine_kernel<T, D>), g4, dim3(D), 0, st, a)
  if (bf16) { if (s.d == 64) DASH_DC(__bf16, 64); else DASH_DC(__bf16, 128); }
  else { if (s.d == 64) DASH_DC(float, 64); else DASH_DC(float, 128); }
#undef DASH_DC
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_summarize_completed(s, kc, max_len, cache_len, w_s, summ, summ_blocks, st);
}

}  // namespace dash
