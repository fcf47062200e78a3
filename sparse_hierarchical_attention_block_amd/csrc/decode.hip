// decode.hip -- one incremental decoding step of DashAttention (the pages'
// kernels support "prefill and incremental decoding"; chunk summaries are
// cached once a chunk is complete -- DashAttention explainer, Technical
// summary, Stage 0 and Contributions).
//
// Per sequence b the new query sits at position L = cache_len[b] - 1:
//   1. decode_scores   x[b,h,j] = (alpha-1) gamma q_h . s_j / sqrt(d) for the
//                      cached summaries j < floor(L / bs)  (HBM scan of the
//                      float32 summary cache, 64 blocks per workgroup); one
//                      more workgroup per (sequence, KV head) writes the
//                      summary of the block the step completes, if any
//                      (cache_len[b] % bs == 0)
//   2. decode_route    one wave per query head finds tau; the G heads of a KV
//                      head average p; the union is compacted into an
//                      ascending list with log pbar per listed block
//   3. decode_attend   split-K over the list [own block, selected blocks...],
//                      32 entries per work item, a persistent grid walking
//                      the items, 4 waves; MFMA 16x16x32 with the G query
//                      heads as MFMA rows (padded to 16); K and V stream from
//                      HBM straight into registers, V is transposed 8x8 in
//                      registers
//   4. decode_combine  log-sum-exp merge of the splits in a fixed order
#include <atomic>

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
  float* summ_w;     // the summary cache, written for a block this step completes
  const float* w_s;
  int64_t nb;
  int64_t n_split;
  int nwords;
  int H, Hkv, G, bs, B;
  int bs_log;        // log2(bs)
  int mode;
  float e, scale, scale_log2;
};

__host__ __device__ inline int64_t min64(int64_t x, int64_t y) { return x < y ? x : y; }

__device__ __forceinline__ int64_t clamp_len(int32_t v, int64_t max_len) {
  int64_t l = v;
  return l < 1 ? 1 : (l > max_len ? max_len : l);
}

// ---- 1. coarse scores ------------------------------------------------------------------------
// One thread per cached summary j; the row is read with 16-byte loads (32
// floats in flight per batch) and serves all G heads, whose queries sit in LDS.
// Summary of one complete block by a 64-thread workgroup, float32 throughout:
// column sums with 16-byte loads (thread = 16-byte column chunk x row group,
// every load of a thread in flight together), reduced over the row groups in
// LDS, then the projection by W_s with 16-byte loads of W_s rows (thread =
// 4 consecutive output columns x a share of the rows), reduced again in LDS.
// sh holds at least 9 D floats.
template <typename T, int D>
__device__ void summarize_block_64(const T* __restrict__ kb, int bs, const float* __restrict__ w_s,
                                   float* __restrict__ out, float* sh) {
  constexpr int EPV = 16 / sizeof(T);   // elements per 16-byte load
  constexpr int CH = D / EPV;           // 16-byte chunks per key row
  constexpr int RG = 64 / CH;           // row groups
  const int t = threadIdx.x;
  {
    const int ch = t % CH, rg = t / CH;
    float acc[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] = 0.f;
#pragma unroll 4
    for (int r = rg; r < bs; r += RG) {
      const u32x4 w = *(const u32x4*)(kb + (int64_t)r * D + ch * EPV);
      if constexpr (sizeof(T) == 2) {
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += bf16_lo(ww[e]);
          acc[2 * e + 1] += bf16_hi(ww[e]);
        }
      } else {
        acc[0] += __uint_as_float(w.x);
        acc[1] += __uint_as_float(w.y);
        acc[2] += __uint_as_float(w.z);
        acc[3] += __uint_as_float(w.w);
      }
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e) sh[rg * D + ch * EPV + e] = acc[e];
  }
  __syncthreads();
  float* mean = sh + 8 * D;
  for (int c = t; c < D; c += 64) {
    float sum = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < RG; ++g2) sum += sh[g2 * D + c];
    mean[c] = sum * (1.0f / (float)bs);
  }
  __syncthreads();
  constexpr int CQ = D / 4;    // column quads
  constexpr int RP = 64 / CQ;  // row shares
  const int cq = t % CQ, rp = t / CQ;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int r = rp; r < D; r += RP) {
    const f32x4 wv = *(const f32x4*)(w_s + r * D + 4 * cq);
    const float m = mean[r];
    o.x = fmaf(m, wv.x, o.x);
    o.y = fmaf(m, wv.y, o.y);
    o.z = fmaf(m, wv.z, o.z);
    o.w = fmaf(m, wv.w, o.w);
  }
  *(f32x4*)(sh + rp * D + 4 * cq) = o;   // sh rows < RP <= 4 do not overlap mean
  __syncthreads();
  for (int c = t; c < D; c += 64) {
    float sum = 0.f;
#pragma unroll
    for (int p2 = 0; p2 < RP; ++p2) sum += sh[p2 * D + c];
    out[c] = sum;
  }
}

// grid.x = ceil(ncand_max / 64) + 1: the last column of workgroups writes the
// summary of the block this step completes, if any (cache_len[b] % bs == 0
// completes block cache_len[b] / bs - 1); it overlaps the score scan.
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_scores_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) float qs[8][D];
  const int64_t bg = blockIdx.y;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t len = clamp_len(a.cache_len[b], a.max_len);
  if (blockIdx.x == gridDim.x - 1) {
    if (len % a.bs == 0) {
      const int64_t j = len / a.bs - 1;
      __shared__ __attribute__((aligned(16))) float sh[9 * D];
      summarize_block_64<T, D>((const T*)a.kc + (bg * a.max_len + j * a.bs) * D, a.bs, a.w_s,
                               a.summ_w + (bg * a.summ_blocks + j) * D, sh);
    }
    return;
  }
  const int64_t ncand = (len - 1) >> a.bs_log;
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
// One workgroup per (sequence, KV head), one wave per query head.  With VPL > 0
// the wave keeps its row of scores in registers (VPL per lane, candidate j in
// lane j % 64, slot j / 64) and solves for tau there (MODE: entmax_mode of
// alpha); VPL = 0 walks the row in memory for lists longer than 64 * 32.
template <int VPL, int MODE>
__global__ __launch_bounds__(512) void decode_route_kernel(DecodeArgs a) {
  extern __shared__ float Ps[];   // [G][nb]
  const int64_t bg = blockIdx.x;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t len = clamp_len(a.cache_len[b], a.max_len);
  const int ncand = (int)((len - 1) >> a.bs_log);
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
  if constexpr (VPL > 0) {
    float xv[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int j = lane + kWave * i;
      xv[i] = j < ncand ? xr[j] : -INFINITY;
    }
    const int nact4 = (ncand + 4 * kWave - 1) / (4 * kWave);
    const float tau = entmax_tau_reg<VPL, MODE>(xv, GroupReduce{kWave}, a.e, nact4);
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
      if (j < ncand) Ps[hh * a.nb + j] = y > 0.f ? entmax_pow(y, MODE, a.e) : 0.f;
    }
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
// One work item: split s of the list of (sequence, KV head) bgi, i.e. entries
// [s * kDecodeSplit, (s + 1) * kDecodeSplit) of [own block, selected blocks...].
// All 256 threads call; ms / ls / os are the workgroup's merge buffers.
template <int D>
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
    const int64_t slot = min64(max(s * kDecodeSplit + wv + 4 * lane - 1, 0), a.nb - 1);
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
  const int n_entries = 1 + count;

  // K/V of this (sequence, KV head) through buffer resources sized to the
  // current length: keys >= len read as zeros (and are masked below)
  const uint32_t len_bytes = (uint32_t)(len * (D * 2));
  const buf_rsrc rk = make_rsrc((const __bf16*)a.kc + bg * a.max_len * D, len_bytes);
  const buf_rsrc rv = make_rsrc((const __bf16*)a.vc + bg * a.max_len * D, len_bytes);

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
    const int64_t j = e == 0 ? own : (int64_t)jraw[ei];
    for (int c64 = 0; c64 < (a.bs >> 6); ++c64) {
      const int64_t key0 = (j << a.bs_log) + 64 * c64;
      if (key0 >= len) break;
      // Issue every load of the chunk before any use (32-bit byte offsets
      // from the chunk's first key).
      const uint32_t c0 = (uint32_t)(key0 * (D * 2));
      u32x4 kw[4][D / 32];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int sp = 0; sp < D / 32; ++sp)
          kw[kt][sp] = buf_load16(rk, c0 + (16 * kt + l16) * (D * 2) + (32 * sp + 8 * lg) * 2);
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
            const u32x4 t = buf_load16(rv, off);
            vin[ks][ep][0] = t.x; vin[ks][ep][1] = t.y; vin[ks][ep][2] = t.z; vin[ks][ep][3] = t.w;
          } else {
            const u32x2 t = buf_load8(rv, off);
            vin[ks][ep][0] = t.x; vin[ks][ep][1] = t.y;
          }
        }
      const float bias2 = e == 0 ? 0.f : a.logp[bg * a.nb + j] * kLog2e;
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
// workgroup derives the work items from the list lengths -- item ranges
// pre[bg] .. pre[bg+1] with ceil((1 + count[bg]) / kDecodeSplit) items per
// (sequence, KV head) -- and takes items blockIdx.x, + gridDim.x, ...  No
// workgroup is launched for a split past its list, so none holds a slot
// waiting only to find it has nothing to do.
template <int D>
__global__ __launch_bounds__(256) void decode_attend_bf16_kernel(DecodeArgs a) {
  __shared__ float ms[4][16], ls[4][16];
  __shared__ float os[4][8][D];
  __shared__ int pre[kDecodeMaxBg + 1];
  __shared__ int wsum[4];
  const int nbg = a.B * a.Hkv;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  // exclusive prefix of the item counts: 256 contiguous ranges, then a scan
  // of the range totals
  const int per = (nbg + 255) / 256;
  const int i0 = min(nbg, (int)threadIdx.x * per), i1 = min(nbg, i0 + per);
  int tot = 0;
  for (int i = i0; i < i1; ++i) {
    const int ns = (a.count[i] + kDecodeSplit) / kDecodeSplit;   // ceil((1 + count) / split)
    pre[i] = ns;
    tot += ns;
  }
  int incl = tot;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int run = incl - tot;
  for (int w = 0; w < wave; ++w) run += wsum[w];
  for (int i = i0; i < i1; ++i) {
    const int ns = pre[i];
    pre[i] = run;
    run += ns;
  }
  const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  if (threadIdx.x == 0) pre[nbg] = total;
  __syncthreads();
  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    int lo = 0, hi = nbg;   // pre[lo] <= it < pre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= it) lo = mid; else hi = mid;
    }
    decode_item<D>(a, lo, it - pre[lo], ms, ls, os);
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

// ---- 4. combine ----------------------------------------------------------------------------
// grid (ceil(G D / 256), B Hkv): workgroup x merges outputs [256 x, 256 x + 256)
// of the G heads x D columns of one (sequence, KV head), one output per
// thread.  The split maxima and sums of the heads it covers are staged in LDS
// and turned into weights exp2(m_s - M) by one thread per head; every thread
// then reads its column of all ns splits, 16 loads in flight.  Fixed order in s.
constexpr int kCombineThreads = 256;
template <typename T, int D>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecodeArgs a) {
  extern __shared__ float wts[];   // [HPW][ns] weights, [HPW][ns] l_s, [HPW] 1 / L
  constexpr int HPW = kCombineThreads / D;   // heads per workgroup (D <= 256)
  const int bgi = blockIdx.y;
  const int64_t bg = bgi;
  const int b = bgi / a.Hkv, g = bgi % a.Hkv;
  const int n_entries = 1 + a.count[bg];
  const int ns = (n_entries + kDecodeSplit - 1) / kDecodeSplit;
  const int G = a.G;
  const int q0 = blockIdx.x * HPW;                 // first head of this workgroup
  const int64_t stride = (int64_t)G * (D + 2);     // one split: G rows of [m, l, o(D)]
  const float* part = a.part + bg * a.n_split * stride;
  float* ls = wts + HPW * ns;
  float* inv_l = ls + HPW * ns;
  for (int e = threadIdx.x; e < HPW * ns; e += kCombineThreads) {
    const int hq = e / ns, sp = e % ns;
    if (q0 + hq < G) {
      const float* pr = part + sp * stride + (q0 + hq) * (D + 2);
      wts[e] = pr[0];
      ls[e] = pr[1];
    }
  }
  __syncthreads();
  if (threadIdx.x < HPW && q0 + (int)threadIdx.x < G) {
    float* w = wts + threadIdx.x * ns;
    const float* l = ls + threadIdx.x * ns;
    float M = -INFINITY;
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, w[sp]);
    float L = 0.f;
    for (int sp = 0; sp < ns; ++sp) {
      const float f = w[sp] == -INFINITY ? 0.f : fast_exp2(w[sp] - M);
      w[sp] = f;
      L += l[sp] * f;
    }
    inv_l[threadIdx.x] = 1.0f / L;
  }
  __syncthreads();
  const int hq = threadIdx.x / D, d = threadIdx.x % D;
  const int qr = q0 + hq;
  if (qr >= G) return;
  const float* col = part + qr * (D + 2) + 2 + d;
  const float* w = wts + hq * ns;
  float O = 0.f;
  int sp = 0;
  for (; sp + 16 <= ns; sp += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = col[(sp + u) * stride];
#pragma unroll
    for (int u = 0; u < 16; ++u) O += v[u] * w[sp + u];
  }
  for (; sp < ns; ++sp) O += col[sp * stride] * w[sp];
  ((T*)a.o)[((int64_t)b * a.H + g * G + qr) * D + d] = from_f32<T>(O * inv_l[hq]);
}

// Workgroups of decode_attend_bf16_kernel<D> resident on the current device at
// once (cached per device).
template <int D>
static int persistent_grid() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int g = cache[dev].load(std::memory_order_relaxed);
  if (g == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, (const void*)decode_attend_bf16_kernel<D>, 256, 0) != hipSuccess)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    g = (per_cu < 1 ? 1 : per_cu) * (cus < 1 ? 1 : cus);
    cache[dev].store(g, std::memory_order_relaxed);
  }
  return g;
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
  a.summ_w = summ;
  a.w_s = w_s;
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
  const bool bf16 = s.dtype == DASH_BF16;
  const unsigned nbg = (unsigned)(s.B * s.Hkv);

  if (L.ncand_max > 0) {
    dim3 g1((unsigned)((L.ncand_max + 63) / 64 + 1), nbg);
#define DASH_DS(T, D) hipLaunchKernelGGL((decode_scores_kernel<T, D>), g1, dim3(64), 0, st, a)
    if (bf16) { if (s.d == 64) DASH_DS(__bf16, 64); else DASH_DS(__bf16, 128); }
    else { if (s.d == 64) DASH_DS(float, 64); else DASH_DS(float, 128); }
#undef DASH_DS
  }
  const size_t lds = sizeof(float) * s.G * L.nb;
  {
    // rows of up to 64 * VPL candidates stay in registers
    const int64_t nc = L.ncand_max;
    const int vpl = nc <= 256 ? 4 : nc <= 512 ? 8 : nc <= 1024 ? 16 : nc <= 2048 ? 32 : 0;
    const int mode = entmax_mode(s.alpha);
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
    if (s.d == 64)
      hipLaunchKernelGGL(decode_attend_bf16_kernel<64>,
                         dim3((unsigned)min64(items_max, persistent_grid<64>())), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(decode_attend_bf16_kernel<128>,
                         dim3((unsigned)min64(items_max, persistent_grid<128>())), dim3(256), 0, st, a);
  } else {
    if (s.d == 64) hipLaunchKernelGGL(decode_attend_f32_kernel<64>, g3, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(decode_attend_f32_kernel<128>, g3, dim3(256), 0, st, a);
  }
  const int hpw = kCombineThreads / s.d;
  dim3 g4((unsigned)((s.G + hpw - 1) / hpw), nbg);
  const size_t lds4 = sizeof(float) * (2 * L.n_split + 1) * hpw;
#define DASH_DC(T, D) \
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), g4, dim3(kCombineThreads), lds4, st, a)
  if (bf16) { if (s.d == 64) DASH_DC(__bf16, 64); else DASH_DC(__bf16, 128); }
  else { if (s.d == 64) DASH_DC(float, 64); else DASH_DC(float, 128); }
#undef DASH_DC
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // with candidates the score kernel wrote the completed block's summary
  if (L.ncand_max > 0) return hipSuccess;
  return launch_summarize_completed(s, kc, max_len, cache_len, w_s, summ, summ_blocks, st);
}

}  // namespace dash
