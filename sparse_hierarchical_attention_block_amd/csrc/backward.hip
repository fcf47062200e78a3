// backward.hip -- gradients of the causal DashAttention prefill (the pages'
// point that alpha-entmax keeps the hierarchy differentiable, so gradients
// reach the chunk summaries through the routing: DashAttention explainer,
// Technical summary and Contributions).
//
// Given the forward inputs and output, its routing result and dO, the
// kernels below produce dq, dk, dv and dW_s (float32) for mean-pooled
// summaries:
//   rows    per (query tile, head): log-sum-exp and delta = dO.o by a first
//           pass over the tile's chunks, then dl_t = P_t (dO.v_t - delta),
//           dq = sum dl_t k_t / sqrt(d), and the bias gradient of every
//           listed block, sigma * sum_{t in block} dl_t, into the head's own
//           slot dlogp[tile, head, list position, row]
//   route   per (query tile, KV head), over the tile's listed blocks only
//           (every other candidate has p = 0 for every head of the group, so
//           no entmax gradient): dpbar = (sum over the heads' slots) / pbar,
//           dp_h = dpbar / G, the entmax Jacobian with
//           u = (x - tau)_+^((2-alpha)/(alpha-1)):
//           dzbar = gamma (u dp - u (u.dp) / sum u); dq += dzbar . s / sqrt(d)
//           and the tile's share of the summaries' gradient, the sum over its
//           rows and heads of dzbar_j q / sqrt(d), into its own partial rows
//   dsum    ds_j += the partial rows of the tiles that list block j, in tile
//           order
//   keys    per 64-key chunk of a (sequence, KV head): every later tile that
//           attends the chunk (branch or list), every head and row of it:
//           dk_t = sum dl_t q / sqrt(d), dv_t = sum P_t dO
//   means   dk of block j += (ds_j W_s^T) / bs; block means m_j
//   w_s     dW_s = sum_j m_j^T ds_j, in slices summed in a fixed order
// The per-tile arrays (dlogp, u, partial summary rows) hold one slab of
// query tiles at a time; rows, route and dsum run slab after slab, so the
// workspace stays bounded for long sequences.  No floating-point atomics:
// every output element is written by one thread, every sum in a fixed order.
// bf16 inputs: the rows and keys products run on MFMA (bf16 operands, float32
// accumulation).  float32 inputs keep plain float32 FMAs, a row or key spread
// over 4 lanes of D/4 columns each.  The routing gradient is float32 FMAs
// for both.
#include "dash_internal.hpp"
#include "device_common.hpp"

namespace dash {

constexpr int kBwdTile = DASH_QUERY_TILE;   // 64 query rows per tile
constexpr int kBwdChunk = 64;               // keys per chunk

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* w_s;
  const float* summ;
  int64_t summ_blocks;
  const float* tau;         // [B, H, n]
  const int32_t* sel_count; // [B, Hkv, n_qt]
  const int32_t* sel_idx;   // [B, Hkv, n_qt, nb]
  const float* sel_logp;    // [B, Hkv, n_qt, nb, 64]
  float* dq;                // [B, H, n, D]
  float* dk;                // [B, Hkv, n, D]
  float* dv;
  float* dw_s;              // [D, D]
  float* lse2;              // [B, H, n] log2-sum-exp2 of the scaled logits
  float* delta;             // [B, H, n] dO . o
  // per slab of query tiles (slot st = qt - slab_q0 < slab), by list position e
  float* dlogp;             // [B, Hkv, slab, G, nb, 64] each head's bias gradient
  float* ucoarse;           // [B, Hkv, slab, G, nb, 64] entmax u of the coarse scores
  float* dspart;            // [B, Hkv, slab, nb, D] each tile's share of ds
  float* ds;                // [B, Hkv, nb, D]
  float* mean;              // [B, Hkv, nb, D]
  float* dm;                // [B, Hkv, nb, D] (ds_j W_s^T) / bs per complete block, else 0
  float* wspart;            // [kWsSplit, D, D] slices of dW_s
  int64_t n, n_qt, nb;
  int64_t slab, slab_q0, slab_nq;   // slab capacity; this slab's first tile and size
  int B, H, Hkv, G, bs, window;
  float scale_log2;         // log2(e) / sqrt(d)
  float rs;                 // 1 / sqrt(d)
  float xscale;             // (alpha - 1) gamma / sqrt(d)
  float gamma, sigma, ue;   // ue = (2 - alpha) / (alpha - 1)
};

template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  return to_f32(((const T*)p)[i]);
}

// sum over the 4 lanes of a row (lanes 4r .. 4r+3)
__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

// The tile's walk: branch chunks first (bias 0; the last one is the diagonal
// chunk), then the chunks of the listed blocks.
struct BwdWalk {
  int64_t own_c0;   // first branch chunk
  int n_own, count, cpb;
};
__device__ __forceinline__ BwdWalk bwd_walk(const BwdArgs& a, int64_t tile, int64_t qt) {
  BwdWalk w;
  w.cpb = a.bs / kBwdChunk;
  const int64_t own = (qt * kBwdTile) / a.bs;
  const int64_t b0 = own - (a.window - 1) > 0 ? own - (a.window - 1) : 0;
  w.own_c0 = b0 * w.cpb;
  w.n_own = (int)(qt - w.own_c0 + 1);
  w.count = a.sel_count[tile];
  return w;
}

// Does tile qt of pair bg attend block blk?  0: no, 1: through its
// near-diagonal branch, 2: through its list (binary search in the ascending
// list).
__device__ __forceinline__ int tile_attends(const BwdArgs& a, int64_t bg, int64_t qt,
                                            int64_t blk) {
  const int64_t tile = bg * a.n_qt + qt;
  const int64_t own = (qt * kBwdTile) / a.bs;
  const int64_t b0 = own - (a.window - 1) > 0 ? own - (a.window - 1) : 0;
  if (blk >= b0 && blk <= own) return 1;
  const int cnt = a.sel_count[tile];
  const int32_t* lst = a.sel_idx + tile * a.nb;
  int lo = 0, hi = cnt;
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    if (lst[mid] < blk) lo = mid + 1; else hi = mid;
  }
  return lo < cnt && lst[lo] == blk ? 2 : 0;
}
// The tiles that attend a chunk are found 256 at a time, one per thread (the
// binary searches run side by side), into an LDS flag array.
constexpr int kFlagTiles = 256;

// ---- rows: lse, delta, dq (fine part), bias gradients ---------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_rows_kernel(BwdArgs a) {
  constexpr int S = D / 4;   // columns per lane
  // K and V of the chunk, [64][D] each, in the input type (bf16 halves the
  // LDS and doubles the workgroups per CU)
  extern __shared__ __attribute__((aligned(16))) char lds_rows[];
  T(*Kc)[D] = (T(*)[D])lds_rows;
  T(*Vc)[D] = (T(*)[D])(lds_rows + sizeof(T) * kBwdChunk * D);
  const int64_t qt = a.slab_q0 + blockIdx.x % a.slab_nq;
  const int64_t bh = blockIdx.x / a.slab_nq;   // b * H + h
  const int b = (int)(bh / a.H), h = (int)(bh % a.H), g = h / a.G;
  const int64_t bg = (int64_t)b * a.Hkv + g;
  const int64_t tile = bg * a.n_qt + qt;
  const int row = threadIdx.x / 4, sl = threadIdx.x % 4;
  const int64_t qpos = qt * kBwdTile + row;
  const bool valid = qpos < a.n;
  const int64_t rbase = (bh * a.n + (valid ? qpos : 0)) * D + sl * S;
  float qv[S], dov[S], acc[S];
  float dlt = 0.f;
#pragma unroll
  for (int c = 0; c < S; ++c) {
    qv[c] = valid ? ld<T>(a.q, rbase + c) : 0.f;
    dov[c] = valid ? ld<T>(a.dO, rbase + c) : 0.f;
    dlt = fmaf(dov[c], valid ? ld<T>(a.o, rbase + c) : 0.f, dlt);
    acc[c] = 0.f;
  }
  dlt = quad_sum(dlt);
  const BwdWalk w = bwd_walk(a, tile, qt);
  const int n_chunks = w.n_own + w.count * w.cpb;
  const T* kb = (const T*)a.k + bg * a.n * D;
  const T* vb = (const T*)a.v + bg * a.n * D;

  // chunk c -> first key, block (-1 for branch chunks)
  auto chunk = [&](int c, int64_t& key0, int64_t& blk) {
    if (c < w.n_own) {
      key0 = (w.own_c0 + c) * kBwdChunk;
      blk = -1;
    } else {
      const int e = (c - w.n_own) / w.cpb;
      blk = a.sel_idx[tile * a.nb + e];
      key0 = blk * a.bs + ((c - w.n_own) % w.cpb) * kBwdChunk;
    }
  };
  auto stage = [&](int64_t key0, bool with_v) {
    for (int e = threadIdx.x; e < kBwdChunk * D; e += 256) {
      const int kk = e / D, c = e % D;
      const bool in = key0 + kk < a.n;
      Kc[kk][c] = in ? kb[(key0 + kk) * D + c] : (T)0.f;
      if (with_v) Vc[kk][c] = in ? vb[(key0 + kk) * D + c] : (T)0.f;
    }
  };
  // scaled logit (log2 units) of key kk of the chunk, -inf when masked
  auto logit = [&](int kk, int64_t key0, int64_t blk, float bias2) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < S; ++c) s = fmaf(qv[c], to_f32(Kc[kk][sl * S + c]), s);
    s = quad_sum(s);
    const int64_t key = key0 + kk;
    if (blk < 0 && key > qpos) return -INFINITY;
    return fmaf(s, a.scale_log2, bias2);
  };

  // pass 1: log-sum-exp
  float m = -INFINITY, l = 0.f;
  for (int c = 0; c < n_chunks; ++c) {
    int64_t key0, blk;
    chunk(c, key0, blk);
    const float bias2 =
        blk < 0 ? 0.f : a.sel_logp[(tile * a.nb + blk) * kBwdTile + row] * kLog2e;
    __syncthreads();
    stage(key0, false);
    __syncthreads();
    if (bias2 == -INFINITY) continue;
    for (int kk = 0; kk < kBwdChunk; ++kk) {
      const float s = logit(kk, key0, blk, bias2);
      if (s == -INFINITY) continue;
      const float mn = fmaxf(m, s);
      l = l * exp2f(m - mn) + exp2f(s - mn);
      m = mn;
    }
  }
  const float lse = m + log2f(l);
  if (valid && sl == 0) {
    a.lse2[bh * a.n + qpos] = lse;
    a.delta[bh * a.n + qpos] = dlt;
  }

  // pass 2: dl, dq, bias gradients
  float bacc = 0.f;
  for (int c = 0; c < n_chunks; ++c) {
    int64_t key0, blk;
    chunk(c, key0, blk);
    const float bias2 =
        blk < 0 ? 0.f : a.sel_logp[(tile * a.nb + blk) * kBwdTile + row] * kLog2e;
    __syncthreads();
    stage(key0, true);
    __syncthreads();
    if (bias2 != -INFINITY) {
      for (int kk = 0; kk < kBwdChunk; ++kk) {
        const float s = logit(kk, key0, blk, bias2);
        const float p = s == -INFINITY ? 0.f : exp2f(s - lse);
        float dp = 0.f;
#pragma unroll
        for (int cc = 0; cc < S; ++cc) dp = fmaf(dov[cc], to_f32(Vc[kk][sl * S + cc]), dp);
        dp = quad_sum(dp);
        const float dl = p * (dp - dlt);
        if (blk >= 0) bacc += dl;
#pragma unroll
        for (int cc = 0; cc < S; ++cc)
          acc[cc] = fmaf(dl * a.rs, to_f32(Kc[kk][sl * S + cc]), acc[cc]);
      }
    }
    // end of a listed block: its bias gradient, into this head's slot
    if (blk >= 0 && (c - w.n_own) % w.cpb == w.cpb - 1) {
      const int e = (c - w.n_own) / w.cpb;
      if (valid && sl == 0)
        a.dlogp[(((bg * a.slab + (qt - a.slab_q0)) * a.G + h % a.G) * a.nb + e) * kBwdTile +
                row] = a.sigma * bacc;
      bacc = 0.f;
    }
  }
  if (valid) {
#pragma unroll
    for (int c = 0; c < S; ++c) a.dq[rbase + c] = acc[c];
  }
}

// ---- rows, bf16 with MFMA: the forward's layout, three products per chunk -------------------
// One workgroup per (sequence, KV head, query tile), 2 G waves of 32 queries
// of one head each, so a staged K/V chunk serves the whole group.  Per chunk
// and wave (keys are the MFMA rows, as in the forward kernel):
//   S^T  (64 keys x 32 queries) = K Q^T          P^T = exp2(S^T scale + bias - lse)
//   dP^T (64 keys x 32 queries) = V dO^T          dS^T = P^T (dP^T - delta)
//   dQ^T (d x 32 queries)      += K^T dS^T        (dS^T rounded to bf16 as the B operand)
// K and V are staged row-major, and K once more transposed with the keys of
// each 16 permuted as the accumulator order of dS^T needs (key 16m+8a+4b+r
// at column 16m+8b+4a+r).  A first pass over the chunks (S^T only) gives lse.
template <int D, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT >= 256 ? 2 : 1)))
void bwd_rows_mfma_kernel(BwdArgs a) {
  constexpr int KP = D + 8;            // row pitch of K and V (bf16)
  constexpr int VP = kBwdChunk + 8;    // row pitch of K^T
  __shared__ __attribute__((aligned(16))) __bf16 Ks[kBwdChunk * KP];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[kBwdChunk * KP];
  __shared__ __attribute__((aligned(16))) __bf16 Kt[D * VP];
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int l32 = lane % 32, lh = lane / 32;
  const int64_t nbg = (int64_t)a.B * a.Hkv;
  const int wpt = (2 * a.G + NT / kWave - 1) / (NT / kWave);   // workgroups per tile
  const int64_t rank = blockIdx.x / wpt;
  const int gw = (int)(blockIdx.x % wpt) * (NT / kWave) + wave;   // wave within the tile
  const int64_t qt = a.slab_q0 + a.slab_nq - 1 - rank / nbg;   // heaviest tiles first
  const int64_t bg = rank % nbg;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t tile = bg * a.n_qt + qt;
  const int h = g * a.G + gw / 2;
  const int qloc = 32 * (gw % 2) + l32;
  const int64_t qpos = qt * kBwdTile + qloc;
  const bool valid = qpos < a.n;
  const int64_t bh = (int64_t)b * a.H + h;
  const __bf16* qrow = (const __bf16*)a.q + (bh * a.n + (valid ? qpos : 0)) * D;
  const __bf16* dorow = (const __bf16*)a.dO + (bh * a.n + (valid ? qpos : 0)) * D;
  const __bf16* orow = (const __bf16*)a.o + (bh * a.n + (valid ? qpos : 0)) * D;
  // Q^T and dO^T operand fragments: column = query l32, k = d in [16 s + 8 lh, +8)
  bf16x8 qf[D / 16], df[D / 16];
  float dlt = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < D / 16; ++s2) {
    u32x4 wq = {0u, 0u, 0u, 0u}, wd = {0u, 0u, 0u, 0u}, wo = {0u, 0u, 0u, 0u};
    if (valid) {
      wq = *(const u32x4*)(qrow + 16 * s2 + 8 * lh);
      wd = *(const u32x4*)(dorow + 16 * s2 + 8 * lh);
      wo = *(const u32x4*)(orow + 16 * s2 + 8 * lh);
    }
    qf[s2] = as_bf16x8(wq);
    df[s2] = as_bf16x8(wd);
    const uint32_t dw[4] = {wd.x, wd.y, wd.z, wd.w}, ow[4] = {wo.x, wo.y, wo.z, wo.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dlt += bf16_lo(dw[e]) * bf16_lo(ow[e]) + bf16_hi(dw[e]) * bf16_hi(ow[e]);
  }
  dlt = xor_reduce<32>(dlt, DppAdd{});   // the two halves of d

  const BwdWalk w = bwd_walk(a, tile, qt);
  const int n_chunks = w.n_own + w.count * w.cpb;
  const uint32_t seq_bytes = (uint32_t)(a.n * (D * 2));
  const buf_rsrc rk = make_rsrc((const __bf16*)a.k + bg * a.n * D, seq_bytes);
  const buf_rsrc rv = make_rsrc((const __bf16*)a.v + bg * a.n * D, seq_bytes);
  auto chunk = [&](int c, int64_t& key0, int64_t& blk) {
    if (c < w.n_own) {
      key0 = (w.own_c0 + c) * kBwdChunk;
      blk = -1;
    } else {
      const int e = (c - w.n_own) / w.cpb;
      blk = a.sel_idx[tile * a.nb + e];
      key0 = blk * a.bs + ((c - w.n_own) % w.cpb) * kBwdChunk;
    }
  };
  auto stage = [&](int64_t key0, bool full) {
    for (int e = threadIdx.x; e < kBwdChunk * (D / 8); e += NT) {
      const int key = e / (D / 8), seg = e % (D / 8);
      const uint32_t off = (uint32_t)((key0 + key) * (D * 2) + seg * 16);
      *(u32x4*)(Ks + key * KP + seg * 8) = buf_load16(rk, off);
      if (full) *(u32x4*)(Vs + key * KP + seg * 8) = buf_load16(rv, off);
    }
    if (!full) return;
    // K^T in 4 x 4 blocks (4 keys x 4 d): four 8-byte loads, register
    // transposes, four 8-byte stores; keys 16 m + 8 a + 4 b + [0, 4) go to
    // columns 16 m + 8 b + 4 a + [0, 4), and 16-byte chunk c of row r sits at
    // c ^ ((r >> 4) & 3) (rows 4 db + [0, 4): c ^ (db >> 2)), so the 16 lanes
    // of a store (rows 4 apart) and of a fragment read cover all banks
    for (int e = threadIdx.x; e < (kBwdChunk / 4) * (D / 4); e += NT) {
      const int db = e % (D / 4), kb4 = e / (D / 4);
      u32x2 in[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        in[rr] = buf_load8(rk, (uint32_t)((key0 + 4 * kb4 + rr) * (D * 2) + db * 8));
      const int col = (16 * (kb4 / 4) + 8 * (kb4 % 2) + 4 * ((kb4 / 2) % 2)) ^ (8 * ((db >> 2) & 3));
      *(u32x2*)(Kt + (4 * db + 0) * VP + col) = (u32x2){pack_lo(in[0].x, in[1].x),
                                                        pack_lo(in[2].x, in[3].x)};
      *(u32x2*)(Kt + (4 * db + 1) * VP + col) = (u32x2){pack_hi(in[0].x, in[1].x),
                                                        pack_hi(in[2].x, in[3].x)};
      *(u32x2*)(Kt + (4 * db + 2) * VP + col) = (u32x2){pack_lo(in[0].y, in[1].y),
                                                        pack_lo(in[2].y, in[3].y)};
      *(u32x2*)(Kt + (4 * db + 3) * VP + col) = (u32x2){pack_hi(in[0].y, in[1].y),
                                                        pack_hi(in[2].y, in[3].y)};
    }
  };
  // acc[kt] += X[32 kt + l32, :] (row-major in LDS, pitch KP) times the
  // register fragments fr, the two chains interleaved and each A fragment
  // read one k-step ahead of its MFMA
  auto two_chains = [&](const __bf16* X, const bf16x8 (&fr)[D / 16], f32x16 (&acc)[2]) {
    const __bf16* x0 = X + l32 * KP + 8 * lh;
    const __bf16* x1 = x0 + 32 * KP;
    u32x4 a0 = *(const u32x4*)x0, a1 = *(const u32x4*)x1;
#pragma unroll
    for (int s2 = 0; s2 < D / 16; ++s2) {
      u32x4 n0 = a0, n1 = a1;
      if (s2 + 1 < D / 16) {
        n0 = *(const u32x4*)(x0 + 16 * (s2 + 1));
        n1 = *(const u32x4*)(x1 + 16 * (s2 + 1));
      }
      acc[0] = mfma32(as_bf16x8(a0), fr[s2], acc[0]);
      acc[1] = mfma32(as_bf16x8(a1), fr[s2], acc[1]);
      a0 = n0;
      a1 = n1;
    }
  };
  // S^T of the staged chunk, masked, in log2 units with the bias: st[kt][i]
  // is query l32, key 32 kt + 8 (i / 4) + 4 lh + i % 4
  auto scores = [&](int c, float bias2, f32x16 (&st)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st[kt][i] = 0.f;
    two_chains(Ks, qf, st);
    const bool diag = c == w.n_own - 1;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * kt + 8 * (i / 4) + 4 * lh + (i % 4);
        st[kt][i] = (diag && key > qloc) ? -INFINITY : fmaf(st[kt][i], a.scale_log2, bias2);
      }
  };

  // pass 1: log2-sum-exp2 per query.  It stages K only, and the next
  // chunk's K is loaded into registers while the current one is computed.
  constexpr int NPK = kBwdChunk * (D / 8) / NT;   // 16-byte pieces of K per thread
  u32x4 kpre[NPK];
  auto load_k = [&](int64_t key0) {
#pragma unroll
    for (int i = 0; i < NPK; ++i) {
      const int e = threadIdx.x + NT * i, key = e / (D / 8), seg = e % (D / 8);
      kpre[i] = buf_load16(rk, (uint32_t)((key0 + key) * (D * 2) + seg * 16));
    }
  };
  float m = -INFINITY, l = 0.f;
  int64_t key0n = 0, blkn = -1;
  if (n_chunks > 0) {
    chunk(0, key0n, blkn);
    load_k(key0n);
  }
  for (int c = 0; c < n_chunks; ++c) {
    const int64_t blk = blkn;
    const float bias2 =
        blk < 0 ? 0.f : a.sel_logp[(tile * a.nb + blk) * kBwdTile + qloc] * kLog2e;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NPK; ++i) {
      const int e = threadIdx.x + NT * i, key = e / (D / 8), seg = e % (D / 8);
      *(u32x4*)(Ks + key * KP + seg * 8) = kpre[i];
    }
    __syncthreads();
    if (c + 1 < n_chunks) {
      chunk(c + 1, key0n, blkn);
      load_k(key0n);
    }
    f32x16 st[2];
    scores(c, bias2, st);
    float cm = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) cm = fmaxf(cm, st[kt][i]);
    cm = xor_reduce<32>(cm, DppMax{});
    if (cm == -INFINITY) continue;
    const float mn = fmaxf(m, cm);
    float cs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) cs += fast_exp2(st[kt][i] - mn);
    cs = xor_reduce<32>(cs, DppAdd{});
    l = l * fast_exp2(m - mn) + cs;
    m = mn;
  }
  const float lse = m + log2f(l);
  if (valid && lh == 0) {
    a.lse2[bh * a.n + qpos] = lse;
    a.delta[bh * a.n + qpos] = dlt;
  }

  // pass 2
  f32x16 dqa[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqa[dt][i] = 0.f;
  float bacc = 0.f;
  for (int c = 0; c < n_chunks; ++c) {
    int64_t key0, blk;
    chunk(c, key0, blk);
    const float bias2 =
        blk < 0 ? 0.f : a.sel_logp[(tile * a.nb + blk) * kBwdTile + qloc] * kLog2e;
    __syncthreads();
    stage(key0, true);
    __syncthreads();
    f32x16 st[2], dp[2];
    scores(c, bias2, st);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dp[kt][i] = 0.f;
    two_chains(Vs, df, dp);
    // dS^T, its column sums (the bias gradient), and the bf16 B operands
    float csum = 0.f;
    bf16x8 dsf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kt = ks / 2, i0 = 8 * (ks % 2);
      float dv8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = fast_exp2(st[kt][i0 + e] - lse);   // 0 where masked
        dv8[e] = pv * (dp[kt][i0 + e] - dlt);
        csum += dv8[e];
      }
      const u32x4 pw = {pack_bf16(dv8[0], dv8[1]), pack_bf16(dv8[2], dv8[3]),
                        pack_bf16(dv8[4], dv8[5]), pack_bf16(dv8[6], dv8[7])};
      dsf[ks] = as_bf16x8(pw);
    }
    csum = xor_reduce<32>(csum, DppAdd{});
    if (blk >= 0) bacc += csum;
    {   // dQ^T += K^T dS^T, each A fragment read one MFMA ahead; chunk
        // 2 ks + lh of row 32 dt + l32 sits at 2 (ks ^ (dt & 1)) + (lh ^ (l32 >> 4))
      constexpr int NQ = 4 * (D / 32);
      const __bf16* ktl = Kt + l32 * VP + 8 * (lh ^ (l32 >> 4));
      auto kto = [&](int ks, int dt) { return (32 * dt) * VP + 16 * (ks ^ (dt & 1)); };
      u32x4 ka = *(const u32x4*)(ktl + kto(0, 0));
#pragma unroll
      for (int x = 0; x < NQ; ++x) {
        const int ks = x / (D / 32), dt = x % (D / 32);
        u32x4 kn = ka;
        if (x + 1 < NQ) {
          const int ks1 = (x + 1) / (D / 32), dt1 = (x + 1) % (D / 32);
          kn = *(const u32x4*)(ktl + kto(ks1, dt1));
        }
        dqa[dt] = mfma32(as_bf16x8(ka), dsf[ks], dqa[dt]);
        ka = kn;
      }
    }
    if (blk >= 0 && (c - w.n_own) % w.cpb == w.cpb - 1) {
      const int e = (c - w.n_own) / w.cpb;
      if (valid && lh == 0)
        a.dlogp[(((bg * a.slab + (qt - a.slab_q0)) * a.G + gw / 2) * a.nb + e) * kBwdTile +
                qloc] = a.sigma * bacc;
      bacc = 0.f;
    }
  }
  // dqa[dt][i] = dQ[query l32][32 dt + 8 (i / 4) + 4 lh + i % 4]
  if (valid) {
    float* dqr = a.dq + (bh * a.n + qpos) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dqr[32 * dt + 8 * (i / 4) + 4 * lh + (i % 4)] = dqa[dt][i] * a.rs;
  }
}

// ---- keys: dk (fine part), dv --------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_keys_kernel(BwdArgs a) {
  constexpr int S = D / 4;
  // q and dO rows of a tile, [64][D] each in the input type, then row data
  extern __shared__ __attribute__((aligned(16))) char lds_keys[];
  T(*Qs)[D] = (T(*)[D])lds_keys;
  T(*Os)[D] = (T(*)[D])(lds_keys + sizeof(T) * kBwdTile * D);
  float* rowl = (float*)(lds_keys + sizeof(T) * 2 * kBwdTile * D);
  float* rowd = rowl + kBwdTile;
  float* rowb = rowd + kBwdTile;
  const int64_t nbg = (int64_t)a.B * a.Hkv;
  const int64_t ch = blockIdx.x / nbg;   // early chunks, attended by the most tiles, first
  const int64_t bg = blockIdx.x % nbg;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int key = threadIdx.x / 4, sl = threadIdx.x % 4;
  const int64_t kpos = ch * kBwdChunk + key;
  const bool valid = kpos < a.n;
  const int64_t kbase = (bg * a.n + (valid ? kpos : 0)) * D + sl * S;
  float kv[S], vv[S], dkv[S], dvv[S];
#pragma unroll
  for (int c = 0; c < S; ++c) {
    kv[c] = valid ? ld<T>(a.k, kbase + c) : 0.f;
    vv[c] = valid ? ld<T>(a.v, kbase + c) : 0.f;
    dkv[c] = 0.f;
    dvv[c] = 0.f;
  }
  const int64_t blk = (ch * kBwdChunk) / a.bs;
  __shared__ int8_t flags[kFlagTiles];
  for (int64_t q0 = ch; q0 < a.n_qt; q0 += kFlagTiles) {
  __syncthreads();
  if (threadIdx.x < kFlagTiles)
    flags[threadIdx.x] =
        q0 + threadIdx.x < a.n_qt ? (int8_t)tile_attends(a, bg, q0 + threadIdx.x, blk) : 0;
  __syncthreads();
  const int nq = (int)min((int64_t)kFlagTiles, a.n_qt - q0);
  for (int tq = 0; tq < nq; ++tq) {
    if (!flags[tq]) continue;
    const int64_t qt = q0 + tq;
    const int64_t tile = bg * a.n_qt + qt;
    const bool branch = flags[tq] == 1;
    for (int hh = 0; hh < a.G; ++hh) {
      const int h = g * a.G + hh;
      const int64_t bh = (int64_t)b * a.H + h;
      __syncthreads();
      for (int e = threadIdx.x; e < kBwdTile * D; e += 256) {
        const int r = e / D, c = e % D;
        const int64_t pos = qt * kBwdTile + r;
        const bool in = pos < a.n;
        Qs[r][c] = in ? ((const T*)a.q)[(bh * a.n + pos) * D + c] : (T)0.f;
        Os[r][c] = in ? ((const T*)a.dO)[(bh * a.n + pos) * D + c] : (T)0.f;
      }
      for (int r = threadIdx.x; r < kBwdTile; r += 256) {
        const int64_t pos = qt * kBwdTile + r;
        const bool in = pos < a.n;
        rowl[r] = in ? a.lse2[bh * a.n + pos] : 0.f;
        rowd[r] = in ? a.delta[bh * a.n + pos] : 0.f;
        rowb[r] = !in ? -INFINITY
                      : (branch ? 0.f : a.sel_logp[(tile * a.nb + blk) * kBwdTile + r] * kLog2e);
      }
      __syncthreads();
      for (int r = 0; r < kBwdTile; ++r) {
        const int64_t pos = qt * kBwdTile + r;
        if (rowb[r] == -INFINITY) continue;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int c = 0; c < S; ++c) {
          s = fmaf(to_f32(Qs[r][sl * S + c]), kv[c], s);
          dp = fmaf(to_f32(Os[r][sl * S + c]), vv[c], dp);
        }
        s = quad_sum(s);
        dp = quad_sum(dp);
        float p = exp2f(fmaf(s, a.scale_log2, rowb[r]) - rowl[r]);
        if (!valid || (branch && kpos > pos)) p = 0.f;
        const float dl = p * (dp - rowd[r]);
#pragma unroll
        for (int c = 0; c < S; ++c) {
          dkv[c] = fmaf(dl * a.rs, to_f32(Qs[r][sl * S + c]), dkv[c]);
          dvv[c] = fmaf(p, to_f32(Os[r][sl * S + c]), dvv[c]);
        }
      }
    }
  }
  }
  if (valid) {
    // plus the summaries' share of the key's block (zero for an incomplete block)
    const float* dmr = a.dm + (bg * a.nb + kpos / a.bs) * D + sl * S;
#pragma unroll
    for (int c = 0; c < S; ++c) {
      a.dk[kbase + c] = dkv[c] + dmr[c];
      a.dv[kbase + c] = dvv[c];
    }
  }
}

// ---- keys, bf16 with MFMA ------------------------------------------------------------------
// One workgroup of 4 waves per 64-key chunk of a (sequence, KV head); wave w
// owns keys 32 (w / 2) .. +32 and half (w % 2) of the d columns of dK and dV.
// For every (tile, head) that attends the chunk, q and dO of the tile are
// staged row-major and transposed (queries of each 16 permuted as the
// accumulator order of P and dS needs), then per 32-query half:
//   S  (32 queries x 32 keys) = Q K^T,  dP = dO V^T      (queries are MFMA rows)
//   P = exp2(S scale + bias - lse),  dS = P (dP - delta)
//   dV^T (d x keys) += dO^T P,  dK^T += Q^T dS            (P, dS as bf16 B operands)
// The wave's K and V fragments stay in registers for the whole walk.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_keys_mfma_kernel(BwdArgs a) {
  constexpr int RP = D + 8;            // row pitch of the staged q / dO rows
  constexpr int TP = kBwdTile + 8;     // row pitch of the transposed ones
  constexpr int NDT = D / 64;          // d tiles of 32 per wave
  extern __shared__ __attribute__((aligned(16))) char lds_km[];
  __bf16* Qr = (__bf16*)lds_km;
  __bf16* Or = Qr + kBwdTile * RP;
  __bf16* Qt = Or + kBwdTile * RP;
  __bf16* Ot = Qt + D * TP;
  float* rowl = (float*)(Ot + D * TP);
  float* rowd = rowl + kBwdTile;
  float* rowb = rowd + kBwdTile;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int l32 = lane % 32, lh = lane / 32;
  const int kt = wave / 2, dh = wave % 2;
  const int64_t nbg = (int64_t)a.B * a.Hkv;
  const int64_t ch = blockIdx.x / nbg;   // early chunks, attended by the most tiles, first
  const int64_t bg = blockIdx.x % nbg;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t kpos = ch * kBwdChunk + 32 * kt + l32;   // this lane's key
  const bool kvalid = kpos < a.n;
  // K^T / V^T operand fragments of the lane's key: k = d in [16 s + 8 lh, +8)
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const __bf16* kr = (const __bf16*)a.k + (bg * a.n + (kvalid ? kpos : 0)) * D;
    const __bf16* vr = (const __bf16*)a.v + (bg * a.n + (kvalid ? kpos : 0)) * D;
#pragma unroll
    for (int s2 = 0; s2 < D / 16; ++s2) {
      u32x4 wk = {0u, 0u, 0u, 0u}, wv = {0u, 0u, 0u, 0u};
      if (kvalid) {
        wk = *(const u32x4*)(kr + 16 * s2 + 8 * lh);
        wv = *(const u32x4*)(vr + 16 * s2 + 8 * lh);
      }
      kf[s2] = as_bf16x8(wk);
      vf[s2] = as_bf16x8(wv);
    }
  }
  f32x16 dka[NDT], dva[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) dka[t][i] = dva[t][i] = 0.f;

  const int64_t blk = (ch * kBwdChunk) / a.bs;
  // Staging: q and dO of a (tile, head) in blocks of 4 rows x 8 d, NBLK per
  // thread, held in registers so that the next item's loads are in flight
  // while the current one is computed.  Block rows 4 rb + [0, 4) land in 4
  // adjacent columns of the transposed copies (rb runs fastest over the
  // lanes, so those 8-byte stores hit distinct banks).
  constexpr int NBLK = D / 64;
  u32x4 pre[NBLK][4];
  float pre_l = 0.f, pre_d = 0.f, pre_b = 0.f;
  // q and dO of one head through buffer resources over its n rows (32-bit
  // offsets; rows past n read as zeros without a compare)
  const uint32_t head_bytes = (uint32_t)(a.n * (D * 2));
  auto prefetch = [&](int64_t qt, int hh, bool branch) {
    const int64_t bh = (int64_t)b * a.H + g * a.G + hh;
#pragma unroll
    for (int m = 0; m < NBLK; ++m) {
      const int e = threadIdx.x + 256 * m;
      // q or dO: uniform within a wave (2 D threads per matrix)
      const int which = __builtin_amdgcn_readfirstlane(e / (2 * D));
      const int e1 = e % (2 * D);
      const int rb = e1 % 16, cb = e1 / 16;
      const buf_rsrc rs = make_rsrc((const __bf16*)(which ? a.dO : a.q) + bh * a.n * D, head_bytes);
      const uint32_t base = (uint32_t)qt * (kBwdTile * D * 2) + (uint32_t)(4 * rb * (D * 2) + 16 * cb);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) pre[m][rr] = buf_load16(rs, base + (uint32_t)(rr * (D * 2)));
    }
    // loads only: any arithmetic on a loaded value here would wait for all of them
    if (threadIdx.x < kBwdTile) {
      const int r = threadIdx.x;
      const int64_t pos = qt * kBwdTile + r;
      if (pos < a.n) {
        pre_l = a.lse2[bh * a.n + pos];
        pre_d = a.delta[bh * a.n + pos];
        if (!branch) pre_b = a.sel_logp[((bg * a.n_qt + qt) * a.nb + blk) * kBwdTile + r];
      }
    }
  };
  auto stage = [&](int64_t qt, bool branch) {
#pragma unroll
    for (int m = 0; m < NBLK; ++m) {
      const int e = threadIdx.x + 256 * m;
      const int which = e / (2 * D), e1 = e % (2 * D);
      const int rb = e1 % 16, cb = e1 / 16;
      __bf16* dr = which ? Or : Qr;
      __bf16* dt = which ? Ot : Qt;
      // 16-byte chunk c of row r sits at chunk c ^ ((r >> 4) & 3), i.e.
      // cb ^ (rb >> 2) here: the 16 lanes of a store (rows 4 rb + rr) then
      // cover all banks, as do the 16 rows of a fragment read
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        *(u32x4*)(dr + (4 * rb + rr) * RP + 8 * (cb ^ (rb >> 2))) = pre[m][rr];
      // queries 16 m' + 8 a' + 4 b' + [0, 4) go to columns 16 m' + 8 b' + 4 a' + [0, 4)
      const int col = 16 * (rb / 4) + 8 * (rb % 2) + 4 * ((rb / 2) % 2);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        *(u32x2*)(dt + (8 * cb + 2 * w) * TP + col) =
            (u32x2){pack_lo(pre[m][0][w], pre[m][1][w]), pack_lo(pre[m][2][w], pre[m][3][w])};
        *(u32x2*)(dt + (8 * cb + 2 * w + 1) * TP + col) =
            (u32x2){pack_hi(pre[m][0][w], pre[m][1][w]), pack_hi(pre[m][2][w], pre[m][3][w])};
      }
    }
    if (threadIdx.x < kBwdTile) {
      const bool in = qt * kBwdTile + threadIdx.x < a.n;
      rowl[threadIdx.x] = in ? pre_l : 0.f;
      rowd[threadIdx.x] = in ? pre_d : 0.f;
      rowb[threadIdx.x] = !in ? -INFINITY : (branch ? 0.f : pre_b * kLog2e);
    }
  };
  __shared__ int8_t flags[kFlagTiles];
  for (int64_t q0 = ch; q0 < a.n_qt; q0 += kFlagTiles) {
    __syncthreads();
    if (threadIdx.x < kFlagTiles)
      flags[threadIdx.x] =
          q0 + threadIdx.x < a.n_qt ? (int8_t)tile_attends(a, bg, q0 + threadIdx.x, blk) : 0;
    __syncthreads();
    const int nq = (int)min((int64_t)kFlagTiles, a.n_qt - q0);
    int tq = 0, hh = 0;
    while (tq < nq && !flags[tq]) ++tq;
    if (tq < nq) prefetch(q0 + tq, 0, flags[tq] == 1);
    while (tq < nq) {
      const int64_t qt = q0 + tq;
      const bool branch = flags[tq] == 1;
      int ntq = tq, nhh = hh + 1;
      if (nhh == a.G) {
        nhh = 0;
        for (++ntq; ntq < nq && !flags[ntq];) ++ntq;
      }
      __syncthreads();   // the previous item is done with the staged rows
      stage(qt, branch);
      __syncthreads();
      if (ntq < nq) prefetch(q0 + ntq, nhh, flags[ntq] == 1);
      const int zero_below =
          !kvalid ? kBwdTile
                  : (branch ? (int)min((int64_t)kBwdTile,
                                       max((int64_t)0, kpos - qt * kBwdTile))
                            : 0);
#pragma unroll 1
      for (int qh = 0; qh < 2; ++qh) {
        // S and dP: queries 32 qh + row, keys of this wave's tile (lane l32)
        f32x16 sv, dpv;
#pragma unroll
        for (int i = 0; i < 16; ++i) sv[i] = dpv[i] = 0.f;
        // A fragments read one k-step ahead of their MFMAs; chunk 2 s2 + lh of
        // row 32 qh + l32 sits at 2 (s2 ^ qh) + (lh ^ (l32 >> 4)) (the swizzle
        // above), so even and odd s2 step from two bases
        const int rbase0 = (32 * qh + l32) * RP + 8 * (lh ^ (l32 >> 4));
        const int roffE = rbase0 + 16 * qh, roffO = rbase0 - 16 * qh;
        auto roff = [&](int s2) { return ((s2 & 1) ? roffO : roffE) + 16 * s2; };
        u32x4 qa = *(const u32x4*)(Qr + roff(0)), oa = *(const u32x4*)(Or + roff(0));
#pragma unroll
        for (int s2 = 0; s2 < D / 16; ++s2) {
          u32x4 qn = qa, on = oa;
          if (s2 + 1 < D / 16) {
            qn = *(const u32x4*)(Qr + roff(s2 + 1));
            on = *(const u32x4*)(Or + roff(s2 + 1));
          }
          sv = mfma32(as_bf16x8(qa), kf[s2], sv);
          dpv = mfma32(as_bf16x8(oa), vf[s2], dpv);
          qa = qn;
          oa = on;
        }
        // element i: query 32 qh + 8 (i / 4) + 4 lh + i % 4, key kpos; rows
        // below `zero_below` get p = 0 (all rows for a key past the end; in
        // the diagonal chunk the rows before the key)
        bf16x8 pf[2], dsf[2];
        const int rbase = 32 * qh + 4 * lh;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          float pv[8], dv8[8];
#pragma unroll
          for (int gq = 0; gq < 2; ++gq) {
            const int r0 = rbase + 8 * (2 * k2 + gq);
            const f32x4 lb = *(const f32x4*)(rowb + r0);
            const f32x4 ll = *(const f32x4*)(rowl + r0);
            const f32x4 ld4 = *(const f32x4*)(rowd + r0);
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const int i = 8 * k2 + 4 * gq + e4;
              float p = fast_exp2(fmaf(sv[i], a.scale_log2, lb[e4]) - ll[e4]);
              if (r0 + e4 < zero_below) p = 0.f;
              pv[4 * gq + e4] = p;
              dv8[4 * gq + e4] = p * (dpv[i] - ld4[e4]);
            }
          }
          pf[k2] = as_bf16x8((u32x4){pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]),
                                     pack_bf16(pv[4], pv[5]), pack_bf16(pv[6], pv[7])});
          dsf[k2] = as_bf16x8((u32x4){pack_bf16(dv8[0], dv8[1]), pack_bf16(dv8[2], dv8[3]),
                                      pack_bf16(dv8[4], dv8[5]), pack_bf16(dv8[6], dv8[7])});
        }
        // dV^T += dO^T P, dK^T += Q^T dS over the two 16-query k-steps
        {   // A fragments read one step ahead of their MFMAs
          auto toff = [&](int x) {
            return (32 * (NDT * dh + x % NDT) + l32) * TP + 16 * (2 * qh + x / NDT) + 8 * lh;
          };
          u32x4 oa = *(const u32x4*)(Ot + toff(0)), qa = *(const u32x4*)(Qt + toff(0));
#pragma unroll
          for (int x = 0; x < 2 * NDT; ++x) {
            const int k2 = x / NDT, t = x % NDT;
            u32x4 on = oa, qn = qa;
            if (x + 1 < 2 * NDT) {
              on = *(const u32x4*)(Ot + toff(x + 1));
              qn = *(const u32x4*)(Qt + toff(x + 1));
            }
            dva[t] = mfma32(as_bf16x8(oa), pf[k2], dva[t]);
            dka[t] = mfma32(as_bf16x8(qa), dsf[k2], dka[t]);
            oa = on;
            qa = qn;
          }
        }
      }
      tq = ntq;
      hh = nhh;
    }
  }
  // dka[t][i] = dK^T[d = 32 dt + 8 (i / 4) + 4 lh + i % 4][key kpos]
  if (kvalid) {
    float* dkr = a.dk + (bg * a.n + kpos) * D;
    float* dvr = a.dv + (bg * a.n + kpos) * D;
    // plus the summaries' share of the key's block (zero for an incomplete block)
    const float* dmr = a.dm + (bg * a.nb + kpos / a.bs) * D;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int dcol = 32 * (NDT * dh + t) + 8 * (i / 4) + 4 * lh + (i % 4);
        dkr[dcol] = dka[t][i] * a.rs + dmr[dcol];
        dvr[dcol] = dva[t][i];
      }
  }
}

// ---- route, tiled: one workgroup per (query tile, KV head) -----------------------------------
// All 64 positions of a tile share their candidates, and only the blocks on
// the tile's list can be in any head's support, so per head the coarse
// scores X = Q S^T (64 x count), the entmax Jacobian, the coarse dq = dZ S
// (64 x d) and the tile's share of the summary gradient dZ^T Q (count x d)
// are small dense products over the listed summary rows: those rows come
// through LDS 32 at a time, each thread owns a 2 x 4 block of X, a 4 x (D / 16)
// block of dq and a 2 x (D / 16) block of the summary gradient, which goes to
// the tile's own rows of dspart (the first head stores, the others add; the
// dsum kernel sums the tiles).  LDS rows are read 4 floats at a time; the row
// pitch D + 4 and the assignment of rows {r, r + 32} and of column groups
// {4 c, 64 + 4 c} to threads keep the 8 lanes of each 16-byte read on
// distinct banks.
constexpr int kRtJ = 32;   // summary rows per LDS chunk
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_route_tile_kernel(BwdArgs a) {
  constexpr int QP = D + 4;      // pitch of Qh and Sc rows (floats)
  constexpr int ZP = kBwdTile + 4;
  constexpr int NV = D / 64;     // float4 column groups per thread (64 apart)
  __shared__ __attribute__((aligned(16))) float Qh[kBwdTile * QP];
  __shared__ __attribute__((aligned(16))) float Sc[kRtJ * QP];
  __shared__ __attribute__((aligned(16))) float Zt[kRtJ * ZP];   // dz, list-major
  __shared__ float red[2][8][kBwdTile];
  __shared__ float corr_s[kBwdTile];
  const int64_t nbg = (int64_t)a.B * a.Hkv;
  const int64_t qt = a.slab_q0 + a.slab_nq - 1 - blockIdx.x / nbg;   // most candidates first
  const int64_t bg = blockIdx.x % nbg;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t p0 = qt * kBwdTile;
  const int64_t tile = bg * a.n_qt + qt;
  const int cnt = a.sel_count[tile];
  if (cnt == 0) return;
  const int32_t* lst = a.sel_idx + tile * a.nb;
  const int64_t slot = bg * a.slab + (qt - a.slab_q0);
  // [G][nb][64] per slot; the head-0 plane is overwritten with dp below
  float* dlg = a.dlogp + slot * a.G * a.nb * kBwdTile;
  float* ucg = a.ucoarse + slot * a.G * a.nb * kBwdTile;
  const int tid = threadIdx.x;
  const float* srow = a.summ + bg * a.summ_blocks * D;

  // dp = (sum of the heads' bias gradients) / pbar / G per (listed block, row),
  // pbar = exp(bias / sigma); with sigma = 0 the bias is 0 on the support and
  // the routing takes no gradient
  for (int e2 = tid; e2 < cnt * kBwdTile; e2 += 256) {
    const int e = e2 / kBwdTile, r = e2 % kBwdTile;
    if (p0 + r >= a.n) continue;
    const float lp = a.sel_logp[(tile * a.nb + lst[e]) * kBwdTile + r];
    float sum = 0.f;
    for (int hh = 0; hh < a.G; ++hh) sum += dlg[((int64_t)hh * a.nb + e) * kBwdTile + r];
    float dp = 0.f;
    if (a.sigma > 0.f && lp != -INFINITY) dp = sum / expf(lp / a.sigma) / (float)a.G;
    dlg[(int64_t)e * kBwdTile + r] = dp;
  }
  // (the __syncthreads() at the top of the head loop orders these stores
  // before the reads of other threads)

  const int rg = tid % 32, jg = tid / 32;   // phase A: rows rg + 32 i; list entries 4 jg + k
  const int rq = tid % 16, cq = tid / 16;   // dq: rows 4 rq + i; columns 64 v + 4 cq + [0, 4)
  const int jq = tid / 16, cc = tid % 16;   // ds: entries 2 jq + {0, 1}; columns as dq's
  // the listed summary rows of the next chunk are loaded (16 bytes at a
  // time) into registers while the current chunk is computed
  constexpr int SV = kRtJ * D / 4 / 256;   // float4s per thread per chunk
  f32x4 spre[SV];
  auto load_s = [&](int j0) {
#pragma unroll
    for (int m = 0; m < SV; ++m) {
      const int e = tid + 256 * m, jr = e / (D / 4), c4 = e % (D / 4);
      spre[m] = j0 + jr < cnt ? *(const f32x4*)(srow + (int64_t)lst[j0 + jr] * D + 4 * c4)
                              : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  };
  auto store_s = [&]() {
#pragma unroll
    for (int m = 0; m < SV; ++m) {
      const int e = tid + 256 * m, jr = e / (D / 4), c4 = e % (D / 4);
      *(f32x4*)(Sc + jr * QP + 4 * c4) = spre[m];
    }
  };
  for (int hh = 0; hh < a.G; ++hh) {
    const int64_t bh = (int64_t)b * a.H + g * a.G + hh;
    __syncthreads();
    // q rows, 16 bytes per load, all of a thread's loads issued before its stores
    constexpr int VE = 16 / (int)sizeof(T);
    constexpr int NQL = kBwdTile * D / VE / 256;
    u32x4 wq[NQL];
#pragma unroll
    for (int k = 0; k < NQL; ++k) {
      const int e = tid + 256 * k, r = e / (D / VE), c = (e % (D / VE)) * VE;
      wq[k] = (u32x4){0u, 0u, 0u, 0u};
      if (p0 + r < a.n) wq[k] = *(const u32x4*)((const T*)a.q + (bh * a.n + p0 + r) * D + c);
    }
    float tau2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t pos = p0 + rg + 32 * i;
      tau2[i] = pos < a.n ? a.tau[bh * a.n + pos] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < NQL; ++k) {
      const int e = tid + 256 * k, r = e / (D / VE), c = (e % (D / VE)) * VE;
      const u32x4 w = wq[k];
      if constexpr (sizeof(T) == 2) {
        *(f32x4*)(Qh + r * QP + c) = (f32x4){bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
        *(f32x4*)(Qh + r * QP + c + 4) =
            (f32x4){bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
      } else {
        *(u32x4*)(Qh + r * QP + c) = w;
      }
    }
    float* uh = ucg + (int64_t)hh * a.nb * kBwdTile;
    // phase A: u and the row sums of u and u dp
    float su[2] = {0.f, 0.f}, sud[2] = {0.f, 0.f};
    if (hh == 0 || cnt > kRtJ) load_s(0);   // one chunk: still held from the last head
    for (int j0 = 0; j0 < cnt; j0 += kRtJ) {
      __syncthreads();
      store_s();
      __syncthreads();
      if (j0 + kRtJ < cnt) load_s(j0 + kRtJ);
      // dp of this thread's (row, entry) pairs, loaded before the scores so
      // that their latency hides behind the FMAs
      float dlv[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int e = j0 + 4 * jg + k;
          const bool in = e < cnt && p0 + rg + 32 * i < a.n;
          dlv[i][k] = in ? dlg[(int64_t)e * kBwdTile + rg + 32 * i] : 0.f;
        }
      float x[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) x[i][k] = 0.f;
      for (int c = 0; c < D; c += 4) {
        const f32x4 q0 = *(const f32x4*)(Qh + rg * QP + c);
        const f32x4 q1 = *(const f32x4*)(Qh + (rg + 32) * QP + c);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const f32x4 sv = *(const f32x4*)(Sc + (4 * jg + k) * QP + c);
#pragma unroll
          for (int cc4 = 0; cc4 < 4; ++cc4) {
            x[0][k] = fmaf(q0[cc4], sv[cc4], x[0][k]);
            x[1][k] = fmaf(q1[cc4], sv[cc4], x[1][k]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = rg + 32 * i;
        const int64_t pos = p0 + r;
        if (pos >= a.n) continue;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int e = j0 + 4 * jg + k;
          if (e >= cnt) continue;
          const float y = x[i][k] * a.xscale - tau2[i];
          const float u = y > 0.f ? (a.ue == 0.f ? 1.f : powf(y, a.ue)) : 0.f;
          su[i] += u;
          sud[i] = fmaf(u, dlv[i][k], sud[i]);
          uh[(int64_t)e * kBwdTile + r] = u;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      red[0][jg][rg + 32 * i] = su[i];
      red[1][jg][rg + 32 * i] = sud[i];
    }
    __syncthreads();
    if (tid < kBwdTile) {   // the row's correction (u . dp) / sum u
      float s_u = 0.f, s_ud = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        s_u += red[0][w][tid];
        s_ud += red[1][w][tid];
      }
      corr_s[tid] = s_u > 0.f ? s_ud / s_u : 0.f;
    }
    // phase B + C: dz = gamma u (dp - corr); dq += dz S / sqrt(d)
    f32x4 dqa[4][NV];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < NV; ++v) dqa[i][v] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // phase B inputs of a chunk (8 (row, entry) pairs per thread), loaded
    // one chunk ahead
    constexpr int NB8 = kBwdTile * kRtJ / 256;
    float bdl[NB8], bu[NB8];
    auto load_b = [&](int j0) {
#pragma unroll
      for (int m = 0; m < NB8; ++m) {
        const int e = tid + 256 * m, r = e % kBwdTile, j = j0 + e / kBwdTile;
        const bool in = j < cnt && p0 + r < a.n;
        bdl[m] = in ? dlg[(int64_t)j * kBwdTile + r] : 0.f;
        bu[m] = in ? uh[(int64_t)j * kBwdTile + r] : 0.f;
      }
    };
    load_b(0);
    if (cnt > kRtJ) load_s(0);   // one chunk: still held from phase A
    for (int j0 = 0; j0 < cnt; j0 += kRtJ) {
      __syncthreads();
      store_s();
#pragma unroll
      for (int m = 0; m < NB8; ++m) {
        const int e = tid + 256 * m, r = e % kBwdTile, jr = e / kBwdTile;
        Zt[jr * ZP + r] = a.gamma * bu[m] * (bdl[m] - corr_s[r]);   // 0 outside (bu = 0)
      }
      __syncthreads();
      if (j0 + kRtJ < cnt) {
        load_b(j0 + kRtJ);
        load_s(j0 + kRtJ);
      }
      const int jn = min(kRtJ, cnt - j0);
      for (int jr = 0; jr < jn; ++jr) {
        const f32x4 zv = *(const f32x4*)(Zt + jr * ZP + 4 * rq);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const f32x4 sv = *(const f32x4*)(Sc + jr * QP + 64 * v + 4 * cq);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) dqa[i][v][kk] = fmaf(zv[i], sv[kk], dqa[i][v][kk]);
        }
      }
      // the summaries' share: ds_j += sum over the tile's rows of dz_j q / sqrt(d)
      {
        f32x4 dsa[2][NV];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int v = 0; v < NV; ++v) dsa[jj][v] = (f32x4){0.f, 0.f, 0.f, 0.f};
        for (int r = 0; r < kBwdTile; ++r) {
          const float z0 = Zt[(2 * jq) * ZP + r], z1 = Zt[(2 * jq + 1) * ZP + r];
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            const f32x4 qv = *(const f32x4*)(Qh + r * QP + 64 * v + 4 * cc);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
              dsa[0][v][kk] = fmaf(z0, qv[kk], dsa[0][v][kk]);
              dsa[1][v][kk] = fmaf(z1, qv[kk], dsa[1][v][kk]);
            }
          }
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int e = j0 + 2 * jq + jj;
          if (e < cnt)
#pragma unroll
            for (int v = 0; v < NV; ++v) {
              f32x4* dst = (f32x4*)(a.dspart + (slot * a.nb + e) * D + 64 * v + 4 * cc);
              const f32x4 val = dsa[jj][v] * a.rs;
              *dst = hh == 0 ? val : *dst + val;
            }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t pos = p0 + 4 * rq + i;
      if (pos >= a.n) continue;
      float* dqr = a.dq + (bh * a.n + pos) * D;
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) dqr[64 * v + 4 * cq + kk] += dqa[i][v][kk] * a.rs;
    }
  }
}

// ---- ds_j += the partial rows of this slab's tiles that list block j ---------------------------
// One workgroup per (sequence, KV head, complete block); the tiles' list
// positions of the block are found first (one binary search per tile, side
// by side), then the listing tiles' partial rows are added in a fixed order.
constexpr int kSlabMax = 256;   // tiles per slab (one search per thread)
template <int D>
__global__ __launch_bounds__(D) void bwd_dsum_kernel(BwdArgs a) {
  __shared__ int pos[kSlabMax];
  const int64_t nbc = a.n / a.bs;
  const int64_t j = blockIdx.x % nbc;
  const int64_t bg = blockIdx.x / nbc;
  // tiles before qt0 have block j in their branch or past their end
  const int64_t qt0 = ((j + a.window) * a.bs + kBwdTile - 1) / kBwdTile;
  for (int e = threadIdx.x; e < kSlabMax; e += D) {
    const int64_t qt = a.slab_q0 + e;
    int found = -1;
    if (e < a.slab_nq && qt >= qt0) {
      const int64_t tile = bg * a.n_qt + qt;
      const int cnt = a.sel_count[tile];
      const int32_t* lst = a.sel_idx + tile * a.nb;
      int lo = 0, hi = cnt;
      while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (lst[mid] < j) lo = mid + 1; else hi = mid;
      }
      if (lo < cnt && lst[lo] == j) found = lo;
    }
    pos[e] = found;
  }
  __syncthreads();
  const int r = threadIdx.x;
  // 16 bytes per load: thread t adds the 4 columns of segment t % (D / 4)
  // over the tiles of group t / (D / 4) (four contiguous ranges of the slab,
  // each in tile order, 8 rows in flight at a time); the groups' sums are
  // then added in group order
  constexpr int NS = D / 4, kGroups = 4, kBatch = 8;
  const int c4 = r % NS, grp = r / NS;
  const int per = (int)((a.slab_nq + kGroups - 1) / kGroups);
  const int e_lo = grp * per, e_hi = min((int)a.slab_nq, e_lo + per);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int e0 = e_lo; e0 < e_hi; e0 += kBatch) {
    f32x4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int e = e0 + u;
      v[u] = e < e_hi && pos[e] >= 0
                 ? *(const f32x4*)(a.dspart + ((bg * a.slab + e) * a.nb + pos[e]) * D + 4 * c4)
                 : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (e0 + u < e_hi && pos[e0 + u] >= 0) {
        const float w4[4] = {v[u][0], v[u][1], v[u][2], v[u][3]};
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) acc[k2] += w4[k2];
      }
  }
  __shared__ float part[kGroups][D];
#pragma unroll
  for (int k2 = 0; k2 < 4; ++k2) part[grp][4 * c4 + k2] = acc[k2];
  __syncthreads();
  float sum = 0.f;
#pragma unroll
  for (int g2 = 0; g2 < kGroups; ++g2) sum += part[g2][r];
  a.ds[(bg * a.nb + j) * D + r] += sum;
}

// ---- block means, and dm_j = (ds_j W_s^T) / bs, which the keys kernels add to the block's dk ---
template <typename T, int D>
__global__ __launch_bounds__(D) void bwd_means_kernel(BwdArgs a) {
  const int64_t j = blockIdx.x % a.nb;
  const int64_t bg = blockIdx.x / a.nb;
  const int r = threadIdx.x;
  float* mrow = a.mean + (bg * a.nb + j) * D;
  float* dmrow = a.dm + (bg * a.nb + j) * D;
  if (j >= a.n / a.bs) {   // incomplete block: no summary, no gradient
    mrow[r] = 0.f;
    dmrow[r] = 0.f;
    return;
  }
  const int64_t k0 = bg * a.n + j * a.bs;
  // The block's key rows in 16-byte pieces: thread t sums the VE columns of
  // segment t % SEG over rows t / SEG + VE i (8 loads in flight at a time),
  // then the VE row groups' partial sums are added in group order.  The
  // pieces are copied into plain arrays before their halves or words are
  // used (reading the vector's components directly compiled to the wrong
  // component here).
  constexpr int VE = 16 / (int)sizeof(T);   // values per 16 bytes
  constexpr int SEG = D / VE;               // segments per row (D threads: VE row groups)
  constexpr int kBatch = 8;
  const int seg = r % SEG, rg = r / SEG;
  float acc[VE];
#pragma unroll
  for (int v = 0; v < VE; ++v) acc[v] = 0.f;
  const T* kb = (const T*)a.k + k0 * D + VE * seg;
  for (int t0 = rg; t0 < a.bs; t0 += VE * kBatch) {
    u32x4 w[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int t = t0 + VE * u;
      w[u] = t < a.bs ? *(const u32x4*)(kb + (int64_t)t * D) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if constexpr (sizeof(T) == 2) {
        const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc[2 * h] += bf16_lo(ww[h]);
          acc[2 * h + 1] += bf16_hi(ww[h]);
        }
      } else {
        const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) acc[h] += __uint_as_float(ww[h]);
      }
    }
  }
  __shared__ float part[VE][D];
#pragma unroll
  for (int v = 0; v < VE; ++v) part[rg][VE * seg + v] = acc[v];
  __syncthreads();
  float m = 0.f;
#pragma unroll
  for (int g2 = 0; g2 < VE; ++g2) m += part[g2][r];
  mrow[r] = m / (float)a.bs;
  __shared__ float dsr[D];
  dsr[r] = a.ds[(bg * a.nb + j) * D + r];
  __syncthreads();
  float dm = 0.f;
  for (int c = 0; c < D; ++c) dm = fmaf(dsr[c], a.w_s[r * D + c], dm);
  dmrow[r] = dm / (float)a.bs;
}

// ---- dW_s = sum_j m_j^T ds_j ---------------------------------------------------------------
// The sum over all blocks of all (sequence, KV head) pairs is cut into
// kWsSplit slices (blockIdx.y), each written to its own plane of wspart;
// bwd_ws_sum_kernel adds the planes in slice order.
constexpr int kWsSplit = 32;
template <int D>
__global__ __launch_bounds__(256) void bwd_ws_kernel(BwdArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)D * D) return;
  const int r = (int)(idx / D), c = (int)(idx % D);
  const int64_t nblk = (int64_t)a.B * a.Hkv * a.nb;
  const int64_t per = (nblk + kWsSplit - 1) / kWsSplit;
  const int64_t u0 = min(nblk, blockIdx.y * per), u1 = min(nblk, u0 + per);
  float acc = 0.f;
#pragma unroll 4
  for (int64_t u = u0; u < u1; ++u) acc = fmaf(a.mean[u * D + r], a.ds[u * D + c], acc);
  a.wspart[blockIdx.y * (int64_t)D * D + idx] = acc;
}
template <int D>
__global__ __launch_bounds__(256) void bwd_ws_sum_kernel(BwdArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)D * D) return;
  float acc = 0.f;
  for (int sl = 0; sl < kWsSplit; ++sl) acc += a.wspart[sl * (int64_t)D * D + idx];
  a.dw_s[idx] = acc;
}

__global__ void bwd_zero_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// Query tiles per slab: the per-tile arrays of one slab stay within
// kBwdSlabBytes (at least one tile, at most kSlabMax).
constexpr int64_t kBwdSlabBytes = (int64_t)1 << 30;
static int64_t bwd_slab_tiles(const Shape& s, int64_t n) {
  const int64_t n_qt = (n + kBwdTile - 1) / kBwdTile, nb = (n + s.bs - 1) / s.bs;
  const int64_t per_tile = (int64_t)sizeof(float) * s.B * s.Hkv * nb *
                           (2 * (int64_t)s.G * kBwdTile + s.d);
  int64_t slab = kBwdSlabBytes / per_tile;
  slab = slab < 1 ? 1 : slab;
  slab = slab > kSlabMax ? kSlabMax : slab;
  return slab < n_qt ? slab : n_qt;
}

BwdLayout bwd_layout(const Shape& s, int64_t n) {
  BwdLayout L;
  const int64_t nb = (n + s.bs - 1) / s.bs, slab = bwd_slab_tiles(s, n);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t per_slot = sizeof(float) * s.B * s.Hkv * slab * s.G * nb * kBwdTile;
  size_t off = 0;
  L.off_lse = off;    off = al(off + sizeof(float) * s.B * s.H * n);
  L.off_delta = off;  off = al(off + sizeof(float) * s.B * s.H * n);
  L.off_dlogp = off;  off = al(off + per_slot);
  L.off_u = off;      off = al(off + per_slot);
  L.off_ds = off;     off = al(off + sizeof(float) * s.B * s.Hkv * nb * s.d);
  L.off_mean = off;   off = al(off + sizeof(float) * s.B * s.Hkv * nb * s.d);
  L.off_dm = off;     off = al(off + sizeof(float) * s.B * s.Hkv * nb * s.d);
  L.off_dspart = off; off = al(off + sizeof(float) * s.B * s.Hkv * slab * nb * s.d);
  L.off_wspart = off; off = al(off + sizeof(float) * kWsSplit * s.d * s.d);
  L.slab = slab;
  L.total = off;
  return L;
}

template <typename T, int D>
static hipError_t bwd_t(BwdArgs a, hipStream_t st) {
  const int64_t nbg = (int64_t)a.B * a.Hkv;
  hipLaunchKernelGGL(bwd_zero_kernel, dim3(256), dim3(256), 0, st, a.ds, nbg * a.nb * D);
  const int64_t nbc = a.n / a.bs;   // complete blocks
  for (int64_t q0 = 0; q0 < a.n_qt; q0 += a.slab) {
    a.slab_q0 = q0;
    a.slab_nq = a.n_qt - q0 < a.slab ? a.n_qt - q0 : a.slab;
    if constexpr (sizeof(T) == 2) {
      // 2 G waves of 32 queries per tile, at most 8 per workgroup
      const int waves = 2 * a.G, wpt = (waves + 7) / 8;
      const dim3 grid((unsigned)(a.slab_nq * nbg * wpt));
      if (waves == 2)
        hipLaunchKernelGGL((bwd_rows_mfma_kernel<D, 128>), grid, dim3(128), 0, st, a);
      else if (waves == 4)
        hipLaunchKernelGGL((bwd_rows_mfma_kernel<D, 256>), grid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((bwd_rows_mfma_kernel<D, 512>), grid, dim3(512), 0, st, a);
    } else {
      const size_t lds_r = sizeof(T) * 2 * kBwdChunk * D;
      (void)hipFuncSetAttribute((const void*)bwd_rows_kernel<T, D>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_r);
      hipLaunchKernelGGL((bwd_rows_kernel<T, D>), dim3((unsigned)(a.slab_nq * a.B * a.H)),
                         dim3(256), lds_r, st, a);
    }
    hipLaunchKernelGGL((bwd_route_tile_kernel<T, D>), dim3((unsigned)(a.slab_nq * nbg)),
                       dim3(256), 0, st, a);
    if (nbc > 0)
      hipLaunchKernelGGL((bwd_dsum_kernel<D>), dim3((unsigned)(nbc * nbg)), dim3(D), 0, st, a);
  }
  hipLaunchKernelGGL((bwd_means_kernel<T, D>), dim3((unsigned)(a.nb * nbg)), dim3(D), 0, st, a);
  const int64_t nch = (a.n + kBwdChunk - 1) / kBwdChunk;
  if constexpr (sizeof(T) == 2) {
    const size_t lds_km = sizeof(__bf16) * (2 * kBwdTile * (D + 8) + 2 * D * (kBwdTile + 8)) +
                          sizeof(float) * 3 * kBwdTile;
    (void)hipFuncSetAttribute((const void*)bwd_keys_mfma_kernel<D>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_km);
    hipLaunchKernelGGL((bwd_keys_mfma_kernel<D>), dim3((unsigned)(nch * nbg)), dim3(256), lds_km,
                       st, a);
  } else {
    const size_t lds_k = sizeof(T) * 2 * kBwdTile * D + sizeof(float) * 3 * kBwdTile;
    (void)hipFuncSetAttribute((const void*)bwd_keys_kernel<T, D>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_k);
    hipLaunchKernelGGL((bwd_keys_kernel<T, D>), dim3((unsigned)(nch * nbg)), dim3(256), lds_k,
                       st, a);
  }
  hipLaunchKernelGGL((bwd_ws_kernel<D>), dim3((unsigned)((D * D + 255) / 256), kWsSplit),
                     dim3(256), 0, st, a);
  hipLaunchKernelGGL((bwd_ws_sum_kernel<D>), dim3((unsigned)((D * D + 255) / 256)), dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

hipError_t launch_prefill_backward(const Shape& s, const void* q, const void* k, const void* v,
                                   const void* o, const void* dO, int64_t n, const float* w_s,
                                   const float* summ, int64_t summ_blocks,
                                   const dash_route_buf& rb, float* dq, float* dk, float* dv,
                                   float* dw_s, const BwdLayout& L, char* ws, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dO = dO;
  a.w_s = w_s;
  a.summ = summ;
  a.summ_blocks = summ_blocks;
  a.tau = rb.tau;
  a.sel_count = rb.sel_count;
  a.sel_idx = rb.sel_idx;
  a.sel_logp = rb.sel_logp;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dw_s = dw_s;
  a.lse2 = (float*)(ws + L.off_lse);
  a.delta = (float*)(ws + L.off_delta);
  a.dlogp = (float*)(ws + L.off_dlogp);
  a.ucoarse = (float*)(ws + L.off_u);
  a.ds = (float*)(ws + L.off_ds);
  a.mean = (float*)(ws + L.off_mean);
  a.dm = (float*)(ws + L.off_dm);
  a.dspart = (float*)(ws + L.off_dspart);
  a.wspart = (float*)(ws + L.off_wspart);
  a.slab = L.slab;
  a.slab_q0 = 0;
  a.slab_nq = 0;
  a.n = n;
  a.n_qt = (n + kBwdTile - 1) / kBwdTile;
  a.nb = (n + s.bs - 1) / s.bs;
  a.B = s.B;
  a.H = s.H;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.bs = s.bs;
  a.window = s.window;
  a.scale_log2 = kLog2e / sqrtf((float)s.d);
  a.rs = 1.0f / sqrtf((float)s.d);
  a.xscale = (s.alpha - 1.0f) * s.gamma / sqrtf((float)s.d);
  a.gamma = s.gamma;
  a.sigma = s.sigma;
  a.ue = (2.0f - s.alpha) / (s.alpha - 1.0f);
  if (s.dtype == DASH_BF16)
    return s.d == 64 ? bwd_t<__bf16, 64>(a, st) : bwd_t<__bf16, 128>(a, st);
  return s.d == 64 ? bwd_t<float, 64>(a, st) : bwd_t<float, 128>(a, st);
}

}  // namespace dash
