// attend.hip -- Stage 2 of DashAttention for causal prefill ("prior-induced
// sparse softmax", DashAttention explainer, Technical summary): attention of
// each query restricted to the blocks its 64-position tile selected, with the
// routing probability as a prior (logit q.k/sqrt(d) + sigma log pbar, the
// bias Stage 1 stored), blocks of probability 0 masked (-inf), and the
// near-diagonal branch -- the query's own block and the window - 1 blocks
// before it -- attended causally with bias 0.  The pages' kernel is a modified
// FlashAttention that walks the active chunks and adds the routing bias before
// the softmax; this is a gfx950 design of that idea.
//
// bf16 kernel: one workgroup per (sequence, KV head, query tile) -- up to 8
// waves; each wave owns 32 queries of one head of the group, so every K/V
// chunk staged in LDS serves all G heads.  The walk goes over 64-key chunks:
// branch chunks first (so every running max is finite), then the selected
// blocks.  Per chunk and wave:
//   S^T (64 keys x 32 queries) = K Q^T     2 x 8 MFMA 32x32x16 (d = 128)
//   online softmax in the exp2 domain, bias added per (query, block)
//   O^T (d x 32 queries) += V^T P^T        4 x 4 MFMA 32x32x16
// Keys are the MFMA rows of S^T, so the accumulator of S^T already has the
// register layout of the P^T operand (the k index of the PV product is a
// permutation of the chunk's keys).  V is transposed into LDS while it is
// staged, with the keys of each group of 16 stored in the order of that
// permutation, so every V^T operand fragment is one 16-byte read; the 16-byte
// segments of each V^T row are XOR-swizzled by the row index so that both
// the staging stores and the fragment reads hit distinct LDS banks.
#include "dash_internal.hpp"
#include "device_common.hpp"

namespace dash {

constexpr int kQTa = DASH_QUERY_TILE;
constexpr int kXcds = 8;   // accelerator complex dies of the part, one L2 each
constexpr int kChunk = 64;

struct AttendArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t n;
  const int32_t* sel_count;
  const int32_t* sel_idx;
  const float* sel_logp;
  int64_t n_qt, nb;
  int H, Hkv, G, bs, B;
  float scale_log2;   // log2(e) / sqrt(d)
  int wg_per_tile;
  int window;         // near-diagonal branch: own block + window - 1 blocks before it
  const int32_t* seq_len;   // [B] valid positions per sequence, or null (all n)
};

// Valid positions of sequence b: seq_len[b] clamped into [0, n], or n.
__device__ __forceinline__ int64_t attend_valid_len(const AttendArgs& a, int b) {
  if (!a.seq_len) return a.n;
  const int64_t l = a.seq_len[b];
  return l < 0 ? 0 : (l > a.n ? a.n : l);
}

// first block of the tile's near-diagonal branch (own block - (window - 1), >= 0)
__device__ __forceinline__ int64_t branch_block0(int64_t p_begin, int bs, int window) {
  const int64_t j = p_begin / bs - (window - 1);
  return j > 0 ? j : 0;
}

// chunk c of the tile's walk -> first key and bias source
struct ChunkRef {
  int64_t key0;
  int64_t block;   // -1 for own-block chunks (bias 0)
  bool diag;       // chunk starting at the tile's first position: causal mask
};

__device__ __forceinline__ ChunkRef chunk_ref(int c, int n_own, int64_t own_c0, int cpb,
                                              const int32_t* idx) {
  ChunkRef r;
  if (c < n_own) {
    r.key0 = (own_c0 + c) * kChunk;
    r.block = -1;
    r.diag = c == n_own - 1;
  } else {
    const int cc = c - n_own;
    const int64_t j = idx[cc / cpb];
    r.key0 = j * (int64_t)(cpb * kChunk) + (cc % cpb) * kChunk;
    r.block = j;
    r.diag = false;
  }
  return r;
}

// ------------------------------------------------------------------------------------------
// bf16, MFMA
// ------------------------------------------------------------------------------------------
// V^T row r (one d, 64 keys = 128 bytes = 8 segments of 16 bytes): logical
// segment s is stored at s ^ vt_swizzle(r).  Staging writes rows 2 dp + {0,1}
// for 8 consecutive d pairs per 8 lanes, fragment reads take 8 consecutive
// rows per 8 lanes: both map those 8 lanes to 8 distinct segments, i.e. to
// distinct banks.  Rows 32 apart share the swizzle, so a lane's read offsets
// are the same for every 32-row tile.
__device__ __forceinline__ int vt_swizzle(int r) { return (r & 7) ^ ((r >> 3) & 3); }

// Staging of one 64-key chunk: K row-major [64][D + 8], V transposed [D][64]
// (keys permuted within each group of 16 and segments swizzled, see store())
// (bf16), and the chunk's 64 per-query biases (float, log pbar of the chunk's
// block; 0 for own-block chunks).  NT threads; each thread owns KPT 16-byte
// pieces of K and VPT (segment, d pair) units of V^T -- the 8 keys of one
// V^T segment at two adjacent d; lanes 0..15 of wave 0 own the bias.
// Loads go through buffer resources, so keys at or past n read as zeros
// without branches, and the bias rides the same in-order load queue as K/V
// (no wait on it can stall on a younger K/V load).
template <int D, int NT>
struct ChunkStage {
  static constexpr int KP = D + 8;
  static constexpr int VP = kChunk;                      // 128-byte rows, swizzled segments
  static constexpr int KTOT = kChunk * (D / 8);          // 16-byte pieces of K
  static constexpr int VTOT = 8 * (D / 2);               // (segment, d pair) units of V^T
  static constexpr int KPT = (KTOT + NT - 1) / NT;
  static constexpr int VPT = (VTOT + NT - 1) / NT;
  u32x4 kr[KPT];
  uint32_t vr[VPT][8];
  u32x4 br;

  // key0: first key of the chunk; block: its block id, -1 for an own-block
  // chunk.  rk / rv cover one sequence's keys / values, rb the tile's bias rows.
  // (32-bit byte offsets: one sequence's keys span less than 2 GiB; the chunk
  // base plus a per-thread part, with the per-key steps of V as instruction
  // offsets)
  __device__ __forceinline__ void load(buf_rsrc rk, buf_rsrc rv, buf_rsrc rb, int key0,
                                       int block) {
    const uint32_t cb = (uint32_t)key0 * (uint32_t)(D * 2);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = threadIdx.x + i * NT;
      const int key = e / (D / 8), seg = e % (D / 8);
      const uint32_t off = cb + (uint32_t)(key * (D * 2) + seg * 16);
      if (KTOT % NT == 0 || e < KTOT) kr[i] = buf_load16(rk, off);
    }
    // V^T unit (segment sg, d pair dp): the keys 16 (sg / 2) + 4 (sg % 2) +
    // 8 a + j (a < 2, j < 4) at d = 2 dp, 2 dp + 1; a wave's lanes take
    // consecutive d pairs, so each load reads whole key rows
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int e = threadIdx.x + i * NT;
      const int dp = e % (D / 2), sg = e / (D / 2);
      const int kbase = 16 * (sg >> 1) + 4 * (sg & 1);
      const uint32_t vb = cb + (uint32_t)(kbase * (D * 2) + dp * 4);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t off = vb + (uint32_t)((8 * a + j) * (D * 2));
          if (VTOT % NT == 0 || e < VTOT) vr[i][4 * a + j] = buf_load4(rv, off);
        }
    }
    if (threadIdx.x < kWave) {   // wave-uniform
      br = (u32x4){0u, 0u, 0u, 0u};
      if (block >= 0)
        br = buf_load16(rb, (uint32_t)block * (kQTa * 4) + (threadIdx.x % 16) * 16);
    }
  }
  __device__ __forceinline__ void store(__bf16* Ks, __bf16* Vt, float* Bs) const {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int e = threadIdx.x + i * NT;
      const int key = e / (D / 8), seg = e % (D / 8);
      if (KTOT % NT == 0 || e < KTOT) *(u32x4*)(Ks + key * KP + seg * 8) = kr[i];
    }
    // keys 16 m + 8 a + 4 b + [0, 4) go to columns 16 m + 8 b + 4 a + [0, 4):
    // the 8 keys one lane needs for a PV k-step form logical segment 2 m + b
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int e = threadIdx.x + i * NT;
      if (VTOT % NT != 0 && e >= VTOT) continue;
      const int dp = e % (D / 2), sg = e / (D / 2);
      const uint32_t* w = vr[i];
      const u32x4 lo = {pack_lo(w[0], w[1]), pack_lo(w[2], w[3]), pack_lo(w[4], w[5]),
                        pack_lo(w[6], w[7])};
      const u32x4 hi = {pack_hi(w[0], w[1]), pack_hi(w[2], w[3]), pack_hi(w[4], w[5]),
                        pack_hi(w[6], w[7])};
      const int r0 = 2 * dp, r1 = 2 * dp + 1;
      *(u32x4*)(Vt + r0 * VP + 8 * (sg ^ vt_swizzle(r0))) = lo;
      *(u32x4*)(Vt + r1 * VP + 8 * (sg ^ vt_swizzle(r1))) = hi;
    }
    if (threadIdx.x < kQTa / 4) *(u32x4*)(Bs + 4 * threadIdx.x) = br;
  }
};

// Workgroup barrier that orders LDS accesses only: global loads issued before
// it stay in flight (__syncthreads would wait for them too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Rescale the running output only when a row max grows by more than 2^8:
// exp2(s - m_ref) then stays <= 256, exact in float32 and in bf16's range.
constexpr float kLazyRescale = 8.0f;

template <int D, int NT>
__global__ __launch_bounds__(NT) void attend_bf16_kernel(AttendArgs a) {
  using Stage = ChunkStage<D, NT>;
  constexpr int KP = Stage::KP, VP = Stage::VP;
  // LDS ring of NBUF chunk buffers: chunk c + 2 is stored while chunk c is
  // computed, so a workgroup barrier is needed once every NBUF - 2 chunks.
  // d = 128: four buffers (133 KB; one workgroup per CU with three as well),
  // a barrier every second chunk; d = 64: three, which keeps more
  // workgroups resident.
  constexpr int NBUF = D == 128 ? 4 : 3;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[NBUF][kChunk * KP];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[NBUF][D * VP];
  __shared__ __attribute__((aligned(16))) float Bs[NBUF][kQTa];

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int l32 = lane % 32, lh = lane / 32;

  const int64_t nbg = (int64_t)a.B * a.Hkv;
  int64_t qt, bg;
  int wi;
  if (nbg > kXcds && nbg % kXcds == 0) {
    // Workgroups go to the XCDs round-robin (workgroup w to XCD w % 8), each
    // XCD with its own L2: give every (sequence, KV head) to one XCD and let
    // that XCD walk its pairs one after another, each pair's tiles heaviest
    // first, so one L2 holds one pair's K/V at a time.
    const int64_t x = blockIdx.x % kXcds, r = blockIdx.x / kXcds;
    const int64_t per_pair = a.n_qt * a.wg_per_tile;
    const int64_t rem = r % per_pair;
    bg = x + kXcds * (r / per_pair);
    qt = a.n_qt - 1 - rem / a.wg_per_tile;
    wi = (int)(rem % a.wg_per_tile);
  } else {
    // at most one pair per XCD (or a count that does not divide evenly): all
    // tiles heaviest first, the pairs of one tile rank side by side
    const int64_t tile_rank = blockIdx.x / a.wg_per_tile;
    wi = blockIdx.x % a.wg_per_tile;
    qt = a.n_qt - 1 - tile_rank / nbg;
    bg = tile_rank % nbg;
  }
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int64_t p_begin = qt * kQTa;
  const int64_t tile = bg * a.n_qt + qt;
  // positions of this sequence (rows are a.n apart); a tile past its end has nothing to do
  const int64_t nv = attend_valid_len(a, b);
  if (p_begin >= nv) return;

  const int gw = wi * (NT / kWave) + wave;   // wave index within the tile
  const int h = g * a.G + gw / 2;            // query head
  const int half = gw % 2;
  const int qloc = 32 * half + l32;          // query row within the tile
  const int64_t qpos = p_begin + qloc;

  const __bf16* qp = (const __bf16*)a.q + (((int64_t)b * a.H + h) * a.n) * D;
  const uint32_t seq_bytes = (uint32_t)(nv * (D * 2));
  const buf_rsrc rk = make_rsrc((const __bf16*)a.k + (bg * a.n) * D, seq_bytes);
  const buf_rsrc rv = make_rsrc((const __bf16*)a.v + (bg * a.n) * D, seq_bytes);
  const buf_rsrc rb = make_rsrc(a.sel_logp + tile * a.nb * kQTa, (uint32_t)(a.nb * kQTa * 4));

  // this lane's V^T fragment of PV k-step ks and d tile dt: row 32 dt + l32
  // (rows 32 apart share the swizzle), logical segment 2 ks + lh, i.e. the
  // element offset vrow + 32 dt VP + (vx ^ 16 ks)
  const int vrow = l32 * VP, vx = 8 * (lh ^ vt_swizzle(l32));

  // Q^T operand fragments: column = query l32, k = d in [16 s + 8 lh, +8)
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qpos < nv) w = *(const u32x4*)(qp + qpos * D + 16 * s + 8 * lh);
    qf[s] = as_bf16x8(w);
  }

  // chunks per block: 1 or 2 (a scalar: the chunk walk's arithmetic stays in
  // SGPRs, in 32 bits -- one sequence's keys span less than 2 GiB)
  const int cpb_log = __builtin_amdgcn_readfirstlane(a.bs == 2 * kChunk ? 1 : 0);
  const int own_c0 = (int)(branch_block0(p_begin, a.bs, a.window) << cpb_log);
  const int n_own = (int)(qt - own_c0 + 1);
  const int count = a.sel_count[tile];
  const int n_chunks = n_own + (count << cpb_log);
  // the tile's selected block ids; chunk c >= n_own belongs to entry
  // (c - n_own) >> cpb_log, other offsets fall outside the range and read 0
  const buf_rsrc ri = make_rsrc(a.sel_idx + tile * a.nb, (uint32_t)(count * 4));
  auto sel_block = [&](int c) -> uint32_t {
    return buf_load4(ri, (uint32_t)(((c - n_own) >> cpb_log) * 4));
  };
  // chunk c (block id j when selected) -> first key, bias block (-1: own block)
  auto key0_of = [&](int c, int j) -> int {
    return c < n_own ? (own_c0 + c) * kChunk
                     : (j << cpb_log) * kChunk + ((c - n_own) & cpb_log) * kChunk;
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  float m_ref = -INFINITY, l_run = 0.f;

  // Chunk c sits in LDS buffer c % NBUF; chunk c+1 is already staged and chunk
  // c+2's K/V/bias are in flight from HBM into registers, preceded in the
  // load queue by the block id of chunk c+3.
  // Prologue: the block ids of chunks 0..3 arrive with one load (slots of
  // own-block chunks and past the list read as 0 and are not used), chunks 0
  // and 1 are loaded together, then chunk 2's loads stay in flight into the
  // loop behind an LDS-only barrier.
  uint32_t j4[4];
  {
    // chunk c >= n_own belongs to list entry (c - n_own) >> cpb_log
    u32x4 w4 = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int c = 0; c < 4; ++c) j4[c] = 0u;
    if (n_own < 4 && count > 0) w4 = buf_load16(ri, 0u);
    const uint32_t wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = (c - n_own) >> cpb_log;   // uniform; negative for own chunks
      uint32_t jj = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) jj = e == q ? wv[q] : jj;
      j4[c] = __builtin_amdgcn_readfirstlane(jj);
    }
  }
  Stage stage, stage1;
  if (n_chunks > 0) stage.load(rk, rv, rb, key0_of(0, (int)j4[0]), 0 < n_own ? -1 : (int)j4[0]);
  if (n_chunks > 1) stage1.load(rk, rv, rb, key0_of(1, (int)j4[1]), 1 < n_own ? -1 : (int)j4[1]);
  if (n_chunks > 0) stage.store(Ks[0], Vt[0], Bs[0]);
  if (n_chunks > 1) stage1.store(Ks[1], Vt[1], Bs[1]);
  uint32_t jv = j4[3];
  if (n_chunks > 2) stage.load(rk, rv, rb, key0_of(2, (int)j4[2]), 2 < n_own ? -1 : (int)j4[2]);
  lds_barrier();

  int bcur = 0;
  for (int c = 0; c < n_chunks; ++c) {
    const int bnx = bcur == NBUF - 1 ? 0 : bcur + 1;
    const int bnx2 = bnx == NBUF - 1 ? 0 : bnx + 1;

    // ---- S^T (64 keys x 32 queries) = K Q^T: two 32-key tiles ----
    const __bf16* Kc = Ks[bcur];
    u32x4 kw[2][D / 16];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        kw[kt][s] = *(const u32x4*)(Kc + (32 * kt + l32) * KP + 16 * s + 8 * lh);
    f32x16 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) st[kt][i] = 0.f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) st[kt] = mfma32(as_bf16x8(kw[kt][s]), qf[s], st[kt]);
    }
    // issue all 2 x D/16 K-fragment reads before the first MFMA (mask 0x100:
    // LDS reads, 0x008: MFMA), so LDS latency is paid once per chunk
    __builtin_amdgcn_sched_group_barrier(0x100, D / 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, D / 8, 0);

    // V^T fragments of the chunk, read while the scores are computed
    const __bf16* Vc = Vt[bcur];
    u32x4 vw[4][D / 32];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        vw[ks][dt] = *(const u32x4*)(Vc + vrow + 32 * dt * VP + (vx ^ (16 * ks)));
      }

    // ---- online softmax of chunk c, exp2 domain: logit2 = s * scale_log2 + bias2 ----
    // (rows past the sequence's end have no stored bias: Stage 1 writes only
    // valid rows, and a value left in memory could otherwise trigger the
    // wave's lazy rescale and change the rounding of the valid rows)
    const float bias2 = qpos < nv ? Bs[bcur][qloc] * kLog2e : 0.f;
    if (c == n_own - 1) {   // the diagonal chunk starts at the tile's first position
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * kt + 8 * (i / 4) + 4 * lh + (i % 4);
          if (key > qloc) st[kt][i] = -INFINITY;
        }
    }
    float smax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) smax = fmaxf(smax, st[kt][i]);
    smax = xor_reduce<32>(smax, DppMax{});
    const float cmax = fmaf(smax, a.scale_log2, bias2);   // -inf when all masked
    if (__any(cmax > m_ref + kLazyRescale)) {
      const float m_new = fmaxf(m_ref, cmax);
      const float corr = m_new == -INFINITY ? 1.f : fast_exp2(m_ref - m_new);
      l_run *= corr;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] *= corr;
      m_ref = m_new;
    }
    const float off = m_ref == -INFINITY ? 0.f : bias2 - m_ref;
    // the row sum adds the bf16 weights the P V product uses, two per
    // v_dot2c_f32_bf16 against (1, 1)
    float psum = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kt = ks / 2, i0 = 8 * (ks % 2);
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(fmaf(st[kt][i0 + e], a.scale_log2, off));
      const u32x4 pw = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]),
                        pack_bf16(pv[4], pv[5]), pack_bf16(pv[6], pv[7])};
      psum = sum2_bf16(pw.x, sum2_bf16(pw.y, sum2_bf16(pw.z, sum2_bf16(pw.w, psum))));
      pf[ks] = as_bf16x8(pw);
    }
    psum = xor_reduce<32>(psum, DppAdd{});
    l_run += psum;

    // ---- O^T += V^T P^T : 4 k-steps of 16 keys ----
    // issued at raised wave priority (the compiler then places the chunk's
    // exponentials before them): the SIMD's other wave, in its softmax,
    // yields the issue slots to these MFMAs (8K attend -1.7 %, 64K -0.7 %)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) acc[dt] = mfma32(as_bf16x8(vw[ks][dt]), pf[ks], acc[dt]);
    __builtin_amdgcn_s_setprio(0);

    // chunk c+2 into the buffer chunk c+2-NBUF used (every wave is past it:
    // the last barrier came after that chunk)
    if (c + 2 < n_chunks) stage.store(Ks[bnx2], Vt[bnx2], Bs[bnx2]);
    if (c % (NBUF - 2) == NBUF - 3) __syncthreads();
    const int c3 = c + 3;
    if (c3 < n_chunks) {
      const int j = __builtin_amdgcn_readfirstlane(jv);
      jv = sel_block(c3 + 1);
      stage.load(rk, rv, rb, key0_of(c3, j), c3 < n_own ? -1 : j);
    }
    bcur = bnx;
  }

  // ---- normalise and store: acc[dt][i] = O[query l32][32 dt + 8 (i/4) + 4 lh + i%4] ----
  if (qpos < nv) {
    const float inv = 1.0f / l_run;
    __bf16* op = (__bf16*)a.o + (((int64_t)b * a.H + h) * a.n + qpos) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        u32x2 w = {pack_bf16(acc[dt][4 * i4 + 0] * inv, acc[dt][4 * i4 + 1] * inv),
                   pack_bf16(acc[dt][4 * i4 + 2] * inv, acc[dt][4 * i4 + 3] * inv)};
        *(u32x2*)(op + 32 * dt + 8 * i4 + 4 * lh) = w;
      }
  }
}

// ------------------------------------------------------------------------------------------
// float32, plain FMAs (one thread per query of one head)
// ------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attend_f32_kernel(AttendArgs a) {
  __shared__ float Ks[kChunk * D];
  __shared__ float Vs[kChunk * D];
  const int64_t nbg = (int64_t)a.B * a.Hkv;
  const int64_t rank = blockIdx.x / a.G;
  const int hh = blockIdx.x % a.G;
  const int64_t qt = a.n_qt - 1 - rank / nbg;
  const int64_t bg = rank % nbg;
  const int b = (int)(bg / a.Hkv), g = (int)(bg % a.Hkv);
  const int h = g * a.G + hh;
  const int64_t p_begin = qt * kQTa;
  const int64_t tile = bg * a.n_qt + qt;
  const int64_t nv = attend_valid_len(a, b);
  if (p_begin >= nv) return;
  const int qloc = threadIdx.x;
  const int64_t qpos = p_begin + qloc;
  const float* kp = (const float*)a.k + (bg * a.n) * D;
  const float* vp = (const float*)a.v + (bg * a.n) * D;

  float qv[D], ov[D];
  const float* qrow = (const float*)a.q + (((int64_t)b * a.H + h) * a.n + qpos) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qv[c] = qpos < nv ? qrow[c] : 0.f;
    ov[c] = 0.f;
  }
  const int cpb = a.bs / kChunk;
  const int64_t own_c0 = branch_block0(p_begin, a.bs, a.window) * cpb;
  const int n_own = (int)(qt - own_c0 + 1);
  const int count = a.sel_count[tile];
  const int32_t* idx = a.sel_idx + tile * a.nb;
  const int n_chunks = n_own + count * cpb;
  float m_run = -INFINITY, l_run = 0.f;
  const float scale = a.scale_log2;

  for (int c = 0; c < n_chunks; ++c) {
    const ChunkRef cr = chunk_ref(c, n_own, own_c0, cpb, idx);
    __syncthreads();
    for (int e = threadIdx.x; e < kChunk * D; e += 64) {
      const int64_t kpos = cr.key0 + e / D;
      Ks[e] = kpos < nv ? kp[cr.key0 * D + e] : 0.f;
      Vs[e] = kpos < nv ? vp[cr.key0 * D + e] : 0.f;
    }
    __syncthreads();
    const float bias2 =
        cr.block >= 0 ? a.sel_logp[(tile * a.nb + cr.block) * kQTa + qloc] * kLog2e : 0.f;
    for (int key = 0; key < kChunk; ++key) {
      if (cr.diag && cr.key0 + key > qpos) break;
      float s = 0.f;
#pragma unroll
      for (int cc = 0; cc < D; ++cc) s = fmaf(qv[cc], Ks[key * D + cc], s);
      s = fmaf(s, scale, bias2);
      const float m_new = fmaxf(m_run, s);
      if (m_new == -INFINITY) continue;
      const float corr = fast_exp2(m_run - m_new), p = fast_exp2(s - m_new);
      l_run = l_run * corr + p;
#pragma unroll
      for (int cc = 0; cc < D; ++cc) ov[cc] = fmaf(p, Vs[key * D + cc], ov[cc] * corr);
      m_run = m_new;
    }
  }
  if (qpos < nv) {
    float* orow = (float*)a.o + (((int64_t)b * a.H + h) * a.n + qpos) * D;
#pragma unroll
    for (int c = 0; c < D; ++c) orow[c] = ov[c] / l_run;
  }
}

hipError_t launch_attend_prefill(const Shape& s, const void* q, const void* k, const void* v,
                                 int64_t n, const dash_route_buf& rb, void* o, hipStream_t st,
                                 const int32_t* seq_len) {
  if (n <= 0) return hipSuccess;
  AttendArgs a;
  a.seq_len = seq_len;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.n = n;
  a.sel_count = rb.sel_count;
  a.sel_idx = rb.sel_idx;
  a.sel_logp = rb.sel_logp;
  a.n_qt = (n + kQTa - 1) / kQTa;
  a.nb = (n + s.bs - 1) / s.bs;
  a.H = s.H;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.bs = s.bs;
  a.B = s.B;
  a.window = s.window;
  a.scale_log2 = kLog2e / sqrtf((float)s.d);
  const int64_t tiles = a.n_qt * s.B * s.Hkv;
  if (s.dtype == DASH_BF16) {
    const int waves = 2 * s.G;                 // 32 queries x 1 head per wave
    a.wg_per_tile = (waves + 7) / 8;
    const int threads = (waves < 8 ? waves : 8) * kWave;
    dim3 grid((unsigned)(tiles * a.wg_per_tile));
#define DASH_AT(D, NT) hipLaunchKernelGGL((attend_bf16_kernel<D, NT>), grid, dim3(NT), 0, st, a)
    if (s.d == 64) {
      if (threads == 128) DASH_AT(64, 128); else if (threads == 256) DASH_AT(64, 256); else DASH_AT(64, 512);
    } else {
      if (threads == 128) DASH_AT(128, 128); else if (threads == 256) DASH_AT(128, 256); else DASH_AT(128, 512);
    }
#undef DASH_AT
  } else {
    a.wg_per_tile = 1;
    dim3 grid((unsigned)(tiles * s.G));
    if (s.d == 64)
      hipLaunchKernelGGL(attend_f32_kernel<64>, grid, dim3(64), 0, st, a);
    else
      hipLaunchKernelGGL(attend_f32_kernel<128>, grid, dim3(64), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace dash
