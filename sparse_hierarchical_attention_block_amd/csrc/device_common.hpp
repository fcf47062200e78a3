// device_common.hpp -- small device helpers shared by the gfx950 kernels of
// the DashAttention library: element types, wave64 reductions and MFMA
// fragment types.  Nothing here is used by the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dash {

// f(std::integral_constant<int, I>{}) for I = Begin .. End - 1, expanded by
// template instantiation: register arrays indexed by I stay in registers
// however long the body (the loop unroller gives up above a size limit and
// leaves such arrays in scratch memory).
template <int Begin, int End, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (Begin < End) {
    f(std::integral_constant<int, Begin>{});
    static_for<Begin + 1, End>(f);
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- element access --------------------------------------------------------

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// bf16 bits <-> float (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// pack the low halves / high halves of two words: (a.lo, b.lo) and (a.hi, b.hi)
// (one v_perm_b32 byte select each: bytes 0-3 of the pair are a, 4-7 are b)
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// two floats -> packed bf16 pair (round to nearest even), x in the low half
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r;
  r.x = (__bf16)x;
  r.y = (__bf16)y;
  return __builtin_bit_cast(uint32_t, r);
}

// 2^x with the hardware instruction (v_exp_f32): no denormal-range fix-up,
// results below 2^-126 flush to zero, which softmax weights can afford.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// c + the two bf16 halves of w (products with 1 are exact): v_dot2c_f32_bf16
__device__ __forceinline__ float sum2_bf16(uint32_t w, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, c, false);
}

// ---- buffer loads with hardware range checking -----------------------------
// A raw buffer resource covers `bytes` bytes from `base`; a load whose byte
// offset lies at or beyond that size returns zeros and touches no memory,
// which replaces per-element bounds branches on ragged tails.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
constexpr int kBufFlags = 0x00020000;   // gfx9 raw-buffer dword 3 (32-bit data format)

__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, kBufFlags);
}
__device__ __forceinline__ u32x4 buf_load16(buf_rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_load8(buf_rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load4(buf_rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// The same loads with the non-temporal cache policy, for data read once per
// call (decode's K/V blocks and summaries): streamed reads reach ~10 % more
// HBM bandwidth on this part than loads that allocate normally.
constexpr int kCacheNT = 2;
__device__ __forceinline__ u32x4 buf_load16_nt(buf_rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCacheNT);
}
__device__ __forceinline__ u32x2 buf_load8_nt(buf_rsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCacheNT);
}

// a store at or beyond the resource's size is dropped
__device__ __forceinline__ void buf_store4(float v, buf_rsrc r, uint32_t off, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, soff, 0);
}

// ---- cross-lane exchange without LDS (DPP and gfx950 permlane swaps) -------
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ float dpp_src(float v, float old) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, BANK_MASK, false));
}
// (v of lane l & ~M, v of lane l | M) for M = 16 (v_permlane16_swap) or 32
// (v_permlane32_swap): the lower and upper partner of every lane
template <int M>
__device__ __forceinline__ void lane_pair(float v, float& lo, float& hi) {
  static_assert(M == 16 || M == 32, "permlane swaps exchange 16- or 32-lane halves");
  const unsigned iv = __builtin_bit_cast(unsigned, v);
  if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(iv, iv, false, false);
    lo = __builtin_bit_cast(float, (unsigned)r[0]);
    hi = __builtin_bit_cast(float, (unsigned)r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(iv, iv, false, false);
    lo = __builtin_bit_cast(float, (unsigned)r[0]);
    hi = __builtin_bit_cast(float, (unsigned)r[1]);
  }
}
// v of lane l ^ M (M a power of two below 64): DPP quad_perm for 1 and 2,
// row_shl / row_shr by 4 on alternate banks of four lanes for 4, row_ror by 8
// for 8, permlane swaps for 16 and 32
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (M == 1) return dpp_src<0xB1>(v, v);            // quad_perm [1,0,3,2]
  else if constexpr (M == 2) return dpp_src<0x4E>(v, v);       // quad_perm [2,3,0,1]
  else if constexpr (M == 4) {
    const float t = dpp_src<0x104, 0xF, 0x5>(v, v);           // banks 0, 2: lane + 4
    return dpp_src<0x114, 0xF, 0xA>(v, t);                     // banks 1, 3: lane - 4
  } else if constexpr (M == 8) return dpp_src<0x128>(v, v);    // row_ror:8
  else {
    float lo, hi;
    lane_pair<M>(v, lo, hi);
    return (__lane_id() & M) ? lo : hi;
  }
}
// op(v, v of lane l ^ M): both lanes of a pair get the same bits (op is
// commutative; for 16 and 32 the lower lane's value is always the left operand)
template <int M, typename Op>
__device__ __forceinline__ float xor_reduce(float v, Op op) {
  if constexpr (M >= 16) {
    float lo, hi;
    lane_pair<M>(v, lo, hi);
    return op(lo, hi);
  } else {
    return op(v, lane_xor<M>(v));
  }
}
// the same over aligned groups of `width` lanes (a power of two <= 64),
// partners at distance 1, 2, 4, ... in that order
template <typename Op>
__device__ __forceinline__ float group_reduce(float v, int width, Op op) {
  if (width > 1) v = xor_reduce<1>(v, op);
  if (width > 2) v = xor_reduce<2>(v, op);
  if (width > 4) v = xor_reduce<4>(v, op);
  if (width > 8) v = xor_reduce<8>(v, op);
  if (width > 16) v = xor_reduce<16>(v, op);
  if (width > 32) v = xor_reduce<32>(v, op);
  return v;
}
// lane_xor for a distance that is a compile-time constant after unrolling
__device__ __forceinline__ float lane_xor_c(float v, int m) {
  switch (m) {
    case 1: return lane_xor<1>(v);
    case 2: return lane_xor<2>(v);
    case 4: return lane_xor<4>(v);
    case 8: return lane_xor<8>(v);
    case 16: return lane_xor<16>(v);
    default: return lane_xor<32>(v);
  }
}
struct DppAdd { __device__ float operator()(float x, float y) const { return x + y; } };
struct DppMax { __device__ float operator()(float x, float y) const { return fmaxf(x, y); } };
struct DppMin { __device__ float operator()(float x, float y) const { return fminf(x, y); } };

// Wave-wide reductions on DPP and permlane swaps: every lane gets the same
// bits; for latency-bound code with few waves per SIMD.
__device__ __forceinline__ float wave_sum(float v) { return group_reduce(v, kWave, DppAdd{}); }
__device__ __forceinline__ float wave_max(float v) { return group_reduce(v, kWave, DppMax{}); }
__device__ __forceinline__ float wave_min(float v) { return group_reduce(v, kWave, DppMin{}); }

// Reductions over aligned groups of `width` lanes (a power of two <= 64)
// through LDS permutes (ds_bpermute): in kernels whose VALU is the busy unit
// these cost less than DPP chains, which add VALU work and wait states.
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float group_max(float v, int width) {
  for (int o = width >> 1; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float group_min(float v, int width) {
  for (int o = width >> 1; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}

// value of lane (l + N) mod 16 within lane l's row of 16 lanes (DPP row_ror);
// summing v, ror 8 and then ror 4 adds up the four lanes l mod 4 + 4 i of a row
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + N, 0xF, 0xF, false));
}

// ---- MFMA (gfx950) ------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16: A 16x32, B 32x16, C 16x16.  Lane l holds row
// (l % 16) of A / column (l % 16) of B with k = 8 * (l / 16) + [0, 8), and
// C[4 * (l / 16) + i][l % 16] in element i.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_32x32x16_bf16: A 32x16, B 16x32, C 32x32.  Lane l holds row
// (l % 32) of A / column (l % 32) of B with k = 8 * (l / 32) + [0, 8), and
// C[8 * (i / 4) + 4 * (l / 32) + i % 4][l % 32] in element i.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_4x4x1_16b_f32: 16 independent 4x4 products with k = 1.  Block
// b = l / 4; lane l holds A_b[l % 4] and B_b[l % 4], and C_b[i][l % 4] in
// element i.
__device__ __forceinline__ f32x4 mfma4x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace dash
