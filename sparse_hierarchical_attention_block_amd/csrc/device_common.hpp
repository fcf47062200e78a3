// device_common.hpp -- small device helpers shared by the gfx950 kernels of
// the DashAttention library: element types, wave64 reductions and MFMA
// fragment types.  Nothing here is used by the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dash {

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
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
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

// ---- wave64 reductions (fixed order, deterministic) -------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}
// Wave-wide reductions on DPP instead of LDS permutes: within each row of 16
// lanes (quad_perm 1,0,3,2 and 2,3,0,1, then half-row and row mirrors every
// lane holds its row's result), then row 0 into row 1 and row 2 into row 3
// (row_bcast:15), then lane 31 into rows 2 and 3 (row_bcast:31); lane 63 ends
// with the whole wave's result, which every lane reads.  Fixed order: all
// lanes get the same bits.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_src(float v, float old) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xF, false));
}
template <typename Op>
__device__ __forceinline__ float wave_reduce_dpp(float v, Op op, float ident) {
  v = op(v, dpp_src<0xB1>(v, ident));         // quad_perm [1,0,3,2]
  v = op(v, dpp_src<0x4E>(v, ident));         // quad_perm [2,3,0,1]
  v = op(v, dpp_src<0x141>(v, ident));        // row_half_mirror
  v = op(v, dpp_src<0x140>(v, ident));        // row_mirror
  v = op(v, dpp_src<0x142, 0xA>(v, ident));   // row_bcast:15 into rows 1 and 3
  v = op(v, dpp_src<0x143, 0xC>(v, ident));   // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
struct DppAdd { __device__ float operator()(float x, float y) const { return x + y; } };
struct DppMax { __device__ float operator()(float x, float y) const { return fmaxf(x, y); } };
struct DppMin { __device__ float operator()(float x, float y) const { return fminf(x, y); } };

// reductions over aligned groups of `width` lanes (width a power of two <= 64)
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
