// entmax_device.hpp -- alpha-entmax threshold on the GPU (Stage 1, "entmax
// chunk routing", DashAttention explainer: w = alpha-entmax(gamma * zbar),
// support size set by the scores).
//
// With inputs in threshold units x_j = (alpha - 1) gamma zbar_j, the
// probabilities are p_j = [x_j - tau]_+^e, e = 1/(alpha-1), where tau is the
// root of f(tau) = sum_j [x_j - tau]_+^e - 1, equivalently of
// phi(tau) = ||[x - tau]_+||_e - 1.  phi is convex and decreasing in tau (a
// norm, nondecreasing in each nonnegative argument, of convex decreasing
// functions), so Newton steps on phi started at tau0 = max_j x_j - 1 (where
// phi >= 0) stay left of the root and increase monotonically.  On a fixed
// support phi is close to linear (exactly linear when the support's values
// are equal), so these steps need fewer passes than Newton on f: with
// S_e = sum y^e and S_{e-1} = sum y^(e-1) over y = [x - tau]_+, the step is
// (S_e - S_e^(1 - 1/e)) / S_{e-1}.  For e = 2 (alpha = 1.5) and e = 1
// (alpha = 2) each pass also solves f = 0 exactly on the current support
// {x_j > tau}; that solution is accepted as soon as it keeps the whole
// support above it, which makes it the (unique) root.
#pragma once

#include "device_common.hpp"

namespace dash {

enum EntmaxMode : int { kSparsemax = 1, kEntmax15 = 2, kEntmaxQuartic = 4, kEntmaxGeneral = 0 };

__host__ __device__ inline int entmax_mode(float alpha) {
  if (alpha == 2.0f) return kSparsemax;
  if (alpha == 1.5f) return kEntmax15;
  if (alpha == 1.25f) return kEntmaxQuartic;
  return kEntmaxGeneral;
}

// Newton step on phi = (sum y^e)^(1/e) - 1 from se = sum y^e, se1 = sum y^(e-1)
__device__ __forceinline__ float entmax_norm_step(float se, float se1, int mode, float e) {
  float root;   // se^(1 - 1/e)
  if (mode == kEntmax15) root = sqrtf(se);
  else if (mode == kEntmaxQuartic) { const float r = sqrtf(se); root = r * sqrtf(r); }
  else root = exp2f((1.f - 1.f / e) * __log2f(se));
  return (se - root) / se1;
}

// y^e for y > 0
__device__ __forceinline__ float entmax_pow(float y, int mode, float e) {
  if (mode == kEntmax15) return y * y;
  if (mode == kSparsemax) return y;
  if (mode == kEntmaxQuartic) { float y2 = y * y; return y2 * y2; }
  return exp2f(e * __log2f(y));
}

// [y]_+^e for any y (0 at and below 0); MODE fixed at compile time
template <int MODE>
__device__ __forceinline__ float entmax_prob(float y, float e) {
  const float yp = fmaxf(y, 0.f);
  if constexpr (MODE == kSparsemax) return yp;
  else if constexpr (MODE == kEntmax15) return yp * yp;
  else if constexpr (MODE == kEntmaxQuartic) { const float y2 = yp * yp; return y2 * y2; }
  else return y > 0.f ? __builtin_amdgcn_exp2f(e * __builtin_amdgcn_logf(y)) : 0.f;
}

// The Stage 2 bias sigma * log(pbar) from sigma * ln 2 and pbar >= 0 (-inf at
// pbar = 0): the hardware log2, its argument held at or above the smallest
// normal float (a pbar below it, a weight under 1e-38 of the row's, gets the
// bias of 2^-126)
__device__ __forceinline__ float prior_bias(float pb, float sigma_ln2) {
  return pb > 0.f ? sigma_ln2 * __builtin_amdgcn_logf(fmaxf(pb, 1.17549435e-38f)) : -INFINITY;
}

// log(y^e) for y > 0
__device__ __forceinline__ float entmax_logpow(float y, int mode, float e) {
  float l = __logf(y);
  if (mode == kEntmax15) return 2.f * l;
  if (mode == kSparsemax) return l;
  if (mode == kEntmaxQuartic) return 4.f * l;
  return e * l;
}

// Threshold of one row whose n values are spread over a group of `width`
// consecutive lanes (lane `sub` of the group reads get(sub), get(sub+width),
// ...).  Every lane of the group returns the same tau.  `get(j)` reads x_j.
template <typename Get>
__device__ float entmax_tau(Get get, int n, int sub, int width, int mode, float e) {
  float xmax = -INFINITY;
  for (int j = sub; j < n; j += width) xmax = fmaxf(xmax, get(j));
  xmax = group_max(xmax, width);
  float tau = xmax - 1.0f;
  for (int it = 0; it < 64; ++it) {
    float k = 0.f, s1 = 0.f, s2 = 0.f, ymin = INFINITY;
    for (int j = sub; j < n; j += width) {
      float y = get(j) - tau;
      if (y > 0.f) {
        k += 1.f;
        ymin = fminf(ymin, y);
        if (mode == kEntmax15) { s1 += y; s2 = fmaf(y, y, s2); }
        else if (mode == kSparsemax) { s1 += y; }
        else if (mode == kEntmaxQuartic) { float y2 = y * y; s1 = fmaf(y2, y, s1); s2 = fmaf(y2, y2, s2); }
        else { float l = __log2f(y); s1 += exp2f((e - 1.f) * l); s2 += exp2f(e * l); }
      }
    }
    k = group_sum(k, width);
    s1 = group_sum(s1, width);
    s2 = group_sum(s2, width);
    ymin = group_min(ymin, width);
    float step;
    if (mode == kSparsemax) {
      // sum_S (y - d) = 1  ->  d = (s1 - 1) / k: Michelot's step, exact once S is the support
      step = (s1 - 1.f) / k;
      tau += step;
      if (step < ymin) break;
    } else if (mode == kEntmax15) {
      // sum_S (y - d)^2 = 1: k d^2 - 2 s1 d + (s2 - 1) = 0, smaller root in stable form
      float disc = s1 * s1 - k * (s2 - 1.f);
      if (disc >= 0.f) {
        float d = (s2 - 1.f) / (s1 + sqrtf(disc));
        if (d < ymin) { tau += d; break; }
      }
      step = entmax_norm_step(s2, s1, mode, e);
      tau += step;
      if (!(step > 1e-7f * fmaxf(1.f, fabsf(tau)))) break;
    } else {
      // s1 = sum y^(e-1), s2 = sum y^e
      step = entmax_norm_step(s2, s1, mode, e);
      tau += step;
      if (!(step > 1e-7f * fmaxf(1.f, fabsf(tau)))) break;
    }
  }
  return tau;
}

// Reductions over the lanes that hold one row.
struct GroupReduce {   // `width` consecutive lanes
  int width;
  __device__ float sum(float v) const { return group_sum(v, width); }
  __device__ float max(float v) const { return group_max(v, width); }
  __device__ float min(float v) const { return group_min(v, width); }
};
// Reductions over aligned groups of W consecutive lanes (W = 2 ... 16, known
// at compile time) on DPP within the lane's row of 16: quad_perm for
// partners 1 and 2, then the half-row and row mirrors (after the quad
// steps every lane of a quad holds the same value, so mirrored partners
// complete the group).  Every lane of a group gets the same bits.
template <int W>
struct DppGroupReduce {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16, "DPP group of 2..16 lanes");
  template <typename Op>
  __device__ static float run(float v, Op op) {
    v = op(v, dpp_src<0xB1>(v, v));
    if constexpr (W > 2) v = op(v, dpp_src<0x4E>(v, v));
    if constexpr (W > 4) v = op(v, dpp_src<0x141>(v, v));
    if constexpr (W > 8) v = op(v, dpp_src<0x140>(v, v));
    return v;
  }
  __device__ float sum(float v) const { return run(v, DppAdd{}); }
  __device__ float max(float v) const { return run(v, DppMax{}); }
  __device__ float min(float v) const { return run(v, DppMin{}); }
};
struct WaveReduce {   // all 64 lanes of the wave
  __device__ float sum(float v) const { return wave_sum(v); }
  __device__ float max(float v) const { return wave_max(v); }
  __device__ float min(float v) const { return wave_min(v); }
};
struct Stride16Reduce {   // lanes l, l^16, l^32, l^48 (one MFMA 16x16 C-fragment row)
  __device__ float sum(float v) const {
    v += __shfl_xor(v, 16, kWave);
    return v + __shfl_xor(v, 32, kWave);
  }
  __device__ float max(float v) const {
    v = fmaxf(v, __shfl_xor(v, 16, kWave));
    return fmaxf(v, __shfl_xor(v, 32, kWave));
  }
  __device__ float min(float v) const {
    v = fminf(v, __shfl_xor(v, 16, kWave));
    return fminf(v, __shfl_xor(v, 32, kWave));
  }
};

// Slot i of a row held in registers: a float array, or MFMA accumulator
// fragments of four (slot i is element i % 4 of fragment i / 4), read in
// place so that no copy of the accumulators is made.
template <int N>
__device__ __forceinline__ float xget(const float (&x)[N], int i) { return x[i]; }
template <int N>
__device__ __forceinline__ float xget(const f32x4 (&x)[N], int i) { return x[i >> 2][i & 3]; }
template <int N>
__device__ __forceinline__ void xset(float (&x)[N], int i, float v) { x[i] = v; }
template <int N>
__device__ __forceinline__ void xset(f32x4 (&x)[N], int i, float v) { x[i >> 2][i & 3] = v; }

// Support statistics of the register-held values at tau: count, s1, s2 and
// the smallest positive y = x - tau (MODE as in entmax_tau).  Only the first
// nact4 groups of four values are visited (nact4 is uniform across the wave,
// so the skipped groups cost no VALU, and the loop leaves at the first
// inactive group).
template <int VPL, int mode, typename XV>
__device__ __forceinline__ void entmax_accumulate(const XV& xv, float tau, float e,
                                                  int nact4, int& kc, float& s1, float& s2,
                                                  float& ymin) {
  kc = 0;
  s1 = 0.f;
  s2 = 0.f;
  ymin = INFINITY;
  static_for<0, VPL / 4>([&](auto G4) {
    constexpr int g4 = decltype(G4)::value;
    if (g4 < nact4) {   // the active groups come first
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const float y = xget(xv, 4 * g4 + ii) - tau;
        const bool in = y > 0.f;
        const float yp = fmaxf(y, 0.f);
        kc += in ? 1 : 0;
        // min(ymin, y over the support) as v_med3(z, ymin, -inf): no NaN
        // quieting of the loop-carried ymin as fminf would need
        ymin = __builtin_amdgcn_fmed3f(in ? y : INFINITY, ymin, -INFINITY);
        if constexpr (mode == kEntmax15) { s1 += yp; s2 = fmaf(yp, yp, s2); }
        else if constexpr (mode == kSparsemax) { s1 += yp; }
        else if constexpr (mode == kEntmaxQuartic) { const float y2 = yp * yp; s1 = fmaf(y2, yp, s1); s2 = fmaf(y2, y2, s2); }
        else if (in) { const float l = __log2f(y); s1 += exp2f((e - 1.f) * l); s2 += exp2f(e * l); }
      }
    }
  });
}

// One update of tau from the statistics of the row's support at tau (k, s1,
// s2, ymin as above); true once tau is final.  Sparsemax: Michelot's step,
// exact once the support is stable; alpha = 1.5: the closed-form root on the
// current support when it keeps the whole support above it, else a Newton
// step on the e-norm form; other alpha: the Newton step.
template <int mode>
__device__ __forceinline__ bool entmax_update(float k, float s1, float s2, float ymin, float e,
                                              float& tau) {
  if constexpr (mode == kSparsemax) {
    const float step = (s1 - 1.f) / k;
    tau += step;
    return step < ymin;
  } else if constexpr (mode == kEntmax15) {
    const float disc = s1 * s1 - k * (s2 - 1.f);
    if (disc >= 0.f) {
      const float d = (s2 - 1.f) / (s1 + sqrtf(disc));
      if (d < ymin) { tau += d; return true; }
    }
    const float step = entmax_norm_step(s2, s1, mode, e);
    tau += step;
    return !(step > 1e-7f * fmaxf(1.f, fabsf(tau)));
  } else {
    const float step = entmax_norm_step(s2, s1, mode, e);
    tau += step;
    return !(step > 1e-7f * fmaxf(1.f, fabsf(tau)));
  }
}

// sum y and sum y^2 over y = [x - tau]_+ of the register-held values: the
// two sums a Newton step on the e-norm form needs at alpha = 1.5.  Since tau
// starts at max x - 1 and only grows, y <= 1, so [x - tau]_+ is the clamp of
// x - tau to [0, 1], one subtraction with the clamp bit: three VALU
// instructions per value against seven and a half for the full statistics.
template <int VPL, typename XV>
__device__ __forceinline__ void entmax_sums15(const XV& xv, float tau, int nact4,
                                              float& s1, float& s2) {
  s1 = 0.f;
  s2 = 0.f;
  static_for<0, VPL / 4>([&](auto G4) {
    constexpr int g4 = decltype(G4)::value;
    if (g4 < nact4) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const float yp = fminf(fmaxf(xget(xv, 4 * g4 + ii) - tau, 0.f), 1.f);
        s1 += yp;
        s2 = fmaf(yp, yp, s2);
      }
    }
  });
}

// Steps above this fraction of max(1, |tau|) are taken from the two sums alone.
constexpr float kEntmaxSumsStop = 1e-2f;

// Same threshold with the row held in registers: each lane of the row's lane
// set holds VPL of its values (-inf for absent entries); `red` reduces over
// that lane set.  At alpha = 1.5 the first Newton steps use only the two sums;
// once a step falls below kEntmaxSumsStop the passes gather the full support
// statistics, so that the closed-form solve can end the search as before.
template <int VPL, int mode, typename XV, typename Red>
__device__ __forceinline__ float entmax_tau_reg(const XV& xv, Red red, float e, int nact4 = VPL / 4) {
  float xmax = -INFINITY;
  static_for<0, VPL / 4>([&](auto G4) {
    constexpr int g4 = decltype(G4)::value;
    if (g4 < nact4)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) xmax = fmaxf(xmax, xget(xv, 4 * g4 + ii));
  });
  xmax = red.max(xmax);
  float tau = xmax - 1.0f;
  int it = 0;
  if constexpr (mode == kEntmax15) {
    for (; it < 64; ++it) {
      float s1, s2;
      entmax_sums15<VPL>(xv, tau, nact4, s1, s2);
      s1 = red.sum(s1);
      s2 = red.sum(s2);
      const float step = entmax_norm_step(s2, s1, mode, e);
      tau += step;
      if (!(step > kEntmaxSumsStop * fmaxf(1.f, fabsf(tau)))) break;
    }
  }
  for (; it < 64; ++it) {
    int kc;
    float s1, s2, ymin;
    entmax_accumulate<VPL, mode>(xv, tau, e, nact4, kc, s1, s2, ymin);
    const float k = red.sum((float)kc);
    s1 = red.sum(s1);
    s2 = red.sum(s2);
    ymin = red.min(ymin);
    if (entmax_update<mode>(k, s1, s2, ymin, e, tau)) break;
  }
  return tau;
}

}  // namespace dash
