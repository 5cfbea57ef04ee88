// Device-side helpers shared by the libeqlinear kernels (gfx950 / CDNA4).
//
// The p4 group DFT used throughout ("Specializzazione per il Gruppo di
// Rotazione p4", Flash EQ-Linear gist.science summary: the length-4 DFT and
// its inverse only need additions, subtractions and power-of-two scalings).
// With omega = exp(-2*pi*i/4) = -i and X[k] = sum_s x[s] omega^(k s):
//     X0 = (x0 + x2) + (x1 + x3)     X2 = (x0 + x2) - (x1 + x3)
//     X1 = Xr + i Xi,  Xr = x0 - x2, Xi = x3 - x1,   X3 = conj(X1)
// and the inverse, written with the kept frequencies only (conjugate
// symmetry of the real DFT, "Approccio Algoritmico"):
//     y0 = (Y0 + Y2)/4 + Yr/2        y1 = (Y0 - Y2)/4 - Yi/2
//     y2 = (Y0 + Y2)/4 - Yr/2        y3 = (Y0 - Y2)/4 + Yi/2
//
// Scaled planes.  Every spectral plane the kernels store is the coefficient
// above times a power of two that bounds it by the largest input magnitude:
// X0 and X2 by 1/4 (|X0|, |X2| <= 4 max|x|), Xr and Xi by 1/2 (|Xr|, |Xi| <=
// 2 max|x|).  So no binary16 plane overflows while its inputs are finite, and
// the layer keeps the input range of the dense fp16-in, fp32-accumulate layer
// it replaces.  Both operands of every product carry the scaling (input planes
// and weight spectra; upstream-gradient planes and input planes in the weight
// gradient), so a product is 1/16 (frequencies 0 and 2) or 1/4 (frequency 1)
// of the unscaled one, and the inverse takes the factors 4 and 2 in place of
// 1/4 and 1/2.  All of these scalings are exact in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eql {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Plane scalings of the forward transform and factors of the inverse.
constexpr float SCALE02 = 0.25f, SCALE1 = 0.5f;
constexpr float INV02 = 4.0f, INV1 = 2.0f;

// Forward length-4 butterfly on one group vector (fp32 arithmetic), scaled
// planes: f0 = X0/4, f2 = X2/4, fr = Xr/2, fi = Xi/2.
struct Spec4 {
  float f0, f2, fr, fi;
};

__device__ __forceinline__ Spec4 dft4(float x0, float x1, float x2, float x3) {
  const float s02 = x0 + x2, s13 = x1 + x3;
  Spec4 s;
  s.f0 = (s02 + s13) * SCALE02;
  s.f2 = (s02 - s13) * SCALE02;
  s.fr = (x0 - x2) * SCALE1;
  s.fi = (x3 - x1) * SCALE1;
  return s;
}

// Inverse length-4 butterfly, fp32, of products of two scaled operands:
// factors 4 and 2 (exact).
__device__ __forceinline__ floatx4 idft4(float Q0, float Q2, float Qr, float Qi) {
  const float a = INV02 * (Q0 + Q2), b = INV02 * (Q0 - Q2);
  const float r = INV1 * Qr, i = INV1 * Qi;
  floatx4 o;
  o[0] = a + r;
  o[1] = b - i;
  o[2] = a - r;
  o[3] = b + i;
  return o;
}

// Inverse with the bias of the output channel (forward epilogues):
// y = 4 (Q0 +- Q2) +- 2 Qr|Qi + b as fused multiply-adds.
__device__ __forceinline__ floatx4 idft4_bias(float Q0, float Q2, float Qr, float Qi, float b) {
  const float u = __builtin_fmaf(Q0, INV02, b);
  const float p = __builtin_fmaf(Q2, INV02, u);   // 4 (Q0 + Q2) + b
  const float m = __builtin_fmaf(Q2, -INV02, u);  // 4 (Q0 - Q2) + b
  floatx4 o;
  o[0] = __builtin_fmaf(Qr, INV1, p);
  o[1] = __builtin_fmaf(Qi, -INV1, m);
  o[2] = __builtin_fmaf(Qr, -INV1, p);
  o[3] = __builtin_fmaf(Qi, INV1, m);
  return o;
}

typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));

// Packed binary16 (Xr/2, -Xi/2) of one group vector held as the pairs
// a01 = (x0, x1), a23 = (x2, x3): (x0 - x2)/2 and (x1 - x3)/2 with one
// rounding each (the halving of a23 is exact for normal values), and no
// overflow for finite inputs.
__device__ __forceinline__ f16x2v half_diff(f16x2v a01, f16x2v a23) {
  const f16x2v h = {(_Float16)SCALE1, (_Float16)SCALE1};
  return __builtin_elementwise_fma(a01, h, a23 * -h);
}

// Binary16 value of v/4 (v in fp32, one rounding)
__device__ __forceinline__ _Float16 quarter_h(float v) {
  return (_Float16)__builtin_fmaf(v, SCALE02, 0.0f);
}

// ---- pointwise activation of the forward epilogue ---------------------------
// Applied after the bias, in fp32, before the rounding to the output dtype.
// It acts on each output value alone, so it commutes with the group action
// and the layer stays equivariant.
//   1: GELU, v * Phi(v) = (v/2) (1 + erf(v / sqrt 2))
//   2: GELU with the tanh approximation,
//      (v/2) (1 + tanh(s)) = v / (1 + exp(-2 s)),  s = sqrt(2/pi) (v + 0.044715 v^3)
// Both are evaluated with the hardware base-2 exponential and reciprocal
// (about 1 ulp each); erf uses formula 7.1.26 of Abramowitz and Stegun,
// Handbook of Mathematical Functions (absolute error <= 1.5e-7):
//   erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),
//   t = 1 / (1 + p z), z >= 0, and erf(-z) = -erf(z).
// The epilogue runs on few waves, so a short instruction sequence matters.
constexpr int ACT_NONE = 0, ACT_GELU = 1, ACT_GELU_TANH = 2;

__device__ __forceinline__ float erf_as(float z) {
  const float a = __builtin_fabsf(z);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, a, 1.0f));
  float q = __builtin_fmaf(1.061405429f, t, -1.453152027f);
  q = __builtin_fmaf(q, t, 1.421413741f);
  q = __builtin_fmaf(q, t, -0.284496736f);
  q = __builtin_fmaf(q, t, 0.254829592f);
  q *= t;
  // exp(-a^2) = 2^(-a^2 log2 e)
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * a * a);
  const float r = __builtin_fmaf(-q, e, 1.0f);
  return __builtin_copysignf(r, z);
}

// The activation with its kind fixed at compile time (no branch).
template <int AK>
__device__ __forceinline__ float activate_k(float v) {
  if constexpr (AK == ACT_GELU) {
    return 0.5f * v * (1.0f + erf_as(v * 0.70710678118654752f));
  } else if constexpr (AK == ACT_GELU_TANH) {
    const float k1 = -2.3022082f, k2 = -0.10294324f;
    const float e = __builtin_amdgcn_exp2f(v * __builtin_fmaf(k2, v * v, k1));
    return v * __builtin_amdgcn_rcpf(1.0f + e);
  } else {
    return v;
  }
}

__device__ __forceinline__ float activate(float v, int act) {
  if (act == ACT_GELU) return 0.5f * v * (1.0f + erf_as(v * 0.70710678118654752f));
  if (act == ACT_GELU_TANH) {
    // -2 s log2(e) = v (k1 + k2 v^2), k1 = -2 sqrt(2/pi) log2 e, k2 = 0.044715 k1
    const float k1 = -2.3022082f, k2 = -0.10294324f;
    const float e = __builtin_amdgcn_exp2f(v * __builtin_fmaf(k2, v * v, k1));
    return v * __builtin_amdgcn_rcpf(1.0f + e);
  }
  return v;
}

// ---- element type traits ---------------------------------------------------
// Loads/stores of one group quad (4 elements of the type) and conversions.
template <typename T>
struct Elem;

template <>
struct Elem<float> {
  typedef floatx4 quad;  // 16 B
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
  static __device__ __forceinline__ quad pack(floatx4 v) { return v; }
  static __device__ __forceinline__ floatx4 unpack(quad q) { return q; }
};

template <>
struct Elem<_Float16> {
  typedef half4 quad;  // 8 B
  static __device__ __forceinline__ float to_f(_Float16 v) { return (float)v; }
  static __device__ __forceinline__ _Float16 from_f(float v) { return (_Float16)v; }
  static __device__ __forceinline__ quad pack(floatx4 v) {
    quad q;
    q[0] = (_Float16)v[0];
    q[1] = (_Float16)v[1];
    q[2] = (_Float16)v[2];
    q[3] = (_Float16)v[3];
    return q;
  }
  static __device__ __forceinline__ floatx4 unpack(quad q) {
    floatx4 v;
    v[0] = (float)q[0];
    v[1] = (float)q[1];
    v[2] = (float)q[2];
    v[3] = (float)q[3];
    return v;
  }
};

// ---- matrix-core step ------------------------------------------------------
// One 32x32 output block, fp32 accumulate.  Operand lane layout (checked on
// gfx950): lane l holds row/column (l % 32) and the k slice owned by lane
// group h = l / 32; the result register r of lane l is row
// 8*(r/4) + 4*h + (r%4), column l % 32.
//   binary16: v_mfma_f32_32x32x16_f16, 8 consecutive k per lane
//   binary32: v_mfma_f32_32x32x2_f32,  1 k per lane
template <typename T>
struct Mma;

template <>
struct Mma<_Float16> {
  typedef half8 frag;
  static constexpr int K_PER_LANE = 8;   // k values one lane feeds per step
  static constexpr int K_STEP = 16;      // k values per instruction
  static __device__ __forceinline__ floatx16 mma(frag a, frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma<float> {
  typedef float frag;
  static constexpr int K_PER_LANE = 1;
  static constexpr int K_STEP = 2;
  static __device__ __forceinline__ floatx16 mma(frag a, frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

}  // namespace eql
