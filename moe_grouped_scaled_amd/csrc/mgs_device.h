// Device helpers shared by the gfx950 kernels: BF16 access, block codecs on hardware converts,
// wavefront reductions over DPP, and the scaled activation functors.
//
// Everything here follows IEEE FP32 with round-to-nearest-even and is compiled with FP contraction
// off, so a functor evaluated in two different kernels gives identical bits (the recompute path
// regenerates the forward's quantized activation and must match it byte for byte).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mgs_internal.h"

namespace mgs {

// ------------------------------------------------------------------------------------------ BF16

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// FP32 -> BF16 pairs with the gfx950 convert: round to nearest, ties to even, subnormals kept (checked
// against the integer definition over all special classes and a million random patterns); a NaN
// stays a quiet NaN, its payload is whatever the hardware keeps.  Low half = first value.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ void unpack8(const uint4& w, float* v) {
  v[0] = bf16lo(w.x); v[1] = bf16hi(w.x); v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
  v[4] = bf16lo(w.z); v[5] = bf16hi(w.z); v[6] = bf16lo(w.w); v[7] = bf16hi(w.w);
}

__device__ __forceinline__ uint4 pack8_bf16(const float* v) {
  uint4 r;
  r.x = bf16x2(v[0], v[1]);
  r.y = bf16x2(v[2], v[3]);
  r.z = bf16x2(v[4], v[5]);
  r.w = bf16x2(v[6], v[7]);
  return r;
}

// ------------------------------------------------------------------------------------------ DPP

// quad_perm / row_ror controls of the DPP modifier (GCN3+ encoding)
constexpr int DPP_QUAD_XOR1 = 0xB1;  // [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;  // [2,3,0,1]
constexpr int DPP_ROW_ROR4 = 0x124;  // rotate right by 4 within each 16-lane row
constexpr int DPP_ROW_ROR8 = 0x128;  // rotate right by 8 within each 16-lane row

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// The lane maxima below are taken over block maxima of magnitudes (non-negative FP32 values), whose
// bit patterns order like unsigned integers: an integer maximum needs none of the NaN-quieting copies
// the compiler puts before a float maximum of a value it cannot prove canonical (a DPP result).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Lane exchanges of gfx950 (VALU, no LDS).  swap16(a, b): lanes of even 16-lane rows get
// (a[l], a[l + 16]), lanes of odd rows (b[l - 16], b[l]); swap32(a, b): lanes 0..31 get (a[l], a[l + 32]),
// lanes 32..63 (b[l - 32], b[l]) (measured on the device).
struct U2 { uint32_t x, y; };
__device__ __forceinline__ U2 swap16(uint32_t a, uint32_t b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  return U2{r[0], r[1]};
}
__device__ __forceinline__ U2 swap32(uint32_t a, uint32_t b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return U2{r[0], r[1]};
}

// max over the 4 lanes of a quad (v >= 0)
__device__ __forceinline__ float quad_max(float v) {
  uint32_t u = __float_as_uint(v);
  u = umax(u, dpp_u<DPP_QUAD_XOR1>(u));
  return __uint_as_float(umax(u, dpp_u<DPP_QUAD_XOR2>(u)));
}
// max over the 2 lanes (l, l^1) (v >= 0)
__device__ __forceinline__ float pair1_max(float v) {
  const uint32_t u = __float_as_uint(v);
  return __uint_as_float(umax(u, dpp_u<DPP_QUAD_XOR1>(u)));
}
// max over the 4 lanes {l mod 4 + 4k} of each 16-lane row (v >= 0)
__device__ __forceinline__ float row4_max(float v) {
  uint32_t u = __float_as_uint(v);
  u = umax(u, dpp_u<DPP_ROW_ROR4>(u));
  return __uint_as_float(umax(u, dpp_u<DPP_ROW_ROR8>(u)));
}
// max over the 2 lanes (l, l^4) (v >= 0)
__device__ __forceinline__ float pair4_max(float v) {
  const uint32_t u = __float_as_uint(v);
  return __uint_as_float(umax(u, (uint32_t)__shfl_xor((int)u, 4)));
}

// relu(x) = max(x, +0) on the bit pattern: negative values (sign bit set, negative as integers),
// -0 included, give +0.  No NaN-quieting copy is needed, unlike a float maximum of an unpacked BF16
// value.
__device__ __forceinline__ float relu(float x) {
  const int b = __float_as_int(x);
  return __int_as_float(b > 0 ? b : 0);
}

// ------------------------------------------------------------------------------------------ MXFP8

// E8M0 scale code of a block with maximum magnitude `amax` (>= 0, finite):
// clamp(floor(log2 amax) - 8 + 127, 0, 254), 0 for amax == 0.  For a normal FP32 amax the biased
// exponent field is floor(log2 amax) + 127; a zero or subnormal amax has field 0 and clamps to 0.
__device__ __forceinline__ uint32_t mx_scale_code(float amax) {
  int e = (int)(__float_as_uint(amax) >> 23);
  return (uint32_t)(e > 8 ? e - 8 : 0);
}

// The block scale 2^(code - 127) as an FP32 number (the subnormal 2^-127 for code 0), code in [0, 246]
__device__ __forceinline__ float mx_scale_value(uint32_t code) {
  return __builtin_amdgcn_ldexpf(1.0f, (int)code - 127);
}

// max |v_i| of eight values, as three-input maxima
__device__ __forceinline__ float absmax8(const float (&v)[8]) {
  float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fabsf(v[2]));
  m = fmaxf(fmaxf(m, fabsf(v[3])), fabsf(v[4]));
  m = fmaxf(fmaxf(m, fabsf(v[5])), fabsf(v[6]));
  return fmaxf(m, fabsf(v[7]));
}

// four FP32 values -> four E4M3 codes of value / s (byte i = value i), s = 2^(code - 127) the block
// scale, RNE, saturating at +-448.  The gfx950 scaled convert divides by the power of two s exactly and
// rounds to nearest-even, but does not saturate (beyond 448 it gives the NaN code), so the values are
// clamped to +-448 s first (`bound` = 448 s, exact).  Checked on the device for every scale code 0..246
// over 2^20 values each: bit for bit the codes of clamping value * 2^(127 - code) at +-448 and
// converting with the unscaled convert.
typedef short mgs_v2s __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e4m3x4_scaled(float a, float b, float c, float d, float s, float bound) {
  a = __builtin_amdgcn_fmed3f(a, -bound, bound);
  b = __builtin_amdgcn_fmed3f(b, -bound, bound);
  c = __builtin_amdgcn_fmed3f(c, -bound, bound);
  d = __builtin_amdgcn_fmed3f(d, -bound, bound);
  mgs_v2s w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, s, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, s, true);
  return __builtin_bit_cast(uint32_t, w);
}

// MXFP8 encode of the eight values a lane holds of one 32-element block whose maximum magnitude is
// `amax`: the E8M0 scale code, and the eight E4M3 codes (value 2k in byte k % 4 of dword k / 4)
struct Mx8 {
  uint32_t code;
  uint2 q;
};
__device__ __forceinline__ Mx8 mx_encode8(const float (&v)[8], float amax) {
  Mx8 r;
  r.code = mx_scale_code(amax);
  const float s = mx_scale_value(r.code), bound = 448.0f * s;
  r.q.x = e4m3x4_scaled(v[0], v[1], v[2], v[3], s, bound);
  r.q.y = e4m3x4_scaled(v[4], v[5], v[6], v[7], s, bound);
  return r;
}

// E4M3 code of one non-negative value (RNE, saturating)
__device__ __forceinline__ uint32_t e4m3_pos(float a) {
  a = __builtin_amdgcn_fmed3f(a, 0.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, 0.0f, 0, false) & 0xffu;
}

// exact value of a non-negative E4M3 code (0..126)
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

// ------------------------------------------------------------------------------------------ NVFP4

// eight FP32 values -> eight E2M1 codes packed in a dword (value 2i in the low nibble of byte i),
// RNE, saturating at +-6 (the gfx950 convert with a unit scale).
__device__ __forceinline__ uint32_t e2m1x8(const float* v) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// per-group encode scale from the group amax: 2688 / amax (1 for amax == 0, FLT_MAX on overflow)
__device__ __forceinline__ float nv_encode_scale(float amax) {
  if (amax == 0.0f) return 1.0f;
  float s = 2688.0f / amax;
  return (__float_as_uint(s) & 0x7fffffffu) == 0x7f800000u ? 3.40282347e+38f : s;
}

struct NvBlock {
  uint32_t code;  // E4M3 block scale code
  float r;        // element multiplier S_enc / s_b (0 when s_b == 0)
};

__device__ __forceinline__ NvBlock nv_block(float amax_b, float s_enc) {
  NvBlock b;
  float sf = (amax_b / 6.0f) * s_enc;
  b.code = e4m3_pos(sf);
  float d = e4m3_value(b.code);
  b.r = d != 0.0f ? s_enc / d : 0.0f;
  return b;
}

// ------------------------------------------------------------------------------------------ acts

struct ActArgs {
  int kind;
  float s, inv_s, limit, alpha, beta;
};

__device__ __forceinline__ float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// tanh(z) for z >= 0 (TanhSReLU's argument relu(x) / s), cheaper than the general library call:
// below 0.25 the odd Maclaurin series of tanh to z^11 (the first omitted term, 21844/6081075 z^13, is
// under 6e-11 relative there); from 0.25 up (1 - e) / (1 + e) with e = exp(-2 z), whose cancellation
// error stays under ~3e-7 relative.  Both are evaluated and one is selected (no divergence).
__device__ __forceinline__ float tanh_nonneg(float z) {
  const float z2 = z * z;
  float p = -1382.0f / 155925.0f;
  p = p * z2 + 62.0f / 2835.0f;
  p = p * z2 - 17.0f / 315.0f;
  p = p * z2 + 2.0f / 15.0f;
  p = p * z2 - 1.0f / 3.0f;
  const float small = z + z * (z2 * p);
  const float e = __expf(-2.0f * z);
  const float large = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
  return z < 0.25f ? small : large;
}

constexpr float INV_SQRT2 = 0.70710678118654752f;    // 1 / sqrt(2)
constexpr float INV_SQRT2PI = 0.39894228040143268f;  // 1 / sqrt(2 pi)

// a(x) for unary kinds
template <int KIND>
__device__ __forceinline__ float act_unary(float x, const ActArgs& aa) {
  if constexpr (KIND == MGS_ACT_IDENTITY) {
    return x;
  } else if constexpr (KIND == MGS_ACT_SRELU) {
    const float r = relu(x);
    return r * r;
  } else if constexpr (KIND == MGS_ACT_GELU) {
    return 0.5f * x * (1.0f + erff(x * INV_SQRT2));
  } else if constexpr (KIND == MGS_ACT_SIGMOID) {
    return sigmoidf_(x);
  } else {
    const float r = relu(x);
    float t = aa.s * tanh_nonneg(r * aa.inv_s);
    return t * t;
  }
}

// da/dx for unary kinds
template <int KIND>
__device__ __forceinline__ float dact_unary(float x, const ActArgs& aa) {
  if constexpr (KIND == MGS_ACT_IDENTITY) {
    return 1.0f;
  } else if constexpr (KIND == MGS_ACT_SRELU) {
    const float r = relu(x);
    return r + r;
  } else if constexpr (KIND == MGS_ACT_GELU) {
    // Phi(x) + x phi(x)
    return 0.5f * (1.0f + erff(x * INV_SQRT2)) + x * (INV_SQRT2PI * __expf(-0.5f * x * x));
  } else if constexpr (KIND == MGS_ACT_SIGMOID) {
    float sg = sigmoidf_(x);
    return sg * (1.0f - sg);
  } else {
    const float r = relu(x);
    float t = tanh_nonneg(r * aa.inv_s);
    float d = (aa.s + aa.s) * t * (1.0f - t * t);
    return x > 0.0f ? d : 0.0f;
  }
}

// a(gate, up) for gated kinds
template <int KIND>
__device__ __forceinline__ float act_gated(float g, float u, const ActArgs& aa) {
  if constexpr (KIND == MGS_ACT_SWIGLU) {
    return g * sigmoidf_(g) * u;
  } else if constexpr (KIND == MGS_ACT_GLU) {
    return sigmoidf_(g) * u;
  } else {
    float gc = fminf(g, aa.limit);
    float uc = fminf(fmaxf(u, -aa.limit), aa.limit);
    return gc * sigmoidf_(aa.alpha * gc) * (uc + aa.beta);
  }
}

// (a, da/dgate, da/dup) for gated kinds
template <int KIND>
__device__ __forceinline__ void dact_gated(float g, float u, const ActArgs& aa, float& a, float& dg,
                                           float& du) {
  if constexpr (KIND == MGS_ACT_SWIGLU) {
    float sg = sigmoidf_(g);
    float silu = g * sg;
    a = silu * u;
    dg = u * sg * (1.0f + g * (1.0f - sg));
    du = silu;
  } else if constexpr (KIND == MGS_ACT_GLU) {
    float sg = sigmoidf_(g);
    a = sg * u;
    dg = u * (sg * (1.0f - sg));
    du = sg;
  } else {
    float gc = fminf(g, aa.limit);
    float uc = fminf(fmaxf(u, -aa.limit), aa.limit);
    float sg = sigmoidf_(aa.alpha * gc);
    float silu = gc * sg;
    float up = uc + aa.beta;
    a = silu * up;
    dg = g <= aa.limit ? up * sg * (1.0f + aa.alpha * gc * (1.0f - sg)) : 0.0f;
    du = (u >= -aa.limit && u <= aa.limit) ? silu : 0.0f;
  }
}

}  // namespace mgs
