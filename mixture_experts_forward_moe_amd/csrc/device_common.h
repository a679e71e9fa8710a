// device_common.h -- gfx950 device helpers shared by the MoE kernels:
// vector types, bf16 / E4M3 / E8M0 / E2M1 conversions on CDNA4 conversion
// instructions, and the NVFP4 / MX block quantisers used by the GEMM1
// epilogue and the input quantisers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define DEV __device__ __forceinline__

// A wave-uniform load through the scalar cache.  Through the constant
// address space, so the compiler does not fall back to a vector load (whose
// wait would also wait for every other load in flight) when the kernel's
// stores might alias; only for values the kernel does not write.
template <typename T>
DEV T ld_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

DEV float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
DEV uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// E4M3 ("fn") code -> fp32, exact.  Codes 0x7f/0xff (NaN) are not produced by
// the quantisers and decode to 480 here.
DEV float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return (c & 0x80u) ? -mag : mag;
}

// E8M0 code as the fp32 whose exponent field is the code: exactly 2^(c-127)
// for c >= 1; c == 0 gives +0.0f, whose exponent field the CDNA4 scaled
// conversions read as 2^-127.
DEV float e8m0_scale_operand(uint32_t c) { return __uint_as_float(c << 23); }

// Eight packed E2M1 codes (one dword, element 0 in the low nibble) times an
// fp32 block scale, as eight bf16.  The product of an E2M1 value and an E4M3
// value has at most 6 significant bits, so the result is exact.
DEV bf16x8_t e2m1x8_scaled_to_bf16(uint32_t w, float scale) {
  f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  u32x4_t r;
  r[0] = pack_bf16x2(p0[0] * scale, p0[1] * scale);
  r[1] = pack_bf16x2(p1[0] * scale, p1[1] * scale);
  r[2] = pack_bf16x2(p2[0] * scale, p2[1] * scale);
  r[3] = pack_bf16x2(p3[0] * scale, p3[1] * scale);
  return __builtin_bit_cast(bf16x8_t, r);
}

// fp32 -> E2M1 code (4 bits), round to nearest even, saturating to +-6; the
// sign of a zero result follows the input.  Scale operand 1.0: no scaling.
DEV uint32_t f32_to_e2m1(float v) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, 0.0f, 1.0f, 0) & 15u;
}
// two values -> one byte (a low nibble, b high nibble), divided by the
// exponent of `scale` (a power of two or an E8M0 operand)
DEV uint32_t f32x2_to_e2m1x2(float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, scale, 0) & 0xffu;
}

// fp32 -> E4M3 code, round to nearest even, saturating to +-448 (the
// conversion itself does not saturate, so clamp first).
DEV uint32_t f32_to_e4m3_sat(float v) {
  v = fminf(fmaxf(v, -448.0f), 448.0f);
  i16x2_t z = {0, 0};
  i16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, v, 0.0f, 1.0f, false);
  return (uint32_t)(uint16_t)r[0] & 0xffu;
}

// x / 2^(code-127) -> E4M3, saturating: clamp to +-448 * 2^(code-127) first
DEV uint32_t f32x2_to_e4m3x2_mx(float a, float b, uint32_t code) {
  float lim = __builtin_ldexpf(448.0f, (int)code - 127);
  a = fminf(fmaxf(a, -lim), lim);
  b = fminf(fmaxf(b, -lim), lim);
  i16x2_t z = {0, 0};
  i16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a, b, e8m0_scale_operand(code), false);
  return (uint32_t)(uint16_t)r[0];
}

// NVFP4 block scale code for a block amax under global scale gs:
// E4M3(bamax / (6 gs)) decided in fp32; 0 when either is 0.
DEV uint32_t nvfp4_scale_code(float bamax, float gs) {
  if (!(gs > 0.0f) || !(bamax > 0.0f)) return 0u;
  float t = __fmul_rn(6.0f, gs);
  float s = __fdiv_rn(bamax, t);
  return f32_to_e4m3_sat(s);
}

// E2M1 code of v for a block with decoded scale sd under global scale gs:
// E2M1(v / (sd * gs)) in fp32; 0 when sd * gs == 0.
DEV uint32_t nvfp4_elem_code(float v, float sd, float gs) {
  float denom = __fmul_rn(sd, gs);
  if (!(denom > 0.0f)) return 0u;
  return f32_to_e2m1(__fdiv_rn(v, denom));
}

// MX shared-exponent code for a block amax (OCP MX v1.0): floor(log2 amax) -
// emax + 127 from the exponent bits, clamped to [0, 254]; 0 for amax == 0.
DEV uint32_t mx_scale_code(float amax, int emax) {
  int be = (int)((__float_as_uint(amax) >> 23) & 255u);
  if (be == 0) return 0u;  // zero or subnormal amax: clamps to 0
  int c = be - emax;
  return (uint32_t)(c < 0 ? 0 : (c > 254 ? 254 : c));
}

DEV float warp_max16(float v) {
  // max over the 16 lanes of a DPP row (lanes 16q .. 16q+15)
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  return v;
}

// SwiGLU with alpha / beta / limit on fp32 gate and up values:
// min(g, l) * sigmoid(a * min(g, l)) * (clamp(u, -l, l) + b).  The sigmoid
// uses the accurate expf and a correctly rounded divide, so y lands within
// about one fp32 ulp of the exact value before its single bf16 rounding.
DEV float swiglu_f32(float g, float u, float alpha, float beta, float limit) {
  float gc = fminf(g, limit);
  float uc = fminf(fmaxf(u, -limit), limit);
  float sig = 1.0f / (1.0f + expf(-alpha * gc));
  return gc * sig * (uc + beta);
}

// The gated FC1 activation ("flashinfer.fused_moe.cute_dsl_fused_moe",
// Parameters activation_type, swiglu_*, situ_beta, situ_linear_beta), one
// block of kernel arguments shared by every GEMM1 epilogue.
enum { ACT_SWIGLU = 0, ACT_GEGLU_TANH = 1, ACT_SITU = 2, ACT_RELU2 = 3 };
struct GateAct {
  int kind;                  // ACT_* (ACT_RELU2: non-gated, each W1 row is an output)
  float alpha, beta, limit;  // SwiGLU
  float situ_beta;           // SiTU gate: situ_beta * tanh(g / situ_beta) * sigmoid(g)
  float situ_lin;            // SiTU up-branch clamp situ_lin * tanh(u / situ_lin); 0 = none
};

// y = act(g, u) in fp32 with accurate expf / tanhf and correctly rounded
// divides, before the single bf16 rounding of y1.
//   SwiGLU: as above.  GeGLU-tanh: g/2 * (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))) * u.
//   SiTU: b tanh(g/b) sigmoid(g) * u', u' = u or c tanh(u/c).
DEV float gated_act_f32(float g, float u, const GateAct& p) {
  if (p.kind == ACT_GEGLU_TANH) {
    const float z = 0.7978845608028654f * (g + 0.044715f * g * g * g);
    return 0.5f * g * (1.0f + tanhf(z)) * u;
  }
  if (p.kind == ACT_SITU) {
    const float gate = p.situ_beta * tanhf(g / p.situ_beta) / (1.0f + expf(-g));
    const float up = p.situ_lin > 0.0f ? p.situ_lin * tanhf(u / p.situ_lin) : u;
    return gate * up;
  }
  return swiglu_f32(g, u, p.alpha, p.beta, p.limit);
}

// gated_act_f32 with the kind fixed at compile time (AK = ACT_SWIGLU,
// ACT_GEGLU_TANH or ACT_SITU): for epilogues unrolled over many elements,
// where carrying every kind's code per element would bloat them.
template <int AK>
DEV float gated_act_k(float g, float u, const GateAct& p) {
  if constexpr (AK == ACT_GEGLU_TANH) {
    const float z = 0.7978845608028654f * (g + 0.044715f * g * g * g);
    return 0.5f * g * (1.0f + tanhf(z)) * u;
  } else if constexpr (AK == ACT_SITU) {
    const float gate = p.situ_beta * tanhf(g / p.situ_beta) / (1.0f + expf(-g));
    const float up = p.situ_lin > 0.0f ? p.situ_lin * tanhf(u / p.situ_lin) : u;
    return gate * up;
  } else {
    return swiglu_f32(g, u, p.alpha, p.beta, p.limit);
  }
}

// ReLU^2 of one FC1 row (activation_type Relu2, non-gated): max(h, 0)^2.
DEV float relu2_f32(float h) {
  const float r = fmaxf(h, 0.0f);
  return r * r;
}
