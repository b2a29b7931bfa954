// Device-side building blocks for the gfx950 kernels of libqlin:
// number codecs (bf16, OCP E4M3, E4M3FNUZ, int8, int4 nibbles), wave and
// block reductions, and thin wrappers over the CDNA4 MFMA builtins.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlin {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round a finite fp32 to bf16, nearest even (integer form).
__device__ __forceinline__ uint32_t f32_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15) via the hardware
// converter (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  v2bf p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

// ---------------------------------------------------------------- FP8
// Encode |x| <= FMAX already clamped; sign handled here. Nearest even.
// OCP E4M3: exponent bias 7, smallest normal 2^-6, subnormal step 2^-9.
// E4M3FNUZ: bias 8, smallest normal 2^-7, subnormal step 2^-10, no -0.
template <bool FNUZ>
__device__ __forceinline__ uint32_t fp8_encode(float x) {
  constexpr float kMax = FNUZ ? 240.0f : 448.0f;
  constexpr float kMinNormal = FNUZ ? 0.0078125f : 0.015625f;  // 2^-7 / 2^-6
  constexpr float kSubScale = FNUZ ? 1024.0f : 512.0f;         // 1 / subnormal step
  constexpr uint32_t kRebias = (127u - (FNUZ ? 8u : 7u)) << 3;
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fminf(fabsf(x), kMax);
  uint32_t mag;
  if (a < kMinNormal) {
    mag = (uint32_t)__builtin_rintf(a * kSubScale);  // 0..8; 8 is the smallest normal
  } else {
    uint32_t v = __float_as_uint(a);
    v = (v + 0x7FFFFu + ((v >> 20) & 1u)) >> 20;  // keep 3 mantissa bits, nearest even
    mag = v - kRebias;
  }
  if (mag == 0) return FNUZ ? 0u : sign;
  return mag | sign;
}

// OCP E4M3 via the hardware converter (v_cvt_pk_fp8_f32) on a pre-clamped
// value; the clamp supplies saturation. Two values -> two bytes.
__device__ __forceinline__ uint32_t fp8_encode_hw2(float x0, float x1) {
  x0 = __builtin_fminf(__builtin_fmaxf(x0, -448.0f), 448.0f);
  x1 = __builtin_fminf(__builtin_fmaxf(x1, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false) & 0xFFFFu;
}

template <bool FNUZ>
__device__ __forceinline__ float fp8_decode(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (FNUZ) {
    v = (e == 0) ? (float)m * 0.0009765625f : __builtin_ldexpf((float)(8u + m), (int)e - 11);
  } else {
    v = (e == 0) ? (float)m * 0.001953125f : __builtin_ldexpf((float)(8u + m), (int)e - 10);
  }
  return (b & 0x80u) ? -v : v;
}

__device__ __forceinline__ int32_t int8_code(float v) {
  float r = __builtin_rintf(v);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int32_t)r;
}

// ---------------------------------------------------------------- int4
// Dequantise 8 nibbles (k = 0..7 at bits 4k) of one 32-bit word to bf16:
// w = bf16(c * step), c = u - 8. c*step is exact in fp32 (<= 12 significant
// bits), computed exactly by one fma as u*step + (-8*step).
__device__ __forceinline__ v8bf dequant8(uint32_t word, float step, float neg8step) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = __builtin_fmaf((float)((word >> (4 * i)) & 15u), step, neg8step);
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  v4i q = {(int)p[0], (int)p[1], (int)p[2], (int)p[3]};
  return __builtin_bit_cast(v8bf, q);
}

// The same dequantisation with fewer VALU operations (17 per word instead
// of 22): each pair of codes (k, k + 4) is placed into the mantissas of two
// fp16 numbers of exponent 10 (ulp 1), as 1024 + u for k = 0, 2 and as
// 1024 + 16u for k = 1, 3 (the nibble's position in its byte, no shift),
// and one mixed-precision fma per value (fp16 operand widened exactly)
// removes the offset and applies the step: (1024 + u) * step - 1032 * step
// and (1024 + 16u) * (step / 16) - 72 * step both equal c * step, which is
// exact, so the bf16 pack gives the single rounding. Values stay in the
// order k = 0..7. Valid for finite steps of magnitude below 2^117 (the
// offsets stay finite); step / 16 is exact down to the fp32 denormals.
struct Int4Step {
  float s, s16, off, off16;
};
__device__ __forceinline__ Int4Step int4_step(float step) {
  return Int4Step{step, step * 0.0625f, -1032.0f * step, -72.0f * step};
}
__device__ __forceinline__ float fma_mix_lo(uint32_t x, float a, float b) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(x), "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ float fma_mix_hi(uint32_t x, float a, float b) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(x), "v"(a), "v"(b));
  return d;
}
// (x & mask) | magic in one VALU operation (the compiler splits it in two
// when both constants are literals)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(x), "s"(mask), "v"(magic));
  return d;
}
__device__ __forceinline__ v8bf dequant8_mix(uint32_t word, const Int4Step& st) {
  constexpr uint32_t kMagic = 0x64006400u;  // fp16 1024.0 in both halves
  const uint32_t t = word >> 8;
  const uint32_t p0 = and_or(word, 0x000F000Fu, kMagic);  // k = 0, 4
  const uint32_t p1 = and_or(word, 0x00F000F0u, kMagic);  // k = 1, 5 (x16)
  const uint32_t p2 = and_or(t, 0x000F000Fu, kMagic);     // k = 2, 6
  const uint32_t p3 = and_or(t, 0x00F000F0u, kMagic);     // k = 3, 7 (x16)
  const float f0 = fma_mix_lo(p0, st.s, st.off), f4 = fma_mix_hi(p0, st.s, st.off);
  const float f1 = fma_mix_lo(p1, st.s16, st.off16), f5 = fma_mix_hi(p1, st.s16, st.off16);
  const float f2 = fma_mix_lo(p2, st.s, st.off), f6 = fma_mix_hi(p2, st.s, st.off);
  const float f3 = fma_mix_lo(p3, st.s16, st.off16), f7 = fma_mix_hi(p3, st.s16, st.off16);
  v4i q = {(int)pack_bf16x2(f0, f1), (int)pack_bf16x2(f2, f3), (int)pack_bf16x2(f4, f5), (int)pack_bf16x2(f6, f7)};
  return __builtin_bit_cast(v8bf, q);
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v |= __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ long long wave_sum_ll(long long v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Block-wide max over `nwaves` waves through a small LDS array.
template <int NWAVES>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NWAVES; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------- MFMA
// D = A*B + C on 16x16 tiles. Operand lane layout (all three): lane l holds
// row/column (l % 16) and K slice (l / 16); the output register i of lane l
// is D[4*(l/16) + i][l % 16]. The K order inside a lane is the same for A
// and B, so any consistent K permutation of both operands gives the same sum.
__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b, v4f c) {
  // f8f6f4 MFMA, both operands OCP E4M3 (type 0), unit E8M0 scales (127).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte global load / store helpers.
__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint4 ldg16_nt(const void* p) {
  const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

}  // namespace qlin
