// Per-token quantisation of one bf16 row by a workgroup: the scale rule, the
// division and the encoders shared by the quantiser kernels of
// qlin_quant.hip and the FP8 mixture-of-experts block's first stage
// (Gemma 4 31B-it FP8 model card: activations quantised to FP8 per token at
// run time).
#pragma once

#include "qlin_device.h"
#include "qlin_internal.h"

namespace qlin {

constexpr int kQThreads = 256;

// 8 fp32 values -> 8 code bytes (two 32-bit words).
template <int FMT>
__device__ __forceinline__ uint2 encode8(const float (&v)[8]) {
  uint32_t w[2];
  if (FMT == QLIN_E4M3) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      w[h] = fp8_encode_hw2(v[4 * h], v[4 * h + 1]) | (fp8_encode_hw2(v[4 * h + 2], v[4 * h + 3]) << 16);
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      w[h] = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t b = FMT == QLIN_INT8 ? ((uint32_t)int8_code(v[4 * h + i]) & 0xFFu)
                                      : fp8_encode<true>(v[4 * h + i]);
        w[h] |= b << (8 * i);
      }
    }
  }
  return make_uint2(w[0], w[1]);
}

// a / s for every value a of a bf16 row whose scale is s = absmax / FMAX
// (absmax a bf16 value, s > 0): the reciprocal quotient with one fused
// multiply-add correction (Markstein's correction of a reciprocal quotient:
// q0 = a*y with y = RN(1/s), r = a - q0*s by an fma, q = q0 + r*y by an
// fma), with a's sign copied onto q so that a zero keeps its sign. For
// s >= 2^-100 it is the IEEE quotient bit for bit wherever either is at
// least 2^-12 in magnitude, and below that both encode to a zero of a's
// sign in every format: an exhaustive check over every positive finite bf16
// absmax, FMAX 448, 240 and 127, and every bf16 a with |a| <= absmax shows it
// (3.1e9 pairs). Rows of a smaller scale, where the remainder can fall among
// the fp32 subnormals, divide.
struct RowScale {
  float s, y;
  bool fast;
};
__device__ __forceinline__ RowScale row_scale(float sc) {
  RowScale r;
  r.s = sc;
  r.y = 1.0f / sc;
  r.fast = sc >= 0x1p-100f && __builtin_isfinite(r.y);
  return r;
}
__device__ __forceinline__ void divide8(float (&v)[8], const RowScale& rs) {
  if (rs.fast) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q0 = v[i] * rs.y;
      v[i] = copysignf(fmaf(fmaf(-q0, rs.s, v[i]), rs.y, q0), v[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = v[i] / rs.s;
  }
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& x, float (&v)[8]) {
  const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(xs[i] << 16);
    v[2 * i + 1] = __uint_as_float(xs[i] & 0xFFFF0000u);
  }
}

// CMAX > 0: the row (K/8 chunks of 8 bf16) is held in registers, CMAX chunks
// per lane. CMAX == 0: two passes over global memory (rows longer than
// 16384 elements). Row m of a is quantised by the whole workgroup (kQThreads
// threads; red: kQThreads / 64 floats of LDS).
template <int FMT, int CMAX>
__device__ __forceinline__ void quant_row(const uint16_t* __restrict__ a, int64_t K, int64_t lda,
                                          uint8_t* __restrict__ q, float* __restrict__ s, int64_t m,
                                          float* red) {
  const uint16_t* row = a + m * lda;
  uint8_t* qrow = q + m * K;
  const int chunks = (int)(K / 8);
  constexpr float kFmax = FMT == QLIN_INT8 ? 127.0f : (FMT == QLIN_E4M3FNUZ ? 240.0f : 448.0f);
  float amax = 0.0f;
  if (CMAX > 0) {
    uint4 cache[CMAX > 0 ? CMAX : 1];
#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
      const int idx = threadIdx.x + c * kQThreads;
      // rows above 8192 elements stream nontemporally (read once; K=14336,
      // M=8192: 58.7 instead of 65.7 us); shorter ones measured slower so
      // (K=4096: 20.7 instead of 17.4 us)
      const uint16_t* src = row + (int64_t)idx * 8;
      cache[c] = idx < chunks ? (CMAX >= 8 ? ldg16_nt(src) : ldg16(src)) : make_uint4(0, 0, 0, 0);
      float v[8];
      unpack_bf16x8(cache[c], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = block_max<kQThreads / 64>(amax, red);
    const float sc = amax > 0.0f ? amax / kFmax : 0.0f;
    const RowScale rs = row_scale(sc);
#pragma unroll
    for (int c = 0; c < CMAX; ++c) {
      const int idx = threadIdx.x + c * kQThreads;
      if (idx < chunks) {
        uint2 out = make_uint2(0, 0);
        if (sc > 0.0f) {
          float v[8];
          unpack_bf16x8(cache[c], v);
          divide8(v, rs);
          out = encode8<FMT>(v);
        }
        *reinterpret_cast<uint2*>(qrow + (int64_t)idx * 8) = out;
      }
    }
    if (threadIdx.x == 0) s[m] = sc;
  } else {
    for (int idx = threadIdx.x; idx < chunks; idx += kQThreads) {
      float v[8];
      unpack_bf16x8(ldg16(row + (int64_t)idx * 8), v);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = block_max<kQThreads / 64>(amax, red);
    const float sc = amax > 0.0f ? amax / kFmax : 0.0f;
    const RowScale rs = row_scale(sc);
    for (int idx = threadIdx.x; idx < chunks; idx += kQThreads) {
      uint2 out = make_uint2(0, 0);
      if (sc > 0.0f) {
        float v[8];
        unpack_bf16x8(ldg16(row + (int64_t)idx * 8), v);
        divide8(v, rs);
        out = encode8<FMT>(v);
      }
      *reinterpret_cast<uint2*>(qrow + (int64_t)idx * 8) = out;
    }
    if (threadIdx.x == 0) s[m] = sc;
  }
}


}  // namespace qlin
