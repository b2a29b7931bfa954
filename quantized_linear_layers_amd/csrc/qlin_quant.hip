// Dynamic per-token activation quantisation for gfx950 (Gemma 4 31B-it FP8
// model card: activations quantised to FP8 per token at run time; "Gemma 4
// From E2B to 31B" article, format table: int8 activations per token).
//   s = max_k |a| / FMAX   (FMAX 448 for OCP E4M3, 127 for int8)
//   q = nearest-even E4M3 code of a / s (saturating)  or  clamp(rint(a/s)).
// Many rows of up to 2048 elements: one wave per row; otherwise one
// workgroup per row. The row is read once into registers (up to 16384
// elements), reduced to its absmax, then encoded and written.
#include "qlin_device.h"
#include "qlin_internal.h"
#include "qlin_quant_row.h"

namespace qlin {

template <int FMT, int CMAX>
__global__ __launch_bounds__(kQThreads) void quant_act_kernel(const uint16_t* __restrict__ a,
                                                              int64_t K, int64_t lda,
                                                              uint8_t* __restrict__ q,
                                                              float* __restrict__ s) {
  __shared__ float red[kQThreads / 64];
  quant_row<FMT, CMAX>(a, K, lda, q, s, blockIdx.x, red);
}

// Rows of at most 2048 elements: one wave per row (four rows per
// workgroup), CPL 16-byte chunks per lane held in registers, the absmax
// reduced within the wave (no LDS, no barrier). The same absmax, scale and
// encoder as above, so the same codes.
template <int FMT, int CPL>
__global__ __launch_bounds__(256) void quant_rows_wave_kernel(const uint16_t* __restrict__ a, int64_t M,
                                                              int64_t K, int64_t lda,
                                                              uint8_t* __restrict__ q,
                                                              float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;  // whole waves leave together
  const uint16_t* row = a + m * lda;
  uint8_t* qrow = q + m * K;
  const int chunks = (int)(K / 8);
  constexpr float kFmax = FMT == QLIN_INT8 ? 127.0f : (FMT == QLIN_E4M3FNUZ ? 240.0f : 448.0f);
  uint4 cache[CPL];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int idx = lane + 64 * c;
    cache[c] = idx < chunks ? ldg16(row + (int64_t)idx * 8) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float v[8];
    unpack_bf16x8(cache[c], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = wave_max(amax);
  const float sc = amax > 0.0f ? amax / kFmax : 0.0f;
  const RowScale rs = row_scale(sc);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int idx = lane + 64 * c;
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
  if (lane == 0) s[m] = sc;
}

template <int FMT>
static void launch_quant_fmt(const uint16_t* a, int64_t M, int64_t K, int64_t lda, uint8_t* q,
                             float* s, hipStream_t st) {
  const int64_t chunks = K / 8;
  const dim3 grid((unsigned)M);
  const dim3 wgrid((unsigned)((M + 3) / 4));
  // many short rows (weights quantised on line, prefill activations): a wave
  // per row keeps every lane busy (C5 bf16 expert banks 540 -> 424 us); a few
  // rows (decode): a workgroup per row spreads each row's divisions over 4x
  // the lanes, which is shorter (K=2048, M <= 64: 2.2-2.5 instead of 2.9-3.1 us)
  const bool tall = M >= 1024;
  if (tall && chunks <= 64)
    quant_rows_wave_kernel<FMT, 1><<<wgrid, kQThreads, 0, st>>>(a, M, K, lda, q, s);
  else if (tall && chunks <= 128)
    quant_rows_wave_kernel<FMT, 2><<<wgrid, kQThreads, 0, st>>>(a, M, K, lda, q, s);
  else if (tall && chunks <= 256)
    quant_rows_wave_kernel<FMT, 4><<<wgrid, kQThreads, 0, st>>>(a, M, K, lda, q, s);
  else if (chunks <= 1 * kQThreads)
    quant_act_kernel<FMT, 1><<<grid, kQThreads, 0, st>>>(a, K, lda, q, s);
  else if (chunks <= 2 * kQThreads)
    quant_act_kernel<FMT, 2><<<grid, kQThreads, 0, st>>>(a, K, lda, q, s);
  else if (chunks <= 4 * kQThreads)
    quant_act_kernel<FMT, 4><<<grid, kQThreads, 0, st>>>(a, K, lda, q, s);
  else if (chunks <= 8 * kQThreads)
    quant_act_kernel<FMT, 8><<<grid, kQThreads, 0, st>>>(a, K, lda, q, s);
  else
    quant_act_kernel<FMT, 0><<<grid, kQThreads, 0, st>>>(a, K, lda, q, s);
}

int launch_quant_act(const uint16_t* a, int64_t M, int64_t K, int64_t lda, int fmt, void* q,
                     float* s, hipStream_t st) {
  uint8_t* qb = reinterpret_cast<uint8_t*>(q);
  if (fmt == QLIN_INT8) launch_quant_fmt<QLIN_INT8>(a, M, K, lda, qb, s, st);
  else if (fmt == QLIN_E4M3FNUZ) launch_quant_fmt<QLIN_E4M3FNUZ>(a, M, K, lda, qb, s, st);
  else launch_quant_fmt<QLIN_E4M3>(a, M, K, lda, qb, s, st);
  return launch_status();
}

// fp32 rows -> OCP E4M3 (the MoE intermediate): same rule, rows of K fp32.
__global__ __launch_bounds__(kQThreads) void quant_rows_f32_kernel(const float* __restrict__ a,
                                                                   int64_t K,
                                                                   uint8_t* __restrict__ q,
                                                                   float* __restrict__ s) {
  __shared__ float red[kQThreads / 64];
  const int64_t m = blockIdx.x;
  const float* row = a + m * K;
  const int chunks = (int)(K / 8);
  float amax = 0.0f;
  for (int idx = threadIdx.x; idx < chunks; idx += kQThreads) {
    const float4 x0 = *reinterpret_cast<const float4*>(row + (int64_t)idx * 8);
    const float4 x1 = *reinterpret_cast<const float4*>(row + (int64_t)idx * 8 + 4);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x0.x), fabsf(x0.y)), fmaxf(fabsf(x0.z), fabsf(x0.w))));
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x1.x), fabsf(x1.y)), fmaxf(fabsf(x1.z), fabsf(x1.w))));
  }
  amax = block_max<kQThreads / 64>(amax, red);
  const float sc = amax > 0.0f ? amax / 448.0f : 0.0f;
  for (int idx = threadIdx.x; idx < chunks; idx += kQThreads) {
    uint2 out = make_uint2(0, 0);
    if (sc > 0.0f) {
      const float4 x0 = *reinterpret_cast<const float4*>(row + (int64_t)idx * 8);
      const float4 x1 = *reinterpret_cast<const float4*>(row + (int64_t)idx * 8 + 4);
      float v[8] = {x0.x / sc, x0.y / sc, x0.z / sc, x0.w / sc,
                    x1.x / sc, x1.y / sc, x1.z / sc, x1.w / sc};
      out = encode8<QLIN_E4M3>(v);
    }
    *reinterpret_cast<uint2*>(q + m * K + (int64_t)idx * 8) = out;
  }
  if (threadIdx.x == 0) s[m] = sc;
}

// Rows of at most 64*8*CPL fp32 values (the MoE intermediate, I = 768): one
// wave per row (four rows per workgroup), CPL chunks of 8 per lane held in
// registers, the absmax reduced within the wave; the same scale, division
// and encoder as above. A workgroup per row left 160 of its 256 threads idle
// at I = 768 and read each row twice (T = 512: 4096 rows).
template <int CPL>
__global__ __launch_bounds__(256) void quant_rows_f32_wave_kernel(const float* __restrict__ a, int64_t M,
                                                                  int64_t K, uint8_t* __restrict__ q,
                                                                  float* __restrict__ s) {
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;  // whole waves leave together
  const float* row = a + m * K;
  const int chunks = (int)(K / 8);
  float4 x[CPL][2];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int idx = lane + 64 * c;
    const bool in = idx < chunks;
    x[c][0] = in ? *reinterpret_cast<const float4*>(row + (int64_t)idx * 8) : make_float4(0, 0, 0, 0);
    x[c][1] = in ? *reinterpret_cast<const float4*>(row + (int64_t)idx * 8 + 4) : make_float4(0, 0, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x[c][h].x), fabsf(x[c][h].y)), fmaxf(fabsf(x[c][h].z), fabsf(x[c][h].w))));
  amax = wave_max(amax);
  const float sc = amax > 0.0f ? amax / 448.0f : 0.0f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int idx = lane + 64 * c;
    if (idx < chunks) {
      uint2 out = make_uint2(0, 0);
      if (sc > 0.0f) {
        float v[8] = {x[c][0].x / sc, x[c][0].y / sc, x[c][0].z / sc, x[c][0].w / sc,
                      x[c][1].x / sc, x[c][1].y / sc, x[c][1].z / sc, x[c][1].w / sc};
        out = encode8<QLIN_E4M3>(v);
      }
      *reinterpret_cast<uint2*>(q + m * K + (int64_t)idx * 8) = out;
    }
  }
  if (lane == 0) s[m] = sc;
}

int launch_quant_rows_f32(const float* a, int64_t M, int64_t K, uint8_t* q, float* s,
                          hipStream_t st) {
  const int64_t chunks = K / 8;
  const dim3 wgrid((unsigned)((M + 3) / 4));
  if (chunks <= 64)
    quant_rows_f32_wave_kernel<1><<<wgrid, 256, 0, st>>>(a, M, K, q, s);
  else if (chunks <= 128)
    quant_rows_f32_wave_kernel<2><<<wgrid, 256, 0, st>>>(a, M, K, q, s);
  else if (chunks <= 256)
    quant_rows_f32_wave_kernel<4><<<wgrid, 256, 0, st>>>(a, M, K, q, s);
  else
    quant_rows_f32_kernel<<<dim3((unsigned)M), kQThreads, 0, st>>>(a, K, q, s);
  return launch_status();
}

// Element-wise encoder (the quantisers' codec), 8 values per lane.
template <int FMT>
__global__ __launch_bounds__(256) void fp8_encode_kernel(const float* __restrict__ x, int64_t n,
                                                         uint8_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i >= n) return;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = (i + j < n) ? x[i + j] : 0.0f;
  const uint2 w = encode8<FMT>(v);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (i + j < n) out[i + j] = (uint8_t)(((j < 4 ? w.x : w.y) >> (8 * (j & 3))) & 0xFFu);
}

int launch_fp8_encode(const float* x, int64_t n, int fmt, uint8_t* out, hipStream_t st) {
  const int64_t blocks = (n + 8 * 256 - 1) / (8 * 256);
  if (fmt == QLIN_E4M3FNUZ)
    fp8_encode_kernel<QLIN_E4M3FNUZ><<<dim3((unsigned)blocks), 256, 0, st>>>(x, n, out);
  else
    fp8_encode_kernel<QLIN_E4M3><<<dim3((unsigned)blocks), 256, 0, st>>>(x, n, out);
  return launch_status();
}

}  // namespace qlin
