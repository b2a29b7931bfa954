// Offline weight repacks for gfx950: q4_0 grid recovery, FP8 / int8
// per-output-channel repacks, E4M3FNUZ -> OCP conversion and the int4 ->
// bf16 dequantiser.
//
// Method (web pages on the weight-format linear layer):
//  - "MI300X: Gemma 4 E2B ..." article, "Step 1": every build starts from
//    the QAT q4_0 checkpoint (4-bit grid, one scale per 32 values, stored as
//    bf16); the 4-bit repack recovers each group's trained step and stores
//    int4 without re-rounding; the FP8 build stores E4M3 with one fp32 scale
//    per output channel; "Tip: E4M3 or E4M3FNUZ": the serving loader
//    converts between the two FP8 flavours at load time.
//  - Gemma 4 31B-it FP8 model card: one float32 scale per output channel,
//    no calibration data.
//  - "Gemma 4 From E2B to 31B" article, format table: int8 per channel.
#include "qlin_device.h"
#include "qlin_internal.h"

namespace qlin {

// ----------------------------------------------------------------------------
// q4_0 grid recovery: one lane per group of 32 values.
// A value whose code is +-1, +-2, +-4 or -8 is step * 2^p exactly, so the
// trained step is among |w_i| * 2^-p (p = 0..3). The smallest step whose grid
// (codes rint(w/step) in [-8, 7]) reproduces all 32 stored bf16 values wins.
// When no bf16 step reproduces the whole group (a trained step that is not a
// bf16 value), the candidate step whose nearest codes reproduce the most
// stored values is kept, the smaller on ties.
// ----------------------------------------------------------------------------
__device__ bool grid_fits(const uint32_t (&w)[32], float step) {
  if (!(step > 0.0f)) return false;
#pragma unroll 4
  for (int j = 0; j < 32; ++j) {
    const float q = __builtin_rintf(bf16_f32(w[j]) / step);
    if (q < -8.0f || q > 7.0f) return false;
    if (f32_bf16_rne(q * step) != w[j]) return false;
  }
  return true;
}

// Stored values reproduced by the nearest codes on `step`, clamped to
// [-8, 7] (0 for a step that is not finite and positive).
__device__ int grid_count(const uint32_t (&w)[32], float step) {
  if (!(step > 0.0f) || !(step < __builtin_inff())) return 0;
  int n = 0;
#pragma unroll 4
  for (int j = 0; j < 32; ++j) {
    const float q = fminf(fmaxf(__builtin_rintf(bf16_f32(w[j]) / step), -8.0f), 7.0f);
    n += f32_bf16_rne(q * step) == w[j];
  }
  return n;
}

__global__ __launch_bounds__(256) void zero_i64_kernel(int64_t* p) { *p = 0; }

__global__ __launch_bounds__(256) void repack_q4_0_kernel(const uint16_t* __restrict__ w,
                                                          int64_t groups,
                                                          uint8_t* __restrict__ codes,
                                                          uint16_t* __restrict__ steps,
                                                          unsigned long long* d_amb) {
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  bool counted = false;
  if (gi < groups) {
    uint32_t v[32];
    const uint4* src = reinterpret_cast<const uint4*>(w + gi * 32);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 x = src[c];
      uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[c * 8 + 2 * i] = xs[i] & 0xFFFFu;
        v[c * 8 + 2 * i + 1] = xs[i] >> 16;
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(bf16_f32(v[j])));

    float best = __builtin_inff(), second = __builtin_inff();
    if (amax > 0.0f) {
      for (int i = 0; i < 32; ++i) {
        const float a = fabsf(bf16_f32(v[i]));
        if (a == 0.0f) continue;
        float s = a;
        for (int p = 0; p < 4; ++p, s *= 0.5f) {
          if (s == best || s == second) continue;
          if (grid_fits(v, s)) {
            if (s < best) { second = best; best = s; }
            else if (s < second) second = s;
          }
        }
      }
    }
    counted = !(amax > 0.0f) || !(best < __builtin_inff()) || (second < __builtin_inff());
    if (amax > 0.0f && !(best < __builtin_inff())) {
      // no power-of-two code: bf16 neighbours of amax / |c| for |c| = 3,5,6,7
      const float div[4] = {3.0f, 5.0f, 6.0f, 7.0f};
      for (int a = 0; a < 4; ++a) {
        const uint32_t c0 = f32_bf16_rne(amax / div[a]);
        for (int d = -8; d <= 8; ++d) {
          const float s = bf16_f32((c0 + (uint32_t)d) & 0xFFFFu);
          if (s < best && grid_fits(v, s)) best = s;
        }
      }
    }
    bool fallback = false;
    if (amax > 0.0f && !(best < __builtin_inff())) {
      // no 4-bit grid fits: the candidate that reproduces the most values
      fallback = true;
      int most = -1;
      for (int i = 0; i < 32; ++i) {
        const float a = fabsf(bf16_f32(v[i]));
        if (a == 0.0f) continue;
        float s = a;
        for (int p = 0; p < 4; ++p, s *= 0.5f) {
          const int n = grid_count(v, s);
          if (n > most || (n == most && s < best)) { most = n; best = s; }
        }
      }
      const float div[4] = {3.0f, 5.0f, 6.0f, 7.0f};
      for (int a = 0; a < 4; ++a) {
        const uint32_t c0 = f32_bf16_rne(amax / div[a]);
        for (int d = -8; d <= 8; ++d) {
          const float s = bf16_f32((c0 + (uint32_t)d) & 0xFFFFu);
          if (!(s > 0.0f) || !(s < __builtin_inff())) continue;
          const int n = grid_count(v, s);
          if (n > most || (n == most && s < best)) { most = n; best = s; }
        }
      }
    }
    // codes on the chosen step
    uint32_t packed[4] = {0, 0, 0, 0};
    if (amax > 0.0f) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        float q = __builtin_rintf(bf16_f32(v[j]) / best);
        if (fallback) q = fminf(fmaxf(q, -8.0f), 7.0f);
        const uint32_t u = (uint32_t)((int)q + 8) & 15u;
        packed[j >> 3] |= u << (4 * (j & 7));
      }
    } else {
      packed[0] = packed[1] = packed[2] = packed[3] = 0x88888888u;
      best = 0.0f;
    }
    *reinterpret_cast<uint4*>(codes + gi * 16) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    steps[gi] = (uint16_t)f32_bf16_rne(best);
  }
  // count per wave, one atomic per wave
  const unsigned long long b = __ballot(counted);
  if (d_amb && (threadIdx.x & 63) == 0 && b) atomicAdd(d_amb, (unsigned long long)__popcll(b));
}

int launch_repack_q4_0(const uint16_t* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* steps,
                       int64_t* d_amb, hipStream_t st) {
  const int64_t groups = N * (K / 32);
  unsigned long long* amb = reinterpret_cast<unsigned long long*>(d_amb);
  if (amb) zero_i64_kernel<<<1, 1, 0, st>>>(d_amb);
  const int64_t blocks = (groups + 255) / 256;
  repack_q4_0_kernel<<<dim3((unsigned)blocks), 256, 0, st>>>(w, groups, codes, steps, amb);
  return launch_status();
}

// ----------------------------------------------------------------------------
// FP8 / int8 per-channel repack: one workgroup per output row.
// grid value w = c * step (exact fp32); s = absmax / FMAX; code(w / s).
// ----------------------------------------------------------------------------
template <int FMT>  // QLIN_E4M3, QLIN_E4M3FNUZ or QLIN_INT8
__global__ __launch_bounds__(256) void repack_w8_kernel(const uint8_t* __restrict__ codes,
                                                        const uint16_t* __restrict__ steps,
                                                        int64_t K, uint8_t* __restrict__ wq,
                                                        float* __restrict__ wscale) {
  __shared__ float red[4];
  const int64_t n = blockIdx.x;
  const int64_t G = K / 32;
  const uint8_t* crow = codes + n * (K / 2);
  const uint16_t* srow = steps + n * G;
  float amax = 0.0f;
  for (int64_t g = threadIdx.x; g < G; g += 256) {
    const uint4 c = ldg16(crow + g * 16);
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    uint32_t cmax = 0;  // largest |code| of the group
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int code = (int)((cw[i >> 3] >> (4 * (i & 7))) & 15u) - 8;
      cmax = max(cmax, (uint32_t)abs(code));
    }
    amax = fmaxf(amax, (float)cmax * bf16_f32(srow[g]));
  }
  amax = block_max<4>(amax, red);
  constexpr float kFmax = FMT == QLIN_INT8 ? 127.0f : (FMT == QLIN_E4M3FNUZ ? 240.0f : 448.0f);
  const float s = amax > 0.0f ? amax / kFmax : 0.0f;
  if (threadIdx.x == 0) wscale[n] = s;
  uint8_t* orow = wq + n * K;
  for (int64_t g = threadIdx.x; g < G; g += 256) {
    const uint4 c = ldg16(crow + g * 16);
    const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
    const float step = bf16_f32(srow[g]);
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = 0;
    if (s > 0.0f) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float w = (float)((int)((cw[i >> 3] >> (4 * (i & 7))) & 15u) - 8) * step;
        const float v = w / s;
        uint32_t b;
        if (FMT == QLIN_INT8) b = (uint32_t)int8_code(v) & 0xFFu;
        else b = fp8_encode<FMT == QLIN_E4M3FNUZ>(v);
        out[i >> 2] |= b << (8 * (i & 3));
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(orow + g * 32);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  }
}

int launch_repack_fp8(const uint8_t* codes, const uint16_t* steps, int64_t N, int64_t K, int fmt,
                      uint8_t* wq, float* ws, hipStream_t st) {
  if (fmt == QLIN_E4M3FNUZ)
    repack_w8_kernel<QLIN_E4M3FNUZ><<<dim3((unsigned)N), 256, 0, st>>>(codes, steps, K, wq, ws);
  else
    repack_w8_kernel<QLIN_E4M3><<<dim3((unsigned)N), 256, 0, st>>>(codes, steps, K, wq, ws);
  return launch_status();
}

int launch_repack_int8(const uint8_t* codes, const uint16_t* steps, int64_t N, int64_t K,
                       int8_t* wq, float* ws, hipStream_t st) {
  repack_w8_kernel<QLIN_INT8><<<dim3((unsigned)N), 256, 0, st>>>(
      codes, steps, K, reinterpret_cast<uint8_t*>(wq), ws);
  return launch_status();
}

// ----------------------------------------------------------------------------
// E4M3FNUZ -> OCP E4M3, one workgroup per row. Same bits decode to twice the
// value in OCP (bias 7 vs 8), so a row without +-240 (0x7F / 0xFF, NaN in
// OCP) keeps its bits with the scale halved; otherwise each value is
// re-encoded at the same scale, nearest even where not representable.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fnuz_to_ocp_kernel(const uint8_t* __restrict__ win,
                                                          const float* __restrict__ sin,
                                                          int64_t K, uint8_t* __restrict__ wout,
                                                          float* __restrict__ sout,
                                                          unsigned long long* d_bad) {
  __shared__ int flag[4];
  const int64_t n = blockIdx.x;
  const uint8_t* r = win + n * K;
  uint8_t* o = wout + n * K;
  int has240 = 0;
  for (int64_t c = threadIdx.x; c < K / 16; c += 256) {
    const uint4 x = ldg16(r + c * 16);
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // byte b has (b & 0x7F) == 0x7F  <=>  (b & 0x7F) + 1 sets bit 7 (no carry
      // crosses into the next byte)
      const uint32_t t = xs[i] & 0x7F7F7F7Fu;
      has240 |= ((t + 0x01010101u) & 0x80808080u) != 0;
    }
  }
  has240 = wave_or(has240);
  if ((threadIdx.x & 63) == 0) flag[threadIdx.x >> 6] = has240;
  __syncthreads();
  has240 = flag[0] | flag[1] | flag[2] | flag[3];
  if (threadIdx.x == 0) sout[n] = has240 ? sin[n] : sin[n] * 0.5f;
  unsigned bad = 0;
  for (int64_t c = threadIdx.x; c < K / 16; c += 256) {
    const uint4 x = ldg16(r + c * 16);
    uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t ow = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t code = (xs[i] >> (8 * b)) & 0xFFu;
        uint32_t outc;
        if (code == 0x80u) {  // the FNUZ NaN: invalid input
          ++bad;
          outc = 0;
        } else if (!has240) {
          outc = code;
        } else {
          const float v = fp8_decode<true>(code);
          outc = fp8_encode<false>(v);
          if (v == 0.0f) outc = 0;
          if (fp8_decode<false>(outc) != v) ++bad;
        }
        ow |= outc << (8 * b);
      }
      xs[i] = ow;
    }
    *reinterpret_cast<uint4*>(o + c * 16) = make_uint4(xs[0], xs[1], xs[2], xs[3]);
  }
  const long long tot = wave_sum_ll((long long)bad);
  if (d_bad && (threadIdx.x & 63) == 0 && tot) atomicAdd(d_bad, (unsigned long long)tot);
}

int launch_fnuz_to_ocp(const uint8_t* win, const float* sin, int64_t N, int64_t K, uint8_t* wout,
                       float* sout, int64_t* d_bad, hipStream_t st) {
  unsigned long long* bad = reinterpret_cast<unsigned long long*>(d_bad);
  if (bad) zero_i64_kernel<<<1, 1, 0, st>>>(d_bad);
  fnuz_to_ocp_kernel<<<dim3((unsigned)N), 256, 0, st>>>(win, sin, K, wout, sout, bad);
  return launch_status();
}

// ----------------------------------------------------------------------------
// int4 -> bf16 dequantiser (the W4A16 GEMM's operand): one lane per group.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dequant_q4_kernel(const uint8_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ steps,
                                                         int64_t groups,
                                                         uint16_t* __restrict__ out) {
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= groups) return;
  const uint4 c = ldg16(codes + gi * 16);
  const float step = bf16_f32(steps[gi]);
  const float n8 = -8.0f * step;
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  uint4* dst = reinterpret_cast<uint4*>(out + gi * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = __builtin_bit_cast(uint4, dequant8(cw[i], step, n8));
}

int launch_dequant_q4(const uint8_t* codes, const uint16_t* steps, int64_t N, int64_t K,
                      uint16_t* out, hipStream_t st) {
  const int64_t groups = N * (K / 32);
  dequant_q4_kernel<<<dim3((unsigned)((groups + 255) / 256)), 256, 0, st>>>(codes, steps, groups,
                                                                            out);
  return launch_status();
}

// int4 vocabulary lookup: the dequantiser above on gathered rows. Each wave
// takes 64 code words (512 values) of one looked-up row, so the row id and
// the row addresses are wave-uniform (scalar loads and arithmetic); each
// lane turns one 32-bit code word and its group's step into one 16-byte
// store, so a wave's loads and stores are contiguous. A row id outside
// [0, V) writes zeros. cpr = ceil(wpr / 64) waves per row.
__global__ __launch_bounds__(256) void embed_q4_kernel(const int32_t* __restrict__ ids, uint32_t T,
                                                       const uint32_t* __restrict__ codes,
                                                       const uint16_t* __restrict__ steps, int64_t V,
                                                       uint32_t wpr, uint32_t cpr, uint4* __restrict__ out) {
  const uint32_t wave = __builtin_amdgcn_readfirstlane(blockIdx.x * 4u + (threadIdx.x >> 6));
  const uint32_t t = wave / cpr;
  if (t >= T) return;
  const uint32_t j = (wave - t * cpr) * 64u + (threadIdx.x & 63u);
  if (j >= wpr) return;
  const int64_t r = ids[t];
  uint4 v = make_uint4(0, 0, 0, 0);
  if (r >= 0 && r < V) {
    const uint32_t cw = __builtin_nontemporal_load(codes + r * wpr + j);
    const float step = bf16_f32(steps[r * (wpr / 4) + j / 4]);
    v = __builtin_bit_cast(uint4, dequant8(cw, step, -8.0f * step));
  }
  out[(size_t)t * wpr + j] = v;
}

int launch_embed_q4(const int32_t* ids, int64_t T, const uint8_t* codes, const uint16_t* steps,
                    int64_t V, int64_t D, uint16_t* out, hipStream_t st) {
  const uint32_t wpr = (uint32_t)(D / 8), cpr = (wpr + 63) / 64;
  const uint64_t waves = (uint64_t)T * cpr;
  embed_q4_kernel<<<dim3((unsigned)((waves + 3) / 4)), 256, 0, st>>>(
      ids, (uint32_t)T, reinterpret_cast<const uint32_t*>(codes), steps, V, wpr, cpr,
      reinterpret_cast<uint4*>(out));
  return launch_status();
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

int launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return QLIN_OK;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  fill_zero_kernel<<<dim3((unsigned)blocks), 256, 0, st>>>(reinterpret_cast<uint4*>(p), n16);
  return launch_status();
}

}  // namespace qlin
