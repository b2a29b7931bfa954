// Decode-shaped quantized GEMMs (M <= 64) for gfx950.
//
//   FP8 W8A8  ("MI300X: Gemma 4 E2B" article, "Step 3": row-wise scaled FP8
//              mm; Gemma 4 31B-it FP8 model card: per-channel weight scale,
//              per-token activation scale)
//              Y = ((sum_k a*w) * s_a[m]) * s_w[n], fp32 accumulation
//   int8 W8A8 (same article, "Step 3" and "Step 2": must accept every M)
//              acc int32, Y = ((float)acc * s_a[m]) * s_w[n]
//   W4A16     ("Gemma 4 From E2B to 31B", "The 4-Bit Builds Stay Slow":
//              weights unpacked to bf16 before each multiply)
//              Y = sum_k a * bf16(c * step)
//
// At M <= 64 the layer is bound by streaming the weights from HBM. Design:
//  * a workgroup of 4 waves owns 64*NB output columns (16*NB per wave) and
//    one K range (split-K across workgroups when the column tiles alone
//    would not fill the device);
//  * the activations of the K range pass through LDS in chunks of 256 K,
//    double buffered and shared by the 4 waves (one barrier per chunk), so
//    each activation byte is fetched once per workgroup, in whole cache
//    lines, and MFMA fragments come from LDS;
//  * each wave streams its own weight rows into a ring of DEPTH 128-K steps
//    of registers, DEPTH steps ahead of use, with branch-free clamped loads;
//  * MFMA with M padded to 16 (padding rows are zero in LDS);
//  * the int4 unpack and every scale are fused into the kernel;
//  * split-K partial sums go to the workspace and the last workgroup of a
//    column tile to arrive (device-scope counter) sums them in split order,
//    so results are deterministic; it applies the epilogue and resets the
//    counter.
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "qlin_device.h"
#include "qlin_internal.h"
#include "qlin_skinny.h"

namespace qlin {

struct GemmArgs {
  const uint8_t* A;       // fp8/int8 codes [M][lda], or bf16 [M][lda] for W4A16
  int64_t lda;            // elements
  const float* sa;        // [M] (fp8 / int8)
  const uint8_t* W;       // fp8/int8 [N][K], or int4 codes [N][K/2]
  const uint16_t* steps;  // W4A16: bf16 [N][K/32]
  const float* sw;        // [N] (fp8 / int8)
  int M, N, K;
  int kc;                 // K per split, multiple of 256
  void* y;
  int out_f32;
  uint32_t* part;         // [S][M][N] fp32 / int32 partial sums
  unsigned* cnt;          // one arrival counter per column tile
};

// Decode-shaped GEMM: the streaming core of qlin_skinny.h over this
// workgroup's 16*NB*NW columns and this split's K range, then the split-K
// reduction and the epilogue. With WK the NW waves share 16*NB columns and
// each takes a quarter of the split's K range (whole 256-K chunks) with its
// own activation chunks; their accumulators are summed through LDS in wave
// order (deterministic) and wave 0 goes on alone. This puts a small layer's
// whole weight matrix in flight at once without a second, global pass.
template <int KIND, int MB, int NB, int DEPTH, bool SB, int NW, bool WK>
__global__ __launch_bounds__(64 * NW) void decode_gemm_kernel(const GemmArgs p) {
  using Acc = SkinnyAcc<KIND>;
  constexpr bool W4 = KIND == kGemmW4;
  constexpr int ESZ = W4 ? 2 : 1;
  constexpr int kPer = skinny_pieces<KIND, MB, NW, WK>();
  constexpr int kLds = skinny_lds_bytes<KIND, MB, NB, DEPTH, NW, WK>();
  static_assert(!WK || kLds >= NW * MB * NB * 64 * 16, "LDS holds the waves' accumulators");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  __shared__ unsigned last_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int split = blockIdx.y, S = gridDim.y;
  const int k0 = split * p.kc, k1 = min(k0 + p.kc, p.K);
  const int n0 = WK ? blockIdx.x * 16 * NB : (blockIdx.x * NW + wave) * 16 * NB;  // this wave's first column
  // this wave's K range
  const int kq = WK ? (k1 - k0 + NW * 256 - 1) / (NW * 256) * 256 : 0;
  const int wk0 = WK ? min(k0 + wave * kq, k1) : k0;
  const int wk1 = WK ? min(wk0 + kq, k1) : k1;

  // operand rows (clamped onto valid rows; padding activation rows masked)
  const uint8_t* wp[NB][2];
  const uint16_t* sp[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = min(n0 + 16 * j + 8 * h + (lane >> 3), p.N - 1);
      wp[j][h] = p.W + (size_t)row * (W4 ? p.K / 2 : p.K) + 16 * (lane & 7);
    }
    sp[j] = W4 ? p.steps + (size_t)min(n0 + 16 * j + (lane & 15), p.N - 1) * (p.K / 32) : nullptr;
  }
  const uint8_t* ap[kPer];
  uint32_t am[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int row = ((WK ? lane : tid) + (WK ? 64 : 64 * NW) * q) / (16 * ESZ);
    ap[q] = p.A + (size_t)min(row, p.M - 1) * p.lda * ESZ;
    am[q] = row < p.M ? 0xFFFFFFFFu : 0u;
  }

  // epilogue scales of this lane's row (one per row block) and its 4
  // columns per column block (the core's output layout), fetched up front
  float sav[MB], swv[NB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) sav[mb] = W4 ? 1.0f : p.sa[min(mb * 16 + r, p.M - 1)];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) swv[j][i] = W4 ? 1.0f : p.sw[min(n0 + 16 * j + 4 * g + i, p.N - 1)];

  Acc acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mb][j] = Acc{0, 0, 0, 0};
  if (wk0 < wk1) skinny_mma<KIND, MB, NB, DEPTH, SB, NW, WK>(lds, wp, sp, ap, am, p.K, wk0, wk1, acc);

  // ---- WK: sum the waves' accumulators (wave order), wave 0 owns the tile
  bool owner = true;
  if constexpr (WK) {
    __syncthreads();  // every wave is done with its LDS regions
    Acc* red = reinterpret_cast<Acc*>(lds);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j) red[((wave * MB + mb) * NB + j) * 64 + lane] = acc[mb][j];
    __syncthreads();
    owner = wave == 0;
    if (owner) {
#pragma unroll
      for (int w = 1; w < NW; ++w)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[mb][j] = acc[mb][j] + red[((w * MB + mb) * NB + j) * 64 + lane];
    }
  }

  // ---- split-K: publish partials, the last workgroup of the tile reduces
  float accf[MB][NB][4];
  int acci[MB][NB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        accf[mb][j][i] = 0.0f;
        acci[mb][j][i] = 0;
        if constexpr (KIND == kGemmI8) acci[mb][j][i] = acc[mb][j][i];
        else accf[mb][j][i] = acc[mb][j][i];
      }
  // Partial sums and the counter use device-scope accesses (the partials:
  // buffer loads and stores with the sc1 cache policy, which bypass the
  // per-XCD L2 caches as relaxed device-scope atomics do); a store is
  // complete (vmcnt) once it is visible device-wide, so waiting for the
  // stores before the counter increment orders them without a cache-wide
  // write-back fence (a fence here would flush and invalidate the whole L2
  // of the XCD on every workgroup). Each lane moves its 4 consecutive
  // columns as one 16-byte access when the rows allow it.
  constexpr int kSc1 = 16;  // cache policy: sc1
  const bool pvec = (p.N & 3) == 0;
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      p.part, (short)0, (int)min((size_t)S * p.M * p.N * 4, (size_t)0x7FFFFFFF), 0x00020000);
  auto part_off = [&](int sp, int m, int n) { return (uint32_t)((((size_t)sp * p.M + m) * p.N + n) * 4); };
  if (S > 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = mb * 16 + r;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = n0 + 16 * j + 4 * g;
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = KIND == kGemmI8 ? (uint32_t)acci[mb][j][i] : __float_as_uint(accf[mb][j][i]);
        if (owner && m < p.M) {
          const uint32_t o = part_off(split, m, n);
          if (pvec && n + 3 < p.N) {
            __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]}, prs, o, 0, kSc1);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (n + i < p.N) __builtin_amdgcn_raw_buffer_store_b32(w[i], prs, o + 4 * i, 0, kSc1);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial sums are visible
    __syncthreads();                // ... and those of the other waves
    if (tid == 0)
      last_flag = __hip_atomic_fetch_add(&p.cnt[blockIdx.x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  (unsigned)(S - 1);
    __syncthreads();
    if (!last_flag || !owner) return;
    // sum the splits in split order; the loads of up to 4 splits are all
    // issued before the first is consumed (each load is a round trip to
    // memory; clamped addresses, no branches before the sums)
    for (int s0 = 0; s0 < S; s0 += 4) {
      uint32_t u[4][MB][NB][4];
      // (one branch around all loads: a branch per load would make the
      // compiler wait for older loads at every block boundary)
      if (pvec) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              const int m = min(mb * 16 + r, p.M - 1), n = min(n0 + 16 * j + 4 * g, p.N - 4);
              const v4i x = __builtin_amdgcn_raw_buffer_load_b128(prs, part_off(min(s0 + b, S - 1), m, n), 0, kSc1);
              u[b][mb][j][0] = (uint32_t)x.x;
              u[b][mb][j][1] = (uint32_t)x.y;
              u[b][mb][j][2] = (uint32_t)x.z;
              u[b][mb][j][3] = (uint32_t)x.w;
            }
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int m = min(mb * 16 + r, p.M - 1), n = min(n0 + 16 * j + 4 * g + i, p.N - 1);
                u[b][mb][j][i] = __builtin_amdgcn_raw_buffer_load_b32(prs, part_off(min(s0 + b, S - 1), m, n), 0, kSc1);
              }
      }
      // every load above is issued before the first sum (the scheduler would
      // otherwise interleave them and keep only a few in flight)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (s0 + b >= S) break;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (s0 + b == 0) {
                if constexpr (KIND == kGemmI8) acci[mb][j][i] = (int)u[b][mb][j][i];
                else accf[mb][j][i] = __uint_as_float(u[b][mb][j][i]);
              } else {
                if constexpr (KIND == kGemmI8) acci[mb][j][i] += (int)u[b][mb][j][i];
                else accf[mb][j][i] = accf[mb][j][i] + __uint_as_float(u[b][mb][j][i]);
              }
            }
      }
    }
    if (tid == 0) __hip_atomic_store(&p.cnt[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!owner) return;

  // ---- epilogue: each lane writes 4 consecutive columns of its row as one
  // 16-byte (fp32) or 8-byte (bf16) store when the row segment is aligned
  // and inside the output, element by element otherwise
  const bool vec = (p.N & 3) == 0 && ((uintptr_t)p.y & (p.out_f32 ? 15u : 7u)) == 0;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = mb * 16 + r;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int n = n0 + 16 * j + 4 * g;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (KIND == kGemmW4) v[i] = accf[mb][j][i];
        else if constexpr (KIND == kGemmI8) v[i] = ((float)acci[mb][j][i] * sav[mb]) * swv[j][i];
        else v[i] = (accf[mb][j][i] * sav[mb]) * swv[j][i];
      }
      const size_t o = (size_t)m * p.N + n;
      if (vec && n + 3 < p.N) {
        if (p.out_f32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.y) + o) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.y) + o) =
              make_uint2(f32_bf16_rne(v[0]) | (f32_bf16_rne(v[1]) << 16), f32_bf16_rne(v[2]) | (f32_bf16_rne(v[3]) << 16));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (n + i < p.N) {
            if (p.out_f32) reinterpret_cast<float*>(p.y)[o + i] = v[i];
            else reinterpret_cast<uint16_t*>(p.y)[o + i] = (uint16_t)f32_bf16_rne(v[i]);
          }
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// launch configuration
// ----------------------------------------------------------------------------
struct DecodeCfg {
  int MB, NB, NW;
  bool WK;
  int tiles, S, kc;
};

// Compute units of the current device (queried once).
static int decode_cus() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    return n;
  }();
  return cus;
}

// Grid: 16*NB*NW columns per workgroup, S splits of K. On a wide layer (the
// 128-column tiles alone reach about three quarters of the CUs) an
// fp8/int8 wave takes two 16-column blocks (more bytes in flight per wave,
// K=5120, N=25600: 22.7 instead of 23.6 us at M = 1). A W4A16 layer of
// 1/4 to 2x the CUs in 128-column tiles runs 8 waves of one block each
// (two waves per SIMD: one wave's unpack hides the other's waits; the 8
// waves share one activation staging), split over K to about one workgroup
// per CU -- none at K=5120, N=25600 (M = 64 41.8 us, M = 48 35.3, M = 32
// 29.7, M = 8 22.3, against 46.2 / 40.3 / 37.6 / 22.8 for two blocks per
// wave with 2 splits above 32 rows and one block with 4 waves and splits
// below; N=32768, K=4096, M = 64: 39.5 against 42.5), 2 at K=5120,
// N=16384 (M = 32 20.7 against 22.5 with 4-wave workgroups) and K=4096,
// N=14336 (M = 64 26.2 against 28.6). Wider W4A16 layers (the K=1536,
// N=262144 lm_head: M = 64 121 against 101 us) take two blocks per wave
// with 8 waves from 33 rows, one block with 4 waves below, unsplit;
// narrower ones one block with 4 waves, split to about two workgroups per
// CU (K=14336, N=4096, M = 64: 26.9 us against 28.6 with 8 waves).
// Split-K costs a write and a read of S*M*N partial sums and a second,
// serial phase. fp8/int8 split when the grid's waves reach fewer than 3/4
// of the SIMDs, to about one wave per SIMD, with at least 2048 K per split
// (512 when the waves reach fewer than half the CUs) (K=14336, N=4096: M =
// 1 12.7 instead of 21.0 us, M = 8 12.9 instead of 21.1, M = 64 18.1
// instead of 24.3, in 4 splits; K=2048, N=8192: 5.5 us unsplit against 6.2
// in 2 splits at M = 1, 8.4 against 10.1 at M = 64). The W4A16 wave-private
// K mode (below) also splits to about two of its 4-wave workgroups per CU.
// W4A16 splits keep >= 4 steps of 128 K.
static DecodeCfg decode_cfg(int kind, int64_t M, int64_t N, int64_t K) {
  DecodeCfg c{};
  const int64_t cus = decode_cus();
  c.MB = (int)((M + 15) / 16);
  const int64_t t128 = (N + 127) / 128;
  const bool wide = t128 >= 3 * cus / 4;
  const bool w4eight = kind == kGemmW4 && 4 * t128 >= cus && t128 < 2 * cus;  // 8 waves of one block
  c.NB = (kind != kGemmW4 || (c.MB >= 3 && !w4eight)) && wide ? 2 : 1;
  // fp8/int8 at M <= 16 with one block per wave: 2 waves per workgroup, so
  // the same waves spread over twice the CUs (K=2048, N=8192: M = 1 5.5 ->
  // 5.3 us, M = 8 6.1 -> 5.7 us; 1 wave per workgroup was slower, and at
  // M = 64 2 waves gained nothing)
  c.NW = kind == kGemmW4 && (w4eight || c.NB == 2) ? 8 : kind != kGemmW4 && c.MB == 1 && c.NB == 1 ? 2 : 4;
  // W4A16 at M <= 16 on a layer too narrow for the column tiles to fill the
  // device: the 4 waves of a workgroup split K instead of the grid (one
  // block each; K=2048, N=8192, M = 1: 5.9 instead of 6.9 us with 2 global
  // splits; for fp8/int8 and on wide layers it was slower)
  c.WK = kind == kGemmW4 && c.MB == 1 && (N + 63) / 64 < 3 * cus / 4;
  if (c.WK) c.NB = 1;
  const int64_t cols = (int64_t)16 * (c.WK ? 1 : c.NW) * c.NB;
  c.tiles = (int)((N + cols - 1) / cols);
  const int64_t ksteps = (K + 127) / 128;
  int64_t S;
  if (kind != kGemmW4) {
    const int64_t waves = (int64_t)c.tiles * c.NW;
    S = waves >= 3 * cus ? 1 : (4 * cus + waves - 1) / waves;
    S = std::max<int64_t>(1, std::min<int64_t>(S, std::min<int64_t>(8, ksteps / (2 * waves >= cus ? 16 : 4))));
  } else {
    S = ((w4eight ? 1 : 2) * cus + c.tiles / 2) / c.tiles;
    S = std::max<int64_t>(1, std::min<int64_t>(S, std::min<int64_t>(8, ksteps / 4)));
  }
  if (c.tiles > (int)(kGemmCounterBytes / 4)) S = 1;  // one counter per tile; such grids need no split
  int64_t steps_per = (ksteps + S - 1) / S;
  steps_per = (steps_per + 1) / 2 * 2;  // whole 256-K chunks
  c.kc = (int)(steps_per * 128);
  c.S = (int)((K + c.kc - 1) / c.kc);
  return c;
}

// Dispatch on (kind, MB, NB, waves, bulk steps) to the instantiation that
// serves it. DEPTH (weight units in flight per wave), as measured: 4
// fp8/int8 128-K units (8 was slower); int4 256-K units: 2 at MB = 1 and
// with two blocks (register bound), 4 otherwise.
template <typename F>
static auto with_decode_inst(int kind, int MB, int NB, int NW, bool wk, bool sb, F&& f) {
#define QLIN_DEC_W4(SB)                                                                       \
  switch (MB) {                                                                               \
    case 1:                                                                                   \
      if (wk) return f.template operator()<kGemmW4, 1, 1, 2, SB, 4, true>();                  \
      if (NW == 8) return f.template operator()<kGemmW4, 1, 1, 2, SB, 8, false>();           \
      return f.template operator()<kGemmW4, 1, 1, 2, SB, 4, false>();                         \
    case 2:                                                                                   \
      if (NW == 8) return f.template operator()<kGemmW4, 2, 1, 4, SB, 8, false>();           \
      return f.template operator()<kGemmW4, 2, 1, 4, SB, 4, false>();                         \
    case 3:                                                                                   \
      if (NB == 2) return f.template operator()<kGemmW4, 3, 2, 2, SB, 8, false>();           \
      if (NW == 8) return f.template operator()<kGemmW4, 3, 1, 4, SB, 8, false>();           \
      return f.template operator()<kGemmW4, 3, 1, 4, SB, 4, false>();                         \
    default:                                                                                  \
      if (NB == 2) return f.template operator()<kGemmW4, 4, 2, 2, SB, 8, false>();           \
      if (NW == 8) return f.template operator()<kGemmW4, 4, 1, 4, SB, 8, false>();           \
      return f.template operator()<kGemmW4, 4, 1, 4, SB, 4, false>();                         \
  }
#define QLIN_DEC_8(K)                                                                         \
  switch (MB) {                                                                               \
    case 1:                                                                                   \
      if (NB == 2) return f.template operator()<K, 1, 2, 4, false, 4, false>();              \
      return f.template operator()<K, 1, 1, 4, false, 2, false>();                            \
    case 2:                                                                                   \
      if (NB == 2) return f.template operator()<K, 2, 2, 4, false, 4, false>();              \
      return f.template operator()<K, 2, 1, 4, false, 4, false>();                            \
    case 3:                                                                                   \
      if (NB == 2) return f.template operator()<K, 3, 2, 4, false, 4, false>();              \
      return f.template operator()<K, 3, 1, 4, false, 4, false>();                            \
    default:                                                                                  \
      if (NB == 2) return f.template operator()<K, 4, 2, 4, false, 4, false>();              \
      return f.template operator()<K, 4, 1, 4, false, 4, false>();                            \
  }
  if (kind == kGemmW4) {
    if (sb) {
      QLIN_DEC_W4(true)
    } else {
      QLIN_DEC_W4(false)
    }
  } else if (kind == kGemmI8) {
    QLIN_DEC_8(kGemmI8)
  } else {
    QLIN_DEC_8(kGemmFP8)
  }
#undef QLIN_DEC_W4
#undef QLIN_DEC_8
}

// Workspace of a split-K call: a fixed counter area (one word per column
// tile, at most kMaxTiles) at offset 0, then the partial sums. Every call
// leaves the counter area zero, and no call ever writes partials there, so a
// workspace zeroed once stays valid across calls of any shape.
constexpr size_t kCounterBytes = kGemmCounterBytes;

size_t decode_workspace_bytes(int kind, int64_t M, int64_t N, int64_t K) {
  if (kind == kGemmW4 && w4_few_applies(M, N, K)) return 0;
  const DecodeCfg c = decode_cfg(kind, M, N, K);
  if (c.S <= 1) return 0;
  return kCounterBytes + round_up((size_t)c.S * M * N * 4, 256);
}

struct LaunchFn {
  const GemmArgs* a;
  const DecodeCfg* c;
  hipStream_t st;
  template <int KIND, int MB, int NB, int DEPTH, bool SB, int NW, bool WK>
  int operator()() const {
    decode_gemm_kernel<KIND, MB, NB, DEPTH, SB, NW, WK><<<dim3((unsigned)c->tiles, (unsigned)c->S), 64 * NW, 0, st>>>(*a);
    return 0;
  }
};

int launch_decode(int kind, const void* a, int64_t lda, const float* sa, const void* w,
                  const void* wsc, int64_t M, int64_t N, int64_t K, void* y, int out_f32,
                  void* ws, size_t ws_bytes, hipStream_t st) {
  if (kind == kGemmW4 && w4_few_applies(M, N, K))
    return launch_w4_few(a, lda, w, wsc, M, N, K, y, out_f32, st);
  const DecodeCfg c = decode_cfg(kind, M, N, K);
  GemmArgs g{};
  g.A = reinterpret_cast<const uint8_t*>(a);
  g.lda = lda;
  g.sa = sa;
  g.W = reinterpret_cast<const uint8_t*>(w);
  if (kind == kGemmW4) g.steps = reinterpret_cast<const uint16_t*>(wsc);
  else g.sw = reinterpret_cast<const float*>(wsc);
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.kc = c.kc;
  g.y = y;
  g.out_f32 = out_f32;
  if (c.S > 1) {
    if (!ws || ws_bytes < decode_workspace_bytes(kind, M, N, K)) return QLIN_ERR_WORKSPACE;
    g.cnt = reinterpret_cast<unsigned*>(ws);
    g.part = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ws) + kCounterBytes);
  }
  // int4 steps in 16-byte pieces of 8 groups: aligned rows, whole pieces
  const bool sb = kind == kGemmW4 && K % 256 == 0 && ((uintptr_t)wsc & 15) == 0;
  with_decode_inst(kind, c.MB, c.NB, c.NW, c.WK, sb, LaunchFn{&g, &c, st});
  return launch_status();
}

}  // namespace qlin
