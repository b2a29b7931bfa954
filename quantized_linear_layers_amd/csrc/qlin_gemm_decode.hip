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
//  * a workgroup of NWK waves owns 16*NB output columns and one K range;
//    its waves take consecutive slices of the range (split-K across
//    workgroups as well when the grid would otherwise be too small);
//  * each wave streams its 16*NB weight rows (16-byte loads) and
//    its activation rows (L2-resident) into registers, DEPTH 128-wide K steps
//    ahead of use, with branch-free loads;
//  * MFMA with M padded to 16 (padding rows masked to zero);
//  * the int4 unpack and every scale are fused into the kernel;
//  * wave partial sums meet in LDS in wave order; split-K partial sums go to
//    the workspace and the last workgroup of a column tile to arrive (device-
//    scope counter) sums them in split order, so results are deterministic,
//    applies the epilogue and resets the counter.
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "qlin_device.h"
#include "qlin_internal.h"

namespace qlin {

struct GemmArgs {
  const uint8_t* A;       // fp8/int8 codes [M][lda], or bf16 [M][lda] for W4A16
  int64_t lda;            // elements
  const float* sa;        // [M] (fp8 / int8)
  const uint8_t* W;       // fp8/int8 [N][K], or int4 codes [N][K/2]
  const uint16_t* steps;  // W4A16: bf16 [N][K/32]
  const float* sw;        // [N] (fp8 / int8)
  int M, N, K;
  int kc;                 // K per split, multiple of 128
  void* y;
  int out_f32;
  uint32_t* part;         // [S][M][N] fp32 / int32 partial sums
  unsigned* cnt;          // one arrival counter per column tile
};

// One 128-wide K step of one wave: the weight fragments of its NB 16-row
// blocks and the activation fragments of its MB 16-row blocks.
//   fp8 / int8: lane (r, g) holds row r, bytes [16g, 16g+16) and
//               [64+16g, 80+16g) of the step (same K order for both
//               operands, as the MFMA requires).
//   W4A16:      lane (r, g) holds row r, the 32 codes of group g (16 bytes)
//               and its step; activations k = 32g + 8w + [0, 8), w = 0..3.
template <int KIND, int MB, int NB>
struct Slot;
template <int MB, int NB>
struct Slot<kGemmFP8, MB, NB> {
  uint4 w[NB][2];
  uint4 a[MB][2];
};
template <int MB, int NB>
struct Slot<kGemmI8, MB, NB> {
  uint4 w[NB][2];
  uint4 a[MB][2];
};
template <int MB, int NB>
struct Slot<kGemmW4, MB, NB> {
  uint4 w[NB];
  float st[NB];
  uint4 a[MB][4];
};

__device__ __forceinline__ uint4 and4(uint4 v, uint32_t m) {
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// Decode-shaped GEMM. A workgroup of NWK waves owns 16*NB output columns and
// one K range (split-K across workgroups); its waves take consecutive slices
// of that range. Each wave streams its weight rows and activation rows into
// registers DEPTH steps ahead of use: loads never depend on a branch (out of
// range addresses are clamped onto data the wave reads anyway, and the
// activation fragment is masked to zero instead), so the steady-state loop is
// straight-line code with DEPTH steps of loads in flight. Partial sums of the
// waves meet in LDS (fixed order); split-K partial sums meet in the workspace
// (fixed order, last arriving workgroup of the tile).
template <int KIND, int MB, int NB, int NWK, int DEPTH>
__global__ __launch_bounds__(NWK * 64) void decode_gemm_kernel(const GemmArgs p) {
  using Acc = typename std::conditional<KIND == kGemmI8, v4i, v4f>::type;
  constexpr int kAccWords = MB * NB * 4;
  __shared__ __attribute__((aligned(16))) uint32_t red[(NWK > 1 ? NWK - 1 : 1) * 64 * kAccWords];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int S = gridDim.y, split = blockIdx.y;
  const int k0 = split * p.kc;
  const int kend = min(k0 + p.kc, p.K);
  const int nsteps = (kend - k0 + 127) >> 7;
  const int spw = (nsteps + NWK - 1) / NWK;
  const int sb = min(wave * spw, nsteps), se = min(sb + spw, nsteps);
  const int kw0 = k0 + sb * 128;
  const int kw1 = min(kend, k0 + se * 128);  // this wave's K range [kw0, kw1)
  const int rounds = (se - sb + DEPTH - 1) / DEPTH;
  constexpr int kChunk = KIND == kGemmW4 ? 32 : 16;  // load granule along K
  const int kclamp = max(kw1 - kChunk, 0);
  const int n0 = blockIdx.x * 16 * NB;

  const uint8_t* wp[NB];
  const uint16_t* sp[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int row = min(n0 + 16 * j + r, p.N - 1);
    if constexpr (KIND == kGemmW4) {
      wp[j] = p.W + (size_t)row * (p.K / 2);
      sp[j] = p.steps + (size_t)row * (p.K / 32);
    } else {
      wp[j] = p.W + (size_t)row * p.K;
      sp[j] = nullptr;
    }
  }
  const uint8_t* ap[MB];
  uint32_t amask[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int row = mb * 16 + r;
    ap[mb] = p.A + (size_t)min(row, p.M - 1) * p.lda * (KIND == kGemmW4 ? 2 : 1);
    amask[mb] = row < p.M ? 0xFFFFFFFFu : 0u;
  }

  // epilogue scales of this lane's rows / columns, fetched up front (clamped
  // addresses, no branches) so that their latency hides under the main loop
  float sav[MB][4], swv[NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sav[mb][i] = KIND == kGemmW4 ? 1.0f : p.sa[min(mb * 16 + 4 * g + i, p.M - 1)];
#pragma unroll
  for (int j = 0; j < NB; ++j) swv[j] = KIND == kGemmW4 ? 1.0f : p.sw[min(n0 + 16 * j + r, p.N - 1)];

  auto load = [&](Slot<KIND, MB, NB>& sl, int t) {
    const int kb = kw0 + t * 128;
    if constexpr (KIND == kGemmW4) {
      const int kg = min(kb + 32 * g, kclamp);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        sl.w[j] = ldg16(wp[j] + (kg >> 1));
        sl.st[j] = bf16_f32(sp[j][kg >> 5]);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int w = 0; w < 4; ++w) sl.a[mb][w] = ldg16(ap[mb] + (size_t)(kg + 8 * w) * 2);
    } else {
      const int kl = min(kb + 16 * g, kclamp), kh = min(kb + 64 + 16 * g, kclamp);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        sl.w[j][0] = ldg16(wp[j] + kl);
        sl.w[j][1] = ldg16(wp[j] + kh);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        sl.a[mb][0] = ldg16(ap[mb] + kl);
        sl.a[mb][1] = ldg16(ap[mb] + kh);
      }
    }
  };

  Acc acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mb][j] = Acc{0, 0, 0, 0};

  auto compute = [&](const Slot<KIND, MB, NB>& sl, int t) {
    const int kb = kw0 + t * 128;
    if constexpr (KIND == kGemmW4) {
      const uint32_t vg = (kb + 32 * g < kw1) ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        v8bf bf[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const uint32_t cw = w == 0 ? sl.w[j].x : w == 1 ? sl.w[j].y : w == 2 ? sl.w[j].z : sl.w[j].w;
          bf[j] = dequant8(cw, sl.st[j], -8.0f * sl.st[j]);
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const v8bf af = __builtin_bit_cast(v8bf, and4(sl.a[mb][w], amask[mb] & vg));
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[mb][j] = mfma_bf16(af, bf[j], acc[mb][j]);
        }
      }
    } else {
      const uint32_t vl = (kb + 16 * g < kw1) ? 0xFFFFFFFFu : 0u;
      const uint32_t vh = (kb + 64 + 16 * g < kw1) ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const uint4 a0 = and4(sl.a[mb][0], amask[mb] & vl);
        const uint4 a1 = and4(sl.a[mb][1], amask[mb] & vh);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const uint4 w0 = sl.w[j][0], w1 = sl.w[j][1];
          if constexpr (KIND == kGemmFP8) {
            const v8i av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                            (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            const v8i wv = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w,
                            (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
            acc[mb][j] = mfma_fp8(av, wv, acc[mb][j]);
          } else {
            const v4i alo = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w};
            const v4i ahi = {(int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            const v4i wlo = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w};
            const v4i whi = {(int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
            acc[mb][j] = mfma_i8(alo, wlo, acc[mb][j]);
            acc[mb][j] = mfma_i8(ahi, whi, acc[mb][j]);
          }
        }
      }
    }
  };

  // The scheduling barriers keep each refill right after the step that
  // freed its slot: without them the scheduler sinks the loads down to their
  // uses one round later, which leaves no load in flight while waiting.
  Slot<KIND, MB, NB> ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load(ring[d], d);
  __builtin_amdgcn_sched_barrier(0);
  for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      compute(ring[d], rd * DEPTH + d);
      __builtin_amdgcn_sched_barrier(0);
      load(ring[d], (rd + 1) * DEPTH + d);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- waves of the workgroup meet in LDS, summed in wave order by wave 0
  float accf[MB][NB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) accf[mb][j][i] = 0.0f;
  int acci[MB][NB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const Acc v = acc[mb][j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (KIND == kGemmI8) acci[mb][j][i] = v[i];
        else accf[mb][j][i] = v[i];
      }
    }
  if constexpr (NWK > 1) {
    if (wave > 0) {
      uint32_t* dst = red + (size_t)(wave - 1) * 64 * kAccWords;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = (mb * NB + j) * 4 + i;
            dst[e * 64 + lane] = KIND == kGemmI8 ? (uint32_t)acci[mb][j][i]
                                                 : __float_as_uint(accf[mb][j][i]);
          }
    }
    __syncthreads();
    if (wave > 0) return;
    for (int w = 1; w < NWK; ++w) {
      const uint32_t* src = red + (size_t)(w - 1) * 64 * kAccWords;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t u = src[((mb * NB + j) * 4 + i) * 64 + lane];
            if constexpr (KIND == kGemmI8) acci[mb][j][i] += (int)u;
            else accf[mb][j][i] = accf[mb][j][i] + __uint_as_float(u);
          }
    }
  }

  // ---- split-K: publish partials, the last workgroup of the tile reduces
  if (S > 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mb * 16 + 4 * g + i, n = n0 + 16 * j + r;
          if (m < p.M && n < p.N)
            p.part[((size_t)split * p.M + m) * p.N + n] =
                KIND == kGemmI8 ? (uint32_t)acci[mb][j][i] : __float_as_uint(accf[mb][j][i]);
        }
    __threadfence();
    unsigned old = 0;
    if (lane == 0) old = atomicAdd(&p.cnt[blockIdx.x], 1u);
    old = __shfl(old, 0, kWave);
    if (old != (unsigned)(S - 1)) return;
    __threadfence();
    // sum the splits in split order; every load of one split is issued
    // before the first is consumed (clamped addresses, no branches)
    const size_t stride = (size_t)p.M * p.N;
    uint32_t off[MB][NB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          off[mb][j][i] = (uint32_t)((size_t)min(mb * 16 + 4 * g + i, p.M - 1) * p.N +
                                     min(n0 + 16 * j + r, p.N - 1));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t u = p.part[off[mb][j][i]];
          if constexpr (KIND == kGemmI8) acci[mb][j][i] = (int)u;
          else accf[mb][j][i] = __uint_as_float(u);
        }
    for (int s = 1; s < S; ++s) {
      const uint32_t* q = p.part + (size_t)s * stride;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t u = q[off[mb][j][i]];
            if constexpr (KIND == kGemmI8) acci[mb][j][i] += (int)u;
            else accf[mb][j][i] = accf[mb][j][i] + __uint_as_float(u);
          }
    }
    if (lane == 0) p.cnt[blockIdx.x] = 0u;
  }

  // ---- epilogue (wave 0 of the workgroup)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mb * 16 + 4 * g + i, n = n0 + 16 * j + r;
        if (m < p.M && n < p.N) {
          float v;
          if constexpr (KIND == kGemmW4) v = accf[mb][j][i];
          else if constexpr (KIND == kGemmI8) v = ((float)acci[mb][j][i] * sav[mb][i]) * swv[j];
          else v = (accf[mb][j][i] * sav[mb][i]) * swv[j];
          if (p.out_f32) reinterpret_cast<float*>(p.y)[(size_t)m * p.N + n] = v;
          else reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.N + n] = (uint16_t)f32_bf16_rne(v);
        }
      }
}

// ----------------------------------------------------------------------------
// launch configuration
// ----------------------------------------------------------------------------
struct DecodeCfg {
  int MB, NB, NWK, DEPTH;
  int tiles, S, kc;
};

template <int KIND, int MB, int NB, int NWK, int DEPTH>
static int resident_waves() {
  // waves of this kernel that fit on the device at once (queried once)
  static int cached = 0;
  if (!cached) {
    int blocks = 0, dev = 0, cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &blocks, reinterpret_cast<const void*>(&decode_gemm_kernel<KIND, MB, NB, NWK, DEPTH>),
            NWK * 64, 0) != hipSuccess || blocks <= 0)
      blocks = 1;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    cached = blocks * NWK * cus;
  }
  return cached;
}

// Per-kind tile shape: NB grows with MB so that activation traffic (from L2)
// stays at or below weight traffic (from HBM).
static void decode_shape(int kind, int MB, int& NB, int& DEPTH) {
  if (kind == kGemmW4) {
    NB = MB >= 3 ? 2 : MB;
    DEPTH = MB >= 3 ? 2 : (MB == 2 ? 3 : 4);
  } else {
    NB = MB >= 3 ? 2 : MB;
    DEPTH = MB >= 3 ? 2 : (MB == 2 ? 3 : 4);
  }
}

// Grid shape: 16*NB columns per workgroup, NWK waves per workgroup along K
// and S splits of K across workgroups. The whole grid should fit in one
// round of resident waves (a second, partly filled round costs a full wave
// run time): take the largest NWK in {4, 2, 1} whose column tiles fit, then
// the largest split that still fits, keeping >= 2*DEPTH steps per wave.
// res[i] = resident waves of the NWK = 1 << i instantiation.
static DecodeCfg decode_cfg_for(int kind, int64_t M, int64_t N, int64_t K, const int res[3]) {
  DecodeCfg c{};
  c.MB = (int)((M + 15) / 16);
  decode_shape(kind, c.MB, c.NB, c.DEPTH);
  const int64_t cols = (int64_t)16 * c.NB;
  c.tiles = (int)((N + cols - 1) / cols);
  const int64_t ksteps = (K + 127) / 128;
  int li = 0;
  for (int i = 2; i >= 0; --i)
    if ((int64_t)c.tiles * (1 << i) <= res[i] && ksteps >= (int64_t)(1 << i) * c.DEPTH) {
      li = i;
      break;
    }
  c.NWK = 1 << li;
  const int64_t waves = (int64_t)c.tiles * c.NWK;
  int64_t S = std::max<int64_t>(1, res[li] / std::max<int64_t>(1, waves));
  S = std::min<int64_t>(S, std::max<int64_t>(1, ksteps / ((int64_t)c.NWK * 2 * c.DEPTH)));
  S = std::max<int64_t>(1, std::min<int64_t>(S, 8));
  if (const char* e = getenv("QLIN_DECODE_SPLIT")) S = std::max(1, atoi(e));  // tuning override
  if (c.tiles > 16384) S = 1;  // counter area bound; such grids need no split
  const int64_t steps_per = (ksteps + S - 1) / S;
  c.kc = (int)(steps_per * 128);
  c.S = (int)((K + c.kc - 1) / c.kc);
  return c;
}

template <int KIND, int MB, int NB, int DEPTH>
static DecodeCfg decode_cfg_t(int64_t M, int64_t N, int64_t K) {
  const int res[3] = {resident_waves<KIND, MB, NB, 1, DEPTH>(), resident_waves<KIND, MB, NB, 2, DEPTH>(),
                      resident_waves<KIND, MB, NB, 4, DEPTH>()};
  return decode_cfg_for(KIND, M, N, K, res);
}

// Dispatch on (kind, MB) to the one instantiation that serves it.
template <typename F>
static auto with_decode_inst(int kind, int MB, F&& f) {
  if (kind == kGemmW4) {
    switch (MB) {
      case 1: return f.template operator()<kGemmW4, 1, 1, 4>();
      case 2: return f.template operator()<kGemmW4, 2, 2, 3>();
      case 3: return f.template operator()<kGemmW4, 3, 2, 2>();
      default: return f.template operator()<kGemmW4, 4, 2, 2>();
    }
  } else if (kind == kGemmI8) {
    switch (MB) {
      case 1: return f.template operator()<kGemmI8, 1, 1, 4>();
      case 2: return f.template operator()<kGemmI8, 2, 2, 3>();
      case 3: return f.template operator()<kGemmI8, 3, 2, 2>();
      default: return f.template operator()<kGemmI8, 4, 2, 2>();
    }
  } else {
    switch (MB) {
      case 1: return f.template operator()<kGemmFP8, 1, 1, 4>();
      case 2: return f.template operator()<kGemmFP8, 2, 2, 3>();
      case 3: return f.template operator()<kGemmFP8, 3, 2, 2>();
      default: return f.template operator()<kGemmFP8, 4, 2, 2>();
    }
  }
}

struct CfgFn {
  int64_t M, N, K;
  template <int KIND, int MB, int NB, int DEPTH>
  DecodeCfg operator()() const { return decode_cfg_t<KIND, MB, NB, DEPTH>(M, N, K); }
};

static DecodeCfg decode_cfg(int kind, int64_t M, int64_t N, int64_t K) {
  return with_decode_inst(kind, (int)((M + 15) / 16), CfgFn{M, N, K});
}

// Workspace of a split-K call: a fixed counter area (one word per column
// tile, at most kMaxTiles) at offset 0, then the partial sums. Every call
// leaves the counter area zero, and no call ever writes partials there, so a
// workspace zeroed once stays valid across calls of any shape.
constexpr int kMaxTiles = 16384;
constexpr size_t kCounterBytes = (size_t)kMaxTiles * 4;

size_t decode_workspace_bytes(int kind, int64_t M, int64_t N, int64_t K) {
  const DecodeCfg c = decode_cfg(kind, M, N, K);
  if (c.S <= 1) return 0;
  return kCounterBytes + round_up((size_t)c.S * M * N * 4, 256);
}

struct LaunchFn {
  const GemmArgs* a;
  const DecodeCfg* c;
  hipStream_t st;
  template <int KIND, int MB, int NB, int DEPTH>
  int operator()() const {
    const dim3 grid((unsigned)c->tiles, (unsigned)c->S);
    if (c->NWK == 1) decode_gemm_kernel<KIND, MB, NB, 1, DEPTH><<<grid, 64, 0, st>>>(*a);
    else if (c->NWK == 2) decode_gemm_kernel<KIND, MB, NB, 2, DEPTH><<<grid, 2 * 64, 0, st>>>(*a);
    else decode_gemm_kernel<KIND, MB, NB, 4, DEPTH><<<grid, 4 * 64, 0, st>>>(*a);
    return 0;
  }
};

int launch_decode(int kind, const void* a, int64_t lda, const float* sa, const void* w,
                  const void* wsc, int64_t M, int64_t N, int64_t K, void* y, int out_f32,
                  void* ws, size_t ws_bytes, hipStream_t st) {
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
  with_decode_inst(kind, c.MB, LaunchFn{&g, &c, st});
  return launch_status();
}

}  // namespace qlin
