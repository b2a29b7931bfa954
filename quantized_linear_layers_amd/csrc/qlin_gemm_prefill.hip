// Prefill-shaped quantized GEMMs (M > 64) for gfx950: the layer is a dense
// contraction here, so it runs as an LDS-tiled MFMA GEMM.
//
//   FP8 W8A8: Y = ((sum_k a*w) * s_a[m]) * s_w[n]   (fp32 accumulation)
//   int8:     Y = ((float)sum_k a*w * s_a[m]) * s_w[n]  (int32 accumulation)
//   W4A16:    Y = sum_k a * bf16(c * step)          (unpacked in the kernel)
// (Row-wise scaled FP8 mm and Int8 scaled mm of the "MI300X: Gemma 4 E2B"
// article, "Step 3"; W4A16 unpack of "Gemma 4 From E2B to 31B", "The 4-Bit
// Builds Stay Slow".)
//
// Workgroup tile BM x BN, K tile of 128 elements, double-buffered LDS; the
// next K tile is fetched into registers while the current one is consumed.
// Waves form a WM x WN grid; each wave owns (BM/WM) x (BN/WN) outputs as
// 16x16 MFMA blocks. Tiles are ordered so that consecutive tiles of one XCD
// share A rows (grouped order, XCD-major block remap).
#include <algorithm>

#include "qlin_device.h"
#include "qlin_internal.h"

namespace qlin {

struct PrefillArgs {
  const uint8_t* A;  // fp8/int8 [M][K] (lda = K) or bf16 [M][lda]
  int64_t lda;
  const float* sa;
  const uint8_t* W;       // fp8/int8 [N][K] or int4 codes [N][K/2]
  const uint16_t* steps;  // [N][K/32] (W4A16)
  const float* sw;
  int M, N, K;
  void* y;
  int out_f32;
};

template <int KIND, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void prefill_gemm_kernel(const PrefillArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int kEsz = KIND == kGemmW4 ? 2 : 1;       // activation bytes / element
  constexpr int kARow = 128 * kEsz + 16;              // LDS row strides (padded)
  constexpr int kWRow = KIND == kGemmW4 ? 128 * 2 + 16 : 128 + 16;  // W stored dequantised (bf16)
  constexpr int MBW = BM / WM / 16, NBW = BN / WN / 16;
  using Acc = typename std::conditional<KIND == kGemmI8, v4i, v4f>::type;
  // global -> register staging: 16-byte pieces per thread
  constexpr int kAPieces = BM * 128 * kEsz / 16 / NT;
  constexpr int kWPieces = KIND == kGemmW4 ? BN * 4 / NT : BN * 128 / 16 / NT;  // W4: one group each
  static_assert(kAPieces * NT == BM * 128 * kEsz / 16, "A tile split");
  static_assert(kWPieces * NT == (KIND == kGemmW4 ? BN * 4 : BN * 8), "W tile split");

  __shared__ __attribute__((aligned(16))) uint8_t lds[2][BM * kARow + BN * kWRow];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile order: XCD-major remap, then grouped rows of tiles
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
  const int nblk = tiles_m * tiles_n;
  int b = blockIdx.x;
  if (nblk % 8 == 0) b = (b % 8) * (nblk / 8) + b / 8;
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int first_m = (b / per_group) * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int tm = first_m + (b % per_group) % gsz;
  const int tn = (b % per_group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  uint4 ra[kAPieces];
  uint4 rw[kWPieces];
  float rstep[KIND == kGemmW4 ? kWPieces : 1];

  // Branch-free tile fetch: rows past M / N are clamped onto the last row
  // (their outputs are never stored); K positions past K read the last valid
  // chunk, and the activation side is zeroed there when the tile is stashed,
  // so they add nothing. Nothing consumes the fetched registers before the
  // stash, which lets the loads fly while the current tile is multiplied.
  auto fetch = [&](int kt) {
    const int kb = kt * 128;
#pragma unroll
    for (int q = 0; q < kAPieces; ++q) {
      const int i = tid + q * NT;
      const int row = i / (8 * kEsz), col = i % (8 * kEsz);
      const int k = kb + col * (16 / kEsz);
      const int m = min(m0 + row, p.M - 1);
      ra[q] = ldg16(p.A + ((size_t)m * p.lda + min(k, p.K - 16 / kEsz)) * kEsz);
    }
#pragma unroll
    for (int q = 0; q < kWPieces; ++q) {
      const int i = tid + q * NT;
      if constexpr (KIND == kGemmW4) {
        const int row = i / 4, grp = i % 4;
        const int k = min(kb + grp * 32, p.K - 32);
        const int n = min(n0 + row, p.N - 1);
        rw[q] = ldg16(p.W + (size_t)n * (p.K / 2) + k / 2);
        rstep[q] = bf16_f32(p.steps[(size_t)n * (p.K / 32) + k / 32]);
      } else {
        const int row = i / 8, col = i % 8;
        const int k = min(kb + col * 16, p.K - 16);
        const int n = min(n0 + row, p.N - 1);
        rw[q] = ldg16(p.W + (size_t)n * p.K + k);
      }
    }
  };
  auto stash = [&](int buf, int kt) {
    uint8_t* la = lds[buf];
    uint8_t* lw = lds[buf] + BM * kARow;
#pragma unroll
    for (int q = 0; q < kAPieces; ++q) {
      const int i = tid + q * NT;
      const int row = i / (8 * kEsz), col = i % (8 * kEsz);
      const uint32_t keep = kt * 128 + col * (16 / kEsz) < p.K ? 0xFFFFFFFFu : 0u;
      const uint4 v = ra[q];
      *reinterpret_cast<uint4*>(la + row * kARow + col * 16) =
          make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
    }
#pragma unroll
    for (int q = 0; q < kWPieces; ++q) {
      const int i = tid + q * NT;
      if constexpr (KIND == kGemmW4) {
        const int row = i / 4, grp = i % 4;
        const uint32_t cw[4] = {rw[q].x, rw[q].y, rw[q].z, rw[q].w};
        const float st = rstep[q], n8 = -8.0f * st;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          *reinterpret_cast<v8bf*>(lw + row * kWRow + (grp * 32 + w * 8) * 2) = dequant8(cw[w], st, n8);
      } else {
        const int row = i / 8, col = i % 8;
        *reinterpret_cast<uint4*>(lw + row * kWRow + col * 16) = rw[q];
      }
    }
  };

  Acc acc[MBW][NBW];
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[i][j] = Acc{0, 0, 0, 0};

  const int KT = (p.K + 127) / 128;
  auto compute = [&](int buf) {
    const uint8_t* la = lds[buf] + (wm * MBW * 16) * kARow;
    const uint8_t* lw = lds[buf] + BM * kARow + (wn * NBW * 16) * kWRow;
    if constexpr (KIND == kGemmW4) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {  // four 32-wide MFMA K slices
        v8bf af[MBW], bf[NBW];
#pragma unroll
        for (int i = 0; i < MBW; ++i)
          af[i] = *reinterpret_cast<const v8bf*>(la + (i * 16 + r) * kARow + (kk * 32 + g * 8) * 2);
#pragma unroll
        for (int j = 0; j < NBW; ++j)
          bf[j] = *reinterpret_cast<const v8bf*>(lw + (j * 16 + r) * kWRow + (kk * 32 + g * 8) * 2);
#pragma unroll
        for (int i = 0; i < MBW; ++i)
#pragma unroll
          for (int j = 0; j < NBW; ++j) acc[i][j] = mfma_bf16(af[i], bf[j], acc[i][j]);
      }
    } else {
      // all B fragments of the wave, then one A fragment at a time
      uint4 w0[NBW], w1[NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const uint8_t* wp = lw + (j * 16 + r) * kWRow + 16 * g;
        w0[j] = *reinterpret_cast<const uint4*>(wp);
        w1[j] = *reinterpret_cast<const uint4*>(wp + 64);
      }
      // A fragments double-buffered: the read of block i+1 is in flight while
      // block i's MFMAs run
      uint4 a0 = *reinterpret_cast<const uint4*>(la + r * kARow + 16 * g);
      uint4 a1 = *reinterpret_cast<const uint4*>(la + r * kARow + 16 * g + 64);
#pragma unroll
      for (int i = 0; i < MBW; ++i) {
        uint4 n0 = a0, n1 = a1;
        if (i + 1 < MBW) {
          const uint8_t* ap = la + ((i + 1) * 16 + r) * kARow + 16 * g;
          n0 = *reinterpret_cast<const uint4*>(ap);
          n1 = *reinterpret_cast<const uint4*>(ap + 64);
        }
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
          if constexpr (KIND == kGemmFP8) {
            const v8i av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                            (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            const v8i wv = {(int)w0[j].x, (int)w0[j].y, (int)w0[j].z, (int)w0[j].w,
                            (int)w1[j].x, (int)w1[j].y, (int)w1[j].z, (int)w1[j].w};
            acc[i][j] = mfma_fp8(av, wv, acc[i][j]);
          } else {
            const v4i alo = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w};
            const v4i ahi = {(int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            const v4i wlo = {(int)w0[j].x, (int)w0[j].y, (int)w0[j].z, (int)w0[j].w};
            const v4i whi = {(int)w1[j].x, (int)w1[j].y, (int)w1[j].z, (int)w1[j].w};
            acc[i][j] = mfma_i8(alo, wlo, acc[i][j]);
            acc[i][j] = mfma_i8(ahi, whi, acc[i][j]);
          }
        }
        a0 = n0;
        a1 = n1;
      }
    }
  };

  fetch(0);
  stash(0, 0);
  __syncthreads();
  for (int kt = 0; kt + 1 < KT; ++kt) {
    fetch(kt + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(kt & 1);
    __builtin_amdgcn_sched_barrier(0);
    stash((kt + 1) & 1, kt + 1);
    __syncthreads();
  }
  compute((KT - 1) & 1);

  // ---- epilogue: scales of this lane's rows / columns (clamped, no
  // branches, all issued before the first use)
  float sav[MBW][4], swv[NBW];
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sav[i][e] = KIND == kGemmW4 ? 1.0f : p.sa[min(m0 + wm * MBW * 16 + i * 16 + 4 * g + e, p.M - 1)];
#pragma unroll
  for (int j = 0; j < NBW; ++j)
    swv[j] = KIND == kGemmW4 ? 1.0f : p.sw[min(n0 + wn * NBW * 16 + j * 16 + r, p.N - 1)];
#pragma unroll
  for (int i = 0; i < MBW; ++i)
#pragma unroll
    for (int j = 0; j < NBW; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * MBW * 16 + i * 16 + 4 * g + e;
        const int n = n0 + wn * NBW * 16 + j * 16 + r;
        if (m < p.M && n < p.N) {
          float v;
          if constexpr (KIND == kGemmW4) v = acc[i][j][e];
          else if constexpr (KIND == kGemmI8) v = ((float)acc[i][j][e] * sav[i][e]) * swv[j];
          else v = (acc[i][j][e] * sav[i][e]) * swv[j];
          if (p.out_f32) reinterpret_cast<float*>(p.y)[(size_t)m * p.N + n] = v;
          else reinterpret_cast<uint16_t*>(p.y)[(size_t)m * p.N + n] = (uint16_t)f32_bf16_rne(v);
        }
      }
}

template <int KIND, int BM, int BN, int WM, int WN>
static void launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  prefill_gemm_kernel<KIND, BM, BN, WM, WN><<<dim3((unsigned)tiles), WM * WN * 64, 0, st>>>(a);
}

int launch_prefill(int kind, const void* a, int64_t lda, const float* sa, const void* w,
                   const void* wsc, int64_t M, int64_t N, int64_t K, void* y, int out_f32,
                   hipStream_t st) {
  PrefillArgs g{};
  g.A = reinterpret_cast<const uint8_t*>(a);
  g.lda = lda;
  g.sa = sa;
  g.W = reinterpret_cast<const uint8_t*>(w);
  if (kind == kGemmW4) g.steps = reinterpret_cast<const uint16_t*>(wsc);
  else g.sw = reinterpret_cast<const float*>(wsc);
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.y = y;
  g.out_f32 = out_f32;
  // large problems: 256x256 tiles (4 waves of 128x128: half the LDS operand
  // traffic per flop of 64x64 wave tiles); small ones keep 128x128 tiles so
  // the grid still fills the device
  const bool big = M >= 1024 && N >= 1024 && (M / 256) * (N / 256) >= 256;
  if (kind == kGemmFP8) {
    if (big) launch_prefill_t<kGemmFP8, 256, 256, 2, 2>(g, st);
    else launch_prefill_t<kGemmFP8, 128, 128, 2, 2>(g, st);
  } else if (kind == kGemmI8) {
    if (big) launch_prefill_t<kGemmI8, 256, 256, 2, 2>(g, st);
    else launch_prefill_t<kGemmI8, 128, 128, 2, 2>(g, st);
  } else {
    launch_prefill_t<kGemmW4, 128, 128, 2, 2>(g, st);
  }
  return launch_status();
}

// ----------------------------------------------------------------------------
// dispatch: M <= 64 -> weight-streaming decode kernel, else tiled MFMA GEMM
// ----------------------------------------------------------------------------
size_t decode_workspace_bytes(int kind, int64_t M, int64_t N, int64_t K);
int launch_decode(int kind, const void* a, int64_t lda, const float* sa, const void* w,
                  const void* wsc, int64_t M, int64_t N, int64_t K, void* y, int out_f32,
                  void* ws, size_t ws_bytes, hipStream_t st);

size_t gemm_workspace_bytes(int kind, int64_t M, int64_t N, int64_t K) {
  if (M <= 64) return decode_workspace_bytes(kind, M, N, K);
  return 0;
}

int launch_gemm(int kind, const void* a, int64_t lda, const float* sa, const void* w,
                const void* wsc, int64_t M, int64_t N, int64_t K, void* y, int out_f32, void* ws,
                size_t ws_bytes, hipStream_t st) {
  if (M <= 64) return launch_decode(kind, a, lda, sa, w, wsc, M, N, K, y, out_f32, ws, ws_bytes, st);
  return launch_prefill(kind, a, lda, sa, w, wsc, M, N, K, y, out_f32, st);
}

}  // namespace qlin
