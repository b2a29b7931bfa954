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

// One "unit" of one wave's weight rows: 16 rows x 128 bytes per 16-row block
// (128 K of fp8/int8, 256 K of int4 codes), fetched as two line-shaped
// loads (lane l: row 8h + l/8, 16-byte chunk l%8) and held in registers
// until it is written to the wave's LDS slot; W4A16 adds the 8 group steps
// of each row (lane l: row l/4, groups 2(l%4) and 2(l%4)+1).
template <int KIND, int NB>
struct Slot {
  uint4 w[NB][2];
};
template <int NB>
struct Slot<kGemmW4, NB> {
  uint4 w[NB][2];
  uint32_t st[NB][2];
};

// Decode-shaped GEMM, see the file comment. Both operands reach the MFMAs
// from LDS in a "fragment-major" layout: the 16 bytes that MFMA lane (r, g)
// reads for one operand piece sit at piece*1024 + g*256 + 16*(r ^ f(c)),
// where c is the 16-byte chunk of the row segment; the XOR spreads the
// line-shaped staging writes over the banks.
//   fp8 / int8 (2 KB per 16-row block and 128-K step): piece = K half h,
//     chunk c = 4h + g, f = 2c. Weights use the same layout.
//   int4 weights (2 KB per block and unit of two steps): piece = step s,
//     chunk c = 4s + g (the 32 codes of group 4s + g), f = 2c.
//   bf16 activations (4 KB per block and step): piece = MFMA w of the step,
//     chunk c = 4g + w (the 8 values k = 32g + 8w .. +8), f = c.
template <int KIND, int MB, int NB, int DEPTH>
__global__ __launch_bounds__(256) void decode_gemm_kernel(const GemmArgs p) {
  using Acc = typename std::conditional<KIND == kGemmI8, v4i, v4f>::type;
  constexpr bool W4 = KIND == kGemmW4;
  constexpr int ESZ = W4 ? 2 : 1;                    // activation bytes per element
  constexpr int kUnitK = W4 ? 256 : 128;             // K per weight unit
  constexpr int UPC = 256 / kUnitK;                  // units per activation chunk
  static_assert(DEPTH % (2 * UPC) == 0, "a round holds an even number of chunks");
  constexpr int kBlk = 16 * 128 * ESZ;               // LDS bytes per (mb, step) of activations
  constexpr int kBuf = MB * 2 * kBlk;                // one 256-K activation chunk
  constexpr int kRowPieces = 16 * ESZ;               // 16-byte pieces per row per chunk
  constexpr int kPer = MB * 16 * kRowPieces / 256;   // activation pieces per thread per chunk
  constexpr int kWSlot = NB * 2048;                  // one wave's weight unit in LDS
  constexpr int kSSlot = W4 ? NB * 256 : 0;          // ... and its int4 group steps
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kBuf + 4 * (kWSlot + kSSlot)];
  __shared__ unsigned last_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int split = blockIdx.y, S = gridDim.y;
  const int k0 = split * p.kc, k1 = min(k0 + p.kc, p.K);
  const int nunits = (k1 - k0 + kUnitK - 1) / kUnitK;
  const int rounds = (nunits + DEPTH - 1) / DEPTH;
  const int n0 = (blockIdx.x * 4 + wave) * 16 * NB;  // this wave's first column
  uint8_t* wslot = lds + 2 * kBuf + wave * kWSlot;
  uint8_t* sslot = lds + 2 * kBuf + 4 * kWSlot + wave * kSSlot;

  // ---- weight rows of this wave (clamped: rows past N repeat the last one)
  const int wc = lane & 7;  // 16-byte chunk of a line-shaped load
  const uint8_t* wp[NB][2];
  const uint16_t* sp[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = min(n0 + 16 * j + 8 * h + (lane >> 3), p.N - 1);
      wp[j][h] = p.W + (size_t)row * (W4 ? p.K / 2 : p.K) + 16 * wc;
    }
    sp[j] = W4 ? p.steps + (size_t)min(n0 + 16 * j + (lane >> 2), p.N - 1) * (p.K / 32) : nullptr;
  }
  // last valid byte offset of a 16-byte chunk within the range, and group
  const int bclamp = (W4 ? k1 / 2 : k1) - 16 - 16 * wc;
  const int gmax = k1 / 32 - 1;
  auto wload = [&](Slot<KIND, NB>& sl, int u) {
    const int kb = k0 + u * kUnitK;
    const int bo = min(W4 ? kb / 2 : kb, bclamp);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      sl.w[j][0] = ldg16_nt(wp[j][0] + bo);
      sl.w[j][1] = ldg16_nt(wp[j][1] + bo);
      if constexpr (W4) {
        const int gi = kb / 32 + 2 * (lane & 3);
        sl.st[j][0] = sp[j][min(gi, gmax)];
        sl.st[j][1] = sp[j][min(gi + 1, gmax)];
      }
    }
  };
  // weight unit -> this wave's LDS slot (wave-private: LDS operations of one
  // wave complete in order, so no barrier is needed before reading it back)
  const int wr = (wc >> 2) * 1024 + (wc & 3) * 256;
  auto wstage = [&](const Slot<KIND, NB>& sl) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int R = 8 * h + (lane >> 3);
        *reinterpret_cast<uint4*>(wslot + j * 2048 + wr + ((R ^ (2 * wc)) & 15) * 16) = sl.w[j][h];
      }
      if constexpr (W4)
        *reinterpret_cast<uint32_t*>(sslot + j * 256 + (lane >> 2) * 16 + (lane & 3) * 4) =
            (sl.st[j][0] & 0xFFFFu) | (sl.st[j][1] << 16);
    }
  };

  // ---- activation chunks: piece q of this thread is row (tid + 256q) / kRowPieces.
  // Loads are clamped and stay unmasked in registers (masking them at load
  // time would make the next instruction wait for every load in flight);
  // rows past M and K past the range are zeroed when written to LDS.
  uint4 aset[2][kPer];
  auto aload = [&](int ci, uint4 (&dst)[kPer]) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int pc = tid + 256 * q;
      const int row = pc / kRowPieces, piece = pc % kRowPieces;
      const int k = k0 + ci * 256 + piece * (16 / ESZ);
      dst[q] = ldg16(p.A + ((size_t)min(row, p.M - 1) * p.lda + min(k, p.K - 16 / ESZ)) * ESZ);
    }
  };
  auto awrite = [&](const uint4 (&src)[kPer], int ci, int buf) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int pc = tid + 256 * q;
      const int row = pc / kRowPieces, piece = pc % kRowPieces;
      const int k = k0 + ci * 256 + piece * (16 / ESZ);
      const uint32_t m = row < p.M && k < k1 ? 0xFFFFFFFFu : 0u;
      const int mb = row >> 4, rr = row & 15;
      const int s = piece / (8 * ESZ), c = piece % (8 * ESZ);
      int off;
      if constexpr (W4) off = (c & 3) * 1024 + (c >> 2) * 256 + ((rr ^ c) & 15) * 16;
      else off = (c >> 2) * 1024 + (c & 3) * 256 + ((rr ^ (2 * c)) & 15) * 16;
      const uint4 v = src[q];
      *reinterpret_cast<uint4*>(lds + buf * kBuf + (mb * 2 + s) * kBlk + off) =
          make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
    }
  };
  // lane offsets of the fragment reads
  const int rd0 = g * 256 + ((r ^ (2 * g)) & 15) * 16;
  const int rd1 = 1024 + g * 256 + ((r ^ (2 * (4 + g))) & 15) * 16;
  const int rdw = g * 256;  // bf16: + w*1024 + ((r ^ (4g + w)) & 15) * 16

  // epilogue scales of this lane's rows / columns, fetched up front
  float sav[MB][4], swv[NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sav[mb][i] = W4 ? 1.0f : p.sa[min(mb * 16 + 4 * g + i, p.M - 1)];
#pragma unroll
  for (int j = 0; j < NB; ++j) swv[j] = W4 ? 1.0f : p.sw[min(n0 + 16 * j + r, p.N - 1)];

  Acc acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mb][j] = Acc{0, 0, 0, 0};

  // multiply the weight unit in the wave's slot (unit u) with the
  // activation chunk that holds it
  auto compute = [&](int u) {
    const uint8_t* abase = lds + ((u / UPC) & 1) * kBuf;
    if constexpr (W4) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint4 cw[NB];
        float st[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          cw[j] = *reinterpret_cast<const uint4*>(wslot + j * 2048 + s * 1024 + g * 256 +
                                                  ((r ^ (2 * (4 * s + g))) & 15) * 16);
          st[j] = bf16_f32(*reinterpret_cast<const uint16_t*>(sslot + j * 256 + r * 16 + (4 * s + g) * 2));
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          v8bf bf[NB];
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const uint32_t word = w == 0 ? cw[j].x : w == 1 ? cw[j].y : w == 2 ? cw[j].z : cw[j].w;
            bf[j] = dequant8(word, st[j], -8.0f * st[j]);
          }
          const int off = s * kBlk + w * 1024 + rdw + ((r ^ (4 * g + w)) & 15) * 16;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const v8bf af = *reinterpret_cast<const v8bf*>(abase + mb * 2 * kBlk + off);
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[mb][j] = mfma_bf16(af, bf[j], acc[mb][j]);
          }
        }
      }
    } else {
      const uint8_t* ab = abase + (u & 1) * kBlk;
      v4i w0[NB], w1[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        w0[j] = *reinterpret_cast<const v4i*>(wslot + j * 2048 + rd0);
        w1[j] = *reinterpret_cast<const v4i*>(wslot + j * 2048 + rd1);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const v4i a0 = *reinterpret_cast<const v4i*>(ab + mb * 2 * kBlk + rd0);
        const v4i a1 = *reinterpret_cast<const v4i*>(ab + mb * 2 * kBlk + rd1);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if constexpr (KIND == kGemmFP8) {
            acc[mb][j] = mfma_fp8(__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7),
                                  __builtin_shufflevector(w0[j], w1[j], 0, 1, 2, 3, 4, 5, 6, 7), acc[mb][j]);
          } else {
            acc[mb][j] = mfma_i8(a0, w0[j], acc[mb][j]);
            acc[mb][j] = mfma_i8(a1, w1[j], acc[mb][j]);
          }
        }
      }
    }
  };

  // ---- prologue: activation chunks 0 and 1 in registers, chunk 0 in LDS,
  // the weight ring filled
  aload(0, aset[0]);
  aload(1, aset[1]);
  Slot<KIND, NB> ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) wload(ring[d], d);
  awrite(aset[0], 0, 0);
  __syncthreads();

  // ---- main loop: DEPTH units per round. Activation chunk ci uses LDS
  // buffer ci & 1 and register set ci & 1; at its start the set is refilled
  // with chunk ci + 2, after its last unit chunk ci + 1 goes to the other
  // buffer. Each unit: its registers go to the wave's slot, the ring slot is
  // refilled DEPTH units ahead, then the unit is multiplied. Units past the
  // range multiply zero activations (clamped weight loads). The scheduling
  // barriers keep each refill right after the write that freed its slot.
  for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int u = rd * DEPTH + d;
      if (d % UPC == 0) aload(u / UPC + 2, aset[(d / UPC) & 1]);
      wstage(ring[d]);
      __builtin_amdgcn_sched_barrier(0);
      wload(ring[d], u + DEPTH);
      __builtin_amdgcn_sched_barrier(0);
      compute(u);
      if (d % UPC == UPC - 1) {
        awrite(aset[((d / UPC) + 1) & 1], u / UPC + 1, (u / UPC + 1) & 1);
        __syncthreads();
      }
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
  // Partial sums and the counter use device-scope relaxed atomic accesses,
  // which bypass the per-XCD L2 caches; a store is complete (vmcnt) once it
  // is visible device-wide, so waiting for the stores before the counter
  // increment orders them without a cache-wide write-back fence (a fence
  // here would flush and invalidate the whole L2 of the XCD on every
  // workgroup).
  if (S > 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = mb * 16 + 4 * g + i, n = n0 + 16 * j + r;
          if (m < p.M && n < p.N)
            __hip_atomic_store(&p.part[((size_t)split * p.M + m) * p.N + n],
                               KIND == kGemmI8 ? (uint32_t)acci[mb][j][i] : __float_as_uint(accf[mb][j][i]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial sums are visible
    __syncthreads();                // ... and those of the other waves
    if (tid == 0)
      last_flag = __hip_atomic_fetch_add(&p.cnt[blockIdx.x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  (unsigned)(S - 1);
    __syncthreads();
    if (!last_flag) return;
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
          const uint32_t u = __hip_atomic_load(&p.part[off[mb][j][i]], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if constexpr (KIND == kGemmI8) acci[mb][j][i] = (int)u;
          else accf[mb][j][i] = __uint_as_float(u);
        }
    for (int s = 1; s < S; ++s) {
      uint32_t* q = p.part + (size_t)s * stride;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t u = __hip_atomic_load(&q[off[mb][j][i]], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if constexpr (KIND == kGemmI8) acci[mb][j][i] += (int)u;
            else accf[mb][j][i] = accf[mb][j][i] + __uint_as_float(u);
          }
    }
    if (tid == 0) __hip_atomic_store(&p.cnt[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- epilogue
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
  int MB, NB, DEPTH;
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

// Per-kind tile shape: a wave takes two column blocks once the activation
// fragments it reads per weight byte would otherwise dominate (MB >= 3).
static int decode_nb(int kind, int MB) {
  if (kind == kGemmW4) return MB >= 2 ? 2 : 1;
  return MB >= 3 ? 2 : 1;
}

// Grid: 64*NB columns per workgroup, S splits of K. Split-K costs a write
// and a read of S*M*N partial sums, so it is used only to reach about three
// quarters of the CUs with column tiles; each split keeps >= 4 steps of
// 128 K. DEPTH (weight units in flight per wave) is the larger choice when
// the split's unit count is a multiple of it or large (a round computes
// DEPTH units; extra units are harmless but cost time).
static DecodeCfg decode_cfg(int kind, int64_t M, int64_t N, int64_t K) {
  DecodeCfg c{};
  c.MB = (int)((M + 15) / 16);
  c.NB = decode_nb(kind, c.MB);
  const int64_t cols = (int64_t)64 * c.NB;
  c.tiles = (int)((N + cols - 1) / cols);
  const int64_t ksteps = (K + 127) / 128;
  const int64_t want = 3 * (int64_t)decode_cus() / 4;
  int64_t S = (want + c.tiles - 1) / c.tiles;
  S = std::max<int64_t>(1, std::min<int64_t>(S, std::min<int64_t>(8, ksteps / 4)));
  if (const char* e = getenv("QLIN_DECODE_SPLIT")) S = std::max(1, atoi(e));  // tuning override
  if (c.tiles > (int)(kGemmCounterBytes / 4)) S = 1;  // one counter per tile; such grids need no split
  int64_t steps_per = (ksteps + S - 1) / S;
  steps_per = (steps_per + 1) / 2 * 2;  // whole 256-K chunks
  c.kc = (int)(steps_per * 128);
  c.S = (int)((K + c.kc - 1) / c.kc);
  const int64_t units = kind == kGemmW4 ? steps_per / 2 : steps_per;
  const int big = kind == kGemmW4 ? 4 : 8;
  c.DEPTH = (c.MB <= 2 && (units % big == 0 || units > 3 * big)) ? big : big / 2;
  return c;
}

// Dispatch on (kind, MB, DEPTH) to the instantiation that serves it.
template <typename F>
static auto with_decode_inst(int kind, int MB, int DEPTH, F&& f) {
#define QLIN_DEC(K, NB1, NB2, D)                                                        \
  switch (MB) {                                                                          \
    case 1: return DEPTH == 2 * D ? f.template operator()<K, 1, NB1, 2 * D>()            \
                                  : f.template operator()<K, 1, NB1, D>();               \
    case 2: return DEPTH == 2 * D ? f.template operator()<K, 2, NB2, 2 * D>()            \
                                  : f.template operator()<K, 2, NB2, D>();               \
    case 3: return f.template operator()<K, 3, 2, D>();                                  \
    default: return f.template operator()<K, 4, 2, D>();                                 \
  }
  if (kind == kGemmW4) {
    QLIN_DEC(kGemmW4, 1, 2, 2)
  } else if (kind == kGemmI8) {
    QLIN_DEC(kGemmI8, 1, 1, 4)
  } else {
    QLIN_DEC(kGemmFP8, 1, 1, 4)
  }
#undef QLIN_DEC
}

// Workspace of a split-K call: a fixed counter area (one word per column
// tile, at most kMaxTiles) at offset 0, then the partial sums. Every call
// leaves the counter area zero, and no call ever writes partials there, so a
// workspace zeroed once stays valid across calls of any shape.
constexpr size_t kCounterBytes = kGemmCounterBytes;

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
    decode_gemm_kernel<KIND, MB, NB, DEPTH><<<dim3((unsigned)c->tiles, (unsigned)c->S), 256, 0, st>>>(*a);
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
  with_decode_inst(kind, c.MB, c.DEPTH, LaunchFn{&g, &c, st});
  return launch_status();
}

}  // namespace qlin
