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
// Large FP8 / int8 problems use a persistent 256x256 kernel, one workgroup
// per CU; when K is a multiple of 128 (and at least 256) its stages are
// loaded straight into LDS by buffer loads, otherwise through registers.
#include <algorithm>
#include <type_traits>

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

// ----------------------------------------------------------------------------
// Large FP8 / int8 problems: persistent 256x256 tiles, software pipelined.
//
// One workgroup of 4 waves per CU loops over output tiles. A K stage is 128
// bytes of K for 256 rows of A and 256 rows of W (64 KB); two stages live in
// LDS. Each wave owns a 128x128 quadrant as 8x8 MFMA blocks and walks it in 8
// "rows" (one A block against the 8 W blocks). While a stage is multiplied:
//   * rows 0..6 write the next stage (already in registers) into the other
//     LDS buffer and issue the global loads of the stage after it;
//   * each row reads the A block of the following row;
//   * row 7 passes the one barrier of the stage, then refills each W block
//     register with the next stage's block right after its last MFMA.
// Global loads: one instruction covers 8 rows x 128 contiguous bytes (whole
// cache lines). LDS keeps every 16-row block "fragment-major": the 16-byte
// piece that MFMA lane (g, r) needs for K half h (chunk c = 4h + g of row r)
// sits at h*1024 + g*256 + 16*((r ^ c) & 15), so both the fragment reads
// (16 lanes of one chunk, r = 0..15) and the line-shaped staging writes (8
// lanes per 128-byte write cycle holding chunks c = 0..7 of one row) hit
// distinct banks.
// The MFMA takes the W block as its first operand, so each lane ends with 4
// consecutive output columns of one row: the epilogue stores 8 (bf16) or 16
// (fp32) bytes per lane per block. The next tile's first loads are issued
// before the epilogue so they overlap the stores.
// Tiles are visited in grouped order, and each round of the workgroups hands
// every XCD a compact block of tiles (workgroups are dispatched round-robin
// over the XCDs), so tiles that share A rows or W rows share an L2.
template <int KIND, bool KTAIL>
__global__ __launch_bounds__(256) void prefill_big_kernel(const PrefillArgs p, int tiles_m,
                                                          int tiles_n) {
  constexpr int kStage = 65536, kWOff = 32768;
  using Acc = typename std::conditional<KIND == kGemmI8, v4i, v4f>::type;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];
  __shared__ __attribute__((aligned(16))) float lds_sc[512];  // the tile's s_a rows, then s_w columns

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, r = lane & 15;
  const int KT = (p.K + 127) >> 7;
  const int tiles = tiles_m * tiles_n, G = gridDim.x;
  const int slot = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;

  // Staging slot q (0..15) of this thread: load instruction 4q + wave, i.e.
  // tile row srow + 32q of A (q < 8) or of W (q >= 8, row srow + 32(q-8)),
  // 16-byte chunk c of the stage's 128 K bytes.
  const int c = lane & 7;
  const int srow = 8 * wave + (lane >> 3);
  const int kofs = 16 * c;
  const int wr_off = (wave >> 1) * 2048 + (c >> 2) * 1024 + (c & 3) * 256 + (((srow & 15) ^ c) * 16);
  const int rd0 = g * 256 + ((r ^ g) * 16);
  const int rd1 = 1024 + g * 256 + ((r ^ (4 + g)) * 16);
  const int ra = wm * 16384, rb = kWOff + wn * 16384;

  uint4 st[16];
  v8i bf[8];  // W blocks of the current stage
  Acc acc[8][8];

  auto tile_origin = [&](int t, int& m0, int& n0) {
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int first_m = (t / per_group) * GM;
    const int gsz = min(tiles_m - first_m, GM);
    m0 = (first_m + (t % per_group) % gsz) * 256;
    n0 = ((t % per_group) / gsz) * 256;
  };
  // Staging addresses: 32-bit byte offsets from the uniform matrix base (the
  // launch checks that M*lda and N*K fit), the row clamp applied to the
  // offset (rows are lda / K bytes apart), then the clamped K chunk.
  const uint32_t lda = (uint32_t)p.lda, ldw = (uint32_t)p.K;
  const uint32_t arow = (uint32_t)srow * lda, wrow = (uint32_t)srow * ldw;
  const uint32_t amax = (uint32_t)(p.M - 1) * lda, wmax = (uint32_t)(p.N - 1) * ldw;
  auto gload_one = [&](int q, int kt, int m0, int n0) {
    const uint32_t kc = (uint32_t)min(kt * 128 + kofs, p.K - 16);
    if (q < 8) {
      const uint32_t o = min((uint32_t)m0 * lda + (uint32_t)(32 * q) * lda + arow, amax) + kc;
      st[q] = ldg16(p.A + o);
    } else {
      const uint32_t o = min((uint32_t)n0 * ldw + (uint32_t)(32 * (q - 8)) * ldw + wrow, wmax) + kc;
      st[q] = ldg16(p.W + o);
    }
  };
  // LDS write of staging slot q (stage kt) into buffer `buf`; A chunks past K
  // are zeroed (only when K is not a multiple of 128)
  auto swrite = [&](int q, int kt, int buf) {
    uint4 v = st[q];
    if (KTAIL && q < 8) {
      const uint32_t keep = kt * 128 + kofs < p.K ? 0xFFFFFFFFu : 0u;
      v = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
    }
    *reinterpret_cast<uint4*>(lds + buf * kStage + wr_off + 4096 * q) = v;
  };
  auto frag = [&](int off) {
    const v4i lo = *reinterpret_cast<const v4i*>(lds + off + rd0);
    const v4i hi = *reinterpret_cast<const v4i*>(lds + off + rd1);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto mma = [&](int i, int j, const v8i& a, const v8i& w) {
    if constexpr (KIND == kGemmFP8) {
      acc[i][j] = mfma_fp8(w, a, acc[i][j]);
    } else {
      acc[i][j] = mfma_i8(__builtin_shufflevector(w, w, 0, 1, 2, 3), __builtin_shufflevector(a, a, 0, 1, 2, 3), acc[i][j]);
      acc[i][j] = mfma_i8(__builtin_shufflevector(w, w, 4, 5, 6, 7), __builtin_shufflevector(a, a, 4, 5, 6, 7), acc[i][j]);
    }
  };

  // The (tile, K stage) pairs of this workgroup form one stream: position
  // pos = n*KT + kt is stage kt of its n-th tile (tile slot + n*G). The
  // pipeline runs across tile boundaries; only the accumulators are flushed.
  // (branch-free: a branch inside the stage body would let the compiler
  // regroup the MFMAs away from the memory operations they hide)
  auto stream_origin = [&](int pos, int& m0, int& n0, int& kk) {
    const int tt = slot + (pos / KT) * G;
    const bool live = tt < tiles;  // past the last tile: a harmless reload of valid memory
    tile_origin(live ? tt : slot, m0, n0);
    kk = live ? pos % KT : KT - 1;
  };

  if (slot >= tiles) return;
  {
    int m0, n0, kk;
    stream_origin(0, m0, n0, kk);
#pragma unroll
    for (int q = 0; q < 16; ++q) gload_one(q, kk, m0, n0);
#pragma unroll
    for (int q = 0; q < 16; ++q) swrite(q, kk, 0);
    stream_origin(1, m0, n0, kk);
#pragma unroll
    for (int q = 0; q < 16; ++q) gload_one(q, kk, m0, n0);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = Acc{0, 0, 0, 0};
  __syncthreads();
  v8i af = frag(ra);
#pragma unroll
  for (int j = 0; j < 8; ++j) bf[j] = frag(rb + 2048 * j);

  int pos = 0;
  for (int t = slot; t < tiles; t += G) {
    int m0, n0;
    tile_origin(t, m0, n0);
    for (int kt = 0; kt < KT; ++kt, ++pos) {
      const int cur = pos & 1, nxt = cur ^ 1;
      const int kw = (pos + 1) % KT;  // stage being written (its K tail mask)
      int lm0, ln0, kl;               // stage being loaded
      stream_origin(pos + 2, lm0, ln0, kl);
      // the tile's scales go to LDS in every stage (unconditionally, see
      // above); the epilogue reads them after the last stage's barrier
      const float sc_a = p.sa[min(m0 + tid, p.M - 1)];
      const float sc_w = p.sw[min(n0 + tid, p.N - 1)];
#pragma unroll
      for (int i = 0; i < 7; ++i) {
        const v8i an = frag(cur * kStage + ra + 2048 * (i + 1));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          mma(i, j, af, bf[j]);
          // staging slots of this row: rows 0,1 take three, rows 2..6 two
          const int q = i < 2 ? 3 * i + (j >> 1) : 6 + 2 * (i - 2) + (j >> 2);
          const bool here = i < 2 ? ((j & 1) && j < 6) : ((j & 3) == 1);
          if (here) {
            swrite(q, kw, nxt);
            gload_one(q, kl, lm0, ln0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        af = an;
      }
      lds_sc[tid] = sc_a;
      lds_sc[256 + tid] = sc_w;
      // row 7: barrier, then the next stage's first A block and W blocks
      mma(7, 0, af, bf[0]);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      const v8i an = frag(nxt * kStage + ra);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j > 0) mma(7, j, af, bf[j]);
        bf[j] = frag(nxt * kStage + rb + 2048 * j);
        __builtin_amdgcn_sched_barrier(0);
      }
      af = an;
    }

    // ---- epilogue. Output element (m, n) of block (i, j): lane (g, r) holds
    // row m = .. + 16i + r, columns n = .. + 16j + 4g + e, e = 0..3.
    // The lane index is made opaque here so that the epilogue's lane-derived
    // offsets are computed where they are used rather than hoisted to the
    // kernel entry (where they would only add to register pressure).
    int el = lane;
    asm volatile("" : "+v"(el));
    const int eg = el >> 4, er = el & 15;
    // The next stage's fragments, loaded by the last row 7, are read again
    // after the epilogue, so they are not live across it; scales are read
    // from LDS where they are used.
    auto scaled = [&](int i, int j, int e) {
      const float sa_i = lds_sc[wm * 128 + i * 16 + er];
      const float sw_e = lds_sc[256 + wn * 128 + j * 16 + 4 * eg + e];
      if constexpr (KIND == kGemmI8) return ((float)acc[i][j][e] * sa_i) * sw_e;
      else return (acc[i][j][e] * sa_i) * sw_e;
    };
    if (p.out_f32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = m0 + wm * 128 + i * 16 + er;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int n = n0 + wn * 128 + j * 16 + 4 * eg;
          if (m < p.M && n < p.N)
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.y) + (size_t)m * p.N + n) =
                make_float4(scaled(i, j, 0), scaled(i, j, 1), scaled(i, j, 2), scaled(i, j, 3));
        }
      }
    } else {
      // bf16: transpose through the LDS buffer the last stage used (free after
      // its barrier), 32 rows of the wave's quadrant at a time, so every
      // store writes whole 256-byte row segments. Rows are padded to 272
      // bytes, which spreads both access shapes over the banks.
      uint8_t* ep = lds + ((pos - 1) & 1) * kStage + wave * (32 * 272);
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = pass * 2 + ii;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t lo = f32_bf16_rne(scaled(i, j, 0)) | (f32_bf16_rne(scaled(i, j, 1)) << 16);
            const uint32_t hi = f32_bf16_rne(scaled(i, j, 2)) | (f32_bf16_rne(scaled(i, j, 3)) << 16);
            *reinterpret_cast<uint2*>(ep + (ii * 16 + er) * 272 + j * 32 + eg * 8) = make_uint2(lo, hi);
          }
        }
        // (LDS operations of one wave complete in order: no wait needed here)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int R = 4 * k + eg, ch = er;
          const uint4 v = *reinterpret_cast<const uint4*>(ep + R * 272 + ch * 16);
          const int m = m0 + wm * 128 + pass * 32 + R;
          const int n = n0 + wn * 128 + 8 * ch;
          if (m < p.M && n < p.N)
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.y) + (size_t)m * p.N + n) = v;
        }
      }
    }
    // the next stage writes the epilogue's LDS buffer and the next scales
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = Acc{0, 0, 0, 0};
    af = frag((pos & 1) * kStage + ra);
#pragma unroll
    for (int j = 0; j < 8; ++j) bf[j] = frag((pos & 1) * kStage + rb + 2048 * j);
  }
}

// ----------------------------------------------------------------------------
// The persistent 256x256 FP8 / int8 GEMM with direct-to-LDS staging (K a
// multiple of 128, at least 256). Each stage's 64 KB arrive through
// buffer_load_dwordx4 ... lds: the memory system writes every lane's 16 bytes
// straight into LDS (lane i of an instruction at byte 16 i of a 1 KB block),
// so staging takes no VGPRs and no LDS write instructions. LDS is row-major (128 bytes of K per row); chunk
// c of row R sits in slot c ^ ((R >> 1) & 7), so one instruction (8 rows,
// 8 lanes per row reading one whole 128-byte line) fills 1 KB contiguously
// and a fragment read (16 lanes, one chunk of 16 consecutive rows) touches
// every bank once.
// Stage s is multiplied in 8 rows of 8 MFMAs. The stage barrier comes after
// row 6: by then each wave has waited for its own loads of stage s + 1, and
// every wave has read all of stage s it needs (row 7's blocks are in
// registers). Row 7 then overlaps the reads of stage s + 1's fragments (each
// W block register refilled right after its last MFMA) and the first loads
// of stage s + 2 into the buffer stage s just released; the rest of those
// loads follow during the first rows of stage s + 1.
// The bf16 epilogue has an LDS area of its own and the scales two copies
// (by tile parity), so loads stay in flight across it and it needs no
// barrier.
template <int KIND>
__global__ __launch_bounds__(256) void prefill_dma_kernel(const PrefillArgs p, int tiles_m,
                                                          int tiles_n) {
  constexpr int kStage = 65536, kWOff = 32768, kEpiRow = 272, kEpi = 16 * kEpiRow;
  using Acc = typename std::conditional<KIND == kGemmI8, v4i, v4f>::type;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];
  __shared__ __attribute__((aligned(16))) float lds_sc[2][512];  // per tile parity: s_a rows, then s_w columns
  __shared__ __attribute__((aligned(16))) uint8_t lds_ep[4 * kEpi];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, r = lane & 15;
  const int KT = p.K >> 7;
  const int tiles = tiles_m * tiles_n, G = gridDim.x;
  const int slot = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;

  // Load q (0..15) of this thread fills 1 KB block 4q + wave of A (q < 8) or
  // W (q >= 8): tile row srow + 32q (or + 32(q-8)), chunk c of the stage.
  const int srow = 8 * wave + (lane >> 3);
  const int c = (lane & 7) ^ (4 * (wave & 1) + (lane >> 4));
  const uint32_t kofs = 16u * (uint32_t)c;
  const int rd0 = r * 128 + ((g ^ (r >> 1)) * 16);
  const int rd1 = r * 128 + (((4 + g) ^ (r >> 1)) * 16);
  const int ra = wm * 16384, rb = kWOff + wn * 16384;

  v8i bf[8];  // W blocks of the current stage
  Acc acc[8][8];

  auto tile_origin = [&](int t, int& m0, int& n0) {
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int first_m = (t / per_group) * GM;
    const int gsz = min(tiles_m - first_m, GM);
    m0 = (first_m + (t % per_group) % gsz) * 256;
    n0 = ((t % per_group) / gsz) * 256;
  };
  // Loads are raw buffer loads (buffer_load_dwordx4 ... lds). The resource
  // of a (matrix, tile, K stage) starts at the stage's first byte of the
  // tile's first row and ends with the matrix, so rows past M (or N) are out
  // of range: they read nothing (only outputs that are never stored depend
  // on them). Each thread's 16 row offsets are fixed for the whole kernel;
  // per stage only scalar registers change.
  const uint32_t lda = (uint32_t)p.lda, ldw = (uint32_t)p.K;
  uint32_t vo[16];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    vo[q] = (uint32_t)(32 * q + srow) * lda + kofs;
    vo[8 + q] = (uint32_t)(32 * q + srow) * ldw + kofs;
  }
  auto rsrc = [&](const uint8_t* base, uint32_t ld, int rows_left, int kt) {
    const uint64_t b = (uint64_t)(uintptr_t)(base + (size_t)kt * 128);
    v4i r;
    r.x = (int)(uint32_t)b;
    r.y = (int)(uint32_t)(b >> 32);  // stride 0 (raw buffer)
    r.z = (int)((uint32_t)rows_left * ld - (uint32_t)kt * 128u);
    r.w = 0x00020000;  // gfx9 data format field (32-bit) as untyped loads need it
    return r;
  };
  // Written as inline assembly: the compiler would otherwise treat every
  // later LDS read as possibly aliasing the load and wait for all loads in
  // flight before it. The kernel orders them itself (each wave waits for its
  // own loads before the stage barrier, and before it exits).
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  auto dma = [&](int q, const v4i& rs, int buf) {
    const uint32_t dst = lds_base + (uint32_t)(buf * kStage + 4096 * q + 1024 * wave);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(dst), "v"(vo[q]), "s"(rs)
                 : "memory", "m0");
  };
  // the resources of stage kt of the tile at (m0, n0): A, then W
  // Each XCD walks K from its own starting stage (k0, wrapping around), so
  // the XCDs finish their tiles at different times and the bursts of output
  // stores spread out; the workgroups of one XCD stay in step and keep
  // sharing their A and W slices in L2.
  const int k0 = (int)(((uint32_t)blockIdx.x % 8u) * (uint32_t)KT / 8u);
  auto stage_rs = [&](int m0, int n0, int kt, v4i& ra_, v4i& rw_) {
    const int kp = kt + k0 < KT ? kt + k0 : kt + k0 - KT;
    ra_ = rsrc(p.A + (size_t)m0 * lda, lda, p.M - m0, kp);
    rw_ = rsrc(p.W + (size_t)n0 * ldw, ldw, p.N - n0, kp);
  };
  auto frag = [&](int off) {
    const v4i lo = *reinterpret_cast<const v4i*>(lds + off + rd0);
    const v4i hi = *reinterpret_cast<const v4i*>(lds + off + rd1);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto mma = [&](int i, int j, const v8i& a, const v8i& w) {
    if constexpr (KIND == kGemmFP8) {
      acc[i][j] = mfma_fp8(w, a, acc[i][j]);
    } else {
      acc[i][j] = mfma_i8(__builtin_shufflevector(w, w, 0, 1, 2, 3), __builtin_shufflevector(a, a, 0, 1, 2, 3), acc[i][j]);
      acc[i][j] = mfma_i8(__builtin_shufflevector(w, w, 4, 5, 6, 7), __builtin_shufflevector(a, a, 4, 5, 6, 7), acc[i][j]);
    }
  };
  // load d of a stage is issued after MFMA number d * kSpread, counted from
  // row 7 of the stage before (the 16 loads occupy the address unit for about
  // half a stage; spreading them wider leaves the last too little time)
  constexpr int kSpread = 2;
  constexpr int kEarly = (8 + kSpread - 1) / kSpread;  // loads issued in row 7

  if (slot >= tiles) return;
  {
    int m0, n0;
    tile_origin(slot, m0, n0);
    v4i r0, r1;
    stage_rs(m0, n0, 0, r0, r1);
#pragma unroll
    for (int q = 0; q < 16; ++q) dma(q, q < 8 ? r0 : r1, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // the first loads of the first step (stage 1), as a row 7 would issue them
    stage_rs(m0, n0, 1, r0, r1);
#pragma unroll
    for (int q = 0; q < kEarly; ++q) dma(q, q < 8 ? r0 : r1, 1);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = Acc{0, 0, 0, 0};
  v8i af = frag(ra);
#pragma unroll
  for (int j = 0; j < 8; ++j) bf[j] = frag(rb + 2048 * j);

  // The stream of (tile, K stage) pairs is cut after each stage barrier:
  // one step is row 7 of stage s - 1 followed by rows 0..6 of stage s, so
  // nothing is pending on the LDS counter where a step begins. All loads of
  // one step go to stage s + 1 (for s + 1 = KT: stage 0 of the workgroup's
  // next tile). A stage's data sits in LDS buffer (position in the stream)
  // & 1.
  //
  // Row 7 of the stage before the one in buffer nb: its MFMAs, the refill of
  // the W block registers and row 0's A block from buffer nb, and the first
  // loads of the step (resources ra_/rw_) into buffer nb ^ 1.
  auto row7 = [&](int nb, const v4i& ra_, const v4i& rw_) {
    const v8i an = frag(nb * kStage + ra);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mma(7, j, af, bf[j]);
      bf[j] = frag(nb * kStage + rb + 2048 * j);
      if (j % kSpread == 0) dma(j / kSpread, j / kSpread < 8 ? ra_ : rw_, nb ^ 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    af = an;
  };
  // Rows 0..6 of the stage in buffer cb (tile at m0, n0; scale copy tp), the
  // remaining loads of the step into buffer cb ^ 1, then the stage barrier.
  // After row 3 (when the step's loads are all issued) `next` computes the
  // next step's resources.
  auto rows06 = [&](int cb, int m0, int n0, int tp, const v4i& ra_, const v4i& rw_, auto&& next) {
    const float sc_a = p.sa[min(m0 + tid, p.M - 1)];
    const float sc_w = p.sw[min(n0 + tid, p.N - 1)];
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      const v8i an = frag(cb * kStage + ra + 2048 * (i + 1));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        mma(i, j, af, bf[j]);
        const int sl = 8 + 8 * i + j;
        if (sl % kSpread == 0 && sl / kSpread < 16) dma(sl / kSpread, sl / kSpread < 8 ? ra_ : rw_, cb ^ 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      af = an;
      if (i == 3) {
        next();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lds_sc[tp][tid] = sc_a;
    lds_sc[tp][256 + tid] = sc_w;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  int tp = 0, cb = 0;
  v4i sa_rs, sw_rs;  // resources of the current step's loads
  {
    int m0, n0;
    tile_origin(slot, m0, n0);
    stage_rs(m0, n0, 1, sa_rs, sw_rs);
  }
  for (int t = slot; t < tiles; t += G, tp ^= 1) {
    int m0, n0, nm0, nn0;
    tile_origin(t, m0, n0);
    // the stages loaded ahead past this tile's last belong to the next tile
    // of the workgroup; past the last tile they reload this tile's last stage
    const bool nlive = t + G < tiles;
    tile_origin(nlive ? t + G : t, nm0, nn0);
    // resources of the loads for stage kt (kt >= KT: the next tile's)
    v4i na_rs, nw_rs;
    auto next_rs = [&](int kt) {
      const bool in = kt < KT;
      stage_rs(in ? m0 : nm0, in ? n0 : nn0, in ? kt : (nlive ? kt - KT : KT - 1), na_rs, nw_rs);
    };
    rows06(cb, m0, n0, tp, sa_rs, sw_rs, [&] { next_rs(2); });
    sa_rs = na_rs;
    sw_rs = nw_rs;
    for (int kt = 1; kt < KT; ++kt) {
      row7(cb ^ 1, sa_rs, sw_rs);
      cb ^= 1;
      rows06(cb, m0, n0, tp, sa_rs, sw_rs, [&] { next_rs(kt + 2); });
      sa_rs = na_rs;
      sw_rs = nw_rs;
    }
    // the tile's last row 7; its loads are the next tile's stage 1
    row7(cb ^ 1, sa_rs, sw_rs);
    cb ^= 1;

    // ---- epilogue (see the kernel above for the lane layout)
    int el = lane;
    asm volatile("" : "+v"(el));
    const int eg = el >> 4, er = el & 15;
    auto scaled = [&](int i, int j, int e) {
      const float sa_i = lds_sc[tp][wm * 128 + i * 16 + er];
      const float sw_e = lds_sc[tp][256 + wn * 128 + j * 16 + 4 * eg + e];
      if constexpr (KIND == kGemmI8) return ((float)acc[i][j][e] * sa_i) * sw_e;
      else return (acc[i][j][e] * sa_i) * sw_e;
    };
    if (p.out_f32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = m0 + wm * 128 + i * 16 + er;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int n = n0 + wn * 128 + j * 16 + 4 * eg;
          if (m < p.M && n < p.N)
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.y) + (size_t)m * p.N + n) =
                make_float4(scaled(i, j, 0), scaled(i, j, 1), scaled(i, j, 2), scaled(i, j, 3));
        }
      }
    } else {
      // bf16: transpose one 16-row block at a time through the wave's own
      // LDS area (rows padded to 272 bytes), storing whole 256-byte row
      // segments; the wave's LDS operations complete in order
      uint8_t* ep = lds_ep + wave * kEpi;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t lo = pack_bf16x2(scaled(i, j, 0), scaled(i, j, 1));
          const uint32_t hi = pack_bf16x2(scaled(i, j, 2), scaled(i, j, 3));
          *reinterpret_cast<uint2*>(ep + er * kEpiRow + j * 32 + eg * 8) = make_uint2(lo, hi);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int R = 4 * k + eg, ch = er;
          const uint4 v = *reinterpret_cast<const uint4*>(ep + R * kEpiRow + ch * 16);
          const int m = m0 + wm * 128 + i * 16 + R;
          const int n = n0 + wn * 128 + 8 * ch;
          // (nontemporal: the output is not read again here)
          if (m < p.M && n < p.N)
            __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(&v),
                                        reinterpret_cast<v4i*>(reinterpret_cast<uint16_t*>(p.y) + (size_t)m * p.N + n));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = Acc{0, 0, 0, 0};
    // the next stage's blocks (read by the last row 7) are read again here
    // rather than kept live across the epilogue
    af = frag(cb * kStage + ra);
#pragma unroll
    for (int j = 0; j < 8; ++j) bf[j] = frag(cb * kStage + rb + 2048 * j);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ----------------------------------------------------------------------------
// Large W4A16 problems (K a multiple of 64, at least 128): the persistent
// 256x256 kernel of the FP8 path with bf16 MFMAs (16x16x32) and the weights
// unpacked in registers. A K stage is 64 elements: 256 rows of bf16 A (32 KB,
// laid out and loaded as the FP8 kernel's stage), the int4 codes of 256
// columns (8 KB, 32 bytes per column) and their group steps (1 KB, two per
// column), all loaded straight into LDS by buffer loads.
// K order inside a stage: MFMA lane group g of K step s takes the stage's
// elements 32s + 8g .. 32s + 8g + 7 (group s of the stage), for A and W
// alike: a lane's A piece for step s is the 16-byte chunk 4s + g of the row
// (the FP8 kernel's fragment reads, conflict-free; the order 16g + 8s, which
// would make a lane's codes one 8-byte read, measured 4 bank-conflict cycles
// per A read) and its codes are dwords g and 4 + g of the column's 32 bytes.
// In LDS the two 16-byte halves of a column's codes swap places when bit 3
// of the column is set, which spreads the dword code reads over all banks.
// Each wave owns 64 columns of the tile and all 256 rows, so every weight
// is unpacked once per tile (the unpack, 17 VALU operations per 8 weights,
// is this kernel's second largest cost after the MFMAs). The 32 A pieces of
// a stage stay in registers; the wave walks its 4 column blocks, K step 0 of
// the 16 row blocks then K step 1 (no MFMA waits for the one before it), and
// spreads the unpack of the next column block over the current block's
// MFMAs. The stage barrier comes after column block 2; column block 3
// overlaps the refill of the A pieces and the unpack of the next stage's
// first block with its MFMAs (as row 7 does in the FP8 kernel).
__global__ __launch_bounds__(256) void prefill_w4_kernel(const PrefillArgs p, int tiles_m, int tiles_n) {
  constexpr int kCOff = 32768, kSOff = 40960, kBuf = 41984;  // A | codes | steps
  constexpr int kEpiRow = 144, kEpi = 16 * kEpiRow;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kBuf];
  __shared__ __attribute__((aligned(16))) uint8_t lds_ep[4 * kEpi];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int KT = p.K >> 6;
  const int tiles = tiles_m * tiles_n, G = gridDim.x;
  const int slot = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;

  // A loads q = 0..7: 1 KB block 4q + wave (tile rows srow + 32q), chunk c
  const int srow = 8 * wave + (lane >> 3);
  const int c = (lane & 7) ^ (4 * (wave & 1) + (lane >> 4));
  const uint32_t lda2 = (uint32_t)p.lda * 2u, kb2 = (uint32_t)p.K / 2u, ks2 = (uint32_t)p.K / 16u;
  uint32_t vo[11];
#pragma unroll
  for (int q = 0; q < 8; ++q) vo[q] = (uint32_t)(32 * q + srow) * lda2 + 16u * (uint32_t)c;
  // code loads h = 0, 1: columns 32 (2 wave + h) + lane / 2, 16-byte half
  // lane & 1 of the column's 32 bytes, swapped for columns with bit 3 set
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int cc = 32 * (2 * wave + h) + (lane >> 1);
    vo[8 + h] = (uint32_t)cc * kb2 + 16u * (uint32_t)((lane & 1) ^ ((cc >> 3) & 1));
  }
  vo[10] = (uint32_t)(64 * wave + lane) * ks2;  // step load: 4 bytes of column 64 wave + lane
  // LDS read offsets: A piece of K step s (row r of a 16-row block), codes
  // and step of column 64 wave + r (+ 16 per column block)
  const int rdA0 = r * 128 + ((g ^ (r >> 1)) & 7) * 16;
  const int rdA1 = r * 128 + (((4 + g) ^ (r >> 1)) & 7) * 16;
  const int sw4 = ((r >> 3) & 1) * 4;  // code dword d of the column sits at d ^ sw4
  const int rdC0 = kCOff + (64 * wave + r) * 32 + 4 * (g ^ sw4);
  const int rdC1 = kCOff + (64 * wave + r) * 32 + 4 * ((4 + g) ^ sw4);
  const int rdS = kSOff + (64 * wave + r) * 4;

  v8bf af[16][2];  // A pieces of the current stage
  v8bf bw[2][2];   // unpacked W: column block j in bw[j & 1]
  v4f acc[16][4];

  auto tile_origin = [&](int t, int& m0, int& n0) {
    constexpr int GM = 8;
    const int per_group = GM * tiles_n;
    const int first_m = (t / per_group) * GM;
    const int gsz = min(tiles_m - first_m, GM);
    m0 = (first_m + (t % per_group) % gsz) * 256;
    n0 = ((t % per_group) / gsz) * 256;
  };
  auto rsrc = [&](const uint8_t* base, uint64_t bytes_left) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    v4i rr;
    rr.x = (int)(uint32_t)b;
    rr.y = (int)(uint32_t)(b >> 32);
    rr.z = (int)(uint32_t)bytes_left;
    rr.w = 0x00020000;
    return rr;
  };
  struct Rs {
    v4i a, c, s;
  };
  const int k0 = (int)(((uint32_t)blockIdx.x % 8u) * (uint32_t)KT / 8u);
  const uint8_t* steps8 = reinterpret_cast<const uint8_t*>(p.steps);
  auto stage_rs = [&](int m0, int n0, int kt) {
    const int kp = kt + k0 < KT ? kt + k0 : kt + k0 - KT;
    Rs q;
    q.a = rsrc(p.A + (size_t)m0 * lda2 + (size_t)kp * 128, (uint64_t)(p.M - m0) * lda2 - (uint64_t)kp * 128);
    q.c = rsrc(p.W + (size_t)n0 * kb2 + (size_t)kp * 32, (uint64_t)(p.N - n0) * kb2 - (uint64_t)kp * 32);
    q.s = rsrc(steps8 + (size_t)n0 * ks2 + (size_t)kp * 4, (uint64_t)(p.N - n0) * ks2 - (uint64_t)kp * 4);
    return q;
  };
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  // load d (0..10) of a stage into buffer buf (inline assembly: see the FP8
  // kernel)
  auto dma = [&](int d, const Rs& q, int buf) {
    if (d < 8) {
      const uint32_t dst = lds_base + (uint32_t)(buf * kBuf + 4096 * d + 1024 * wave);
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(dst), "v"(vo[d]), "s"(q.a)
                   : "memory", "m0");
    } else if (d < 10) {
      const uint32_t dst = lds_base + (uint32_t)(buf * kBuf + kCOff + 1024 * (2 * wave + d - 8));
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(dst), "v"(vo[d]), "s"(q.c)
                   : "memory", "m0");
    } else {
      const uint32_t dst = lds_base + (uint32_t)(buf * kBuf + kSOff + 256 * wave);
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(dst), "v"(vo[10]), "s"(q.s)
                   : "memory", "m0");
    }
  };
  auto apiece = [&](int off) { return *reinterpret_cast<const v8bf*>(lds + off); };
  // The unpack of one column block, in pieces placed between MFMAs:
  // piece 0 reads the two code words and the column's two steps, 1 and 6
  // turn a step into the unpack constants, 2..5 and 6..9 unpack a word.
  struct Unpack {
    uint32_t w0, w1, sb;
    Int4Step st;
    uint32_t t, p0, p1, p2, p3;
    float f[8];
  };
  auto unpack_piece = [&](int k, int bb, int j, Unpack& u, v8bf& out0, v8bf& out1) {
    constexpr uint32_t kMagic = 0x64006400u;
    switch (k) {
      case 0:
        u.w0 = *reinterpret_cast<const uint32_t*>(lds + bb * kBuf + rdC0 + 512 * j);
        u.w1 = *reinterpret_cast<const uint32_t*>(lds + bb * kBuf + rdC1 + 512 * j);
        u.sb = *reinterpret_cast<const uint32_t*>(lds + bb * kBuf + rdS + 64 * j);
        break;
      case 1: u.st = int4_step(__uint_as_float(u.sb << 16)); break;
      case 2: case 6: {
        if (k == 6) u.st = int4_step(__uint_as_float(u.sb & 0xFFFF0000u));
        const uint32_t x = k == 2 ? u.w0 : u.w1;
        u.t = x >> 8;
        u.p0 = and_or(x, 0x000F000Fu, kMagic);
        u.p1 = and_or(x, 0x00F000F0u, kMagic);
        break;
      }
      case 3: case 7:
        u.p2 = and_or(u.t, 0x000F000Fu, kMagic);
        u.p3 = and_or(u.t, 0x00F000F0u, kMagic);
        u.f[0] = fma_mix_lo(u.p0, u.st.s, u.st.off);
        u.f[4] = fma_mix_hi(u.p0, u.st.s, u.st.off);
        break;
      case 4: case 8:
        u.f[1] = fma_mix_lo(u.p1, u.st.s16, u.st.off16);
        u.f[5] = fma_mix_hi(u.p1, u.st.s16, u.st.off16);
        u.f[2] = fma_mix_lo(u.p2, u.st.s, u.st.off);
        u.f[6] = fma_mix_hi(u.p2, u.st.s, u.st.off);
        break;
      default: {  // 5, 9
        u.f[3] = fma_mix_lo(u.p3, u.st.s16, u.st.off16);
        u.f[7] = fma_mix_hi(u.p3, u.st.s16, u.st.off16);
        v4i q = {(int)pack_bf16x2(u.f[0], u.f[1]), (int)pack_bf16x2(u.f[2], u.f[3]),
                 (int)pack_bf16x2(u.f[4], u.f[5]), (int)pack_bf16x2(u.f[6], u.f[7])};
        (k == 5 ? out0 : out1) = __builtin_bit_cast(v8bf, q);
      }
    }
  };
  auto mma = [&](int i, int j, int s) { acc[i][j] = mfma_bf16(bw[j & 1][s], af[i][s], acc[i][j]); };
  // load d of a step is issued after MFMA number 4 d + 1 of the step (the
  // step's first 32 MFMAs are column block 3 of the stage before)
  constexpr int kEarly = 8;  // loads issued in column block 3

  if (slot >= tiles) return;
  {
    int m0, n0;
    tile_origin(slot, m0, n0);
    const Rs q0 = stage_rs(m0, n0, 0);
#pragma unroll
    for (int d = 0; d < 11; ++d) dma(d, q0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const Rs q1 = stage_rs(m0, n0, 1);
#pragma unroll
    for (int d = 0; d < kEarly; ++d) dma(d, q1, 1);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    af[i][0] = apiece(2048 * i + rdA0);
    af[i][1] = apiece(2048 * i + rdA1);
  }
  {
    Unpack u;
#pragma unroll
    for (int k = 0; k < 10; ++k) unpack_piece(k, 0, 0, u, bw[0][0], bw[0][1]);
  }

  // Column block 3 of the stage before the one in buffer nb, with the
  // refill of the A pieces and the unpack of column block 0 from buffer nb,
  // and the first loads of the step (resources q) into buffer nb ^ 1.
  auto col3 = [&](int nb, const Rs& q) {
    Unpack u;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const int i = t & 15, s = t >> 4;
      mma(i, 3, s);
      if (s == 1) {
        af[i][0] = apiece(nb * kBuf + 2048 * i + rdA0);
        af[i][1] = apiece(nb * kBuf + 2048 * i + rdA1);
      }
      if (t % 3 == 2 && t / 3 < 10) unpack_piece(t / 3, nb, 0, u, bw[0][0], bw[0][1]);
      if (t % 4 == 1) dma(t / 4, q, nb ^ 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Column blocks 0..2 of the stage in buffer cb, the remaining loads of the
  // step into buffer cb ^ 1, then the stage barrier; `next` computes the
  // next step's resources once its loads are issued.
  auto cols02 = [&](int cb, const Rs& q, auto&& next) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      Unpack u;
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        mma(t & 15, j, t >> 4);  // consecutive MFMAs on different accumulators
        // (one unpack piece after every third MFMA)
        if (t % 3 == 1 && t / 3 < 10) unpack_piece(t / 3, cb, j + 1, u, bw[(j + 1) & 1][0], bw[(j + 1) & 1][1]);
        const int sl = 32 * (j + 1) + t;
        if (sl % 4 == 1 && sl / 4 < 11) dma(sl / 4, q, cb ^ 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j == 1) {
        next();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  int cb = 0;
  Rs cur_rs;
  {
    int m0, n0;
    tile_origin(slot, m0, n0);
    cur_rs = stage_rs(m0, n0, 1);
  }
  for (int t = slot; t < tiles; t += G) {
    int m0, n0, nm0, nn0;
    tile_origin(t, m0, n0);
    const bool nlive = t + G < tiles;
    tile_origin(nlive ? t + G : t, nm0, nn0);
    Rs nrs;
    auto next_rs = [&](int kt) {
      const bool in = kt < KT;
      nrs = stage_rs(in ? m0 : nm0, in ? n0 : nn0, in ? kt : (nlive ? kt - KT : KT - 1));
    };
    cols02(cb, cur_rs, [&] { next_rs(2); });
    cur_rs = nrs;
    for (int kt = 1; kt < KT; ++kt) {
      col3(cb ^ 1, cur_rs);
      cb ^= 1;
      cols02(cb, cur_rs, [&] { next_rs(kt + 2); });
      cur_rs = nrs;
    }
    col3(cb ^ 1, cur_rs);
    cb ^= 1;

    // ---- epilogue: lane (g, r) of block (i, j) holds row 16i + r, columns
    // 16j + 4g .. 16j + 4g + 3 of the wave's 256 x 64 part
    int el = lane;
    asm volatile("" : "+v"(el));
    const int eg = el >> 4, er = el & 15;
    if (p.out_f32) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + i * 16 + er;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + 64 * wave + j * 16 + 4 * eg;
          if (m < p.M && n < p.N)
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.y) + (size_t)m * p.N + n) =
                make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
      }
    } else {
      // bf16: transpose each 16-row block through the wave's LDS area (rows
      // of 128 bytes padded to 144) and store whole 128-byte row segments
      uint8_t* ep = lds_ep + wave * kEpi;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
          const uint32_t hi = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
          *reinterpret_cast<uint2*>(ep + er * kEpiRow + j * 32 + eg * 8) = make_uint2(lo, hi);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int R = 8 * k + (el >> 3), ch = el & 7;
          const uint4 v = *reinterpret_cast<const uint4*>(ep + R * kEpiRow + ch * 16);
          const int m = m0 + i * 16 + R;
          const int n = n0 + 64 * wave + 8 * ch;
          if (m < p.M && n < p.N)
            __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(&v),
                                        reinterpret_cast<v4i*>(reinterpret_cast<uint16_t*>(p.y) + (size_t)m * p.N + n));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0, 0, 0, 0};
    // the next stage's A pieces and first unpacked block (made by the last
    // column block 3) are made again here rather than kept live across the
    // epilogue; buffer cb is not written before the next barrier
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      af[i][0] = apiece(cb * kBuf + 2048 * i + rdA0);
      af[i][1] = apiece(cb * kBuf + 2048 * i + rdA1);
    }
    Unpack u;
#pragma unroll
    for (int kk = 0; kk < 10; ++kk) unpack_piece(kk, cb, 0, u, bw[0][0], bw[0][1]);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int KIND, int BM, int BN, int WM, int WN>
static void launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  prefill_gemm_kernel<KIND, BM, BN, WM, WN><<<dim3((unsigned)tiles), WM * WN * 64, 0, st>>>(a);
}

// Compute units of the current device (one persistent workgroup each).
static int device_cus() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    return n;
  }();
  return cus;
}

template <int KIND>
static void launch_prefill_big(const PrefillArgs& a, hipStream_t st) {
  const int tm = (a.M + 255) / 256, tn = (a.N + 255) / 256;
  const int grid = std::min(tm * tn, device_cus());
  if (a.K % 128 == 0 && a.K >= 256) {
    prefill_dma_kernel<KIND><<<dim3((unsigned)grid), 256, 0, st>>>(a, tm, tn);
    return;
  }
  if (a.K % 128 == 0) prefill_big_kernel<KIND, false><<<dim3((unsigned)grid), 256, 0, st>>>(a, tm, tn);
  else prefill_big_kernel<KIND, true><<<dim3((unsigned)grid), 256, 0, st>>>(a, tm, tn);
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
  // enough 256x256 tiles to occupy half the device or more: the persistent
  // pipelined kernel; otherwise 128x128 tiles so the grid still fills it
  // (its staging offsets are 32-bit: both operands under 2 GiB)
  const bool big = ((M + 255) / 256) * ((N + 255) / 256) >= device_cus() / 2 &&
                   (uint64_t)M * (uint64_t)lda < (1ull << 31) && (uint64_t)N * (uint64_t)K < (1ull << 31);
  if (kind == kGemmFP8) {
    if (big) launch_prefill_big<kGemmFP8>(g, st);
    else launch_prefill_t<kGemmFP8, 128, 128, 2, 2>(g, st);
  } else if (kind == kGemmI8) {
    if (big) launch_prefill_big<kGemmI8>(g, st);
    else launch_prefill_t<kGemmI8, 128, 128, 2, 2>(g, st);
  } else {
    // the persistent kernel loads the group steps as dwords straight into
    // LDS: it needs 4-byte aligned steps (the ABI accepts 2-byte alignment)
    const int tm = (int)((M + 255) / 256), tn = (int)((N + 255) / 256);
    if (tm * tn >= device_cus() / 2 && K % 64 == 0 && K >= 128 && (uint64_t)M * (uint64_t)lda * 2 < (1ull << 31) &&
        (uint64_t)N * (uint64_t)K / 2 < (1ull << 31) && ((uintptr_t)wsc & 3) == 0)
      prefill_w4_kernel<<<dim3((unsigned)std::min(tm * tn, device_cus())), 256, 0, st>>>(g, tm, tn);
    else
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
