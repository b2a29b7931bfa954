// W4A16 GEMM for decode batches (M <= 64) of layers too small for one wave
// per 16 output columns to fill the device, on gfx950 ("Gemma 4 From E2B to 31B",
// "The 4-Bit Builds Stay Slow": the kernel unpacks the group-32 int4 weights
// to bf16 before each multiply):
//   Y[m,n] = sum_k a[m,k] * bf16(c[n,k] * step[n,k/32]),  fp32 accumulation.
//
// Such a layer (K=2048, N=8192: 9.4 MB of codes and steps) is too small for
// one wave per 16 columns to keep the device busy, and splitting K across
// workgroups costs a write and a read of fp32 partial sums per split. Here
// the four waves of a workgroup split the work among themselves instead:
// NC column groups x NQ K parts (x NR row blocks, which would read the same
// weights and each unpack them for their rows: the launcher uses NR = 1).
// The K parts of a column group are summed through LDS in part order
// (deterministic, nothing in memory).
//  * each wave owns 16*NB output columns, all 16*MB rows (each unpacked
//    weight feeds MB MFMAs) and a range of whole 256-K units;
//  * weights are fetched in whole lines (each load instruction reads 128
//    bytes of each of 8 rows: one 256-K unit of those rows) and pass through
//    a wave-private LDS slot into MFMA fragment layout (LDS operations of one
//    wave complete in order: no barrier). Lane (r, g) then holds, for h = 0,
//    1, the 32 codes of group 4h + g of row r, and loads that group's bf16
//    step itself. Word i of piece h holds the codes of k = 128h + 32g + 8i +
//    t (nibble t); the MFMA step (h, i) multiplies them with the activations
//    at the same k: the same K permutation for both operands of every MFMA.
//    The slot is fragment-major with an XOR swizzle of the row, so both the
//    line-shaped writes (8 lanes = 8 chunks of one row) and the fragment
//    reads (16 rows, one chunk) are free of bank conflicts;
//  * the weights of DEPTH units per wave are in flight at any time (a ring
//    of registers, refilled right after a slot is consumed);
//  * activations pass through LDS compactly: only the M real rows, in rounds
//    of CK units per K part, double buffered and staged by the whole
//    workgroup, one barrier per round. Lanes of rows >= M read a zero row.
//    LDS row stride 512*CK + 16 bytes, so the 8 lanes of one 16-byte read
//    cycle (8 rows, one k) fall in distinct bank groups.
#include <algorithm>

#include "qlin_device.h"
#include "qlin_internal.h"

namespace qlin {

struct W4FewArgs {
  const uint16_t* A;      // bf16 [M][lda]
  int64_t lda;            // elements
  const uint8_t* codes;   // [N][K/2]
  const uint16_t* steps;  // [N][K/32]
  int M, N, K;
  int kq;                 // units (256 K) per K part
  void* y;
  int out_f32;
};

template <int CK>
constexpr int w4few_row_bytes() { return CK * 512 + 16; }
// LDS of the activations: 2 buffers x NQ parts x MR rows, and the zero row
template <int MR, int CK, int NQ>
constexpr int w4few_act_bytes() { return (2 * NQ * MR + 1) * w4few_row_bytes<CK>(); }

template <int NB, int MB, int DEPTH, int NC, int NQ, int NR, int MR, int CK>
__global__ __launch_bounds__(256) void decode_w4_few_kernel(const W4FewArgs p) {
  static_assert(NC * NQ * NR == 4, "four waves per workgroup");
  static_assert(MR <= 16 * MB * NR, "the row blocks cover the staged rows");
  constexpr int RS = w4few_row_bytes<CK>();            // LDS row stride
  constexpr int kPartBuf = MR * RS;                    // one K part's rows of one buffer
  constexpr int kAct = w4few_act_bytes<MR, CK, NQ>();  // activations and the zero row
  constexpr int kLds = kAct + 4 * NB * 2048;           // + one weight slot per wave
  static_assert(kAct >= 4 * MB * NB * 64 * 16, "LDS holds the waves' accumulators for the reduction");
  // activation pieces (16 bytes) staged per round: NQ parts x MR rows x CK
  // units x 32 pieces, over 256 threads
  constexpr int kPieces = NQ * MR * CK * 32;
  constexpr int kPer = (kPieces + 255) / 256;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int cg = wave % NC, q = wave / NC % NQ, qr = wave / (NC * NQ);  // column group, K part, row block
  const int n0 = (blockIdx.x * NC + cg) * 16 * NB;
  const int units = p.K / 256;
  const int u0 = q * p.kq;                            // this wave's first unit
  const int nu = max(0, min(p.kq, units - u0));       // its unit count (uniform per wave)
  const int rounds = (p.kq + CK - 1) / CK;            // uniform over the workgroup
  const int zero_off = 2 * NQ * kPartBuf;             // the zero row

  // weight rows of this lane (clamped onto valid rows; their columns are not
  // stored): line-shaped code loads (row 8h + lane/8 of block j, 16-byte
  // chunk lane%8) and fragment-shaped step loads (row r, group 4h + g)
  const uint8_t* wrow[NB][2];
  const uint16_t* srow[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      wrow[j][h] = p.codes + (size_t)min(n0 + 16 * j + 8 * h + (lane >> 3), p.N - 1) * (p.K / 2) + 16 * (lane & 7);
    srow[j] = p.steps + (size_t)min(n0 + 16 * j + r, p.N - 1) * (p.K / 32) + g;
  }
  uint8_t* const wslot = lds + kAct + wave * NB * 2048;
  const int wc = lane & 7;
  const int wwr = (wc >> 2) * 1024 + (wc & 3) * 256;  // write: piece wc/4, lane group wc%4

  struct Slot {
    uint4 c[NB][2];
    uint16_t s[NB][2];
  };
  // unit u of this wave, clamped onto the wave's last unit and onto the
  // row's last unit (a wave may have no unit at all): valid memory, never used
  auto wload = [&](Slot& sl, int u) {
    const int uu = min(u0 + max(0, min(u, nu - 1)), units - 1);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      sl.c[j][0] = ldg16(wrow[j][0] + (size_t)uu * 128);
      sl.c[j][1] = ldg16(wrow[j][1] + (size_t)uu * 128);
      sl.s[j][0] = srow[j][(size_t)uu * 8];
      sl.s[j][1] = srow[j][(size_t)uu * 8 + 4];
    }
  };

  // ---- activation staging: piece x = tid + 256 e -> (part, row, unit, piece)
  uint4 areg[kPer];
  auto apiece = [&](int x, int& part, int& row, int& cu, int& pc) {
    pc = x & 31;
    cu = (x >> 5) % CK;
    row = (x >> 5) / CK % MR;
    part = (x >> 5) / CK / MR;
  };
  // Rows >= M are staged from row M - 1 (valid memory) and never read (their
  // lanes read the zero row): no divergent branch per piece, which had cost
  // each load and each LDS write an exec-mask save, branch and restore.
  auto aload = [&](int rd) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int x = tid + 256 * e;
      int part, row, cu, pc;
      apiece(x, part, row, cu, pc);
      if (kPieces % 256 == 0 || x < kPieces) {
        // clamp past the part's units or K (read valid memory; never used)
        const int u = min(part * p.kq + min(rd * CK + cu, p.kq - 1), units - 1);
        areg[e] = ldg16(p.A + (size_t)min(row, p.M - 1) * p.lda + (size_t)u * 256 + pc * 8);
      }
    }
  };
  auto awrite = [&](int buf) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int x = tid + 256 * e;
      int part, row, cu, pc;
      apiece(x, part, row, cu, pc);
      if (kPieces % 256 == 0 || x < kPieces)
        *reinterpret_cast<uint4*>(lds + (buf * NQ + part) * kPartBuf + row * RS + cu * 512 + pc * 16) = areg[e];
    }
  };

  // this lane's activation rows in LDS, one per 16-row block (rows >= M
  // read the zero row)
  int arow[MB], abuf[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int ar = 16 * (qr * MB + mb) + r;
    arow[mb] = ar < p.M ? (q * kPartBuf + ar * RS) : zero_off;
    abuf[mb] = ar < p.M ? NQ * kPartBuf : 0;  // offset of buffer 1 (0 for the zero row)
  }

  v4f acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mb][j] = v4f{0, 0, 0, 0};

  auto compute = [&](const Slot& sl, int buf, int cu) {
    // line-shaped code registers -> the wave's slot -> fragment pieces
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int R = 8 * h + (lane >> 3);
        *reinterpret_cast<uint4*>(wslot + j * 2048 + wwr + ((R ^ wc) & 15) * 16) = sl.c[j][h];
      }
    uint4 frag[NB][2];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        frag[j][h] = *reinterpret_cast<const uint4*>(wslot + j * 2048 + h * 1024 + g * 256 +
                                                     ((r ^ (4 * h + g)) & 15) * 16);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      Int4Step st[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) st[j] = int4_step(bf16_f32(sl.s[j][h]));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // the activation fragments are requested before the unpack, which
        // covers their LDS latency (scheduling barriers keep the order)
        v8bf af[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          af[mb] = *reinterpret_cast<const v8bf*>(lds + arow[mb] + buf * abuf[mb] + cu * 512 + g * 64 +
                                                  h * 256 + i * 16);
        __builtin_amdgcn_sched_barrier(0);
        v8bf bf[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const uint4& cw = frag[j][h];
          const uint32_t word = i == 0 ? cw.x : i == 1 ? cw.y : i == 2 ? cw.z : cw.w;
          bf[j] = dequant8_mix(word, st[j]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[mb][j] = mfma_bf16(bf[j], af[mb], acc[mb][j]);
      }
    }
  };

  // ---- prologue: zero row, first activation round, weight ring
  for (int x = tid; x < RS / 16; x += 256)
    *reinterpret_cast<uint4*>(lds + zero_off + x * 16) = make_uint4(0, 0, 0, 0);
  aload(0);
  Slot ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) wload(ring[d], d);
  awrite(0);
  __syncthreads();
  if (rounds > 1) aload(1);

  // ---- units in groups of DEPTH (the ring slot is known at compile time).
  // At the start of round rd (> 0) the activations fetched during round
  // rd - 1 go to buffer rd & 1, last read in round rd - 2 (before the barrier
  // that opened round rd - 1), then the next round's are fetched. The loop
  // bounds and round boundaries are uniform over the workgroup.
  for (int ub = 0; ub < p.kq; ub += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int u = ub + d;
      if (u < p.kq) {
        const int rd = u / CK, cu = u - rd * CK;
        if (rd > 0 && cu == 0) {
          awrite(rd & 1);
          __syncthreads();
          if (rd + 1 < rounds) aload(rd + 1);
        }
        if (u < nu) {  // uniform per wave
          Slot cur = ring[d];
          __builtin_amdgcn_sched_barrier(0);
          wload(ring[d], u + DEPTH);
          __builtin_amdgcn_sched_barrier(0);
          compute(cur, rd & 1, cu);
        }
      }
    }
  }

  // ---- sum the K parts in part order; part 0's waves store
  if constexpr (NQ > 1) {
    __syncthreads();  // every wave is done with the activation buffers
    v4f* red = reinterpret_cast<v4f*>(lds);
    const int slot = (qr * NQ + q) * NC + cg;
    if (q > 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NB; ++j) red[((slot * MB + mb) * NB + j) * 64 + lane] = acc[mb][j];
    }
    __syncthreads();
    if (q > 0) return;
#pragma unroll
    for (int qq = 1; qq < NQ; ++qq)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[mb][j] = acc[mb][j] + red[(((((qr * NQ + qq) * NC + cg) * MB + mb) * NB + j) * 64) + lane];
  }
  // the weights are the MFMA's first operand: lane (r, g) holds row r of
  // each row block and columns 4g..4g+3 of each column block, stored as one
  // 16-byte (fp32) or 8-byte (bf16) piece when aligned and inside the output
  const bool vec = (p.N & 3) == 0 && ((uintptr_t)p.y & (p.out_f32 ? 15u : 7u)) == 0;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = 16 * (qr * MB + mb) + r;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int n = n0 + 16 * j + 4 * g;
      const v4f v = acc[mb][j];
      const size_t o = (size_t)m * p.N + n;
      if (vec && n + 3 < p.N) {
        if (p.out_f32)
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.y) + o) = make_float4(v[0], v[1], v[2], v[3]);
        else
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.y) + o) =
              make_uint2(f32_bf16_rne(v[0]) | (f32_bf16_rne(v[1]) << 16), f32_bf16_rne(v[2]) | (f32_bf16_rne(v[3]) << 16));
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

// Compute units of the current device (queried once).
static int w4few_cus() {
  static const int cus = [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    return n;
  }();
  return cus;
}

// Where this kernel serves, as measured at 256 CUs against the split-K
// streaming core:
//  * at most 16 rows on layers with fewer 16-column blocks than SIMDs
//    (K=2048, N=8192: M = 1 5.2 us, M = 8 6.2 us, M = 16 6.8 us, against
//    6.0 / 7.4 / 9.0 us; wider layers keep one wave per column block busy);
//  * 17..64 rows where one workgroup per CU covers the layer: 3/4 of the CUs
//    < N/32 <= CUs (K=2048, N=8192: M = 32 8.8 us, M = 48 11.8 us, M = 64
//    13.0 us, against 10.0 / 12.2 / 14.1 us; with their 74 and 141 KB of LDS
//    a grid of half the CUs (N=4096, K=4096: 19.8 against 15.9 us) or of 1.75
//    workgroups per CU (N=14336: 39.6 against 36.4 us) was slower).
bool w4_few_applies(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > 64 || K % 256 != 0) return false;
  const int64_t cus = w4few_cus();
  if (M <= 16) return (N + 15) / 16 < 4 * cus;
  const int64_t wgs = (N + 31) / 32;
  return 4 * wgs > 3 * cus && wgs <= cus;
}

template <int NB, int MB, int DEPTH, int NC, int NQ, int NR, int MR, int CK>
static void w4few_launch(const W4FewArgs& a, hipStream_t st) {
  const int cols = 16 * NB * NC;
  const int grid = (a.N + cols - 1) / cols;
  decode_w4_few_kernel<NB, MB, DEPTH, NC, NQ, NR, MR, CK><<<dim3((unsigned)grid), 256, 0, st>>>(a);
}

// Launch rule, as measured (one 16-column block per wave): at M = 1 the
// fewest K parts that give every SIMD a wave (K=2048, N=8192: 2 parts, 5.2
// us against 5.6 in 4; K=4096, N=14336: 2 parts, 11.4 us against 14.7 in 1
// and 13.9 in 4; K=14336, N=4096: 4 parts, 14.8 us against 23.4 in 2);
// above, 4 parts (K=2048, N=8192, M = 8: 6.2 us against 7.1 in 2), and 2
// at 16 rows.
template <int MR, int CK>
static void w4few_rows(W4FewArgs& a, hipStream_t st) {
  const int units = a.K / 256;
  const int64_t blocks = (a.N + 15) / 16, simds = 4 * (int64_t)w4few_cus();
  int nq = 4;
  if (MR <= 1)
    for (nq = 1; nq < 4 && blocks * nq < simds;) nq *= 2;
  if (MR == 16) nq = 2;  // 16 rows x 4 parts would not fit LDS twice
  nq = std::max(1, std::min(nq, units));
  if (nq == 3) nq = 2;
  a.kq = (units + nq - 1) / nq;
  if (nq == 1) w4few_launch<1, 1, 2, 4, 1, 1, MR, CK>(a, st);
  else if (nq == 2) w4few_launch<1, 1, 2, 2, 2, 1, MR, CK>(a, st);
  else w4few_launch<1, 1, 2, 1, 4, 1, MR, CK>(a, st);
}

int launch_w4_few(const void* a, int64_t lda, const void* codes, const void* steps, int64_t M,
                  int64_t N, int64_t K, void* y, int out_f32, hipStream_t st) {
  W4FewArgs g{};
  g.A = reinterpret_cast<const uint16_t*>(a);
  g.lda = lda;
  g.codes = reinterpret_cast<const uint8_t*>(codes);
  g.steps = reinterpret_cast<const uint16_t*>(steps);
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.y = y;
  g.out_f32 = out_f32;
  const int units = (int)(K / 256);
  if (M <= 1) w4few_rows<1, 8>(g, st);
  else if (M <= 4) w4few_rows<4, 2>(g, st);
  else if (M <= 8) w4few_rows<8, 2>(g, st);
  else if (M <= 16) w4few_rows<16, 2>(g, st);
  else {
    // 32 or 64 staged rows in every wave (each unpacked weight feeds 2 or 4
    // MFMAs), the waves split as 2 column groups x 2 K parts; one 256-K unit
    // per round keeps the 64-row double buffer at 135 KB of LDS
    const int nq = units >= 2 ? 2 : 1;
    g.kq = (units + nq - 1) / nq;
    if (M <= 32) {
      if (nq == 2) w4few_launch<1, 2, 2, 2, 2, 1, 32, 1>(g, st);
      else w4few_launch<1, 2, 2, 4, 1, 1, 32, 1>(g, st);
    } else {
      if (nq == 2) w4few_launch<1, 4, 2, 2, 2, 1, 64, 1>(g, st);
      else w4few_launch<1, 4, 2, 4, 1, 1, 64, 1>(g, st);
    }
  }
  return launch_status();
}

}  // namespace qlin
