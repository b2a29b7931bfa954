// FP8 mixture-of-experts block for gfx950 ("Gemma 4 From E2B to 31B",
// "Step 1 -- Build the Larger Repacks": the fused expert banks gate_up_proj /
// down_proj are split per expert and quantised like the dense layers, the
// router stays outside in bf16; vLLM PR #45854 report: the fp8 MoE takes
// per-token activation and per-output-channel weight scales).
//
// Stages (intermediates live in the workspace):
//   1. per-token FP8 quant of x                    -> xq [T][H], sx [T]
//   2. routing bookkeeping (one workgroup): rows of each expert
//      (1 and 2 share one launch below 1024 tokens)
//   3. grouped gate_up: for every touched expert, its 2I x H FP8 weights are
//      streamed once for all of its rows; h = (xq.w13^T)*sx*s13, then
//      act = SiLU(h[:I]) * h[I:] in fp32        -> act [R][I]   (R = T*topk)
//      (or the SwiGLU-OAI activation with alpha, beta and a clamp limit, the
//      variant the PR carries into the fp8 MoE config)
//   4. per-row FP8 requant of act                 -> aq [R][I], sa [R]
//   5. grouped down: d = (aq.w2^T)*sa*s2           -> d [R][H] fp32
//   6. combine: y[t] = bf16(sum_j p[t,j] * d[t*topk+j]) in slot order.
// Experts that no token routes to are never read.
// The W4A16 block (the 4-bit builds' WNA16 expert path, "The 4-Bit Builds
// Stay Slow") runs the same grouped GEMMs on bf16 activations and int4
// expert banks unpacked in the kernel: no quantisation stages, and
// act = bf16(SiLU(g) * u) is written by the gate_up epilogue.
#include <mutex>

#include "qlin_device.h"
#include "qlin_internal.h"
#include "qlin_quant_row.h"
#include "qlin_skinny.h"

namespace qlin {

// Stage buffers of the allocation-free FP8 MoE entry point: one array per
// GPU, alive until the process ends. Every call on a GPU reuses it (calls
// that overlap on one GPU race) and overwrites what the previous call left;
// no part of it has to start at zero.
static __device__ __align__(256) uint8_t scratch[kMoeScratchBytes];

int moe_scratch_ptr(void** out) {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return QLIN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return QLIN_OK;
}

MoeLayout moe_layout(int64_t T, int64_t H, int64_t I, int64_t E, int topk) {
  const int64_t R = T * topk;
  MoeLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round_up(bytes, 256);
    return at;
  };
  L.xq = take((size_t)T * H);
  L.sx = take((size_t)T * 4);
  L.act = take((size_t)R * I * 4);
  L.aq = take((size_t)R * I);
  L.sa = take((size_t)R * 4);
  L.d = take((size_t)R * H * 4);
  L.cnt = take((size_t)E * 4);
  L.off = take((size_t)(E + 1) * 4);
  L.rows = take((size_t)R * 4);
  L.total = o;
  return L;
}

MoeW4Layout moe_w4_layout(int64_t T, int64_t H, int64_t I, int64_t E, int topk) {
  const int64_t R = T * topk;
  MoeW4Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round_up(bytes, 256);
    return at;
  };
  L.act = take((size_t)R * I * 2);
  L.d = take((size_t)R * H * 4);
  L.off = take((size_t)(E + 1) * 4);
  L.rows = take((size_t)R * 4);
  L.total = o;
  return L;
}

// ---------------------------------------------------------------- routing
// off[e] = first position of expert e in rows[]; rows[] lists r = t*topk+j.
// The order of rows inside an expert does not affect any result (every
// output row is computed from its own activation row only).
// One workgroup (any size that is a multiple of 64); sh: 2E ints of LDS.
// The first KEEP ids of each thread stay in registers for the scatter (one
// global read of them instead of two).
template <int KEEP>
__device__ __forceinline__ void moe_route(const int32_t* __restrict__ ids, int R, int E,
                                          int* __restrict__ off, int* __restrict__ rows, int* sh) {
  int* cnt = sh;
  int* cur = sh + E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  constexpr int kKeep = KEEP;
  int keep[kKeep];
#pragma unroll
  for (int i = 0; i < kKeep; ++i) {
    const int r = threadIdx.x + i * blockDim.x;
    keep[i] = r < R ? ids[r] : -1;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kKeep; ++i)
    if (keep[i] >= 0 && keep[i] < E) atomicAdd(&cnt[keep[i]], 1);
  for (int r = threadIdx.x + kKeep * blockDim.x; r < R; r += blockDim.x) {
    const int e = ids[r];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // exclusive prefix over the experts by the first wave, 64 at a time
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int run = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < E ? cnt[e] : 0;
      int incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      if (e < E) {
        off[e] = run + incl - c;
        cur[e] = run + incl - c;
      }
      run += __shfl(incl, 63, 64);
    }
    if (lane == 0) off[E] = run;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kKeep; ++i)
    if (keep[i] >= 0 && keep[i] < E) rows[atomicAdd(&cur[keep[i]], 1)] = threadIdx.x + i * blockDim.x;
  for (int r = threadIdx.x + kKeep * blockDim.x; r < R; r += blockDim.x) {
    const int e = ids[r];
    if (e >= 0 && e < E) rows[atomicAdd(&cur[e], 1)] = r;
  }
}

__global__ __launch_bounds__(1024) void moe_route_kernel(const int32_t* __restrict__ ids, int R,
                                                         int E, int* __restrict__ off,
                                                         int* __restrict__ rows) {
  extern __shared__ int sh[];  // cnt[E], cur[E]
  moe_route<4>(ids, R, E, off, rows, sh);  // 1024 threads: R <= 4096 in registers
}

// Stages 1 and 2 of the FP8 block in one launch: workgroup 0 does the
// routing bookkeeping (the longest workgroup, dispatched first), workgroups
// 1..T quantise one token each (the two share nothing; as separate launches
// the routing kernel added its own launch to the block's critical path).
template <int CMAX>
__global__ __launch_bounds__(kQThreads) void moe_prep_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                             uint8_t* __restrict__ xq, float* __restrict__ sx,
                                                             const int32_t* __restrict__ ids, int R, int E,
                                                             int* __restrict__ off, int* __restrict__ rows) {
  extern __shared__ int sh[];  // routing: cnt[E], cur[E]
  __shared__ float red[kQThreads / 64];
  if (blockIdx.x == 0) moe_route<16>(ids, R, E, off, rows, sh);  // R <= 4096 in registers
  else quant_row<QLIN_E4M3, CMAX>(x, H, H, xq, sx, (int64_t)blockIdx.x - 1, red);
}

// ---------------------------------------------------------------- grouped GEMM
struct MoeGemmArgs {
  const uint8_t* A;       // gate_up: xq [T][H] (W4A16: x bf16); down: aq [R][I] (W4A16: act bf16)
  const float* sa;        // gate_up: sx [T]; down: sa [R] (FP8 only)
  const uint8_t* W;       // gate_up: w13 [E][2I][H]; down: w2 [E][H][I] (W4A16: packed codes, K/2 per row)
  const float* sw;        // s13 [E][2I] / s2 [E][H] (FP8 only)
  const uint16_t* steps;  // W4A16 group steps [E][rows][K/32]
  const int* off;         // [E+1]
  const int* rows;        // [R]
  int topk;
  int K;                  // H (gate_up) or I (down)
  int nout;               // I (gate_up: pairs) or H (down)
  void* out;              // act [R][I] (fp32; W4A16: bf16) or d [R][H] fp32
  MoeAct act;             // gate_up epilogue activation
};

// gate_up epilogue: SiLU(g) * u, or SwiGLU-OAI with the call's alpha, beta
// and clamp limit (the same expression order as the SiLU form, so alpha 1,
// beta 0 and an infinite limit give SiLU(g) * u).
__device__ __forceinline__ float moe_activation(const MoeAct& a, float g, float u) {
  if (a.kind == kMoeActSwigluOai) {
    g = fminf(g, a.limit);
    u = fminf(fmaxf(u, -a.limit), a.limit);
    return (g / (1.0f + expf(-(a.alpha * g)))) * (u + a.beta);
  }
  const float silu = g / (1.0f + expf(-g));
  return silu * u;
}

// One workgroup: 64 output columns of one expert (gate_up: 64 gate
// columns and the matching 64 up columns of the bank), for up to MB*16 of
// the expert's routed rows at a time; the weights stream once per row block
// through the skinny GEMM core (qlin_skinny.h), gathered activation rows
// pass through LDS.
// gate_up: each wave owns 16 gate columns and the matching 16 up columns
// (NB = 2 blocks); down: each wave owns two blocks of 16 columns, 128
// columns per workgroup, so that its short K (I) still streams enough bytes
// per workgroup.
template <bool GATEUP>
constexpr int moe_cols_per_wg() { return GATEUP ? 64 : 128; }

template <int KIND, bool GATEUP, int MB, bool SB>
__device__ __forceinline__ void moe_tile(const MoeGemmArgs& p, uint8_t* lds, int tile, int e, int rbeg, int nrows) {
  constexpr bool W4 = KIND == kGemmW4;
  constexpr int ESZ = W4 ? 2 : 1;
  constexpr int NB = 2;
  constexpr int DEPTH = W4 ? 2 : 4;
  constexpr int CW = GATEUP ? 16 : 32;  // distinct output columns per wave
  constexpr int kPer = skinny_pieces<KIND, MB, 4>();
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int K = p.K;
  const int c0 = tile * moe_cols_per_wg<GATEUP>() + wave * CW;  // this wave's first output column
  const size_t wrows = GATEUP ? 2 * (size_t)p.nout : (size_t)p.nout;
  const size_t wrow_bytes = W4 ? (size_t)K / 2 : (size_t)K;
  const uint8_t* wbase = p.W + (size_t)e * wrows * wrow_bytes;

  const uint8_t* wp[NB][2];
  const uint16_t* sp[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // gate_up block j: bank rows j*I + column; down block j: column 16j + ..
      const int col = min(c0 + (GATEUP ? 0 : 16 * j) + 8 * h + (lane >> 3), p.nout - 1);
      wp[j][h] = wbase + (size_t)((GATEUP ? j * p.nout : 0) + col) * wrow_bytes + 16 * (lane & 7);
    }
    if constexpr (W4) {
      const int col = min(c0 + (GATEUP ? 0 : 16 * j) + r, p.nout - 1);
      sp[j] = p.steps + ((size_t)e * wrows + (GATEUP ? j * p.nout : 0) + col) * (K / 32);
    } else {
      sp[j] = nullptr;
    }
  }
  const uint8_t* ap[kPer];
  uint32_t am[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = (tid + 256 * q) / (16 * ESZ);  // tile row of this thread's chunk piece
    const int rr = p.rows[rbeg + min(i, nrows - 1)];
    ap[q] = p.A + (size_t)(GATEUP ? rr / p.topk : rr) * K * ESZ;
    am[q] = i < nrows ? 0xFFFFFFFFu : 0u;
  }
  v4f acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0, 0, 0, 0};
  skinny_mma<KIND, MB, NB, DEPTH, SB>(lds, wp, sp, ap, am, K, 0, K, acc);

  // epilogue operands (the core's output layout: lane (r, g) holds row
  // i*16 + r of each row block and 4 consecutive columns 4g..4g+3 of each
  // column block), fetched after the main loop so that they hold no
  // registers during it
  int rid[MB];
  float sav[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int rr = p.rows[rbeg + min(i * 16 + r, nrows - 1)];
    rid[i] = rr;
    sav[i] = W4 ? 1.0f : p.sa[GATEUP ? rr / p.topk : rr];
  }
  // whole 4-column pieces of aligned rows are stored at once (16 bytes of
  // fp32, 8 of bf16)
  const bool vec = (p.nout & 3) == 0 && ((uintptr_t)p.out & (W4 && GATEUP ? 7u : 15u)) == 0;
  if constexpr (GATEUP) {
    const int col = c0 + 4 * g;
    float swg[4], swu[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int colc = min(col + q, p.nout - 1);
      swg[q] = W4 ? 1.0f : p.sw[(size_t)e * wrows + colc];
      swu[q] = W4 ? 1.0f : p.sw[(size_t)e * wrows + p.nout + colc];
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (i * 16 + r >= nrows) continue;
      float av[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float gv, uv;
        if constexpr (W4) {
          gv = acc[i][0][q];
          uv = acc[i][1][q];
        } else {
          gv = (acc[i][0][q] * sav[i]) * swg[q];
          uv = (acc[i][1][q] * sav[i]) * swu[q];
        }
        av[q] = moe_activation(p.act, gv, uv);
      }
      const size_t o = (size_t)rid[i] * p.nout + col;
      if (vec && col + 3 < p.nout) {
        if constexpr (W4)
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + o) =
              make_uint2(f32_bf16_rne(av[0]) | (f32_bf16_rne(av[1]) << 16),
                         f32_bf16_rne(av[2]) | (f32_bf16_rne(av[3]) << 16));
        else
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + o) = make_float4(av[0], av[1], av[2], av[3]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (col + q < p.nout) {
            if constexpr (W4) reinterpret_cast<uint16_t*>(p.out)[o + q] = (uint16_t)f32_bf16_rne(av[q]);
            else reinterpret_cast<float*>(p.out)[o + q] = av[q];
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int col = c0 + 16 * j + 4 * g;
      float sw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) sw[q] = W4 ? 1.0f : p.sw[(size_t)e * wrows + min(col + q, p.nout - 1)];
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        if (i * 16 + r >= nrows) continue;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = W4 ? acc[i][j][q] : (acc[i][j][q] * sav[i]) * sw[q];
        const size_t o = (size_t)rid[i] * p.nout + col;
        if (vec && col + 3 < p.nout) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + o) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (col + q < p.nout) reinterpret_cast<float*>(p.out)[o + q] = v[q];
        }
      }
    }
  }
  __syncthreads();  // the next row block reuses the LDS
}

// Each workgroup walks its expert's routed rows in blocks of MBMAX*16 rows
// (one pass of the weights per block). MBMAX is chosen per call from the
// average number of rows per expert: 2 (32-row blocks) for light loads, 3
// (48-row blocks) otherwise, so that nearly every expert is served by one
// pass while the registers still allow two workgroups per CU (the 48-row
// W4A16 kernels fit the 256 VGPRs of that bound without spilling).
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup L to XCD
// L % 8), each with its own L2; when the expert count is a multiple of 8,
// the k-th workgroup of XCD x takes column tile k % tiles of expert
// x + 8 * (k / tiles), so all tiles of an expert share one L2 and its
// gathered activation rows are fetched into one L2 instead of eight.
template <int KIND, bool GATEUP, int MBMAX, bool SB>
__global__ __launch_bounds__(256, 2) void moe_gemm_kernel(const MoeGemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[skinny_lds_bytes<KIND, MBMAX, 2, KIND == kGemmW4 ? 2 : 1>()];
  constexpr int kXcds = 8;
  int tile = blockIdx.x, e = blockIdx.y;
  if (gridDim.y % kXcds == 0) {
    const int L = blockIdx.y * gridDim.x + blockIdx.x, k = L / kXcds;
    e = L % kXcds + kXcds * (k / gridDim.x);
    tile = k % gridDim.x;
  }
  const int beg = p.off[e], n = p.off[e + 1] - beg;
  for (int rb = 0; rb < n; rb += 16 * MBMAX) {
    const int nr = min(16 * MBMAX, n - rb);
    const int mb = (nr + 15) / 16;
    if (mb == 1) moe_tile<KIND, GATEUP, 1, SB>(p, lds, tile, e, beg + rb, nr);
    else if (mb == 2 || MBMAX == 2) moe_tile<KIND, GATEUP, 2, SB>(p, lds, tile, e, beg + rb, nr);
    else moe_tile<KIND, GATEUP, (MBMAX > 2 ? 3 : 2), SB>(p, lds, tile, e, beg + rb, nr);
  }
}

// ---------------------------------------------------------------- combine
// y[t][h] = bf16(sum_j p[t][j] * d[t*topk + j][h]), j ascending; slots with
// an expert id outside [0, E) contribute nothing. One thread per (t, 4 h).
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ d,
                                                          const int32_t* __restrict__ ids,
                                                          const float* __restrict__ wts, int T, int topk,
                                                          int H, int E, uint16_t* __restrict__ y) {
  const int hq = H / 4;
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)T * hq) return;
  const int t = (int)(i / hq), h = (int)(i % hq) * 4;
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
  // slots in batches of 8: every load of a batch is issued before the first
  // sum (clamped slot indices, no branch between the loads), then the sums
  // run in slot order
  for (int j0 = 0; j0 < topk; j0 += 8) {
    int ev[8];
    float wv[8];
    float4 dv[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int j = min(j0 + b, topk - 1);
      ev[b] = ids[t * topk + j];
      wv[b] = wts[t * topk + j];
      dv[b] = *reinterpret_cast<const float4*>(d + ((size_t)t * topk + j) * H + h);
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if (j0 + b < topk && ev[b] >= 0 && ev[b] < E) {
        a0 = a0 + wv[b] * dv[b].x;
        a1 = a1 + wv[b] * dv[b].y;
        a2 = a2 + wv[b] * dv[b].z;
        a3 = a3 + wv[b] * dv[b].w;
      }
    }
  }
  const uint32_t lo = f32_bf16_rne(a0) | (f32_bf16_rne(a1) << 16);
  const uint32_t hi = f32_bf16_rne(a2) | (f32_bf16_rne(a3) << 16);
  *reinterpret_cast<uint2*>(y + (size_t)t * H + h) = make_uint2(lo, hi);
}

int launch_moe_fp8(const uint16_t* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                   const int32_t* ids, const float* wts, const uint8_t* w13, const float* s13,
                   const uint8_t* w2, const float* s2, uint16_t* y, void* ws, hipStream_t st,
                   const MoeAct& act) {
  const MoeLayout L = moe_layout(T, H, I, E, topk);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  uint8_t* xq = base + L.xq;
  float* sx = reinterpret_cast<float*>(base + L.sx);
  float* act32 = reinterpret_cast<float*>(base + L.act);
  uint8_t* aq = base + L.aq;
  float* sa = reinterpret_cast<float*>(base + L.sa);
  float* dd = reinterpret_cast<float*>(base + L.d);
  int* off = reinterpret_cast<int*>(base + L.off);
  int* rows = reinterpret_cast<int*>(base + L.rows);
  const int R = (int)(T * topk);

  // token quantisation and routing in one launch where the quantiser takes
  // a workgroup per token (fewer than 1024 tokens of at most 16384
  // elements, as launch_quant_act would)
  int rc = QLIN_OK;
  const int64_t chunks = H / 8;
  const dim3 pgrid((unsigned)(T + 1));
  const size_t psh = 2 * E * sizeof(int);
  if (T < 1024 && chunks <= 1 * kQThreads)
    moe_prep_kernel<1><<<pgrid, kQThreads, psh, st>>>(x, (int)T, (int)H, xq, sx, ids, R, (int)E, off, rows);
  else if (T < 1024 && chunks <= 2 * kQThreads)
    moe_prep_kernel<2><<<pgrid, kQThreads, psh, st>>>(x, (int)T, (int)H, xq, sx, ids, R, (int)E, off, rows);
  else if (T < 1024 && chunks <= 4 * kQThreads)
    moe_prep_kernel<4><<<pgrid, kQThreads, psh, st>>>(x, (int)T, (int)H, xq, sx, ids, R, (int)E, off, rows);
  else if (T < 1024 && chunks <= 8 * kQThreads)
    moe_prep_kernel<8><<<pgrid, kQThreads, psh, st>>>(x, (int)T, (int)H, xq, sx, ids, R, (int)E, off, rows);
  else {
    if ((rc = launch_quant_act(x, T, H, H, QLIN_E4M3, xq, sx, st))) return rc;
    moe_route_kernel<<<1, 1024, psh, st>>>(ids, R, (int)E, off, rows);
  }
  if ((rc = launch_status())) return rc;

  // row blocks of 32 rows when an expert averages at most 8 routed rows,
  // else 48
  const bool light = R <= 8 * E;
  MoeGemmArgs gu{xq, sx, w13, s13, nullptr, off, rows, topk, (int)H, (int)I, act32, act};
  const dim3 ggrid((unsigned)((I + moe_cols_per_wg<true>() - 1) / moe_cols_per_wg<true>()), (unsigned)E);
  if (light) moe_gemm_kernel<kGemmFP8, true, 2, false><<<ggrid, 256, 0, st>>>(gu);
  else moe_gemm_kernel<kGemmFP8, true, 3, false><<<ggrid, 256, 0, st>>>(gu);
  if ((rc = launch_status())) return rc;

  if ((rc = launch_quant_rows_f32(act32, R, I, aq, sa, st))) return rc;

  MoeGemmArgs dn{aq, sa, w2, s2, nullptr, off, rows, topk, (int)I, (int)H, dd};
  const dim3 dgrid((unsigned)((H + moe_cols_per_wg<false>() - 1) / moe_cols_per_wg<false>()), (unsigned)E);
  if (light) moe_gemm_kernel<kGemmFP8, false, 2, false><<<dgrid, 256, 0, st>>>(dn);
  else moe_gemm_kernel<kGemmFP8, false, 3, false><<<dgrid, 256, 0, st>>>(dn);
  if ((rc = launch_status())) return rc;

  const long long threads = T * (H / 4);
  moe_combine_kernel<<<dim3((unsigned)((threads + 255) / 256)), 256, 0, st>>>(dd, ids, wts, (int)T, topk,
                                                                             (int)H, (int)E, y);
  return launch_status();
}

// W4A16 block (the 4-bit MoE's WNA16 expert path: bf16 activations, group-32
// int4 expert banks): routing bookkeeping, grouped gate_up on x itself with
// act = bf16(SiLU(g) * u) in its epilogue, grouped down on act, combine.
int launch_moe_w4a16(const uint16_t* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                     const int32_t* ids, const float* wts, const uint8_t* p13, const uint16_t* st13,
                     const uint8_t* p2, const uint16_t* st2, uint16_t* y, void* ws, hipStream_t st) {
  const MoeW4Layout L = moe_w4_layout(T, H, I, E, topk);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  uint16_t* act = reinterpret_cast<uint16_t*>(base + L.act);
  float* dd = reinterpret_cast<float*>(base + L.d);
  int* off = reinterpret_cast<int*>(base + L.off);
  int* rows = reinterpret_cast<int*>(base + L.rows);
  const int R = (int)(T * topk);

  moe_route_kernel<<<1, 1024, 2 * E * sizeof(int), st>>>(ids, R, (int)E, off, rows);
  int rc = launch_status();
  if (rc) return rc;

  const bool light = R <= 8 * E;
  // bulk int4 step loads need 256-element K chunks and 16-byte aligned step rows
  auto bulk = [](const uint16_t* s, int64_t K) { return K % 256 == 0 && (reinterpret_cast<uintptr_t>(s) & 15) == 0; };
  MoeGemmArgs gu{reinterpret_cast<const uint8_t*>(x), nullptr, p13, nullptr, st13, off, rows, topk, (int)H, (int)I, act};
  const dim3 ggrid((unsigned)((I + moe_cols_per_wg<true>() - 1) / moe_cols_per_wg<true>()), (unsigned)E);
  const bool sg = bulk(st13, H);
  if (light) {
    if (sg) moe_gemm_kernel<kGemmW4, true, 2, true><<<ggrid, 256, 0, st>>>(gu);
    else moe_gemm_kernel<kGemmW4, true, 2, false><<<ggrid, 256, 0, st>>>(gu);
  } else {
    if (sg) moe_gemm_kernel<kGemmW4, true, 3, true><<<ggrid, 256, 0, st>>>(gu);
    else moe_gemm_kernel<kGemmW4, true, 3, false><<<ggrid, 256, 0, st>>>(gu);
  }
  if ((rc = launch_status())) return rc;

  MoeGemmArgs dn{reinterpret_cast<const uint8_t*>(act), nullptr, p2, nullptr, st2, off, rows, topk, (int)I, (int)H, dd};
  const dim3 dgrid((unsigned)((H + moe_cols_per_wg<false>() - 1) / moe_cols_per_wg<false>()), (unsigned)E);
  const bool sd = bulk(st2, I);
  if (light) {
    if (sd) moe_gemm_kernel<kGemmW4, false, 2, true><<<dgrid, 256, 0, st>>>(dn);
    else moe_gemm_kernel<kGemmW4, false, 2, false><<<dgrid, 256, 0, st>>>(dn);
  } else {
    if (sd) moe_gemm_kernel<kGemmW4, false, 3, true><<<dgrid, 256, 0, st>>>(dn);
    else moe_gemm_kernel<kGemmW4, false, 3, false><<<dgrid, 256, 0, st>>>(dn);
  }
  if ((rc = launch_status())) return rc;

  const long long threads = T * (H / 4);
  moe_combine_kernel<<<dim3((unsigned)((threads + 255) / 256)), 256, 0, st>>>(dd, ids, wts, (int)T, topk,
                                                                             (int)H, (int)E, y);
  return launch_status();
}

}  // namespace qlin
