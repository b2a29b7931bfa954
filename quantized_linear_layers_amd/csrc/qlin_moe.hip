// FP8 mixture-of-experts block for gfx950 ("Gemma 4 From E2B to 31B",
// "Step 1 -- Build the Larger Repacks": the fused expert banks gate_up_proj /
// down_proj are split per expert and quantised like the dense layers, the
// router stays outside in bf16; vLLM PR #45854 report: the fp8 MoE takes
// per-token activation and per-output-channel weight scales).
//
// Stages (one kernel each; intermediates live in the workspace):
//   1. per-token FP8 quant of x                    -> xq [T][H], sx [T]
//   2. routing bookkeeping (one workgroup): rows of each expert
//   3. grouped gate_up: for every touched expert, its 2I x H FP8 weights are
//      streamed once for all of its rows; h = (xq.w13^T)*sx*s13, then
//      act = SiLU(h[:I]) * h[I:] in fp32        -> act [R][I]   (R = T*topk)
//   4. per-row FP8 requant of act                 -> aq [R][I], sa [R]
//   5. grouped down: d = (aq.w2^T)*sa*s2           -> d [R][H] fp32
//   6. combine: y[t] = bf16(sum_j p[t,j] * d[t*topk+j]) in slot order.
// Experts that no token routes to are never read.
#include "qlin_device.h"
#include "qlin_internal.h"

namespace qlin {

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

// ---------------------------------------------------------------- routing
// off[e] = first position of expert e in rows[]; rows[] lists r = t*topk+j.
// The order of rows inside an expert does not affect any result (every
// output row is computed from its own activation row only).
__global__ __launch_bounds__(1024) void moe_route_kernel(const int32_t* __restrict__ ids, int R,
                                                         int E, int* __restrict__ off,
                                                         int* __restrict__ rows) {
  extern __shared__ int sh[];  // cnt[E], cur[E]
  int* cnt = sh;
  int* cur = sh + E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    const int e = ids[r];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = run;
      cur[e] = run;
      run += cnt[e];
    }
    off[E] = run;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    const int e = ids[r];
    if (e >= 0 && e < E) rows[atomicAdd(&cur[e], 1)] = r;
  }
}

// ---------------------------------------------------------------- grouped GEMM
struct MoeGemmArgs {
  const uint8_t* A;    // gate_up: xq [T][H]; down: aq [R][I]
  const float* sa;     // gate_up: sx [T]; down: sa [R]
  const uint8_t* W;    // gate_up: w13 [E][2I][H]; down: w2 [E][H][I]
  const float* sw;     // s13 [E][2I] / s2 [E][H]
  const int* off;      // [E+1]
  const int* rows;     // [R]
  int topk;
  int K;               // H (gate_up) or I (down)
  int nout;            // I (gate_up: pairs) or H (down)
  float* out;          // act [R][I] or d [R][H]
};

constexpr int kMoeNW = 4;

__device__ __forceinline__ uint4 and4m(uint4 v, uint32_t m) {
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// One wave owns 16 output columns of one expert (gate_up: 16 gate rows and
// the matching 16 up rows of the bank), the workgroup 64 columns, for up to
// MB*16 routed rows of that expert. Same streaming scheme as the dense decode
// GEMM: weight rows (HBM) and the gathered activation rows (L2) go
// into a DEPTH-step register ring with branch-free, clamped loads; padding
// rows and positions past K are masked to zero on the activation side.
template <bool GATEUP, int MB>
__device__ __forceinline__ void moe_tile(const MoeGemmArgs& p, int e, int rbeg, int nrows) {
  constexpr int NB = GATEUP ? 2 : 1;
  constexpr int DEPTH = MB <= 1 ? 6 : (MB == 2 ? 4 : 2);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int K = p.K;
  const int col = blockIdx.x * (kMoeNW * 16) + wave * 16 + r;  // output column of this lane
  const int colc = min(col, p.nout - 1);
  const size_t wrows = GATEUP ? 2 * (size_t)p.nout : (size_t)p.nout;
  const uint8_t* wbase = p.W + (size_t)e * wrows * K;
  const uint8_t* wr[NB];
  wr[0] = wbase + (size_t)colc * K;
  if (GATEUP) wr[NB - 1] = wbase + (size_t)(p.nout + colc) * K;

  // activation rows this lane loads (MFMA operand row r of each block)
  const uint8_t* ap[MB];
  uint32_t amask[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int rl = i * 16 + r;
    const int rr = p.rows[rbeg + min(rl, nrows - 1)];
    ap[i] = p.A + (size_t)(GATEUP ? rr / p.topk : rr) * K;
    amask[i] = rl < nrows ? 0xFFFFFFFFu : 0u;
  }
  // epilogue operands (output rows 4g+q of each block, this lane's column)
  int rid[MB][4];
  float sav[MB][4];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = p.rows[rbeg + min(i * 16 + 4 * g + q, nrows - 1)];
      rid[i][q] = rr;
      sav[i][q] = p.sa[GATEUP ? rr / p.topk : rr];
    }
  float swv[NB];
  swv[0] = p.sw[(size_t)e * wrows + colc];
  if (GATEUP) swv[NB - 1] = p.sw[(size_t)e * wrows + p.nout + colc];

  v4f acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = v4f{0, 0, 0, 0};

  struct Sl {
    uint4 w[NB][2];
    uint4 a[MB][2];
  };
  const int kclamp = K - 16;
  auto load = [&](Sl& sl, int t) {
    const int kl = min(t * 128 + 16 * g, kclamp), kh = min(t * 128 + 64 + 16 * g, kclamp);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      sl.w[j][0] = ldg16(wr[j] + kl);
      sl.w[j][1] = ldg16(wr[j] + kh);
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      sl.a[i][0] = ldg16(ap[i] + kl);
      sl.a[i][1] = ldg16(ap[i] + kh);
    }
  };
  auto compute = [&](const Sl& sl, int t) {
    const uint32_t vl = (t * 128 + 16 * g < K) ? 0xFFFFFFFFu : 0u;
    const uint32_t vh = (t * 128 + 64 + 16 * g < K) ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const uint4 a0 = and4m(sl.a[i][0], amask[i] & vl);
      const uint4 a1 = and4m(sl.a[i][1], amask[i] & vh);
      const v8i av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                      (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const uint4 w0 = sl.w[j][0], w1 = sl.w[j][1];
        const v8i wv = {(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w,
                        (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
        acc[i][j] = mfma_fp8(av, wv, acc[i][j]);
      }
    }
  };

  const int nsteps = (K + 127) / 128;
  const int rounds = (nsteps + DEPTH - 1) / DEPTH;
  Sl ring[DEPTH];
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

  // epilogue: lane holds rows 4g+q of each block, column `col`
  if (col < p.nout) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = i * 16 + 4 * g + q;
        if (row < nrows) {
          const int rr = rid[i][q];
          if (GATEUP) {
            const float gv = (acc[i][0][q] * sav[i][q]) * swv[0];
            const float uv = (acc[i][1][q] * sav[i][q]) * swv[NB - 1];
            const float silu = gv / (1.0f + expf(-gv));
            p.out[(size_t)rr * p.nout + col] = silu * uv;
          } else {
            p.out[(size_t)rr * p.nout + col] = (acc[i][0][q] * sav[i][q]) * swv[0];
          }
        }
      }
  }
}

template <bool GATEUP>
__global__ __launch_bounds__(kMoeNW * 64) void moe_gemm_kernel(const MoeGemmArgs p) {
  const int e = blockIdx.y;
  const int beg = p.off[e], n = p.off[e + 1] - beg;
  for (int rb = 0; rb < n; rb += 64) {
    const int nr = min(64, n - rb);
    const int mb = (nr + 15) / 16;
    if (mb == 1) moe_tile<GATEUP, 1>(p, e, beg + rb, nr);
    else if (mb == 2) moe_tile<GATEUP, 2>(p, e, beg + rb, nr);
    else if (mb == 3) moe_tile<GATEUP, 3>(p, e, beg + rb, nr);
    else moe_tile<GATEUP, 4>(p, e, beg + rb, nr);
  }
}

// ---------------------------------------------------------------- combine
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ d,
                                                          const int32_t* __restrict__ ids,
                                                          const float* __restrict__ wts, int topk,
                                                          int H, int E, uint16_t* __restrict__ y) {
  const int t = blockIdx.x;
  for (int h = threadIdx.x; h < H; h += blockDim.x) {
    float acc = 0.0f;
    for (int j = 0; j < topk; ++j) {
      const int e = ids[t * topk + j];
      if (e >= 0 && e < E) acc = acc + wts[t * topk + j] * d[((size_t)t * topk + j) * H + h];
    }
    y[(size_t)t * H + h] = (uint16_t)f32_bf16_rne(acc);
  }
}

int launch_moe_fp8(const uint16_t* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                   const int32_t* ids, const float* wts, const uint8_t* w13, const float* s13,
                   const uint8_t* w2, const float* s2, uint16_t* y, void* ws, hipStream_t st) {
  const MoeLayout L = moe_layout(T, H, I, E, topk);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  uint8_t* xq = base + L.xq;
  float* sx = reinterpret_cast<float*>(base + L.sx);
  float* act = reinterpret_cast<float*>(base + L.act);
  uint8_t* aq = base + L.aq;
  float* sa = reinterpret_cast<float*>(base + L.sa);
  float* dd = reinterpret_cast<float*>(base + L.d);
  int* off = reinterpret_cast<int*>(base + L.off);
  int* rows = reinterpret_cast<int*>(base + L.rows);
  const int R = (int)(T * topk);

  int rc = launch_quant_act(x, T, H, H, QLIN_E4M3, xq, sx, st);
  if (rc) return rc;
  moe_route_kernel<<<1, 1024, 2 * E * sizeof(int), st>>>(ids, R, (int)E, off, rows);
  if ((rc = launch_status())) return rc;

  MoeGemmArgs gu{xq, sx, w13, s13, off, rows, topk, (int)H, (int)I, act};
  moe_gemm_kernel<true><<<dim3((unsigned)((I + 63) / 64), (unsigned)E), kMoeNW * 64, 0, st>>>(gu);
  if ((rc = launch_status())) return rc;

  if ((rc = launch_quant_rows_f32(act, R, I, aq, sa, st))) return rc;

  MoeGemmArgs dn{aq, sa, w2, s2, off, rows, topk, (int)I, (int)H, dd};
  moe_gemm_kernel<false><<<dim3((unsigned)((H + 63) / 64), (unsigned)E), kMoeNW * 64, 0, st>>>(dn);
  if ((rc = launch_status())) return rc;

  moe_combine_kernel<<<dim3((unsigned)T), 256, 0, st>>>(dd, ids, wts, topk, (int)H, (int)E, y);
  return launch_status();
}

}  // namespace qlin
