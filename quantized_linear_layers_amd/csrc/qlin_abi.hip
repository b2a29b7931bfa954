// C ABI of libqlin: argument validation, device check, dispatch.
// Validation happens on the host before any HIP call, so an invalid call
// returns a status without touching the device.
#include <mutex>
#include <string.h>

#include <algorithm>

#include "qlin_internal.h"
#include <cmath>

namespace qlin {

static thread_local int g_last_hip = 0;

int hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return QLIN_ERR_HIP;
}

// Once-per-device check that the current device is gfx950.
static int device_ok() {
  static std::mutex mu;
  static signed char state[64] = {0};  // 0 unknown, 1 ok, -1 unsupported
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return QLIN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(mu);
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e);
    state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  return state[dev] == 1 ? QLIN_OK : QLIN_ERR_UNSUPPORTED;
}

static bool a16(const void* p) { return aligned16(p); }

}  // namespace qlin

using namespace qlin;

#define QLIN_CHECK(cond, code) \
  do {                         \
    if (!(cond)) return (code); \
  } while (0)

extern "C" {

int qlin_abi_version(void) { return QLIN_ABI_VERSION; }

const char* qlin_status_str(int s) {
  switch (s) {
    case QLIN_OK: return "ok";
    case QLIN_ERR_ARG: return "invalid argument (null pointer or unknown enum)";
    case QLIN_ERR_SHAPE: return "invalid shape";
    case QLIN_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case QLIN_ERR_WORKSPACE: return "workspace missing or too small";
    case QLIN_ERR_UNSUPPORTED: return "device is not gfx950";
    case QLIN_ERR_HIP: return "HIP call failed";
    default: return "unknown status";
  }
}

int qlin_last_hip_error(void) { return g_last_hip; }

// ------------------------------------------------------------------ repacks
int qlin_repack_q4_0(const qlin_bf16* w, int64_t N, int64_t K, uint8_t* codes, qlin_bf16* steps,
                     int64_t* d_n_ambiguous, qlin_stream_t stream) {
  QLIN_CHECK(N >= 0 && K >= 0 && K % 32 == 0, QLIN_ERR_SHAPE);
  if (N == 0 || K == 0) return QLIN_OK;
  QLIN_CHECK(w && codes && steps, QLIN_ERR_ARG);
  QLIN_CHECK(a16(w) && a16(codes) && ((uintptr_t)steps & 1) == 0 &&
                 ((uintptr_t)d_n_ambiguous & 7) == 0,
             QLIN_ERR_ALIGN);
  int rc = device_ok();
  if (rc) return rc;
  return launch_repack_q4_0(w, N, K, codes, steps, d_n_ambiguous, as_stream(stream));
}

int qlin_repack_fp8(const uint8_t* codes, const qlin_bf16* steps, int64_t N, int64_t K, int fmt,
                    uint8_t* w_q, float* w_scale, qlin_stream_t stream) {
  QLIN_CHECK(fmt == QLIN_E4M3 || fmt == QLIN_E4M3FNUZ, QLIN_ERR_ARG);
  QLIN_CHECK(N >= 0 && K >= 0 && K % 32 == 0 && N <= 0x7FFFFFFF, QLIN_ERR_SHAPE);
  if (N == 0) return QLIN_OK;
  QLIN_CHECK(codes && steps && w_q && w_scale, QLIN_ERR_ARG);
  QLIN_CHECK(a16(codes) && a16(w_q) && ((uintptr_t)steps & 1) == 0 && ((uintptr_t)w_scale & 3) == 0,
             QLIN_ERR_ALIGN);
  int rc = device_ok();
  if (rc) return rc;
  return launch_repack_fp8(codes, steps, N, K, fmt, w_q, w_scale, as_stream(stream));
}

int qlin_repack_int8(const uint8_t* codes, const qlin_bf16* steps, int64_t N, int64_t K,
                     int8_t* w_q, float* w_scale, qlin_stream_t stream) {
  QLIN_CHECK(N >= 0 && K >= 0 && K % 32 == 0 && N <= 0x7FFFFFFF, QLIN_ERR_SHAPE);
  if (N == 0) return QLIN_OK;
  QLIN_CHECK(codes && steps && w_q && w_scale, QLIN_ERR_ARG);
  QLIN_CHECK(a16(codes) && a16(w_q) && ((uintptr_t)steps & 1) == 0 && ((uintptr_t)w_scale & 3) == 0,
             QLIN_ERR_ALIGN);
  int rc = device_ok();
  if (rc) return rc;
  return launch_repack_int8(codes, steps, N, K, w_q, w_scale, as_stream(stream));
}

int qlin_fp8_fnuz_to_ocp(const uint8_t* w_fnuz, const float* s_in, int64_t N, int64_t K,
                         uint8_t* w_ocp, float* s_out, int64_t* d_n_inexact,
                         qlin_stream_t stream) {
  QLIN_CHECK(N >= 0 && K >= 0 && K % 16 == 0 && N <= 0x7FFFFFFF, QLIN_ERR_SHAPE);
  if (N == 0) return QLIN_OK;
  QLIN_CHECK(w_fnuz && s_in && w_ocp && s_out, QLIN_ERR_ARG);
  QLIN_CHECK(a16(w_fnuz) && a16(w_ocp) && ((uintptr_t)s_in & 3) == 0 &&
                 ((uintptr_t)s_out & 3) == 0 && ((uintptr_t)d_n_inexact & 7) == 0,
             QLIN_ERR_ALIGN);
  int rc = device_ok();
  if (rc) return rc;
  return launch_fnuz_to_ocp(w_fnuz, s_in, N, K, w_ocp, s_out, d_n_inexact, as_stream(stream));
}

int qlin_dequant_q4_bf16(const uint8_t* codes, const qlin_bf16* steps, int64_t N, int64_t K,
                         qlin_bf16* out, qlin_stream_t stream) {
  QLIN_CHECK(N >= 0 && K >= 0 && K % 32 == 0, QLIN_ERR_SHAPE);
  if (N == 0 || K == 0) return QLIN_OK;
  QLIN_CHECK(codes && steps && out, QLIN_ERR_ARG);
  QLIN_CHECK(a16(codes) && a16(out) && ((uintptr_t)steps & 1) == 0, QLIN_ERR_ALIGN);
  int rc = device_ok();
  if (rc) return rc;
  return launch_dequant_q4(codes, steps, N, K, out, as_stream(stream));
}

int qlin_embed_q4(const int32_t* ids, int64_t T, const uint8_t* codes, const qlin_bf16* steps,
                  int64_t V, int64_t D, qlin_bf16* out, qlin_stream_t stream) {
  QLIN_CHECK(T >= 0 && V > 0 && D > 0 && D % 32 == 0 && V <= 0x7FFFFFFF && D <= 0x7FFFFFFF &&
                 T <= 0x7FFFFFFF && T * (D / 8) < ((int64_t)1 << 31),
             QLIN_ERR_SHAPE);
  if (T == 0) return QLIN_OK;
  QLIN_CHECK(ids && codes && steps && out, QLIN_ERR_ARG);
  QLIN_CHECK(a16(codes) && a16(out) && ((uintptr_t)steps & 1) == 0 && ((uintptr_t)ids & 3) == 0,
             QLIN_ERR_ALIGN);
  int rc = device_ok();
  if (rc) return rc;
  return launch_embed_q4(ids, T, codes, steps, V, D, out, as_stream(stream));
}

// ------------------------------------------------------------------ quantisers
int qlin_quant_act(const qlin_bf16* a, int64_t M, int64_t K, int64_t lda, int fmt, void* a_q,
                   float* a_scale, qlin_stream_t stream) {
  QLIN_CHECK(fmt == QLIN_E4M3 || fmt == QLIN_E4M3FNUZ || fmt == QLIN_INT8, QLIN_ERR_ARG);
  QLIN_CHECK(M >= 0 && K >= 0 && K % 16 == 0 && lda >= K && M <= 0x7FFFFFFF, QLIN_ERR_SHAPE);
  if (M == 0 || K == 0) return QLIN_OK;
  QLIN_CHECK(a && a_q && a_scale, QLIN_ERR_ARG);
  QLIN_CHECK(a16(a) && a16(a_q) && lda % 8 == 0 && ((uintptr_t)a_scale & 3) == 0, QLIN_ERR_ALIGN);
  int rc = device_ok();
  if (rc) return rc;
  return launch_quant_act(a, M, K, lda, fmt, a_q, a_scale, as_stream(stream));
}

int qlin_quant_weight(const qlin_bf16* w, int64_t N, int64_t K, int fmt, void* w_q, float* w_scale,
                      qlin_stream_t stream) {
  // one output channel = one row of W: the per-row quantiser of the activations
  return qlin_quant_act(w, N, K, K, fmt, w_q, w_scale, stream);
}

int qlin_fp8_encode_f32(const float* x, int64_t n, int fmt, uint8_t* out, qlin_stream_t stream) {
  QLIN_CHECK(fmt == QLIN_E4M3 || fmt == QLIN_E4M3FNUZ, QLIN_ERR_ARG);
  QLIN_CHECK(n >= 0 && n < ((int64_t)1 << 40), QLIN_ERR_SHAPE);
  if (n == 0) return QLIN_OK;
  QLIN_CHECK(x && out, QLIN_ERR_ARG);
  QLIN_CHECK(((uintptr_t)x & 3) == 0, QLIN_ERR_ALIGN);
  int rc = device_ok();
  if (rc) return rc;
  return launch_fp8_encode(x, n, fmt, out, as_stream(stream));
}

// ------------------------------------------------------------------ GEMMs
static int gemm_shape_ok(int64_t M, int64_t N, int64_t K, int kmult) {
  return M >= 0 && N >= 0 && K > 0 && K % kmult == 0 && N % 16 == 0 && M <= 0x7FFFFFFF &&
         N <= 0x7FFFFFFF && K <= 133144;
}

// A linear call keeps the GEMM's own workspace (counter area always
// reserved, so the counters stay at offset 0 for every call) in front of
// the quantised activations and their scales.
static size_t linear_gemm_bytes(int kind, int64_t M, int64_t N, int64_t K) {
  return round_up(std::max(gemm_workspace_bytes(kind, M, N, K), kGemmCounterBytes), 256);
}

size_t qlin_workspace_bytes(int op, int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  switch (op) {
    case QLIN_OP_GEMM_FP8: return gemm_workspace_bytes(kGemmFP8, M, N, K);
    case QLIN_OP_GEMM_W8A8: return gemm_workspace_bytes(kGemmI8, M, N, K);
    case QLIN_OP_GEMM_W4A16: return gemm_workspace_bytes(kGemmW4, M, N, K);
    case QLIN_OP_LINEAR_FP8:
      return linear_gemm_bytes(kGemmFP8, M, N, K) + round_up((size_t)M * K, 256) + round_up((size_t)M * 4, 256);
    case QLIN_OP_LINEAR_W8A8:
      return linear_gemm_bytes(kGemmI8, M, N, K) + round_up((size_t)M * K, 256) + round_up((size_t)M * 4, 256);
    default: return 0;
  }
}

int qlin_workspace_init(void* ws, size_t bytes, qlin_stream_t stream) {
  if (bytes == 0) return QLIN_OK;
  QLIN_CHECK(ws, QLIN_ERR_ARG);
  QLIN_CHECK(a16(ws) && bytes % 16 == 0, QLIN_ERR_ALIGN);
  int rc = device_ok();
  if (rc) return rc;
  return launch_fill_zero(ws, bytes, as_stream(stream));
}

static int gemm_common(int kind, const void* a, int64_t lda, const float* sa, const void* w,
                       const void* wsc, int64_t M, int64_t N, int64_t K, void* y, int out_dtype,
                       void* ws, size_t ws_bytes, qlin_stream_t stream) {
  QLIN_CHECK(out_dtype == QLIN_OUT_BF16 || out_dtype == QLIN_OUT_F32, QLIN_ERR_ARG);
  QLIN_CHECK(gemm_shape_ok(M, N, K, kind == kGemmW4 ? 32 : 16) && lda >= K, QLIN_ERR_SHAPE);
  if (M == 0 || N == 0) return QLIN_OK;
  QLIN_CHECK(a && w && wsc && y && (kind == kGemmW4 || sa), QLIN_ERR_ARG);
  QLIN_CHECK(a16(a) && a16(w) && a16(y) && (kind == kGemmW4 ? lda % 8 == 0 : lda % 16 == 0) &&
                 ((uintptr_t)wsc & 1) == 0,
             QLIN_ERR_ALIGN);
  const size_t need = gemm_workspace_bytes(kind, M, N, K);
  QLIN_CHECK(ws_bytes >= need && (need == 0 || ws), QLIN_ERR_WORKSPACE);
  QLIN_CHECK(need == 0 || ((uintptr_t)ws & 255) == 0, QLIN_ERR_ALIGN);
  int rc = device_ok();
  if (rc) return rc;
  return launch_gemm(kind, a, lda, sa, w, wsc, M, N, K, y, out_dtype == QLIN_OUT_F32, ws, ws_bytes,
                     as_stream(stream));
}

int qlin_gemm_fp8(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q,
                  const float* w_scale, int64_t M, int64_t N, int64_t K, void* y, int out_dtype,
                  void* ws, size_t ws_bytes, qlin_stream_t stream) {
  return gemm_common(kGemmFP8, a_q, K, a_scale, w_q, w_scale, M, N, K, y, out_dtype, ws, ws_bytes,
                     stream);
}

int qlin_gemm_w8a8(const int8_t* a_q, const float* a_scale, const int8_t* w_q,
                   const float* w_scale, int64_t M, int64_t N, int64_t K, void* y, int out_dtype,
                   void* ws, size_t ws_bytes, qlin_stream_t stream) {
  return gemm_common(kGemmI8, a_q, K, a_scale, w_q, w_scale, M, N, K, y, out_dtype, ws, ws_bytes,
                     stream);
}

int qlin_gemm_w4a16(const qlin_bf16* a, int64_t lda, const uint8_t* codes,
                    const qlin_bf16* steps, int64_t M, int64_t N, int64_t K, void* y,
                    int out_dtype, void* ws, size_t ws_bytes, qlin_stream_t stream) {
  return gemm_common(kGemmW4, a, lda, nullptr, codes, steps, M, N, K, y, out_dtype, ws, ws_bytes,
                     stream);
}

static int linear_common(int kind, const qlin_bf16* x, int64_t lda, const void* w_q,
                         const float* w_scale, int64_t M, int64_t N, int64_t K, qlin_bf16* y,
                         void* ws, size_t ws_bytes, qlin_stream_t stream) {
  QLIN_CHECK(gemm_shape_ok(M, N, K, 16) && lda >= K, QLIN_ERR_SHAPE);
  if (M == 0 || N == 0) return QLIN_OK;
  QLIN_CHECK(x && w_q && w_scale && y, QLIN_ERR_ARG);
  QLIN_CHECK(a16(x) && a16(w_q) && a16(y) && lda % 8 == 0 && ((uintptr_t)w_scale & 3) == 0,
             QLIN_ERR_ALIGN);
  const int op = kind == kGemmFP8 ? QLIN_OP_LINEAR_FP8 : QLIN_OP_LINEAR_W8A8;
  QLIN_CHECK(ws && ws_bytes >= qlin_workspace_bytes(op, M, N, K), QLIN_ERR_WORKSPACE);
  QLIN_CHECK(((uintptr_t)ws & 255) == 0, QLIN_ERR_ALIGN);
  int rc = device_ok();
  if (rc) return rc;
  uint8_t* gws = reinterpret_cast<uint8_t*>(ws);
  const size_t gbytes = linear_gemm_bytes(kind, M, N, K);
  uint8_t* aq = gws + gbytes;
  float* sa = reinterpret_cast<float*>(aq + round_up((size_t)M * K, 256));
  hipStream_t st = as_stream(stream);
  rc = launch_quant_act(x, M, K, lda, kind == kGemmFP8 ? QLIN_E4M3 : QLIN_INT8, aq, sa, st);
  if (rc) return rc;
  return launch_gemm(kind, aq, K, sa, w_q, w_scale, M, N, K, y, 0, gws, gbytes, st);
}

int qlin_linear_fp8(const qlin_bf16* x, int64_t lda, const uint8_t* w_q, const float* w_scale,
                    int64_t M, int64_t N, int64_t K, qlin_bf16* y, void* ws, size_t ws_bytes,
                    qlin_stream_t stream) {
  return linear_common(kGemmFP8, x, lda, w_q, w_scale, M, N, K, y, ws, ws_bytes, stream);
}

int qlin_linear_w8a8(const qlin_bf16* x, int64_t lda, const int8_t* w_q, const float* w_scale,
                     int64_t M, int64_t N, int64_t K, qlin_bf16* y, void* ws, size_t ws_bytes,
                     qlin_stream_t stream) {
  return linear_common(kGemmI8, x, lda, w_q, w_scale, M, N, K, y, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ MoE
size_t qlin_moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int topk) {
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return 0;
  return moe_layout(T, H, I, E, topk).total;
}

int qlin_moe_workspace_layout(int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                              size_t offsets[6]) {
  QLIN_CHECK(offsets, QLIN_ERR_ARG);
  const MoeLayout L = moe_layout(T, H, I, E, topk);
  offsets[0] = L.xq;
  offsets[1] = L.sx;
  offsets[2] = L.act;
  offsets[3] = L.aq;
  offsets[4] = L.sa;
  offsets[5] = L.d;
  return QLIN_OK;
}

// Arguments of the FP8 MoE calls other than the workspace; 1 = nothing to
// do (T == 0), else a status.
static int moe_fp8_args(const qlin_bf16* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                        const int32_t* topk_ids, const float* topk_w, const uint8_t* w13,
                        const float* s13, const uint8_t* w2, const float* s2, qlin_bf16* y) {
  QLIN_CHECK(T >= 0 && H > 0 && I > 0 && E > 0 && topk > 0 && H % 32 == 0 && I % 32 == 0 &&
                 E <= 4096 && T * topk <= 0x7FFFFFFF && topk <= E,
             QLIN_ERR_SHAPE);
  if (T == 0) return 1;
  QLIN_CHECK(x && topk_ids && topk_w && w13 && s13 && w2 && s2 && y, QLIN_ERR_ARG);
  QLIN_CHECK(a16(x) && a16(w13) && a16(w2) && a16(y) && ((uintptr_t)topk_ids & 3) == 0 &&
                 ((uintptr_t)topk_w & 3) == 0 && ((uintptr_t)s13 & 3) == 0 &&
                 ((uintptr_t)s2 & 3) == 0,
             QLIN_ERR_ALIGN);
  return QLIN_OK;
}

static int moe_fp8_call(const qlin_bf16* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                        const int32_t* topk_ids, const float* topk_w, const uint8_t* w13,
                        const float* s13, const uint8_t* w2, const float* s2, qlin_bf16* y,
                        void* ws, size_t ws_bytes, qlin_stream_t stream, const MoeAct& act) {
  int rc = moe_fp8_args(x, T, H, I, E, topk, topk_ids, topk_w, w13, s13, w2, s2, y);
  if (rc) return rc == 1 ? QLIN_OK : rc;
  QLIN_CHECK(ws && ws_bytes >= qlin_moe_workspace_bytes(T, H, I, E, topk), QLIN_ERR_WORKSPACE);
  QLIN_CHECK(((uintptr_t)ws & 255) == 0, QLIN_ERR_ALIGN);
  rc = device_ok();
  if (rc) return rc;
  return launch_moe_fp8(x, T, H, I, E, topk, topk_ids, topk_w, w13, s13, w2, s2, y, ws,
                        as_stream(stream), act);
}

int qlin_moe_fp8(const qlin_bf16* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                 const int32_t* topk_ids, const float* topk_w, const uint8_t* w13,
                 const float* s13, const uint8_t* w2, const float* s2, qlin_bf16* y, void* ws,
                 size_t ws_bytes, qlin_stream_t stream) {
  return moe_fp8_call(x, T, H, I, E, topk, topk_ids, topk_w, w13, s13, w2, s2, y, ws, ws_bytes,
                      stream, MoeAct{});
}

int qlin_moe_fp8_noalloc(const qlin_bf16* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                         const int32_t* topk_ids, const float* topk_w, const uint8_t* w13,
                         const float* s13, const uint8_t* w2, const float* s2, qlin_bf16* y,
                         qlin_stream_t stream) {
  int rc = moe_fp8_args(x, T, H, I, E, topk, topk_ids, topk_w, w13, s13, w2, s2, y);
  if (rc) return rc == 1 ? QLIN_OK : rc;
  QLIN_CHECK(qlin_moe_workspace_bytes(T, H, I, E, topk) <= kMoeScratchBytes, QLIN_ERR_WORKSPACE);
  rc = device_ok();
  if (rc) return rc;
  void* ws = nullptr;
  rc = moe_scratch_ptr(&ws);
  if (rc) return rc;
  return launch_moe_fp8(x, T, H, I, E, topk, topk_ids, topk_w, w13, s13, w2, s2, y, ws,
                        as_stream(stream), MoeAct{});
}

int qlin_moe_fp8_swiglu_oai(const qlin_bf16* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                            const int32_t* topk_ids, const float* topk_w, const uint8_t* w13,
                            const float* s13, const uint8_t* w2, const float* s2, float alpha,
                            float beta, float limit, qlin_bf16* y, void* ws, size_t ws_bytes,
                            qlin_stream_t stream) {
  QLIN_CHECK(std::isfinite(alpha) && std::isfinite(beta) && limit > 0.0f, QLIN_ERR_ARG);
  MoeAct act;
  act.kind = kMoeActSwigluOai;
  act.alpha = alpha;
  act.beta = beta;
  act.limit = limit;
  return moe_fp8_call(x, T, H, I, E, topk, topk_ids, topk_w, w13, s13, w2, s2, y, ws, ws_bytes,
                      stream, act);
}

size_t qlin_moe_w4a16_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int topk) {
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return 0;
  return moe_w4_layout(T, H, I, E, topk).total;
}

int qlin_moe_w4a16_workspace_layout(int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                                    size_t offsets[2]) {
  QLIN_CHECK(offsets, QLIN_ERR_ARG);
  const MoeW4Layout L = moe_w4_layout(T, H, I, E, topk);
  offsets[0] = L.act;
  offsets[1] = L.d;
  return QLIN_OK;
}

int qlin_moe_w4a16(const qlin_bf16* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                   const int32_t* topk_ids, const float* topk_w, const uint8_t* codes13,
                   const qlin_bf16* steps13, const uint8_t* codes2, const qlin_bf16* steps2,
                   qlin_bf16* y, void* ws, size_t ws_bytes, qlin_stream_t stream) {
  QLIN_CHECK(T >= 0 && H > 0 && I > 0 && E > 0 && topk > 0 && H % 32 == 0 && I % 32 == 0 &&
                 E <= 4096 && T * topk <= 0x7FFFFFFF && topk <= E,
             QLIN_ERR_SHAPE);
  if (T == 0) return QLIN_OK;
  QLIN_CHECK(x && topk_ids && topk_w && codes13 && steps13 && codes2 && steps2 && y, QLIN_ERR_ARG);
  QLIN_CHECK(a16(x) && a16(codes13) && a16(codes2) && a16(y) && ((uintptr_t)topk_ids & 3) == 0 &&
                 ((uintptr_t)topk_w & 3) == 0 && ((uintptr_t)steps13 & 1) == 0 &&
                 ((uintptr_t)steps2 & 1) == 0,
             QLIN_ERR_ALIGN);
  QLIN_CHECK(ws && ws_bytes >= qlin_moe_w4a16_workspace_bytes(T, H, I, E, topk), QLIN_ERR_WORKSPACE);
  QLIN_CHECK(((uintptr_t)ws & 255) == 0, QLIN_ERR_ALIGN);
  int rc = device_ok();
  if (rc) return rc;
  return launch_moe_w4a16(x, T, H, I, E, topk, topk_ids, topk_w, codes13, steps13, codes2, steps2, y,
                          ws, as_stream(stream));
}

}  // extern "C"
