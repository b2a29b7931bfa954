// Host-side internals shared by the libqlin translation units: launcher
// declarations, workspace sizing and the status plumbing of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qlin.h"

namespace qlin {

// Records a failed HIP call (thread-local) and maps it to QLIN_ERR_HIP.
int hip_fail(hipError_t e);

// Checks the launch that was just enqueued.
inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? QLIN_OK : hip_fail(e);
}

inline hipStream_t as_stream(qlin_stream_t s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- repack / conversion launchers (qlin_repack.hip)
int launch_repack_q4_0(const uint16_t* w, int64_t N, int64_t K, uint8_t* codes, uint16_t* steps,
                       int64_t* d_amb, hipStream_t st);
int launch_repack_fp8(const uint8_t* codes, const uint16_t* steps, int64_t N, int64_t K, int fmt,
                      uint8_t* wq, float* ws, hipStream_t st);
int launch_repack_int8(const uint8_t* codes, const uint16_t* steps, int64_t N, int64_t K,
                       int8_t* wq, float* ws, hipStream_t st);
int launch_fnuz_to_ocp(const uint8_t* win, const float* sin, int64_t N, int64_t K, uint8_t* wout,
                       float* sout, int64_t* d_bad, hipStream_t st);
int launch_embed_q4(const int32_t* ids, int64_t T, const uint8_t* codes, const uint16_t* steps,
                    int64_t V, int64_t D, uint16_t* out, hipStream_t st);
int launch_dequant_q4(const uint8_t* codes, const uint16_t* steps, int64_t N, int64_t K,
                      uint16_t* out, hipStream_t st);
int launch_fill_zero(void* p, size_t bytes, hipStream_t st);

// ---- quantisers (qlin_quant.hip)
int launch_quant_act(const uint16_t* a, int64_t M, int64_t K, int64_t lda, int fmt, void* q,
                     float* s, hipStream_t st);
int launch_quant_rows_f32(const float* a, int64_t M, int64_t K, uint8_t* q, float* s,
                          hipStream_t st);
int launch_fp8_encode(const float* x, int64_t n, int fmt, uint8_t* out, hipStream_t st);

// ---- GEMMs (qlin_gemm_decode.hip, qlin_gemm_prefill.hip)
enum GemmKind { kGemmFP8 = 0, kGemmI8 = 1, kGemmW4 = 2 };
size_t gemm_workspace_bytes(int kind, int64_t M, int64_t N, int64_t K);
// Split-K arrival counters occupy the first kGemmCounterBytes of every GEMM
// workspace (zero between calls); partial sums follow them.
constexpr size_t kGemmCounterBytes = 65536;
// W4A16 at M <= 64, K % 256 == 0, on layers too small for one wave per 16
// columns to fill the device (qlin_gemm_w4_decode.hip): no workspace.
bool w4_few_applies(int64_t M, int64_t N, int64_t K);
int launch_w4_few(const void* a, int64_t lda, const void* codes, const void* steps, int64_t M,
                  int64_t N, int64_t K, void* y, int out_f32, hipStream_t st);
int launch_gemm(int kind, const void* a, int64_t lda, const float* sa, const void* w,
                const void* wsc, int64_t M, int64_t N, int64_t K, void* y, int out_f32, void* ws,
                size_t ws_bytes, hipStream_t st);

// ---- MoE (qlin_moe.hip)
// Activation of the gate_up epilogue: SiLU(g) * u, or SwiGLU-OAI (gate
// clamped from above at limit, up to [-limit, limit], then
// g * sigmoid(alpha g) * (u + beta)).
constexpr int kMoeActSilu = 0;
constexpr int kMoeActSwigluOai = 1;
struct MoeAct {
  int kind = kMoeActSilu;
  float alpha = 1.0f, beta = 0.0f, limit = __builtin_inff();
};
struct MoeLayout {
  size_t xq, sx, act, aq, sa, d, cnt, off, rows, total;
};
MoeLayout moe_layout(int64_t T, int64_t H, int64_t I, int64_t E, int topk);
int launch_moe_fp8(const uint16_t* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                   const int32_t* ids, const float* wts, const uint8_t* w13, const float* s13,
                   const uint8_t* w2, const float* s2, uint16_t* y, void* ws, hipStream_t st,
                   const MoeAct& act = MoeAct{});
// Allocation-free FP8 MoE (qlin_moe_fp8_noalloc): the stage buffers live in
// a static device array of this many bytes on each GPU (qlin_moe.hip).
constexpr size_t kMoeScratchBytes = QLIN_MOE_NOALLOC_MAX_BYTES;
// Device address of the current GPU's scratch array, resolved once per
// device (a host-side reference to the array itself is not an address).
int moe_scratch_ptr(void** ptr);
struct MoeW4Layout {
  size_t act, d, off, rows, total;
};
MoeW4Layout moe_w4_layout(int64_t T, int64_t H, int64_t I, int64_t E, int topk);
int launch_moe_w4a16(const uint16_t* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                     const int32_t* ids, const float* wts, const uint8_t* p13, const uint16_t* st13,
                     const uint8_t* p2, const uint16_t* st2, uint16_t* y, void* ws, hipStream_t st);

}  // namespace qlin
