/*
 * qlin -- quantized linear layers for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libqlin.so. Every entry point takes plain pointers and sizes; no
 * framework types cross this boundary.
 *
 * Conventions (all entry points):
 *   - Shapes follow a PyTorch Linear: activations A [M,K] row-major, weights
 *     W [N,K] with K contiguous (one row per output channel), outputs Y [M,N].
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The
 *     library allocates and frees no device memory and keeps no per-call
 *     state; inputs must not alias outputs.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream). Arguments are validated on the host before any
 *     launch, so a call that returns an error has enqueued nothing.
 *     QLIN_OK means the work was enqueued, not that it has finished.
 *   - Device-side counters (int64) are written asynchronously; synchronise
 *     the stream before reading them.
 *   - Pointers must be 16-byte aligned; K must be a multiple of 16 (32 for
 *     int4 data); N must be a multiple of 16. M = 0 (or N = 0) is a no-op.
 *   - bf16 values travel as uint16_t bit patterns (qlin_bf16).
 *
 * Sources: the web pages on the weight-format linear layer of LLM serving,
 * cited by page and section:
 *   [E2B]  "MI300X: Gemma 4 E2B, fp8 fastest yet farthest from the original
 *          weights" (geoz.com.cn article)
 *   [SIZES] "Gemma 4 From E2B to 31B on an AMD MI300X" (dev.to)
 *   [CARD] "Gemma 4 31B-it QAT, FP8 E4M3 W8A8, text only" (model card)
 *   [PR]   vLLM PR #45854 report, "Enable fp8_per_channel for bf16 weights
 *          on mi300x" (prhub.com.cn)
 */
#ifndef QLIN_H
#define QLIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t qlin_bf16;
typedef void* qlin_stream_t; /* hipStream_t */

#define QLIN_ABI_VERSION 1

/* Status codes. */
enum {
  QLIN_OK = 0,
  QLIN_ERR_ARG = 1,         /* null pointer or unknown enum value */
  QLIN_ERR_SHAPE = 2,       /* negative size, K/N/lda not allowed */
  QLIN_ERR_ALIGN = 3,       /* pointer not 16-byte aligned */
  QLIN_ERR_WORKSPACE = 4,   /* workspace missing or too small */
  QLIN_ERR_UNSUPPORTED = 5, /* current device is not gfx950 */
  QLIN_ERR_HIP = 6          /* a HIP call failed; see qlin_last_hip_error() */
};

/* Element formats. */
enum {
  QLIN_E4M3 = 0,     /* OCP FP8 E4M3: max 448, signed zero */
  QLIN_E4M3FNUZ = 1, /* FP8 E4M3FNUZ: max 240, no negative zero */
  QLIN_INT8 = 2      /* symmetric int8, [-127, 127] */
};

/* Output element types. */
enum { QLIN_OUT_BF16 = 0, QLIN_OUT_F32 = 1 };

/* Workspace-using operations (for qlin_workspace_bytes). */
enum {
  QLIN_OP_GEMM_FP8 = 0,
  QLIN_OP_GEMM_W8A8 = 1,
  QLIN_OP_GEMM_W4A16 = 2,
  QLIN_OP_LINEAR_FP8 = 3,
  QLIN_OP_LINEAR_W8A8 = 4
};

/* Version of this ABI (QLIN_ABI_VERSION). */
int qlin_abi_version(void);

/* Static string for a status code. */
const char* qlin_status_str(int status);

/* hipError_t of the last failed HIP call on this host thread (0 if none). */
int qlin_last_hip_error(void);

/* ------------------------------------------------------------------------
 * Offline repacks
 * ------------------------------------------------------------------------ */

/* q4_0 repack: recover the trained 4-bit grid of a QAT weight stored as
 * bf16 ([E2B] "Step 1": the 4-bit repack recovers each group's trained step
 * and stores the values as int4 without re-rounding; [SIZES] format table:
 * int4 holding the QAT grid exactly; [CARD]: one scale per group of 32).
 *   w        [N][K] bf16, the QAT values (each group of 32 along K is c*step
 *            rounded to bf16, c in [-8, 7]).
 *   codes    [N][K/2] output, offset-binary u = c + 8, two per byte, the low
 *            nibble holds the even k.
 *   steps    [N][K/32] output bf16 step per group: the smallest step whose
 *            grid reproduces all 32 stored values; when no bf16 step does (a
 *            trained step that is not a bf16 value), the candidate step whose
 *            nearest codes (clamped to [-8, 7]) reproduce the most values,
 *            the smaller on ties. Candidates: |w_i| / p, p in {1, 2, 4, 8},
 *            and the 17 bf16 values nearest absmax/a, a in {3, 5, 6, 7}.
 *   d_n_ambiguous  device int64 output: number of groups not recovered
 *            unambiguously (all-zero group, several steps fit, no power-of-two
 *            code so the step came from the neighbour search, or no 4-bit
 *            grid fits). May be NULL.
 * Requires K % 32 == 0. */
int qlin_repack_q4_0(const qlin_bf16* w, int64_t N, int64_t K, uint8_t* codes, qlin_bf16* steps,
                     int64_t* d_n_ambiguous, qlin_stream_t stream);

/* FP8 per-output-channel repack of a q4 grid ([E2B] "Step 1" fp8 build and
 * its verify report; [CARD]: every Linear stored as FP8 E4M3 with one
 * float32 scale per output channel, no calibration data).
 *   grid value w = c * step (exact in fp32); s = max_k |w| / FMAX
 *   (448 for QLIN_E4M3, 240 for QLIN_E4M3FNUZ); q = nearest-even code of
 *   w / s, saturating. An all-zero row gets s = 0 and codes 0.
 *   codes/steps as produced by qlin_repack_q4_0; w_q [N][K] bytes;
 *   w_scale [N] fp32. fmt: QLIN_E4M3 or QLIN_E4M3FNUZ. K % 32 == 0. */
int qlin_repack_fp8(const uint8_t* codes, const qlin_bf16* steps, int64_t N, int64_t K, int fmt,
                    uint8_t* w_q, float* w_scale, qlin_stream_t stream);

/* int8 per-output-channel repack of a q4 grid ([SIZES] format table: int8
 * weights per channel; [E2B] fidelity section: 255 levels per row).
 *   s = max_k |c*step| / 127; q = clamp(rint(w / s), -127, 127).
 *   w_q [N][K] int8; w_scale [N] fp32. K % 32 == 0. */
int qlin_repack_int8(const uint8_t* codes, const qlin_bf16* steps, int64_t N, int64_t K,
                     int8_t* w_q, float* w_scale, qlin_stream_t stream);

/* E4M3FNUZ -> OCP E4M3 conversion of per-channel FP8 weights ([E2B] "Tip:
 * E4M3 or E4M3FNUZ": the serving loader converts the FP8 flavour at load
 * time; this GPU's FP8 is OCP, so the conversion runs the other way).
 * Per row: without any +-240 code the bits are kept and the scale halved
 * (exact); otherwise the scale is kept and each value re-encoded in OCP
 * (exact except odd mantissas in the two lowest binades, which round to
 * nearest even). d_n_inexact (device int64, may be NULL) receives the number
 * of inexact values plus invalid (0x80) inputs, which are written as 0.
 *   w_fnuz, w_ocp [N][K] bytes; s_in, s_out [N] fp32. */
int qlin_fp8_fnuz_to_ocp(const uint8_t* w_fnuz, const float* s_in, int64_t N, int64_t K,
                         uint8_t* w_ocp, float* s_out, int64_t* d_n_inexact,
                         qlin_stream_t stream);

/* Dequantise int4 codes to bf16: out[n][k] = bf16(c * step), the operand the
 * W4A16 GEMM multiplies ([SIZES] "The 4-Bit Builds Stay Slow": the kernel
 * unpacks the weights to bf16 before each multiply). out [N][K]. */
int qlin_dequant_q4_bf16(const uint8_t* codes, const qlin_bf16* steps, int64_t N, int64_t K,
                         qlin_bf16* out, qlin_stream_t stream);

/* int4 vocabulary table lookup ([E2B] tip on the int4 vocabulary tables;
 * [SIZES] "Tip: int4 Embedding Tables Cost More at Larger Sizes": the
 * embedding, untied lm_head and per-layer embedding tables packed int4 in
 * groups of 32 as trained). out[t][k] = bf16(c * step) of row ids[t] of the
 * table, the values qlin_dequant_q4_bf16 gives for that row; an id outside
 * [0, V) yields a row of zeros (ids are device data, so they are not an
 * error). ids [T] int32 (4-byte aligned); codes [V][D/2] (16-byte aligned),
 * steps [V][D/32] bf16; out [T][D] bf16 (16-byte aligned); D % 32 == 0,
 * V <= 2^31 - 1, T * D / 8 < 2^31 (else QLIN_ERR_SHAPE). The untied lm_head
 * is qlin_gemm_w4a16 with N = V. */
int qlin_embed_q4(const int32_t* ids, int64_t T, const uint8_t* codes, const qlin_bf16* steps,
                  int64_t V, int64_t D, qlin_bf16* out, qlin_stream_t stream);

/* ------------------------------------------------------------------------
 * Dynamic per-token activation quantisation ([CARD]: activations quantised
 * to FP8 per token at run time; [SIZES] format table: int8 activations per
 * token).
 *   s[m] = max_k |a[m,k]| / FMAX (448 for QLIN_E4M3, 127 for QLIN_INT8);
 *   q = nearest-even E4M3 code of a / s (saturating), or
 *   clamp(rint(a / s), -127, 127). A row of zeros gets s = 0 and codes 0.
 *   a [M][lda] bf16 (lda >= K, lda % 8 == 0); a_q [M][K] bytes; a_scale [M].
 * ------------------------------------------------------------------------ */
int qlin_quant_act(const qlin_bf16* a, int64_t M, int64_t K, int64_t lda, int fmt, void* a_q,
                   float* a_scale, qlin_stream_t stream);

/* Online per-channel quantisation of bf16 (non-QAT) weights ([PR]:
 * fp8_per_channel enabled for bf16 weights on the GPU, one scale per output
 * channel): each row n of W [N][K] gets w_scale[n] = max_k |w[n,k]| / FMAX
 * and codes enc(w / w_scale[n]), exactly qlin_quant_act on W's rows (FMAX
 * 448 QLIN_E4M3, 240 QLIN_E4M3FNUZ, 127 QLIN_INT8). w [N][K] bf16, K % 16
 * == 0; w_q [N][K] bytes; w_scale [N] fp32. Errors as for qlin_quant_act. */
int qlin_quant_weight(const qlin_bf16* w, int64_t N, int64_t K, int fmt, void* w_q, float* w_scale,
                      qlin_stream_t stream);

/* Element-wise fp32 -> FP8 encoder (nearest even, saturating), the codec the
 * quantisers use. fmt: QLIN_E4M3 or QLIN_E4M3FNUZ. x, out: n elements. */
int qlin_fp8_encode_f32(const float* x, int64_t n, int fmt, uint8_t* out, qlin_stream_t stream);

/* ------------------------------------------------------------------------
 * GEMMs. Workspace: the split-K paths keep per-tile arrival counters (the
 * first 64 KiB) and fp32/int32 partial sums (after them) in a caller-provided
 * workspace of qlin_workspace_bytes(op, M, N, K) bytes (256-byte aligned;
 * 0 means none is needed). The counter area must be ZERO before the first
 * call that uses the workspace (allocate it zeroed, or call
 * qlin_workspace_init); every call leaves it zero again, whatever its shape,
 * so one zeroed workspace serves all later calls. Calls that share one
 * workspace must be ordered on one stream. The MoE calls overwrite their
 * whole workspace: a buffer lent to them must be zeroed again
 * (qlin_workspace_init) before it serves a GEMM.
 * ------------------------------------------------------------------------ */
size_t qlin_workspace_bytes(int op, int64_t M, int64_t N, int64_t K);

/* Zero a workspace of `bytes` bytes (with a fill kernel). */
int qlin_workspace_init(void* ws, size_t bytes, qlin_stream_t stream);

/* Row-wise scaled FP8 W8A8 GEMM ([E2B] "Step 3": RowWiseTorchFP8Scaled-
 * MMLinearKernel for compressed-tensors W8A8 FP8; [CARD]: per-channel
 * weight scale, per-token activation scale):
 *   Y[m,n] = ((sum_k a[m,k] * w[n,k]) * a_scale[m]) * w_scale[n],
 *   fp32 accumulation, OCP E4M3 operands, written as bf16 (nearest even)
 *   or fp32 (out_dtype).
 *   a_q [M][K], w_q [N][K] OCP E4M3 codes; y [M][N]. */
int qlin_gemm_fp8(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q,
                  const float* w_scale, int64_t M, int64_t N, int64_t K, void* y, int out_dtype,
                  void* ws, size_t ws_bytes, qlin_stream_t stream);

/* int8 W8A8 GEMM ([E2B] "Step 3": TritonInt8ScaledMMLinearKernel; "Step 2":
 * the framework int8 matmul refuses M <= 16 -- here every M >= 1 works):
 *   acc = sum_k a*w in int32 (exact for K <= 133144);
 *   Y = ((float)acc * a_scale[m]) * w_scale[n]. */
int qlin_gemm_w8a8(const int8_t* a_q, const float* a_scale, const int8_t* w_q,
                   const float* w_scale, int64_t M, int64_t N, int64_t K, void* y, int out_dtype,
                   void* ws, size_t ws_bytes, qlin_stream_t stream);

/* W4A16 GEMM with group-32 int4 weights and bf16 activations ([SIZES] "The
 * 4-Bit Builds Stay Slow": TritonW4A16LinearKernel unpacks the weights to
 * bf16 before each multiply; [E2B]: the card has no int4 multiply):
 *   Y[m,n] = sum_k a[m,k] * bf16(c[n,k] * step[n,k/32]), fp32 accumulation.
 *   a [M][lda] bf16 (lda % 8 == 0); codes/steps as from qlin_repack_q4_0.
 *   Steps must be finite with magnitude below 2^117 (the unpack computes
 *   c*step as (1024 + u)*step - 1032*step; larger steps overflow to inf;
 *   q4_0 steps are fp16 values, far below this). K % 32 == 0; the fastest
 *   step loads need K % 256 == 0 and a 16-byte aligned steps pointer. */
int qlin_gemm_w4a16(const qlin_bf16* a, int64_t lda, const uint8_t* codes,
                    const qlin_bf16* steps, int64_t M, int64_t N, int64_t K, void* y,
                    int out_dtype, void* ws, size_t ws_bytes, qlin_stream_t stream);

/* FP8 linear with the per-token quantisation in front ([CARD]: activations
 * quantised to FP8 per token at run time): qlin_quant_act(QLIN_E4M3) into
 * the workspace, then qlin_gemm_fp8. x [M][lda] bf16, y [M][N] bf16.
 * Workspace of qlin_workspace_bytes(QLIN_OP_LINEAR_*, M, N, K): the GEMM's
 * counter area (first 64 KiB, same zero rule as above) and partial sums,
 * then the quantised activations and their scales. */
int qlin_linear_fp8(const qlin_bf16* x, int64_t lda, const uint8_t* w_q, const float* w_scale,
                    int64_t M, int64_t N, int64_t K, qlin_bf16* y, void* ws, size_t ws_bytes,
                    qlin_stream_t stream);

/* int8 linear: qlin_quant_act(QLIN_INT8) into the workspace, then
 * qlin_gemm_w8a8. */
int qlin_linear_w8a8(const qlin_bf16* x, int64_t lda, const int8_t* w_q, const float* w_scale,
                     int64_t M, int64_t N, int64_t K, qlin_bf16* y, void* ws, size_t ws_bytes,
                     qlin_stream_t stream);

/* ------------------------------------------------------------------------
 * FP8 mixture-of-experts block ([SIZES] "Step 1 -- Build the Larger
 * Repacks": fused gate_up / down expert banks split per expert, router kept
 * outside in bf16; [PR]: fp8 MoE with per-token activation scales and
 * per-output-channel weight scales). Routing is an input.
 *   x [T][H] bf16; topk_ids [T][topk] int32 in [0,E); topk_w [T][topk] fp32;
 *   w13 [E][2I][H] OCP E4M3 (rows 0..I-1 gate, I..2I-1 up), s13 [E][2I];
 *   w2 [E][H][I] OCP E4M3, s2 [E][H]; y [T][H] bf16.
 * For token t and slot j (expert e, weight p):
 *   (xq, sx) = per-token FP8 quant of x;
 *   h = (xq . w13[e]^T) * sx * s13[e]   (fp32);  g = h[:I], u = h[I:];
 *   act = SiLU(g) * u (fp32); (aq, sa) = per-row FP8 quant of act;
 *   d = (aq . w2[e]^T) * sa * s2[e]       (fp32);
 *   y[t] = bf16(sum_j p_j * d_j), summed in slot order j = 0..topk-1.
 * Expert ids outside [0, E) contribute nothing. H, I multiples of 32.
 * Workspace: qlin_moe_workspace_bytes(T, H, I, E, topk) bytes (no zeroing
 * needed); after the call it holds the stage results at the offsets given by
 * qlin_moe_workspace_layout. */
int qlin_moe_fp8(const qlin_bf16* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                 const int32_t* topk_ids, const float* topk_w, const uint8_t* w13,
                 const float* s13, const uint8_t* w2, const float* s2, qlin_bf16* y, void* ws,
                 size_t ws_bytes, qlin_stream_t stream);

/* Allocation-free variant of qlin_moe_fp8, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same block, kernels and results,
 * with the stage buffers in a static device array that the library holds on
 * each GPU it runs on, QLIN_MOE_NOALLOC_MAX_BYTES bytes, until the process
 * ends. The caller passes inputs and outputs only. A call whose
 * qlin_moe_workspace_bytes(T, H, I, E, topk) exceeds the array returns
 * QLIN_ERR_WORKSPACE (E=128, H=2048, I=768, top-8 needs about 50 MiB at
 * T = 512). Every call on one GPU uses that GPU's array, which keeps what
 * the last call wrote: calls that overlap in time on one GPU (two streams,
 * two host threads) race, and the caller must order them. The array's
 * device address is looked up on the first call on each device; no call
 * allocates or frees memory. Other errors as for qlin_moe_fp8. */
#define QLIN_MOE_NOALLOC_MAX_BYTES ((size_t)64 << 20)
int qlin_moe_fp8_noalloc(const qlin_bf16* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                         const int32_t* topk_ids, const float* topk_w, const uint8_t* w13,
                         const float* s13, const uint8_t* w2, const float* s2, qlin_bf16* y,
                         qlin_stream_t stream);

/* The same block with the SwiGLU-OAI activation in place of SiLU(g) * u
 * ([PR]: the fp8 MoE config carries gemm1_alpha / gemm1_beta, 1.702 / 1.0
 * for MiniMax-M3, and a clamp limit):
 *   g' = min(g, limit); u' = min(max(u, -limit), limit);
 *   act = g' * sigmoid(alpha * g') * (u' + beta)   (fp32).
 * alpha and beta finite, limit > 0 (+inf: no clamp), else QLIN_ERR_ARG.
 * Arguments, workspace and stage results as for qlin_moe_fp8. */
int qlin_moe_fp8_swiglu_oai(const qlin_bf16* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                            const int32_t* topk_ids, const float* topk_w, const uint8_t* w13,
                            const float* s13, const uint8_t* w2, const float* s2, float alpha,
                            float beta, float limit, qlin_bf16* y, void* ws, size_t ws_bytes,
                            qlin_stream_t stream);

/* Workspace bytes of qlin_moe_fp8 and qlin_moe_fp8_swiglu_oai. */
size_t qlin_moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int topk);

/* Byte offsets of the MoE stage results inside its workspace (R = T*topk):
 *   [0] xq  [T][H] u8     [1] sx  [T] f32      [2] act [R][I] f32
 *   [3] aq  [R][I] u8     [4] sa  [R] f32      [5] d   [R][H] f32
 * Row r = t*topk + j. Returns QLIN_OK, or QLIN_ERR_ARG for a NULL out. */
int qlin_moe_workspace_layout(int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                              size_t offsets[6]);

/* ------------------------------------------------------------------------
 * W4A16 mixture-of-experts block ([SIZES] "The 4-Bit Builds Stay Slow": the
 * 4-bit builds of the MoE model run a WNA16 expert path -- bf16 activations,
 * group-32 int4 expert weights -- on the expert banks split per expert as in
 * "Step 1"). Routing is an input, as for qlin_moe_fp8.
 *   x [T][H] bf16; topk_ids [T][topk] int32 in [0,E); topk_w [T][topk] fp32;
 *   codes13 [E][2I][H/2] packed int4 (layout of qlin_repack_q4_0; rows
 *   0..I-1 gate, I..2I-1 up), steps13 [E][2I][H/32] bf16;
 *   codes2 [E][H][I/2], steps2 [E][H][I/32]; y [T][H] bf16.
 * With wd = bf16(c * step), for token t and slot j (expert e, weight p):
 *   h = x . W13d[e]^T (fp32);  g = h[:I], u = h[I:];
 *   act = bf16(SiLU(g) * u)   (computed in fp32, rounded once);
 *   d = act . W2d[e]^T        (fp32);
 *   y[t] = bf16(sum_j p_j * d_j), summed in slot order j = 0..topk-1.
 * Expert ids outside [0, E) contribute nothing. H, I multiples of 32; x,
 * codes and y 16-byte aligned, steps 2-byte aligned (16-byte aligned step
 * rows with H, I multiples of 256 take the faster bulk step loads).
 * Workspace: qlin_moe_w4a16_workspace_bytes(T, H, I, E, topk) bytes,
 * 256-byte aligned (no zeroing needed); after the call it holds the stage
 * results at the offsets given by qlin_moe_w4a16_workspace_layout.
 * Errors as for qlin_moe_fp8. */
int qlin_moe_w4a16(const qlin_bf16* x, int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                   const int32_t* topk_ids, const float* topk_w, const uint8_t* codes13,
                   const qlin_bf16* steps13, const uint8_t* codes2, const qlin_bf16* steps2,
                   qlin_bf16* y, void* ws, size_t ws_bytes, qlin_stream_t stream);

/* Workspace bytes of qlin_moe_w4a16 (0 for a non-positive size). */
size_t qlin_moe_w4a16_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int topk);

/* Byte offsets of its stage results (R = T*topk, row r = t*topk + j):
 *   [0] act [R][I] bf16     [1] d [R][H] f32
 * Returns QLIN_OK, or QLIN_ERR_ARG for a NULL out. */
int qlin_moe_w4a16_workspace_layout(int64_t T, int64_t H, int64_t I, int64_t E, int topk,
                                    size_t offsets[2]);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_H */
