"""qlin: quantized linear layers for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libqlin.so`` (``include/qlin.h``).
Every computation runs in the library's HIP kernels; this module only checks
tensors, allocates outputs with torch and passes raw device pointers plus
the current HIP stream. Importing it fails loudly if the library has not been
built (``python quantized_linear_layers_amd/build.py``).

bf16 tensors are ``torch.bfloat16``; FP8 codes are ``torch.uint8`` holding
OCP E4M3 (or E4M3FNUZ) bit patterns; int8 codes are ``torch.int8``; int4
codes are ``torch.uint8`` [N, K/2] (low nibble = even k, value c + 8).
"""

from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlin.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libqlin.so not found at {LIB_PATH}: build it with "
        "`python quantized_linear_layers_amd/build.py` (hipcc, gfx950)")

_lib = C.CDLL(LIB_PATH)

# ---------------------------------------------------------------- constants
OK, ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP = range(7)
E4M3, E4M3FNUZ, INT8 = 0, 1, 2
OUT_BF16, OUT_F32 = 0, 1
OP_GEMM_FP8, OP_GEMM_W8A8, OP_GEMM_W4A16, OP_LINEAR_FP8, OP_LINEAR_W8A8 = range(5)

_P, _I64, _INT, _SZ = C.c_void_p, C.c_int64, C.c_int, C.c_size_t
_SIGS = {
    "qlin_abi_version": (_INT, []),
    "qlin_status_str": (C.c_char_p, [_INT]),
    "qlin_last_hip_error": (_INT, []),
    "qlin_repack_q4_0": (_INT, [_P, _I64, _I64, _P, _P, _P, _P]),
    "qlin_repack_fp8": (_INT, [_P, _P, _I64, _I64, _INT, _P, _P, _P]),
    "qlin_repack_int8": (_INT, [_P, _P, _I64, _I64, _P, _P, _P]),
    "qlin_fp8_fnuz_to_ocp": (_INT, [_P, _P, _I64, _I64, _P, _P, _P, _P]),
    "qlin_dequant_q4_bf16": (_INT, [_P, _P, _I64, _I64, _P, _P]),
    "qlin_quant_act": (_INT, [_P, _I64, _I64, _I64, _INT, _P, _P, _P]),
    "qlin_quant_weight": (_INT, [_P, _I64, _I64, _INT, _P, _P, _P]),
    "qlin_embed_q4": (_INT, [_P, _I64, _P, _P, _I64, _I64, _P, _P]),
    "qlin_fp8_encode_f32": (_INT, [_P, _I64, _INT, _P, _P]),
    "qlin_workspace_bytes": (_SZ, [_INT, _I64, _I64, _I64]),
    "qlin_workspace_init": (_INT, [_P, _SZ, _P]),
    "qlin_gemm_fp8": (_INT, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _INT, _P, _SZ, _P]),
    "qlin_gemm_w8a8": (_INT, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _INT, _P, _SZ, _P]),
    "qlin_gemm_w4a16": (_INT, [_P, _I64, _P, _P, _I64, _I64, _I64, _P, _INT, _P, _SZ, _P]),
    "qlin_linear_fp8": (_INT, [_P, _I64, _P, _P, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "qlin_linear_w8a8": (_INT, [_P, _I64, _P, _P, _I64, _I64, _I64, _P, _P, _SZ, _P]),
    "qlin_moe_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _INT]),
    "qlin_moe_workspace_layout": (_INT, [_I64, _I64, _I64, _I64, _INT, C.POINTER(_SZ)]),
    "qlin_moe_fp8": (_INT, [_P, _I64, _I64, _I64, _I64, _INT, _P, _P, _P, _P, _P, _P, _P, _P,
                            _SZ, _P]),
    "qlin_moe_fp8_noalloc": (_INT, [_P, _I64, _I64, _I64, _I64, _INT, _P, _P, _P, _P, _P, _P, _P,
                                    _P]),
    "qlin_moe_fp8_swiglu_oai": (_INT, [_P, _I64, _I64, _I64, _I64, _INT, _P, _P, _P, _P, _P, _P,
                                       C.c_float, C.c_float, C.c_float, _P, _P, _SZ, _P]),
    "qlin_moe_w4a16_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _INT]),
    "qlin_moe_w4a16_workspace_layout": (_INT, [_I64, _I64, _I64, _I64, _INT, C.POINTER(_SZ)]),
    "qlin_moe_w4a16": (_INT, [_P, _I64, _I64, _I64, _I64, _INT, _P, _P, _P, _P, _P, _P, _P, _P,
                              _SZ, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


class QlinError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.qlin_status_str(status).decode()
        if status == ERR_HIP:
            msg += f" (hipError {_lib.qlin_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")
        self.status = status


def lib():
    """The raw ctypes handle of libqlin.so."""
    return _lib


def _call(name: str, *args):
    st = getattr(_lib, name)(*args)
    if st != OK:
        raise QlinError(name, st)


def _ptr(t: torch.Tensor | None):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(t: torch.Tensor, name: str, dtype, ndim: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_FMT = {"e4m3": E4M3, "e4m3fnuz": E4M3FNUZ, "int8": INT8, E4M3: E4M3, E4M3FNUZ: E4M3FNUZ,
        INT8: INT8}

# ---------------------------------------------------------------- workspace
# Buffers are cached per (device, stream): calls on one stream are ordered,
# so they may share a buffer, while calls on two streams may overlap and
# must not share split-K counters, partial sums or MoE stage data. A buffer
# that a call outgrows is replaced by one at least twice its size, and the
# old one is kept alive until the process ends: a HIP graph captured
# earlier, or a kernel still queued on the stream, may hold its address.
# (The retired buffers add up to less than the live one.)
_ws_cache: dict[tuple[int, int], torch.Tensor] = {}
_scratch_cache: dict[tuple[int, int], torch.Tensor] = {}
_retired: list[torch.Tensor] = []


def _cache_key(device: torch.device) -> tuple[int, int]:
    idx = device.index if device.index is not None else torch.cuda.current_device()
    return idx, torch.cuda.current_stream(idx).cuda_stream


def _cached(cache, nbytes: int, device: torch.device, zero: bool) -> torch.Tensor:
    key = _cache_key(device)
    ws = cache.get(key)
    if ws is None or ws.numel() < nbytes:
        size = max(nbytes, 1 << 20, 0 if ws is None else 2 * ws.numel())
        new = (torch.zeros if zero else torch.empty)(size, dtype=torch.uint8,
                                                     device=torch.device("cuda", key[0]))
        if ws is not None:
            _retired.append(ws)
        cache[key] = ws = new
    return ws


def workspace(nbytes: int, device: torch.device) -> torch.Tensor:
    """Zero-initialised workspace of at least nbytes for the current stream
    of `device` (kept for reuse; the library leaves its counter area zero
    after every call)."""
    return _cached(_ws_cache, nbytes, device, True)


def scratch(nbytes: int, device: torch.device) -> torch.Tensor:
    """Scratch of at least nbytes for the current stream of `device`, for
    calls that overwrite their whole workspace (the MoE blocks). Kept apart
    from `workspace`, whose counter area the split-K GEMMs need to find
    zero."""
    return _cached(_scratch_cache, nbytes, device, False)


def workspace_bytes(op: int, M: int, N: int, K: int) -> int:
    return int(_lib.qlin_workspace_bytes(op, M, N, K))


# ---------------------------------------------------------------- repacks
def repack_q4_0(w: torch.Tensor):
    """bf16 QAT weight [N,K] -> (codes u8 [N,K/2], steps bf16 [N,K/32],
    n_ambiguous int64 [1] on device)."""
    _check(w, "w", torch.bfloat16, 2)
    N, K = w.shape
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    steps = torch.empty((N, K // 32), dtype=torch.bfloat16, device=w.device)
    amb = torch.empty(1, dtype=torch.int64, device=w.device)
    _call("qlin_repack_q4_0", _ptr(w), N, K, _ptr(codes), _ptr(steps), _ptr(amb), _stream(w.device))
    return codes, steps, amb


def repack_fp8(codes: torch.Tensor, steps: torch.Tensor, fmt="e4m3"):
    """q4 grid -> (FP8 codes u8 [N,K], per-channel scale f32 [N])."""
    _check(codes, "codes", torch.uint8, 2)
    _check(steps, "steps", torch.bfloat16, 2)
    N, K = codes.shape[0], codes.shape[1] * 2
    wq = torch.empty((N, K), dtype=torch.uint8, device=codes.device)
    ws = torch.empty(N, dtype=torch.float32, device=codes.device)
    _call("qlin_repack_fp8", _ptr(codes), _ptr(steps), N, K, _FMT[fmt], _ptr(wq), _ptr(ws),
          _stream(codes.device))
    return wq, ws


def repack_int8(codes: torch.Tensor, steps: torch.Tensor):
    _check(codes, "codes", torch.uint8, 2)
    _check(steps, "steps", torch.bfloat16, 2)
    N, K = codes.shape[0], codes.shape[1] * 2
    wq = torch.empty((N, K), dtype=torch.int8, device=codes.device)
    ws = torch.empty(N, dtype=torch.float32, device=codes.device)
    _call("qlin_repack_int8", _ptr(codes), _ptr(steps), N, K, _ptr(wq), _ptr(ws),
          _stream(codes.device))
    return wq, ws


def fp8_fnuz_to_ocp(w_fnuz: torch.Tensor, s_in: torch.Tensor):
    """E4M3FNUZ weights + scales -> (OCP codes, scales, n_inexact int64 [1])."""
    _check(w_fnuz, "w_fnuz", torch.uint8, 2)
    _check(s_in, "s_in", torch.float32, 1)
    N, K = w_fnuz.shape
    wo = torch.empty_like(w_fnuz)
    so = torch.empty_like(s_in)
    bad = torch.empty(1, dtype=torch.int64, device=w_fnuz.device)
    _call("qlin_fp8_fnuz_to_ocp", _ptr(w_fnuz), _ptr(s_in), N, K, _ptr(wo), _ptr(so), _ptr(bad),
          _stream(w_fnuz.device))
    return wo, so, bad


def dequant_q4_bf16(codes: torch.Tensor, steps: torch.Tensor) -> torch.Tensor:
    _check(codes, "codes", torch.uint8, 2)
    _check(steps, "steps", torch.bfloat16, 2)
    N, K = codes.shape[0], codes.shape[1] * 2
    out = torch.empty((N, K), dtype=torch.bfloat16, device=codes.device)
    _call("qlin_dequant_q4_bf16", _ptr(codes), _ptr(steps), N, K, _ptr(out), _stream(codes.device))
    return out


# ---------------------------------------------------------------- quantisers
def quant_act(a: torch.Tensor, fmt="e4m3", out=None):
    """bf16 [M,K] (row stride may exceed K) -> (codes [M,K], scale f32 [M]).
    `out` may pass preallocated (codes, scale) tensors."""
    if not (isinstance(a, torch.Tensor) and a.is_cuda and a.dtype == torch.bfloat16 and a.dim() == 2
            and a.stride(1) == 1):
        raise ValueError("a must be a 2-D bf16 device tensor with unit column stride")
    M, K = a.shape
    f = _FMT[fmt]
    if out is not None:
        q, s = out
        _check(q, "out codes", torch.int8 if f == INT8 else torch.uint8, 2)
        _check(s, "out scale", torch.float32, 1)
        if q.shape != (M, K) or s.numel() != M:
            raise ValueError("out shape mismatch")
    else:
        q = torch.empty((M, K), dtype=torch.int8 if f == INT8 else torch.uint8, device=a.device)
        s = torch.empty(M, dtype=torch.float32, device=a.device)
    _call("qlin_quant_act", _ptr(a), M, K, a.stride(0), f, _ptr(q), _ptr(s), _stream(a.device))
    return q, s


def fp8_encode_f32(x: torch.Tensor, fmt="e4m3") -> torch.Tensor:
    _check(x, "x", torch.float32)
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _call("qlin_fp8_encode_f32", _ptr(x), x.numel(), _FMT[fmt], _ptr(out), _stream(x.device))
    return out


# ---------------------------------------------------------------- GEMMs
def _out(M, N, dev, out_dtype):
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out_dtype must be bfloat16 or float32")
    return torch.empty((M, N), dtype=out_dtype, device=dev), (OUT_F32 if out_dtype == torch.float32
                                                              else OUT_BF16)


def gemm_fp8(a_q, a_scale, w_q, w_scale, out_dtype=torch.bfloat16, out=None):
    """Y = ((A_q . W_q^T) * a_scale[:,None]) * w_scale[None,:], OCP E4M3."""
    _check(a_q, "a_q", torch.uint8, 2)
    _check(w_q, "w_q", torch.uint8, 2)
    _check(a_scale, "a_scale", torch.float32, 1)
    _check(w_scale, "w_scale", torch.float32, 1)
    M, K = a_q.shape
    N = w_q.shape[0]
    if w_q.shape[1] != K or a_scale.numel() != M or w_scale.numel() != N:
        raise ValueError("shape mismatch")
    y, od = (out, OUT_F32 if out.dtype == torch.float32 else OUT_BF16) if out is not None else \
        _out(M, N, a_q.device, out_dtype)
    nb = workspace_bytes(OP_GEMM_FP8, M, N, K)
    ws = workspace(nb, a_q.device)
    _call("qlin_gemm_fp8", _ptr(a_q), _ptr(a_scale), _ptr(w_q), _ptr(w_scale), M, N, K, _ptr(y), od,
          _ptr(ws), ws.numel(), _stream(a_q.device))
    return y


def gemm_w8a8(a_q, a_scale, w_q, w_scale, out_dtype=torch.bfloat16, out=None):
    """Y = ((float)(A_q . W_q^T) * a_scale) * w_scale, int32 accumulation."""
    _check(a_q, "a_q", torch.int8, 2)
    _check(w_q, "w_q", torch.int8, 2)
    _check(a_scale, "a_scale", torch.float32, 1)
    _check(w_scale, "w_scale", torch.float32, 1)
    M, K = a_q.shape
    N = w_q.shape[0]
    if w_q.shape[1] != K or a_scale.numel() != M or w_scale.numel() != N:
        raise ValueError("shape mismatch")
    y, od = (out, OUT_F32 if out.dtype == torch.float32 else OUT_BF16) if out is not None else \
        _out(M, N, a_q.device, out_dtype)
    nb = workspace_bytes(OP_GEMM_W8A8, M, N, K)
    ws = workspace(nb, a_q.device)
    _call("qlin_gemm_w8a8", _ptr(a_q), _ptr(a_scale), _ptr(w_q), _ptr(w_scale), M, N, K, _ptr(y),
          od, _ptr(ws), ws.numel(), _stream(a_q.device))
    return y


def gemm_w4a16(a, codes, steps, out_dtype=torch.bfloat16, out=None):
    """Y = A . bf16(c * step)^T with group-32 int4 weights, bf16 activations."""
    if not (isinstance(a, torch.Tensor) and a.is_cuda and a.dtype == torch.bfloat16 and a.dim() == 2
            and a.stride(1) == 1):
        raise ValueError("a must be a 2-D bf16 device tensor with unit column stride")
    _check(codes, "codes", torch.uint8, 2)
    _check(steps, "steps", torch.bfloat16, 2)
    M, K = a.shape
    N = codes.shape[0]
    if codes.shape[1] * 2 != K or steps.shape != (N, K // 32):
        raise ValueError("shape mismatch")
    y, od = (out, OUT_F32 if out.dtype == torch.float32 else OUT_BF16) if out is not None else \
        _out(M, N, a.device, out_dtype)
    nb = workspace_bytes(OP_GEMM_W4A16, M, N, K)
    ws = workspace(nb, a.device)
    _call("qlin_gemm_w4a16", _ptr(a), a.stride(0), _ptr(codes), _ptr(steps), M, N, K, _ptr(y), od,
          _ptr(ws), ws.numel(), _stream(a.device))
    return y


def _linear(name, op, x, w_q, w_scale, wdtype, out=None):
    if not (isinstance(x, torch.Tensor) and x.is_cuda and x.dtype == torch.bfloat16 and x.dim() == 2
            and x.stride(1) == 1):
        raise ValueError("x must be a 2-D bf16 device tensor with unit column stride")
    _check(w_q, "w_q", wdtype, 2)
    _check(w_scale, "w_scale", torch.float32, 1)
    M, K = x.shape
    N = w_q.shape[0]
    if w_q.shape[1] != K or w_scale.numel() != N:
        raise ValueError("shape mismatch")
    if out is not None:
        _check(out, "out", torch.bfloat16, 2)
        if out.shape != (M, N):
            raise ValueError("out shape mismatch")
        y = out
    else:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    ws = workspace(workspace_bytes(op, M, N, K), x.device)
    _call(name, _ptr(x), x.stride(0), _ptr(w_q), _ptr(w_scale), M, N, K, _ptr(y), _ptr(ws),
          ws.numel(), _stream(x.device))
    return y


def linear_fp8(x, w_q, w_scale, out=None):
    """Per-token FP8 quantisation of x followed by the FP8 GEMM (bf16 out)."""
    return _linear("qlin_linear_fp8", OP_LINEAR_FP8, x, w_q, w_scale, torch.uint8, out)


def linear_w8a8(x, w_q, w_scale, out=None):
    """Per-token int8 quantisation of x followed by the int8 GEMM."""
    return _linear("qlin_linear_w8a8", OP_LINEAR_W8A8, x, w_q, w_scale, torch.int8, out)


# ---------------------------------------------------------------- MoE
def moe_workspace_layout(T, H, I, E, topk):
    offs = (C.c_size_t * 6)()
    _call("qlin_moe_workspace_layout", T, H, I, E, topk, offs)
    return [int(o) for o in offs]


def embed_q4(ids, codes, steps):
    """Rows ids [T] (int32) of an int4 table (codes u8 [V,D/2], steps bf16
    [V,D/32]) as bf16 [T,D]; ids outside [0,V) give zero rows."""
    _check(ids, "ids", torch.int32, 1)
    _check(codes, "codes", torch.uint8, 2)
    _check(steps, "steps", torch.bfloat16, 2)
    V, D2 = codes.shape
    D = 2 * D2
    if steps.shape != (V, D // 32):
        raise ValueError("shape mismatch")
    out = torch.empty((ids.numel(), D), dtype=torch.bfloat16, device=codes.device)
    _call("qlin_embed_q4", _ptr(ids), ids.numel(), _ptr(codes), _ptr(steps), V, D, _ptr(out),
          _stream(codes.device))
    return out


def quant_weight(w: torch.Tensor, fmt="e4m3"):
    """Online per-channel quantisation of a bf16 weight [N,K] (contiguous):
    (codes [N,K], scale f32 [N]), one scale per output channel."""
    _check(w, "w", torch.bfloat16, 2)
    N, K = w.shape
    f = _FMT[fmt]
    q = torch.empty((N, K), dtype=torch.int8 if f == INT8 else torch.uint8, device=w.device)
    s = torch.empty(N, dtype=torch.float32, device=w.device)
    _call("qlin_quant_weight", _ptr(w), N, K, f, _ptr(q), _ptr(s), _stream(w.device))
    return q, s


def moe_fp8(x, topk_ids, topk_w, w13, s13, w2, s2, return_stages=False, swiglu_oai=None):
    """FP8 MoE block. x [T,H] bf16; topk_ids int32 [T,k]; topk_w f32 [T,k];
    w13 u8 [E,2I,H], s13 f32 [E,2I]; w2 u8 [E,H,I], s2 f32 [E,H].
    swiglu_oai: None for SiLU(g)*u, or (alpha, beta, limit) for SwiGLU-OAI."""
    _check(x, "x", torch.bfloat16, 2)
    _check(topk_ids, "topk_ids", torch.int32, 2)
    _check(topk_w, "topk_w", torch.float32, 2)
    _check(w13, "w13", torch.uint8, 3)
    _check(s13, "s13", torch.float32, 2)
    _check(w2, "w2", torch.uint8, 3)
    _check(s2, "s2", torch.float32, 2)
    T, H = x.shape
    E, I2, H2 = w13.shape
    I = I2 // 2
    topk = topk_ids.shape[1]
    if H2 != H or w2.shape != (E, H, I) or s13.shape != (E, I2) or s2.shape != (E, H) or \
            topk_w.shape != topk_ids.shape or topk_ids.shape[0] != T:
        raise ValueError("shape mismatch")
    nb = int(_lib.qlin_moe_workspace_bytes(T, H, I, E, topk))
    ws = scratch(nb, x.device) if not return_stages else \
        torch.empty(max(nb, 256), dtype=torch.uint8, device=x.device)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if swiglu_oai is None:
        _call("qlin_moe_fp8", _ptr(x), T, H, I, E, topk, _ptr(topk_ids), _ptr(topk_w), _ptr(w13),
              _ptr(s13), _ptr(w2), _ptr(s2), _ptr(y), _ptr(ws), ws.numel(), _stream(x.device))
    else:
        alpha, beta, limit = (float(v) for v in swiglu_oai)
        _call("qlin_moe_fp8_swiglu_oai", _ptr(x), T, H, I, E, topk, _ptr(topk_ids), _ptr(topk_w),
              _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2), alpha, beta, limit, _ptr(y), _ptr(ws),
              ws.numel(), _stream(x.device))
    if not return_stages:
        return y
    o = moe_workspace_layout(T, H, I, E, topk)
    R = T * topk

    def view(off, n, dt):
        return ws[off: off + n * torch.tensor([], dtype=dt).element_size()].view(dt)

    stages = dict(xq=view(o[0], T * H, torch.uint8).view(T, H), sx=view(o[1], T, torch.float32),
                  act=view(o[2], R * I, torch.float32).view(R, I),
                  aq=view(o[3], R * I, torch.uint8).view(R, I), sa=view(o[4], R, torch.float32),
                  d=view(o[5], R * H, torch.float32).view(R, H))
    return y, stages


MOE_NOALLOC_MAX_BYTES = 64 << 20


def moe_fp8_noalloc(x, topk_ids, topk_w, w13, s13, w2, s2, out=None):
    """The FP8 MoE block through the allocation-free entry point: stage
    buffers in the library's static per-GPU array (calls that overlap on one
    GPU race). `out` may pass a preallocated y [T,H] bf16."""
    _check(x, "x", torch.bfloat16, 2)
    _check(topk_ids, "topk_ids", torch.int32, 2)
    _check(topk_w, "topk_w", torch.float32, 2)
    _check(w13, "w13", torch.uint8, 3)
    _check(s13, "s13", torch.float32, 2)
    _check(w2, "w2", torch.uint8, 3)
    _check(s2, "s2", torch.float32, 2)
    T, H = x.shape
    E, I2, H2 = w13.shape
    I = I2 // 2
    topk = topk_ids.shape[1]
    if H2 != H or w2.shape != (E, H, I) or s13.shape != (E, I2) or s2.shape != (E, H) or \
            topk_w.shape != topk_ids.shape or topk_ids.shape[0] != T:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    else:
        _check(out, "out", torch.bfloat16, 2)
        if out.shape != (T, H):
            raise ValueError("out shape mismatch")
    _call("qlin_moe_fp8_noalloc", _ptr(x), T, H, I, E, topk, _ptr(topk_ids), _ptr(topk_w), _ptr(w13),
          _ptr(s13), _ptr(w2), _ptr(s2), _ptr(out), _stream(x.device))
    return out


def moe_w4a16(x, topk_ids, topk_w, codes13, steps13, codes2, steps2, return_stages=False):
    """W4A16 MoE block. x [T,H] bf16; topk_ids int32 [T,k]; topk_w f32 [T,k];
    codes13 u8 [E,2I,H/2], steps13 bf16 [E,2I,H/32]; codes2 u8 [E,H,I/2],
    steps2 bf16 [E,H,I/32]."""
    _check(x, "x", torch.bfloat16, 2)
    _check(topk_ids, "topk_ids", torch.int32, 2)
    _check(topk_w, "topk_w", torch.float32, 2)
    _check(codes13, "codes13", torch.uint8, 3)
    _check(steps13, "steps13", torch.bfloat16, 3)
    _check(codes2, "codes2", torch.uint8, 3)
    _check(steps2, "steps2", torch.bfloat16, 3)
    T, H = x.shape
    E, I2, H2 = codes13.shape
    I = I2 // 2
    topk = topk_ids.shape[1]
    if H2 * 2 != H or codes2.shape != (E, H, I // 2) or steps13.shape != (E, I2, H // 32) or \
            steps2.shape != (E, H, I // 32) or topk_w.shape != topk_ids.shape or topk_ids.shape[0] != T:
        raise ValueError("shape mismatch")
    nb = int(_lib.qlin_moe_w4a16_workspace_bytes(T, H, I, E, topk))
    ws = scratch(nb, x.device) if not return_stages else \
        torch.empty(max(nb, 256), dtype=torch.uint8, device=x.device)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _call("qlin_moe_w4a16", _ptr(x), T, H, I, E, topk, _ptr(topk_ids), _ptr(topk_w), _ptr(codes13),
          _ptr(steps13), _ptr(codes2), _ptr(steps2), _ptr(y), _ptr(ws), ws.numel(), _stream(x.device))
    if not return_stages:
        return y
    offs = (_SZ * 2)()
    _call("qlin_moe_w4a16_workspace_layout", T, H, I, E, topk, offs)
    R = T * topk
    act = ws[offs[0]: offs[0] + R * I * 2].view(torch.bfloat16).view(R, I)
    d = ws[offs[1]: offs[1] + R * H * 4].view(torch.float32).view(R, H)
    return y, dict(act=act, d=d)
