"""qlin CPU oracle -- TEST INFRASTRUCTURE ONLY.

ctypes wrapper around ``liboracle.so`` (built from ``qlin_oracle.c`` with
gcc). Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import this package; the GPU library never does.

All arrays are numpy; bf16 tensors travel as uint16 bit patterns.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

OCP, FNUZ, INT8 = 0, 1, 2

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _b

        _b.build()
    lib = C.CDLL(LIB_PATH)
    P = C.c_void_p
    I64 = C.c_int64
    sig = {
        "qo_bf16_value": (C.c_float, [C.c_uint16]),
        "qo_bf16_nearest": (C.c_uint16, [C.c_float]),
        "qo_fp8_value": (C.c_double, [C.c_uint8, C.c_int]),
        "qo_fp8_encode": (C.c_uint8, [C.c_float, C.c_int]),
        "qo_fp8_encode_array": (None, [P, I64, C.c_int, P]),
        "qo_bf16_nearest_array": (None, [P, I64, P]),
        "qo_repack_q4_0": (None, [P, I64, I64, P, P, P]),
        "qo_unpack_q4": (None, [P, I64, I64, P]),
        "qo_repack_fp8": (None, [P, P, I64, I64, C.c_int, P, P]),
        "qo_repack_int8": (None, [P, P, I64, I64, P, P]),
        "qo_repack_stats": (None, [P, P, P, P, I64, I64, C.c_int, P, P]),
        "qo_frac_bit_identical": (C.c_double, [P, P, P, I64, I64]),
        "qo_fnuz_to_ocp": (None, [P, P, I64, I64, P, P, P]),
        "qo_quant_act": (None, [P, I64, I64, I64, C.c_int, P, P]),
        "qo_quant_rows_f32": (None, [P, I64, I64, C.c_int, P, P]),
        "qo_gemm_fp8": (None, [P, P, P, P, I64, I64, I64, P, P]),
        "qo_gemm_w8a8": (None, [P, P, P, P, I64, I64, I64, P, P, P]),
        "qo_gemm_w4a16": (None, [P, I64, P, P, I64, I64, I64, P, P]),
        "qo_gemm_bf16": (None, [P, I64, P, I64, I64, I64, P, P]),
        "qo_gemm_fp8_sample": (None, [P, P, P, P, I64, P, P, I64, P]),
        "qo_gemm_w8a8_sample": (None, [P, P, P, P, I64, P, P, I64, P, P]),
        "qo_gemm_w4a16_sample": (None, [P, I64, P, P, I64, P, P, I64, P]),
        "qo_moe_gate_up": (None, [P, P, I64, I64, I64, C.c_int, P, P, P, P]),
        "qo_moe_gate_up_act": (None, [P, P, I64, I64, I64, C.c_int, P, P, P, C.c_int, C.c_float,
                                      C.c_float, C.c_float, P]),
        "qo_quant_weight": (None, [P, I64, I64, C.c_int, P, P]),
        "qo_swiglu_oai": (C.c_float, [C.c_float, C.c_float, C.c_float, C.c_float, C.c_float]),
        "qo_swiglu_oai_array": (None, [P, P, I64, C.c_float, C.c_float, C.c_float, P]),
        "qo_moe_down": (None, [P, P, I64, I64, I64, C.c_int, P, P, P, P, P, P, P]),
        "qo_moe_fp8": (None, [P, I64, I64, I64, I64, C.c_int, P, P, P, P, P, P, P, P, P, P, P, P]),
        "qo_moe_fp8_act": (None, [P, I64, I64, I64, I64, C.c_int, P, P, P, P, P, P, C.c_int,
                                  C.c_float, C.c_float, C.c_float, P, P, P, P, P, P]),
        "qo_moe_w4a16": (None, [P, I64, I64, I64, I64, C.c_int, P, P, P, P, P, P, P, P, P, P]),
        "qo_embed_q4": (None, [P, I64, P, P, I64, I64, P]),
        "qo_max_threads": (C.c_int, []),
        "qo_set_threads": (None, [C.c_int]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---------------------------------------------------------------- codecs
def fp8_value(code: int, fmt: int = OCP) -> float:
    return _load().qo_fp8_value(code, fmt)


def fp8_encode(x: float, fmt: int = OCP) -> int:
    return _load().qo_fp8_encode(x, fmt)


def fp8_encode_array(x: np.ndarray, fmt: int = OCP) -> np.ndarray:
    flat = _c(x, np.float32).ravel()
    out = np.empty(flat.shape, np.uint8)
    _load().qo_fp8_encode_array(_p(flat), flat.size, fmt, _p(out))
    return out.reshape(np.shape(x))


def bf16_nearest_array(x: np.ndarray) -> np.ndarray:
    flat = _c(x, np.float32).ravel()
    out = np.empty(flat.shape, np.uint16)
    _load().qo_bf16_nearest_array(_p(flat), flat.size, _p(out))
    return out.reshape(np.shape(x))


def fp8_decode_table(fmt: int = OCP) -> np.ndarray:
    lib = _load()
    return np.array([lib.qo_fp8_value(b, fmt) for b in range(256)], np.float64)


def bf16_nearest(x: float) -> int:
    return _load().qo_bf16_nearest(x)


def bf16_value(b: int) -> float:
    return _load().qo_bf16_value(b)


# ---------------------------------------------------------------- repacks
def repack_q4_0(w_bf16: np.ndarray):
    """bf16 bits [N,K] -> (packed u8 [N,K/2], steps bf16 bits [N,K/32], n_ambiguous)."""
    w = _c(w_bf16, np.uint16)
    N, K = w.shape
    packed = np.empty((N, K // 2), np.uint8)
    steps = np.empty((N, K // 32), np.uint16)
    amb = np.zeros(1, np.int64)
    _load().qo_repack_q4_0(_p(w), N, K, _p(packed), _p(steps), _p(amb))
    return packed, steps, int(amb[0])


def unpack_q4(packed: np.ndarray, K: int) -> np.ndarray:
    p = _c(packed, np.uint8)
    N = p.shape[0]
    out = np.empty((N, K), np.int8)
    _load().qo_unpack_q4(_p(p), N, K, _p(out))
    return out


def repack_fp8(packed, steps, K: int, fmt: int = OCP):
    p, s = _c(packed, np.uint8), _c(steps, np.uint16)
    N = p.shape[0]
    wq = np.empty((N, K), np.uint8)
    ws = np.empty(N, np.float32)
    _load().qo_repack_fp8(_p(p), _p(s), N, K, fmt, _p(wq), _p(ws))
    return wq, ws


def repack_int8(packed, steps, K: int):
    p, s = _c(packed, np.uint8), _c(steps, np.uint16)
    N = p.shape[0]
    wq = np.empty((N, K), np.int8)
    ws = np.empty(N, np.float32)
    _load().qo_repack_int8(_p(p), _p(s), N, K, _p(wq), _p(ws))
    return wq, ws


def repack_stats(packed, steps, wq, wscale, K: int, fmt: int):
    p, s = _c(packed, np.uint8), _c(steps, np.uint16)
    q = np.ascontiguousarray(wq)
    sc = _c(wscale, np.float32)
    N = p.shape[0]
    rr = np.zeros(1, np.float64)
    mr = np.zeros(1, np.float64)
    _load().qo_repack_stats(_p(p), _p(s), _p(q), _p(sc), N, K, fmt, _p(rr), _p(mr))
    return float(rr[0]), float(mr[0])


def frac_bit_identical(packed, steps, w_bf16) -> float:
    p, s, w = _c(packed, np.uint8), _c(steps, np.uint16), _c(w_bf16, np.uint16)
    N, K = w.shape
    return _load().qo_frac_bit_identical(_p(p), _p(s), _p(w), N, K)


def fnuz_to_ocp(w_fnuz, s_in):
    w, s = _c(w_fnuz, np.uint8), _c(s_in, np.float32)
    N, K = w.shape
    wo = np.empty_like(w)
    so = np.empty_like(s)
    bad = np.zeros(1, np.int64)
    _load().qo_fnuz_to_ocp(_p(w), _p(s), N, K, _p(wo), _p(so), _p(bad))
    return wo, so, int(bad[0])


# ---------------------------------------------------------------- quantisers
def quant_act(a_bf16, fmt: int = OCP):
    a = _c(a_bf16, np.uint16)
    M, K = a.shape
    q = np.empty((M, K), np.int8 if fmt == INT8 else np.uint8)
    s = np.empty(M, np.float32)
    _load().qo_quant_act(_p(a), M, K, K, fmt, _p(q), _p(s))
    return q, s


def quant_weight(w_bf16, fmt: int = OCP):
    """Online per-channel quantisation of bf16 weights W [N,K]: one fp32
    scale per output channel. Returns (codes [N,K], scales [N])."""
    w = _c(w_bf16, np.uint16)
    N, K = w.shape
    q = np.empty((N, K), np.int8 if fmt == INT8 else np.uint8)
    s = np.empty(N, np.float32)
    _load().qo_quant_weight(_p(w), N, K, fmt, _p(q), _p(s))
    return q, s


def swiglu_oai(g, u, alpha: float, beta: float, limit: float):
    """Elementwise SwiGLU-OAI of fp32 gate and up values (same shape)."""
    g, u = _c(g, np.float32), _c(u, np.float32)
    assert g.shape == u.shape
    out = np.empty(g.shape, np.float32)
    _load().qo_swiglu_oai_array(_p(g), _p(u), g.size, alpha, beta, limit, _p(out))
    return out


ACT_SILU, ACT_SWIGLU_OAI = 0, 1


def _act_args(act):
    """act None -> SiLU(g)*u; act (alpha, beta, limit) -> SwiGLU-OAI."""
    if act is None:
        return ACT_SILU, 1.0, 0.0, float("inf")
    alpha, beta, limit = act
    return ACT_SWIGLU_OAI, float(alpha), float(beta), float(limit)


def quant_rows_f32(x, fmt: int = OCP):
    a = _c(x, np.float32)
    M, K = a.shape
    q = np.empty((M, K), np.int8 if fmt == INT8 else np.uint8)
    s = np.empty(M, np.float32)
    _load().qo_quant_rows_f32(_p(a), M, K, fmt, _p(q), _p(s))
    return q, s


# ---------------------------------------------------------------- GEMMs
def gemm_fp8(aq, sa, wq, sw):
    aq, sa, wq, sw = _c(aq, np.uint8), _c(sa, np.float32), _c(wq, np.uint8), _c(sw, np.float32)
    M, K = aq.shape
    N = wq.shape[0]
    y32 = np.empty((M, N), np.float32)
    y16 = np.empty((M, N), np.uint16)
    _load().qo_gemm_fp8(_p(aq), _p(sa), _p(wq), _p(sw), M, N, K, _p(y32), _p(y16))
    return y32, y16


def gemm_w8a8(aq, sa, wq, sw):
    aq, sa, wq, sw = _c(aq, np.int8), _c(sa, np.float32), _c(wq, np.int8), _c(sw, np.float32)
    M, K = aq.shape
    N = wq.shape[0]
    acc = np.empty((M, N), np.int32)
    y32 = np.empty((M, N), np.float32)
    y16 = np.empty((M, N), np.uint16)
    _load().qo_gemm_w8a8(_p(aq), _p(sa), _p(wq), _p(sw), M, N, K, _p(acc), _p(y32), _p(y16))
    return acc, y32, y16


def gemm_w4a16(a_bf16, packed, steps):
    a, p, s = _c(a_bf16, np.uint16), _c(packed, np.uint8), _c(steps, np.uint16)
    M, K = a.shape
    N = p.shape[0]
    y32 = np.empty((M, N), np.float32)
    y16 = np.empty((M, N), np.uint16)
    _load().qo_gemm_w4a16(_p(a), K, _p(p), _p(s), M, N, K, _p(y32), _p(y16))
    return y32, y16


def gemm_bf16(a_bf16, w_bf16):
    a, w = _c(a_bf16, np.uint16), _c(w_bf16, np.uint16)
    M, K = a.shape
    N = w.shape[0]
    y32 = np.empty((M, N), np.float32)
    y16 = np.empty((M, N), np.uint16)
    _load().qo_gemm_bf16(_p(a), K, _p(w), M, N, K, _p(y32), _p(y16))
    return y32, y16


def gemm_fp8_sample(aq, sa, wq, sw, mi, ni):
    aq, sa, wq, sw = _c(aq, np.uint8), _c(sa, np.float32), _c(wq, np.uint8), _c(sw, np.float32)
    mi, ni = _c(mi, np.int64), _c(ni, np.int64)
    out = np.empty(len(mi), np.float32)
    _load().qo_gemm_fp8_sample(_p(aq), _p(sa), _p(wq), _p(sw), aq.shape[1], _p(mi), _p(ni),
                               len(mi), _p(out))
    return out


def gemm_w8a8_sample(aq, sa, wq, sw, mi, ni):
    aq, sa, wq, sw = _c(aq, np.int8), _c(sa, np.float32), _c(wq, np.int8), _c(sw, np.float32)
    mi, ni = _c(mi, np.int64), _c(ni, np.int64)
    acc = np.empty(len(mi), np.int32)
    out = np.empty(len(mi), np.float32)
    _load().qo_gemm_w8a8_sample(_p(aq), _p(sa), _p(wq), _p(sw), aq.shape[1], _p(mi), _p(ni),
                                len(mi), _p(acc), _p(out))
    return acc, out


def gemm_w4a16_sample(a_bf16, packed, steps, mi, ni):
    a, p, s = _c(a_bf16, np.uint16), _c(packed, np.uint8), _c(steps, np.uint16)
    mi, ni = _c(mi, np.int64), _c(ni, np.int64)
    out = np.empty(len(mi), np.float32)
    K = a.shape[1]
    _load().qo_gemm_w4a16_sample(_p(a), K, _p(p), _p(s), K, _p(mi), _p(ni), len(mi), _p(out))
    return out


# ---------------------------------------------------------------- MoE
def moe_fp8(x_bf16, ids, probs, w13, s13, w2, s2, act=None):
    """Full fp8 MoE block. w13 [E,2I,H] u8, s13 [E,2I], w2 [E,H,I] u8, s2 [E,H].
    act: None for SiLU(g)*u, or (alpha, beta, limit) for SwiGLU-OAI.

    Returns dict with act32 [T*topk,I], aq, sa, d32 [T*topk,H], y32 [T,H], y16.
    """
    x = _c(x_bf16, np.uint16)
    ids, probs = _c(ids, np.int32), _c(probs, np.float32)
    w13, s13, w2, s2 = _c(w13, np.uint8), _c(s13, np.float32), _c(w2, np.uint8), _c(s2, np.float32)
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    topk = ids.shape[1]
    R = T * topk
    out = dict(act32=np.empty((R, I), np.float32), aq=np.empty((R, I), np.uint8),
               sa=np.empty(R, np.float32), d32=np.empty((R, H), np.float32),
               y32=np.empty((T, H), np.float32), y16=np.empty((T, H), np.uint16))
    _load().qo_moe_fp8_act(_p(x), T, H, I, E, topk, _p(ids), _p(probs), _p(w13), _p(s13), _p(w2),
                           _p(s2), *_act_args(act), _p(out["act32"]), _p(out["aq"]), _p(out["sa"]), _p(out["d32"]),
                       _p(out["y32"]), _p(out["y16"]))
    return out


def moe_gate_up(xq, sx, ids, w13, s13, act=None):
    xq, sx, ids = _c(xq, np.uint8), _c(sx, np.float32), _c(ids, np.int32)
    w13, s13 = _c(w13, np.uint8), _c(s13, np.float32)
    T, H = xq.shape
    I = w13.shape[1] // 2
    topk = ids.shape[1]
    out = np.empty((T * topk, I), np.float32)
    _load().qo_moe_gate_up_act(_p(xq), _p(sx), T, H, I, topk, _p(ids), _p(w13), _p(s13),
                               *_act_args(act), _p(out))
    return out


def moe_down(aq, sa, ids, probs, w2, s2):
    aq, sa = _c(aq, np.uint8), _c(sa, np.float32)
    ids, probs = _c(ids, np.int32), _c(probs, np.float32)
    w2, s2 = _c(w2, np.uint8), _c(s2, np.float32)
    T, topk = ids.shape
    H, I = w2.shape[1], w2.shape[2]
    d32 = np.empty((T * topk, H), np.float32)
    y32 = np.empty((T, H), np.float32)
    y16 = np.empty((T, H), np.uint16)
    _load().qo_moe_down(_p(aq), _p(sa), T, H, I, topk, _p(ids), _p(probs), _p(w2), _p(s2),
                        _p(d32), _p(y32), _p(y16))
    return d32, y32, y16


def moe_w4a16(x_bf16, ids, probs, p13, st13, p2, st2):
    """Full W4A16 MoE block. p13 [E,2I,H/2] u8 codes, st13 [E,2I,H/32] bf16
    steps, p2 [E,H,I/2], st2 [E,H,I/32].

    Returns dict with act16 [T*topk,I] (bf16 bits), d32 [T*topk,H], y32 [T,H], y16.
    """
    x = _c(x_bf16, np.uint16)
    ids, probs = _c(ids, np.int32), _c(probs, np.float32)
    p13, st13, p2, st2 = _c(p13, np.uint8), _c(st13, np.uint16), _c(p2, np.uint8), _c(st2, np.uint16)
    T, H = x.shape
    E, I2, _ = p13.shape
    I = I2 // 2
    topk = ids.shape[1]
    R = T * topk
    out = dict(act16=np.empty((R, I), np.uint16), d32=np.empty((R, H), np.float32),
               y32=np.empty((T, H), np.float32), y16=np.empty((T, H), np.uint16))
    _load().qo_moe_w4a16(_p(x), T, H, I, E, topk, _p(ids), _p(probs), _p(p13), _p(st13), _p(p2),
                         _p(st2), _p(out["act16"]), _p(out["d32"]), _p(out["y32"]), _p(out["y16"]))
    return out


def embed_q4(ids, packed, steps):
    """Rows ids [T] of an int4 table (packed [V,D/2] u8, steps [V,D/32] bf16)
    as bf16 bits [T,D]; ids outside [0,V) give zero rows."""
    ids, p, s = _c(ids, np.int32), _c(packed, np.uint8), _c(steps, np.uint16)
    V, D2 = p.shape
    D = 2 * D2
    out = np.empty((ids.size, D), np.uint16)
    _load().qo_embed_q4(_p(ids), ids.size, _p(p), _p(s), V, D, _p(out))
    return out


def max_threads() -> int:
    return _load().qo_max_threads()


def set_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on (timing only)."""
    _load().qo_set_threads(int(n))
