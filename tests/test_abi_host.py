"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every entry point the header declares, and rejects invalid arguments with
the documented status before touching the device."""

import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlin.h")


@pytest.fixture(scope="module")
def q():
    import quantized_linear_layers_amd as qlin

    return qlin


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s*(qlin_\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol(q):
    names = _declared()
    assert len(names) >= 20
    lib = C.CDLL(q.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(q.EXPORTED)


def test_version_and_status_strings(q):
    lib = q.lib()
    assert lib.qlin_abi_version() == 1
    for s in range(7):
        assert lib.qlin_status_str(s)
    assert lib.qlin_status_str(99) == b"unknown status"


# fake (never dereferenced) device addresses: validation fails before use
A16 = C.c_void_p(0x10000)
A_ODD = C.c_void_p(0x10001)


def test_gemm_validation(q):
    lib = q.lib()
    ws = C.c_void_p(0x100000)
    # K not a multiple of 16
    assert lib.qlin_gemm_fp8(A16, A16, A16, A16, 4, 512, 17, A16, 0, ws, 1 << 20, None) == q.ERR_SHAPE
    # N not a multiple of 16
    assert lib.qlin_gemm_w8a8(A16, A16, A16, A16, 4, 500, 256, A16, 0, ws, 1 << 20, None) == q.ERR_SHAPE
    # negative M
    assert lib.qlin_gemm_fp8(A16, A16, A16, A16, -1, 512, 256, A16, 0, ws, 1 << 20, None) == q.ERR_SHAPE
    # null operand
    assert lib.qlin_gemm_fp8(None, A16, A16, A16, 4, 512, 256, A16, 0, ws, 1 << 20, None) == q.ERR_ARG
    # bad output dtype
    assert lib.qlin_gemm_fp8(A16, A16, A16, A16, 4, 512, 256, A16, 7, ws, 1 << 20, None) == q.ERR_ARG
    # misaligned weight pointer
    assert lib.qlin_gemm_fp8(A16, A16, A_ODD, A16, 4, 512, 256, A16, 0, ws, 1 << 20, None) == q.ERR_ALIGN
    # W4A16 needs K % 32 == 0
    assert lib.qlin_gemm_w4a16(A16, 48, A16, A16, 4, 512, 48, A16, 0, ws, 1 << 20, None) == q.ERR_SHAPE
    # lda < K
    assert lib.qlin_gemm_w4a16(A16, 32, A16, A16, 4, 512, 64, A16, 0, ws, 1 << 20, None) == q.ERR_SHAPE
    # M = 0 is a no-op (returns before any device call)
    assert lib.qlin_gemm_fp8(None, None, None, None, 0, 512, 256, None, 0, None, 0, None) == q.OK


def test_workspace_validation(q):
    lib = q.lib()
    # a narrow, deep decode shape: few column tiles, so K is split across
    # workgroups and a workspace is needed
    need = lib.qlin_workspace_bytes(q.OP_GEMM_FP8, 64, 512, 16384)
    assert need > 65536
    assert lib.qlin_gemm_fp8(A16, A16, A16, A16, 64, 512, 16384, A16, 0, C.c_void_p(0x100000),
                             need - 1, None) == q.ERR_WORKSPACE
    assert lib.qlin_gemm_fp8(A16, A16, A16, A16, 64, 512, 16384, A16, 0, None, need, None) == q.ERR_WORKSPACE
    # workspace must be 256-byte aligned
    assert lib.qlin_gemm_fp8(A16, A16, A16, A16, 64, 512, 16384, A16, 0, C.c_void_p(0x100010),
                             need, None) == q.ERR_ALIGN
    assert lib.qlin_workspace_bytes(q.OP_GEMM_FP8, 0, 8192, 2048) == 0
    assert lib.qlin_workspace_bytes(99, 4, 512, 256) == 0
    lin = lib.qlin_workspace_bytes(q.OP_LINEAR_FP8, 4, 512, 256)
    assert lin >= 4 * 256 + 16
    assert lib.qlin_moe_workspace_bytes(64, 2048, 768, 128, 8) > 64 * 8 * (768 * 5 + 2048 * 4)


def test_repack_quant_validation(q):
    lib = q.lib()
    assert lib.qlin_repack_q4_0(A16, 16, 48, A16, A16, None, None) == q.ERR_SHAPE
    assert lib.qlin_repack_q4_0(None, 16, 64, A16, A16, None, None) == q.ERR_ARG
    assert lib.qlin_repack_q4_0(A_ODD, 16, 64, A16, A16, None, None) == q.ERR_ALIGN
    assert lib.qlin_repack_fp8(A16, A16, 16, 64, 2, A16, A16, None) == q.ERR_ARG  # int8 is not fp8
    assert lib.qlin_repack_int8(A16, A16, 16, 40, A16, A16, None) == q.ERR_SHAPE
    assert lib.qlin_fp8_fnuz_to_ocp(A16, A16, 4, 24, A16, A16, None, None) == q.ERR_SHAPE
    assert lib.qlin_quant_act(A16, 4, 64, 32, 0, A16, A16, None) == q.ERR_SHAPE  # lda < K
    assert lib.qlin_quant_act(A16, 4, 64, 68, 0, A16, A16, None) == q.ERR_ALIGN  # lda % 8
    assert lib.qlin_quant_act(A16, 4, 64, 64, 9, A16, A16, None) == q.ERR_ARG
    assert lib.qlin_quant_act(A16, 0, 64, 64, 0, A16, A16, None) == q.OK
    assert lib.qlin_fp8_encode_f32(A16, 16, 2, A16, None) == q.ERR_ARG
    assert lib.qlin_quant_weight(A16, 16, 40, 0, A16, A16, None) == q.ERR_SHAPE  # K % 16
    assert lib.qlin_quant_weight(A16, 16, 64, 9, A16, A16, None) == q.ERR_ARG
    assert lib.qlin_quant_weight(A_ODD, 16, 64, 1, A16, A16, None) == q.ERR_ALIGN
    assert lib.qlin_quant_weight(A16, 0, 64, 0, A16, A16, None) == q.OK
    assert lib.qlin_embed_q4(A16, 4, A16, A16, 100, 48, A16, None) == q.ERR_SHAPE  # D % 32
    assert lib.qlin_embed_q4(A16, 4, A16, A16, 0, 64, A16, None) == q.ERR_SHAPE
    assert lib.qlin_embed_q4(None, 4, A16, A16, 100, 64, A16, None) == q.ERR_ARG
    assert lib.qlin_embed_q4(A16, 4, A_ODD, A16, 100, 64, A16, None) == q.ERR_ALIGN
    assert lib.qlin_embed_q4(A16, 0, A16, A16, 100, 64, A16, None) == q.OK
    assert lib.qlin_embed_q4(A16, 1 << 20, A16, A16, 100, 1 << 14, A16, None) == q.ERR_SHAPE


def test_moe_validation(q):
    lib = q.lib()
    args = [A16] * 6  # ids, weights, w13, s13, w2, s2
    ws = C.c_void_p(0x100000)
    need = lib.qlin_moe_workspace_bytes(8, 256, 128, 8, 2)
    assert lib.qlin_moe_fp8(A16, 8, 250, 128, 8, 2, *args, A16, ws, need, None) == q.ERR_SHAPE
    assert lib.qlin_moe_fp8(A16, 8, 256, 128, 8, 9, *args, A16, ws, need, None) == q.ERR_SHAPE
    assert lib.qlin_moe_fp8(A16, 8, 256, 128, 8, 2, *args, A16, ws, need - 1, None) == q.ERR_WORKSPACE
    assert lib.qlin_moe_fp8(A16, 0, 256, 128, 8, 2, *args, A16, ws, 0, None) == q.OK
    offs = (C.c_size_t * 6)()
    assert lib.qlin_moe_workspace_layout(8, 256, 128, 8, 2, offs) == q.OK
    assert list(offs) == sorted(offs) and all(o % 256 == 0 for o in offs)


def test_moe_swiglu_oai_validation(q):
    lib = q.lib()
    args = [A16] * 6  # ids, weights, w13, s13, w2, s2
    ws = C.c_void_p(0x100000)
    need = lib.qlin_moe_workspace_bytes(8, 256, 128, 8, 2)
    f = lib.qlin_moe_fp8_swiglu_oai
    ok = (1.702, 1.0, 7.0)
    for bad in ((float("nan"), 1.0, 7.0), (1.702, float("inf"), 7.0), (1.702, 1.0, 0.0),
                (1.702, 1.0, -1.0), (1.702, 1.0, float("nan"))):
        assert f(A16, 8, 256, 128, 8, 2, *args, *bad, A16, ws, need, None) == q.ERR_ARG
    assert f(A16, 8, 250, 128, 8, 2, *args, *ok, A16, ws, need, None) == q.ERR_SHAPE
    assert f(A16, 8, 256, 128, 8, 2, *args, *ok, A16, ws, need - 1, None) == q.ERR_WORKSPACE
    assert f(A16, 8, 256, 128, 8, 2, *args, *ok, A16, C.c_void_p(0x100010), need, None) == q.ERR_ALIGN
    assert f(A16, 0, 256, 128, 8, 2, *args, 1.702, 1.0, float("inf"), A16, ws, 0, None) == q.OK


def test_moe_w4a16_validation(q):
    lib = q.lib()
    args = [A16] * 6  # ids, weights, codes13, steps13, codes2, steps2
    ws = C.c_void_p(0x100000)
    need = lib.qlin_moe_w4a16_workspace_bytes(8, 256, 128, 8, 2)
    assert need >= 16 * 128 * 2 + 16 * 256 * 4
    assert lib.qlin_moe_w4a16(A16, 8, 250, 128, 8, 2, *args, A16, ws, need, None) == q.ERR_SHAPE
    assert lib.qlin_moe_w4a16(A16, 8, 256, 100, 8, 2, *args, A16, ws, need, None) == q.ERR_SHAPE
    assert lib.qlin_moe_w4a16(A16, 8, 256, 128, 8, 9, *args, A16, ws, need, None) == q.ERR_SHAPE
    assert lib.qlin_moe_w4a16(A16, 8, 256, 128, 8, 2, *args, A16, ws, need - 1, None) == q.ERR_WORKSPACE
    assert lib.qlin_moe_w4a16(A16, 8, 256, 128, 8, 2, *args, A16, C.c_void_p(0x100010), need,
                              None) == q.ERR_ALIGN
    assert lib.qlin_moe_w4a16(A16, 0, 256, 128, 8, 2, *args, A16, ws, 0, None) == q.OK
    assert lib.qlin_moe_w4a16(None, 8, 256, 128, 8, 2, *args, A16, ws, need, None) == q.ERR_ARG
    offs = (C.c_size_t * 2)()
    assert lib.qlin_moe_w4a16_workspace_layout(8, 256, 128, 8, 2, offs) == q.OK
    assert list(offs) == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lib.qlin_moe_w4a16_workspace_layout(8, 256, 128, 8, 2, None) == q.ERR_ARG


def test_binding_rejects_host_tensors(q):
    import torch

    with pytest.raises(ValueError):
        q.quant_act(torch.zeros(4, 64, dtype=torch.bfloat16))
