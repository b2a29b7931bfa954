"""GPU parity of the in-kernel int4 unpack, bit for bit.

The W4A16 GEMMs multiply bf16 activations by bf16(c * step), the weight
rounded once to bf16 ("Gemma 4 From E2B to 31B", "The 4-Bit Builds Stay
Slow": the kernel unpacks the weights to bf16 before each multiply). With a
one-hot activation row a = e_k the fp32 output is exactly that unpacked
weight: y[m, n] = 1.0 * bf16(c[n,k] * step[n,k/32]) plus exact zeros. So an
F32-output GEMM whose rows are one-hot reads the kernel's unpack back, and
it must equal the oracle's bf16(c * step) (its int4 table lookup) as a
value, for every weight.

The weights hold every finite bf16 step of magnitude below 2^117 (both
signs, zeros and subnormals included; the bound the W4A16 entry point
states), one per group of 32, and every group holds all 16 codes twice,
rotated by the group index so every lane position meets every code. Each
shape below selects one launch path of the decode (M <= 64) or prefill
kernels; the MoE blocks are read back through their stage results.
"""

import numpy as np
import pytest
import torch

import gen
from helpers import bf16_to_f32, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import quantized_linear_layers_amd as qlin

    assert torch.cuda.is_available()
    return qlin


def step_table() -> np.ndarray:
    """bf16 bit patterns of every finite step with |step| < 2^117: exponent
    fields 0..243 with every mantissa, both signs (62464 patterns)."""
    mags = np.arange(0, 244 * 128, dtype=np.uint16)
    return np.concatenate([mags, mags | np.uint16(0x8000)])


def table_weights(N: int, K: int, shift: int = 0):
    """Packed codes [N, K/2] and steps [N, K/32] (bf16 bits): group g (row-
    major over (row, group)) takes step table[(g + shift) % len] and codes
    c_j = ((j + g) % 16) - 8."""
    tab = step_table()
    G = N * K // 32
    g = np.arange(G)
    steps = tab[(g + shift) % tab.size].reshape(N, K // 32)
    j = np.arange(32)
    u = ((j[None, :] + g[:, None]) % 16).astype(np.uint8)  # offset-binary c + 8
    packed = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8).reshape(N, K // 2)
    return packed, steps


def reference(oracle, packed, steps):
    """The oracle's bf16(c * step) for every weight, [N, K] as fp32."""
    N = packed.shape[0]
    return bf16_to_f32(oracle.embed_q4(np.arange(N, dtype=np.int32), packed, steps))


def check_equal(got: np.ndarray, want: np.ndarray, what: str):
    bad = got != want  # values: +0 and -0 compare equal
    if bad.any():
        i = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} unpacked weights differ; first at "
                             f"{i.tolist()}: gpu {got[bad][:5].tolist()} oracle {want[bad][:5].tolist()}")


def windows(K: int, M: int):
    """Row offsets of one-hot windows of M rows that cover k = 0..K-1 (the
    last window is moved back inside K)."""
    offs = list(range(0, K - M + 1, M))
    if offs[-1] + M < K:
        offs.append(K - M)
    return offs


def run_decode(q, oracle, N, K, Ms, misalign=False, extra_m1=()):
    packed, steps = table_weights(N, K)
    ref = reference(oracle, packed, steps)
    eye = torch.eye(K, dtype=torch.bfloat16, device="cuda")
    pk = dev(packed)
    st = dev(steps)
    if misalign:  # step rows 2 bytes past an aligned address: per-unit step loads
        buf = torch.empty(st.numel() + 8, dtype=st.dtype, device="cuda")
        sv = buf[1:1 + st.numel()].view(st.shape)
        sv.copy_(st)
        assert sv.data_ptr() % 16 != 0
        st = sv
    for M in Ms:
        for off in windows(K, M):
            y = host(q.gemm_w4a16(eye[off:off + M], pk, st, out_dtype=torch.float32))
            check_equal(y, ref[:, off:off + M].T, f"N={N} K={K} M={M} rows {off}..{off + M - 1}")
    for k in extra_m1:
        y = host(q.gemm_w4a16(eye[k:k + 1], pk, st, out_dtype=torch.float32))
        check_equal(y, ref[:, k:k + 1].T, f"N={N} K={K} M=1 row {k}")


# ------------------------------------------------------------------ decode paths
# The launch rules at 256 CUs: with K % 256 == 0, M <= 16 on a layer of
# fewer than 16384 columns, and M = 17..64 on one of 6145..8192 columns, run
# the small-layer kernel (waves splitting K in 1, 2 or 4 parts; 1, 4, 8, 16,
# 32 or 64 staged rows). Otherwise the streaming core: one
# 16-row block (M <= 16) on a layer of at most 12224 columns splits K over
# the 4 waves of a workgroup (WK); wider layers give each wave its own
# columns; a layer of 24449..65536 columns runs 8-wave workgroups over the
# whole K range at every M, a wider one two column blocks per wave in 8-wave
# workgroups at M = 33..64. K % 256 == 0 with 16-byte aligned step rows
# loads the steps in bulk, otherwise per unit.
DECODE_CASES = [
    # id, N, K, Ms, misalign, M=1 rows
    ("small_layer_one_unit", 7808, 256, (16,), False, (0, 1, 131, 255)),
    ("small_layer_k_parts", 1952, 1024, (1, 3, 4, 5, 8, 12, 16), False, ()),
    ("small_layer_unaligned_steps", 7808, 256, (16,), True, (3,)),
    ("small_layer_32_64_rows", 8192, 512, (32, 48, 64), False, (0, 300)),
    ("small_layer_64_rows_one_part", 8160, 256, (17, 64), False, ()),
    ("wk_per_unit_k288", 6944, 288, (16,), False, (0, 287)),
    ("wide_mb1_bulk", 16384, 256, (16,), False, (0, 200)),
    ("wide_mb1_per_unit", 12288, 288, (16,), False, ()),
    ("mb2_mb3_mb4_bulk", 4096, 512, (32, 48, 64), False, ()),
    ("mb2_mb4_per_unit", 4096, 288, (32, 64), False, ()),
    ("wide_8_waves_bulk", 24576, 256, (1, 17, 48, 64), False, (0, 255)),
    ("wide_8_waves_per_unit", 24576, 288, (16, 32, 64), False, ()),
    ("wide_8_waves_unaligned_steps", 24576, 512, (8, 64), True, ()),
    ("two_blocks_8_waves_bulk", 65664, 256, (48, 64), False, ()),
    ("two_blocks_8_waves_per_unit", 65664, 288, (64,), False, ()),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_unpack_one_hot(q, oracle, case):
    _, N, K, Ms, mis, m1 = case
    run_decode(q, oracle, N, K, Ms, misalign=mis, extra_m1=m1)


# ------------------------------------------------------------------ prefill paths
@pytest.mark.parametrize("case", [
    # persistent 256x256 kernel (>= 128 tiles, K % 64 == 0, 4-byte aligned steps)
    ("persistent", 512, 16384, 512, False),
    # 128x128 tiled kernel (fewer tiles)
    ("tiled", 512, 4096, 512, False),
    # tile count of the persistent kernel, ragged M and N, steps only 2-byte
    # aligned: the tiled kernel serves it
    ("persistent_shape_unaligned_steps", 2000, 4112, 384, True),
    ("persistent_ragged", 2000, 4112, 384, False),
], ids=lambda c: c[0])
def test_prefill_unpack_one_hot(q, oracle, case):
    _, M, N, K, mis = case
    packed, steps = table_weights(N, K, shift=7)
    ref = reference(oracle, packed, steps)
    ks = np.arange(M) % K
    a = torch.zeros(M, K, dtype=torch.bfloat16, device="cuda")
    a[torch.arange(M, device="cuda"), torch.from_numpy(ks).cuda()] = 1.0
    st = dev(steps)
    if mis:
        buf = torch.empty(st.numel() + 8, dtype=st.dtype, device="cuda")
        sv = buf[1:1 + st.numel()].view(st.shape)
        sv.copy_(st)
        assert sv.data_ptr() % 4 != 0
        st = sv
    y = host(q.gemm_w4a16(a, dev(packed), st, out_dtype=torch.float32))
    check_equal(y, ref[:, ks].T, f"prefill M={M} N={N} K={K}")


# ------------------------------------------------------------------ MoE W4A16
def _const_rows(rows: int, K: int, code: int, step: float):
    u = np.uint8(code + 8)
    packed = np.full((rows, K // 2), u | (u << 4), np.uint8)
    steps = np.full((rows, K // 32), gen.to_bf16_bits(np.float32([step]))[0], np.uint16)
    return packed, steps


def _moe_call(q, x, E, codes13, steps13, codes2, steps2, misalign):
    T = x.shape[0]
    ids = torch.zeros(T, 1, dtype=torch.int32, device="cuda")
    pr = torch.ones(T, 1, dtype=torch.float32, device="cuda")
    args = [dev(codes13), dev(steps13), dev(codes2), dev(steps2)]
    if misalign:
        for i in (1, 3):
            s = args[i]
            buf = torch.empty(s.numel() + 8, dtype=s.dtype, device="cuda")
            sv = buf[1:1 + s.numel()].view(s.shape)
            sv.copy_(s)
            args[i] = sv
    _, stages = q.moe_w4a16(x, ids, pr, *args, return_stages=True)
    return host(stages["act"]), stages["d"].cpu().numpy()


@pytest.mark.parametrize("misalign", [False, True], ids=["bulk_steps", "per_unit_steps"])
def test_moe_gate_up_unpack_one_hot(q, oracle, misalign):
    """gate_up: token t is e_t, every gate weight is 4 * 8 = 32 and the up
    rows hold the table, so g = 32, SiLU(32) = 32 exactly (exp(-32) vanishes
    beside 1 in fp32) and act[t, i] = bf16(32 * u) = 32 * bf16(c * step) of
    up row i at column t (a power-of-two scaling, exact). T = 2048 rows of
    one expert run 48-row blocks and a 32-row tail; T = 16 one 16-row block."""
    H, I = 2048, 1024
    up_p, up_s = table_weights(I, H, shift=3)
    ref = reference(oracle, up_p, up_s)  # [I, H]
    g_p, g_s = _const_rows(I, H, 4, 8.0)
    codes13 = np.concatenate([g_p, up_p])[None]
    steps13 = np.concatenate([g_s, up_s])[None]
    codes2, steps2 = _const_rows(H, I, 0, 1.0)
    eye = torch.eye(H, dtype=torch.bfloat16, device="cuda")
    for T in (2048, 16):
        act, _ = _moe_call(q, eye[:T].contiguous(), 1, codes13, steps13, codes2[None], steps2[None],
                           misalign)
        check_equal(bf16_to_f32(act), 32.0 * ref[:, :T].T, f"MoE gate_up T={T}")


@pytest.mark.parametrize("misalign", [False, True], ids=["bulk_steps", "per_unit_steps"])
def test_moe_down_unpack_one_hot(q, oracle, misalign):
    """down: token t is e_t, gate weights 32 and up weight 2^-5 exactly where
    up row i meets column t = i (else 0), so act = e_t; the down rows hold the
    table and d[t, h] = bf16(c * step) of down row h at column t."""
    H, I = 2048, 1024
    dn_p, dn_s = table_weights(H, I, shift=11)
    ref = reference(oracle, dn_p, dn_s)  # [H, I]
    g_p, g_s = _const_rows(I, H, 4, 8.0)
    k = np.arange(H)
    u = np.where(k[None, :] == np.arange(I)[:, None], 9, 8).astype(np.uint8)  # c = 1 on the diagonal
    up_p = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    up_s = np.full((I, H // 32), gen.to_bf16_bits(np.float32([2.0 ** -5]))[0], np.uint16)
    codes13 = np.concatenate([g_p, up_p])[None]
    steps13 = np.concatenate([g_s, up_s])[None]
    eye = torch.eye(H, dtype=torch.bfloat16, device="cuda")
    T = I
    act, d = _moe_call(q, eye[:T].contiguous(), 1, codes13, steps13, dn_p[None], dn_s[None], misalign)
    assert np.array_equal(bf16_to_f32(act), np.eye(I, dtype=np.float32)), "act is not one-hot"
    check_equal(d, ref[:, :T].T, "MoE down")
