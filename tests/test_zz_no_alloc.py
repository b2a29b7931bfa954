"""The allocation-free FP8 MoE entry point.

qlin_moe_fp8_noalloc runs the kernels of qlin_moe_fp8 with its stage
buffers in the library's static per-GPU array instead of a caller
workspace. Called through the C ABI it must equal qlin_moe_fp8 bit for bit,
on two calls in a row with the second smaller (the array keeps the first
call's contents), and refuse before any launch a call whose stage buffers
exceed the array.
"""

import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import quantized_linear_layers_amd as qlin

    assert torch.cuda.is_available()
    return qlin


def _block(q, E, H, I, T, topk, seed):
    """Seeded synthetic FP8 MoE operands: per-channel FP8 banks of N(0, 0.02)
    bf16 weights (the library's own quantiser), N(0, 1) activations, top-k
    routing of N(0, 1) logits."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    w13, s13 = q.quant_weight((torch.randn(E * 2 * I, H, device="cuda", generator=g) * 0.02)
                              .to(torch.bfloat16))
    w2, s2 = q.quant_weight((torch.randn(E * H, I, device="cuda", generator=g) * 0.02).to(torch.bfloat16))
    x = torch.randn(T, H, device="cuda", generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    ids, pr = gen.route_topk(rng.standard_normal((T, E), dtype=np.float32), topk)
    return (x, torch.from_numpy(ids).cuda(), torch.from_numpy(pr).cuda(), w13.view(E, 2 * I, H),
            s13.view(E, 2 * I), w2.view(E, H, I), s2.view(E, H))


def test_noalloc_equals_workspace_entry_point(q):
    E, H, I, topk = 128, 2048, 768, 8
    # the largest token count of the MoE workload first (about 50 MiB of
    # stage buffers), then a smaller block with other routing
    for T, seed in ((512, 31), (40, 32)):
        ops = _block(q, E, H, I, T, topk, seed)
        need = int(q.lib().qlin_moe_workspace_bytes(T, H, I, E, topk))
        assert need <= q.MOE_NOALLOC_MAX_BYTES
        y = q.moe_fp8_noalloc(*ops)
        ref = q.moe_fp8(*ops)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"T={T}"
    # repeated call on the same operands: same bits
    y2 = q.moe_fp8_noalloc(*ops)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), ref.view(torch.int16))


def test_noalloc_refuses_oversize_call(q):
    E, H, I, topk = 8, 2048, 768, 8
    T = 2048  # stage buffers of about 200 MiB
    assert int(q.lib().qlin_moe_workspace_bytes(T, H, I, E, topk)) > q.MOE_NOALLOC_MAX_BYTES
    x = torch.zeros(T, H, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(T, topk, dtype=torch.int32, device="cuda")
    pr = torch.zeros(T, topk, dtype=torch.float32, device="cuda")
    w13 = torch.zeros(E, 2 * I, H, dtype=torch.uint8, device="cuda")
    s13 = torch.zeros(E, 2 * I, dtype=torch.float32, device="cuda")
    w2 = torch.zeros(E, H, I, dtype=torch.uint8, device="cuda")
    s2 = torch.zeros(E, H, dtype=torch.float32, device="cuda")
    y = torch.full((T, H), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(q.QlinError) as ei:
        q.moe_fp8_noalloc(x, ids, pr, w13, s13, w2, s2, out=y)
    assert ei.value.status == q.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all()), "a refused call wrote its output"
