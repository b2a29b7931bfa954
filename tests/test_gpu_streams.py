"""Workspaces of the Python binding under concurrency and graph capture.

The C ABI requires that calls sharing a workspace be ordered on one stream
(split-K arrival counters and partial sums, MoE stage data). The binding
keeps one workspace per (device, stream) and never frees a workspace a call
has outgrown, because a captured graph may still hold its address.
"""

import numpy as np
import pytest
import torch

import gen
from helpers import dev, host

pytestmark = pytest.mark.gpu

OCP = 0


@pytest.fixture(scope="module")
def q():
    import quantized_linear_layers_amd as qlin

    assert torch.cuda.is_available()
    return qlin


def _ops(oracle):
    d = gen.linear_config(2, n=4096, k=2048, m=64)
    p, s, _ = oracle.repack_q4_0(d["w_bf16"])
    wq, ws = oracle.repack_fp8(p, s, d["K"], OCP)
    aq, sa = oracle.quant_act(d["a"], OCP)
    dm = gen.moe_config(E=16, H=512, I=256, T=48, topk=4, seed=21)
    m13 = [oracle.repack_q4_0(dm["w13_bf16"][e]) for e in range(dm["E"])]
    m2 = [oracle.repack_q4_0(dm["w2_bf16"][e]) for e in range(dm["E"])]
    moe = [np.stack([m[0] for m in m13]), np.stack([m[1] for m in m13]),
           np.stack([m[0] for m in m2]), np.stack([m[1] for m in m2])]
    return dict(a=dev(d["a"]), p=dev(p), s=dev(s), wq=dev(wq), ws=dev(ws), aq=dev(aq), sa=dev(sa),
                x=dev(dm["x"]), ids=dev(dm["ids"]), pr=dev(dm["probs"]), moe=[dev(t) for t in moe])


def test_two_streams_match_serial(q, oracle):
    """Split-K FP8 GEMMs and linears (1024 columns: 32 column tiles, K split
    4 ways), W4A16 GEMMs and W4A16 MoE blocks issued on two streams at once
    equal the serial results bit for bit, five rounds in a row."""
    o = _ops(oracle)
    w1k, s1k = o["wq"][:1024], o["ws"][:1024]

    def work_a():
        return [q.gemm_w4a16(o["a"], o["p"], o["s"]), q.linear_fp8(o["a"][:8], w1k, s1k),
                q.gemm_fp8(o["aq"][:2], o["sa"][:2], w1k, s1k),
                q.moe_w4a16(o["x"], o["ids"], o["pr"], *o["moe"])]

    def work_b():
        return [q.gemm_w4a16(o["a"][:8], o["p"], o["s"]), q.moe_w4a16(o["x"][:20], o["ids"][:20],
                                                                       o["pr"][:20], *o["moe"]),
                q.gemm_fp8(o["aq"][:5], o["sa"][:5], w1k, s1k), q.linear_fp8(o["a"][:3], w1k, s1k)]

    ref_a = [host(t) for t in work_a()]
    ref_b = [host(t) for t in work_b()]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rnd in range(5):
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        outs_a, outs_b = [], []
        for _ in range(4):
            with torch.cuda.stream(s1):
                outs_a.append(work_a())
            with torch.cuda.stream(s2):
                outs_b.append(work_b())
        torch.cuda.synchronize()
        for ya in outs_a:
            for i, t in enumerate(ya):
                assert np.array_equal(host(t), ref_a[i]), f"round {rnd}, stream 1, output {i}"
        for yb in outs_b:
            for i, t in enumerate(yb):
                assert np.array_equal(host(t), ref_b[i]), f"round {rnd}, stream 2, output {i}"


def test_graph_replay_after_workspace_grew(q, oracle):
    """A graph captured with a split-K GEMM on stream s replays correctly
    after an eager call on s needed a larger workspace (the old one stays
    allocated: memory handed out afterwards is not overwritten by the
    replay's partial sums)."""
    o = _ops(oracle)
    small_w = (o["wq"][:1024], o["ws"][:1024])  # 32 column tiles: K split 4 ways
    wide = gen.linear_config(2, n=16384, k=2048, m=64)
    wp, wst, _ = oracle.repack_q4_0(wide["w_bf16"])
    wp, wst = dev(wp), dev(wst)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y = torch.empty(8, 1024, dtype=torch.bfloat16, device="cuda")
        q.gemm_fp8(o["aq"][:8], o["sa"][:8], *small_w, out=y)
        torch.cuda.synchronize()
        ref = host(y)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            q.gemm_fp8(o["aq"][:8], o["sa"][:8], *small_w, out=y)
        need_small = q.workspace_bytes(q.OP_GEMM_FP8, 8, 1024, 2048)
        need_big = q.workspace_bytes(q.OP_GEMM_W4A16, 64, 16384, 2048)
        assert need_small > 0 and need_big > max(need_small, 1 << 20)
        big = q.gemm_w4a16(o["a"], wp, wst)  # outgrows the workspace of s
        torch.cuda.synchronize()
        # fresh allocations that would reuse a freed workspace
        fill = [torch.full((1 << 20,), 77, dtype=torch.uint8, device="cuda") for _ in range(8)]
        for rep in range(3):
            y.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(host(y), ref), f"replay {rep}"
            for t in fill:
                assert bool((t == 77).all()), "replay wrote into memory allocated after the growth"
        assert host(big).shape == (64, 16384)
