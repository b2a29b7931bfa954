"""Pins for the oracle's FP8 mixture-of-experts block (CPU only).

The block (dev.to sizes article, "Step 1 -- Build the Larger Repacks": the
fused expert banks split per expert into gate/up/down, the router stays
outside; vLLM PR #45854 report: per-token activation and per-output-channel
weight scales for the fp8 MoE) reduces to per-expert FP8 linears. A
brute-force fp64 numpy version at a tiny size checks each stage; the
requantisation between the two GEMMs is checked bit-exact against a
brute-force quantiser on the oracle's own intermediate.

The W4A16 block (sizes article, "The 4-Bit Builds Stay Slow": the 4-bit MoE
runs vLLM's WNA16 expert path) is pinned the same way on the generator's
materialised bf16 banks, plus its reduction to the W4A16 GEMM oracle at one
expert per token and its linearity in the routing probabilities.
"""

import numpy as np
import pytest

import gen

OCP = 0


def _small_block(oracle, E=4, H=64, I=32, T=5, topk=2, seed=21):
    d = gen.moe_config(E=E, H=H, I=I, T=T, topk=topk, seed=seed)
    w13 = np.empty((E, 2 * I, H), np.uint8); s13 = np.empty((E, 2 * I), np.float32)
    w2 = np.empty((E, H, I), np.uint8); s2 = np.empty((E, H), np.float32)
    for e in range(E):
        p, st, amb = oracle.repack_q4_0(d["w13_bf16"][e]); assert amb == 0
        w13[e], s13[e] = oracle.repack_fp8(p, st, H, OCP)
        p, st, amb = oracle.repack_q4_0(d["w2_bf16"][e]); assert amb == 0
        w2[e], s2[e] = oracle.repack_fp8(p, st, I, OCP)
    d.update(w13=w13, s13=s13, w2=w2, s2=s2)
    return d


def _close(x, ref, rel=1e-5):
    rms = np.sqrt(np.mean(ref.astype(np.float64) ** 2))
    return np.all(np.abs(x - ref) <= rel * np.abs(ref) + 1e-5 * rms)


def test_moe_stages_bruteforce(oracle):
    d = _small_block(oracle)
    t = oracle.fp8_decode_table(OCP)
    out = oracle.moe_fp8(d["x"], d["ids"], d["probs"], d["w13"], d["s13"], d["w2"], d["s2"])
    xq, sx = oracle.quant_act(d["x"], OCP)
    T, topk, I = d["T"], d["topk"], d["I"]
    # stage 1: gate_up + SiLU(g) * u
    act = np.empty((T * topk, I))
    for r in range(T * topk):
        tok, e = r // topk, d["ids"].ravel()[r]
        h = (t[xq[tok]] @ t[d["w13"][e]].T) * float(sx[tok]) * d["s13"][e].astype(np.float64)
        g, u = h[:I], h[I:]
        act[r] = g / (1.0 + np.exp(-g)) * u
    assert _close(out["act32"], act)
    # stage 2: requant of the oracle's own fp32 intermediate, brute force
    top = t[:0x7F]
    for r in range(T * topk):
        row = out["act32"][r]
        s = np.float32(np.abs(row).max()) / np.float32(448.0)
        assert out["sa"][r] == s
        v = row / s
        dd = np.abs(top[None, :] - np.abs(v.astype(np.float64))[:, None])
        for i in range(I):
            best = np.flatnonzero(dd[i] == dd[i].min())
            c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
            neg = np.signbit(v[i])
            want = (0x80 if neg else 0) if c == 0 else (c | (0x80 if neg else 0))
            assert out["aq"][r, i] == want
    # stage 3: down + combine in slot order, given the oracle's aq / sa
    y = np.zeros((T, d["H"]))
    for r in range(T * topk):
        tok, e = r // topk, d["ids"].ravel()[r]
        dr = (t[out["aq"][r]] @ t[d["w2"][e]].T) * float(out["sa"][r]) * d["s2"][e].astype(np.float64)
        assert _close(out["d32"][r], dr)
        y[tok] += float(d["probs"].ravel()[r]) * dr
    assert _close(out["y32"], y, rel=1e-4)
    assert np.array_equal(out["y16"], oracle.bf16_nearest_array(out["y32"]))


def test_moe_stage_functions_compose(oracle):
    d = _small_block(oracle, seed=5)
    out = oracle.moe_fp8(d["x"], d["ids"], d["probs"], d["w13"], d["s13"], d["w2"], d["s2"])
    xq, sx = oracle.quant_act(d["x"], OCP)
    act = oracle.moe_gate_up(xq, sx, d["ids"], d["w13"], d["s13"])
    assert np.array_equal(act, out["act32"])
    aq, sa = oracle.quant_rows_f32(act, OCP)
    assert np.array_equal(aq, out["aq"]) and np.array_equal(sa, out["sa"])
    d32, y32, y16 = oracle.moe_down(aq, sa, d["ids"], d["probs"], d["w2"], d["s2"])
    assert np.array_equal(y32, out["y32"]) and np.array_equal(y16, out["y16"])


def test_moe_single_expert_is_dense_linear(oracle):
    """topk=1 with probability 1: the down projection of a token equals the
    dense FP8 GEMM of its requantised intermediate through that expert."""
    d = _small_block(oracle, T=3, topk=1, seed=9)
    probs = np.ones_like(d["probs"])
    out = oracle.moe_fp8(d["x"], d["ids"], probs, d["w13"], d["s13"], d["w2"], d["s2"])
    for tok in range(3):
        e = d["ids"][tok, 0]
        y32, _ = oracle.gemm_fp8(out["aq"][tok:tok + 1], out["sa"][tok:tok + 1], d["w2"][e], d["s2"][e])
        assert np.array_equal(out["y32"][tok], y32[0])


# ---------------------------------------------------------------- W4A16 block
def _w4_block(oracle, E=4, H=64, I=32, T=5, topk=2, seed=31):
    """Packed codes and bf16 steps of every expert, recovered from the
    generator's bf16 expert banks by the (separately pinned) q4_0 repack."""
    d = gen.moe_config(E=E, H=H, I=I, T=T, topk=topk, seed=seed)
    p13 = np.empty((E, 2 * I, H // 2), np.uint8); st13 = np.empty((E, 2 * I, H // 32), np.uint16)
    p2 = np.empty((E, H, I // 2), np.uint8); st2 = np.empty((E, H, I // 32), np.uint16)
    for e in range(E):
        p13[e], st13[e], amb = oracle.repack_q4_0(d["w13_bf16"][e]); assert amb == 0
        p2[e], st2[e], amb = oracle.repack_q4_0(d["w2_bf16"][e]); assert amb == 0
    d.update(p13=p13, st13=st13, p2=p2, st2=st2)
    return d


def test_moe_w4a16_stages_bruteforce(oracle):
    """fp64 numpy on the generator's materialised bf16 banks (bf16(c*step)
    bit for bit under the bf16-step recipe): gate rows first, SiLU(g)*u
    rounded once to bf16, down, probability-weighted sum in slot order."""
    d = _w4_block(oracle)
    out = oracle.moe_w4a16(d["x"], d["ids"], d["probs"], d["p13"], d["st13"], d["p2"], d["st2"])
    T, topk, I, H = d["T"], d["topk"], d["I"], d["H"]
    x = gen.bf16_bits_to_f32(d["x"]).astype(np.float64)
    w13 = gen.bf16_bits_to_f32(d["w13_bf16"]).astype(np.float64)
    w2 = gen.bf16_bits_to_f32(d["w2_bf16"]).astype(np.float64)
    act16 = gen.bf16_bits_to_f32(out["act16"]).astype(np.float64)
    y = np.zeros((T, H))
    for r in range(T * topk):
        tok, e = r // topk, d["ids"].ravel()[r]
        h = x[tok] @ w13[e].T
        g, u = h[:I], h[I:]
        act = g / (1.0 + np.exp(-g)) * u
        # one bf16 rounding (half an ulp) plus fp32 summation error
        assert np.all(np.abs(act16[r] - act) <= 2.0 ** -8 * np.abs(act) + 1e-5 * np.sqrt(np.mean(act ** 2)))
        dr = act16[r] @ w2[e].T
        assert _close(out["d32"][r], dr)
        y[tok] += float(d["probs"].ravel()[r]) * dr
    assert _close(out["y32"], y, rel=1e-4)
    assert np.array_equal(out["y16"], oracle.bf16_nearest_array(out["y32"]))


def test_moe_w4a16_single_expert_is_w4a16_linear(oracle):
    """topk=1 with probability 1: each token's output equals the W4A16 GEMM
    oracle on its bf16 intermediate through that expert's down bank."""
    d = _w4_block(oracle, T=3, topk=1, seed=13)
    probs = np.ones_like(d["probs"])
    out = oracle.moe_w4a16(d["x"], d["ids"], probs, d["p13"], d["st13"], d["p2"], d["st2"])
    for tok in range(3):
        e = d["ids"][tok, 0]
        y32, _ = oracle.gemm_w4a16(out["act16"][tok:tok + 1], d["p2"][e], d["st2"][e])
        assert np.array_equal(out["y32"][tok], y32[0])


def test_moe_w4a16_linear_in_probabilities(oracle):
    """Doubling every routing probability doubles the fp32 output exactly;
    zero probabilities give zero."""
    d = _w4_block(oracle, seed=17)
    a = oracle.moe_w4a16(d["x"], d["ids"], d["probs"], d["p13"], d["st13"], d["p2"], d["st2"])
    b = oracle.moe_w4a16(d["x"], d["ids"], 2 * d["probs"], d["p13"], d["st13"], d["p2"], d["st2"])
    z = oracle.moe_w4a16(d["x"], d["ids"], 0 * d["probs"], d["p13"], d["st13"], d["p2"], d["st2"])
    assert np.array_equal(b["y32"], 2 * a["y32"])
    assert np.array_equal(b["act16"], a["act16"])
    assert not np.any(z["y32"])
