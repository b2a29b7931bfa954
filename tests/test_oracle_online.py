"""Pins for the oracle's online per-channel FP8 of bf16 weights and the
SwiGLU-OAI MoE activation (CPU only).

vLLM PR #45854 report (sections on the motivation and the implementation
breakdown): fp8_per_channel quantises bf16, non-QAT weights per output
channel at load, with per-token activations, and the fp8 MoE config gains
gemm1_alpha / gemm1_beta (1.702 / 1.0 for MiniMax-M3) and a clamp limit for
the SwiGLU-OAI activation. The quantiser is checked by brute force over the
decoded code table; the activation by identities of x*sigmoid(a*x) that
hold for any alpha, its value where the sigmoid is exactly 3/4, its zero at
up = -beta, the clamp rules, and its reduction to SiLU(g)*u.
"""

import math

import numpy as np
import pytest

import gen

OCP, FNUZ, INT8 = 0, 1, 2
ALPHA, BETA = 1.702, 1.0


def _nearest_codes(v, table, fmax_code_limit):
    """Brute force: nearest finite code of each |v| among codes 0..limit-1
    of the decoded table, ties to the even code; sign bit from v."""
    top = table[:fmax_code_limit].astype(np.float64)
    out = np.empty(v.shape, np.uint8)
    for i, x in enumerate(v.ravel()):
        d = np.abs(top - abs(float(x)))
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        out.ravel()[i] = c
    return out


@pytest.mark.parametrize("fmt", [OCP, FNUZ])
def test_quant_weight_fp8_bruteforce(oracle, fmt):
    rng = np.random.default_rng(40 + fmt)
    w = gen.dense_bf16(rng, 12, 96)
    q, s = oracle.quant_weight(w, fmt)
    wf = gen.bf16_bits_to_f32(w)
    fmax = np.float32(448.0 if fmt == OCP else 240.0)
    t = oracle.fp8_decode_table(fmt)
    for n in range(w.shape[0]):
        amax = np.float32(np.abs(wf[n]).max())
        assert s[n] == amax / fmax
        v = wf[n] / s[n]
        mag = _nearest_codes(v, t, 0x7F if fmt == OCP else 0x80)
        neg = np.signbit(v)
        if fmt == OCP:
            want = np.where(mag == 0, np.where(neg, 0x80, 0), mag | np.where(neg, 0x80, 0))
        else:  # FNUZ has no negative zero: 0x80 is its NaN
            want = np.where(mag == 0, 0, mag | np.where(neg, 0x80, 0))
        assert np.array_equal(q[n], want.astype(np.uint8))
        # the channel's largest weight lands on the format's largest code
        k = int(np.argmax(np.abs(wf[n])))
        assert t[q[n, k]] == (fmax if wf[n, k] > 0 else -fmax)


def test_quant_weight_int8_bruteforce(oracle):
    rng = np.random.default_rng(43)
    w = gen.dense_bf16(rng, 12, 64)
    q, s = oracle.quant_weight(w, INT8)
    wf = gen.bf16_bits_to_f32(w)
    for n in range(w.shape[0]):
        assert s[n] == np.float32(np.abs(wf[n]).max()) / np.float32(127.0)
        v = (wf[n] / s[n]).astype(np.float64)
        want = np.clip(np.round(v), -127, 127)  # numpy rounds half to even
        assert np.array_equal(q[n].astype(np.int64), want.astype(np.int64))


def test_quant_weight_zero_channel(oracle):
    w = gen.dense_bf16(np.random.default_rng(44), 4, 64)
    w[2] = 0
    q, s = oracle.quant_weight(w, OCP)
    assert s[2] == 0 and not q[2].any() and np.all(s[[0, 1, 3]] > 0)


# ------------------------------------------------------------ SwiGLU-OAI
def test_swiglu_oai_odd_part_is_identity(oracle):
    """x*sigmoid(a x) - (-x)*sigmoid(-a x) = x for every a, since
    sigmoid(z) + sigmoid(-z) = 1: act(g,u) - act(-g,u) = g*(u+beta)."""
    rng = np.random.default_rng(1)
    limit = 7.0
    g = rng.uniform(-limit, limit, 4000).astype(np.float32)
    u = rng.uniform(-limit, limit, 4000).astype(np.float32)
    for alpha in (ALPHA, 0.5, 3.0):
        a = oracle.swiglu_oai(g, u, alpha, BETA, limit).astype(np.float64)
        b = oracle.swiglu_oai(-g, u, alpha, BETA, limit).astype(np.float64)
        want = g.astype(np.float64) * (u.astype(np.float64) + BETA)
        scale = np.maximum(np.abs(want), np.maximum(np.abs(a), np.abs(b)))
        assert np.all(np.abs((a - b) - want) <= 4e-6 * scale + 1e-30)


def test_swiglu_oai_sigmoid_three_quarters(oracle):
    """At alpha*g = ln 3 the sigmoid is exactly 3/4: act = 0.75 g (u+beta)."""
    g0 = math.log(3.0) / ALPHA
    u = np.float32([-3.0, -0.25, 0.0, 0.5, 2.0, 6.5])
    g = np.full_like(u, g0)
    a = oracle.swiglu_oai(g, u, ALPHA, BETA, 7.0).astype(np.float64)
    want = 0.75 * np.float64(np.float32(g0)) * (u.astype(np.float64) + BETA)
    assert np.all(np.abs(a - want) <= 2e-6 * np.abs(want))


def test_swiglu_oai_zero_at_minus_beta(oracle):
    g = np.float32([-5.0, -1.0, 0.3, 2.0, 6.9, 40.0])
    u = np.full_like(g, -BETA)
    assert not np.any(oracle.swiglu_oai(g, u, ALPHA, BETA, 7.0))


def test_swiglu_oai_clamps(oracle):
    """The gate is clamped from above only, the up value on both sides."""
    rng = np.random.default_rng(2)
    limit = 2.5
    g = rng.uniform(-6, 6, 2000).astype(np.float32)
    u = rng.uniform(-6, 6, 2000).astype(np.float32)
    a = oracle.swiglu_oai(g, u, ALPHA, BETA, limit)
    gc = np.minimum(g, np.float32(limit))
    uc = np.clip(u, np.float32(-limit), np.float32(limit))
    assert np.array_equal(a, oracle.swiglu_oai(gc, uc, ALPHA, BETA, np.inf))
    # a gate below -limit is not clamped: it differs from the gate at -limit
    lo = g < -limit
    assert lo.sum() > 100
    at = oracle.swiglu_oai(np.full(lo.sum(), -limit, np.float32), uc[lo], ALPHA, BETA, np.inf)
    assert np.all(a[lo] != at)
    # above the limit the result no longer depends on the gate
    hi = g > limit
    assert np.array_equal(a[hi], oracle.swiglu_oai(np.full(hi.sum(), limit, np.float32), uc[hi],
                                                   ALPHA, BETA, np.inf))


# ------------------------------------------------------- MoE with SwiGLU-OAI
def _online_block(oracle, E=4, H=64, I=32, T=5, topk=2, seed=51):
    """bf16 (non-QAT) banks quantised per channel on line."""
    d = gen.moe_bf16_config(E=E, H=H, I=I, T=T, topk=topk, seed=seed)
    w13, s13 = oracle.quant_weight(d["w13_bf16"].reshape(E * 2 * I, H), OCP)
    w2, s2 = oracle.quant_weight(d["w2_bf16"].reshape(E * H, I), OCP)
    d.update(w13=w13.reshape(E, 2 * I, H), s13=s13.reshape(E, 2 * I),
             w2=w2.reshape(E, H, I), s2=s2.reshape(E, H))
    return d


def test_moe_oai_reduces_to_silu(oracle):
    """alpha 1, beta 0, no clamp: the SwiGLU-OAI block is the SiLU block bit
    for bit."""
    d = _online_block(oracle)
    a = oracle.moe_fp8(d["x"], d["ids"], d["probs"], d["w13"], d["s13"], d["w2"], d["s2"])
    b = oracle.moe_fp8(d["x"], d["ids"], d["probs"], d["w13"], d["s13"], d["w2"], d["s2"],
                       act=(1.0, 0.0, np.inf))
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_moe_oai_gate_up_bruteforce(oracle):
    """fp64 numpy gate_up on the decoded per-channel FP8 banks with the
    SwiGLU-OAI activation (at H = 64 the gate and up values are ~0.2, so a
    limit of 0.2 clamps often)."""
    d = _online_block(oracle, seed=52)
    limit = 0.2
    out = oracle.moe_fp8(d["x"], d["ids"], d["probs"], d["w13"], d["s13"], d["w2"], d["s2"],
                         act=(ALPHA, BETA, limit))
    t = oracle.fp8_decode_table(OCP)
    xq, sx = oracle.quant_act(d["x"], OCP)
    T, topk, I = d["T"], d["topk"], d["I"]
    n_clamped = 0
    for r in range(T * topk):
        tok, e = r // topk, d["ids"].ravel()[r]
        h = (t[xq[tok]] @ t[d["w13"][e]].T) * float(sx[tok]) * d["s13"][e].astype(np.float64)
        g, u = h[:I], h[I:]
        n_clamped += int(np.sum(g > limit) + np.sum(np.abs(u) > limit))
        g = np.minimum(g, limit)
        u = np.clip(u, -limit, limit)
        act = g / (1.0 + np.exp(-ALPHA * g)) * (u + BETA)
        rms = np.sqrt(np.mean(act ** 2))
        assert np.all(np.abs(out["act32"][r] - act) <= 1e-5 * np.abs(act) + 1e-5 * rms)
    assert n_clamped > 20
    # the rest of the block is the pinned requant / down / combine
    aq, sa = oracle.quant_rows_f32(out["act32"], OCP)
    assert np.array_equal(aq, out["aq"]) and np.array_equal(sa, out["sa"])
    d32, y32, y16 = oracle.moe_down(aq, sa, d["ids"], d["probs"], d["w2"], d["s2"])
    assert np.array_equal(y32, out["y32"]) and np.array_equal(y16, out["y16"])


def test_moe_gate_up_act_matches_block(oracle):
    d = _online_block(oracle, seed=53)
    act = (ALPHA, BETA, 0.2)
    out = oracle.moe_fp8(d["x"], d["ids"], d["probs"], d["w13"], d["s13"], d["w2"], d["s2"], act=act)
    xq, sx = oracle.quant_act(d["x"], OCP)
    assert np.array_equal(oracle.moe_gate_up(xq, sx, d["ids"], d["w13"], d["s13"], act=act),
                          out["act32"])
