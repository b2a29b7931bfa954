"""Seeded synthetic inputs for the quantized-linear workloads.

This module only draws inputs; it holds none of the arithmetic of the
quantized linear layer (no quantization, no GEMM, no repack). Both the test
suite and the benchmark draw their inputs from here, so the GPU path and the
CPU oracle always see identical bytes.

Workload shapes and distributions:

* QAT grid weights ("Gemma 4 ... QAT q4_0 unquantized" release, as described
  in the MI300X article, section "Ten builds", and the 31B model card): every
  Linear weight lies on a 4-bit grid with one scale per 32 consecutive values
  along K, stored as bf16. Synthetic stand-in: codes uniform in [-8, 7], one
  fp32 step per (output row, group of 32) drawn lognormal(ln 0.01, 0.5) and
  rounded to the nearest bf16 (so the stored bf16 tensor determines the step
  exactly), materialised as bf16(code * step).
* Activations: bf16 N(0, 1) with 1 % of entries multiplied by 20 (outliers),
  drawn once at the largest M of a configuration; smaller M use leading rows.
* MoE routing (router outside the block): N(0, 1) fp32 router logits, top-8
  of the softmax, weights not renormalised. Ties go to the lower expert id.

Draw order inside one configuration: weights (per matrix codes, then steps;
for the MoE experts in ascending order, gate_up then down), then activations,
then router logits.
"""

from __future__ import annotations

import numpy as np

GROUP = 32


# --------------------------------------------------------------------------
# bf16 storage helpers (input materialisation only)
# --------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# element generators
# --------------------------------------------------------------------------
def qat_grid(rng: np.random.Generator, n: int, k: int, bf16_steps: bool = True):
    """One Linear weight on the QAT q4_0 grid.

    Returns (codes int8 [n,k] in [-8,7], steps float32 [n,k/32] holding bf16
    values, w_bf16 uint16 [n,k] = bf16(code*step)). With bf16_steps=False the
    steps keep their full fp32 draw (a trained checkpoint's steps need not be
    bf16 values), so bf16(code*step) rounds values whose product needs more
    than bf16's 8 significant bits.
    """
    assert k % GROUP == 0
    codes = rng.integers(-8, 8, size=(n, k), dtype=np.int8)
    steps = rng.lognormal(np.log(0.01), 0.5, size=(n, k // GROUP)).astype(np.float32)
    if bf16_steps:
        steps = bf16_bits_to_f32(to_bf16_bits(steps))
    w = codes.astype(np.float32).reshape(n, k // GROUP, GROUP) * steps[:, :, None]
    w_bf16 = to_bf16_bits(w.reshape(n, k))
    return codes, steps, w_bf16


def dense_bf16(rng: np.random.Generator, n: int, k: int) -> np.ndarray:
    """One non-QAT bf16 weight [n,k] (bits): N(0,1) entries times a per-row
    lognormal magnitude around 0.02, so that the output channels differ in
    scale as trained channels do, with 0.1 % of entries scaled by 8 (heavy
    tails set each channel's absmax)."""
    w = rng.standard_normal(size=(n, k), dtype=np.float32)
    w *= rng.lognormal(np.log(0.02), 0.3, size=(n, 1)).astype(np.float32)
    mask = rng.random(size=(n, k), dtype=np.float32) < 0.001
    w[mask] *= 8.0
    return to_bf16_bits(w)


def activations(rng: np.random.Generator, m: int, k: int) -> np.ndarray:
    """bf16 bits [m,k]: N(0,1) with 1 % of entries scaled by 20."""
    x = rng.standard_normal(size=(m, k), dtype=np.float32)
    mask = rng.random(size=(m, k), dtype=np.float32) < 0.01
    x[mask] *= 20.0
    return to_bf16_bits(x)


def wide_range_rows(rng: np.random.Generator, m: int, k: int) -> np.ndarray:
    """bf16 bits [m,k] spread over the whole bf16 range: row i draws a top
    exponent field e_i in [1, 254] and a width w_i in [0, 40]; each value
    takes an exponent field uniform in [max(0, e_i - w_i), e_i] (field 0:
    subnormals), a uniform mantissa and sign; 1 % of values are +0 or -0."""
    e_hi = rng.integers(1, 255, size=(m, 1))
    w = rng.integers(0, 41, size=(m, 1))
    e = np.maximum(e_hi - rng.integers(0, 1 << 30, size=(m, k)) % (w + 1), 0)
    mant = rng.integers(0, 128, size=(m, k))
    sign = rng.integers(0, 2, size=(m, k))
    bits = (sign << 15) | (e << 7) | mant
    zero = rng.random(size=(m, k)) < 0.01
    bits[zero] = sign[zero] << 15
    return bits.astype(np.uint16)


def route_topk(logits: np.ndarray, topk: int):
    """Router stand-in: softmax over experts, top-k ids and probabilities.

    The router sits outside the MoE block; its output is an input of the
    block. Returns (ids int32 [T,topk], probs float32 [T,topk]).
    """
    lg = logits.astype(np.float64)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    # stable sort on -p: equal probabilities keep ascending expert order
    order = np.argsort(-p, axis=1, kind="stable")[:, :topk]
    ids = order.astype(np.int32)
    probs = np.take_along_axis(p, order, axis=1).astype(np.float32)
    return ids, probs


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------
CONFIGS = {
    1: dict(name="C1 single layer M=4 K=256 N=512", seed=0, K=256, N=512, M=(4,)),
    2: dict(name="C2 decode K=2048 N=8192", seed=1, K=2048, N=8192, M=(1, 8, 64)),
    3: dict(name="C3 large decode K=5120 N=25600", seed=2, K=5120, N=25600, M=(1, 8, 64)),
    4: dict(name="C4 prefill M=8192", seed=3, M=8192, shapes=((4096, 14336), (14336, 4096))),
    5: dict(name="C5 MoE E=128 H=2048 I=768 top-8", seed=4, E=128, H=2048, I=768, topk=8,
            T=(64, 512)),
}


def linear_config(cfg: int, n: int | None = None, k: int | None = None, m: int | None = None,
                  bf16_steps: bool = True):
    """Inputs of a dense configuration (1, 2 or 3).

    Optional n/k/m override the sizes (same seed and draw order), for small
    parity cases of the same distribution. bf16_steps=False draws the same
    grid with unrounded fp32 steps (see qat_grid).
    """
    c = CONFIGS[cfg]
    rng = np.random.default_rng(c["seed"])
    N = c["N"] if n is None else n
    K = c["K"] if k is None else k
    M = max(c["M"]) if m is None else m
    codes, steps, w_bf16 = qat_grid(rng, N, K, bf16_steps)
    a = activations(rng, M, K)
    return dict(codes=codes, steps=steps, w_bf16=w_bf16, a=a, M=M, N=N, K=K)


def prefill_config(which: int, m: int | None = None, rows_n: int | None = None):
    """Inputs of configuration 4, shape index 0 (K=4096,N=14336) or 1.

    Weights for both shapes are drawn first, then both activations, so the
    draw order is fixed whichever shape is asked for. `m` / `rows_n` keep
    only the leading rows (same bytes as the full draw).
    """
    c = CONFIGS[4]
    rng = np.random.default_rng(c["seed"])
    ws = [qat_grid(rng, n, k) for (k, n) in c["shapes"]]
    acts = []
    for (k, _n) in c["shapes"]:
        acts.append(activations(rng, c["M"], k))
    K, N = c["shapes"][which]
    codes, steps, w_bf16 = ws[which]
    a = acts[which]
    if m is not None:
        a = a[:m]
    if rows_n is not None:
        codes, steps, w_bf16 = codes[:rows_n], steps[:rows_n], w_bf16[:rows_n]
        N = rows_n
    return dict(codes=codes, steps=steps, w_bf16=w_bf16, a=np.ascontiguousarray(a),
                M=a.shape[0], N=N, K=K)


def moe_config(E: int | None = None, H: int | None = None, I: int | None = None,
               T: int | None = None, topk: int | None = None, seed: int | None = None):
    """Inputs of configuration 5 (or a smaller block of the same recipe).

    Returns q4 grids of every expert: gate_up [E, 2I, H] and down [E, H, I]
    (codes, steps, bf16), activations x [T,H] and routing ids/probs [T,topk].
    """
    c = CONFIGS[5]
    E = c["E"] if E is None else E
    H = c["H"] if H is None else H
    I = c["I"] if I is None else I
    T = max(c["T"]) if T is None else T
    topk = c["topk"] if topk is None else topk
    rng = np.random.default_rng(c["seed"] if seed is None else seed)
    c13 = np.empty((E, 2 * I, H), np.int8)
    s13 = np.empty((E, 2 * I, H // GROUP), np.float32)
    w13 = np.empty((E, 2 * I, H), np.uint16)
    c2 = np.empty((E, H, I), np.int8)
    s2 = np.empty((E, H, I // GROUP), np.float32)
    w2 = np.empty((E, H, I), np.uint16)
    for e in range(E):
        c13[e], s13[e], w13[e] = qat_grid(rng, 2 * I, H)
        c2[e], s2[e], w2[e] = qat_grid(rng, H, I)
    x = activations(rng, T, H)
    logits = rng.standard_normal(size=(T, E), dtype=np.float32)
    ids, probs = route_topk(logits, topk)
    return dict(E=E, H=H, I=I, T=T, topk=topk, codes13=c13, steps13=s13, w13_bf16=w13,
                codes2=c2, steps2=s2, w2_bf16=w2, x=x, logits=logits, ids=ids, probs=probs)


def moe_bf16_config(E: int | None = None, H: int | None = None, I: int | None = None,
                    T: int | None = None, topk: int | None = None, seed: int | None = None):
    """A bf16 (non-QAT) MoE block of configuration 5's shape: the expert
    banks are dense_bf16 weights, quantised per channel on line. Returns
    w13_bf16 [E, 2I, H], w2_bf16 [E, H, I], x [T,H], ids/probs [T,topk]."""
    c = CONFIGS[5]
    E = c["E"] if E is None else E
    H = c["H"] if H is None else H
    I = c["I"] if I is None else I
    T = max(c["T"]) if T is None else T
    topk = c["topk"] if topk is None else topk
    rng = np.random.default_rng((c["seed"] + 100) if seed is None else seed)
    w13 = np.empty((E, 2 * I, H), np.uint16)
    w2 = np.empty((E, H, I), np.uint16)
    for e in range(E):
        w13[e] = dense_bf16(rng, 2 * I, H)
        w2[e] = dense_bf16(rng, H, I)
    x = activations(rng, T, H)
    logits = rng.standard_normal(size=(T, E), dtype=np.float32)
    ids, probs = route_topk(logits, topk)
    return dict(E=E, H=H, I=I, T=T, topk=topk, w13_bf16=w13, w2_bf16=w2, x=x, logits=logits,
                ids=ids, probs=probs)


def vocab_config(V: int = 262144, D: int = 1536, T: int = 64, seed: int = 7):
    """An int4 vocabulary table on the QAT grid (the pages give no table
    shape: 2^18 rows of 1536 by default) with T token ids uniform in [0, V)
    and T hidden rows (activations) for the untied lm_head."""
    rng = np.random.default_rng(seed)
    codes, steps, w_bf16 = qat_grid(rng, V, D)
    ids = rng.integers(0, V, size=T, dtype=np.int32)
    h = activations(rng, T, D)
    return dict(V=V, D=D, T=T, codes=codes, steps=steps, w_bf16=w_bf16, ids=ids, h=h)
