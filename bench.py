#!/usr/bin/env python3
"""Benchmark of the quantized linear layer on one MI355X.

One step = one pass of the per-call hot path over one batch at the decode
layer K=2048, N=8192 (seed 1) for M in {1, 8, 64}:
  FP8 W8A8   : per-token FP8 quantisation of x[:M] + row-scaled FP8 GEMM
  int8 W8A8  : per-token int8 quantisation of x[:M] + int8 GEMM
  W4A16      : group-32 int4 GEMM with in-kernel unpack
(9 GEMMs + 6 quantisations). The weights rotate through enough copies
(>= 1 GiB per format pass) that every launch streams them from HBM, not
from the 256 MB Infinity Cache; activations stay warm as in serving. Each
step is a captured HIP graph, replayed (launch overhead excluded, as in the
pages' GEMM micro-benchmark).

value = weight bytes streamed per step / step time  (GB/s)

Also reported in the same JSON line:
  roofline      the dominant kernel of the step, achieved weight GB/s from
                HIP events around its launches vs the 8 TB/s HBM peak;
  cpu_baseline  the CPU oracle running the same step on the host cores;
  rows          per-kernel figures: every decode GEMM of the step, the large
                decode layer (K=5120, N=25600), the prefill GEMMs (M=8192,
                TFLOP/s vs MFMA peak), the MoE block and the offline repacks.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
for _p in (ROOT, os.path.join(ROOT, "tests")):
    if _p not in sys.path:
        sys.path.insert(0, _p)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "int8": 5000.0, "bf16": 2500.0}
GIB = 1 << 30


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extras", action="store_true", help="skip the C3/C4/C5/repack rows")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--kernel-iters", type=int, default=64,
                    help="event-timed launches per kernel for the per-kernel rows")
    ap.add_argument("--pmc-workload", choices=("prefill", "moe"), default=None,
                    help="counter-collection workload for rocprofv3 --pmc: the C4 prefill GEMMs "
                         "(fp8, int8, W4A16, torch bf16; 3 launches each) or the C5 MoE blocks "
                         "(fp8, fp8 + SwiGLU-OAI, W4A16 at T = 64 and 512; 3 launches each), "
                         "then the 256 MiB copy that calibrates FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="counter-collection workload: every decode GEMM of the step, 8 eager "
                         "launches each, then a 256 MiB device copy (the counters' calibration); "
                         "run under rocprofv3 --pmc")
    return ap.parse_args()


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def dev(a, torch):
    import numpy as np

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def weight_bytes(fmt, N, K):
    if fmt in ("fp8", "int8"):
        return N * K + 4 * N  # codes + fp32 per-channel scales
    if fmt == "w4a16":
        return N * K // 2 + 2 * N * (K // 32)  # int4 codes + bf16 group steps
    if fmt == "bf16":
        return 2 * N * K
    raise ValueError(fmt)


class Timer:
    """Per-launch device time with HIP events on the launching stream. A
    queue filler keeps the device busy while the host enqueues, so each
    event pair brackets one kernel without host gaps."""

    def __init__(self, torch):
        self.torch = torch

    def time(self, fn, iters, filler_ms=30.0):
        torch = self.torch
        st = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        torch.cuda.synchronize()
        _filler(torch, filler_ms)
        for i in range(iters):
            ev[i][0].record(st)
            fn(i)
            ev[i][1].record(st)
        torch.cuda.synchronize()
        d = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)  # us
        return dict(mean_us=sum(d) / len(d), median_us=d[len(d) // 2], min_us=d[0])


class GraphTimer:
    """Average device time per launch: `reps` launches of one call (rotating
    over weight copies) captured in one HIP graph, replayed with events
    around each replay on the replaying stream; time per launch = replay
    time / reps. Back-to-back graph launches leave little idle time between
    kernels, so this agrees with the profiler's kernel durations."""

    def __init__(self, torch):
        self.torch = torch

    def time(self, fn, reps=32, replays=5):
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(2):
                fn(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(reps):
                fn(i)
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        g.replay()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(replays)]
        for a, b in ev:
            a.record(st)
            g.replay()
            b.record(st)
        torch.cuda.synchronize()
        d = sorted(a.elapsed_time(b) * 1e3 / reps for a, b in ev)  # us per launch
        del g
        return dict(mean_us=sum(d) / len(d), median_us=d[len(d) // 2], min_us=d[0])


_FILL = {}


def _filler(torch, ms):
    """Busy the stream for ~ms milliseconds (bf16 matmuls, calibrated once)."""
    if "a" not in _FILL:
        _FILL["a"] = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
        a = _FILL["a"]
        for _ in range(3):
            a @ a
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(10):
            a @ a
        e.record()
        torch.cuda.synchronize()
        _FILL["ms"] = max(s.elapsed_time(e) / 10, 1e-3)
    a = _FILL["a"]
    for _ in range(max(1, int(ms / _FILL["ms"]))):
        a @ a


# ----------------------------------------------------------------------------
# the decode step at K=2048, N=8192
# ----------------------------------------------------------------------------
class DecodeLayer:
    """Weights of one layer in the three formats, rotated over `copies`."""

    def __init__(self, q, torch, d, copies):
        self.q, self.torch = q, torch
        self.N, self.K = d["N"], d["K"]
        w = dev(d["w_bf16"], torch)
        codes, steps, amb = q.repack_q4_0(w)
        wq8, ws8 = q.repack_fp8(codes, steps)
        wi8, wsi8 = q.repack_int8(codes, steps)
        torch.cuda.synchronize()
        self.n_ambiguous = int(amb.item())
        self.copies = copies
        self.fp8 = [(wq8.clone(), ws8.clone()) for _ in range(copies)]
        self.int8 = [(wi8.clone(), wsi8.clone()) for _ in range(copies)]
        self.w4 = [(codes.clone(), steps.clone()) for _ in range(copies)]
        self.w_bf16 = w
        del wq8, wi8


def run_step_fn(q, torch, L, x, Ms, bufs):
    def step(i):
        c = i % L.copies
        for M in Ms:
            b = bufs[M]
            xm = x[:M]
            q.quant_act(xm, "e4m3", out=(b["aq8"], b["sa8"]))
            q.gemm_fp8(b["aq8"], b["sa8"], *L.fp8[c], out=b["y8"])
            q.quant_act(xm, "int8", out=(b["aqi"], b["sai"]))
            q.gemm_w8a8(b["aqi"], b["sai"], *L.int8[c], out=b["yi"])
            q.gemm_w4a16(xm, *L.w4[c], out=b["y4"])
    return step


def make_bufs(torch, Ms, N, K):
    out = {}
    for M in Ms:
        out[M] = dict(aq8=torch.empty(M, K, dtype=torch.uint8, device="cuda"),
                      sa8=torch.empty(M, dtype=torch.float32, device="cuda"),
                      aqi=torch.empty(M, K, dtype=torch.int8, device="cuda"),
                      sai=torch.empty(M, dtype=torch.float32, device="cuda"),
                      y8=torch.empty(M, N, dtype=torch.bfloat16, device="cuda"),
                      yi=torch.empty(M, N, dtype=torch.bfloat16, device="cuda"),
                      y4=torch.empty(M, N, dtype=torch.bfloat16, device="cuda"))
    return out


def gemm_calls(q, L, x, Ms, bufs):
    """(row name suffix, M, format, call(i)) for every decode GEMM of the step
    and the FP8 activation quantisation (operands prepared outside)."""
    out = []
    for M in Ms:
        b = bufs[M]
        xm = x[:M]
        q.quant_act(xm, "e4m3", out=(b["aq8"], b["sa8"]))
        q.quant_act(xm, "int8", out=(b["aqi"], b["sai"]))
        out += [
            (f"fp8_M{M}", M, "fp8",
             lambda i, b=b: q.gemm_fp8(b["aq8"], b["sa8"], *L.fp8[i % L.copies], out=b["y8"])),
            (f"int8_M{M}", M, "int8",
             lambda i, b=b: q.gemm_w8a8(b["aqi"], b["sai"], *L.int8[i % L.copies], out=b["yi"])),
            (f"w4a16_M{M}", M, "w4a16",
             lambda i, xm=xm, b=b: q.gemm_w4a16(xm, *L.w4[i % L.copies], out=b["y4"])),
            (f"quant_fp8_M{M}", M, "quant_fp8",
             lambda i, xm=xm, b=b: q.quant_act(xm, "e4m3", out=(b["aq8"], b["sa8"]))),
        ]
    return out


def per_kernel_rows(q, torch, L, x, Ms, bufs, iters, tag):
    """Per-launch device time of each GEMM of the step (graph-timed, see
    GraphTimer), weight GB/s and the fraction of the HBM peak."""
    T = GraphTimer(torch)
    rows = {}
    for name, M, fmt, fn in gemm_calls(q, L, x, Ms, bufs):
        t = T.time(fn, reps=min(32, max(8, iters // 2)))
        r = dict(M=M, us=round(t["mean_us"], 3), min_us=round(t["min_us"], 3))
        if fmt != "quant_fp8":
            wb = weight_bytes(fmt, L.N, L.K)
            r["weight_bytes"] = wb
            r["GBps"] = round(wb / (t["mean_us"] * 1e3), 1)
            r["frac_hbm"] = round(r["GBps"] / HBM_PEAK_GBS, 4)
        rows[f"{tag}_{name}"] = r
    return rows


def bf16_rows(torch, L, x, Ms, iters, tag):
    """torch's bf16 GEMM on the materialised weights (the comparator): the
    faster of x @ W^T and (W @ x^T)^T, graph-timed like the other rows."""
    T = GraphTimer(torch)
    ws = [L.w_bf16.clone() for _ in range(max(4, int(math.ceil(1.5 * GIB / (2 * L.N * L.K)))))]
    rows = {}
    for M in Ms:
        xm = x[:M].contiguous()
        xt = xm.t().contiguous()
        best = None
        for form, fn in (("x@Wt", lambda i, xm=xm: torch.matmul(xm, ws[i % len(ws)].t())),
                         ("(W@xt)t", lambda i, xt=xt: torch.matmul(ws[i % len(ws)], xt))):
            t = T.time(fn, reps=min(16, len(ws)))
            if best is None or t["mean_us"] < best[1]["mean_us"]:
                best = (form, t)
        wb = weight_bytes("bf16", L.N, L.K)
        rows[f"{tag}_bf16_torch_M{M}"] = dict(M=M, us=round(best[1]["mean_us"], 3), form=best[0],
                                             GBps=round(wb / (best[1]["mean_us"] * 1e3), 1))
    del ws
    return rows


# ----------------------------------------------------------------------------
# extras
# ----------------------------------------------------------------------------
def repack_fidelity(torch, codes, steps, wq, ws, fmt, rows_per=2048):
    """Fidelity of an FP8 repack against the QAT grid values it came from:
    relative RMS error sqrt(sum (dec(q)*s - w)^2 / sum w^2) and the largest
    per-row max error over the row's max |w| (w = c*step, exact), in fp64
    with torch on the device, a block of rows at a time."""
    f8 = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e4m3fnuz
    num = den = 0.0
    mx = 0.0
    N = codes.shape[0]
    for n0 in range(0, N, rows_per):
        c = codes[n0:n0 + rows_per].to(torch.int32)
        grid = torch.stack(((c & 15) - 8, (c >> 4) - 8), dim=-1).reshape(c.shape[0], -1).to(torch.float64)
        st = steps[n0:n0 + rows_per].to(torch.float64).repeat_interleave(32, dim=1)
        w = grid * st
        d = wq[n0:n0 + rows_per].view(f8).to(torch.float64) * ws[n0:n0 + rows_per].to(torch.float64)[:, None]
        e = d - w
        num += float((e * e).sum())
        den += float((w * w).sum())
        amax = w.abs().amax(dim=1)
        r = torch.where(amax > 0, e.abs().amax(dim=1) / amax, torch.zeros_like(amax))
        mx = max(mx, float(r.max()))
    return (num / den) ** 0.5 if den > 0 else 0.0, mx


def c3_rows(q, torch, gen, iters):
    d = gen.linear_config(3)
    copies = max(2, int(math.ceil(1.1 * GIB / weight_bytes("fp8", d["N"], d["K"]))))
    L = DecodeLayer(q, torch, d, copies)
    x = dev(d["a"], torch)
    Ms = (1, 8, 64)
    bufs = make_bufs(torch, Ms, L.N, L.K)
    rows = per_kernel_rows(q, torch, L, x, Ms, bufs, iters, "C3")
    rows = {k: v for k, v in rows.items() if "_int8_" not in k}
    rows.update(bf16_rows(torch, L, x, Ms, iters, "C3"))
    # offline repacks on this layer
    T = Timer(torch)
    w = L.w_bf16
    t = T.time(lambda i: q.repack_q4_0(w), 4, filler_ms=5)
    rows["C3_repack_q4_0"] = dict(us=round(t["mean_us"], 1), n_ambiguous=L.n_ambiguous)
    codes, steps = L.w4[0]
    t = T.time(lambda i: q.repack_fp8(codes, steps), 8, filler_ms=5)
    rows["C3_repack_fp8"] = dict(us=round(t["mean_us"], 1))
    for fmt in ("e4m3", "e4m3fnuz"):
        wq_, ws_ = q.repack_fp8(codes, steps, fmt)
        rr, mr = repack_fidelity(torch, codes, steps, wq_, ws_, fmt)
        rows["C3_repack_fp8"][f"rel_rms_{fmt}"] = round(rr, 6)
        rows["C3_repack_fp8"][f"max_err_over_row_max_{fmt}"] = round(mr, 6)
        del wq_, ws_
    wf, sf = q.repack_fp8(codes, steps, "e4m3fnuz")
    wo, so, bad = q.fp8_fnuz_to_ocp(wf, sf)
    t = T.time(lambda i: q.fp8_fnuz_to_ocp(wf, sf), 8, filler_ms=5)
    torch.cuda.synchronize()
    rows["C3_fnuz_to_ocp"] = dict(us=round(t["mean_us"], 1), n_inexact=int(bad.item()),
                                  bit_identical_to_ocp_repack=bool(torch.equal(wo, L.fp8[0][0])))
    del L
    torch.cuda.empty_cache()
    return rows


def c4_rows(q, torch, gen, iters):
    rows = {}
    T = Timer(torch)
    for which in (0, 1):
        d = gen.prefill_config(which)
        M, N, K = d["M"], d["N"], d["K"]
        flops = 2.0 * M * N * K
        w = dev(d["w_bf16"], torch)
        codes, steps, _ = q.repack_q4_0(w)
        wq8, ws8 = q.repack_fp8(codes, steps)
        wi8, wsi8 = q.repack_int8(codes, steps)
        x = dev(d["a"], torch)
        aq8, sa8 = q.quant_act(x, "e4m3")
        aqi, sai = q.quant_act(x, "int8")
        y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        n_it = max(4, iters // 8)
        t_q = T.time(lambda i: q.quant_act(x, "e4m3", out=(aq8, sa8)), n_it, filler_ms=5)
        t_g8 = T.time(lambda i: q.gemm_fp8(aq8, sa8, wq8, ws8, out=y), n_it, filler_ms=5)
        t_gi = T.time(lambda i: q.gemm_w8a8(aqi, sai, wi8, wsi8, out=y), n_it, filler_ms=5)
        # W4A16 at the prefill shape (bf16 activations, int4 weights unpacked
        # in the kernel) and torch's bf16 matmul on the same bf16 weights
        t_w4 = T.time(lambda i: q.gemm_w4a16(x, codes, steps, out=y), n_it, filler_ms=5)
        t_bf = T.time(lambda i: torch.matmul(x, w.t(), out=y), n_it, filler_ms=5)
        tag = f"C4_K{K}_N{N}"
        for name, t, peak in (("fp8_gemm", t_g8, "fp8"), ("int8_gemm", t_gi, "int8"),
                              ("w4a16_gemm", t_w4, "bf16"), ("bf16_torch", t_bf, "bf16")):
            tf = flops / (t["mean_us"] * 1e-6) / 1e12
            rows[f"{tag}_{name}"] = dict(us=round(t["mean_us"], 1), TFLOPs=round(tf, 1),
                                         frac_mfma=round(tf / MFMA_PEAK_TFLOPS[peak], 4))
        tot = t_q["mean_us"] + t_g8["mean_us"]
        tf = flops / (tot * 1e-6) / 1e12
        rows[f"{tag}_fp8_linear_incl_quant"] = dict(us=round(tot, 1), quant_us=round(t_q["mean_us"], 1),
                                                    TFLOPs=round(tf, 1),
                                                    frac_mfma=round(tf / MFMA_PEAK_TFLOPS["fp8"], 4))
        del wq8, wi8, x, aq8, aqi, y, w, codes, steps
        torch.cuda.empty_cache()
    return rows


def c5_rows(q, torch, gen, iters):
    rows = {}
    d = gen.moe_config()
    E, H, I = d["E"], d["H"], d["I"]
    w13 = torch.empty(E, 2 * I, H, dtype=torch.uint8, device="cuda")
    s13 = torch.empty(E, 2 * I, dtype=torch.float32, device="cuda")
    w2 = torch.empty(E, H, I, dtype=torch.uint8, device="cuda")
    s2 = torch.empty(E, H, dtype=torch.float32, device="cuda")
    for e in range(E):
        c, s, _ = q.repack_q4_0(dev(d["w13_bf16"][e], torch))
        w13[e], s13[e] = q.repack_fp8(c, s)
        c, s, _ = q.repack_q4_0(dev(d["w2_bf16"][e], torch))
        w2[e], s2[e] = q.repack_fp8(c, s)
    copies = [(w13, s13, w2, s2)] + [(w13.clone(), s13.clone(), w2.clone(), s2.clone())
                                     for _ in range(2)]
    T = Timer(torch)
    for Tn in (64, 512):
        x = dev(d["x"][:Tn], torch)
        ids = dev(d["ids"][:Tn], torch)
        pr = dev(d["probs"][:Tn], torch)
        touched = len(set(d["ids"][:Tn].ravel().tolist()))
        wb = touched * (2 * I * H + 4 * 2 * I + H * I + 4 * H)
        t = T.time(lambda i: q.moe_fp8(x, ids, pr, *copies[i % len(copies)]), max(6, iters // 4),
                   filler_ms=5)
        gbs = wb / (t["mean_us"] * 1e3)
        rows[f"C5_moe_fp8_T{Tn}"] = dict(us=round(t["mean_us"], 1), experts_touched=touched,
                                         weight_bytes=wb, GBps=round(gbs, 1),
                                         frac_hbm=round(gbs / HBM_PEAK_GBS, 4))
    del copies, w13, w2
    torch.cuda.empty_cache()
    # W4A16 block: packed codes and bf16 group steps of every expert, read
    # in place by the grouped GEMMs
    c13 = torch.empty(E, 2 * I, H // 2, dtype=torch.uint8, device="cuda")
    t13 = torch.empty(E, 2 * I, H // 32, dtype=torch.bfloat16, device="cuda")
    c2 = torch.empty(E, H, I // 2, dtype=torch.uint8, device="cuda")
    t2 = torch.empty(E, H, I // 32, dtype=torch.bfloat16, device="cuda")
    for e in range(E):
        c13[e], t13[e], _ = q.repack_q4_0(dev(d["w13_bf16"][e], torch))
        c2[e], t2[e], _ = q.repack_q4_0(dev(d["w2_bf16"][e], torch))
    copies = [(c13, t13, c2, t2)] + [tuple(a.clone() for a in (c13, t13, c2, t2)) for _ in range(2)]
    for Tn in (64, 512):
        x = dev(d["x"][:Tn], torch)
        ids = dev(d["ids"][:Tn], torch)
        pr = dev(d["probs"][:Tn], torch)
        touched = len(set(d["ids"][:Tn].ravel().tolist()))
        wb = touched * (2 * I * H // 2 + 2 * I * (H // 32) * 2 + H * I // 2 + H * (I // 32) * 2)
        t = T.time(lambda i: q.moe_w4a16(x, ids, pr, *copies[i % len(copies)]), max(6, iters // 4),
                   filler_ms=5)
        gbs = wb / (t["mean_us"] * 1e3)
        rows[f"C5_moe_w4a16_T{Tn}"] = dict(us=round(t["mean_us"], 1), experts_touched=touched,
                                           weight_bytes=wb, GBps=round(gbs, 1),
                                           frac_hbm=round(gbs / HBM_PEAK_GBS, 4))
    del copies, c13, c2
    torch.cuda.empty_cache()
    # bf16 (non-QAT) banks quantised per channel on line, then the FP8 block
    # with the SwiGLU-OAI activation (alpha 1.702, beta 1.0, clamp 7.0)
    d = gen.moe_bf16_config()
    b13 = dev(d["w13_bf16"].reshape(E * 2 * I, H), torch)
    b2 = dev(d["w2_bf16"].reshape(E * H, I), torch)
    tq = T.time(lambda i: (q.quant_weight(b13), q.quant_weight(b2)), max(4, iters // 8), filler_ms=5)
    qb = (b13.numel() + b2.numel()) * 3 + 4 * (E * 2 * I + E * H)
    rows["C5_quant_weight_bf16_banks"] = dict(us=round(tq["mean_us"], 1), bytes=qb,
                                              GBps=round(qb / (tq["mean_us"] * 1e3), 1))
    w13, s13 = q.quant_weight(b13)
    w2, s2 = q.quant_weight(b2)
    del b13, b2
    w13, s13, w2, s2 = w13.view(E, 2 * I, H), s13.view(E, 2 * I), w2.view(E, H, I), s2.view(E, H)
    copies = [(w13, s13, w2, s2)] + [(w13.clone(), s13.clone(), w2.clone(), s2.clone())
                                     for _ in range(2)]
    for Tn in (64, 512):
        x = dev(d["x"][:Tn], torch)
        ids = dev(d["ids"][:Tn], torch)
        pr = dev(d["probs"][:Tn], torch)
        touched = len(set(d["ids"][:Tn].ravel().tolist()))
        wb = touched * (2 * I * H + 4 * 2 * I + H * I + 4 * H)
        t = T.time(lambda i: q.moe_fp8(x, ids, pr, *copies[i % len(copies)],
                                       swiglu_oai=(1.702, 1.0, 7.0)), max(6, iters // 4), filler_ms=5)
        gbs = wb / (t["mean_us"] * 1e3)
        rows[f"C5_moe_fp8_swiglu_oai_T{Tn}"] = dict(us=round(t["mean_us"], 1), experts_touched=touched,
                                                    weight_bytes=wb, GBps=round(gbs, 1),
                                                    frac_hbm=round(gbs / HBM_PEAK_GBS, 4))
    del copies, w13, w2
    torch.cuda.empty_cache()
    return rows


def vocab_rows(q, torch, gen, iters):
    """int4 vocabulary tables (262144 x 1536): the untied lm_head as a W4A16
    GEMM with N = 262144 and the embedding lookup, each beside torch on the
    same table in bf16."""
    import numpy as np

    rows = {}
    d = gen.vocab_config()
    V, D = d["V"], d["D"]
    w = dev(d["w_bf16"], torch)
    codes, steps, _ = q.repack_q4_0(w)
    cps = [(codes, steps)] + [(codes.clone(), steps.clone()) for _ in range(3)]
    ws = [w, w.clone()]
    h = dev(d["h"], torch)
    T = GraphTimer(torch)
    wb4, wb16 = weight_bytes("w4a16", V, D), weight_bytes("bf16", V, D)
    for M in (1, 8, 64):
        xm = h[:M].contiguous()
        xt = xm.t().contiguous()
        y = torch.empty(M, V, dtype=torch.bfloat16, device="cuda")
        t = T.time(lambda i, xm=xm, y=y: q.gemm_w4a16(xm, *cps[i % len(cps)], out=y), reps=16)
        gbs = wb4 / (t["mean_us"] * 1e3)
        rows[f"V_lm_head_w4a16_M{M}"] = dict(us=round(t["mean_us"], 2), weight_bytes=wb4,
                                             GBps=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4))
        best = None
        for form, fn in (("x@Wt", lambda i, xm=xm: torch.matmul(xm, ws[i % 2].t())),
                         ("(W@xt)t", lambda i, xt=xt: torch.matmul(ws[i % 2], xt))):
            tb = T.time(fn, reps=8)
            if best is None or tb["mean_us"] < best[1]["mean_us"]:
                best = (form, tb)
        rows[f"V_lm_head_bf16_torch_M{M}"] = dict(us=round(best[1]["mean_us"], 2), form=best[0],
                                                  GBps=round(wb16 / (best[1]["mean_us"] * 1e3), 1))
    for Tn in (64, 8192):
        ids_np = np.random.default_rng(Tn).integers(0, V, size=Tn, dtype=np.int32)
        ids = dev(ids_np, torch)
        ids64 = ids.long()
        t = T.time(lambda i: q.embed_q4(ids, *cps[i % len(cps)]), reps=16)
        moved = Tn * (D // 2 + 2 * (D // 32) + 2 * D)
        rows[f"V_embed_q4_T{Tn}"] = dict(us=round(t["mean_us"], 2), bytes=moved,
                                         GBps=round(moved / (t["mean_us"] * 1e3), 1))
        tb = T.time(lambda i: torch.index_select(ws[i % 2], 0, ids64), reps=16)
        rows[f"V_embed_bf16_torch_T{Tn}"] = dict(us=round(tb["mean_us"], 2))
    rows["V_table_bytes"] = dict(int4=wb4, bf16=wb16, ratio=round(wb4 / wb16, 4))
    del cps, ws, codes, steps, w
    torch.cuda.empty_cache()
    return rows


# ----------------------------------------------------------------------------
# HBM traffic from hardware counters
# ----------------------------------------------------------------------------
TRAFFIC_MD = os.path.join(ROOT, "profiles", "decode_gemm_K2048_N8192_pmc_traffic.md")
DECODE_SOURCES = ("qlin_gemm_decode.hip", "qlin_skinny.h", "qlin_device.h")


def decode_sources_sha256():
    import hashlib

    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "quantized_linear_layers_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def pmc_pass(q, torch, L, x, Ms, bufs, launches=8):
    """Counter-collection workload (run under rocprofv3 --pmc): every decode
    GEMM of the step, `launches` eager launches each in a fixed order, then a
    plain 256 MiB device-to-device copy four times, whose FETCH_SIZE /
    WRITE_SIZE readings calibrate the counters (known bytes / reading)."""
    order = []
    for name, M, fmt, fn in gemm_calls(q, L, x, Ms, bufs):
        if fmt == "quant_fp8":
            continue
        torch.cuda.synchronize()
        for i in range(launches):
            fn(i)
        torch.cuda.synchronize()
        order.append("C2_" + name)
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_pass": order, "launches": launches, "copy_bytes": n, "copies": 4,
                      "sources_sha256": decode_sources_sha256()}), flush=True)


def pmc_workload(q, torch, which, launches=3):
    """Counter-collection workloads beyond the decode step (run under
    rocprofv3 --pmc): synthetic operands of the C4 / C5 shapes built on the
    device (uniform random codes, bf16 steps in [0.001, 0.021], N(0,1)
    activations, N(0, 0.02) bf16 weights quantised per channel), each call
    launched `launches` times in a fixed order, then the calibration copy."""
    torch.manual_seed(0)
    order = []

    def rep(name, fn):
        torch.cuda.synchronize()
        for _ in range(launches):
            fn()
        torch.cuda.synchronize()
        order.append(name)

    if which == "prefill":
        M = 8192
        for K, N in ((4096, 14336), (14336, 4096)):
            a = torch.randn(M, K, device="cuda").to(torch.bfloat16)
            w = (torch.randn(N, K, device="cuda") * 0.02).to(torch.bfloat16)
            aq, sa = q.quant_act(a, "e4m3")
            ai, sai = q.quant_act(a, "int8")
            wq, ws = q.quant_weight(w, "e4m3")
            wi, wsi = q.quant_weight(w, "int8")
            codes = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda")
            steps = (torch.rand(N, K // 32, device="cuda") * 0.02 + 0.001).to(torch.bfloat16)
            tag = f"C4_K{K}_N{N}"
            rep(f"{tag}_fp8", lambda: q.gemm_fp8(aq, sa, wq, ws))
            rep(f"{tag}_int8", lambda: q.gemm_w8a8(ai, sai, wi, wsi))
            rep(f"{tag}_w4a16", lambda: q.gemm_w4a16(a, codes, steps))
            rep(f"{tag}_bf16_torch", lambda: torch.matmul(a, w.t()))
            del a, w, aq, ai, wq, wi, codes, steps
    else:
        import numpy as np

        import gen
        E, H, I, topk = 128, 2048, 768, 8
        w13, s13 = q.quant_weight((torch.randn(E * 2 * I, H, device="cuda") * 0.02).to(torch.bfloat16))
        w2, s2 = q.quant_weight((torch.randn(E * H, I, device="cuda") * 0.02).to(torch.bfloat16))
        fp8w = (w13.view(E, 2 * I, H), s13.view(E, 2 * I), w2.view(E, H, I), s2.view(E, H))
        w4 = (torch.randint(0, 256, (E, 2 * I, H // 2), dtype=torch.uint8, device="cuda"),
              (torch.rand(E, 2 * I, H // 32, device="cuda") * 0.02 + 0.001).to(torch.bfloat16),
              torch.randint(0, 256, (E, H, I // 2), dtype=torch.uint8, device="cuda"),
              (torch.rand(E, H, I // 32, device="cuda") * 0.02 + 0.001).to(torch.bfloat16))
        rng = np.random.default_rng(0)
        for T in (64, 512):
            ids, pr = gen.route_topk(rng.standard_normal((T, E), dtype=np.float32), topk)
            ids, pr = dev(ids, torch), dev(pr, torch)
            x = torch.randn(T, H, device="cuda").to(torch.bfloat16)
            rep(f"C5_moe_fp8_T{T}", lambda: q.moe_fp8(x, ids, pr, *fp8w))
            rep(f"C5_moe_fp8_swiglu_oai_T{T}", lambda: q.moe_fp8(x, ids, pr, *fp8w, swiglu_oai=(1.702, 1.0, 7.0)))
            rep(f"C5_moe_w4a16_T{T}", lambda: q.moe_w4a16(x, ids, pr, *w4))
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_workload": which, "order": order, "launches": launches, "copy_bytes": n,
                      "copies": 4}), flush=True)


def traffic_table():
    """Per-launch HBM bytes of each decode GEMM of the step, from the
    committed counter summary, if it was taken on the current kernel sources
    (else None: the counters no longer describe this code)."""
    try:
        with open(TRAFFIC_MD) as fh:
            txt = fh.read()
        blob = txt[txt.index("```json") + 7:]
        blob = blob[:blob.index("```")]
        tab = json.loads(blob)
    except (OSError, ValueError):
        return None
    if tab.get("sources_sha256") != decode_sources_sha256():
        return None
    return tab


# ----------------------------------------------------------------------------
# CPU baseline: the oracle running the same step on the host
# ----------------------------------------------------------------------------
def cpu_baseline(gen, d, Ms, step_weight_bytes, budget_s=12.0):
    import numpy as np
    import oracle

    p, s, _ = oracle.repack_q4_0(d["w_bf16"])
    K = d["K"]
    wq8, ws8 = oracle.repack_fp8(p, s, K, oracle.OCP)
    wi8, wsi8 = oracle.repack_int8(p, s, K)

    def one():
        for M in Ms:
            a = d["a"][:M]
            aq, sa = oracle.quant_act(a, oracle.OCP)
            oracle.gemm_fp8(aq, sa, wq8, ws8)
            ai, sai = oracle.quant_act(a, oracle.INT8)
            oracle.gemm_w8a8(ai, sai, wi8, wsi8)
            oracle.gemm_w4a16(a, p, s)

    t0 = time.perf_counter()
    one()
    reps = 1
    while time.perf_counter() - t0 < budget_s and reps < 1000:
        one()
        reps += 1
    dt = time.perf_counter() - t0
    _ = np
    return dict(value=round(step_weight_bytes * reps / dt / 1e9, 3), unit="GB/s",
                cores=oracle.max_threads(), kind="oracle",
                sample=f"{reps} full steps (M=1,8,64 x fp8/int8/W4A16, quant + GEMM, K=2048 N=8192) "
                       f"in {dt:.1f} s")


# ----------------------------------------------------------------------------
def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}): this build measures the "
              "single-GPU kernel; multi-GPU sharding is a design note, not a measured path.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import gen
    import quantized_linear_layers_amd as q

    torch.cuda.set_device(0)
    t_start = time.time()
    if a.pmc_workload:
        pmc_workload(q, torch, a.pmc_workload)
        return
    cfg = gen.CONFIGS[2]
    d = gen.linear_config(2)
    N, K, Ms = d["N"], d["K"], cfg["M"]
    fmt_bytes = {f: weight_bytes(f, N, K) for f in ("fp8", "int8", "w4a16")}
    step_wb = sum(fmt_bytes.values()) * len(Ms)
    copies = max(8, int(math.ceil(1.0 * GIB / fmt_bytes["fp8"])))
    log(f"C2 decode layer N={N} K={K}, M={Ms}, weight copies={copies}")
    L = DecodeLayer(q, torch, d, copies)
    x = dev(d["a"], torch)
    bufs = make_bufs(torch, Ms, N, K)
    if a.pmc_pass:
        pmc_pass(q, torch, L, x, Ms, bufs)
        return
    step = run_step_fn(q, torch, L, x, Ms, bufs)

    # capture one graph per rotation slot (eager warm-up first)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):
            step(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graphs = []
    for c in range(copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(c)
        graphs.append(g)
    torch.cuda.synchronize()
    log(f"captured {len(graphs)} step graphs")

    for i in range(a.warmup):
        graphs[i % copies].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        graphs[(a.warmup + i) % copies].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / a.steps
    value = step_wb / (ms_per_step * 1e-3) / 1e9
    log(f"step {ms_per_step * 1e3:.1f} us -> {value:.1f} GB/s")

    # per-kernel rows of the step (event timed, eager launches behind a filler)
    rows = per_kernel_rows(q, torch, L, x, Ms, bufs, a.kernel_iters, "C2")
    rows.update(bf16_rows(torch, L, x, Ms, a.kernel_iters, "C2"))
    share = {}
    for k, r in rows.items():
        if k.startswith("C2_") and "weight_bytes" in r:
            share[k] = r["us"]
    dom = max(share, key=share.get)
    dr = rows[dom]
    fmt_dom = dom.split("_")[1]
    kname = {"fp8": "decode_gemm_kernel<FP8>", "int8": "decode_gemm_kernel<INT8>",
             "w4a16": "decode_gemm_kernel<W4A16>"}[fmt_dom]
    tab = traffic_table()
    traffic = None
    if tab and dom in tab.get("rows", {}):
        traffic = tab["rows"][dom]["hbm_bytes"]
    roofline = dict(bound="hbm", achieved=dr["GBps"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(dr["GBps"] / HBM_PEAK_GBS, 4), traffic=traffic,
                    kernel=f"{kname} M={dr['M']}", bytes_per_launch=dr["weight_bytes"],
                    launch_us=dr["us"],
                    traffic_note="HBM bytes per launch from FETCH_SIZE + WRITE_SIZE (rocprofv3 "
                                 "--pmc), calibrated on a 256 MiB copy; null when the counters "
                                 "were taken on other kernel sources")
    del graphs
    del L
    torch.cuda.empty_cache()

    if not a.no_extras:
        for name, fn in (("C3", c3_rows), ("C4", c4_rows), ("C5", c5_rows), ("V", vocab_rows)):
            tt = time.time()
            try:
                rows.update(fn(q, torch, gen, a.kernel_iters))
            except Exception as e:  # report, never hide
                rows[f"{name}_error"] = repr(e)
            log(f"{name} rows done in {time.time() - tt:.1f} s")

    cpu = None
    if not a.no_cpu:
        tt = time.time()
        cpu = cpu_baseline(gen, d, Ms, step_wb)
        log(f"cpu baseline done in {time.time() - tt:.1f} s")

    out = {
        "metric": "quantized GEMM weight GB/s (M<=64) and TFLOP/s (prefill) vs MI355X roofline",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8/int8/bf16",
        "data": "synthetic",
        "config": {"workload": "decode layer K=2048 N=8192 (seed 1), M in {1,8,64}: FP8 W8A8 and "
                               "int8 W8A8 each with per-token quantisation, W4A16 group-32; "
                               "weights rotated over %d copies (cold HBM), HIP-graph replay" % copies,
                   "K": K, "N": N, "M": list(Ms), "weight_bytes_per_step": step_wb},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "rows": rows,
        "wall_s": round(time.time() - t_start, 1),
    }
    _ = np
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
