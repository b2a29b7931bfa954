#!/usr/bin/env python3
"""Benchmark of the quantized linear layer on one MI355X.

One step = one pass of the per-call hot path over one batch at the large
dense decode layer K=5120, N=25600 (seed 2) for M in {1, 8, 64}:
  FP8 W8A8 : the FP8 linear (per-token FP8 quantisation of x[:M] + the
             row-scaled FP8 GEMM against per-channel E4M3 weights)
  W4A16    : the group-32 int4 GEMM with the unpack in the kernel
(3 linears + 3 W4A16 GEMMs). The weights rotate through enough copies
(>= 1 GiB per format) that every launch streams them from HBM, not from the
256 MB Infinity Cache; activations stay warm as in serving. Each step is a
captured HIP graph, replayed (launch overhead excluded, as in the pages'
GEMM micro-benchmark).

value = weight bytes streamed per step / step time  (GB/s)

Also reported in the same JSON line:
  roofline          the dominant GEMM kernel of the step: weight bytes per
                    launch over its mean launch time (HIP events on its
                    stream) against the 8 TB/s HBM peak, and its HBM bytes
                    per launch from the committed rocprofv3 counter summary;
  roofline_prefill  the FP8 linear (quantisation included) at the two
                    M=8192 prefill shapes, TFLOP/s against the FP8 MFMA peak;
  cpu_baseline      the CPU oracle running the same step on the host cores
                    (plus a 1-thread run, prefill and MoE samples);
  rows              per-kernel figures: the step's kernels, the K=2048 N=8192
                    decode layer (fp8, int8, W4A16), the prefill GEMMs, the MoE
                    blocks, the int4 vocabulary tables, the repacks and their
                    fidelity statistics.

Counter tools (rocprofv3 runs of committed code):
  --pmc-pass               decode GEMMs of both decode layers, eager launches
  --pmc-workload prefill|moe   the M=8192 GEMMs or the MoE blocks
  --summarize-pmc DIR ...  turn the counter CSVs of those runs into the
                           markdown summaries kept under profiles/
  --summarize-trace CSV    group a rocprofv3 --kernel-trace CSV by kernel
                           and grid
  --summarize-clock DIR ... shader clock per kernel (wave lifetime and
                           GRBM_GUI_ACTIVE) from the counter runs above
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
    ap.add_argument("--no-extras", action="store_true", help="skip the C1/C2/C4/C5/vocabulary rows")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--kernel-iters", type=int, default=64,
                    help="event-timed launches per kernel for the per-kernel rows")
    ap.add_argument("--pmc-workload", choices=("prefill", "moe"), default=None,
                    help="counter-collection workload for rocprofv3 --pmc: the M=8192 prefill "
                         "GEMMs (fp8, int8, W4A16, the fp8 linear, torch bf16) or the MoE blocks "
                         "(fp8, fp8 + SwiGLU-OAI, W4A16 at T = 64 and 512), 3 launches each, "
                         "then the 256 MiB copy that calibrates FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="counter-collection workload: every decode GEMM and quantisation of the "
                         "K=5120 N=25600 step and of the K=2048 N=8192 layer, 8 eager launches "
                         "each (weights rotating), then the 256 MiB calibration copy; run under "
                         "rocprofv3 --pmc")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR", default=None,
                    help="write the counter summary of rocprofv3 --pmc runs of one workload (one "
                         "directory per counter pass) to --pmc-out")
    ap.add_argument("--pmc-out", default=None, help="markdown file written by --summarize-pmc")
    ap.add_argument("--pmc-cmd", action="append", default=[],
                    help="the rocprofv3 command of each pass, quoted in the summary")
    ap.add_argument("--summarize-trace", metavar="CSV", default=None,
                    help="print the dispatches of a rocprofv3 --kernel-trace CSV grouped by kernel "
                         "and grid (count, average and minimum duration), largest total first")
    ap.add_argument("--trace-top", type=int, default=70, help="groups printed by --summarize-trace")
    ap.add_argument("--summarize-clock", nargs="+", metavar="DIR", default=None,
                    help="print the shader clock of each kernel (and grid) over its dispatches of at least "
                         "20 us, bracketed by wave lifetime and GRBM_GUI_ACTIVE, from rocprofv3 --pmc runs")
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


_GEN = {}


def cached_config(gen, kind, *args):
    """Generated inputs kept for the run: the GPU rows and the CPU baseline
    use the same draws without generating them twice."""
    key = (kind,) + args
    if key not in _GEN:
        _GEN[key] = {"prefill": gen.prefill_config, "moe": gen.moe_config}[kind](*args)
    return _GEN[key]


class Timer:
    """Per-launch device time with HIP events on the launching stream, after
    one untimed call. A queue filler keeps the device busy while the host
    enqueues, so each event pair brackets one call without host gaps."""

    def __init__(self, torch):
        self.torch = torch

    def time(self, fn, iters, filler_ms=30.0):
        torch = self.torch
        st = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        fn(0)  # one-time work (a workspace that grows) stays out of the timed launches
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
# decode layers and their per-call hot path
# ----------------------------------------------------------------------------
class DecodeLayer:
    """Weights of one layer in the requested formats, rotated over `copies`
    (FP8 and int8 per-channel repacks of the GPU's q4_0 repack)."""

    def __init__(self, q, torch, d, copies, fmts=("fp8", "int8", "w4a16")):
        self.q, self.torch = q, torch
        self.N, self.K = d["N"], d["K"]
        self.fmts = fmts
        w = dev(d["w_bf16"], torch)
        codes, steps, amb = q.repack_q4_0(w)
        torch.cuda.synchronize()
        self.n_ambiguous = int(amb.item())
        self.copies = copies
        self.fp8 = self.int8 = None
        if "fp8" in fmts:
            wq8, ws8 = q.repack_fp8(codes, steps)
            self.fp8 = [(wq8, ws8)] + [(wq8.clone(), ws8.clone()) for _ in range(copies - 1)]
        if "int8" in fmts:
            wi8, wsi8 = q.repack_int8(codes, steps)
            self.int8 = [(wi8, wsi8)] + [(wi8.clone(), wsi8.clone()) for _ in range(copies - 1)]
        self.w4 = [(codes, steps)] + [(codes.clone(), steps.clone()) for _ in range(copies - 1)]
        self.w_bf16 = w


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


def step_fn(q, L, x, Ms, bufs):
    """One step of the headline: for each M the FP8 linear (quantisation +
    GEMM) and the W4A16 GEMM, on weight copy i % copies."""
    def step(i):
        c = i % L.copies
        for M in Ms:
            b = bufs[M]
            xm = x[:M]
            q.linear_fp8(xm, *L.fp8[c], out=b["y8"])
            q.gemm_w4a16(xm, *L.w4[c], out=b["y4"])
    return step


def gemm_calls(q, L, x, Ms, bufs):
    """(row suffix, M, kind, call(i)) for every decode GEMM of the layer's
    formats and the per-token quantisations (operands prepared here)."""
    out = []
    for M in Ms:
        b = bufs[M]
        xm = x[:M]
        if L.fp8 is not None:
            q.quant_act(xm, "e4m3", out=(b["aq8"], b["sa8"]))
            out += [(f"fp8_M{M}", M, "fp8",
                     lambda i, b=b: q.gemm_fp8(b["aq8"], b["sa8"], *L.fp8[i % L.copies], out=b["y8"])),
                    (f"quant_fp8_M{M}", M, "quant",
                     lambda i, xm=xm, b=b: q.quant_act(xm, "e4m3", out=(b["aq8"], b["sa8"])))]
        if L.int8 is not None:
            q.quant_act(xm, "int8", out=(b["aqi"], b["sai"]))
            out += [(f"int8_M{M}", M, "int8",
                     lambda i, b=b: q.gemm_w8a8(b["aqi"], b["sai"], *L.int8[i % L.copies], out=b["yi"]))]
        out += [(f"w4a16_M{M}", M, "w4a16",
                 lambda i, xm=xm, b=b: q.gemm_w4a16(xm, *L.w4[i % L.copies], out=b["y4"]))]
    return out


def per_kernel_rows(q, torch, L, x, Ms, bufs, iters, tag):
    """Per-launch device time of each GEMM and quantisation of the layer
    (graph-timed, see GraphTimer), weight GB/s and the fraction of the HBM
    peak; plus the FP8 linear (quantisation + GEMM) per M."""
    T = GraphTimer(torch)
    rows = {}
    for name, M, kind, fn in gemm_calls(q, L, x, Ms, bufs):
        t = T.time(fn, reps=min(32, max(8, iters // 2)))
        r = dict(M=M, us=round(t["mean_us"], 3), min_us=round(t["min_us"], 3))
        if kind != "quant":
            wb = weight_bytes(kind, L.N, L.K)
            r["weight_bytes"] = wb
            r["GBps"] = round(wb / (t["mean_us"] * 1e3), 1)
            r["frac_hbm"] = round(r["GBps"] / HBM_PEAK_GBS, 4)
        rows[f"{tag}_{name}"] = r
    if L.fp8 is not None:
        for M in Ms:
            b = bufs[M]
            t = T.time(lambda i, xm=x[:M], b=b: q.linear_fp8(xm, *L.fp8[i % L.copies], out=b["y8"]),
                       reps=min(32, max(8, iters // 2)))
            wb = weight_bytes("fp8", L.N, L.K)
            rows[f"{tag}_fp8_linear_M{M}"] = dict(M=M, us=round(t["mean_us"], 3), weight_bytes=wb,
                                                  GBps=round(wb / (t["mean_us"] * 1e3), 1),
                                                  frac_hbm=round(wb / (t["mean_us"] * 1e3) / HBM_PEAK_GBS, 4))
    return rows


def bf16_rows(torch, L, x, Ms, iters, tag):
    """torch's bf16 GEMM on the materialised weights (the comparator): the
    faster of x @ W^T and (W @ x^T)^T, graph-timed like the other rows."""
    T = GraphTimer(torch)
    ws = [L.w_bf16] + [L.w_bf16.clone() for _ in range(max(3, int(math.ceil(1.5 * GIB / (2 * L.N * L.K)))) - 1)]
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
# repack rows: fidelity statistics and conversion checks (GPU results, fp64
# statistics with torch on the device)
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


def fnuz_ocp_value_equal(torch, wf, sf, wo, so, rows_per=4096):
    """Every converted element keeps its value: dec_ocp(b') * s' ==
    dec_fnuz(b) * s in fp64 (both decodes and products exact)."""
    for n0 in range(0, wf.shape[0], rows_per):
        a = wf[n0:n0 + rows_per].view(torch.float8_e4m3fnuz).to(torch.float64) * \
            sf[n0:n0 + rows_per, None].to(torch.float64)
        b = wo[n0:n0 + rows_per].view(torch.float8_e4m3fn).to(torch.float64) * \
            so[n0:n0 + rows_per, None].to(torch.float64)
        if not torch.equal(a, b):
            return False
    return True


def repack_rows(q, torch, gen, L):
    """The offline repacks on the K=5120 N=25600 layer (times, fidelity of
    the FP8 repack in both formats, the FNUZ -> OCP copy with its inexact
    count and value check), the FP8 repack fidelity at the single-layer
    size (M=4 K=256 N=512), and the q4_0 repack of a grid whose steps are
    not bf16 values (share of unpacked values bit-identical to the stored
    ones, the E2B article's 90.0 % statistic)."""
    rows = {}
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
                                  every_value_preserved=fnuz_ocp_value_equal(torch, wf, sf, wo, so))
    del wf, wo
    # single layer M=4 K=256 N=512 (seed 0)
    d = gen.linear_config(1)
    c1, s1, _ = q.repack_q4_0(dev(d["w_bf16"], torch))
    rows["C1_repack_fp8"] = {}
    for fmt in ("e4m3", "e4m3fnuz"):
        wq_, ws_ = q.repack_fp8(c1, s1, fmt)
        rr, mr = repack_fidelity(torch, c1, s1, wq_, ws_, fmt)
        rows["C1_repack_fp8"][f"rel_rms_{fmt}"] = round(rr, 6)
        rows["C1_repack_fp8"][f"max_err_over_row_max_{fmt}"] = round(mr, 6)
    # fp32 (not bf16) trained steps, K=2048 N=8192 layer drawn with seed 1
    d = gen.linear_config(2, bf16_steps=False)
    wr = dev(d["w_bf16"], torch)
    cr, sr, ar = q.repack_q4_0(wr)
    back = q.dequant_q4_bf16(cr, sr)
    same = float((back.view(torch.int16) == wr.view(torch.int16)).double().mean())
    rows["C2_unrounded_steps_repack_q4_0"] = dict(frac_bit_identical=round(same, 6),
                                                  n_ambiguous=int(ar.item()),
                                                  groups=d["N"] * d["K"] // 32)
    del wr, cr, sr, back
    torch.cuda.empty_cache()
    return rows


def c2_rows(q, torch, gen, iters):
    """The K=2048 N=8192 decode layer (seed 1): fp8, int8 and W4A16 GEMMs,
    the quantisations and the FP8 linear at M = 1, 8, 64, torch bf16 beside."""
    d = gen.linear_config(2)
    copies = max(8, int(math.ceil(1.0 * GIB / weight_bytes("fp8", d["N"], d["K"]))))
    L = DecodeLayer(q, torch, d, copies)
    x = dev(d["a"], torch)
    Ms = (1, 8, 64)
    bufs = make_bufs(torch, Ms, L.N, L.K)
    rows = per_kernel_rows(q, torch, L, x, Ms, bufs, iters, "C2")
    rows.update(bf16_rows(torch, L, x, Ms, iters, "C2"))
    del L
    torch.cuda.empty_cache()
    return rows


def c4_rows(q, torch, gen, iters):
    """M=8192 prefill GEMMs at (K=4096, N=14336) and (K=14336, N=4096):
    fp8, int8 and W4A16 GEMMs, the FP8 linear (quantisation included, the
    timed call) and torch's bf16 matmul on the same weights. Returns (rows,
    roofline objects of the FP8 linear)."""
    rows, roof = {}, []
    T = Timer(torch)
    for which in (0, 1):
        d = cached_config(gen, "prefill", which)
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
        # the quantizer alone: graph-replayed launches over enough copies of
        # x (>= 512 MB) that every launch reads it from HBM
        xs = [x] + [x.clone() for _ in range(max(1, math.ceil((512 << 20) / (2 * M * K))) - 1)]
        t_q = GraphTimer(torch).time(lambda i: q.quant_act(xs[i % len(xs)], "e4m3", out=(aq8, sa8)), reps=16)
        del xs
        t_g8 = T.time(lambda i: q.gemm_fp8(aq8, sa8, wq8, ws8, out=y), n_it, filler_ms=5)
        t_lin = T.time(lambda i: q.linear_fp8(x, wq8, ws8, out=y), n_it, filler_ms=5)
        t_gi = T.time(lambda i: q.gemm_w8a8(aqi, sai, wi8, wsi8, out=y), n_it, filler_ms=5)
        t_li = T.time(lambda i: q.linear_w8a8(x, wi8, wsi8, out=y), n_it, filler_ms=5)
        t_w4 = T.time(lambda i: q.gemm_w4a16(x, codes, steps, out=y), n_it, filler_ms=5)
        t_bf = T.time(lambda i: torch.matmul(x, w.t(), out=y), n_it, filler_ms=5)
        tag = f"C4_K{K}_N{N}"
        for name, t, peak in (("fp8_gemm", t_g8, "fp8"), ("int8_gemm", t_gi, "int8"),
                              ("fp8_linear_incl_quant", t_lin, "fp8"),
                              ("int8_linear_incl_quant", t_li, "int8"),
                              ("w4a16_gemm", t_w4, "bf16"), ("bf16_torch", t_bf, "bf16")):
            tf = flops / (t["mean_us"] * 1e-6) / 1e12
            rows[f"{tag}_{name}"] = dict(us=round(t["mean_us"], 1), TFLOPs=round(tf, 1),
                                         frac_mfma=round(tf / MFMA_PEAK_TFLOPS[peak], 4))
        rows[f"{tag}_quant_fp8"] = dict(us=round(t_q["mean_us"], 1),
                                        GBps=round((M * K * 3 + 4 * M) / (t_q["mean_us"] * 1e3), 1))
        tf = flops / (t_lin["mean_us"] * 1e-6) / 1e12
        roof.append(dict(bound="mfma", achieved=round(tf, 1), peak=MFMA_PEAK_TFLOPS["fp8"],
                         unit="TFLOP/s", frac=round(tf / MFMA_PEAK_TFLOPS["fp8"], 4), traffic=None,
                         kernel=f"qlin_linear_fp8 M={M} K={K} N={N} (per-token quantisation + FP8 GEMM)",
                         flops_per_launch=flops, launch_us=round(t_lin["mean_us"], 1), M=M, K=K, N=N))
        del wq8, wi8, x, aq8, aqi, y, w, codes, steps
        torch.cuda.empty_cache()
    return rows, roof


def c5_rows(q, torch, gen, iters):
    rows = {}
    d = cached_config(gen, "moe")
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
# hardware-counter workloads (run under rocprofv3 --pmc) and their summary
# ----------------------------------------------------------------------------
CSRC = os.path.join(ROOT, "quantized_linear_layers_amd", "csrc")
DECODE_SOURCES = ("qlin_gemm_decode.hip", "qlin_gemm_w4_decode.hip", "qlin_skinny.h", "qlin_device.h",
                  "qlin_quant.hip", "qlin_quant_row.h", "qlin_abi.hip")
PREFILL_SOURCES = ("qlin_gemm_prefill.hip", "qlin_device.h", "qlin_quant.hip", "qlin_quant_row.h", "qlin_abi.hip")
MOE_SOURCES = ("qlin_moe.hip", "qlin_skinny.h", "qlin_device.h", "qlin_quant.hip", "qlin_quant_row.h")
PMC_SOURCES = {"decode": DECODE_SOURCES, "prefill": PREFILL_SOURCES, "moe": MOE_SOURCES}
TRAFFIC_MD = {"decode": os.path.join(ROOT, "profiles", "decode_gemms_K5120_N25600_K2048_N8192_pmc_counters.md"),
              "prefill": os.path.join(ROOT, "profiles", "prefill_gemms_M8192_pmc_counters.md"),
              "moe": os.path.join(ROOT, "profiles", "moe_blocks_E128_H2048_I768_pmc_counters.md")}
COPY_BYTES = 256 << 20
# kernels the library launches per call (the counter summary assigns
# dispatches to calls by these counts)
LINEAR_KERNELS = 2       # per-token quantisation, GEMM
MOE_FP8_KERNELS = 5      # quantisation with routing, gate_up, requantisation, down, combine
MOE_W4A16_KERNELS = 4    # routing, gate_up, down, combine


def sources_sha256(which):
    import hashlib

    h = hashlib.sha256()
    for f in PMC_SOURCES[which]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _pmc_marker(q, torch):
    """One launch of the element-wise FP8 encoder (used nowhere else in the
    counter workloads): the summary starts reading dispatches after it."""
    q.fp8_encode_f32(torch.zeros(64, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()


def _pmc_copy(torch):
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()


def _pmc_plan(which, plan, launches):
    print(json.dumps({"pmc_plan": which, "rows": plan, "launches": launches, "copy_bytes": COPY_BYTES,
                      "copies": 4, "sources_sha256": sources_sha256(which)}), flush=True)
    os.makedirs(os.path.join(ROOT, "gpurun_out"), exist_ok=True)
    with open(os.path.join(ROOT, "gpurun_out", f"pmc_plan_{which}.json"), "w") as fh:
        json.dump({"rows": plan, "launches": launches, "copy_bytes": COPY_BYTES, "copies": 4,
                   "sources_sha256": sources_sha256(which)}, fh)


def pmc_pass(q, torch, gen, launches=8):
    """Decode counter workload: every GEMM and quantisation of the K=5120
    N=25600 step and of the K=2048 N=8192 layer (weights rotating over
    copies, so they come from HBM), `launches` eager launches each, then the
    256 MiB calibration copy four times."""
    plan = []
    for cfg, tag, fmts in ((3, "C3", ("fp8", "w4a16")), (2, "C2", ("fp8", "int8", "w4a16"))):
        d = gen.linear_config(cfg)
        copies = max(4, int(math.ceil(1.0 * GIB / weight_bytes("fp8", d["N"], d["K"]))))
        L = DecodeLayer(q, torch, d, copies, fmts)
        x = dev(d["a"], torch)
        Ms = (1, 8, 64)
        bufs = make_bufs(torch, Ms, L.N, L.K)
        calls = gemm_calls(q, L, x, Ms, bufs)
        for name, M, kind, fn in calls:
            fn(launches)  # warm-up: workspaces exist before the marker
            _pmc_marker(q, torch)
            for i in range(launches):
                fn(i)
            torch.cuda.synchronize()
            plan.append([f"{tag}_{name}", 1, weight_bytes(kind, L.N, L.K) if kind != "quant" else 0])
        del L, bufs, calls
        torch.cuda.empty_cache()
    _pmc_marker(q, torch)
    _pmc_copy(torch)
    _pmc_plan("decode", plan, launches)


def pmc_workload(q, torch, which, launches=3):
    """Counter workloads beyond the decode step: synthetic operands of the
    M=8192 prefill shapes or the MoE block built on the device (uniform
    random codes, bf16 steps in [0.001, 0.021], N(0,1) activations, N(0,
    0.02) bf16 weights quantised per channel), each call launched `launches`
    times in a fixed order, then the calibration copy."""
    torch.manual_seed(0)
    plan = []

    def rep(name, kpc, fn):
        fn()  # warm-up: workspaces exist before the marker
        _pmc_marker(q, torch)
        for _ in range(launches):
            fn()
        torch.cuda.synchronize()
        plan.append([name, kpc, 0])

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
            y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            q.linear_fp8(a, wq, ws, out=y)  # workspace allocated before the marker
            q.linear_w8a8(a, wi, wsi, out=y)
            tag = f"C4_K{K}_N{N}"
            lin_k = LINEAR_KERNELS
            rep(f"{tag}_fp8_gemm", 1, lambda: q.gemm_fp8(aq, sa, wq, ws, out=y))
            rep(f"{tag}_int8_gemm", 1, lambda: q.gemm_w8a8(ai, sai, wi, wsi, out=y))
            rep(f"{tag}_fp8_linear", lin_k, lambda: q.linear_fp8(a, wq, ws, out=y))
            rep(f"{tag}_quant_fp8", 1, lambda: q.quant_act(a, "e4m3", out=(aq, sa)))
            rep(f"{tag}_w4a16_gemm", 1, lambda: q.gemm_w4a16(a, codes, steps, out=y))
            rep(f"{tag}_bf16_torch", 1, lambda: torch.matmul(a, w.t(), out=y))
            del a, w, aq, ai, wq, wi, codes, steps, y
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
            q.moe_fp8(x, ids, pr, *fp8w)  # scratch allocated before the marker
            q.moe_w4a16(x, ids, pr, *w4)
            rep(f"C5_moe_fp8_T{T}", MOE_FP8_KERNELS, lambda: q.moe_fp8(x, ids, pr, *fp8w))
            rep(f"C5_moe_fp8_swiglu_oai_T{T}", MOE_FP8_KERNELS,
                lambda: q.moe_fp8(x, ids, pr, *fp8w, swiglu_oai=(1.702, 1.0, 7.0)))
            rep(f"C5_moe_w4a16_T{T}", MOE_W4A16_KERNELS, lambda: q.moe_w4a16(x, ids, pr, *w4))
    _pmc_marker(q, torch)
    _pmc_copy(torch)
    _pmc_plan(which, plan, launches)


def _read_dispatches(d):
    """Dispatches of one rocprofv3 --pmc run directory, in dispatch order:
    [{'id', 'kernel', 'grid', 'wg', 'vgpr', 'lds', 'ns', 'ctr': {name: value}}]."""
    import csv
    import glob

    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {d}")
    disp = {}
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                key = (f, int(r["Dispatch_Id"]))
                e = disp.get(key)
                if e is None:
                    e = disp[key] = dict(id=key, kernel=r.get("Kernel_Name", ""),
                                         grid=r.get("Grid_Size", ""), wg=r.get("Workgroup_Size", ""),
                                         vgpr=r.get("VGPR_Count", r.get("Arch_VGPR_Count", "")),
                                         lds=r.get("LDS_Block_Size", ""),
                                         ns=int(r.get("End_Timestamp", 0)) - int(r.get("Start_Timestamp", 0)),
                                         ctr={})
                n = r["Counter_Name"]
                e["ctr"][n] = e["ctr"].get(n, 0.0) + float(r["Counter_Value"])
    return [disp[k] for k in sorted(disp)]


def _short(kernel):
    k = kernel
    if k.startswith("void "):
        k = k[5:]
    k = k.split("(")[0]
    return k.replace("qlin::", "")


def summarize_clock(dirs, min_us=20.0):
    """Shader clock per kernel and grid, bracketed by two counter ratios
    over dispatches of at least `min_us` (median per group):
    * wave lifetime / duration (4 x SQ_WAVE_CYCLES / SQ_WAVES, quad-cycles,
      over the dispatch time): a lower bound, close to the clock for kernels
      whose waves all live the whole dispatch (one round of workgroups:
      the decode GEMMs at these shapes, the persistent prefill kernels);
    * GRBM_GUI_ACTIVE / 8 / duration: GPU clock cycles of each of the 8
      XCDs (the counter summed over their instances, so a 3.3 ms
      memory-bound kernel reads 2.31 GHz); the counter window is longer
      than the kernel by about 16 k cycles per XCD (a 25 us repack reads
      2.95 GHz against 2.33 at 128 us), an upper bound that is tight only
      for long dispatches."""
    import collections
    import statistics

    for d in dirs:
        g = collections.defaultdict(list)
        for e in _read_dispatches(d):
            c = e["ctr"]
            if "GRBM_GUI_ACTIVE" in c and c.get("SQ_WAVES") and e["ns"] >= min_us * 1e3:
                life = 4.0 * c["SQ_WAVE_CYCLES"] / c["SQ_WAVES"]
                g[(_short(e["kernel"]), e["grid"])].append((e["ns"], life / e["ns"], c["GRBM_GUI_ACTIVE"] / e["ns"] / 8))
        print(f"{d}: kernel, grid (work-items), dispatches, median us, GHz from wave lifetime (lower "
              f"bound), GHz from GRBM_GUI_ACTIVE (upper bound)")
        for (k, grid), v in sorted(g.items(), key=lambda kv: -statistics.median(x[0] for x in kv[1])):
            print(f"  {k[:64]:64s} {grid:>9s} {len(v):4d} {statistics.median(x[0] for x in v) / 1e3:9.1f} "
                  f"{statistics.median(x[1] for x in v):6.2f} {statistics.median(x[2] for x in v):6.2f}")


def summarize_trace(csv_path, top):
    """Group the dispatches of a kernel-trace CSV by kernel (name without
    namespace and argument list) and grid in workgroups; one line per group,
    largest total duration first."""
    import csv
    import collections

    def short(name):
        name = name.replace("qlin::", "")
        depth = 0
        for i, ch in enumerate(name):
            if ch == "<":
                depth += 1
            elif ch == ">":
                depth -= 1
            elif ch == "(" and depth == 0:
                return name[:i][:60]
        return name[:60]

    groups = collections.defaultdict(list)
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            wx = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
            wy = int(r["Grid_Size_Y"]) // max(1, int(r["Workgroup_Size_Y"]))
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            groups[(short(r["Kernel_Name"]), wx, wy)].append(us)
    items = sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:top]
    for (name, wx, wy), d in items:
        print(f"{name:60s} grid=({wx},{wy}) n={len(d):5d} avg={sum(d) / len(d):10.2f}us min={min(d):10.2f}us")


def summarize_pmc(dirs, out_md, cmds):
    """Counter summary of one workload: a row's `launches` calls follow its
    marker dispatch (then the next row's warm-up call and the next marker);
    the kernels per call are the planned count when the dispatch names
    repeat with that period, else the shortest period they repeat with (a
    call's kernel count can depend on the shape); per row and
    kernel the median dispatch is kept. FETCH_SIZE / WRITE_SIZE are scaled
    by what they read for the 256 MiB copy (known bytes)."""
    import statistics

    plan_path = None
    for d in dirs:
        for root, _, files in os.walk(d):
            for f in files:
                if f.startswith("pmc_plan_") and f.endswith(".json"):
                    plan_path = os.path.join(root, f)
    which = None
    if plan_path is None:
        for w in ("decode", "prefill", "moe"):
            p = os.path.join(ROOT, "gpurun_out", f"pmc_plan_{w}.json")
            if os.path.exists(p) and w in out_md:
                plan_path = p
    if plan_path is None:
        raise FileNotFoundError("no pmc_plan_*.json (written by the counter workload)")
    which = os.path.basename(plan_path)[len("pmc_plan_"):-5]
    plan = json.load(open(plan_path))
    rows = {}
    copy_ctr = {}
    for d in dirs:
        try:
            ds = _read_dispatches(d)
        except FileNotFoundError:
            continue  # a directory holding only the plan
        marks = [i for i, e in enumerate(ds) if "fp8_encode" in e["kernel"]]
        if len(marks) < len(plan["rows"]) + 1:
            raise ValueError(f"{d}: {len(marks)} marker dispatches for {len(plan['rows'])} rows")
        for ri, ((name, kpc_plan, wbytes), m) in enumerate(zip(plan["rows"], marks)):
            names = [_short(e["kernel"]) for e in ds[m + 1:marks[ri + 1]]]
            L = plan["launches"]

            def periodic(p):
                return 0 < L * p <= len(names) and all(names[j] == names[j % p] for j in range(L * p))
            kpc = kpc_plan if periodic(kpc_plan) else next((p for p in range(1, len(names) // L + 1)
                                                            if periodic(p)), None)
            if kpc is None:
                raise ValueError(f"{d}: row {name}: no {L} repeated calls after the marker")
            if kpc != kpc_plan:
                print(f"{d}: row {name}: {kpc} kernels per call (planned {kpc_plan})", file=sys.stderr)
            seq = ds[m + 1:m + 1 + kpc * L]
            r = rows.setdefault(name, dict(weight_bytes=wbytes, kernels={}))
            for j in range(kpc):
                calls = seq[j::kpc]
                kn = _short(calls[0]["kernel"])
                kr = r["kernels"].setdefault(f"{j}:{kn}", dict(kernel=kn, grid=calls[0]["grid"],
                                                              wg=calls[0]["wg"], vgpr=calls[0]["vgpr"],
                                                              lds=calls[0]["lds"], ctr={}, us=[]))
                for c in calls:
                    for n, v in c["ctr"].items():
                        kr["ctr"].setdefault(n, []).append(v)
                    kr["us"].append(c["ns"] / 1e3)
        copies = [e for e in ds[marks[-1] + 1:] if "fp8_encode" not in e["kernel"]][-plan["copies"]:]
        for c in copies:
            for n, v in c["ctr"].items():
                copy_ctr.setdefault(n, []).append(v)
    med = {n: statistics.median(v) for n, v in copy_ctr.items()}
    kib = COPY_BYTES / 1024
    ff = kib / med["FETCH_SIZE"] if med.get("FETCH_SIZE") else None
    wf = kib / med["WRITE_SIZE"] if med.get("WRITE_SIZE") else None
    table = dict(sources_sha256=plan["sources_sha256"], copy_bytes=COPY_BYTES,
                 copy_fetch_kib=med.get("FETCH_SIZE"), copy_write_kib=med.get("WRITE_SIZE"),
                 fetch_factor=ff, write_factor=wf, rows={})
    lines = []
    cols = ["row", "kernel", "grid", "VGPR", "us", "FETCH KiB", "WRITE KiB", "HBM bytes", "HBM / weight",
            "VALU share", "LDS share", "wait share", "MFMA busy", "VALU / MFMA", "L2 hit"]
    lines.append("| " + " | ".join(cols) + " |")
    lines.append("|" + "---|" * len(cols))
    for name, r in rows.items():
        trow = dict(kernels=[])
        tot_hbm = 0.0
        have_hbm = ff is not None and wf is not None
        for key, kr in r["kernels"].items():
            c = {n: statistics.median(v) for n, v in kr["ctr"].items()}
            us = statistics.median(kr["us"])
            hbm = (c["FETCH_SIZE"] * ff + c["WRITE_SIZE"] * wf) * 1024 if have_hbm and \
                "FETCH_SIZE" in c and "WRITE_SIZE" in c else None
            if hbm is not None:
                tot_hbm += hbm

            def ratio(a, b):
                return round(c[a] / c[b], 3) if a in c and b in c and c[b] else None

            mfma_busy = None
            if c.get("SQ_VALU_MFMA_BUSY_CYCLES") and c.get("SQ_WAVE_CYCLES") and c.get("SQ_WAVES"):
                # SQ_WAVE_CYCLES counts quad-cycles: one wave's lifetime in cycles
                life = 4.0 * c["SQ_WAVE_CYCLES"] / c["SQ_WAVES"]
                mfma_busy = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * life), 3)
            l2 = None
            if "TCC_HIT_sum" in c and "TCC_MISS_sum" in c and (c["TCC_HIT_sum"] + c["TCC_MISS_sum"]):
                l2 = round(c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"]), 3)
            k = dict(kernel=kr["kernel"], grid=kr["grid"], wg=kr["wg"], vgpr=kr["vgpr"], us=round(us, 2),
                     fetch_kib=c.get("FETCH_SIZE"), write_kib=c.get("WRITE_SIZE"),
                     hbm_bytes=round(hbm) if hbm is not None else None,
                     valu_share=ratio("SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES"),
                     lds_share=ratio("SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES"),
                     wait_share=ratio("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
                     mfma_busy=mfma_busy, valu_per_mfma=ratio("SQ_INSTS_VALU", "SQ_INSTS_MFMA"), l2_hit=l2)
            trow["kernels"].append(k)

            def f(v):
                if v is None:
                    return "-"
                if isinstance(v, float):
                    return f"{v:.3f}" if abs(v) < 10 else f"{v:.1f}"
                return str(v)

            lines.append("| " + " | ".join([
                name, k["kernel"], str(k["grid"]), str(k["vgpr"]), f(k["us"]), f(k["fetch_kib"]),
                f(k["write_kib"]), f(k["hbm_bytes"]),
                f(round(hbm / r["weight_bytes"], 2)) if hbm is not None and r["weight_bytes"] else "-",
                f(k["valu_share"]), f(k["lds_share"]), f(k["wait_share"]), f(k["mfma_busy"]),
                f(k["valu_per_mfma"]), f(k["l2_hit"])]) + " |")
        if tot_hbm:
            trow["hbm_bytes"] = round(tot_hbm)
        trow["weight_bytes"] = r["weight_bytes"]
        table["rows"][name] = trow
    title = {"decode": "Decode GEMMs (K=5120 N=25600 and K=2048 N=8192, M = 1, 8, 64)",
             "prefill": "Prefill GEMMs at M=8192 (K=4096 N=14336 and K=14336 N=4096)",
             "moe": "MoE blocks (E=128, H=2048, I=768, top-8, T = 64 and 512)"}[which]
    with open(out_md, "w") as fh:
        fh.write(f"# {title}: rocprofv3 counters\n\n")
        fh.write("Commands (from the repository root, on one MI355X; one counter set per pass), then the "
                 "summary:\n\n")
        for c in cmds:
            fh.write(f"    {c}\n")
        fh.write(f"    python bench.py --summarize-pmc {' '.join(dirs)} --pmc-out "
                 f"{os.path.relpath(out_md, ROOT)}\n\n")
        fh.write(
            "Each row is one call launched `launches` times after a marker dispatch (weights rotating over "
            "copies in the decode workload); per kernel the median dispatch is shown. Durations are those of "
            "the counter runs (serialised dispatches). HBM bytes = FETCH_SIZE x fetch_factor + WRITE_SIZE x "
            "write_factor (KiB x 1024), the factors being what the counters read for a 256 MiB device copy "
            "(known bytes). Shares are of SQ_WAVE_CYCLES: VALU / LDS = cycles with such an instruction "
            "active, wait = cycles waiting on an instruction's operands; MFMA busy = "
            "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x one wave's lifetime, 4 x SQ_WAVE_CYCLES / SQ_WAVES, "
            "SQ_WAVE_CYCLES counting quad-cycles): the busy share of the MFMA pipes for the persistent "
            "kernels with one wave per SIMD (prefill_*, hipBLASLt), a lower bound elsewhere; VALU / MFMA "
            "counts instructions; "
            "L2 hit = TCC hits / (hits + misses). `-`: the counter was not in the passes given.\n\n")
        fh.write("\n".join(lines) + "\n\n")
        fh.write("Machine-readable table (bench.py reads `hbm_bytes` per row; `sources_sha256` hashes the "
                 "kernel sources the counters were taken on, and bench.py reports no traffic when the "
                 "current sources differ):\n\n```json\n")
        fh.write(json.dumps(table, indent=1))
        fh.write("\n```\n")
    print(f"wrote {out_md}: {len(rows)} rows", flush=True)


def traffic_table(which):
    """Per-launch HBM bytes per row from the committed counter summary of a
    workload, if it was taken on the current kernel sources (else None: the
    counters no longer describe this code)."""
    try:
        with open(TRAFFIC_MD[which]) as fh:
            txt = fh.read()
        blob = txt[txt.index("```json") + 7:]
        blob = blob[:blob.index("```")]
        tab = json.loads(blob)
    except (OSError, ValueError):
        return None
    if tab.get("sources_sha256") != sources_sha256(which):
        return None
    return tab


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on the host cores
# ----------------------------------------------------------------------------
def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(gen, d, Ms, step_wb, budget_s=12.0):
    """The oracle (as it stands) on the headline step, on every host thread
    it gets, repeated for about budget_s; beside it a 1-thread run of the
    same step on the first 1600 of the 25600 output channels, one FP8 linear
    at K=4096 N=14336 on 16 of the 8192 rows, and the FP8 MoE block at T=64
    (median of 3)."""
    import statistics

    import numpy as np

    import oracle

    p, s, _ = oracle.repack_q4_0(d["w_bf16"])
    K, N = d["K"], d["N"]
    wq8, ws8 = oracle.repack_fp8(p, s, K, oracle.OCP)

    def step(wq, ws, pp, ss):
        for M in Ms:
            a = d["a"][:M]
            aq, sa = oracle.quant_act(a, oracle.OCP)
            oracle.gemm_fp8(aq, sa, wq, ws)
            oracle.gemm_w4a16(a, pp, ss)

    threads = oracle.max_threads()
    t0 = time.perf_counter()
    step(wq8, ws8, p, s)
    reps = 1
    while time.perf_counter() - t0 < budget_s and reps < 1000:
        step(wq8, ws8, p, s)
        reps += 1
    dt = time.perf_counter() - t0
    value = step_wb * reps / dt / 1e9
    # one thread, 1/16 of the output channels
    n1 = N // 16
    sub = (np.ascontiguousarray(wq8[:n1]), np.ascontiguousarray(ws8[:n1]), np.ascontiguousarray(p[:n1]),
           np.ascontiguousarray(s[:n1]))
    oracle.set_threads(1)
    t1 = time.perf_counter()
    step(*sub)
    dt1 = time.perf_counter() - t1
    oracle.set_threads(threads)
    one = step_wb / 16 / dt1 / 1e9
    # prefill: FP8 linear at K=4096 N=14336 on 16 rows
    dp = cached_config(gen, "prefill", 0)
    pp, sp, _ = oracle.repack_q4_0(dp["w_bf16"])
    wqp, wsp = oracle.repack_fp8(pp, sp, dp["K"], oracle.OCP)
    a16 = np.ascontiguousarray(dp["a"][:16])
    t2 = time.perf_counter()
    aq, sa = oracle.quant_act(a16, oracle.OCP)
    oracle.gemm_fp8(aq, sa, wqp, wsp)
    dt2 = time.perf_counter() - t2
    pre_tf = 2.0 * 16 * dp["N"] * dp["K"] / dt2 / 1e12
    # MoE T=64 (the leading 64 tokens of the T=512 draw)
    dm = dict(cached_config(gen, "moe"))
    dm.update(x=dm["x"][:64], ids=dm["ids"][:64], probs=dm["probs"][:64])
    E = dm["E"]
    w13 = np.empty((E, 2 * dm["I"], dm["H"]), np.uint8)
    s13 = np.empty((E, 2 * dm["I"]), np.float32)
    w2 = np.empty((E, dm["H"], dm["I"]), np.uint8)
    s2 = np.empty((E, dm["H"]), np.float32)
    for e in range(E):
        pe, se, _ = oracle.repack_q4_0(dm["w13_bf16"][e])
        w13[e], s13[e] = oracle.repack_fp8(pe, se, dm["H"], oracle.OCP)
        pe, se, _ = oracle.repack_q4_0(dm["w2_bf16"][e])
        w2[e], s2[e] = oracle.repack_fp8(pe, se, dm["I"], oracle.OCP)
    tm = []
    for _ in range(3):
        t3 = time.perf_counter()
        oracle.moe_fp8(dm["x"], dm["ids"], dm["probs"], w13, s13, w2, s2)
        tm.append(time.perf_counter() - t3)
    touched = len(set(dm["ids"].ravel().tolist()))
    moe_wb = touched * (2 * dm["I"] * dm["H"] + 8 * dm["I"] + dm["H"] * dm["I"] + 4 * dm["H"])
    moe_t = statistics.median(tm)
    return dict(value=round(value, 3), unit="GB/s", cores=threads, kind="oracle",
                sample=f"{reps} full steps (M = 1, 8, 64: FP8 quantisation + GEMM and W4A16 GEMM, "
                       f"K={K} N={N}) in {dt:.1f} s on {threads} threads",
                host=dict(nproc=os.cpu_count(), cpu_model=_cpu_model()),
                one_thread=dict(value=round(one, 4), unit="GB/s", cores=1,
                                sample=f"the same step on output channels 0..{n1 - 1}, {dt1:.1f} s"),
                prefill_fp8_linear=dict(value=round(pre_tf, 5), unit="TFLOP/s", cores=threads,
                                        sample=f"quantisation + FP8 GEMM, K=4096 N=14336, 16 of the 8192 "
                                               f"rows, one run, {dt2:.2f} s"),
                moe_fp8_T64=dict(value=round(moe_wb / moe_t / 1e9, 3), unit="GB/s", cores=threads,
                                 sample=f"FP8 MoE block, T=64, E=128 top-8, median of 3 runs "
                                        f"({moe_t * 1e3:.0f} ms)"))


# ----------------------------------------------------------------------------
def main():
    a = parse()
    if a.summarize_pmc:
        summarize_pmc(a.summarize_pmc, a.pmc_out, a.pmc_cmd)
        return
    if a.summarize_trace:
        summarize_trace(a.summarize_trace, a.trace_top)
        return
    if a.summarize_clock:
        summarize_clock(a.summarize_clock)
        return
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
    if a.pmc_pass:
        pmc_pass(q, torch, gen)
        return
    cfg = gen.CONFIGS[3]
    d = gen.linear_config(3)
    N, K, Ms = d["N"], d["K"], cfg["M"]
    fmt_bytes = {f: weight_bytes(f, N, K) for f in ("fp8", "w4a16")}
    step_wb = sum(fmt_bytes.values()) * len(Ms)
    copies = max(4, int(math.ceil(1.02 * GIB / fmt_bytes["fp8"])))
    log(f"C3 decode layer N={N} K={K}, M={Ms}, weight copies={copies}")
    L = DecodeLayer(q, torch, d, copies, ("fp8", "w4a16"))
    x = dev(d["a"], torch)
    bufs = make_bufs(torch, Ms, N, K)
    step = step_fn(q, L, x, Ms, bufs)

    # capture one graph per rotation slot (eager warm-up first, on the
    # capture stream so its workspaces exist before capture)
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
        with torch.cuda.graph(g, stream=s):
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
    del graphs

    # per-kernel rows of the step
    rows = per_kernel_rows(q, torch, L, x, Ms, bufs, a.kernel_iters, "C3")
    rows.update(bf16_rows(torch, L, x, Ms, a.kernel_iters, "C3"))
    share = {k: r["us"] for k, r in rows.items()
             if k.startswith("C3_") and "weight_bytes" in r and "linear" not in k}
    dom = max(share, key=share.get)
    dr = rows[dom]
    fmt_dom = dom.split("_")[1]
    tab = traffic_table("decode")
    traffic = None
    kname = {"fp8": "decode_gemm_kernel<FP8>", "w4a16": "decode_gemm_kernel<W4A16>"}[fmt_dom]
    if tab and dom in tab.get("rows", {}):
        traffic = tab["rows"][dom].get("hbm_bytes")
        kname = tab["rows"][dom]["kernels"][0]["kernel"]
    roofline = dict(bound="hbm", achieved=dr["GBps"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(dr["GBps"] / HBM_PEAK_GBS, 4), traffic=traffic,
                    kernel=f"{kname} M={dr['M']} K={K} N={N}", bytes_per_launch=dr["weight_bytes"],
                    launch_us=dr["us"],
                    traffic_note="HBM bytes per launch from FETCH_SIZE + WRITE_SIZE (rocprofv3 --pmc), "
                                 "calibrated on a 256 MiB copy; null when the counters were taken on "
                                 "other kernel sources")
    rows.update(repack_rows(q, torch, gen, L))
    del L
    torch.cuda.empty_cache()

    roof_pre = None
    if not a.no_extras:
        for name, fn in (("C2", c2_rows), ("C4", c4_rows), ("C5", c5_rows), ("V", vocab_rows)):
            tt = time.time()
            try:
                r = fn(q, torch, gen, a.kernel_iters)
                if name == "C4":
                    r, roof_pre = r
                    ptab = traffic_table("prefill")
                    for ro in roof_pre:
                        key = "C4_K%d_N%d_fp8_linear" % (ro["K"], ro["N"])
                        if ptab and key in ptab.get("rows", {}):
                            ro["traffic"] = ptab["rows"][key].get("hbm_bytes")
                rows.update(r)
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
        "dtype": "fp8/bf16",
        "data": "synthetic",
        "config": {"workload": "large dense decode layer K=5120 N=25600 (seed 2), M in {1,8,64}: FP8 "
                               "W8A8 linear (per-token quantisation + per-channel FP8 GEMM) and W4A16 "
                               "group-32 GEMM; weights rotated over %d copies (cold HBM), HIP-graph "
                               "replay" % copies,
                   "K": K, "N": N, "M": list(Ms), "weight_bytes_per_step": step_wb},
        "roofline": roofline,
        "roofline_prefill": roof_pre,
        "cpu_baseline": cpu,
        "rows": rows,
        "wall_s": round(time.time() - t_start, 1),
    }
    _ = np
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
