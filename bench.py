#!/usr/bin/env python3
"""Benchmark: one training step of the MXFP4 GEMM path at Llama-3.1-8B MLP shapes on one MI355X.

A step is the whole hot path for each MLP projection (gate/up 8192x28672x4096
and down 8192x4096x14336, M = 8192 tokens, one GPU's share):
    forward : dual casts of A and W (one launch), out = A . W^T (FP4 GEMM)
    backward: dual cast dOut, dA = dOut . W (NN) and dW = dOut^T . A (NT wgrad),
              the two in one persistent launch where that is faster
every kernel launched through the C ABI on torch's current stream, inputs
resident in HBM before timing starts.

Prints ONE JSON line.  `value` is the whole step's throughput (6*M*N*K
summed over the projections, divided by the step time including the casts),
from K steps after W warm-up steps with nothing between the launches.
`roofline` describes the dominant kernel (the GEMM): algorithmic FLOPs per
launch over its average launch time, timed with events on the launch stream
over a second pass of K steps that records an event after every launch.
`cpu_baseline` times the CPU oracle on a bounded slab of the same workload.

Other modes: `--workload llama70b | llama8b_attn` (the same step at other
projection shapes), `--workload ragged` (the edge sweep), `--ceilings` (the
sustained MFMA and HBM rates of the bench's probes), `--cast-scaling` (the dual
cast's marginal rate and fixed cost per launch), `--gemm-data` (the MLP GEMM
products on random against constant operands), `--copy-calibration`
(a plain device copy for scaling HBM counters).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP4_PEAK_TFLOPS = 10100.0   # MI355X dense MXFP4 MFMA
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense FP8 MFMA
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
METRIC = "MXFP4 GEMM TFLOP/s + % of MI355X FP4 peak (fwd+dA+dB), cast GB/s"

WORKLOADS = {
    "llama8b_mlp": ("Llama-3.1-8B MLP projections, one GPU's share (M=8192 tokens): gate/up 8192x28672x4096 "
                    "and down 8192x4096x14336, fwd + dA + dB with dual casts"),
    "llama8b_attn": ("Llama-3.1-8B attention projections, one GPU's share (M=8192): QKV 8192x6144x4096 and "
                     "O 8192x4096x4096, fwd + dA + dB with dual casts"),
    "llama70b": ("Llama-3-70B per-GPU projections (M=8192): QKV 8192x10240x8192, gate/up 8192x57344x8192, "
                 "down 8192x8192x28672, fwd + dA + dB with dual casts"),
    "ragged": ("edge / ragged sweep: all 36 (M, N, K) with M in {1, 17, 4096, 16384}, N in {128, 4096, 128256}, "
               "K in {32, 4096, 14336}, U(-1e3, 1e3) with 5% zero and 5% subnormal 32x32 tiles; "
               "fwd + dA + dB with dual casts per combination"),
}


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    # defaults: 100 timed steps after 50 warm-up steps (the chip's clock and power settle over the
    # first ~50 ms of back-to-back steps); the ragged sweep: 5 after 2 per combination
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="llama8b_mlp", choices=sorted(WORKLOADS))
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target wall time of the CPU-oracle sample (0 skips the CPU baseline)")
    p.add_argument("--cached-weights", action="store_true",
                   help="weights quantized once before timing (WeightWorkspace reuse): the step skips W's dual cast")
    p.add_argument("--hadamard-grad", action="store_true",
                   help="the Hadamard gradient recipe: column copies of A and W and both copies of dOut transformed")
    p.add_argument("--fp8-wgrad", action="store_true",
                   help="dB as an MXFP8 GEMM (column copies of A and dOut in MXFP8), as in the FP8 dB variant")
    p.add_argument("--fused-producers", action="store_true",
                   help="A operands made by the fused producers: RMSNorm + cast for gate/up (of the block input), "
                        "SiLU-and-mul + cast for down (of the gate/up output) instead of plain casts")
    p.add_argument("--headline-only", action="store_true",
                   help="the default 8B MLP line without the secondary 70B and 8B-attention configs")
    p.add_argument("--no-kernel-events", action="store_true",
                   help="time only the whole step (no per-kernel events)")
    p.add_argument("--ceilings", action="store_true",
                   help="only measure the chip's sustained FP4 MFMA rate (random and constant operands) and HBM "
                        "stream rates (read, copy, the dual cast's read/write mix) with the bench's probes")
    p.add_argument("--cast-scaling", action="store_true",
                   help="only time the dual cast at several sizes (1 GiB read before each launch) and report its "
                        "marginal rate and fixed cost per launch")
    p.add_argument("--gemm-data", action="store_true",
                   help="only time the 8B MLP step's six GEMM products back to back on random and on constant "
                        "operands (the same kernel, launches and bytes; less switching power), with the clock")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain device copy of COPY_BYTES (for scaling HBM counters), then exit")
    a = p.parse_args()
    if a.steps is None:
        a.steps = 5 if a.workload == "ragged" else 100
    if a.warmup is None:
        a.warmup = 2 if a.workload == "ragged" else 50
    return a


COPY_BYTES = 1 << 30  # plain copy used to calibrate FETCH_SIZE / WRITE_SIZE


def copy_calibration():
    import torch
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "calls": 3}), flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_llama8b_mlp_traffic.json")


def measured_traffic():
    """Per-launch HBM bytes of the GEMM kernel from the committed counter summary, if the kernel is unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        import bench_rocprof as rs
        if t.get("source_hash") != rs.source_hash(rs.GEMM_SOURCES):
            return None
        return round(t["traffic_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def gemm_roofline(m, n, k, fmt=4):
    """Algorithmic FLOPs and minimum HBM bytes of out[m, n] = sum over k (MXFP4 or, fmt 8, MXFP8
    operands), and the bound they imply."""
    flops = 2.0 * m * n * k
    code = 0.5 if fmt == 4 else 1.0
    nbytes = m * k * code + n * k * code + (m + n) * k / 32 + 2.0 * m * n
    t_mfma = flops / ((FP4_PEAK_TFLOPS if fmt == 4 else FP8_PEAK_TFLOPS) * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBPS * 1e9)
    return flops, nbytes, ("mfma" if t_mfma >= t_hbm else "hbm"), max(t_mfma, t_hbm)


def step_ops(P, L, sp, N, cached_weights=False, hadamard=False, fp8_wgrad=False):
    """The training step of one projection: (kind, label, launch, work, roofline-ideal seconds).
    With cached_weights, W's copies are made once beforehand and the step has no W cast.
    With hadamard, the casts apply the gradient recipe's block transform (A and W: column copy;
    dOut: both copies, divided by 32).  With fp8_wgrad, A and dOut get MXFP8 column copies and
    dB is the MXFP8 GEMM (kind "gemm8")."""

    def cast_dual(x, row, col, t_row=False, t_col=False, shift=0):
        R, C = x.shape
        if col.fmt == 8:
            return lambda: L.mxfp4_cast_dual_fp8col(x.data_ptr(), R, C, C, row.q.data_ptr(), row.s.data_ptr(),
                                                    col.q.data_ptr(), col.s.data_ptr(), sp)
        if hadamard:
            return lambda: L.mxfp4_cast_hadamard(x.data_ptr(), R, C, C, row.q.data_ptr(), row.s.data_ptr(),
                                                 col.q.data_ptr(), col.s.data_ptr(), int(t_row), int(t_col), shift, sp)
        return lambda: L.mxfp4_cast_dual(x.data_ptr(), R, C, C, row.q.data_ptr(), row.s.data_ptr(),
                                         col.q.data_ptr(), col.s.data_ptr(), sp)

    def gemm(fn, a, b, out):
        # MXFP4 products go through the workspace form (a long contraction behind a small output
        # is split over several workgroups); the same kernels as mxfp4_gemm_nt / _nn otherwise
        M, Nn = a.rows, b.rows
        ws = P["gemm_ws"]
        if a.fmt == 8:
            return lambda: fn(a.q.data_ptr(), a.s.data_ptr(), b.q.data_ptr(), b.s.data_ptr(), M, Nn, a.k,
                              out.data_ptr(), Nn, sp)
        return lambda: L.mxfp4_gemm_nt_ws(a.q.data_ptr(), a.s.data_ptr(), b.q.data_ptr(), b.s.data_ptr(), M, Nn, a.k,
                                          out.data_ptr(), Nn, ws.data_ptr(), ws.numel(), sp)

    M, Nn, K, name = P["M"], P["N"], P["K"], P["name"]
    ops = []
    casts = [] if P.get("producer") else [("cast_dual(A)", P["a"], P["a_row"], P["a_col"])]
    if P.get("producer"):
        ops.append(producer_op(P, L, sp))
    if not cached_weights:
        casts.append(("cast_dual(W)", P["w"], P["w_row"], P["w_col"]))
    def cast_bytes(x, col):
        # bytes per element: bf16 read, FP4 row codes, column codes (FP4 or FP8), two scale bytes per 32
        return (2.5 + (1.0 if col.fmt == 8 else 0.5) + 2.0 / 32) * x.shape[0] * x.shape[1]

    if len(casts) == 2 and not hadamard and all(c[3].fmt == 4 for c in casts):
        # the forward's two dual casts in one launch, as the training step's forward does them
        (_, xa, ra, ca), (_, xw, rw, cw) = casts
        nb = cast_bytes(xa, ca) + cast_bytes(xw, cw)
        launch = lambda: L.mxfp4_cast_dual_pair(
            xa.data_ptr(), xa.shape[0], xa.shape[1], xa.shape[1], ra.q.data_ptr(), ra.s.data_ptr(), ca.q.data_ptr(),
            ca.s.data_ptr(), xw.data_ptr(), xw.shape[0], xw.shape[1], xw.shape[1], rw.q.data_ptr(), rw.s.data_ptr(),
            cw.q.data_ptr(), cw.s.data_ptr(), sp)
        ops.append(("cast", name + ".cast_dual(A,W)", launch, nb, nb / (HBM_PEAK_GBPS * 1e9)))
        casts = []
    for label, x, row, col in casts:
        nb = cast_bytes(x, col)
        ops.append(("cast", name + "." + label, cast_dual(x, row, col, False, True, 0), nb, nb / (HBM_PEAK_GBPS * 1e9)))
    fl, _, _, t = gemm_roofline(M, Nn, K)
    ops.append(("gemm", name + ".fwd", gemm(L.mxfp4_gemm_nt, P["a_row"], P["w_row"], P["out"]), fl, t))
    nb = (2.5 + (1.0 if fp8_wgrad else 0.5) + 2.0 / 32) * M * Nn
    ops.append(("cast", name + ".cast_dual(dOut)", cast_dual(P["g"], P["g_row"], P["g_col"], True, True, 5), nb,
                nb / (HBM_PEAK_GBPS * 1e9)))
    fl, _, _, t = gemm_roofline(M, K, Nn)
    if fp8_wgrad:
        ops.append(("gemm", name + ".dA", gemm(L.mxfp4_gemm_nn, P["g_row"], P["w_col"], P["da"]), fl, t))
        fl, _, _, t = gemm_roofline(Nn, K, M, fmt=8)
        ops.append(("gemm8", name + ".dB(fp8)", gemm(L.mxfp8_gemm_nt, P["g_col"], P["a_col"], P["dw"]), fl, t))
    else:
        # dA and dB in one call, as the training backward makes them: one persistent launch with
        # the XCDs divided between the two where that is faster, else two launches
        fl1, _, _, t1 = gemm_roofline(Nn, K, M)
        gr, wc, gc, ac, ws = P["g_row"], P["w_col"], P["g_col"], P["a_col"], P["gemm_ws"]
        pair = lambda: L.mxfp4_gemm_nt_pair_ws(
            gr.q.data_ptr(), gr.s.data_ptr(), wc.q.data_ptr(), wc.s.data_ptr(), M, K, Nn, P["da"].data_ptr(), K,
            gc.q.data_ptr(), gc.s.data_ptr(), ac.q.data_ptr(), ac.s.data_ptr(), Nn, K, gc.k, P["dw"].data_ptr(), K,
            ws.data_ptr(), ws.numel(), sp)
        ops.append(("gemm", name + ".dA+dB", pair, fl + fl1, t + t1))
    return ops


def gemm_kernel_launches(label, projs, L):
    """GEMM kernel launches behind one GEMM op of step_ops: the paired dA + dB call is one launch
    when it pairs and two otherwise; every other GEMM op one."""
    if not label.endswith(".dA+dB"):
        return 1
    P = {p["name"]: p for p in projs}[label[:-len(".dA+dB")]]
    return 1 if L.mxfp4_gemm_pair_split(P["M"], P["K"], P["N"], P["N"], P["K"], P["Mp"]) > 0 else 2


def producer_op(P, L, sp):
    """The A operand made by a fused producer + cast instead of a plain cast: RMSNorm of the
    block input (gate/up) or SiLU-and-mul of the gate/up output (down).  Work: the producer's
    inputs read once plus the copies written (minimum bytes); an unfused producer would also
    write its bf16 output and the cast read it back (4 B more per element)."""
    kind = P["producer"][0]
    M, K = P["M"], P["K"]
    row, col = P["a_row"], P["a_col"]
    copies = 0.5 + (1.0 if col.fmt == 8 else 0.5) + 2.0 / 32
    if kind == "rms":
        _, x, gamma, rstd, eps = P["producer"]
        launch = lambda: L.mxfp4_rmsnorm_cast(x.data_ptr(), None, gamma.data_ptr(), eps, M, K, row.q.data_ptr(),
                                              row.s.data_ptr(), col.q.data_ptr(), col.s.data_ptr(), col.fmt, None,
                                              rstd.data_ptr(), None, sp)
        nb = (2.0 + copies) * M * K
        label = "rmsnorm_cast(A)"
    else:
        _, src = P["producer"]
        launch = lambda: L.mxfp4_silu_mul_cast(src.data_ptr(), M, K, src.stride(0), row.q.data_ptr(),
                                               row.s.data_ptr(), col.q.data_ptr(), col.s.data_ptr(), col.fmt, None, sp)
        nb = (4.0 + copies) * M * K
        label = "silu_mul_cast(A)"
    return ("cast", P["name"] + "." + label, launch, nb, nb / (HBM_PEAK_GBPS * 1e9))


def alloc_projection(name, M, Nn, K, a, w, g, mx, torch, dev, fp8_wgrad=False):
    """Device operands of one projection's step (a, w, g: bf16 device tensors); with fp8_wgrad
    the column copies of A and dOut (dB's operands) are MXFP8."""
    Mp = -(-M // 32) * 32
    cf = 8 if fp8_wgrad else 4
    P = dict(name=name, M=M, N=Nn, K=K, Mp=Mp, a=a, w=w, g=g)
    P["a_row"], P["a_col"] = mx.empty_operand(M, K, dev), mx.empty_operand(K, Mp, dev, cf)
    P["w_row"], P["w_col"] = mx.empty_operand(Nn, K, dev), mx.empty_operand(K, Nn, dev)
    P["g_row"], P["g_col"] = mx.empty_operand(M, Nn, dev), mx.empty_operand(Nn, Mp, dev, cf)
    P["out"] = torch.empty((M, Nn), dtype=torch.bfloat16, device=dev)
    P["da"] = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    P["dw"] = torch.empty((Nn, K), dtype=torch.bfloat16, device=dev)
    # split-contraction scratch shared by the step's three products (run in order on one stream)
    P["gemm_ws"] = mx.gemm_workspace([(M, Nn, K), (M, K, Nn), (Nn, K, Mp)], dev)
    return P


def time_ops(ops, steps, warmup, stream, torch, N, per_kernel=True, before_step=None):
    """Warm up, then time `steps` passes over `ops` on `stream`.  With per_kernel, one event
    goes before the first launch and after every launch, so kernel i is timed between
    events i and i+1 (no extra gaps between launches).  `before_step` (e.g. a cache flush)
    runs before every timed pass, outside the events; the pass time is then the sum of the
    per-pass event spans instead of one bracket around all passes.
    Returns (ms per pass, per-op lists of per-pass ms, or None)."""

    def run(events):
        if events is not None:
            events[0].record(stream)
        for i, (_, label, launch, _, _) in enumerate(ops):
            st = launch()
            if st != 0:
                raise N.Mxfp4Error(st, label)
            if events is not None:
                events[i + 1].record(stream)

    for _ in range(warmup):
        if before_step is not None:
            before_step()
        run(None)
    torch.cuda.synchronize()
    use_events = per_kernel or before_step is not None
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(steps)] \
        if use_events else None
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s_ in range(steps):
        if before_step is not None:
            before_step()
        run(ev[s_] if use_events else None)
    end.record(stream)
    torch.cuda.synchronize()
    if before_step is not None:
        ms = sum(ev[s_][0].elapsed_time(ev[s_][-1]) for s_ in range(steps)) / steps
    else:
        ms = start.elapsed_time(end) / steps
    if not per_kernel:
        return ms, None
    return ms, [[ev[s_][i].elapsed_time(ev[s_][i + 1]) for s_ in range(steps)] for i in range(len(ops))]


def percentiles(xs):
    import numpy as np
    p10, p50, p90 = np.percentile(np.asarray(xs, dtype=np.float64), [10, 50, 90])
    return {"p10": round(float(p10), 4), "p50": round(float(p50), 4), "p90": round(float(p90), 4)}


class ClockSampler:
    """Samples the GPU's shader clock (MHz) and board power (W) from sysfs in a thread.
    Reads the first card exposing pp_dpm_sclk; `summary()` is None where sysfs has neither."""

    def __init__(self, period_s=0.002):
        import glob
        import threading
        cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.sclk = cards[0] if cards else None
        base = os.path.dirname(self.sclk) if self.sclk else None
        powers = sorted(glob.glob(os.path.join(base, "hwmon", "hwmon*", "power1_input"))) if base else []
        self.power = powers[0] if powers else None
        self.period = period_s
        self.mhz, self.watts = [], []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        if self.sclk:
            try:
                for line in open(self.sclk):
                    if line.rstrip().endswith("*"):
                        self.mhz.append(float(line.split(":")[1].strip().split("M")[0]))
            except (OSError, ValueError, IndexError):
                pass
        if self.power:
            try:
                self.watts.append(float(open(self.power).read()) / 1e6)
            except (OSError, ValueError):
                pass

    def _run(self):
        while not self._stop.is_set():
            self._read()
            self._stop.wait(self.period)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join()

    def summary(self):
        import numpy as np
        if not self.mhz and not self.watts:
            return None
        out = {"samples": len(self.mhz)}
        if self.mhz:
            out["sclk_mhz"] = {"p50": float(np.median(self.mhz)), "min": min(self.mhz), "max": max(self.mhz)}
        if self.watts:
            out["power_w"] = {"p50": round(float(np.median(self.watts)), 1), "max": round(max(self.watts), 1)}
        return out


def ragged_sweep(args, torch, mx, N, W, L, dev):
    """Every (M, N, K) of the edge sweep: one step each, per-kernel times against each kernel's roofline."""
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    cid = W.CONFIG_IDS["ragged"]
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    combos = []
    tot_flops = tot_ms = 0.0
    for ci, (M, Nn, K) in enumerate(W.ragged_combos()):
        seed = W.seed_of(cid, 0, ci)
        a = W.ragged_values_torch((M, K), seed + W.A, dev).view(torch.bfloat16)
        w = W.ragged_values_torch((Nn, K), seed + W.W, dev).view(torch.bfloat16)
        g = W.ragged_values_torch((M, Nn), seed + W.DOUT, dev).view(torch.bfloat16)
        P = alloc_projection("M%d-N%d-K%d" % (M, Nn, K), M, Nn, K, a, w, g, mx, torch, dev)
        ops = step_ops(P, L, sp, N)
        # a 1 GiB read before every timed step: small operands would otherwise stay in the 256 MB MALL
        # (a read leaves clean lines, so the step pays no write-back of the flush)
        ms, per = time_ops(ops, args.steps, args.warmup, stream, torch, N, before_step=lambda: torch.sum(flush))
        fl = 6.0 * M * Nn * K
        tot_flops += fl
        tot_ms += ms
        kernels = {}
        for (kind, label, _, work, ideal), ts in zip(ops, per):
            t = sum(ts) / len(ts)
            rate = work / (t * 1e-3)
            kernels[label.split(".", 1)[1]] = {
                "ms": round(t, 4), ("tflops" if kind == "gemm" else "gbps"): round(rate / (1e12 if kind == "gemm" else 1e9), 1),
                "roofline_frac": round(ideal / (t * 1e-3), 3)}
        combos.append({"M": M, "N": Nn, "K": K, "ms_step": round(ms, 4), "kernels": kernels})
        print("[ragged %2d/36] M=%d N=%d K=%d step %.3f ms" % (ci + 1, M, Nn, K, ms), file=sys.stderr, flush=True)
        del P, ops, a, w, g
        torch.cuda.empty_cache()
    value = tot_flops / (tot_ms * 1e-3) / 1e12
    return {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(tot_ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "mxfp4", "data": "synthetic",
            "config": {"workload": WORKLOADS["ragged"], "combos": len(combos),
                       "step_tflop": round(tot_flops / 1e12, 4), "cache": "1 GiB read before every timed step"},
            "per_combo": combos}


def ceilings():
    """What the chip sustains on the path's two bounds, measured with the bench's probes
    (bench_probes.hip, a library of their own): the GEMM's inner loop of FP4 32x32x64 scaled MFMAs over
    register-resident operands, on random codes and on constant codes (the power limit shows
    in the difference), and 16-byte HBM streams: read only, copy, and the dual cast's 2 : 1.0625
    mix of read and written bytes.  Prints one JSON line."""
    import torch
    import bench_probes as N
    L = N.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    def timed(launch, reps):
        N.check(launch(), "probe")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            N.check(launch(), "probe")
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    result = {"metric": "sustained rates (probes)", "cus": cus}
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    words = cus * 256 * 32  # 128 bytes per lane
    ops = {"mfma_random": torch.randint(-2 ** 31, 2 ** 31 - 1, (words,), dtype=torch.int32, device=dev, generator=g),
           "mfma_constant": torch.full((words,), 0x24242424, dtype=torch.int32, device=dev)}  # E2M1 1.0 and 2.0
    out_f = torch.empty(cus * 256, dtype=torch.float32, device=dev)
    iters = 40000
    flop = cus * 4 * iters * 16 * 2.0 * 32 * 32 * 64
    for name, buf in ops.items():
        t = timed(lambda: L.probe_mfma(buf.data_ptr(), iters, cus, out_f.data_ptr(), sp), 10)
        tf = flop / t / 1e12
        # each SIMD issues one 32-cycle MFMA after another: the clock implied if none is lost
        result[name] = {"tflops": round(tf, 1), "frac_of_peak": round(tf / FP4_PEAK_TFLOPS, 4),
                        "implied_clock_mhz": round(2400.0 * tf / FP4_PEAK_TFLOPS)}
    nbytes = 4 << 30
    src = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).random_(generator=g)
    out_u = torch.empty(cus * 8 * 256, dtype=torch.int32, device=dev)
    for name, w in (("hbm_read", 0), ("hbm_copy", 32), ("hbm_cast_mix", 17)):
        dst_bytes = -(-nbytes // 512) * w * 16
        dst = torch.empty(max(dst_bytes // 4, 4), dtype=torch.int32, device=dev) if w else None
        t = timed(lambda: L.probe_stream(src.data_ptr(), nbytes, dst.data_ptr() if w else None, w, cus * 8,
                                                     out_u.data_ptr(), sp), 10)
        moved = nbytes + dst_bytes
        result[name] = {"gbps": round(moved / t / 1e9, 1), "frac_of_hbm": round(moved / t / 1e9 / HBM_PEAK_GBPS, 4),
                        "read_bytes": nbytes, "write_bytes": dst_bytes}
        del dst
    print(json.dumps(result), flush=True)


def cast_scaling():
    """Dual cast of x [R, C] (bf16 N(0,1)) for R = 4096 .. 32768 at C = 4096 and 14336, a 1 GiB read
    before every launch (no operand served from the MALL), hip events around each launch: per size the
    median time and rate, and per C the marginal rate between the two largest sizes (the stream's own
    rate) and the fixed cost per launch it leaves (launch latency, ramp and tail).  Prints one JSON line."""
    import numpy as np
    import torch
    import mxfp4_block_scaled_cast_amd as mx
    dev = torch.device("cuda:0")
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    result = {"metric": "dual cast time against size", "bytes_per_element": 3.0625, "sizes": [], "fits": []}
    for C in (4096, 14336):
        pts = []
        for R in (4096, 8192, 16384, 32768):
            x = torch.randn(R, C, device=dev, generator=g).to(torch.bfloat16)
            t = mx.cast_dual(x)
            ts = []
            for rep in range(15):
                flush.sum()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                mx.cast_dual(x, t.row, t.col)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            us = float(np.median(ts[3:]))
            nb = R * C * 3.0625
            pts.append((nb, us))
            result["sizes"].append({"R": R, "C": C, "us": round(us, 2), "gbps": round(nb / us * 1e-3, 1),
                                    "frac_of_hbm": round(nb / us * 1e-3 / HBM_PEAK_GBPS, 4)})
            del x, t
        (b0, t0), (b1, t1) = pts[-2], pts[-1]
        marginal = (b1 - b0) / (t1 - t0) * 1e-3
        result["fits"].append({"C": C, "marginal_gbps": round(marginal, 1),
                               "marginal_frac_of_hbm": round(marginal / HBM_PEAK_GBPS, 4),
                               "fixed_us": round(t1 - b1 / marginal * 1e-3, 2)})
    print(json.dumps(result), flush=True)


def gemm_data():
    """The 8B MLP step's six GEMM products (fwd, dA, dB of gate/up and down), each launched back to back
    (20 untimed, then 60 timed between two events) on random operands (bf16 N(0, 1) cast to MXFP4) and
    on constant ones (every element 1.0: one code, one scale), alternating, with the shader clock
    sampled over each timed run.  Same kernel, launch sequence and bytes moved; only the operands'
    switching activity differs.  Prints one JSON line."""
    import numpy as np
    import torch
    import mxfp4_block_scaled_cast_amd as mx
    from mxfp4_block_scaled_cast_amd import workloads as W
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(17)
    out = {"metric": "MXFP4 GEMM TFLOP/s by operand data (8B MLP products)", "products": []}
    tot = {"random": [0.0, 0.0], "constant": [0.0, 0.0]}
    for name, M, Nn, K in W.LLAMA8B_MLP:
        for what, (m, n, k) in (("fwd", (M, Nn, K)), ("dA", (M, K, Nn)), ("dB", (Nn, K, M))):
            ops = {}
            for kind in ("random", "constant"):
                if kind == "random":
                    xa = torch.randn(m, k, device=dev, generator=g).to(torch.bfloat16)
                    xb = torch.randn(n, k, device=dev, generator=g).to(torch.bfloat16)
                else:
                    xa = torch.ones(m, k, device=dev, dtype=torch.bfloat16)
                    xb = torch.ones(n, k, device=dev, dtype=torch.bfloat16)
                ops[kind] = (mx.cast(xa), mx.cast(xb))
                del xa, xb
            o = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
            row = {"product": "%s.%s" % (name, what), "M": m, "N": n, "K": k}
            for kind in ("random", "constant", "random", "constant"):
                a, b = ops[kind]
                for _ in range(20):
                    mx.gemm_nt(a, b, out=o)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                with ClockSampler() as cs:
                    e0.record()
                    for _ in range(60):
                        mx.gemm_nt(a, b, out=o)
                    e1.record()
                    torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / 60
                clk = cs.summary()
                tf = 2.0 * m * n * k / us * 1e-6
                row.setdefault(kind, []).append({"us": round(us, 1), "tflops": round(tf, 1),
                                                 "sclk_mhz": clk["sclk_mhz"]["p50"] if clk and "sclk_mhz" in clk
                                                 else None})
            for kind in ("random", "constant"):
                best = min(row[kind], key=lambda r: r["us"])
                tot[kind][0] += 2.0 * m * n * k
                tot[kind][1] += best["us"]
            out["products"].append(row)
            del ops, o
            torch.cuda.empty_cache()
    for kind, (fl, us) in tot.items():
        tf = fl / us * 1e-6
        out[kind] = {"tflops": round(tf, 1), "frac_of_fp4_peak": round(tf / FP4_PEAK_TFLOPS, 4)}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gemm_data:
        gemm_data()
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.cast_scaling:
        cast_scaling()
        return
    if args.ceilings:
        ceilings()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.stderr.write("bench.py measures one GPU only: the library has no multi-GPU path "
                         "(--gpus %d, WORLD_SIZE %d requested)\n" % (args.gpus, world))
        sys.exit(2)

    import torch

    import mxfp4_block_scaled_cast_amd as mx
    from mxfp4_block_scaled_cast_amd import _native as N
    from mxfp4_block_scaled_cast_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = N.lib()

    if args.workload == "ragged":
        print(json.dumps(ragged_sweep(args, torch, mx, N, W, L, dev)), flush=True)
        return
    result = measure_workload(args.workload, args, args.steps, args.warmup, args.cpu_seconds, torch, mx, N, W, L,
                              dev)
    plain = not (args.cached_weights or args.hadamard_grad or args.fp8_wgrad or args.fused_producers)
    if args.workload == "llama8b_mlp" and plain and not args.headline_only:
        # the other per-GPU projection configs, as secondary fields of the same line (fewer steps)
        for wl in SECONDARY:
            r = measure_workload(wl, args, min(args.steps, SECONDARY_STEPS), min(args.warmup, SECONDARY_WARMUP),
                                 min(args.cpu_seconds, SECONDARY_CPU_S), torch, mx, N, W, L, dev)
            result[wl] = {k: r[k] for k in SECONDARY_KEYS if k in r}
    print(json.dumps(result), flush=True)


SECONDARY = ("llama70b", "llama8b_attn")
SECONDARY_STEPS, SECONDARY_WARMUP, SECONDARY_CPU_S = 30, 20, 8.0
SECONDARY_KEYS = ("config", "steps", "warmup", "ms_per_step", "value", "frac_of_fp4_peak", "gemm_tflops",
                  "gemm_frac_of_fp4_peak", "cast_gbps", "cast_frac_of_hbm", "per_kernel", "roofline", "clock",
                  "cpu_baseline")


def measure_workload(workload, args, steps, warmup, cpu_seconds, torch, mx, N, W, L, dev):
    """The training step of one projection config: inputs made and resident, `warmup` untimed
    steps, `steps` timed steps bracketed by two events (the step time), the same steps again
    with an event after every launch (per-kernel times), the clock over 0.5 s more, and the
    CPU oracle on a bounded sample.  Returns the result dict; frees the config's buffers."""
    import numpy as np
    projections = {"llama8b_mlp": W.LLAMA8B_MLP, "llama8b_attn": W.LLAMA8B_ATTN, "llama70b": W.LLAMA70B}[workload]

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    # ---- inputs and preallocated operands (resident before timing)
    t0 = time.time()
    projs = []
    host_inputs = {}
    for idx, (name, M, Nn, K) in enumerate(projections):
        a, w, g = W.projection_inputs(workload, idx, M, Nn, K)
        if idx == 0:
            host_inputs = {"a": a, "w": w, "M": M, "N": Nn, "K": K, "name": name}
        projs.append(alloc_projection(name, M, Nn, K, to_dev(a), to_dev(w), to_dev(g), mx, torch, dev,
                                      args.fp8_wgrad))
        del a, w, g
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    if args.fused_producers:
        if workload != "llama8b_mlp" and workload != "llama70b":
            sys.stderr.write("--fused-producers needs an MLP workload (gate/up then down)\n")
            sys.exit(2)
        byname = {P["name"]: P for P in projs}
        gu, dn = byname["gate_up"], byname["down"]
        g = torch.from_numpy(W.bf16_bits((1 + 0.1 * np.random.default_rng(5).standard_normal(gu["K"]))
                                         .astype(np.float32)).view(np.int16)).view(torch.bfloat16).to(dev)
        gu["producer"] = ("rms", gu["a"], g, torch.empty(gu["M"], dtype=torch.float64, device=dev),
                          float(np.float32(1e-5)))
        # down's A is SiLU-and-mul of the gate/up output [M, 2 * K_down]
        dn["producer"] = ("silu", gu["out"])
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    ops = []
    step_flops = 0.0
    for P in projs:
        step_flops += 6.0 * P["M"] * P["N"] * P["K"]
        ops += step_ops(P, L, sp, N, cached_weights=args.cached_weights, hadamard=args.hadamard_grad,
                        fp8_wgrad=args.fp8_wgrad)
        if args.cached_weights:
            # the WeightWorkspace fill: W's dual cast once, outside the timed region
            R, C = P["w"].shape
            N.check(L.mxfp4_cast_hadamard(P["w"].data_ptr(), R, C, C, P["w_row"].q.data_ptr(),
                                          P["w_row"].s.data_ptr(), P["w_col"].q.data_ptr(), P["w_col"].s.data_ptr(),
                                          0, int(args.hadamard_grad), 0, sp), "mxfp4_cast_hadamard")

    if args.fp8_wgrad and args.hadamard_grad:
        sys.stderr.write("--fp8-wgrad and --hadamard-grad do not combine (the transform is MXFP4-only)\n")
        sys.exit(2)
    use_events = not args.no_kernel_events
    # the timed region: K steps bracketed by two events, nothing between the launches
    ms_per_step, _ = time_ops(ops, steps, warmup, stream, torch, N, per_kernel=False)
    per = None
    if use_events:
        # per-kernel durations: the same K steps again with an event after every launch
        # (each event adds a few microseconds between launches, so the step time above
        # comes from the uninstrumented pass)
        _, per = time_ops(ops, steps, 0, stream, torch, N, per_kernel=True)

    per_op = {}
    gemm_ms = cast_ms = 0.0
    gemm_launches = 0
    gemm_work = cast_bytes = 0.0
    gemm8_ms = gemm8_work = 0.0
    if use_events:
        for (kind, label, _, work, _), ts in zip(ops, per):
            avg = sum(ts) / len(ts)
            rate = work / (avg * 1e-3)
            is_gemm = kind in ("gemm", "gemm8")
            per_op[label] = {"ms": round(avg, 4),
                             ("tflops" if is_gemm else "gbps"): round(rate / (1e12 if is_gemm else 1e9), 1),
                             **percentiles(ts)}
            if kind == "gemm8":
                gemm8_ms += avg
                gemm8_work += work
            elif kind == "gemm":
                gemm_ms += avg
                gemm_launches += gemm_kernel_launches(label, projs, L)
                gemm_work += work
            else:
                cast_ms += avg
                cast_bytes += work

    value = step_flops / (ms_per_step * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4+mxfp8" if args.fp8_wgrad else "mxfp4",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[workload] + (
                       "; weights quantized once (cached), no W cast in the step" if args.cached_weights else "") + (
                       "; Hadamard gradient recipe" if args.hadamard_grad else "") + (
                       "; dB as an MXFP8 GEMM (FP8 wgrad)" if args.fp8_wgrad else "") + (
                       "; A operands from fused RMSNorm + cast (gate/up) and SiLU-and-mul + cast (down)"
                       if args.fused_producers else ""),
                   "projections": [[P["name"], P["M"], P["N"], P["K"]] for P in projs],
                   "step_tflop": round(step_flops / 1e12, 4)},
        "frac_of_fp4_peak": round(value / FP4_PEAK_TFLOPS, 4),
    }
    if use_events:
        gemm_tflops = gemm_work / (gemm_ms * 1e-3) / 1e12
        cast_gbps = cast_bytes / (cast_ms * 1e-3) / 1e9
        avg_gemm_ms = gemm_ms / gemm_launches
        result["gemm_tflops"] = round(gemm_tflops, 1)
        result["gemm_frac_of_fp4_peak"] = round(gemm_tflops / FP4_PEAK_TFLOPS, 4)
        result["cast_gbps"] = round(cast_gbps, 1)
        result["cast_frac_of_hbm"] = round(cast_gbps / HBM_PEAK_GBPS, 4)
        result["per_kernel"] = per_op
        if gemm8_ms > 0:
            t8 = gemm8_work / (gemm8_ms * 1e-3) / 1e12
            result["fp8_gemm"] = {"kernel": "mxfp8 block-scaled GEMM (dB launches)", "achieved": round(t8, 1),
                                  "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(t8 / FP8_PEAK_TFLOPS, 4)}
        result["roofline"] = {"kernel": "mxfp4 block-scaled GEMM (%s launches)" % (
                                  "fwd, dA" if gemm8_ms > 0 else "fwd; dA + dB paired"),
                              "bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": FP4_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(gemm_tflops / FP4_PEAK_TFLOPS, 4),
                              "launches_per_step": gemm_launches,
                              "avg_launch_ms": round(avg_gemm_ms, 4),
                              "flop_per_launch": gemm_work / gemm_launches,
                              # counters were taken over the 8B MLP step's MXFP4 GEMM launches: the
                              # figure belongs to that workload's GEMM set only
                              "traffic": measured_traffic()
                              if workload == "llama8b_mlp" and gemm8_ms == 0 else None}
        # sustained clock and power over ~0.5 s of further steps (not part of the timed region)
        with ClockSampler() as cs:
            t_end = time.time() + 0.5
            while time.time() < t_end:
                time_ops(ops, 5, 0, stream, torch, N, per_kernel=False)
        clk = cs.summary()
        result["clock"] = clk
        if clk and "sclk_mhz" in clk:
            peak_clk = FP4_PEAK_TFLOPS * clk["sclk_mhz"]["p50"] / 2400.0
            result["roofline"]["peak_at_clock"] = round(peak_clk, 1)
            result["roofline"]["frac_at_clock"] = round(gemm_tflops / peak_clk, 4)

    # free the config's device buffers before the CPU sample (and the next config)
    del ops, projs
    P = gu = dn = None  # noqa: F841 (the loop variables held the last projection's buffers)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(host_inputs, cpu_seconds)
    result["setup_s"] = round(setup_s, 1)
    return result




def cpu_baseline(inp, target_s):
    """The CPU oracle on a slab of the first projection's forward GEMM: cast the slab's
    rows of A and all of W, then the exact fp64 GEMM for those rows."""
    import numpy as np
    import oracle

    cores = len(os.sched_getaffinity(0))
    a, w, K, Nn = inp["a"], inp["w"], inp["K"], inp["N"]

    def run(rows):
        t = time.perf_counter()
        qa, sa = oracle.cast_rows(np.ascontiguousarray(a[:rows]), nthreads=cores)
        qw, sw = oracle.cast_rows(w, nthreads=cores)
        oracle.gemm(qa, sa, qw, sw, nthreads=cores)
        return time.perf_counter() - t

    # calibrate: a fixed part (W's cast, B's unpacking) plus a part linear in the rows
    r1, r2 = 8, 8 * cores
    t1, t2 = run(r1), run(r2)
    per_row = max((t2 - t1) / (r2 - r1), 1e-6)
    fixed = max(t1 - per_row * r1, 0.0)
    rows = int(max(target_s - fixed, per_row * r2) / per_row)
    rows = max(r2, min(a.shape[0], rows // 8 * 8))

    dt = run(rows)
    flops = 2.0 * rows * Nn * K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "%s forward, first %d of %d rows of A (%d x %d x %d): oracle cast of those rows and of W, "
                      "then the exact fp64 GEMM; %.1f s" % (inp["name"], rows, a.shape[0], rows, Nn, K, dt)}


if __name__ == "__main__":
    main()
