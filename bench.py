"""Benchmark of the k-quant prefill GEMM hot path on one MI355X.

A step is one pass of the whole hot path over the FFN gate/up workload of a 7B prefill:
quantize_q8_1 of the f32 activation X [512 x 4096] (per-token gains) followed by the
q4_K MMQ against W [11008 x 4096] q4_K, output Y [512 x 11008] f32. Inputs are seeded
synthetic data resident in HBM before timing starts.

Prints ONE JSON line (metric, value in TMAC/s = M*N*K / step time, roofline of the MMQ
kernel, CPU-oracle baseline). Defaults: 200 warm-up and 1000 timed steps (~100 ms of GPU
time): the first ~10-20 ms of a run are up to 10 % slower while the clock ramps up.
Other modes:
  --shards                   the N/8 shares of the 7B layer GEMMs, plain vs K-split entry
                             points (one JSON line per shape)
  --msweep                   the 7B layer GEMM shapes at M = 16 .. 2048 tokens, likewise
  --q6forms                  the raw, prepared and expanded q6_K forms on the v and down
                             shapes at M = 16 .. 1024, likewise
For rocprofv3 runs:
  --profile {q4K,q6K,q6Kp,q6Kx,quant}  a few launches of one kernel (q6_K raw / prepared /
                             expanded), no timing output
  --copy-calibration         a device-to-device copy of known size (HBM counter scale)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "int8 TMAC/s of q4_K/q6_K MMQ at 7B prefill shapes (M=512); % of MFMA peak"
PEAK_INT8_TOPS = 5000.0          # MI355X dense int8 MFMA, TOP/s (2 ops per MAC)
PEAK_HBM_GBS = 8000.0
PEAK_F32_VALU_TFLOPS = 157.3     # MI355X f32 vector peak (FMA = 2 FLOP)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_mmq_q4K_512x11008x4096.txt")
KERNEL_SOURCES = ["quantized_prefill_gemm_amd/csrc/mmq_q4k.hip", "quantized_prefill_gemm_amd/csrc/qpg_common.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch of the MMQ kernel from committed rocprofv3 counter runs, or None
    when the kernel source changed since the counters were taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def algorithmic_bytes(M, N, K, wbytes_per_block=144):
    """Bytes the MMQ kernel must move at least once: weights (bytes per row and 256 weights:
    144 q4_K, 210 q6_K, 256 prepared q6_K, 548 expanded q6_K), q8_1 activations, f32 output."""
    return N * (K // 256) * wbytes_per_block + (M * K + 4 * M * (K // 32)) + 4 * M * N


def setup(cfg: int):
    import torch
    from quantized_prefill_gemm_amd import binding as B
    from quantized_prefill_gemm_amd import inputs
    wtype, M, N, K, W, X = inputs.make_config(cfg)
    dev = torch.device("cuda:0")
    w = torch.from_numpy(W.reshape(-1)).to(dev)
    x = torch.from_numpy(X).to(dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = torch.empty(B.q8_1_bytes(M, K), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    return B, wtype, M, N, K, W, X, w, x, y, ws


ROUNDS = 5


def run_gpu(cfg: int, steps: int, warmup: int, q6: str = "raw"):
    """Warm-up steps, then exactly `steps` timed steps (the line's value). Afterwards, outside
    the timed region, ROUNDS rounds that alternate `steps` steps, `steps` MMQ launches alone
    and `steps` quantize launches alone, each bracketed by HIP events on the launch stream,
    with the shader clock read right after each round: the per-kernel figures are the
    medians of those rounds, taken under the same clock as the step figure they are
    compared with."""
    import statistics
    import torch
    B, wtype, M, N, K, W, X, w, x, y, ws = setup(cfg)
    mmq_q8 = B.mmq_q4K_q8 if wtype == "q4_K" else B.mmq_q6K_q8
    if q6 == "prepared" and wtype == "q6_K":
        w = B.q6K_prepare(w, N, K)          # one-time repack, outside the timed region
        mmq_q8 = B.mmq_q6K_prep_q8
    elif q6 == "expanded" and wtype == "q6_K":
        w = B.q6K_expand(w, N, K)           # one-time expansion, outside the timed region
        mmq_q8 = B.mmq_q6K_exp_q8
    stream = torch.cuda.current_stream()

    def step():
        B.quantize_q8_1(x, ws, stream=stream)
        mmq_q8(w, ws, M, N, K, y, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    def bracketed(fn, n):
        """Average over n back-to-back calls, HIP events on the launch stream around them all
        (an event between two launches costs ~3 us of GPU time on this device, so none is
        recorded inside)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # timed region: exactly `steps` steps
    t0 = time.perf_counter()
    step_ms = bracketed(step, steps)
    wall = time.perf_counter() - t0
    rounds = {"step": [], "mmq": [], "quant": [], "clock_ghz": []}
    clock = ClockProbe()
    for _ in range(ROUNDS):
        rounds["step"].append(bracketed(step, steps))
        rounds["mmq"].append(bracketed(lambda: mmq_q8(w, ws, M, N, K, y, stream=stream), steps))
        rounds["quant"].append(bracketed(lambda: B.quantize_q8_1(x, ws, stream=stream), steps))
        rounds["clock_ghz"].append(clock.read())
    med = {k: statistics.median(v) for k, v in rounds.items()}
    return dict(wtype=wtype, M=M, N=N, K=K, W=W, X=X, wall_s=wall, step_ms=step_ms,
                quant_ms=med["quant"], mmq_ms=med["mmq"], step_rounds_ms=med["step"],
                clock_ghz=med["clock_ghz"], rounds=rounds)


class ClockProbe:
    """Shader clock right now: a short run of libqpg_calib.so's matrix-core chains on every CU
    (s_memtime ticks over the 100 MHz s_memrealtime ticks of the same loop, median over the
    workgroups). ~20 us, so it reads the clock the preceding work left the device at."""

    def __init__(self, blocks: int = 256, iters: int = 100):
        import ctypes
        import torch
        self.lib = ctypes.CDLL(os.path.join(ROOT, "quantized_prefill_gemm_amd", "libqpg_calib.so"))
        self.lib.qpg_calib_mfma_i8.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        self.lib.qpg_calib_mfma_i8.restype = ctypes.c_int
        self.blocks, self.iters = blocks, iters
        self.out = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda:0")
        self.sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def read(self) -> float:
        import ctypes
        import statistics
        import torch
        if self.lib.qpg_calib_mfma_i8(self.blocks, self.iters, ctypes.c_void_p(self.out.data_ptr()), self.sp) != 0:
            raise RuntimeError("qpg_calib_mfma_i8 failed")
        torch.cuda.synchronize()
        v = self.out.view(self.blocks, 4).cpu().numpy()
        return statistics.median(t / (r / 100e6) for t, r in zip(v[:, 0], v[:, 1]) if r > 0) / 1e9


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wtype, W, X):
    """The oracle (untuned) on the full workload: one warm run, then the median of three."""
    import statistics
    from oracle import oracle as O
    nth = O.default_threads()
    M, K = X.shape
    N = W.shape[0]
    O.mmq(wtype, W, X, nthreads=nth)                 # warm: page-in, thread start-up
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        O.mmq(wtype, W, X, nthreads=nth)
        runs.append(time.perf_counter() - t0)
    dt = statistics.median(runs)
    return {"value": M * N * K / dt / 1e12, "unit": "TMAC/s", "cores": nth, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"full workload {M}x{N}x{K} {wtype}: quantize_q8_1 + exact int32 sums + fp64 fold; "
                      f"median of 3 runs after one warm run ({', '.join(f'{r:.2f}' for r in runs)} s) "
                      f"on {nth} threads"}


def measured_mfma_peak(iters: int = 20000, blocks: int = 512):
    """Measured int8 matrix-core peak and shader clock (libqpg_calib.so: chains of
    v_mfma_i32_32x32x32_i8 only, two waves per SIMD)."""
    import ctypes
    import statistics
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "quantized_prefill_gemm_amd", "libqpg_calib.so"))
    lib.qpg_calib_mfma_i8.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.qpg_calib_mfma_i8.restype = ctypes.c_int
    out = torch.zeros(blocks * 4, dtype=torch.int64, device="cuda:0")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    if lib.qpg_calib_mfma_i8(blocks, 100, ctypes.c_void_p(out.data_ptr()), sp) != 0:
        raise RuntimeError("qpg_calib_mfma_i8 failed")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    rc = lib.qpg_calib_mfma_i8(blocks, iters, ctypes.c_void_p(out.data_ptr()), sp)
    e1.record(stream)
    torch.cuda.synchronize()
    if rc != 0:
        raise RuntimeError("qpg_calib_mfma_i8 failed")
    secs = e0.elapsed_time(e1) * 1e-3
    ops = blocks * 4 * iters * 16 * 65536
    v = out.view(blocks, 4).cpu().numpy()
    clocks = [t / (r / 100e6) for t, r in zip(v[:, 0], v[:, 1]) if r > 0]
    ghz = statistics.median(clocks) / 1e9
    return {"value": round(ops / secs / 1e12, 1), "unit": "TOP/s", "clock_ghz": round(ghz, 3),
            "spec_at_this_clock": round(PEAK_INT8_TOPS * ghz / 2.4, 1),
            "kernel": "v_mfma_i32_32x32x32_i8 chains, 2 waves per SIMD", "seconds": round(secs, 5)}


STEP_MODES = {0: "mfma_only", 1: "fold_only", 2: "kernel_step", 3: "mfma_and_independent_fold",
              4: "mfma_then_own_fold", 5: "kernel_step_operands_from_lds",
              6: "kernel_step_operands_from_lds_one_step_ahead", 7: "kernel_step_fold_in_groups_of_4"}


def measured_step_ceiling(waves=(1, 2, 3, 4), iters: int = 4000):
    """The q4_K kernel's compute step alone (libqpg_calib.so qpg_calib_step: one
    v_mfma_i32_32x32x32_i8 issued a step ahead plus the 32 fold FMAs of the previous result,
    per wave and step; no memory traffic, barriers, decode or min term), at 1-4 waves per
    SIMD (one: a short prompt's split, one four-wave workgroup per CU). Each mode is timed with HIP events around one launch; the rate is counted in the
    int8 ops of the MFMAs (2 per MAC) the steps stand for, also for the fold-only mode.
    Returns the rate of the kernel's step at its production occupancy (3 waves per SIMD) as
    the ceiling of its arithmetic, plus every mode and occupancy."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "quantized_prefill_gemm_amd", "libqpg_calib.so"))
    lib.qpg_calib_step.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.qpg_calib_step.restype = ctypes.c_int
    lib.qpg_calib_step_blocks.argtypes = [ctypes.c_int]
    lib.qpg_calib_step_blocks.restype = ctypes.c_int64
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    table = {}
    for w in waves:
        nb = lib.qpg_calib_step_blocks(w)
        out = torch.zeros(nb * 4, dtype=torch.int64, device="cuda:0")
        row = {}
        for mode, name in STEP_MODES.items():
            if lib.qpg_calib_step(mode, w, 50, ctypes.c_void_p(out.data_ptr()), sp) != 0:   # warm
                raise RuntimeError("qpg_calib_step failed")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            rc = lib.qpg_calib_step(mode, w, iters, ctypes.c_void_p(out.data_ptr()), sp)
            e1.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError("qpg_calib_step failed")
            secs = e0.elapsed_time(e1) * 1e-3
            v = out.view(nb, 4).cpu().numpy()
            ghz = float(np.median(v[:, 0] / (v[:, 1] / 100e6))) / 1e9
            steps_per_simd = iters * 8 * w
            row[name] = {"tops": round(2 * nb * 4 * iters * 8 * 32768 / secs / 1e12, 1),
                         "ns_per_step_per_simd": round(secs * 1e9 / steps_per_simd, 2),
                         "clock_ghz": round(ghz, 3)}
        table[f"{w}_waves_per_simd"] = row
    ks = table["3_waves_per_simd"]
    m0, m1, m2, m3 = (ks[STEP_MODES[i]]["ns_per_step_per_simd"] for i in range(4))
    return {"value": ks["kernel_step"]["tops"], "unit": "TOP/s",
            "frac_of_peak": round(ks["kernel_step"]["tops"] / PEAK_INT8_TOPS, 4),
            "clock_ghz": ks["kernel_step"]["clock_ghz"],
            "what": "q4_K compute step alone at 3 waves per SIMD (1 MFMA 32x32x32 i8 + 32 fold FMAs per "
                    "wave and step, no memory, barriers, decode or min term)",
            "overlap": {"mfma_ns": m0, "fold_ns": m1, "sum_ns": round(m0 + m1, 2), "max_ns": max(m0, m1),
                        "both_independent_ns": m3, "kernel_step_ns": m2},
            "modes": table}


def run_stack(steps: int, warmup: int, q6: str):
    """Config 5: the 32-layer 7B-shaped stack at M = 1024 (quantized_prefill_gemm_amd.stack),
    each of the 7 GEMMs of a layer preceded by its quantize_q8_1 (448 launches per pass), and
    with one quantize per distinct input (4 per layer), and the GEMMs alone; each timed both as
    one HIP graph replayed and launched eagerly. Weights: the seeded per-layer generator
    (4.15 GB of q4_K / q6_K blocks resident in HBM); activations: one seeded input per
    distinct input position, reused by every layer."""
    import torch
    from quantized_prefill_gemm_amd import inputs
    from quantized_prefill_gemm_amd.stack import MODES, SOURCES, Stack
    M, L = inputs.STACK_M, inputs.STACK_LAYERS
    dev = torch.device("cuda:0")
    weights = []
    for layer in range(L):
        weights.append([torch.from_numpy(inputs.make_stack_matrix(layer, idx)[4].reshape(-1)).to(dev)
                        for idx in range(len(inputs.STACK_LAYER))])
        if layer % 8 == 7:
            print(f"stack weights: {layer + 1}/{L} layers resident", file=sys.stderr, flush=True)
    st = Stack(weights, M, q6=q6)
    del weights
    for src in SOURCES:
        st.set_input(0, src, torch.from_numpy(inputs.make_stack_input(0, src)).to(dev))
    st.run("all")
    torch.cuda.synchronize()
    res = {}
    for mode in MODES:
        g = st.capture(mode)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for e0, e1 in ev:
            e0.record()
            g.replay()
            e1.record()
        torch.cuda.synchronize()
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        res[mode + "_graph"] = ms[len(ms) // 2]
        del g
        # the same pass launched eagerly (the host stays ahead of the GPU: ~15 us per launch
        # against ~60 us per kernel), timed as a whole
        for _ in range(warmup):
            st.run(mode)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            st.run(mode)
        e1.record()
        torch.cuda.synchronize()
        res[mode + "_eager"] = e0.elapsed_time(e1) / steps
        res[mode] = min(res[mode + "_graph"], res[mode + "_eager"])
        print(f"stack '{mode}': graph median {res[mode + '_graph']:.3f} ms, eager mean "
              f"{res[mode + '_eager']:.3f} ms per pass", file=sys.stderr, flush=True)
    return st.macs(), res


def stack_cpu_baseline():
    """Oracle on each distinct GEMM shape of the stack at M = 1024 once (plus the
    quantize it includes), extrapolated with the multiplicities 3 / 1 / 2 / 1 x 32 layers."""
    from oracle import oracle as O
    from quantized_prefill_gemm_amd import inputs
    nth = O.default_threads()
    per = {}
    for idx in (0, 2, 4, 6):
        name, wtype, N, K, W = inputs.make_stack_matrix(0, idx)
        X = inputs.make_stack_input(0, idx)
        t0 = time.perf_counter()
        O.mmq(wtype, W, X, nthreads=nth)
        per[idx] = time.perf_counter() - t0
    total = inputs.STACK_LAYERS * (3 * per[0] + per[2] + 2 * per[4] + per[6])
    macs = inputs.STACK_M * inputs.STACK_LAYERS * sum(N * K for _, _, N, K in inputs.STACK_LAYER)
    return {"value": macs / total / 1e12, "unit": "TMAC/s", "cores": nth, "kind": "oracle",
            "sample": "the 4 distinct GEMM shapes of layer 0 at M=1024 once each (quantize + exact int32 "
                      f"sums + fp64 fold), {sum(per.values()):.2f} s, extrapolated x(3,1,2,1) x 32 layers "
                      f"to {total:.1f} s"}


def profile_mode(which: str, launches: int):
    import torch
    cfg = {"q4K": 3, "q6K": 4, "q6Kp": 4, "q6Kx": 4, "quant": 3}[which]
    B, wtype, M, N, K, W, X, w, x, y, ws = setup(cfg)
    mmq = B.mmq_q4K_q8 if wtype == "q4_K" else B.mmq_q6K_q8
    if which == "q6Kp":
        w, mmq = B.q6K_prepare(w, N, K), B.mmq_q6K_prep_q8
    elif which == "q6Kx":
        w, mmq = B.q6K_expand(w, N, K), B.mmq_q6K_exp_q8
    for _ in range(launches):
        B.quantize_q8_1(x, ws)
        if which != "quant":
            mmq(w, ws, M, N, K, y)
    torch.cuda.synchronize()
    print(f"profiled {which}: {launches} launches of {wtype} {M}x{N}x{K}", flush=True)


MSWEEP_M = (16, 64, 128, 256, 512, 1024, 2048)
MSWEEP_SHAPES = [("q4K", 4096, 4096, "q/k/o 4096x4096 q4_K"), ("q6K_exp", 4096, 4096, "v 4096x4096 q6_K expanded"),
                 ("q4K", 11008, 4096, "gate/up 11008x4096 q4_K"), ("q6K_exp", 4096, 11008, "down 4096x11008 q6_K expanded")]

Q6FORMS_M = (16, 64, 128, 256, 512, 1024)
Q6FORMS_SHAPES = [(4096, 4096, "v 4096x4096"), (4096, 11008, "down 4096x11008")]

SHARD_SHAPES = [("q4K", 512, 1376, 4096, "gate/up share"), ("q4K", 512, 512, 4096, "q/k/v/o share"),
                ("q6K", 512, 512, 11008, "down share, raw q6_K"), ("q6K_prep", 512, 512, 11008, "down share, prepared"),
                ("q6K_exp", 512, 512, 11008, "down share, expanded"), ("q4K", 128, 4096, 4096, "short prompt")]


def run_shards(steps: int, warmup: int, shapes=None):
    """One GPU's N/8 share of each 7B layer GEMM (M = 512) and a short prompt, or with
    `shapes` any (form, M, N, K, label) list: the plain entry point against the K-split entry
    point (partial tiles + reduce; the plain kernel when the shape needs no split): HIP events
    around `steps` back-to-back calls, five rounds with the two alternating, median per entry.
    One JSON line per shape."""
    import torch
    from quantized_prefill_gemm_amd import binding as B
    from quantized_prefill_gemm_amd import inputs
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    # rate of torch's spin kernel (its cycle count is the shader clock's), measured once
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1_000_000)
    e0.record(stream)
    torch.cuda._sleep(4_000_000)
    e1.record(stream)
    torch.cuda.synchronize()
    spin_cycles_per_us = 4_000_000 / (e0.elapsed_time(e1) * 1e3)
    for form, M, N, K, what in (shapes or SHARD_SHAPES):
        wtype = "q4_K" if form == "q4K" else "q6_K"
        W, X = inputs.small_case(wtype, M, N, K, seed=1)
        w = torch.from_numpy(W.reshape(-1)).to(dev)
        if form == "q6K_prep":
            w = B.q6K_prepare(w, N, K)
        elif form == "q6K_exp":
            w = B.q6K_expand(w, N, K)
        xq = B.quantize_q8_1(torch.from_numpy(X).to(dev))
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        nws = B.mmq_sk_bytes(M, N, K, form)
        ws = torch.empty(max(nws // 4, 1), dtype=torch.float32, device=dev)
        plain = {"q4K": B.mmq_q4K_q8, "q6K": B.mmq_q6K_q8, "q6K_prep": B.mmq_q6K_prep_q8,
                 "q6K_exp": B.mmq_q6K_exp_q8}[form]
        sk = {"q4K": B.mmq_q4K_q8_sk, "q6K": B.mmq_q6K_q8_sk, "q6K_prep": B.mmq_q6K_prep_q8_sk,
              "q6K_exp": B.mmq_q6K_exp_q8_sk}[form]
        fns = {"plain": lambda: plain(w, xq, M, N, K, y, stream=stream),
               "split": lambda: sk(w, xq, M, N, K, y, ws if nws else None, stream=stream)}
        host_us = {}
        for name, fn in fns.items():
            h0 = time.perf_counter()
            for _ in range(warmup):
                fn()
            host_us[name] = (time.perf_counter() - h0) / warmup * 1e6
            torch.cuda.synchronize()
        # Each timed round starts behind a spin kernel long enough for the host to enqueue all
        # `steps` calls (1.5x the host time the warm-up measured), so the events time the
        # calls running back to back on the GPU, not the binding's per-call host work (which
        # exceeds the GPU time of the smallest shapes). `host_bound` reports any round whose
        # enqueueing outlasted its spin kernel. Five rounds, the two entry points alternating
        # (the clock ramps after a change of shape); median per entry.
        t = {name: [] for name in fns}
        host_bound = False
        for _ in range(5):
            for name, fn in fns.items():
                spin_us = 1.5 * host_us[name] * steps + 200.0
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(int(spin_us * spin_cycles_per_us))
                h0 = time.perf_counter()
                e0.record(stream)
                for _ in range(steps):
                    fn()
                e1.record(stream)
                host_bound |= e0.query()          # the GPU reached e0 before the host finished
                enq_us = (time.perf_counter() - h0) * 1e6
                torch.cuda.synchronize()
                t[name].append(e0.elapsed_time(e1) / steps * 1e3)
                host_us[name] = max(host_us[name], enq_us / steps)
        t = {name: sorted(v)[2] for name, v in t.items()}
        macs = M * N * K
        print(json.dumps({"shard": what, "form": form, "M": M, "N": N, "K": K,
                          "pieces": nws // (4 * M * N) if nws else 1,
                          "plain_us": round(t["plain"], 2), "split_us": round(t["split"], 2),
                          "plain_tmacs": round(macs / t["plain"] / 1e6, 1),
                          "split_tmacs": round(macs / t["split"] / 1e6, 1),
                          "host_us_per_call": {k: round(v, 1) for k, v in host_us.items()},
                          "host_bound": bool(host_bound)}), flush=True)


def copy_calibration(nbytes: int, launches: int):
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(launches):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copy calibration: {launches} copies of {nbytes} bytes", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", type=int, default=3,
                    help="workload 2/3 (q4_K), 4 (q6_K) or 5 (the 32-layer stack as one graph)")
    ap.add_argument("--q6k", choices=["raw", "prepared", "expanded"], default=None,
                    help="q6_K weight form: raw blocks, the prepared repack or the expanded digits "
                         "(made once, outside the timed region); default raw for config 4, expanded "
                         "for config 5")
    ap.add_argument("--prepared", action="store_true", help="same as --q6k prepared")
    ap.add_argument("--expanded", action="store_true", help="same as --q6k expanded")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--profile", choices=["q4K", "q6K", "q6Kp", "q6Kx", "quant"])
    ap.add_argument("--launches", type=int, default=20)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--shards", action="store_true",
                    help="time the N/8 shares of the 7B layer GEMMs: plain vs K-split entry points")
    ap.add_argument("--msweep", action="store_true",
                    help="time the 7B layer GEMM shapes over M = 16..2048 tokens: plain vs K-split entry points")
    ap.add_argument("--q6forms", action="store_true",
                    help="time the three q6_K weight forms on the v and down shapes over M = 16..1024")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}): this build has no multi-GPU path; "
              f"the per-GPU kernel at its sharded shape is the unit that scales.", file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration(a.copy_calibration, a.launches)
        return
    if a.profile:
        profile_mode(a.profile, a.launches)
        return
    if a.shards or a.msweep or a.q6forms:
        if a.shards:
            shapes = None
        elif a.msweep:
            shapes = [(f, m, n, k, f"{what}, M={m}") for f, n, k, what in MSWEEP_SHAPES for m in MSWEEP_M]
        else:
            shapes = [(f, m, n, k, f"{what} {f} M={m}") for n, k, what in Q6FORMS_SHAPES for m in Q6FORMS_M
                      for f in ("q6K", "q6K_prep", "q6K_exp")]
        run_shards(a.steps if a.steps != ap.get_default("steps") else (300 if a.shards else 100),
                   a.warmup if a.warmup != ap.get_default("warmup") else (100 if a.shards else 30), shapes)
        return

    if a.config == 5:
        steps = a.steps if a.steps != ap.get_default("steps") else 10
        warmup = a.warmup if a.warmup != ap.get_default("warmup") else 2
        q6 = a.q6k or ("prepared" if a.prepared else "expanded")
        macs, res = run_stack(steps, warmup, q6)
        ms = res["all"]
        out = {
            "metric": METRIC, "value": round(macs / (ms * 1e-3) / 1e12, 3), "unit": "TMAC/s", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
            "config": {"workload": "32-layer 7B-shaped stack, M=1024: q/k/o 4096x4096 q4_K, v 4096x4096 q6_K, "
                                   "gate/up 11008x4096 q4_K, down 4096x11008 q6_K, quantize_q8_1 before each "
                                   "GEMM; 448 launches per pass, as one HIP graph or eagerly, whichever is faster",
                       "M": 1024, "layers": 32, "q6_K": {"raw": "raw blocks", "prepared": "prepared",
                                                         "expanded": "expanded digits"}[q6]},
            "stack_ms": {k: round(v, 4) for k, v in res.items()},
            "launch": "graph" if res["all_graph"] <= res["all_eager"] else "eager",
            "stack_tmacs": {"with_7_quantizes": round(macs / (res["all"] * 1e-3) / 1e12, 3),
                            "with_4_shared_quantizes": round(macs / (res["shared"] * 1e-3) / 1e12, 3),
                            "gemms_only": round(macs / (res["gemm"] * 1e-3) / 1e12, 3)},
        }
        if not a.no_cpu:
            out["cpu_baseline"] = stack_cpu_baseline()
        print(json.dumps(out), flush=True)
        return

    q6 = a.q6k or ("prepared" if a.prepared else "expanded" if a.expanded else "raw")
    r = run_gpu(a.config, a.steps, a.warmup, q6=q6)
    M, N, K = r["M"], r["N"], r["K"]
    macs = M * N * K
    ms_step = r["step_ms"]
    value = macs / (ms_step * 1e-3) / 1e12
    mmq_s = r["mmq_ms"] * 1e-3
    achieved = 2 * macs / mmq_s / 1e12
    traffic = load_traffic() if a.config == 3 else None
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TMAC/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": f"{r['wtype']} MMQ + q8_1 quantize, M={M} tokens x N={N} x K={K}"
                               + (" (FFN gate/up shape, per-token gains U[0.5,2])" if a.config == 3 else "")
                               + ({"prepared": " (q6_K weights prepared once, outside the timed steps)",
                                   "expanded": " (q6_K weights expanded once, outside the timed steps)"}
                                  .get(q6, "") if r["wtype"] == "q6_K" else ""),
                   "M": M, "N": N, "K": K, "weights": r["wtype"]},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_INT8_TOPS,
                     "unit": "TOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 5), "traffic": traffic,
                     "kernel": f"mmq_{r['wtype'].replace('_', '')}{'_exp' if q6 == 'expanded' and r['wtype'] == 'q6_K' else ''}_kernel",
                     "avg_us": round(r["mmq_ms"] * 1e3, 3),
                     "note": "int8 ops counted as 2 per MAC, as in the 5.0 POP/s dense int8 peak"},
        "kernels_us": {"quantize_q8_1": round(r["quant_ms"] * 1e3, 3), "mmq": round(r["mmq_ms"] * 1e3, 3),
                       "step": round(r["step_rounds_ms"] * 1e3, 3),
                       "timing": f"after the K timed steps, {ROUNDS} rounds alternating K steps, K MMQ "
                                 "launches alone and K quantize launches alone, HIP events on the launch "
                                 "stream around each; medians",
                       "rounds_us": {k: [round(t * 1e3, 3) for t in v] for k, v in r["rounds"].items()
                                     if k != "clock_ghz"}},
        "clock_ghz": {"median": round(r["clock_ghz"], 3), "rounds": [round(c, 3) for c in r["rounds"]["clock_ghz"]],
                      "how": "shader clock read right after each round (s_memtime over s_memrealtime)"},
        "mmq_tmacs": round(macs / mmq_s / 1e12, 3),
        "mmq_hbm_gbs_algorithmic": round(algorithmic_bytes(M, N, K, 144 if r["wtype"] == "q4_K" else
                                                           {"raw": 210, "prepared": 256, "expanded": 548}[q6])
                                         / mmq_s / 1e9, 1),
        "wall_s": round(r["wall_s"], 4),
    }
    # consistency of the line: the MMQ alone cannot take longer than quantize + MMQ measured in
    # the same rounds; a line where it does is flagged, not silently printed
    out["self_check"] = {"mmq_us_below_step_us": r["mmq_ms"] < r["step_rounds_ms"],
                         "quant_plus_mmq_over_step": round((r["mmq_ms"] + r["quant_ms"]) / r["step_rounds_ms"], 4)}
    # The fold (2 f32 FMAs per output and 32-chunk for q4_K, 4 for q6_K, 3 for expanded q6_K) on the VALU, against
    # the f32 vector peak.
    fold_fma = M * N * (K // 32) * (2 if r["wtype"] == "q4_K" else 3 if q6 == "expanded" else 4)
    fold_tflops = 2 * fold_fma / mmq_s / 1e12
    out["fold_valu"] = {"achieved": round(fold_tflops, 2), "peak": PEAK_F32_VALU_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(fold_tflops / PEAK_F32_VALU_TFLOPS, 4)}
    pk = measured_mfma_peak()
    pk["achieved_frac_of_measured"] = round(achieved / pk["value"], 5)
    out["mfma_peak_measured"] = pk
    if r["wtype"] == "q4_K":
        ceil = measured_step_ceiling()
        ceil["achieved_frac_of_ceiling"] = round(achieved / ceil["value"], 4)
        out["roofline"]["ceiling"] = ceil["value"]
        out["roofline"]["ceiling_frac"] = ceil["achieved_frac_of_ceiling"]
        out["step_ceiling"] = ceil
    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(r["wtype"], r["W"], r["X"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
