"""Benchmark of the k-quant prefill GEMM hot path on one MI355X.

A step is one pass of the whole hot path over the FFN gate/up workload of a 7B prefill:
quantize_q8_1 of the f32 activation X [512 x 4096] (per-token gains) followed by the
q4_K MMQ against W [11008 x 4096] q4_K, output Y [512 x 11008] f32. Inputs are seeded
synthetic data resident in HBM before timing starts.

Prints ONE JSON line (metric, value in TMAC/s = M*N*K / step time, roofline of the MMQ
kernel, CPU-oracle baseline). Other modes (for rocprofv3 runs):
  --profile {q4K,q6K,quant}  a few launches of one kernel, no timing output
  --copy-calibration         a device-to-device copy of known size (HBM counter scale)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "int8 TMAC/s of q4_K/q6_K MMQ at 7B prefill shapes (M=512); % of MFMA peak"
PEAK_INT8_TOPS = 5000.0          # MI355X dense int8 MFMA, TOP/s (2 ops per MAC)
PEAK_HBM_GBS = 8000.0
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
    """Bytes the MMQ kernel must move at least once: weights, q8_1 activations, f32 output."""
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


def run_gpu(cfg: int, steps: int, warmup: int):
    import torch
    B, wtype, M, N, K, W, X, w, x, y, ws = setup(cfg)
    mmq_q8 = B.mmq_q4K_q8 if wtype == "q4_K" else B.mmq_q6K_q8
    stream = torch.cuda.current_stream()

    def step():
        B.quantize_q8_1(x, ws, stream=stream)
        mmq_q8(w, ws, M, N, K, y, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        B.quantize_q8_1(x, ws, stream=stream)
        ev[i][1].record(stream)
        mmq_q8(w, ws, M, N, K, y, stream=stream)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    q_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(steps)]
    m_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(steps)]
    span_ms = ev[0][0].elapsed_time(ev[-1][2])
    return dict(wtype=wtype, M=M, N=N, K=K, W=W, X=X, wall_s=wall, span_ms=span_ms,
                quant_ms=sum(q_ms) / steps, mmq_ms=sum(m_ms) / steps, mmq_min_ms=min(m_ms))


def cpu_baseline(wtype, W, X):
    from oracle import oracle as O
    nth = O.default_threads()
    M, K = X.shape
    N = W.shape[0]
    t0 = time.perf_counter()
    O.mmq(wtype, W, X, nthreads=nth)
    dt = time.perf_counter() - t0
    return {"value": M * N * K / dt / 1e12, "unit": "TMAC/s", "cores": nth, "kind": "oracle",
            "sample": f"full workload {M}x{N}x{K} {wtype}, one run: quantize_q8_1 + exact int32 sums + fp64 fold, "
                      f"{dt:.2f} s wall on {nth} threads"}


def profile_mode(which: str, launches: int):
    import torch
    cfg = {"q4K": 3, "q6K": 4, "quant": 3}[which]
    B, wtype, M, N, K, W, X, w, x, y, ws = setup(cfg)
    for _ in range(launches):
        if which == "quant":
            B.quantize_q8_1(x, ws)
        else:
            B.quantize_q8_1(x, ws)
            (B.mmq_q4K_q8 if wtype == "q4_K" else B.mmq_q6K_q8)(w, ws, M, N, K, y)
    torch.cuda.synchronize()
    print(f"profiled {which}: {launches} launches of {wtype} {M}x{N}x{K}", flush=True)


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
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, help="workload 2/3 (q4_K) or 4 (q6_K)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--profile", choices=["q4K", "q6K", "quant"])
    ap.add_argument("--launches", type=int, default=20)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
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

    r = run_gpu(a.config, a.steps, a.warmup)
    M, N, K = r["M"], r["N"], r["K"]
    macs = M * N * K
    ms_step = r["span_ms"] / a.steps
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
                               + (" (FFN gate/up shape, per-token gains U[0.5,2])" if a.config == 3 else ""),
                   "M": M, "N": N, "K": K, "weights": r["wtype"]},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_INT8_TOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 5), "traffic": traffic,
                     "kernel": f"mmq_{r['wtype'].replace('_', '')}_kernel", "avg_us": round(r["mmq_ms"] * 1e3, 3),
                     "note": "int8 ops counted as 2 per MAC, as in the 5.0 POP/s dense peak"},
        "kernels_us": {"quantize_q8_1": round(r["quant_ms"] * 1e3, 3), "mmq": round(r["mmq_ms"] * 1e3, 3),
                       "mmq_min": round(r["mmq_min_ms"] * 1e3, 3)},
        "mmq_tmacs": round(macs / mmq_s / 1e12, 3),
        "mmq_hbm_gbs_algorithmic": round(algorithmic_bytes(M, N, K, 144 if r["wtype"] == "q4_K" else 210)
                                         / mmq_s / 1e9, 1),
        "wall_s": round(r["wall_s"], 4),
    }
    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(r["wtype"], r["W"], r["X"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
