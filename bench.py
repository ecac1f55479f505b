"""Benchmark of the IM-Unpack integer GEMM path on one MI355X.

A step is one call of imu_imunpack_matmul on the LLaMA-7B-shaped linear
workload (X 2048x4096 bf16 times W^T with W 4096x4096 bf16, beta=15, b=5,
p=95%, Mix unpacking): percentile scale, RTN + outlier counts, Mix residuals,
plan (one device->host header read), digit unpacking of both operands, int8
MFMA GEMM with shift-and-accumulate fold and dequantization.  Inputs are
resident in HBM before the timed region.

The printed JSON line reports effective int-TOPS on the original shape
(2*M*N*K / step time), the unpack ratio, the GEMM's share of the dense int8
MFMA peak (roofline object), per-stage times from HIP events, and the CPU
oracle timed on the host cores (cpu_baseline).  Only one GPU is supported.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective int-TOPS (orig M·N·K) + unpack ratio + % int8 MFMA peak, 1×MI355X"
INT8_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA, 5.0 POP/s
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, help="workload recipe index (default 1: LLaMA linear)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-repeats", type=int, default=1)
    return ap.parse_args()


def device_matrix(op, torch, B):
    s = op.stored
    if op.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(s).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(s))
    t = t.to("cuda")
    return B.Matrix(t[0] if op.batch == 1 else t, op.layout)


def cpu_baseline(pr, repeats: int):
    """The oracle as it stands, on the whole workload (all stages, unpacked GEMM included)."""
    from oracle import imunpack_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = os.cpu_count() or 1
    a = O.widen(pr.a.logical_bits(0), pr.a.dtype)
    b = O.widen(pr.b.logical_bits(0), pr.b.dtype)
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        O.imunpack_matmul(a, b, pr.beta, pr.bits, pr.p_num, pr.p_den, pr.strat_a, pr.strat_b, pr.gamma,
                          unpacked=True)
        times.append(time.perf_counter() - t0)
    M, K, N = pr.mnk
    t = min(times)
    return {"value": round(2.0 * M * N * K / t / 1e12, 6), "unit": "TOPS", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"whole {pr.name} problem ({M}x{K} @ {K}x{N}), every oracle stage incl. the unpacked "
                      f"GEMM + fold, best of {repeats}; {t:.2f} s; numpy/BLAS threads={blas_threads}, "
                      f"host cpus={os.cpu_count()}"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the IM-Unpack path here is single-GPU", file=sys.stderr)
        sys.exit(2)

    import torch
    from outlier_unpacking_quantization_amd import binding as B
    from outlier_unpacking_quantization_amd import workloads as W

    pr = W.config(args.config)[0]
    M, K, N = pr.mnk
    a = device_matrix(pr.a, torch, B)
    b = device_matrix(pr.b, torch, B)
    p = B.params(beta=pr.beta, bits=pr.bits, p=(pr.p_num, pr.p_den), strat_a=pr.strat_a,
                 strat_b=pr.strat_b, gamma=pr.gamma)
    ws = B.Workspace("cuda")
    c = torch.empty((pr.a.batch, M, N), dtype=torch.int32, device="cuda")
    out = torch.empty((pr.a.batch, M, N), dtype=torch.float32, device="cuda")

    def step():
        return B.imunpack_matmul(a, b, p, out=out, c=c, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        _, _, infos = step()
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    info = infos[0]

    # per-stage HIP events through the staged entry points (same kernels)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
    names = ["quantize_a", "quantize_b", "plan", "unpack_a", "unpack_b", "gemm"]
    acc = np.zeros(6)
    reps = max(3, min(args.steps, 20))
    for it in range(reps + 1):
        ev[0].record()
        sa = B.quantize_rtn(a, p)
        ev[1].record()
        sb = B.quantize_rtn(b, p)
        ev[2].record()
        plan = B.plan_unpack(a, b, p, sa, sb)
        ev[3].record()
        a_u = B.unpack(a, 0, p, sa, plan)
        ev[4].record()
        b_u = B.unpack(b, 1, p, sb, plan)
        ev[5].record()
        B.unpacked_gemm(a_u, b_u, p, sa, sb, plan)
        ev[6].record()
        torch.cuda.synchronize()
        if it:
            acc += [ev[i].elapsed_time(ev[i + 1]) for i in range(6)]
    stages_us = {n: round(float(v) * 1000.0 / reps, 2) for n, v in zip(names, acc)}

    # dominant kernel: the unpacked int8 GEMM, timed alone over back-to-back launches
    gc, gout = torch.empty_like(c), torch.empty_like(out)
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        B.unpacked_gemm(a_u, b_u, p, sa, sb, plan)
    g0.record()
    greps = max(10, args.steps)
    for _ in range(greps):
        B.unpacked_gemm(a_u, b_u, p, sa, sb, plan)
    g1.record()
    torch.cuda.synchronize()
    t_gemm = g0.elapsed_time(g1) / 1000.0 / greps
    gemm_ops = 2.0 * info["m_u"] * info["k_u"] * info["n_u"]
    gemm_tops = gemm_ops / t_gemm / 1e12

    eff_tops = 2.0 * M * N * K / t_step / 1e12
    rec = {
        "metric": METRIC,
        "value": round(eff_tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"{pr.name}: A {M}x{K} {pr.a.dtype} ({pr.a.layout}) @ B {K}x{N} {pr.b.dtype} "
                               f"({pr.b.layout}), beta={pr.beta} b={pr.bits} p={pr.p_num}/{pr.p_den} "
                               f"{pr.strat_a}/{pr.strat_b}",
                   "M": M, "K": K, "N": N, "batch": pr.a.batch},
        "unpack_ratio": round(info["unpack_ratio"], 4),
        "plan": {"choice": list(info["choice"]), "m_u": info["m_u"], "k_u": info["k_u"], "n_u": info["n_u"],
                 "k_pad": info["k_pad"], "segments": info["n_seg"]},
        "gemm_pct_int8_peak": round(100.0 * gemm_tops / INT8_PEAK_TOPS, 2),
        "stages_us": stages_us,
        "roofline": {"bound": "mfma", "kernel": "gemm_kernel (imu_unpacked_gemm)",
                     "achieved": round(gemm_tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                     "frac": round(gemm_tops / INT8_PEAK_TOPS, 4), "traffic": None,
                     "launch_us": round(t_gemm * 1e6, 2), "ops_per_launch": gemm_ops},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(pr, args.cpu_repeats)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
