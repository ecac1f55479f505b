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


# HBM traffic of one GEMM launch on the default workload, from two rocprofv3
# --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by the
# factor that maps the same counter onto the known bytes of a plain 256 MiB
# device copy (bench.py --copy-calibration).  The readings belong to one
# version of the GEMM source: when gemm.hip no longer hashes to `source_sha256`
# the traffic is reported as null.
GEMM_TRAFFIC = {
    "source_sha256": "9f179b4b771cddb04e32901c9ce05bb9939bf615b38f57d1d4242e0c8bdcd7b9",
    "fetch_kib": 151790.0, "write_kib": 65536.0,        # counter readings per launch
    "fetch_factor": 1.99980, "write_factor": 1.00000,  # copy calibration
    "bytes_per_launch": 377943480,
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, help="workload recipe index (default 1: LLaMA linear)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-repeats", type=int, default=1)
    ap.add_argument("--training-step", action="store_true",
                    help="time the quantized-training linear step (forward, data gradient, weight gradient) "
                         "at the training workload size instead")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy 5 times (counter calibration)")
    return ap.parse_args()


def gemm_source_sha() -> str:
    import hashlib
    path = os.path.join(ROOT, "outlier_unpacking_quantization_amd", "csrc", "gemm.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


class HipEvents:
    """Raw HIP events (timing enabled) through the HIP runtime torch has loaded.

    They are recorded with a device-scope release: a default event writes back
    the L2 to system scope when it is recorded, which would leave the GPU idle
    for microseconds inside every timed step."""

    kReleaseToDevice = 0x40000000  # hipEventReleaseToDevice

    def __init__(self, n: int):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(h), self.kReleaseToDevice) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(h.value)

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(h)


def copy_calibration():
    import torch
    n = 256 << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 5}))


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


def training_step(args):
    """One step = the three GEMMs of a linear layer's training step (forward,
    data gradient, weight gradient), each the whole IM-Unpack path, on the
    training workload (8192 tokens, 768 -> 3072, beta=31, b=4, Mix)."""
    import torch
    from outlier_unpacking_quantization_amd import binding as B
    from outlier_unpacking_quantization_amd import training as T
    from outlier_unpacking_quantization_amd import workloads as W

    fwd, dgrad, _ = W.training()
    dev = "cuda"
    bf = lambda st: torch.from_numpy(np.ascontiguousarray(st[0]).view(np.int16)).view(torch.bfloat16).to(dev)
    x = bf(fwd.a.stored)          # tokens x d_in
    w = bf(fwd.b.stored)          # d_out x d_in (W^T stored transposed)
    dy = bf(dgrad.a.stored).float()  # tokens x d_out, entering as float32
    tokens, d_in = x.shape
    d_out = w.shape[0]
    p = B.params(beta=fwd.beta, bits=fwd.bits)
    ws = B.Workspace(dev)

    def step():
        T.linear_forward(x, w, p, ws)
        T.linear_data_grad(dy, w, p, ws)
        T.linear_weight_grad(dy, x, p, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / args.steps
    ops = 3 * 2.0 * tokens * d_in * d_out
    print(json.dumps({"metric": "effective int-TOPS of a quantized-training linear step (fwd + dgrad + wgrad)",
                      "value": round(ops / t / 1e12, 3), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "ms_per_step": round(t * 1e3, 4), "higher_is_better": True,
                      "dtype": "i8", "data": "synthetic",
                      "config": {"workload": f"training linear: X {tokens}x{d_in} bf16, W {d_out}x{d_in} bf16, "
                                             f"dY {tokens}x{d_out} (float32 from bf16), beta={fwd.beta} b={fwd.bits} "
                                             "p=95/100 mix/mix"}}))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the IM-Unpack path here is single-GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.training_step:
        training_step(args)
        return

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
    # the GEMM launches of every timed step are bracketed by a pair of HIP
    # events recorded by the library on the launch stream
    hev = HipEvents(2 * args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        B.set_gemm_events(hev.ev[2 * i], hev.ev[2 * i + 1])
        _, _, infos = step()
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    B.set_gemm_events(None, None)
    t_gemm = sum(hev.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)) / 1000.0 / args.steps
    hev.close()
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

    # dominant kernel: the unpacked int8 GEMM of the timed steps (events above)
    gemm_ops = sum(2.0 * f["m_u"] * f["k_u"] * f["n_u"] for f in infos)  # every batch entry
    gemm_tops = gemm_ops / t_gemm / 1e12
    traffic = None
    if GEMM_TRAFFIC is not None and GEMM_TRAFFIC["source_sha256"] == gemm_source_sha():
        traffic = GEMM_TRAFFIC["bytes_per_launch"]

    eff_tops = 2.0 * M * N * K * pr.a.batch / t_step / 1e12
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
        "unpack_ratio": round(sum(f["m_u"] * f["k_u"] * f["n_u"] for f in infos) / (pr.a.batch * M * K * N), 4),
        "plan": {"choice": list(info["choice"]), "m_u": info["m_u"], "k_u": info["k_u"], "n_u": info["n_u"],
                 "k_pad": info["k_pad"], "segments": info["n_seg"]},
        "gemm_pct_int8_peak": round(100.0 * gemm_tops / INT8_PEAK_TOPS, 2),
        "stages_us": stages_us,
        "roofline": {"bound": "mfma", "kernel": "gemm_kernel (imu_unpacked_gemm)",
                     "achieved": round(gemm_tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                     "frac": round(gemm_tops / INT8_PEAK_TOPS, 4), "traffic": traffic,
                     "launch_us": round(t_gemm * 1e6, 2), "ops_per_launch": gemm_ops},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(pr, args.cpu_repeats)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
