"""Benchmark of the IM-Unpack integer GEMM path on one MI355X.

A step is one call of imu_imunpack_matmul: percentile scale, RTN + outlier
counts, Mix residuals, plan (one device->host header read), digit unpacking
of both operands, int8 MFMA GEMM with shift-and-accumulate fold and
dequantization.  The default workload is the MLP up-projection (X 2048x4096
bf16 times W^T with W 11008x4096 bf16, beta=31, b=4, p=95%, Mix unpacking),
the largest single-GPU configuration; --config 1 selects the LLaMA-7B-shaped
linear layer.  Inputs are resident in HBM before the timed region.

The printed JSON line reports effective int-TOPS on the original shape
(2*M*N*K / step time) over back-to-back (warm) steps, the same steps with the
L2 and the 256 MB MALL flushed before each (cold, a 512 MiB write between the
steps, outside their events), the unpack ratio of Mix and of the four fixed
row/column pairings (next to the ratios the IM-Unpack page reports for
LLaMA-7B, as context), the GEMM's share of the dense int8 MFMA peak (roofline
object), per-stage times from HIP events, and the CPU oracle timed on the host
cores on a sampled block (cpu_baseline).  Only one GPU is supported.
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
FP6_PEAK_TFLOPS = 10100.0  # MI355X dense fp6 / fp4 MFMA, 10.1 PFLOP/s
HBM_PEAK_GBS = 8000.0
FLUSH_BYTES = 512 << 20  # written between cold steps: more than the 256 MB MALL and the 8 x 4 MB L2

# Unpack ratios the IM-Unpack summary page reports ("Measured effects" table,
# unpack-ratio rows: LLaMA-7B linear-layer GEMMs, beta=15, b=5).  Context only:
# those matrices are not available, the synthetic workloads are not them.
PAGE_RATIOS = {"mix": 1.06, "row/row": 2.02, "row/col": 5.36, "col/row": 1.64, "col/col": 4.01}

# HBM traffic of one GEMM launch per workload and digit format, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by the factor
# that maps the same counter onto the known bytes of a plain 256 MiB device
# copy (bench.py --copy-calibration).  The readings belong to one version of
# the GEMM source: when gemm.hip no longer hashes to `source_sha256` the
# traffic is reported as null.
GEMM_TRAFFIC = {
    ("mlp_up", "fp6"): {"source_sha256": "f12a4fb5a112327b4d7dd453fd11369b1645b15aece5d5cf52fb55a3cbf4fbee",
                        "fetch_kib": 1675866.7, "write_kib": 384852.2, "fetch_factor": 1.9998, "write_factor": 1.0000,
                        "bytes_per_launch": 3825920437},
    ("llama_linear", "int8"): {"source_sha256": "f12a4fb5a112327b4d7dd453fd11369b1645b15aece5d5cf52fb55a3cbf4fbee",
                               "fetch_kib": 151217.5, "write_kib": 65536.0, "fetch_factor": 1.9998,
                               "write_factor": 1.0000, "bytes_per_launch": 376771335},
}


WARMUP_MIN_S = 0.3  # warm-up lasts at least this long, whatever --warmup says


def warm_up(fn, n_min: int, torch) -> int:
    """Untimed steps: at least n_min, and at least WARMUP_MIN_S of them.  The
    GPU clocks take a while to come up from idle: on the LLaMA-shaped layer
    50 steps after 5 warm-up steps ran at 0.315 ms each, after 300 at 0.284.
    Returns the number of steps run."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < n_min or time.perf_counter() - t0 < WARMUP_MIN_S:
        fn()
        n += 1
        if n >= n_min:
            torch.cuda.synchronize()
    return n


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2,
                    help="workload recipe index (default 2: MLP up-projection; 1: LLaMA-shaped linear)")
    ap.add_argument("--cold-steps", type=int, default=20, help="steps timed after a cache flush each")
    ap.add_argument("--digits", choices=("auto", "int8", "fp6"), default="auto",
                    help="digit format of the unpacked operands (auto: fp6 where it applies)")
    ap.add_argument("--pair-steps", type=int, default=5, help="timed steps of each fixed row/column pairing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-logits", action="store_true",
                    help="attention workload: time imu_softmax_prepare on its logits only (for profiler runs)")
    ap.add_argument("--only-steps", action="store_true",
                    help="run the warm steps only (no cold, per-stage, fixed-pair or CPU legs): for profiler runs")
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

    def record(self, i: int, stream: int) -> None:
        if self.hip.hipEventRecord(self.ct.c_void_p(self.ev[i]), self.ct.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(pr, rows: int = 256, col_frac: int = 8):
    """The oracle as it stands, timed on the host cores on a bounded sample of
    the workload: quantization (percentile, RTN, counts) and the plan of the
    full operands, then the low bit-width route (unpack, segment GEMMs, fold)
    for the output block of the first `rows` rows and the first N/col_frac
    columns, checked against the direct product of that block.  The per-block
    time is scaled to all of C (the route's work is proportional to the output
    block at fixed K), so `value` is the oracle's effective int-TOPS on the
    whole problem."""
    from oracle import imunpack_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = os.cpu_count() or 1
    M, K, N = pr.mnk
    ms, ns = min(rows, M), max(1, N // col_frac)
    a = O.widen(pr.a.logical_bits(0), pr.a.dtype)
    b = O.widen(pr.b.logical_bits(0), pr.b.dtype)
    t0 = time.perf_counter()
    qa = O.quantize(a, pr.beta, pr.p_num, pr.p_den, pr.bits)
    qb = O.quantize(b, pr.beta, pr.p_num, pr.p_den, pr.bits)
    pl = O.plan(qa, qb, pr.strat_a, pr.strat_b, pr.gamma)
    t_qp = time.perf_counter() - t0
    t1 = time.perf_counter()
    da_r, db_c = pl.da_r[:ms], pl.db_c[:ns]
    rows_a, cols_b = O.level_lines(da_r), O.level_lines(db_c)
    Ap = O.unpack_a(qa.q[:ms], pr.bits, da_r, pl.da_c, pl.db_r, rows_a, pl.trip)
    Bp = O.unpack_b(qb.q[:, :ns], pr.bits, pl.db_r, db_c, pl.da_c, cols_b, pl.trip)
    P = O.segment_products(Ap, Bp, pl.trip, pr.bits)
    Cb = O.fold(P, rows_a, cols_b, ms, ns, pr.bits)
    t_blk = time.perf_counter() - t1
    if not np.array_equal(Cb, O.direct_product(qa.q[:ms], qb.q[:, :ns])):
        raise AssertionError("oracle: sampled unpacked block differs from the direct product")
    t_est = t_qp + t_blk * (M * N) / (ms * ns)
    return {"value": round(2.0 * M * N * K / t_est / 1e12, 6), "unit": "TOPS", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{pr.name}: quantize + plan of the full operands ({t_qp:.2f} s), then unpack + segment "
                      f"GEMMs + fold for the C block of rows 0..{ms - 1} x columns 0..{ns - 1} ({t_blk:.2f} s, "
                      f"checked against the direct product), scaled by {M * N / (ms * ns):.0f} to all of C; "
                      f"numpy/BLAS threads={blas_threads}, host cpus={os.cpu_count()}, cpu '{cpu_model()}'"}


def training_step(args):
    """One step = the three GEMMs of a linear layer's training step (forward,
    data gradient, weight gradient), each the whole IM-Unpack path, on the
    training workload (8192 tokens, 768 -> 3072, beta=31, b=4, Mix), with X, W
    and dY quantized once per step and shared by the products they enter.  The
    same step quantizing every operand per product is timed beside it."""
    import torch
    from outlier_unpacking_quantization_amd import binding as B
    from outlier_unpacking_quantization_amd import training as T
    from outlier_unpacking_quantization_amd import workloads as W

    fwd, dgrad, _ = W.training()
    dev = "cuda"
    bf = lambda st: torch.from_numpy(np.ascontiguousarray(st[0]).view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    x = bf(fwd.a.stored)          # tokens x d_in
    w = bf(fwd.b.stored)          # d_out x d_in (W^T stored transposed)
    dy = bf(dgrad.a.stored).float()  # tokens x d_out, entering as float32
    tokens, d_in = x.shape
    d_out = w.shape[0]
    p = B.params(beta=fwd.beta, bits=fwd.bits)
    ws = B.Workspace(dev)

    def shared():
        T.training_step(x, w, dy, p, ws)

    def per_use():
        T.linear_forward(x, w, p, ws)
        T.linear_data_grad(dy, w, p, ws)
        T.linear_weight_grad(dy, x, p, ws)

    def timed(fn, n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    # both variants warm up before either is timed
    n_warm = warm_up(lambda: (shared(), per_use()), args.warmup, torch)
    t = timed(shared, args.steps)
    t_per_use = timed(per_use, max(3, args.steps // 2))
    ops = 3 * 2.0 * tokens * d_in * d_out
    print(json.dumps({"metric": "effective int-TOPS of a quantized-training linear step (fwd + dgrad + wgrad)",
                      "value": round(ops / t / 1e12, 3), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
                      "warmup": args.warmup, "warmup_steps_run": n_warm, "ms_per_step": round(t * 1e3, 4),
                      "higher_is_better": True,
                      "dtype": "fp6+i8", "data": "synthetic",
                      "digits": {"forward X W^T": "fp6 (b = 4, both operands K-contiguous)",
                                 "data gradient dY W": "int8 (W enters N x K row-major)",
                                 "weight gradient dY^T X": "int8 (dY^T is outer-contiguous)"},
                      "quantization": "X, W, dY quantized once per step (3 passes), shared by the products",
                      "per_use": {"ms_per_step": round(t_per_use * 1e3, 4), "tops": round(ops / t_per_use / 1e12, 3),
                                  "quantization": "every operand quantized per product (6 passes)"},
                      "config": {"workload": f"training linear: X {tokens}x{d_in} bf16, W {d_out}x{d_in} bf16, "
                                             f"dY {tokens}x{d_out} (float32 from bf16), beta={fwd.beta} b={fwd.bits} "
                                             "p=95/100 mix/mix"}}))


def static_weight(pr, a, b, p_mix, prm, steps: int, warmup: int):
    """Inference with a fixed weight (B = W^T): (1) W's statistics prepared
    once, every call quantizes only the activation; (2) A row-unpacked, so that
    K' depends on W alone and W's unpacked B'^T is made once and reused: a call
    quantizes and unpacks the activation only (staged entry points)."""
    import torch
    from outlier_unpacking_quantization_amd import binding as B

    M, K, N = pr.mnk
    ops = 2.0 * M * N * K
    w_stats = B.prepare_operand(B.Matrix(b.stored), p_mix)  # W as stored; used transposed
    ws = B.Workspace("cuda")
    c = torch.empty((1, M, N), dtype=torch.int32, device="cuda")
    out = torch.empty((1, M, N), dtype=torch.float32, device="cuda")

    def run(fn, n):
        warm_up(fn, warmup, torch)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    t1 = run(lambda: B.imunpack_matmul_prepared(a, b, p_mix, None, (w_stats, True), out=out, c=c, ws=ws), steps)
    # B's candidate when A is row-unpacked does not depend on A: take it from a
    # plan with A restricted to rows, then plan with it fixed (no residual pass)
    p_row = prm("row", pr.strat_b)
    sa0, sb0 = B.quantize_rtn(a, p_row), B.quantize_rtn(b, p_row)
    choice_b = B.plan_unpack(a, b, p_row, sa0, sb0).entry(0)["choice"][1]
    fixed_b = choice_b if choice_b in ("row", "col") else pr.strat_b
    p_c = prm("row", fixed_b)
    sb = B.quantize_rtn(b, p_c)
    sa = B.quantize_rtn(a, p_c)
    plan = B.plan_unpack(a, b, p_c, sa, sb)
    b_u = B.unpack(b, 1, p_c, sb, plan)
    info = plan.entry(0)

    def cached_call():
        sa_ = B.quantize_rtn(a, p_c)
        pl = B.plan_unpack(a, b, p_c, sa_, sb)
        a_u = B.unpack(a, 0, p_c, sa_, pl)
        B.unpacked_gemm(a_u, b_u, p_c, sa_, sb, pl)

    t2 = run(cached_call, steps)
    return {"prepared_weight_stats": {"ms_per_step": round(t1 * 1e3, 4), "tops": round(ops / t1 / 1e12, 3),
                                      "plan": "mix/mix as the dynamic call"},
            "cached_unpacked_weight": {"ms_per_step": round(t2 * 1e3, 4), "tops": round(ops / t2 / 1e12, 3),
                                       "plan": f"row/{info['choice'][1]}",
                                       "unpack_ratio": round(info["unpack_ratio"], 4),
                                       "note": "A row-unpacked so that B'^T depends on W alone; staged entry points"}}


def only_logits(args):
    """imu_softmax_prepare on the attention workload's logits, warm steps only."""
    import torch
    from outlier_unpacking_quantization_amd import binding as B
    from outlier_unpacking_quantization_amd import workloads as W
    pr = W.config(3)[0]
    z = torch.from_numpy(W.attn_logits(1003, pr.a.batch, pr.a.rows)).to("cuda")
    P = torch.empty(z.shape, dtype=torch.bfloat16, device="cuda")
    p = B.params(beta=pr.beta, bits=pr.bits, p=(pr.p_num, pr.p_den))

    def call():
        return B.softmax_prepare(z, p, p_out=P)

    n_warm = warm_up(call, args.warmup, torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"workload": "attn_out logits", "shape": list(z.shape), "steps": args.steps,
                      "warmup_steps_run": n_warm, "softmax_prepare_us": round(t * 1e6, 2)}))


def from_logits(v, p, M, N, K, nb, steps: int):
    """The attention output from its logits (fused softmax -> quantize): the
    logits of this workload's P (fp32, resident), imu_softmax_prepare against
    torch's softmax + bf16 cast + imu_prepare_operand, and the whole step
    logits -> P.V through the prepared product.  Algorithmic bytes of the
    fused softmax: 4 (logit read) + 2 (P write) per element."""
    import torch
    from outlier_unpacking_quantization_amd import binding as B
    from outlier_unpacking_quantization_amd import workloads as W
    z = torch.from_numpy(W.attn_logits(1003, nb, M)).to("cuda")
    P = torch.empty(z.shape, dtype=torch.bfloat16, device="cuda")
    c = torch.empty((nb, M, N), dtype=torch.int32, device="cuda")
    out = torch.empty((nb, M, N), dtype=torch.float32, device="cuda")
    ws = B.Workspace("cuda")

    def fused():
        return B.softmax_prepare(z, p, p_out=P)[1]

    def separate():
        P.copy_(torch.softmax(z, dim=-1))
        return B.prepare_operand(B.Matrix(P), p)

    def whole():
        st = fused()
        return B.imunpack_matmul_prepared(B.Matrix(P), v, p, pre_a=st, out=out, c=c, ws=ws)

    def timed(fn):
        warm_up(fn, 2, torch)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
        for i in range(steps):
            ev[2 * i].record()
            fn()
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        return float(np.median([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)])) / 1000.0

    t_fused, t_sep, t_whole = timed(fused), timed(separate), timed(whole)
    elems = nb * M * K
    # algorithmic bytes of the call: logits read (4) and P written (2) by the
    # fused softmax + histogram, P read by the count (2) and residual (2) passes
    call_bytes = 10 * elems
    return {"logits": f"{nb} x {M} x {K} fp32 (the softmax inputs of this workload's P, resident)",
            "softmax_prepare_us": round(t_fused * 1e6, 2),
            "torch_softmax_then_prepare_us": round(t_sep * 1e6, 2),
            "step_ms": round(t_whole * 1e3, 4), "tops": round(2.0 * M * N * K * nb / t_whole / 1e12, 3),
            "softmax_prepare_hbm": {"bytes": call_bytes, "gbs": round(call_bytes / t_fused / 1e9, 1),
                                    "frac_of_8tbs": round(call_bytes / t_fused / 8e12, 4),
                                    "note": "whole call; 10 B per element (4 + 2 softmax, 2 count, 2 residual)"}}


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
    if args.only_logits:
        only_logits(args)
        return

    import torch
    from outlier_unpacking_quantization_amd import binding as B
    from outlier_unpacking_quantization_amd import workloads as W

    pr = W.config(args.config)[0]
    M, K, N = pr.mnk
    nb = pr.a.batch
    a = device_matrix(pr.a, torch, B)
    b = device_matrix(pr.b, torch, B)

    def prm(sa, sb, digits=args.digits):
        return B.params(beta=pr.beta, bits=pr.bits, p=(pr.p_num, pr.p_den), strat_a=sa, strat_b=sb,
                        gamma=pr.gamma, digits=digits)

    p = prm(pr.strat_a, pr.strat_b)
    ws = B.Workspace("cuda")
    c = torch.empty((nb, M, N), dtype=torch.int32, device="cuda")
    out = torch.empty((nb, M, N), dtype=torch.float32, device="cuda")

    def step(pp=p):
        return B.imunpack_matmul(a, b, pp, out=out, c=c, ws=ws)

    n_warm = warm_up(step, args.warmup, torch)
    # warm: back-to-back steps, the GEMM launches of every step bracketed by a
    # pair of HIP events the library records on the launch stream
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

    fp6 = info["digits"] == B.DIGITS["fp6"]
    if args.only_steps:
        print(json.dumps({"workload": pr.name, "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": n_warm,
                          "digits": "fp6" if fp6 else "int8",
                          "ms_per_step": round(t_step * 1e3, 4), "gemm_us": round(t_gemm * 1e6, 2)}))
        return

    # cold: a 512 MiB write before each step evicts the L2s and the MALL; the
    # step's own events start after it
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    nc = max(1, args.cold_steps)
    sev, gev = HipEvents(2 * nc), HipEvents(2 * nc)
    sh = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    for i in range(nc):
        flush.fill_(i & 0xFF)
        sev.record(2 * i, sh)
        B.set_gemm_events(gev.ev[2 * i], gev.ev[2 * i + 1])
        step()
        sev.record(2 * i + 1, sh)
    torch.cuda.synchronize()
    B.set_gemm_events(None, None)
    cold_step = float(np.median([sev.elapsed_ms(2 * i, 2 * i + 1) for i in range(nc)])) / 1000.0
    cold_gemm = float(np.median([gev.elapsed_ms(2 * i, 2 * i + 1) for i in range(nc)])) / 1000.0
    sev.close()
    gev.close()
    del flush

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
    del sa, sb, plan, a_u, b_u

    # the four fixed row/column pairings: unpack ratio (the Mix plan's table
    # holds the sizes of every pair) and the whole step with that strategy
    base_mnk = M * K * N
    ratios = {"mix": round(info["m_u"] * info["k_u"] * info["n_u"] / base_mnk, 4)}
    pair_ms = {}
    for sa_, sb_ in (("row", "row"), ("row", "col"), ("col", "row"), ("col", "col")):
        key = f"{sa_}/{sb_}"
        mu, ku, nu = info["pairs"][(sa_, sb_)]
        ratios[key] = round(mu * ku * nu / base_mnk, 4)
        pp = prm(sa_, sb_)
        for _ in range(2):
            _, _, pinfo = step(pp)
        if (pinfo[0]["m_u"], pinfo[0]["k_u"], pinfo[0]["n_u"]) != (mu, ku, nu):
            raise AssertionError(f"fixed pairing {key}: sizes differ from the Mix plan's table")
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(max(1, args.pair_steps)):
            step(pp)
        torch.cuda.synchronize()
        pair_ms[key] = round((time.perf_counter() - t1) / max(1, args.pair_steps) * 1e3, 4)

    # the greedy line-at-a-time planner on both operands (plan quality against Mix)
    pg = prm("greedy", "greedy")
    for _ in range(2):
        _, _, ginfo = step(pg)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(max(1, args.pair_steps)):
        step(pg)
    torch.cuda.synchronize()
    ratios["greedy/greedy"] = round(ginfo[0]["unpack_ratio"], 4)
    pair_ms["greedy/greedy"] = round((time.perf_counter() - t1) / max(1, args.pair_steps) * 1e3, 4)

    # quantizer variants of the page's ablation rows on the same operands: p =
    # 100% with beta = 255, and clipping at the 99.5-percentile
    variants = {}
    for key, vb, vp, vclip in (("p100_beta255", 255, (100, 100), False), ("clip_p995", pr.beta, (995, 1000), True)):
        pv = B.params(beta=vb, bits=pr.bits, p=vp, strat_a=pr.strat_a, strat_b=pr.strat_b, gamma=pr.gamma,
                      clip=vclip, digits=args.digits)
        for _ in range(2):
            _, _, vinfo = step(pv)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(max(1, args.pair_steps)):
            step(pv)
        torch.cuda.synchronize()
        tv = (time.perf_counter() - t1) / max(1, args.pair_steps)
        variants[key] = {"beta": vb, "p": f"{vp[0]}/{vp[1]}", "clip": vclip,
                         "unpack_ratio": round(vinfo[0]["unpack_ratio"], 4),
                         "ms_per_step": round(tv * 1e3, 4), "tops": round(2.0 * M * N * K * nb / tv / 1e12, 3)}

    # the other digit format on the same plan (where fp6 applies): whole step and GEMM
    formats = {}
    if fp6 or pr.bits <= 4:
        for dg in ("int8", "fp6"):
            pd = prm(pr.strat_a, pr.strat_b, dg)
            try:
                for _ in range(2):
                    step(pd)
            except B.ImunpackError:
                continue
            dev = HipEvents(2 * max(1, args.pair_steps))
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for i in range(max(1, args.pair_steps)):
                B.set_gemm_events(dev.ev[2 * i], dev.ev[2 * i + 1])
                step(pd)
            torch.cuda.synchronize()
            B.set_gemm_events(None, None)
            td = (time.perf_counter() - t1) / max(1, args.pair_steps)
            gd = sum(dev.elapsed_ms(2 * i, 2 * i + 1) for i in range(max(1, args.pair_steps))) / max(1, args.pair_steps)
            dev.close()
            formats[dg] = {"ms_per_step": round(td * 1e3, 4), "tops": round(2.0 * M * N * K * nb / td / 1e12, 3),
                           "gemm_us": round(gd * 1e3, 2)}

    # dominant kernel: the unpacked digit GEMM of the warm steps (events above),
    # against the dense MFMA peak of its operand type
    gemm_ops = sum(2.0 * f["m_u"] * f["k_u"] * f["n_u"] for f in infos)  # every batch entry
    gemm_tops = gemm_ops / t_gemm / 1e12
    peak = FP6_PEAK_TFLOPS if fp6 else INT8_PEAK_TOPS
    tr = GEMM_TRAFFIC.get((pr.name, "fp6" if fp6 else "int8"))
    traffic = tr["bytes_per_launch"] if tr and tr["source_sha256"] == gemm_source_sha() else None

    eff = lambda t: 2.0 * M * N * K * nb / t / 1e12  # noqa: E731
    rec = {
        "metric": METRIC,
        "value": round(eff(t_step), 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_warm,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp6" if fp6 else "i8",
        "data": "synthetic",
        "config": {"workload": f"{pr.name}: A {M}x{K} {pr.a.dtype} ({pr.a.layout}) @ B {K}x{N} {pr.b.dtype} "
                               f"({pr.b.layout}), beta={pr.beta} b={pr.bits} p={pr.p_num}/{pr.p_den} "
                               f"{pr.strat_a}/{pr.strat_b}, digits {'fp6 (e2m3)' if fp6 else 'int8'}",
                   "M": M, "K": K, "N": N, "batch": nb},
        "warm": {"ms_per_step": round(t_step * 1e3, 4), "tops": round(eff(t_step), 3),
                 "gemm_us": round(t_gemm * 1e6, 2)},
        "cold": {"ms_per_step": round(cold_step * 1e3, 4), "tops": round(eff(cold_step), 3),
                 "gemm_us": round(cold_gemm * 1e6, 2), "steps": nc,
                 "flush": f"{FLUSH_BYTES >> 20} MiB written before each step, outside its events (median)"},
        "unpack_ratio": round(sum(f["m_u"] * f["k_u"] * f["n_u"] for f in infos) / (nb * base_mnk), 4),
        "unpack_ratios": ratios,
        "pair_ms_per_step": pair_ms,
        "quantizer_variants": variants,
        "page_unpack_ratios": {"values": PAGE_RATIOS,
                               "note": "IM-Unpack page, LLaMA-7B linear layers, beta=15 b=5: context only"},
        "plan": {"choice": list(info["choice"]), "m_u": info["m_u"], "k_u": info["k_u"], "n_u": info["n_u"],
                 "k_pad": info["k_pad"], "segments": info["n_seg"]},
        "gemm_pct_int8_peak": round(100.0 * gemm_tops / INT8_PEAK_TOPS, 2),
        "digit_formats": formats,
        "stages_us": stages_us,
        "roofline": {"bound": "mfma", "kernel": f"gemm_kernel ({'fp6' if fp6 else 'int8'} digits, imu_unpacked_gemm)",
                     "achieved": round(gemm_tops, 2), "peak": peak, "unit": "TFLOP/s" if fp6 else "TOP/s",
                     "frac": round(gemm_tops / peak, 4), "traffic": traffic,
                     "launch_us": round(t_gemm * 1e6, 2), "ops_per_launch": gemm_ops},
    }
    if nb == 1 and pr.b.layout == "transposed":
        rec["static_weight"] = static_weight(pr, a, b, p, prm, max(3, args.pair_steps), 2)
    if pr.name == "attn_out":
        rec["from_logits"] = from_logits(b, p, M, N, K, nb, max(5, args.pair_steps))
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(pr)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
