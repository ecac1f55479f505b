"""Python binding of ``libimunpack.so`` (the IM-Unpack C ABI in include/imunpack.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory (tensors) and the current HIP stream.
torch is imported before the library is loaded, so the library binds to the
HIP runtime torch already loaded (both carry the soname libamdhip64.so.7).

The function names match the C entry points without the ``imu_`` prefix:
``quantize_rtn``, ``plan_unpack``, ``unpack``, ``unpacked_gemm`` and
``imunpack_matmul``.  A missing library raises ``ImunpackError``; there is no
fallback implementation.
"""
from __future__ import annotations

import atexit
import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libimunpack.so")

OK, ERR_INVALID_ARG, ERR_NONFINITE, ERR_RANGE, ERR_WORKSPACE, ERR_HIP, ERR_UNSUPPORTED = range(7)
F32, BF16 = 0, 1
NORMAL, TRANSPOSED = 0, 1
STRATEGY = {"row": 0, "col": 1, "mix": 2, "greedy": 3}
CANDIDATES = ("row", "col", "cr", "rc", "greedy")
DIGITS = {"auto": 0, "int8": 1, "fp6": 2}  # imu_digits


class ImunpackError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class ImuMatrix(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("ld", ctypes.c_int64),
                ("batch", ctypes.c_int64), ("batch_stride", ctypes.c_int64)]


class ImuParams(ctypes.Structure):
    _fields_ = [("beta", ctypes.c_int32), ("p_num", ctypes.c_int32), ("p_den", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("gamma", ctypes.c_int32), ("strat_a", ctypes.c_int32),
                ("strat_b", ctypes.c_int32), ("clip", ctypes.c_int32), ("digits", ctypes.c_int32)]


class ImuPrepared(ctypes.Structure):
    _fields_ = [("stats", ctypes.c_void_p), ("transposed", ctypes.c_int32), ("pad_", ctypes.c_int32)]


class ImuPlanInfo(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("k", ctypes.c_int64), ("n", ctypes.c_int64),
                ("m_u", ctypes.c_int64), ("k_u", ctypes.c_int64), ("n_u", ctypes.c_int64),
                ("m_alloc", ctypes.c_int64), ("n_alloc", ctypes.c_int64), ("k_pad", ctypes.c_int64),
                ("m_base", ctypes.c_int64), ("n_base", ctypes.c_int64),
                ("a_offset", ctypes.c_int64), ("b_offset", ctypes.c_int64),
                ("n_seg", ctypes.c_int32), ("choice_a", ctypes.c_int32), ("choice_b", ctypes.c_int32),
                ("digits", ctypes.c_int32), ("unpack_ratio", ctypes.c_double),
                ("pair_sizes", (ctypes.c_int64 * 3) * 25)]

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in self._fields_ if f != "pair_sizes"}
        d["choice"] = (CANDIDATES[self.choice_a], CANDIDATES[self.choice_b])
        pairs = {}
        for ia, ca in enumerate(CANDIDATES):
            for ib, cb in enumerate(CANDIDATES):
                s = tuple(int(v) for v in self.pair_sizes[ia * len(CANDIDATES) + ib])
                if s[0] >= 0:
                    pairs[(ca, cb)] = s
        d["pairs"] = pairs
        return d


class ImuStatsView(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int64) for f in ("stride", "row_oob", "col_oob", "row_maxdig", "col_maxdig",
                                              "cr_rowdig", "rc_coldig", "hist")]


class ImuPlanView(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int64) for f in ("header_stride", "headers_bytes", "entry_stride", "da_r",
                                              "da_c", "db_r", "db_c", "lvl_a", "lvl_b", "kpre", "amap",
                                              "bmap", "levels", "segments", "m_alloc_max",
                                              "n_alloc_max")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library (once).  Raises ImunpackError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImunpackError(ERR_UNSUPPORTED, f"{LIB_PATH} is missing: build it with "
                                             "outlier_unpacking_quantization_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, S, I64, I32 = ctypes.POINTER, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int32
    V = ctypes.c_void_p
    sig = {
        "imu_stats_bytes": (S, [P(ImuMatrix)]),
        "imu_stats_layout": (I32, [P(ImuMatrix), P(ImuStatsView)]),
        "imu_plan_bytes": (S, [P(ImuMatrix), P(ImuMatrix), P(ImuParams)]),
        "imu_plan_layout": (I32, [P(ImuMatrix), P(ImuMatrix), P(ImuParams), P(ImuPlanView)]),
        "imu_workspace_fixed_bytes": (S, [P(ImuMatrix), P(ImuMatrix), P(ImuParams)]),
        "imu_quantize_rtn": (I32, [P(ImuMatrix), P(ImuParams), V, V, V]),
        "imu_plan_unpack": (I32, [P(ImuMatrix), P(ImuMatrix), P(ImuParams), V, V, V, P(ImuPlanInfo), V]),
        "imu_unpack": (I32, [P(ImuMatrix), I32, P(ImuParams), V, V, P(ImuPlanInfo), V, V]),
        "imu_unpacked_gemm": (I32, [V, V, P(ImuParams), V, V, V, P(ImuPlanInfo), I64, V, I64, I64, V, V]),
        "imu_imunpack_matmul": (I32, [P(ImuMatrix), P(ImuMatrix), P(ImuParams), V, V, V, S, P(S),
                                      P(ImuPlanInfo), V]),
        "imu_status_string": (ctypes.c_char_p, [I32]),
        "imu_last_error": (ctypes.c_char_p, []),
        "imu_version": (ctypes.c_char_p, []),
        "imu_set_gemm_events": (I32, [V, V]),
        "imu_imunpack_matmul_noalloc": (I32, [P(ImuMatrix), P(ImuMatrix), P(ImuParams), V, V, P(S),
                                              P(ImuPlanInfo), V]),
        "imu_noalloc_scratch_bytes": (S, []),
        "imu_prepare_operand": (I32, [P(ImuMatrix), P(ImuParams), V, V]),
        "imu_softmax_prepare": (I32, [P(ImuMatrix), P(ImuMatrix), P(ImuParams), V, V]),
        "imu_imunpack_matmul_prepared": (I32, [P(ImuMatrix), P(ImuMatrix), P(ImuParams), P(ImuPrepared),
                                               P(ImuPrepared), V, V, V, S, P(S), P(ImuPlanInfo), V]),
        "imu_init": (I32, [I64]),
        "imu_release": (I32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


EXPORTED = ("imu_init", "imu_release", "imu_stats_bytes", "imu_stats_layout", "imu_plan_bytes",
            "imu_plan_layout", "imu_workspace_fixed_bytes", "imu_quantize_rtn", "imu_plan_unpack",
            "imu_unpack", "imu_unpacked_gemm", "imu_imunpack_matmul", "imu_status_string", "imu_last_error",
            "imu_version", "imu_set_gemm_events", "imu_imunpack_matmul_noalloc", "imu_noalloc_scratch_bytes",
            "imu_prepare_operand", "imu_imunpack_matmul_prepared", "imu_softmax_prepare")


def _check(status: int):
    if status != OK:
        raise ImunpackError(status, lib().imu_last_error().decode())


# batch entries imu_init has set up per device index (the library's per-device
# context: pinned header buffer and events)
_ready = {}
_MIN_BATCH = 256


def ensure_init(device, batch: int = 1) -> None:
    """imu_init for `device` (a torch device or index) with room for `batch`
    entries; the first call also registers imu_release for interpreter exit."""
    idx = torch.device(device).index if not isinstance(device, int) else device
    if idx is None:
        idx = torch.cuda.current_device()
    if _ready.get(idx, 0) >= batch:
        return
    want = max(batch, _MIN_BATCH, _ready.get(idx, 0))
    with torch.cuda.device(idx):
        _check(lib().imu_init(want))
    if not _ready:
        atexit.register(release_all)
    _ready[idx] = want


def release_all() -> None:
    """imu_release on every device set up through this binding."""
    for idx in list(_ready):
        with torch.cuda.device(idx):
            lib().imu_release()
        del _ready[idx]


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------------
# operands and parameters
# ---------------------------------------------------------------------------

@dataclass
class Matrix:
    """A device operand as it enters C = A @ B.

    ``stored``: (srows, scols) or (batch, srows, scols) tensor, float32 or
    bfloat16, unit stride in the last dimension.  ``layout`` "normal": the
    logical matrix is ``stored``; "transposed": it is ``stored``'s transpose.
    """
    stored: torch.Tensor
    layout: str = "normal"

    def c(self) -> ImuMatrix:
        t = self.stored
        if t.dim() == 2:
            batch, bstride, sr, sc = 1, 0, t.shape[0], t.shape[1]
            ld = t.stride(0)
        elif t.dim() == 3:
            batch, sr, sc = t.shape
            bstride, ld = t.stride(0), t.stride(1)
        else:
            raise ImunpackError(ERR_INVALID_ARG, "operand must be 2-D or 3-D")
        # strides of size-1 dimensions address nothing: numpy and torch leave them arbitrary
        if t.stride(-1) != 1 and sc > 1:
            raise ImunpackError(ERR_INVALID_ARG, "operand must have unit stride in its last dimension")
        if sr == 1:
            ld = sc
        if t.dtype == torch.float32:
            dt = F32
        elif t.dtype == torch.bfloat16:
            dt = BF16
        else:
            raise ImunpackError(ERR_INVALID_ARG, f"unsupported dtype {t.dtype}")
        tr = self.layout == "transposed"
        rows, cols = (sc, sr) if tr else (sr, sc)
        return ImuMatrix(t.data_ptr(), dt, TRANSPOSED if tr else NORMAL, rows, cols, ld, batch,
                         bstride if batch > 1 else 0)

    @property
    def rows(self) -> int:
        return self.c().rows

    @property
    def cols(self) -> int:
        return self.c().cols

    @property
    def batch(self) -> int:
        return self.c().batch


def params(beta: int = 15, bits: int = 5, p: Tuple[int, int] = (95, 100), strat_a: str = "mix",
           strat_b: str = "mix", gamma: int = 2, clip: bool = False, digits: str = "auto") -> ImuParams:
    return ImuParams(beta, p[0], p[1], bits, gamma, STRATEGY[strat_a], STRATEGY[strat_b], 1 if clip else 0,
                     DIGITS[digits])


def _as_matrix(x) -> Matrix:
    return x if isinstance(x, Matrix) else Matrix(x)


# ---------------------------------------------------------------------------
# statistics and plan handles
# ---------------------------------------------------------------------------

class Stats:
    """Device statistics of one operand (percentile scale, outlier counts)."""

    def __init__(self, x: Matrix):
        m = x.c()
        self.rows, self.cols, self.batch = m.rows, m.cols, m.batch
        n = lib().imu_stats_bytes(ctypes.byref(m))
        if n == 0:
            _check(ERR_INVALID_ARG)
        self.view = ImuStatsView()
        _check(lib().imu_stats_layout(ctypes.byref(m), ctypes.byref(self.view)))
        self.buf = torch.empty(n, dtype=torch.uint8, device=x.stored.device)
        self.q: Optional[torch.Tensor] = None

    def _entry(self, b: int) -> torch.Tensor:
        s = self.view.stride
        return self.buf[b * s:(b + 1) * s]

    def header(self, b: int = 0) -> dict:
        h = self._entry(b)[:64].cpu()
        f = h[:16].view(torch.float32)
        u = h[16:32].view(torch.int32)
        return {"alpha": float(f[0]), "r": float(f[1]), "s": float(f[2]), "kth": float(f[3]),
                "maxkey": int(u[0]) & 0xFFFFFFFF, "status": int(u[1]),
                "total": int(h[32:40].view(torch.int64)[0]),
                "alpha_bits": int(h[0:4].view(torch.int32)[0]), "r_bits": int(h[4:8].view(torch.int32)[0]),
                "s_bits": int(h[8:12].view(torch.int32)[0])}

    def array(self, name: str, b: int = 0) -> torch.Tensor:
        n = self.rows if name in ("row_oob", "row_maxdig", "cr_rowdig") else self.cols
        off = getattr(self.view, name)
        return self._entry(b)[off:off + 4 * n].view(torch.int32)


class Plan:
    """Device plan buffer plus the host summary of every batch entry."""

    def __init__(self, a: Matrix, b: Matrix, p: ImuParams):
        ma, mb = a.c(), b.c()
        n = lib().imu_plan_bytes(ctypes.byref(ma), ctypes.byref(mb), ctypes.byref(p))
        if n == 0:
            _check(ERR_INVALID_ARG)
        self.view = ImuPlanView()
        _check(lib().imu_plan_layout(ctypes.byref(ma), ctypes.byref(mb), ctypes.byref(p),
                                     ctypes.byref(self.view)))
        self.buf = torch.empty(n, dtype=torch.uint8, device=a.stored.device)
        self.batch = ma.batch
        self.M, self.K, self.N = ma.rows, ma.cols, mb.cols
        self.info = (ImuPlanInfo * self.batch)()
        self.params = p

    def entry(self, b: int) -> dict:
        return self.info[b].as_dict()

    def header_raw(self, b: int = 0) -> torch.Tensor:
        s = self.view.header_stride
        return self.buf[b * s:(b + 1) * s]

    def array(self, name: str, b: int = 0) -> torch.Tensor:
        v = self.view
        base = v.headers_bytes + b * v.entry_stride + getattr(v, name)
        n = {"da_r": self.M, "da_c": self.K, "db_r": self.K, "db_c": self.N,
             "lvl_a": self.M * v.levels, "lvl_b": self.N * v.levels,
             "kpre": (self.K + 1) * v.segments, "amap": v.m_alloc_max, "bmap": v.n_alloc_max}[name]
        return self.buf[base:base + 4 * n].view(torch.int32)

    def segments(self, b: int = 0) -> Tuple[List[int], List[int]]:
        """(padded offsets, lengths) of the exponent segments of K'."""
        h = self.header_raw(b).cpu()
        n_seg = int(h[12:16].view(torch.int32)[0])
        # PlanHeader: 4 ints, 3 + 4 + 1 int64, 4 ints, 25*3 int64, then seg_off[65] int64, seg_len[64] int32
        off0 = 16 + 8 * 8 + 16 + 25 * 3 * 8
        seg_off = h[off0:off0 + 8 * 65].view(torch.int64)[:n_seg + 1].tolist()
        seg_len = h[off0 + 8 * 65:off0 + 8 * 65 + 4 * 64].view(torch.int32)[:n_seg].tolist()
        return seg_off, seg_len


# ---------------------------------------------------------------------------
# the five entry points
# ---------------------------------------------------------------------------

def quantize_rtn(x, p: ImuParams, want_q: bool = False, stream=None) -> Stats:
    """RTN quantization + outlier statistics of one operand (imu_quantize_rtn)."""
    x = _as_matrix(x)
    st = Stats(x)
    m = x.c()
    if want_q:
        st.q = torch.empty((m.batch, m.rows, m.cols), dtype=torch.int32, device=x.stored.device)
    _check(lib().imu_quantize_rtn(ctypes.byref(m), ctypes.byref(p), _ptr(st.buf), _ptr(st.q),
                                  ctypes.c_void_p(_stream(stream))))
    return st


def plan_unpack(a, b, p: ImuParams, stats_a: Stats, stats_b: Stats, stream=None) -> Plan:
    """Unpacking plan for A and B (imu_plan_unpack); waits once for the device."""
    a, b = _as_matrix(a), _as_matrix(b)
    pl = Plan(a, b, p)
    ma, mb = a.c(), b.c()
    ensure_init(a.stored.device, ma.batch)
    _check(lib().imu_plan_unpack(ctypes.byref(ma), ctypes.byref(mb), ctypes.byref(p), _ptr(stats_a.buf),
                                 _ptr(stats_b.buf), _ptr(pl.buf), pl.info, ctypes.c_void_p(_stream(stream))))
    return pl


def unpacked_bytes(plan: Plan, operand: int) -> int:
    last = plan.info[plan.batch - 1]
    rows = last.m_alloc if operand == 0 else last.n_alloc
    off = last.a_offset if operand == 0 else last.b_offset
    row_bytes = last.k_pad * 3 // 4 if last.digits == DIGITS["fp6"] else last.k_pad
    return int(off + (rows * row_bytes + 255) // 256 * 256)


def unpack(x, operand: int, p: ImuParams, stats: Stats, plan: Plan, stream=None) -> torch.Tensor:
    """Digits of one operand (imu_unpack): A' (operand 0) or B'^T (operand 1) as
    int8 bytes or fp6 codes (the plan's format, info[b].digits), all batch
    entries in one flat byte buffer at info[b].a_offset / b_offset."""
    x = _as_matrix(x)
    out = torch.empty(unpacked_bytes(plan, operand), dtype=torch.int8, device=x.stored.device)
    m = x.c()
    _check(lib().imu_unpack(ctypes.byref(m), operand, ctypes.byref(p), _ptr(stats.buf), _ptr(plan.buf),
                            plan.info, _ptr(out), ctypes.c_void_p(_stream(stream))))
    return out


def unpacked_gemm(a_u: torch.Tensor, b_u: torch.Tensor, p: ImuParams, stats_a: Stats, stats_b: Stats,
                  plan: Plan, want_out: bool = True, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """int8 MFMA GEMMs + shift-and-accumulate fold + dequant (imu_unpacked_gemm).
    Returns (C int32, out float32) shaped (batch, M, N)."""
    dev = a_u.device
    ensure_init(dev, plan.batch)
    c = torch.empty((plan.batch, plan.M, plan.N), dtype=torch.int32, device=dev)
    out = torch.empty((plan.batch, plan.M, plan.N), dtype=torch.float32, device=dev) if want_out else None
    _check(lib().imu_unpacked_gemm(_ptr(a_u), _ptr(b_u), ctypes.byref(p), _ptr(stats_a.buf), _ptr(stats_b.buf),
                                   _ptr(plan.buf), plan.info, plan.batch, _ptr(c), plan.N, plan.M * plan.N,
                                   _ptr(out), ctypes.c_void_p(_stream(stream))))
    return c, out


class Workspace:
    """Device workspace for imunpack_matmul that grows on demand (torch allocator)."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = torch.empty(0, dtype=torch.uint8, device=device)

    def ensure(self, n: int) -> torch.Tensor:
        if self.buf.numel() < n:
            self.buf = torch.empty(int(n * 1.1) + 4096, dtype=torch.uint8, device=self.device)
        return self.buf


_default_ws = {}


def imunpack_matmul(a, b, p: ImuParams, out: Optional[torch.Tensor] = None, c: Optional[torch.Tensor] = None,
                    want_out: bool = True, ws: Optional[Workspace] = None, stream=None):
    """The whole path (imu_imunpack_matmul).  Returns (out float32 or None, C int32, [info dict])."""
    a, b = _as_matrix(a), _as_matrix(b)
    ma, mb = a.c(), b.c()
    dev = a.stored.device
    ensure_init(dev, ma.batch)
    shape = (ma.batch, ma.rows, mb.cols)
    if c is None:
        c = torch.empty(shape, dtype=torch.int32, device=dev)
    if want_out and out is None:
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    if ws is None:
        ws = _default_ws.setdefault(str(dev), Workspace(dev))
    info = (ImuPlanInfo * ma.batch)()
    need = ctypes.c_size_t(0)
    for _ in range(3):
        buf = ws.buf
        st = lib().imu_imunpack_matmul(ctypes.byref(ma), ctypes.byref(mb), ctypes.byref(p), _ptr(c),
                                       _ptr(out) if want_out else None,
                                       _ptr(buf) if buf.numel() else None, buf.numel(), ctypes.byref(need),
                                       info, ctypes.c_void_p(_stream(stream)))
        if st == ERR_WORKSPACE:
            ws.ensure(need.value)
            continue
        _check(st)
        return (out if want_out else None), c, [info[i].as_dict() for i in range(ma.batch)]
    _check(ERR_WORKSPACE)


def imunpack_matmul_noalloc(a, b, p: ImuParams, out: Optional[torch.Tensor] = None,
                            c: Optional[torch.Tensor] = None, want_out: bool = True, stream=None):
    """The whole path in the library's static scratch (imu_imunpack_matmul_noalloc):
    no workspace argument.  Returns (out float32 or None, C int32, [info dict])."""
    a, b = _as_matrix(a), _as_matrix(b)
    ma, mb = a.c(), b.c()
    dev = a.stored.device
    ensure_init(dev, ma.batch)
    shape = (ma.batch, ma.rows, mb.cols)
    if c is None:
        c = torch.empty(shape, dtype=torch.int32, device=dev)
    if want_out and out is None:
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    info = (ImuPlanInfo * ma.batch)()
    need = ctypes.c_size_t(0)
    _check(lib().imu_imunpack_matmul_noalloc(ctypes.byref(ma), ctypes.byref(mb), ctypes.byref(p), _ptr(c),
                                             _ptr(out) if want_out else None, ctypes.byref(need), info,
                                             ctypes.c_void_p(_stream(stream))))
    return (out if want_out else None), c, [info[i].as_dict() for i in range(ma.batch)]


def prepare_operand(x, p: ImuParams, stream=None) -> Stats:
    """Statistics of one operand for later calls (imu_prepare_operand): scale,
    counts and the Mix residuals of both line directions."""
    x = _as_matrix(x)
    st = Stats(x)
    _check(lib().imu_prepare_operand(ctypes.byref(x.c()), ctypes.byref(p), _ptr(st.buf),
                                     ctypes.c_void_p(_stream(stream))))
    return st


def softmax_prepare(logits, p: ImuParams, p_out: Optional[torch.Tensor] = None, stream=None):
    """imu_softmax_prepare: P = row softmax of `logits` (2-D or 3-D, float32 or
    bfloat16, row-major) as bfloat16 and P's statistics.  Returns (P, Stats)."""
    z = _as_matrix(logits)
    if z.layout != "normal":
        raise ImunpackError(ERR_INVALID_ARG, "logits must be row-major (layout normal)")
    t = z.stored
    if p_out is None:
        p_out = torch.empty(t.shape, dtype=torch.bfloat16, device=t.device)
    pm = Matrix(p_out)
    st = Stats(pm)
    _check(lib().imu_softmax_prepare(ctypes.byref(z.c()), ctypes.byref(pm.c()), ctypes.byref(p), _ptr(st.buf),
                                     ctypes.c_void_p(_stream(stream))))
    return p_out, st


def _prepared(pre) -> Optional[ImuPrepared]:
    """None, a Stats (used as prepared) or a (Stats, transposed) pair."""
    if pre is None:
        return None
    st, tr = pre if isinstance(pre, tuple) else (pre, False)
    return ImuPrepared(st.buf.data_ptr(), 1 if tr else 0, 0)


def imunpack_matmul_prepared(a, b, p: ImuParams, pre_a=None, pre_b=None, out: Optional[torch.Tensor] = None,
                             c: Optional[torch.Tensor] = None, want_out: bool = True,
                             ws: Optional[Workspace] = None, stream=None):
    """imu_imunpack_matmul_prepared: pre_a / pre_b are None, a Stats from
    prepare_operand, or (Stats, transposed).  Returns (out or None, C, [info])."""
    a, b = _as_matrix(a), _as_matrix(b)
    ma, mb = a.c(), b.c()
    dev = a.stored.device
    ensure_init(dev, ma.batch)
    shape = (ma.batch, ma.rows, mb.cols)
    if c is None:
        c = torch.empty(shape, dtype=torch.int32, device=dev)
    if want_out and out is None:
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    if ws is None:
        ws = _default_ws.setdefault(str(dev), Workspace(dev))
    pa, pb = _prepared(pre_a), _prepared(pre_b)
    info = (ImuPlanInfo * ma.batch)()
    need = ctypes.c_size_t(0)
    for _ in range(3):
        buf = ws.buf
        st = lib().imu_imunpack_matmul_prepared(ctypes.byref(ma), ctypes.byref(mb), ctypes.byref(p),
                                                ctypes.byref(pa) if pa else None, ctypes.byref(pb) if pb else None,
                                                _ptr(c), _ptr(out) if want_out else None,
                                                _ptr(buf) if buf.numel() else None, buf.numel(), ctypes.byref(need),
                                                info, ctypes.c_void_p(_stream(stream)))
        if st == ERR_WORKSPACE:
            ws.ensure(need.value)
            continue
        _check(st)
        return (out if want_out else None), c, [info[i].as_dict() for i in range(ma.batch)]
    _check(ERR_WORKSPACE)


def version() -> str:
    return lib().imu_version().decode()


def set_gemm_events(before: int | None, after: int | None) -> None:
    """imu_set_gemm_events with raw hipEvent_t handles (None, None switches it off)."""
    _check(lib().imu_set_gemm_events(ctypes.c_void_p(before), ctypes.c_void_p(after)))
