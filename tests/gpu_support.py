"""Helpers shared by the GPU parity tests: upload seeded operands, run the
oracle per batch entry, and map the HIP path's padded unpacked layout back to
the canonical one.  The padded layout is the documented one (include/imunpack.h):
extra lines start at m_base / n_base, and every exponent segment of K' starts
at a multiple of 128 bytes; both are reconstructed here from the oracle's own
index maps, not read from the GPU plan arrays."""
from __future__ import annotations

import numpy as np
import torch

from oracle import imunpack_oracle as O
from outlier_unpacking_quantization_amd import binding as B
from outlier_unpacking_quantization_amd import workloads as W

KPAD = 128


def to_device(op: W.Operand) -> B.Matrix:
    s = op.stored
    if op.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(s).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(s))
    t = t.to("cuda")
    if op.batch == 1:
        t = t[0]
    return B.Matrix(t, op.layout)


def logical_f32(op: W.Operand, b: int) -> np.ndarray:
    return O.widen(op.logical_bits(b), op.dtype)


def params_of(pr: W.Problem, digits: str = "auto") -> B.ImuParams:
    return B.params(beta=pr.beta, bits=pr.bits, p=(pr.p_num, pr.p_den), strat_a=pr.strat_a,
                    strat_b=pr.strat_b, gamma=pr.gamma, clip=pr.clip, digits=digits)


def oracle_entries(pr: W.Problem, unpacked: bool = True):
    out = []
    for b in range(pr.a.batch):
        out.append(O.imunpack_matmul(logical_f32(pr.a, b), logical_f32(pr.b, b), pr.beta, pr.bits,
                                     pr.p_num, pr.p_den, pr.strat_a, pr.strat_b, pr.gamma,
                                     unpacked=unpacked, clip=pr.clip))
    return out


def padded_segment_offsets(seg_sizes) -> list:
    off = [0]
    for s in seg_sizes:
        off.append(off[-1] + -(-int(s) // KPAD) * KPAD)
    return off


def padded_line_index(lines: np.ndarray, n_orig: int, base: int) -> np.ndarray:
    """Canonical level-major index -> padded row (extra lines start at `base`)."""
    idx = np.arange(lines.shape[0])
    return np.where(idx < n_orig, idx, idx - n_orig + base)


def depth_order_col_index(cols: np.ndarray, db_c: np.ndarray, base: int) -> np.ndarray:
    """Canonical level-major B' column (n, w) -> row of B'^T as the HIP path
    lays it out (include/imunpack.h): the columns in depth order (descending
    depth, ties by index); level 0 at rows 0..N-1 in that order, level w >= 1 at
    base + (columns deeper than 1..w-1) + the column's position in the order."""
    d = np.asarray(db_c, np.int64)
    order = np.lexsort((np.arange(d.size), -d))  # depth descending, then index
    pos = np.empty(d.size, np.int64)
    pos[order] = np.arange(d.size)
    dmax = int(d.max()) if d.size else 1
    deeper = np.array([int((d > w).sum()) for w in range(dmax + 1)], np.int64)
    lvbase = np.zeros(dmax + 1, np.int64)
    for w in range(2, dmax + 1):
        lvbase[w] = lvbase[w - 1] + deeper[w - 1]
    n, w = cols[:, 0], cols[:, 1]
    return np.where(w == 0, pos[n], base + lvbase[np.minimum(w, dmax)] + pos[n])


def padded_k_index(trip: np.ndarray) -> np.ndarray:
    """Canonical K' index (sorted by e, k, v) -> padded column."""
    sizes = np.bincount(trip[:, 3]) if trip.size else np.zeros(0, int)
    off = padded_segment_offsets(sizes)
    start = np.concatenate([[0], np.cumsum(sizes)])
    e = trip[:, 3]
    return np.array(off)[e] + (np.arange(trip.shape[0]) - start[e])


def untile_a(flat: np.ndarray, m_alloc: int, kp: int) -> np.ndarray:
    """A' as stored (MFMA fragment order, include/imunpack.h) -> row-major m_alloc x kp.

    Block (row block rb, K' block c) is 1 KB at (rb * kp/32 + c) * 1024; inside
    it, 16-byte half h of row r of the block is lane r + 32 h."""
    t = np.asarray(flat).reshape(m_alloc // 32, kp // 32, 2, 32, 16)  # rb, c, h, r, byte
    return t.transpose(0, 3, 1, 2, 4).reshape(m_alloc, kp)


# e2m3 (fp6) codes of the integers 0..7: 1 sign, 2 exponent (bias 1) and 3
# mantissa bits, value 2^(e-1) (1 + m/8) for e > 0 and m/8 for e = 0.  The
# table is derived from that definition here, so it pins the HIP side's table.
def _e2m3_value(code: int) -> float:
    e, m = (code >> 3) & 3, code & 7
    v = m / 8.0 if e == 0 else 2.0 ** (e - 1) * (1 + m / 8.0)
    return -v if code & 0x20 else v


E2M3_DIGIT = np.full(64, 99, np.int64)  # 99: a code that is no integer digit, or a signed zero
for _c in range(64):
    _v = _e2m3_value(_c)
    if _v == int(_v) and (_v != 0 or _c == 0):
        E2M3_DIGIT[_c] = int(_v)


def fp6_digits(codes: np.ndarray) -> np.ndarray:
    """e2m3 codes -> integer digits, 99 for a code that is no integer digit
    (or a negative zero: zero digits are stored as code 0), which no oracle
    digit equals.  Rows past the valid ones are never written and may hold
    anything."""
    return E2M3_DIGIT[np.asarray(codes, np.int64)]


def unpack_6bit(rows: np.ndarray, n: int) -> np.ndarray:
    """Byte rows holding 6-bit fields (field j at bits [6j, 6j + 6), little
    endian) -> the first n fields of each row."""
    bits = np.unpackbits(np.ascontiguousarray(rows, np.uint8), axis=-1, bitorder="little")
    f = bits[..., :6 * n].reshape(*rows.shape[:-1], n, 6).astype(np.int64)
    return (f << np.arange(6)).sum(-1)


def b_rows(b_u: np.ndarray, info: dict) -> np.ndarray:
    """B'^T as stored -> n_alloc x k_pad integer digits (int8 bytes, or fp6
    bit-stream rows of 3/4 k_pad bytes)."""
    n, kp = info["n_alloc"], info["k_pad"]
    if info["digits"] == B.DIGITS["fp6"]:
        raw = np.asarray(b_u)[:n * kp * 3 // 4].view(np.uint8).reshape(n, kp * 3 // 4)
        return fp6_digits(unpack_6bit(raw, kp))
    return np.asarray(b_u)[:n * kp].view(np.int8).reshape(n, kp).astype(np.int64)


def a_rows(a_u: np.ndarray, info: dict) -> np.ndarray:
    """A' as stored (MFMA fragment order) -> m_alloc x k_pad integer digits.

    int8: untile_a.  fp6: blocks of 32 rows x 64 positions, 1536 bytes, at
    (rb * k_pad/64 + c) * 1536; inside, lane r + 32 h holds 24 bytes: the 6-bit
    codes of positions 32 h .. 32 h + 31 of the block's row r."""
    m, kp = info["m_alloc"], info["k_pad"]
    if info["digits"] == B.DIGITS["fp6"]:
        raw = np.asarray(a_u)[:m * kp * 3 // 4].view(np.uint8).reshape(m // 32, kp // 64, 2, 32, 24)
        codes = unpack_6bit(raw, 32)  # rb, c, h, r, j
        return fp6_digits(codes.transpose(0, 3, 1, 2, 4).reshape(m, kp))
    return untile_a(np.asarray(a_u)[:m * kp].view(np.int8), m, kp).astype(np.int64)


def ulp_diff(a: np.ndarray, b: np.ndarray) -> int:
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return int(np.abs(ia - ib).max(initial=0))


def f32_bits(x) -> int:
    return int(np.float32(x).view(np.int32))
