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


def params_of(pr: W.Problem) -> B.ImuParams:
    return B.params(beta=pr.beta, bits=pr.bits, p=(pr.p_num, pr.p_den), strat_a=pr.strat_a,
                    strat_b=pr.strat_b, gamma=pr.gamma, clip=pr.clip)


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


def ulp_diff(a: np.ndarray, b: np.ndarray) -> int:
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return int(np.abs(ia - ib).max(initial=0))


def f32_bits(x) -> int:
    return int(np.float32(x).view(np.int32))
