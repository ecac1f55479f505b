"""CPU oracle for the IM-Unpack integer GEMM path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run this module.  The product path (the HIP
library and its Python binding) never calls it and shares no code with it.

Source: the summary page "IM-Unpack: Training and Inference with Arbitrarily
Low Precision Integers" (atlas.scime.ai).  The page fixes what is computed:

* round-to-nearest (RTN) integer quantization with a scale chosen so that a
  p-percentile magnitude maps to the integer beta ("Measured effects" table:
  p=95%, beta=15/31; p=100% restricts every value to the range);
* heavy hitters stay as out-of-range integers, they are not clipped
  (summary paragraph and "Problem");
* each out-of-range integer is split into several in-range narrow integers
  held in added rows or columns, the row/column choice made for each matrix
  from how many outliers its lines hold; narrow-integer products, each
  multiplied by a power of two and summed, then give back the integer product
  without error ("Approach");
* the Mix strategy beats every fixed row/column pairing ("Measured effects"
  table, unpack-ratio rows).

The page gives no formula for the percentile, the in-range interval, the digit
base, the Mix rule or the layout of the unpacked matrices.  This oracle takes
one reading of each (numbered R-1 ... R-17 in the docstrings below, the same
numbering the design notes use) and implements it plainly:

* integer arithmetic is int64 (Python integers where int64 could overflow);
* the quantizer's decisions are taken in IEEE binary32, the precision the
  HIP kernels use, so that a quantized code is decided the same way on both
  sides;
* every matrix product is a library matmul whose exactness is guaranteed by
  a magnitude bound checked before the call (float64 BLAS when every partial
  sum is an integer below 2**53, int64 below 2**62, Python integers above).

Pins (tests/test_oracle_*.py) check every step against brute force, exact
rational arithmetic, closed forms and the exactness invariant.  The plan
choice (Mix rule) has no value on the page to compare with: parity with the
paper's own plans is unpinned; only its invariants are pinned.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

# status codes, same meaning as the C ABI's (values are part of the contract)
OK, ERR_INVALID_ARG, ERR_NONFINITE, ERR_RANGE = 0, 1, 2, 3

CANDIDATE_ORDER = ("row", "col", "cr", "rc", "greedy")  # tie order of the joint choice (R-7)
ALLOWED = {"row": ("row",), "col": ("col",), "mix": ("row", "col", "cr", "rc"), "greedy": ("greedy",)}


class OracleError(Exception):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


# ----------------------------------------------------------------------------
# input widening
# ----------------------------------------------------------------------------

def widen(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Stored operand -> float32 values.  bfloat16 is the top half of binary32,
    so widening is exact: the 16 stored bits become the high half of the word."""
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32)
    if dtype == "bf16":
        bits = np.asarray(stored, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32)
    raise OracleError(ERR_INVALID_ARG, f"dtype {dtype}")


# ----------------------------------------------------------------------------
# O1-O3: percentile, scale, RTN   (page: "Measured effects" table, p and beta rows)
# ----------------------------------------------------------------------------

def percentile_rank(count: int, p_num: int, p_den: int) -> int:
    """R-1 nearest rank: k = ceil(p * N) with p = p_num / p_den held exactly, clamped to [1, N]."""
    k = -((-p_num * count) // p_den)
    return min(max(k, 1), count)


@dataclass
class Scale:
    alpha: np.float32  # the p-percentile magnitude (after the R-2 fallback)
    r: np.float32  # multiplier that quantizes: q = rne(fl32(x * r))
    s: np.float32  # dequantization step alpha / beta
    kth: np.float32  # the raw k-th smallest |x| before the fallback
    maxabs: np.float32


def percentile_scale(x32: np.ndarray, beta: int, p_num: int, p_den: int) -> Scale:
    """O1 + O2 for one matrix.

    alpha = k-th smallest |x| (R-1).  If alpha is 0 the largest |x| is used; if
    that is 0 too the matrix is all zeros and r = s = 0 (R-2).  Non-finite
    input is rejected (R-3).  r = fl32(beta / alpha) and s = fl32(alpha / beta),
    each one IEEE binary32 division (R-4).
    """
    a = np.abs(np.asarray(x32, dtype=np.float32)).ravel()
    if a.size == 0:
        raise OracleError(ERR_INVALID_ARG, "empty matrix")
    if not np.all(np.isfinite(a)):
        raise OracleError(ERR_NONFINITE, "non-finite input")
    k = percentile_rank(a.size, p_num, p_den)
    kth = np.partition(a, k - 1)[k - 1]
    maxabs = a.max()
    alpha = kth if kth > 0 else maxabs
    if alpha == 0:
        z = np.float32(0)
        return Scale(z, z, z, kth, maxabs)
    r = np.float32(beta) / np.float32(alpha)
    s = np.float32(alpha) / np.float32(beta)
    return Scale(np.float32(alpha), np.float32(r), np.float32(s), kth, maxabs)


def rtn(x32: np.ndarray, r: np.float32) -> np.ndarray:
    """O3: y = fl32(x * r) (one binary32 product), q = round-half-to-even(y).

    No clipping: heavy hitters keep their large integer (page summary and
    "Problem").  |y| >= 2**31 cannot be held as an int32 code and is an error.
    """
    with np.errstate(over="ignore"):
        y = np.asarray(x32, dtype=np.float32) * np.float32(r)
    if y.size and np.abs(y).max() >= np.float32(2.0 ** 31):
        raise OracleError(ERR_RANGE, "|x * r| >= 2**31")
    return np.rint(y).astype(np.int64)


def rtn_clipped(x32: np.ndarray, r: np.float32, beta: int) -> np.ndarray:
    """R-13: the clipping quantizer of the page's ablation rows ("Measured
    effects" table, the 99.5-percentile clipping row, set against p = 100% with
    beta = 255, R-14): the RTN code of fl32(x * r), rounded half to even, then
    clamped to [-beta, beta].  A product that overflows binary32 is clamped like
    any other code beyond beta."""
    with np.errstate(over="ignore"):
        y = np.asarray(x32, dtype=np.float32) * np.float32(r)
    return np.clip(np.rint(y), -beta, beta).astype(np.int64)


# ----------------------------------------------------------------------------
# O4-O5: digits and outlier statistics   (page: "Approach")
# ----------------------------------------------------------------------------

def digit_base(bits: int) -> int:
    """R-5: an in-range code is a symmetric signed b-bit integer, |q| <= 2**(b-1) - 1,
    and unpacking uses sign-magnitude digits in base S = 2**(b-1)."""
    return 1 << (bits - 1)


def max_digits(bits: int) -> int:
    """Largest digit count of a code with |q| < 2**31."""
    return -(-31 // (bits - 1))


def digit_count(q: np.ndarray, bits: int) -> np.ndarray:
    """n(q): 1 if |q| < S, else 1 + n(|q| // S) -- the number of base-S digits."""
    S = digit_base(bits)
    m = np.abs(np.asarray(q, dtype=np.int64)) // S
    n = np.ones(m.shape, dtype=np.int64)
    while np.any(m > 0):
        n += (m > 0)
        m //= S
    return n


def digit(q: np.ndarray, bits: int, t: int) -> np.ndarray:
    """digit_t(q) = sign(q) * (floor(|q| / S**t) mod S), so that sum_t digit_t * S**t = q."""
    S = digit_base(bits)
    q = np.asarray(q, dtype=np.int64)
    mag = (np.abs(q) // (S ** t)) % S
    return np.sign(q) * mag


@dataclass
class LineStats:
    row_oob: np.ndarray  # out-of-range codes per row
    col_oob: np.ndarray  # per column
    row_maxdig: np.ndarray  # largest digit count per row
    col_maxdig: np.ndarray
    total: int  # T: out-of-range codes in the matrix


def line_stats(n: np.ndarray) -> LineStats:
    """O5: a code is out of range iff it needs two or more digits.  Rows and
    columns are those of the operand as it enters C = A @ B."""
    oob = (n >= 2)
    return LineStats(oob.sum(axis=1).astype(np.int64), oob.sum(axis=0).astype(np.int64),
                     n.max(axis=1).astype(np.int64), n.max(axis=0).astype(np.int64),
                     int(oob.sum()))


# ----------------------------------------------------------------------------
# O6-O7: candidate depth maps and the joint choice   (page: "Approach", Mix rows)
# ----------------------------------------------------------------------------

def candidates(n: np.ndarray, st: LineStats, strategy: str, gamma: int = 2
               ) -> Dict[str, Tuple[np.ndarray, np.ndarray]]:
    """R-7: depth maps (d_r per row, d_c per column) of each allowed candidate.

    row: every row gets its largest digit count, columns stay single.
    col: the mirror image.
    cr : heavy columns H_c = {k : col_oob[k] * C > gamma * T} take their largest
         digit count; every row then takes the largest digit count over the
         columns outside H_c (at least 1).
    rc : the mirror of cr with heavy rows H_r = {i : row_oob[i] * R > gamma * T}.
    greedy: the line-at-a-time depths of greedy_depths (strategy "greedy" only).
    Every candidate covers every code: d_r[i] + d_c[k] - 1 >= n[i, k].
    """
    R, C = n.shape
    out: Dict[str, Tuple[np.ndarray, np.ndarray]] = {}
    for name in ALLOWED[strategy]:
        if name == "row":
            d_r, d_c = st.row_maxdig.copy(), np.ones(C, np.int64)
        elif name == "col":
            d_r, d_c = np.ones(R, np.int64), st.col_maxdig.copy()
        elif name == "cr":
            heavy = st.col_oob * C > gamma * st.total
            d_c = np.where(heavy, st.col_maxdig, 1)
            rest = n[:, ~heavy]
            d_r = np.maximum(1, rest.max(axis=1)) if rest.shape[1] else np.ones(R, np.int64)
        elif name == "rc":
            heavy = st.row_oob * R > gamma * st.total
            d_r = np.where(heavy, st.row_maxdig, 1)
            rest = n[~heavy, :]
            d_c = np.maximum(1, rest.max(axis=0)) if rest.shape[0] else np.ones(C, np.int64)
        elif name == "greedy":
            d_r, d_c = greedy_depths(n)
        else:
            raise OracleError(ERR_INVALID_ARG, name)
        out[name] = (d_r.astype(np.int64), d_c.astype(np.int64))
    return out


def greedy_depths(n: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """R-15: line-at-a-time unpacking (the page's per-matrix choice from
    outlier counts, "Approach", read as a greedy): all depths start at 1; while some code is not
    covered (n[i, k] > d_r[i] + d_c[k] - 1), the line holding the most
    uncovered codes gets one more level, rows before columns and lower indices
    first on equal counts.  Raising row i to depth d covers exactly the codes
    with n[i, k] = d + d_c[k] - 1 (they needed one more level than the row
    had), so the counts are updated along that line only."""
    R, C = n.shape
    d_r = np.ones(R, np.int64)
    d_c = np.ones(C, np.int64)
    unc = n > 1
    cnt_r = unc.sum(axis=1).astype(np.int64)
    cnt_c = unc.sum(axis=0).astype(np.int64)
    while True:
        mr = int(cnt_r.max()) if R else 0
        mc = int(cnt_c.max()) if C else 0
        if max(mr, mc) == 0:
            return d_r, d_c
        if mr >= mc:
            i = int(np.argmax(cnt_r))  # first line with the largest count
            d_r[i] += 1
            newly = n[i, :] == d_r[i] + d_c - 1
            cnt_c -= newly
            cnt_r[i] -= int(newly.sum())
        else:
            k = int(np.argmax(cnt_c))
            d_c[k] += 1
            newly = n[:, k] == d_r + d_c[k] - 1
            cnt_r -= newly
            cnt_c[k] -= int(newly.sum())


@dataclass
class Choice:
    cand_a: str
    cand_b: str
    m_u: int  # M' = sum of A's row depths
    k_u: int  # K' = sum over k of (A's column depth) * (B's row depth)
    n_u: int  # N' = sum of B's column depths
    table: Dict[Tuple[str, str], Tuple[int, int, int]] = field(default_factory=dict)


def unpacked_sizes(da_r, da_c, db_r, db_c) -> Tuple[int, int, int]:
    return int(np.sum(da_r)), int(np.sum(da_c * db_r)), int(np.sum(db_c))


def joint_choice(cand_a, cand_b) -> Choice:
    """R-7: the allowed pair with the smallest M'*K'*N'; ties go to the first pair
    in A-major order row < col < cr < rc."""
    best = None
    table = {}
    for na in CANDIDATE_ORDER:
        if na not in cand_a:
            continue
        for nb in CANDIDATE_ORDER:
            if nb not in cand_b:
                continue
            m_u, k_u, n_u = unpacked_sizes(cand_a[na][0], cand_a[na][1], cand_b[nb][0], cand_b[nb][1])
            table[(na, nb)] = (m_u, k_u, n_u)
            cost = m_u * k_u * n_u  # Python integers: exact
            if best is None or cost < best[0]:
                best = (cost, na, nb, m_u, k_u, n_u)
    _, na, nb, m_u, k_u, n_u = best
    return Choice(na, nb, m_u, k_u, n_u, table)


# ----------------------------------------------------------------------------
# O8-O10: index maps and unpacked operands
# ----------------------------------------------------------------------------

def level_lines(d: np.ndarray) -> np.ndarray:
    """R-8 level-major line order: for level u = 0, 1, ... every line with depth > u
    in ascending order.  Returns (L', 2) rows of (line, level); the first len(d)
    entries are the original lines at level 0."""
    out = []
    for u in range(int(d.max()) if d.size else 0):
        idx = np.nonzero(d > u)[0]
        out.append(np.stack([idx, np.full(idx.size, u)], axis=1))
    return np.concatenate(out).astype(np.int64) if out else np.zeros((0, 2), np.int64)


def k_triples(da_c: np.ndarray, db_r: np.ndarray) -> np.ndarray:
    """R-8 order of the unpacked inner dimension: triples (k, v, v') with v < A's
    depth of column k and v' < B's depth of row k, sorted by exponent e = v + v',
    then k, then v.  Returns (K', 4) rows of (k, v, v', e); the e = 0 segment is
    exactly the original K columns."""
    out = []
    emax = int((da_c.max() - 1) + (db_r.max() - 1)) if da_c.size else -1
    for e in range(emax + 1):
        ks, vs = [], []
        for v in range(e + 1):
            k = np.nonzero((v < da_c) & (e - v < db_r))[0]
            ks.append(k)
            vs.append(np.full(k.size, v))
        k, v = np.concatenate(ks), np.concatenate(vs)
        order = np.lexsort((v, k))  # by k, then v
        k, v = k[order], v[order]
        out.append(np.stack([k, v, e - v, np.full(k.size, e)], axis=1))
    return np.concatenate(out).astype(np.int64) if out else np.zeros((0, 4), np.int64)


def _positions(lines: np.ndarray, n_lines: int, depth_max: int) -> np.ndarray:
    pos = np.full((n_lines, max(depth_max, 1)), -1, np.int64)
    pos[lines[:, 0], lines[:, 1]] = np.arange(lines.shape[0])
    return pos


def _triple_positions(trip: np.ndarray, K: int, da_max: int, db_max: int) -> np.ndarray:
    pos = np.full((K, max(da_max, 1), max(db_max, 1)), -1, np.int64)
    pos[trip[:, 0], trip[:, 1], trip[:, 2]] = np.arange(trip.shape[0])
    return pos


def placement(t: int, d_k: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """R-9 "inner line first" placement of digit t of a code whose inner (K-side)
    line has depth d_k: K-side index min(t, d_k - 1), outer index the rest."""
    kv = np.minimum(t, d_k - 1)
    return kv, t - kv


def unpack_a(qA: np.ndarray, bits: int, da_r, da_c, db_r, rows_a, trip) -> np.ndarray:
    """O9-O10 for A (M x K): A'[(i,u), (k,v,v')] = digit placed at (u, v) of entry
    (i, k), repeated for every v' < B's depth of row k.  Returns M' x K' int8
    (every digit lies in [-(S-1), S-1] with S <= 128)."""
    M, K = qA.shape
    n = digit_count(qA, bits)
    rowpos = _positions(rows_a, M, int(da_r.max()))
    tpos = _triple_positions(trip, K, int(da_c.max()), int(db_r.max()))
    Ap = np.zeros((rows_a.shape[0], trip.shape[0]), np.int8)
    ii, kk = np.meshgrid(np.arange(M), np.arange(K), indexing="ij")
    for t in range(int(n.max())):
        dg = digit(qA, bits, t)
        kv, u = placement(t, np.broadcast_to(da_c[None, :], qA.shape))
        live = dg != 0
        if np.any(u[live] >= da_r[ii[live]]):
            raise AssertionError("plan does not cover a digit of A")
        for vp in range(int(db_r.max())):
            m = live & (vp < db_r[None, :])
            Ap[rowpos[ii[m], u[m]], tpos[kk[m], kv[m], vp]] = dg[m]
    return Ap


def unpack_b(qB: np.ndarray, bits: int, db_r, db_c, da_c, cols_b, trip) -> np.ndarray:
    """O9-O10 for B (K x N): B'[(k,v,v'), (n,w)] = digit placed at (v', w) of entry
    (k, n), repeated for every v < A's depth of column k.  Returns K' x N' int8."""
    K, N = qB.shape
    n = digit_count(qB, bits)
    colpos = _positions(cols_b, N, int(db_c.max()))
    tpos = _triple_positions(trip, K, int(da_c.max()), int(db_r.max()))
    Bp = np.zeros((trip.shape[0], cols_b.shape[0]), np.int8)
    kk, nn = np.meshgrid(np.arange(K), np.arange(N), indexing="ij")
    for t in range(int(n.max())):
        dg = digit(qB, bits, t)
        kv, w = placement(t, np.broadcast_to(db_r[:, None], qB.shape))
        live = dg != 0
        if np.any(w[live] >= db_c[nn[live]]):
            raise AssertionError("plan does not cover a digit of B")
        for v in range(int(da_c.max())):
            m = live & (v < da_c[:, None])
            Bp[tpos[kk[m], v, kv[m]], colpos[nn[m], w[m]]] = dg[m]
    return Bp


# ----------------------------------------------------------------------------
# O11-O15: low bit-width GEMMs, shift-and-accumulate, int32 result, dequant
# ----------------------------------------------------------------------------

def exact_matmul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Integer matrix product, exact.  Chooses the arithmetic from the bound
    max|a| * max|b| * K on every partial sum: float64 BLAS below 2**53 (all
    partial sums are then exactly representable integers), int64 below 2**62,
    Python integers otherwise."""
    if a.shape[1] == 0 or a.size == 0 or b.size == 0:
        return np.zeros((a.shape[0], b.shape[1]), np.int64)
    amax = max(abs(int(a.min())), abs(int(a.max())))
    bmax = max(abs(int(b.min())), abs(int(b.max())))
    bound = amax * bmax * a.shape[1]
    if bound < 2 ** 53:
        return np.rint(a.astype(np.float64) @ b.astype(np.float64)).astype(np.int64)
    if bound < 2 ** 62:
        return a.astype(np.int64) @ b.astype(np.int64)
    return a.astype(object) @ b.astype(object)


def segment_products(Ap: np.ndarray, Bp: np.ndarray, trip: np.ndarray, bits: int,
                     big: bool = False) -> np.ndarray:
    """O11: P_e = A'[:, K'_e] @ B'[K'_e, :] for every exponent segment e, then
    P = sum_e S**e * P_e (power-of-two scaling and summation, "Approach" section)."""
    S = digit_base(bits)
    P = np.zeros((Ap.shape[0], Bp.shape[1]), object if big else np.int64)
    for e in np.unique(trip[:, 3]) if trip.size else []:
        sel = trip[:, 3] == e
        Pe = exact_matmul(Ap[:, sel], Bp[sel, :])
        P = P + (Pe.astype(object) * (S ** int(e)) if big else Pe * (S ** int(e)))
    return P


def fold(P: np.ndarray, rows_a: np.ndarray, cols_b: np.ndarray, M: int, N: int, bits: int,
         big: bool = False) -> np.ndarray:
    """O12: C[i, n] = sum over unpacked rows (i, u) and columns (n, w) of
    S**(u + w) * P[(i,u), (n,w)] (the accumulation back to the original shape)."""
    S = digit_base(bits)
    dt = object if big else np.int64
    scale_r = np.array([S ** int(u) for u in rows_a[:, 1]], dtype=dt)
    scale_c = np.array([S ** int(w) for w in cols_b[:, 1]], dtype=dt)
    Cr = np.zeros((M, P.shape[1]), dt)
    np.add.at(Cr, rows_a[:, 0], P * scale_r[:, None])
    C = np.zeros((N, M), dt)
    np.add.at(C, cols_b[:, 0], (Cr * scale_c[None, :]).T)
    return C.T


def direct_product(qA: np.ndarray, qB: np.ndarray) -> np.ndarray:
    """O13: the original integer GEMM C = A_q @ B_q, exact."""
    return exact_matmul(qA, qB)


def wrap_int32(C: np.ndarray) -> np.ndarray:
    """O14: C mod 2**32 as two's-complement int32 (R-10)."""
    if C.dtype == object:
        w = np.array([(int(v) + 2 ** 31) % 2 ** 32 - 2 ** 31 for v in C.ravel()], np.int64)
        return w.reshape(C.shape).astype(np.int32)
    return (((C.astype(np.int64) + 2 ** 31) % 2 ** 32) - 2 ** 31).astype(np.int32)


def dequant(C32: np.ndarray, sA: np.float32, sB: np.float32) -> np.ndarray:
    """O15 (R-10): out = fl32(fl32(C32) * fl32(sA * sB)), each step one binary32 rounding."""
    sab = np.float32(np.float32(sA) * np.float32(sB))
    return (np.asarray(C32, dtype=np.int32).astype(np.float32) * sab).astype(np.float32)


# ----------------------------------------------------------------------------
# whole path for one problem
# ----------------------------------------------------------------------------

@dataclass
class Quantized:
    scale: Scale
    q: np.ndarray
    n: np.ndarray
    stats: LineStats


def quantize(x32: np.ndarray, beta: int, p_num: int, p_den: int, bits: int, clip: bool = False) -> Quantized:
    """O1-O5 for one matrix; `clip` selects the clipping quantizer (rtn_clipped)."""
    sc = percentile_scale(x32, beta, p_num, p_den)
    if sc.alpha == 0:
        q = np.zeros(x32.shape, np.int64)
    else:
        q = rtn_clipped(x32, sc.r, beta) if clip else rtn(x32, sc.r)
    n = digit_count(q, bits)
    return Quantized(sc, q, n, line_stats(n))


@dataclass
class Plan:
    choice: Choice
    da_r: np.ndarray
    da_c: np.ndarray
    db_r: np.ndarray
    db_c: np.ndarray
    rows_a: np.ndarray  # (M', 2) (i, u)
    cols_b: np.ndarray  # (N', 2) (n, w)
    trip: np.ndarray  # (K', 4) (k, v, v', e)

    @property
    def segment_sizes(self) -> np.ndarray:
        if self.trip.shape[0] == 0:
            return np.zeros(0, np.int64)
        return np.bincount(self.trip[:, 3])


def plan(qa: Quantized, qb: Quantized, strat_a: str, strat_b: str, gamma: int = 2) -> Plan:
    ca = candidates(qa.n, qa.stats, strat_a, gamma)
    cb = candidates(qb.n, qb.stats, strat_b, gamma)
    ch = joint_choice(ca, cb)
    da_r, da_c = ca[ch.cand_a]
    db_r, db_c = cb[ch.cand_b]
    return Plan(ch, da_r, da_c, db_r, db_c, level_lines(da_r), level_lines(db_c),
                k_triples(da_c, db_r))


@dataclass
class Result:
    qa: Quantized
    qb: Quantized
    plan: Plan
    unpack_ratio: float
    C: np.ndarray  # exact int64 (object when it exceeds int64)
    C32: np.ndarray
    out: np.ndarray
    Ap: Optional[np.ndarray] = None
    Bp: Optional[np.ndarray] = None
    C_unpacked: Optional[np.ndarray] = None


def imunpack_matmul(a32: np.ndarray, b32: np.ndarray, beta: int, bits: int, p_num: int = 95,
                    p_den: int = 100, strat_a: str = "mix", strat_b: str = "mix",
                    gamma: int = 2, unpacked: bool = True, clip: bool = False) -> Result:
    """The whole path for one (non-batched) problem C = A @ B.

    With ``unpacked`` the low bit-width route (O9-O12) is run as well and its
    result is checked against the direct product (O13, the page's exactness
    claim); without it only the direct product is formed.
    """
    if not 2 <= bits <= 8:
        raise OracleError(ERR_INVALID_ARG, "bits must be in [2, 8]")
    if beta < 1 or not (0 < p_num <= p_den):
        raise OracleError(ERR_INVALID_ARG, "beta >= 1 and 0 < p <= 1 required")
    qa = quantize(a32, beta, p_num, p_den, bits, clip)
    qb = quantize(b32, beta, p_num, p_den, bits, clip)
    pl = plan(qa, qb, strat_a, strat_b, gamma)
    M, K = qa.q.shape
    N = qb.q.shape[1]
    ch = pl.choice
    ratio = (ch.m_u * ch.k_u * ch.n_u) / (M * K * N)
    C = direct_product(qa.q, qb.q)
    big = C.dtype == object
    res = Result(qa, qb, pl, ratio, C, wrap_int32(C), None)
    res.out = dequant(res.C32, qa.scale.s, qb.scale.s)
    if unpacked:
        Ap = unpack_a(qa.q, bits, pl.da_r, pl.da_c, pl.db_r, pl.rows_a, pl.trip)
        Bp = unpack_b(qb.q, bits, pl.db_r, pl.db_c, pl.da_c, pl.cols_b, pl.trip)
        P = segment_products(Ap, Bp, pl.trip, bits, big)
        Cu = fold(P, pl.rows_a, pl.cols_b, M, N, bits, big)
        if not np.array_equal(np.asarray(Cu, dtype=object), np.asarray(C, dtype=object)):
            raise AssertionError("unpacked GEMM + fold differs from the direct product")
        res.Ap, res.Bp, res.C_unpacked = Ap, Bp, Cu
    return res


# ----------------------------------------------------------------------------
# row softmax of attention logits (the P of the attention-output GEMM P.V)
# ----------------------------------------------------------------------------
# The page's attention-output GEMMs ("Key results", third bullet; the
# "Measured effects" row that quantizes all GEMMs) multiply the softmax
# probabilities P by V.  The page fixes no softmax arithmetic.  R-17: P is the
# binary32 softmax of each row of logits, rounded to bf16, with every step
# fixed so that one result is defined:
#
#   m   = the largest logit of the row (NaNs ignored, as IEEE maxNum);
#   t   = x - m, y = t * L with L = binary32(log2 e), both rounded;
#   e   = 0 when y < -100, else 2^n * poly(f) with n = y rounded to the nearest
#         integer (ties to even) and f = y - n (exact): poly is the Taylor
#         polynomial of 2^f = exp(f ln 2) to degree 7, coefficients
#         binary32((ln 2)^k / k!), evaluated by Horner with a rounded product
#         and a rounded sum per step (no fused multiply-add);
#   S   = the sum of the row's e: the row is taken in chunks of 256 positions;
#         "lane" l (0..63) adds, in order, positions 256 j + 4 l + c for
#         j = 0, 1, ... and c = 0..3 (those inside the row) to a binary32 sum
#         that starts at 0; the 64 lane sums are then halved pairwise
#         (lanes l and l + 32, then l and l + 16, ... down to 1);
#   P   = e / S rounded to binary32, then to bf16 (nearest, ties to even; any
#         NaN becomes the quiet NaN 0x7FC0).
#
# A row holding a NaN or +Inf gives a NaN row (the statistics then report a
# non-finite operand); -Inf logits give P = 0 (masked positions).
# Pins: tests/test_oracle_softmax.py.

SOFTMAX_LOG2E = np.float32(1.4426950408889634)
SOFTMAX_EXP_CUT = -100.0
SOFTMAX_LANES, SOFTMAX_CHUNK = 64, 4


def exp2_coefficients() -> List[np.float32]:
    """binary32((ln 2)^k / k!) for k = 0..7 (R-17)."""
    import math
    return [np.float32(math.log(2.0) ** k / math.factorial(k)) for k in range(8)]


def softmax_exp(t: np.ndarray) -> np.ndarray:
    """e = exp(t) for binary32 t <= 0 (or NaN) by the steps of R-17."""
    t = np.asarray(t, dtype=np.float32)
    y = (t * SOFTMAX_LOG2E).astype(np.float32)
    e = np.zeros_like(y)
    nan = np.isnan(y)
    e[nan] = np.float32(np.nan)
    live = ~nan & ~(y < np.float32(SOFTMAX_EXP_CUT))
    yl = y[live]
    n = np.rint(yl).astype(np.float32)
    f = (yl - n).astype(np.float32)
    c = exp2_coefficients()
    p = np.full_like(f, c[7])
    for k in range(6, -1, -1):
        p = ((p * f).astype(np.float32) + c[k]).astype(np.float32)
    e[live] = np.ldexp(p, n.astype(np.int32)).astype(np.float32)
    return e


def softmax_row_sum(e: np.ndarray) -> np.float32:
    """S of R-17: per-lane sums in chunk order, then the pairwise halving over the 64 lanes."""
    e = np.asarray(e, dtype=np.float32)
    n = e.shape[0]
    span = SOFTMAX_LANES * SOFTMAX_CHUNK
    J = max(1, -(-n // span))
    padded = np.zeros(J * span, dtype=np.float32)  # +0 leaves a sum of non-negative terms unchanged
    padded[:n] = e
    lanes = padded.reshape(J, SOFTMAX_LANES, SOFTMAX_CHUNK).transpose(1, 0, 2).reshape(SOFTMAX_LANES, -1)
    v = np.add.accumulate(lanes, axis=1, dtype=np.float32)[:, -1]  # left to right, binary32
    s = SOFTMAX_LANES // 2
    while s >= 1:
        v = (v[:s] + v[s:2 * s]).astype(np.float32)
        s //= 2
    return np.float32(v[0])


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 bits, nearest with ties to even; NaN -> 0x7FC0."""
    x = np.atleast_1d(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[np.isnan(x)] = np.uint16(0x7FC0)
    return r


def softmax_f32(row: np.ndarray) -> np.ndarray:
    """e / S of R-17 for one row of binary32 logits, before the bf16 rounding."""
    row = np.asarray(row, dtype=np.float32)
    m = np.fmax.reduce(row) if row.size else np.float32(0)
    with np.errstate(invalid="ignore", divide="ignore"):
        t = (row - np.float32(m)).astype(np.float32)
        e = softmax_exp(t)
        S = softmax_row_sum(e)
        return (e / S).astype(np.float32)


def softmax_bf16(logits: np.ndarray) -> np.ndarray:
    """P of R-17 for every row of ``logits`` (rows x cols, binary32): bf16 bits."""
    z = np.asarray(logits, dtype=np.float32)
    out = np.empty(z.shape, dtype=np.uint16)
    for i in range(z.shape[0]):
        out[i] = f32_to_bf16_rne(softmax_f32(z[i]))
    return out
