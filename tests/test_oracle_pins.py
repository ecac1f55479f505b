"""Pins of the CPU oracle against things other than itself.

Every check here uses an independent route: brute force over tiny inputs in
plain Python integers, exact rational arithmetic (``fractions.Fraction``)
with a rounding-to-binary32 routine written here from the IEEE definition,
closed forms, the page's exactness claim, and hand-worked examples stored in
``tests/golden``.  Source page: "IM-Unpack: Training and Inference with
Arbitrarily Low Precision Integers" (summary, "Approach", "Measured effects").
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import imunpack_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent helpers
# ---------------------------------------------------------------------------

def f32_round(x: Fraction) -> np.float32:
    """Round an exact rational to the nearest binary32 value, ties to even
    (normal and subnormal range), straight from the definition."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    m = abs(x)
    e = m.numerator.bit_length() - m.denominator.bit_length()
    while Fraction(2) ** e > m:
        e -= 1
    while Fraction(2) ** (e + 1) <= m:
        e += 1
    qexp = max(e - 23, -149)
    scaled = m / Fraction(2) ** qexp
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * n * 2.0 ** qexp)


def brute_alpha(x, p_num, p_den):
    vals = sorted(abs(float(v)) for v in np.ravel(x))
    k = math.ceil(Fraction(p_num * len(vals), p_den))
    k = min(max(k, 1), len(vals))
    return vals[k - 1]


def brute_digits(q: int, bits: int):
    """Sign-magnitude base-2^(b-1) digits of q, least significant first."""
    S = 2 ** (bits - 1)
    m, out = abs(q), []
    while True:
        out.append((1 if q > 0 else -1 if q < 0 else 0) * (m % S))
        m //= S
        if m == 0:
            return out


def brute_matmul(a, b):
    a = [[int(v) for v in row] for row in np.asarray(a, dtype=object)]
    b = [[int(v) for v in row] for row in np.asarray(b, dtype=object)]
    K = len(b)
    N = len(b[0]) if K else 0
    return [[sum(a[i][k] * b[k][n] for k in range(K)) for n in range(N)] for i in range(len(a))]


def rand_codes(rng, shape, bits, oob_frac=0.1, big=2000):
    S = 2 ** (bits - 1)
    q = rng.integers(-(S - 1), S, size=shape)
    mask = rng.random(shape) < oob_frac
    q[mask] = rng.integers(-big, big + 1, size=int(mask.sum()))
    return q.astype(np.int64)


def solve(a, b, **kw):
    return O.imunpack_matmul(np.asarray(a, np.float32), np.asarray(b, np.float32), **kw)


# ---------------------------------------------------------------------------
# input widening (bf16 operands of the linear, attention and training GEMMs)
# ---------------------------------------------------------------------------

def bf16_value(bits: int) -> float:
    """Value of a bfloat16 bit pattern from the format's definition: 1 sign bit,
    8 exponent bits (bias 127), 7 fraction bits; exponent 0 is subnormal
    (2^-126 * f/128), exponent 255 is Inf (f = 0) or NaN."""
    s = -1.0 if bits >> 15 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        return s * math.inf if f == 0 else math.nan
    if e == 0:
        return s * math.ldexp(f, -126 - 7)
    return s * math.ldexp(128 + f, e - 127 - 7)


def test_widen_every_bf16_pattern():
    """All 65536 bf16 patterns: the oracle's widening equals the value the
    format defines (±0, subnormals, the largest finite values, Inf, NaN) and
    torch's own bfloat16 -> float32 conversion."""
    torch = pytest.importorskip("torch")
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.widen(bits, "bf16")
    assert got.dtype == np.float32 and got.shape == bits.shape
    ref = np.array([bf16_value(int(b)) for b in bits], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].astype(np.float64), ref[~nan])
    # signed zeros keep their sign; the extremes land where the format puts them
    assert np.signbit(got[0x8000]) and not np.signbit(got[0x0000]) and got[0x8000] == 0
    assert got[0x0001] == np.float32(2.0 ** -133) and got[0x007F] == np.float32(127 * 2.0 ** -133)
    assert got[0x7F7F] == np.float32((2 - 2.0 ** -7) * 2.0 ** 127) and got[0xFF7F] == -got[0x7F7F]
    assert got[0x7F80] == np.inf and got[0xFF80] == -np.inf
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(np.isnan(t), nan)
    assert np.array_equal(t[~nan].view(np.uint32), got[~nan].view(np.uint32))
    # 2-D operands widen element by element, in their stored orientation
    m = bits[:4096].reshape(64, 64)
    assert np.array_equal(O.widen(m, "bf16").ravel().view(np.uint32), got[:4096].view(np.uint32))
    assert np.array_equal(O.widen(m.T, "bf16"), O.widen(m, "bf16").T)
    f = np.array([[1.5, -2.25]], np.float32)
    assert O.widen(f, "f32") is not None and np.array_equal(O.widen(f, "f32"), f)


# ---------------------------------------------------------------------------
# O1 percentile, O2 scale, O3 RTN
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("p", [(95, 100), (1, 2), (995, 1000), (1, 1), (1, 1000), (3, 4)])
def test_percentile_matches_sorted_bruteforce(p):
    rng = np.random.default_rng(1)
    for trial in range(30):
        shape = (int(rng.integers(1, 9)), int(rng.integers(1, 9)))
        x = rng.standard_normal(shape).astype(np.float32)
        if trial % 3 == 0:  # ties and zeros
            x = np.round(x * 2).astype(np.float32) / 2
        sc = O.percentile_scale(x, 15, *p)
        assert float(sc.kth) == brute_alpha(x, *p)


def test_alpha_zero_falls_back_to_max_and_all_zero_gives_zero_codes():
    x = np.zeros((10, 10), np.float32)
    x[3, 4] = -7.5
    sc = O.percentile_scale(x, 15, 95, 100)
    assert sc.kth == 0 and sc.alpha == np.float32(7.5)
    q = O.quantize(x, 15, 95, 100, 5)
    assert q.q[3, 4] == -15 and np.count_nonzero(q.q) == 1
    z = np.zeros((4, 6), np.float32)
    res = solve(z, z.T.copy(), beta=15, bits=5)
    assert res.qa.scale.r == 0 and res.qa.scale.s == 0
    assert not res.C.any() and not res.out.any() and res.unpack_ratio == 1.0


def test_negative_zero_counts_as_zero():
    x = np.array([[-0.0, 0.0, 3.0, -3.0]], np.float32)
    sc = O.percentile_scale(x, 15, 1, 2)
    assert sc.kth == 0 and sc.alpha == 3.0


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_nonfinite_is_rejected(bad):
    x = np.ones((3, 3), np.float32)
    x[1, 2] = bad
    with pytest.raises(O.OracleError) as e:
        O.percentile_scale(x, 15, 95, 100)
    assert e.value.code == O.ERR_NONFINITE


def test_scale_is_correctly_rounded_division():
    rng = np.random.default_rng(2)
    for _ in range(300):
        alpha = np.float32(abs(rng.standard_normal()) * 10.0 ** rng.integers(-30, 30))
        if alpha == 0:
            continue
        beta = int(rng.choice([1, 5, 7, 15, 31, 127, 255]))
        x = np.array([[alpha]], np.float32)
        sc = O.percentile_scale(x, beta, 1, 1)
        assert sc.r == f32_round(Fraction(beta) / Fraction(float(alpha)))
        assert sc.s == f32_round(Fraction(float(alpha)) / Fraction(beta))


def test_rtn_matches_exact_rational_rounding():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 64)) * 3).astype(np.float32)
    x[rng.random(x.shape) < 0.02] *= 40
    for beta in (1, 15, 31, 255):
        sc = O.percentile_scale(x, beta, 95, 100)
        q = O.rtn(x, sc.r)
        for idx in zip(rng.integers(0, 64, 200), rng.integers(0, 64, 200)):
            y = f32_round(Fraction(float(x[idx])) * Fraction(float(sc.r)))
            assert q[idx] == round(Fraction(float(y)))  # Fraction rounds half to even


def test_rtn_ties_go_to_even():
    x = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 4.5, 5.0], np.float32)
    assert O.rtn(x, np.float32(1.0)).tolist() == [0, 2, 2, 4, 0, -2, -2, 4, 5]
    assert O.rtn(np.array([5.0, 7.0, -3.0], np.float32), np.float32(0.5)).tolist() == [2, 4, -2]


def test_no_clipping_of_heavy_hitters():
    x = np.ones((4, 5), np.float32)
    x[2, 3] = 1000.0
    q = O.quantize(x, 15, 95, 100, 5)
    assert q.scale.alpha == 1.0 and q.q[2, 3] == 15000  # kept, far outside [-15, 15]


def test_range_overflow_is_rejected():
    x = np.full((10, 10), 1e-30, np.float32)
    x[0, 0] = 1e10
    with pytest.raises(O.OracleError) as e:
        O.quantize(x, 15, 95, 100, 5)
    assert e.value.code == O.ERR_RANGE


# ---------------------------------------------------------------------------
# O4 digits, O5 statistics
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bits", range(2, 9))
def test_digits_closed_form_and_reconstruction(bits):
    S = 2 ** (bits - 1)
    rng = np.random.default_rng(bits)
    special = [0, 1, -1, S - 1, -(S - 1), S, -S, S * S - 1, S * S, 2 ** 31 - 128, -(2 ** 31 - 128)]
    q = np.array(special + list(rng.integers(-2 ** 31 + 128, 2 ** 31 - 128, 400)), np.int64)
    n = O.digit_count(q, bits)
    for j, qv in enumerate(q.tolist()):
        # closed form: a code needs ceil(bitlength / (b-1)) digits (one for 0)
        assert n[j] == max(1, -(-abs(qv).bit_length() // (bits - 1)))
        ds = [int(O.digit(q[j:j + 1], bits, t)[0]) for t in range(O.max_digits(bits) + 1)]
        assert sum(d * S ** t for t, d in enumerate(ds)) == qv
        assert all(abs(d) <= S - 1 for d in ds)
        assert all(d == 0 for d in ds[n[j]:])
        assert qv == 0 or ds[n[j] - 1] != 0
        assert ds[:n[j]] == brute_digits(qv, bits)[:n[j]]
    assert n.max() <= O.max_digits(bits)


def test_in_range_means_one_digit():
    for bits in range(2, 9):
        S = 2 ** (bits - 1)
        q = np.arange(-3 * S, 3 * S + 1)
        n = O.digit_count(q, bits)
        assert np.array_equal(n == 1, np.abs(q) <= S - 1)


def test_line_stats_bruteforce():
    rng = np.random.default_rng(4)
    for _ in range(20):
        R, C = int(rng.integers(1, 7)), int(rng.integers(1, 7))
        q = rand_codes(rng, (R, C), 4, 0.3)
        n = O.digit_count(q, 4)
        st = O.line_stats(n)
        nd = [[len(brute_digits(int(q[i, k]), 4)) for k in range(C)] for i in range(R)]
        for i in range(R):
            assert st.row_oob[i] == sum(1 for k in range(C) if nd[i][k] >= 2)
            assert st.row_maxdig[i] == max(nd[i])
        for k in range(C):
            assert st.col_oob[k] == sum(1 for i in range(R) if nd[i][k] >= 2)
            assert st.col_maxdig[k] == max(nd[i][k] for i in range(R))
        assert st.total == sum(1 for i in range(R) for k in range(C) if nd[i][k] >= 2)


# ---------------------------------------------------------------------------
# O6 candidates, O7 joint choice
# ---------------------------------------------------------------------------

def brute_candidates(nd, strategy, gamma=2):
    R, C = len(nd), len(nd[0])
    oob = [[1 if nd[i][k] >= 2 else 0 for k in range(C)] for i in range(R)]
    T = sum(map(sum, oob))
    row_oob = [sum(oob[i]) for i in range(R)]
    col_oob = [sum(oob[i][k] for i in range(R)) for k in range(C)]
    out = {}
    if strategy in ("row", "mix"):
        out["row"] = ([max(nd[i]) for i in range(R)], [1] * C)
    if strategy in ("col", "mix"):
        out["col"] = ([1] * R, [max(nd[i][k] for i in range(R)) for k in range(C)])
    if strategy == "mix":
        hc = [k for k in range(C) if col_oob[k] * C > gamma * T]
        out["cr"] = ([max([1] + [nd[i][k] for k in range(C) if k not in hc]) for i in range(R)],
                     [max(nd[i][k] for i in range(R)) if k in hc else 1 for k in range(C)])
        hr = [i for i in range(R) if row_oob[i] * R > gamma * T]
        out["rc"] = ([max(nd[i]) if i in hr else 1 for i in range(R)],
                     [max([1] + [nd[i][k] for i in range(R) if i not in hr]) for k in range(C)])
    return out


def test_candidates_bruteforce_and_coverage():
    rng = np.random.default_rng(5)
    for trial in range(60):
        R, C = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        bits = int(rng.integers(2, 9))
        q = rand_codes(rng, (R, C), bits, float(rng.choice([0.0, 0.05, 0.3, 1.0])))
        if trial % 4 == 0:  # one heavy column / row
            q[:, 0] = rng.integers(500, 5000, R)
        n = O.digit_count(q, bits)
        st = O.line_stats(n)
        nd = n.tolist()
        for strat in ("row", "col", "mix"):
            got = O.candidates(n, st, strat)
            ref = brute_candidates(nd, strat)
            assert set(got) == set(ref)
            for name, (d_r, d_c) in got.items():
                assert d_r.tolist() == ref[name][0] and d_c.tolist() == ref[name][1]
                assert (d_r >= 1).all() and (d_c >= 1).all()
                # coverage: every code fits into its d_r x d_c sub-block
                assert (d_r[:, None] + d_c[None, :] - 1 >= n).all()


def test_joint_choice_bruteforce_min_and_tie_order():
    rng = np.random.default_rng(6)
    order = O.ALLOWED["mix"]  # the Mix candidates, in tie order
    for _ in range(40):
        M, K, N = (int(v) for v in rng.integers(1, 7, 3))
        bits = int(rng.integers(2, 7))
        na = O.digit_count(rand_codes(rng, (M, K), bits, 0.3), bits)
        nb = O.digit_count(rand_codes(rng, (K, N), bits, 0.3), bits)
        ca = O.candidates(na, O.line_stats(na), "mix")
        cb = O.candidates(nb, O.line_stats(nb), "mix")
        ch = O.joint_choice(ca, cb)
        best = None
        for ia, xa in enumerate(order):
            for ib, xb in enumerate(order):
                rows = [(i, u) for i in range(M) for u in range(ca[xa][0][i])]
                cols = [(n, w) for n in range(N) for w in range(cb[xb][1][n])]
                trip = [(k, v, vp) for k in range(K) for v in range(ca[xa][1][k])
                        for vp in range(cb[xb][0][k])]
                key = (len(rows) * len(trip) * len(cols), ia, ib)
                if best is None or key < best[0]:
                    best = (key, xa, xb, len(rows), len(trip), len(cols))
        assert (ch.cand_a, ch.cand_b, ch.m_u, ch.k_u, ch.n_u) == best[1:]


def test_mix_never_worse_than_fixed_pairs():
    rng = np.random.default_rng(7)
    for _ in range(10):
        a = rng.standard_normal((24, 40)).astype(np.float32)
        b = rng.standard_normal((40, 16)).astype(np.float32)
        a[:, rng.integers(0, 40, 3)] *= 30
        b[rng.random(b.shape) < 0.05] *= 25
        mix = solve(a, b, beta=15, bits=5, unpacked=False).unpack_ratio
        for sa, sb in itertools.product(("row", "col"), repeat=2):
            fixed = solve(a, b, beta=15, bits=5, strat_a=sa, strat_b=sb, unpacked=False)
            assert mix <= fixed.unpack_ratio


# ---------------------------------------------------------------------------
# O8-O10 index maps and unpacked operands
# ---------------------------------------------------------------------------

def test_level_lines_and_triples_bruteforce():
    rng = np.random.default_rng(8)
    for _ in range(30):
        K = int(rng.integers(1, 9))
        da_c = rng.integers(1, 5, K)
        db_r = rng.integers(1, 5, K)
        trip = O.k_triples(da_c, db_r)
        ref = sorted(((v + vp, k, v), (k, v, vp, v + vp)) for k in range(K)
                     for v in range(da_c[k]) for vp in range(db_r[k]))
        assert trip.tolist() == [list(r[1]) for r in ref]
        assert (trip[trip[:, 3] == 0][:, 0] == np.arange(K)).all()
        d = rng.integers(1, 5, K)
        ll = O.level_lines(d)
        ref_l = sorted(((u, i), (i, u)) for i in range(K) for u in range(d[i]))
        assert ll.tolist() == [list(r[1]) for r in ref_l]
        assert (ll[:K, 0] == np.arange(K)).all() and (ll[:K, 1] == 0).all()


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_unpacked_operands_reconstruct_codes(bits):
    rng = np.random.default_rng(100 + bits)
    S = 2 ** (bits - 1)
    for trial in range(12):
        M, K, N = (int(v) for v in rng.integers(1, 7, 3))
        qa = rand_codes(rng, (M, K), bits, 0.3, 300)
        qb = rand_codes(rng, (K, N), bits, 0.3, 300)
        na, nb = O.digit_count(qa, bits), O.digit_count(qb, bits)
        ca = O.candidates(na, O.line_stats(na), "mix")
        cb = O.candidates(nb, O.line_stats(nb), "mix")
        ca.update(O.candidates(na, O.line_stats(na), "greedy"))  # every candidate map, greedy included
        cb.update(O.candidates(nb, O.line_stats(nb), "greedy"))
        for xa, xb in itertools.product(O.CANDIDATE_ORDER, repeat=2):
            da_r, da_c = ca[xa]
            db_r, db_c = cb[xb]
            rows, cols = O.level_lines(da_r), O.level_lines(db_c)
            trip = O.k_triples(da_c, db_r)
            Ap = O.unpack_a(qa, bits, da_r, da_c, db_r, rows, trip)
            Bp = O.unpack_b(qb, bits, db_r, db_c, da_c, cols, trip)
            assert Ap.shape == (int(da_r.sum()), int((da_c * db_r).sum()))
            assert Bp.shape == (int((da_c * db_r).sum()), int(db_c.sum()))
            assert np.abs(Ap.astype(int)).max(initial=0) <= S - 1
            assert np.abs(Bp.astype(int)).max(initial=0) <= S - 1
            # A' repeats over v', B' over v
            for j, (k, v, vp, e) in enumerate(trip.tolist()):
                j0 = [jj for jj, t in enumerate(trip.tolist()) if t[:2] == [k, v] and t[2] == 0][0]
                assert np.array_equal(Ap[:, j], Ap[:, j0])
                j1 = [jj for jj, t in enumerate(trip.tolist()) if t[0] == k and t[2] == vp and t[1] == 0][0]
                assert np.array_equal(Bp[j, :], Bp[j1, :])
            # folding the sub-blocks back gives every code exactly
            for i in range(M):
                for k in range(K):
                    acc = 0
                    for r, (ii, u) in enumerate(rows.tolist()):
                        for j, (kk, v, vp, e) in enumerate(trip.tolist()):
                            if ii == i and kk == k and vp == 0:
                                acc += int(Ap[r, j]) * S ** (u + v)
                    assert acc == qa[i, k]
            for k in range(K):
                for n in range(N):
                    acc = 0
                    for c, (nn, w) in enumerate(cols.tolist()):
                        for j, (kk, v, vp, e) in enumerate(trip.tolist()):
                            if nn == n and kk == k and v == 0:
                                acc += int(Bp[j, c]) * S ** (vp + w)
                    assert acc == qb[k, n]


# ---------------------------------------------------------------------------
# O11-O15 exactness, int32 result, dequantization
# ---------------------------------------------------------------------------

def test_exactness_against_bruteforce_all_pairs():
    """The page's central claim: low bit-width GEMMs + shift-and-accumulate equal
    the integer GEMM exactly; checked against a plain triple loop."""
    rng = np.random.default_rng(9)
    for trial in range(16):
        M, K, N = (int(v) for v in rng.integers(1, 10, 3))
        bits = int(rng.integers(2, 9))
        beta = int(rng.choice([1, 7, 15, 31, 255]))
        a = rng.standard_normal((M, K)).astype(np.float32)
        b = rng.standard_normal((K, N)).astype(np.float32)
        a[rng.random(a.shape) < 0.1] *= 40
        b[rng.random(b.shape) < 0.1] *= 40
        for sa, sb in itertools.product(("row", "col", "mix"), repeat=2):
            res = solve(a, b, beta=beta, bits=bits, strat_a=sa, strat_b=sb)
            ref = brute_matmul(res.qa.q, res.qb.q)
            assert np.asarray(res.C, dtype=object).tolist() == ref
            assert np.asarray(res.C_unpacked, dtype=object).tolist() == ref


def test_identity_when_everything_is_in_range():
    rng = np.random.default_rng(10)
    a = rng.uniform(-1, 1, (5, 7)).astype(np.float32)
    b = rng.uniform(-1, 1, (7, 3)).astype(np.float32)
    res = solve(a, b, beta=7, bits=8)  # |q| <= 7 * max/alpha stays far below S = 128
    assert res.unpack_ratio == 1.0 and res.qa.stats.total == 0 and res.qb.stats.total == 0
    assert np.array_equal(res.Ap, res.qa.q) and np.array_equal(res.Bp, res.qb.q)


def test_int32_wraps_modulo_2_32():
    a = np.ones((4, 8), np.float32)
    a[1, 2] = 1e6
    b = np.ones((8, 3), np.float32)
    b[2, 1] = 1e6
    res = solve(a, b, beta=15, bits=5)
    big = 15_000_000 * 15_000_000 + 6 * 15 * 15 + 15 * 15
    assert int(res.C[1, 1]) == big
    assert int(res.C32[1, 1]) == (big + 2 ** 31) % 2 ** 32 - 2 ** 31


def test_python_integer_route_for_huge_codes():
    a = np.ones((3, 8), np.float32)
    a[0, 0] = 2.0 ** 26
    b = np.ones((8, 2), np.float32)
    b[0, 1] = 2.0 ** 26
    res = solve(a, b, beta=15, bits=8, p_num=1, p_den=2)
    assert res.qa.q[0, 0] == res.qb.q[0, 1] == 15 * 2 ** 26
    ref = brute_matmul(res.qa.q, res.qb.q)
    assert res.C.dtype == object and res.C.tolist() == ref
    assert np.asarray(res.C_unpacked, dtype=object).tolist() == ref
    assert [[int(v) for v in r] for r in res.C32.tolist()] == \
        [[(v + 2 ** 31) % 2 ** 32 - 2 ** 31 for v in r] for r in ref]


def test_dequant_is_three_binary32_roundings():
    rng = np.random.default_rng(11)
    c = np.array([0, 1, -1, 2 ** 24 + 1, -(2 ** 24 + 3), 2 ** 31 - 1, -2 ** 31, 123456789]
                 + list(rng.integers(-2 ** 31, 2 ** 31, 50)), np.int64).astype(np.int32)
    for _ in range(20):
        sa = np.float32(rng.uniform(1e-4, 1))
        sb = np.float32(rng.uniform(1e-4, 1))
        out = O.dequant(c, sa, sb)
        sab = f32_round(Fraction(float(sa)) * Fraction(float(sb)))
        for j in range(c.size):
            cf = f32_round(Fraction(int(c[j])))
            assert out[j] == f32_round(Fraction(float(cf)) * Fraction(float(sab)))


# ---------------------------------------------------------------------------
# hand-worked examples and the page's qualitative claims
# ---------------------------------------------------------------------------

def test_hand_worked_examples():
    with open(os.path.join(GOLDEN, "hand_worked_examples.json")) as f:
        ex = json.load(f)["examples"]
    for e in ex:
        res = solve(e["A"], e["B"], beta=e["beta"], bits=e["bits"], p_num=e["p_num"],
                    p_den=e["p_den"], strat_a=e["strat_a"], strat_b=e["strat_b"])
        assert float(res.qa.scale.alpha) == e["alpha_a"] and float(res.qb.scale.alpha) == e["alpha_b"]
        assert float(res.qa.scale.r) == e["r_a"] and float(res.qa.scale.s) == e["s_a"]
        assert float(res.qb.scale.r) == e["r_b"] and float(res.qb.scale.s) == e["s_b"]
        assert res.qa.q.tolist() == e["qA"] and res.qb.q.tolist() == e["qB"]
        assert res.qa.stats.total == e["total_oob_a"] and res.qb.stats.total == e["total_oob_b"]
        ch = res.plan.choice
        assert [ch.cand_a, ch.cand_b] == e["choice"]
        assert (ch.m_u, ch.k_u, ch.n_u) == (e["m_u"], e["k_u"], e["n_u"])
        assert res.plan.rows_a.tolist() == e["rows_a"] and res.plan.cols_b.tolist() == e["cols_b"]
        assert res.plan.trip.tolist() == e["triples"]
        assert res.Ap.tolist() == e["Ap"] and res.Bp.tolist() == e["Bp"]
        assert res.C.tolist() == e["C"] and res.out.tolist() == e["out"]
        assert res.unpack_ratio == e["unpack_ratio"]


def test_pages_table_is_consistent_with_mix_being_best():
    with open(os.path.join(GOLDEN, "pages_unpack_ratios.json")) as f:
        g = json.load(f)
    assert all(g["mix"] <= v for v in g["fixed"].values())


def test_overhead_grows_with_heavy_hitters():
    """Limitations section: unpacking overhead grows with the number of heavy
    hitters.  For the fixed row/column strategies the depth of a line can only
    grow as out-of-range codes are added, so the ratio is monotone."""
    rng = np.random.default_rng(12)
    bits = 5
    qa = rand_codes(rng, (16, 24), bits, 0.0)
    qb = rand_codes(rng, (24, 12), bits, 0.0)
    prev = {}
    for step in range(6):
        idx = (rng.integers(0, 16, 3), rng.integers(0, 24, 3))
        qa[idx] = rng.integers(16, 5000, 3)
        na, nb = O.digit_count(qa, bits), O.digit_count(qb, bits)
        for sa, sb in itertools.product(("row", "col"), repeat=2):
            ca = O.candidates(na, O.line_stats(na), sa)
            cb = O.candidates(nb, O.line_stats(nb), sb)
            ch = O.joint_choice(ca, cb)
            r = ch.m_u * ch.k_u * ch.n_u
            assert r >= prev.get((sa, sb), 0)
            prev[(sa, sb)] = r


def test_invalid_parameters():
    a = np.ones((2, 2), np.float32)
    for kw in ({"bits": 1}, {"bits": 9}, {"beta": 0, "bits": 5}, {"bits": 5, "p_num": 0},
               {"bits": 5, "p_num": 101}):
        kw.setdefault("beta", 15)
        with pytest.raises(O.OracleError) as e:
            solve(a, a, **kw)
        assert e.value.code == O.ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# quantizer variants of the page's ablation rows ("Measured effects":
# p = 100% with beta = 255; clipping at the 99.5-percentile)
# ---------------------------------------------------------------------------

def _rne(x: Fraction) -> int:
    """Round an exact rational half to even."""
    n = math.floor(x)
    rem = x - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def test_clipping_quantizer_is_rounding_then_clamp():
    rng = np.random.default_rng(71)
    for trial in range(40):
        x = (rng.standard_normal((5, 7)) * 4).astype(np.float32)
        x[rng.random(x.shape) < 0.1] *= 300
        if trial % 4 == 0:  # exact halves
            x = (np.round(x * 2) / 2).astype(np.float32)
        beta = int(rng.choice([1, 3, 7, 15, 31, 255]))
        r = np.float32(rng.choice([1.0, 0.5, 2.0, rng.uniform(0.1, 9.0)]))
        q = O.rtn_clipped(x, r, beta)
        for v, got in zip(x.ravel(), q.ravel()):
            y = Fraction(float(f32_round(Fraction(float(v)) * Fraction(float(r)))))
            assert got == max(-beta, min(beta, _rne(y))), (v, r, beta)
    # a product that overflows binary32 is clamped too
    big = np.array([[3e38, -3e38, 1.0]], np.float32)
    assert O.rtn_clipped(big, np.float32(10.0), 15).tolist() == [[15, -15, 10]]


def test_clipped_path_is_in_range_when_beta_fits():
    """beta = 15 at b = 5 with clipping: every code is in range, so no line is
    unpacked (ratio 1) and C is the product of the clipped codes."""
    rng = np.random.default_rng(72)
    a = rng.standard_normal((40, 50)).astype(np.float32)
    b = rng.standard_normal((50, 30)).astype(np.float32)
    a.flat[rng.choice(a.size, 25, replace=False)] *= 40.0  # heavy hitters above the 99.5-percentile
    b.flat[rng.choice(b.size, 20, replace=False)] *= -30.0
    res = O.imunpack_matmul(a, b, 15, 5, 995, 1000, clip=True)
    assert res.unpack_ratio == 1.0
    assert np.abs(res.qa.q).max() == 15 and np.abs(res.qb.q).max() == 15
    assert res.C.tolist() == brute_matmul(res.qa.q, res.qb.q)
    plain = O.imunpack_matmul(a, b, 15, 5, 995, 1000)
    assert plain.unpack_ratio > 1.0  # the same input unclipped has heavy hitters


def test_p100_beta255_maps_the_largest_magnitude_to_beta():
    rng = np.random.default_rng(73)
    a = (rng.standard_normal((7, 10)) * 2).astype(np.float32)
    b = rng.standard_normal((10, 6)).astype(np.float32)
    for bits in (5, 8):
        res = O.imunpack_matmul(a, b, 255, bits, 100, 100)
        assert float(res.qa.scale.alpha) == float(np.abs(a).max())
        assert np.abs(res.qa.q).max() == 255 and np.abs(res.qb.q).max() == 255
        assert res.C.tolist() == brute_matmul(res.qa.q, res.qb.q)
        S = 2 ** (bits - 1)
        assert res.qa.n.max() == (2 if 255 >= S else 1)


# ---------------------------------------------------------------------------
# greedy line-at-a-time Mix (strategy "greedy")
# ---------------------------------------------------------------------------

def greedy_from_scratch(n):
    """The greedy rule with every count recounted from the whole matrix at
    every step (no incremental bookkeeping)."""
    n = np.asarray(n)
    R, C = n.shape
    d_r, d_c = [1] * R, [1] * C
    while True:
        unc = [[n[i][k] > d_r[i] + d_c[k] - 1 for k in range(C)] for i in range(R)]
        rows = [sum(unc[i]) for i in range(R)]
        cols = [sum(unc[i][k] for i in range(R)) for k in range(C)]
        best = max(rows + cols)
        if best == 0:
            return d_r, d_c
        lines = [("r", i) for i in range(R)] + [("c", k) for k in range(C)]
        counts = rows + cols
        kind, idx = lines[counts.index(best)]  # rows first, then the lowest index
        if kind == "r":
            d_r[idx] += 1
        else:
            d_c[idx] += 1


def test_greedy_closed_forms():
    n = np.ones((6, 7), np.int64)
    n[2, 5] = 4  # one code of four digits: its row takes all three extra levels (rows first)
    d_r, d_c = O.greedy_depths(n)
    assert d_r.tolist() == [1, 1, 4, 1, 1, 1] and d_c.tolist() == [1] * 7
    n = np.ones((6, 7), np.int64)
    n[:, 3] = 2  # a whole column of two-digit codes: one column level covers them
    d_r, d_c = O.greedy_depths(n)
    assert d_r.tolist() == [1] * 6 and d_c.tolist() == [1, 1, 1, 2, 1, 1, 1]
    assert [v.tolist() for v in O.greedy_depths(np.ones((3, 4), np.int64))] == [[1] * 3, [1] * 4]


def test_greedy_matches_recount_from_scratch_and_covers():
    rng = np.random.default_rng(81)
    for trial in range(60):
        R, C = int(rng.integers(1, 7)), int(rng.integers(1, 7))
        bits = int(rng.choice([2, 3, 5]))
        q = rand_codes(rng, (R, C), bits, oob_frac=float(rng.choice([0.1, 0.4])), big=600)
        n = O.digit_count(q, bits)
        d_r, d_c = O.greedy_depths(n)
        ref_r, ref_c = greedy_from_scratch(n)
        assert d_r.tolist() == ref_r and d_c.tolist() == ref_c, (trial, n.tolist())
        assert np.all(d_r[:, None] + d_c[None, :] - 1 >= n)


def test_greedy_strategy_path_is_exact():
    rng = np.random.default_rng(82)
    for trial in range(12):
        M, K, N = (int(v) for v in rng.integers(2, 9, size=3))
        bits = int(rng.choice([3, 5]))
        a = rng.standard_normal((M, K)).astype(np.float32)
        b = rng.standard_normal((K, N)).astype(np.float32)
        a[rng.random(a.shape) < 0.15] *= 40
        res = O.imunpack_matmul(a, b, 15 if bits == 5 else 3, bits, 90, 100, "greedy", "mix")
        assert res.plan.choice.cand_a == "greedy"
        assert set(k[0] for k in res.plan.choice.table) == {"greedy"}
        assert res.C.tolist() == brute_matmul(res.qa.q, res.qb.q)
