"""Pins of the oracle's row softmax (R-17: the P of the attention-output GEMM).

The softmax arithmetic is fixed step by step so that one P is defined; these
tests tie it to what mathematics fixes: the exponential within its error
bound, closed forms (a constant row, a masked row), the float64 softmax of
the same rounded differences within the binary32 error bound, exact sums,
bf16 rounding on hand-picked ties, and non-finite rows.  The last test plants
plausible mistakes in the oracle and checks that some pin fails.
"""
import contextlib
import math

import numpy as np
import pytest

from oracle import imunpack_oracle as O

U = 2.0 ** -24  # unit roundoff of binary32


def _exp_bound(t):
    """Relative error bound of R-17's exp for binary32 t <= 0: half an ulp of
    y = t log2(e) (the rounding of the product) carried through 2^y, plus
    the rounding of L itself, the Horner steps and the degree-7 truncation."""
    y = np.abs(np.asarray(t, np.float64)) * math.log2(math.e)
    ulp_y = np.where(y > 0, 2.0 ** (np.floor(np.log2(np.maximum(y, 1e-300))) - 23), 0.0)
    return math.log(2.0) * (0.5 * ulp_y + y * U) + 12 * U


def test_exp_within_bound_and_special_values():
    t = np.concatenate([np.linspace(-69.0, 0.0, 200001), -np.logspace(-12, 1.8, 5000)]).astype(np.float32)
    e = O.softmax_exp(t)
    ref = np.exp(t.astype(np.float64))
    rel = np.abs(e.astype(np.float64) - ref) / ref
    assert np.all(rel <= _exp_bound(t)), float((rel / _exp_bound(t)).max())
    assert O.softmax_exp(np.float32([0.0]))[0] == np.float32(1.0)       # 2^0 * c0
    assert O.softmax_exp(np.float32([-np.inf]))[0] == 0.0               # masked logit
    assert O.softmax_exp(np.float32([-75.0]))[0] == 0.0                 # y < -100
    assert O.softmax_exp(np.float32([-69.0]))[0] > 0.0                  # y > -100
    assert np.isnan(O.softmax_exp(np.float32([np.nan]))[0])


def test_exp2_polynomial_matches_2_to_the_f():
    # the polynomial alone on [-1/2, 1/2] (n = 0): within a few ulp of 2^f
    f = np.linspace(-0.5, 0.5, 100001).astype(np.float32)
    c = O.exp2_coefficients()
    p = np.full_like(f, c[7])
    for k in range(6, -1, -1):
        p = ((p * f).astype(np.float32) + c[k]).astype(np.float32)
    ref = np.exp2(f.astype(np.float64))
    assert np.max(np.abs(p - ref) / ref) <= 4 * U
    assert float(c[0]) == 1.0 and abs(float(c[1]) - math.log(2.0)) <= U


@pytest.mark.parametrize("n", [1, 5, 63, 256, 257, 2048, 3000])
def test_constant_row_is_one_over_n(n):
    p = O.softmax_f32(np.full(n, 2.5, np.float32))
    assert np.all(p == np.float32(1.0) / np.float32(n))  # e = 1 exactly, S = n exactly
    bits = O.softmax_bf16(np.full((1, n), -7.0, np.float32))
    assert np.all(bits == O.f32_to_bf16_rne(np.float32(1.0) / np.float32(n)))


def test_masked_row_is_one_hot():
    row = np.full(300, -np.inf, np.float32)
    row[123] = 4.0
    p = O.softmax_f32(row)
    assert p[123] == 1.0 and np.count_nonzero(p) == 1


@pytest.mark.parametrize("n,shift", [(1, 0.0), (64, 0.0), (255, 0.0), (300, 50.0), (2048, 0.0), (2048, 120.0),
                                     (5000, -30.0)])
def test_against_float64_softmax_of_the_same_differences(n, shift):
    rng = np.random.default_rng(17 + n)
    row = (rng.standard_normal(n) * 3.0 + shift).astype(np.float32)
    p = O.softmax_f32(row)
    t = (row - np.fmax.reduce(row)).astype(np.float32).astype(np.float64)
    e = np.exp(t)
    ref = e / e.sum()
    # e: exp bound; S: n - 1 additions of non-negative terms; the division: 1 rounding
    bound = _exp_bound(t) + (n + 2) * U + _exp_bound(t).max()
    assert np.all(np.abs(p - ref) <= bound * ref + 1e-45)
    assert abs(float(p.astype(np.float64).sum()) - 1.0) <= (2 * n + 4) * U + float(_exp_bound(t).max())


def test_row_sum_exact_cases_and_bound():
    assert O.softmax_row_sum(np.ones(3000, np.float32)) == np.float32(3000.0)
    pw = np.float32(2.0) ** -np.arange(0, 20, dtype=np.float32)  # exact binary sums
    assert O.softmax_row_sum(pw) == np.float32(math.fsum(pw.astype(np.float64)))
    rng = np.random.default_rng(5)
    for n in (1, 3, 255, 256, 257, 1000, 4097):
        e = rng.random(n, dtype=np.float32)
        s = float(O.softmax_row_sum(e))
        exact = math.fsum(e.astype(np.float64))
        assert abs(s - exact) <= n * U * exact
        e2 = e.copy()
        e2[-1] += 1.0  # the last (tail) element counts
        assert float(O.softmax_row_sum(e2)) > s + 0.5


def test_bf16_rounding_golden():
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, 0.2,
                  3.4028234663852886e38, 0.0, -0.0, np.nan, -1.0 - 2.0 ** -8], np.float32)
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0x3E4D, 0x7F80, 0x0000, 0x8000, 0x7FC0, 0xBF80]
    assert [int(x) for x in O.f32_to_bf16_rne(v)] == want


def test_nonfinite_rows():
    for bad in (np.nan, np.inf):
        row = np.zeros(40, np.float32)
        row[7] = bad
        assert np.all(O.softmax_bf16(row[None, :]) == 0x7FC0)
    assert np.all(O.softmax_bf16(np.full((1, 9), -np.inf, np.float32)) == 0x7FC0)


PINS = [test_exp_within_bound_and_special_values, test_exp2_polynomial_matches_2_to_the_f, test_masked_row_is_one_hot,
        test_row_sum_exact_cases_and_bound, test_bf16_rounding_golden, test_nonfinite_rows]
PINS_N = [(test_constant_row_is_one_over_n, {"n": 257}),
          (test_against_float64_softmax_of_the_same_differences, {"n": 2048, "shift": 120.0}),
          (test_against_float64_softmax_of_the_same_differences, {"n": 300, "shift": 50.0})]

_orig_exp, _orig_sum, _orig_f32 = O.softmax_exp, O.softmax_row_sum, O.softmax_f32


def _exp_floor(t):  # n = floor(y): f in [0, 1), where the degree-7 polynomial is short
    t = np.asarray(t, np.float32)
    y = (t * O.SOFTMAX_LOG2E).astype(np.float32)
    e = np.zeros_like(y)
    live = ~np.isnan(y) & ~(y < -100)
    n = np.floor(y[live]).astype(np.float32)
    f = (y[live] - n).astype(np.float32)
    c = O.exp2_coefficients()
    p = np.full_like(f, c[7])
    for k in range(6, -1, -1):
        p = ((p * f).astype(np.float32) + c[k]).astype(np.float32)
    e[live] = np.ldexp(p, n.astype(np.int32))
    e[np.isnan(y)] = np.nan
    return e


def _exp_natural_base(t):  # forgets the log2(e) factor
    return _orig_exp((np.asarray(t, np.float32) / O.SOFTMAX_LOG2E).astype(np.float32))


def _sum_drops_tail(e):
    e = np.asarray(e, np.float32)
    span = O.SOFTMAX_LANES * O.SOFTMAX_CHUNK
    n = (e.shape[0] // span) * span
    return _orig_sum(e[:n]) if n else np.float32(0.0)


def _sum_half_lanes(e):  # the halving stops one step early (lanes 0..1 only)
    e = np.asarray(e, np.float32)
    span = O.SOFTMAX_LANES * O.SOFTMAX_CHUNK
    J = max(1, -(-e.shape[0] // span))
    pad = np.zeros(J * span, np.float32)
    pad[:e.shape[0]] = e
    lanes = pad.reshape(J, 64, 4).transpose(1, 0, 2).reshape(64, -1)
    v = np.add.accumulate(lanes, axis=1, dtype=np.float32)[:, -1]
    s = 32
    while s >= 2:
        v = (v[:s] + v[s:2 * s]).astype(np.float32)
        s //= 2
    return np.float32(v[0])


def _f32_no_max(row):  # exp of the raw logits
    row = np.asarray(row, np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(row.astype(np.float32))
        return (e / O.softmax_row_sum(e)).astype(np.float32)


def _bf16_truncate(x):
    x = np.asarray(x, np.float32)
    x = np.atleast_1d(x)
    r = (x.view(np.uint32) >> 16).astype(np.uint16)
    r[np.isnan(x)] = 0x7FC0
    return r


MUTATIONS = {
    "exp_floor_reduction": ("softmax_exp", _exp_floor),
    "exp_natural_base": ("softmax_exp", _exp_natural_base),
    "sum_drops_tail_chunk": ("softmax_row_sum", _sum_drops_tail),
    "sum_halving_stops_early": ("softmax_row_sum", _sum_half_lanes),
    "no_max_subtraction": ("softmax_f32", _f32_no_max),
    "bf16_truncates": ("f32_to_bf16_rne", _bf16_truncate),
}


@contextlib.contextmanager
def _patched(name, fn):
    old = getattr(O, name)
    setattr(O, name, fn)
    try:
        yield
    finally:
        setattr(O, name, old)


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_softmax_mistake_is_caught(mutation):
    name, fn = MUTATIONS[mutation]
    caught = []
    with _patched(name, fn):
        for pin in PINS:
            try:
                pin()
            except Exception as e:  # noqa: BLE001 - any failure counts as caught
                caught.append((pin.__name__, type(e).__name__))
        for pin, kw in PINS_N:
            try:
                pin(**kw)
            except Exception as e:  # noqa: BLE001
                caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {mutation}"
