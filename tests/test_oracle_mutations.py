"""Planted mistakes in the CPU oracle must be caught by its pins.

Each mutation below is a plausible slip (a dropped term, a wrong sign, a
wrong rounding rule, a wrong order, a transposed operand).  The mutation is
patched into the oracle module on the CPU, the pins of
``test_oracle_pins`` are run, and at least one of them must fail.
"""
import contextlib

import numpy as np
import pytest

from oracle import imunpack_oracle as O
from tests import test_oracle_pins as P

PINS = [
    P.test_widen_every_bf16_pattern,
    P.test_percentile_matches_sorted_bruteforce,
    P.test_scale_is_correctly_rounded_division,
    P.test_rtn_matches_exact_rational_rounding,
    P.test_rtn_ties_go_to_even,
    P.test_digits_closed_form_and_reconstruction,
    P.test_line_stats_bruteforce,
    P.test_candidates_bruteforce_and_coverage,
    P.test_joint_choice_bruteforce_min_and_tie_order,
    P.test_level_lines_and_triples_bruteforce,
    P.test_unpacked_operands_reconstruct_codes,
    P.test_exactness_against_bruteforce_all_pairs,
    P.test_int32_wraps_modulo_2_32,
    P.test_dequant_is_three_binary32_roundings,
    P.test_hand_worked_examples,
    P.test_clipping_quantizer_is_rounding_then_clamp,
    P.test_clipped_path_is_in_range_when_beta_fits,
    P.test_greedy_closed_forms,
    P.test_greedy_matches_recount_from_scratch_and_covers,
]
PARAMS = {
    "test_percentile_matches_sorted_bruteforce": {"p": (95, 100)},
    "test_digits_closed_form_and_reconstruction": {"bits": 5},
    "test_unpacked_operands_reconstruct_codes": {"bits": 3},
}


@contextlib.contextmanager
def patched(name, fn):
    old = getattr(O, name)
    setattr(O, name, fn)
    try:
        yield
    finally:
        setattr(O, name, old)


def _rtn_half_up(x32, r):
    y = np.asarray(x32, np.float32) * np.float32(r)
    return np.floor(y + np.float32(0.5)).astype(np.int64)


def _rank_floor(count, p_num, p_den):
    return min(max((p_num * count) // p_den, 1), count)


def _digit_unsigned(q, bits, t):
    S = 1 << (bits - 1)
    return (np.abs(np.asarray(q, np.int64)) // (S ** t)) % S


def _widen_shift_15(stored, dtype):
    if dtype == "bf16":
        bits = np.asarray(stored, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return bits.view(np.float32)
    return np.asarray(stored, dtype=np.float32)


def _widen_through_f16(stored, dtype):
    # reads the stored half-word as IEEE binary16 instead of bfloat16
    if dtype == "bf16":
        return np.asarray(stored, dtype=np.uint16).view(np.float16).astype(np.float32)
    return np.asarray(stored, dtype=np.float32)


def _placement_outer_first(t, d_k):
    return np.zeros_like(d_k) + np.minimum(t, 0), t + 0 * d_k


_orig_segments = O.segment_products
_orig_fold = O.fold
_orig_triples = O.k_triples
_orig_joint = O.joint_choice
_orig_cands = O.candidates
_orig_unpack_b = O.unpack_b


def _segments_no_shift(Ap, Bp, trip, bits, big=False):
    t = trip.copy()
    t[:, 3] = 0
    return _orig_segments(Ap, Bp, t, bits, big)


def _fold_rows_only(P_, rows_a, cols_b, M, N, bits, big=False):
    c = cols_b.copy()
    c[:, 1] = 0
    return _orig_fold(P_, rows_a, c, M, N, bits, big)


def _triples_k_major(da_c, db_r):
    t = _orig_triples(da_c, db_r)
    return t[np.lexsort((t[:, 2], t[:, 1], t[:, 0]))] if t.size else t


def _joint_max(ca, cb):
    best = None
    for na in O.CANDIDATE_ORDER:
        for nb in O.CANDIDATE_ORDER:
            if na in ca and nb in cb:
                m, k, n = O.unpacked_sizes(ca[na][0], ca[na][1], cb[nb][0], cb[nb][1])
                if best is None or m * k * n > best[0]:
                    best = (m * k * n, na, nb, m, k, n)
    return O.Choice(*best[1:])


def _cands_ge(n, st, strategy, gamma=2):
    # heavy-line test with >= instead of >
    return _orig_cands(n, st, strategy, gamma - 1 if gamma > 0 else gamma)


def _dequant_one_scale(C32, sA, sB):
    return (np.asarray(C32, np.int32).astype(np.float32) * np.float32(sA)).astype(np.float32)


def _scale_swapped(x32, beta, p_num, p_den):
    sc = _orig_scale(x32, beta, p_num, p_den)
    return O.Scale(sc.alpha, sc.s, sc.r, sc.kth, sc.maxabs)


_orig_scale = O.percentile_scale


def _unpack_b_transposed_depths(qB, bits, db_r, db_c, da_c, cols_b, trip):
    # uses A's inner depths where B's belong
    return _orig_unpack_b(qB, bits, da_c, db_c, db_r, cols_b, trip)


def _exact_matmul_drop_last_column(a, b):
    c = a.astype(np.int64) @ b.astype(np.int64) if a.size and b.size else \
        np.zeros((a.shape[0], b.shape[1]), np.int64)
    if a.shape[1] > 1:
        c = c - np.outer(a[:, -1].astype(np.int64), b[-1, :].astype(np.int64))
    return c


def _clip_dropped(x32, r, beta):
    with np.errstate(over="ignore"):
        y = np.asarray(x32, np.float32) * np.float32(r)
    return np.rint(np.nan_to_num(y, posinf=2.0 ** 31 - 1, neginf=-(2.0 ** 31 - 1))).astype(np.int64)


def _greedy_columns_first(n):
    d_r, d_c = _orig_greedy(n.T)
    return d_c, d_r


def _greedy_stale_update(n):
    # covers the codes the line needed before its new level (off by one)
    R, C = n.shape
    d_r, d_c = np.ones(R, np.int64), np.ones(C, np.int64)
    unc = n > 1
    cr, cc = unc.sum(1), unc.sum(0)
    for _ in range(R * C * 40):
        if max(cr.max(initial=0), cc.max(initial=0)) == 0:
            break
        if cr.max(initial=0) >= cc.max(initial=0):
            i = int(np.argmax(cr))
            newly = n[i, :] == d_r[i] + d_c - 1
            d_r[i] += 1
            cc -= newly
            cr[i] -= int(newly.sum())
        else:
            k = int(np.argmax(cc))
            newly = n[:, k] == d_r + d_c[k] - 1
            d_c[k] += 1
            cr -= newly
            cc[k] -= int(newly.sum())
    return d_r, d_c


_orig_greedy = O.greedy_depths


MUTATIONS = {
    "greedy_columns_first": ("greedy_depths", _greedy_columns_first),
    "greedy_stale_update": ("greedy_depths", _greedy_stale_update),
    "clip_dropped": ("rtn_clipped", _clip_dropped),
    "widen_shift_15": ("widen", _widen_shift_15),
    "widen_reads_binary16": ("widen", _widen_through_f16),
    "rtn_half_up": ("rtn", _rtn_half_up),
    "percentile_floor_rank": ("percentile_rank", _rank_floor),
    "digit_drops_sign": ("digit", _digit_unsigned),
    "placement_outer_first": ("placement", _placement_outer_first),
    "segment_shift_dropped": ("segment_products", _segments_no_shift),
    "fold_drops_column_shift": ("fold", _fold_rows_only),
    "triples_k_major": ("k_triples", _triples_k_major),
    "joint_choice_max": ("joint_choice", _joint_max),
    "heavy_line_ge": ("candidates", _cands_ge),
    "dequant_one_scale": ("dequant", _dequant_one_scale),
    "scale_r_s_swapped": ("percentile_scale", _scale_swapped),
    "unpack_b_wrong_depths": ("unpack_b", _unpack_b_transposed_depths),
    "matmul_drops_a_term": ("exact_matmul", _exact_matmul_drop_last_column),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation):
    name, fn = MUTATIONS[mutation]
    caught = []
    with patched(name, fn):
        for pin in PINS:
            try:
                pin(**PARAMS.get(pin.__name__, {}))
            except Exception as e:  # noqa: BLE001 - any failure counts as caught
                caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {mutation}"
