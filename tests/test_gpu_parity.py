"""GPU parity of the HIP path against the CPU oracle, stage by stage.

Bar (all through the C ABI): bit-exact percentile scale (alpha, r, s), codes q,
per-line counts and maxima, Mix residuals, plan (choice, sizes of every
candidate pair, depth maps, segment sizes), unpacked int8 operands with the
padding stripped, int32 C; the dequantized output within 1 ulp of binary32
(expected bit-exact: the formula is fixed).  Small shapes span several 128-wide
tiles and ragged tails; the full workload sizes run in the same launch
configuration as bench.py (imu_imunpack_matmul with a reused workspace).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import imunpack_oracle as O  # noqa: E402
from outlier_unpacking_quantization_amd import binding as B  # noqa: E402
from outlier_unpacking_quantization_amd import workloads as W  # noqa: E402
from tests import gpu_support as G  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


SMALL = [
    dict(seed=1, m=300, k=700, n=260, kind="linear", dtype="bf16", layout_b="transposed"),
    dict(seed=2, m=130, k=257, n=129, kind="gauss", dtype="f32"),
    dict(seed=3, m=200, k=333, n=150, kind="grad", dtype="bf16", layout_a="transposed", beta=31, bits=4),
    dict(seed=4, m=160, k=160, n=64, kind="attn", dtype="bf16", batch=3),
    dict(seed=5, m=260, k=384, n=200, kind="linear", strat_a="row", strat_b="row"),
    dict(seed=6, m=260, k=384, n=200, kind="linear", strat_a="row", strat_b="col"),
    dict(seed=7, m=260, k=384, n=200, kind="linear", strat_a="col", strat_b="row"),
    dict(seed=8, m=260, k=384, n=200, kind="gauss", strat_a="col", strat_b="col"),
    dict(seed=9, m=100, k=90, n=70, kind="gauss", bits=2, beta=1),
    dict(seed=10, m=140, k=130, n=90, kind="gauss", bits=3, beta=7, layout_a="transposed",
         layout_b="transposed"),
    dict(seed=11, m=129, k=200, n=131, kind="linear", bits=6, beta=31, dtype="f32"),
    dict(seed=12, m=70, k=500, n=90, kind="grad", bits=8, beta=255),
    # quantizer variants of the page's ablation rows: clipping at the
    # 99.5-percentile (beta = 15 at b = 5 leaves every code in range; beta = 7
    # at b = 3 still unpacks the clipped codes) and p = 100% with beta = 255
    dict(seed=16, m=200, k=300, n=150, kind="linear", p=(995, 1000), clip=True, layout_b="transposed"),
    dict(seed=17, m=150, k=260, n=140, kind="gauss", beta=7, bits=3, p=(995, 1000), clip=True, dtype="f32"),
    dict(seed=18, m=180, k=260, n=140, kind="linear", beta=255, bits=5, p=(100, 100)),
    dict(seed=19, m=140, k=200, n=130, kind="grad", beta=255, bits=8, p=(100, 100), layout_a="transposed"),
    # the greedy line-at-a-time planner (strategy "greedy"), alone and against Mix
    dict(seed=20, m=200, k=300, n=150, kind="linear", strat_a="greedy", strat_b="greedy", layout_b="transposed"),
    dict(seed=21, m=130, k=257, n=129, kind="gauss", dtype="f32", strat_a="greedy", strat_b="mix"),
    dict(seed=22, m=150, k=200, n=140, kind="grad", bits=4, beta=31, strat_a="mix", strat_b="greedy",
         layout_a="transposed", batch=2),
]


# fp6 digits (bits <= 4, A row-major, B stored N x K): several 128-wide tiles,
# ragged tails, K over several 512-wide unpack windows (so segments end inside
# 16-position groups at window ends), each digit base, Mix / fixed / greedy
# plans, clipping, batches
FP6 = [
    dict(seed=31, m=300, k=1100, n=260, kind="linear", dtype="bf16", layout_b="transposed", beta=31, bits=4),
    dict(seed=32, m=130, k=257, n=129, kind="gauss", dtype="f32", layout_b="transposed", beta=15, bits=4),
    dict(seed=33, m=200, k=1333, n=150, kind="grad", dtype="bf16", layout_b="transposed", beta=7, bits=3, batch=2),
    dict(seed=34, m=100, k=90, n=70, kind="gauss", layout_b="transposed", beta=1, bits=2),
    dict(seed=35, m=150, k=700, n=140, kind="gauss", dtype="f32", layout_b="transposed", beta=7, bits=3,
         p=(995, 1000), clip=True),
    dict(seed=36, m=200, k=600, n=150, kind="linear", layout_b="transposed", beta=31, bits=4,
         strat_a="greedy", strat_b="mix"),
    dict(seed=37, m=260, k=640, n=200, kind="linear", layout_b="transposed", beta=15, bits=4,
         strat_a="row", strat_b="col"),
    dict(seed=38, m=160, k=520, n=64, kind="attn", dtype="bf16", layout_b="transposed", beta=15, bits=4, batch=3),
]


def _id(c):
    return f"s{c['seed']}_{c['m']}x{c['k']}x{c['n']}_{c['kind']}"


def check_stats(st: B.Stats, q_entries, b: int, tag: str):
    h = st.header(b)
    q = q_entries
    assert h["status"] == 0, tag
    assert h["alpha_bits"] == G.f32_bits(q.scale.alpha), f"{tag} alpha {h['alpha']} vs {q.scale.alpha}"
    assert h["r_bits"] == G.f32_bits(q.scale.r), f"{tag} r"
    assert h["s_bits"] == G.f32_bits(q.scale.s), f"{tag} s"
    assert np.array_equal(st.q[b].cpu().numpy().astype(np.int64), q.q), f"{tag} codes"
    s = q.stats
    assert h["total"] == s.total, f"{tag} T"
    for name, ref in (("row_oob", s.row_oob), ("col_oob", s.col_oob), ("row_maxdig", s.row_maxdig),
                      ("col_maxdig", s.col_maxdig)):
        assert np.array_equal(st.array(name, b).cpu().numpy(), ref), f"{tag} {name}"


@pytest.mark.parametrize("cfg", SMALL, ids=[_id(c) for c in SMALL])
def test_staged_path_matches_oracle(cfg):
    _staged(cfg)


@pytest.mark.parametrize("cfg", FP6, ids=[_id(c) for c in FP6])
def test_fp6_digits_match_oracle(cfg):
    """The fp6 digit format (e2m3 codes on the f8f6f4 MFMA, the Horner sum in
    the fp32 accumulators): the same plan, the digits
    decoded from the fp6 buffers equal the oracle's A' and B', and C is the
    same integer product."""
    _staged_problem(W.random_problem(**cfg), digits="fp6")


def test_fp6_wide_codes_and_levels():
    """fp6 with codes of five and more base-8 digits (|q| >= 2^12 at b = 4):
    the unpack stages sign-magnitude codes and writes levels u > 0."""
    pr = W.random_problem(seed=39, m=96, k=700, n=80, kind="gauss", dtype="f32", layout_b="transposed",
                          beta=15, bits=4)
    rng = np.random.Generator(np.random.PCG64(39))
    for op, scale in ((pr.a, 3e3), (pr.b, 1e3)):
        flat = op.stored.reshape(-1)
        idx = rng.choice(flat.size, 7, replace=False)
        flat[idx] *= np.float32(scale)
    _staged_problem(pr, digits="fp6")


@pytest.mark.parametrize("strats", [("mix", "mix"), ("row", "col"), ("col", "col"), ("col", "row")], ids="/".join)
@pytest.mark.parametrize("fold", ["1", "0"], ids=["fold_columns", "atomic_columns"])
def test_fp6_partial_sums_flushed_into_c(fold, strats, monkeypatch):
    """fp6 products far beyond 2^24 (and beyond int32): the fp32 accumulators
    cannot hold them, so waves add their exact partial sums into C on the way
    (base tiles that store, base tiles that add after the extra-row pass, and
    extra tiles) and C still equals the oracle's product modulo 2^32."""
    monkeypatch.setenv("IMU_FOLD_COLUMNS", fold)
    rng = np.random.Generator(np.random.PCG64(41))
    a = rng.standard_normal((300, 1000)).astype(np.float32)
    b = rng.standard_normal((1000, 260)).astype(np.float32)
    a[5, 17], a[40, 3], a[280, 900] = 3e5, -2e5, 1e5
    b[17, 9], b[3, 250], b[900, 140] = 4e5, 3e5, -2e5
    ref = O.imunpack_matmul(a, b, 7, 4, strat_a=strats[0], strat_b=strats[1])
    big = np.abs(np.asarray(ref.C, np.float64))
    assert big.max() > 2 ** 31 and (big > 2 ** 24).sum() >= 3
    print(f"\n[fp6 flush] fold={fold} {strats} plan {ref.plan.choice.m_u}x{ref.plan.choice.k_u}x"
          f"{ref.plan.choice.n_u}", flush=True)
    da = B.Matrix(torch.from_numpy(a).to("cuda"))
    db = B.Matrix(torch.from_numpy(np.ascontiguousarray(b.T)).to("cuda"), "transposed")
    out, c, info = B.imunpack_matmul(da, db, B.params(beta=7, bits=4, strat_a=strats[0], strat_b=strats[1],
                                                       digits="fp6"))
    assert info[0]["digits"] == B.DIGITS["fp6"]
    assert np.array_equal(c[0].cpu().numpy(), ref.C32)
    assert G.ulp_diff(out[0].cpu().numpy(), ref.out) <= 1


@pytest.mark.parametrize("fold", ["1", "0"], ids=["fold_columns", "atomic_columns"])
def test_fp6_and_int8_give_the_same_bytes(fold, monkeypatch):
    """The two digit formats of one problem: same plan, same C and output."""
    monkeypatch.setenv("IMU_FOLD_COLUMNS", fold)
    pr = W.random_problem(seed=40, m=300, k=900, n=260, kind="linear", dtype="bf16", layout_b="transposed",
                          beta=31, bits=4, strat_a="row", strat_b="col")
    a, b = G.to_device(pr.a), G.to_device(pr.b)
    out8, c8, i8 = B.imunpack_matmul(a, b, G.params_of(pr, "int8"))
    out6, c6, i6 = B.imunpack_matmul(a, b, G.params_of(pr, "fp6"))
    outa, ca, ia = B.imunpack_matmul(a, b, G.params_of(pr, "auto"))
    assert i8[0]["digits"] == B.DIGITS["int8"] and i6[0]["digits"] == B.DIGITS["fp6"]
    assert ia[0]["digits"] == B.DIGITS["fp6"]
    assert torch.equal(c8, c6) and torch.equal(out8, out6) and torch.equal(ca, c6)
    ref = G.oracle_entries(pr, unpacked=False)[0]
    assert np.array_equal(c6[0].cpu().numpy(), ref.C32)


def test_wide_codes_match_oracle():
    """Codes of five and more digits (|q| >= 2^16 at b=5) take the unpack
    kernels' code-word staging; the other cases stay within four digits."""
    pr = W.random_problem(seed=13, m=96, k=300, n=80, kind="gauss", dtype="f32")
    rng = np.random.Generator(np.random.PCG64(13))
    for op, scale in ((pr.a, 1e5), (pr.b, 3e4)):
        flat = op.stored.reshape(-1)
        idx = rng.choice(flat.size, 5, replace=False)
        flat[idx] *= np.float32(scale)
    _staged_problem(pr)


@pytest.mark.parametrize("fold", ["1", "0"], ids=["fold_columns", "atomic_columns"])
def test_batch_entries_with_and_without_extra_tiles(fold, monkeypatch):
    """One GEMM launch per pass serves every batch entry: here entry 0 has no
    out-of-range code (its plan has no extra rows or columns) while entry 1's
    heavy hitters unpack B into extra columns, so the extra-tile pass and the
    base pass see entries of both kinds.  Run with the extra columns folded
    inside the base tiles and with the atomic pass (IMU_FOLD_COLUMNS)."""
    monkeypatch.setenv("IMU_FOLD_COLUMNS", fold)
    pr = W.random_problem(seed=14, m=200, k=300, n=140, kind="gauss", dtype="f32", batch=2,
                          strat_a="col", strat_b="col")
    rng = np.random.Generator(np.random.PCG64(14))
    for op in (pr.a, pr.b):
        op.stored[0] = rng.choice(np.array([-1.0, 1.0], np.float32), size=op.stored[0].shape)
    _staged_problem(pr)


def test_batch_mixing_extra_rows_and_folded_extra_columns(monkeypatch):
    """A (row unpacking) is all in range in entry 0, so that entry has extra
    columns only (from B, column unpacking) and folds them inside its base
    tiles, while entry 1 also has extra rows and takes the atomic pass: both
    kinds share the two GEMM launches (folding forced: the problem has fewer
    base tiles than the GPU has CUs)."""
    monkeypatch.setenv("IMU_FOLD_COLUMNS", "1")
    pr = W.random_problem(seed=15, m=260, k=200, n=300, kind="gauss", dtype="f32", batch=2,
                          strat_a="row", strat_b="col")
    rng = np.random.Generator(np.random.PCG64(15))
    pr.a.stored[0] = rng.choice(np.array([-1.0, 1.0], np.float32), size=pr.a.stored[0].shape)
    refs = G.oracle_entries(pr)
    assert refs[0].plan.choice.m_u == 260 and refs[0].plan.choice.n_u > 300
    assert refs[1].plan.choice.m_u > 260 and refs[1].plan.choice.n_u > 300
    _staged_problem(pr)


def _staged(cfg):
    _staged_problem(W.random_problem(**cfg))


def _staged_problem(pr, digits="auto"):
    print(f"\n[case] {pr.name} a={pr.a.dtype}/{pr.a.layout} b={pr.b.layout} bits={pr.bits} beta={pr.beta} "
          f"strat={pr.strat_a}/{pr.strat_b} batch={pr.a.batch} digits={digits}", flush=True)
    refs = G.oracle_entries(pr)
    a, b = G.to_device(pr.a), G.to_device(pr.b)
    p = G.params_of(pr, digits)
    sa = B.quantize_rtn(a, p, want_q=True)
    sb = B.quantize_rtn(b, p, want_q=True)
    plan = B.plan_unpack(a, b, p, sa, sb)
    a_u = B.unpack(a, 0, p, sa, plan)
    b_u = B.unpack(b, 1, p, sb, plan)
    c, out = B.unpacked_gemm(a_u, b_u, p, sa, sb, plan)
    torch.cuda.synchronize()
    M, K, N = pr.mnk
    for e, ref in enumerate(refs):
        tag = f"{pr.name}[{e}]"
        check_stats(sa, ref.qa, e, tag + " A")
        check_stats(sb, ref.qb, e, tag + " B")
        info = plan.entry(e)
        ch = ref.plan.choice
        assert info["choice"] == (ch.cand_a, ch.cand_b), tag
        assert (info["m_u"], info["k_u"], info["n_u"]) == (ch.m_u, ch.k_u, ch.n_u), tag
        assert info["pairs"] == ch.table, tag
        assert info["unpack_ratio"] == pytest.approx(ref.unpack_ratio, rel=1e-12)
        # Mix residuals against the oracle's cr / rc candidates
        for st, qq, strat, side in ((sa, ref.qa, pr.strat_a, "A"), (sb, ref.qb, pr.strat_b, "B")):
            if strat == "mix":
                cand = O.candidates(qq.n, qq.stats, "mix", pr.gamma)
                assert np.array_equal(np.maximum(1, st.array("cr_rowdig", e).cpu().numpy()), cand["cr"][0]), side
                assert np.array_equal(np.maximum(1, st.array("rc_coldig", e).cpu().numpy()), cand["rc"][1]), side
        pl = ref.plan
        for name, arr in (("da_r", pl.da_r), ("da_c", pl.da_c), ("db_r", pl.db_r), ("db_c", pl.db_c)):
            assert np.array_equal(plan.array(name, e).cpu().numpy(), arr), f"{tag} {name}"
        seg_off, seg_len = plan.segments(e)
        assert seg_len == pl.segment_sizes.tolist(), tag
        assert seg_off == G.padded_segment_offsets(seg_len), tag
        assert info["k_pad"] == seg_off[-1]
        # unpacked operands, padding stripped through the documented layout
        kp = info["k_pad"]
        assert info["digits"] == B.DIGITS[digits if digits != "auto" else "int8"], tag
        A_g = G.a_rows(a_u[info["a_offset"]:].cpu().numpy(), info)
        B_g = G.b_rows(b_u[info["b_offset"]:].cpu().numpy(), info)
        rows = G.padded_line_index(pl.rows_a, M, info["m_base"])
        cols = G.depth_order_col_index(pl.cols_b, pl.db_c, info["n_base"])
        bmap = plan.array("bmap", e).cpu().numpy()
        assert np.array_equal(bmap[cols], pl.cols_b[:, 0] | (pl.cols_b[:, 1] << 24)), f"{tag} B' row map"
        kidx = G.padded_k_index(pl.trip)
        assert np.array_equal(A_g[np.ix_(rows, kidx)], ref.Ap), f"{tag} A'"
        assert np.array_equal(B_g[np.ix_(cols, kidx)], ref.Bp.T), f"{tag} B'^T"
        pad = np.ones(kp, bool)
        pad[kidx] = False
        assert not A_g[rows][:, pad].any() and not B_g[cols][:, pad].any(), f"{tag} K padding not zero"
        # integer product and dequantized output
        assert np.array_equal(c[e].cpu().numpy(), ref.C32), f"{tag} C"
        assert G.ulp_diff(out[e].cpu().numpy(), ref.out) <= 1, f"{tag} out"
    # the fused entry point gives the same bytes
    out2, c2, info2 = B.imunpack_matmul(a, b, p)
    assert torch.equal(c2, c) and torch.equal(out2, out)
    assert [i["choice"] for i in info2] == [plan.entry(e)["choice"] for e in range(pr.a.batch)]


def _single(a_np, b_np, beta=15, bits=5, p=(95, 100), dtype=torch.float32):
    a = B.Matrix(torch.from_numpy(np.ascontiguousarray(a_np, np.float32)).to("cuda", dtype))
    b = B.Matrix(torch.from_numpy(np.ascontiguousarray(b_np, np.float32)).to("cuda", dtype))
    prm = B.params(beta=beta, bits=bits, p=p)
    out, c, info = B.imunpack_matmul(a, b, prm)
    return out[0].cpu().numpy(), c[0].cpu().numpy(), info[0]


EDGE = {
    "all_zero": (np.zeros((40, 50)), np.zeros((50, 30))),
    "mostly_zero_alpha_fallback": (np.pad(np.full((1, 3), 2.5), ((0, 39), (0, 47))),
                                   np.eye(50, 30) * 3.0),
    "one_by_one": (np.array([[37.0]]), np.array([[-11.0]])),
    "k_equals_one": (np.linspace(-5, 90, 33)[:, None], np.linspace(-3, 70, 17)[None, :]),
    "single_row": (np.linspace(-9, 400, 300)[None, :], np.linspace(-1, 2, 300 * 5).reshape(300, 5)),
    "single_col": (np.linspace(-9, 40, 77)[:, None] * np.ones((1, 129)),
                   np.linspace(-1, 90, 129)[:, None]),
    "negative_ties": (np.array([[-2.5, 2.5, -0.5, 1.5, 3.5, -3.5, 0.5, 4.5]] * 8),
                      np.array([[1.5, -2.5, 0.5, 3.0, -4.5, 2.0, 1.0, 5.5]] * 8).T),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_cases(name):
    a_np, b_np = (np.asarray(x, np.float32) for x in EDGE[name])
    print(f"\n[edge] {name} {a_np.shape}x{b_np.shape}", flush=True)
    ref = O.imunpack_matmul(a_np, b_np, 15, 5)
    out, c, info = _single(a_np, b_np)
    assert np.array_equal(c, ref.C32)
    assert G.ulp_diff(out, ref.out) <= 1
    assert (info["m_u"], info["k_u"], info["n_u"]) == (ref.plan.choice.m_u, ref.plan.choice.k_u,
                                                        ref.plan.choice.n_u)


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_cases_fp6(name):
    """The same degenerate shapes through the 6-bit digit path (b = 4, B given as its
    transpose so that every digit row is K-contiguous)."""
    a_np, b_np = (np.asarray(x, np.float32) for x in EDGE[name])
    print(f"\n[edge fp6] {name} {a_np.shape}x{b_np.shape}", flush=True)
    ref = O.imunpack_matmul(a_np, b_np, 7, 4)
    a = B.Matrix(torch.from_numpy(np.ascontiguousarray(a_np)).to("cuda"))
    b = B.Matrix(torch.from_numpy(np.ascontiguousarray(b_np.T)).to("cuda"), "transposed")
    out, c, info = B.imunpack_matmul(a, b, B.params(beta=7, bits=4, digits="fp6"))
    assert info[0]["digits"] == B.DIGITS["fp6"]
    assert np.array_equal(c[0].cpu().numpy(), ref.C32)
    assert G.ulp_diff(out[0].cpu().numpy(), ref.out) <= 1
    assert (info[0]["m_u"], info[0]["k_u"], info[0]["n_u"]) == (ref.plan.choice.m_u, ref.plan.choice.k_u,
                                                              ref.plan.choice.n_u)


def test_plan_with_many_chunks():
    """A plan over 57 chunks of 512 lines (28000 rows of A, one chunk each of k
    and of B's columns): more than one round of the planner's record reads
    (56 records a round in the choice, 16 in the layout), with heavy rows and
    columns so that A takes extra rows."""
    rng = np.random.default_rng(2024)
    a_np = rng.standard_normal((28000, 64)).astype(np.float32)
    a_np[rng.choice(28000, 40, replace=False)] *= 30
    a_np[:, [3, 17]] *= 25
    b_np = rng.standard_normal((64, 128)).astype(np.float32)
    b_np[:, 5] *= 40
    print(f"\n[chunks] {a_np.shape}x{b_np.shape}", flush=True)
    ref = O.imunpack_matmul(a_np, b_np, 15, 5)
    out, c, info = _single(a_np, b_np)
    ch = ref.plan.choice
    assert info["choice"] == (ch.cand_a, ch.cand_b)
    assert (info["m_u"], info["k_u"], info["n_u"]) == (ch.m_u, ch.k_u, ch.n_u)
    assert info["pairs"] == ch.table
    assert np.array_equal(c, ref.C32)
    assert G.ulp_diff(out, ref.out) <= 1


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_nonfinite_input_is_reported(bad):
    a = np.ones((20, 30), np.float32)
    a[3, 7] = bad
    with pytest.raises(B.ImunpackError) as e:
        _single(a, np.ones((30, 10), np.float32))
    assert e.value.status == B.ERR_NONFINITE


def test_range_overflow_is_reported():
    a = np.full((10, 10), 1e-30, np.float32)
    a[0, 0] = 1e10
    with pytest.raises(B.ImunpackError) as e:
        _single(a, np.ones((10, 4), np.float32))
    assert e.value.status == B.ERR_RANGE


def test_int32_wraparound_matches_modular_oracle():
    """The exact product exceeds int32; MFMA accumulation and the fold wrap mod 2^32."""
    a = np.ones((64, 160), np.float32)
    a[5, 17] = 1e6
    a[40, 3] = -7e5
    b = np.ones((160, 96), np.float32)
    b[17, 9] = 1e6
    b[3, 50] = 9e5
    ref = O.imunpack_matmul(a, b, 15, 5)
    assert np.abs(np.asarray(ref.C, np.float64)).max() > 2 ** 31
    out, c, info = _single(a, b)
    assert np.array_equal(c, ref.C32)
    assert G.ulp_diff(out, ref.out) <= 1


def test_plan_log_lines(monkeypatch, capfd):
    """IMU_LOG=1: one stderr line per batch entry naming the plan the call
    made, which is the oracle's (candidates and unpacked sizes)."""
    pr = W.random_problem(seed=60, m=130, k=257, n=129, kind="linear", batch=2)
    a, b = G.to_device(pr.a), G.to_device(pr.b)
    ws = B.Workspace("cuda")
    B.imunpack_matmul(a, b, G.params_of(pr), ws=ws)  # sizes the workspace (a call that reports
    torch.cuda.synchronize()                        # IMU_ERR_WORKSPACE also logs its plan)
    monkeypatch.setenv("IMU_LOG", "1")
    capfd.readouterr()
    _, _, info = B.imunpack_matmul(a, b, G.params_of(pr), ws=ws)
    torch.cuda.synchronize()
    lines = [ln for ln in capfd.readouterr().err.splitlines() if ln.startswith("imu plan: entry")]
    assert len(lines) == 2
    for e, (ln, ref) in enumerate(zip(lines, G.oracle_entries(pr, unpacked=False))):
        ch = ref.plan.choice
        assert ln.startswith(f"imu plan: entry {e}: 130x257x129 choice {info[e]['choice'][0]}/{info[e]['choice'][1]} ")
        assert f"M'={ch.m_u} K'={ch.k_u} N'={ch.n_u} " in ln and "status 0" in ln


def test_workspace_grows_and_results_repeat():
    pr = W.random_problem(21, 150, 300, 140, kind="linear")
    a, b = G.to_device(pr.a), G.to_device(pr.b)
    p = G.params_of(pr)
    ws = B.Workspace("cuda")
    out1, c1, _ = B.imunpack_matmul(a, b, p, ws=ws)
    out2, c2, _ = B.imunpack_matmul(a, b, p, ws=ws)
    assert torch.equal(c1, c2) and torch.equal(out1, out2)
    ref = G.oracle_entries(pr, unpacked=False)[0]
    assert np.array_equal(c1[0].cpu().numpy(), ref.C32)


# ---------------------------------------------------------------------------
# full workload sizes, bench launch configuration
# ---------------------------------------------------------------------------

# (config, sub-problem, digit format): "auto" takes fp6 where it applies (the
# MLP up-projection and the training forward GEMM, b = 4), which also run with
# int8 digits
FULL = [(0, 0, "auto"), (1, 0, "auto"), (2, 0, "auto"), (2, 0, "int8"), (3, 0, "auto"), (4, 0, "auto"),
        (4, 0, "int8"), (4, 1, "auto"), (4, 2, "auto")]


@pytest.mark.parametrize("idx,sub,digits", FULL, ids=[f"config{i}_{j}_{d}" for i, j, d in FULL])
def test_full_size_workload(idx, sub, digits):
    pr = W.config(idx)[sub]
    M, K, N = pr.mnk
    print(f"\n[full] {pr.name} M={M} K={K} N={N} batch={pr.a.batch} digits={digits}", flush=True)
    a, b = G.to_device(pr.a), G.to_device(pr.b)
    p = G.params_of(pr, digits)
    ws = B.Workspace("cuda")
    out, c, infos = B.imunpack_matmul(a, b, p, ws=ws)
    torch.cuda.synchronize()
    refs = G.oracle_entries(pr, unpacked=False)
    for e, ref in enumerate(refs):
        ch = ref.plan.choice
        info = infos[e]
        assert info["choice"] == (ch.cand_a, ch.cand_b), (pr.name, e)
        assert (info["m_u"], info["k_u"], info["n_u"]) == (ch.m_u, ch.k_u, ch.n_u), (pr.name, e)
        assert info["pairs"] == ch.table
        assert np.array_equal(c[e].cpu().numpy(), ref.C32), (pr.name, e)
        assert G.ulp_diff(out[e].cpu().numpy(), ref.out) <= 1, (pr.name, e)
    print(f"[full] {pr.name} ok ratio={infos[0]['unpack_ratio']:.3f} choice={infos[0]['choice']} "
          f"digits={infos[0]['digits']}", flush=True)


def test_full_size_fp32_gradient_operand():
    """The training data gradient at full size with the gradient entering as
    float32 (Student-t draws, not bf16-rounded), so the percentile takes the
    fp32 route (16-bit key prefix, then two 256-bin refinements) over 25.2 M
    elements, in the launch configuration of the training step."""
    rng = np.random.Generator(np.random.PCG64(1104))
    dy = W.gradients(rng, 8192, 3072)
    w = W.config(4)[1].b  # W (3072 x 768, bf16) as it enters dY @ W
    print("\n[full-f32] dY 8192x3072 f32 @ W 3072x768 bf16", flush=True)
    a = B.Matrix(torch.from_numpy(dy).to("cuda"))
    b = G.to_device(w)
    p = B.params(beta=31, bits=4)
    out, c, infos = B.imunpack_matmul(a, b, p, ws=B.Workspace("cuda"))
    torch.cuda.synchronize()
    ref = O.imunpack_matmul(dy, G.logical_f32(w, 0), 31, 4, 95, 100, unpacked=False)
    ch = ref.plan.choice
    assert infos[0]["choice"] == (ch.cand_a, ch.cand_b)
    assert (infos[0]["m_u"], infos[0]["k_u"], infos[0]["n_u"]) == (ch.m_u, ch.k_u, ch.n_u)
    assert np.array_equal(c[0].cpu().numpy(), ref.C32)
    assert G.ulp_diff(out[0].cpu().numpy(), ref.out) <= 1
    # the scale itself, through the staged entry point
    st = B.quantize_rtn(a, p)
    h = st.header(0)
    assert h["alpha_bits"] == G.f32_bits(ref.qa.scale.alpha) and h["r_bits"] == G.f32_bits(ref.qa.scale.r)
    assert h["total"] == ref.qa.stats.total


def test_entry_points_need_init_and_release_frees():
    """imu_release frees the device's context; the planner then refuses to run
    until imu_init sets it up again (through the binding here)."""
    pr = W.random_problem(31, 96, 130, 70, kind="gauss", dtype="f32")
    a, b = G.to_device(pr.a), G.to_device(pr.b)
    p = G.params_of(pr)
    out1, c1, _ = B.imunpack_matmul(a, b, p)
    torch.cuda.synchronize()
    B.release_all()
    sa, sb = B.quantize_rtn(a, p), B.quantize_rtn(b, p)
    pl = B.Plan(a, b, p)
    ma, mb = a.c(), b.c()
    import ctypes
    st = B.lib().imu_plan_unpack(ctypes.byref(ma), ctypes.byref(mb), ctypes.byref(p), B._ptr(sa.buf),
                                 B._ptr(sb.buf), B._ptr(pl.buf), pl.info,
                                 ctypes.c_void_p(B._stream(None)))
    assert st == B.ERR_INVALID_ARG and b"imu_init" in B.lib().imu_last_error()
    out2, c2, _ = B.imunpack_matmul(a, b, p)  # the binding sets the device up again
    assert torch.equal(c1, c2) and torch.equal(out1, out2)


def test_full_size_greedy_plan():
    """The greedy planner on the LLaMA-shaped linear layer at full size (2681
    and 4405 greedy steps): plan sizes and C against the oracle."""
    pr = W.config(1)[0].with_strategies("greedy", "greedy")
    print(f"\n[full] {pr.name} greedy/greedy", flush=True)
    a, b = G.to_device(pr.a), G.to_device(pr.b)
    out, c, infos = B.imunpack_matmul(a, b, G.params_of(pr), ws=B.Workspace("cuda"))
    torch.cuda.synchronize()
    ref = G.oracle_entries(pr, unpacked=False)[0]
    ch = ref.plan.choice
    assert infos[0]["choice"] == ("greedy", "greedy")
    assert (infos[0]["m_u"], infos[0]["k_u"], infos[0]["n_u"]) == (ch.m_u, ch.k_u, ch.n_u)
    assert np.array_equal(c[0].cpu().numpy(), ref.C32)
    assert G.ulp_diff(out[0].cpu().numpy(), ref.out) <= 1
