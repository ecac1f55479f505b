"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and its host-only functions (sizes, layouts, argument validation)
behave as documented in include/imunpack.h.  No kernel is launched here:
every call below either touches no device memory or fails validation first."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "imunpack.h")

torch = pytest.importorskip("torch")
from outlier_unpacking_quantization_amd import binding as B  # noqa: E402


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(imu_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from outlier_unpacking_quantization_amd import build
        build.build()
    return B.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), f"{n} declared in imunpack.h but not exported"
    assert set(B.EXPORTED) == set(names)


def test_init_validates_before_touching_a_device(lib):
    for bad in (0, -1, 65536):
        assert lib.imu_init(bad) == B.ERR_INVALID_ARG
        assert b"max_batch" in lib.imu_last_error()


def test_version_and_status_strings(lib):
    assert "gfx950" in B.version()
    for s in range(7):
        assert lib.imu_status_string(s)
    assert lib.imu_status_string(99) == b"unknown status"


def cpu_matrix(rows, cols, dtype=torch.bfloat16, layout="normal", batch=1):
    shape = (cols, rows) if layout == "transposed" else (rows, cols)
    t = torch.zeros((batch, *shape) if batch > 1 else shape, dtype=dtype)
    return B.Matrix(t, layout)


def test_stats_layout_sizes(lib):
    m = cpu_matrix(100, 37).c()
    v = B.ImuStatsView()
    assert lib.imu_stats_layout(ctypes.byref(m), ctypes.byref(v)) == 0
    assert lib.imu_stats_bytes(ctypes.byref(m)) == v.stride
    offs = [v.row_oob, v.col_oob, v.row_maxdig, v.col_maxdig, v.cr_rowdig, v.rc_coldig, v.hist]
    assert offs == sorted(offs) and offs[0] >= 64 and all(o % 256 == 0 for o in offs)
    assert v.hist + 4 * 32768 <= v.stride
    mb = cpu_matrix(100, 37, batch=3).c()
    assert lib.imu_stats_bytes(ctypes.byref(mb)) == 3 * v.stride


def test_plan_layout_bounds(lib):
    a, b = cpu_matrix(300, 700).c(), cpu_matrix(700, 260, layout="transposed").c()
    for bits in range(2, 9):
        p = B.params(bits=bits)
        v = B.ImuPlanView()
        assert lib.imu_plan_layout(ctypes.byref(a), ctypes.byref(b), ctypes.byref(p), ctypes.byref(v)) == 0
        levels = -(-31 // (bits - 1))
        assert v.levels == levels and v.segments == 2 * levels - 1
        assert v.m_alloc_max >= 300 * levels and v.n_alloc_max >= 260 * levels
        assert lib.imu_plan_bytes(ctypes.byref(a), ctypes.byref(b), ctypes.byref(p)) == \
            v.headers_bytes + v.entry_stride
        assert lib.imu_workspace_fixed_bytes(ctypes.byref(a), ctypes.byref(b), ctypes.byref(p)) >= \
            v.headers_bytes + v.entry_stride


@pytest.mark.parametrize("bad", [
    {"bits": 1}, {"bits": 9}, {"beta": 0}, {"p": (0, 100)}, {"p": (101, 100)}, {"gamma": -1},
])
def test_invalid_params_rejected_before_any_device_work(lib, bad):
    kw = dict(beta=15, bits=5, p=(95, 100), gamma=2)
    kw.update(bad)
    p = B.params(**kw)
    m = cpu_matrix(8, 8).c()
    st = lib.imu_quantize_rtn(ctypes.byref(m), ctypes.byref(p), ctypes.c_void_p(1), None, None)
    assert st == B.ERR_INVALID_ARG
    assert lib.imu_last_error()


def test_fp6_digits_need_bits_4_and_k_contiguous_operands(lib):
    """fp6 digits (e2m3 holds integers up to 7) need bits <= 4 and the
    K-contiguous layouts; asked for elsewhere they are refused before any
    device work, and an unknown format is an argument error."""
    a = cpu_matrix(64, 128).c()
    bt = cpu_matrix(128, 64, layout="transposed").c()
    bn = cpu_matrix(128, 64).c()
    at = cpu_matrix(64, 128, layout="transposed").c()
    size = lambda x, y, p: lib.imu_plan_bytes(ctypes.byref(x), ctypes.byref(y), ctypes.byref(p))
    for bits in (2, 3, 4):
        assert size(a, bt, B.params(bits=bits, digits="fp6")) > 0
    assert size(a, bt, B.params(bits=5, digits="fp6")) == 0
    assert b"fp6" in lib.imu_last_error()
    assert size(a, bn, B.params(bits=4, digits="fp6")) == 0
    assert size(at, bt, B.params(bits=4, digits="fp6")) == 0
    for digits in ("auto", "int8"):  # fall back / ask for int8: always valid
        assert size(a, bn, B.params(bits=4, digits=digits)) > 0
        assert size(a, bt, B.params(bits=5, digits=digits)) > 0
    bad = B.params(bits=4)
    bad.digits = 3
    assert size(a, bt, bad) == 0 and b"digits" in lib.imu_last_error()
    need = ctypes.c_size_t(0)
    p = B.params(bits=5, digits="fp6")
    st = lib.imu_imunpack_matmul(ctypes.byref(a), ctypes.byref(bt), ctypes.byref(p), ctypes.c_void_p(1), None,
                                 None, 0, ctypes.byref(need), None, None)
    assert st == B.ERR_UNSUPPORTED


def test_invalid_shapes_rejected(lib):
    p = B.params()
    a, b = cpu_matrix(8, 9).c(), cpu_matrix(10, 4).c()  # K mismatch
    info = (B.ImuPlanInfo * 1)()
    st = lib.imu_plan_unpack(ctypes.byref(a), ctypes.byref(b), ctypes.byref(p), ctypes.c_void_p(1),
                             ctypes.c_void_p(1), ctypes.c_void_p(1), info, None)
    assert st == B.ERR_INVALID_ARG and b"K" in lib.imu_last_error()
    z = B.ImuMatrix(1, B.BF16, B.NORMAL, 0, 5, 5, 1, 0)  # empty
    assert lib.imu_stats_bytes(ctypes.byref(z)) == 0
    bad_ld = B.ImuMatrix(1, B.BF16, B.NORMAL, 4, 8, 7, 1, 0)  # ld below the row length
    assert lib.imu_stats_bytes(ctypes.byref(bad_ld)) == 0
    bad_dt = B.ImuMatrix(1, 7, B.NORMAL, 4, 8, 8, 1, 0)
    assert lib.imu_stats_bytes(ctypes.byref(bad_dt)) == 0
    null = B.ImuMatrix(None, B.BF16, B.NORMAL, 4, 8, 8, 1, 0)
    assert lib.imu_quantize_rtn(ctypes.byref(null), ctypes.byref(p), ctypes.c_void_p(1), None, None) \
        == B.ERR_INVALID_ARG
    huge = B.ImuMatrix(1, B.BF16, B.NORMAL, 1 << 24, 8, 8, 1, 0)
    assert lib.imu_quantize_rtn(ctypes.byref(huge), ctypes.byref(p), ctypes.c_void_p(1), None, None) \
        == B.ERR_UNSUPPORTED


def test_workspace_too_small_reports_fixed_size(lib):
    a, b = cpu_matrix(64, 128).c(), cpu_matrix(128, 64).c()
    p = B.params()
    need = ctypes.c_size_t(0)
    st = lib.imu_imunpack_matmul(ctypes.byref(a), ctypes.byref(b), ctypes.byref(p), ctypes.c_void_p(1), None,
                                 None, 0, ctypes.byref(need), None, None)
    assert st == B.ERR_WORKSPACE
    assert need.value == lib.imu_workspace_fixed_bytes(ctypes.byref(a), ctypes.byref(b), ctypes.byref(p))


def test_binding_matrix_marshalling():
    t = torch.zeros((3, 40, 24), dtype=torch.bfloat16)
    m = B.Matrix(t, "transposed").c()
    assert (m.rows, m.cols, m.ld, m.batch, m.batch_stride, m.layout, m.dtype) == \
        (24, 40, 24, 3, 960, B.TRANSPOSED, B.BF16)
    with pytest.raises(B.ImunpackError):
        B.Matrix(torch.zeros((4, 4), dtype=torch.float64)).c()
    with pytest.raises(B.ImunpackError):
        B.Matrix(torch.zeros((4, 4)).t()).c()  # non-unit last stride
    # size-1 dimensions may carry any stride (numpy's contiguous (17, 1) transpose of a (1, 17) row)
    col = torch.zeros((1, 17)).t()
    assert col.stride() == (1, 17)
    m = B.Matrix(col, "transposed").c()
    assert (m.rows, m.cols, m.ld) == (1, 17, 1)
    m = B.Matrix(torch.zeros(17).as_strided((1, 17), (1, 1))).c()  # one stored row, torch row stride 1
    assert (m.rows, m.cols, m.ld) == (1, 17, 17)


def test_training_wrapper_rejects_bad_shapes():
    torch = pytest.importorskip("torch")
    from outlier_unpacking_quantization_amd import training as T
    p = B.params(beta=31, bits=4)
    with pytest.raises(B.ImunpackError):
        T.imunpack_linear(torch.zeros(4, 3), torch.zeros(5, 2), p)
    with pytest.raises(B.ImunpackError):
        T.imunpack_linear(torch.zeros(4, 3, 2), torch.zeros(5, 3), p)


def test_softmax_prepare_validates_before_any_device_work(lib):
    """imu_softmax_prepare: P must be bf16, row-major, the logits' shape, and
    apart from the logits; each violation is refused synchronously."""
    p = B.params()
    st = ctypes.c_void_p(1)  # never written: every call below fails validation
    call = lambda z, o, prm=p, s=st: lib.imu_softmax_prepare(ctypes.byref(z), ctypes.byref(o), ctypes.byref(prm),
                                                             s, None)
    z = B.Matrix(torch.zeros((16, 40), dtype=torch.float32)).c()
    assert call(z, B.Matrix(torch.zeros((16, 40), dtype=torch.float32)).c()) == B.ERR_INVALID_ARG
    assert b"bf16" in lib.imu_last_error().lower() or b"BF16" in lib.imu_last_error()
    assert call(z, B.Matrix(torch.zeros((16, 41), dtype=torch.bfloat16)).c()) == B.ERR_INVALID_ARG
    assert call(z, B.Matrix(torch.zeros((40, 16), dtype=torch.bfloat16), "transposed").c()) == B.ERR_UNSUPPORTED
    zt = B.Matrix(torch.zeros((40, 16), dtype=torch.float32), "transposed").c()
    assert call(zt, B.Matrix(torch.zeros((16, 40), dtype=torch.bfloat16)).c()) == B.ERR_UNSUPPORTED
    buf = torch.zeros((16, 40), dtype=torch.bfloat16)
    same = B.Matrix(buf).c()
    assert call(same, same) == B.ERR_INVALID_ARG and b"overlap" in lib.imu_last_error()
    assert call(z, B.Matrix(buf).c(), s=None) == B.ERR_INVALID_ARG
    bad = B.params()
    bad.bits = 9
    assert call(z, B.Matrix(buf).c(), prm=bad) == B.ERR_INVALID_ARG
