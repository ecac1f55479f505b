"""imu_imunpack_matmul_noalloc (the whole path in the library's static scratch
array) against imu_imunpack_matmul (caller workspace) through the C ABI: two
calls in a row, the second on a smaller, ragged problem (the array keeps the
first call's contents), each compared bit for bit (C and the dequantized
output) and with the oracle's C; a problem larger than the array is rejected
with IMU_ERR_WORKSPACE and the size it needs."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

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


def _both(pr):
    a, b = G.to_device(pr.a), G.to_device(pr.b)
    p = G.params_of(pr)
    out0, c0, info0 = B.imunpack_matmul(a, b, p, ws=B.Workspace("cuda"))
    out1, c1, info1 = B.imunpack_matmul_noalloc(a, b, p)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1) and torch.equal(out0, out1), pr.name
    assert [i["choice"] for i in info0] == [i["choice"] for i in info1]
    assert [(i["m_u"], i["k_u"], i["n_u"]) for i in info0] == [(i["m_u"], i["k_u"], i["n_u"]) for i in info1]
    return c1


def test_noalloc_matches_workspace_entry_point_twice():
    assert B.lib().imu_noalloc_scratch_bytes() == 128 << 20
    big = W.config(1)[0]  # LLaMA-shaped linear: about 112 MiB of workspace
    print("\n[noalloc] llama_linear full size", flush=True)
    c_big = _both(big)
    small = W.random_problem(41, 300, 700, 260, kind="linear", layout_b="transposed", batch=2)
    print("[noalloc] small ragged batch 2", flush=True)
    c_small = _both(small)
    for e, ref in enumerate(G.oracle_entries(small, unpacked=False)):
        assert np.array_equal(c_small[e].cpu().numpy(), ref.C32)
    ref = G.oracle_entries(big, unpacked=False)[0]
    assert np.array_equal(c_big[0].cpu().numpy(), ref.C32)


def test_noalloc_rejects_a_problem_above_the_scratch():
    pr = W.config(2)[0]  # MLP up-projection: its unpacked operands need about 430 MB
    print("\n[noalloc] mlp_up (too large)", flush=True)
    a, b = G.to_device(pr.a), G.to_device(pr.b)
    with pytest.raises(B.ImunpackError) as e:
        B.imunpack_matmul_noalloc(a, b, G.params_of(pr))
    assert e.value.status == B.ERR_WORKSPACE and "scratch" in str(e.value)
    # the array still serves a problem that fits
    _both(W.random_problem(42, 129, 257, 131, kind="gauss", dtype="f32"))
