"""GPU parity of the quantized-training linear layer (forward, data gradient,
weight gradient through imu_imunpack_matmul) against the CPU oracle, and of
its autograd gradients against those products.

Bar: int32 C bit-exact, dequantized output within 1 ulp of binary32, for each
of the three GEMMs; autograd returns exactly those products in the dtype of
the tensor they belong to.  Shapes are ragged and span several GEMM tiles; the
value models are the training recipe's (activations with outlier channels,
N(0, 0.02) weights with heavy hitters, Student-t gradients), beta = 31, b = 4.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import imunpack_oracle as O  # noqa: E402
from outlier_unpacking_quantization_amd import binding as B  # noqa: E402
from outlier_unpacking_quantization_amd import training as T  # noqa: E402
from outlier_unpacking_quantization_amd import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    torch.cuda.synchronize()


def _max_ulp(got: np.ndarray, ref: np.ndarray) -> int:
    g = got.astype(np.float32).view(np.int32).astype(np.int64)
    r = ref.astype(np.float32).view(np.int32).astype(np.int64)
    return int(np.abs(g - r).max()) if g.size else 0


def test_training_linear_step_matches_oracle():
    rng = np.random.Generator(np.random.PCG64(21))
    tokens, d_in, d_out = 320, 200, 260
    x = torch.from_numpy(W.activations(rng, tokens, d_in)).to("cuda").to(torch.bfloat16)
    w = torch.from_numpy(W.weights(rng, d_out, d_in)).to("cuda").to(torch.bfloat16)
    dy32 = W.gradients(rng, tokens, d_out)
    dy = torch.from_numpy(dy32).to("cuda")
    xa, wa = x.float().cpu().numpy(), w.float().cpu().numpy()  # the bf16 values, exactly
    p = B.params(beta=31, bits=4)
    ws = B.Workspace("cuda")
    print(f"\n[case] training linear tokens={tokens} d_in={d_in} d_out={d_out}", flush=True)
    y, cy = T.linear_forward(x, w, p, ws)
    dx, cdx = T.linear_data_grad(dy, w, p, ws)
    dw, cdw = T.linear_weight_grad(dy, x, p, ws)
    torch.cuda.synchronize()
    for out, c, a, b, tag in ((y, cy, xa, wa.T, "forward"), (dx, cdx, dy32, wa, "data gradient"),
                              (dw, cdw, dy32.T, xa, "weight gradient")):
        ref = O.imunpack_matmul(np.ascontiguousarray(a), np.ascontiguousarray(b), 31, 4, 95, 100)
        assert np.array_equal(c.cpu().numpy().astype(np.int64), ref.C32.astype(np.int64)), f"{tag}: int32 C"
        assert _max_ulp(out.cpu().numpy(), ref.out) <= 1, f"{tag}: dequantized output"

    xr, wr = x.clone().requires_grad_(True), w.clone().requires_grad_(True)
    yr = T.imunpack_linear(xr, wr, p, ws)
    yr.backward(dy)
    torch.cuda.synchronize()
    assert torch.equal(yr.detach(), y)
    assert xr.grad.dtype == torch.bfloat16 and torch.equal(xr.grad, dx.to(torch.bfloat16))
    assert wr.grad.dtype == torch.bfloat16 and torch.equal(wr.grad, dw.to(torch.bfloat16))
