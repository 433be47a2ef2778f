"""signmuon_polar_ns_static (PolarNS with the library's per-GPU scratch
array, no workspace argument) against signmuon_polar_ns with a caller
workspace: the same kernels on the same inputs give the same bits, on two
calls in a row, the second on a smaller matrix (the array keeps the first
call's contents)."""
import numpy as np
import pytest

from distributed_bit_matrix_amd import binding as B

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _x(shape, seed):
    rng = np.random.default_rng(seed)
    G = 0.5 * rng.standard_normal(shape) + rng.standard_normal(shape)
    return torch.from_numpy((0.1 * G).astype(np.float32)).cuda()


CASES = [
    # (first shape, second smaller shape, hyper-parameters)
    ((768, 3072), (192, 576), B.HParams(K=5, scale="fro", precision="bf16")),
    ((1024, 4096), (300, 10), B.HParams(K=5, scale="spectral", P=8, precision="bf16")),
    ((512, 1536), (64, 147), B.HParams(K=5, scale="spectral", P=5,
                                       coeffs=(3.4445, -4.7750, 2.0315),
                                       precision="bf16x3")),
    ((384, 640), (33, 7), B.HParams(K=3, scale="fro", precision="f32")),
]


@pytest.mark.parametrize("first,second,hp", CASES)
def test_polar_ns_static_matches_workspace_entry(first, second, hp):
    for shape, seed in ((first, 1), (second, 2)):
        print(f"polar_ns_static {shape} {hp.precision} {hp.scale}", flush=True)
        X = _x(shape, seed)
        u0 = None
        if hp.scale == "spectral":
            u0 = torch.from_numpy(np.random.default_rng(seed + 10).standard_normal(
                min(shape)).astype(np.float32)).cuda()
        U_static = B.polar_ns_static(X, hp, u0=u0)
        U_ws = B.polar_ns(X, hp, u0=u0)
        torch.cuda.synchronize()
        assert torch.equal(U_static.view(torch.int32), U_ws.view(torch.int32)), shape


def test_polar_ns_static_rejects_oversize():
    X = torch.zeros((4096, 4096), dtype=torch.float32, device="cuda")
    with pytest.raises(B.SignMuonError) as e:
        B.polar_ns_static(X, B.HParams(K=5))
    assert e.value.status == B.SM_ERANGE
