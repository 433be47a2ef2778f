"""GPU parity of signmuon_polar_ns (PolarNS: pre-scale + Newton-Schulz)
against the oracle's Newton-Schulz at the same K, coefficients, scale and
start vector."""
import numpy as np
import pytest

import oracle as O
from distributed_bit_matrix_amd import binding as B
from distributed_bit_matrix_amd import workloads as WL
from tests.gpu_common import f32, oracle_hp, polar_tol, sign_gate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
QUINTIC = WL.QUINTIC


def momentum_like(shape, seed, signal=0.5):
    """A momentum matrix after one step from zero, G = S + N (Gaussian)."""
    rng = np.random.default_rng(seed)
    G = signal * rng.standard_normal(shape) + rng.standard_normal(shape)
    return (0.1 * G).astype(np.float32)


def run(X, hp, u0=None):
    Xt = torch.from_numpy(X).cuda()
    u0t = None if u0 is None else torch.from_numpy(u0).cuda()
    U = B.polar_ns(Xt, hp, u0=u0t)
    torch.cuda.synchronize()
    return U.cpu().numpy().astype(np.float64)


def check(X, hp, u0=None, max_abs=None, gate=True):
    print(f"polar_ns {X.shape} {hp.precision} {hp.scale} K={hp.K} c={hp.coeffs[2]}",
          flush=True)
    Ug = run(X, hp, u0)
    o = oracle_hp(hp)
    Uo, _ = O.polar_ns(X.astype(np.float64), o["K"], o["eps"], o["scale"], o["P"],
                       o["coeffs"], None if u0 is None else u0.astype(np.float64))
    err = float(np.abs(Ug - Uo).max())
    tol = polar_tol(hp.precision) if max_abs is None else max_abs
    assert err <= tol, (err, tol)
    if gate:
        ok, st = sign_gate(Ug < 0, Uo)
        assert ok, st
    return err


SHAPES = [(256, 512), (512, 256), (128, 128), (64, 147), (147, 64), (10, 300),
          (300, 10), (384, 640), (1, 64), (200, 1000)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("precision", ["f32", "bf16", "bf16x3"])
def test_polar_fro_cubic(shape, precision):
    X = momentum_like(shape, 1)
    check(X, B.HParams(K=5, scale="fro", precision=precision))


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("K", [1, 2, 5])
def test_polar_fro_cubic_iterate_form(shape, K, monkeypatch):
    # bfloat16 cubic with the Frobenius scale runs in Gram space by default;
    # the iterate form is held to the same gates
    monkeypatch.setenv("SIGNMUON_NS_FORM", "iterate")
    X = momentum_like(shape, 1)
    check(X, B.HParams(K=K, scale="fro", precision="bf16"))


@pytest.mark.parametrize("shape", [(256, 512), (512, 256), (64, 147), (1, 64), (200, 1000)])
@pytest.mark.parametrize("K", [1, 2, 3])
def test_polar_fro_cubic_gram_space_few_steps(shape, K):
    # the Gram-space form with K = 1 (no symmetric products), 2 and 3
    X = momentum_like(shape, 6)
    check(X, B.HParams(K=K, scale="fro", precision="bf16"))


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("precision", ["f32", "bf16"])
def test_polar_spectral_cubic(shape, precision):
    X = momentum_like(shape, 2)
    u0 = np.random.default_rng(3).standard_normal(min(shape)).astype(np.float32)
    check(X, B.HParams(K=5, scale="spectral", P=5, precision=precision), u0=u0)


@pytest.mark.parametrize("shape", [(256, 512), (512, 256), (384, 640)])
@pytest.mark.parametrize("precision", ["f32", "bf16x3"])
def test_polar_quintic(shape, precision):
    X = momentum_like(shape, 4)
    check(X, B.HParams(K=5, scale="spectral", P=10, coeffs=QUINTIC, precision=precision))


# Long k with few Gram tiles: the Gram (and the raw Gram of the spectral
# scale) is split along k into partial tiles that a second kernel sums.
SPLIT_K = [((128, 4096), "bf16", "fro", (1.5, -0.5, 0.0)),
           ((4096, 128), "bf16", "spectral", (1.5, -0.5, 0.0)),
           ((256, 3000), "bf16x3", "fro", QUINTIC),
           ((200, 2600), "f32", "spectral", (1.5, -0.5, 0.0)),
           ((384, 2176), "bf16", "spectral", (1.5, -0.5, 0.0))]


@pytest.mark.parametrize("shape,precision,scale,coeffs", SPLIT_K)
def test_polar_split_k(shape, precision, scale, coeffs):
    X = momentum_like(shape, 5)
    u0 = np.random.default_rng(6).standard_normal(min(shape)).astype(np.float32)
    hp = B.HParams(K=5, scale=scale, P=6, coeffs=coeffs, precision=precision)
    check(X, hp, u0=u0 if scale == "spectral" else None)


@pytest.mark.parametrize("K", [0, 1, 2])
@pytest.mark.parametrize("scale", ["fro", "spectral"])
def test_polar_few_steps(K, scale):
    X = momentum_like((192, 320), 5)
    check(X, B.HParams(K=K, scale=scale, P=3, precision="f32"))
    check(X, B.HParams(K=K, scale=scale, P=3, precision="bf16"))


def test_polar_default_start_vector():
    X = momentum_like((100, 260), 6)
    check(X, B.HParams(K=5, scale="spectral", P=4, precision="f32"), u0=None)


def test_polar_zero_matrix():
    X = np.zeros((64, 96), np.float32)
    for scale in ("fro", "spectral"):
        Ug = run(X, B.HParams(K=5, scale=scale, P=3))
        assert np.all(Ug == 0.0)


def test_polar_rank_one_signs_exact():
    x = np.random.default_rng(7).standard_normal(96).astype(np.float32)
    y = np.random.default_rng(8).standard_normal(224).astype(np.float32)
    X = np.outer(x, y).astype(np.float32)
    Ug = run(X, B.HParams(K=5, scale="fro", precision="bf16"))
    assert np.array_equal(np.sign(Ug), np.outer(np.sign(x), np.sign(y)))


def test_polar_orthogonal_fixed_point():
    Q, _ = np.linalg.qr(np.random.default_rng(9).standard_normal((256, 256)))
    Q = Q.astype(np.float32)
    Ug = run(Q, B.HParams(K=5, scale="spectral", P=3, precision="f32"))
    assert np.abs(Ug - Q).max() < 1e-4
