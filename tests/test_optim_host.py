"""Host-side checks of the torch.optim front end (no GPU work)."""
import pytest

torch = pytest.importorskip("torch")

from distributed_bit_matrix_amd import optim as SO  # noqa: E402


def test_matrix_shapes():
    assert SO.matrix_shape((768, 2304)) == (768, 2304)
    assert SO.matrix_shape((64, 3, 7, 7)) == (64, 147)        # conv kernel, flattened
    assert SO.matrix_shape((512, 256, 3, 3)) == (512, 2304)
    assert SO.matrix_shape((10,)) == (1, 10)                   # vector: 1 x n
    assert SO.matrix_shape(()) == (1, 1)


def test_arguments():
    p = torch.nn.Parameter(torch.zeros(4, 4))
    with pytest.raises(ValueError):
        SO.SignMuon([p], workers=0)
    with pytest.raises(ValueError):
        SO.SignMuon([p], workers=4)                            # no source of other signs
    opt = SO.SignMuon([p], lr=0.01, K=3)
    assert opt.param_groups[0]["K"] == 3
