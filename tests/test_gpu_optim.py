"""The torch.optim front end on the GPU: one step of a small model matches
the oracle's step (M = 1) given the library's own sign buffer, and a short
synthetic regression trains."""
import numpy as np
import pytest

import oracle as O
from distributed_bit_matrix_amd import binding as B
from distributed_bit_matrix_amd import optim as SO
from tests.gpu_common import f32, momentum_tol, sign_gate, unpack_neg

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def test_one_step_matches_oracle():
    torch.manual_seed(0)
    shapes = [(96, 160), (64, 3, 5, 5), (40,)]
    params = [torch.nn.Parameter((0.02 * torch.randn(s)).cuda()) for s in shapes]
    W0 = [p.detach().cpu().numpy().astype(np.float64).reshape(-1) for p in params]
    grads = [torch.randn(s).cuda() for s in shapes]
    for p, g in zip(params, grads):
        p.grad = g.clone()
    opt = SO.SignMuon(params, lr=0.02, beta=0.9, weight_decay=0.01, K=5, scale="fro",
                      ns_precision="f32")
    print("optim one step", shapes, flush=True)
    opt.step()
    torch.cuda.synchronize()
    st = opt._groups[0]
    bits = st.bits.cpu().numpy().view(np.uint32)
    hp = dict(eta=f32(0.02), beta=f32(0.9), lam=f32(0.01), eps=f32(1e-7), K=5, scale="fro",
              P=5)
    for i, (p, g, w0) in enumerate(zip(params, grads, W0)):
        r, c, off, woff = st.layout[i]
        n = r * c
        G = g.cpu().numpy().astype(np.float64).reshape(-1)
        Mom = O.momentum_update(np.zeros(n), G, w0, hp["beta"], hp["lam"])
        Mg = st.Mom[off:off + n].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(Mg - Mom) <= momentum_tol(np.zeros(n), G, w0, hp["beta"],
                                                        hp["lam"]))
        U, _ = O.polar_ns(Mom.reshape(r, c), 5, hp["eps"], "fro")
        seg = bits[0, woff:woff + (n + 31) // 32]
        ok, stats = sign_gate(unpack_neg(seg, n), U)
        assert ok, (i, stats)
        # M = 1: the vote is the local buffer; W given those signs, bit for bit
        D = O.majority_from_sums(O.vote_sums_from_bits(seg[None, :], n), 0)
        Wn = O.apply_update(w0.astype(np.float32), D, hp["eta"], "f32")
        got = p.detach().cpu().numpy().reshape(-1)
        assert np.array_equal(got.view(np.uint32), Wn.view(np.uint32)), i
        assert p.data.data_ptr() == st.W[off:].data_ptr()      # a view of the flat buffer


def test_synthetic_regression_trains():
    torch.manual_seed(1)
    X = torch.randn(4096, 64, device="cuda")
    Wt = torch.randn(64, 32, device="cuda") / 8
    Y = torch.tanh(X @ Wt)
    model = torch.nn.Sequential(torch.nn.Linear(64, 128), torch.nn.Tanh(),
                                torch.nn.Linear(128, 32)).cuda()
    opt = SO.SignMuon(model.parameters(), lr=0.01, beta=0.9, K=5, scale="fro")
    losses = []
    print("optim regression", flush=True)
    for step in range(60):
        idx = torch.randint(0, X.shape[0], (512,), device="cuda")
        loss = torch.nn.functional.mse_loss(model(X[idx]), Y[idx])
        opt.zero_grad(set_to_none=False)
        loss.backward()
        opt.step()
        losses.append(float(loss.detach()))
    assert not opt.nonfinite()
    assert np.mean(losses[-10:]) < 0.3 * np.mean(losses[:5]), losses[::10]
