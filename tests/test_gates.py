"""The parity gates of the GPU tests, checked on the CPU with planted
mistakes: what they must reject and what they must let through."""
import numpy as np

from tests.gpu_common import sign_gate, w_round_tol


def _u(n, seed=0):
    return np.random.default_rng(seed).standard_normal(n)


def test_sign_gate_exact_and_near_zero_flips():
    U = _u(1216)
    assert sign_gate(U < 0, U)[0]
    small = np.argsort(np.abs(U))[:2]          # the entries closest to zero
    neg = U < 0
    one = neg.copy(); one[small[0]] ^= True
    assert sign_gate(one, U)[0]                 # one undecidable entry: 0.08%
    two = neg.copy(); two[small] ^= True
    assert not sign_gate(two, U)[0]             # a second is over 0.1%
    # a tiny matrix has no room for any disagreement
    V = _u(9, 3)
    flip = V < 0; flip[np.argmin(np.abs(V))] ^= True
    assert not sign_gate(flip, V)[0]


def test_sign_gate_rejects_planted_mistakes():
    U = _u(20000, 1)
    neg = U < 0
    big = neg.copy(); big[np.argmax(np.abs(U))] ^= True
    assert not sign_gate(big, U)[0]             # one large entry flipped
    assert not sign_gate(~neg, U)[0]            # sign convention inverted
    assert not sign_gate(np.roll(neg, 1), U)[0]  # index shifted by one
    # many flips below the magnitude bound still exceed the fraction
    many = neg.copy(); many[np.argsort(np.abs(U))[:40]] ^= True
    assert not sign_gate(many, U)[0]
    few = neg.copy(); few[np.argsort(np.abs(U))[:20]] ^= True
    assert sign_gate(few, U)[0]                 # 0.1% of the entries, all tiny


def test_w_round_tol_bounds_bf16_rounding():
    rng = np.random.default_rng(2)
    W = rng.standard_normal(5000).astype(np.float32) * 0.05
    U = rng.standard_normal(5000) * 0.02
    eta = 0.02
    exact = W.astype(np.float64) - eta * U
    # round to bfloat16 (nearest even) by hand
    b = exact.astype(np.float32).view(np.uint32)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    Wn = b.view(np.float32)
    Ur = (W.astype(np.float64) - Wn.astype(np.float64)) / eta
    assert np.all(np.abs(Ur - U) <= w_round_tol(Wn, "bf16", eta) * 1.0001 + 1e-9)
    assert np.all(w_round_tol(Wn, "f32", eta) == 0)
