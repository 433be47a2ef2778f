"""Pins of the CPU oracle to what the pages and the mathematics fix.

None of these tests re-types the oracle's formula: each compares it with a
worked example printed on the pages, a value derived by hand, a closed form,
an exhaustive enumeration, or a library routine that computes the same
quantity by another route (SVD, torch's bfloat16 cast).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle as O

QUINTIC = (3.4445, -4.7750, 2.0315)


# --------------------------------------------------------------------------
# Majority vote, sign and ties
# --------------------------------------------------------------------------
def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_blog_example_ternary(golden_dir):
    g = _load(golden_dir, "blog_vote_example.json")
    dirs = np.array(g["directions"])
    signs = O.sign_ternary(dirs)
    sums = O.vote_sums_from_signs(signs)
    # Per entry by hand: (+1-1-1), (-1-1+1), (+1+1+1), (+1-1+1).
    assert sums.tolist() == [[-1, -1], [3, 1]]
    assert O.majority_from_sums(sums, 0).tolist() == g["majority"]


def test_blog_example_packed(golden_dir):
    g = _load(golden_dir, "blog_vote_example.json")
    dirs = np.array(g["directions"])
    bits = np.stack([O.pack_signs(w) for w in dirs])
    sums = O.vote_sums_from_bits(bits, 4)
    D = O.majority_from_sums(sums, 0).reshape(2, 2)
    assert D.tolist() == g["majority"]


def test_mean_versus_majority(golden_dir):
    g = _load(golden_dir, "blog_mean_vs_majority.json")
    x = np.array(g["directions"])
    assert np.sign(x.mean()) == g["mean_sign"]
    signs = O.sign_ternary(x.reshape(3, 1))
    D = O.majority_from_sums(O.vote_sums_from_signs(signs), 0)
    assert D.tolist() == [g["majority"]]
    bits = np.stack([O.pack_signs(x[i:i + 1]) for i in range(3)])
    assert O.majority_from_sums(O.vote_sums_from_bits(bits, 1)).tolist() == [-1]


@pytest.mark.parametrize("tie", [0, 1])
def test_ties(tie):
    signs = np.array([[1, -1, 1, 1], [-1, 1, 1, -1]])  # M=2 workers, 4 entries
    D = O.majority_from_sums(O.vote_sums_from_signs(signs), tie)
    assert D.tolist() == [tie, tie, 1, tie]
    signs4 = np.array([[1], [1], [-1], [-1]])
    assert O.majority_from_sums(O.vote_sums_from_signs(signs4), tie).tolist() == [tie]
    with pytest.raises(ValueError):
        O.majority_from_sums(np.zeros(3, np.int32), -1)


@pytest.mark.parametrize("M", list(range(1, 13)))
@pytest.mark.parametrize("tie", [0, 1])
def test_vote_exhaustive_pm1(M, tie):
    pats = np.array(list(itertools.product([1, -1], repeat=M)), dtype=np.int8).T
    pos = (pats == 1).sum(axis=0)
    neg = (pats == -1).sum(axis=0)
    want = np.where(pos > neg, 1, np.where(neg > pos, -1, tie))
    got = O.majority_from_sums(O.vote_sums_from_signs(pats), tie)
    assert np.array_equal(got, want)
    # the same through the 1-bit packed buffers
    bits = np.stack([O.pack_signs(pats[m].astype(np.float64)) for m in range(M)])
    got2 = O.majority_from_sums(O.vote_sums_from_bits(bits, pats.shape[1]), tie)
    assert np.array_equal(got2, want)


@pytest.mark.parametrize("M", list(range(1, 7)))
def test_vote_exhaustive_ternary(M):
    pats = np.array(list(itertools.product([1, 0, -1], repeat=M)), dtype=np.int8).T
    pos = (pats == 1).sum(axis=0)
    neg = (pats == -1).sum(axis=0)
    want = np.where(pos > neg, 1, np.where(neg > pos, -1, 0))
    got = O.majority_from_sums(O.vote_sums_from_signs(pats), 0)
    assert np.array_equal(got, want)


def test_int8_accumulator_overflow():
    # Blog, bytes section: an int8 sum of many signs overflows.
    for M, wrapped in [(127, 127), (128, -128), (200, -56), (255, -1)]:
        signs = [np.ones(1, np.int8)] * M
        assert int(O.vote_sums_int8_wrapping(signs)[0]) == wrapped
        assert int(O.vote_sums_from_signs(np.ones((M, 1)))[0]) == M
    # at M=200 the int8 route would even flip the majority
    signs = [np.ones(1, np.int8)] * 200
    assert O.majority_from_sums(O.vote_sums_int8_wrapping(signs)).tolist() == [-1]
    assert O.majority_from_sums(O.vote_sums_from_signs(np.ones((200, 1)))).tolist() == [1]


def test_sign_of_zero():
    x = np.array([0.0, -0.0, 1e-300, -1e-300, 5.0, -2.0])
    assert O.sign_ternary(x).tolist() == [0, 0, 1, -1, 1, -1]
    # packed: bit set only for strictly negative entries (indices 3 and 5)
    assert O.pack_signs(x).tolist() == [(1 << 3) | (1 << 5)]


# --------------------------------------------------------------------------
# 1-bit packing layout
# --------------------------------------------------------------------------
def test_pack_every_byte_pattern():
    for v in range(256):
        for byte_pos in range(4):
            U = np.ones(32)
            for i in range(8):
                if (v >> i) & 1:
                    U[8 * byte_pos + i] = -1.0
            w = O.pack_signs(U)
            assert w.shape == (1,)
            assert int(w[0]) == v << (8 * byte_pos)


def test_pack_layout_by_hand():
    U = np.ones(40)
    U[[0, 31, 32, 39]] = -1.0
    w = O.pack_signs(U)
    assert w.tolist() == [0x80000001, 0x00000081]   # tail bits 40..63 are 0


def test_pack_roundtrip():
    rng = np.random.default_rng(1)
    for n in [1, 31, 32, 33, 1000]:
        s = rng.choice([-1, 1], size=n).astype(np.int8)
        assert np.array_equal(O.unpack_signs(O.pack_signs(s), n), s)


# --------------------------------------------------------------------------
# Momentum
# --------------------------------------------------------------------------
def test_momentum_by_hand():
    Mom = np.array([[1.0, 2.0]])
    G = np.array([[4.0, -8.0]])
    W = np.array([[2.0, 4.0]])
    # G~ = G + 0.25 W = [4.5, -7];  Mom' = 0.5 Mom + 0.5 G~ = [2.75, -2.5]
    out = O.momentum_update(Mom, G, W, beta=0.5, lam=0.25)
    assert out.tolist() == [[2.75, -2.5]]


def test_momentum_special_cases():
    rng = np.random.default_rng(2)
    Mom, G, W = rng.standard_normal((3, 4, 5))
    assert np.array_equal(O.momentum_update(Mom, G, W, 0.0, 0.1), G + 0.1 * W)
    assert np.allclose(O.momentum_update(Mom, G, W, 0.9, 0.0), 0.9 * Mom + 0.1 * G,
                       rtol=0, atol=1e-15)
    assert np.array_equal(O.momentum_update(np.zeros((2, 2)), np.zeros((2, 2)),
                                            np.ones((2, 2)), 0.5, 0.0), np.zeros((2, 2)))


# --------------------------------------------------------------------------
# Pre-scaling
# --------------------------------------------------------------------------
def test_frobenius_by_hand():
    assert O.frobenius_scale(np.array([[3.0, 4.0]])) == 5.0
    assert O.frobenius_scale(np.array([[1.0, 2.0], [2.0, 4.0]])) == 5.0


def test_spectral_power_iteration_by_hand():
    Mom = np.diag([3.0, 1.0])
    # A = diag(9, 1); from u0 = (1, 1): |A u0| / |u0| = sqrt(82/2) = sqrt(41)
    assert np.isclose(O.spectral_scale(Mom, 1, np.array([1.0, 1.0])), 41 ** 0.25,
                      rtol=1e-15)
    # P=2: |A^2 u0| / |A u0| = sqrt(6562 / 82)
    assert np.isclose(O.spectral_scale(Mom, 2, np.array([1.0, 1.0])),
                      (6562 / 82) ** 0.25, rtol=1e-15)
    assert np.isclose(O.spectral_scale(Mom, 200), 3.0, rtol=1e-12)
    assert O.spectral_scale(np.zeros((3, 4)), 5) == 0.0


@pytest.mark.parametrize("shape", [(5, 9), (9, 5), (6, 6)])
@pytest.mark.parametrize("P", [1, 2, 5])
def test_spectral_closed_form(shape, P):
    # Normalised power iteration: the last |w| equals |A^P u0| / |A^(P-1) u0|,
    # with A the smaller Gram.  Evaluated here by repeated multiplication
    # without normalisation, and the Gram built from the SVD.
    rng = np.random.default_rng(3)
    Mom = rng.standard_normal(shape)
    r = min(shape)
    u0 = rng.standard_normal(r)
    Us, sv, Vt = np.linalg.svd(Mom if shape[0] <= shape[1] else Mom.T,
                               full_matrices=False)
    A = (Us * sv ** 2) @ Us.T
    v = u0.copy()
    for _ in range(P - 1):
        v = A @ v
    lam = np.linalg.norm(A @ v) / np.linalg.norm(v)
    assert np.isclose(O.spectral_scale(Mom, P, u0), np.sqrt(lam), rtol=1e-12)
    # the estimate never exceeds sigma_max
    assert O.spectral_scale(Mom, P, u0) <= sv[0] * (1 + 1e-12)


def test_spectral_transpose_invariant():
    rng = np.random.default_rng(4)
    Mom = rng.standard_normal((7, 3))
    u0 = rng.standard_normal(3)
    assert np.isclose(O.spectral_scale(Mom, 4, u0), O.spectral_scale(Mom.T, 4, u0),
                      rtol=1e-14)


# --------------------------------------------------------------------------
# Newton-Schulz and the polar factor
# --------------------------------------------------------------------------
def _scalar_ns(sig, K, coeffs):
    a, b, c = coeffs
    for _ in range(K):
        sig = a * sig + b * sig ** 3 + c * sig ** 5
    return sig


@pytest.mark.parametrize("shape", [(5, 9), (9, 5), (6, 6), (1, 8), (8, 1)])
@pytest.mark.parametrize("scale,P", [("fro", 0), ("spectral", 3)])
@pytest.mark.parametrize("coeffs", [O.CUBIC, QUINTIC])
@pytest.mark.parametrize("K", [0, 1, 3, 5])
def test_ns_spectral_identity(shape, scale, P, coeffs, K):
    # NS applies the odd scalar polynomial p(s) = a s + b s^3 + c s^5 to every
    # singular value and keeps the singular vectors.
    rng = np.random.default_rng(5)
    Mom = rng.standard_normal(shape)
    u0 = rng.standard_normal(min(shape))
    eps = 1e-7
    U, s = O.polar_ns(Mom, K, eps, scale, P, coeffs, u0)
    Us, sv, Vt = np.linalg.svd(Mom, full_matrices=False)
    want = (Us * _scalar_ns(sv / (s + eps), K, coeffs)) @ Vt
    assert U.shape == shape
    assert np.allclose(U, want, rtol=0, atol=1e-12 * max(1.0, np.abs(want).max()))


def test_ns_zero_steps_is_prescale():
    rng = np.random.default_rng(6)
    Mom = rng.standard_normal((4, 6))
    U, s = O.polar_ns(Mom, 0, 1e-7, "fro")
    assert s == O.frobenius_scale(Mom)
    assert np.array_equal(U, Mom / (s + 1e-7))


def test_ns_rank_one_fixed_point():
    x = np.array([1.0, -2.0, 0.5, 3.0])
    y = np.array([-1.0, 4.0, 2.0, -0.25, 1.5, -3.0])
    Mom = np.outer(x, y)
    U, s = O.polar_ns(Mom, 5, 1e-7, "fro")
    # one singular value, fro scale puts it at 1/(1+eps/|x||y|): cubic fixed point
    assert np.allclose(U, Mom / (np.linalg.norm(x) * np.linalg.norm(y)), atol=1e-6)
    assert np.array_equal(O.sign_ternary(U), np.outer(np.sign(x), np.sign(y)))


def test_ns_diagonal_gives_exact_zeros():
    Mom = np.zeros((3, 5))
    Mom[0, 0], Mom[1, 1], Mom[2, 2] = 3.0, -2.0, 1.0
    U, _ = O.polar_ns(Mom, 5, 1e-7, "fro")
    off = np.ones((3, 5), bool)
    off[[0, 1, 2], [0, 1, 2]] = False
    assert np.all(U[off] == 0.0)
    assert O.sign_ternary(U).tolist() == [[1, 0, 0, 0, 0], [0, -1, 0, 0, 0],
                                          [0, 0, 1, 0, 0]]
    # zeros pack as the +1 bit: only entry (1,1) = flat 6 is negative
    assert O.pack_signs(U).tolist() == [1 << 6]


def test_ns_orthogonal_input_spectral():
    rng = np.random.default_rng(7)
    Q, _ = np.linalg.qr(rng.standard_normal((6, 6)))
    U, s = O.polar_ns(Q, 5, 1e-7, "spectral", 3, O.CUBIC, rng.standard_normal(6))
    assert np.isclose(s, 1.0, rtol=1e-13)
    assert np.allclose(U, Q, atol=1e-6)          # p(1) = 1 for the cubic
    U5, _ = O.polar_ns(Q, 1, 1e-7, "spectral", 3, QUINTIC, rng.standard_normal(6))
    assert np.allclose(U5, (3.4445 - 4.7750 + 2.0315) * Q, atol=1e-6)


@pytest.mark.parametrize("shape", [(2, 2), (3, 3), (3, 5), (5, 3)])
def test_orthogonality_residual(shape):
    rng = np.random.default_rng(8)
    Mom = rng.standard_normal(shape) + 2.0 * np.eye(*shape)
    I = np.eye(min(shape))
    for U in (O.polar_svd(Mom), O.polar_ns(Mom, 60, 1e-7, "fro")[0]):
        G = U @ U.T if shape[0] <= shape[1] else U.T @ U
        assert np.abs(G - I).max() < 1e-6
    assert np.allclose(O.polar_ns(Mom, 60, 1e-7, "fro")[0], O.polar_svd(Mom), atol=1e-6)


@pytest.mark.parametrize("seed", range(6))
def test_polar_svd_2x2_closed_form(seed):
    # For 2x2 M with cof(M) = [[d, -c], [-b, a]], the polar factor is
    # (M + t cof M) / sqrt(|det(M + t cof M)|) with t = sign(det M).
    rng = np.random.default_rng(100 + seed)
    M = rng.standard_normal((2, 2))
    (a, b), (c, d) = M
    cof = np.array([[d, -c], [-b, a]])
    t = np.sign(np.linalg.det(M))
    N = M + t * cof
    R = N / np.sqrt(abs(np.linalg.det(N)))
    assert np.allclose(O.polar_svd(M), R, atol=1e-12)


def test_polar_ns_transpose_equivariant():
    rng = np.random.default_rng(9)
    Mom = rng.standard_normal((4, 7))
    u0 = rng.standard_normal(4)
    for scale, P in [("fro", 0), ("spectral", 4)]:
        A, _ = O.polar_ns(Mom, 5, 1e-7, scale, P, O.CUBIC, u0)
        B, _ = O.polar_ns(Mom.T, 5, 1e-7, scale, P, O.CUBIC, u0)
        assert np.allclose(A, B.T, atol=1e-14)


# --------------------------------------------------------------------------
# Apply and bfloat16 rounding
# --------------------------------------------------------------------------
def _bf16(bits):
    return np.array([bits << 16], dtype=np.uint32).view(np.float32)


def _bits(x):
    return int(np.asarray(x, np.float32).view(np.uint32)[0]) >> 16


@pytest.mark.parametrize("eta,D,want", [
    (2.0 ** -9, 1, 0x3F80),        # 1 - 2^-9: halfway, even neighbour is 1.0
    (3 * 2.0 ** -9, 1, 0x3F7E),    # 1 - 3*2^-9: halfway between 0x3F7F and 0x3F7E
    (2.0 ** -9, -1, 0x3F80),       # 1 + 2^-9: a quarter step, rounds down
    (2.0 ** -8, -1, 0x3F80),       # 1 + 2^-8: halfway, even is 0x3F80
    (3 * 2.0 ** -8, -1, 0x3F82),   # 1 + 3*2^-8: halfway between 0x3F81 and 0x3F82
    (2.0 ** -7, 0, 0x3F80),        # D = 0 leaves W
])
def test_apply_bf16_by_hand(eta, D, want):
    W = _bf16(0x3F80)                              # 1.0
    out = O.apply_update(W, np.array([D]), eta, "bf16")
    assert _bits(out) == want


def test_apply_eta_zero_is_identity():
    rng = np.random.default_rng(10)
    W32 = rng.standard_normal(1000).astype(np.float32)
    D = rng.choice([-1, 0, 1], 1000)
    assert np.array_equal(O.apply_update(W32, D, 0.0, "f32").view(np.uint32),
                          W32.view(np.uint32))
    Wb = O.bf16_round_nearest_even(W32)
    assert np.array_equal(O.apply_update(Wb, D, 0.0, "bf16").view(np.uint32),
                          Wb.view(np.uint32))


def test_apply_f32_single_rounding():
    # Difference of two float32 values with nearby exponents is exact in
    # float64; one rounding to float32 must then match the oracle.
    rng = np.random.default_rng(11)
    W = rng.uniform(0.5, 2.0, 5000).astype(np.float32)
    D = rng.choice([-1, 0, 1], 5000)
    eta = np.float32(0.02)
    want = (W.astype(np.float64) - float(eta) * D).astype(np.float32)
    assert np.array_equal(O.apply_update(W, D, eta, "f32"), want)


def test_bf16_rounding_against_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        # exact halfway cases: low 16 bits = 0x8000
                        ((rng.integers(0x3000, 0x5000, 5000).astype(np.uint32) << 16)
                         | np.uint32(0x8000)).view(np.float32)])
    ours = O.bf16_round_nearest_even(x).view(np.uint32) >> 16
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(ours.astype(np.uint16), ref.view(np.uint16))


# --------------------------------------------------------------------------
# The whole step: closed forms and invariances
# --------------------------------------------------------------------------
HP = dict(eta=0.02, beta=0.9, lam=0.01, eps=1e-7, K=5, scale="fro", P=0)


def _set(rng, mats, M):
    d = sum(r * c for r, c in mats)
    W = O.bf16_round_nearest_even((0.02 * rng.standard_normal(d)).astype(np.float32))
    Gs = [rng.standard_normal(d) for _ in range(M)]
    Moms = [0.1 * rng.standard_normal(d) for _ in range(M)]
    return W, Gs, Moms


def test_step_zero_steps_single_worker_closed_form():
    # K = 0 and M = 1: U = Mom'/(s+eps) so D = sign(Mom') with zero -> +1 bit.
    rng = np.random.default_rng(13)
    mats = [(4, 8), (8, 4)]
    W, Gs, Moms = _set(rng, mats, 1)
    hp = dict(HP, K=0)
    out = O.step(mats, W, Moms, Gs, hp, 0, False, "bf16")
    Mnew = 0.9 * Moms[0] + 0.1 * (Gs[0] + 0.01 * W.astype(np.float64))
    assert np.allclose(out["Mom"][0], Mnew, rtol=1e-13, atol=1e-16)
    want_D = np.where(Mnew < 0, -1, 1)
    assert np.array_equal(out["D"], want_D)
    assert np.array_equal(out["Wn"], O.bf16_round_nearest_even(
        (W - np.float32(0.02) * want_D.astype(np.float32)).astype(np.float32)))


def test_step_worker_permutation_invariant():
    rng = np.random.default_rng(14)
    mats = [(6, 10), (10, 6), (8, 8)]
    W, Gs, Moms = _set(rng, mats, 4)
    a = O.step(mats, W, Moms, Gs, HP, 0, False, "bf16")
    perm = [2, 0, 3, 1]
    b = O.step(mats, W, [Moms[i] for i in perm], [Gs[i] for i in perm], HP, 0,
               False, "bf16")
    assert np.array_equal(a["D"], b["D"])
    assert np.array_equal(a["Wn"].view(np.uint32), b["Wn"].view(np.uint32))
    assert np.array_equal(a["bits"][perm], b["bits"])


def test_step_eta_zero_and_bits_layout():
    rng = np.random.default_rng(15)
    mats = [(3, 7), (5, 5)]                   # 21 and 25 entries: ragged words
    W, Gs, Moms = _set(rng, mats, 3)
    out = O.step(mats, W, Moms, Gs, dict(HP, eta=0.0), 0, False, "bf16")
    assert np.array_equal(out["Wn"].view(np.uint32), W.view(np.uint32))
    assert out["bits"].shape == (3, 2)        # one word per matrix
    for m in range(3):
        assert np.array_equal(out["bits"][m, 0:1],
                              O.pack_signs(out["U"][m][0]))


def test_step_both_polar_steps_rank_one_closed_form():
    # post_vote = 2 with identical rank-one momenta x y^T (W = 0, Mom = 0):
    # every worker's polar factor is x y^T / (|x| |y|), whose signs are
    # s t^T (s = sign x, t = sign y); the vote of M = 3 identical buffers is
    # D = s t^T; D / sqrt(mn) has its one singular value at 1, a fixed point
    # of the cubic, so the update is W = -eta D / sqrt(mn).
    rng = np.random.default_rng(17)
    r, c = 5, 8
    x = rng.standard_normal(r) + np.sign(rng.standard_normal(r)) * 0.5
    y = rng.standard_normal(c) + np.sign(rng.standard_normal(c)) * 0.5
    G = np.outer(x, y).reshape(-1)
    d = r * c
    W = np.zeros(d, np.float32)
    out = O.step([(r, c)], W, [np.zeros(d)] * 3, [G] * 3, dict(HP, lam=0.0), 0, 2, "f32")
    st = np.outer(np.sign(x), np.sign(y))
    u = np.outer(x, y) / (np.linalg.norm(x) * np.linalg.norm(y))
    assert np.allclose(out["U"][0][0], u, atol=1e-12)
    assert np.array_equal(out["D"].reshape(r, c), st)
    assert np.allclose(out["Upost"][0], st / np.sqrt(d), atol=1e-12)
    want = (np.float32(0.0) - np.float32(0.02) * (st / np.sqrt(d)).astype(np.float32)).reshape(-1)
    assert np.allclose(out["Wn"], want, rtol=2e-7, atol=0)


def test_step_both_polar_steps_is_algorithm2_then_post_vote():
    # post_vote = 2: the buffers are Algorithm 2's (signs of the polar factor,
    # not of the momentum), and W moves by eta times the polar factor of the
    # majority, not by the majority itself.
    rng = np.random.default_rng(18)
    mats = [(6, 10), (9, 5)]
    W, Gs, Moms = _set(rng, mats, 3)
    a2 = O.step(mats, W, Moms, Gs, HP, 0, 0, "bf16")
    pv = O.step(mats, W, Moms, Gs, HP, 0, 1, "bf16")
    both = O.step(mats, W, Moms, Gs, HP, 0, 2, "bf16")
    assert np.array_equal(both["bits"], a2["bits"])
    assert not np.array_equal(both["bits"], pv["bits"])
    assert np.array_equal(both["D"], a2["D"])
    assert not np.array_equal(both["Wn"], a2["Wn"])
    with pytest.raises(ValueError):
        O.step(mats, W, Moms, Gs, HP, 0, 3, "bf16")


def test_step_post_vote_uses_majority_of_momentum_signs():
    rng = np.random.default_rng(16)
    mats = [(4, 6)]
    W, Gs, Moms = _set(rng, mats, 3)
    hp = dict(HP, scale="spectral", P=8)
    out = O.step(mats, W, Moms, Gs, hp, 0, True, "f32")
    signs = np.stack([np.where(m < 0, -1, 1) for m in out["Mom"]])
    want_D = np.sign(signs.sum(axis=0))       # M = 3 is odd: no ties
    assert np.array_equal(out["D"], want_D)
    Up, _ = O.polar_ns(want_D.reshape(4, 6).astype(np.float64), 5, 1e-7,
                       "spectral", 8)
    assert np.allclose(out["Upost"][0], Up, atol=1e-15)


# --------------------------------------------------------------------------
# Ternary sign buffers (section 3: sign(0) = 0; Algorithm 2 and Figure 1: the
# workers' signs summed as int8).  Diagonal momenta give polar factors that
# are exactly zero off the diagonal: sent as ternary signs those entries add
# nothing to the vote, which ties at 0 there and leaves W unchanged; sent as
# packed bits the same zeros vote +1 and move W by -eta.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("post_vote", [0, 2])
def test_step_ternary_diagonal_closed_form(post_vote):
    r, c, M = 4, 7, 3
    d = r * c
    diag = np.zeros((r, c), bool)
    diag[np.arange(r), np.arange(r)] = True
    # worker m's gradient is diagonal with signs s[m] on the diagonal
    s = np.array([[1, -1, 1, -1], [1, 1, -1, -1], [-1, -1, 1, 1]])
    Gs = []
    for m in range(M):
        G = np.zeros((r, c))
        G[np.arange(r), np.arange(r)] = s[m] * (1.0 + 0.25 * np.arange(r))
        Gs.append(G.reshape(-1))
    W = O.bf16_round_nearest_even(np.linspace(-0.05, 0.05, d).astype(np.float32))
    hp = dict(HP, lam=0.0)
    tern = O.step([(r, c)], W, [np.zeros(d)] * M, Gs, hp, 0, post_vote, "bf16",
                  encoding="ternary")
    pack = O.step([(r, c)], W, [np.zeros(d)] * M, Gs, hp, 0, post_vote, "bf16")
    # every worker's polar factor is diagonal with the signs of its gradient
    for m in range(M):
        U = tern["U"][m][0]
        assert np.all(U[~diag] == 0.0)
        assert np.array_equal(np.sign(U[np.arange(r), np.arange(r)]), s[m])
        assert np.array_equal(tern["signs"][m].reshape(r, c),
                              np.where(diag, np.sign(Gs[m].reshape(r, c)), 0))
    maj = np.sign(s.sum(axis=0))                       # M = 3: no ties
    want_t = np.zeros((r, c), np.int64)
    want_t[np.arange(r), np.arange(r)] = maj
    assert np.array_equal(tern["D"].reshape(r, c), want_t)
    want_p = np.ones((r, c), np.int64)                 # zeros travel as +1
    want_p[np.arange(r), np.arange(r)] = maj
    assert np.array_equal(pack["D"].reshape(r, c), want_p)
    assert "bits" not in tern and "signs" not in pack
    if post_vote == 0:
        # off the diagonal the ternary step leaves W bit for bit unchanged
        Wt = tern["Wn"].reshape(r, c)
        assert np.array_equal(Wt[~diag].view(np.uint32), W.reshape(r, c)[~diag].view(np.uint32))
        Wp = pack["Wn"].reshape(r, c)
        want = O.bf16_round_nearest_even(
            (W.reshape(r, c)[~diag] - np.float32(0.02)).astype(np.float32))
        assert np.array_equal(Wp[~diag].view(np.uint32), want.view(np.uint32))
    else:
        # the majority is diagonal with r singular values 1: the Frobenius
        # scale puts them at 1/sqrt(r), and K cubic steps map that through
        # the scalar polynomial; off the diagonal the factor stays exactly 0
        Up = tern["Upost"][0]
        assert np.all(Up[~diag] == 0.0)
        sig = 1.0 / (np.sqrt(r) + 1e-7)
        for _ in range(5):
            sig = 1.5 * sig - 0.5 * sig ** 3
        assert np.allclose(Up[np.arange(r), np.arange(r)], maj * sig, rtol=1e-12, atol=0)
        # packed: the +1 votes off the diagonal give a dense majority instead
        assert np.all(pack["Upost"][0][~diag] != 0.0)


def test_step_ternary_matches_packed_without_zeros():
    # with no exact zeros the two encodings carry the same signs
    rng = np.random.default_rng(19)
    mats = [(6, 10), (9, 5)]
    W, Gs, Moms = _set(rng, mats, 4)
    a = O.step(mats, W, Moms, Gs, HP, 0, 0, "bf16")
    b = O.step(mats, W, Moms, Gs, HP, 0, 0, "bf16", encoding="ternary")
    assert np.array_equal(a["D"], b["D"])
    assert np.array_equal(a["Wn"].view(np.uint32), b["Wn"].view(np.uint32))
    offs = np.cumsum([0] + [r * c for r, c in mats])
    woffs = np.cumsum([0] + [(r * c + 31) // 32 for r, c in mats])
    for m in range(4):
        for i, (r, c) in enumerate(mats):
            t = b["signs"][m, offs[i]:offs[i + 1]]
            assert np.all(t != 0)
            assert np.array_equal(O.pack_signs(t), a["bits"][m, woffs[i]:woffs[i + 1]])
    with pytest.raises(ValueError):
        O.step(mats, W, Moms, Gs, HP, 0, 0, "bf16", encoding="int4")


# --------------------------------------------------------------------------
# The spectral-norm normalized sign step (post_vote = 3): W moves by
# eta D / (||D||_2 + eps), ||D||_2 from P power steps.
# --------------------------------------------------------------------------
def test_normalized_sign_rank_one_closed_form():
    # D = s t^T with s, t in {-1, +1}: D D^T = n s s^T has one eigenvalue
    # m n, reached exactly after the first power step, so ||D||_2 = sqrt(mn)
    rng = np.random.default_rng(21)
    for (m, n) in [(4, 9), (9, 4), (6, 6)]:
        st = np.outer(rng.choice([-1, 1], m), rng.choice([-1, 1], n)).astype(np.float64)
        u0 = rng.standard_normal(min(m, n))
        for P in (2, 3, 7):
            got = O.normalized_sign(st, P, 1e-7, u0)
            assert np.allclose(got, st / (np.sqrt(m * n) + 1e-7), rtol=1e-14, atol=0)
    # a diagonal +-1 majority has all singular values 1
    D = np.zeros((3, 5)); D[0, 0], D[1, 1], D[2, 2] = 1, -1, 1
    assert np.allclose(O.normalized_sign(D, 4, 1e-7), D / (1 + 1e-7), rtol=1e-15)
    # a zero majority (every vote tied) gives a zero step
    assert np.all(O.normalized_sign(np.zeros((4, 4)), 3, 1e-7) == 0.0)


def test_normalized_sign_converges_to_spectral_norm():
    rng = np.random.default_rng(22)
    D = np.sign(rng.standard_normal((12, 30)))
    sig = np.linalg.norm(D, 2)
    got = O.normalized_sign(D, 200, 1e-7, rng.standard_normal(12))
    assert np.allclose(got, D / (sig + 1e-7), rtol=1e-10)
    assert abs(np.linalg.norm(got, 2) - 1.0) < 1e-6


def test_step_normalized_sign_uses_algorithm2_signs():
    rng = np.random.default_rng(23)
    mats = [(6, 10), (9, 5)]
    W, Gs, Moms = _set(rng, mats, 3)
    hp = dict(HP, P=6)
    a2 = O.step(mats, W, Moms, Gs, hp, 0, 0, "f32")
    ns = O.step(mats, W, Moms, Gs, hp, 0, 3, "f32")
    assert np.array_equal(ns["bits"], a2["bits"])          # the same workers
    assert np.array_equal(ns["D"], a2["D"])
    offs = np.cumsum([0] + [r * c for r, c in mats])
    for i, (r, c) in enumerate(mats):
        D = a2["D"][offs[i]:offs[i + 1]].astype(np.float64).reshape(r, c)
        assert np.array_equal(ns["Upost"][i], O.normalized_sign(D, 6, 1e-7))
        # a step of spectral norm at most about 1 (the estimate is below
        # ||D||_2, so slightly above 1 is possible)
        assert np.linalg.norm(ns["Upost"][i], 2) < 1.2
    want = (W - (np.float32(0.02) * np.concatenate(
        [u.reshape(-1) for u in ns["Upost"]]).astype(np.float32))).astype(np.float32)
    assert np.array_equal(ns["Wn"], want)
