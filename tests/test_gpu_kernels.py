"""GPU parity of the unit entry points (sign_pack, majority_vote, apply,
momentum) against the CPU oracle, through the C ABI."""
import json
import os

import numpy as np
import pytest

import oracle as O
from distributed_bit_matrix_amd import binding as B
from tests.gpu_common import f32, momentum_tol

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def u32(t):
    return host(t).view(np.uint32)


# --------------------------------------------------------------------------
# sign + 1-bit pack
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 31, 32, 33, 64, 65, 1000, 100003, 1 << 20])
def test_sign_pack_bit_exact(n):
    print(f"sign_pack n={n}", flush=True)
    rng = np.random.default_rng(n)
    U = rng.standard_normal(n).astype(np.float32)
    U[rng.random(n) < 0.05] = 0.0
    U[rng.random(n) < 0.05] = -0.0
    bits = B.sign_pack(dev(U))
    assert np.array_equal(u32(bits), O.pack_signs(U))


def test_sign_pack_tail_bits_zero():
    U = -np.ones(40, np.float32)
    out = dev(np.full(2, -1, np.int32))
    B.sign_pack(dev(U), bits=out)
    assert u32(out).tolist() == [0xFFFFFFFF, 0x000000FF]


# --------------------------------------------------------------------------
# majority vote
# --------------------------------------------------------------------------
def test_vote_blog_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "blog_vote_example.json")))
    dirs = np.array(g["directions"], np.float32).reshape(3, 4)
    bits = torch.cat([B.sign_pack(dev(dirs[m])) for m in range(3)])
    D, S = B.majority_vote(bits, 3, 4, 0, stride=1, want_sums=True)
    assert host(D).reshape(2, 2).tolist() == g["majority"]
    assert host(S).tolist() == [-1, -1, 3, 1]


def test_vote_mean_versus_majority(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "blog_mean_vs_majority.json")))
    x = np.array(g["directions"], np.float32)
    bits = torch.cat([B.sign_pack(dev(x[m:m + 1])) for m in range(3)])
    assert host(B.majority_vote(bits, 3, 1, 0, stride=1)).tolist() == [g["majority"]]


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 15, 16, 200, 255, 256, 1001])
@pytest.mark.parametrize("n", [7, 32, 1000, 65536 + 17])
def test_vote_bit_exact(M, n):
    print(f"vote M={M} n={n}", flush=True)
    rng = np.random.default_rng(M * 7919 + n)
    words = (n + 31) // 32
    stride = words + (3 if M > 1 else 0)
    bits = rng.integers(0, 2 ** 32, size=(M, stride), dtype=np.uint32)
    for tie in (0, 1):
        D, S = B.majority_vote(dev(bits.view(np.int32)), M, n, tie, stride=stride,
                               want_sums=True)
        sums = O.vote_sums_from_bits(bits[:, :words], n)
        assert np.array_equal(host(S).astype(np.int32), sums)
        assert np.array_equal(host(D), O.majority_from_sums(sums, tie))


@pytest.mark.parametrize("M", [2, 8, 200, 1000])
def test_vote_planted_ties(M):
    rng = np.random.default_rng(M)
    n = 4096 * 8
    words = n // 32
    bits = rng.integers(0, 2 ** 32, size=(M, words), dtype=np.uint32)
    mask = rng.integers(0, 2 ** 32, size=words, dtype=np.uint32) & \
        rng.integers(0, 2 ** 32, size=words, dtype=np.uint32)   # ~25% of entries
    bits[: M // 2] &= ~mask
    bits[M // 2:] |= mask
    sums = O.vote_sums_from_bits(bits, n)
    assert (sums == 0).mean() > 0.2
    for tie in (0, 1):
        D = B.majority_vote(dev(bits.view(np.int32)), M, n, tie)
        assert np.array_equal(host(D), O.majority_from_sums(sums, tie))


def test_vote_sums_beyond_int8():
    # 200 agreeing workers: sums of +-200 need more than int8
    M, n = 200, 64
    bits = np.zeros((M, 2), np.uint32)
    bits[:, 1] = 0xFFFFFFFF
    D, S = B.majority_vote(dev(bits.view(np.int32)), M, n, 0, want_sums=True)
    assert host(S).tolist() == [200] * 32 + [-200] * 32
    assert host(D).tolist() == [1] * 32 + [-1] * 32


# --------------------------------------------------------------------------
# apply
# --------------------------------------------------------------------------
@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["ternary", "float"])
@pytest.mark.parametrize("n", [5, 4096, 1000003])
def test_apply_bit_exact(w_dtype, kind, n):
    print(f"apply {w_dtype} {kind} n={n}", flush=True)
    rng = np.random.default_rng(n)
    W = (0.05 * rng.standard_normal(n)).astype(np.float32)
    if w_dtype == "bf16":
        W = O.bf16_round_nearest_even(W)
    eta = 0.0123
    if kind == "ternary":
        D = rng.integers(-1, 2, n).astype(np.int8)
        Wt = dev(W, torch.bfloat16 if w_dtype == "bf16" else None)
        B.apply(Wt, eta, D=dev(D))
    else:
        D = (0.3 * rng.standard_normal(n)).astype(np.float32)
        Wt = dev(W, torch.bfloat16 if w_dtype == "bf16" else None)
        B.apply(Wt, eta, Df=dev(D))
    want = O.apply_update(W, D, f32(eta), w_dtype)
    got = host(Wt.float())
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_apply_bf16_rounding_ties_by_hand():
    # W = 1.0; see the oracle pins for the derivation of each expected pattern
    cases = [(2.0 ** -9, 1, 0x3F80), (3 * 2.0 ** -9, 1, 0x3F7E), (2.0 ** -9, -1, 0x3F80),
             (2.0 ** -8, -1, 0x3F80), (3 * 2.0 ** -8, -1, 0x3F82)]
    for eta, d, want in cases:
        Wt = torch.ones(1, dtype=torch.bfloat16, device="cuda")
        B.apply(Wt, eta, D=torch.tensor([d], dtype=torch.int8, device="cuda"))
        assert int(host(Wt.view(torch.int16))[0]) & 0xFFFF == want


def test_apply_eta_zero_identity():
    W = torch.randn(10000, device="cuda").to(torch.bfloat16)
    W0 = W.clone()
    B.apply(W, 0.0, D=torch.ones(10000, dtype=torch.int8, device="cuda"))
    assert torch.equal(W.view(torch.int16), W0.view(torch.int16))


# --------------------------------------------------------------------------
# momentum
# --------------------------------------------------------------------------
@pytest.mark.parametrize("w_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [3, 1024, 500001])
def test_momentum_tolerance(w_dtype, n):
    rng = np.random.default_rng(n)
    G = rng.standard_normal(n).astype(np.float32)
    Mom = (0.3 * rng.standard_normal(n)).astype(np.float32)
    W = (0.02 * rng.standard_normal(n)).astype(np.float32)
    if w_dtype == "bf16":
        W = O.bf16_round_nearest_even(W)
    beta, lam = 0.9, 0.01
    Mt = dev(Mom)
    B.momentum(dev(G), dev(W, torch.bfloat16 if w_dtype == "bf16" else None), Mt, beta, lam)
    want = O.momentum_update(Mom, G, W, f32(beta), f32(lam))
    got = host(Mt).astype(np.float64)
    tol = momentum_tol(Mom, G, W, f32(beta), f32(lam))
    assert np.all(np.abs(got - want) <= tol)


def test_momentum_beta_zero_exact():
    # beta = 0, lambda = 0: Mom' = G exactly
    G = np.random.default_rng(0).standard_normal(999).astype(np.float32)
    Mt = dev(np.zeros(999, np.float32))
    B.momentum(dev(G), dev(np.zeros(999, np.float32)), Mt, 0.0, 0.0)
    assert np.array_equal(host(Mt), G)


# --------------------------------------------------------------------------
# ternary (int8) sign buffers and their vote: bit-exact against the oracle
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 15, 16, 17, 4095, 4096, 4097, 100003])
def test_sign_ternary_bit_exact(n):
    rng = np.random.default_rng(n)
    U = rng.standard_normal(n).astype(np.float32)
    U[rng.integers(0, n, max(1, n // 10))] = 0.0
    U[rng.integers(0, n, max(1, n // 20))] = -0.0
    S = host(B.sign_ternary(dev(U)))
    assert np.array_equal(S, O.sign_ternary(U))


def test_sign_ternary_nan_and_inf():
    # NaN has no sign: the library writes 0 for it (the pages define sign on
    # real numbers only); +-inf keep their signs
    U = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1e-45, -1e-45], np.float32)
    assert host(B.sign_ternary(dev(U))).tolist() == [0, 1, -1, 0, 0, 1, -1]


def test_vote_ternary_blog_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "blog_vote_example.json")))
    dirs = np.array(g["directions"], np.float32).reshape(3, 4)
    S = B.sign_ternary(dev(dirs.reshape(-1)))
    D, sums = B.majority_vote_ternary(S, 3, 4, 0, stride=4, want_sums=True)
    assert host(D).reshape(2, 2).tolist() == g["majority"]
    assert host(sums).tolist() == [-1, -1, 3, 1]


@pytest.mark.parametrize("M,n,stride", [(1, 100003, None), (2, 4096, None), (3, 4097, 4112),
                                        (8, 100000, None), (8, 100003, 100003),
                                        (200, 70001, 70016), (301, 4099, 4099)])
@pytest.mark.parametrize("tie", [0, 1])
def test_vote_ternary_bit_exact(M, n, stride, tie):
    # aligned strides take the 16-byte path, odd ones the byte path; signs
    # include zeros, and even M plants ties
    print(f"vote ternary M={M} n={n} stride={stride} tie={tie}", flush=True)
    rng = np.random.default_rng(M * 7919 + n)
    st = n if stride is None else stride
    Sg = rng.integers(-1, 2, size=(M, st)).astype(np.int8)
    if M % 2 == 0:
        Sg[M // 2:, : n // 3] = -Sg[: M // 2, : n // 3]       # exact ties
    D, sums = B.majority_vote_ternary(dev(Sg.reshape(-1)), M, n, tie, stride=st,
                                      want_sums=True)
    want_sums = O.vote_sums_from_signs(Sg[:, :n])
    assert np.array_equal(host(sums).astype(np.int32), want_sums)
    assert np.array_equal(host(D), O.majority_from_sums(want_sums, tie))


def test_vote_ternary_unaligned_start_and_sums_beyond_int8():
    M, n = 300, 5000
    buf = torch.ones(M * n + 1, dtype=torch.int8, device="cuda")
    S = buf[1:]                                   # start off a 16-byte boundary
    D, sums = B.majority_vote_ternary(S, M, n, 0, stride=n, want_sums=True)
    assert host(sums).tolist() == [300] * n
    assert host(D).tolist() == [1] * n


def test_vote_ternary_full_nanogpt_size():
    # the nanoGPT set's 84,934,656 entries over M = 8 int8 buffers
    from distributed_bit_matrix_amd import workloads as WL
    w = WL.get("nanogpt")
    n, M = w.d, w.M
    rng = np.random.default_rng(5)
    Sg = rng.integers(-1, 2, size=(M, n), dtype=np.int8)
    D = B.majority_vote_ternary(dev(Sg.reshape(-1)), M, n, 0)
    assert np.array_equal(host(D), O.majority_from_sums(O.vote_sums_from_signs(Sg), 0))


# --------------------------------------------------------------------------
# every flat call past 2^31 entries (64-bit indexing), checked at samples
# --------------------------------------------------------------------------
def _sampled_words(n):
    """Words (32-entry groups) to check: the first ones, those around entry
    2^31, the last ones (the last one partial), and 600 at random."""
    nw = (n + 31) // 32
    rng = np.random.default_rng(2031)
    mid = (1 << 31) // 32
    w = [0, 1, 2] + list(range(mid - 3, mid + 3)) + list(range(nw - 3, nw)) + \
        rng.integers(0, nw, 600).tolist()
    return np.unique(np.array(w, np.int64))


def _entries_of(words, n):
    """Entry index of every entry of the given words (past n: -1)."""
    e = words[:, None] * 32 + np.arange(32)[None, :]
    return np.where(e < n, e, -1)


def _gather(t, idx):
    """Values of device tensor t at host indices idx (-1 gives 0)."""
    i = torch.from_numpy(np.where(idx < 0, 0, idx).reshape(-1)).cuda()
    v = host(t.index_select(0, i)).reshape(idx.shape)
    return np.where(idx < 0, np.zeros((), v.dtype), v)


def test_flat_calls_past_2_31_entries():
    n = (1 << 31) + 4099          # neither a whole 32-entry word nor a whole vector
    free, _ = torch.cuda.mem_get_info()
    if free < (48 << 30):
        pytest.skip("needs 48 GiB of free device memory")
    print(f"flat calls n={n}", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2031)
    words = _sampled_words(n)
    ent = _entries_of(words, n)                       # (k, 32)
    valid = ent >= 0
    nw = (n + 31) // 32

    # momentum, bfloat16 W
    G = torch.randn(n, device="cuda", generator=gen)
    Mom = torch.randn(n, device="cuda", generator=gen).mul_(0.3)
    W = torch.randn(n, device="cuda", generator=gen).mul_(0.02).to(torch.bfloat16)
    g_s, m_s = _gather(G, ent), _gather(Mom, ent)
    w_s = _gather(W.view(torch.int16), ent).astype(np.uint16).astype(np.uint32) << 16
    w_s = w_s.view(np.float32)
    beta, lam = 0.9, 0.01
    B.momentum(G, W, Mom, beta, lam)
    del G
    got = _gather(Mom, ent).astype(np.float64)
    want = O.momentum_update(m_s, g_s, w_s, f32(beta), f32(lam))
    tol = momentum_tol(m_s, g_s, w_s, f32(beta), f32(lam))
    assert np.all((np.abs(got - want) <= tol)[valid])

    # signs of the new momentum, with zeros planted in the sampled words
    zero_at = torch.from_numpy(ent[valid][::5].copy()).cuda()
    Mom.index_fill_(0, zero_at, 0.0)
    U = Mom
    u_s = _gather(U, ent)
    bits = torch.empty((3, nw), dtype=torch.int32, device="cuda")
    B.sign_pack(U, bits=bits[0])
    bits[1:].random_(-(1 << 31), 1 << 31, generator=gen)     # workers 1 and 2
    b_s = host(bits.index_select(1, torch.from_numpy(words).cuda())).view(np.uint32)  # (3, k)
    for r, wd in enumerate(words):
        m = valid[r]
        assert O.pack_signs(u_s[r][m])[0] == b_s[0, r], ("pack", int(wd))

    # vote over the three packed buffers, then the apply with its result
    D, S = B.majority_vote(bits, 3, n, 0, stride=nw, want_sums=True)
    d_s, s_s = _gather(D, ent), _gather(S, ent).astype(np.int32)
    for r, wd in enumerate(words):
        m = int(valid[r].sum())
        sums = O.vote_sums_from_bits(b_s[:, r:r + 1], m)
        assert np.array_equal(s_s[r, :m], sums), ("vote sums", int(wd))
        assert np.array_equal(d_s[r, :m], O.majority_from_sums(sums, 0)), ("vote", int(wd))
    del S, bits
    eta = 0.0123
    B.apply(W, eta, D=D)
    got_w = _gather(W.view(torch.int16), ent).astype(np.uint16)
    want_w = O.apply_update(w_s[valid], d_s[valid], f32(eta), "bf16")
    assert np.array_equal(got_w[valid].astype(np.uint32) << 16, want_w.view(np.uint32))
    del D, W

    # ternary signs and their vote over two buffers (16-byte stride)
    st = (n + 15) // 16 * 16
    T = torch.empty(2 * st, dtype=torch.int8, device="cuda")
    B.sign_ternary(U, S=T[:n])
    T[st:].random_(-1, 2, generator=gen)
    t0 = _gather(T, ent)
    assert np.array_equal(t0[valid], O.sign_ternary(u_s[valid]))
    t1 = _gather(T, np.where(ent < 0, -1, ent + st))
    D2, S2 = B.majority_vote_ternary(T, 2, n, 1, stride=st, want_sums=True)
    got_s2 = _gather(S2, ent).astype(np.int32)[valid]
    want_s2 = O.vote_sums_from_signs(np.stack([t0[valid], t1[valid]]))
    assert np.array_equal(got_s2, want_s2)
    assert np.array_equal(_gather(D2, ent)[valid], O.majority_from_sums(want_s2, 1))


# --------------------------------------------------------------------------
# the largest worker count: sums reach +-32767 (int16)
# --------------------------------------------------------------------------
def test_vote_max_workers():
    M, n = 32767, 4099
    print(f"vote M={M} n={n}", flush=True)
    rng = np.random.default_rng(32767)
    words = (n + 31) // 32
    bits = rng.integers(0, 2 ** 32, size=(M, words), dtype=np.uint32)
    bits[:, 0] = 0                       # entries 0..31: every worker +1
    bits[:, 1] = 0xFFFFFFFF              # entries 32..63: every worker -1
    D, S = B.majority_vote(dev(bits.view(np.int32)), M, n, 0, want_sums=True)
    sums = O.vote_sums_from_bits(bits, n)
    assert sums[0] == M and sums[32] == -M
    assert np.array_equal(host(S).astype(np.int32), sums)
    assert np.array_equal(host(D), O.majority_from_sums(sums, 0))


def test_vote_ternary_max_workers():
    M, n = 32767, 4099
    print(f"vote ternary M={M} n={n}", flush=True)
    rng = np.random.default_rng(32768)
    Sg = rng.integers(-1, 2, size=(M, n)).astype(np.int8)
    Sg[:, :16] = 1
    Sg[:, 16:32] = -1
    for tie in (0, 1):
        D, sums = B.majority_vote_ternary(dev(Sg.reshape(-1)), M, n, tie, stride=n,
                                          want_sums=True)
        want = O.vote_sums_from_signs(Sg)
        assert want[0] == M and want[16] == -M
        assert np.array_equal(host(sums).astype(np.int32), want)
        assert np.array_equal(host(D), O.majority_from_sums(want, tie))
