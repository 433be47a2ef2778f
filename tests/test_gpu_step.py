"""GPU parity of the fused signmuon_step against the oracle's step.

Every step starts from a state the oracle produced (its W_t and its float64
momentum rounded to float32), so differences do not compound; the other
workers' packed buffers are the oracle's own.  The checks per step:
* momentum of the local worker within the float32 evaluation bound;
* the local worker's packed signs pass the sign gate against the oracle's
  polar factor (post-vote: against its momentum; with both polar steps,
  post_vote = 2, against the polar factor as in Algorithm 2);
* W is bit-exact wherever the local worker's bit equals the oracle's (every
  vote input is then identical), and otherwise moves by at most one step;
* post-vote and both polar steps: the polar factor recovered from the W
  update is within the polar tolerance of the oracle's and passes the sign
  gate.
Full-size workloads are checked on sampled matrices the oracle can afford.
"""
import numpy as np
import pytest

import oracle as O
from distributed_bit_matrix_amd import binding as B
from distributed_bit_matrix_amd import workloads as WL
from tests.gpu_common import (f32, momentum_tol, oracle_hp, polar_tol, sign_gate, unpack_neg,
                               w_round_tol)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def hparams(w):
    return B.HParams(eta=w.eta, beta=w.beta, lam=w.lam, eps=w.eps, K=w.K, scale=w.scale,
                     P=w.P, coeffs=w.coeffs, precision=w.ns_precision,
                     tie_value=w.tie_value)


class GpuState:
    def __init__(self, w, hp):
        self.w = w
        self.layout, self.d, self.words = B.default_layout(w.mats)
        self.plan = B.StepPlan(self.layout, hp, w.post_vote)
        self.wdt = torch.bfloat16 if w.w_dtype == "bf16" else torch.float32

    def run(self, W, Mom0, G0, bits, u0):
        W_t = torch.from_numpy(np.ascontiguousarray(W, np.float32)).cuda().to(self.wdt)
        M_t = torch.from_numpy(np.ascontiguousarray(Mom0, np.float32)).cuda()
        G_t = torch.from_numpy(np.ascontiguousarray(G0, np.float32)).cuda()
        b_t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int32)).cuda()
        u_t = None if u0 is None else torch.from_numpy(u0).cuda()
        self.plan(G_t, W_t, M_t, b_t, self.words, bits.shape[0], 0, u0=u_t)
        st = self.plan.status()
        torch.cuda.synchronize()
        return (W_t.float().cpu().numpy(), M_t.cpu().numpy(),
                b_t.cpu().numpy().view(np.uint32), st)


def u0_concat(w):
    return np.concatenate(WL.power_start(w)).astype(np.float32) if w.scale == "spectral" \
        else None


def check_step(w, st, hp, W, Moms, Gs, u0s, sample=None, other_bits=None):
    """One step from the oracle's state; returns the oracle's output."""
    o = oracle_hp(hp)
    mats = list(w.mats)
    offs, woffs = w.elem_offsets, w.word_offsets
    idx = list(range(len(mats))) if sample is None else sample
    M = len(Gs) if other_bits is None else other_bits.shape[0]
    # oracle: local worker (0) on the sampled matrices
    Mom_new0 = O.momentum_update(Moms[0], Gs[0], W, o["beta"], o["lam"])
    U0 = {}
    for i in idx:
        r, c = mats[i]
        blk = Mom_new0[offs[i]:offs[i] + r * c].reshape(r, c)
        if w.post_vote == 1:
            U0[i] = blk
        else:
            U0[i], _ = O.polar_ns(blk, o["K"], o["eps"], o["scale"], o["P"], o["coeffs"],
                                  None if u0s is None else u0s[i].astype(np.float64))
    if other_bits is None:
        # the other workers are the oracle's own pipelines
        out = O.step(mats, W, Moms, Gs, o, w.tie_value, w.post_vote, w.w_dtype,
                     None if u0s is None else [u.astype(np.float64) for u in u0s])
        bits_in = out["bits"].copy()
    else:
        out = None
        bits_in = other_bits.copy()
        for i in idx:
            bits_in[0, woffs[i]:woffs[i] + (mats[i][0] * mats[i][1] + 31) // 32] = \
                O.pack_signs(U0[i])
    u0 = None if u0s is None else np.concatenate(u0s).astype(np.float32)
    Wg, Mg, bg, status = st.run(W, np.float32(Moms[0]), Gs[0], bits_in, u0)
    assert status == B.SM_OK
    # momentum (all entries)
    tol = momentum_tol(np.float32(Moms[0]), Gs[0], W, o["beta"], o["lam"])
    assert np.all(np.abs(Mg.astype(np.float64) - Mom_new0) <= tol)
    for i in idx:
        r, c = mats[i]
        n = r * c
        sl = slice(offs[i], offs[i] + n)
        wsl = slice(woffs[i], woffs[i] + (n + 31) // 32)
        gneg = unpack_neg(bg[0, wsl], n)
        ok, stats = sign_gate(gneg, U0[i])
        assert ok, (i, mats[i], stats)
        oneg = unpack_neg(bits_in[0, wsl], n)
        same = gneg == oneg
        # vote inputs identical where the local bit agrees
        sums = O.vote_sums_from_bits(bits_in[:, wsl], n)
        if w.post_vote:
            D = O.majority_from_sums(sums, w.tie_value).astype(np.float64).reshape(r, c)
            Upost, _ = O.polar_ns(D, o["K"], o["eps"], o["scale"], o["P"], o["coeffs"],
                                  None if u0s is None else u0s[i].astype(np.float64))
            if same.all():
                Ug = (W[sl].astype(np.float64) - Wg[sl].astype(np.float64)) / o["eta"]
                tol = polar_tol(hp.precision) + 1e-6 + w_round_tol(Wg[sl], w.w_dtype, o["eta"])
                assert np.all(np.abs(Ug - Upost.reshape(-1)) <= tol), (i, "post-vote")
                if w.w_dtype == "f32":
                    # (a bfloat16 W keeps too few bits for the signs of small U)
                    ok, stats = sign_gate(Ug < 0, Upost.reshape(-1))
                    assert ok, (i, "post-vote", stats)
            continue
        D = O.majority_from_sums(sums, w.tie_value)
        Wn = O.apply_update(W[sl], D, o["eta"], w.w_dtype)
        assert np.array_equal(Wg[sl][same].view(np.uint32), Wn[same].view(np.uint32)), i
        moved = np.abs(Wg[sl][~same].astype(np.float64) - W[sl][~same])
        assert np.all(moved <= 1.01 * o["eta"] + 1e-2 * np.abs(W[sl][~same])), i
    return out


def gradients(w, t, M):
    return [WL.gradient(w, t, m).astype(np.float64) for m in range(M)]


# --------------------------------------------------------------------------
# Oracle-sized workloads, several steps (common state from the oracle)
# --------------------------------------------------------------------------
SMALL = {
    "single": (WL.get("single"), None, 10),
    "resnet50": (WL.scaled(WL.get("resnet50"), [(64, 147), (128, 576), (256, 512),
                                                (512, 256), (10, 256)]), None, 3),
    "nanogpt": (WL.scaled(WL.get("nanogpt"), [(192, 576), (192, 192), (192, 768),
                                              (768, 192)] * 2), None, 3),
    "llm_mlp": (WL.scaled(WL.get("llm_mlp"), [(256, 256), (256, 1024)]), None, 2),
    "llm_mlp_quintic": (WL.scaled(WL.get("llm_mlp"), [(256, 256), (256, 1024)],
                                  name="llm_mlp-q").replace(coeffs=WL.QUINTIC,
                                                            ns_precision="bf16x3"), None, 2),
    "postvote": (WL.scaled(WL.get("postvote"), [(128, 128)] * 6 + [(256, 512)] * 2,
                           M=40), None, 3),
    # both polar steps: Algorithm 2's worker pipeline, then PolarNS of the vote
    "prepost": (WL.scaled(WL.get("nanogpt_prepost"), [(192, 576), (192, 192), (192, 768),
                                                      (768, 192)] * 2), None, 3),
    "prepost_spectral": (WL.scaled(WL.get("resnet50"), [(64, 147), (128, 576), (256, 512),
                                                        (512, 256), (10, 256)],
                                   name="resnet50-prepost").replace(post_vote=2), None, 2),
}


@pytest.fixture(params=["auto", "chains"])
def chain_mode(request, monkeypatch):
    """auto: the library's choice (one chain for these small sets); chains:
    the concurrent chains forced (SIGNMUON_CHAIN_MIN_GFLOP=0)."""
    if request.param == "chains":
        monkeypatch.setenv("SIGNMUON_CHAIN_MIN_GFLOP", "0")
    return request.param


@pytest.mark.parametrize("name", list(SMALL))
def test_step_multistep_small(name, chain_mode):
    w, _, T = SMALL[name]
    print(f"step {name} mats={len(w.mats)} M={w.M} T={T} {chain_mode}", flush=True)
    hp = hparams(w)
    st = GpuState(w, hp)
    W = WL.init_weights(w)
    Moms = [np.zeros(w.d) for _ in range(w.M)]
    u0s = WL.power_start(w) if w.scale == "spectral" else None
    for t in range(T):
        Gs = gradients(w, t, w.M)
        out = check_step(w, st, hp, W, Moms, Gs, u0s)
        W, Moms = out["Wn"], out["Mom"]


def test_step_nanogpt_iterate_form(monkeypatch):
    # the nanoGPT set's steps run in Gram space by default; the iterate form
    # is held to the same gates
    monkeypatch.setenv("SIGNMUON_NS_FORM", "iterate")
    w, _, T = SMALL["nanogpt"]
    hp = hparams(w)
    st = GpuState(w, hp)
    W = WL.init_weights(w)
    Moms = [np.zeros(w.d) for _ in range(w.M)]
    for t in range(T):
        out = check_step(w, st, hp, W, Moms, gradients(w, t, w.M), None)
        W, Moms = out["Wn"], out["Mom"]


# Sizes whose entry counts are odd: matrices start at unaligned offsets (no
# 16-byte vector access of W), widths are not multiples of 32 (signs packed
# by the separate pass), and the vote covers partial 2048-entry stretches.
ODD_MATS = [(5, 37), (33, 7), (45, 71), (64, 19), (3, 3)]
ODD = {
    "f32_M5": WL.scaled(WL.get("single"), ODD_MATS, M=5, name="odd-f32"),
    "bf16_M6": WL.scaled(WL.get("nanogpt"), ODD_MATS, M=6, name="odd-bf16"),
    "prepost_M5": WL.scaled(WL.get("nanogpt_prepost"), ODD_MATS, M=5, name="odd-prepost"),
}


@pytest.mark.parametrize("name", list(ODD))
def test_step_odd_sizes(name, chain_mode):
    w = ODD[name]
    assert any(o % 8 for o in w.elem_offsets)
    print(f"odd-size step {name} mats={w.mats} M={w.M}", flush=True)
    hp = hparams(w)
    st = GpuState(w, hp)
    W = WL.init_weights(w)
    Moms = [np.zeros(w.d) for _ in range(w.M)]
    for t in range(2):
        out = check_step(w, st, hp, W, Moms, gradients(w, t, w.M), None)
        W, Moms = out["Wn"], out["Mom"]


def test_step_nonfinite_skips_update():
    w = SMALL["nanogpt"][0]
    hp = hparams(w)
    st = GpuState(w, hp)
    W = WL.init_weights(w)
    G = WL.gradient(w, 0, 0)
    G[12345] = np.inf
    bits = WL.random_bits(w, w.M)
    Wg, Mg, bg, status = st.run(W, np.zeros(w.d, np.float32), G, bits, None)
    assert status == B.SM_ENONFINITE
    assert np.array_equal(Wg.view(np.uint32), W.view(np.uint32))
    # the next finite step clears the flag
    Wg, Mg, bg, status = st.run(W, np.zeros(w.d, np.float32), WL.gradient(w, 0, 0), bits,
                                None)
    assert status == B.SM_OK


def test_step_deterministic_and_permutation_invariant():
    w = SMALL["nanogpt"][0]
    hp = hparams(w)
    st = GpuState(w, hp)
    W = WL.init_weights(w)
    Mom = WL.init_momentum(w, 0, std=0.1)
    G = WL.gradient(w, 0, 0)
    bits = WL.random_bits(w, w.M)
    a = st.run(W, Mom, G, bits, None)
    b = st.run(W, Mom, G, bits, None)
    assert all(np.array_equal(x, y) for x, y in zip(a[:3], b[:3]))
    perm = np.concatenate([[0], 1 + np.random.default_rng(0).permutation(w.M - 1)])
    c = st.run(W, Mom, G, bits[perm], None)
    assert np.array_equal(a[0].view(np.uint32), c[0].view(np.uint32))


@pytest.mark.parametrize("post_vote", [0, 2])
def test_step_zero_steps_K0(post_vote):
    w = SMALL["nanogpt"][0].replace(K=0, post_vote=post_vote)
    hp = hparams(w)
    st = GpuState(w, hp)
    W = WL.init_weights(w)
    Moms = [WL.init_momentum(w, m, std=0.1).astype(np.float64) for m in range(w.M)]
    check_step(w, st, hp, W, Moms, gradients(w, 0, w.M), None)


# --------------------------------------------------------------------------
# Full-size workloads (the shapes the benchmark times), sampled matrices
# --------------------------------------------------------------------------
def full_case(name, sample, bits_kind="random"):
    w = WL.get(name)
    print(f"full-size step {name} d={w.d} M={w.M} sample={sample}", flush=True)
    hp = hparams(w)
    st = GpuState(w, hp)
    W = WL.init_weights(w)
    Mom0 = WL.init_momentum(w, 0, std=0.05).astype(np.float64)
    G0 = WL.gradient(w, 0, 0).astype(np.float64)
    if bits_kind == "ties":
        bits, _ = WL.planted_tie_bits(w)
    else:
        bits = WL.random_bits(w, w.M)
    u0s = WL.power_start(w) if w.scale == "spectral" else None
    check_step(w, st, hp, W, [Mom0], [G0], u0s, sample=sample, other_bits=bits)


def test_step_full_nanogpt():
    full_case("nanogpt", sample=[0, 1, 2, 3, 46, 47])


def test_step_full_resnet50():
    full_case("resnet50", sample=list(range(9)))


def test_step_full_nanogpt_prepost():
    full_case("nanogpt_prepost", sample=[0, 1, 46, 47])


@pytest.mark.slow
def test_step_full_llm_mlp():
    full_case("llm_mlp", sample=[0])


@pytest.mark.slow
def test_step_full_postvote():
    full_case("postvote", sample=[0, 1, 511, 512], bits_kind="ties")


# --------------------------------------------------------------------------
# Every worker's pipeline on the GPU (signmuon_worker_pipeline for workers
# 1..M-1, then signmuon_step for worker 0): each buffer against the oracle's
# worker, W unchanged by the worker calls, and the final W bit-exact wherever
# every worker's bit equals the oracle's.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["nanogpt", "postvote", "prepost"])
def test_all_workers_on_gpu(name, chain_mode):
    w, _, _ = SMALL[name]
    if name == "postvote":
        w = w.replace(M=12)
    print(f"all workers {name} mats={len(w.mats)} M={w.M}", flush=True)
    hp = hparams(w)
    o = oracle_hp(hp)
    st = GpuState(w, hp)
    mats = list(w.mats)
    offs, woffs = w.elem_offsets, w.word_offsets
    M = w.M
    W = WL.init_weights(w)
    Moms = [0.05 * WL.init_momentum(w, m, std=1.0) for m in range(M)]
    Gs = gradients(w, 0, M)
    u0s = WL.power_start(w) if w.scale == "spectral" else None
    out = O.step(mats, W, Moms, Gs, o, w.tie_value, w.post_vote, w.w_dtype,
                 None if u0s is None else [u.astype(np.float64) for u in u0s])

    W_t = torch.from_numpy(np.ascontiguousarray(W, np.float32)).cuda().to(st.wdt)
    W_in = W_t.clone()
    Mt = [torch.from_numpy(np.ascontiguousarray(np.float32(Moms[m]))).cuda() for m in range(M)]
    Gt = [torch.from_numpy(np.ascontiguousarray(Gs[m], np.float32)).cuda() for m in range(M)]
    rng = np.random.default_rng(7)
    b_t = torch.from_numpy(rng.integers(0, 2**31, size=(M, st.words), dtype=np.int64)
                           .astype(np.int32)).cuda()
    u_t = None if u0s is None else torch.from_numpy(np.concatenate(u0s).astype(np.float32)).cuda()
    for m in range(1, M):
        st.plan.worker_pipeline(Gt[m], W_t, Mt[m], b_t, st.words, M, m, u0=u_t)
    torch.cuda.synchronize()
    assert st.plan.status() == B.SM_OK
    assert torch.equal(W_t.view(torch.int16) if st.wdt == torch.bfloat16 else W_t.view(torch.int32),
                       W_in.view(torch.int16) if st.wdt == torch.bfloat16 else W_in.view(torch.int32))
    st.plan(Gt[0], W_t, Mt[0], b_t, st.words, M, 0, u0=u_t)
    assert st.plan.status() == B.SM_OK
    torch.cuda.synchronize()
    Wg = W_t.float().cpu().numpy()
    bg = b_t.cpu().numpy().view(np.uint32)
    for m in range(M):
        tol = momentum_tol(np.float32(Moms[m]), Gs[m], W, o["beta"], o["lam"])
        assert np.all(np.abs(Mt[m].cpu().numpy().astype(np.float64) - out["Mom"][m]) <= tol), m
    all_same = []
    for i, (r, c) in enumerate(mats):
        n = r * c
        wsl = slice(woffs[i], woffs[i] + (n + 31) // 32)
        same = np.ones(n, bool)
        for m in range(M):
            gneg = unpack_neg(bg[m, wsl], n)
            ref = out["Mom"][m][offs[i]:offs[i] + n] if w.post_vote == 1 \
                else out["U"][m][i].reshape(-1)
            ok, stats = sign_gate(gneg, ref)
            assert ok, (m, i, stats)
            same &= gneg == unpack_neg(out["bits"][m, wsl], n)
        all_same.append(same)
        if not w.post_vote:
            sl = slice(offs[i], offs[i] + n)
            assert np.array_equal(Wg[sl][same].view(np.uint32),
                                  out["Wn"][sl][same].view(np.uint32)), i
    if w.post_vote:
        # the post-vote update of a matrix is exact only if its whole majority matrix is
        for i, (r, c) in enumerate(mats):
            if all_same[i].all():
                sl = slice(offs[i], offs[i] + r * c)
                Ug = (W[sl].astype(np.float64) - Wg[sl].astype(np.float64)) / o["eta"]
                Uo = (W[sl].astype(np.float64) - out["Wn"][sl].astype(np.float64)) / o["eta"]
                tol = (polar_tol(hp.precision) + 1e-6 + w_round_tol(Wg[sl], w.w_dtype, o["eta"])
                       + w_round_tol(out["Wn"][sl], w.w_dtype, o["eta"]))
                assert np.all(np.abs(Ug - Uo) <= tol), i
