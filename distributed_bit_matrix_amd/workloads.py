"""Seeded synthetic workloads for the Sign-Muon step (inputs only).

This module holds parameter-set shapes, hyper-parameter presets and seeded
NumPy generators for weights, gradients, power-iteration start vectors and
resident worker sign buffers.  It performs none of the method's arithmetic
and imports nothing but NumPy, so both the HIP path's tests and the CPU
oracle can be fed from it.

Workloads (the pages train ResNet-50 on CIFAR-10 and nanoGPT on OpenWebText;
those datasets are not used: parameter sets of the same shapes with Gaussian
gradients stand in for them):

* ``single``   one 256 x 512 float32 matrix, M = 3, float32 Newton-Schulz.
* ``resnet50`` the ResNet-50-shaped set of nine float32 matrices (conv
  kernels flattened to (out, in*kh*kw), plus the 10-class head), M = 4,
  bf16 Newton-Schulz with spectral scaling (P = 5).
* ``nanogpt``  12 transformer layers x {qkv 768x2304, attn-out 768x768,
  fc 768x3072, proj 3072x768}, bf16 weights, M = 8, Frobenius scaling.
* ``llm_mlp``  4096x4096 and 4096x16384 bf16, M = 16, spectral P = 10,
  gradients with a rank-16 signal, cubic coefficients; ``llm_mlp_quintic``
  the same with the quintic coefficients in split-bfloat16.
* ``postvote`` 512 x (128x128) + 64 x (1024x4096) float32, M = 200, the
  post-vote polar variant with spectral P = 8 and correlated worker noise.
* ``nanogpt_ternary`` the nanoGPT set with int8 ternary sign buffers;
  ``nanogpt_prepost`` the nanoGPT set with both polar steps;
  ``nanogpt_normalized`` the nanoGPT set with the normalized sign step.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

BASE_SEED = 20260504
QUINTIC = (3.4445, -4.7750, 2.0315)
CUBIC = (1.5, -0.5, 0.0)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    mats: Tuple[Tuple[int, int], ...]
    w_dtype: str            # "f32" | "bf16"
    M: int
    eta: float
    beta: float
    lam: float
    eps: float
    K: int
    scale: str              # "fro" | "spectral"
    P: int
    coeffs: Tuple[float, float, float]
    ns_precision: str       # "f32" | "bf16" | "bf16x3"
    tie_value: int
    T: int
    warmup: int
    post_vote: int          # 0: Algorithm 2; 1: polar after the vote; 2: both;
                            # 3: the spectral-norm normalized sign step
    signal_std: float       # std of the shared signal S
    seed_index: int
    encoding: str = "packed"   # worker sign buffers: "packed" | "ternary" (int8)

    @property
    def d(self) -> int:
        return sum(r * c for r, c in self.mats)

    @property
    def elem_offsets(self) -> List[int]:
        offs, o = [], 0
        for r, c in self.mats:
            offs.append(o)
            o += r * c
        return offs

    @property
    def word_offsets(self) -> List[int]:
        offs, o = [], 0
        for r, c in self.mats:
            offs.append(o)
            o += (r * c + 31) // 32
        return offs

    @property
    def words(self) -> int:
        return sum((r * c + 31) // 32 for r, c in self.mats)

    @property
    def seed(self) -> int:
        return BASE_SEED + self.seed_index

    def hp(self) -> dict:
        return dict(eta=self.eta, beta=self.beta, lam=self.lam, eps=self.eps,
                    K=self.K, scale=self.scale, P=self.P, coeffs=self.coeffs)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def ns_gflop(self) -> float:
        """Newton-Schulz flops per worker-step: K (4 m^2 n [+ 2 m^3]), m = min dim."""
        tot = 0.0
        for r, c in self.mats:
            m, n = min(r, c), max(r, c)
            per = 4.0 * m * m * n
            if self.coeffs[2] != 0.0:
                per += 2.0 * m ** 3
            tot += self.K * per
        return tot / 1e9


_COMMON = dict(eta=0.02, beta=0.9, lam=0.01, eps=1e-7, K=5, coeffs=CUBIC,
               tie_value=0)

RESNET50_MATS = ((64, 147), (64, 576), (128, 1152), (256, 2304), (512, 4608),
                 (256, 1024), (512, 2048), (2048, 512), (10, 2048))
NANOGPT_LAYER = ((768, 2304), (768, 768), (768, 3072), (3072, 768))

WORKLOADS = {
    "single": Workload(
        name="single", mats=((256, 512),), w_dtype="f32", M=3, scale="fro", P=0,
        ns_precision="f32", T=10, warmup=2, post_vote=False, signal_std=0.5,
        seed_index=0, **_COMMON),
    "resnet50": Workload(
        name="resnet50", mats=RESNET50_MATS, w_dtype="f32", M=4,
        scale="spectral", P=5, ns_precision="bf16", T=20, warmup=3,
        post_vote=False, signal_std=0.5, seed_index=1, **_COMMON),
    "nanogpt": Workload(
        name="nanogpt", mats=NANOGPT_LAYER * 12, w_dtype="bf16", M=8,
        scale="fro", P=0, ns_precision="bf16", T=20, warmup=3,
        post_vote=False, signal_std=0.3, seed_index=2, **_COMMON),
    "llm_mlp": Workload(
        name="llm_mlp", mats=((4096, 4096), (4096, 16384)), w_dtype="bf16", M=16,
        scale="spectral", P=10, ns_precision="bf16", T=5, warmup=2,
        post_vote=False, signal_std=0.0, seed_index=3, **_COMMON),
    # The same matrices with the quintic coefficients, in split-bfloat16 (the
    # precision in which the quintic meets the sign gate).
    "llm_mlp_quintic": Workload(
        name="llm_mlp_quintic", mats=((4096, 4096), (4096, 16384)), w_dtype="bf16", M=16,
        scale="spectral", P=10, ns_precision="bf16x3", T=5, warmup=2,
        post_vote=False, signal_std=0.0, seed_index=3,
        **dict(_COMMON, coeffs=QUINTIC)),
    "postvote": Workload(
        name="postvote", mats=((128, 128),) * 512 + ((1024, 4096),) * 64,
        w_dtype="f32", M=200, scale="spectral", P=8, ns_precision="bf16", T=10,
        warmup=2, post_vote=True, signal_std=0.5, seed_index=4, **_COMMON),
    # The nanoGPT set with int8 ternary sign buffers (one byte per entry and
    # worker, a zero sign kept as 0).
    "nanogpt_ternary": Workload(
        name="nanogpt_ternary", mats=NANOGPT_LAYER * 12, w_dtype="bf16", M=8,
        scale="fro", P=0, ns_precision="bf16", T=20, warmup=3,
        post_vote=False, signal_std=0.3, seed_index=6, encoding="ternary", **_COMMON),
    # The nanoGPT set with the spectral-norm normalized sign step
    # (post_vote = 3): ||D||_2 of each majority matrix from P = 5 power steps.
    "nanogpt_normalized": Workload(
        name="nanogpt_normalized", mats=NANOGPT_LAYER * 12, w_dtype="bf16", M=8,
        scale="fro", P=5, ns_precision="bf16", T=20, warmup=3,
        post_vote=3, signal_std=0.3, seed_index=7, **_COMMON),
    # The nanoGPT set with both polar steps (no configuration of its own is
    # given for this variant).
    "nanogpt_prepost": Workload(
        name="nanogpt_prepost", mats=NANOGPT_LAYER * 12, w_dtype="bf16", M=8,
        scale="fro", P=0, ns_precision="bf16", T=20, warmup=3,
        post_vote=2, signal_std=0.3, seed_index=5, **_COMMON),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(w: Workload, mats, M: Optional[int] = None, name=None) -> Workload:
    """The same recipe on a smaller parameter set (for oracle-sized tests)."""
    return w.replace(mats=tuple(mats), M=w.M if M is None else M,
                     name=name or (w.name + "-small"))


# --------------------------------------------------------------------------
# Generators.  Every stream is drawn from PCG64(SeedSequence([seed, tag...])).
# --------------------------------------------------------------------------
_TAG_W, _TAG_S, _TAG_N, _TAG_U0, _TAG_BITS, _TAG_MOM, _TAG_LR, _TAG_C = range(8)


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Map float32 inputs onto bfloat16-representable values by truncating
    the low 16 mantissa bits (input synthesis only)."""
    b = np.ascontiguousarray(np.asarray(x, np.float32)).view(np.uint32)
    return (b & np.uint32(0xFFFF0000)).view(np.float32)


def init_weights(w: Workload) -> np.ndarray:
    """W0 ~ N(0, 0.02^2), float32 values (bfloat16-representable for bf16 W)."""
    W = (0.02 * _rng(w.seed, _TAG_W).standard_normal(w.d, dtype=np.float32))
    return to_bf16_values(W) if w.w_dtype == "bf16" else W.astype(np.float32)


def init_momentum(w: Workload, worker: int = 0, std: float = 0.0) -> np.ndarray:
    """Initial momentum: zeros (the method's Mom_0), or N(0, std^2) for tests."""
    if std == 0.0:
        return np.zeros(w.d, np.float32)
    return (std * _rng(w.seed, _TAG_MOM, worker).standard_normal(
        w.d, dtype=np.float32)).astype(np.float32)


def _signal(w: Workload) -> np.ndarray:
    if w.name.startswith("llm_mlp"):
        # rank-16 signal per matrix: L = A B^T / 4 with A, B ~ N(0, 1)
        out = np.empty(w.d, np.float32)
        for i, ((r, c), off) in enumerate(zip(w.mats, w.elem_offsets)):
            g = _rng(w.seed, _TAG_LR, i)
            A = g.standard_normal((r, 16), dtype=np.float32)
            B = g.standard_normal((c, 16), dtype=np.float32)
            out[off:off + r * c] = ((A @ B.T) * 0.25).reshape(-1)
        return out
    return (w.signal_std * _rng(w.seed, _TAG_S).standard_normal(
        w.d, dtype=np.float32)).astype(np.float32)


_SIGNAL_CACHE = {}


def signal(w: Workload) -> np.ndarray:
    key = (w.name, w.mats, w.seed, w.signal_std)
    if key not in _SIGNAL_CACHE:
        _SIGNAL_CACHE.clear()
        _SIGNAL_CACHE[key] = _signal(w)
    return _SIGNAL_CACHE[key]


def gradient(w: Workload, t: int, worker: int) -> np.ndarray:
    """G_{t}^{(worker)} as float32: shared signal plus per-worker noise.

    postvote: S + 0.7 C_t + 0.3 E_{t,worker}; otherwise S + N_{t,worker}.
    """
    S = signal(w)
    if w.name.startswith("postvote"):
        C = _rng(w.seed, _TAG_C, t).standard_normal(w.d, dtype=np.float32)
        E = _rng(w.seed, _TAG_N, t, worker).standard_normal(w.d, dtype=np.float32)
        return (S + 0.7 * C + 0.3 * E).astype(np.float32)
    N = _rng(w.seed, _TAG_N, t, worker).standard_normal(w.d, dtype=np.float32)
    return (S + N).astype(np.float32)


def power_start(w: Workload) -> List[np.ndarray]:
    """Per-matrix power-iteration start vectors, N(0, 1), length min(r, c)."""
    return [_rng(w.seed, _TAG_U0, i).standard_normal(min(r, c)).astype(np.float32)
            for i, (r, c) in enumerate(w.mats)]


def random_bits(w: Workload, workers: int, tag: int = 0) -> np.ndarray:
    """Uniform random packed sign buffers, shape (workers, words), uint32."""
    g = _rng(w.seed, _TAG_BITS, tag)
    return g.integers(0, 2 ** 32, size=(workers, w.words), dtype=np.uint32)


def random_ternary(w: Workload, workers: int, zero_frac: float = 0.02,
                   tag: int = 0) -> np.ndarray:
    """Random int8 sign buffers, shape (workers, d): +1 or -1 with equal
    probability, 0 on a fraction zero_frac of the entries."""
    g = _rng(w.seed, _TAG_BITS, 100 + tag)
    s = np.where(g.random((workers, w.d)) < 0.5, -1, 1).astype(np.int8)
    s[g.random((workers, w.d)) < zero_frac] = 0
    return s


def planted_tie_bits(w: Workload, frac: float = 0.01, tag: int = 1) -> np.ndarray:
    """M buffers with exact ties planted on a fixed random entry mask.

    Off the mask every bit is uniform; on the mask, workers [0, M/2) hold
    the +1 bit (0) and the rest the -1 bit (1), so the vote there ties
    whenever M is even.
    """
    g = _rng(w.seed, _TAG_BITS, tag)
    bits = g.integers(0, 2 ** 32, size=(w.M, w.words), dtype=np.uint32)
    mask_words = np.zeros(w.words, np.uint32)
    for (r, c), woff in zip(w.mats, w.word_offsets):
        n = r * c
        m = g.random(n) < frac
        pad = np.zeros(((n + 31) // 32) * 32, bool)
        pad[:n] = m
        mask_words[woff:woff + (n + 31) // 32] = np.packbits(
            pad, bitorder="little").view("<u4")
    half = w.M // 2
    bits[:half] &= ~mask_words
    bits[half:] |= mask_words
    return bits, mask_words
