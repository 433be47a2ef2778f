"""Helpers shared by the GPU parity tests (not a test module).

The gates below are the parity bars for this method:
* packing, vote, ties and the apply given D are bit-exact;
* the polar factor is within 2e-2 max-abs error when the Newton-Schulz
  products use bfloat16 operands, 1e-4 when they are float32;
* signs agree on at least 99.9% of entries and every disagreement sits where
  |U_oracle| < 1e-2 * rms(U_oracle);
* momentum agrees elementwise within 2^-22 * (beta |Mom| + (1-beta)(|G| +
  lambda |W|)) (float32 evaluation of the float64 recurrence).
"""
import numpy as np

import oracle as O


def f32(x):
    """A hyper-parameter as the GPU sees it (float32), back in float64."""
    return float(np.float32(x))


def oracle_hp(hp):
    """Binding HParams -> oracle dict with float32-rounded values."""
    return dict(eta=f32(hp.eta), beta=f32(hp.beta), lam=f32(hp.lam), eps=f32(hp.eps),
                K=hp.K, scale=hp.scale, P=hp.P,
                coeffs=tuple(f32(c) for c in hp.coeffs))


def sign_gate(U_gpu_signs_neg, U_oracle, min_agree=0.999, rel=1e-2):
    """Check packed-sign agreement.  U_gpu_signs_neg: bool array (GPU bit = 1,
    i.e. negative); U_oracle: float64 oracle polar factor.  Returns stats.

    At most a fraction 1 - min_agree of the entries may disagree, and every
    disagreement must sit within rel * rms of zero (where the operand
    precision cannot decide the sign)."""
    Uo = np.asarray(U_oracle, np.float64).reshape(-1)
    gneg = np.asarray(U_gpu_signs_neg, bool).reshape(-1)
    oneg = Uo < 0
    mis = gneg != oneg
    rms = float(np.sqrt(np.mean(Uo ** 2))) if Uo.size else 0.0
    agree = 1.0 - float(mis.mean()) if Uo.size else 1.0
    worst = float(np.abs(Uo[mis]).max() / rms) if mis.any() and rms > 0 else 0.0
    ok = agree >= min_agree and (not mis.any() or worst < rel)
    return ok, dict(agree=agree, worst_over_rms=worst, mismatches=int(mis.sum()))


def ternary_gate(S_gpu, U_oracle, min_agree=0.999, rel=1e-2):
    """sign_gate for int8 signs in {-1, 0, +1}: a disagreement is any entry
    whose sign differs from the oracle's (np.sign, with sign(0) = 0), held to
    the same fraction and magnitude bounds."""
    Uo = np.asarray(U_oracle, np.float64).reshape(-1)
    Sg = np.asarray(S_gpu).astype(np.int64).reshape(-1)
    mis = Sg != np.sign(Uo).astype(np.int64)
    rms = float(np.sqrt(np.mean(Uo ** 2))) if Uo.size else 0.0
    agree = 1.0 - float(mis.mean()) if Uo.size else 1.0
    worst = float(np.abs(Uo[mis]).max() / rms) if mis.any() and rms > 0 else 0.0
    ok = agree >= min_agree and (not mis.any() or worst < rel) and \
        bool(np.all(np.isin(Sg, (-1, 0, 1))))
    return ok, dict(agree=agree, worst_over_rms=worst, mismatches=int(mis.sum()))


def unpack_neg(words, n):
    """GPU packed words -> bool 'negative' array (test-side decoding)."""
    by = np.asarray(words).astype("<u4").view(np.uint8)
    return np.unpackbits(by, bitorder="little")[:n].astype(bool)


def momentum_tol(Mom_prev, G, W, beta, lam):
    return 2.0 ** -22 * (beta * np.abs(Mom_prev) + (1 - beta) * (np.abs(G) + lam * np.abs(W))) \
        + 1e-30


def polar_tol(precision):
    return 1e-4 if precision == "f32" else 2e-2


def w_round_tol(Wn, w_dtype, eta):
    """Per-entry bound on |U - (W - Wn) / eta| from storing Wn = W - eta U in
    w_dtype: half a unit in the last place of Wn (bfloat16: 8 significant
    bits), divided by eta; float32 rounding is far below the polar tolerances."""
    if w_dtype != "bf16":
        return np.zeros(np.shape(Wn))
    a = np.abs(np.asarray(Wn, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -126)))
    return 0.5 * 2.0 ** (e - 7) / eta
