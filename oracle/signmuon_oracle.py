"""Slow, plain CPU oracle for the Sign-Muon optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants
or helpers with the HIP library; it depends on NumPy alone.

Every floating-point quantity is carried in float64 unless the method fixes
a storage precision (the parameter W is float32 or bfloat16, and the apply
step is specified in float32 arithmetic).  Each function names the passage
of the pages it follows.  Sources:

* "SignMuon: Communication-Efficient Distributed Muon Optimization"
  (Mishra, Trivedi, Kumar; arXiv 2605.16311), rendering of the arXiv HTML:
  Algorithm 1 (single worker), Algorithm 2 (distributed, all-reduce),
  Figure 1, section 3 (preliminaries and notation), section 4 (the
  algorithm, including the Newton-Schulz paragraph), section 6
  (communication model).
* Blog "SignMuon: Matrix Directions, Majority Votes, and the Actual Bytes
  Sent" (the first author's site): sections "Keep local and shared
  operations separate", "A tiny aggregation calculation", "One bit of
  information is not automatically a one-bit all-reduce".

Readings taken where the pages are silent or disagree (each is also pinned
by a test under ``tests/``):

* sign(0) = 0 (section 3).  The 1-bit packed encoding stores bit = 1 iff the
  value is negative, so a zero packs as the +1 bit.
* A tied vote maps to 0 (the blog); a tie value of +1 (Algorithm 2's
  convention) is selectable.
* epsilon is added to the pre-scale: X0 = Mom / (s + eps).
* Power iteration (section 4 names it, without details): it runs on the
  smaller Gram matrix of Mom, from a caller-given start vector (default: all
  ones, normalised); each step is w = A u, u = w / |w|; after P steps
  s = sqrt(|w_P|).
* Newton-Schulz for an m x n matrix uses the smaller Gram: for m <= n,
  X <- a X + (b A + c A^2) X with A = X X^T; for m > n the same on X^T.
  This equals X (a I + b X^T X + c (X^T X)^2) in exact arithmetic.  The cubic
  is (a, b, c) = (1.5, -0.5, 0) as in section 4.
* Post-vote variant: workers send sign(Mom); after the vote the local polar
  step is applied to the majority matrix and W <- W - eta * U (U not
  re-signed).

Parity pins: every function below is pinned by ``tests/test_oracle_pins.py``
(worked examples from the pages, closed forms, exhaustive small cases).
"""
from __future__ import annotations

import numpy as np

CUBIC = (1.5, -0.5, 0.0)
SCALE_FRO = "fro"
SCALE_SPECTRAL = "spectral"


# --------------------------------------------------------------------------
# Momentum (Algorithm 1 and Algorithm 2: weight decay, then the EMA)
# --------------------------------------------------------------------------
def weight_decayed_gradient(G, W, lam):
    """G~ = G + lambda * W (Algorithm 1, weight-decay line; coupled L2)."""
    return np.asarray(G, np.float64) + float(lam) * np.asarray(W, np.float64)


def momentum_update(Mom, G, W, beta, lam):
    """Mom_{t+1} = beta * Mom_t + (1 - beta) * (G + lambda W), in float64.

    Algorithm 1 / Algorithm 2, local momentum line; Mom_0 = 0.
    """
    Gt = weight_decayed_gradient(G, W, lam)
    return float(beta) * np.asarray(Mom, np.float64) + (1.0 - float(beta)) * Gt


# --------------------------------------------------------------------------
# Pre-scaling (section 4, Newton-Schulz paragraph: spectral or Frobenius)
# --------------------------------------------------------------------------
def _short_side(X):
    """Return (Y, transposed) with Y the orientation having rows <= cols."""
    X = np.asarray(X, np.float64)
    if X.shape[0] > X.shape[1]:
        return X.T, True
    return X, False


def frobenius_scale(Mom):
    """s = ||Mom||_F = sqrt(sum of squares)."""
    Mom = np.asarray(Mom, np.float64)
    return float(np.sqrt(np.sum(Mom * Mom)))


def spectral_scale(Mom, P, u0=None):
    """Estimate sigma_max(Mom) by P power-iteration steps on the smaller Gram.

    A = Y Y^T with Y the short-side orientation of Mom.  u starts at u0
    normalised (default: the all-ones vector normalised).  Each step:
    w = A u, lam = |w|, u = w / lam.  Returns sqrt(lam) of the last step.
    A zero matrix gives 0.
    """
    if P < 1:
        raise ValueError("spectral scaling needs P >= 1")
    Y, _ = _short_side(Mom)
    A = Y @ Y.T
    r = A.shape[0]
    u = np.ones(r) if u0 is None else np.asarray(u0, np.float64).copy()
    if u.shape != (r,):
        raise ValueError("u0 must have min(rows, cols) entries")
    nu = np.linalg.norm(u)
    if nu == 0.0:
        raise ValueError("u0 must be nonzero")
    u = u / nu
    lam = 0.0
    for _ in range(P):
        w = A @ u
        lam = float(np.linalg.norm(w))
        if lam == 0.0:
            return 0.0
        u = w / lam
    return float(np.sqrt(lam))


def prescale(Mom, eps, scale, P=0, u0=None):
    """Return s for X0 = Mom / (s + eps)."""
    if scale == SCALE_FRO:
        return frobenius_scale(Mom)
    if scale == SCALE_SPECTRAL:
        return spectral_scale(Mom, P, u0)
    raise ValueError(f"unknown scale {scale!r}")


# --------------------------------------------------------------------------
# PolarNS (Algorithm 1 polar line; section 3 Muon paragraph; section 4)
# --------------------------------------------------------------------------
def newton_schulz(X0, K, coeffs=CUBIC):
    """K Newton-Schulz steps X <- a X + (b A + c A^2) X, A = X X^T.

    Runs on the short-side orientation and returns in the input's shape.
    """
    a, b, c = (float(v) for v in coeffs)
    Y, transposed = _short_side(X0)
    X = Y.copy()
    for _ in range(int(K)):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if transposed else X


def polar_ns(Mom, K, eps, scale, P=0, coeffs=CUBIC, u0=None):
    """PolarNS(Mom; K, eps, scale, P): pre-scale, then K Newton-Schulz steps.

    Returns (U, s) with U = X_K and s the scale used in X0 = Mom / (s + eps).
    """
    Mom = np.asarray(Mom, np.float64)
    s = prescale(Mom, eps, scale, P, u0)
    X0 = Mom / (s + float(eps))
    return newton_schulz(X0, K, coeffs), s


def polar_svd(Mom):
    """Exact polar factor U_s V_s^T from the thin SVD (section 3, Muon).

    Singular values below max(m, n) * 2^-52 * sigma_max are treated as zero,
    so a rank-deficient input gives U_r V_r^T.
    """
    Mom = np.asarray(Mom, np.float64)
    Us, sv, Vt = np.linalg.svd(Mom, full_matrices=False)
    if sv.size == 0 or sv[0] == 0.0:
        return np.zeros_like(Mom)
    keep = sv > max(Mom.shape) * np.finfo(np.float64).eps * sv[0]
    return Us[:, keep] @ Vt[keep, :]


# --------------------------------------------------------------------------
# Entrywise sign and 1-bit packing (section 3; section 6; blog bytes section)
# --------------------------------------------------------------------------
def sign_ternary(U):
    """Entrywise sign with sign(0) = 0, as int8 in {-1, 0, +1}."""
    return np.sign(np.asarray(U, np.float64)).astype(np.int8)


def pack_signs(U):
    """Pack entrywise signs of flattened U into little-endian uint32 words.

    Flat index j goes to bit (j mod 32) of word j // 32; bit = 1 iff U_j < 0.
    Tail bits of the last word are 0.  Implemented with numpy.packbits.
    """
    neg = (np.asarray(U).reshape(-1) < 0)
    n = neg.size
    nwords = (n + 31) // 32
    padded = np.zeros(nwords * 32, dtype=bool)
    padded[:n] = neg
    by = np.packbits(padded, bitorder="little")
    return by.view("<u4").astype(np.uint32)


def unpack_signs(words, n):
    """Inverse of pack_signs: +1 / -1 (int8) for the first n flat entries."""
    by = np.asarray(words, dtype="<u4").view(np.uint8)
    bits = np.unpackbits(by, bitorder="little")[:n]
    return (1 - 2 * bits.astype(np.int8)).astype(np.int8)


# --------------------------------------------------------------------------
# Majority vote (Algorithm 2 all-reduce and threshold; blog example)
# --------------------------------------------------------------------------
def vote_sums_from_signs(signs):
    """Integer sum over workers (axis 0) of sign arrays, in int32."""
    return np.sum(np.asarray(signs, dtype=np.int32), axis=0, dtype=np.int32)


def vote_sums_from_bits(bits, n):
    """Sum over workers of the +1/-1 signs decoded from packed buffers.

    bits: array of shape (M, words) of uint32; returns int32 sums of length n.
    """
    bits = np.asarray(bits, dtype=np.uint32)
    total = np.zeros(n, dtype=np.int32)
    for m in range(bits.shape[0]):
        total += unpack_signs(bits[m], n).astype(np.int32)
    return total


def vote_sums_int8_wrapping(signs):
    """The same sum accumulated in int8 with two's-complement wrap-around.

    Shows the overflow the blog warns about for large worker counts; not
    used by the step.
    """
    acc = np.zeros(np.asarray(signs[0]).shape, dtype=np.int8)
    with np.errstate(over="ignore"):
        for s in signs:
            acc = (acc.astype(np.int16) + np.asarray(s, np.int16))
            acc = ((acc + 128) % 256 - 128).astype(np.int8)
    return acc


def majority_from_sums(sums, tie_value=0):
    """D = sign(sum), with a zero sum (a tie) mapped to tie_value (0 or +1)."""
    if tie_value not in (0, 1):
        raise ValueError("tie_value must be 0 or 1")
    sums = np.asarray(sums, dtype=np.int64)
    D = np.sign(sums).astype(np.int8)
    D[sums == 0] = tie_value
    return D


# --------------------------------------------------------------------------
# Apply (Algorithm 1 / Algorithm 2 update line), specified in float32
# --------------------------------------------------------------------------
def bf16_round_nearest_even(x):
    """Round float32 values to the nearest bfloat16 value, ties to even.

    Finite inputs only.  Works from the definition: the two bfloat16
    neighbours of x (truncation toward zero and the next value away from
    zero) are formed from the bit pattern and compared in float64.
    Returns float32 arrays holding bfloat16-representable values.
    """
    x = np.ascontiguousarray(np.asarray(x, np.float32))
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding oracle expects finite values")
    bits = x.view(np.uint32)
    lo_bits = bits & np.uint32(0xFFFF0000)
    hi_bits = lo_bits + np.uint32(0x10000)  # next bfloat16 away from zero
    lo = lo_bits.view(np.float32).astype(np.float64)
    hi = hi_bits.view(np.float32).astype(np.float64)
    xv = x.astype(np.float64)
    d_lo = np.abs(xv - lo)
    d_hi = np.abs(hi - xv)
    lo_even = ((lo_bits >> np.uint32(16)) & np.uint32(1)) == 0
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~lo_even)
    out = np.where(pick_hi, hi_bits, lo_bits).astype(np.uint32)
    return out.view(np.float32)


def apply_update(W, D, eta, w_dtype="f32"):
    """W <- W - eta * D in float32 arithmetic, then stored in w_dtype.

    t = fl32(eta * D) (exact when D is ternary), W' = fl32(W - t); for a
    bfloat16 parameter W' is then rounded to bfloat16 (nearest, ties even).
    W must hold values representable in w_dtype.
    """
    W32 = np.asarray(W, np.float32)
    t = (np.float32(eta) * np.asarray(D, np.float32)).astype(np.float32)
    Wn = (W32 - t).astype(np.float32)
    if w_dtype == "f32":
        return Wn
    if w_dtype == "bf16":
        return bf16_round_nearest_even(Wn)
    raise ValueError(f"unknown w_dtype {w_dtype!r}")


# --------------------------------------------------------------------------
# One worker's local direction and one full step over a parameter set
# --------------------------------------------------------------------------
def worker_direction(Mom_new, hp, u0=None, post_vote=0):
    """What one worker transmits for one matrix.

    Pre-sign polar (Algorithm 2, and the first half of the variant with both
    polar steps, post_vote = 2): U = PolarNS(Mom_new), signs of U.
    Post-vote variant (post_vote = 1): the signs of Mom_new itself (polar
    happens after the vote).  Returns (values whose signs are sent, polar
    factor or None).
    """
    if post_vote == 1:
        return np.asarray(Mom_new, np.float64), None
    # post_vote 0, 2 and 3: Algorithm 2's worker pipeline
    U, _ = polar_ns(Mom_new, hp["K"], hp["eps"], hp["scale"], hp.get("P", 0),
                    hp.get("coeffs", CUBIC), u0)
    return U, U


def normalized_sign(D, P, eps, u0=None):
    """The spectral-norm normalized sign step of the analysis: D / ||D||_2.

    The abstract states the O(1/sqrt(T)) rate for the spectral-norm
    normalized sign step; section 4 (single-worker variant) normalizes D_t
    explicitly in the analysis, and section 4 (Newton-Schulz paragraph)
    estimates spectral norms by power iteration, all locally.  ||D||_2 is
    estimated as in the spectral pre-scale (P power steps on the smaller
    Gram from u0, s = sqrt(|w_P|)) and, as there, eps is added:
    returns D / (s + eps), so a zero D gives a zero step.
    """
    D = np.asarray(D, np.float64)
    s = spectral_scale(D, P, u0)
    return D / (s + float(eps))


def step(mats, W, Moms, Gs, hp, tie_value=0, post_vote=0, w_dtype="f32",
         u0s=None, encoding="packed"):
    """One Sign-Muon step for M workers over a parameter set.

    post_vote = 0: Algorithm 2 of the bittide.aicompass.dev rendering (polar
    before the sign, W moves by eta times the majority).  1: the post-vote
    variant (the momentum's signs are voted, W moves by eta times the polar
    factor of the majority matrix).  2: both polar steps, the abstract's
    optional local polar step on the sota2.com record read as a PolarNS of
    the voted matrix after Algorithm 2's exchange, with the same settings.
    3: the spectral-norm normalized sign step (Algorithm 2's workers, then
    W moves by eta times normalized_sign(majority), with hp's P and eps).

    mats: list of (rows, cols) in storage order; the flat arrays W (length
    d, values exact in w_dtype), Moms[m] and Gs[m] (length d each) hold the
    matrices row-major back to back.  hp: dict with eta, beta, lam, eps, K,
    scale, P and optionally coeffs.  u0s: optional list (per matrix) of
    power-iteration start vectors.

    encoding: what each worker sends.  "packed": the 1-bit buffers of the
    blog's byte count, where a zero travels as the +1 bit.  "ternary": the
    signs as int8 values in {-1, 0, +1} (section 3 defines sign(0) = 0;
    Algorithm 2 and Figure 1 sum the workers' signs as int8 in one
    all-reduce), so an exact zero adds nothing to the vote.

    Returns a dict: Mom (list of new momenta, float64), U (per worker, list
    of per-matrix polar factors or None), bits (M x words, uint32 per matrix
    concatenated with each matrix starting on a word boundary; packed only),
    signs (M x d int8 ternary signs; ternary only), sums (int32, length d),
    D (int8 ternary majority), Wn (new W, float32 array of w_dtype values),
    and for the post-vote variant Upost (per-matrix polar factor of the
    majority matrix).
    """
    if encoding not in ("packed", "ternary"):
        raise ValueError(f"encoding must be 'packed' or 'ternary', not {encoding!r}")
    M = len(Gs)
    offs = np.cumsum([0] + [r * c for r, c in mats])
    d = int(offs[-1])
    words = [((r * c) + 31) // 32 for r, c in mats]
    woffs = np.cumsum([0] + words)
    W = np.asarray(W, np.float64)
    new_moms, Us = [], []
    bits = np.zeros((M, int(woffs[-1])), dtype=np.uint32)
    signs = np.zeros((M, d), dtype=np.int8)
    for m in range(M):
        Mom_new = momentum_update(Moms[m], Gs[m], W, hp["beta"], hp["lam"])
        new_moms.append(Mom_new)
        per = []
        for i, (r, c) in enumerate(mats):
            blk = Mom_new[offs[i]:offs[i + 1]].reshape(r, c)
            u0 = None if u0s is None else u0s[i]
            vals, U = worker_direction(blk, hp, u0, post_vote)
            per.append(U)
            if encoding == "packed":
                bits[m, woffs[i]:woffs[i + 1]] = pack_signs(vals)
            else:
                signs[m, offs[i]:offs[i + 1]] = sign_ternary(vals).reshape(-1)
        Us.append(per)
    sums = np.zeros(d, dtype=np.int32)
    for i, (r, c) in enumerate(mats):
        if encoding == "packed":
            sums[offs[i]:offs[i + 1]] = vote_sums_from_bits(
                bits[:, woffs[i]:woffs[i + 1]], r * c)
        else:
            sums[offs[i]:offs[i + 1]] = vote_sums_from_signs(signs[:, offs[i]:offs[i + 1]])
    D = majority_from_sums(sums, tie_value)
    out = {"Mom": new_moms, "U": Us, "sums": sums, "D": D}
    if encoding == "packed":
        out["bits"] = bits
    else:
        out["signs"] = signs
    if post_vote not in (0, 1, 2, 3):
        raise ValueError(f"post_vote must be 0, 1, 2 or 3, not {post_vote!r}")
    if post_vote == 0:
        out["Wn"] = apply_update(W, D, hp["eta"], w_dtype)
        return out
    # Post-vote variant and the second half of post_vote = 2: local polar
    # step on the aggregated sign matrix; post_vote = 3: the majority
    # normalized by its spectral norm.
    Uflat = np.zeros(d, dtype=np.float64)
    Upost = []
    for i, (r, c) in enumerate(mats):
        Sbar = D[offs[i]:offs[i + 1]].astype(np.float64).reshape(r, c)
        u0 = None if u0s is None else u0s[i]
        if post_vote == 3:
            U = normalized_sign(Sbar, hp["P"], hp["eps"], u0)
        else:
            U, _ = polar_ns(Sbar, hp["K"], hp["eps"], hp["scale"], hp.get("P", 0),
                            hp.get("coeffs", CUBIC), u0)
        Upost.append(U)
        Uflat[offs[i]:offs[i + 1]] = U.reshape(-1)
    out["Upost"] = Upost
    # The update uses U as stored in float32 on the way into the apply.
    out["Wn"] = apply_update(W, Uflat.astype(np.float32), hp["eta"], w_dtype)
    return out
