"""ctypes binding of libsignmuon.so (argument marshalling only).

Every step of the Sign-Muon path runs in the HIP library; this module turns
torch tensors (device memory) and the current torch stream into the plain
pointers and sizes of the C ABI declared in ``include/signmuon.h``, and
raises ``SignMuonError`` on a non-zero status.  There is no fallback: if the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
# SIGNMUON_LIB may name another build of the same library (e.g. a tuning
# variant); the default is the in-tree build.
LIB_PATH = os.environ.get("SIGNMUON_LIB") or os.path.join(_HERE, "libsignmuon.so")

SM_OK, SM_EINVAL, SM_EWORKSPACE, SM_EHIP, SM_ENONFINITE, SM_ERANGE, SM_EUNSUPPORTED = \
    0, -1, -2, -3, -4, -5, -6
SM_F32, SM_BF16 = 0, 1
NS_F32, NS_BF16, NS_BF16X3 = 0, 1, 2
SCALE_FRO, SCALE_SPECTRAL = 0, 1
SIGNS_PACKED, SIGNS_TERNARY = 0, 1
MAX_WORKERS = 32767

EXPORTS = (
    "signmuon_strerror", "signmuon_abi_version", "signmuon_momentum",
    "signmuon_polar_ns_workspace", "signmuon_polar_ns", "signmuon_sign_pack",
    "signmuon_majority_vote", "signmuon_apply", "signmuon_step_workspace",
    "signmuon_step", "signmuon_step_profiled", "signmuon_get_status",
    "signmuon_worker_pipeline", "signmuon_sign_ternary", "signmuon_majority_vote_ternary",
    "signmuon_executor_create", "signmuon_executor_destroy", "signmuon_reset_status",
    "signmuon_polar_ns_static",
)
PHASES = {0: "start", 1: "momentum", 2: "prescale", 3: "gemm", 4: "pack", 5: "vote",
          6: "gram", 7: "square", 8: "update", 9: "gap"}


class SignMuonError(RuntimeError):
    def __init__(self, func: str, status: int, msg: str):
        super().__init__(f"{func}: {msg} (status {status})")
        self.status = status


class SmHparams(ctypes.Structure):
    _fields_ = [("eta", ctypes.c_float), ("beta", ctypes.c_float),
                ("lambda_", ctypes.c_float), ("eps", ctypes.c_float),
                ("K", ctypes.c_int32), ("scale", ctypes.c_int32),
                ("P", ctypes.c_int32), ("ns_a", ctypes.c_float),
                ("ns_b", ctypes.c_float), ("ns_c", ctypes.c_float),
                ("ns_precision", ctypes.c_int32), ("tie_value", ctypes.c_int32),
                ("sign_encoding", ctypes.c_int32)]


class SmProfile(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)),
                ("kinds", ctypes.POINTER(ctypes.c_int32)),
                ("capacity", ctypes.c_int32), ("count", ctypes.c_int32)]


class SmMatrix(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("elem_off", ctypes.c_int64), ("word_off", ctypes.c_int64)]


@dataclasses.dataclass
class HParams:
    eta: float = 0.02
    beta: float = 0.9
    lam: float = 0.01
    eps: float = 1e-7
    K: int = 5
    scale: str = "fro"              # "fro" | "spectral"
    P: int = 0
    coeffs: Tuple[float, float, float] = (1.5, -0.5, 0.0)
    precision: str = "bf16"         # "f32" | "bf16" | "bf16x3"
    tie_value: int = 0
    encoding: str = "packed"        # worker sign buffers: "packed" | "ternary"

    def to_c(self) -> SmHparams:
        prec = {"f32": NS_F32, "bf16": NS_BF16, "bf16x3": NS_BF16X3}[self.precision]
        scale = {"fro": SCALE_FRO, "spectral": SCALE_SPECTRAL}[self.scale]
        enc = {"packed": SIGNS_PACKED, "ternary": SIGNS_TERNARY}[self.encoding]
        a, b, c = self.coeffs
        return SmHparams(self.eta, self.beta, self.lam, self.eps, int(self.K), scale,
                         int(self.P), a, b, c, prec, int(self.tie_value), enc)


_LIB = None


def lib():
    """Load libsignmuon.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m distributed_bit_matrix_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                 ctypes.c_float, ctypes.c_size_t)
        hp = ctypes.POINTER(SmHparams)
        mats = ctypes.POINTER(SmMatrix)
        sig = {
            "signmuon_strerror": (ctypes.c_char_p, [ctypes.c_int]),
            "signmuon_abi_version": (i32, []),
            "signmuon_momentum": (i32, [vp, vp, i32, vp, i64, f32, f32, vp]),
            "signmuon_polar_ns_workspace": (sz, [i64, i64, hp]),
            "signmuon_polar_ns": (i32, [vp, vp, i64, i64, hp, vp, vp, sz, vp]),
            "signmuon_polar_ns_static": (i32, [vp, vp, i64, i64, hp, vp, vp]),
            "signmuon_sign_pack": (i32, [vp, vp, i64, vp]),
            "signmuon_majority_vote": (i32, [vp, i64, i32, i64, i32, vp, vp, vp]),
            "signmuon_sign_ternary": (i32, [vp, vp, i64, vp]),
            "signmuon_majority_vote_ternary": (i32, [vp, i64, i32, i64, i32, vp, vp, vp]),
            "signmuon_apply": (i32, [vp, i32, vp, vp, f32, i64, vp]),
            "signmuon_step_workspace": (sz, [mats, i32, hp, i32]),
            "signmuon_step": (i32, [mats, i32, hp, vp, vp, i32, vp, vp, i64, i32,
                                    i32, i32, vp, vp, sz, vp, vp]),
            "signmuon_worker_pipeline": (i32, [mats, i32, hp, vp, vp, i32, vp, vp, i64,
                                               i32, i32, i32, vp, vp, sz, vp, vp]),
            "signmuon_step_profiled": (i32, [mats, i32, hp, vp, vp, i32, vp, vp, i64,
                                             i32, i32, i32, vp, vp, sz,
                                             ctypes.POINTER(SmProfile), vp, vp]),
            "signmuon_get_status": (i32, [vp, vp]),
            "signmuon_executor_create": (i32, [ctypes.POINTER(vp)]),
            "signmuon_executor_destroy": (i32, [vp]),
            "signmuon_reset_status": (i32, [vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def strerror(status: int) -> str:
    return lib().signmuon_strerror(int(status)).decode()


def _check(func: str, status: int):
    if status != SM_OK:
        raise SignMuonError(func, status, strerror(status))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _wdtype(W) -> int:
    import torch
    if W.dtype == torch.float32:
        return SM_F32
    if W.dtype == torch.bfloat16:
        return SM_BF16
    raise TypeError("W must be float32 or bfloat16")


def _require(t, dtype, name):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous {dtype} CUDA tensor")


def mats_array(mats: Sequence[Tuple[int, int, int, int]]):
    arr = (SmMatrix * len(mats))()
    for i, (r, c, eo, wo) in enumerate(mats):
        arr[i] = SmMatrix(r, c, eo, wo)
    return arr


def default_layout(shapes: Sequence[Tuple[int, int]]):
    """Back-to-back layout: (rows, cols, elem_off, word_off) per matrix, the
    entry count d and the packed words per worker (int8 sign buffers take d
    bytes per worker, each matrix at its elem_off)."""
    out, eo, wo = [], 0, 0
    for r, c in shapes:
        out.append((r, c, eo, wo))
        eo += r * c
        wo += (r * c + 31) // 32
    return out, eo, wo


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------
def momentum(G, W, Mom, beta: float, lam: float, stream=None):
    import torch
    _require(G, torch.float32, "G")
    _require(Mom, torch.float32, "Mom")
    n = Mom.numel()
    if G.numel() != n or W.numel() != n:
        raise ValueError("G, W and Mom must have the same size")
    _check("signmuon_momentum", lib().signmuon_momentum(
        _ptr(G), _ptr(W), _wdtype(W), _ptr(Mom), n, beta, lam, _stream(stream)))


def polar_ns_workspace(rows: int, cols: int, hp: HParams) -> int:
    return int(lib().signmuon_polar_ns_workspace(rows, cols, ctypes.byref(hp.to_c())))


def polar_ns(X, hp: HParams, u0=None, U=None, ws=None, stream=None):
    import torch
    _require(X, torch.float32, "X")
    rows, cols = X.shape
    if U is None:
        U = torch.empty_like(X)
    nbytes = polar_ns_workspace(rows, cols, hp)
    if nbytes == 0:
        raise SignMuonError("signmuon_polar_ns_workspace", SM_EINVAL, "invalid arguments")
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=X.device)
    if u0 is not None:
        _require(u0, torch.float32, "u0")
    _check("signmuon_polar_ns", lib().signmuon_polar_ns(
        _ptr(X), _ptr(U), rows, cols, ctypes.byref(hp.to_c()), _ptr(u0), _ptr(ws),
        ws.numel(), _stream(stream)))
    return U


STATIC_SCRATCH_BYTES = 64 << 20


def polar_ns_static(X, hp: HParams, u0=None, U=None, stream=None):
    """PolarNS with the library's own per-GPU scratch array (no workspace,
    no allocation by the library; calls on one GPU must not overlap)."""
    import torch
    _require(X, torch.float32, "X")
    rows, cols = X.shape
    if U is None:
        U = torch.empty_like(X)
    _require(U, torch.float32, "U")
    if u0 is not None:
        _require(u0, torch.float32, "u0")
    _check("signmuon_polar_ns_static", lib().signmuon_polar_ns_static(
        _ptr(X), _ptr(U), rows, cols, ctypes.byref(hp.to_c()), _ptr(u0), _stream(stream)))
    return U


def sign_pack(U, bits=None, stream=None):
    import torch
    _require(U, torch.float32, "U")
    n = U.numel()
    if bits is None:
        bits = torch.empty((n + 31) // 32, dtype=torch.int32, device=U.device)
    _check("signmuon_sign_pack", lib().signmuon_sign_pack(_ptr(U), _ptr(bits), n,
                                                          _stream(stream)))
    return bits


def majority_vote(bits, M: int, n: int, tie_value: int = 0, stride: Optional[int] = None,
                  D=None, sums=None, want_sums: bool = False, stream=None):
    """bits: int32 tensor holding M worker buffers of `stride` words each."""
    import torch
    if stride is None:
        stride = (n + 31) // 32
    if D is None:
        D = torch.empty(n, dtype=torch.int8, device=bits.device)
    if want_sums and sums is None:
        sums = torch.empty(n, dtype=torch.int16, device=bits.device)
    _check("signmuon_majority_vote", lib().signmuon_majority_vote(
        _ptr(bits), stride, M, n, tie_value, _ptr(D), _ptr(sums), _stream(stream)))
    return (D, sums) if want_sums else D


def sign_ternary(U, S=None, stream=None):
    """int8 signs of U: +1, -1, or 0 for zero / NaN."""
    import torch
    _require(U, torch.float32, "U")
    n = U.numel()
    if S is None:
        S = torch.empty(n, dtype=torch.int8, device=U.device)
    _check("signmuon_sign_ternary", lib().signmuon_sign_ternary(_ptr(U), _ptr(S), n,
                                                                _stream(stream)))
    return S


def majority_vote_ternary(S, M: int, n: int, tie_value: int = 0,
                          stride: Optional[int] = None, D=None, sums=None,
                          want_sums: bool = False, stream=None):
    """S: int8 tensor holding M worker sign buffers of `stride` bytes each."""
    import torch
    if stride is None:
        stride = n
    if D is None:
        D = torch.empty(n, dtype=torch.int8, device=S.device)
    if want_sums and sums is None:
        sums = torch.empty(n, dtype=torch.int16, device=S.device)
    _check("signmuon_majority_vote_ternary", lib().signmuon_majority_vote_ternary(
        _ptr(S), stride, M, n, tie_value, _ptr(D), _ptr(sums), _stream(stream)))
    return (D, sums) if want_sums else D


def apply(W, eta: float, D=None, Df=None, stream=None):
    n = W.numel()
    _check("signmuon_apply", lib().signmuon_apply(
        _ptr(W), _wdtype(W), _ptr(D), _ptr(Df), eta, n, _stream(stream)))
    return W


def step_workspace(mats, hp: HParams, post_vote: int) -> int:
    arr = mats_array(mats)
    return int(lib().signmuon_step_workspace(arr, len(mats), ctypes.byref(hp.to_c()),
                                             int(post_vote)))


class Executor:
    """Owner of a signmuon_executor (the streams and events of the concurrent
    PolarNS chains), created on the current device; freed on close() or
    garbage collection."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check("signmuon_executor_create", lib().signmuon_executor_create(ctypes.byref(h)))
        self.handle = h

    def close(self):
        if self.handle is not None and self.handle.value:
            _check("signmuon_executor_destroy", lib().signmuon_executor_destroy(self.handle))
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class StepPlan:
    """Cached ctypes arguments of one parameter set for repeated steps.

    concurrent: run the PolarNS chains concurrently on an executor owned by
    the plan (default); False enqueues every kernel on the caller's stream."""

    def __init__(self, mats, hp: HParams, post_vote: int, device=None,
                 concurrent: bool = True):
        import torch
        self.mats = list(mats)
        self.arr = mats_array(self.mats)
        self.hp = hp
        self.hpc = hp.to_c()
        # 0: Algorithm 2; 1: polar step after the vote; 2: both
        self.post_vote = int(post_vote)
        nbytes = step_workspace(self.mats, hp, post_vote)
        if nbytes == 0:
            raise SignMuonError("signmuon_step_workspace", SM_EINVAL, "invalid arguments")
        dev = torch.device(device or "cuda")
        # zero-filled: the first bytes carry the non-finite flags
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        self.executor = None
        if concurrent:
            with torch.cuda.device(self.ws.device):
                self.executor = Executor()

    def _ex(self):
        return None if self.executor is None else self.executor.handle

    def set_eta(self, eta: float):
        self.hp.eta = eta
        self.hpc.eta = eta

    def __call__(self, G, W, Mom, bits, stride: int, M: int, local_worker: int = 0,
                 u0=None, stream=None):
        _check("signmuon_step", lib().signmuon_step(
            self.arr, len(self.mats), ctypes.byref(self.hpc), _ptr(G), _ptr(W),
            _wdtype(W), _ptr(Mom), _ptr(bits), stride, M, local_worker,
            int(self.post_vote), _ptr(u0), _ptr(self.ws), self.ws.numel(),
            self._ex(), _stream(stream)))

    def worker_pipeline(self, G, W, Mom, bits, stride: int, M: int, worker: int,
                        u0=None, stream=None):
        """Worker `worker`'s momentum, PolarNS and sign packing (no vote,
        W unchanged)."""
        _check("signmuon_worker_pipeline", lib().signmuon_worker_pipeline(
            self.arr, len(self.mats), ctypes.byref(self.hpc), _ptr(G), _ptr(W),
            _wdtype(W), _ptr(Mom), _ptr(bits), stride, M, worker,
            int(self.post_vote), _ptr(u0), _ptr(self.ws), self.ws.numel(),
            self._ex(), _stream(stream)))

    def profiled(self, prof: "SmProfile", G, W, Mom, bits, stride: int, M: int,
                 local_worker: int = 0, u0=None, stream=None):
        """Same step, recording prof's events after each phase."""
        _check("signmuon_step_profiled", lib().signmuon_step_profiled(
            self.arr, len(self.mats), ctypes.byref(self.hpc), _ptr(G), _ptr(W),
            _wdtype(W), _ptr(Mom), _ptr(bits), stride, M, local_worker,
            int(self.post_vote), _ptr(u0), _ptr(self.ws), self.ws.numel(),
            ctypes.byref(prof), self._ex(), _stream(stream)))

    def status(self, stream=None) -> int:
        return int(lib().signmuon_get_status(_ptr(self.ws), _stream(stream)))

    def reset_status(self, stream=None):
        _check("signmuon_reset_status", lib().signmuon_reset_status(_ptr(self.ws),
                                                                    _stream(stream)))

    def capture(self, G, W, Mom, bits, stride: int, M: int, local_worker: int = 0,
                u0=None):
        """Recording the step into a HIP graph is switched off: with this
        ROCm release, ending the capture of a step (torch.cuda.graph around
        one call) ended the process with a segmentation fault inside the
        runtime, also for sets that run as one chain on the capturing stream
        (so the fork and join of the executor's streams is not the cause),
        and no cause in the library has been found.  Steps are enqueued
        eagerly."""
        raise SignMuonError("StepPlan.capture", SM_EUNSUPPORTED,
                            "HIP graph capture of the step is disabled")
