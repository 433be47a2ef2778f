"""torch.optim front end of libsignmuon: the Sign-Muon step over a model's
parameters, every step run by the HIP library.

Each parameter is one matrix of the step: a 2-D weight as it is, a
convolution kernel (out, in, kh, kw) flattened to (out, in*kh*kw) (the layout
of the ResNet-50-shaped parameter set), and a vector (bias, norm weight) as a
1 x n matrix, whose polar factor is the vector over its norm, so its signed
update is the sign of its momentum.  The pages define the method for
matrices and say nothing of other parameters; this is the reading taken
here.  Parameters of one group must share a device and a dtype (float32 or
bfloat16): at the first step they are moved into one flat buffer (each
parameter becomes a view of it), which the library updates in place.

Single process: the local worker is worker 0 of M.  With workers = 1 the
vote is over the local buffer alone (Algorithm 1).  With workers > 1,
`fill_other_workers(bits, stride, M)` is called before every step to write
the other M - 1 workers' sign buffers (slots 1..M-1 of `bits`), e.g. from an
exchange; the step then votes over all M.
"""
from __future__ import annotations

from typing import Callable, Optional

import torch

from . import binding as B


def matrix_shape(shape) -> tuple:
    """The (rows, cols) matrix a parameter of this shape is updated as."""
    shape = tuple(int(s) for s in shape)
    if len(shape) == 0:
        return (1, 1)
    if len(shape) == 1:
        return (1, shape[0])
    rows = shape[0]
    cols = 1
    for s in shape[1:]:
        cols *= s
    return (rows, cols)


class _GroupState:
    def __init__(self, params, group, post_vote, workers, encoding):
        dev = params[0].device
        dtype = params[0].dtype
        for p in params:
            if p.device != dev or p.dtype != dtype:
                raise ValueError("SignMuon: parameters of one group must share device and dtype")
            if dtype not in (torch.float32, torch.bfloat16):
                raise TypeError("SignMuon: parameters must be float32 or bfloat16")
            if not p.is_cuda:
                raise ValueError("SignMuon: parameters must be on a GPU")
        shapes = [matrix_shape(p.shape) for p in params]
        self.layout, self.d, self.words = B.default_layout(shapes)
        self.params = params
        # one flat W; every parameter becomes a view of it
        self.W = torch.empty(self.d, dtype=dtype, device=dev)
        for p, (_, _, off, _) in zip(params, self.layout):
            n = p.numel()
            self.W[off:off + n].copy_(p.detach().reshape(-1))
            p.data = self.W[off:off + n].view_as(p)
        self.G = torch.zeros(self.d, dtype=torch.float32, device=dev)
        self.Mom = torch.zeros(self.d, dtype=torch.float32, device=dev)
        self.M = int(workers)
        self.tern = encoding == "ternary"
        self.stride = self.d if self.tern else self.words
        self.bits = torch.zeros((self.M, self.stride),
                                dtype=torch.int8 if self.tern else torch.int32, device=dev)
        self.hp = B.HParams(eta=group["lr"], beta=group["beta"], lam=group["weight_decay"],
                            eps=group["eps"], K=group["K"], scale=group["scale"], P=group["P"],
                            coeffs=tuple(group["coeffs"]), precision=group["ns_precision"],
                            tie_value=group["tie_value"], encoding=encoding)
        with torch.cuda.device(dev):
            self.plan = B.StepPlan(self.layout, self.hp, post_vote, device=dev)


class SignMuon(torch.optim.Optimizer):
    """Sign-Muon (momentum, PolarNS, sign, majority vote, W <- W - lr D) on
    the GPU through libsignmuon.

    lr, beta, weight_decay, eps, K, scale ("fro" | "spectral"), P, coeffs
    (Newton-Schulz (a, b, c)), ns_precision ("bf16" | "bf16x3" | "f32") and
    tie_value are Algorithm 1's inputs and the library's hyper-parameters
    (per parameter group).  post_vote: 0 Algorithm 2, 1 polar step after the
    vote, 2 both, 3 the normalized sign step.  encoding: "packed" (1-bit
    buffers) or "ternary" (int8 signs)."""

    def __init__(self, params, lr: float = 0.02, beta: float = 0.9,
                 weight_decay: float = 0.0, eps: float = 1e-7, K: int = 5,
                 scale: str = "spectral", P: int = 5, coeffs=(1.5, -0.5, 0.0),
                 ns_precision: str = "bf16", tie_value: int = 0, post_vote: int = 0,
                 encoding: str = "packed", workers: int = 1,
                 fill_other_workers: Optional[Callable] = None):
        if workers < 1:
            raise ValueError("workers must be >= 1")
        if workers > 1 and fill_other_workers is None:
            raise ValueError("workers > 1 needs fill_other_workers to supply their signs")
        defaults = dict(lr=lr, beta=beta, weight_decay=weight_decay, eps=eps, K=K,
                        scale=scale, P=P, coeffs=tuple(coeffs), ns_precision=ns_precision,
                        tie_value=tie_value)
        super().__init__(params, defaults)
        self.post_vote = int(post_vote)
        self.encoding = encoding
        self.workers = int(workers)
        self.fill_other_workers = fill_other_workers
        self._groups = {}

    def _state(self, gi, group):
        st = self._groups.get(gi)
        if st is None:
            params = [p for p in group["params"]]
            st = _GroupState(params, group, self.post_vote, self.workers, self.encoding)
            self._groups[gi] = st
        return st

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        for gi, group in enumerate(self.param_groups):
            if not group["params"]:
                continue
            st = self._state(gi, group)
            for p, (_, _, off, _) in zip(st.params, st.layout):
                n = p.numel()
                if p.grad is None:
                    st.G[off:off + n].zero_()
                else:
                    st.G[off:off + n].copy_(p.grad.reshape(-1))
            st.plan.set_eta(float(group["lr"]))
            if self.workers > 1:
                self.fill_other_workers(st.bits, st.stride, self.workers)
            st.plan(st.G, st.W, st.Mom, st.bits, st.stride, self.workers, 0)
        return loss

    def nonfinite(self) -> bool:
        """Whether the last step of any group met a non-finite value (and
        skipped its update); waits for the GPU."""
        return any(st.plan.status() == B.SM_ENONFINITE for st in self._groups.values())
