"""Sign-Muon optimizer step for MI355X (gfx950): HIP kernels behind a C ABI.

The compute path lives in ``libsignmuon.so`` (built from ``csrc/``); the
Python side only marshals arguments (see ``binding``); ``optim`` is a
torch.optim front end over it.  ``workloads`` holds seeded synthetic inputs.
"""
__all__ = ["binding", "optim", "workloads"]
