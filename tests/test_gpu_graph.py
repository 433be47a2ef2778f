"""A step recorded into a HIP graph (StepPlan.capture) and replayed gives
the eager step's results bit for bit (the step is deterministic: every
reduction has a fixed order), on every replay, with eager work between the
replays.  Inputs are reset to the same state before each replay."""
import numpy as np
import pytest

from distributed_bit_matrix_amd import binding as B
from distributed_bit_matrix_amd import workloads as WL
from tests.test_gpu_step import SMALL, hparams

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.skip(reason="HIP graph capture of the step is disabled: ending the capture "
                         "segfaulted inside the HIP runtime (host side); the sets here run "
                         "as one chain on the capturing stream, so the multi-stream fork "
                         "and join is not the cause, and no cause has been shown")
@pytest.mark.parametrize("name", ["nanogpt", "resnet50", "postvote", "llm_mlp_quintic"])
def test_graph_replay_matches_eager(name):
    w = SMALL[name][0]
    print(f"graph replay {name} mats={len(w.mats)} M={w.M}", flush=True)
    hp = hparams(w)
    layout, d, words = B.default_layout(w.mats)
    plan = B.StepPlan(layout, hp, w.post_vote)
    wdt = torch.bfloat16 if w.w_dtype == "bf16" else torch.float32
    W0 = torch.from_numpy(WL.init_weights(w)).cuda().to(wdt)
    Mom0 = torch.from_numpy(WL.init_momentum(w, 0, std=0.1).astype(np.float32)).cuda()
    G = torch.from_numpy(WL.gradient(w, 0, 0)).cuda()
    bits0 = torch.from_numpy(WL.random_bits(w, w.M).view(np.int32)).cuda()
    u0 = (torch.from_numpy(np.concatenate(WL.power_start(w))).cuda()
          if w.scale == "spectral" else None)

    W, Mom, bits = W0.clone(), Mom0.clone(), bits0.clone()
    plan(G, W, Mom, bits, words, w.M, 0, u0=u0)       # eager reference (and first call)
    torch.cuda.synchronize()
    assert plan.status() == B.SM_OK

    Wg, Mg, bg = W0.clone(), Mom0.clone(), bits0.clone()
    graph = plan.capture(G, Wg, Mg, bg, words, w.M, 0, u0=u0)
    for rep in range(3):
        Wg.copy_(W0)
        Mg.copy_(Mom0)
        bg.copy_(bits0)
        graph.replay()
        # eager work between replays, on other buffers, same workspace
        W2, M2, b2 = W0.clone(), Mom0.clone(), bits0.clone()
        plan(G, W2, M2, b2, words, w.M, 0, u0=u0)
        torch.cuda.synchronize()
        assert same(Wg, W) and same(Mg, Mom) and same(bg, bits), rep
        assert same(W2, W) and same(M2, Mom) and same(b2, bits), rep
    assert not same(W, W0)      # the step moved W
