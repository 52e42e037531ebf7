"""The benchmark's training step captured into a HIP graph (torch.cuda.CUDAGraph
over the library's calls) and replayed: the library records no memset and
allocates nothing, so the captured step must reproduce the eager step's
results exactly (every reduction of the path runs in a fixed order).

Each replay is checked against the eager results byte for byte, with the
outputs overwritten and unrelated eager work (and a synchronization) between
replays, so that a replay that skipped a kernel, or one whose launch depended
on state from the capture, would show.  GPT-2-small layer shapes (T = 8192,
adapter rank 16): every kernel of the step, the weight gradient's token split
included.
"""
import pytest
import torch

import bench as B
import sparse_gemm_02_amd as S
from workloads import WORKLOADS

from gpu_util import say

pytestmark = pytest.mark.gpu

OUTS = ("vs", "ms", "ps", "pd", "Y", "dX", "Xp", "dYp", "dW", "dL", "dR")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _snapshot(lins):
    return [{k: getattr(li, k).clone() for k in OUTS} for li in lins]


def _scramble(lins):
    for li in lins:
        for k in OUTS:
            getattr(li, k).view(torch.uint8).fill_(0xA5)


def _same(lins, ref):
    for li, r in zip(lins, ref):
        for k in OUTS:
            a, b = getattr(li, k).view(torch.uint8), r[k].view(torch.uint8)
            assert torch.equal(a, b), f"{li.name}.{k} differs from the eager step"


def test_step_replayed_from_a_graph_matches_eager():
    wl = WORKLOADS["gpt2_small"]
    say(f"[graph] gpt2_small T={wl.T} r={wl.r}")
    lins = [B.Linear(l.name, l.K, l.N, wl.T, wl.r, seed=0, index=i) for i, l in enumerate(wl.linears)]
    B.step(lins, S)                                  # eager warm-up: attributes set, plans made
    torch.cuda.synchronize()
    _scramble(lins)
    B.step(lins, S)
    torch.cuda.synchronize()
    ref = _snapshot(lins)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.step(lins, S)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.step(lins, S)
    torch.cuda.synchronize()

    a = torch.randn((1024, 1024), device="cuda")
    for rep in range(3):
        _scramble(lins)
        b = a @ a                                    # the program's own eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(lins, ref)
        assert torch.isfinite(b).all()
        say(f"[graph] replay {rep} equal")
    # an eager step after the replays still gives the same results
    _scramble(lins)
    B.step(lins, S)
    torch.cuda.synchronize()
    _same(lins, ref)
    del g
