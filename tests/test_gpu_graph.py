"""A whole decode step captured into a HIP graph and replayed: every replay
equals the eager step bit for bit (indices, candidate blocks, outputs, lse).

The library's group step enqueues kernels only (no memset nodes, no host
synchronisation), so a caller may capture it.  Each replay starts from
outputs overwritten with garbage, and the program's own eager work (another
eager step, a synchronisation) runs between replays.  The eager step itself is
checked against the oracle by the layer and full-size tests."""
import pytest
import torch

from fp4_kv_cache_02_amd import group, synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _state(run):
    return [run.topk_idx.clone(), run.cand.clone()] + [o.clone() for o in run.out] + [x.clone() for x in run.lse]


def _scribble(run):
    """Garbage into every buffer the step writes."""
    run.topk_idx.fill_(-5)
    if run.w.hier:
        run.cand.fill_(-5)
    for li in run.attended_layers():
        run.out[li].fill_(float("nan"))
        run.lse[li].fill_(float("nan"))


@pytest.mark.parametrize("kind,reduced", [("decode_128k", True), ("decode_1m", True), ("serving", True),
                                          ("decode_128k", False)])
def test_graph_replay_equals_eager(kind, reduced):
    w = synth.workload(kind, reduced=reduced)
    say("graph replay", w.name)
    run = group.GroupRunner(w, group.build_inputs(w))
    other = group.GroupRunner(w, group.build_inputs(w))      # eager work between replays
    run.step()
    torch.cuda.synchronize()
    ref = _state(run)

    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        run.step()
    torch.cuda.synchronize()
    for rep in range(3):
        _scribble(run)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _state(run)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), (w.name, rep, i)
        other.step()                 # eager work of the program between replays
        torch.cuda.synchronize()
