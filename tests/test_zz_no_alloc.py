"""csa2_group_step_noalloc (the group step on the library's static scratch)
against csa2_group_step with a workspace of its own (GPU only): two calls in
a row, the second on a smaller input, each compared with the workspace
call on the same inputs -- Top-512 indices and candidate blocks bit-exact,
attention within 2e-3 max relative error per (row, head) (the same kernels
run, so the outputs agree bit for bit in practice)."""
import numpy as np
import pytest
import torch

from fp4_kv_cache_02_amd import group, synth
from tests.gpu_util import ATTN_TOL, host, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def C():
    from fp4_kv_cache_02_amd import csa2
    return csa2


def _compare(C, w):
    run = group.GroupRunner(w, group.build_inputs(w))
    need = max(C.csa2_group_workspace_bytes(synth.MODES[w.schedule[li0]], n, w.R, w.n_max, w.hier)
               for li0, n in run.groups)
    assert need <= C.NOALLOC_SCRATCH_BYTES
    for gi, (li0, n) in enumerate(run.groups):
        say("no-alloc", w.name, "group", gi, "layers", w.schedule[li0:li0 + n])
        mode = synth.MODES[w.schedule[li0]]
        # with a workspace of its own
        C.csa2_group_step(mode, run.group_args[gi], run.shared, run.ws)
        torch.cuda.synchronize()
        ref_idx, ref_cand = host(run.topk_idx).copy(), host(run.cand).copy()
        ref_out = [host(run.out[li]).copy() for li in range(li0, li0 + n)]
        ref_lse = [host(run.lse[li]).copy() for li in range(li0, li0 + n)]
        for li in range(li0, li0 + n):
            run.out[li].fill_(float("nan"))
            run.lse[li].fill_(float("nan"))
        # on the static scratch (the Reindex/Reuse inputs left by the group
        # before are the same for both calls)
        C.csa2_group_step_noalloc(mode, run.group_args[gi], run.shared)
        torch.cuda.synchronize()
        assert np.array_equal(host(run.topk_idx), ref_idx)
        assert np.array_equal(host(run.cand), ref_cand)
        for j, li in enumerate(range(li0, li0 + n)):
            if w.schedule[li] == "F" and w.hier and w.full_blocks_only:
                continue
            g = host(run.out[li])
            assert np.all(rel_err(g, ref_out[j]) <= ATTN_TOL), (w.name, li)
            assert np.array_equal(np.isneginf(host(run.lse[li])), np.isneginf(ref_lse[j]))
            fin = np.isfinite(ref_lse[j])
            assert np.allclose(host(run.lse[li])[fin], ref_lse[j][fin], rtol=1e-5, atol=1e-5)


def test_noalloc_matches_workspace_call(C):
    # first: the reduced 128K decode group (Full + 3 Reuse, 3 rows up to 12000
    # positions) and the hierarchical 1M group's structure at 40000 positions
    _compare(C, synth.workload("decode_128k", reduced=True))
    _compare(C, synth.workload("decode_1m", reduced=True))
    # then a smaller input on the same scratch
    _compare(C, synth.Workload("noalloc_small_F3R_b1_L3000", 1107, [3000], "FRRR"))


def test_noalloc_refuses_calls_beyond_its_scratch(C):
    """A Full layer over 32 rows of 1M positions needs ~194 MB of workspace:
    refused with CSA2_ERR_WORKSPACE before anything is enqueued."""
    w = synth.workload("full_4k")
    run = group.GroupRunner(w, group.build_inputs(w))
    s = C.make_shared(run.kv, run.kidx, run.inp.seq_len, 1 << 20, run.topk_idx, run.cand, hier=True)
    big = C.make_layer_args(run.inp.layers[0].q, run.inp.layers[0].swa_k, run.inp.layers[0].swa_v,
                            run.inp.layers[0].swa_start, run.inp.layers[0].swa_len, group.SM_SCALE, run.out[0],
                            q_idx=run.inp.layers[0].q_idx, R=32)
    arr = C.make_layer_array([big])
    assert C.csa2_group_workspace_bytes(C.FULL, 1, 32, 1 << 20, True) > C.NOALLOC_SCRATCH_BYTES
    with pytest.raises(C.Csa2Error) as e:
        C.csa2_group_step_noalloc(C.FULL, arr, s)
    assert e.value.status == 4
