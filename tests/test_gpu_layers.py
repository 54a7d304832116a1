"""End-to-end parity of CSA2 layer groups against the oracle, on the five
workloads at reduced sizes (same structure: schedules, planted keys,
hierarchical candidates, paging, prefill rows), through both entry points:
csa2_layer_step (one layer per call) and csa2_group_step (a Full/Reindex
layer and its Reuse layers per call, attention of the whole group in one
launch).  Indices and candidate blocks bit-exact after every group; outputs
within 2e-3."""
import numpy as np
import pytest
import torch

from fp4_kv_cache_02_amd import synth
from oracle import csa2_oracle as O
from tests.gpu_util import ATTN_TOL, host, lse_ok, rel_err, say

pytestmark = pytest.mark.gpu


def numpy_caches(w):
    """Main KV (quantised by the oracle from the seeded N(0,1) values, or raw
    FP4 bytes) and indexer keys at their slots."""
    n_slots, pt, _ = synth.slots_layout(w)
    if w.raw_fp4:
        P, S = synth.gen_fp4_raw(w, n_slots)
    else:
        P = np.zeros((n_slots, 256), np.uint8)
        S = np.zeros((n_slots, 32), np.uint8)
        for b in range(w.B):
            L = w.seq_lens[b]
            p, s = O.quantize_fp4(synth.gen_kv_values(w, b, 0, L))
            sl = synth.slot_index(w, pt, b, np.arange(L))
            P[sl], S[sl] = p, s
    from fp4_kv_cache_02_amd.group import k_idx_slots_from_synth
    K = k_idx_slots_from_synth(w, n_slots, pt)
    return P, S, K, pt, n_slots


def run_and_compare(w, by_group: bool, check_rows=None, equal_keys=False, zero_query=False):
    """equal_keys: every indexer key the same vector; zero_query: every
    indexer query zero -- both tie every score of a row (the Top-k and the
    candidate blocks are then the lowest positions / blocks)."""
    from fp4_kv_cache_02_amd import group
    P, S, K, pt, n_slots = numpy_caches(w)
    if equal_keys:
        K[:] = K[0]
    inp = group.build_inputs(w, kv_fp4=P, kv_scale=S, k_idx=K if equal_keys else None)
    if zero_query:
        for L in inp.layers:
            if L.q_idx is not None:
                L.q_idx.zero_()
    run = group.GroupRunner(w, inp)
    cache = O.Cache(P, S, K, w.seq_lens, pt, 64, w.slot_stride)
    row_seq = w.row_seq()
    state = O.GroupState(w.R)
    rows = list(range(w.R)) if check_rows is None else check_rows
    units = run.groups if by_group else [(li, 1) for li in range(len(w.schedule))]
    for ui, (li0, n) in enumerate(units):
        say(w.name, "group" if by_group else "layer", li0, n, w.schedule[li0:li0 + n])
        if by_group:
            run.step_group(ui)
        else:
            run.step_layer(li0)
        torch.cuda.synchronize()
        for li in range(li0, li0 + n):
            m = w.schedule[li]
            k, v, _, st, ln = synth.gen_swa(w, li)
            qi = synth.gen_q_idx(w, li) if m in "FI" else None
            if qi is not None and zero_query:
                qi = np.zeros_like(qi)
            q = synth.gen_q(w, li)
            blocks_only = m == "F" and w.hier and w.full_blocks_only
            res = O.layer_step(synth.MODES[m], cache, state, row_seq, qi, q, k, v, st, ln, group.SM_SCALE,
                               hier=w.hier, blocks_only=blocks_only, rows=rows, swa_shared=w.shared_slots)
            if m == "F" and w.hier:
                gc = host(run.cand)
                for r in rows:
                    assert np.array_equal(gc[r], state.cand[r]), (w.name, li, r)
            if blocks_only:
                continue
            gt = host(run.topk_idx)
            go, gl = host(run.out[li]), host(run.lse[li])
            for r in rows:
                assert np.array_equal(gt[r], state.topk[r]), (w.name, li, r)
                e = rel_err(go[r], res[r][0])
                assert np.all(e <= ATTN_TOL), (w.name, li, r, e.max())
                assert lse_ok(gl[r], res[r][1]), (w.name, li, r)


@pytest.mark.parametrize("kind", ["full_4k", "decode_128k", "decode_1m", "serving"])
def test_group_reduced_by_layer(kind):
    run_and_compare(synth.workload(kind, reduced=True), by_group=False)


@pytest.mark.parametrize("kind", ["full_4k", "decode_128k", "decode_1m", "serving"])
def test_group_reduced_by_group(kind):
    run_and_compare(synth.workload(kind, reduced=True), by_group=True)


def test_group_prefill_reduced():
    run_and_compare(synth.workload("prefill", reduced=True), by_group=True)


def test_group_causal_prefill_reduced():
    """A prefill chunk whose rows also see the chunk's own compressed entries
    once complete (each row a sequence of its own over shared slots, one
    shared window buffer)."""
    run_and_compare(synth.workload("causal_prefill", reduced=True), by_group=True)
    run_and_compare(synth.workload("causal_prefill", reduced=True), by_group=False, check_rows=[0, 1, 2, 31, 62, 63])


def test_group_prefill_rows_mode():
    """Enough rows x layers (128 x 6) that every (layer, row) is one block
    writing its output directly (no partials)."""
    w = synth.workload("prefill", reduced=True)
    w = synth.Workload("prefill_reduced_F5R_C128_E8192", w.seed, [8192], "FRRRRR", prefill_rows=128,
                       prefill_pos=16384, raw_fp4=True)
    run_and_compare(w, by_group=True, check_rows=list(range(0, 128, 9)) + [127])


@pytest.mark.parametrize("wl", ["decode_128k", "decode_1m"])
@pytest.mark.parametrize("kind", ["equal_keys", "zero_query"])
def test_group_tied_scores(wl, kind):
    """Degenerate indexer inputs: every score of a row tied, so the Top-512
    (and the candidate blocks) must be the lowest positions; the selections
    overflow their fast paths and take the general ones."""
    run_and_compare(synth.workload(wl, reduced=True), by_group=True, equal_keys=kind == "equal_keys",
                    zero_query=kind == "zero_query")


@pytest.mark.parametrize("sched,hier,blocks_only", [("FRRR", False, False), ("FIRRR", True, True),
                                                    ("FRRRIRRR", True, False)])
@pytest.mark.parametrize("by_group", [True, False])
def test_group_ragged_short_rows(sched, hier, blocks_only, by_group):
    """A batch of rows around the kernels' boundaries: an empty sequence (no
    Top-k entry, no window: lse -inf), rows shorter than one 8-position block,
    than one 64-position step and than the Top-512, and rows just past each;
    every Top-k keeps min(L, 512) positions, the candidate set min(ceil(L/8),
    2048) blocks."""
    w = synth.Workload(f"ragged_{sched}", 1201, [0, 1, 7, 63, 64, 65, 511, 512, 513, 2047, 5000], sched,
                       hier=hier, full_blocks_only=blocks_only)
    run_and_compare(w, by_group=by_group)


@pytest.mark.parametrize("R", [160, 300])
def test_group_many_decode_rows(R):
    """Decode batches past the split layouts: 160 rows x 4 layers = 640
    row-layers (one attention block per row-layer, per-sequence windows;
    split Top-512 over up to 256 rows) and 300 rows (one Top-k block per
    row); lengths uniform in [0, 5000], one empty sequence, raw FP4 bytes
    as the main KV, sampled rows checked."""
    r = np.random.default_rng(1300 + R)
    lens = [int(x) for x in r.integers(0, 5001, size=R)]
    lens[0], lens[1] = 0, 5000
    w = synth.Workload(f"decode_many_rows_b{R}", 1300 + R, lens, "FRRR", planted=0.01, raw_fp4=True)
    run_and_compare(w, by_group=True, check_rows=[0, 1, 2, 57, 101, 159, R - 1])


@pytest.mark.parametrize("lens,paged", [
    ([1048576, 131073, 32767, 32768, 32769, 500001, 65, 0], True),
    ([262144, 131073, 200000, 163840], False),
])
@pytest.mark.parametrize("kind", ["planted", "equal_keys"])
def test_group_long_full_rows(lens, paged, kind):
    """Full-layer Top-512 on rows past 131072 positions (one block per row
    descending the scan's maxima): a row of 2^20 positions, rows just past
    131072 and around multiples of 32768, short and empty rows in the same
    batch, paged and contiguous caches.  With every indexer key equal, every
    score of a row ties and the selection takes its general path."""
    w = synth.Workload(f"long_full_rows_{'paged' if paged else 'contig'}", 1600 + len(lens), lens, "FR",
                       paged=paged, planted=0.02, raw_fp4=True)
    run_and_compare(w, by_group=True, equal_keys=kind == "equal_keys")


@pytest.mark.parametrize("R", [24, 150])
def test_group_blocks_only_full_then_reuse(R):
    """A hierarchical Full layer that only builds the candidate blocks, with
    three Reuse layers in its group (they attend over the Top-K the Reindex
    layer of the group before left): the group's attention covers one layer
    fewer than the group holds, and at these batch sizes three layers take
    more attention partials than four would (24 rows: 6 blocks per
    row-layer for three layers against 4 for four, 432 partials against
    384; 150 rows: partials and a merge for three layers, one block per
    row-layer and no partials for four), so the group workspace must be
    sized for both counts."""
    r = np.random.default_rng(1700 + R)
    lens = [int(x) for x in r.integers(600, 5001, size=R)]
    w = synth.Workload(f"blocks_only_FIRRR_FRRR_b{R}", 1700 + R, lens, "FIRRRFRRR", hier=True,
                       full_blocks_only=True, planted=0.01, raw_fp4=True)
    run_and_compare(w, by_group=True, check_rows=sorted(set([0, 1, R // 2, R - 1])))


@pytest.mark.parametrize("kind", ["planted", "equal_keys"])
def test_group_paged_ragged_small_batch(kind):
    """A small paged batch whose attention launches fit on the CUs (8 rows x
    4 layers), so the Top-512's final selection runs inside the attention
    launch: ragged lengths with an empty row, rows shorter than the Top-512
    and rows of several segments, a Full and a Reindex group over the
    candidate blocks; with every indexer key equal the selection takes its
    general path there."""
    w = synth.Workload(f"paged_ragged_small_{kind}", 1701, [0, 1, 700, 2049, 5000, 12000, 3000, 64], "FRRRIRRR",
                       hier=True, paged=True, planted=0.02, raw_fp4=True)
    run_and_compare(w, by_group=True, equal_keys=kind == "equal_keys")
