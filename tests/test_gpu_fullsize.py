"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (the same inputs, the GPU-quantised main KV, the same group calls), on
sampled rows the oracle computes one by one: Top-512 indices and candidate
blocks bit-exact, outputs within 2e-3, and the GPU-quantised main-KV bytes
equal to the oracle's quantisation at every gathered position."""
import numpy as np
import pytest
import torch

from fp4_kv_cache_02_amd import synth
from oracle import csa2_oracle as O
from tests.gpu_util import ATTN_TOL, host, lse_ok, rel_err, say

pytestmark = pytest.mark.gpu


def oracle_caches(w, K, K_scale=None):
    """The oracle's own main KV (quantised by the oracle from the seeded source
    values) and the indexer keys at their slots (FP8 codes with K_scale when
    given)."""
    n_slots, pt, _ = synth.slots_layout(w)
    if w.raw_fp4:
        P, S = synth.gen_fp4_raw(w, n_slots)
    else:
        P = np.zeros((n_slots, 256), np.uint8)
        S = np.zeros((n_slots, 32), np.uint8)
        if w.kv_pool:
            pp, ps = O.quantize_fp4(synth.gen_kv_pool(w))
        for b in range(w.B):
            L = w.seq_lens[b]
            sl = synth.slot_index(w, pt, b, np.arange(L))
            if w.kv_pool:
                m = synth.gen_kv_pool_map(w, b)
                P[sl], S[sl] = pp[m], ps[m]
            else:
                P[sl], S[sl] = O.quantize_fp4(synth.gen_kv_values(w, b, 0, L))
    return O.Cache(P, S, K, w.seq_lens, pt, 64, w.slot_stride, k_idx_scale=K_scale), P, S, pt


def run_fullsize(w, rows, fp8_keys=False):
    """fp8_keys: the indexer keys in the FP8 form bench.py times, made from the
    workload's bf16 keys by the library's FP8 key quantiser; its bytes must
    equal the oracle's quantisation at every slot, and the oracle scores its
    own FP8 entries."""
    import dataclasses
    from fp4_kv_cache_02_amd import csa2, group
    n_slots, pt, _ = synth.slots_layout(w)
    say(w.name, "building inputs, rows checked", rows, "fp8 keys" if fp8_keys else "")
    K = group.k_idx_slots_from_synth(w, n_slots, pt)
    inp = group.build_inputs(w, k_idx=K)
    K_scale = None
    if fp8_keys:
        codes = torch.zeros((inp.k_idx.shape[0], 64), dtype=torch.uint8, device="cuda")
        scale = torch.zeros((inp.k_idx.shape[0],), dtype=torch.float32, device="cuda")
        csa2.csa2_fp8_key_quantize(inp.k_idx, codes, scale)
        inp = dataclasses.replace(inp, k_idx=codes, k_scale=scale)
        K, K_scale = O.quantize_fp8_keys(K)
        assert np.array_equal(host(codes), K) and np.array_equal(host(scale).view(np.uint32), K_scale.view(np.uint32))
    run = group.GroupRunner(w, inp)
    cache, P, S, _ = oracle_caches(w, K, K_scale)
    gP, gS = host(inp.kv_fp4), host(inp.kv_scale)
    row_seq = w.row_seq()
    state = O.GroupState(w.R)
    emax = 0.0
    for gi, (li0, n) in enumerate(run.groups):
        say(w.name, "group", gi, w.schedule[li0:li0 + n])
        run.step_group(gi)
        torch.cuda.synchronize()
        for li in range(li0, li0 + n):
            m = w.schedule[li]
            k, v, _, st, ln = synth.gen_swa(w, li)
            qi = synth.gen_q_idx(w, li) if m in "FI" else None
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
                b = int(row_seq[r])
                pos = state.topk[r][state.topk[r] >= 0]
                sl = O.slot_of(b, pos, pt, 64, w.slot_stride)
                assert np.array_equal(gP[sl], P[sl]) and np.array_equal(gS[sl], S[sl]), (w.name, li, r)
                e = rel_err(go[r], res[r][0])
                assert np.all(e <= ATTN_TOL), (w.name, li, r, e.max())
                assert lse_ok(gl[r], res[r][1]), (w.name, li, r)
                emax = max(emax, float(e.max()))
    say(w.name, "attention max relative error", f"{emax:.3e}")


def test_fullsize_decode_128k():
    w = synth.workload("decode_128k")
    run_fullsize(w, list(range(w.R)))


def test_fullsize_decode_128k_fp8_keys():
    """The 128K decode group on FP8 indexer keys (64 E4M3 codes + a float32
    scale per position), every row."""
    w = synth.workload("decode_128k")
    run_fullsize(w, list(range(w.R)), fp8_keys=True)


def test_fullsize_decode_1m():
    w = synth.workload("decode_1m")
    run_fullsize(w, [0])


def test_fullsize_decode_1m_fp8_keys():
    """The 1M hierarchical group on FP8 indexer keys: the Full layer's scan and
    candidate blocks, then the Reindex scoring of the candidates."""
    w = synth.workload("decode_1m")
    run_fullsize(w, [0], fp8_keys=True)


def test_fullsize_prefill():
    w = synth.workload("prefill")
    rng = np.random.default_rng(7)
    rows = sorted(set([0, 1, 127, 2048, w.R - 1] + list(rng.choice(w.R, size=5, replace=False))))
    run_fullsize(w, rows)


def test_fullsize_mixed_serving():
    w = synth.workload("serving")
    lens = np.array(w.seq_lens)
    rows = sorted(set([int(lens.argmax()), int(lens.argmin()), 5, 17]))
    run_fullsize(w, rows)


def test_fullsize_mixed_serving_fp8_keys():
    """The mixed paged serving batch on FP8 indexer keys (paged FP8 scan, the
    Top-512 of rows past 131072 positions, Reindex scoring of candidates)."""
    w = synth.workload("serving")
    lens = np.array(w.seq_lens)
    rows = sorted(set([int(lens.argmax()), int(lens.argmin()), 9]))
    run_fullsize(w, rows, fp8_keys=True)


def test_fullsize_causal_prefill():
    """Config 3 with the chunk's own 2048 entries under the completion mask
    (matrix-core indexer with per-row lengths)."""
    w = synth.workload("causal_prefill")
    rng = np.random.default_rng(8)
    rows = sorted(set([0, 1, 2, 127, 2048, w.R - 2, w.R - 1] + list(rng.choice(w.R, size=5, replace=False))))
    run_fullsize(w, rows)
