"""Per-kernel parity of the HIP library against the CPU oracle (GPU only).

Bars: quantiser bytes, indexer scores, block maxima, Top-K indices and
candidate blocks bit-exact; attention outputs within 2e-3 max relative error
per (row, head) of the float64 oracle."""
import math

import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O
from tests.gpu_util import (ATTN_TOL, bf16, dev, host, lse_ok, paged_layout, place, rand_fp4, rel_err, say,
                            workspace)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def C():
    from fp4_kv_cache_02_amd import csa2
    return csa2


# --------------------------------------------------------------- quantiser --

def test_quantize_bitexact(C):
    rng = np.random.default_rng(101)
    N = 3000
    x = rng.standard_normal((N, 512)).astype(np.float32)
    blk = np.exp(rng.uniform(-14, 9, size=(N, 32))).astype(np.float32)
    x = (x.reshape(N, 32, 16) * blk[:, :, None]).reshape(N, 512).astype(np.float32)
    x[0, :16] = 0.0
    x[1, :16] = -0.0
    x[2, 16:32] = 3000.0               # saturating scale
    x[3, :] = rng.choice(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32), 512)
    say("quantize N", N)
    ref_p, ref_s = O.quantize_fp4(x)
    fp4 = torch.zeros((N, 256), dtype=torch.uint8, device="cuda")
    sc = torch.zeros((N, 32), dtype=torch.uint8, device="cuda")
    C.csa2_fp4_quantize(dev(x), fp4, sc)
    torch.cuda.synchronize()
    assert np.array_equal(host(sc), ref_s)
    assert np.array_equal(host(fp4), ref_p)
    # scattered destination slots
    perm = rng.permutation(N + 100)[:N].astype(np.int64)
    fp4b = torch.zeros((N + 100, 256), dtype=torch.uint8, device="cuda")
    scb = torch.zeros((N + 100, 32), dtype=torch.uint8, device="cuda")
    C.csa2_fp4_quantize(dev(x), fp4b, scb, dst_slot=dev(perm))
    torch.cuda.synchronize()
    assert np.array_equal(host(fp4b)[perm], ref_p) and np.array_equal(host(scb)[perm], ref_s)


# ------------------------------------------------------------ index score --

@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("weighted", [False, True])
def test_index_score_bitexact(C, paged, weighted):
    rng = np.random.default_rng(202 + paged * 2 + weighted)
    lens = [5000, 1, 777, 64, 3000]
    B = len(lens)
    n_max = max(lens) + 13
    kseq = [bf16(rng, (L, 64), 1.0 + 3 * (b == 0)) for b, L in enumerate(lens)]
    kseq[2][5] = 0  # an all-zero key
    if paged:
        pt, n_slots = paged_layout(rng, lens)
        stride = 0
    else:
        pt, stride, n_slots = None, n_max, B * n_max
    kslots = place(kseq, lens, n_slots, pt, stride, 64, np.uint16)
    # rows: two rows read sequence 0
    row_seq = np.array([0, 1, 2, 3, 4, 0], np.int32)
    R = len(row_seq)
    q = bf16(rng, (R, 4, 64))
    q[1] = 0
    w = rng.uniform(-0.5, 2.0, size=(R, 4)).astype(np.float32) if weighted else None
    say("index_score paged", paged, "weighted", weighted, "R", R)
    kc = C.make_cache(dev(kslots), page_table=dev(pt) if paged else None, seq_stride=stride)
    scores = torch.full((R, n_max), float("nan"), device="cuda")
    bmax = torch.full((R, (n_max + 7) // 8), float("nan"), device="cuda")
    C.csa2_index_score(dev(q), kc, dev(np.array(lens, np.int32)), scores, row_seq=dev(row_seq),
                       head_w=dev(w) if weighted else None, block_max=bmax)
    torch.cuda.synchronize()
    g, gb = host(scores), host(bmax)
    for r in range(R):
        b = row_seq[r]
        L = lens[b]
        ref = O.index_scores(q[r], kseq[b], None if w is None else w[r])
        assert np.array_equal(g[r, :L].view(np.uint32), ref.view(np.uint32)), r
        assert np.all(np.isnan(g[r, L:]))
        nb = (L + 7) // 8
        assert np.array_equal(gb[r, :nb].view(np.uint32), O.block_max(ref, L).view(np.uint32)), r


def test_index_score_candidates_bitexact(C):
    rng = np.random.default_rng(303)
    lens = [20000, 3000, 100]
    B = len(lens)
    n_max = max(lens)
    kseq = [bf16(rng, (L, 64)) for L in lens]
    kslots = place(kseq, lens, B * n_max, None, n_max, 64, np.uint16)
    n_cand = 2048
    cand = np.full((B, n_cand), -1, np.int32)
    for b, L in enumerate(lens):
        nb = (L + 7) // 8
        pick = np.sort(rng.choice(nb, size=min(nb, n_cand - 5), replace=False))
        cand[b, :len(pick)] = pick
    q = bf16(rng, (B, 4, 64))
    say("index_score candidates")
    kc = C.make_cache(dev(kslots), seq_stride=n_max)
    scores = torch.zeros((B, n_cand * 8), device="cuda")
    C.csa2_index_score(dev(q), kc, dev(np.array(lens, np.int32)), scores, cand_blocks=dev(cand), n_max=n_max)
    torch.cuda.synchronize()
    g = host(scores)
    for b, L in enumerate(lens):
        pos = (cand[b][:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
        ok = (np.repeat(cand[b], 8) >= 0) & (pos < L)
        ref = np.full(n_cand * 8, -np.inf, np.float32)
        ref[ok] = O.index_scores(q[b], kseq[b][pos[ok]])
        assert np.array_equal(g[b].view(np.uint32), ref.view(np.uint32)), b


# ------------------------------------------------------------------ top-k --

def _topk_case(rng, kind, n):
    if kind == "normal":
        return rng.standard_normal(n).astype(np.float32)
    if kind == "ties":
        return rng.integers(0, 5, size=n).astype(np.float32)
    if kind == "zeros":
        s = np.maximum(rng.standard_normal(n), 0).astype(np.float32)
        s[rng.random(n) < 0.3] = -0.0
        return s
    if kind == "equal":
        return np.full(n, 2.5, np.float32)
    if kind == "clustered":   # all the large values in one segment -> exactness fallback
        s = rng.standard_normal(n).astype(np.float32)
        s[:min(n, 3000)] += 100
        return s
    if kind == "copies":      # ~8 copies of each value: ties inside the bin that holds the k-th value
        pool = rng.standard_normal(max(1, n // 8)).astype(np.float32)
        return pool[rng.integers(0, len(pool), size=n)]
    if kind == "neginf":
        s = rng.standard_normal(n).astype(np.float32)
        s[rng.random(n) < 0.5] = -np.inf
        return s
    raise ValueError(kind)


@pytest.mark.parametrize("k", [1, 7, 512, 1024, 2048])
def test_topk_bitexact(C, k):
    rng = np.random.default_rng(400 + k)
    kinds = ["normal", "ties", "zeros", "equal", "clustered", "neginf", "copies"]
    ns = [0, 5, k, 4096, 4097, 9000, 70000, 131072]
    rows = [(kd, n) for kd in kinds for n in ns]
    R = len(rows)
    n_max = max(ns)
    scores = np.full((R, n_max), np.nan, np.float32)
    nv = np.zeros(R, np.int32)
    for r, (kd, n) in enumerate(rows):
        scores[r, :n] = _topk_case(rng, kd, n)
        nv[r] = n
    say("topk k", k, "R", R)
    ws = workspace(C.csa2_topk_workspace_bytes(R, n_max, k))
    out = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
    C.csa2_topk(dev(scores), k, out, ws, n_valid=dev(nv))
    torch.cuda.synchronize()
    g = host(out)
    for r, (kd, n) in enumerate(rows):
        ref = O.topk(scores[r, :n], k)
        assert np.array_equal(g[r], ref), (kd, n, k)
    # a second call on the same workspace (tickets were left at zero)
    C.csa2_topk(dev(scores), k, out, ws, n_valid=dev(nv))
    torch.cuda.synchronize()
    assert np.array_equal(host(out), g)


@pytest.mark.parametrize("k", [7, 512, 1024])
def test_topk_bitexact_long_rows(C, k):
    """Rows of 131073 .. 1048576 values (one block per row descending three
    levels of maxima), every distribution, beside a short row in the same
    launch."""
    rng = np.random.default_rng(800 + k)
    kinds = ["normal", "ties", "zeros", "equal", "clustered", "neginf", "copies"]
    ns = [131073, 1048576, 300000]
    rows = [(kd, n) for kd in kinds for n in ns] + [("normal", 5000)]
    R = len(rows)
    n_max = max(n for _, n in rows)
    scores = np.full((R, n_max), np.nan, np.float32)
    nv = np.zeros(R, np.int32)
    for r, (kd, n) in enumerate(rows):
        scores[r, :n] = _topk_case(rng, kd, n)
        nv[r] = n
    say("topk long rows k", k, "R", R)
    ws = workspace(C.csa2_topk_workspace_bytes(R, n_max, k))
    out = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
    C.csa2_topk(dev(scores), k, out, ws, n_valid=dev(nv))
    torch.cuda.synchronize()
    g = host(out)
    for r, (kd, n) in enumerate(rows):
        assert np.array_equal(g[r], O.topk(scores[r, :n], k)), (kd, n, k)


@pytest.mark.parametrize("k", [7, 512])
@pytest.mark.parametrize("mapped", [False, True])
def test_topk_bitexact_short_rows(C, k, mapped):
    """Rows of at most 16384 values (the Reindex candidates' size): the
    selection split over 1024-value segments, with and without a candidate
    block map (output position = 8 * cand_blocks[i // 8] + i % 8)."""
    rng = np.random.default_rng(700 + k + 7 * mapped)
    kinds = ["normal", "ties", "zeros", "equal", "clustered", "neginf", "copies"]
    ns = [0, 5, k, 2048, 2049, 9000, 16383, 16384]
    rows = [(kd, n) for kd in kinds for n in ns]
    R = len(rows)
    n_max = 16384
    scores = np.full((R, n_max), np.nan, np.float32)
    nv = np.zeros(R, np.int32)
    for r, (kd, n) in enumerate(rows):
        scores[r, :n] = _topk_case(rng, kd, n)
        if n < n_max:
            scores[r, n:] = -np.inf if mapped else np.nan
        nv[r] = n
    cand = None
    if mapped:
        cand = np.sort(np.stack([rng.choice(1 << 20, n_max // 8, replace=False) for _ in range(R)]), axis=1)
        cand = cand.astype(np.int32)
    say("topk short rows k", k, "mapped", mapped, "R", R)
    ws = workspace(C.csa2_topk_workspace_bytes(R, n_max, k))
    out = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
    # (a candidate map covers whole rows: every value is present or -inf)
    C.csa2_topk(dev(scores), k, out, ws, n_valid=None if mapped else dev(nv),
                cand_blocks=dev(cand) if mapped else None)
    torch.cuda.synchronize()
    g = host(out)
    for r, (kd, n) in enumerate(rows):
        ref = O.topk(scores[r] if mapped else scores[r, :n], k)
        if mapped:
            ref = np.where(ref >= 0, cand[r][np.maximum(ref, 0) // 8] * 8 + np.maximum(ref, 0) % 8, -1)
        assert np.array_equal(g[r], ref), (kd, n, k)


def test_hier_candidates_bitexact(C):
    rng = np.random.default_rng(505)
    lens = [1048576 // 4, 16384, 12345, 7]
    R = len(lens)
    n_max = max(lens)
    nb_max = (n_max + 7) // 8
    bm = np.full((R, nb_max), np.nan, np.float32)
    for r, L in enumerate(lens):
        s = rng.standard_normal(L).astype(np.float32)
        if r == 2:
            s = rng.integers(0, 3, size=L).astype(np.float32)
        bm[r, :(L + 7) // 8] = O.block_max(s, L)
    say("hier candidates R", R)
    ws = workspace(C.csa2_topk_workspace_bytes(R, nb_max, 2048))
    out = torch.full((R, 2048), -7, dtype=torch.int32, device="cuda")
    C.csa2_hier_candidates(dev(bm), dev(np.array(lens, np.int32)), n_max, 2048, out, ws)
    torch.cuda.synchronize()
    g = host(out)
    for r, L in enumerate(lens):
        assert np.array_equal(g[r], O.topk(bm[r, :(L + 7) // 8], 2048)), r


@pytest.mark.parametrize("lens", [[1048576, 1048576, 600000, 524288], [131072, 131072, 100000, 70000]])
def test_hier_candidates_long_rows(C, lens):
    """Rows of 65536 .. 131072 block maxima (512K .. 1M positions): segment
    thresholds taken on the maxima of 8 block maxima; rows of at most 16384
    block maxima (128K positions): two segments."""
    rng = np.random.default_rng(506 + len(str(lens)))
    R = len(lens)
    n_max = max(lens)
    nb_max = (n_max + 7) // 8
    bm = np.full((R, nb_max), np.nan, np.float32)
    for r, L in enumerate(lens):
        if r == 1:      # ~8 copies of each value: ties at the selection edge
            pool = rng.standard_normal(L // 8).astype(np.float32)
            s = pool[rng.integers(0, len(pool), size=L)]
        else:
            s = rng.standard_normal(L).astype(np.float32)
        bm[r, :(L + 7) // 8] = O.block_max(s, L)
    say("hier candidates long rows R", R)
    ws = workspace(C.csa2_topk_workspace_bytes(R, nb_max, 2048))
    out = torch.full((R, 2048), -7, dtype=torch.int32, device="cuda")
    C.csa2_hier_candidates(dev(bm), dev(np.array(lens, np.int32)), n_max, 2048, out, ws)
    torch.cuda.synchronize()
    g = host(out)
    for r, L in enumerate(lens):
        assert np.array_equal(g[r], O.topk(bm[r, :(L + 7) // 8], 2048)), r


# -------------------------------------------------------------- attention --

@pytest.mark.parametrize("paged", [False, True])
def test_attention_parity(C, paged):
    rng = np.random.default_rng(606 + paged)
    lens = [3000, 700, 64, 2000]
    B = len(lens)
    n_max = max(lens)
    kvp = [rand_fp4(rng, L) for L in lens]
    if paged:
        pt, n_slots = paged_layout(rng, lens)
        stride = 0
    else:
        pt, stride, n_slots = None, n_max, B * n_max
    P = place([p for p, _ in kvp], lens, n_slots, pt, stride, 256, np.uint8)
    Sc = place([s for _, s in kvp], lens, n_slots, pt, stride, 32, np.uint8)
    row_seq = np.array([0, 1, 2, 3, 0], np.int32)
    R = len(row_seq)
    k = 512
    idx = np.full((R, k), -1, np.int32)
    for r in range(R):
        L = lens[row_seq[r]]
        m = min(L, [512, 300, 64, 511, 512][r])
        idx[r, :m] = np.sort(rng.choice(L, size=m, replace=False))
    idx[3, 10] = 99999          # out of range: skipped
    idx[4, :] = -1              # no sparse entries: window only
    S = 140
    swk, swv = bf16(rng, (B, S, 512)), bf16(rng, (B, S, 512))
    st = np.array([0, 12, 0, 3, 0], np.int32)
    ln = np.array([128, 128, 0, 77, 128], np.int32)
    q = bf16(rng, (R, 16, 512))
    q[0] *= 0
    sm = 1.0 / math.sqrt(512)
    say("attention paged", paged, "R", R)
    kv = C.make_cache(dev(P), dev(Sc), page_table=dev(pt) if paged else None, seq_stride=stride)
    out = torch.full((R, 16, 512), float("nan"), device="cuda")
    lse = torch.full((R, 16), float("nan"), device="cuda")
    ws = workspace(C.csa2_attn_workspace_bytes(R))
    C.csa2_fp4_sparse_attn(dev(q), kv, dev(np.array(lens, np.int32)), dev(idx), dev(swk), dev(swv), dev(st),
                           dev(ln), sm, out, lse, ws, row_seq=dev(row_seq))
    torch.cuda.synchronize()
    g, gl = host(out), host(lse)
    cache = O.Cache(P, Sc, np.zeros((n_slots, 64), np.uint16), lens, pt, 64, stride)
    for r in range(R):
        b = row_seq[r]
        sel = idx[r][(idx[r] >= 0) & (idx[r] < lens[b])]
        ref, rl = O.attention(q[r], cache.kv_rows(b, sel), swk[b, st[r]:st[r] + ln[r]],
                              swv[b, st[r]:st[r] + ln[r]], sm)
        e = rel_err(g[r], ref)
        assert np.all(e <= ATTN_TOL), (r, e.max())
        assert lse_ok(gl[r], rl), (r, gl[r], rl)


@pytest.mark.parametrize("R", [7, 64, 96])
def test_attention_window_lengths(C, R):
    """Window lengths across the two 64-key halves of the window step (0, 1,
    40, 64, 65, 100, 128; windows ending at the buffer's last entry), one
    launch of R rows: 7 rows run one block per CU, 64 rows two blocks per CU
    (both with the window step split over two blocks), 96 rows two main steps
    per block."""
    rng = np.random.default_rng(909 + R)
    lens = [3000, 700, 2000, 1200]
    B = len(lens)
    n_max = max(lens)
    kvp = [rand_fp4(rng, L) for L in lens]
    pt, stride, n_slots = None, n_max, B * n_max
    P = place([p for p, _ in kvp], lens, n_slots, pt, stride, 256, np.uint8)
    Sc = place([s for _, s in kvp], lens, n_slots, pt, stride, 32, np.uint8)
    row_seq = (np.arange(R) % B).astype(np.int32)
    k = 512
    idx = np.full((R, k), -1, np.int32)
    for r in range(R):
        L = lens[row_seq[r]]
        m = int(rng.integers(0, min(L, k) + 1))
        idx[r, :m] = np.sort(rng.choice(L, size=m, replace=False))
    S = 140
    swk, swv = bf16(rng, (B, S, 512)), bf16(rng, (B, S, 512))
    choices = [0, 1, 40, 64, 65, 100, 128]
    ln = np.array([choices[r % len(choices)] for r in range(R)], np.int32)
    st = np.array([S - ln[r] if r % 2 else int(rng.integers(0, S - ln[r] + 1)) for r in range(R)], np.int32)
    q = bf16(rng, (R, 16, 512))
    sm = 1.0 / math.sqrt(512)
    say("attention window lengths R", R)
    kv = C.make_cache(dev(P), dev(Sc), seq_stride=stride)
    out = torch.full((R, 16, 512), float("nan"), device="cuda")
    lse = torch.full((R, 16), float("nan"), device="cuda")
    ws = workspace(C.csa2_attn_workspace_bytes(R))
    C.csa2_fp4_sparse_attn(dev(q), kv, dev(np.array(lens, np.int32)), dev(idx), dev(swk), dev(swv), dev(st),
                           dev(ln), sm, out, lse, ws, row_seq=dev(row_seq))
    torch.cuda.synchronize()
    g, gl = host(out), host(lse)
    cache = O.Cache(P, Sc, np.zeros((n_slots, 64), np.uint16), lens, pt, 64, stride)
    for r in range(R):
        b = row_seq[r]
        sel = idx[r][idx[r] >= 0]
        ref, rl = O.attention(q[r], cache.kv_rows(b, sel), swk[b, st[r]:st[r] + ln[r]],
                              swv[b, st[r]:st[r] + ln[r]], sm)
        if sel.size == 0 and ln[r] == 0:
            assert np.all(g[r] == 0) and np.all(np.isneginf(gl[r])), r
            continue
        e = rel_err(g[r], ref)
        assert np.all(e <= ATTN_TOL), (r, ln[r], e.max())
        assert lse_ok(gl[r], rl), (r, gl[r], rl)


def test_attention_empty_row_and_single_key(C):
    rng = np.random.default_rng(707)
    P, Sc = rand_fp4(rng, 10)
    Sc[:] = 0x38
    R = 2
    idx = np.full((R, 512), -1, np.int32)
    idx[1, 0] = 4
    q = bf16(rng, (R, 16, 512))
    swk = bf16(rng, (R, 128, 512))
    kv = C.make_cache(dev(P), dev(Sc), seq_stride=0)
    out = torch.full((R, 16, 512), float("nan"), device="cuda")
    lse = torch.full((R, 16), float("nan"), device="cuda")
    ws = workspace(C.csa2_attn_workspace_bytes(R))
    zero = dev(np.zeros(R, np.int32))
    C.csa2_fp4_sparse_attn(dev(q), kv, dev(np.array([10, 10], np.int32)), dev(idx), dev(swk), dev(swk),
                           zero, zero, 0.05, out, lse, ws, row_seq=dev(np.array([0, 0], np.int32)))
    torch.cuda.synchronize()
    g, gl = host(out), host(lse)
    assert np.all(g[0] == 0) and np.all(np.isneginf(gl[0]))
    v = O.dequantize_fp4(P[4:5], Sc[4:5])[0]
    assert np.array_equal(g[1], np.broadcast_to(v, (16, 512)).astype(np.float32))


def test_attention_deterministic(C):
    rng = np.random.default_rng(808)
    P, Sc = rand_fp4(rng, 4096)
    R = 3
    idx = np.sort(rng.choice(4096, size=(R, 512)), axis=1).astype(np.int32)
    q = bf16(rng, (R, 16, 512))
    swk, swv = bf16(rng, (R, 128, 512)), bf16(rng, (R, 128, 512))
    kv = C.make_cache(dev(P), dev(Sc), seq_stride=0)
    ws = workspace(C.csa2_attn_workspace_bytes(R))
    outs = []
    for _ in range(3):
        out = torch.empty((R, 16, 512), device="cuda")
        C.csa2_fp4_sparse_attn(dev(q), kv, dev(np.full(R, 4096, np.int32)), dev(idx), dev(swk), dev(swv),
                               dev(np.zeros(R, np.int32)), dev(np.full(R, 128, np.int32)), 0.04, out, None, ws,
                               row_seq=dev(np.zeros(R, np.int32)))
        outs.append(host(out))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
