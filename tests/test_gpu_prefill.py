"""Parity of the prefill-chunk indexer (every row of a Full layer scores the
same sequence; at least 256 rows over at least 65536 positions): the
matrix-core pass finds a candidate superset per row and the exact selection
must equal the oracle's Top-512 bit for bit, including rows whose scores are
tied or nearly tied (exact rescoring inside the error band) and rows with too
many candidates (exact scan fallback)."""
import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O
from tests.gpu_util import bf16, dev, host, rand_fp4, say, workspace

pytestmark = pytest.mark.gpu

FULL = 0


@pytest.fixture(scope="module")
def C():
    from fp4_kv_cache_02_amd import csa2
    return csa2


def _keys(rng, L, kind):
    k = bf16(rng, (L, 64))
    if kind == "dup":
        # a third of the positions hold one large key: rows that score it
        # highly see tens of thousands of exact ties (too many candidates)
        u = bf16(rng, (1, 64), 3.0)
        k[rng.choice(L, size=L // 3, replace=False)] = u
    elif kind == "near":
        # 3000 near-copies of a strong key (one channel one bf16 step up):
        # their scores differ by less than the matrix-core error band
        v = bf16(rng, (1, 64), 2.5)
        n = 3000
        kk = np.repeat(v, n, axis=0)
        ch = rng.integers(0, 64, n)
        bits = kk[np.arange(n), ch]
        safe = ((bits & 0x7FFF) > 0) & ((bits & 0x7FFF) < 0x7F00)
        kk[np.arange(n)[safe], ch[safe]] = bits[safe] + 1
        k[rng.choice(L, size=n, replace=False)] = kk
        # and some exact zeros
        k[rng.choice(L, size=500, replace=False)] = 0
    return k


def _run(C, R, L, n_max, kind, paged, weighted, seed, n_check=20):
    rng = np.random.default_rng(seed)
    keys = _keys(rng, L, kind)
    if paged:
        npg = (n_max + 63) // 64
        perm = rng.permutation(npg).astype(np.int32)
        pt = perm[None, :].copy()
        n_slots = npg * 64
        kslots = np.zeros((n_slots, 64), np.uint16)
        pos = np.arange(L)
        kslots[perm[pos // 64].astype(np.int64) * 64 + pos % 64] = keys
        stride = 0
    else:
        pt = None
        n_slots = n_max
        kslots = np.zeros((n_slots, 64), np.uint16)
        kslots[:L] = keys
        stride = n_max
    q_idx = bf16(rng, (R, 4, 64))
    q_idx[3] = 0                                   # a row whose scores are all zero
    w = rng.uniform(-0.5, 2.0, size=(R, 4)).astype(np.float32) if weighted else None
    P, S = rand_fp4(rng, n_slots)
    q = bf16(rng, (R, 16, 512))
    Sw = R + 127
    swk, swv = bf16(rng, (1, Sw, 512)), bf16(rng, (1, Sw, 512))
    say("prefill indexer", kind, "paged", paged, "weighted", weighted, "R", R, "L", L, "n_max", n_max)

    kv = C.make_cache(dev(P), dev(S), page_table=dev(pt) if paged else None, seq_stride=stride)
    kc = C.make_cache(dev(kslots), page_table=dev(pt) if paged else None, seq_stride=stride)
    seq_len = dev(np.array([L], np.int32))
    topk = torch.full((R, 512), -7, dtype=torch.int32, device="cuda")
    sh = C.make_shared(kv, kc, seq_len, n_max, topk)
    out = torch.zeros((R, 16, 512), device="cuda")
    args = C.make_layer_args(dev(q), dev(swk), dev(swv), dev(np.arange(R, dtype=np.int32)),
                             dev(np.full(R, 128, np.int32)), 512 ** -0.5, out, q_idx=dev(q_idx),
                             head_w=dev(w) if weighted else None, row_seq=dev(np.zeros(R, np.int32)))
    ws = workspace(C.csa2_workspace_bytes(FULL, R, n_max, False))
    C.csa2_layer_step(FULL, args, sh, ws)
    torch.cuda.synchronize()
    g = host(topk)
    rows = sorted(set([0, 3, R - 1] + list(rng.choice(R, size=n_check, replace=False))))
    for r in rows:
        ref = O.topk(O.index_scores_chunked(q_idx[r], keys, None if w is None else w[r]), 512)
        assert np.array_equal(g[r], ref), (kind, r, np.setdiff1d(g[r], ref)[:8], np.setdiff1d(ref, g[r])[:8])
    assert np.all(np.isfinite(host(out)))


def test_prefill_indexer_random(C):
    _run(C, R=320, L=100000, n_max=104000, kind="random", paged=False, weighted=False, seed=501)


def test_prefill_indexer_weighted_paged(C):
    _run(C, R=256, L=131072, n_max=131072, kind="random", paged=True, weighted=True, seed=502)


def test_prefill_indexer_near_ties(C):
    _run(C, R=256, L=70001, n_max=70001, kind="near", paged=False, weighted=False, seed=503)


def test_prefill_indexer_duplicates_fallback(C):
    _run(C, R=288, L=90000, n_max=90000, kind="dup", paged=False, weighted=True, seed=504, n_check=24)


def test_prefill_indexer_causal_rows(C):
    """Rows with their own visible lengths (row i sees L0 + floor((i + 1) / 2)
    positions of one shared cache: each row a sequence of its own with
    seq_stride 0) on the matrix-core indexer."""
    rng = np.random.default_rng(505)
    R, L0 = 288, 66000
    lens = [L0 + (i + 1) // 2 for i in range(R)]
    n_max = max(lens)
    keys = _keys(rng, n_max, "random")
    q_idx = bf16(rng, (R, 4, 64))
    P, S = rand_fp4(rng, n_max)
    q = bf16(rng, (R, 16, 512))
    Sw = R + 127
    swk, swv = bf16(rng, (1, Sw, 512)), bf16(rng, (1, Sw, 512))
    say("prefill indexer, causal rows R", R, "L0", L0, "n_max", n_max)
    kv = C.make_cache(dev(P), dev(S), seq_stride=0)
    kc = C.make_cache(dev(keys), seq_stride=0)
    seq_len = dev(np.array(lens, np.int32))
    topk = torch.full((R, 512), -7, dtype=torch.int32, device="cuda")
    sh = C.make_shared(kv, kc, seq_len, n_max, topk)
    out = torch.zeros((R, 16, 512), device="cuda")
    args = C.make_layer_args(dev(q), dev(swk), dev(swv), dev(np.arange(R, dtype=np.int32)),
                             dev(np.full(R, 128, np.int32)), 512 ** -0.5, out, q_idx=dev(q_idx),
                             row_seq=dev(np.arange(R, dtype=np.int32)), swa_shared=True)
    ws = workspace(C.csa2_workspace_bytes(FULL, R, n_max, False))
    C.csa2_layer_step(FULL, args, sh, ws)
    torch.cuda.synchronize()
    g = host(topk)
    rows = sorted(set([0, 1, 2, R - 2, R - 1] + list(rng.choice(R, size=20, replace=False))))
    for r in rows:
        ref = O.topk(O.index_scores_chunked(q_idx[r], keys[:lens[r]]), 512)
        assert np.array_equal(g[r], ref), (r, np.setdiff1d(g[r], ref)[:8], np.setdiff1d(ref, g[r])[:8])
    assert np.all(np.isfinite(host(out)))


def test_prefill_indexer_short_and_ragged_rows(C):
    """Rows of their own lengths in one chunk: empty rows, rows of a few
    positions, rows below 512 groups of 64 (no threshold: every visible
    position is a candidate, within the 4096 the selection holds), rows past
    that (the exact-scan fallback) and rows ending on and beside group
    boundaries, among long rows."""
    rng = np.random.default_rng(506)
    R = 256
    special = [0, 1, 7, 63, 64, 65, 511, 513, 2047, 4000, 4096, 4097, 20000, 32767, 32768, 32769, 65535, 65536]
    lens = special + list(rng.integers(60000, 70001, size=R - len(special)))
    n_max = 70001
    lens[-1] = n_max
    keys = _keys(rng, n_max, "random")
    q_idx = bf16(rng, (R, 4, 64))
    P, S = rand_fp4(rng, n_max)
    q = bf16(rng, (R, 16, 512))
    Sw = R + 127
    swk, swv = bf16(rng, (1, Sw, 512)), bf16(rng, (1, Sw, 512))
    say("prefill indexer, short and ragged rows R", R, "n_max", n_max)
    kv = C.make_cache(dev(P), dev(S), seq_stride=0)
    kc = C.make_cache(dev(keys), seq_stride=0)
    seq_len = dev(np.array(lens, np.int32))
    topk = torch.full((R, 512), -7, dtype=torch.int32, device="cuda")
    sh = C.make_shared(kv, kc, seq_len, n_max, topk)
    out = torch.zeros((R, 16, 512), device="cuda")
    args = C.make_layer_args(dev(q), dev(swk), dev(swv), dev(np.arange(R, dtype=np.int32)),
                             dev(np.full(R, 128, np.int32)), 512 ** -0.5, out, q_idx=dev(q_idx),
                             row_seq=dev(np.arange(R, dtype=np.int32)), swa_shared=True)
    ws = workspace(C.csa2_workspace_bytes(FULL, R, n_max, False))
    C.csa2_layer_step(FULL, args, sh, ws)
    torch.cuda.synchronize()
    g = host(topk)
    rows = list(range(len(special))) + sorted(set([R - 1] + list(rng.choice(np.arange(len(special), R), size=8,
                                                                              replace=False))))
    for r in rows:
        ref = O.topk(O.index_scores_chunked(q_idx[r], keys[:lens[r]]), 512)
        assert np.array_equal(g[r], ref), (r, lens[r], np.setdiff1d(g[r], ref)[:8], np.setdiff1d(ref, g[r])[:8])
    assert np.all(np.isfinite(host(out)))


def test_prefill_indexer_max_positions(C):
    """The largest chunk the matrix-core indexer takes: 262144 positions per
    row (its stored bf16 scores, positions and group indices at their limits)."""
    _run(C, R=256, L=262144, n_max=262144, kind="random", paged=False, weighted=True, seed=507, n_check=8)
