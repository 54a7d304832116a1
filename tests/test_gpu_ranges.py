"""Parity of the exported calls over the parameter ranges the layer modes do
not use (GPU only): sparse attention with k below 512 (index rows of stride
k, in the split-plus-merge layout of few rows and the one-block-per-row layout
of many), Reindex scoring of fewer than 2048 candidate blocks, candidate
builds that keep fewer than 2048 blocks, and queries whose heads lie far
outside fp16's range.

Bars as elsewhere: scores, indices and candidate blocks bit-exact; attention
within 2e-3 max relative error per (row, head) of the float64 oracle."""
import math

import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O
from tests.gpu_util import ATTN_TOL, bf16, dev, host, lse_ok, place, rand_fp4, rel_err, say, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def C():
    from fp4_kv_cache_02_amd import csa2
    return csa2


def _attn_case(C, rng, R, k, q=None, lens=(3000, 700, 2000, 1200)):
    lens = list(lens)
    B = len(lens)
    n_max = max(lens)
    kvp = [rand_fp4(rng, L) for L in lens]
    P = place([p for p, _ in kvp], lens, B * n_max, None, n_max, 256, np.uint8)
    Sc = place([s for _, s in kvp], lens, B * n_max, None, n_max, 32, np.uint8)
    row_seq = (np.arange(R) % B).astype(np.int32)
    idx = np.full((R, k), -1, np.int32)
    for r in range(R):
        L = lens[row_seq[r]]
        # mostly full rows, some partly padded; positions in ascending order
        m = min(L, k) if r % 3 else int(rng.integers(0, min(L, k) + 1))
        idx[r, :m] = np.sort(rng.choice(L, size=m, replace=False))
    S = 140
    swk, swv = bf16(rng, (B, S, 512)), bf16(rng, (B, S, 512))
    ln = np.array([(128, 0, 77, 1)[r % 4] for r in range(R)], np.int32)
    st = np.array([int(rng.integers(0, S - ln[r] + 1)) for r in range(R)], np.int32)
    if q is None:
        q = bf16(rng, (R, 16, 512))
    sm = 1.0 / math.sqrt(512)
    kv = C.make_cache(dev(P), dev(Sc), seq_stride=n_max)
    out = torch.full((R, 16, 512), float("nan"), device="cuda")
    lse = torch.full((R, 16), float("nan"), device="cuda")
    ws = workspace(C.csa2_attn_workspace_bytes(R))
    C.csa2_fp4_sparse_attn(dev(q), kv, dev(np.array(lens, np.int32)), dev(idx), dev(swk), dev(swv), dev(st),
                           dev(ln), sm, out, lse, ws, row_seq=dev(row_seq))
    torch.cuda.synchronize()
    g, gl = host(out), host(lse)
    cache = O.Cache(P, Sc, np.zeros((B * n_max, 64), np.uint16), lens, None, 64, n_max)
    for r in range(R):
        b = row_seq[r]
        sel = idx[r][idx[r] >= 0]
        ref, rl = O.attention(q[r], cache.kv_rows(b, sel), swk[b, st[r]:st[r] + ln[r]],
                              swv[b, st[r]:st[r] + ln[r]], sm)
        if sel.size == 0 and ln[r] == 0:
            assert np.all(g[r] == 0) and np.all(np.isneginf(gl[r])), r
            continue
        e = rel_err(g[r], ref)
        assert np.all(e <= ATTN_TOL), (r, k, e.max())
        assert lse_ok(gl[r], rl), (r, gl[r], rl)


@pytest.mark.parametrize("k", [1, 64, 128, 129, 300, 384, 511])
@pytest.mark.parametrize("R", [3, 90, 520])
def test_attention_k_below_512(C, k, R):
    """k sets the number of 128-key main steps, the blocks per row and the
    row stride of idx.  3 rows: one step per block and the window in two
    halves; 90 rows: two blocks per CU (k = 300 and 384 take more blocks per
    row than k = 512 there); 520 rows: one block per row over every step."""
    rng = np.random.default_rng(1100 + k + R)
    say("attention k", k, "R", R)
    _attn_case(C, rng, R, k)


def test_attention_query_magnitudes(C):
    """Query heads far outside fp16's range (up to 2^100) and far below it
    (2^-60), a head with a single huge element among ordinary ones, and an
    all-zero head: the main steps run the fp16 matrix cores on each head's
    query scaled by its own power of two."""
    rng = np.random.default_rng(1200)
    R = 5
    q = np.stack([bf16(rng, (16, 512)) for _ in range(R)])
    qf = O.bf16_to_f64(q)
    mags = [2.0 ** 100, 2.0 ** 40, 2.0 ** 17, 2.0 ** -20, 2.0 ** -60, 1.0, 3.0e4, 7.0e4]
    for r in range(R):
        for h in range(16):
            qf[r, h] *= mags[(r + h) % len(mags)]
    qf[1, 3] = 0.0
    qf[2, 5, 17] = 2.0 ** 90
    from fp4_kv_cache_02_amd import synth
    q = synth.f32_to_bf16_bits(qf.astype(np.float32))
    say("attention query magnitudes")
    _attn_case(C, rng, R, 512, q=q)


@pytest.mark.parametrize("n_cand", [1, 7, 100, 2047])
def test_index_score_few_candidates(C, n_cand):
    rng = np.random.default_rng(1300 + n_cand)
    lens = [20000, 3000, 100, 9]
    B = len(lens)
    n_max = max(lens)
    kseq = [bf16(rng, (L, 64)) for L in lens]
    kslots = place(kseq, lens, B * n_max, None, n_max, 64, np.uint16)
    cand = np.full((B, n_cand), -1, np.int32)
    for b, L in enumerate(lens):
        nb = (L + 7) // 8
        m = min(nb, n_cand if b % 2 == 0 else max(0, n_cand - 3))
        cand[b, :m] = np.sort(rng.choice(nb, size=m, replace=False))
    cand[0, -1] = (lens[0] + 7) // 8 + 5 if n_cand > 1 else cand[0, -1]   # a block past the row's end
    q = bf16(rng, (B, 4, 64))
    say("index_score n_cand", n_cand)
    kc = C.make_cache(dev(kslots), seq_stride=n_max)
    scores = torch.full((B, n_cand * 8), float("nan"), device="cuda")
    C.csa2_index_score(dev(q), kc, dev(np.array(lens, np.int32)), scores, cand_blocks=dev(cand), n_max=n_max)
    torch.cuda.synchronize()
    g = host(scores)
    for b, L in enumerate(lens):
        pos = (cand[b][:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
        ok = (np.repeat(cand[b], 8) >= 0) & (pos < L)
        ref = np.full(n_cand * 8, -np.inf, np.float32)
        ref[ok] = O.index_scores(q[b], kseq[b][pos[ok]])
        assert np.array_equal(g[b].view(np.uint32), ref.view(np.uint32)), b


@pytest.mark.parametrize("keep", [1, 512, 2047])
def test_hier_candidates_keep_below_2048(C, keep):
    rng = np.random.default_rng(1400 + keep)
    lens = [1048576, 131072, 16384, 12345, 4000, 7]
    R = len(lens)
    n_max = max(lens)
    nb_max = (n_max + 7) // 8
    bm = np.full((R, nb_max), np.nan, np.float32)
    for r, L in enumerate(lens):
        if r == 2:     # ties at the selection edge
            s = rng.integers(0, 3, size=L).astype(np.float32)
        else:
            s = rng.standard_normal(L).astype(np.float32)
        bm[r, :(L + 7) // 8] = O.block_max(s, L)
    say("hier candidates keep", keep)
    ws = workspace(C.csa2_topk_workspace_bytes(R, nb_max, keep))
    out = torch.full((R, keep), -7, dtype=torch.int32, device="cuda")
    C.csa2_hier_candidates(dev(bm), dev(np.array(lens, np.int32)), n_max, keep, out, ws)
    torch.cuda.synchronize()
    g = host(out)
    for r, L in enumerate(lens):
        assert np.array_equal(g[r], O.topk(bm[r, :(L + 7) // 8], keep)), (r, keep)


def test_attention_every_scale_code(C):
    """Each row attends one main key and no window, so its output is that
    key's dequantised vector times a softmax weight of exactly 1: the FP4
    values times their E4M3 scales, which the kernel converts to fp16 with the
    hardware conversion.  Eight rows cover the 254 scale codes that are
    numbers (zero, subnormals, 448, negative scales; the two NaN codes are
    left out, padded with 1.0); the outputs must equal the float64 decode
    exactly."""
    rng = np.random.default_rng(1500)
    R = 8
    L = 40
    packed = rng.integers(0, 256, size=(L, 256), dtype=np.uint8)
    scale = rng.integers(0x28, 0x40, size=(L, 32), dtype=np.uint8)
    keys = rng.choice(L, size=R, replace=False)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)] + [0x38, 0x38], np.uint8)
    for r in range(R):
        scale[keys[r]] = codes[32 * r:32 * r + 32]
    idx = keys.astype(np.int32).reshape(R, 1)
    q = bf16(rng, (R, 16, 512))
    swk, swv = bf16(rng, (1, 8, 512)), bf16(rng, (1, 8, 512))
    say("attention every scale code")
    kv = C.make_cache(dev(packed), dev(scale), seq_stride=L)
    out = torch.full((R, 16, 512), float("nan"), device="cuda")
    lse = torch.full((R, 16), float("nan"), device="cuda")
    ws = workspace(C.csa2_attn_workspace_bytes(R))
    C.csa2_fp4_sparse_attn(dev(q), kv, dev(np.array([L], np.int32)), dev(idx), dev(swk), dev(swv),
                           dev(np.zeros(R, np.int32)), dev(np.zeros(R, np.int32)), 1.0 / math.sqrt(512), out, lse, ws,
                           row_seq=dev(np.zeros(R, np.int32)))
    torch.cuda.synchronize()
    g = host(out)
    ref = O.dequantize_fp4(packed[keys], scale[keys])
    for r in range(R):
        for h in range(16):
            assert np.array_equal(g[r, h].astype(np.float64), ref[r]), (r, h)
