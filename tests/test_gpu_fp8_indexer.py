"""Parity of the FP8 indexer-key variant (64 E4M3 codes and a float32 scale
per position) against the oracle: indexer scores and block maxima bit-exact
(scan and Reindex candidate scoring, contiguous and paged, with and without
head weights), and whole layers -- the hierarchical Full layer's Top-512 and
candidate blocks, then a Reindex layer -- bit-exact, outputs within 2e-3."""
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


def fp8_keys(rng, L, kind="normal"):
    """(codes [L, 64] uint8, scales [L] float32).  normal: N(0,1) keys with a
    per-position scale amax / 448; raw: uniform codes (subnormals included,
    no NaN codes) with scales spread over 2^-12 .. 2^6 and some zeros."""
    if kind == "raw":
        c = rng.integers(0, 256, size=(L, 64)).astype(np.uint8)
        c[(c & 0x7F) == 0x7F] ^= 1
        sc = np.exp2(rng.uniform(-12, 6, size=L)).astype(np.float32)
        sc[rng.random(L) < 0.05] = 0.0
        return c, sc
    k = rng.standard_normal((L, 64))
    sc = (np.abs(k).max(axis=1) / 448.0).astype(np.float32)
    mag = np.abs(k) / np.maximum(sc, np.float32(1e-30))[:, None].astype(np.float64)
    c = O.e4m3_encode(mag.astype(np.float32)) | np.where(k < 0, 0x80, 0).astype(np.uint8)
    return c.astype(np.uint8), sc


def place_fp8(seqs, lens, n_slots, pt, stride):
    codes = place([s[0] for s in seqs], lens, n_slots, pt, stride, 64, np.uint8)
    sc = place([s[1][:, None] for s in seqs], lens, n_slots, pt, stride, 1, np.float32)[:, 0].copy()
    return codes, sc


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("weighted", [False, True])
def test_index_score_fp8_bitexact(C, paged, weighted):
    rng = np.random.default_rng(702 + paged * 2 + weighted)
    lens = [5000, 1, 777, 64, 3000]
    B = len(lens)
    n_max = max(lens) + 13
    seqs = [fp8_keys(rng, L, "raw" if b % 2 else "normal") for b, L in enumerate(lens)]
    seqs[2][0][5] = 0  # an all-zero key
    if paged:
        pt, n_slots = paged_layout(rng, lens)
        stride = 0
    else:
        pt, stride, n_slots = None, n_max, B * n_max
    codes, sc = place_fp8(seqs, lens, n_slots, pt, stride)
    row_seq = np.array([0, 1, 2, 3, 4, 0], np.int32)
    R = len(row_seq)
    q = bf16(rng, (R, 4, 64))
    q[1] = 0
    w = rng.uniform(-0.5, 2.0, size=(R, 4)).astype(np.float32) if weighted else None
    say("fp8 index_score paged", paged, "weighted", weighted, "R", R)
    kc = C.make_cache(dev(codes), scale=dev(sc), page_table=dev(pt) if paged else None, seq_stride=stride)
    scores = torch.full((R, n_max), float("nan"), device="cuda")
    bmax = torch.full((R, (n_max + 7) // 8), float("nan"), device="cuda")
    C.csa2_index_score(dev(q), kc, dev(np.array(lens, np.int32)), scores, row_seq=dev(row_seq),
                       head_w=dev(w) if weighted else None, block_max=bmax)
    torch.cuda.synchronize()
    g, gb = host(scores), host(bmax)
    for r in range(R):
        b = row_seq[r]
        L = lens[b]
        ref = O.index_scores_fp8(q[r], seqs[b][0], seqs[b][1], None if w is None else w[r])
        assert np.array_equal(g[r, :L].view(np.uint32), ref.view(np.uint32)), r
        assert np.all(np.isnan(g[r, L:]))
        nb = (L + 7) // 8
        assert np.array_equal(gb[r, :nb].view(np.uint32), O.block_max(ref, L).view(np.uint32)), r


def test_index_score_fp8_candidates_bitexact(C):
    rng = np.random.default_rng(803)
    lens = [20000, 3000, 100]
    B = len(lens)
    n_max = max(lens)
    seqs = [fp8_keys(rng, L) for L in lens]
    codes, sc = place_fp8(seqs, lens, B * n_max, None, n_max)
    n_cand = 2048
    cand = np.full((B, n_cand), -1, np.int32)
    for b, L in enumerate(lens):
        nb = (L + 7) // 8
        pick = np.sort(rng.choice(nb, size=min(nb, n_cand - 5), replace=False))
        cand[b, :len(pick)] = pick
    q = bf16(rng, (B, 4, 64))
    say("fp8 index_score candidates")
    kc = C.make_cache(dev(codes), scale=dev(sc), seq_stride=n_max)
    scores = torch.zeros((B, n_cand * 8), device="cuda")
    C.csa2_index_score(dev(q), kc, dev(np.array(lens, np.int32)), scores, cand_blocks=dev(cand), n_max=n_max)
    torch.cuda.synchronize()
    g = host(scores)
    for b, L in enumerate(lens):
        pos = (cand[b][:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
        ok = (np.repeat(cand[b], 8) >= 0) & (pos < L)
        ref = np.full(n_cand * 8, -np.inf, np.float32)
        ref[ok] = O.index_scores_fp8(q[b], seqs[b][0][pos[ok]], seqs[b][1][pos[ok]])
        assert np.array_equal(g[b].view(np.uint32), ref.view(np.uint32)), b


@pytest.mark.parametrize("paged", [False, True])
def test_fp8_layers_parity(C, paged):
    """Hierarchical Full layer (Top-512 + 2048 candidate blocks) then a Reindex
    layer over the candidates, on FP8 indexer keys."""
    rng = np.random.default_rng(904 + paged)
    lens = [20000, 7001]
    B = len(lens)
    n_max = max(lens)
    seqs = [fp8_keys(rng, L) for L in lens]
    if paged:
        pt, n_slots = paged_layout(rng, lens)
        stride = 0
    else:
        pt, stride, n_slots = None, n_max, B * n_max
    codes, sc = place_fp8(seqs, lens, n_slots, pt, stride)
    P, S = rand_fp4(rng, n_slots)
    cache = O.Cache(P, S, codes, lens, pt, 64, stride, k_idx_scale=sc)
    kv = C.make_cache(dev(P), dev(S), page_table=dev(pt) if paged else None, seq_stride=stride)
    kc = C.make_cache(dev(codes), scale=dev(sc), page_table=dev(pt) if paged else None, seq_stride=stride)
    seq_len = dev(np.array(lens, np.int32))
    topk = torch.full((B, 512), -7, dtype=torch.int32, device="cuda")
    cand = torch.full((B, 2048), -7, dtype=torch.int32, device="cuda")
    sh = C.make_shared(kv, kc, seq_len, n_max, topk, cand, hier=True)
    ws = workspace(max(C.csa2_workspace_bytes(m, B, n_max, True) for m in (0, 1)))
    state = O.GroupState(B)
    rs = np.arange(B)
    for li, mode in enumerate((O.FULL, O.REINDEX)):
        qi = bf16(rng, (B, 4, 64))
        q = bf16(rng, (B, 16, 512))
        sk, sv = bf16(rng, (B, 128, 512)), bf16(rng, (B, 128, 512))
        st, ln = np.zeros(B, np.int32), np.array([128, 77], np.int32)
        out = torch.zeros((B, 16, 512), device="cuda")
        lse = torch.zeros((B, 16), device="cuda")
        say("fp8 layers paged", paged, "layer", li, "mode", mode)
        args = C.make_layer_args(dev(q), dev(sk), dev(sv), dev(st), dev(ln), 512 ** -0.5, out, lse, q_idx=dev(qi),
                                 row_seq=dev(rs.astype(np.int32)))
        C.csa2_layer_step(mode, args, sh, ws)
        torch.cuda.synchronize()
        res = O.layer_step(mode, cache, state, rs, qi, q, sk, sv, st, ln, 512 ** -0.5, hier=True)
        gt, go, gl = host(topk), host(out), host(lse)
        for r in range(B):
            assert np.array_equal(gt[r], state.topk[r]), (li, r)
            if mode == O.FULL:
                assert np.array_equal(host(cand)[r], state.cand[r]), (li, r)
            assert np.all(rel_err(go[r], res[r][0]) <= ATTN_TOL), (li, r)
            assert lse_ok(gl[r], res[r][1]), (li, r)


@pytest.mark.parametrize("n_cand", [1, 7, 100, 2047])
def test_index_score_fp8_few_candidates(C, n_cand):
    """Reindex scoring over FP8 keys (raw codes with subnormals and zero
    scales) for candidate counts that leave the last 16-block step partly
    empty."""
    rng = np.random.default_rng(820 + n_cand)
    lens = [20000, 3000, 100, 9]
    B = len(lens)
    n_max = max(lens)
    seqs = [fp8_keys(rng, L, "raw" if b % 2 else "normal") for b, L in enumerate(lens)]
    codes, sc = place_fp8(seqs, lens, B * n_max, None, n_max)
    cand = np.full((B, n_cand), -1, np.int32)
    for b, L in enumerate(lens):
        nb = (L + 7) // 8
        m = min(nb, n_cand)
        cand[b, :m] = np.sort(rng.choice(nb, size=m, replace=False))
    q = bf16(rng, (B, 4, 64))
    say("fp8 index_score n_cand", n_cand)
    kc = C.make_cache(dev(codes), scale=dev(sc), seq_stride=n_max)
    scores = torch.full((B, n_cand * 8), float("nan"), device="cuda")
    C.csa2_index_score(dev(q), kc, dev(np.array(lens, np.int32)), scores, cand_blocks=dev(cand), n_max=n_max)
    torch.cuda.synchronize()
    g = host(scores)
    for b, L in enumerate(lens):
        pos = (cand[b][:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
        ok = (np.repeat(cand[b], 8) >= 0) & (pos < L)
        ref = np.full(n_cand * 8, -np.inf, np.float32)
        ref[ok] = O.index_scores_fp8(q[b], seqs[b][0][pos[ok]], seqs[b][1][pos[ok]])
        assert np.array_equal(g[b].view(np.uint32), ref.view(np.uint32)), b


def test_index_score_fp8_unaligned_codes(C):
    """FP8 codes whose array starts 8 bytes off a 16-byte boundary (allowed:
    8-byte alignment) take the 8-byte-load scan; scores and block maxima equal
    the oracle's as on aligned codes."""
    rng = np.random.default_rng(830)
    lens = [5000, 777]
    B = len(lens)
    n_max = max(lens) + 3
    seqs = [fp8_keys(rng, L) for L in lens]
    codes, sc = place_fp8(seqs, lens, B * n_max, None, n_max)
    raw = torch.zeros(codes.size + 8, dtype=torch.uint8, device="cuda")
    view = raw[8:].view(B * n_max, 64)
    view.copy_(dev(codes))
    assert view.data_ptr() % 16 == 8
    q = bf16(rng, (B, 4, 64))
    say("fp8 index_score unaligned codes")
    kc = C.make_cache(view, scale=dev(sc), seq_stride=n_max)
    scores = torch.full((B, n_max), float("nan"), device="cuda")
    bmax = torch.full((B, (n_max + 7) // 8), float("nan"), device="cuda")
    C.csa2_index_score(dev(q), kc, dev(np.array(lens, np.int32)), scores, block_max=bmax)
    torch.cuda.synchronize()
    g, gb = host(scores), host(bmax)
    for b, L in enumerate(lens):
        ref = O.index_scores_fp8(q[b], seqs[b][0], seqs[b][1])
        assert np.array_equal(g[b, :L].view(np.uint32), ref.view(np.uint32)), b
        assert np.array_equal(gb[b, :(L + 7) // 8].view(np.uint32), O.block_max(ref, L).view(np.uint32)), b


def test_fp8_key_quantize_bitexact(C):
    """The library's FP8 key quantiser against the oracle's: codes and scales
    bit-exact (zero and -0 keys, single-element keys, magnitudes 2^-120 ..
    2^40), contiguous and into scattered slots."""
    rng = np.random.default_rng(840)
    N = 5000
    k = rng.standard_normal((N, 64)).astype(np.float32)
    k *= np.exp2(rng.uniform(-120, 40, size=(N, 1))).astype(np.float32)
    k[0] = 0.0
    k[1] = -0.0
    k[2, :] = 0.0
    k[2, 7] = -5.5
    k[3, ::2] = -0.0
    from fp4_kv_cache_02_amd import synth
    kb = synth.f32_to_bf16_bits(k)
    ref_c, ref_s = O.quantize_fp8_keys(kb)
    say("fp8 key quantize N", N)
    codes = torch.zeros((N, 64), dtype=torch.uint8, device="cuda")
    sc = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    C.csa2_fp8_key_quantize(dev(kb), codes, sc)
    torch.cuda.synchronize()
    assert np.array_equal(host(sc).view(np.uint32), ref_s.view(np.uint32))
    assert np.array_equal(host(codes), ref_c)
    perm = rng.permutation(N + 77)[:N].astype(np.int64)
    codes2 = torch.zeros((N + 77, 64), dtype=torch.uint8, device="cuda")
    sc2 = torch.zeros((N + 77,), dtype=torch.float32, device="cuda")
    C.csa2_fp8_key_quantize(dev(kb), codes2, sc2, dst_slot=dev(perm))
    torch.cuda.synchronize()
    assert np.array_equal(host(codes2)[perm], ref_c)
    assert np.array_equal(host(sc2)[perm].view(np.uint32), ref_s.view(np.uint32))
