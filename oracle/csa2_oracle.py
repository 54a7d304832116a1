"""Plain CPU oracle for the CSA2 (Compressed Sparse Attention 2) hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the GPU library.

What it computes, and where the pages say so (DeepSeek-V4.1-Flash coverage):

* FP4 main KV -- E2M1 values with one E4M3 scale per 16 channels, the NVFP4
  pattern without its global scale: page "DeepSeek lança V4.1-Flash com
  contexto de um milhão de tokens..." (conexaotc.com.br), paragraph on the KV
  quantisation; page "DeepSeek V4.1-Flash abre pesos e corta o cache KV em 4
  vezes" (plugged.ninja), bullet "Cache KV principal em FP4"; page
  "DeepSeek AI lanzó DeepSeek-V4.1-Flash..." (7minutos.es), section "FP4 KV,
  repetición limitada y otras extensiones".
* The three static layer modes (Full computes its own main KV and indexer K
  and selects new Top-512 indices; Reindex re-scores the shared indexer K of
  the last Full layer with its own indexer Q; Reuse re-uses the main KV and the
  most recent Top-K and runs no indexer); the decoder's hierarchical indexer
  (candidate set of up to 16 384 positions, 2 048 blocks of 8, built by the
  Full layer): conexaotc page, paragraph on CSA2; 7minutos page, section
  "Atención escasa comprimida 2 (CSA2)"; e-cogni summary of the preprint
  "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression", section
  "Como funciona".
* Every layer keeps its own global Q and its own sliding-window KV, and
  combines global (sparse) attention with a 128-token SWA: e-cogni summary,
  sections "Como funciona" and "O que os autores propõem"; conexaotc page,
  paragraph on the Causal Encoder-Decoder (window of 128 tokens).

The pages leave open how the indexer heads are combined, the rounding order of
the score, the Top-K tie rule and output order, how a block is scored for the
hierarchical indexer, and how the sparse and window branches are combined.
The readings taken here:

* score = sum_h w_h * ReLU(q_h . k) over the 4 indexer heads (w defaults to 1)
  with a fixed fp32 evaluation order (``index_scores``);
* Top-K orders by (score descending, position ascending) and returns the kept
  positions in ascending order, padded with -1;
* a block's score is the maximum of its positions' Full-layer scores;
* one softmax over the union of the Top-K entries and the window entries, the
  512-d main-KV vector serving as both key and value; scale 1/sqrt(512).

Floating point: attention in float64 from exactly converted inputs.  Where a
floating-point value decides an integer (the FP4/E4M3 codes, the Top-K order)
the decision is taken in float32, the precision of the GPU kernels.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# bf16 inputs
# ---------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# O1 / O2: the two element formats
# ---------------------------------------------------------------------------

E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_value(code) -> np.ndarray:
    """Decode 4-bit E2M1 codes: bit 3 sign, bits 2..1 exponent (bias 1),
    bit 0 mantissa.  Exponent 0 is subnormal: 0 or 0.5."""
    c = np.asarray(code, dtype=np.int64) & 0xF
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(c & 8, -mag, mag).astype(np.float64)


def e4m3_value(code) -> np.ndarray:
    """Decode OCP E4M3FN bytes: bit 7 sign, bits 6..3 exponent (bias 7),
    bits 2..0 mantissa; exponent 0 is subnormal (m/8 * 2^-6); no infinities;
    0x7F and 0xFF are NaN."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where(c & 0x80, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, val).astype(np.float64)


_E4M3_POS = e4m3_value(np.arange(0x7F))          # codes 0x00..0x7E, ascending, 0 .. 448
_E2M1_POS = np.array(E2M1_MAGNITUDES)             # codes 0..7


def _round_to_table(a: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the nearest table entry to each a >= 0 (table ascending,
    index parity == code parity); ties go to the even index; values above the
    table's last entry saturate to it."""
    a = np.asarray(a, dtype=np.float64)
    hi = np.clip(np.searchsorted(table, a, side="left"), 1, len(table) - 1)
    lo = hi - 1
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(a >= table[-1], len(table) - 1, idx)
    return idx.astype(np.int64)


def e4m3_encode(a) -> np.ndarray:
    """Round non-negative float32 values to E4M3FN codes: nearest, ties to even,
    saturating at 448 (code 0x7E)."""
    a = np.asarray(a, dtype=np.float32)
    if np.any(a < 0) or not np.all(np.isfinite(a)):
        raise ValueError("e4m3_encode expects finite non-negative values")
    return _round_to_table(a, _E4M3_POS).astype(np.uint8)


def e2m1_encode(y) -> np.ndarray:
    """Round float32 values to E2M1 codes: nearest magnitude, ties to the even
    code, saturating at 6; the sign bit of y is kept (so -0 gives code 8)."""
    y = np.asarray(y, dtype=np.float32)
    mag = _round_to_table(np.abs(y), _E2M1_POS)
    return (mag | np.where(np.signbit(y), 8, 0)).astype(np.uint8)


# ---------------------------------------------------------------------------
# O3: quantising main-KV vectors (the write side of the cache)
# ---------------------------------------------------------------------------


def quantize_fp4(x) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise float32 vectors [N, 512] to (packed [N, 256] u8, scale [N, 32] u8).

    Per 16-channel block j: amax = max |x|; scale code = E4M3(amax / 6), the
    division in float32; the element codes are E2M1(x / decoded scale), the
    division in float32; a block whose decoded scale is 0 gets all codes 0.
    Channel 2i goes to the low nibble of byte i, channel 2i+1 to the high
    nibble; byte j of the scale row covers channels 16j .. 16j+15.  There is no
    per-tensor (global) scale.
    """
    x = np.asarray(x, dtype=np.float32)
    N, Dm = x.shape
    if Dm % 16:
        raise ValueError("dim must be a multiple of 16")
    blocks = x.reshape(N, Dm // 16, 16)
    amax = np.max(np.abs(blocks), axis=2)
    scale_code = e4m3_encode(amax / np.float32(6.0))
    s = e4m3_value(scale_code).astype(np.float32)
    safe = np.where(s == 0, np.float32(1.0), s)
    codes = e2m1_encode(blocks / safe[:, :, None])
    codes = np.where((s == 0)[:, :, None], np.uint8(0), codes).reshape(N, Dm)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale_code.astype(np.uint8)


def quantize_fp8_keys(k_bits) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise bf16 indexer keys [N, 64] to FP8 entries: (codes [N, 64] u8
    OCP E4M3FN, scale [N] float32) -- the 68-B entry of index_scores_fp8.

    The pages give only the entry size (890 B per token, conexaotc.com.br
    page, opening paragraph); the reading taken here: one scale per position,
    s = float32(amax / 448) with amax = max |k| (so the largest element maps
    to the largest E4M3 value), codes = E4M3(|k| / s) rounded to nearest-even
    (the division in float32), saturating at 448, with the sign of k; a key
    whose s is 0 gets s = 0 and all codes 0.
    """
    k = bf16_to_f64(k_bits).astype(np.float32)
    amax = np.max(np.abs(k), axis=1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(s == 0, np.float32(1.0), s)
    y = (np.abs(k) / safe[:, None]).astype(np.float32)
    codes = e4m3_encode(y) | np.where(np.signbit(k), 0x80, 0).astype(np.uint8)
    codes = np.where((s == 0)[:, None], np.uint8(0), codes).astype(np.uint8)
    return codes, s


def dequantize_fp4(packed, scale) -> np.ndarray:
    """Decode (packed [N, 256], scale [N, 32]) to float64 [N, 512] exactly."""
    packed = np.asarray(packed, dtype=np.uint8)
    scale = np.asarray(scale, dtype=np.uint8)
    N = packed.shape[0]
    codes = np.empty((N, packed.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    s = np.repeat(e4m3_value(scale), 16, axis=1)
    return e2m1_value(codes) * s


# ---------------------------------------------------------------------------
# O4: the indexer score
# ---------------------------------------------------------------------------


def _fma32(c: np.ndarray, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """float32(c + a*b) with the product exact and one rounding.

    a, b are bf16 values, so a*b (at most 16 significant bits) and c + a*b are
    formed exactly in float64 whenever the result can round differently from
    the exact sum; the single conversion to float32 is then the one rounding.
    """
    return (c.astype(np.float64) + a * b).astype(np.float32)


def _head_dots(q_bits, k_vals) -> np.ndarray:
    """The four heads' dot products d_h, float32 [N, 4], in the fixed order:
    eight partial sums c_j over channels 8j .. 8j+7, each accumulated from +0
    in channel order with one fused multiply-add per channel, then
    ((c0+c1)+(c2+c3)) + ((c4+c5)+(c6+c7)).  k_vals: [N, 64] float64 holding
    values exactly representable in bf16."""
    q = bf16_to_f64(q_bits).reshape(4, 8, 8)           # [head, chunk, lane]
    N = k_vals.shape[0]
    k = np.asarray(k_vals, dtype=np.float64).reshape(N, 1, 8, 8)   # [pos, -, chunk, lane]
    c = np.zeros((N, 4, 8), dtype=np.float32)
    for i in range(8):
        c = _fma32(c, q[None, :, :, i], k[:, :, :, i])
    return ((c[..., 0] + c[..., 1]) + (c[..., 2] + c[..., 3])) + \
        ((c[..., 4] + c[..., 5]) + (c[..., 6] + c[..., 7]))


def _head_sum(d, w) -> np.ndarray:
    """(w0*r0 + w1*r1) + (w2*r2 + w3*r3), r_h = ReLU(d_h), every product and
    sum rounded to float32."""
    r = np.where(d > 0, d, np.float32(0.0)).astype(np.float32)
    if w is None:
        w = np.ones(4, dtype=np.float32)
    w = np.asarray(w, dtype=np.float32)
    p = (r * w[None, :]).astype(np.float32)
    return ((p[:, 0] + p[:, 1]) + (p[:, 2] + p[:, 3])).astype(np.float32)


def index_scores(q_bits, k_bits, w=None) -> np.ndarray:
    """Indexer scores of N keys for one query: float32 [N].

    q_bits: [4, 64] bf16 bits (the layer's own indexer query, 4 heads);
    k_bits: [N, 64] bf16 bits (the shared indexer keys); w: optional float32 [4]
    head weights (default 1).

    score = (w0*r0 + w1*r1) + (w2*r2 + w3*r3), r_h = ReLU(d_h), and the dot
    product d_h is evaluated as eight partial sums c_j over channels
    8j .. 8j+7, each accumulated from +0 in channel order with one fused
    multiply-add per channel, then combined as
    ((c0+c1)+(c2+c3)) + ((c4+c5)+(c6+c7)).  Every operation rounds to float32;
    each w_h*r_h product is rounded on its own.
    """
    return _head_sum(_head_dots(q_bits, bf16_to_f64(k_bits)), w)


def index_scores_fp8(q_bits, k_codes, k_scale, w=None) -> np.ndarray:
    """Indexer scores against FP8 indexer keys: float32 [N].

    The variant in which an indexer entry is 64 E4M3 codes and one 4-byte
    scale, 68 B per position -- the entry size under which the pages' global
    KV cache of 890 B per token adds up with the 288-B FP4 main-KV entry
    (890 = 2.5 x (288 + 68); the figure: conexaotc.com.br page, opening
    paragraph; 7minutos.es page, opening section).  The pages give no
    formula; the reading taken here: the entry's value is the decoded
    E4M3 vector times its scale, and the scale multiplies each head's dot
    product, d'_h = float32(s * d_h), with d_h evaluated over the exact E4M3
    values in the order of index_scores; then ReLU and the head sum as there.

    k_codes: [N, 64] OCP E4M3FN bytes (no NaN codes); k_scale: [N] float32,
    finite and >= 0.
    """
    d = _head_dots(q_bits, e4m3_value(k_codes))
    sc = np.asarray(k_scale, dtype=np.float32).astype(np.float64)
    d = (d.astype(np.float64) * sc[:, None]).astype(np.float32)     # exact product, one rounding
    return _head_sum(d, w)


def index_scores_chunked(q_bits, k_bits, w=None, chunk: int = 1 << 16) -> np.ndarray:
    out = np.empty(k_bits.shape[0], dtype=np.float32)
    for s in range(0, k_bits.shape[0], chunk):
        out[s:s + chunk] = index_scores(q_bits, k_bits[s:s + chunk], w)
    return out


def index_scores_fp8_chunked(q_bits, k_codes, k_scale, w=None, chunk: int = 1 << 16) -> np.ndarray:
    out = np.empty(k_codes.shape[0], dtype=np.float32)
    for s in range(0, k_codes.shape[0], chunk):
        out[s:s + chunk] = index_scores_fp8(q_bits, k_codes[s:s + chunk], k_scale[s:s + chunk], w)
    return out


# ---------------------------------------------------------------------------
# O5: Top-K
# ---------------------------------------------------------------------------


def order_key(scores) -> np.ndarray:
    """Order-preserving uint32 key of float32 scores (-0 sorts below +0)."""
    u = np.asarray(scores, dtype=np.float32).view(np.uint32)
    return np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)


def topk(scores, k: int, ignore_neg_inf: bool = True) -> np.ndarray:
    """Top-k of float32 scores [n] -> int32 [k].

    Keeps the first min(k, n_present) entries in the order (score descending,
    index ascending), where an entry equal to -inf counts as absent; returns
    their indices in ascending order, padded with -1.
    """
    s = np.asarray(scores, dtype=np.float32)
    idx = np.arange(s.shape[0], dtype=np.int64)
    if ignore_neg_inf:
        keep = ~(s == -np.inf)
        s, idx = s[keep], idx[keep]
    key = order_key(s).astype(np.int64)
    order = np.lexsort((idx, -key))
    chosen = np.sort(idx[order[:k]])
    out = np.full(k, -1, dtype=np.int32)
    out[:chosen.shape[0]] = chosen
    return out


# ---------------------------------------------------------------------------
# O6 / O7: hierarchical candidates and Reindex
# ---------------------------------------------------------------------------


def block_max(scores, L: int, block: int = 8) -> np.ndarray:
    """Score of each block of `block` positions: the maximum (in the Top-K
    order) of the scores of its positions below L."""
    s = np.asarray(scores, dtype=np.float32)[:L]
    nb = (L + block - 1) // block
    pad = np.full(nb * block, -np.inf, dtype=np.float32)
    pad[:L] = s
    key = order_key(pad).reshape(nb, block)
    best = np.argmax(key, axis=1)
    return pad.reshape(nb, block)[np.arange(nb), best]


def hier_candidates(scores, L: int, keep: int = 2048, block: int = 8) -> np.ndarray:
    """Candidate blocks built by the Full layer: the `keep` best blocks by
    (block score descending, block index ascending), ascending ids, -1 pad."""
    return topk(block_max(scores, L, block), keep)


def candidate_positions(cand_blocks, L: int, block: int = 8) -> np.ndarray:
    """Positions covered by the candidate blocks (ascending), below L."""
    cb = np.asarray(cand_blocks, dtype=np.int64)
    cb = cb[cb >= 0]
    pos = (cb[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return pos[pos < L]


def reindex_topk(q_bits, k_bits_seq, cand_blocks, L: int, k: int = 512, w=None,
                 block: int = 8) -> np.ndarray:
    """Reindex layer: re-score the candidate positions with the layer's own
    indexer query against the shared indexer keys, then Top-k over them with
    ties to the lower position.  Without candidates every position is scored."""
    return reindex_topk_from(lambda pos: index_scores_chunked(q_bits, k_bits_seq[pos], w), cand_blocks, L, k,
                             block)


def reindex_topk_from(score_fn, cand_blocks, L: int, k: int = 512, block: int = 8) -> np.ndarray:
    """reindex_topk with the scores of given positions from score_fn(pos)."""
    if cand_blocks is None:
        return topk(score_fn(np.arange(L)), k)
    pos = candidate_positions(cand_blocks, L, block)
    sel = topk(score_fn(pos), k)
    out = np.full(k, -1, dtype=np.int32)
    n = int(np.sum(sel >= 0))
    out[:n] = pos[sel[:n]]
    return out


# ---------------------------------------------------------------------------
# O8: attention over the selected main-KV entries and the window
# ---------------------------------------------------------------------------


def attention(q_bits, kv_sel, swa_k_bits, swa_v_bits, sm_scale: float):
    """One query row: q [16, 512] bf16 bits; kv_sel [n, 512] float64 (the
    dequantised selected main-KV vectors, each serving as key and value);
    swa_k/swa_v [w, 512] bf16 bits (the window).  One softmax per head over all
    n + w entries with logits sm_scale * (q_h . key).

    Returns (out [16, 512] float64, lse [16] float64); with no entries at all
    the output is 0 and the lse is -inf.
    """
    q = bf16_to_f64(q_bits)
    keys = [np.asarray(kv_sel, dtype=np.float64).reshape(-1, q.shape[1])]
    vals = [keys[0]]
    if swa_k_bits is not None and len(swa_k_bits):
        keys.append(bf16_to_f64(swa_k_bits))
        vals.append(bf16_to_f64(swa_v_bits))
    K = np.concatenate(keys, axis=0)
    V = np.concatenate(vals, axis=0)
    if K.shape[0] == 0:
        return np.zeros_like(q), np.full(q.shape[0], -np.inf)
    z = float(sm_scale) * (q @ K.T)                     # [16, n+w]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ V) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def merge_partials(outs, lses):
    """Combine attention results over disjoint entry sets into the result over
    their union (weights exp(lse_i - lse))."""
    lses = np.stack(lses)                                # [p, 16]
    m = np.max(lses, axis=0)
    wts = np.exp(lses - m)
    tot = wts.sum(axis=0)
    out = sum(wts[i][:, None] * outs[i] for i in range(len(outs))) / tot[:, None]
    return out, m + np.log(tot)


# ---------------------------------------------------------------------------
# O10: paged addressing
# ---------------------------------------------------------------------------


def slot_of(b: int, pos, page_table=None, page_size: int = 64, seq_stride: int = 0) -> np.ndarray:
    """Physical slot of logical position `pos` of sequence b: through the page
    table (page_table[b][pos // page_size] * page_size + pos % page_size) or,
    without one, b * seq_stride + pos.  The main KV and the indexer keys share
    the same slots."""
    pos = np.asarray(pos, dtype=np.int64)
    if page_table is None:
        return b * seq_stride + pos
    pt = np.asarray(page_table)
    return pt[b, pos // page_size].astype(np.int64) * page_size + pos % page_size


# ---------------------------------------------------------------------------
# O9: one layer step in each mode
# ---------------------------------------------------------------------------

FULL, REINDEX, REUSE = 0, 1, 2


class Cache:
    """Per-slot caches shared by a layer group: FP4 main KV and the indexer K
    (bf16, or FP8: E4M3 codes with a float32 scale per slot when k_idx_scale
    is given), with the slot mapping of every sequence."""

    def __init__(self, kv_packed, kv_scale, k_idx_bits, seq_lens, page_table=None,
                 page_size: int = 64, seq_stride: int = 0, k_idx_scale=None):
        self.kv_packed = kv_packed
        self.kv_scale = kv_scale
        self.k_idx = k_idx_bits
        self.k_idx_scale = k_idx_scale
        self.seq_lens = list(seq_lens)
        self.page_table = page_table
        self.page_size = page_size
        self.seq_stride = seq_stride

    def scores(self, q_bits, b: int, pos, w=None) -> np.ndarray:
        """Indexer scores of positions `pos` of sequence b (O4)."""
        s = self.slots(b, np.asarray(pos, dtype=np.int64))
        if self.k_idx_scale is None:
            return index_scores_chunked(q_bits, self.k_idx[s], w)
        return index_scores_fp8_chunked(q_bits, self.k_idx[s], self.k_idx_scale[s], w)

    def slots(self, b: int, pos) -> np.ndarray:
        return slot_of(b, pos, self.page_table, self.page_size, self.seq_stride)

    def k_idx_seq(self, b: int, L: Optional[int] = None) -> np.ndarray:
        L = self.seq_lens[b] if L is None else L
        return self.k_idx[self.slots(b, np.arange(L))]

    def kv_rows(self, b: int, pos) -> np.ndarray:
        pos = np.asarray(pos, dtype=np.int64)
        pos = pos[pos >= 0]
        s = self.slots(b, pos)
        return dequantize_fp4(self.kv_packed[s], self.kv_scale[s])


class GroupState:
    """What a layer hands to the next one: the most recent Top-K per row and
    the hierarchical candidate blocks per row."""

    def __init__(self, R: int):
        self.topk = [None] * R
        self.cand = [None] * R


def layer_step(mode: int, cache: Cache, state: GroupState, row_seq, q_idx_bits, q_bits,
               swa_k, swa_v, swa_start, swa_len, sm_scale: float, hier: bool = False,
               head_w=None, k: int = 512, keep: int = 2048, blocks_only: bool = False,
               rows=None, swa_shared: bool = False):
    """One CSA2 layer over the query rows `rows` (default all).

    Full: score every visible position with the layer's indexer query, keep
    Top-k (and, with `hier`, the candidate blocks), attend.  Reindex: score the
    candidate positions with the layer's own indexer query, keep Top-k, attend.
    Reuse: attend over the most recent Top-k.  Every mode attends with the
    layer's own query and window (swa_k[b], or swa_k[0] for every row when
    `swa_shared`).  `blocks_only` stops a Full layer after the candidate
    build (no Top-k, no attention).

    Returns {row: (out, lse)} for the rows attended.
    """
    R = len(row_seq)
    rows = range(R) if rows is None else rows
    results = {}
    for r in rows:
        b = int(row_seq[r])
        L = cache.seq_lens[b]
        w = None if head_w is None else head_w[r]
        if mode == FULL:
            s = cache.scores(q_idx_bits[r], b, np.arange(L), w)
            if hier:
                state.cand[r] = hier_candidates(s, L, keep)
            if blocks_only:
                continue
            state.topk[r] = topk(s, k)
        elif mode == REINDEX:
            state.topk[r] = reindex_topk_from(lambda pos: cache.scores(q_idx_bits[r], b, pos, w),
                                              state.cand[r], L, k)
        elif mode != REUSE:
            raise ValueError(mode)
        sel = state.topk[r]
        kv = cache.kv_rows(b, sel)
        st, ln = int(swa_start[r]), int(swa_len[r])
        bw = 0 if swa_shared else b
        results[r] = attention(q_bits[r], kv, swa_k[bw, st:st + ln], swa_v[bw, st:st + ln], sm_scale)
    return results
