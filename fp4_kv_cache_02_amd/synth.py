"""Seeded synthetic inputs for the CSA2 decode/prefill hot path.

This module draws random numbers and lays them out; it performs none of the
method's arithmetic (no quantisation, no scoring, no selection, no attention).
Both the CPU checker and the GPU path consume what it produces.

Workloads follow the shapes the pages give for DeepSeek-V4.1-Flash CSA2
layers: 16 query heads sharing one 512-d main-KV vector, a 4-head x 64-d
indexer, Top-512 selection, a 128-token sliding window, hierarchical
candidates of 2048 blocks of 8 positions, pages of 64 positions.

Random streams: ``np.random.SeedSequence(seed, spawn_key=(tensor, seq, layer))``
with a fixed seed per workload kind -- one independent stream per
(tensor, sequence, layer), so any slice can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

# model dimensions
H = 16          # query heads (MQA: all share one main-KV vector)
D = 512         # main-KV / query head dim
HI = 4          # indexer heads
DI = 64         # indexer head dim
TOPK = 512
WINDOW = 128
BLOCK = 8       # hierarchical indexer block
KEEP_BLOCKS = 2048
PAGE = 64

# tensor ids for the spawn keys
T_QIDX, T_KIDX, T_KV, T_Q, T_SWAK, T_SWAV, T_PLANT, T_LENS, T_PAGES, T_W, T_KVMAP, T_FP4RAW = range(12)

MODES = {"F": 0, "I": 1, "R": 2}   # Full, Reindex, Reuse


def rng_for(seed: int, tensor: int, seq: int = 0, layer: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tensor, seq, layer)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One synthetic workload. Decode: one query row per sequence."""
    name: str
    seed: int
    seq_lens: List[int]          # context positions (or compressed entries) per sequence
    schedule: str                # e.g. "FRRR", "IRRR", "FRRRIRRRIRRR..."
    hier: bool = False           # Full layer also builds the hierarchical candidate set
    paged: bool = False
    planted: float = 0.0         # fraction of planted high-similarity indexer keys
    prefill_rows: int = 0        # >0: one sequence, this many query rows (prefill chunk)
    prefill_pos: int = 0         # absolute position of the first chunk row (prefill)
    raw_fp4: bool = False        # main KV drawn directly as FP4 / E4M3 bytes
    kv_pool: int = 0             # >0: main-KV vectors drawn from a pool of this size
    full_blocks_only: bool = False  # Full layer stops after the candidate build
    shared_slots: bool = False   # every sequence reads the same slots (prefill rows with their own lengths)

    @property
    def B(self) -> int:
        return len(self.seq_lens)

    @property
    def R(self) -> int:
        return self.prefill_rows if self.prefill_rows else self.B

    @property
    def n_max(self) -> int:
        return max(self.seq_lens)

    @property
    def layers(self) -> int:
        return len(self.schedule)

    @property
    def slot_stride(self) -> int:
        """Contiguous caches: slot = seq * slot_stride + pos (0: shared slots)."""
        return 0 if (self.paged or self.shared_slots) else self.n_max

    def row_seq(self) -> np.ndarray:
        """Sequence of every query row: one sequence for a prefill chunk, one
        per row otherwise (rows of a chunk with their own lengths included)."""
        if self.prefill_rows and not self.shared_slots:
            return np.zeros(self.R, np.int64)
        return np.arange(self.R, dtype=np.int64)


def _loguniform_lengths(seed: int, B: int, lo: int, hi: int) -> List[int]:
    r = rng_for(seed, T_LENS)
    u = r.uniform(math.log(lo), math.log(hi), size=B)
    return [int(round(math.exp(v))) for v in u]


WORKLOADS = ("full_4k", "decode_128k", "decode_1m", "prefill", "causal_prefill", "serving")


def workload(kind: str, reduced: bool = False) -> Workload:
    """The seeded workloads, by kind (one of ``WORKLOADS``).  ``reduced`` keeps
    the structure at test-friendly sizes."""
    if kind == "full_4k":
        return Workload("full_b1_L4096", 1000, [4096], "F")
    if kind == "decode_128k":
        if reduced:
            return Workload("decode_reduced_F3R_b3_L12000", 1001, [12000, 9001, 4096], "FRRR",
                            planted=0.01)
        return Workload("decode_F3R_b8_L131072", 1001, [131072] * 8, "FRRR", planted=0.01,
                        kv_pool=65536)
    if kind == "decode_1m":
        if reduced:
            return Workload("decode_reduced_hier_FIRRR_b1_L40000", 1002, [40000], "FIRRR", hier=True,
                            full_blocks_only=True)
        return Workload("decode_hier_FIRRR_b1_L1048576", 1002, [1048576], "FIRRR", hier=True,
                        full_blocks_only=True, kv_pool=65536)
    if kind == "prefill":
        if reduced:
            return Workload("prefill_reduced_F5R_C64_E8192", 1003, [8192], "FRRRRR",
                            prefill_rows=64, prefill_pos=16384, raw_fp4=True)
        return Workload("prefill_F5R_C4096_E131072", 1003, [131072], "FRRRRR",
                        prefill_rows=4096, prefill_pos=262144, raw_fp4=True)
    if kind == "causal_prefill":
        # the prefill chunk with its own compressed entries (ratio 2: entry j
        # of the chunk covers its tokens 2j, 2j+1): row i sees the E prior
        # entries and the chunk entries completed by its token,
        # j < floor((i + 1) / 2) -- a completion mask over one shared cache
        C, E = (64, 8192) if reduced else (4096, 131072)
        lens = [E + (i + 1) // 2 for i in range(C)]
        name = f"causal_prefill_F5R_C{C}_E{E}+{C // 2}" + ("_reduced" if reduced else "")
        return Workload(name, 1106, lens, "FRRRRR", prefill_rows=C, prefill_pos=2 * E, raw_fp4=True,
                        shared_slots=True)
    if kind == "serving":
        if reduced:
            lens = _loguniform_lengths(1004, 5, 2048, 40000)
            return Workload("serving_reduced_20L_b5_paged", 1004, lens, "FRRR" + "IRRR" * 4,
                            hier=True, paged=True)
        lens = _loguniform_lengths(1004, 32, 32768, 1048576)
        return Workload("serving_20L_b32_loguniform_paged", 1004, lens, "FRRR" + "IRRR" * 4,
                        hier=True, paged=True, kv_pool=65536)
    raise ValueError(f"unknown workload kind {kind!r}; expected one of {WORKLOADS}")


def model_step(reduced: bool = False) -> List[Workload]:
    """The 38 CSA2 layers of one decode step as two workloads over their own
    caches: the encoder's 18 layers at compression ratio 2 (three groups of
    Full + 5 Reuse over L/2 compressed entries) and the decoder's 20 (Full +
    3 Reuse, the Full layer also building the hierarchical candidate set, then
    four groups of Reindex + 3 Reuse over L positions) -- the layer pattern of
    the 7minutos.es page, section "Atención escasa comprimida 2 (CSA2)", and
    the conexaotc.com.br page, paragraph on CSA2.  Decode batch 8 at L = 131072."""
    if reduced:
        return [Workload("model38_reduced_enc18_b2_E5000", 1005, [5000, 2048], "FRRRRR" * 3, planted=0.01),
                Workload("model38_reduced_dec20_b2_L20000", 1006, [20000, 9000], "FRRR" + "IRRR" * 4,
                         hier=True, planted=0.01)]
    return [Workload("model38_enc18_F5Rx3_b8_E65536", 1005, [65536] * 8, "FRRRRR" * 3, planted=0.01,
                     kv_pool=65536),
            Workload("model38_dec20_F3R_4xI3R_b8_L131072", 1006, [131072] * 8, "FRRR" + "IRRR" * 4,
                     hier=True, planted=0.01, kv_pool=65536)]


# --------------------------------------------------------------------------
# generators (numpy, host)
# --------------------------------------------------------------------------

def slots_layout(w: Workload):
    """Physical slot layout for the per-position caches.

    Contiguous: slot = seq * n_max + pos.  Paged: pages of 64 positions; the
    physical page ids are a seeded permutation of all pages in use.
    Returns (n_slots, page_table [B, max_pages] int32 or None, max_pages).
    """
    if w.shared_slots:
        return w.n_max, None, 0
    if not w.paged:
        return w.B * w.n_max, None, 0
    npages = [(L + PAGE - 1) // PAGE for L in w.seq_lens]
    total = sum(npages)
    perm = rng_for(w.seed, T_PAGES).permutation(total).astype(np.int32)
    max_pages = max(npages)
    table = np.full((w.B, max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(npages):
        table[b, :n] = perm[off:off + n]
        off += n
    return total * PAGE, table, max_pages


def slot_index(w: Workload, page_table, b: int, pos: np.ndarray) -> np.ndarray:
    pos = np.asarray(pos, dtype=np.int64)
    if page_table is None:
        return b * w.slot_stride + pos
    return page_table[b, pos // PAGE].astype(np.int64) * PAGE + pos % PAGE


def gen_q_idx(w: Workload, layer: int) -> np.ndarray:
    """Indexer query of one Full/Reindex layer: [R, 4, 64] bf16 bits."""
    out = np.empty((w.R, HI, DI), dtype=np.uint16)
    if w.prefill_rows:
        out[:] = f32_to_bf16_bits(rng_for(w.seed, T_QIDX, 0, layer).standard_normal(
            (w.R, HI, DI), dtype=np.float32))
        return out
    for b in range(w.B):
        out[b] = f32_to_bf16_bits(rng_for(w.seed, T_QIDX, b, layer).standard_normal(
            (HI, DI), dtype=np.float32))
    return out


def gen_k_idx_seq(w: Workload, b: int, q_idx_full: Optional[np.ndarray], L: Optional[int] = None) -> np.ndarray:
    """Indexer keys of sequence b, [L_b, 64] bf16 bits, with optional planted keys.

    Planted keys (a fraction ``w.planted`` of positions, chosen without
    replacement) are bf16(u + 0.5 z) with u = 8 * qbar / |qbar|, qbar the sum of
    the Full layer's four indexer query heads and z ~ N(0, I).
    """
    L = w.seq_lens[b] if L is None else L
    k = rng_for(w.seed, T_KIDX, b).standard_normal((L, DI), dtype=np.float32)
    if w.planted > 0:
        r = rng_for(w.seed, T_PLANT, b)
        n = int(round(w.planted * L))
        where = r.choice(L, size=n, replace=False)
        qbar = bf16_bits_to_f32(q_idx_full[b]).astype(np.float64).sum(axis=0)
        u = 8.0 * qbar / np.linalg.norm(qbar)
        z = r.standard_normal((n, DI))
        k[where] = (u[None, :] + 0.5 * z).astype(np.float32)
    return f32_to_bf16_bits(k)


def gen_q(w: Workload, layer: int) -> np.ndarray:
    """Per-layer global query: [R, 16, 512] bf16 bits."""
    if w.prefill_rows:
        return f32_to_bf16_bits(rng_for(w.seed, T_Q, 0, layer).standard_normal(
            (w.R, H, D), dtype=np.float32))
    out = np.empty((w.R, H, D), dtype=np.uint16)
    for b in range(w.B):
        out[b] = f32_to_bf16_bits(rng_for(w.seed, T_Q, b, layer).standard_normal(
            (H, D), dtype=np.float32))
    return out


def gen_swa(w: Workload, layer: int):
    """Per-layer sliding-window K and V (bf16 bits) and per-row window.

    Decode: [B, 128, 512] each; row b attends window entries [0, 128).
    Prefill: one buffer [C + 127, 512]; row i attends entries [i, i + 128),
    i.e. itself and the 127 tokens before it.
    Returns (swa_k, swa_v, S, start[R], length[R]).
    """
    if w.prefill_rows:
        S = w.prefill_rows + WINDOW - 1
        k = f32_to_bf16_bits(rng_for(w.seed, T_SWAK, 0, layer).standard_normal((1, S, D), dtype=np.float32))
        v = f32_to_bf16_bits(rng_for(w.seed, T_SWAV, 0, layer).standard_normal((1, S, D), dtype=np.float32))
        start = np.arange(w.R, dtype=np.int32)
        length = np.full(w.R, WINDOW, dtype=np.int32)
        return k, v, S, start, length
    S = WINDOW
    k = np.empty((w.B, S, D), dtype=np.uint16)
    v = np.empty((w.B, S, D), dtype=np.uint16)
    for b in range(w.B):
        k[b] = f32_to_bf16_bits(rng_for(w.seed, T_SWAK, b, layer).standard_normal((S, D), dtype=np.float32))
        v[b] = f32_to_bf16_bits(rng_for(w.seed, T_SWAV, b, layer).standard_normal((S, D), dtype=np.float32))
    start = np.zeros(w.B, dtype=np.int32)
    length = np.array([min(WINDOW, L) for L in w.seq_lens], dtype=np.int32)
    return k, v, S, start, length


def gen_kv_values(w: Workload, b: int, pos0: int, n: int) -> np.ndarray:
    """Main-KV source values (float32 N(0,1)) for positions [pos0, pos0+n) of seq b.

    Drawn per sequence from one stream; only for workloads without a pool.
    """
    r = rng_for(w.seed, T_KV, b)
    if pos0:
        r.standard_normal((pos0, D), dtype=np.float32)  # advance deterministically
    return r.standard_normal((n, D), dtype=np.float32)


def gen_kv_pool(w: Workload) -> np.ndarray:
    """Pool of main-KV source vectors, float32 N(0,1) [P, 512]."""
    return rng_for(w.seed, T_KV, 0, 1).standard_normal((w.kv_pool, D), dtype=np.float32)


def gen_kv_pool_map(w: Workload, b: int) -> np.ndarray:
    """For pooled workloads: pool entry of every position of sequence b."""
    return rng_for(w.seed, T_KVMAP, b).integers(0, w.kv_pool, size=w.seq_lens[b], dtype=np.int64)


def gen_fp4_raw(w: Workload, n_slots: int):
    """Main KV drawn directly as bytes: nibbles uniform over 0..15, scale codes
    uniform over 0x20..0x37 (E4M3 values 0.125 .. 0.9375)."""
    r = rng_for(w.seed, T_FP4RAW)
    packed = r.integers(0, 256, size=(n_slots, D // 2), dtype=np.uint8)
    scale = r.integers(0x20, 0x38, size=(n_slots, D // 16), dtype=np.uint8)
    return packed, scale


def gen_head_w(w: Workload, layer: int) -> Optional[np.ndarray]:
    """Indexer head weights are not part of the workloads (all ones); tests draw
    their own when they exercise the weighted form."""
    return None
