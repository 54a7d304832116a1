"""Helpers for the GPU parity tests: move seeded numpy inputs to the GPU and
compare against the oracle."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from fp4_kv_cache_02_amd import synth
from oracle import csa2_oracle as O

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray) -> torch.Tensor:
    """numpy -> CUDA tensor (uint16 bit patterns travel as int16)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    if x.dtype == np.uint32:
        x = x.view(np.int32)
    return torch.from_numpy(x).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def workspace(nbytes: int) -> torch.Tensor:
    from fp4_kv_cache_02_amd import csa2
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    csa2.csa2_workspace_init(ws)
    return ws


def rel_err(g: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Per (row, head): max_c |g - o| / max_c |o|  (the parity metric)."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    num = np.abs(g - o).max(axis=-1)
    den = np.abs(o).max(axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


ATTN_TOL = 2e-3


def lse_ok(g, o) -> bool:
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    both_inf = np.isneginf(g) & np.isneginf(o)
    fin = ~both_inf
    return bool(np.all(np.isfinite(g[fin])) and np.all(np.abs(g[fin] - o[fin]) <= 1e-3 + 1e-4 * np.abs(o[fin])))


def rand_fp4(rng, n, scale_lo=0x28, scale_hi=0x40):
    packed = rng.integers(0, 256, size=(n, 256), dtype=np.uint8)
    scale = rng.integers(scale_lo, scale_hi, size=(n, 32), dtype=np.uint8)
    return packed, scale


def bf16(rng, shape, scale=1.0):
    return synth.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def paged_layout(rng, lens, page=64):
    npg = [(L + page - 1) // page for L in lens]
    perm = rng.permutation(sum(npg)).astype(np.int32)
    pt = np.full((len(lens), max(npg)), -1, np.int32)
    off = 0
    for b, n in enumerate(npg):
        pt[b, :n] = perm[off:off + n]
        off += n
    return pt, sum(npg) * page


def place(per_seq, lens, n_slots, page_table, stride, width, dtype):
    """Scatter per-sequence rows into the slot array of a (paged or contiguous) cache."""
    out = np.zeros((n_slots, width), dtype)
    for b, L in enumerate(lens):
        sl = O.slot_of(b, np.arange(L), page_table, 64, stride)
        out[sl] = per_seq[b][:L]
    return out
