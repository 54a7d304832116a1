"""Run a CSA2 layer group (a static Full / Reindex / Reuse schedule) on the GPU.

Layer schedules from the pages: the decoder's 20 layers are five groups of
four, Full + 3 Reuse first, then Reindex + 3 Reuse; the encoder's 18 CSA2
layers (compression ratio 2) are three groups of Full + 5 Reuse
(conexaotc.com.br page "DeepSeek lança V4.1-Flash...", paragraph on CSA2;
7minutos.es page, section "Atención escasa comprimida 2 (CSA2)").

This module only allocates device memory and calls the library; every step
of the path runs in libcsa2.so.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

from . import csa2
from . import synth

SM_SCALE = 1.0 / math.sqrt(synth.D)


def _dev(x: np.ndarray, device="cuda") -> torch.Tensor:
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).to(device)


@dataclasses.dataclass
class LayerInputs:
    q: torch.Tensor            # [R, 16, 512] bf16 bits (int16)
    swa_k: torch.Tensor        # [B, S, 512]
    swa_v: torch.Tensor
    swa_start: torch.Tensor    # [R] int32
    swa_len: torch.Tensor      # [R] int32
    q_idx: Optional[torch.Tensor] = None   # [R, 4, 64] (Full / Reindex)


@dataclasses.dataclass
class GroupInputs:
    kv_fp4: torch.Tensor       # [n_slots, 256] uint8
    kv_scale: torch.Tensor     # [n_slots, 32] uint8
    k_idx: torch.Tensor        # [n_slots, 64] bf16 bits
    seq_len: torch.Tensor      # [B] int32
    page_table: Optional[torch.Tensor]
    seq_stride: int
    row_seq: Optional[torch.Tensor]
    layers: List[LayerInputs]
    k_scale: Optional[torch.Tensor] = None   # FP8 indexer keys: [n_slots] float32 (k_idx then holds E4M3 codes)


def layer_inputs_from_synth(w: synth.Workload, device="cuda") -> List[LayerInputs]:
    out = []
    for li, m in enumerate(w.schedule):
        k, v, S, st, ln = synth.gen_swa(w, li)
        qi = _dev(synth.gen_q_idx(w, li), device) if m in "FI" else None
        out.append(LayerInputs(q=_dev(synth.gen_q(w, li), device), swa_k=_dev(k, device), swa_v=_dev(v, device),
                               swa_start=_dev(st, device), swa_len=_dev(ln, device), q_idx=qi))
    return out


def k_idx_slots_from_synth(w: synth.Workload, n_slots: int, page_table) -> np.ndarray:
    """Indexer keys of every sequence placed at their slots ([n_slots, 64] bf16 bits)."""
    q_full = synth.gen_q_idx(w, 0) if w.planted > 0 else None
    out = np.zeros((n_slots, synth.DI), np.uint16)
    if w.shared_slots:          # one set of keys that every row's sequence reads
        out[:w.n_max] = synth.gen_k_idx_seq(w, 0, q_full, L=w.n_max)
        return out
    for b in range(w.B):
        kb = synth.gen_k_idx_seq(w, b, q_full)
        out[synth.slot_index(w, page_table, b, np.arange(w.seq_lens[b]))] = kb
    return out


def kv_slots_gpu_quantized(w: synth.Workload, n_slots: int, page_table, device="cuda"):
    """Main KV for the benchmark: N(0,1) source vectors quantised on the GPU by
    the library's own quantiser (pooled workloads: the pool is quantised and
    positions take pool entries through the seeded map)."""
    fp4 = torch.zeros((n_slots, 256), dtype=torch.uint8, device=device)
    sc = torch.zeros((n_slots, 32), dtype=torch.uint8, device=device)
    if w.raw_fp4:
        p, s = synth.gen_fp4_raw(w, n_slots)
        return _dev(p, device), _dev(s, device)
    if w.kv_pool:
        pool = torch.from_numpy(synth.gen_kv_pool(w)).to(device)
        pf = torch.zeros((w.kv_pool, 256), dtype=torch.uint8, device=device)
        ps = torch.zeros((w.kv_pool, 32), dtype=torch.uint8, device=device)
        csa2.csa2_fp4_quantize(pool, pf, ps)
        for b in range(w.B):
            sl = torch.from_numpy(synth.slot_index(w, page_table, b, np.arange(w.seq_lens[b]))).to(device)
            m = torch.from_numpy(synth.gen_kv_pool_map(w, b)).to(device)
            fp4[sl] = pf[m]
            sc[sl] = ps[m]
        return fp4, sc
    for b in range(w.B):
        L = w.seq_lens[b]
        x = torch.from_numpy(synth.gen_kv_values(w, b, 0, L)).to(device)
        sl = torch.from_numpy(synth.slot_index(w, page_table, b, np.arange(L))).to(device)
        csa2.csa2_fp4_quantize(x, fp4, sc, dst_slot=sl)
    return fp4, sc


def build_inputs(w: synth.Workload, kv_fp4=None, kv_scale=None, device="cuda", k_idx=None) -> GroupInputs:
    """Device inputs of a workload.  kv_fp4/kv_scale (numpy or tensors) may be
    given; otherwise they are quantised on the GPU.  k_idx: the indexer keys at
    their slots when already generated (k_idx_slots_from_synth)."""
    n_slots, page_table, _ = synth.slots_layout(w)
    kidx = k_idx_slots_from_synth(w, n_slots, page_table) if k_idx is None else k_idx
    if kv_fp4 is None:
        kv_fp4, kv_scale = kv_slots_gpu_quantized(w, n_slots, page_table, device)
    elif isinstance(kv_fp4, np.ndarray):
        kv_fp4, kv_scale = _dev(kv_fp4, device), _dev(kv_scale, device)
    row_seq = None
    if w.prefill_rows:
        row_seq = _dev(w.row_seq().astype(np.int32), device)
    return GroupInputs(kv_fp4=kv_fp4, kv_scale=kv_scale, k_idx=_dev(kidx, device),
                       seq_len=_dev(np.array(w.seq_lens, np.int32), device),
                       page_table=_dev(page_table, device) if page_table is not None else None,
                       seq_stride=w.slot_stride, row_seq=row_seq,
                       layers=layer_inputs_from_synth(w, device))


def split_groups(schedule: str):
    """(first layer, layer count) of each group: a Full or Reindex layer and
    the Reuse layers after it (a leading run of Reuse layers is a group too).
    A Full layer that only builds candidates forms a group of its own when a
    Reindex layer follows it."""
    groups = []
    for li, m in enumerate(schedule):
        if li == 0 or m in "FI" or groups[-1][1] >= csa2.MAX_GROUP_LAYERS:
            groups.append([li, 1])
        else:
            groups[-1][1] += 1
    return [tuple(g) for g in groups]


class GroupRunner:
    """Owns the outputs, the shared Top-K / candidate buffers and the workspace
    of one layer group; ``step()`` runs every layer of the schedule once."""

    def __init__(self, w: synth.Workload, inp: GroupInputs, device="cuda"):
        self.w = w
        self.inp = inp
        R = w.R
        self.kv = csa2.make_cache(inp.kv_fp4, inp.kv_scale, inp.page_table, seq_stride=inp.seq_stride)
        self.kidx = csa2.make_cache(inp.k_idx, inp.k_scale, inp.page_table, seq_stride=inp.seq_stride)
        self.topk_idx = torch.full((R, csa2.TOPK), -1, dtype=torch.int32, device=device)
        self.cand = torch.full((R, csa2.KEEP_BLOCKS), -1, dtype=torch.int32, device=device)
        self.shared = csa2.make_shared(self.kv, self.kidx, inp.seq_len, w.n_max, self.topk_idx, self.cand,
                                       hier=w.hier)
        self.groups = split_groups(w.schedule)
        ws_bytes = max(csa2.csa2_workspace_bytes(m, R, w.n_max, w.hier) for m in (0, 1, 2))
        for li0, n in self.groups:
            ws_bytes = max(ws_bytes, csa2.csa2_group_workspace_bytes(synth.MODES[w.schedule[li0]], n, R, w.n_max,
                                                                     w.hier))
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
        csa2.csa2_workspace_init(self.ws)
        self.out = [torch.zeros((R, 16, 512), dtype=torch.float32, device=device) for _ in w.schedule]
        self.lse = [torch.zeros((R, 16), dtype=torch.float32, device=device) for _ in w.schedule]
        self.args = []
        for li, m in enumerate(w.schedule):
            L = inp.layers[li]
            blocks_only = (m == "F" and w.hier and w.full_blocks_only)
            self.args.append(csa2.make_layer_args(L.q, L.swa_k, L.swa_v, L.swa_start, L.swa_len, SM_SCALE,
                                                  self.out[li], self.lse[li], q_idx=L.q_idx, row_seq=inp.row_seq,
                                                  blocks_only=blocks_only, R=R, swa_shared=w.shared_slots))

        self.group_args = [csa2.make_layer_array(self.args[li0:li0 + n]) for li0, n in self.groups]

    def step_layer(self, li: int, stream=None):
        """One layer on its own (csa2_layer_step)."""
        csa2.csa2_layer_step(synth.MODES[self.w.schedule[li]], self.args[li], self.shared, self.ws, stream)

    def step_group(self, gi: int, stream=None):
        """One group: a Full/Reindex layer and the Reuse layers after it (csa2_group_step)."""
        li0, _ = self.groups[gi]
        csa2.csa2_group_step(synth.MODES[self.w.schedule[li0]], self.group_args[gi], self.shared, self.ws, stream)

    def step(self, stream=None):
        """Every layer of the schedule once, one group call per group."""
        for gi in range(len(self.groups)):
            self.step_group(gi, stream)

    def attended_layers(self) -> List[int]:
        return [li for li, m in enumerate(self.w.schedule)
                if not (m == "F" and self.w.hier and self.w.full_blocks_only)]
