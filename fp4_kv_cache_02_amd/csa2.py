"""Thin ctypes binding of libcsa2.so (include/csa2.h), same entry-point names.

Argument marshalling only: every step runs in the library's HIP kernels.
Tensors are torch tensors on the GPU (plumbing for device memory); streams
default to torch's current stream.  A non-zero status raises ``Csa2Error``.
The library must have been built (``fp4_kv_cache_02_amd.build``); importing
this module fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("CSA2_LIB") or os.path.join(HERE, "libcsa2.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run python -m fp4_kv_cache_02_amd.build "
                      "or __graft_entry__.build()")
_lib = ctypes.CDLL(LIB_PATH)

# constants mirrored from csa2.h
HEADS, DIM, IDX_HEADS, IDX_DIM = 16, 512, 4, 64
BLOCK, MAX_WINDOW, TOPK, KEEP_BLOCKS, MAX_K, PAGE, MAX_ROWS = 8, 128, 512, 2048, 2048, 64, 65536
MAX_GROUP_LAYERS = 8
FULL, REINDEX, REUSE = 0, 1, 2

c_i32p = ctypes.c_void_p
c_ptr = ctypes.c_void_p


class csa2_cache(ctypes.Structure):
    _fields_ = [("data", c_ptr), ("scale", c_ptr), ("page_table", c_ptr), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("seq_stride", ctypes.c_int64), ("n_slots", ctypes.c_int64)]


class csa2_shared(ctypes.Structure):
    _fields_ = [("kv", csa2_cache), ("k_idx", csa2_cache), ("seq_len", c_ptr), ("B", ctypes.c_int32),
                ("n_max", ctypes.c_int32), ("hier", ctypes.c_int32), ("topk_idx", c_ptr),
                ("cand_blocks", c_ptr)]


class csa2_layer_args(ctypes.Structure):
    _fields_ = [("R", ctypes.c_int32), ("row_seq", c_ptr), ("q_idx", c_ptr), ("head_w", c_ptr), ("q", c_ptr),
                ("swa_k", c_ptr), ("swa_v", c_ptr), ("S", ctypes.c_int32), ("swa_start", c_ptr),
                ("swa_len", c_ptr), ("sm_scale", ctypes.c_float), ("blocks_only", ctypes.c_int32),
                ("out", c_ptr), ("lse", c_ptr), ("swa_shared", ctypes.c_int32)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_st = ctypes.c_int
_sz = ctypes.c_size_t
_i32, _i64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_P = ctypes.POINTER

_index_score = _sig("csa2_index_score", _st, [c_ptr, c_ptr, _P(csa2_cache), c_ptr, c_ptr, c_ptr, _i32, _i32,
                                               _i32, c_ptr, c_ptr, c_ptr])
_topk = _sig("csa2_topk", _st, [c_ptr, _i64, c_ptr, c_ptr, _i32, _i32, _i32, c_ptr, c_ptr, c_ptr, _sz, c_ptr])
_topk_ws = _sig("csa2_topk_workspace_bytes", _sz, [_i32, _i32, _i32])
_hier = _sig("csa2_hier_candidates", _st, [c_ptr, c_ptr, c_ptr, _i32, _i32, _i32, c_ptr, c_ptr, _sz, c_ptr])
_attn = _sig("csa2_fp4_sparse_attn", _st, [c_ptr, _P(csa2_cache), c_ptr, c_ptr, c_ptr, _i32, c_ptr, c_ptr, _i32,
                                           c_ptr, c_ptr, _f32, _i32, c_ptr, c_ptr, c_ptr, _sz, c_ptr])
_attn_ws = _sig("csa2_attn_workspace_bytes", _sz, [_i32])
_quant = _sig("csa2_fp4_quantize", _st, [c_ptr, _i64, c_ptr, c_ptr, c_ptr, _i64, c_ptr])
_fp8q = _sig("csa2_fp8_key_quantize", _st, [c_ptr, _i64, c_ptr, c_ptr, c_ptr, _i64, c_ptr])
_layer = _sig("csa2_layer_step", _st, [_i32, _P(csa2_layer_args), _P(csa2_shared), c_ptr, _sz, c_ptr])
_ws_bytes = _sig("csa2_workspace_bytes", _sz, [_i32, _i32, _i32, _i32])
_group = _sig("csa2_group_step", _st, [_i32, _i32, ctypes.c_void_p, _P(csa2_shared), c_ptr, _sz, c_ptr])
_group_ws = _sig("csa2_group_workspace_bytes", _sz, [_i32, _i32, _i32, _i32, _i32])
_group_noalloc = _sig("csa2_group_step_noalloc", _st, [_i32, _i32, ctypes.c_void_p, _P(csa2_shared), c_ptr])
_ws_init = _sig("csa2_workspace_init", _st, [c_ptr, _sz, c_ptr])
_status_string = _sig("csa2_status_string", ctypes.c_char_p, [_st])
_version = _sig("csa2_version", ctypes.c_char_p, [])

EXPORTED = ("csa2_index_score", "csa2_topk", "csa2_topk_workspace_bytes", "csa2_hier_candidates",
            "csa2_fp4_sparse_attn", "csa2_attn_workspace_bytes", "csa2_fp4_quantize", "csa2_layer_step",
            "csa2_workspace_bytes", "csa2_group_step", "csa2_group_workspace_bytes", "csa2_workspace_init",
            "csa2_status_string", "csa2_version", "csa2_group_step_noalloc",
            "csa2_fp8_key_quantize")
NOALLOC_SCRATCH_BYTES = 64 << 20


class Csa2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({csa2_status_string(status)})")


def _check(status: int, where: str):
    if status != 0:
        raise Csa2Error(status, where)


def _p(t) -> Optional[int]:
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def csa2_status_string(status: int) -> str:
    return _status_string(status).decode()


def csa2_version() -> str:
    return _version().decode()


def make_cache(data, scale=None, page_table=None, seq_stride: int = 0, n_slots: Optional[int] = None,
               page_size: int = PAGE) -> csa2_cache:
    """Describe a per-position cache.  data: [n_slots, 256] uint8 (main KV),
    [n_slots, 64] bf16/int16 (indexer keys) or [n_slots, 64] uint8 E4M3 codes
    (FP8 indexer keys); scale: [n_slots, 32] uint8 (main KV), None (bf16
    indexer keys) or [n_slots] float32 (FP8 indexer keys); page_table:
    [B, max_pages] int32 or None (then slot = b*seq_stride + p)."""
    c = csa2_cache()
    c.data = _p(data)
    c.scale = _p(scale)
    c.page_table = _p(page_table)
    c.page_size = page_size if page_table is not None else 0
    c.max_pages = int(page_table.shape[1]) if page_table is not None else 0
    c.seq_stride = int(seq_stride)
    c.n_slots = int(data.shape[0]) if n_slots is None else int(n_slots)
    c._keep = (data, scale, page_table)  # keep tensors alive while the struct is
    return c


def csa2_index_score(q_idx, k_idx: csa2_cache, seq_len, scores, row_seq=None, head_w=None, cand_blocks=None,
                     n_max: Optional[int] = None, block_max=None, stream=None):
    R = int(q_idx.shape[0])
    n_cand = int(cand_blocks.shape[1]) if cand_blocks is not None else 0
    if n_max is None:
        n_max = int(scores.shape[1]) if cand_blocks is None else 0
    _check(_index_score(_p(q_idx), _p(head_w), ctypes.byref(k_idx), _p(row_seq), _p(seq_len), _p(cand_blocks),
                        n_cand, R, n_max, _p(scores), _p(block_max), _stream(stream)), "csa2_index_score")


def csa2_topk_workspace_bytes(R: int, n_max: int, k: int) -> int:
    return int(_topk_ws(R, n_max, k))


def csa2_topk(scores, k: int, idx, ws, n_valid=None, row_seq=None, n_max: Optional[int] = None,
              cand_blocks=None, stream=None):
    R = int(scores.shape[0])
    stride = int(scores.stride(0))
    n_max = int(scores.shape[1]) if n_max is None else n_max
    _check(_topk(_p(scores), stride, _p(row_seq), _p(n_valid), R, n_max, k, _p(cand_blocks), _p(idx), _p(ws),
                 ws.numel() * ws.element_size(), _stream(stream)), "csa2_topk")


def csa2_hier_candidates(block_max, seq_len, n_max: int, keep: int, cand_blocks, ws, row_seq=None, stream=None):
    R = int(block_max.shape[0])
    _check(_hier(_p(block_max), _p(row_seq), _p(seq_len), R, n_max, keep, _p(cand_blocks), _p(ws),
                 ws.numel() * ws.element_size(), _stream(stream)), "csa2_hier_candidates")


def csa2_attn_workspace_bytes(R: int) -> int:
    return int(_attn_ws(R))


def csa2_fp4_sparse_attn(q, kv: csa2_cache, seq_len, idx, swa_k, swa_v, swa_start, swa_len, sm_scale: float,
                         out, lse=None, ws=None, row_seq=None, stream=None):
    R = int(q.shape[0])
    k = int(idx.shape[1])
    S = int(swa_k.shape[1])
    _check(_attn(_p(q), ctypes.byref(kv), _p(row_seq), _p(seq_len), _p(idx), k, _p(swa_k), _p(swa_v), S,
                 _p(swa_start), _p(swa_len), float(sm_scale), R, _p(out), _p(lse), _p(ws),
                 ws.numel() * ws.element_size(), _stream(stream)), "csa2_fp4_sparse_attn")


def csa2_fp4_quantize(x, fp4, scale, dst_slot=None, stream=None):
    n = int(x.shape[0])
    _check(_quant(_p(x), n, _p(dst_slot), _p(fp4), _p(scale), int(fp4.shape[0]), _stream(stream)),
           "csa2_fp4_quantize")


def csa2_fp8_key_quantize(k, codes, scale, dst_slot=None, stream=None):
    """k: [n, 64] bf16 bits (int16/bf16); codes: [n_slots, 64] uint8; scale: [n_slots] float32."""
    n = int(k.shape[0])
    _check(_fp8q(_p(k), n, _p(dst_slot), _p(codes), _p(scale), int(codes.shape[0]), _stream(stream)),
           "csa2_fp8_key_quantize")


def csa2_workspace_bytes(mode: int, R: int, n_max: int, hier: bool) -> int:
    return int(_ws_bytes(mode, R, n_max, 1 if hier else 0))


def csa2_workspace_init(ws, stream=None):
    _check(_ws_init(_p(ws), ws.numel() * ws.element_size(), _stream(stream)), "csa2_workspace_init")


def make_shared(kv: csa2_cache, k_idx: csa2_cache, seq_len, n_max: int, topk_idx, cand_blocks=None,
                hier: bool = False) -> csa2_shared:
    s = csa2_shared()
    s.kv = kv
    s.k_idx = k_idx
    s.seq_len = _p(seq_len)
    s.B = int(seq_len.shape[0])
    s.n_max = int(n_max)
    s.hier = 1 if hier else 0
    s.topk_idx = _p(topk_idx)
    s.cand_blocks = _p(cand_blocks)
    s._keep = (kv, k_idx, seq_len, topk_idx, cand_blocks)
    return s


def make_layer_args(q, swa_k, swa_v, swa_start, swa_len, sm_scale: float, out, lse=None, q_idx=None,
                    head_w=None, row_seq=None, blocks_only: bool = False, R: Optional[int] = None,
                    swa_shared: bool = False) -> csa2_layer_args:
    a = csa2_layer_args()
    a.R = int(R if R is not None else (q.shape[0] if q is not None else q_idx.shape[0]))
    a.row_seq = _p(row_seq)
    a.q_idx = _p(q_idx)
    a.head_w = _p(head_w)
    a.q = _p(q)
    a.swa_k = _p(swa_k)
    a.swa_v = _p(swa_v)
    a.S = int(swa_k.shape[1]) if swa_k is not None else 0
    a.swa_start = _p(swa_start)
    a.swa_len = _p(swa_len)
    a.sm_scale = float(sm_scale)
    a.blocks_only = 1 if blocks_only else 0
    a.out = _p(out)
    a.lse = _p(lse)
    a.swa_shared = 1 if swa_shared else 0
    a._keep = (q, swa_k, swa_v, swa_start, swa_len, out, lse, q_idx, head_w, row_seq)
    return a


def csa2_layer_step(mode: int, args: csa2_layer_args, shared: csa2_shared, ws, stream=None):
    _check(_layer(mode, ctypes.byref(args), ctypes.byref(shared), _p(ws), ws.numel() * ws.element_size(),
                  _stream(stream)), "csa2_layer_step")


def csa2_group_workspace_bytes(first_mode: int, n_layers: int, R: int, n_max: int, hier: bool) -> int:
    return int(_group_ws(first_mode, n_layers, R, n_max, 1 if hier else 0))


def make_layer_array(layers):
    """A contiguous C array of csa2_layer_args (kept alive with its inputs)."""
    arr = (csa2_layer_args * len(layers))(*layers)
    arr._keep = layers
    return arr


def csa2_group_step(first_mode: int, layers, shared: csa2_shared, ws, stream=None):
    """layers: a csa2_layer_args array from make_layer_array (layer 0 in
    first_mode, the rest Reuse)."""
    _check(_group(first_mode, len(layers), ctypes.cast(layers, ctypes.c_void_p), ctypes.byref(shared), _p(ws),
                  ws.numel() * ws.element_size(), _stream(stream)), "csa2_group_step")


def csa2_group_step_noalloc(first_mode: int, layers, shared: csa2_shared, stream=None):
    """csa2_group_step on the library's static scratch (no workspace, no
    allocation); layers as for csa2_group_step."""
    _check(_group_noalloc(first_mode, len(layers), ctypes.cast(layers, ctypes.c_void_p), ctypes.byref(shared),
                          _stream(stream)), "csa2_group_step_noalloc")
