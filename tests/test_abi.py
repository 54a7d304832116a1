"""The C-ABI library loads, exports every entry point its header declares, and
rejects bad arguments on the host before launching anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def C():
    from fp4_kv_cache_02_amd import csa2
    return csa2


def test_every_declared_symbol_is_exported(C):
    names = _declared()
    assert len(names) >= 12
    lib = ctypes.CDLL(C.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(C.EXPORTED)


def test_status_strings_and_version(C):
    for s in range(6):
        assert C.csa2_status_string(s)
    assert C.csa2_status_string(0) == "ok"
    assert "gfx950" in C.csa2_version()


def test_workspace_sizes_are_monotone(C):
    a = C.csa2_workspace_bytes(C.FULL, 8, 131072, False)
    b = C.csa2_workspace_bytes(C.FULL, 8, 131072, True)
    c = C.csa2_workspace_bytes(C.REUSE, 8, 131072, False)
    assert 0 < c < a <= b
    assert C.csa2_workspace_bytes(C.FULL, 16, 131072, False) > a
    assert C.csa2_topk_workspace_bytes(8, 131072, 512) > C.csa2_topk_workspace_bytes(8, 4096, 512)
    assert C.csa2_attn_workspace_bytes(16) > C.csa2_attn_workspace_bytes(8)


def test_workspace_covers_the_split_and_large_k_paths(C):
    """The workspace of a Top-k holds the split path's per-segment lists
    (32 segments x 1024 values x (key, position) per row, for k below 1024 on
    rows of 2049 .. 131072 values and at most 256 rows) and the large-k path's
    (16 segments x 8192 per row, k of 1024 and more on rows of 16384 ..
    131072); shapes outside them need no lists."""
    lists = 32 * 1024 * 8
    split_8 = C.csa2_topk_workspace_bytes(8, 131072, 512)
    split_16 = C.csa2_topk_workspace_bytes(16, 131072, 512)
    assert split_16 - split_8 >= 8 * lists                    # per-row lists grow with the rows
    assert C.csa2_topk_workspace_bytes(8, 2048, 512) < 8 * lists   # short rows: one block per row
    assert C.csa2_topk_workspace_bytes(300, 131072, 512) < 300 * lists      # too many rows: no lists
    large = C.csa2_topk_workspace_bytes(1, 131072, 2048)
    assert large >= 16 * 8192 * 8                              # 16 segment lists of 8192
    assert C.csa2_topk_workspace_bytes(1, 16384, 2048) >= 2 * 8192 * 8
    # a group's workspace holds its Full layer's lists
    assert C.csa2_group_workspace_bytes(C.FULL, 4, 8, 131072, 0) >= C.csa2_group_workspace_bytes(C.REUSE, 4, 8,
                                                                                                 131072, 0) \
        + 8 * lists


def _lib(C):
    return ctypes.CDLL(C.LIB_PATH)


def test_host_validation_errors(C):
    lib = _lib(C)
    P = ctypes.c_void_p
    fake = P(0x1000)  # never dereferenced: validation fails first
    cache = C.csa2_cache()
    # NULL inputs
    lib.csa2_index_score.restype = ctypes.c_int
    lib.csa2_index_score.argtypes = C._index_score.argtypes
    assert lib.csa2_index_score(None, None, ctypes.byref(cache), None, None, None, 0, 1, 16, None, None, None) \
        == 1
    cache.data = 0x1000
    cache.n_slots = 16
    # R out of range
    assert lib.csa2_index_score(fake, None, ctypes.byref(cache), None, fake, None, 0, 0, 16, fake, None,
                                None) == 2
    # too many candidate blocks
    assert lib.csa2_index_score(fake, None, ctypes.byref(cache), None, fake, fake, 4096, 1, 16, fake, None,
                                None) == 2
    # unsupported: block maxima with candidates
    assert lib.csa2_index_score(fake, None, ctypes.byref(cache), None, fake, fake, 8, 1, 16, fake, fake,
                                None) == 3
    # paged cache with a page size other than 64
    cache.page_table = 0x1000
    cache.page_size = 32
    cache.max_pages = 4
    assert lib.csa2_index_score(fake, None, ctypes.byref(cache), None, fake, None, 0, 1, 16, fake, None,
                                None) == 3
    cache.page_size = 64
    cache.max_pages = 0
    assert lib.csa2_index_score(fake, None, ctypes.byref(cache), None, fake, None, 0, 1, 16, fake, None,
                                None) == 2
    cache.page_table = None
    cache.max_pages = 0
    # Top-k: k out of range, missing workspace, too small workspace
    assert C._topk(fake, 16, None, None, 1, 16, 0, None, fake, fake, 1 << 30, None) == 2
    assert C._topk(fake, 16, None, None, 1, 16, 4096, None, fake, fake, 1 << 30, None) == 2
    assert C._topk(fake, 16, None, None, 1, 16, 8, None, fake, None, 0, None) == 4
    assert C._topk(fake, 1 << 20, None, None, 4, 1 << 20, 512, None, fake, fake, 1024, None) == 4
    # stride smaller than the row
    assert C._topk(fake, 8, None, None, 1, 16, 8, None, fake, fake, 1 << 30, None) == 2
    # attention: k above 512, NULL window
    kv = C.csa2_cache()
    kv.data, kv.scale, kv.n_slots = 0x1000, 0x1000, 16
    assert C._attn(fake, ctypes.byref(kv), None, fake, fake, 513, fake, fake, 128, fake, fake, 0.1, 1, fake,
                   None, fake, 1 << 30, None) == 2
    assert C._attn(fake, ctypes.byref(kv), None, fake, fake, 512, None, fake, 128, fake, fake, 0.1, 1, fake,
                   None, fake, 1 << 30, None) == 1
    # main KV without scales
    kv.scale = None
    assert C._attn(fake, ctypes.byref(kv), None, fake, fake, 512, fake, fake, 128, fake, fake, 0.1, 1, fake,
                   None, fake, 1 << 30, None) == 1
    # layer step: bad mode, missing workspace
    a = C.csa2_layer_args()
    s = C.csa2_shared()
    assert C._layer(7, ctypes.byref(a), ctypes.byref(s), None, 0, None) == 3
    a.R = 1
    s.B, s.n_max = 1, 16
    s.seq_len = s.topk_idx = 0x1000
    s.kv.data, s.kv.scale, s.kv.n_slots = 0x1000, 0x1000, 16
    a.q = a.swa_k = a.swa_v = a.swa_start = a.swa_len = a.out = 0x1000
    assert C._layer(C.REUSE, ctypes.byref(a), ctypes.byref(s), None, 0, None) == 4
    assert C._layer(C.REUSE, ctypes.byref(a), ctypes.byref(s), fake, 100, None) == 4
    # Full needs an indexer query
    assert C._layer(C.FULL, ctypes.byref(a), ctypes.byref(s), fake, 1 << 40, None) == 1
    # group step: layer count out of range, rows differing between layers,
    # rows x layers above the limit, context above the Top-k limit
    arr = C.make_layer_array([a, a])
    assert C._group(C.REUSE, 0, ctypes.cast(arr, ctypes.c_void_p), ctypes.byref(s), fake, 1 << 40, None) == 2
    assert C._group(C.REUSE, C.MAX_GROUP_LAYERS + 1, ctypes.cast(arr, ctypes.c_void_p), ctypes.byref(s), fake,
                    1 << 40, None) == 2
    b2 = C.csa2_layer_args()
    ctypes.pointer(b2)[0] = a
    b2.R = 2
    arr2 = C.make_layer_array([a, b2])
    assert C._group(C.REUSE, 2, ctypes.cast(arr2, ctypes.c_void_p), ctypes.byref(s), fake, 1 << 40, None) == 2
    big = C.csa2_layer_args()
    ctypes.pointer(big)[0] = a
    big.R = C.MAX_ROWS // 2 + 1
    arr3 = C.make_layer_array([big, big])
    assert C._group(C.REUSE, 2, ctypes.cast(arr3, ctypes.c_void_p), ctypes.byref(s), fake, 1 << 40, None) == 2
    s.n_max = (1 << 20) + 1
    assert C._group(C.REUSE, 2, ctypes.cast(arr, ctypes.c_void_p), ctypes.byref(s), fake, 1 << 40, None) == 3
    s.n_max = 16
    assert C._topk(fake, (1 << 20) + 1, None, None, 1, (1 << 20) + 1, 8, None, fake, fake, 1 << 40, None) == 3
    # the group workspace grows with the layer count
    assert C.csa2_group_workspace_bytes(C.FULL, 4, 8, 131072, False) > \
        C.csa2_group_workspace_bytes(C.FULL, 1, 8, 131072, False)
    assert C.csa2_group_workspace_bytes(C.FULL, 9, 8, 131072, False) == 0
    # quantiser: negative count; workspace init with a tiny buffer
    assert C._quant(fake, -1, None, fake, fake, 16, None) == 2
    assert C._quant(fake, 32, None, fake, fake, 16, None) == 2
    assert C._ws_init(fake, 16, None) == 4
    assert C._ws_init(None, 1 << 20, None) == 1


# Without a GPU every launch fails with CSA2_ERR_HIP (5); the entry points carve
# their workspace and check it against ws_bytes before the first launch, so a
# call that gets as far as status 5 was given enough workspace by the sizing
# function, while CSA2_ERR_WORKSPACE (4) would mean the sizing fell short.
ATTN_KS = (1, 100, 127, 128, 129, 200, 255, 256, 257, 300, 383, 384, 385, 450, 511, 512)


def _kv_desc(C, paged=False, page_size=64):
    kv = C.csa2_cache()
    kv.data, kv.scale, kv.n_slots = 0x1000, 0x1000, 1 << 20
    if paged:
        kv.page_table, kv.page_size, kv.max_pages = 0x1000, page_size, 16
    return kv


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="relies on launches failing without a GPU")
def test_attention_workspace_covers_every_k(C):
    """csa2_attn_workspace_bytes(R) suffices for every k of 1..512: the
    partials depend on k through its number of 128-key steps, and fewer steps
    can take more blocks per row (e.g. k = 300 at R = 90)."""
    fake = ctypes.c_void_p(0x1000)
    kv = _kv_desc(C)
    for R in range(1, 601):
        ws = C.csa2_attn_workspace_bytes(R)
        for k in ATTN_KS:
            st = C._attn(fake, ctypes.byref(kv), None, fake, fake, k, fake, fake, 128, fake, fake, 0.1, R, fake,
                         None, fake, ws, None)
            assert st == 5, (R, k, st)
    # and a workspace one byte short of a case that needs partials is refused
    ws = C.csa2_attn_workspace_bytes(90)
    assert C._attn(fake, ctypes.byref(kv), None, fake, fake, 300, fake, fake, 128, fake, fake, 0.1, 90, fake, None,
                   fake, 1024, None) == 4
    assert ws > 1024


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="relies on launches failing without a GPU")
def test_group_workspace_covers_every_layer_count(C):
    """csa2_group_workspace_bytes suffices for groups of 1..8 layers at any R,
    including a hierarchical Full layer that only builds candidates (its
    group attends n_layers - 1 layers, which can need more partials)."""
    fake = 0x1000
    s = C.csa2_shared()
    s.kv = _kv_desc(C)
    s.k_idx.data, s.k_idx.n_slots = fake, 1 << 20
    s.B, s.n_max = 1, 4096
    s.seq_len = s.topk_idx = s.cand_blocks = fake
    for hier, blocks_only, mode in ((0, 0, C.REUSE), (1, 1, C.FULL), (1, 0, C.FULL), (0, 0, C.FULL)):
        s.hier = hier
        for n in range(1, C.MAX_GROUP_LAYERS + 1):
            for R in list(range(1, 200)) + list(range(200, 601, 7)):
                a = C.csa2_layer_args()
                a.R = R
                a.q = a.swa_k = a.swa_v = a.swa_start = a.swa_len = a.out = a.q_idx = fake
                a.blocks_only = blocks_only
                arr = C.make_layer_array([a] * n)
                ws = C.csa2_group_workspace_bytes(mode, n, R, s.n_max, bool(hier))
                st = C._group(mode, n, ctypes.cast(arr, ctypes.c_void_p), ctypes.byref(s), ctypes.c_void_p(fake),
                              ws, None)
                assert st == 5, (mode, hier, blocks_only, n, R, st)


def test_page_size_other_than_64_is_unsupported(C):
    fake = ctypes.c_void_p(0x1000)
    kv = _kv_desc(C, paged=True, page_size=32)
    assert C._attn(fake, ctypes.byref(kv), None, fake, fake, 512, fake, fake, 128, fake, fake, 0.1, 1, fake, None,
                   fake, 1 << 30, None) == 3
    s = C.csa2_shared()
    s.kv = kv
    s.B, s.n_max = 1, 16
    s.seq_len = s.topk_idx = 0x1000
    a = C.csa2_layer_args()
    a.R = 1
    a.q = a.swa_k = a.swa_v = a.swa_start = a.swa_len = a.out = 0x1000
    assert C._layer(C.REUSE, ctypes.byref(a), ctypes.byref(s), fake, 1 << 30, None) == 3
