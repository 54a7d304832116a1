// Host side of the C ABI: argument validation, workspace layout, dispatch of
// the CSA2 layer modes (Full / Reindex / Reuse) onto the kernels.
//
// Modes as the pages describe them (conexaotc.com.br page "DeepSeek lança
// V4.1-Flash...", paragraph on CSA2; 7minutos.es page, section "Atención
// escasa comprimida 2 (CSA2)"): Full scores every position with its own
// indexer query and keeps a new Top-512 (and, in the decoder, the candidate
// set of 2048 blocks of 8); Reindex re-scores the candidate positions of the
// last Full layer with its own indexer query and keeps a new Top-512; Reuse
// takes the most recent Top-K.  Every mode attends with the layer's own query
// and window.
#include <algorithm>

#include "kernels.h"

using namespace csa2;

namespace {

constexpr size_t kAlign = 256;
// control words: topk tickets, attention tickets (must be zero between calls)
constexpr size_t kCtrlTopk = 0;
constexpr size_t kCtrlAttn = (size_t)CSA2_MAX_ROWS * 4;
constexpr size_t kCtrlBytes = (size_t)CSA2_MAX_ROWS * 8;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Bump {
  char* base;
  size_t off;
  template <class T>
  T* take(size_t n) {
    T* p = base ? (T*)(base + off) : nullptr;
    off = align_up(off + n * sizeof(T));
    return p;
  }
};

struct TopkWs {
  uint32_t* cand_key;
  int32_t* cand_idx;
  int32_t* seg_info;
};

TopkWs carve_topk(Bump& bp, int R, int n_max, int k) {
  const int S = topk_segments(n_max);
  const int kcap = topk_kcap(k);
  TopkWs t;
  if (S <= 1) {  // single segment per row: selection is direct, no candidates
    t.cand_key = nullptr;
    t.cand_idx = nullptr;
    t.seg_info = nullptr;
    return t;
  }
  t.cand_key = bp.take<uint32_t>((size_t)R * S * kcap);
  t.cand_idx = bp.take<int32_t>((size_t)R * S * kcap);
  t.seg_info = bp.take<int32_t>((size_t)R * S * 4);
  return t;
}

struct AttnWs {
  float* part_o;
  float* part_ml;
  int n_main, n_splits;
};

AttnWs carve_attn(Bump& bp, int R, int k) {
  AttnWs w;
  w.n_splits = attn_splits(k, &w.n_main);
  w.part_o = bp.take<float>((size_t)R * w.n_splits * 16 * 512);
  w.part_ml = bp.take<float>((size_t)R * w.n_splits * 32);
  return w;
}

bool cache_ok(const csa2_cache* c, bool need_scale) {
  if (!c || !c->data) return false;
  if (need_scale && !c->scale) return false;
  if (c->n_slots < 0) return false;
  if (c->page_table && (c->page_size != CSA2_PAGE || c->max_pages <= 0)) return false;
  if (!c->page_table && c->seq_stride < 0) return false;
  return true;
}

csa2_status hip_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

csa2_status do_index_score(const uint16_t* q_idx, const float* head_w, const csa2_cache* k_idx,
                           const int32_t* row_seq, const int32_t* seq_len, const int32_t* cand,
                           int32_t n_cand, int32_t R, int32_t n_max, float* scores, float* bmax,
                           hipStream_t st) {
  IdxArgs a;
  a.q32 = (const uint32_t*)q_idx;
  a.head_w = head_w;
  a.kdata = (const uint4*)k_idx->data;
  a.map = make_slot_map(*k_idx);
  a.row_seq = row_seq;
  a.seq_len = seq_len;
  a.cand = cand;
  a.n_cand = n_cand;
  a.R = R;
  a.n_max = n_max;
  a.tiles_per_row = cand ? (n_cand * 8 + 255) / 256 : (n_max + 255) / 256;
  a.score_stride = cand ? (int64_t)n_cand * 8 : n_max;
  a.bmax_stride = (n_max + 7) / 8;
  a.scores = scores;
  a.block_max = bmax;
  return hip_status(launch_index_score(a, cand != nullptr, head_w != nullptr, bmax != nullptr, st));
}

csa2_status do_topk(const float* scores, int64_t stride, const int32_t* row_seq, const int32_t* n_valid,
                    int n_div, int R, int n_max, int k, const int32_t* cand_blocks, int cand_stride,
                    int32_t* out, const TopkWs& tw, char* ws, hipStream_t st) {
  TopkArgs a;
  a.scores = scores;
  a.row_stride = stride;
  a.row_seq = row_seq;
  a.n_valid = n_valid;
  a.n_max = n_max;
  a.n_div = n_div;
  a.R = R;
  a.k = k;
  a.S_max = topk_segments(n_max);
  a.kcap = topk_kcap(k);
  a.cand_blocks = cand_blocks;
  a.cand_stride = cand_stride;
  a.out = out;
  a.out_stride = k;
  a.cand_key = tw.cand_key;
  a.cand_idx = tw.cand_idx;
  a.seg_info = tw.seg_info;
  a.ticket = (uint32_t*)(ws + kCtrlTopk);
  return hip_status(launch_topk(a, st));
}

csa2_status do_attn(const uint16_t* q, const csa2_cache* kv, const int32_t* row_seq,
                    const int32_t* seq_len, const int32_t* idx, int32_t k, const uint16_t* swa_k,
                    const uint16_t* swa_v, int32_t S, const int32_t* swa_start, const int32_t* swa_len,
                    float sm_scale, int32_t R, float* out, float* lse, const AttnWs& aw, char* ws,
                    hipStream_t st) {
  AttnArgs a;
  a.q = (const uint4*)q;
  a.kv = (const uint8_t*)kv->data;
  a.kv_scale = kv->scale;
  a.map = make_slot_map(*kv);
  a.row_seq = row_seq;
  a.seq_len = seq_len;
  a.idx = idx;
  a.k = k;
  a.swa_k = (const uint4*)swa_k;
  a.swa_v = (const uint4*)swa_v;
  a.S = S;
  a.swa_start = swa_start;
  a.swa_len = swa_len;
  a.sm_scale = sm_scale;
  a.R = R;
  a.out = out;
  a.lse = lse;
  a.part_o = aw.part_o;
  a.part_ml = aw.part_ml;
  a.ticket = (uint32_t*)(ws + kCtrlAttn);
  a.n_main_splits = aw.n_main;
  a.n_splits = aw.n_splits;
  return hip_status(launch_attn(a, st));
}

size_t topk_region(int R, int n_max, int k) {
  Bump bp{nullptr, 0};
  carve_topk(bp, R, n_max, k);
  return bp.off;
}

size_t attn_region(int R, int k) {
  Bump bp{nullptr, 0};
  carve_attn(bp, R, k);
  return bp.off;
}

}  // namespace

extern "C" {

const char* csa2_status_string(csa2_status s) {
  switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_NULL: return "a required pointer is NULL";
    case CSA2_ERR_SHAPE: return "a size or count is out of range";
    case CSA2_ERR_UNSUPPORTED: return "unsupported layout or parameter";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* csa2_version(void) { return "csa2-gfx950 0.1"; }

csa2_status csa2_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws) return CSA2_ERR_NULL;
  if (ws_bytes < kCtrlBytes) return CSA2_ERR_WORKSPACE;
  return hip_status(launch_fill_u32((uint32_t*)ws, (int64_t)(kCtrlBytes / 4), 0u, stream));
}

size_t csa2_topk_workspace_bytes(int32_t R, int32_t n_max, int32_t k) {
  if (R < 0 || n_max < 0 || k < 1) return 0;
  return kCtrlBytes + topk_region(R, n_max, k);
}

size_t csa2_attn_workspace_bytes(int32_t R) {
  if (R < 0) return 0;
  return kCtrlBytes + attn_region(R, CSA2_TOPK);
}

csa2_status csa2_index_score(const uint16_t* q_idx, const float* head_w, const csa2_cache* k_idx,
                             const int32_t* row_seq, const int32_t* seq_len, const int32_t* cand_blocks,
                             int32_t n_cand, int32_t R, int32_t n_max, float* scores, float* block_max,
                             hipStream_t stream) {
  if (!q_idx || !k_idx || !seq_len || !scores) return CSA2_ERR_NULL;
  if (!cache_ok(k_idx, false)) return CSA2_ERR_NULL;
  if (R < 1 || R > CSA2_MAX_ROWS || n_max < 0) return CSA2_ERR_SHAPE;
  if (cand_blocks) {
    if (n_cand < 1 || n_cand > CSA2_KEEP_BLOCKS) return CSA2_ERR_SHAPE;
    if (block_max) return CSA2_ERR_UNSUPPORTED;
  }
  return do_index_score(q_idx, head_w, k_idx, row_seq, seq_len, cand_blocks, n_cand, R, n_max, scores,
                        block_max, stream);
}

csa2_status csa2_topk(const float* scores, int64_t row_stride, const int32_t* row_seq,
                      const int32_t* n_valid, int32_t R, int32_t n_max, int32_t k,
                      const int32_t* cand_blocks, int32_t* idx, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  if (!scores || !idx) return CSA2_ERR_NULL;
  if (R < 1 || R > CSA2_MAX_ROWS || n_max < 0 || k < 1 || k > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  if (row_stride < n_max) return CSA2_ERR_SHAPE;
  if (cand_blocks && n_max % 8) return CSA2_ERR_SHAPE;
  if (!ws) return CSA2_ERR_WORKSPACE;
  if (ws_bytes < csa2_topk_workspace_bytes(R, n_max, k)) return CSA2_ERR_WORKSPACE;
  Bump bp{(char*)ws, kCtrlBytes};
  TopkWs tw = carve_topk(bp, R, n_max, k);
  return do_topk(scores, row_stride, row_seq, n_valid, 1, R, n_max, k, cand_blocks, n_max / 8, idx, tw,
                 (char*)ws, stream);
}

csa2_status csa2_hier_candidates(const float* block_max, const int32_t* row_seq, const int32_t* seq_len,
                                 int32_t R, int32_t n_max, int32_t keep, int32_t* cand_blocks, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  if (!block_max || !seq_len || !cand_blocks) return CSA2_ERR_NULL;
  if (R < 1 || R > CSA2_MAX_ROWS || n_max < 0 || keep < 1 || keep > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  const int nb = (n_max + 7) / 8;
  if (!ws) return CSA2_ERR_WORKSPACE;
  if (ws_bytes < csa2_topk_workspace_bytes(R, nb, keep)) return CSA2_ERR_WORKSPACE;
  Bump bp{(char*)ws, kCtrlBytes};
  TopkWs tw = carve_topk(bp, R, nb, keep);
  return do_topk(block_max, nb, row_seq, seq_len, 8, R, nb, keep, nullptr, 0, cand_blocks, tw, (char*)ws,
                 stream);
}

csa2_status csa2_fp4_sparse_attn(const uint16_t* q, const csa2_cache* kv, const int32_t* row_seq,
                                 const int32_t* seq_len, const int32_t* idx, int32_t k, const uint16_t* swa_k,
                                 const uint16_t* swa_v, int32_t S, const int32_t* swa_start,
                                 const int32_t* swa_len, float sm_scale, int32_t R, float* out, float* lse,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!q || !kv || !seq_len || !idx || !swa_k || !swa_v || !swa_start || !swa_len || !out)
    return CSA2_ERR_NULL;
  if (!cache_ok(kv, true)) return CSA2_ERR_NULL;
  if (R < 1 || R > CSA2_MAX_ROWS || k < 1 || k > CSA2_TOPK || S < 0) return CSA2_ERR_SHAPE;
  if (!ws) return CSA2_ERR_WORKSPACE;
  if (ws_bytes < csa2_attn_workspace_bytes(R)) return CSA2_ERR_WORKSPACE;
  Bump bp{(char*)ws, kCtrlBytes};
  AttnWs aw = carve_attn(bp, R, k);
  return do_attn(q, kv, row_seq, seq_len, idx, k, swa_k, swa_v, S, swa_start, swa_len, sm_scale, R, out, lse,
                 aw, (char*)ws, stream);
}

csa2_status csa2_fp4_quantize(const float* x, int64_t n, const int64_t* dst_slot, uint8_t* fp4,
                              uint8_t* scale, int64_t n_slots, hipStream_t stream) {
  if (n > 0 && (!x || !fp4 || !scale)) return CSA2_ERR_NULL;
  if (n < 0 || n_slots < 0) return CSA2_ERR_SHAPE;
  if (!dst_slot && n > n_slots) return CSA2_ERR_SHAPE;
  if (n / 4 >= (int64_t)0x7FFFFFFF) return CSA2_ERR_SHAPE;
  return hip_status(launch_quant(x, n, dst_slot, fp4, scale, n_slots, stream));
}

size_t csa2_workspace_bytes(csa2_mode mode, int32_t R, int32_t n_max, int32_t hier) {
  if (R < 0 || n_max < 0) return 0;
  Bump bp{nullptr, kCtrlBytes};
  if (mode == CSA2_FULL) {
    bp.take<float>((size_t)R * n_max);
    if (hier) bp.take<float>((size_t)R * ((n_max + 7) / 8));
    const size_t t1 = topk_region(R, n_max, CSA2_TOPK);
    const size_t t2 = hier ? topk_region(R, (n_max + 7) / 8, CSA2_KEEP_BLOCKS) : 0;
    bp.off = align_up(bp.off + std::max(t1, t2));
  } else if (mode == CSA2_REINDEX) {
    const int nc = hier ? CSA2_KEEP_BLOCKS * 8 : n_max;
    bp.take<float>((size_t)R * nc);
    bp.off = align_up(bp.off + topk_region(R, nc, CSA2_TOPK));
  }
  bp.off = align_up(bp.off + attn_region(R, CSA2_TOPK));
  return bp.off;
}

csa2_status csa2_layer_step(csa2_mode mode, const csa2_layer_args* a, const csa2_shared* sh, void* ws,
                            size_t ws_bytes, hipStream_t st) {
  if (!a || !sh) return CSA2_ERR_NULL;
  if (mode != CSA2_FULL && mode != CSA2_REINDEX && mode != CSA2_REUSE) return CSA2_ERR_UNSUPPORTED;
  const int R = a->R, n_max = sh->n_max;
  if (R < 1 || R > CSA2_MAX_ROWS || n_max < 0 || sh->B < 1) return CSA2_ERR_SHAPE;
  if (!sh->seq_len || !sh->topk_idx) return CSA2_ERR_NULL;
  if (!cache_ok(&sh->kv, true)) return CSA2_ERR_NULL;
  const bool blocks_only = mode == CSA2_FULL && sh->hier && a->blocks_only;
  if (!blocks_only) {
    if (!a->q || !a->swa_k || !a->swa_v || !a->swa_start || !a->swa_len || !a->out) return CSA2_ERR_NULL;
    if (a->S < 0) return CSA2_ERR_SHAPE;
  }
  if (mode != CSA2_REUSE) {
    if (!a->q_idx) return CSA2_ERR_NULL;
    if (!cache_ok(&sh->k_idx, false)) return CSA2_ERR_NULL;
  }
  if (sh->hier && mode != CSA2_REUSE && !sh->cand_blocks) return CSA2_ERR_NULL;
  if (!ws) return CSA2_ERR_WORKSPACE;
  if (ws_bytes < csa2_workspace_bytes(mode, R, n_max, sh->hier)) return CSA2_ERR_WORKSPACE;

  char* w = (char*)ws;
  Bump bp{w, kCtrlBytes};
  csa2_status s = CSA2_OK;
  if (mode == CSA2_FULL) {
    float* scores = bp.take<float>((size_t)R * n_max);
    float* bmax = sh->hier ? bp.take<float>((size_t)R * ((n_max + 7) / 8)) : nullptr;
    const size_t mark = bp.off;
    s = do_index_score(a->q_idx, a->head_w, &sh->k_idx, a->row_seq, sh->seq_len, nullptr, 0, R, n_max, scores,
                       bmax, st);
    if (s) return s;
    if (!blocks_only) {
      TopkWs tw = carve_topk(bp, R, n_max, CSA2_TOPK);
      s = do_topk(scores, n_max, a->row_seq, sh->seq_len, 1, R, n_max, CSA2_TOPK, nullptr, 0, sh->topk_idx, tw,
                  w, st);
      if (s) return s;
    }
    if (sh->hier) {
      bp.off = mark;
      const int nb = (n_max + 7) / 8;
      TopkWs tw = carve_topk(bp, R, nb, CSA2_KEEP_BLOCKS);
      s = do_topk(bmax, nb, a->row_seq, sh->seq_len, 8, R, nb, CSA2_KEEP_BLOCKS, nullptr, 0, sh->cand_blocks,
                  tw, w, st);
      if (s) return s;
    }
    bp.off = mark;
    bp.off = align_up(bp.off + std::max(topk_region(R, n_max, CSA2_TOPK),
                                        sh->hier ? topk_region(R, (n_max + 7) / 8, CSA2_KEEP_BLOCKS) : 0));
    if (blocks_only) return CSA2_OK;
  } else if (mode == CSA2_REINDEX) {
    if (sh->hier) {
      const int nc = CSA2_KEEP_BLOCKS * 8;
      float* scores = bp.take<float>((size_t)R * nc);
      s = do_index_score(a->q_idx, a->head_w, &sh->k_idx, a->row_seq, sh->seq_len, sh->cand_blocks,
                         CSA2_KEEP_BLOCKS, R, n_max, scores, nullptr, st);
      if (s) return s;
      const size_t mark = bp.off;
      TopkWs tw = carve_topk(bp, R, nc, CSA2_TOPK);
      s = do_topk(scores, nc, nullptr, nullptr, 1, R, nc, CSA2_TOPK, sh->cand_blocks, CSA2_KEEP_BLOCKS,
                  sh->topk_idx, tw, w, st);
      if (s) return s;
      bp.off = align_up(mark + topk_region(R, nc, CSA2_TOPK));
    } else {
      float* scores = bp.take<float>((size_t)R * n_max);
      s = do_index_score(a->q_idx, a->head_w, &sh->k_idx, a->row_seq, sh->seq_len, nullptr, 0, R, n_max,
                         scores, nullptr, st);
      if (s) return s;
      const size_t mark = bp.off;
      TopkWs tw = carve_topk(bp, R, n_max, CSA2_TOPK);
      s = do_topk(scores, n_max, a->row_seq, sh->seq_len, 1, R, n_max, CSA2_TOPK, nullptr, 0, sh->topk_idx, tw,
                  w, st);
      if (s) return s;
      bp.off = align_up(mark + topk_region(R, n_max, CSA2_TOPK));
    }
  }
  AttnWs aw = carve_attn(bp, R, CSA2_TOPK);
  return do_attn(a->q, &sh->kv, a->row_seq, sh->seq_len, sh->topk_idx, CSA2_TOPK, a->swa_k, a->swa_v, a->S,
                 a->swa_start, a->swa_len, a->sm_scale, R, a->out, a->lse, aw, w, st);
}

}  // extern "C"
