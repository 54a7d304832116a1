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
#include <mutex>

#include "kernels.h"

using namespace csa2;

namespace {

constexpr size_t kAlign = 256;
// reserved control words at the start of every workspace (zeroed by
// csa2_workspace_init; no kernel of this version uses them)
constexpr size_t kCtrlBytes = kAlign;
constexpr int64_t kSelCapHost = 16384;        // values one Top-k block holds
constexpr int64_t kMaxTopkN = kSelCapHost * 64;  // two levels of maxima

#ifdef CSA2_TRACE
uint64_t* g_trace[3] = {nullptr, nullptr, nullptr};   // scan, top-k, attention
#define CSA2_SET_TRACE(args, which) (args).trace = g_trace[which]
#else
#define CSA2_SET_TRACE(args, which) (void)0
#endif

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Carves a workspace into aligned regions.  A sizing pass runs with a null
// base; a real carve records an overrun of `end` in `over`, which the entry
// points check before launching anything that uses the carved regions.
struct Bump {
  char* base;
  size_t off;
  size_t end = SIZE_MAX;
  bool over = false;
  template <class T>
  T* take(size_t n) {
    T* p = base ? (T*)(base + off) : nullptr;
    off = align_up(off + n * sizeof(T));
    if (off > end) over = true;
    return p;
  }
};

// Checks a cache descriptor: missing pointers give CSA2_ERR_NULL, negative
// sizes CSA2_ERR_SHAPE, a page size other than CSA2_PAGE CSA2_ERR_UNSUPPORTED.
csa2_status cache_status(const csa2_cache* c, bool need_scale) {
  if (!c || !c->data) return CSA2_ERR_NULL;
  if (need_scale && !c->scale) return CSA2_ERR_NULL;
  if (c->n_slots < 0) return CSA2_ERR_SHAPE;
  if (c->page_table) {
    if (c->max_pages <= 0) return CSA2_ERR_SHAPE;
    if (c->page_size != CSA2_PAGE) return CSA2_ERR_UNSUPPORTED;
  } else if (c->seq_stride < 0) {
    return CSA2_ERR_SHAPE;
  }
  return CSA2_OK;
}

csa2_status hip_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

// The indexer-key cache: bf16 keys (scale NULL, 16-byte aligned rows) or FP8
// keys (64 E4M3 codes per slot, 8-byte aligned rows, and a float32 scale per
// slot, 4-byte aligned).
csa2_status idx_cache_status(const csa2_cache* c) {
  if (const csa2_status cs = cache_status(c, false)) return cs;
  if (c->n_slots < 1 || c->n_slots > 0x7FFFFFFFll) return CSA2_ERR_SHAPE;
  if (c->scale && (((uintptr_t)c->scale & 3u) || ((uintptr_t)c->data & 7u))) return CSA2_ERR_SHAPE;
  if (!c->scale && ((uintptr_t)c->data & 15u)) return CSA2_ERR_SHAPE;
  return CSA2_OK;
}

// ---------------------------------------------------------------- scoring --

csa2_status do_index_score(const uint16_t* q_idx, const float* head_w, const csa2_cache* k_idx,
                           const int32_t* row_seq, const int32_t* seq_len, const int32_t* cand,
                           int32_t n_cand, int32_t R, int32_t n_max, float* scores, float* bmax, float* max64,
                           hipStream_t st) {
  IdxArgs a;
  a.q32 = (const uint32_t*)q_idx;
  a.head_w = head_w;
  a.kdata = (const uint4*)k_idx->data;
  a.kscale = (const float*)k_idx->scale;
  a.map = make_slot_map(*k_idx);
  a.row_seq = row_seq;
  a.seq_len = seq_len;
  a.cand = cand;
  a.n_cand = n_cand;
  a.R = R;
  a.n_max = n_max;
  a.steps_per_row = cand ? (int32_t)cdiv(n_cand, 8) : (int32_t)cdiv(n_max, 64);
  a.score_stride = cand ? (int64_t)n_cand * 8 : n_max;
  a.bmax_stride = cand ? (int64_t)n_cand : cdiv(n_max, 8);
  a.max64_stride = cdiv(n_max, 64);
  a.scores = scores;
  a.block_max = bmax;
  a.max64 = max64;
  a.row_list = nullptr;
  a.row_list_count = nullptr;
  CSA2_SET_TRACE(a, 0);
  return hip_status(launch_index_score(a, cand != nullptr, head_w != nullptr, bmax != nullptr, st));
}

// ------------------------------------------------------------------ top-k --

// Levels of maxima a Top-k over n values needs beyond level 0.
int topk_levels_needed(int64_t n) {
  if (n <= kSelCapHost) return 0;
  if (cdiv(n, 8) <= kSelCapHost) return 1;
  return 2;
}

struct TopkWs {
  float* lv1 = nullptr;
  float* lv2 = nullptr;
  uint32_t* seg_kth = nullptr;    // large-k path (segment thresholds, gathered values)
  uint32_t* seg_cnt = nullptr;
  uint32_t* seg_key = nullptr;
  int32_t* seg_pos = nullptr;
  uint32_t* desc_cnt = nullptr;   // split path (per-segment lists)
  uint32_t* desc_key = nullptr;
  int32_t* desc_pos = nullptr;
};

// Top-k spread over the CUs: k below 1024, rows of 2049 .. kDescMaxN values,
// a bounded number of rows (the lists take 256 KiB per row).
constexpr int kDescMaxRows = 256;
bool topk_desc_shape(int R, int64_t n_max, int k) {
  return k < 1024 && R <= kDescMaxRows && n_max > 2048 && n_max <= kDescMaxN;
}
// its top level for the longest row: 1 up to 16384 values, else 2
int desc_top_level(int64_t n_max) { return n_max <= 16384 ? 1 : 2; }

void carve_desc(Bump& bp, TopkWs& t, int R, int64_t n_max, int k) {
  if (!topk_desc_shape(R, n_max, k)) return;
  t.desc_cnt = bp.take<uint32_t>((size_t)R * kDescMaxSeg);
  t.desc_key = bp.take<uint32_t>((size_t)R * kDescMaxSeg * kDescCap);
  t.desc_pos = bp.take<int32_t>((size_t)R * kDescMaxSeg * kDescCap);
}

// Large k over long rows: per-segment gathers above one threshold per row.
bool topk_large_shape(int64_t n_max, int k) { return k >= 1024 && n_max >= kSelCapHost && n_max <= kTauMaxN; }

void carve_large(Bump& bp, TopkWs& t, int R, int64_t n_max, int k) {
  if (!topk_large_shape(n_max, k)) return;
  const size_t nseg = (size_t)cdiv(n_max, kSegLen);
  t.seg_kth = bp.take<uint32_t>((size_t)R * nseg);
  t.seg_cnt = bp.take<uint32_t>((size_t)R * nseg);
  t.seg_key = bp.take<uint32_t>((size_t)R * nseg * kSegLen);
  t.seg_pos = bp.take<int32_t>((size_t)R * nseg * kSegLen);
}

// Workspace for the levels of maxima a generic Top-k must build itself.
// (the split path needs its top level stored)
int topk_levels_built(int R, int64_t n_max, int k) {
  int need = topk_levels_needed(n_max);
  if (topk_desc_shape(R, n_max, k) && !topk_large_shape(n_max, k)) need = max(need, desc_top_level(n_max));
  return need;
}

TopkWs carve_topk(Bump& bp, int R, int64_t n_max, int k) {
  TopkWs t;
  const int need = topk_levels_built(R, n_max, k);
  if (need >= 1) t.lv1 = bp.take<float>((size_t)R * cdiv(n_max, 8));
  if (need >= 2) t.lv2 = bp.take<float>((size_t)R * cdiv(n_max, 64));
  carve_large(bp, t, R, n_max, k);
  carve_desc(bp, t, R, n_max, k);
  return t;
}

size_t topk_region(int R, int64_t n_max, int k) {
  Bump bp{nullptr, 0};
  carve_topk(bp, R, n_max, k);
  return bp.off;
}

TopkArgs topk_args(const float* lv0, int64_t stride, const int32_t* row_seq, const int32_t* n_valid, int n_div,
                   int R, int n_max, int k, int32_t* out) {
  TopkArgs a;
  a.lv[0] = lv0;
  a.lv[1] = a.lv[2] = nullptr;
  a.lv_stride[0] = stride;
  a.lv_stride[1] = cdiv(n_max, 8);
  a.lv_stride[2] = cdiv(n_max, 64);
  a.row_seq = row_seq;
  a.n_valid = n_valid;
  a.n_div = n_div;
  a.n_max = n_max;
  a.R = R;
  a.k = k;
  a.cand_blocks = nullptr;
  a.cand_stride = 0;
  a.out = out;
  a.out_stride = k;
  a.row_list = nullptr;
  a.row_list_count = nullptr;
  a.nseg = 0;
  a.seg_kth = nullptr;
  a.seg_cnt = nullptr;
  a.seg_key = nullptr;
  a.seg_pos = nullptr;
  return a;
}

// Builds the missing levels of maxima into the workspace, then selects.
// defer (optional): when the split path is taken, only its segment lists are
// built here and *defer receives the arguments of its final selection, which
// the attention launch that follows takes over (defer->out stays null
// otherwise).
// The path a Top-k takes, chosen (and its arguments completed, building
// missing levels of maxima first) by plan_topk, launched by launch_planned.
enum TopkPath { kPathOneBlock, kPathDesc, kPathLarge, kPathError };

TopkPath plan_topk(TopkArgs& a, const TopkWs& tw, hipStream_t st) {
  const int need = topk_levels_built(a.R, a.n_max, a.k);
  for (int l = 1; l <= need; ++l) {
    if (a.lv[l]) continue;
    if (!((l == 1) ? tw.lv1 : tw.lv2)) break;     // (a caller's levels only)
    float* dst = (l == 1) ? tw.lv1 : tw.lv2;
    MaximaArgs m;
    m.in = a.lv[l - 1];
    m.in_stride = a.lv_stride[l - 1];
    m.out = dst;
    m.out_stride = a.lv_stride[l];
    m.n_out_max = a.lv_stride[l];
    m.div_in = (l == 1) ? 1 : 8;
    m.row_seq = a.row_seq;
    m.n_valid = a.n_valid;
    m.n_div = a.n_div;
    m.n_max = a.n_max;
    m.R = a.R;
    hipError_t e = launch_maxima(m, st);
    if (e != hipSuccess) return kPathError;
    a.lv[l] = dst;
  }
  CSA2_SET_TRACE(a, 1);
  if (tw.seg_cnt && a.lv[1] && !a.cand_blocks && !a.row_list && topk_large_shape(a.n_max, a.k)) {
    a.seg_kth = tw.seg_kth;
    a.nseg = (int32_t)cdiv(a.n_max, kSegLen);
    a.seg_cnt = tw.seg_cnt;
    a.seg_key = tw.seg_key;
    a.seg_pos = tw.seg_pos;
    return kPathLarge;
  }
  if (tw.desc_cnt && !a.row_list && topk_desc_shape(a.R, a.n_max, a.k) && a.lv[1] &&
      (desc_top_level(a.n_max) < 2 || a.lv[2])) {
    a.nseg = (int32_t)cdiv(a.n_max, desc_seg_len(a.n_max));
    a.seg_cnt = tw.desc_cnt;
    a.seg_key = tw.desc_key;
    a.seg_pos = tw.desc_pos;
    return kPathDesc;
  }
  return kPathOneBlock;
}

// defer: the split path's final selection is left to the caller (*defer).
csa2_status launch_planned(const TopkArgs& a, TopkPath p, hipStream_t st, TopkArgs* defer = nullptr) {
  switch (p) {
    case kPathLarge: return hip_status(launch_topk_large(a, st));
    case kPathDesc:
      if (defer) {
        *defer = a;
        return hip_status(launch_desc_seg(a, st));
      }
      return hip_status(launch_topk_desc(a, st));
    case kPathOneBlock: return hip_status(launch_topk(a, st));
    default: return CSA2_ERR_HIP;
  }
}

csa2_status run_topk(TopkArgs a, const TopkWs& tw, hipStream_t st, TopkArgs* defer = nullptr) {
  const TopkPath p = plan_topk(a, tw, st);
  return launch_planned(a, p, st, defer);
}

// -------------------------------------------------------------- attention --

struct AttnWs {
  float* part_o;
  float* part_ml;
  int n_blocks, cpb;
};

AttnWs carve_attn(Bump& bp, int R, int n_layers, int k) {
  AttnWs w;
  w.n_blocks = attn_blocks(k, R * n_layers, &w.cpb);
  if (w.n_blocks > 1) {
    w.part_o = bp.take<float>((size_t)n_layers * R * w.n_blocks * 16 * 512);
    w.part_ml = bp.take<float>((size_t)n_layers * R * w.n_blocks * 32);
  } else {
    w.part_o = w.part_ml = nullptr;
  }
  return w;
}

size_t attn_region(int R, int n_layers, int k) {
  Bump bp{nullptr, 0};
  carve_attn(bp, R, n_layers, k);
  return bp.off;
}

// The attention's partials depend on k only through its number of 128-key
// main steps, and not monotonically (fewer steps can take more blocks per
// row-layer): the largest region over k = 1 .. kmax.
size_t attn_region_any_k(int R, int n_layers, int kmax) {
  size_t m = 0;
  for (int steps = 1; (steps - 1) * 128 < kmax; ++steps) m = std::max(m, attn_region(R, n_layers, std::min(kmax, 128 * steps)));
  return m;
}

struct AttnLayerIn {
  const uint16_t *q, *swa_k, *swa_v;
  int32_t S;
  const int32_t *swa_start, *swa_len;
  float *out, *lse;
  float sm_scale;
  int32_t swa_shared;
};

// fin (optional): the split Top-k's final selection, still to run (it
// writes idx); the attention launch takes it over or launches it first.
csa2_status do_attn(const AttnLayerIn* L, int n_layers, const csa2_cache* kv, const int32_t* row_seq,
                    const int32_t* seq_len, const int32_t* idx, int32_t k, int32_t R,
                    const AttnWs& aw, char* ws, hipStream_t st, const TopkArgs* fin = nullptr,
                    const TopkArgs* cand = nullptr) {
  AttnArgs a;
  a.sel = fin ? *fin : TopkArgs{};
  if (!fin) a.sel.out = nullptr;
  for (int i = 0; i < n_layers; ++i) {
    a.layer[i].q = (const uint4*)L[i].q;
    a.layer[i].swa_k = (const uint4*)L[i].swa_k;
    a.layer[i].swa_v = (const uint4*)L[i].swa_v;
    a.layer[i].swa_start = L[i].swa_start;
    a.layer[i].swa_len = L[i].swa_len;
    a.layer[i].out = L[i].out;
    a.layer[i].lse = L[i].lse;
    a.layer[i].S = L[i].S;
    a.layer[i].sm_scale = L[i].sm_scale;
    a.layer[i].swa_shared = L[i].swa_shared ? 1 : 0;
  }
  a.n_layers = n_layers;
  a.kv = (const uint8_t*)kv->data;
  a.kv_scale = kv->scale;
  a.map = make_slot_map(*kv);
  a.row_seq = row_seq;
  a.seq_len = seq_len;
  a.idx = idx;
  a.k = k;
  a.R = R;
  a.n_blocks = aw.n_blocks;
  a.steps_per_block = aw.cpb;
  a.part_o = aw.part_o;
  a.part_ml = aw.part_ml;
  CSA2_SET_TRACE(a, 2);
  return hip_status(launch_attn(a, st, cand));
}

bool attn_layer_ok(const csa2_layer_args* a) {
  return a->q && a->swa_k && a->swa_v && a->swa_start && a->swa_len && a->out && a->S >= 0;
}

AttnLayerIn layer_in(const csa2_layer_args* a) {
  return AttnLayerIn{a->q, a->swa_k, a->swa_v, a->S, a->swa_start, a->swa_len, a->out, a->lse, a->sm_scale,
                     a->swa_shared};
}

// ------------------------------------------------------- layer index part --

// Rows of a prefill chunk (all rows score one sequence) that are many enough
// for the matrix-core indexer; the caller also requires a single sequence.
bool prefill_shape(csa2_mode mode, int R, int n_max, int hier) {
  return (mode == CSA2_FULL || mode == CSA2_REINDEX) && !hier && R >= kPrefMinRows && n_max >= kPrefMinN &&
         n_max <= kPrefMaxN;
}

struct PrefWs {
  float* gmax;
  float* kmax_part;
  float* theta;
  uint32_t* cand_count;
  int32_t* cand;
  int32_t* fb_list;
  uint32_t* fb_count;
};

PrefWs carve_prefill(Bump& bp, int R, int n_max) {
  PrefWs p;
  p.gmax = bp.take<float>((size_t)R * cdiv(n_max, 64));
  p.kmax_part = bp.take<float>((size_t)cdiv(n_max, 2048));
  p.theta = bp.take<float>((size_t)R);
  p.cand_count = bp.take<uint32_t>((size_t)R);
  p.cand = bp.take<int32_t>((size_t)R * kPrefCap);
  p.fb_list = bp.take<int32_t>((size_t)R);
  p.fb_count = bp.take<uint32_t>(1);
  return p;
}

// Workspace of the indexer part of a layer in `mode` (scores, maxima, Top-k levels).
size_t index_region(csa2_mode mode, int R, int n_max, int hier) {
  Bump bp{nullptr, 0};
  if (mode == CSA2_FULL || (mode == CSA2_REINDEX && !hier)) {
    bp.take<float>((size_t)R * n_max);
    bp.take<float>((size_t)R * cdiv(n_max, 8));
    bp.take<float>((size_t)R * cdiv(n_max, 64));
    if (prefill_shape(mode, R, n_max, hier)) carve_prefill(bp, R, n_max);
    TopkWs t;
    carve_desc(bp, t, R, n_max, CSA2_TOPK);
    if (mode == CSA2_FULL && hier) carve_large(bp, t, R, cdiv(n_max, 8), CSA2_KEEP_BLOCKS);
  } else if (mode == CSA2_REINDEX) {
    bp.take<float>((size_t)R * CSA2_KEEP_BLOCKS * 8);
    bp.take<float>((size_t)R * CSA2_KEEP_BLOCKS);
    TopkWs t;
    carve_desc(bp, t, R, CSA2_KEEP_BLOCKS * 8, CSA2_TOPK);
  }
  return bp.off;
}

// Scoring + selection of a Full or Reindex layer; leaves the Top-512 in
// shared->topk_idx (and the candidate blocks of a hierarchical Full layer in
// shared->cand_blocks).
// cand_defer: when given, a hierarchical Full layer's candidate build may
// leave its final selection to the caller (*cand_defer, out non-null), its
// first launch paired with the Top-512's.
csa2_status run_index(csa2_mode mode, const csa2_layer_args* a, const csa2_shared* sh, Bump& bp, bool blocks_only,
                      hipStream_t st, TopkArgs* defer, TopkArgs* cand_defer = nullptr) {
  const int R = a->R, n_max = sh->n_max;
  csa2_status s;
  if (mode == CSA2_FULL || (mode == CSA2_REINDEX && !sh->hier)) {
    float* scores = bp.take<float>((size_t)R * n_max);
    float* bmax = bp.take<float>((size_t)R * cdiv(n_max, 8));
    float* m64 = bp.take<float>((size_t)R * cdiv(n_max, 64));
    // every row reads the same slots: one sequence, or sequences that share
    // them (contiguous caches with seq_stride 0: a chunk whose rows see
    // different lengths of one context)
    const bool one_context = sh->B == 1 || (!sh->kv.page_table && sh->kv.seq_stride == 0 &&
                                            !sh->k_idx.page_table && sh->k_idx.seq_stride == 0);
    if (one_context && a->row_seq && !blocks_only && !sh->k_idx.scale && prefill_shape(mode, R, n_max, sh->hier)) {
      // prefill chunk: matrix-core indexer with exact selection; the rows it
      // lists (too many candidates) take the exact scan and Top-k below
      const PrefWs pw = carve_prefill(bp, R, n_max);
      if (bp.over) return CSA2_ERR_WORKSPACE;
      PrefArgs p;
      p.q32 = (const uint32_t*)a->q_idx;
      p.head_w = a->head_w;
      p.kdata = (const uint4*)sh->k_idx.data;
      p.map = make_slot_map(sh->k_idx);
      p.seq_len = sh->seq_len;
      p.row_seq = a->row_seq;
      p.R = R;
      p.n_max = n_max;
      p.k = CSA2_TOPK;
      p.gmax = pw.gmax;
      p.gmax_stride = cdiv(n_max, 64);
      p.kmax_part = pw.kmax_part;
      p.theta = pw.theta;
      p.cand_count = pw.cand_count;
      p.cand = pw.cand;
      p.cap = kPrefCap;
      p.fb_list = pw.fb_list;
      p.fb_count = pw.fb_count;
      p.out = sh->topk_idx;
      // the approximate scores in bf16 share the memory of the exact scores,
      // which only the listed rows' exact scan writes, after the selection
      p.sb = (uint16_t*)scores;
      p.sb_stride = cdiv(n_max, 64) * 64;     // whole groups of 64 per row (<= 2 n_max: fits)
      hipError_t e = launch_prefill_index(p, a->head_w != nullptr, st);
      if (e != hipSuccess) return CSA2_ERR_HIP;
      IdxArgs ia;
      ia.q32 = p.q32;
      ia.head_w = a->head_w;
      ia.kdata = p.kdata;
      ia.kscale = nullptr;            // (the matrix-core path runs on bf16 keys only)
      ia.map = p.map;
      ia.row_seq = a->row_seq;
      ia.seq_len = sh->seq_len;
      ia.cand = nullptr;
      ia.n_cand = 0;
      ia.R = R;
      ia.n_max = n_max;
      ia.steps_per_row = (int32_t)cdiv(n_max, 64);
      ia.score_stride = n_max;
      ia.bmax_stride = cdiv(n_max, 8);
      ia.max64_stride = cdiv(n_max, 64);
      ia.scores = scores;
      ia.block_max = bmax;
      ia.max64 = m64;
      ia.row_list = pw.fb_list;
      ia.row_list_count = pw.fb_count;
      CSA2_SET_TRACE(ia, 0);
      e = launch_index_score(ia, false, a->head_w != nullptr, true, st);
      if (e != hipSuccess) return CSA2_ERR_HIP;
      TopkArgs t = topk_args(scores, n_max, a->row_seq, sh->seq_len, 1, R, n_max, CSA2_TOPK, sh->topk_idx);
      t.lv[1] = bmax;
      t.lv[2] = m64;
      t.row_list = pw.fb_list;
      t.row_list_count = pw.fb_count;
      return run_topk(t, TopkWs{}, st);
    }
    TopkWs dw, tw;
    carve_desc(bp, dw, R, n_max, CSA2_TOPK);
    const int nb = (int)cdiv(n_max, 8);
    if (mode == CSA2_FULL && sh->hier) carve_large(bp, tw, R, nb, CSA2_KEEP_BLOCKS);
    if (bp.over) return CSA2_ERR_WORKSPACE;
    s = do_index_score(a->q_idx, a->head_w, &sh->k_idx, a->row_seq, sh->seq_len, nullptr, 0, R, n_max, scores,
                       bmax, m64, st);
    if (s) return s;
    TopkArgs t512{}, tc{};
    TopkPath p512 = kPathError, pc = kPathError;
    const bool cands = mode == CSA2_FULL && sh->hier;
    if (!blocks_only) {
      t512 = topk_args(scores, n_max, a->row_seq, sh->seq_len, 1, R, n_max, CSA2_TOPK, sh->topk_idx);
      t512.lv[1] = bmax;
      t512.lv[2] = m64;
      p512 = plan_topk(t512, dw, st);
      if (p512 == kPathError) return CSA2_ERR_HIP;
    }
    if (cands) {
      tc = topk_args(bmax, nb, a->row_seq, sh->seq_len, 8, R, nb, CSA2_KEEP_BLOCKS, sh->cand_blocks);
      tc.lv[1] = m64;     // maxima of 8 block maxima
      tc.lv_stride[1] = cdiv(n_max, 64);
      pc = plan_topk(tc, tw, st);
      if (pc == kPathError) return CSA2_ERR_HIP;
    }
    // the Top-512 and the candidate build read only the scan's outputs: their
    // first launches share one, and the candidates' final selection joins the
    // merge after the attention (the next group reads the candidates)
    if (!blocks_only && cands && cand_defer && pc == kPathLarge) {
      if (p512 == kPathDesc && defer && tc.n_max <= kSelCapHost) {
        *defer = t512;
        *cand_defer = tc;
        return hip_status(launch_desc_seg_tau(t512, tc, st));
      }
      if (p512 == kPathOneBlock && tc.n_max > kSelCapHost) {
        *cand_defer = tc;
        return hip_status(launch_topk_kth_gather(t512, tc, st));
      }
    }
    if (!blocks_only) {
      s = launch_planned(t512, p512, st, defer);
      if (s) return s;
    }
    if (cands) {
      s = launch_planned(tc, pc, st);
      if (s) return s;
    }
    return CSA2_OK;
  }
  // Reindex over the candidate blocks of the last (hierarchical) Full layer
  const int nc = CSA2_KEEP_BLOCKS * 8;
  float* scores = bp.take<float>((size_t)R * nc);
  float* cmax = bp.take<float>((size_t)R * CSA2_KEEP_BLOCKS);     // maxima of the candidate blocks
  TopkWs dw;
  carve_desc(bp, dw, R, nc, CSA2_TOPK);
  if (bp.over) return CSA2_ERR_WORKSPACE;
  s = do_index_score(a->q_idx, a->head_w, &sh->k_idx, a->row_seq, sh->seq_len, sh->cand_blocks, CSA2_KEEP_BLOCKS,
                     R, n_max, scores, cmax, nullptr, st);
  if (s) return s;
  TopkArgs t = topk_args(scores, nc, nullptr, nullptr, 1, R, nc, CSA2_TOPK, sh->topk_idx);
  t.lv[1] = cmax;
  t.cand_blocks = sh->cand_blocks;
  t.cand_stride = CSA2_KEEP_BLOCKS;
  return run_topk(t, dw, st, defer);
}

csa2_status check_shared(const csa2_shared* sh, int R) {
  if (!sh) return CSA2_ERR_NULL;
  if (R < 1 || R > CSA2_MAX_ROWS || sh->n_max < 0 || sh->B < 1) return CSA2_ERR_SHAPE;
  if (sh->n_max > kMaxTopkN) return CSA2_ERR_UNSUPPORTED;
  if (!sh->seq_len || !sh->topk_idx) return CSA2_ERR_NULL;
  if (const csa2_status cs = cache_status(&sh->kv, true)) return cs;
  if (sh->kv.n_slots > 0x7FFFFFFFll) return CSA2_ERR_UNSUPPORTED;
  return CSA2_OK;
}

// Scratch of csa2_group_step_noalloc: a static device array (zero when the
// code object is loaded; each GPU holds its own copy until the process ends).
// In host code `scratch` names a host-side stand-in: kernels get the device
// address that hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = CSA2_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
csa2_status device_scratch(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return CSA2_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return CSA2_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSA2_ERR_HIP;
    g_scratch_ptr[dev] = (char*)p;
  }
  *out = g_scratch_ptr[dev];
  return CSA2_OK;
}

}  // namespace

extern "C" {

#ifdef CSA2_TRACE
// Tuning builds only: device buffers (2048 uint64 each) that receive phase
// timestamps and per-block spans of the scan (0), Top-k (1) and attention (2)
// kernels; NULL stops recording.
void csa2_trace_set(int which, uint64_t* dev_buf) {
  if (which >= 0 && which < 3) g_trace[which] = dev_buf;
}
#endif

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

const char* csa2_version(void) { return "csa2-gfx950 0.2"; }

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
  return kCtrlBytes + attn_region_any_k(R, 1, CSA2_TOPK);
}

csa2_status csa2_index_score(const uint16_t* q_idx, const float* head_w, const csa2_cache* k_idx,
                             const int32_t* row_seq, const int32_t* seq_len, const int32_t* cand_blocks,
                             int32_t n_cand, int32_t R, int32_t n_max, float* scores, float* block_max,
                             hipStream_t stream) {
  if (!q_idx || !k_idx || !seq_len || !scores) return CSA2_ERR_NULL;
  if (const csa2_status cs = idx_cache_status(k_idx)) return cs;
  if (R < 1 || R > CSA2_MAX_ROWS || n_max < 0) return CSA2_ERR_SHAPE;
  if (cand_blocks) {
    if (n_cand < 1 || n_cand > CSA2_KEEP_BLOCKS) return CSA2_ERR_SHAPE;
    if (block_max) return CSA2_ERR_UNSUPPORTED;
  }
  if ((int64_t)R * (cand_blocks ? cdiv(n_cand, 8) : cdiv(n_max, 64)) > 0xFFFFFFFFll) return CSA2_ERR_SHAPE;
  return do_index_score(q_idx, head_w, k_idx, row_seq, seq_len, cand_blocks, n_cand, R, n_max, scores, block_max,
                        nullptr, stream);
}

csa2_status csa2_topk(const float* scores, int64_t row_stride, const int32_t* row_seq,
                      const int32_t* n_valid, int32_t R, int32_t n_max, int32_t k,
                      const int32_t* cand_blocks, int32_t* idx, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  if (!scores || !idx) return CSA2_ERR_NULL;
  if (R < 1 || R > CSA2_MAX_ROWS || n_max < 0 || k < 1 || k > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  if (row_stride < n_max) return CSA2_ERR_SHAPE;
  if (n_max > kMaxTopkN) return CSA2_ERR_UNSUPPORTED;
  if (cand_blocks && n_max % 8) return CSA2_ERR_SHAPE;
  if (cand_blocks && n_max > 8 * CSA2_KEEP_BLOCKS) return CSA2_ERR_UNSUPPORTED;
  if (!ws) return CSA2_ERR_WORKSPACE;
  if (ws_bytes < csa2_topk_workspace_bytes(R, n_max, k)) return CSA2_ERR_WORKSPACE;
  Bump bp{(char*)ws, kCtrlBytes, ws_bytes};
  const TopkWs tw = carve_topk(bp, R, n_max, k);
  if (bp.over) return CSA2_ERR_WORKSPACE;
  TopkArgs t = topk_args(scores, row_stride, row_seq, n_valid, 1, R, n_max, k, idx);
  t.cand_blocks = cand_blocks;
  t.cand_stride = n_max / 8;
  return run_topk(t, tw, stream);
}

csa2_status csa2_hier_candidates(const float* block_max, const int32_t* row_seq, const int32_t* seq_len,
                                 int32_t R, int32_t n_max, int32_t keep, int32_t* cand_blocks, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  if (!block_max || !seq_len || !cand_blocks) return CSA2_ERR_NULL;
  if (R < 1 || R > CSA2_MAX_ROWS || n_max < 0 || keep < 1 || keep > CSA2_MAX_K) return CSA2_ERR_SHAPE;
  if (n_max > kMaxTopkN) return CSA2_ERR_UNSUPPORTED;
  const int nb = (int)cdiv(n_max, 8);
  if (!ws) return CSA2_ERR_WORKSPACE;
  if (ws_bytes < csa2_topk_workspace_bytes(R, nb, keep)) return CSA2_ERR_WORKSPACE;
  Bump bp{(char*)ws, kCtrlBytes, ws_bytes};
  const TopkWs tw = carve_topk(bp, R, nb, keep);
  if (bp.over) return CSA2_ERR_WORKSPACE;
  return run_topk(topk_args(block_max, nb, row_seq, seq_len, 8, R, nb, keep, cand_blocks), tw, stream);
}

csa2_status csa2_fp4_sparse_attn(const uint16_t* q, const csa2_cache* kv, const int32_t* row_seq,
                                 const int32_t* seq_len, const int32_t* idx, int32_t k, const uint16_t* swa_k,
                                 const uint16_t* swa_v, int32_t S, const int32_t* swa_start,
                                 const int32_t* swa_len, float sm_scale, int32_t R, float* out, float* lse,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!q || !kv || !seq_len || !idx || !swa_k || !swa_v || !swa_start || !swa_len || !out)
    return CSA2_ERR_NULL;
  if (const csa2_status cs = cache_status(kv, true)) return cs;
  if (R < 1 || R > CSA2_MAX_ROWS || k < 1 || k > CSA2_TOPK || S < 0) return CSA2_ERR_SHAPE;
  if (kv->n_slots > 0x7FFFFFFFll) return CSA2_ERR_UNSUPPORTED;
  if (!ws) return CSA2_ERR_WORKSPACE;
  if (ws_bytes < csa2_attn_workspace_bytes(R)) return CSA2_ERR_WORKSPACE;
  Bump bp{(char*)ws, kCtrlBytes, ws_bytes};
  const AttnWs aw = carve_attn(bp, R, 1, k);
  if (bp.over) return CSA2_ERR_WORKSPACE;
  const AttnLayerIn L{q, swa_k, swa_v, S, swa_start, swa_len, out, lse, sm_scale, 0};
  return do_attn(&L, 1, kv, row_seq, seq_len, idx, k, R, aw, (char*)ws, stream);
}

csa2_status csa2_fp4_quantize(const float* x, int64_t n, const int64_t* dst_slot, uint8_t* fp4,
                              uint8_t* scale, int64_t n_slots, hipStream_t stream) {
  if (n > 0 && (!x || !fp4 || !scale)) return CSA2_ERR_NULL;
  if (n < 0 || n_slots < 0) return CSA2_ERR_SHAPE;
  if (!dst_slot && n > n_slots) return CSA2_ERR_SHAPE;
  if (n / 4 >= (int64_t)0x7FFFFFFF) return CSA2_ERR_SHAPE;
  return hip_status(launch_quant(x, n, dst_slot, fp4, scale, n_slots, stream));
}

csa2_status csa2_fp8_key_quantize(const uint16_t* k, int64_t n, const int64_t* dst_slot, uint8_t* codes,
                                  float* scale, int64_t n_slots, hipStream_t stream) {
  if (n > 0 && (!k || !codes || !scale)) return CSA2_ERR_NULL;
  if (n < 0 || n_slots < 0) return CSA2_ERR_SHAPE;
  if (!dst_slot && n > n_slots) return CSA2_ERR_SHAPE;
  if (n / 4 >= (int64_t)0x7FFFFFFF) return CSA2_ERR_SHAPE;
  return hip_status(launch_fp8_key_quant(k, n, dst_slot, codes, scale, n_slots, stream));
}

size_t csa2_group_workspace_bytes(csa2_mode first_mode, int32_t n_layers, int32_t R, int32_t n_max, int32_t hier) {
  if (R < 0 || n_max < 0 || n_layers < 1 || n_layers > CSA2_MAX_GROUP_LAYERS) return 0;
  size_t off = kCtrlBytes;
  off = align_up(off + index_region(first_mode, R, n_max, hier));
  // a hierarchical Full layer that only builds candidates leaves n_layers - 1
  // attended layers, which can need more partials than n_layers
  size_t attn = attn_region(R, n_layers, CSA2_TOPK);
  if (first_mode == CSA2_FULL && hier && n_layers > 1) attn = std::max(attn, attn_region(R, n_layers - 1, CSA2_TOPK));
  off = align_up(off + attn);
  return off;
}

size_t csa2_workspace_bytes(csa2_mode mode, int32_t R, int32_t n_max, int32_t hier) {
  return csa2_group_workspace_bytes(mode, 1, R, n_max, hier);
}

csa2_status csa2_group_step(csa2_mode first_mode, int32_t n_layers, const csa2_layer_args* layers,
                            const csa2_shared* sh, void* ws, size_t ws_bytes, hipStream_t st) {
  if (!layers) return CSA2_ERR_NULL;
  if (first_mode != CSA2_FULL && first_mode != CSA2_REINDEX && first_mode != CSA2_REUSE) return CSA2_ERR_UNSUPPORTED;
  if (n_layers < 1 || n_layers > CSA2_MAX_GROUP_LAYERS) return CSA2_ERR_SHAPE;
  const int R = layers[0].R;
  csa2_status s = check_shared(sh, R);
  if (s) return s;
  const bool blocks_only = first_mode == CSA2_FULL && sh->hier && layers[0].blocks_only;
  // attended layers: all, except a Full layer that only builds candidates
  const int a0 = blocks_only ? 1 : 0;
  for (int i = 0; i < n_layers; ++i) {
    if (layers[i].R != R || layers[i].row_seq != layers[0].row_seq) return CSA2_ERR_SHAPE;
    if (i >= a0 && !attn_layer_ok(&layers[i])) return CSA2_ERR_NULL;
  }
  if ((int64_t)R * n_layers > CSA2_MAX_ROWS) return CSA2_ERR_SHAPE;
  if (first_mode != CSA2_REUSE) {
    if (!layers[0].q_idx) return CSA2_ERR_NULL;
    if (const csa2_status cs = idx_cache_status(&sh->k_idx)) return cs;
    if (sh->hier && !sh->cand_blocks) return CSA2_ERR_NULL;
  }
  if (!ws) return CSA2_ERR_WORKSPACE;
  if (ws_bytes < csa2_group_workspace_bytes(first_mode, n_layers, R, sh->n_max, sh->hier)) return CSA2_ERR_WORKSPACE;

  // workspace: the indexer part's region, then the attention's partials;
  // both carved (and checked against ws_bytes) before anything is launched
  char* w = (char*)ws;
  Bump bp{w, kCtrlBytes, ws_bytes};
  const size_t index_off = bp.off;
  if (first_mode != CSA2_REUSE) bp.off = align_up(bp.off + index_region(first_mode, R, sh->n_max, sh->hier));
  const size_t index_end = bp.off;
  if (index_end > ws_bytes) return CSA2_ERR_WORKSPACE;
  const int na = n_layers - a0;
  const AttnWs aw = na > 0 ? carve_attn(bp, R, na, CSA2_TOPK) : AttnWs{nullptr, nullptr, 0, 0};
  if (bp.over) return CSA2_ERR_WORKSPACE;
  // the split Top-512's final selection may be left to the attention launch
  TopkArgs fin{}, cfin{};
  fin.out = nullptr;
  cfin.out = nullptr;
  if (first_mode != CSA2_REUSE) {
    Bump ib{w, index_off, index_end};
    s = run_index(first_mode, &layers[0], sh, ib, blocks_only, st, na > 0 ? &fin : nullptr,
                  na > 0 ? &cfin : nullptr);
    if (s) return s;
  }
  if (na == 0) return CSA2_OK;
  AttnLayerIn L[CSA2_MAX_GROUP_LAYERS];
  for (int i = 0; i < na; ++i) L[i] = layer_in(&layers[a0 + i]);
  return do_attn(L, na, &sh->kv, layers[0].row_seq, sh->seq_len, sh->topk_idx, CSA2_TOPK, R, aw, w, st,
                 fin.out ? &fin : nullptr, cfin.out ? &cfin : nullptr);
}

csa2_status csa2_layer_step(csa2_mode mode, const csa2_layer_args* a, const csa2_shared* sh, void* ws,
                            size_t ws_bytes, hipStream_t st) {
  if (!a || !sh) return CSA2_ERR_NULL;
  return csa2_group_step(mode, 1, a, sh, ws, ws_bytes, st);
}

csa2_status csa2_group_step_noalloc(csa2_mode first_mode, int32_t n_layers, const csa2_layer_args* layers,
                                    const csa2_shared* sh, hipStream_t st) {
  if (!layers || !sh) return CSA2_ERR_NULL;
  if (n_layers < 1 || n_layers > CSA2_MAX_GROUP_LAYERS) return CSA2_ERR_SHAPE;
  if (layers[0].R < 0 || sh->n_max < 0) return CSA2_ERR_SHAPE;
  // the static scratch stands in for the caller's workspace: a call needing
  // more is refused before anything touches the device
  const size_t need = csa2_group_workspace_bytes(first_mode, n_layers, layers[0].R, sh->n_max, sh->hier);
  if (need > kScratchBytes) return CSA2_ERR_WORKSPACE;
  char* ptr = nullptr;
  if (const csa2_status s = device_scratch(&ptr)) return s;
  return csa2_group_step(first_mode, n_layers, layers, sh, ptr, kScratchBytes, st);
}

}  // extern "C"
