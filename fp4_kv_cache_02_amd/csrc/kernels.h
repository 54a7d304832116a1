// Kernel argument blocks and launch entry points shared by the kernels and
// the host dispatcher.
#pragma once
#include "common.h"

namespace csa2 {

// (every optional pointer defaults to null: a new field left unset by a caller
// must select no variant)
struct IdxArgs {
  const uint32_t* q32 = nullptr;        // [R][4][32] bf16 pairs
  const float* head_w = nullptr;        // [R][4] or null
  const uint4* kdata = nullptr;         // bf16 keys: [n_slots][8] 16-byte chunks; FP8 keys: [n_slots][4] (64 codes)
  const float* kscale = nullptr;        // FP8 keys: [n_slots] scales; null for bf16 keys
  SlotMap map = {};
  const int32_t* row_seq = nullptr;
  const int32_t* seq_len = nullptr;
  const int32_t* cand = nullptr;        // [R][n_cand] or null
  int32_t n_cand = 0;
  int32_t R = 0;
  int32_t n_max = 0;
  int32_t steps_per_row = 0;            // 64-position steps: ceil(n_max/64) (scan) or ceil(n_cand/8) (Reindex)
  int64_t score_stride = 0;
  int64_t bmax_stride = 0;
  int64_t max64_stride = 0;
  float* scores = nullptr;
  float* block_max = nullptr;           // [R][ceil(n_max/8)] maxima of 8 positions (scan, optional)
  float* max64 = nullptr;               // [R][ceil(n_max/64)] maxima of 64 positions (scan, optional)
  const int32_t* row_list = nullptr;    // optional: score only rows row_list[0 .. *row_list_count)
  const uint32_t* row_list_count = nullptr;
#ifdef CSA2_TRACE
  uint64_t* trace = nullptr;
#endif
};

// Top-k over level 0 of a tree of maxima (level l+1 = maxima of 8 of level l).
struct TopkArgs {
  const float* lv[3];         // level arrays (lv[1], lv[2] may be null when not needed)
  int64_t lv_stride[3];
  const int32_t* row_seq;
  const int32_t* n_valid;     // per sequence, or null (n = n_max)
  int32_t n_div;              // level-0 count = ceil(n_valid / n_div)
  int32_t n_max;              // level-0 count cap
  int32_t R;
  int32_t k;
  const int32_t* cand_blocks; // optional index -> position map of the output
  int32_t cand_stride;
  int32_t* out;
  int32_t out_stride;
  const int32_t* row_list;    // optional: select only rows row_list[0 .. *row_list_count)
  const uint32_t* row_list_count;
  // segmented paths: per (row, segment) thresholds (rows of more than 16384
  // values) and lists of gathered values
  uint32_t* seg_kth;          // [R][nseg] or null
  int32_t nseg;
  uint32_t* seg_cnt;          // [R][nseg]: values >= tau gathered per segment
  uint32_t* seg_key;          // [R][nseg][kSegLen]: their keys, in index order
  int32_t* seg_pos;           // [R][nseg][kSegLen]: their indices
  CSA2_TRACE_ARG
};

constexpr int kSegLen = 8192;             // level-0 values per segment of the large-k path
constexpr int kTauMaxN = 131072;          // level-0 values per row it handles (8 x 16384)
// Top-k spread over the CUs (k below 1024): rows of at most kDescMaxN values,
// at most 32 segments per row, kDescCap listed values per segment
constexpr int kDescMaxN = 131072;
constexpr int kDescCap = 1024;
constexpr int kDescMaxSeg = 32;
inline int desc_seg_len(int64_t n_max) { return n_max <= 16 * 1024 ? 1024 : 4096; }

// Prefill-chunk indexer on MFMA: every query row sees the positions of one
// sequence (sequence 0).
struct PrefArgs {
  const uint32_t* q32 = nullptr;        // [R][4][32] bf16 pairs
  const float* head_w = nullptr;        // [R][4] or null
  const uint4* kdata = nullptr;         // indexer keys
  SlotMap map = {};
  const int32_t* seq_len = nullptr;     // visible positions of row r: seq_len[row_seq[r]] (row_seq null: seq_len[0])
  const int32_t* row_seq = nullptr;     // every row reads the same slots (one sequence, or sequences sharing them)
  int32_t R = 0;
  int32_t n_max = 0;
  int32_t k = 0;
  float* gmax = nullptr;                // [R][ceil(n_max/64)] maxima of the approximate scores per 64 positions
  int64_t gmax_stride = 0;
  float* kmax_part = nullptr;           // [ceil(n_max/2048)] largest |key element| per chunk of 2048 positions
  float* theta = nullptr;               // [R] candidate threshold
  uint16_t* sb = nullptr;               // [R][sb_stride] approximate scores rounded to bf16 (NaN: not visible)
  int64_t sb_stride = 0;                // a multiple of 64, >= n_max
  uint32_t* cand_count = nullptr;       // [R]
  int32_t* cand = nullptr;              // [R][cap] candidate positions
  int32_t cap = 0;
  int32_t* fb_list = nullptr;           // [R] rows whose candidates overflowed
  uint32_t* fb_count = nullptr;         // [1]
  int32_t* out = nullptr;               // [R][k] Top-k positions
};

struct MaximaArgs {
  const float* in;
  int64_t in_stride;
  float* out;
  int64_t out_stride;
  int64_t n_out_max;          // groups per row at the largest row
  int64_t div_in;             // this input level holds ceil(n0 / div_in) values
  const int32_t* row_seq;
  const int32_t* n_valid;
  int32_t n_div;
  int32_t n_max;              // level-0 count cap
  int32_t R;
};

constexpr int kMaxAttnLayers = CSA2_MAX_GROUP_LAYERS;
constexpr int kMaxAttnBlocks = 8;   // 4 main steps + the window step in four quarters

struct AttnLayer {
  const uint4* q;               // [R][16][64] uint4 (8 bf16 each)
  const uint4* swa_k;           // [B][S][64] uint4
  const uint4* swa_v;
  const int32_t* swa_start;     // [R]
  const int32_t* swa_len;       // [R]
  float* out;                   // [R][16][512]
  float* lse;                   // [R][16] or null
  int32_t S;
  float sm_scale;
  int32_t swa_shared;           // every row reads window buffer 0
};

struct AttnArgs {
  AttnLayer layer[kMaxAttnLayers];
  int32_t n_layers;
  const uint8_t* kv;            // [n_slots][256]
  const uint8_t* kv_scale;      // [n_slots][32]
  SlotMap map;
  const int32_t* row_seq;
  const int32_t* seq_len;
  const int32_t* idx;           // [R][k], shared by every layer of the launch
  int32_t k;
  int32_t R;
  int32_t n_blocks;             // blocks per (layer, row)
  int32_t steps_per_block;    // 128-key steps per block
  float* part_o;                // [n_layers][R][n_blocks][16][512]
  float* part_ml;               // [n_layers][R][n_blocks][16][2]
  // the final selection of the split Top-k, when it is left to this launch
  // (sel.out non-null: the segment lists are ready, idx = sel.out is still to
  // be written)
  TopkArgs sel;
  CSA2_TRACE_ARG
};

hipError_t launch_index_score(const IdxArgs& a, bool cand, bool has_w, bool maxima, hipStream_t st);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
hipError_t launch_topk_large(const TopkArgs& a, hipStream_t st);
hipError_t launch_topk_desc(const TopkArgs& a, hipStream_t st);
hipError_t launch_desc_seg(const TopkArgs& a, hipStream_t st);
hipError_t launch_desc_final(const TopkArgs& a, hipStream_t st);
// launches that pair a group step's independent pieces (topk.hip)
hipError_t launch_desc_seg_tau(const TopkArgs& d, const TopkArgs& g, hipStream_t st);
hipError_t launch_topk_kth_gather(const TopkArgs& t, const TopkArgs& g, hipStream_t st);
hipError_t launch_seg_final(const TopkArgs& g, hipStream_t st);
hipError_t launch_maxima(const MaximaArgs& a, hipStream_t st);
// cand: the candidate blocks' final selection, when it is to share the
// merge's launch (after the attention)
hipError_t launch_attn(const AttnArgs& a, hipStream_t st, const TopkArgs* cand = nullptr);
hipError_t launch_merge_final(const AttnArgs& a, const TopkArgs& g, hipStream_t st);
hipError_t launch_quant(const float* x, int64_t n, const int64_t* dst, uint8_t* fp4, uint8_t* scale,
                        int64_t n_slots, hipStream_t st);
hipError_t launch_fp8_key_quant(const uint16_t* k, int64_t n, const int64_t* dst, uint8_t* codes, float* scale,
                                int64_t n_slots, hipStream_t st);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st);
hipError_t launch_prefill_index(const PrefArgs& a, bool has_w, hipStream_t st);
constexpr int kPrefMinRows = 256;        // rows from which the MFMA prefill indexer is used
constexpr int kPrefMinN = 128 * CSA2_TOPK;  // positions from which it is used (>= 2k groups of 64)
constexpr int kPrefMaxN = 262144;        // positions it supports
constexpr int kPrefCap = 4096;           // candidate positions kept per row
int attn_steps(int k);
int attn_blocks(int k, int rows_x_layers, int* steps_per_block);

}  // namespace csa2
