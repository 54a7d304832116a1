// Kernel argument blocks and launch entry points shared by the kernels and
// the host dispatcher.
#pragma once
#include "common.h"

namespace csa2 {

struct IdxArgs {
  const uint32_t* q32;        // [R][4][32] bf16 pairs
  const float* head_w;        // [R][4] or null
  const uint4* kdata;         // [n_slots][8] 16-byte chunks of the indexer key
  SlotMap map;
  const int32_t* row_seq;
  const int32_t* seq_len;
  const int32_t* cand;        // [R][n_cand] or null
  int32_t n_cand;
  int32_t R;
  int32_t n_max;
  int32_t tiles_per_row;      // ceil(n_max/256) (scan) or n_cand/32 (Reindex)
  int64_t score_stride;
  int64_t bmax_stride;
  float* scores;
  float* block_max;
};

struct TopkArgs {
  const float* scores;
  int64_t row_stride;
  const int32_t* row_seq;
  const int32_t* n_valid;
  int32_t n_max;
  int32_t n_div;       // n = ceil(n_valid / n_div)
  int32_t R;
  int32_t k;
  int32_t S_max;        // segments per row at n_max
  int32_t kcap;         // candidate slots per segment = min(k, kSeg)
  const int32_t* cand_blocks;   // optional index -> position map
  int32_t cand_stride;
  int32_t* out;
  int32_t out_stride;
  uint32_t* cand_key;   // [R][S_max*kcap]
  int32_t* cand_idx;    // [R][S_max*kcap]
  int32_t* seg_info;    // [R][S_max][4]: truncated, worst key, worst index
  uint32_t* ticket;     // [R], zero between calls
};

struct AttnArgs {
  const uint4* q;               // [R][16][64] uint4 (8 bf16 each)
  const uint8_t* kv;            // [n_slots][256]
  const uint8_t* kv_scale;      // [n_slots][32]
  SlotMap map;
  const int32_t* row_seq;
  const int32_t* seq_len;
  const int32_t* idx;           // [R][k]
  int32_t k;
  const uint4* swa_k;           // [B][S][64] uint4
  const uint4* swa_v;
  int32_t S;
  const int32_t* swa_start;
  const int32_t* swa_len;
  float sm_scale;
  int32_t R;
  float* out;                   // [R][16][512]
  float* lse;                   // [R][16] or null
  float* part_o;                // [R][n_splits][16][512]
  float* part_ml;               // [R][n_splits][16][2]
  uint32_t* ticket;             // [R]
  int32_t n_main_splits;
  int32_t n_splits;
};

hipError_t launch_index_score(const IdxArgs& a, bool cand, bool has_w, bool bmax, hipStream_t st);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
hipError_t launch_attn(const AttnArgs& a, hipStream_t st);
hipError_t launch_quant(const float* x, int64_t n, const int64_t* dst, uint8_t* fp4, uint8_t* scale,
                        int64_t n_slots, hipStream_t st);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st);
int topk_segments(int n_max);
int topk_kcap(int k);
int attn_splits(int k, int* n_main);

}  // namespace csa2
