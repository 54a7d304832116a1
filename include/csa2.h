/*
 * csa2.h -- C ABI of the MI355X (gfx950) CSA2 decode/prefill hot path.
 *
 * CSA2 (Compressed Sparse Attention 2) is the attention of DeepSeek-V4.1-Flash
 * as the pages covering its release describe it: every layer is statically one
 * of three modes -- Full (computes its own main KV and indexer K, selects new
 * Top-512 indices), Reindex (re-scores the indexer K of the last Full layer
 * with its own indexer Q and selects a new Top-K), Reuse (re-uses the main KV
 * and the most recent Top-K, no indexer) -- and in the decoder a hierarchical
 * indexer lets the Full layer build a candidate set of up to 16 384 positions
 * (2 048 blocks of 8) that later Reindex layers score instead of the whole
 * context.  Sources: page "DeepSeek lança V4.1-Flash com contexto de um milhão
 * de tokens..." (conexaotc.com.br), paragraph on CSA2; page "DeepSeek AI lanzó
 * DeepSeek-V4.1-Flash..." (7minutos.es), section "Atención escasa comprimida 2
 * (CSA2)"; e-cogni summary of "DeepSeek-V4.1-Flash: Pushing the Limits of KV
 * Cache Compression", section "Como funciona".  The main KV is E2M1 with one
 * E4M3 scale per 16 channels (NVFP4 without its global scale): conexaotc page,
 * paragraph on KV quantisation.  Every layer keeps its own global Q and its own
 * 128-token sliding-window KV: e-cogni summary, section "Como funciona";
 * conexaotc page, paragraph on the Causal Encoder-Decoder.
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers to memory the caller owns.  The
 *    library allocates nothing and keeps no state between calls; scratch space
 *    comes from the caller's workspace (see csa2_workspace_bytes).
 *  - bf16 tensors are passed as uint16_t bit patterns.  Row-major, contiguous.
 *  - Work is enqueued on `stream`; calls return without synchronising.
 *  - Host-side validation runs before any launch and returns an error code
 *    (nothing is enqueued then).  A launch failure returns CSA2_ERR_HIP.
 *    Asynchronous device faults surface at the caller's next synchronisation.
 *  - Inputs must be finite and row_seq entries must be valid sequence indices
 *    (preconditions, not checked).  Top-K indices, candidate blocks, window
 *    ranges and page-table entries that fall outside their tensors are skipped
 *    by the kernels, never dereferenced; seq_len is clamped to n_max.
 *  - Two calls that share a workspace must not run concurrently.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

/* Fixed model dimensions. */
#define CSA2_HEADS 16        /* query heads, all sharing one main-KV vector (MQA) */
#define CSA2_DIM 512         /* main-KV / query head dimension                     */
#define CSA2_IDX_HEADS 4     /* indexer heads                                       */
#define CSA2_IDX_DIM 64      /* indexer head dimension                              */
#define CSA2_BLOCK 8         /* positions per hierarchical-indexer block            */
#define CSA2_MAX_WINDOW 128  /* sliding-window length                               */
#define CSA2_TOPK 512        /* Top-K of the layer modes                            */
#define CSA2_KEEP_BLOCKS 2048/* candidate blocks kept by a hierarchical Full layer  */
#define CSA2_MAX_K 2048      /* largest k accepted by csa2_topk                     */
#define CSA2_PAGE 64         /* positions per page of a paged cache                 */
#define CSA2_MAX_ROWS 65536  /* largest number of query rows per call               */
#define CSA2_MAX_GROUP_LAYERS 8 /* layers one csa2_group_step call may run          */

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_NULL = 1,        /* a required pointer is NULL                    */
  CSA2_ERR_SHAPE = 2,       /* a size or count is out of range               */
  CSA2_ERR_UNSUPPORTED = 3, /* a layout the library does not implement      */
  CSA2_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required    */
  CSA2_ERR_HIP = 5          /* a HIP launch failed                           */
} csa2_status;

typedef enum { CSA2_FULL = 0, CSA2_REINDEX = 1, CSA2_REUSE = 2 } csa2_mode;

/*
 * A per-position cache: the FP4 main KV or the bf16 indexer keys.  Both use
 * the same slot mapping (a position owns one slot in each).
 *   main KV:     data  = [n_slots][256] uint8, channel 2i in the low nibble of
 *                        byte i, channel 2i+1 in the high nibble (E2M1 codes:
 *                        bit 3 sign, bits 2..1 exponent, bit 0 mantissa);
 *                scale = [n_slots][32] uint8, E4M3 (OCP E4M3FN) scale of
 *                        channels 16j .. 16j+15 in byte j.
 *   indexer K:   data  = [n_slots][64] bf16 (16-byte aligned); scale = NULL;
 *                or, FP8 indexer keys, data = [n_slots][64] uint8 OCP E4M3FN
 *                codes (no NaN codes; 8-byte aligned) and scale = [n_slots]
 *                float32 (4-byte aligned, finite, >= 0), passed through
 *                this uint8 pointer: 68 B per position, the entry under which
 *                the pages' 890 B per token of global KV cache adds up with
 *                the 288-B FP4 main-KV entry (890 = 2.5 x (288 + 68)).
 *                The FP8 form is read by csa2_index_score and by the
 *                Full/Reindex layers of csa2_layer_step / csa2_group_step.
 * Slot of position p of sequence b:
 *   page_table == NULL : b * seq_stride + p
 *   page_table != NULL : page_table[b * max_pages + p / page_size] * page_size
 *                        + p % page_size          (page_size must be 64)
 * A slot outside [0, n_slots) is treated as absent.  Every entry point
 * returns CSA2_ERR_NULL for a missing data (or main-KV scale) pointer,
 * CSA2_ERR_SHAPE for a negative n_slots, seq_stride or max_pages, and
 * CSA2_ERR_UNSUPPORTED for a page table with page_size other than 64.
 */
typedef struct {
  const void* data;
  const uint8_t* scale;
  const int32_t* page_table;
  int32_t page_size;
  int32_t max_pages;
  int64_t seq_stride;
  int64_t n_slots;
} csa2_cache;

/*
 * Indexer scoring (the Full layer's scan, or the Reindex layer's scoring of
 * its candidate positions).  Defined by: conexaotc.com.br page "DeepSeek lança
 * V4.1-Flash com contexto de um milhão de tokens...", paragraph on CSA2 (a Full
 * layer scores the context with its own indexer query against the indexer
 * keys; a Reindex layer re-scores, with its own indexer query, the candidate
 * positions of the hierarchical indexer); e-cogni summary of
 * "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression", section
 * "Como funciona" (Reindex uses the shared indexer K of the preceding Full
 * layer).  The pages do not give the head combination; the form below is
 * the one this library fixes.
 * For query row r of sequence b = row_seq[r]
 * (row_seq NULL: b = r), with L = seq_len[b] visible positions,
 *   score(p) = sum_h w_h * ReLU(q_idx[r][h] . k_idx(b, p)),  h = 0..3,
 * w = head_w[r] (head_w NULL: all ones), evaluated in float32 in a fixed order:
 * per head, eight partial sums over channels 8j..8j+7, each a chain of fused
 * multiply-adds in channel order starting from +0, combined as
 * ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)); then ReLU; then
 * (w0*r0 + w1*r1) + (w2*r2 + w3*r3) with each product rounded on its own.
 * FP8 indexer keys: the chains run over the exact E4M3 values and each head's
 * dot product is multiplied by the position's scale (one float32 rounding)
 * before the ReLU.
 *
 * cand_blocks == NULL (scan):  scores[r][p] for p < L (entries p >= L are not
 *   written; a position below L whose slot is absent scores -inf); if
 *   block_max != NULL, block_max[r][j] = the largest score of block j
 *   (positions 8j..8j+7 below L, -0 below +0) for j < ceil(L/8), -inf when
 *   the block has no present position.
 * cand_blocks != NULL (Reindex): cand_blocks[r][0..n_cand) are block ids
 *   (-1 = none); scores[r][8i + t] is the score of position 8*cand[i] + t, or
 *   -inf when the block is -1 or that position is >= L.  block_max must be NULL.
 * Row stride of scores is n_max (scan) or 8*n_cand (Reindex); of block_max
 * ceil(n_max/8).  Requires 1 <= R <= CSA2_MAX_ROWS, every L <= n_max,
 * n_cand <= CSA2_KEEP_BLOCKS.
 */
csa2_status csa2_index_score(const uint16_t* q_idx /* [R][4][64] */, const float* head_w,
                             const csa2_cache* k_idx, const int32_t* row_seq,
                             const int32_t* seq_len /* [B] */, const int32_t* cand_blocks,
                             int32_t n_cand, int32_t R, int32_t n_max, float* scores,
                             float* block_max, hipStream_t stream);

/*
 * Top-k selection.  Defined by: conexaotc.com.br page, paragraph on CSA2 (each
 * Full or Reindex layer keeps the Top-512 positions by indexer score);
 * 7minutos.es page "DeepSeek AI lanzó DeepSeek-V4.1-Flash...", section
 * "Atención escasa comprimida 2 (CSA2)".  Ties and output order are not given
 * there: ties go to the lower index, indices come out ascending.
 * For row r, among scores[r][0 .. n) with
 * n = n_valid[row_seq ? row_seq[r] : r] (n_valid NULL: n = n_max), entries equal
 * to -inf being absent, keep the first min(k, present) in the order (score
 * descending, index ascending; -0 below +0) and write their indices in
 * ascending order to idx[r][0..k), padding with -1.  If cand_blocks is given
 * ([R][n_max/8], n_max a multiple of 8 and at most 8*CSA2_KEEP_BLOCKS), index
 * i is written as the position 8*cand_blocks[r][i/8] + i%8 instead.
 * The result is exact.  Row stride of scores is `row_stride` elements.
 * Requires 1 <= k <= CSA2_MAX_K, 0 <= n_max <= 1048576 (larger:
 * CSA2_ERR_UNSUPPORTED), workspace of at least
 * csa2_topk_workspace_bytes(R, n_max, k) bytes (prepared by
 * csa2_workspace_init).
 */
csa2_status csa2_topk(const float* scores, int64_t row_stride, const int32_t* row_seq,
                      const int32_t* n_valid, int32_t R, int32_t n_max, int32_t k,
                      const int32_t* cand_blocks, int32_t* idx, void* ws, size_t ws_bytes,
                      hipStream_t stream);
size_t csa2_topk_workspace_bytes(int32_t R, int32_t n_max, int32_t k);

/*
 * Hierarchical candidate build.  Defined by: conexaotc.com.br page, paragraph
 * on CSA2 (in the decoder the Full layer builds a candidate set of up to 2048
 * blocks of 8 positions, 16384 positions, that the Reindex layers score
 * instead of the whole context); e-cogni summary, section "Como funciona".
 * The block score is not given there: it is the largest score in the block.
 * For row r with L = seq_len[row_seq[r]], keep
 * the `keep` best of the ceil(L/8) block scores block_max[r][..] (order:
 * score descending, block id ascending) and write their block ids ascending
 * to cand_blocks[r][0..keep), padding with -1.  Row stride of block_max is
 * ceil(n_max/8).  With keep >= 512 the candidate positions contain the Full
 * layer's Top-512.  Requires 1 <= keep <= CSA2_MAX_K, n_max <= 1048576, and
 * workspace as for csa2_topk(R, ceil(n_max/8), keep).
 */
csa2_status csa2_hier_candidates(const float* block_max, const int32_t* row_seq,
                                 const int32_t* seq_len, int32_t R, int32_t n_max, int32_t keep,
                                 int32_t* cand_blocks, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * Sparse FP4 attention with the sliding window.  Defined by: e-cogni summary
 * of "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression",
 * sections "O que os autores propõem" and "Como funciona" (every layer attends
 * with its own query over the selected main-KV entries and its own 128-token
 * sliding window); conexaotc.com.br page, paragraph on the KV quantisation
 * (the main KV is E2M1 with one E4M3 scale per 16 channels and no global
 * scale).  How the two branches combine is not given there: one softmax over
 * their union.
 * For query row r of sequence b = row_seq[r] (row_seq NULL: b = r), L = seq_len[b]:
 *   entries = { main-KV vector of position idx[r][i] : 0 <= idx < L }
 *           U { window entry w : swa_start[r] <= w < swa_start[r] + swa_len[r] }
 *   out[r][h] = sum_e softmax_e(sm_scale * q[r][h] . key_e) * value_e
 *   lse[r][h] = log sum_e exp(sm_scale * q[r][h] . key_e)
 * The dequantised main-KV vector (E2M1 code * E4M3 scale, exact) is both key
 * and value; window entries use swa_k[b][w] as key and swa_v[b][w] as value
 * ([B][S][512] bf16).  One softmax per head over the union (no de-duplication
 * between the two branches).  A row with no entries gets out = 0, lse = -inf.
 * idx entries < 0 or >= L are skipped, and so are window entries outside
 * [0, S).  Requires 1 <= k <= CSA2_TOPK, swa_len <= 128 (longer windows are
 * cut to 128 entries), kv->n_slots < 2^31; any finite bf16 query (the main
 * keys' products run on fp16 matrix cores with each head's query scaled by a
 * power of two into fp16's range, elements more than 2^28 below the head's
 * largest one dropping out).  A paged kv with page_size other than 64 returns
 * CSA2_ERR_UNSUPPORTED.  Accumulation in float32; output float32.
 * Workspace: csa2_attn_workspace_bytes(R), enough for every k.
 */
csa2_status csa2_fp4_sparse_attn(const uint16_t* q /* [R][16][512] */, const csa2_cache* kv,
                                 const int32_t* row_seq, const int32_t* seq_len,
                                 const int32_t* idx /* [R][k] */, int32_t k,
                                 const uint16_t* swa_k, const uint16_t* swa_v, int32_t S,
                                 const int32_t* swa_start, const int32_t* swa_len,
                                 float sm_scale, int32_t R, float* out /* [R][16][512] */,
                                 float* lse /* [R][16] or NULL */, void* ws, size_t ws_bytes,
                                 hipStream_t stream);
size_t csa2_attn_workspace_bytes(int32_t R);

/*
 * FP4 quantisation of new main-KV vectors (the write side of the cache).
 * Defined by: conexaotc.com.br page, paragraph on the KV quantisation (E2M1
 * values with one E4M3 scale per 16 channels, the NVFP4 pattern without its
 * global scale); 7minutos.es page, section "FP4 KV, repetición limitada y
 * otras extensiones".  Rounding and saturation are not given there:
 * x[i] (512 float32) -> main-KV slot dst_slot[i] (dst_slot NULL: slot i).
 * Per 16-channel block: amax = max|x|; scale = E4M3 round-to-nearest-even of
 * amax/6 (float32 division), saturating at 448; codes = E2M1
 * round-to-nearest-even of x / scale (float32 division), saturating at +-6,
 * sign kept; a zero scale gives all-zero codes.  Slots outside [0, n_slots)
 * are skipped.
 */
csa2_status csa2_fp4_quantize(const float* x, int64_t n, const int64_t* dst_slot,
                              uint8_t* fp4 /* [n_slots][256] */,
                              uint8_t* scale /* [n_slots][32] */, int64_t n_slots,
                              hipStream_t stream);

/*
 * FP8 quantisation of new indexer keys (the write side of the FP8 indexer-key
 * cache).  The pages give only the entry size -- 890 B of global KV cache per
 * token, which adds up with a 68-B indexer entry beside the 288-B FP4 main-KV
 * entry (conexaotc.com.br page, opening paragraph; 7minutos.es page, opening
 * section); the encoding is this library's reading: k[i] (64 bf16 channels)
 * -> slot dst_slot[i] (dst_slot NULL: slot i) of codes ([n_slots][64] uint8,
 * OCP E4M3FN) and scale ([n_slots] float32): s = amax / 448 (amax = max |k|,
 * float32 division), code = E4M3 round-to-nearest-even of |k| / s (float32
 * division, saturating at 448) with the sign of k; s == 0 gives all codes 0.
 * The largest element of a key maps to +-448.  Slots outside [0, n_slots) are
 * skipped.
 */
csa2_status csa2_fp8_key_quantize(const uint16_t* k, int64_t n, const int64_t* dst_slot, uint8_t* codes,
                                  float* scale, int64_t n_slots, hipStream_t stream);

/* State handed from layer to layer within a group (Full -> Reindex/Reuse). */
typedef struct {
  csa2_cache kv;           /* main KV shared by the group                          */
  csa2_cache k_idx;        /* indexer keys shared by the group                     */
  const int32_t* seq_len;  /* [B] visible positions per sequence                   */
  int32_t B;
  int32_t n_max;           /* >= every seq_len                                     */
  int32_t hier;            /* Full layers build candidate blocks                   */
  int32_t* topk_idx;       /* [R][512]: the most recent Top-K (positions, -1 pad)  */
  int32_t* cand_blocks;    /* [R][2048]: candidate blocks of the last Full layer   */
} csa2_shared;

/* One layer's own inputs and outputs. */
typedef struct {
  int32_t R;
  const int32_t* row_seq;  /* [R] or NULL (row r is sequence r)                    */
  const uint16_t* q_idx;   /* [R][4][64] indexer query (Full, Reindex)             */
  const float* head_w;     /* [R][4] indexer head weights or NULL                  */
  const uint16_t* q;       /* [R][16][512] query                                   */
  const uint16_t* swa_k;   /* [B][S][512] window keys                              */
  const uint16_t* swa_v;   /* [B][S][512] window values                            */
  int32_t S;
  const int32_t* swa_start;/* [R] */
  const int32_t* swa_len;  /* [R] */
  float sm_scale;
  int32_t blocks_only;     /* Full + hier: stop after the candidate build          */
  float* out;              /* [R][16][512]                                         */
  float* lse;              /* [R][16] or NULL                                      */
  int32_t swa_shared;      /* nonzero: swa_k/swa_v hold one buffer [1][S][512] that
                              every row reads at its own swa_start (the rows of a
                              prefill chunk given as sequences of their own that
                              share the caches' slots, seq_stride 0)              */
} csa2_layer_args;

/*
 * A group of layers that share one Top-K: layers[0] runs in first_mode
 * (Full, Reindex or Reuse) and layers[1 .. n_layers) run as Reuse layers over
 * the Top-K it leaves in shared->topk_idx -- the decoder's Full + 3 Reuse or
 * Reindex + 3 Reuse, the encoder's Full + 5 Reuse (conexaotc.com.br page,
 * paragraph on CSA2; 7minutos.es page, section "Atención escasa comprimida 2
 * (CSA2)").  Results equal n_layers csa2_layer_step calls; the attention of
 * every layer of the group runs in one launch.  All layers must have the same
 * R and row_seq.  Requires 1 <= n_layers <= CSA2_MAX_GROUP_LAYERS,
 * R * n_layers <= CSA2_MAX_ROWS, shared->n_max <= 1048576, workspace of
 * csa2_group_workspace_bytes(first_mode, n_layers, R, n_max, hier) bytes.
 */
csa2_status csa2_group_step(csa2_mode first_mode, int32_t n_layers, const csa2_layer_args* layers,
                            const csa2_shared* shared, void* ws, size_t ws_bytes, hipStream_t stream);
size_t csa2_group_workspace_bytes(csa2_mode first_mode, int32_t n_layers, int32_t R, int32_t n_max,
                                  int32_t hier);

/*
 * csa2_group_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The library's own scratch stands in for
 * the workspace: a static device array of CSA2_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the first call on that GPU until the process ends (its device
 * address is looked up once per device, on the device current at the call;
 * `stream` must belong to that device).  Results equal csa2_group_step's with
 * a workspace of its own.  A call whose csa2_group_workspace_bytes exceeds
 * CSA2_NOALLOC_SCRATCH_BYTES returns CSA2_ERR_WORKSPACE before anything is
 * enqueued (64 MiB covers, for instance, a Full + 3 Reuse group at batch 32 and
 * 131072 positions, or the 1M-position hierarchical groups at batch 1; not a
 * 32-row Full layer at 1M positions, nor a prefill chunk).  Every call on one
 * GPU uses the same scratch, which keeps the last call's contents (nothing in
 * it needs clearing: the kernels reset their own counters): calls that
 * overlap on one GPU (other streams, other host threads) race and must be
 * serialised by the caller.  This entry point calls no allocator.
 */
#define CSA2_NOALLOC_SCRATCH_BYTES (64ull << 20)
csa2_status csa2_group_step_noalloc(csa2_mode first_mode, int32_t n_layers, const csa2_layer_args* layers,
                                    const csa2_shared* shared, hipStream_t stream);

/*
 * One CSA2 layer.  Defined by: conexaotc.com.br page, paragraph on CSA2 (the
 * static Full / Reindex / Reuse modes); 7minutos.es page, section "Atención
 * escasa comprimida 2 (CSA2)"; e-cogni summary, section "Como funciona" (each
 * layer's own query and window).
 *   CSA2_FULL    : scan all L positions -> Top-512 into shared->topk_idx (and,
 *                  if shared->hier, candidate blocks into shared->cand_blocks)
 *                  -> attention.  With blocks_only: candidates only.
 *   CSA2_REINDEX : score the 8*2048 candidate positions of shared->cand_blocks
 *                  with this layer's q_idx -> Top-512 into shared->topk_idx ->
 *                  attention.  Without a hierarchical Full layer before it
 *                  (shared->hier == 0) every position is scored.
 *   CSA2_REUSE   : attention over shared->topk_idx.
 * Workspace: csa2_workspace_bytes(mode, R, n_max, hier).
 */
csa2_status csa2_layer_step(csa2_mode mode, const csa2_layer_args* args,
                            const csa2_shared* shared, void* ws, size_t ws_bytes,
                            hipStream_t stream);
size_t csa2_workspace_bytes(csa2_mode mode, int32_t R, int32_t n_max, int32_t hier);

/*
 * Prepare a freshly allocated workspace (zero its control words).  Needed once
 * per allocation; every call leaves the control words as it found them.
 */
csa2_status csa2_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/* Human-readable description of a status code (static string). */
const char* csa2_status_string(csa2_status status);

/* Library version string. */
const char* csa2_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
