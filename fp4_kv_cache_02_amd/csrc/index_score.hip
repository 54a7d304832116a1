// Indexer scoring (Full-layer scan / Reindex candidate scoring).
//
// The indexer of a CSA2 layer scores context positions by its own indexer
// query against the shared indexer keys (e-cogni summary of "DeepSeek-V4.1-Flash:
// Pushing the Limits of KV Cache Compression", section "Como funciona"; the
// Reindex layer scores only the candidate blocks built by the Full layer:
// 7minutos.es page, section "Atención escasa comprimida 2 (CSA2)").
//
// score = (w0*r0 + w1*r1) + (w2*r2 + w3*r3), r_h = ReLU(d_h), with d_h the dot
// product of head h evaluated as eight fused-multiply-add chains over channels
// 8j..8j+7 (from +0, channel order) combined as ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)).
//
// Layout of the work: a tile is 256 positions (32 KiB of bf16 keys).  The tile
// is read from HBM with fully coalesced 16-byte loads (thread t loads piece
// i*256+t), written to LDS with an XOR swizzle of the 16-byte chunks
// (chunk j of row p at slot j ^ (p & 7)) so that both the writes and the
// per-position reads are bank-conflict free, and then each thread scores one
// position from LDS.  The next tile's loads are issued before the current tile
// is scored.  The query (4 x 64) is uniform over the block and is read through
// the scalar cache.  Persistent grid: each block walks work items (row, tile)
// with a stride of gridDim.x.
#include "kernels.h"

namespace csa2 {

constexpr int kTile = 256;           // positions per tile (one per thread)


template <bool CAND, bool HAS_W, bool BMAX>
__global__ __launch_bounds__(256) void index_score_kernel(IdxArgs a, const uint32_t* __restrict__ q32,
                                                          const uint4* __restrict__ kdata,
                                                          float* __restrict__ scores,
                                                          float* __restrict__ block_max) {
  __shared__ uint4 lds[kTile * 8];
  const int tid = threadIdx.x;
  const int64_t n_items = (int64_t)a.R * a.tiles_per_row;

  // per-thread piece geometry: piece i covers position P = i*32 + tid/8, chunk tid%8
  const int pchunk = tid & 7;
  uint4 regs[8];

  auto load_item = [&](int64_t item) {
    const int r = (int)(item / a.tiles_per_row);
    const int t = (int)(item % a.tiles_per_row);
    const int b = a.row_seq ? a.row_seq[r] : r;
    const int L = min(a.seq_len[b], a.n_max);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int P = i * 32 + (tid >> 3);
      int64_t pos;
      bool ok;
      if (CAND) {
        const int ci = t * kTile + P;
        const int blk = (ci < a.n_cand * 8) ? a.cand[(int64_t)r * a.n_cand + (ci >> 3)] : -1;
        pos = (int64_t)blk * 8 + (ci & 7);
        ok = blk >= 0 && pos < L;
      } else {
        pos = (int64_t)t * kTile + P;
        ok = pos < L;
      }
      int64_t slot = ok ? a.map(b, pos) : -1;
      ok = slot >= 0;
      regs[i] = ok ? kdata[slot * 8 + pchunk] : make_uint4(0, 0, 0, 0);
    }
  };

  int64_t item = blockIdx.x;
  if (item >= n_items) return;
  load_item(item);

  for (; item < n_items; item += gridDim.x) {
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int P = i * 32 + (tid >> 3);
      lds[P * 8 + (pchunk ^ (P & 7))] = regs[i];
    }
    __syncthreads();
    const int64_t next = item + gridDim.x;
    const int r = (int)(item / a.tiles_per_row);
    const int t = (int)(item % a.tiles_per_row);
    if (next < n_items) load_item(next);

    // ---- score position p = tile*256 + tid ----
    const int b = a.row_seq ? a.row_seq[r] : r;
    const int L = min(a.seq_len[b], a.n_max);
    int64_t pos;
    bool ok;
    if (CAND) {
      const int ci = t * kTile + tid;
      const int blk = (ci < a.n_cand * 8) ? a.cand[(int64_t)r * a.n_cand + (ci >> 3)] : -1;
      pos = (int64_t)blk * 8 + (ci & 7);
      ok = blk >= 0 && pos < L && a.map(b, pos) >= 0;
    } else {
      pos = (int64_t)t * kTile + tid;
      ok = pos < L && a.map(b, pos) >= 0;
    }
    const uint32_t* q = q32 + (int64_t)r * 128;
    float c[4][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 kw = lds[tid * 8 + (j ^ (tid & 7))];
      const float kf[8] = {bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y),
                           bf16_lo(kw.z), bf16_hi(kw.z), bf16_lo(kw.w), bf16_hi(kw.w)};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t q0 = q[h * 32 + j * 4 + 0], q1 = q[h * 32 + j * 4 + 1];
        const uint32_t q2 = q[h * 32 + j * 4 + 2], q3 = q[h * 32 + j * 4 + 3];
        float acc = 0.0f;
        acc = __builtin_fmaf(kf[0], bf16_lo(q0), acc);
        acc = __builtin_fmaf(kf[1], bf16_hi(q0), acc);
        acc = __builtin_fmaf(kf[2], bf16_lo(q1), acc);
        acc = __builtin_fmaf(kf[3], bf16_hi(q1), acc);
        acc = __builtin_fmaf(kf[4], bf16_lo(q2), acc);
        acc = __builtin_fmaf(kf[5], bf16_hi(q2), acc);
        acc = __builtin_fmaf(kf[6], bf16_lo(q3), acc);
        acc = __builtin_fmaf(kf[7], bf16_hi(q3), acc);
        c[h][j] = acc;
      }
    }
    float rr[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float d = ((c[h][0] + c[h][1]) + (c[h][2] + c[h][3])) +
                      ((c[h][4] + c[h][5]) + (c[h][6] + c[h][7]));
      rr[h] = (d > 0.0f) ? d : 0.0f;
    }
    float s;
    if (HAS_W) {
      const float* w = a.head_w + (int64_t)r * 4;
      const float p0 = w[0] * rr[0], p1 = w[1] * rr[1], p2 = w[2] * rr[2], p3 = w[3] * rr[3];
      s = (p0 + p1) + (p2 + p3);
    } else {
      s = (rr[0] + rr[1]) + (rr[2] + rr[3]);
    }
    if (CAND) {
      const int64_t ci = (int64_t)t * kTile + tid;
      if (ci < a.score_stride) scores[(int64_t)r * a.score_stride + ci] = ok ? s : -__builtin_inff();
    } else {
      if (ok) scores[(int64_t)r * a.score_stride + pos] = s;
      if (BMAX) {
        uint32_t k = ok ? order_key(s) : 0u;
        k = max(k, (uint32_t)__shfl_xor((int)k, 1, kWave));
        k = max(k, (uint32_t)__shfl_xor((int)k, 2, kWave));
        k = max(k, (uint32_t)__shfl_xor((int)k, 4, kWave));
        if ((tid & 7) == 0 && k != 0u) block_max[(int64_t)r * a.bmax_stride + (pos >> 3)] = key_to_float(k);
      }
    }
  }
}

hipError_t launch_index_score(const IdxArgs& a, bool cand, bool has_w, bool bmax, hipStream_t st) {
  const int64_t items = (int64_t)a.R * a.tiles_per_row;
  if (items == 0) return hipSuccess;
  const int grid = (int)(items < 2048 ? items : 2048);
#define CSA2_IDX_LAUNCH(C, W, M) \
  hipLaunchKernelGGL((index_score_kernel<C, W, M>), dim3(grid), dim3(256), 0, st, a, a.q32, a.kdata, \
                     a.scores, a.block_max)
  if (cand) {
    if (has_w) CSA2_IDX_LAUNCH(true, true, false); else CSA2_IDX_LAUNCH(true, false, false);
  } else if (bmax) {
    if (has_w) CSA2_IDX_LAUNCH(false, true, true); else CSA2_IDX_LAUNCH(false, false, true);
  } else {
    if (has_w) CSA2_IDX_LAUNCH(false, true, false); else CSA2_IDX_LAUNCH(false, false, false);
  }
#undef CSA2_IDX_LAUNCH
  return hipGetLastError();
}

}  // namespace csa2
