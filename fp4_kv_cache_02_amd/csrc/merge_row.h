// The merge of a split decode attention's partial softmax states, per block
// of 256 threads; launched on its own (attn.hip) or beside the candidate
// blocks' final selection (topk.hip, merge_final_kernel).
#pragma once
#include "kernels.h"

namespace csa2 {

// One merge block of 256 threads, block id `bid` = quarter of the heads *
// (layers x rows) + layer * R + row, thread `tid`: out = sum_j w_j O_j /
// sum_j w_j l_j with w_j = exp(m_j - max_j m_j), the partials of the row's
// attention blocks merged as one softmax; lse = max + log(sum).
CSA2_DEV void merge_block(const AttnArgs& a, int bid, int tid) {
  const int nlr = a.n_layers * a.R;
  const int hq = bid / nlr, lr = bid - hq * nlr;   // lr = li * R + r
  const int li = lr / a.R, r = lr - li * a.R;
  const AttnLayer& Ly = a.layer[li];
  const int th = 4 * hq + (tid >> 6), tc = tid & 63;   // head th, dims 8tc .. 8tc+7
  const int64_t prow = (int64_t)lr * a.n_blocks;
  CSA2_MARK(a, 16);
  CSA2_SPAN(a, 1280, 0);
  // every load is unconditional (blocks past n_blocks re-read the last one
  // and get weight 0), so all of them are in flight at once
  float mj[kMaxAttnBlocks], lj[kMaxAttnBlocks];
  float4 v[kMaxAttnBlocks][2];
#pragma unroll
  for (int j = 0; j < kMaxAttnBlocks; ++j) {
    const int64_t pj = prow + min(j, a.n_blocks - 1);
    mj[j] = a.part_ml[pj * 32 + th * 2 + 0];
    lj[j] = a.part_ml[pj * 32 + th * 2 + 1];
    const float* po = a.part_o + pj * (16 * 512) + th * 512 + tc * 8;
    v[j][0] = *(const float4*)po;
    v[j][1] = *(const float4*)(po + 4);
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < kMaxAttnBlocks; ++j) M = fmaxf(M, j < a.n_blocks ? mj[j] : -__builtin_inff());
  CSA2_MARK(a, 17);
  float Lsum = 0.f, wj[kMaxAttnBlocks];
#pragma unroll
  for (int j = 0; j < kMaxAttnBlocks; ++j) {
    wj[j] = (j >= a.n_blocks || mj[j] == -__builtin_inff()) ? 0.f : __expf(mj[j] - M);
    Lsum += wj[j] * lj[j];
  }
  float4 acc[2];
#pragma unroll
  for (int q4 = 0; q4 < 2; ++q4) acc[q4] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < kMaxAttnBlocks; ++j) {
#pragma unroll
    for (int q4 = 0; q4 < 2; ++q4) {
      acc[q4].x += wj[j] * v[j][q4].x;
      acc[q4].y += wj[j] * v[j][q4].y;
      acc[q4].z += wj[j] * v[j][q4].z;
      acc[q4].w += wj[j] * v[j][q4].w;
    }
  }
  const float inv = (Lsum > 0.f) ? 1.0f / Lsum : 0.f;
  float* out_row = Ly.out + ((int64_t)r * 16 + th) * 512 + tc * 8;
#pragma unroll
  for (int q4 = 0; q4 < 2; ++q4)
    *(float4*)(out_row + 4 * q4) = make_float4(acc[q4].x * inv, acc[q4].y * inv, acc[q4].z * inv, acc[q4].w * inv);
  if (Ly.lse && tc == 0) Ly.lse[(int64_t)r * 16 + th] = (Lsum > 0.f) ? M + __logf(Lsum) : -__builtin_inff();
  CSA2_MARK(a, 18);
  CSA2_SPAN(a, 1280, 1);
}

}  // namespace csa2
