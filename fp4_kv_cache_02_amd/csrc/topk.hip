// Exact Top-k selection (the "Top-512" of the CSA2 Full and Reindex layers and
// the 2048 candidate blocks of the hierarchical indexer: conexaotc.com.br page
// "DeepSeek lança V4.1-Flash...", paragraph on CSA2).
//
// Order: score descending, index ascending (-0 below +0); -inf = absent;
// output ascending indices, -1 padding.
//
// Two stages in one launch.  Grid (rows, segments); a segment is 4096 scores.
//  1. Every segment block selects its local top-kloc exactly (radix select on
//     order-preserving keys) and writes it, in index order, to a padded slot
//     of the row's candidate array (unused entries: key 0 = absent).
//     kloc is sized from k*4096/n (expected share plus margin).
//  2. The last segment block of a row to finish (atomic ticket) selects the
//     top-k of the candidate union.  The union holds the true top-k unless a
//     segment that dropped elements kept a worst element that ranks above the
//     k-th selected one; that is checked, and in that case the row is
//     re-selected exactly from all its scores.
#include "select.h"
#include "kernels.h"

namespace csa2 {

constexpr int kSeg = 4096;
constexpr int kTopkThreads = 512;
constexpr int kPer = kSeg / kTopkThreads;   // 8


struct ScoreSrc {
  const float* p;
  int64_t n;
  CSA2_DEV void load(int64_t base, int tid, uint32_t (&k)[kPer]) const {
    const int64_t e0 = base + (int64_t)tid * kPer;
#pragma unroll
    for (int j = 0; j < kPer; ++j) k[j] = (e0 + j < n) ? order_key(p[e0 + j]) : 0u;
  }
};

struct KeySrc {
  const uint32_t* p;
  int64_t n;
  CSA2_DEV void load(int64_t base, int tid, uint32_t (&k)[kPer]) const {
    const int64_t e0 = base + (int64_t)tid * kPer;
#pragma unroll
    for (int j = 0; j < kPer; ++j) k[j] = (e0 + j < n) ? p[e0 + j] : 0u;
  }
};

CSA2_DEV int row_n(const TopkArgs& a, int r) {
  int n = a.n_max;
  if (a.n_valid) {
    const int v = a.n_valid[a.row_seq ? a.row_seq[r] : r];
    n = v <= 0 ? 0 : (v + a.n_div - 1) / a.n_div;
  }
  return n > a.n_max ? a.n_max : n;
}

CSA2_DEV int kloc_for(int k, int n, int S) {
  if (S <= 1) return k < kSeg ? k : kSeg;
  const float mu = (float)k * (float)kSeg / (float)n;
  const float v = mu + 4.0f * sqrtf(mu) + 8.0f;
  int kl = 16;
  while ((float)kl < v) kl <<= 1;
  const int cap = k < kSeg ? k : kSeg;
  return kl > cap ? cap : kl;
}

CSA2_DEV int32_t map_index(const TopkArgs& a, int r, int64_t i) {
  if (!a.cand_blocks) return (int32_t)i;
  const int32_t blk = a.cand_blocks[(int64_t)r * a.cand_stride + (i >> 3)];
  return blk * 8 + (int32_t)(i & 7);
}

// Exact top-k of a whole row from its scores, written to the output.
CSA2_DEV uint32_t select_row_direct(SelectSmem<kTopkThreads>& sm, const TopkArgs& a, int r,
                                    const float* row, int64_t n) {
  ScoreSrc src{row, n};
  uint32_t gt, eq;
  const uint32_t T = radix_select<kTopkThreads, kPer>(sm, src, n, (uint32_t)a.k, gt, eq);
  const uint32_t need_eq = T ? (uint32_t)a.k - gt : 0u;
  int32_t* out = a.out + (int64_t)r * a.out_stride;
  int64_t last;
  return compact<kTopkThreads, kPer>(
      sm, src, n, T, need_eq,
      [&](uint32_t pos, uint32_t, int64_t e) { out[pos] = map_index(a, r, e); }, last);
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  __shared__ SelectSmem<kTopkThreads> sm;
  const int r = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int n = row_n(a, r);
  const int S = n > kSeg ? (n + kSeg - 1) / kSeg : 1;
  if (s >= S) return;
  const float* row = a.scores + (int64_t)r * a.row_stride;
  int32_t* out = a.out + (int64_t)r * a.out_stride;

  if (S == 1) {
    const uint32_t m = select_row_direct(sm, a, r, row, n);
    for (int i = (int)m + tid; i < a.k; i += kTopkThreads) out[i] = -1;
    return;
  }

  // ---- stage 1: local selection of this segment ----
  const int kloc = kloc_for(a.k, n, S);
  const int64_t base = (int64_t)s * kSeg;
  const int64_t cnt = (n - base) < kSeg ? (n - base) : kSeg;
  ScoreSrc src{row + base, cnt};
  uint32_t gt, eq;
  const uint32_t T = radix_select<kTopkThreads, kPer>(sm, src, cnt, (uint32_t)kloc, gt, eq);
  const uint32_t need_eq = T ? (uint32_t)kloc - gt : 0u;
  const int64_t row_cbase = (int64_t)r * a.S_max * a.kcap;
  uint32_t* ck = a.cand_key + row_cbase + (int64_t)s * kloc;
  int32_t* ci = a.cand_idx + row_cbase + (int64_t)s * kloc;
  int64_t last_tie;
  const uint32_t m = compact<kTopkThreads, kPer>(
      sm, src, cnt, T, need_eq,
      [&](uint32_t pos, uint32_t key, int64_t e) { ck[pos] = key; ci[pos] = (int32_t)(base + e); },
      last_tie);
  for (int i = (int)m + tid; i < kloc; i += kTopkThreads) ck[i] = 0u;
  if (tid == 0) {
    // A segment with T != 0 kept exactly kloc elements and may have dropped
    // others ("truncated"); record its worst kept element: key T, and the
    // largest index among its kept elements equal to T.
    int32_t* info = a.seg_info + ((int64_t)r * a.S_max + s) * 4;
    info[0] = T != 0u ? 1 : 0;
    info[1] = (int32_t)T;
    info[2] = (int32_t)(base + last_tie);
    info[3] = (int32_t)m;
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = atomicAdd(&a.ticket[r], 1u);
    sm.bcast[4] = (old == (uint32_t)(S - 1)) ? 1u : 0u;
  }
  __syncthreads();
  if (sm.bcast[4] == 0u) return;
  __threadfence();

  // ---- stage 2: the last block of the row selects from the union ----
  const int64_t un = (int64_t)S * kloc;
  KeySrc usrc{a.cand_key + row_cbase, un};
  const int32_t* uidx = a.cand_idx + row_cbase;
  uint32_t ugt, ueq;
  const uint32_t UT = radix_select<kTopkThreads, kPer>(sm, usrc, un, (uint32_t)a.k, ugt, ueq);
  const uint32_t uneed = UT ? (uint32_t)a.k - ugt : 0u;
  int64_t ulast;
  uint32_t um = compact<kTopkThreads, kPer>(
      sm, usrc, un, UT, uneed,
      [&](uint32_t pos, uint32_t, int64_t e) { out[pos] = map_index(a, r, uidx[e]); }, ulast);
  const int64_t tk_idx = (UT != 0u && ulast >= 0) ? (int64_t)uidx[ulast] : -1;

  // safety check: a segment that kept exactly kloc of more present elements is
  // "truncated"; its worst kept element must not rank above the k-th selected.
  uint32_t unsafe = 0;
  for (int seg = tid; seg < S; seg += kTopkThreads) {
    const int32_t* info = a.seg_info + ((int64_t)r * a.S_max + seg) * 4;
    if (info[0] == 0) continue;               // kept every present element
    if (UT == 0u) { unsafe = 1; continue; }   // union has < k present but a segment dropped some
    const uint32_t Ts = (uint32_t)info[1];
    const int64_t ws_idx = info[2];
    if (Ts > UT || (Ts == UT && ws_idx < tk_idx)) unsafe = 1;
  }
  if (tid == 0) sm.bcast[5] = 0u;
  __syncthreads();
  if (unsafe) atomicOr(&sm.bcast[5], 1u);
  __syncthreads();
  if (sm.bcast[5]) um = select_row_direct(sm, a, r, row, n);
  for (int i = (int)um + tid; i < a.k; i += kTopkThreads) out[i] = -1;
  if (tid == 0) a.ticket[r] = 0u;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.R == 0) return hipSuccess;
  dim3 grid(a.R, a.S_max > 0 ? a.S_max : 1);
  hipLaunchKernelGGL(topk_kernel, grid, dim3(kTopkThreads), 0, st, a);
  return hipGetLastError();
}

int topk_segments(int n_max) { return n_max > kSeg ? (n_max + kSeg - 1) / kSeg : 1; }
int topk_kcap(int k) { return k < kSeg ? k : kSeg; }

}  // namespace csa2
