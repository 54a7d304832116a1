// Exact Top-k selection (the "Top-512" of the CSA2 Full and Reindex layers and
// the 2048 candidate blocks of the hierarchical indexer: conexaotc.com.br page
// "DeepSeek lança V4.1-Flash...", paragraph on CSA2).
//
// Order: value descending, index ascending (-0 below +0); -inf = absent;
// output ascending indices, -1 padding.
//
// Three paths share the selection primitives of select.h: the split path
// (desc_seg_kernel + desc_final_kernel, below) for k below 1024 on rows of up
// to 131072 values, the large-k path (seg_*_kernel) for the 2048 candidate
// blocks, and topk_kernel for every other shape and as the fallback of both.
//
// topk_kernel: one block per row descends a tree of maxima.  Level 0 holds the n values;
// level l+1 holds the maximum of each group of 8 consecutive level-l values
// (the indexer scan emits levels 1 and 2 as it scores; `maxima_kernel` builds
// them for other callers).  The descent rests on one fact: if a group holds an
// element of the top k of its level, the group's maximum is in the top k of
// the level above.  (Were k groups ranked above it, each would contain an
// element ranked above that element -- with equal values the group with the
// lower index holds the lower element indices -- so it would not be in the top
// k.)  Hence, starting at the coarsest level with at most 16384 values:
//   * keep a superset of the level's top-k groups: every group whose maximum
//     is at or above a bin edge T with k <= #{>= T} <= 2048 (a radix search
//     that stops early) -- or, when ties prevent that, the exact top k;
//   * the children of the kept groups (at most 2048 * 8 = 16384 values, in
//     index order) are the candidates one level down;
//   * at level 0 the exact top k is taken (ties cut by index) and written in
//     index order.
#include "topk_row.h"
#include "merge_row.h"

namespace csa2 {

// One block's work; every kernel of this file is a thin launch of such a
// function (block index -> (segment, row)), so that two of them can share a
// launch (topk_kth_kernel, desc_seg_tau_kernel, attn.hip's merge_final_kernel).
CSA2_DEV void topk_block(const TopkArgs& a, int r0) {
  __shared__ SelSmem sm;
  __shared__ int32_t par[2][kSelCap / 8];
  __shared__ int32_t cmap[kSelCap / 8];     // the row's candidate blocks (output index map)
  const int tid = threadIdx.x;
  CSA2_SPAN(a, 256, 0);
  int r = r0;
  if (a.row_list) {
    if ((uint32_t)r >= *a.row_list_count) return;
    r = a.row_list[r];
  }
  if (a.cand_blocks)
    for (int i = tid; i < a.cand_stride; i += kSelThreads) cmap[i] = a.cand_blocks[(int64_t)r * a.cand_stride + i];
  const int64_t n0 = row_count(a, r);
  int32_t* out = a.out + (int64_t)r * a.out_stride;
  CSA2_MARK(a, 0);
  if (n0 == 0) {
    for (int i = tid; i < a.k; i += kSelThreads) out[i] = -1;
    return;
  }
  __syncthreads();   // cmap visible
  if (!topk_threshold(a, r, n0, sm, par, cmap, out)) {
    __syncthreads();
    topk_general(a, r, n0, sm, par, cmap, out);
  }
  CSA2_MARK(a, 8);
  CSA2_SPAN(a, 256, 1);
}


// ---- large k over a long row (the 2048 candidate blocks of a hierarchical
// indexer at up to 1M positions) ----
//
// seg_tau_gather_kernel, grid (segments of kSegLen level-0 values, rows):
// every block of a row takes the same threshold tau from the row's lowest
// level of at most kSelCap values (level 0 on rows of at most kSelCap values,
// else the maxima of 8), held in registers: a bin edge with k <= #{level
// values >= tau} <= 1.5 k (tau = 1, every present value, when at most k are
// present).  Each level value >= tau is the maximum of its own group, so at
// least k level-0 values are >= tau and the row's top k lie among them.  The
// block gathers its segment's values >= tau, in index order, into the
// segment's own list (every segment on its own CU: one CU fetching the whole
// row is bound by the misses it keeps in flight).
// seg_final_kernel, one block per row: the lists concatenated in segment
// order (= index order) and the exact top k of them; a row with more than
// kTauCap gathered values takes the general path in the same block.

CSA2_DEV void seg_tau_gather_block(const TopkArgs& a, int s, int r) {
  __shared__ SelSmemT<1> sm;                       // (the keys stay in registers)
  __shared__ uint32_t cnt[kSegPer * kSelWaves];    // values kept per (round, wave)
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int64_t n0 = row_count(a, r);
  const int64_t lo = (int64_t)s * kSegLen;
  const int n = (int)max((int64_t)0, min(n0 - lo, (int64_t)kSegLen));
  const int64_t rs = (int64_t)r * a.nseg + s;
  if (n == 0) {
    if (tid == 0) a.seg_cnt[rs] = 0u;
    return;
  }
  // every load at once: the threshold level (element t + 512 j) and the
  // segment (element t + 512 j: coalesced; index order = (round, wave, lane))
  const int T = n0 <= kSelCap ? 0 : 1;
  const int64_t nT = lv_count(n0, T);
  const float* tb = lv_row(a, T, r);
  float tv[kTopPer];
#pragma unroll
  for (int j = 0; j < kTopPer; ++j) tv[j] = tb[min((int64_t)(tid + j * kSelThreads), nT - 1)];
  const float* base = a.lv[0] + (int64_t)r * a.lv_stride[0] + lo;
  float v[kSegPer];
#pragma unroll
  for (int j = 0; j < kSegPer; ++j) v[j] = base[min(tid + j * kSelThreads, n - 1)];
  RegKeysN<kTopPer> top;
#pragma unroll
  for (int j = 0; j < kTopPer; ++j) top.v[j] = (tid + j * kSelThreads < nT) ? order_key(tv[j]) : 0u;
  const uint32_t K = (uint32_t)a.k;
  const SelResult sr = block_select(sm, top, K, K + K / 2);
  const uint32_t tau = max(sr.T, 1u);
  uint32_t keepm = 0u;
#pragma unroll
  for (int j = 0; j < kSegPer; ++j) {
    const bool kp = tid + j * kSelThreads < n && order_key(v[j]) >= tau;
    keepm |= kp ? (1u << j) : 0u;
    const uint64_t b = __ballot(kp);
    if (lane == 0) cnt[j * kSelWaves + wv] = (uint32_t)__popcll(b);
  }
  __syncthreads();
  // offsets of the (round, wave) runs: an exclusive scan in that order
  uint32_t tot;
  const uint32_t off = block_excl_scan(sm, tid < kSegPer * kSelWaves ? cnt[tid] : 0u, tot);
  if (tid < kSegPer * kSelWaves) cnt[tid] = off;
  __syncthreads();
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  uint32_t* kd = a.seg_key + rs * kSegLen;
  int32_t* pd = a.seg_pos + rs * kSegLen;
#pragma unroll
  for (int j = 0; j < kSegPer; ++j) {
    const bool kp = (keepm >> j) & 1u;
    const uint64_t b = __ballot(kp);
    if (kp) {
      const uint32_t p = cnt[j * kSelWaves + wv] + (uint32_t)__popcll(b & lt_mask);
      kd[p] = order_key(v[j]);
      pd[p] = (int32_t)(lo + tid + j * kSelThreads);
    }
  }
  if (tid == 0) a.seg_cnt[rs] = tot;
}

// Rows longer than kSelCap values: the threshold per segment instead, from
// the segment's own values, in a launch of its own (seg_kth_kernel: on rows of
// at least 32 k values from the segment's 1024 maxima of 8, in registers); the
// minimum over the row's segments tau has at least k values at or above it,
// and seg_gather_kernel gathers each segment's values >= tau.  (One block
// per segment selecting over the row's 16384 maxima of 8 costs more than the
// extra launch.)

CSA2_DEV void seg_kth_block(const TopkArgs& a, int s, int r) {
  __shared__ SelSmemT<kSegLen + kSegLen / 32> sm;
  const int tid = threadIdx.x;
  const int64_t n0 = row_count(a, r);
  const int64_t lo = (int64_t)s * kSegLen;
  const int n = (int)max((int64_t)0, min(n0 - lo, (int64_t)kSegLen));
  if (n == 0) {
    if (tid == 0) a.seg_kth[(int64_t)r * a.nseg + s] = 0xFFFFFFFFu;
    return;
  }
  const uint32_t m_s = (uint32_t)(((int64_t)a.k * n + n0 - 1) / n0);
  if (a.lv[1] && n0 >= 32 * (int64_t)a.k) {
    // the segment's level-1 values (maxima of 8): each is the maximum of its
    // own group of level-0 values, so a key with m_s of them at or above it
    // has m_s level-0 values at or above it (1024 keys in registers; on rows
    // of at least 32 k values, m_s is at most a quarter of them)
    const int64_t n1 = lv_count(n0, 1);
    const int64_t lo1 = lo / 8;
    const int m1 = (int)max((int64_t)0, min(n1 - lo1, (int64_t)(kSegLen / 8)));
    const float* b1 = a.lv[1] + (int64_t)r * a.lv_stride[1] + lo1;
    RegKeys ks;
#pragma unroll
    for (int j = 0; j < kRegPer; ++j) {
      const int e = kRegPer * tid + j;
      const float x = b1[min(e, m1 - 1)];
      ks.v[j] = e < m1 ? order_key(x) : 0u;
    }
    const SelResult res = block_select(sm, ks, m_s, 2u * m_s);
    if (tid == 0) a.seg_kth[(int64_t)r * a.nseg + s] = res.T;
    return;
  }
  const float* base = a.lv[0] + (int64_t)r * a.lv_stride[0] + lo;
  float v[kSegPer];
#pragma unroll
  for (int j = 0; j < kSegPer; ++j) v[j] = base[min(tid + j * kSelThreads, n - 1)];
#pragma unroll
  for (int j = 0; j < kSegPer; ++j) {
    const int e = tid + j * kSelThreads;
    sm.key[skew(e)] = e < n ? order_key(v[j]) : 0u;
  }
  __syncthreads();
  const LdsKeysT<SelSmemT<kSegLen + kSegLen / 32>> ks{&sm, kSegLen};
  // any key with at least m_s values at or above it serves: stop at the first
  // bin edge with at most 2 m_s above it
  const SelResult res = block_select(sm, ks, m_s, 2u * m_s);
  if (tid == 0) a.seg_kth[(int64_t)r * a.nseg + s] = res.T;
}

// tau of row r: the minimum of its segment keys (every lane of every wave)
CSA2_DEV uint32_t row_tau(const TopkArgs& a, int r) {
  const int lane = threadIdx.x & 63;
  const uint32_t t = lane < a.nseg ? a.seg_kth[(int64_t)r * a.nseg + lane] : 0xFFFFFFFFu;
  return max(wave_min_u32(t), 1u);
}

struct GatherSmem {
  uint32_t wa[kSelWaves];
  uint32_t cnt[kSegPer * kSelWaves];   // values kept per (round, wave)
};

__global__ __launch_bounds__(kSelThreads) void seg_gather_kernel(TopkArgs a) {
  __shared__ GatherSmem sm;
  const int s = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int64_t n0 = row_count(a, r);
  const int64_t lo = (int64_t)s * kSegLen;
  const int n = (int)max((int64_t)0, min(n0 - lo, (int64_t)kSegLen));
  const int64_t rs = (int64_t)r * a.nseg + s;
  if (n == 0) {
    if (tid == 0) a.seg_cnt[rs] = 0u;
    return;
  }
  const uint32_t tau = row_tau(a, r);
  // element e = 512 j + 64 w + l: round j, wave w, lane l (coalesced loads;
  // index order = (round, wave, lane) order)
  const float* base = a.lv[0] + (int64_t)r * a.lv_stride[0] + lo;
  float v[kSegPer];
#pragma unroll
  for (int j = 0; j < kSegPer; ++j) v[j] = base[min(tid + j * kSelThreads, n - 1)];
  uint32_t keepm = 0u;
#pragma unroll
  for (int j = 0; j < kSegPer; ++j) {
    const bool kp = tid + j * kSelThreads < n && order_key(v[j]) >= tau;
    keepm |= kp ? (1u << j) : 0u;
    const uint64_t b = __ballot(kp);
    if (lane == 0) sm.cnt[j * kSelWaves + wv] = (uint32_t)__popcll(b);
  }
  __syncthreads();
  // offsets of the (round, wave) runs: an exclusive scan in that order
  uint32_t tot;
  const uint32_t off = block_excl_scan(sm, tid < kSegPer * kSelWaves ? sm.cnt[tid] : 0u, tot);
  __syncthreads();
  if (tid < kSegPer * kSelWaves) sm.cnt[tid] = off;
  __syncthreads();
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  uint32_t* kd = a.seg_key + rs * kSegLen;
  int32_t* pd = a.seg_pos + rs * kSegLen;
#pragma unroll
  for (int j = 0; j < kSegPer; ++j) {
    const bool kp = (keepm >> j) & 1u;
    const uint64_t b = __ballot(kp);
    if (kp) {
      const uint32_t p = sm.cnt[j * kSelWaves + wv] + (uint32_t)__popcll(b & lt_mask);
      kd[p] = order_key(v[j]);
      pd[p] = (int32_t)(lo + tid + j * kSelThreads);
    }
  }
  if (tid == 0) a.seg_cnt[rs] = tot;
}

CSA2_DEV void seg_final_block(const TopkArgs& a, int r) {
  __shared__ FinalOrGeneral u;
  FinalSmem& sm = u.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint32_t K = (uint32_t)a.k;
  int32_t* out = a.out + (int64_t)r * a.out_stride;
  const int64_t n0 = row_count(a, r);
  if (n0 == 0) {
    for (int i = tid; i < a.k; i += kSelThreads) out[i] = -1;
    return;
  }
  CSA2_MARK(a, 20);
  // segment counts and their offsets (one segment per lane; every wave alike)
  // and, in the same round of loads, the fixed register slots of the fast
  // path below: segment s owns slots [spp s, spp (s+1)), thread t slots
  // 16t .. 16t+15
  const int nseg = (int)((n0 + kSegLen - 1) / kSegLen);
  const uint32_t c = lane < nseg ? a.seg_cnt[(int64_t)r * a.nseg + lane] : 0u;
  constexpr int kPer = kTauCap / kSelThreads;
  const int spp = min(kTauCap / nseg, kSegLen) & ~(kPer - 1);
  const int sg = kPer * tid / spp, sl0 = kPer * tid - sg * spp;
  const int64_t rb0 = (int64_t)r * a.nseg * kSegLen;
  const int64_t g0 = sg < nseg ? rb0 + (int64_t)sg * kSegLen + sl0 : rb0;
  uint32_t kk[kPer];
  int32_t pp[kPer];
#pragma unroll
  for (int q = 0; q < kPer / 4; ++q) {
    const uint4 x = *(const uint4*)(a.seg_key + g0 + 4 * q);
    const int4 y = *(const int4*)(a.seg_pos + g0 + 4 * q);
    kk[4 * q] = x.x; kk[4 * q + 1] = x.y; kk[4 * q + 2] = x.z; kk[4 * q + 3] = x.w;
    pp[4 * q] = y.x; pp[4 * q + 1] = y.y; pp[4 * q + 2] = y.z; pp[4 * q + 3] = y.w;
  }
  const uint32_t inc = wave_incl_scan_u32(c);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  if (total > (uint32_t)kTauCap) {
    // too many values at or above tau (ties, or scores that favour one
    // segment): this block takes the row through the general path
    if (!topk_threshold(a, r, n0, u.g.sel, u.g.par, u.g.cmap, out)) {
      __syncthreads();
      topk_general(a, r, n0, u.g.sel, u.g.par, u.g.cmap, out);
    }
    return;
  }
  // fast path: every list fits its slots; thread order is then (segment,
  // list position) order = index order, slots past a list's length absent
  if (__ballot(c > (uint32_t)spp) == 0ull) {
    const uint32_t cs = (uint32_t)__shfl((int)c, sg < nseg ? sg : 0, 64);
    RegKeysN<kPer> ks;
#pragma unroll
    for (int j = 0; j < kPer; ++j) ks.v[j] = (sg < nseg && (uint32_t)(sl0 + j) < cs) ? kk[j] : 0u;
    CSA2_MARK(a, 21);
    const SelResult res = block_select(sm.sel, ks, K, 0u);
    CSA2_MARK(a, 22);
    const uint32_t m = block_compact(sm.sel, ks, res, K, [&](uint32_t o, int e) { out[o] = pp[e & (kPer - 1)]; });
    for (int i = (int)m + tid; i < a.k; i += kSelThreads) out[i] = -1;
    CSA2_MARK(a, 23);
    return;
  }
  const int n_pad = sel_padded((int)total);
  lists_to_lds<kTauMaxN / kSegLen>(sm, a.seg_key, a.seg_pos, rb0, kSegLen, nseg, c, inc, total);
  __syncthreads();
  CSA2_MARK(a, 21);
  const LdsKeysT<SelSmemT<kTauKeyWords>> ks{&sm.sel, n_pad};
  const SelResult res = block_select(sm.sel, ks, K, 0u, CSA2_TRACE_AT(a, 24));
  CSA2_MARK(a, 22);
  const uint32_t m = block_compact(sm.sel, ks, res, K, [&](uint32_t o, int e) { out[o] = sm.pos[e]; });
  for (int i = (int)m + tid; i < a.k; i += kSelThreads) out[i] = -1;
  CSA2_MARK(a, 23);
}

// ---- Top-k spread over the CUs: k below 1024 over rows of at most kDescMaxN
// values whose top level (the lowest level with at most kRegCap values) is
// stored ----
//
// One block per row descending the tree is bound by the cache misses one CU
// keeps in flight (the children of ~1000 groups at two levels).  Instead:
// desc_seg_kernel, grid (segments, rows), segments of SEGPER * 512 level-0
// values: every block of a row loads the row's top level and finds the same
// bin edge tau with k <= #{top-level values >= tau} <= 1.5 k (tau = 1, every
// present value, when at most k are present).  Each of those top-level values
// is the maximum of its own group of level-0 values, so at least k level-0
// values are >= tau: the row's k-th largest value is >= tau and its top k lie
// among the level-0 values >= tau.  The block's segment of level 0, loaded in
// full at the start (in flight while tau is found), is filtered at tau into
// the segment's list in index order; a segment with more than kDescCap such
// values marks the row.  desc_final_kernel, one block per row: the lists
// concatenated in segment order (= index order) and the exact top k; a marked
// row, or one with more than kTauCap listed values, takes the general path in
// the same block.

template <int SEGPER>
CSA2_DEV void desc_seg_block(const TopkArgs& a, int s, int r) {
  constexpr int kSeg = SEGPER * kSelThreads;
  __shared__ SelSmemT<1> sm;                  // the keys stay in registers
  __shared__ uint32_t cnt[SEGPER * kSelWaves];
  __shared__ int32_t cm[kSeg / 8];            // the segment's candidate blocks
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const uint32_t K = (uint32_t)a.k;
  const int64_t n0 = row_count(a, r);
  const int64_t rs = (int64_t)r * a.nseg + s;
  const int64_t lo = (int64_t)s * kSeg;
  const int n = (int)max((int64_t)0, min(n0 - lo, (int64_t)kSeg));
  if (n == 0) {
    if (tid == 0) a.seg_cnt[rs] = 0u;
    return;
  }
  CSA2_MARK(a, 0);
  int T = 0;
  while (T < 2 && lv_count(n0, T) > kRegCap) ++T;
  const int64_t nT = lv_count(n0, T);
  // every load at once: the top level, the segment, its candidate blocks
  const float* tb = lv_row(a, T, r);
  float tv[kRegPer];
  if (((uintptr_t)tb & 15u) == 0 && kRegPer * tid + kRegPer <= nT) {
    const float4 x = *(const float4*)(tb + kRegPer * tid);
    tv[0] = x.x; tv[1] = x.y; tv[2] = x.z; tv[3] = x.w;
  } else {
#pragma unroll
    for (int j = 0; j < kRegPer; ++j) tv[j] = tb[min((int64_t)(kRegPer * tid + j), nT - 1)];
  }
  const float* base = a.lv[0] + (int64_t)r * a.lv_stride[0] + lo;
  float v[SEGPER];
#pragma unroll
  for (int j = 0; j < SEGPER; ++j) v[j] = base[min(tid + j * kSelThreads, n - 1)];
  int32_t cbv = 0;
  if (a.cand_blocks && tid < kSeg / 8) {
    const int64_t cb = min((lo >> 3) + tid, (int64_t)a.cand_stride - 1);
    cbv = a.cand_blocks[(int64_t)r * a.cand_stride + cb];
  }
  RegKeys top;
#pragma unroll
  for (int j = 0; j < kRegPer; ++j) top.v[j] = (kRegPer * tid + j < nT) ? order_key(tv[j]) : 0u;
  const SelResult sr = block_select(sm, top, K, K + K / 2);
  const uint32_t tau = max(sr.T, 1u);
  CSA2_MARK(a, 1);
  if (a.cand_blocks && tid < kSeg / 8) cm[tid] = cbv;
  // the kept values in (round, wave, lane) order = index order
  uint32_t keepm = 0u;
#pragma unroll
  for (int j = 0; j < SEGPER; ++j) {
    const bool kp = tid + j * kSelThreads < n && order_key(v[j]) >= tau;
    keepm |= kp ? (1u << j) : 0u;
    const uint64_t b = __ballot(kp);
    if (lane == 0) cnt[j * kSelWaves + wv] = (uint32_t)__popcll(b);
  }
  __syncthreads();
  uint32_t tot;
  const uint32_t off = block_excl_scan(sm, tid < SEGPER * kSelWaves ? cnt[tid] : 0u, tot);
  if (tid < SEGPER * kSelWaves) cnt[tid] = off;
  __syncthreads();
  if (tot > (uint32_t)kDescCap) {           // uniform
    if (tid == 0) a.seg_cnt[rs] = (uint32_t)kDescCap + 1u;
    return;
  }
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  uint32_t* kd = a.seg_key + rs * kDescCap;
  int32_t* pd = a.seg_pos + rs * kDescCap;
#pragma unroll
  for (int j = 0; j < SEGPER; ++j) {
    const bool kp = (keepm >> j) & 1u;
    const uint64_t b = __ballot(kp);
    if (kp) {
      const uint32_t p = cnt[j * kSelWaves + wv] + (uint32_t)__popcll(b & lt_mask);
      const int e = tid + j * kSelThreads;
      kd[p] = order_key(v[j]);
      pd[p] = a.cand_blocks ? cm[e >> 3] * 8 + (e & 7) : (int32_t)(lo + e);
    }
  }
  if (tid == 0) a.seg_cnt[rs] = tot;
  CSA2_MARK(a, 2);
}

__global__ __launch_bounds__(kSelThreads) void topk_kernel(TopkArgs a) { topk_block(a, blockIdx.x); }
__global__ __launch_bounds__(kSelThreads) void seg_tau_gather_kernel(TopkArgs a) {
  seg_tau_gather_block(a, blockIdx.x, blockIdx.y);
}
__global__ __launch_bounds__(kSelThreads) void seg_kth_kernel(TopkArgs a) { seg_kth_block(a, blockIdx.x, blockIdx.y); }
__global__ __launch_bounds__(kSelThreads) void seg_final_kernel(TopkArgs a) { seg_final_block(a, blockIdx.x); }
template <int SEGPER>
__global__ __launch_bounds__(kSelThreads) void desc_seg_kernel(TopkArgs a) {
  desc_seg_block<SEGPER>(a, blockIdx.x, blockIdx.y);
}

// Two independent pieces of a group step in one launch (both read only the
// scan's outputs): blocks [0, d.nseg * d.R) build the split Top-512's segment
// lists, the rest take the candidate blocks' threshold and gather
// (seg_tau_gather); the candidates' final selection joins the merge launch.
template <int SEGPER>
__global__ __launch_bounds__(kSelThreads) void desc_seg_tau_kernel(TopkArgs d, TopkArgs g) {
  const int nd = d.nseg * d.R;
  const int b = blockIdx.x;
  if (b < nd) {
    desc_seg_block<SEGPER>(d, b % d.nseg, b / d.nseg);
  } else {
    const int b2 = b - nd;
    seg_tau_gather_block(g, b2 % g.nseg, b2 / g.nseg);
  }
}
// ... and for rows past kSelCap block maxima: blocks [0, t.R) take the
// Top-512 one row per block, the rest the candidate segments' thresholds
// (seg_kth), which the one-block rows leave most CUs free for.
__global__ __launch_bounds__(kSelThreads) void topk_kth_kernel(TopkArgs t, TopkArgs g) {
  const int b = blockIdx.x;
  if (b < t.R) {
    topk_block(t, b);
  } else {
    const int b2 = b - t.R;
    seg_kth_block(g, b2 % g.nseg, b2 / g.nseg);
  }
}

// The attention's merge and the candidate blocks' final selection in one
// launch of 512-thread blocks: the first ceil(4 n_layers R / 2) each run two
// merge blocks of 256 threads, the rest one final selection (seg_final) each.
__global__ __launch_bounds__(kSelThreads) void merge_final_kernel(AttnArgs a, TopkArgs g) {
  const int nm = 4 * a.n_layers * a.R;
  const int np = (nm + 1) / 2;
  const int b = blockIdx.x;
  if (b < np) {
    const int unit = 2 * b + (int)(threadIdx.x >> 8);
    if (unit < nm) merge_block(a, unit, threadIdx.x & 255);
  } else {
    seg_final_block(g, b - np);
  }
}

hipError_t launch_merge_final(const AttnArgs& a, const TopkArgs& g, hipStream_t st) {
  const int nm = 4 * a.n_layers * a.R;
  hipLaunchKernelGGL(merge_final_kernel, dim3((unsigned)((nm + 1) / 2 + g.R)), dim3(kSelThreads), 0, st, a, g);
  return hipGetLastError();
}
hipError_t launch_seg_final(const TopkArgs& g, hipStream_t st) {
  if (g.R == 0) return hipSuccess;
  hipLaunchKernelGGL(seg_final_kernel, dim3(g.R), dim3(kSelThreads), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_desc_seg_tau(const TopkArgs& d, const TopkArgs& g, hipStream_t st) {
  if (d.R == 0) return hipSuccess;
  const unsigned nb = (unsigned)(d.nseg * d.R + g.nseg * g.R);
  if (d.n_max <= 16 * 2 * kSelThreads)
    hipLaunchKernelGGL(desc_seg_tau_kernel<2>, dim3(nb), dim3(kSelThreads), 0, st, d, g);
  else
    hipLaunchKernelGGL(desc_seg_tau_kernel<8>, dim3(nb), dim3(kSelThreads), 0, st, d, g);
  return hipGetLastError();
}
hipError_t launch_topk_kth_gather(const TopkArgs& t, const TopkArgs& g, hipStream_t st) {
  if (t.R == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kth_kernel, dim3((unsigned)(t.R + g.nseg * g.R)), dim3(kSelThreads), 0, st, t, g);
  hipLaunchKernelGGL(seg_gather_kernel, dim3(g.nseg, g.R), dim3(kSelThreads), 0, st, g);
  return hipGetLastError();
}

__global__ __launch_bounds__(kSelThreads) void desc_final_kernel(TopkArgs a) {
  __shared__ DescFinalSmem u;
  const int r = blockIdx.x;
  desc_final_row(a, r, u, a.out + (int64_t)r * a.out_stride);
}

// out[r][g] = maximum (in the Top-k order) of in[r][8g .. 8g+7] below the
// row's count, -inf when none is present.  The row's count at this level is
// ceil(n0 / div) with n0 the level-0 count of the row.
__global__ __launch_bounds__(256) void maxima_kernel(MaximaArgs a) {
  const int64_t total = (int64_t)a.R * a.n_out_max;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(t / a.n_out_max);
    const int64_t g = t - (int64_t)r * a.n_out_max;
    int64_t n0 = a.n_max;
    if (a.n_valid) {
      const int64_t v = a.n_valid[a.row_seq ? a.row_seq[r] : r];
      n0 = v <= 0 ? 0 : (v + a.n_div - 1) / a.n_div;
      if (n0 > a.n_max) n0 = a.n_max;
    }
    const int64_t n_in = (n0 + a.div_in - 1) / a.div_in;
    if (g * 8 >= n_in) continue;
    const float* src = a.in + (int64_t)r * a.in_stride + g * 8;
    uint32_t k = 0u;
    for (int c = 0; c < 8 && g * 8 + c < n_in; ++c) k = max(k, order_key(src[c]));
    a.out[(int64_t)r * a.out_stride + g] = k ? key_to_float(k) : -__builtin_inff();
  }
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  if (a.R == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(a.R), dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
}

// Large k over rows of at most kTauMaxN values: the per-segment gather above
// the row's threshold, the final selection.
hipError_t launch_topk_large(const TopkArgs& a, hipStream_t st) {
  if (a.R == 0) return hipSuccess;
  if (a.n_max <= kSelCap) {
    hipLaunchKernelGGL(seg_tau_gather_kernel, dim3(a.nseg, a.R), dim3(kSelThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL(seg_kth_kernel, dim3(a.nseg, a.R), dim3(kSelThreads), 0, st, a);
    hipLaunchKernelGGL(seg_gather_kernel, dim3(a.nseg, a.R), dim3(kSelThreads), 0, st, a);
  }
  hipLaunchKernelGGL(seg_final_kernel, dim3(a.R), dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
}

// Top-k spread over the CUs: segments of 1024 values for rows of at most
// 16384 (top level 1), else of 4096 (top level 2).
hipError_t launch_desc_seg(const TopkArgs& a, hipStream_t st) {
  if (a.R == 0) return hipSuccess;
  if (a.n_max <= 16 * 2 * kSelThreads)
    hipLaunchKernelGGL(desc_seg_kernel<2>, dim3(a.nseg, a.R), dim3(kSelThreads), 0, st, a);
  else
    hipLaunchKernelGGL(desc_seg_kernel<8>, dim3(a.nseg, a.R), dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_desc_final(const TopkArgs& a, hipStream_t st) {
  if (a.R == 0) return hipSuccess;
  hipLaunchKernelGGL(desc_final_kernel, dim3(a.R), dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_topk_desc(const TopkArgs& a, hipStream_t st) {
  const hipError_t e = launch_desc_seg(a, st);
  return e != hipSuccess ? e : launch_desc_final(a, st);
}

hipError_t launch_maxima(const MaximaArgs& a, hipStream_t st) {
  const int64_t total = (int64_t)a.R * a.n_out_max;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(maxima_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa2
