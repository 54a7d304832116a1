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
#include "select.h"
#include "kernels.h"

namespace csa2 {

CSA2_DEV int64_t row_count(const TopkArgs& a, int r) {
  int64_t n = a.n_max;
  if (a.n_valid) {
    const int64_t v = a.n_valid[a.row_seq ? a.row_seq[r] : r];
    n = v <= 0 ? 0 : (v + a.n_div - 1) / a.n_div;
  }
  return n > a.n_max ? a.n_max : n;
}


// Level l's values of row r, and the number of values of level l over n0
// level-0 values (selects, not an indexed array: a runtime index into an
// array of the kernel's arguments or of locals is served from scratch memory).
CSA2_DEV const float* lv_row(const TopkArgs& a, int l, int r) {
  // the three row bases first, then the choice: a choice between two loads
  // would be folded into one load at a runtime offset
  const float* b0 = a.lv[0] ? a.lv[0] + (int64_t)r * a.lv_stride[0] : nullptr;
  const float* b1 = a.lv[1] ? a.lv[1] + (int64_t)r * a.lv_stride[1] : nullptr;
  const float* b2 = a.lv[2] ? a.lv[2] + (int64_t)r * a.lv_stride[2] : nullptr;
  return (l == 0) ? b0 : (l == 1) ? b1 : b2;
}
CSA2_DEV int64_t lv_count(int64_t n0, int l) {
  return (l == 0) ? n0 : (l == 1) ? (n0 + 7) / 8 : (l == 2) ? (n0 + 63) / 64 : (n0 + 511) / 512;
}

// Threshold path.  tau = the k-th largest value of the top level T (the
// lowest level with at most kRegCap values, taken as maxima of 8 of level T-1
// when level T is not stored).  By the fact above applied level by level,
// tau <= the k-th largest value of every level below, so the top k of level
// 0 lie among the positions whose value is >= tau, and those are found by
// descending through the groups whose value is >= tau.  Only two selections
// run (at the top and among the final survivors), each over at most kRegCap
// keys held in registers.  Returns false -- the row then takes the general
// path -- when a level or the survivors would exceed kRegCap.
CSA2_DEV bool topk_threshold(const TopkArgs& a, int r, int64_t n0, SelSmem& sm, int32_t (*par)[kSelCap / 8],
                             const int32_t* cmap, int32_t* out) {
  const int tid = threadIdx.x;
  const uint32_t K = (uint32_t)a.k;
  int T = 0;
  while (T < 3 && lv_count(n0, T) > kRegCap) ++T;
  const int64_t nT = lv_count(n0, T);
  if (nT > kRegCap) return false;
  const bool direct = (T == 0) || (T <= 2 && lv_row(a, T, r) != nullptr);
  if (!direct && (T - 1 > 2 || lv_row(a, T - 1, r) == nullptr)) return false;
  for (int l = 0; l < T; ++l)
    if (l > 2 || lv_row(a, l, r) == nullptr) return false;

  // ---- top level: 4 values per thread ----
  RegKeys top;
  // top level built from level 0 (T == 1 without stored maxima): the 32
  // level-0 values of this thread's 4 groups stay in registers and are the
  // children of the descent (no reload, no compaction of the top level)
  const bool from0 = !direct && T == 1;
  float v0[kRegPer * 8];
  if (direct) {
    const float* base = lv_row(a, T, r);
    float v[kRegPer];
    if (((uintptr_t)base & 15u) == 0 && kRegPer * tid + kRegPer <= nT) {
      const float4 x = *(const float4*)(base + kRegPer * tid);
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
#pragma unroll
      for (int j = 0; j < kRegPer; ++j) v[j] = base[min((int64_t)(kRegPer * tid + j), nT - 1)];
    }
#pragma unroll
    for (int j = 0; j < kRegPer; ++j) top.v[j] = (kRegPer * tid + j < nT) ? order_key(v[j]) : 0u;
  } else {
    const float* base = lv_row(a, T - 1, r);
    const int64_t nb = lv_count(n0, T - 1);
    float (&v)[kRegPer * 8] = v0;
    if (((uintptr_t)base & 15u) == 0 && 8 * kRegPer * tid + 8 * kRegPer <= nb) {
#pragma unroll
      for (int q = 0; q < 2 * kRegPer; ++q) {
        const float4 x = *(const float4*)(base + 8 * kRegPer * tid + 4 * q);
        v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kRegPer * 8; ++j) v[j] = base[min((int64_t)(8 * kRegPer * tid + j), nb - 1)];
    }
#pragma unroll
    for (int j = 0; j < kRegPer; ++j) {
      uint32_t m = 0u;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        m = max(m, (8 * (kRegPer * tid + j) + c < nb) ? order_key(v[8 * j + c]) : 0u);
      top.v[j] = m;
    }
  }
  CSA2_MARK(a, 9);
  // Above level 0 any threshold at or below the k-th largest value serves
  // (the descent keeps every child >= it), so the search may stop at the
  // first bin edge with at most 1.5 k values above it (usually one pass).
  const uint32_t cap = (T == 0) ? 0u : K + K / 2;
  const SelResult s = block_select(sm, top, K, cap, CSA2_TRACE_PTR(a) ? CSA2_TRACE_PTR(a) + 10 : nullptr);
  CSA2_MARK(a, 1);
  if (T == 0) {
    const uint32_t m = block_compact(sm, top, s, K, [&](uint32_t pos, int e) {
      out[pos] = a.cand_blocks ? cmap[e >> 3] * 8 + (e & 7) : e;
    });
    for (int i = (int)m + tid; i < (int)K; i += kSelThreads) out[i] = -1;
    return true;
  }
  const uint32_t tau = max(s.T, 1u);     // s.T == 0: fewer than k present, all present qualify
  SelResult ge;
  ge.T = tau;
  ge.n_gt = 0;
  ge.n_eq = 0;
  ge.exact = false;
  int cur = 0;
  int n_par = 0;
  if (!from0) {
    n_par = (int)block_compact(sm, top, ge, K, [&](uint32_t pos, int e) { par[0][pos] = e; });
    __syncthreads();
  }

  // ---- descend: children of the kept groups with value >= tau ----
  for (int l = T - 1; l >= 0; --l) {
    const float* base = lv_row(a, l, r);
    const int64_t n = lv_count(n0, l);
    // children of this thread's parents kRegPer*t .. +kRegPer-1; every load
    // is unconditional (clamped index) so all of them are in flight at once
    // (a load under a branch is waited for before the next branch)
    int32_t idx[kRegPer * 8];       // (level counts stay below 2^31)
    float v[kRegPer * 8];
    if (from0) {
      // parents: this thread's own top-level groups kRegPer*t + p
#pragma unroll
      for (int p = 0; p < kRegPer; ++p) {
        const int64_t g = top.v[p] >= tau ? (int64_t)(kRegPer * tid + p) : -1;
#pragma unroll
        for (int c = 0; c < 8; ++c) idx[8 * p + c] = (g >= 0 && g * 8 + c < n) ? (int32_t)(g * 8 + c) : -1;
      }
#pragma unroll
      for (int j = 0; j < kRegPer * 8; ++j) v[j] = v0[j];
    } else {
#pragma unroll
      for (int p = 0; p < kRegPer; ++p) {
        const int pi = kRegPer * tid + p;
        const int64_t g = (pi < n_par) ? (int64_t)par[cur][pi] : -1;
#pragma unroll
        for (int c = 0; c < 8; ++c) idx[8 * p + c] = (g >= 0 && g * 8 + c < n) ? (int32_t)(g * 8 + c) : -1;
      }
#pragma unroll
      for (int j = 0; j < kRegPer * 8; ++j) v[j] = base[idx[j] >= 0 ? idx[j] : 0];
    }
    uint32_t cnt = 0;
    uint32_t keepm = 0;           // bit j: child j kept
#pragma unroll
    for (int j = 0; j < kRegPer * 8; ++j) {
      const bool kp = idx[j] >= 0 && order_key(v[j]) >= tau;
      keepm |= kp ? (1u << j) : 0u;
      cnt += kp ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t pos = block_excl_scan(sm, cnt, tot);
    if (tot > (uint32_t)kRegCap) return false;      // uniform: every thread sees the same total
    int32_t* dst = par[cur ^ 1];
    if (l > 0) {
#pragma unroll
      for (int j = 0; j < kRegPer * 8; ++j)
        if ((keepm >> j) & 1u) dst[pos++] = (int32_t)idx[j];
      __syncthreads();
      cur ^= 1;
      n_par = (int)tot;
      CSA2_MARK(a, 2 + l);
      continue;
    }
    // level 0: survivors (key, position) in index order, then the exact top k
#pragma unroll
    for (int j = 0; j < kRegPer * 8; ++j)
      if ((keepm >> j) & 1u) {
        dst[pos] = (int32_t)idx[j];
        sm.key[pos] = order_key(v[j]);
        ++pos;
      }
    __syncthreads();
    RegKeys sv;
#pragma unroll
    for (int j = 0; j < kRegPer; ++j) {
      const int e = kRegPer * tid + j;
      sv.v[j] = (e < (int)tot) ? sm.key[e] : 0u;
    }
    const SelResult f = block_select(sm, sv, K, 0u);
    CSA2_MARK(a, 6);
    const uint32_t m = block_compact(sm, sv, f, K, [&](uint32_t o, int e) {
      const int32_t i = dst[e];
      out[o] = a.cand_blocks ? cmap[i >> 3] * 8 + (i & 7) : i;
    });
    for (int i = (int)m + tid; i < (int)K; i += kSelThreads) out[i] = -1;
    CSA2_MARK(a, 7);
    return true;
  }
  return true;
}

// General path: at each level keep a superset of the top-k groups bounded by
// 2048 (a radix search that stops early, or the exact top k when ties prevent
// that), descending to the exact top k at level 0.  Handles any value
// distribution; the keys of a level are staged in LDS.
CSA2_DEV void topk_general(const TopkArgs& a, int r, int64_t n0, SelSmem& sm, int32_t (*par)[kSelCap / 8],
                           const int32_t* cmap, int32_t* out) {
  const int tid = threadIdx.x;
  int level = 0;
  if (n0 > kSelCap) level = (lv_count(n0, 1) > kSelCap) ? 2 : 1;
  bool all = true;     // candidates = every index of the level
  int n_par = 0;       // otherwise: children of par[cur][0 .. n_par)
  int cur = 0;
  for (;;) {
    const float* base = lv_row(a, level, r);
    const int64_t n = lv_count(n0, level);
    const int n_elem = all ? (int)n : 8 * n_par;
    // candidates of this level into LDS in index order, padded with absent
    // keys to a multiple of kSelPad; every read is in bounds (an absent
    // candidate reads element 0 of the row, which exists when n_elem > 0)
    const int n_pad = sel_padded(n_elem);
    // two batches of loads in flight per round trip (n_pad is a multiple of kSelPad)
    for (int e00 = tid; e00 < n_pad; e00 += 2 * kSelPad) {
      int64_t src[2 * kSelBatch];
      bool ok[2 * kSelBatch];
#pragma unroll
      for (int j = 0; j < 2 * kSelBatch; ++j) {
        const int e = e00 + j * kSelThreads;
        const int ec = min(e, max(n_elem - 1, 0));
        const int64_t i = all ? (int64_t)ec : (int64_t)par[cur][ec >> 3] * 8 + (ec & 7);
        ok[j] = e < n_elem && i < n;
        src[j] = ok[j] ? i : 0;
      }
      float v[2 * kSelBatch];
#pragma unroll
      for (int j = 0; j < 2 * kSelBatch; ++j) v[j] = base[src[j]];
#pragma unroll
      for (int j = 0; j < 2 * kSelBatch; ++j) {
        const int e = e00 + j * kSelThreads;
        if (e < n_pad) sm.key[skew(e)] = ok[j] ? order_key(v[j]) : 0u;
      }
    }
    __syncthreads();
    const LdsKeys ks{&sm, n_pad};
    auto index_of = [&](int e) -> int64_t {
      return all ? (int64_t)e : (int64_t)par[cur][e >> 3] * 8 + (e & 7);
    };
    if (level > 0) {
      const SelResult s = block_select(sm, ks, (uint32_t)a.k, kSelCap / 8);
      int32_t* dst = par[cur ^ 1];
      const uint32_t m = block_compact(sm, ks, s, (uint32_t)a.k, [&](uint32_t pos, int e) { dst[pos] = (int32_t)index_of(e); });
      __syncthreads();
      all = false;
      n_par = (int)m;
      cur ^= 1;
      --level;
    } else {
      const SelResult s = block_select(sm, ks, (uint32_t)a.k, 0u);
      const uint32_t m = block_compact(sm, ks, s, (uint32_t)a.k, [&](uint32_t pos, int e) {
        const int64_t i = index_of(e);
        out[pos] = a.cand_blocks ? cmap[i >> 3] * 8 + (int32_t)(i & 7) : (int32_t)i;
      });
      for (int i = (int)m + tid; i < a.k; i += kSelThreads) out[i] = -1;
      return;
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void topk_kernel(TopkArgs a) {
  __shared__ SelSmem sm;
  __shared__ int32_t par[2][kSelCap / 8];
  __shared__ int32_t cmap[kSelCap / 8];     // the row's candidate blocks (output index map)
  const int tid = threadIdx.x;
  CSA2_SPAN(a, 256, 0);
  int r = blockIdx.x;
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

constexpr int kTauCap = 8192;             // gathered values a row's final selection holds
constexpr int kTauKeyWords = kTauCap + kTauCap / 32;
constexpr int kSegPer = kSegLen / kSelThreads;   // values per thread of a segment
constexpr int kTopPer = kSelCap / kSelThreads;   // values per thread of the threshold level
static_assert(kTauMaxN / kSegLen <= kWave, "one segment per lane of a wave");
static_assert(kSegLen == 2 * kSelPad, "a segment is two LDS key batches");
static_assert(kTauMaxN <= 8 * kSelCap, "the maxima of 8 of a row fit the threshold level");

__global__ __launch_bounds__(kSelThreads) void seg_tau_gather_kernel(TopkArgs a) {
  __shared__ SelSmemT<1> sm;                       // (the keys stay in registers)
  __shared__ uint32_t cnt[kSegPer * kSelWaves];    // values kept per (round, wave)
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

__global__ __launch_bounds__(kSelThreads) void seg_kth_kernel(TopkArgs a) {
  __shared__ SelSmemT<kSegLen + kSegLen / 32> sm;
  const int s = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
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

struct FinalSmem {
  SelSmemT<kTauKeyWords> sel;     // the gathered keys
  int32_t pos[kTauCap];           // their indices
};
struct GeneralSmem {              // the general path, for a row with more
  SelSmem sel;
  int32_t par[2][kSelCap / 8];
  int32_t cmap[1];                // (no candidate map on this path)
};
union FinalOrGeneral {
  FinalSmem f;
  GeneralSmem g;
};

// The per-segment lists of a row (segment s: length c and inclusive prefix
// inc in lane s, list at rb + s * stride) into LDS at their offsets in the
// concatenation (segment order = index order), keys padded with absent ones to
// a multiple of kSelPad.  Thread t takes element t of every list (all loads at
// once; a segment's lane is a constant, so its length and offset are two
// readlanes), then, rarely, the elements past 512 of a longer list.
template <int MAXSEG>
CSA2_DEV void lists_to_lds(FinalSmem& sm, const uint32_t* keys, const int32_t* pos, int64_t rb, int64_t stride,
                           int nseg, uint32_t c, uint32_t inc, uint32_t total) {
  const int tid = threadIdx.x;
  uint32_t kv[MAXSEG];
  int32_t pv[MAXSEG];
#pragma unroll
  for (int q = 0; q < MAXSEG; ++q) {
    const uint32_t cq = q < nseg ? (uint32_t)__builtin_amdgcn_readlane((int)c, q) : 0u;
    const int64_t g = (uint32_t)tid < cq ? rb + (int64_t)q * stride + tid : rb;
    kv[q] = keys[g];
    pv[q] = pos[g];
  }
  const int n_pad = sel_padded((int)total);
  for (int e = (int)total + tid; e < n_pad; e += kSelThreads) sm.sel.key[skew(e)] = 0u;
#pragma unroll
  for (int q = 0; q < MAXSEG; ++q) {
    const uint32_t cq = q < nseg ? (uint32_t)__builtin_amdgcn_readlane((int)c, q) : 0u;
    const uint32_t sq = q < nseg ? (uint32_t)__builtin_amdgcn_readlane((int)inc, q) - cq : 0u;
    if ((uint32_t)tid < cq) {
      sm.sel.key[skew((int)(sq + tid))] = kv[q];
      sm.pos[sq + tid] = pv[q];
    }
    for (uint32_t i = tid + kSelThreads; i < cq; i += kSelThreads) {
      const int64_t g = rb + (int64_t)q * stride + i;
      sm.sel.key[skew((int)(sq + i))] = keys[g];
      sm.pos[sq + i] = pos[g];
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void seg_final_kernel(TopkArgs a) {
  __shared__ FinalOrGeneral u;
  FinalSmem& sm = u.f;
  const int r = blockIdx.x, tid = threadIdx.x;
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
  const SelResult res = block_select(sm.sel, ks, K, 0u, CSA2_TRACE_PTR(a) ? CSA2_TRACE_PTR(a) + 24 : nullptr);
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
__global__ __launch_bounds__(kSelThreads) void desc_seg_kernel(TopkArgs a) {
  constexpr int kSeg = SEGPER * kSelThreads;
  __shared__ SelSmemT<1> sm;                  // the keys stay in registers
  __shared__ uint32_t cnt[SEGPER * kSelWaves];
  __shared__ int32_t cm[kSeg / 8];            // the segment's candidate blocks
  const int s = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
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

struct DescGeneralSmem {          // the general path of a marked row
  SelSmem sel;
  int32_t par[2][kSelCap / 8];
  int32_t cmap[kSelCap / 8];
};
union DescFinalSmem {
  FinalSmem f;
  DescGeneralSmem g;
};

__global__ __launch_bounds__(kSelThreads) void desc_final_kernel(TopkArgs a) {
  __shared__ DescFinalSmem u;
  FinalSmem& sm = u.f;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63;
  const uint32_t K = (uint32_t)a.k;
  int32_t* out = a.out + (int64_t)r * a.out_stride;
  const int64_t n0 = row_count(a, r);
  if (n0 == 0) {
    for (int i = tid; i < a.k; i += kSelThreads) out[i] = -1;
    return;
  }
  CSA2_MARK(a, 3);
  // list lengths (one segment per lane; every wave alike) and, in the same
  // round of loads, the fixed register slots of the fast path below: segment
  // s owns slots [spp s, spp (s+1)), thread t slots 4t .. 4t+3
  const uint32_t c = lane < a.nseg ? a.seg_cnt[(int64_t)r * a.nseg + lane] : 0u;
  const int64_t rb = (int64_t)r * a.nseg * kDescCap;
  const int spp = min(kRegCap / a.nseg, kDescCap) & ~(kRegPer - 1);
  const int sg = kRegPer * tid / spp, sl0 = kRegPer * tid - sg * spp;
  const int64_t g0 = sg < a.nseg ? rb + (int64_t)sg * kDescCap + sl0 : rb;
  const uint4 kk = *(const uint4*)(a.seg_key + g0);
  const int4 pp = *(const int4*)(a.seg_pos + g0);
  const bool marked = __ballot(c > (uint32_t)kDescCap) != 0ull;
  const uint32_t inc = wave_incl_scan_u32(c);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  if (marked || total > (uint32_t)kTauCap) {
    if (a.cand_blocks)
      for (int i = tid; i < a.cand_stride; i += kSelThreads) u.g.cmap[i] = a.cand_blocks[(int64_t)r * a.cand_stride + i];
    __syncthreads();
    if (!topk_threshold(a, r, n0, u.g.sel, u.g.par, u.g.cmap, out)) {
      __syncthreads();
      topk_general(a, r, n0, u.g.sel, u.g.par, u.g.cmap, out);
    }
    return;
  }
  // Fast path: every list fits its slots.  Thread order is then (segment,
  // list position) order = index order; slots past a list's length are absent.
  {
    const bool fits = __ballot(c > (uint32_t)spp) == 0ull;
    if (fits) {
      const uint32_t cs = (uint32_t)__shfl((int)c, sg < a.nseg ? sg : 0, 64);
      RegKeys ks;
      ks.v[0] = (sg < a.nseg && (uint32_t)sl0 + 0u < cs) ? kk.x : 0u;
      ks.v[1] = (sg < a.nseg && (uint32_t)sl0 + 1u < cs) ? kk.y : 0u;
      ks.v[2] = (sg < a.nseg && (uint32_t)sl0 + 2u < cs) ? kk.z : 0u;
      ks.v[3] = (sg < a.nseg && (uint32_t)sl0 + 3u < cs) ? kk.w : 0u;
      CSA2_MARK(a, 4);
      const SelResult res = block_select(sm.sel, ks, K, 0u);
      const uint32_t m = block_compact(sm.sel, ks, res, K, [&](uint32_t o, int e) {
        const int j = e & (kRegPer - 1);
        out[o] = (j == 0) ? pp.x : (j == 1) ? pp.y : (j == 2) ? pp.z : pp.w;
      });
      for (int i = (int)m + tid; i < a.k; i += kSelThreads) out[i] = -1;
      CSA2_MARK(a, 5);
      return;
    }
  }
  // lists longer than their slots: concatenated in LDS
  const int n_pad = sel_padded((int)total);
  lists_to_lds<kDescMaxSeg>(sm, a.seg_key, a.seg_pos, rb, kDescCap, a.nseg, c, inc, total);
  __syncthreads();
  const LdsKeysT<SelSmemT<kTauKeyWords>> ks{&sm.sel, n_pad};
  const SelResult res = block_select(sm.sel, ks, K, 0u);
  const uint32_t m = block_compact(sm.sel, ks, res, K, [&](uint32_t o, int e) { out[o] = sm.pos[e]; });
  for (int i = (int)m + tid; i < a.k; i += kSelThreads) out[i] = -1;
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
hipError_t launch_topk_desc(const TopkArgs& a, hipStream_t st) {
  if (a.R == 0) return hipSuccess;
  if (a.n_max <= 16 * 2 * kSelThreads)
    hipLaunchKernelGGL(desc_seg_kernel<2>, dim3(a.nseg, a.R), dim3(kSelThreads), 0, st, a);
  else
    hipLaunchKernelGGL(desc_seg_kernel<8>, dim3(a.nseg, a.R), dim3(kSelThreads), 0, st, a);
  hipLaunchKernelGGL(desc_final_kernel, dim3(a.R), dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
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
