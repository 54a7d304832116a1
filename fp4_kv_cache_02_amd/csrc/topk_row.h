// The row-level pieces of the exact Top-k selection that more than one
// kernel runs: the threshold and general paths of one block per row, the
// final selection over the per-segment lists of the split path (also run at
// the head of the decode attention), and their LDS layouts.  The selection
// rules are those stated in topk.hip.
#pragma once
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
  const SelResult s = block_select(sm, top, K, cap, CSA2_TRACE_AT(a, 10));
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

constexpr int kTauCap = 8192;             // gathered values a row's final selection holds
constexpr int kTauKeyWords = kTauCap + kTauCap / 32;
constexpr int kSegPer = kSegLen / kSelThreads;   // values per thread of a segment
constexpr int kTopPer = kSelCap / kSelThreads;   // values per thread of the threshold level
static_assert(kTauMaxN / kSegLen <= kWave, "one segment per lane of a wave");
static_assert(kSegLen == 2 * kSelPad, "a segment is two LDS key batches");
static_assert(kTauMaxN <= 8 * kSelCap, "the maxima of 8 of a row fit the threshold level");

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

struct DescGeneralSmem {          // the general path of a marked row
  SelSmem sel;
  int32_t par[2][kSelCap / 8];
  int32_t cmap[kSelCap / 8];
};
union DescFinalSmem {
  FinalSmem f;
  DescGeneralSmem g;
};

// The final selection of the split path for row r: the top k of the row's
// segment lists, written to out[0 .. k) (ascending indices, -1 padding) --
// global memory, or a block's LDS (a generic pointer) when the selection runs
// at the head of the attention that consumes it.  Every thread of a block of
// kSelThreads calls it; u is the block's LDS.
CSA2_DEV void desc_final_row(const TopkArgs& a, int r, DescFinalSmem& u, int32_t* out) {
  FinalSmem& sm = u.f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const uint32_t K = (uint32_t)a.k;
  // list lengths (one segment per lane; every wave alike) and, in the same
  // round of loads, the fixed register slots of the fast path below: segment
  // s owns slots [spp s, spp (s+1)), thread t slots 4t .. 4t+3.  Issued
  // beside the row's length (every segment of an empty row has length 0, and
  // the slots are read only below a list's length).
  const uint32_t c = lane < a.nseg ? a.seg_cnt[(int64_t)r * a.nseg + lane] : 0u;
  const int64_t rb = (int64_t)r * a.nseg * kDescCap;
  const int spp = min(kRegCap / a.nseg, kDescCap) & ~(kRegPer - 1);
  const int sg = kRegPer * tid / spp, sl0 = kRegPer * tid - sg * spp;
  const int64_t g0 = sg < a.nseg ? rb + (int64_t)sg * kDescCap + sl0 : rb;
  const uint4 kk = *(const uint4*)(a.seg_key + g0);
  const int4 pp = *(const int4*)(a.seg_pos + g0);
  const int64_t n0 = row_count(a, r);
  if (n0 == 0) {
    for (int i = tid; i < a.k; i += kSelThreads) out[i] = -1;
    return;
  }
  CSA2_MARK(a, 3);
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

}  // namespace csa2
