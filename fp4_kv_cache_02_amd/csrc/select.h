// Block-wide exact selection on order-preserving uint32 keys (key 0 = absent).
//
// A block (kSelThreads threads) selects among keys held either in registers
// (RegKeys: kRegPer keys per thread, thread t holding elements
// kRegPer*t .. kRegPer*t+kRegPer-1) or in LDS (LdsKeys: up to kSelCap keys,
// element e at a skewed index so that per-thread contiguous runs are read
// with few bank conflicts, padded with absent keys to a multiple of kSelPad).
//
// The k-th largest key is found by a radix search over an adaptive key range:
// each pass histograms (key - lo) >> shift into kSelBins LDS bins, the shift
// chosen so the current range fills the bins, which keeps same-bin collisions
// (and LDS atomic serialisation) low even when the keys share their top bits.
// A search may stop early once the keys at or above a bin edge are few enough
// (a superset of the top k).
//
// Cost model (one CU per row): every pass touches every key a few times at 64
// lanes per cycle, so the callers keep the key sets they search small.
#pragma once
#include "common.h"

namespace csa2 {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelCap = 16384;                 // keys an LDS key set may hold
constexpr int kSelBins = 2048;
constexpr int kSelBinsPerThread = kSelBins / kSelThreads;
constexpr int kRegPer = 4;                     // keys per thread of a register key set
constexpr int kRegCap = kSelThreads * kRegPer; // 2048

CSA2_DEV int skew(int e) { return e + (e >> 5); }
constexpr int kSelKeyWords = kSelCap + kSelCap / 32;

// KW: LDS words of the key set (skewed), e.g. kSelKeyWords for kSelCap keys.
template <int KW>
struct SelSmemT {
  uint32_t key[KW];
  uint32_t bins[kSelBins];
  uint32_t wa[kSelWaves];
  uint32_t wb[kSelWaves];
  uint32_t wc[kSelWaves];
  uint32_t bc[4];
  uint32_t fin[kWave];       // keys of the final bin, ranked by one wave
};
using SelSmem = SelSmemT<kSelKeyWords>;

// LDS key sets are read in batches of kSelBatch independent reads without
// bounds tests (a test per read would make the compiler wait on each read).
constexpr int kSelBatch = 8;
constexpr int kSelPad = kSelBatch * kSelThreads;    // 4096
CSA2_DEV int sel_padded(int n) { return (n + kSelPad - 1) / kSelPad * kSelPad; }

// Keys in registers: thread t holds elements N*t .. N*t+N-1 (the element
// order matters only to block_compact).
template <int N>
struct RegKeysN {
  uint32_t v[N];
  template <class F>
  CSA2_DEV void each(const F& f) const {
#pragma unroll
    for (int j = 0; j < N; ++j) f(v[j]);
  }
  template <class F>
  CSA2_DEV void each_owned(const F& f) const {       // contiguous, in element order
#pragma unroll
    for (int j = 0; j < N; ++j) f(v[j], N * (int)threadIdx.x + j);
  }
};
using RegKeys = RegKeysN<kRegPer>;

// Keys in LDS: sm.key[skew(e)] for e < n (n a multiple of kSelPad).
template <class Sm>
struct LdsKeysT {
  const Sm* sm;
  int n;
  template <class F>
  CSA2_DEV void each(const F& f) const {
    for (int e0 = threadIdx.x; e0 < n; e0 += kSelPad) {
      uint32_t v[kSelBatch];
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) v[j] = sm->key[skew(e0 + j * kSelThreads)];
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) f(v[j]);
    }
  }
  template <class F>
  CSA2_DEV void each_owned(const F& f) const {       // thread t: elements [t*C, (t+1)*C)
    const int C = n / kSelThreads;                    // a multiple of kSelBatch
    const int e0 = (int)threadIdx.x * C;
    for (int b = e0; b < e0 + C; b += kSelBatch) {
      uint32_t v[kSelBatch];
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) v[j] = sm->key[skew(b + j)];
#pragma unroll
      for (int j = 0; j < kSelBatch; ++j) f(v[j], b + j);
    }
  }
};
using LdsKeys = LdsKeysT<SelSmem>;

// Wave-wide inclusive scan and reductions through DPP lane shifts (no LDS
// round trips): shifts by 1, 2, 4, 8 within each row of 16 lanes, then the
// last lane of a row is broadcast into the next row(s).  Lanes whose source
// lies outside the row receive 0 (the `old` operand).
#define CSA2_DPP_U(v, ctrl, rmask) \
  ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(v), (ctrl), (rmask), 0xF, false))
CSA2_DEV uint32_t wave_incl_scan_u32(uint32_t v) {
  v += CSA2_DPP_U(v, 0x111, 0xF);   // row_shr:1
  v += CSA2_DPP_U(v, 0x112, 0xF);   // row_shr:2
  v += CSA2_DPP_U(v, 0x114, 0xF);   // row_shr:4
  v += CSA2_DPP_U(v, 0x118, 0xF);   // row_shr:8
  v += CSA2_DPP_U(v, 0x142, 0xA);   // row_bcast:15 into rows 1, 3
  v += CSA2_DPP_U(v, 0x143, 0xC);   // row_bcast:31 into rows 2, 3
  return v;
}
// min / sum over the wave, valid in every lane (max: common.h)
CSA2_DEV uint32_t wave_min_u32(uint32_t v) {
  // shifted-in zeros must not win: complement, take the max, complement back
  return ~wave_max_u32(~v);
}
CSA2_DEV uint32_t wave_sum_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan_u32(v), 63);
}

// Exclusive prefix sum of v in thread order; total returned through `total`.
template <class Sm>
CSA2_DEV uint32_t block_excl_scan(Sm& sm, uint32_t v, uint32_t& total) {
  const int tid = threadIdx.x, w = tid / kWave;
  const uint32_t inc = wave_incl_scan_u32(v);
  if (lane_id() == kWave - 1) sm.wa[w] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const uint32_t t = sm.wa[i];
    before += (i < w) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

// Minimum and maximum present key, and the number of present keys.
template <class Keys, class Sm>
CSA2_DEV void block_range(Sm& sm, const Keys& ks, uint32_t& kmin, uint32_t& kmax, uint32_t& count) {
  uint32_t mn = 0xFFFFFFFFu, mx = 0u, c = 0u;
  ks.each([&](uint32_t v) {
    mn = v ? min(mn, v) : mn;
    mx = max(mx, v);
    c += v ? 1u : 0u;
  });
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  c = wave_sum_u32(c);
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) {
    sm.wa[w] = mn;
    sm.wb[w] = mx;
    sm.wc[w] = c;
  }
  __syncthreads();
  mn = 0xFFFFFFFFu;
  mx = 0u;
  c = 0u;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    mn = min(mn, sm.wa[i]);
    mx = max(mx, sm.wb[i]);
    c += sm.wc[i];
  }
  __syncthreads();
  kmin = mn;
  kmax = mx;
  count = c;
}

struct SelResult {
  uint32_t T;       // threshold key: keep keys > T, and keys == T as below
  uint32_t n_gt;    // present keys > T
  uint32_t n_eq;    // present keys == T
  bool exact;       // T is the k-th largest key (ties at T must be cut by element order)
};

// The k-th largest present key (exact = true), or, when `cap` > 0, an earlier
// bin edge T such that k <= #{keys >= T} <= cap (exact = false; keep every
// key >= T).  With at most k present keys: T = 0, n_gt = count (keep all).
// Once the bin holding the k-th largest key has at most 64 keys, one wave
// ranks them instead of running further passes over every key.
template <class Keys, class Sm>
CSA2_DEV SelResult block_select(Sm& sm, const Keys& ks, uint32_t kth, uint32_t cap, uint64_t* tr = nullptr) {
  const int tid = threadIdx.x;
  uint32_t lo, hi, count;
  block_range(sm, ks, lo, hi, count);
  CSA2_MARKP(tr, 0);
  [[maybe_unused]] int pass = 0;     // (numbers the trace marks)
  SelResult res;
  if (count <= kth) {
    res.T = 0u;
    res.n_gt = count;
    res.n_eq = 0u;
    res.exact = true;
    return res;
  }
  uint32_t above = 0u;   // keys > hi
  for (;;) {
    // the range [lo, hi] holds the k-th largest; `above` keys lie above it
    const uint32_t width = hi - lo;
    int shift = 0;
    while (shift < 32 && (width >> shift) >= (uint32_t)kSelBins) ++shift;
#pragma unroll
    for (int i = 0; i < kSelBinsPerThread; ++i) sm.bins[tid + i * kSelThreads] = 0u;
    if (tid == 0) sm.bc[3] = 0u;     // fill count of sm.fin
    __syncthreads();
    ks.each([&](uint32_t v) {
      if (v >= lo && v <= hi && v != 0u) atomicAdd(&sm.bins[(v - lo) >> shift], 1u);
    });
    __syncthreads();
    // thread t owns the kSelBinsPerThread bins just below B - BPT*t, scanned from the top
    const int top = kSelBins - kSelBinsPerThread * tid;
    uint32_t hb[kSelBinsPerThread];
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < kSelBinsPerThread; ++i) {
      hb[i] = sm.bins[top - 1 - i];
      cnt += hb[i];
    }
    uint32_t tot;
    const uint32_t before = above + block_excl_scan(sm, cnt, tot);
    if (before < kth && before + cnt >= kth) {
      uint32_t acc = before;
#pragma unroll
      for (int i = 0; i < kSelBinsPerThread; ++i) {
        if (acc < kth && acc + hb[i] >= kth) {
          sm.bc[0] = (uint32_t)(top - 1 - i);
          sm.bc[1] = acc;
          sm.bc[2] = hb[i];
        }
        acc += hb[i];
      }
    }
    __syncthreads();
    const uint32_t bin = sm.bc[0], acc = sm.bc[1], h = sm.bc[2];
    __syncthreads();
    CSA2_MARKP(tr, 1 + (pass++));
    const uint32_t blo = lo + (bin << shift);
    const uint32_t bhi =
        (shift == 0) ? blo : (uint32_t)min((uint64_t)hi, (uint64_t)blo + ((1ull << shift) - 1ull));
    if (cap && acc + h <= cap) {
      res.T = blo;
      res.n_gt = acc + h;
      res.n_eq = 0u;
      res.exact = false;
      return res;
    }
    if (blo == bhi) {
      res.T = blo;
      res.n_gt = acc;
      res.n_eq = h;
      res.exact = true;
      return res;
    }
    if (h <= (uint32_t)kWave) {
      // the bin's h keys into sm.fin (any order): acc keys lie above the bin
      // and the k-th largest is the need-th largest of the bin
      ks.each([&](uint32_t v) {
        if (v >= blo && v <= bhi && v != 0u) sm.fin[atomicAdd(&sm.bc[3], 1u)] = v;
      });
      __syncthreads();
      if (tid < kWave) {
        const uint32_t need = kth - acc;
        const uint32_t mine = (tid < (int)h) ? sm.fin[tid] : 0u;
        uint32_t gt = 0u, ge = 0u;
        for (int j = 0; j < (int)h; ++j) {
          const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)mine, j);
          gt += (o > mine) ? 1u : 0u;
          ge += (o >= mine) ? 1u : 0u;
        }
        // the lanes holding the need-th largest value (all equal) publish it
        if (tid < (int)h && gt < need && ge >= need) {
          sm.bc[0] = mine;
          sm.bc[1] = acc + gt;
          sm.bc[2] = ge - gt;
        }
      }
      __syncthreads();
      res.T = sm.bc[0];
      res.n_gt = sm.bc[1];
      res.n_eq = sm.bc[2];
      res.exact = true;
      __syncthreads();
      return res;
    }
    above = acc;
    lo = blo;
    hi = bhi;
  }
}

// Order-preserving compaction of the selection described by `s` with k
// wanted: keys > T, plus (exact) the first k - n_gt keys == T in element
// order, or (not exact) every key >= T.  emit(out_pos, element) is called for
// each kept element; returns the number kept.
template <class Keys, class Emit, class Sm>
CSA2_DEV uint32_t block_compact(Sm& sm, const Keys& ks, const SelResult& s, uint32_t kth, const Emit& emit) {
  const uint32_t need_eq = s.exact ? (kth > s.n_gt ? kth - s.n_gt : 0u) : 0u;
  const bool keep_all = (s.T == 0u);
  const uint32_t T = s.T;
  const bool cut_eq = !keep_all && s.exact;
  // keep-all: every present key; exact: keys > T (ties separately); superset: keys >= T
  const uint32_t gt_lo = keep_all ? 1u : (s.exact ? T + 1u : T);
  const bool none_gt = s.exact && !keep_all && T == 0xFFFFFFFFu;
  uint32_t n_keep = 0, n_eq = 0;
  ks.each_owned([&](uint32_t v, int) {
    n_keep += (!none_gt && v >= gt_lo) ? 1u : 0u;
    n_eq += (cut_eq && v == T) ? 1u : 0u;
  });
  // one scan of both counts (each total <= kSelCap < 2^16)
  uint32_t tot;
  const uint32_t pre = block_excl_scan(sm, n_keep | (n_eq << 16), tot);
  uint32_t eq_rank = pre >> 16;
  uint32_t pos = (pre & 0xFFFFu) + min(eq_rank, need_eq);
  ks.each_owned([&](uint32_t v, int e) {
    bool keep = !none_gt && v >= gt_lo;
    if (cut_eq && v == T) {
      keep = eq_rank < need_eq;
      ++eq_rank;
    }
    if (keep) emit(pos++, e);
  });
  const uint32_t total_gt = tot & 0xFFFFu, total_eq = tot >> 16;
  return total_gt + min(total_eq, need_eq);
}

}  // namespace csa2
