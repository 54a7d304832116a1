// Block-wide exact selection primitives (radix select on order-preserving
// uint32 keys, order-preserving compaction).  Used by the Top-K kernels.
//
// Ordering everywhere: key descending, index ascending.  Key 0 = absent.
#pragma once
#include "common.h"

namespace csa2 {

// Threads own contiguous runs of PER elements ("chunk" = NT*PER elements);
// element e of a chunk belongs to thread e / PER.
template <int NT>
struct SelectSmem {
  uint32_t hist[4096];
  uint32_t wtot[NT / kWave];
  uint32_t bcast[8];
  unsigned long long last;   // 1 + largest kept tie index (0: none)
};

CSA2_DEV uint32_t wave_incl_scan(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint32_t t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

// Exclusive prefix sum of v over the block (thread order); also returns the total.
template <int NT>
CSA2_DEV uint32_t block_excl_scan(SelectSmem<NT>& sm, uint32_t v, uint32_t& total) {
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  uint32_t inc = wave_incl_scan(v);
  if (lane == kWave - 1) sm.wtot[w] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) {
    uint32_t t = sm.wtot[i];
    before += (i < w) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

// Source of keys: a functor load(chunk_base, tid, out[PER]) filling the PER keys
// of thread tid for elements chunk_base + tid*PER + j (absent -> 0).

// Radix select: the kth largest present key among n elements.
// Returns T (0 if fewer than kth keys are present) and sets cnt_gt to the number
// of present keys > T and cnt_eq to the number equal to T (both exact).
template <int NT, int PER, class Src>
CSA2_DEV uint32_t radix_select(SelectSmem<NT>& sm, const Src& src, int64_t n, uint32_t kth,
                               uint32_t& cnt_gt, uint32_t& cnt_eq) {
  const int tid = threadIdx.x;
  constexpr int CH = NT * PER;
  uint32_t prefix = 0, mask = 0, remaining = kth;
  const int shifts[3] = {20, 8, 0};
  const int nbins[3] = {4096, 4096, 256};
  uint32_t last_count = 0;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass], nb = nbins[pass];
    for (int b = tid; b < nb; b += NT) sm.hist[b] = 0;
    __syncthreads();
    for (int64_t base = 0; base < n; base += CH) {
      uint32_t k[PER];
      src.load(base, tid, k);
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (k[j] != 0u && (k[j] & mask) == prefix) atomicAdd(&sm.hist[(k[j] >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    // thread t covers bins from the top: [nb - (t+1)*bpt, nb - t*bpt)
    const int bpt = (nb + NT - 1) / NT;
    const int hi = nb - tid * bpt;            // exclusive upper bound
    const int lo = hi - bpt < 0 ? 0 : hi - bpt;
    uint32_t mine = 0;
    for (int b = lo; b < hi; ++b) mine += sm.hist[b];
    uint32_t total;
    uint32_t above = block_excl_scan<NT>(sm, hi > 0 ? mine : 0u, total);
    if (pass == 0 && total < remaining) {
      // fewer present keys than kth: everything present is "greater than" T = 0
      cnt_gt = total;
      cnt_eq = 0;
      return 0u;
    }
    if (hi > 0 && above < remaining && above + mine >= remaining) {
      uint32_t acc = above;
      for (int b = hi - 1; b >= lo; --b) {
        uint32_t h = sm.hist[b];
        if (acc + h >= remaining) {
          sm.bcast[0] = (uint32_t)b;
          sm.bcast[1] = acc;
          sm.bcast[2] = h;
          break;
        }
        acc += h;
      }
    }
    __syncthreads();
    const uint32_t d = sm.bcast[0], acc = sm.bcast[1];
    last_count = sm.bcast[2];
    __syncthreads();
    remaining -= acc;
    prefix |= d << shift;
    mask |= (uint32_t)(nb - 1) << shift;
  }
  cnt_gt = kth - remaining;
  cnt_eq = last_count;
  return prefix;
}

// Order-preserving compaction of the selection {key > T} U {the first need_eq
// keys == T in index order}; T == 0 keeps every present key.  For each kept
// element calls emit(out_pos, key, element_index).  Returns the number kept.
// Also reports the index of the last kept element equal to T (or -1).
template <int NT, int PER, class Src, class Emit>
CSA2_DEV uint32_t compact(SelectSmem<NT>& sm, const Src& src, int64_t n, uint32_t T,
                          uint32_t need_eq, const Emit& emit, int64_t& last_tie_idx) {
  const int tid = threadIdx.x;
  constexpr int CH = NT * PER;
  uint32_t out_before = 0, eq_before = 0;
  int64_t last_tie = -1;
  for (int64_t base = 0; base < n; base += CH) {
    uint32_t k[PER];
    src.load(base, tid, k);
    uint32_t n_eq = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) n_eq += (T != 0u && k[j] == T) ? 1u : 0u;
    uint32_t eq_tot;
    uint32_t eq_rank = eq_before + block_excl_scan<NT>(sm, n_eq, eq_tot);
    bool keep[PER];
    uint32_t n_keep = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      bool gt = (T == 0u) ? (k[j] != 0u) : (k[j] > T);
      bool eq = (T != 0u) && (k[j] == T);
      bool kt = eq && (eq_rank < need_eq);
      if (eq) {
        if (kt) last_tie = base + (int64_t)tid * PER + j;
        ++eq_rank;
      }
      keep[j] = gt || kt;
      n_keep += keep[j] ? 1u : 0u;
    }
    uint32_t keep_tot;
    uint32_t pos = out_before + block_excl_scan<NT>(sm, n_keep, keep_tot);
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (keep[j]) emit(pos++, k[j], base + (int64_t)tid * PER + j);
    out_before += keep_tot;
    eq_before += eq_tot;
  }
  // largest index among kept ties (the worst kept element)
  if (tid == 0) sm.last = 0ull;
  __syncthreads();
  if (last_tie >= 0) atomicMax(&sm.last, (unsigned long long)(last_tie + 1));
  __syncthreads();
  last_tie_idx = (int64_t)sm.last - 1;
  __syncthreads();
  return out_before;
}

}  // namespace csa2
