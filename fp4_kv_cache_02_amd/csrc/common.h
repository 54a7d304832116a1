// Shared device helpers for the CSA2 kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa2.h"

#define CSA2_DEV __device__ __forceinline__

namespace csa2 {

constexpr int kWave = 64;

// Order-preserving key of a float32 score: larger score -> larger key, -0 < +0.
// Key 0 is reserved for "absent" (it would be a NaN bit pattern); -inf, the
// marker of an absent entry, is mapped to it as well.
CSA2_DEV uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (s == -__builtin_inff()) ? 0u : k;
}
CSA2_DEV float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Physical slot of position p of sequence b (-1 when outside the cache).
struct SlotMap {
  const int32_t* page_table;
  int64_t seq_stride;
  int64_t n_slots;
  int32_t max_pages;
  CSA2_DEV int64_t operator()(int b, int64_t p) const {
    int64_t s;
    if (page_table) {
      int64_t pg = p >> 6;
      if (pg >= max_pages) return -1;
      int32_t phys = page_table[(int64_t)b * max_pages + pg];
      s = (int64_t)phys * 64 + (p & 63);
    } else {
      s = (int64_t)b * seq_stride + p;
    }
    return (s >= 0 && s < n_slots) ? s : -1;
  }
};

inline SlotMap make_slot_map(const csa2_cache& c) {
  SlotMap m;
  m.page_table = c.page_table;
  m.seq_stride = c.seq_stride;
  m.n_slots = c.n_slots;
  m.max_pages = c.max_pages;
  return m;
}

// bf16 bit pattern -> float (exact).
CSA2_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
CSA2_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// E4M3 (OCP E4M3FN) byte -> float, exact: the bits are placed in a float32
// whose exponent field is the E4M3 exponent, then rescaled by 2^120 (bias 127
// -> 7); exponent 0 lands in float32's subnormal range and scales correctly.
CSA2_DEV float e4m3_to_float(uint32_t c) {
  float v = __uint_as_float(((c & 0x7Fu) << 20)) * 0x1p120f;
  return (c & 0x80u) ? -v : v;
}

CSA2_DEV int lane_id() { return __lane_id(); }

// Maximum over the wave through DPP lane shifts (rows of 16 lanes, then row
// broadcasts); shifted-in lanes contribute 0.  Result valid in every lane.
CSA2_DEV uint32_t wave_max_u32(uint32_t v) {
#define CSA2_DPPMAX(ctrl, rmask) \
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, (ctrl), (rmask), 0xF, false))
  CSA2_DPPMAX(0x111, 0xF);   // row_shr:1
  CSA2_DPPMAX(0x112, 0xF);   // row_shr:2
  CSA2_DPPMAX(0x114, 0xF);   // row_shr:4
  CSA2_DPPMAX(0x118, 0xF);   // row_shr:8
  CSA2_DPPMAX(0x142, 0xA);   // row_bcast:15
  CSA2_DPPMAX(0x143, 0xC);   // row_bcast:31
#undef CSA2_DPPMAX
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Phase timestamps for kernel tuning: only a build with -DCSA2_TRACE records
// them (thread 0 of block CSA2_TRACE_BLOCK, default 0, writes the 100 MHz
// wall clock into slot i of the trace buffer set by csa2_trace_set).
#ifdef CSA2_TRACE
#ifndef CSA2_TRACE_BLOCK
#define CSA2_TRACE_BLOCK 0
#endif
#define CSA2_TRACE_ARG uint64_t* trace;
#define CSA2_MARK(a, i)                                                                       \
  do {                                                                                         \
    if ((a).trace && threadIdx.x == 0 && blockIdx.x == CSA2_TRACE_BLOCK && blockIdx.y == 0 && blockIdx.z == 0) { \
      (a).trace[(i)] = wall_clock64();                                                         \
      (a).trace[32 + (i)] = __builtin_amdgcn_s_memtime();                                      \
    }                                                                                          \
  } while (0)
// inner marks: a trace pointer passed down explicitly
#define CSA2_MARKP(tr, i)                                                                        \
  do {                                                                                           \
    if ((tr) && threadIdx.x == 0 && blockIdx.x == CSA2_TRACE_BLOCK && blockIdx.y == 0 && blockIdx.z == 0) { \
      (tr)[(i)] = wall_clock64();                                                                \
      (tr)[32 + (i)] = __builtin_amdgcn_s_memtime();                                             \
    }                                                                                            \
  } while (0)
#define CSA2_TRACE_PTR(a) (a).trace
// slot `off` of the trace buffer, or null when none is set
#define CSA2_TRACE_AT(a, off) ((a).trace ? (a).trace + (off) : (uint64_t*)nullptr)
// per-block start (i = 0) and end (i = 1) times of a 1-D grid at slots
// base + 2 * block + i of a 2048-slot trace buffer
#define CSA2_SPAN(a, base, i)                                                                     \
  do {                                                                                            \
    if ((a).trace && threadIdx.x == 0 && blockIdx.y == 0 && (base) + 2 * blockIdx.x + 1 < 2048)   \
      (a).trace[(base) + 2 * blockIdx.x + (i)] = wall_clock64();                                  \
  } while (0)
#else
#define CSA2_SPAN(a, base, i) \
  do {                        \
  } while (0)
#define CSA2_TRACE_ARG
#define CSA2_MARK(a, i) \
  do {                  \
  } while (0)
#define CSA2_MARKP(tr, i) \
  do {                    \
  } while (0)
#define CSA2_TRACE_PTR(a) ((uint64_t*)nullptr)
#define CSA2_TRACE_AT(a, off) ((uint64_t*)nullptr)
#endif

}  // namespace csa2
