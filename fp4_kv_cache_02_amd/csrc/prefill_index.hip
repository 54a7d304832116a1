// Indexer of a prefill chunk on the matrix cores, with the exact Top-k.
//
// In a prefill chunk every query row of the layer scores the same context
// positions (the encoder prefill of a CSA2 layer group: 7minutos.es page,
// section "Atención escasa comprimida 2 (CSA2)"), so the indexer is a dense
// product [rows x 4 heads x 64] . [64 x positions] followed by ReLU and the
// head sum.  The selection must equal the one made on the canonical score
// (eight fused-multiply-add chains per head, see index_score.hip), which the
// matrix cores do not reproduce bit for bit.  The matrix-core score s~ is
// therefore only used to find, for each row, a small superset of the Top-k,
// with a proven error band, and the superset is then rescored exactly:
//
//   1. pass 0 (MFMA): s~ for every (row, position), stored rounded to bf16;
//      per row and group of 64 positions the maximum of s~ (gmax); the
//      largest |key| element (kmax).
//   2. threshold (the row's pass-1 block, before its filter): tau = (a
//      lower bound of) the k-th largest gmax of the row.
//      At least k groups hold a position with s~ >= tau, so at least k
//      positions have a canonical score >= tau - D, where D bounds |s~ - s|;
//      hence every position of the exact Top-k has s >= tau - D and
//      s~ >= theta = tau - 2D.
//   3. pass 1 (filter): the positions whose stored bf16 score is >=
//      bf16(theta) are the candidates, read only in the groups whose gmax
//      is >= theta (the same arithmetic produced gmax).  Rounding to nearest
//      even is monotone, so every position with s~ >= theta passes.
//   4. select: the candidates are put in position order, rescored with the
//      canonical arithmetic and the exact Top-k (ties to the lower position)
//      is written in ascending position order.
//   A row with more than kPrefCap candidates (near-constant scores) is listed
//   and scored by the exact scan + Top-k kernels instead.
//
// The band D.  For head h let M_h = sum_c |q_hc k_c| <= |q_h|_1 * kmax.
// The canonical dot product makes at most 11 roundings in float32
// (u = 2^-24): |d_h - e_h| <= 11u M_h (1 + O(u)), e_h the exact value.  The
// matrix core multiplies bf16 values exactly and adds 64 products in float32;
// the order and the rounding of its additions are not specified, so its error
// is taken as at most 73 u' M_h with u' = 2^-20 (four bits fewer than float32
// rounding to nearest).  ReLU does not increase a difference, and the head
// sums of s and s~ each round three times.  With w = head weights:
//   |s~ - s| <= sum_h |w_h| M_h (11u + 73u' + 6u)(1 + 2^-10) =: D,
// and a subnormal product the hardware might flush adds at most 2^-120.
#include "select.h"
#include <type_traits>
#include "kernels.h"

namespace csa2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

CSA2_DEV bf16x8_t to_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
// float -> bf16 bits, rounded to nearest even (monotone: x <= y gives bf16(x) <= bf16(y))
CSA2_DEV uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
constexpr uint16_t kBf16NaN = 0x7FC0u;
// ReLU as a signed integer maximum of the bits: a negative float (-0 too) is a
// negative integer and becomes +0; one instruction, with none of the NaN
// canonicalisation a float maximum adds in IEEE mode
CSA2_DEV float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

constexpr int kPWaves = 4;                  // waves per workgroup of the MFMA passes
constexpr int kPRows = 16 * kPWaves;        // query rows per workgroup (16 per wave)
constexpr int kPChunk = 2048;               // positions per workgroup
constexpr int kPStage = 128;                // positions per LDS stage
constexpr int kPGroup = 64;                 // positions per gmax group

// DPP lane patterns inside a row of 16 lanes
#define PF_DPP(v, ctrl) \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (v)), (ctrl), 0xF, 0xF, false))
constexpr int kQuadSwap1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;     // lane i <-> 7 - i within 8
constexpr int kMirror = 0x140;         // lane i <-> 15 - i within 16

// maximum over the 16 lanes of a DPP row, in every lane of the row
CSA2_DEV float row16_max(float v) {
  v = fmaxf(v, PF_DPP(v, kQuadSwap1));
  v = fmaxf(v, PF_DPP(v, kQuadSwap2));
  v = fmaxf(v, PF_DPP(v, kHalfMirror));
  v = fmaxf(v, PF_DPP(v, kMirror));
  return v;
}
CSA2_DEV float row16_sum(float v) {
  v += PF_DPP(v, kQuadSwap1);
  v += PF_DPP(v, kQuadSwap2);
  v += PF_DPP(v, kHalfMirror);
  v += PF_DPP(v, kMirror);
  return v;
}

struct PassSmem {
  uint4 keys[kPStage * 8];            // chunk c of stage position p at p*8 + (c ^ (p & 7))
  uint32_t present[kPStage + kPWaves * 64];   // [kPStage, ...): sink of the non-writing lanes
  uint32_t kmax[kPWaves];
};

// Pass 0.  Workgroup (x, y): positions
// [2048x, 2048x + 2048) of rows [64y, 64y + 64); wave w owns rows 64y + 16w
// .. +15 as four MFMA row tiles of 4 rows x 4 heads.
//
// MFMA 16x16x32 bf16 operand layout (lane l, c = l % 16, g = l / 16):
//   A (query): row m = c of the tile = (row 4mt + c/4, head c%4), elements
//     k = 8g .. 8g+7 of the 32-wide K slice;
//   B (keys): column n = c = position, elements k = 8g .. 8g+7;
//   D: lane holds rows 4g .. 4g+3 of column c = the four heads of row 4mt+g
//     at position c, so each lane finishes one (row, position) score.
// Visible positions of row r (rows past R: none).
CSA2_DEV int pref_row_len(const PrefArgs& a, int r) {
  if (r >= a.R) return 0;
  return min(a.seq_len[a.row_seq ? a.row_seq[r] : 0], a.n_max);
}

template <bool HAS_W>
__global__ __launch_bounds__(kPWaves * 64) void pref_pass_kernel(PrefArgs a) {
  __shared__ PassSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 15, g = lane >> 4;
  // positions any row may see (rows with their own lengths: all up to n_max;
  // each row's own length masks its scores below)
  const int L = a.row_seq ? a.n_max : min(a.seq_len[0], a.n_max);
  const int64_t x0 = (int64_t)blockIdx.x * kPChunk;
  if (x0 >= L) return;
  const int n_here = (int)min((int64_t)kPChunk, (int64_t)L - x0);
  const int n_stage = (n_here + kPStage - 1) / kPStage;
  // first row of the wave (uniform: the score buffer resource below lives in
  // scalar registers)
  const int rw0 = blockIdx.y * kPRows + 16 * __builtin_amdgcn_readfirstlane(wave);

  // query fragments (rows past R read row R-1; their results are dropped)
  bf16x8_t A[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int row = min(rw0 + 4 * mt + (c >> 2), a.R - 1);
    const uint4* qp = (const uint4*)(a.q32 + ((int64_t)row * 4 + (c & 3)) * 32);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) A[mt][kh] = to_bf16x8(qp[4 * kh + g]);
  }
  // this lane's output rows and their visible lengths
  int orow[4];
  int olen[4];
  float w[4][4];
  // the wave's rows of stored scores through buffer resources (rows 4 mt ..
  // 15 for the lane's row 4 mt + g): a store to a row past R lies past the
  // resource's end, a position past L gets an offset far past it, and the
  // hardware drops both, so the epilogue stores without a branch (16 rows x
  // 262144 positions x 2 bytes: 32-bit offsets)
  const int sstride = (int)a.sb_stride * 2;             // bytes per row
  const int nrow_w = max(0, min(16, a.R - rw0));
  const uint64_t sbase = (uint64_t)(a.sb + (int64_t)min(rw0, a.R - 1) * a.sb_stride);
  bool sw[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    orow[mt] = rw0 + 4 * mt + g;
    olen[mt] = pref_row_len(a, orow[mt]);
    const int rr = min(orow[mt], a.R - 1);
    sw[mt] = orow[mt] < a.R;
#pragma unroll
    for (int h = 0; h < 4; ++h) w[mt][h] = HAS_W ? a.head_w[(int64_t)rr * 4 + h] : 1.0f;
  }
  // the shortest visible length over the wave's rows below R (uniform)
  int mlen = 0x7FFFFFFF;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) mlen = sw[mt] ? min(mlen, olen[mt]) : mlen;
  mlen = min(min(__builtin_amdgcn_readlane(mlen, 0), __builtin_amdgcn_readlane(mlen, 16)),
             min(__builtin_amdgcn_readlane(mlen, 32), __builtin_amdgcn_readlane(mlen, 48)));
  const bool want_kmax = blockIdx.y == 0;
  uint32_t kmx = 0u;

  // stage loads: thread t loads chunk (t & 7) of stage positions (t >> 3) + 32i
  const int lq = tid & 7;
  uint4 pf0, pf1, pf2, pf3;             // prefetched stage (one variable per load:
  uint32_t pp0, pp1, pp2, pp3;           // an array here was kept in scratch memory)
#define PF_LOAD1(S, I)                                                          \
  {                                                                            \
    const int64_t p = x0 + (int64_t)(S) * kPStage + (tid >> 3) + 32 * (I);     \
    const int64_t slot = p < L ? a.map(0, p) : -1;                             \
    pp##I = slot >= 0 ? 1u : 0u;                                               \
    pf##I = a.kdata[(slot >= 0 ? slot : 0) * 8 + lq];                          \
  }
#define PF_LOAD_STAGE(S) PF_LOAD1(S, 0) PF_LOAD1(S, 1) PF_LOAD1(S, 2) PF_LOAD1(S, 3)
  PF_LOAD_STAGE(0);

  float gm[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) gm[mt] = -__builtin_inff();

  for (int s = 0; s < n_stage; ++s) {
    __syncthreads();                       // the previous stage is consumed
    {
      const uint4 pv[4] = {pf0, pf1, pf2, pf3};
      const uint32_t pr[4] = {pp0, pp1, pp2, pp3};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pl = (tid >> 3) + 32 * i;
        sm.keys[pl * 8 + (lq ^ (pl & 7))] = pv[i];
        sm.present[lq == 0 ? pl : kPStage + tid] = pr[i];     // unconditional store
        if (want_kmax) {
          const uint32_t wv[4] = {pv[i].x, pv[i].y, pv[i].z, pv[i].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t m = wv[e] & 0x7FFF7FFFu;
            kmx = max(kmx, max(m & 0xFFFFu, m >> 16));
          }
        }
      }
    }
    __syncthreads();
    if (s + 1 < n_stage) { PF_LOAD_STAGE(s + 1); }

    // a stage whose 128 positions are present and visible to every row of the
    // wave (uniform) takes the epilogue without the visibility selects
    const int sp0 = (int)x0 + s * kPStage;
    const bool full = sp0 + kPStage <= min(L, mlen) &&
                      __ballot(sm.present[lane] == 0u || sm.present[64 + lane] == 0u) == 0ull;
    auto tile_loop = [&](auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
#pragma unroll 4
    for (int nt = 0; nt < kPStage / 16; ++nt) {
      const int pl = 16 * nt + c;
      const uint4 b0 = sm.keys[pl * 8 + (g ^ (pl & 7))];
      const uint4 b1 = sm.keys[pl * 8 + ((4 + g) ^ (pl & 7))];
      const bool pres = FULL || sm.present[pl] != 0u;
      const int pos = (int)x0 + s * kPStage + pl;          // < kPrefMaxN
      const bool in_l = FULL || pos < L;
      // byte offset of (row 4 mt + g, pos) from row 4 mt; far past the rows when pos >= L
      const int po = in_l ? g * sstride + 2 * pos : 0x40000000;
      f32x4_t acc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        acc[mt] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][0], to_bf16x8(b0), acc[mt], 0, 0, 0);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][1], to_bf16x8(b1), acc[mt], 0, 0, 0);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float r0 = relu_bits(acc[mt][0]), r1 = relu_bits(acc[mt][1]);
        const float r2 = relu_bits(acc[mt][2]), r3 = relu_bits(acc[mt][3]);
        float sc;
        if (HAS_W)
          sc = (w[mt][0] * r0 + w[mt][1] * r1) + (w[mt][2] * r2 + w[mt][3] * r3);
        else
          sc = (r0 + r1) + (r2 + r3);
        const bool vis = FULL || (pres && pos < olen[mt]);
        gm[mt] = fmaxf(gm[mt], vis ? sc : -__builtin_inff());
        // the score for pass 1 (NaN where not visible: no comparison passes),
        // through a resource over rows 4 mt .. 15 of the wave (rebuilt here
        // from values read as uniform: one kept across the loop ends up in
        // vector registers and each store in a loop over its distinct values)
        const uint64_t bmt = (((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(sbase >> 32)) << 32) |
                              (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)sbase)) +
                             (uint64_t)(4 * mt) * (uint32_t)__builtin_amdgcn_readfirstlane(sstride);
        const int nmt = max(0, __builtin_amdgcn_readfirstlane(nrow_w) - 4 * mt) * __builtin_amdgcn_readfirstlane(sstride);
        const __amdgpu_buffer_rsrc_t sbuf = __builtin_amdgcn_make_buffer_rsrc((void*)bmt, 0, nmt, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(vis ? bf16_bits(sc) : kBf16NaN), sbuf, po, 0, 0);
      }
      if ((nt & 3) == 3) {      // end of a group of 64 positions
        const int grp = ((int)x0 + s * kPStage) / kPGroup + (nt >> 2);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const float v = row16_max(gm[mt]);
          if (c == 0 && sw[mt] && grp * kPGroup < olen[mt]) a.gmax[(int64_t)orow[mt] * a.gmax_stride + grp] = v;
          gm[mt] = -__builtin_inff();
        }
      }
    }
    };
    if (full) tile_loop(std::true_type{});
    else tile_loop(std::false_type{});
  }

  if (want_kmax) {
    kmx = wave_max_u32(kmx);
    if (lane == 0) sm.kmax[wave] = kmx;
    __syncthreads();
    if (tid == 0) {
      uint32_t m = sm.kmax[0];
      for (int i = 1; i < kPWaves; ++i) m = max(m, sm.kmax[i]);
      a.kmax_part[blockIdx.x] = __uint_as_float(m << 16);
    }
  }
#undef PF_LOAD_STAGE
#undef PF_LOAD1
}

// The error margin D of row r (one wave; lane is its lane; valid in every
// lane): sum_h |w_h| |q_h|_1 * kmax * (17 u + 73 u') (1 + 2^-10) + 2^-120,
// kmax the largest |key element| over the row's visible chunks.
template <bool HAS_W>
CSA2_DEV double pref_margin(const PrefArgs& a, int r, int lane) {
  const int L = pref_row_len(a, r);
  const int nchunk = (L + kPChunk - 1) / kPChunk;
  float km = 0.0f;
  for (int i = lane; i < nchunk; i += 64) km = fmaxf(km, a.kmax_part[i]);
  km = __uint_as_float(wave_max_u32(__float_as_uint(km)));
  // sum_h |w_h| |q_h|_1: lane l holds elements 4l .. 4l+3, head l / 16
  const uint2 qv = ((const uint2*)(a.q32 + (int64_t)r * 128))[lane];
  float s1 = (fabsf(bf16_lo(qv.x)) + fabsf(bf16_hi(qv.x))) + (fabsf(bf16_lo(qv.y)) + fabsf(bf16_hi(qv.y)));
  s1 = row16_sum(s1);
  if (HAS_W) s1 *= fabsf(a.head_w[(int64_t)r * 4 + (lane >> 4)]);
  const float aq = (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(s1), 0)) +
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s1), 16))) +
                   (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(s1), 32)) +
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s1), 48)));
  const double u = 0x1p-24, u2 = 0x1p-20;
  return (double)aq * (double)km * (17.0 * u + 73.0 * u2) * (1.0 + 0x1p-10) + 0x1p-120;
}

// One 8-bit digit of the row's threshold key, over the whole block (256
// threads, one histogram bin each).  Among the keys whose bits above
// shift + 8 equal `pre` (every key for the leading digit), the largest digit
// d (bits shift .. shift + 7) with above + #{keys with digit >= d} >= k;
// `above` then also counts the keys whose digit is larger.  Returns -1 when
// even d = 0 falls short (only possible for the leading digit: fewer than k
// keys).  The leading digit (sign and high exponent bits) takes few values,
// so each wave adds one count per distinct value instead of one atomic per
// key into the same bin.
struct FiltSmem {
  uint32_t hist[256];
  uint32_t wsum[4];
  uint32_t above;
  int dig;
};
template <int KPT>
CSA2_DEV int theta_digit(const uint32_t (&key)[KPT], int shift, uint32_t pre, bool lead, uint32_t k, uint32_t& above,
                         FiltSmem& f, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  f.hist[tid] = 0u;
  if (tid == 0) f.dig = -1;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool on = key[i] != 0u && (lead || (uint32_t)((uint64_t)key[i] >> (shift + 8)) == pre);
    const uint32_t d = (key[i] >> shift) & 255u;
    if (lead) {
      uint64_t act = __ballot(on);
      while (act) {                                  // uniform
        const int l0 = __ffsll((unsigned long long)act) - 1;
        const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)d, l0);
        const uint64_t m = __ballot(on && d == d0);
        if (lane == l0) atomicAdd(&f.hist[d0], (uint32_t)__popcll(m));
        act &= ~m;
      }
    } else if (on) {
      atomicAdd(&f.hist[d], 1u);
    }
  }
  __syncthreads();
  // thread t: bin 255 - t; its inclusive prefix = #{keys with digit >= 255 - t}
  const uint32_t v = f.hist[255 - tid];
  uint32_t P = wave_incl_scan_u32(v);
  if (lane == 63) f.wsum[wave] = P;
  __syncthreads();
  for (int w = 0; w < wave; ++w) P += f.wsum[w];
  if (above + P >= k && above + P - v < k) {
    f.dig = 255 - tid;
    f.above = above + P - v;
  }
  __syncthreads();
  const int dg = f.dig;
  if (dg >= 0) above = f.above;
  __syncthreads();                                   // (the next digit rewrites f)
  return dg;
}

// Pass 1: the candidates of row r are the positions, inside the groups whose
// maximum is >= theta, whose stored score is >= theta once both are rounded
// to bf16.  Rounding to nearest even never reverses an order, so every
// position with s~ >= theta passes; the few others that pass (less than one
// bf16 step below theta) are rescored exactly like every candidate.  One
// block per row: the row's groups at or above theta listed in LDS (ballot
// compaction, one LDS reservation per wave), then eight lanes per group,
// 16 bytes (8 scores) each, kFUnroll groups in flight per lane; the hits of
// a wave take one reservation (a wave prefix sum of the lanes' counts).  The
// list is in no particular order: the selection sorts it.
//
// The row's threshold first: tau = the largest key T with its low 8 bits
// zero such that at least k group maxima have keys >= T (a lower bound of
// the k-th largest group maximum), found digit by digit (bits 31..24,
// 23..16, 15..8) with block-wide histograms; theta = tau - 2D, or -inf
// when fewer than k groups hold a visible position.
constexpr int kFWaves = 4;
constexpr int kFUnroll = 4;
template <int NREG, bool HAS_W>
__global__ __launch_bounds__(kFWaves * 64) void pref_filter_kernel(PrefArgs a) {
  constexpr int kMaxG = kPrefMaxN / kPGroup;
  constexpr int kGPer = NREG / kFWaves;          // group maxima per thread (64 NREG per row at most)
  static_assert(kFWaves * 64 == 256, "one histogram bin per thread");
  __shared__ int32_t grp[kMaxG];
  __shared__ uint32_t ng, nc;
  __shared__ float s_th;
  __shared__ FiltSmem fs;
  const int r = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint64_t lt = (1ull << lane) - 1ull;
  const int L = pref_row_len(a, r);
  const int G = (L + kPGroup - 1) / kPGroup;
  if (tid == 0) {
    ng = 0u;
    nc = 0u;
    if (r == 0) *a.fb_count = 0u;      // the selection lists its overflowing rows there
  }
  float gv[kGPer];
  uint32_t key[kGPer];
#pragma unroll
  for (int i = 0; i < kGPer; ++i) {
    const int gi = tid + kFWaves * 64 * i;
    gv[i] = gi < G ? a.gmax[(int64_t)r * a.gmax_stride + gi] : -__builtin_inff();
    key[i] = order_key(gv[i]);                    // 0: absent, or no visible position
  }
  double D = 0.0;
  if (wave == 0) D = pref_margin<HAS_W>(a, r, lane);
  const uint32_t K = (uint32_t)a.k;
  uint32_t above = 0u, T = 0u;
  const int d0 = theta_digit<kGPer>(key, 24, 0u, true, K, above, fs, tid);
  if (d0 >= 0) {                                  // uniform
    const int d1 = theta_digit<kGPer>(key, 16, (uint32_t)d0, false, K, above, fs, tid);
    const int d2 = theta_digit<kGPer>(key, 8, ((uint32_t)d0 << 8) | (uint32_t)d1, false, K, above, fs, tid);
    // (d1, d2 >= 0: the keys of the chosen prefix reach k with those above)
    T = (d1 < 0 || d2 < 0) ? 0u : ((uint32_t)d0 << 24) | ((uint32_t)d1 << 16) | ((uint32_t)d2 << 8);
  }
  if (tid == 0) {
    float theta = -__builtin_inff();
    if (T != 0u) {
      float t = (float)((double)key_to_float(T) - 2.0 * D);
      theta = t - fabsf(t) * 0x1p-20f;
    }
    s_th = theta;
    a.theta[r] = theta;
  }
  __syncthreads();
  const float th = s_th;
  const float thb = __uint_as_float((uint32_t)bf16_bits(th) << 16);
#pragma unroll
  for (int i = 0; i < kGPer; ++i) {
    const int gi = tid + kFWaves * 64 * i;
    const bool q = gi < G && gv[i] >= th;
    const uint64_t bq = __ballot(q);
    if (bq) {                                      // uniform
      uint32_t base = 0u;
      if (lane == 0) base = atomicAdd(&ng, (uint32_t)__popcll(bq));
      base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
      if (q) grp[base + (uint32_t)__popcll(bq & lt)] = gi;
    }
  }
  __syncthreads();
  const uint32_t n_g = ng;
  const uint4* row = (const uint4*)(a.sb + (int64_t)r * a.sb_stride);
  int32_t* cl = a.cand + (int64_t)r * a.cap;
  const int part = lane & 7;
  for (uint32_t j0 = 0; j0 < n_g; j0 += kFUnroll * kFWaves * 8) {
    int gg[kFUnroll];
    uint4 v[kFUnroll];
#pragma unroll
    for (int u = 0; u < kFUnroll; ++u) {
      const uint32_t j = j0 + (uint32_t)((u * kFWaves + wave) * 8 + (lane >> 3));
      gg[u] = j < n_g ? grp[j] : -1;
      v[u] = row[(int64_t)(gg[u] >= 0 ? gg[u] : 0) * 8 + part];
    }
    uint32_t hits[kFUnroll];
    uint32_t cnt = 0u;
#pragma unroll
    for (int u = 0; u < kFUnroll; ++u) {
      const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      const int p0 = gg[u] * kPGroup + 8 * part;
      uint32_t h = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (e & 1) ? (w4[e >> 1] & 0xFFFF0000u) : (w4[e >> 1] << 16);
        h |= (gg[u] >= 0 && p0 + e < L && __uint_as_float(bits) >= thb) ? (1u << e) : 0u;
      }
      hits[u] = h;
      cnt += (uint32_t)__popc(h);
    }
    const uint32_t inc = wave_incl_scan_u32(cnt);
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    if (tot) {                                     // uniform
      uint32_t base = 0u;
      if (lane == 0) base = atomicAdd(&nc, tot);
      uint32_t o = (uint32_t)__builtin_amdgcn_readfirstlane((int)base) + inc - cnt;
#pragma unroll
      for (int u = 0; u < kFUnroll; ++u) {
        uint32_t h = hits[u];
        const int p0 = gg[u] * kPGroup + 8 * part;
        while (h) {
          const int e = __ffs(h) - 1;
          h &= h - 1u;
          if (o < (uint32_t)a.cap) cl[o] = p0 + e;
          ++o;
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) a.cand_count[r] = nc;
}

// Exact selection among the candidates of a row (one block per row).
constexpr int kPSelKeyWords = kPrefCap + kPrefCap / 32;
constexpr int kPBuckets = kSelThreads;                 // positions >> 9
static_assert(kPrefMaxN / kPBuckets == 512, "bucket width");
static_assert(kPrefCap % kSelPad == 0, "candidate capacity is a multiple of the LDS key padding");

struct PrefSelSmem {
  SelSmemT<kPSelKeyWords> sel;
  int32_t pos[kPrefCap];
  uint32_t bcnt[kPBuckets];
  uint32_t boff[kPBuckets];
};

template <bool HAS_W>
__global__ __launch_bounds__(kSelThreads) void pref_select_kernel(PrefArgs a) {
  __shared__ PrefSelSmem sm;
  const int r = blockIdx.x, tid = threadIdx.x;
  const uint32_t n = a.cand_count[r];
  int32_t* out = a.out + (int64_t)r * a.k;
  if (n > (uint32_t)a.cap) {
    if (tid == 0) a.fb_list[atomicAdd(a.fb_count, 1u)] = r;
    return;
  }
  const int32_t* cl = a.cand + (int64_t)r * a.cap;
  // ---- candidates into position order: bucket by position / 512, then rank within the bucket
  sm.bcnt[tid] = 0u;
  __syncthreads();
  for (uint32_t e = tid; e < n; e += kSelThreads) atomicAdd(&sm.bcnt[cl[e] >> 9], 1u);
  __syncthreads();
  uint32_t total;
  const uint32_t my_cnt = sm.bcnt[tid];
  const uint32_t off = block_excl_scan(sm.sel, my_cnt, total);
  sm.boff[tid] = off;
  sm.bcnt[tid] = 0u;
  __syncthreads();
  for (uint32_t e = tid; e < n; e += kSelThreads) {
    const int32_t p = cl[e];
    const uint32_t b = (uint32_t)p >> 9;
    sm.pos[sm.boff[b] + atomicAdd(&sm.bcnt[b], 1u)] = p;
  }
  __syncthreads();
  constexpr int kPer = kPrefCap / kSelThreads;
  int32_t rp[kPer];
  int32_t rd[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint32_t e = tid + i * kSelThreads;
    rd[i] = -1;
    if (e < n) {
      const int32_t p = sm.pos[e];
      const uint32_t b = (uint32_t)p >> 9;
      const uint32_t lo = sm.boff[b], hi = lo + sm.bcnt[b];
      uint32_t rank = 0;
      for (uint32_t j = lo; j < hi; ++j) rank += sm.pos[j] < p ? 1u : 0u;
      rp[i] = p;
      rd[i] = (int32_t)(lo + rank);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (rd[i] >= 0) sm.pos[rd[i]] = rp[i];
  __syncthreads();

  // ---- canonical scores: 8 lanes per candidate (lane j: channels 8j .. 8j+7)
  const int j = tid & 7, grp = tid >> 3;
  float qf[4][8];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint4 v = ((const uint4*)(a.q32 + (int64_t)r * 128))[h * 8 + j];
    qf[h][0] = bf16_lo(v.x); qf[h][1] = bf16_hi(v.x);
    qf[h][2] = bf16_lo(v.y); qf[h][3] = bf16_hi(v.y);
    qf[h][4] = bf16_lo(v.z); qf[h][5] = bf16_hi(v.z);
    qf[h][6] = bf16_lo(v.w); qf[h][7] = bf16_hi(v.w);
  }
  float wt[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  if (HAS_W) {
#pragma unroll
    for (int h = 0; h < 4; ++h) wt[h] = a.head_w[(int64_t)r * 4 + h];
  }
  const int n_pad = n ? sel_padded((int)n) : kSelPad;
  for (int e0 = 0; e0 < (int)n; e0 += kSelThreads / 8) {
    const int e = e0 + grp;
    const int32_t p = e < (int)n ? sm.pos[e] : -1;
    const int64_t slot = p >= 0 ? a.map(0, p) : -1;
    const uint4 kw = a.kdata[(slot >= 0 ? slot : 0) * 8 + j];
    const float kf[8] = {bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y),
                         bf16_lo(kw.z), bf16_hi(kw.z), bf16_lo(kw.w), bf16_hi(kw.w)};
    float d[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(kf[i], qf[h][i], acc);
      acc = acc + PF_DPP(acc, kQuadSwap1);     // c_j + c_(j^1)
      acc = acc + PF_DPP(acc, kQuadSwap2);     // (c0+c1)+(c2+c3) in lanes 0..3
      acc = acc + PF_DPP(acc, kHalfMirror);    // + ((c4+c5)+(c6+c7))
      d[h] = acc;
    }
    float rr[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) rr[h] = d[h] > 0.0f ? d[h] : 0.0f;
    float sc;
    if (HAS_W)
      sc = (wt[0] * rr[0] + wt[1] * rr[1]) + (wt[2] * rr[2] + wt[3] * rr[3]);
    else
      sc = (rr[0] + rr[1]) + (rr[2] + rr[3]);
    if (j == 0 && e < (int)n) sm.sel.key[skew(e)] = slot >= 0 ? order_key(sc) : 0u;
  }
  for (int e = (int)n + tid; e < n_pad; e += kSelThreads) sm.sel.key[skew(e)] = 0u;
  __syncthreads();

  // ---- exact Top-k in position order (keys in registers when they fit)
  uint32_t kept;
  if (n <= (uint32_t)kRegCap) {
    RegKeys rk;
#pragma unroll
    for (int j = 0; j < kRegPer; ++j) rk.v[j] = sm.sel.key[skew(kRegPer * tid + j)];
    __syncthreads();
    const SelResult res = block_select(sm.sel, rk, (uint32_t)a.k, 0u);
    kept = block_compact(sm.sel, rk, res, (uint32_t)a.k, [&](uint32_t o, int e) { out[o] = sm.pos[e]; });
  } else {
    const LdsKeysT<SelSmemT<kPSelKeyWords>> ks{&sm.sel, n_pad};
    const SelResult res = block_select(sm.sel, ks, (uint32_t)a.k, 0u);
    kept = block_compact(sm.sel, ks, res, (uint32_t)a.k, [&](uint32_t o, int e) { out[o] = sm.pos[e]; });
  }
  for (int i = (int)kept + tid; i < a.k; i += kSelThreads) out[i] = -1;
}

}  // namespace

hipError_t launch_prefill_index(const PrefArgs& a, bool has_w, hipStream_t st) {
  if (a.R <= 0) return hipSuccess;
  if (a.n_max > kPrefMaxN || a.cap != kPrefCap || a.k > kPrefCap || !a.sb || a.sb_stride < a.n_max ||
      (a.sb_stride & 63) != 0 || ((uintptr_t)a.sb & 15u) != 0)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.n_max + kPChunk - 1) / kPChunk), (unsigned)((a.R + kPRows - 1) / kPRows));
  const int G = (a.n_max + kPGroup - 1) / kPGroup;
  if (has_w) {
    hipLaunchKernelGGL((pref_pass_kernel<true>), grid, dim3(kPWaves * 64), 0, st, a);
    if (G <= 2048) hipLaunchKernelGGL((pref_filter_kernel<32, true>), dim3(a.R), dim3(kFWaves * 64), 0, st, a);
    else hipLaunchKernelGGL((pref_filter_kernel<64, true>), dim3(a.R), dim3(kFWaves * 64), 0, st, a);
    hipLaunchKernelGGL((pref_select_kernel<true>), dim3(a.R), dim3(kSelThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((pref_pass_kernel<false>), grid, dim3(kPWaves * 64), 0, st, a);
    if (G <= 2048) hipLaunchKernelGGL((pref_filter_kernel<32, false>), dim3(a.R), dim3(kFWaves * 64), 0, st, a);
    else hipLaunchKernelGGL((pref_filter_kernel<64, false>), dim3(a.R), dim3(kFWaves * 64), 0, st, a);
    hipLaunchKernelGGL((pref_select_kernel<false>), dim3(a.R), dim3(kSelThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace csa2
