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
// Work layout (no LDS): a wave scores one "step" of 64 positions at a time.
// Lane l = 8g + j owns channel chunk j (channels 8j..8j+7, one 16-byte load)
// of the eight positions of group g; register i of the lane holds position
// (step base) + 8g + i.  One load instruction therefore reads eight whole
// 128-byte key rows, and the eight instructions of a step read 8 KiB.
// Each lane forms its chunk's partial c_j of every position for the four heads
// with eight FMAs each; the tree over the eight chunks is a three-level
// reduce-scatter inside the group of eight lanes: at each level a lane keeps
// half of its positions, adds the partner's partials of those positions (DPP
// lane exchange: partner j^1, then j^2, then 7-j) and hands over the other
// half, so the pairs combined are exactly ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7))
// (IEEE addition is commutative) and every lane ends with one position whose
// score it finishes alone.  Loads of the next step are issued register by
// register as the current step consumes them (unconditional loads: an absent
// position reads slot 0), so each wave keeps 8 KiB in flight.
//
// Epilogue: each lane writes its position's score (32 contiguous bytes per
// group).  In scan mode the wave also emits the maxima the Top-K selection
// descends through: the maximum of each block of 8 positions (the
// hierarchical indexer's block score) and of the 64-position step.
#include "kernels.h"

namespace csa2 {

constexpr int kScanWaves = 4;            // waves per block

#define CSA2_DPP(v, ctrl) \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (v)), (ctrl), 0xF, 0xF, false))

// Geometry of one step: the row is wave-uniform (scalar registers), the
// position group and its slot are per lane.
struct StepGeo {
  int r;          // query row
  int b;          // sequence
  int L;          // visible positions of the row
  int t;          // step index within the row
  int64_t pos0;   // first position of this lane's group (scan: 64t + 8g)
  int64_t s0;     // slot of pos0 (0 when the group is absent: a safe address)
  int nv;         // positions i < nv of the group are present
};

template <bool CAND>
CSA2_DEV StepGeo step_geo(const IdxArgs& a, uint32_t item, int g) {
  StepGeo s;
  s.r = __builtin_amdgcn_readfirstlane((int)(item / (uint32_t)a.steps_per_row));
  s.t = __builtin_amdgcn_readfirstlane((int)(item - (uint32_t)s.r * (uint32_t)a.steps_per_row));
  if (a.row_list) s.r = __builtin_amdgcn_readfirstlane(a.row_list[s.r]);
  s.b = a.row_seq ? a.row_seq[s.r] : s.r;
  s.L = __builtin_amdgcn_readfirstlane(min(a.seq_len[s.b], a.n_max));
  int64_t pos0;
  if (CAND) {
    const int ci = s.t * 8 + g;
    const int blk = ci < a.n_cand ? a.cand[(int64_t)s.r * a.n_cand + ci] : -1;
    pos0 = blk >= 0 ? (int64_t)blk * 8 : (int64_t)1 << 40;
  } else {
    pos0 = (int64_t)s.t * 64 + g * 8;
  }
  s.pos0 = pos0;
  int64_t s0 = -1;
  int nv = 0;
  if (pos0 < s.L) {
    s0 = a.map(s.b, pos0);    // a group of 8 never straddles a page (pages are 64)
    if (s0 >= 0) {
      const int64_t lim = min((int64_t)s.L - pos0, a.map.n_slots - s0);
      nv = (int)min(lim, (int64_t)8);
    }
  }
  s.s0 = nv > 0 ? s0 : 0;
  s.nv = nv;
  return s;
}

// Chunk j (channels 8j .. 8j+7) of the key of position i of the group (slot
// 0 stands in for absent positions: every load is unconditional and in
// bounds): 16 bytes of bf16, or 8 bytes of E4M3 codes for FP8 keys (in .x,
// .y).  The keys are streamed once per scan: non-temporal loads (measured
// ~10 % faster than ordinary ones at 8 x 128K positions).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
template <bool FP8>
CSA2_DEV uint4 key_chunk(const uint4* __restrict__ kd, const StepGeo& s, int i, int j) {
  const int64_t slot = (i < s.nv) ? s.s0 + i : 0;
  if (FP8) {
    const u32x2_t v = __builtin_nontemporal_load((const u32x2_t*)kd + slot * 8 + j);
    return make_uint4(v[0], v[1], 0u, 0u);
  }
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)&kd[slot * 8 + j]);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// The eight channel values of a chunk as exact floats.
template <bool FP8>
CSA2_DEV void chunk_values(uint4 kw, float (&kf)[8]) {
  if (FP8) {
    // the hardware conversion of two OCP E4M3 codes (bytes 0-1 or 2-3 of the
    // word) to float32, exact
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)kw.x, false);
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)kw.x, true);
    const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)kw.y, false);
    const f32x2_t d = __builtin_amdgcn_cvt_pk_f32_fp8((int)kw.y, true);
    kf[0] = a[0]; kf[1] = a[1]; kf[2] = b[0]; kf[3] = b[1];
    kf[4] = c[0]; kf[5] = c[1]; kf[6] = d[0]; kf[7] = d[1];
  } else {
    kf[0] = bf16_lo(kw.x); kf[1] = bf16_hi(kw.x); kf[2] = bf16_lo(kw.y); kf[3] = bf16_hi(kw.y);
    kf[4] = bf16_lo(kw.z); kf[5] = bf16_hi(kw.z); kf[6] = bf16_lo(kw.w); kf[7] = bf16_hi(kw.w);
  }
}

// One step per wave: the register budget of six waves per SIMD (~80 VGPRs,
// no spill) -- measured 51.9 against 52.7 us per 128K group step at the
// compiler's four; the persistent variant keeps four (it would spill).
template <bool CAND, bool HAS_W, bool MAXIMA, bool PERSIST, bool FP8>
__global__ __launch_bounds__(kScanWaves * 64) __attribute__((amdgpu_waves_per_eu(PERSIST ? 4 : 6)))
void index_scan_kernel(IdxArgs a) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 3, j = lane & 7;
  // reduce-scatter roles: lanes j and 7-j play the same part in the two
  // quads; lane j finishes position pj of its group
  const int vj = (j < 4) ? j : 7 - j;
  const int pj = (j < 4) ? j : 11 - j;
  const bool b0 = vj & 1, b1 = (vj >> 1) & 1, upper = j >= 4;
  const uint32_t W = gridDim.x * kScanWaves;
  const uint32_t n_rows = a.row_list ? min(*a.row_list_count, (uint32_t)a.R) : (uint32_t)a.R;
  const uint32_t n_items = n_rows * (uint32_t)a.steps_per_row;
  uint32_t item = __builtin_amdgcn_readfirstlane(blockIdx.x * kScanWaves + (threadIdx.x >> 6));
  if (item >= n_items) return;

  const uint4* __restrict__ kd = a.kdata;
  uint4 regs[8];
  StepGeo cur = step_geo<CAND>(a, item, g);
  // a scan step past its row's visible positions writes nothing: leave before
  // any load (rows of a batch differ in length; the grid covers the longest)
  if (!CAND && !PERSIST && cur.t * 64 >= cur.L) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) regs[i] = key_chunk<FP8>(kd, cur, i, j);
  // FP8 keys: the scale of the position this lane finishes (slot 0 when absent)
  float ksc = 1.0f;
  if (FP8) ksc = a.kscale[pj < cur.nv ? cur.s0 + pj : 0];

  int qrow = -1;
  float qf[4][8];
  float w[4] = {1.f, 1.f, 1.f, 1.f};

  for (;;) {
    if (cur.r != qrow) {
      qrow = cur.r;
      const uint4* qp = (const uint4*)(a.q32 + (int64_t)qrow * 128);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint4 v = qp[h * 8 + j];
        qf[h][0] = bf16_lo(v.x); qf[h][1] = bf16_hi(v.x);
        qf[h][2] = bf16_lo(v.y); qf[h][3] = bf16_hi(v.y);
        qf[h][4] = bf16_lo(v.z); qf[h][5] = bf16_hi(v.z);
        qf[h][6] = bf16_lo(v.w); qf[h][7] = bf16_hi(v.w);
      }
      if (HAS_W) {
#pragma unroll
        for (int h = 0; h < 4; ++h) w[h] = a.head_w[(int64_t)qrow * 4 + h];
      }
    }
    const uint32_t next = item + W;
    const bool has_next = PERSIST && next < n_items;
    StepGeo nxt = cur;
    if (has_next) nxt = step_geo<CAND>(a, next, g);
    float ksc_next = ksc;
    if (FP8 && has_next) ksc_next = a.kscale[pj < nxt.nv ? nxt.s0 + pj : 0];

    // chunk partials c_j of the eight positions, four heads
    float P[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 kw = regs[i];
      if (has_next) regs[i] = key_chunk<FP8>(kd, nxt, i, j);
      float kf[8];
      chunk_values<FP8>(kw, kf);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(kf[e], qf[h][e], acc);
        P[i][h] = acc;
      }
    }
    // reduce-scatter over the 8 lanes of the group
    float Q[4][4], Rr[2][4], d[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float keep = b0 ? P[2 * r + 1][h] : P[2 * r][h];
        const float send = b0 ? P[2 * r][h] : P[2 * r + 1][h];
        Q[r][h] = keep + CSA2_DPP(send, 0xB1);          // partner j ^ 1
      }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float keep = b1 ? Q[2 * s2 + 1][h] : Q[2 * s2][h];
        const float send = b1 ? Q[2 * s2][h] : Q[2 * s2 + 1][h];
        Rr[s2][h] = keep + CSA2_DPP(send, 0x4E);        // partner j ^ 2
      }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float keep = upper ? Rr[1][h] : Rr[0][h];
      const float send = upper ? Rr[0][h] : Rr[1][h];
      d[h] = keep + CSA2_DPP(send, 0x141);              // partner 7 - j
    }
    // FP8 keys: the entry's scale multiplies each head's dot product (one rounding)
    if (FP8) {
#pragma unroll
      for (int h = 0; h < 4; ++h) d[h] = d[h] * ksc;
    }
    float rr[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) rr[h] = (d[h] > 0.0f) ? d[h] : 0.0f;
    float sc;
    if (HAS_W) {
      const float p0 = w[0] * rr[0], p1 = w[1] * rr[1], p2 = w[2] * rr[2], p3 = w[3] * rr[3];
      sc = (p0 + p1) + (p2 + p3);
    } else {
      sc = (rr[0] + rr[1]) + (rr[2] + rr[3]);
    }
    const bool present = pj < cur.nv;

    // ---- outputs of the step ----
    if (CAND) {
      const int64_t ci8 = (int64_t)cur.t * 64 + g * 8 + pj;     // 8 * candidate index + pj
      if (ci8 < (int64_t)a.n_cand * 8)
        a.scores[(int64_t)cur.r * a.score_stride + ci8] = present ? sc : -__builtin_inff();
      if (MAXIMA) {
        // maximum of the candidate block (the lane group's 8 positions)
        uint32_t k = present ? order_key(sc) : 0u;
        k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0xB1, 0xF, 0xF, false));
        k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x4E, 0xF, 0xF, false));
        k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x141, 0xF, 0xF, false));
        const int ci = cur.t * 8 + g;
        if (j == 0 && ci < a.n_cand)
          a.block_max[(int64_t)cur.r * a.bmax_stride + ci] = k ? key_to_float(k) : -__builtin_inff();
      }
    } else {
      const int64_t p = cur.pos0 + pj;
      if (p < cur.L) a.scores[(int64_t)cur.r * a.score_stride + p] = present ? sc : -__builtin_inff();
      if (MAXIMA) {
        uint32_t k = present ? order_key(sc) : 0u;
        k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0xB1, 0xF, 0xF, false));
        k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x4E, 0xF, 0xF, false));
        k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x141, 0xF, 0xF, false));
        if (j == 0 && cur.pos0 < cur.L)
          a.block_max[(int64_t)cur.r * a.bmax_stride + (cur.pos0 >> 3)] = k ? key_to_float(k) : -__builtin_inff();
        if (a.max64) {
          const uint32_t k2 = wave_max_u32(k);
          if (lane == 0 && (int64_t)cur.t * 64 < cur.L)
            a.max64[(int64_t)cur.r * a.max64_stride + cur.t] = k2 ? key_to_float(k2) : -__builtin_inff();
        }
      }
    }
    if (!has_next) break;
    item = next;
    cur = nxt;
    ksc = ksc_next;
  }
}

// ---- FP8 indexer keys: 16-byte loads ----
//
// A 68-byte FP8 entry moves half the bytes of a bf16 one, so with the layout
// above a wave step carries 4 KiB.  Here lane 4g + q (g = 0..15, q = 0..3)
// loads 16 bytes -- the E4M3 codes of channels 16q .. 16q+15, i.e. chunks 2q
// and 2q+1 -- of each of the eight positions of group g: a wave step is 128
// positions and 8 KiB, as for bf16 keys.  The lane runs the two FMA chains of
// its chunks and adds them (the first level of the canonical tree,
// c_{2q} + c_{2q+1}); the two levels left are a reduce-scatter over the four
// lanes of the group (partner q ^ 1, then q ^ 2), after which lane q holds
// positions q and q + 4 of its group, each scaled, ReLU'd and summed over the
// heads as in the kernel above.  Candidate mode: group g of step t is
// candidate block 16 t + g.
template <bool CAND, bool HAS_W, bool MAXIMA>
__global__ __launch_bounds__(kScanWaves * 64) __attribute__((amdgpu_waves_per_eu(4)))
void index_scan_fp8_kernel(IdxArgs a) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 2, q = lane & 3;
  const bool b0 = q & 1, b1 = (q >> 1) & 1;
  const uint32_t n_items = (uint32_t)a.R * (uint32_t)a.steps_per_row;
  const uint32_t item = __builtin_amdgcn_readfirstlane(blockIdx.x * kScanWaves + (threadIdx.x >> 6));
  if (item >= n_items) return;
  const int r = __builtin_amdgcn_readfirstlane((int)(item / (uint32_t)a.steps_per_row));
  const int t = __builtin_amdgcn_readfirstlane((int)(item - (uint32_t)r * (uint32_t)a.steps_per_row));
  const int b = a.row_seq ? a.row_seq[r] : r;
  const int L = __builtin_amdgcn_readfirstlane(min(a.seq_len[b], a.n_max));
  if (!CAND && t * 128 >= L) return;      // past the row's visible positions: nothing to write
  int64_t pos0;
  int ci = 0;
  if (CAND) {
    ci = t * 16 + g;
    const int blk = ci < a.n_cand ? a.cand[(int64_t)r * a.n_cand + ci] : -1;
    pos0 = blk >= 0 ? (int64_t)blk * 8 : (int64_t)1 << 40;
  } else {
    pos0 = (int64_t)t * 128 + g * 8;
  }
  int64_t s0 = 0;
  int nv = 0;
  if (pos0 < L) {
    const int64_t sl = a.map(b, pos0);    // a group of 8 never straddles a page
    if (sl >= 0) {
      nv = (int)min(min((int64_t)L - pos0, a.map.n_slots - sl), (int64_t)8);
      s0 = sl;
    }
  }
  // the eight 16-byte loads at once (slot 0 for absent positions)
  const u32x4_t* kd = (const u32x4_t*)a.kdata;
  u32x4_t kr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) kr[i] = __builtin_nontemporal_load(kd + ((i < nv) ? s0 + i : 0) * 4 + q);
  // scales of the two positions this lane finishes: q and q + 4
  const float sc0 = a.kscale[(q < nv) ? s0 + q : 0];
  const float sc1 = a.kscale[(q + 4 < nv) ? s0 + q + 4 : 0];
  // query channels 16q .. 16q+15 of each head
  float qf[4][16];
  {
    const uint4* qp = (const uint4*)(a.q32 + (int64_t)r * 128);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint4 v = qp[h * 8 + 2 * q + u];
        qf[h][8 * u + 0] = bf16_lo(v.x); qf[h][8 * u + 1] = bf16_hi(v.x);
        qf[h][8 * u + 2] = bf16_lo(v.y); qf[h][8 * u + 3] = bf16_hi(v.y);
        qf[h][8 * u + 4] = bf16_lo(v.z); qf[h][8 * u + 5] = bf16_hi(v.z);
        qf[h][8 * u + 6] = bf16_lo(v.w); qf[h][8 * u + 7] = bf16_hi(v.w);
      }
    }
  }
  float w[4] = {1.f, 1.f, 1.f, 1.f};
  if (HAS_W) {
#pragma unroll
    for (int h = 0; h < 4; ++h) w[h] = a.head_w[(int64_t)r * 4 + h];
  }
  // level 1 in the lane: (c_{2q} + c_{2q+1}) of the eight positions, four heads
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  float P[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float kf[16];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)kr[i][d], false);
      const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)kr[i][d], true);
      kf[4 * d + 0] = lo[0]; kf[4 * d + 1] = lo[1]; kf[4 * d + 2] = hi[0]; kf[4 * d + 3] = hi[1];
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float c0 = 0.0f, c1 = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        c0 = __builtin_fmaf(kf[e], qf[h][e], c0);
        c1 = __builtin_fmaf(kf[8 + e], qf[h][8 + e], c1);
      }
      P[i][h] = c0 + c1;
    }
  }
  // level 2 (partner q ^ 1): lane keeps positions i with (i & 1) == b0
  float Q[4][4], d[2][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float keep = b0 ? P[2 * m + 1][h] : P[2 * m][h];
      const float send = b0 ? P[2 * m][h] : P[2 * m + 1][h];
      Q[m][h] = keep + CSA2_DPP(send, 0xB1);          // quad_perm 1,0,3,2
    }
  // level 3 (partner q ^ 2): of positions b0 + 2m (m = 0..3) keep m with (m & 1) == b1
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float keep = b1 ? Q[2 * u + 1][h] : Q[2 * u][h];
      const float send = b1 ? Q[2 * u][h] : Q[2 * u + 1][h];
      d[u][h] = keep + CSA2_DPP(send, 0x4E);          // quad_perm 2,3,0,1
    }
  // lane q now holds positions b0 + 2 b1 + 4u = q + 4u, u = 0, 1
  float sc[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float scale = u ? sc1 : sc0;
    float rr[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float dh = d[u][h] * scale;
      rr[h] = (dh > 0.0f) ? dh : 0.0f;
    }
    if (HAS_W) {
      const float p0 = w[0] * rr[0], p1 = w[1] * rr[1], p2 = w[2] * rr[2], p3 = w[3] * rr[3];
      sc[u] = (p0 + p1) + (p2 + p3);
    } else {
      sc[u] = (rr[0] + rr[1]) + (rr[2] + rr[3]);
    }
  }
  const bool pres0 = q < nv, pres1 = q + 4 < nv;
  uint32_t k = max(pres0 ? order_key(sc[0]) : 0u, pres1 ? order_key(sc[1]) : 0u);
  if (CAND) {
    const int64_t base = (int64_t)r * a.score_stride + (int64_t)ci * 8;
    if (ci < a.n_cand) {
      a.scores[base + q] = pres0 ? sc[0] : -__builtin_inff();
      a.scores[base + q + 4] = pres1 ? sc[1] : -__builtin_inff();
    }
    if (MAXIMA) {
      k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0xB1, 0xF, 0xF, false));
      k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x4E, 0xF, 0xF, false));
      if (q == 0 && ci < a.n_cand)
        a.block_max[(int64_t)r * a.bmax_stride + ci] = k ? key_to_float(k) : -__builtin_inff();
    }
  } else {
    float* srow = a.scores + (int64_t)r * a.score_stride;
    if (pos0 + q < L) srow[pos0 + q] = pres0 ? sc[0] : -__builtin_inff();
    if (pos0 + q + 4 < L) srow[pos0 + q + 4] = pres1 ? sc[1] : -__builtin_inff();
    if (MAXIMA) {
      k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0xB1, 0xF, 0xF, false));
      k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x4E, 0xF, 0xF, false));
      if (q == 0 && pos0 < L)
        a.block_max[(int64_t)r * a.bmax_stride + (pos0 >> 3)] = k ? key_to_float(k) : -__builtin_inff();
      if (a.max64) {
        // 64-position maxima: lanes 0-31 and 32-63 each cover 64 positions
        k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x124, 0xF, 0xF, false));   // row_ror:4
        k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x128, 0xF, 0xF, false));   // row_ror:8
        k = max(k, (uint32_t)__shfl_xor((int)k, 16, 64));
        const int64_t p64 = (int64_t)t * 128 + (lane >> 5) * 64;
        if ((lane & 31) == 0 && p64 < L)
          a.max64[(int64_t)r * a.max64_stride + (p64 >> 6)] = k ? key_to_float(k) : -__builtin_inff();
      }
    }
  }
}

hipError_t launch_index_score(const IdxArgs& a, bool cand, bool has_w, bool maxima, hipStream_t st) {
  if (a.kscale && !a.row_list && ((uintptr_t)a.kdata & 15u) == 0) {
    // FP8 keys in 16-byte loads: 128 positions (16 candidate blocks) per wave step
    IdxArgs f = a;
    f.steps_per_row = cand ? (a.n_cand + 15) / 16 : (a.n_max + 127) / 128;
    const int64_t items = (int64_t)f.R * f.steps_per_row;
    if (items == 0) return hipSuccess;
    if (items > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((items + kScanWaves - 1) / kScanWaves)), blk(kScanWaves * 64);
#define CSA2_FP8_LAUNCH(C, Wt, M) hipLaunchKernelGGL((index_scan_fp8_kernel<C, Wt, M>), grid, blk, 0, st, f)
    if (cand && maxima) { if (has_w) CSA2_FP8_LAUNCH(true, true, true); else CSA2_FP8_LAUNCH(true, false, true); }
    else if (cand) { if (has_w) CSA2_FP8_LAUNCH(true, true, false); else CSA2_FP8_LAUNCH(true, false, false); }
    else if (maxima) { if (has_w) CSA2_FP8_LAUNCH(false, true, true); else CSA2_FP8_LAUNCH(false, false, true); }
    else { if (has_w) CSA2_FP8_LAUNCH(false, true, false); else CSA2_FP8_LAUNCH(false, false, false); }
#undef CSA2_FP8_LAUNCH
    return hipGetLastError();
  }
  const int64_t items = (int64_t)a.R * a.steps_per_row;
  if (items == 0) return hipSuccess;
  if (items > 0x7FFFFFFFll) return hipErrorInvalidValue;
  // One step per wave: every wave issues its eight loads at once and the
  // hardware refills freed wave slots (measured faster than persistent waves
  // that prefetch their next step).  A row list (device-side count) runs on
  // a persistent grid of ~4 resident blocks per CU instead.
  const bool persist = a.row_list != nullptr;
  int64_t blocks = (items + kScanWaves - 1) / kScanWaves;
  if (persist && blocks > 256 * 4) blocks = 256 * 4;
  const bool fp8 = a.kscale != nullptr;
#define CSA2_IDX_LAUNCH4(C, Wt, M, F)                                                                      \
  do {                                                                                                     \
    if (persist)                                                                                           \
      hipLaunchKernelGGL((index_scan_kernel<C, Wt, M, true, F>), dim3((unsigned)blocks), dim3(kScanWaves * 64), 0, st, a); \
    else                                                                                                   \
      hipLaunchKernelGGL((index_scan_kernel<C, Wt, M, false, F>), dim3((unsigned)blocks), dim3(kScanWaves * 64), 0, st, a); \
  } while (0)
#define CSA2_IDX_LAUNCH(C, Wt, M)              \
  do {                                         \
    if (fp8) CSA2_IDX_LAUNCH4(C, Wt, M, true); \
    else CSA2_IDX_LAUNCH4(C, Wt, M, false);    \
  } while (0)
  if (cand && maxima) {
    if (has_w) CSA2_IDX_LAUNCH(true, true, true); else CSA2_IDX_LAUNCH(true, false, true);
  } else if (cand) {
    if (has_w) CSA2_IDX_LAUNCH(true, true, false); else CSA2_IDX_LAUNCH(true, false, false);
  } else if (maxima) {
    if (has_w) CSA2_IDX_LAUNCH(false, true, true); else CSA2_IDX_LAUNCH(false, false, true);
  } else {
    if (has_w) CSA2_IDX_LAUNCH(false, true, false); else CSA2_IDX_LAUNCH(false, false, false);
  }
#undef CSA2_IDX_LAUNCH
#undef CSA2_IDX_LAUNCH4
  return hipGetLastError();
}

}  // namespace csa2
