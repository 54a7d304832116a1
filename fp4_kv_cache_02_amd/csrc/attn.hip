// Sparse FP4 attention + sliding window (decode rows and prefill-chunk rows).
//
// Every CSA2 layer combines global (sparse) attention over the selected Top-K
// main-KV entries with a 128-token sliding window, using its own query
// (e-cogni summary of "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
// Compression", sections "O que os autores propõem" and "Como funciona").
// The main KV is E2M1 with one E4M3 scale per 16 channels (conexaotc.com.br
// page, paragraph on the KV quantisation).  Reading taken: one softmax per
// head over the union of both branches; the 512-d main-KV vector is both key
// and value.
//
// Work decomposition.  The keys of a (layer, row) are its k selected main-KV
// entries followed by its window entries, cut into "steps" of 128 keys
// (ceil(k/128) main steps, one window step).  A block of NW waves (4, or 8
// for launches that fit on the CUs at one block each) processes steps of one
// (layer, row); with KPW = 128 / NW keys and DPW = 512 / NW output dims per
// wave:
//   1. wave w computes the logits of keys KPW w .. KPW w + KPW - 1 of the step
//      for all 16 heads: S^T[KPW keys x 16 heads] = K Q^T as KPW / 16 MFMA
//      groups of 16 keys (16x16x32, 16 steps over the 512 dims; lane (c, g) =
//      (l % 16, l / 16) loads key 16u + c of the wave's keys, dims 128g ..
//      128g+127, and reads the query fragment of head c from LDS);
//   2. the block's softmax statistics per head are combined through LDS and
//      P is written to LDS as [16 heads x 128 keys]: for main steps in fp16
//      (11 significant bits; the softmax sum is taken over those rounded
//      weights), for the window step as bf16 hi + lo halves (16 bits);
//   3. wave w computes O[16 heads x dims DPW w .. DPW w + DPW - 1] = P V over
//      all 128 keys: 4 K-steps of 32 keys, NT = DPW / 16 output tiles, tile j
//      covering dims {DPW w + NT c + j : c = 0..15}, so lane (c, g) needs one
//      NT-dim word of each of its 8 keys -- V is read straight from the cache
//      in that layout.
// A block that covers every step of its row (many rows) keeps an online
// softmax over the steps and writes the output; otherwise (few rows: decode)
// each block takes one or two steps (the window step split over two or four
// blocks, so that one CU fetches a half or a quarter of the window K/V) and
// writes a partial (O, max, sum), and
// attn_merge_kernel combines the partials of each row as one softmax.  (A
// cross-block hand-off inside one kernel would need a device-scope release,
// which on this chip writes back the whole L2 of the issuing XCD.)  Several
// layers that share the Top-K (a Full or Reindex layer and its Reuse layers)
// run in one launch.
//
// FP4 -> fp16 is exact: the hardware E2M1 conversion at unit scale (the
// conversion's own scale operand applies only a power of two), then an fp16
// multiply by the E4M3 scale (products have <= 6 significant bits within
// fp16's normal range).  Window steps use bf16 throughout.
#include "attn_util.h"
#include "topk_row.h"
#include "merge_row.h"


namespace csa2 {

constexpr int kStepKeys = 128;                  // keys per step
constexpr int kMaxWaves = 8;                    // waves per block, at most
constexpr int kQRow = 65;                       // uint4 per head row of Q in LDS (64 + 1 pad)
constexpr int kPRow = kStepKeys + 8;            // halves per head row of P in LDS

constexpr int kCodeRow = 68;                   // dwords per staged key row (256 B of codes + 16 B pad)
constexpr int kSh2Row = 34;                    // dwords per staged scale row (32 fp16 pairs + 2 pad)

// Per-wave shape of an NW-wave block.
template <int NW>
struct Shape {
  static constexpr int KPW = kStepKeys / NW;   // keys per wave in QK (32, 16)
  static constexpr int NU = KPW / 16;          // 16-key MFMA groups per wave (2, 1)
  static constexpr int DPW = 512 / NW;         // output dims per wave in PV (128, 64)
  static constexpr int NT = DPW / 16;          // output tiles per wave = dims per lane column (8, 4)
  static constexpr int NQ = 16 * 64 / (64 * NW);   // query uint4 per thread (4, 2)
};

struct AttnSmem {
  uint4 q[16 * kQRow];         // query of the step kind: fp16 (main steps) or bf16 (window step)
  uint16_t p_hi[16 * kPRow];
  uint16_t p_lo[16 * kPRow];
  int32_t slot[kStepKeys];     // slot of each main key of the step (-1: absent)
  uint32_t code[kStepKeys * kCodeRow];   // FP4 codes of the step's main keys
  uint32_t sh2[kStepKeys * kSh2Row];     // their scales as fp16 pairs {s, s}, one per 16 channels (0: absent)
  float red_m[kMaxWaves][16];
  float red_l[kMaxWaves][16];
  float qscale[16];            // main steps: sm_scale * 2^t_h, the query of head h held as q * 2^-t_h
};

// Per-wave running state over the steps of one (layer, row).
template <int NT>
struct RowState {
  f32x4 o[NT];     // O[head 4g+i][dim DPW w + NT c + j] in o[j][i]
  float m[4];      // running max of heads 4g+i (block-wide)
  float l[4];      // running sum of heads 4g+i
};

// ---- phase 1: logits of this wave's keys (lane (c, g): head c, keys sigma(g, e)) ----
// sigma(g, e) = 16 (e / 4) + 4g + e % 4 among the wave's KPW keys
template <int NW>
CSA2_DEV void qk_main(const AttnSmem& sm, int w, int c, int g, float (&s)[4 * Shape<NW>::NU]) {
  using S = Shape<NW>;
  const uint4* qrow = sm.q + c * kQRow + 16 * g;
#pragma unroll
  for (int u = 0; u < S::NU; ++u) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int key = S::KPW * w + 16 * u + c;
    const uint4* src = (const uint4*)&sm.code[key * kCodeRow + 16 * g];
    uint4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = src[i];
    // the fp16 scale pairs of channel blocks 8g .. 8g+7
    const uint2* sp = (const uint2*)&sm.sh2[key * kSh2Row + 8 * g];
    uint32_t sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint2 x = sp[i];
      sv[2 * i] = x.x;
      sv[2 * i + 1] = x.y;
    }
    const uint32_t rw[16] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w,
                             raw[2].x, raw[2].y, raw[2].z, raw[2].w, raw[3].x, raw[3].y, raw[3].z, raw[3].w};
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const half8_t kf = dequant8(rw[t], u2h(sv[t >> 1]));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, as_h8(qrow[t]), acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s[4 * u + i] = acc[i];
  }
}

// Window keys of this wave's 16-key groups: lane (c, g) holds key
// KPW w + 16u + c of the step (window entry koff + that), dims 32t + 8g ..
// 32t + 8g + 7 in its t-th word, so that the four lanes of a key read one
// 64-byte piece of its row per load (a lane reading a contiguous quarter of
// the row touched four times as many cache lines per load; the MFMA's t-th
// step then sums dims 32t .. 32t + 31).  Entry 0 of the buffer stands in for
// an absent key: its logits are replaced by -inf, whatever the entry holds.
// Loaded at the head of the window step, with the query, so that one round
// trip brings both.
template <int NW>
struct WinK {
  uint4 k[Shape<NW>::NU][16];
};
template <int NW>
CSA2_DEV void win_k_load(const AttnLayer& Ly, int b, int wst, int wl, int koff, int nkeys, int w, int c, int g,
                         WinK<NW>& wk) {
  using S = Shape<NW>;
#pragma unroll
  for (int u = 0; u < S::NU; ++u) {
    const int e = S::KPW * w + 16 * u + c, kk = koff + e;
    const bool ok = e < nkeys && kk < wl && wst >= 0 && (int64_t)wst + kk < Ly.S;
    const uint4* src = Ly.swa_k + ((int64_t)b * Ly.S + (ok ? wst + kk : 0)) * 64 + g;
#pragma unroll
    for (int t = 0; t < 16; ++t) wk.k[u][t] = src[4 * t];
  }
}

template <int NW>
CSA2_DEV void qk_win(const AttnSmem& sm, const WinK<NW>& wk, int c, int g, float (&s)[4 * Shape<NW>::NU]) {
  const uint4* qrow = sm.q + c * kQRow + g;
#pragma unroll
  for (int u = 0; u < Shape<NW>::NU; ++u) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 16; ++t)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(wk.k[u][t]), as_bf8(qrow[4 * t]), acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) s[4 * u + i] = acc[i];
  }
}

// ---- phase 3: O[16 heads x dims DPW w .. DPW w + DPW - 1] += P V over the step's 128 keys ----
// Lane (c, g) covers dims DPW w + NT c .. + NT - 1 of keys 32 ks + 8g + i: one
// dword of FP4 codes (NT = 8) or its half (NT = 4), under one scale.
template <int NW>
CSA2_DEV void pv_main(const AttnSmem& sm, RowState<Shape<NW>::NT>& st, int w, int c, int g) {
  using S = Shape<NW>;
  constexpr int NSEL = S::NT / 2;               // code bytes (dim pairs) per lane and key
  const int d0 = S::DPW * w + S::NT * c;        // the lane's first dim
  const int cw = d0 >> 3;                       // its code dword
  const int csh = (d0 & 7) * 4;                 // bit offset of its first code in the dword
  const int sb = d0 >> 4;                       // its scale block
#pragma unroll 1
  for (int ks = 0; ks < 4; ++ks) {
    const int key0 = 32 * ks + 8 * g;
    uint32_t dw[8];
    half2_t sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = key0 + i;
      dw[i] = sm.code[key * kCodeRow + cw] >> csh;
      sv[i] = u2h(sm.sh2[key * kSh2Row + sb]);
    }
    const uint4 ph = *(const uint4*)&sm.p_hi[c * kPRow + key0];
#pragma unroll
    for (int sel = 0; sel < NSEL; ++sel) {
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = h2u(fp4x2(dw[i], sel) * sv[i]);
      const uint4 b0 = make_uint4(pack_lo(h[0], h[1]), pack_lo(h[2], h[3]), pack_lo(h[4], h[5]), pack_lo(h[6], h[7]));
      const uint4 b1 = make_uint4(pack_hi(h[0], h[1]), pack_hi(h[2], h[3]), pack_hi(h[4], h[5]), pack_hi(h[6], h[7]));
      st.o[2 * sel] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(ph), as_h8(b0), st.o[2 * sel], 0, 0, 0);
      st.o[2 * sel + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(ph), as_h8(b1), st.o[2 * sel + 1], 0, 0, 0);
    }
  }
}

// The window keys of a step: entries koff .. koff + nkeys - 1 of the row's
// window (b: the window buffer's sequence).
struct WinGeo {
  int b, wst, wl, koff;
};
CSA2_DEV bool win_key_ok(const AttnLayer& Ly, const WinGeo& wg, int kk) {
  return kk < wg.wl && wg.wst >= 0 && (int64_t)wg.wst + kk < Ly.S;
}

// A lane's window V word for one key: NT bf16 dims (NT = 8: a uint4; NT = 4: a uint2).
template <int NT>
struct VWord;
template <>
struct VWord<8> {
  uint4 v;
  CSA2_DEV uint32_t dw(int m) const { return (m == 0) ? v.x : (m == 1) ? v.y : (m == 2) ? v.z : v.w; }
};
template <>
struct VWord<4> {
  uint2 v;
  CSA2_DEV uint32_t dw(int m) const { return (m == 0) ? v.x : v.y; }
};

// Window V words of keys 32 ks + 8g + i (i < 8) of the step (window entries
// koff + those), dims DPW w + NT c .. + NT - 1; an absent key reads entry 0
// and is zeroed (P is 0 there, but the entry may hold any bits).  The lane's
// word is element 16 w + c of a 1024-B window row in units of its own size.
template <int NW>
CSA2_DEV void win_v_load(const AttnLayer& Ly, const WinGeo& wg, int ks, int w, int c, int g,
                         VWord<Shape<NW>::NT> (&vr)[8]) {
  constexpr int NT = Shape<NW>::NT;
  const int key0 = wg.koff + 32 * ks + 8 * g;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int kk = key0 + i;
    const bool ok = win_key_ok(Ly, wg, kk);
    const int64_t row = (int64_t)wg.b * Ly.S + (ok ? wg.wst + kk : 0);
    const uint32_t m = ok ? 0xFFFFFFFFu : 0u;
    if constexpr (NT == 8) {
      const uint4 x = Ly.swa_v[row * 64 + 16 * w + c];
      vr[i].v = mask4(x, m);
    } else {
      const uint2 x = ((const uint2*)Ly.swa_v)[row * 128 + 16 * w + c];
      vr[i].v = make_uint2(x.x & m, x.y & m);
    }
  }
}

// O += P V over keys 32 ks .. 32 ks + 31 of the window step.
template <int NW>
CSA2_DEV void pv_win_part(const AttnSmem& sm, RowState<Shape<NW>::NT>& st, int ks, int c, int g,
                          const VWord<Shape<NW>::NT> (&v)[8]) {
  const int key0 = 32 * ks + 8 * g;
  const uint4 ph = *(const uint4*)&sm.p_hi[c * kPRow + key0];
  const uint4 pl = *(const uint4*)&sm.p_lo[c * kPRow + key0];
#pragma unroll
  for (int m = 0; m < Shape<NW>::NT / 2; ++m) {
    uint32_t x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = v[i].dw(m);
    const uint4 b0 = make_uint4(pack_lo_w(x[0], x[1]), pack_lo_w(x[2], x[3]), pack_lo_w(x[4], x[5]), pack_lo_w(x[6], x[7]));
    const uint4 b1 = make_uint4(pack_hi_w(x[0], x[1]), pack_hi_w(x[2], x[3]), pack_hi_w(x[4], x[5]), pack_hi_w(x[6], x[7]));
    st.o[2 * m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(ph), as_bf8(b0), st.o[2 * m], 0, 0, 0);
    st.o[2 * m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(pl), as_bf8(b0), st.o[2 * m], 0, 0, 0);
    st.o[2 * m + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(ph), as_bf8(b1), st.o[2 * m + 1], 0, 0, 0);
    st.o[2 * m + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(pl), as_bf8(b1), st.o[2 * m + 1], 0, 0, 0);
  }
}

// Window keys loaded one 16-key group at a time (two blocks per CU: their
// register budget does not hold a wave's keys at once).
template <int NW>
CSA2_DEV void qk_win_seq(const AttnLayer& Ly, const AttnSmem& sm, int b, int wst, int wl, int koff, int nkeys, int w,
                         int c, int g, float (&s)[4 * Shape<NW>::NU]) {
  using S = Shape<NW>;
  const uint4* qrow = sm.q + c * kQRow + g;
#pragma unroll 1
  for (int u = 0; u < S::NU; ++u) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int e = S::KPW * w + 16 * u + c, kk = koff + e;
    const bool ok = e < nkeys && kk < wl && wst >= 0 && (int64_t)wst + kk < Ly.S;
    const uint4* src = Ly.swa_k + ((int64_t)b * Ly.S + (ok ? wst + kk : 0)) * 64 + g;   // as in win_k_load
    uint4 kr[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) kr[t] = src[4 * t];
#pragma unroll
    for (int t = 0; t < 16; ++t)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(kr[t]), as_bf8(qrow[4 * t]), acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) s[4 * u + i] = acc[i];
  }
}
// The window step's P V over its 32-key parts (4, 2 or 1), each part's values
// loaded just ahead of its MFMAs (a wave's registers do not hold the values
// of several parts beside its output tiles at two waves per SIMD).
template <int NW>
CSA2_DEV void pv_win_seq(const AttnLayer& Ly, const WinGeo& wg, const AttnSmem& sm, RowState<Shape<NW>::NT>& st,
                         int nparts, int w, int c, int g) {
#pragma unroll 1
  for (int ks = 0; ks < nparts; ++ks) {
    VWord<Shape<NW>::NT> vr[8];
    win_v_load<NW>(Ly, wg, ks, w, c, g, vr);
    pv_win_part<NW>(sm, st, ks, c, g, vr);
  }
}

// ---- phase 2: softmax statistics of the step (head c), P into LDS, running
// statistics of this lane's output heads 4g+i (O rescaled) ----
template <bool MAIN, int NW>
CSA2_DEV void step_softmax(AttnSmem& sm, RowState<Shape<NW>::NT>& st, float (&s)[4 * Shape<NW>::NU], uint64_t vmask,
                           float sm_scale, int w, int c, int g) {
    using S = Shape<NW>;
    constexpr int NE = 4 * S::NU;
    float cmax = -__builtin_inff();
    // main steps: the logits of head c carry the power of two its fp16 query was scaled by
    const float f = MAIN ? sm.qscale[c] : sm_scale;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int key = 16 * (e >> 2) + 4 * g + (e & 3);
      const bool ok = (vmask >> key) & 1ull;
      s[e] = ok ? s[e] * f : -__builtin_inff();
      cmax = fmaxf(cmax, s[e]);
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    if (g == 0) sm.red_m[w][c] = cmax;
    __syncthreads();
    float mstep = sm.red_m[0][c];
#pragma unroll
    for (int v = 1; v < NW; ++v) mstep = fmaxf(mstep, sm.red_m[v][c]);
    // running max of head c before this step: kept in st.m[c & 3] by the lanes
    // of group c >> 2 (lane 16 * (c >> 2) + c evaluates pick4 with its own c)
    const float mold_c = __shfl(pick4(st.m, c & 3), 16 * (c >> 2) + c, 64);
    const float mnew_c = fmaxf(mold_c, mstep);
    float p[NE], psum = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      p[e] = (mnew_c == -__builtin_inff()) ? 0.f : __expf(s[e] - mnew_c);
      // main steps: the weights as the fp16 values the P V product takes, so
      // that the output is a convex combination of the values
      if (MAIN) p[e] = (float)(_Float16)p[e];
      psum += p[e];
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    if (g == 0) sm.red_l[w][c] = psum;
    // P -> LDS [head c][key KPW w + sigma(g, e)]: fp16 for main steps, bf16
    // hi + lo halves for the window step
    {
      uint32_t hw[NE / 2], lw[NE / 2];
#pragma unroll
      for (int e = 0; e < NE; e += 2) {
        uint32_t h0, h1, l0, l1;
        if (MAIN) {
          h0 = __builtin_bit_cast(uint16_t, (_Float16)p[e]);       // (exact: p is an fp16 value)
          h1 = __builtin_bit_cast(uint16_t, (_Float16)p[e + 1]);
          l0 = l1 = 0;
        } else {
          h0 = f32_to_bf16_rne(p[e]);
          h1 = f32_to_bf16_rne(p[e + 1]);
          l0 = f32_to_bf16_rne(p[e] - __uint_as_float(h0 << 16));
          l1 = f32_to_bf16_rne(p[e + 1] - __uint_as_float(h1 << 16));
        }
        hw[e / 2] = h0 | (h1 << 16);
        lw[e / 2] = l0 | (l1 << 16);
      }
      uint16_t* ph = &sm.p_hi[c * kPRow + S::KPW * w];
      uint16_t* pl = &sm.p_lo[c * kPRow + S::KPW * w];
#pragma unroll
      for (int u = 0; u < S::NU; ++u) {
        *(uint2*)(ph + 16 * u + 4 * g) = make_uint2(hw[2 * u], hw[2 * u + 1]);
        if (!MAIN) *(uint2*)(pl + 16 * u + 4 * g) = make_uint2(lw[2 * u], lw[2 * u + 1]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      float mh = sm.red_m[0][h], lh = sm.red_l[0][h];
#pragma unroll
      for (int v = 1; v < NW; ++v) {
        mh = fmaxf(mh, sm.red_m[v][h]);
        lh += sm.red_l[v][h];
      }
      const float mn = fmaxf(st.m[i], mh);
      const float alpha = (st.m[i] == -__builtin_inff()) ? 0.f : __expf(st.m[i] - mn);
      st.l[i] = st.l[i] * alpha + lh;
      st.m[i] = mn;
      if (alpha != 1.f) {
#pragma unroll
        for (int j = 0; j < S::NT; ++j) st.o[j][i] *= alpha;
      }
    }
}

// The query of the row into LDS from loads issued earlier (uint4 e = tid +
// 64 NW i: head e / 64, piece e % 64): fp16 for main steps, bf16 for the
// window step (per-word selects: a select of whole uint4s becomes a branch
// per load, each waiting for its load).
//
// fp16 holds a narrower range than bf16, so for main steps each head's query
// is first scaled by a power of two 2^-t_h (exact) that puts its largest
// element in [2^14, 2^15); the logits of that head are multiplied by
// sm_scale * 2^t_h instead of sm_scale.  Elements more than 2^28 below the
// head's largest one become fp16 subnormals or zero (a relative change of the
// head's logits below 2^-28 of sum |q| |k|).  Wave w holds heads w + NW i.
template <int NW>
CSA2_DEV void store_q(AttnSmem& sm, const uint4 (&qv)[Shape<NW>::NQ], bool to_f16, int tid, float sm_scale) {
  constexpr int NQ = Shape<NW>::NQ;
  if (!to_f16) {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int e = tid + 64 * NW * i;
      sm.q[(e >> 6) * kQRow + (e & 63)] = qv[i];
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int e = tid + 64 * NW * i;
    // bf16 exponent field of the head's largest |element|; t = exponent - 14,
    // kept >= -126 so that 2^-t and sm_scale * 2^t stay normal floats
    const uint32_t ex = wave_max_u32(bf16_abs_max8(qv[i])) >> 7;
    const int t = max((int)ex - 127 - 14, -126);
    const float down = __uint_as_float((uint32_t)(127 - t) << 23);
    sm.q[(e >> 6) * kQRow + (e & 63)] = bf16x8_to_f16x8_scaled(qv[i], down);
    if ((tid & 63) == 0) sm.qscale[e >> 6] = sm_scale * __uint_as_float((uint32_t)(127 + t) << 23);
  }
}

// BPC: blocks per CU; NW: waves per block.  BPC = 1 (a launch whose blocks
// all fit on the CUs at once, as in decode) runs NW = 8 waves (two per SIMD,
// each with half a step's work): the window step issues all of its keys with
// the query, a main step its indices with the query.  BPC = 2 (many blocks:
// prefill, large decode batches) runs NW = 4 waves and loads the window keys
// one 16-key group at a time.
// LDS of a block: the attention's; with SEL also the final Top-k selection's
// (used first, then given over to the attention) and the selected positions.
template <bool SEL>
struct AttnShared {
  AttnSmem at;
};
template <>
struct AttnShared<true> {
  union {
    AttnSmem at;
    DescFinalSmem topk;
  };
  int32_t sel_pos[CSA2_TOPK];
};

// SEL: the split Top-k's final selection runs at the head of every block of
// main steps (each repeats its row's selection from the segment lists and
// keeps the row's k positions in LDS; one block per row also writes them to
// idx), instead of in a launch of its own whose end the attention would wait
// for.  Window blocks need no indices and start at once.
template <int BPC, int NW, bool SEL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(BPC * NW / 4, BPC * NW / 4)))
void fp4_attn_kernel(AttnArgs a) {
  using S = Shape<NW>;
  constexpr bool kEarly = BPC == 1;
  constexpr int NT = S::NT;
  static_assert(!SEL || NW * 64 == kSelThreads, "the selection runs on blocks of kSelThreads threads");
  __shared__ AttnShared<SEL> shm;
  AttnSmem& sm = shm.at;
  // flat grid: block id = (li * R + r) * n_blocks + blk
  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin by id, so
  // within each run of 8 rows, row 8q + x takes every id = x (mod 8): all
  // layers and steps of a row share one XCD's L2 (the gathered rows, the
  // indices and, for neighbouring prefill rows, the window)
  const int per = a.n_layers * a.n_blocks;                // blocks of one row
  const int full = (a.R / 8) * 8 * per;                   // ids in complete runs of 8 rows
  int r, sub;
  if ((int)blockIdx.x < full) {
    const int q = blockIdx.x / (8 * per), rem = blockIdx.x - q * 8 * per;
    r = 8 * q + (rem & 7);
    sub = rem >> 3;
  } else {
    const int rem = blockIdx.x - full;
    r = (a.R / 8) * 8 + rem / per;
    sub = rem - (rem / per) * per;
  }
  const int li = sub / a.n_blocks, blk = sub - li * a.n_blocks;
  const int lr = li * a.R + r;
  const AttnLayer& Ly = a.layer[li];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, c = lane & 15, g = lane >> 4;
  const int b = a.row_seq ? a.row_seq[r] : r;
  const int L = a.seq_len[b];
  const int n_main = (a.k + kStepKeys - 1) / kStepKeys;
  // One block per row-layer (n_blocks 1, many rows): every step.  Otherwise
  // (decode) the main steps in blocks of steps_per_block (1 or 2), then the
  // window step in one block, or split over nwb = 2 or 4 blocks of 128 / nwb
  // keys (the blocks of the row-layer past its main-step blocks).
  int st0, st1, nwb = 1, wpart = 0;
  bool main_block = true;
  if (a.n_blocks == 1) {
    st0 = 0;
    st1 = n_main + 1;
  } else {
    const int mpb = a.steps_per_block;
    const int nmb = (n_main + mpb - 1) / mpb;           // blocks of main steps
    if (blk < nmb) {
      st0 = blk * mpb;
      st1 = min(n_main, st0 + mpb);
    } else {
      st0 = n_main;
      st1 = n_main + 1;
      nwb = a.n_blocks - nmb;
      wpart = blk - nmb;
      main_block = false;
    }
  }
  const int nwk = kStepKeys / nwb;                                  // the window step's keys in this block
  const int koff = nwk * wpart;                                     // its first window entry
  const int nwp = nwk / 32;                                         // 32-key parts
  const int32_t* idx_row = a.idx + (int64_t)r * a.k;
  CSA2_MARK(a, 0);
  CSA2_SPAN(a, 256, 0);
  if constexpr (SEL) {
    if (main_block) {     // uniform over the block
      desc_final_row(a.sel, r, shm.topk, shm.sel_pos);
      __syncthreads();    // positions visible; the selection's LDS is free
      CSA2_MARK(a, 6);
      if (li == 0 && blk == 0)
        for (int i = threadIdx.x; i < a.k; i += NW * 64) a.sel.out[(int64_t)r * a.sel.out_stride + i] = shm.sel_pos[i];
    }
  }
  // position of rank kk of the row's Top-k (kk < k)
  auto rank_pos = [&](int kk) -> int {
    if constexpr (SEL) return shm.sel_pos[kk];
    else return idx_row[kk];
  };
  const int wst = Ly.swa_start[r];
  const int wl = min(Ly.swa_len[r], CSA2_MAX_WINDOW);

  RowState<NT> st;
#pragma unroll
  for (int j = 0; j < NT; ++j) st.o[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    st.m[i] = -__builtin_inff();
    st.l[i] = 0.f;
  }

  const uint4* qsrc = Ly.q + (int64_t)r * 16 * 64;
  const int wb = Ly.swa_shared ? 0 : b;
  // staging of a main step's rows: thread t loads part t % (NW / 2) of key
  // t / (NW / 2) -- 256 / (NW / 2) bytes of codes and 32 / (NW / 2) of scales;
  // the codes as the 16-byte pieces p + i NW / 2 of the row (i = 0, 1, ...),
  // so that the threads of a key read adjacent pieces with each load
  constexpr int TPK = NW / 2;                 // threads per key (2, 4)
  constexpr int CPT = 16 / TPK;               // uint4 of codes per thread (8, 4)
  constexpr int SPT = 32 / TPK;               // scale bytes per thread (16, 8)
  const int skey = tid / TPK, spart = tid % TPK;
  // The two kinds of step are separate code paths (their registers do not
  // overlap).  In each, the loads that head its longest chain go first -- the
  // main keys' indices (their slots, then their rows), or the window keys --
  // with the query in flight beside them.
  // a block with several main steps loads the next step's indices while the
  // current step runs (the index heads each step's chain of loads)
  int pos_next = -1;
  for (int step = st0; step < st1; ++step) {
    const bool is_main = step < n_main;
    const bool need_q = step == st0 || !is_main;
    if (is_main) {
      // each thread finds the slot of the key it stages (its index, then the
      // slot: no hand-off through LDS ahead of the row loads)
      const int kk = step * kStepKeys + skey;
      const int pos = (step > st0) ? pos_next : (kk < a.k ? rank_pos(kk) : -1);
      uint4 qv[S::NQ];
      if (need_q) {
#pragma unroll
        for (int i = 0; i < S::NQ; ++i) qv[i] = qsrc[tid + 64 * NW * i];   // uint4 e: head e / 64, piece e % 64
        if (!kEarly) store_q<NW>(sm, qv, true, tid, Ly.sm_scale);
      }
      const int32_t sl = (pos >= 0 && pos < L) ? (int32_t)a.map(b, pos) : -1;
      if (spart == 0) sm.slot[skey] = sl;
      // the step's FP4 rows (unconditional loads from slot 0 for absent keys;
      // their scales are zeroed below, so their values are zero)
      const int64_t ss = sl >= 0 ? sl : 0;
      const uint4* src = (const uint4*)(a.kv + ss * 256) + spart;
      uint4 rv[CPT];
#pragma unroll
      for (int i = 0; i < CPT; ++i) rv[i] = src[TPK * i];
      uint32_t rs[SPT / 4];
      if constexpr (SPT == 16) {
        const uint4 x = *(const uint4*)(a.kv_scale + ss * 32 + 16 * spart);
        rs[0] = x.x; rs[1] = x.y; rs[2] = x.z; rs[3] = x.w;
      } else {
        const uint2 x = *(const uint2*)(a.kv_scale + ss * 32 + 8 * spart);
        rs[0] = x.x; rs[1] = x.y;
      }
      const uint32_t rmask = sl >= 0 ? 0xFFFFFFFFu : 0u;
      if (step + 1 < min(st1, n_main)) {
        const int kn = (step + 1) * kStepKeys + skey;
        pos_next = kn < a.k ? rank_pos(kn) : -1;
      }
      if (kEarly && need_q) store_q<NW>(sm, qv, true, tid, Ly.sm_scale);
      // codes as loaded; an absent key's scales are zero, so its values are
      // zero whatever slot 0 holds (its logits are masked as well)
      uint4* dst = (uint4*)&sm.code[skey * kCodeRow] + spart;
#pragma unroll
      for (int i = 0; i < CPT; ++i) dst[TPK * i] = rv[i];
      {
        uint2* sd = (uint2*)&sm.sh2[skey * kSh2Row + SPT * spart];
#pragma unroll
        for (int i = 0; i < SPT / 4; ++i) {
          uint32_t o[4];
          scale_pairs4(rs[i] & rmask, o);
          sd[2 * i] = make_uint2(o[0], o[1]);
          sd[2 * i + 1] = make_uint2(o[2], o[3]);
        }
      }
      __syncthreads();    // query, slots, codes and scales visible
      const uint64_t vmask = __ballot(sm.slot[S::KPW * w + (lane & (S::KPW - 1))] >= 0);
      CSA2_MARK(a, 1);
      float s[4 * S::NU];
      qk_main<NW>(sm, w, c, g, s);
      CSA2_MARK(a, 2);
      step_softmax<true, NW>(sm, st, s, vmask, Ly.sm_scale, w, c, g);
      CSA2_MARK(a, 3);
      pv_main<NW>(sm, st, w, c, g);
      CSA2_MARK(a, 4);
    } else if (!kEarly) {
      uint4 qv[S::NQ];
#pragma unroll
      for (int i = 0; i < S::NQ; ++i) qv[i] = qsrc[tid + 64 * NW * i];
      store_q<NW>(sm, qv, false, tid, Ly.sm_scale);
      const int e = S::KPW * w + (lane & (S::KPW - 1));
      const uint64_t vmask = __ballot(e < nwk && koff + e < wl && wst >= 0 && (int64_t)wst + koff + e < Ly.S);
      __syncthreads();    // query visible
      float s[4 * S::NU];
      qk_win_seq<NW>(Ly, sm, wb, wst, wl, koff, nwk, w, c, g, s);
      step_softmax<false, NW>(sm, st, s, vmask, Ly.sm_scale, w, c, g);
      const WinGeo wg{wb, wst, wl, koff};
      pv_win_seq<NW>(Ly, wg, sm, st, nwp, w, c, g);
    } else {
      WinK<NW> wk;
      win_k_load<NW>(Ly, wb, wst, wl, koff, nwk, w, c, g, wk);
      uint4 qv[S::NQ];
#pragma unroll
      for (int i = 0; i < S::NQ; ++i) qv[i] = qsrc[tid + 64 * NW * i];
      store_q<NW>(sm, qv, false, tid, Ly.sm_scale);
      const int e = S::KPW * w + (lane & (S::KPW - 1));
      const uint64_t vmask = __ballot(e < nwk && koff + e < wl && wst >= 0 && (int64_t)wst + koff + e < Ly.S);
      __syncthreads();    // query visible
      float s[4 * S::NU];
      qk_win<NW>(sm, wk, c, g, s);
      const WinGeo wg{wb, wst, wl, koff};
      step_softmax<false, NW>(sm, st, s, vmask, Ly.sm_scale, w, c, g);
      pv_win_seq<NW>(Ly, wg, sm, st, nwp, w, c, g);
    }
    __syncthreads();    // P, slots and statistics may be overwritten by the next step
  }

  // ---- output (one block per row) or partial: lane (c, g) holds heads 4g+i,
  // dims DPW w + NT c + j ----
  const int d0 = S::DPW * w + NT * c;
  if (a.n_blocks == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      const float inv = (st.l[i] > 0.f) ? 1.0f / st.l[i] : 0.f;
      float* dst = Ly.out + ((int64_t)r * 16 + h) * 512 + d0;
#pragma unroll
      for (int j4 = 0; j4 < NT / 4; ++j4)
        *(float4*)(dst + 4 * j4) = make_float4(st.o[4 * j4][i] * inv, st.o[4 * j4 + 1][i] * inv,
                                               st.o[4 * j4 + 2][i] * inv, st.o[4 * j4 + 3][i] * inv);
      if (Ly.lse && w == 0 && c == 0)
        Ly.lse[(int64_t)r * 16 + h] = (st.l[i] > 0.f) ? st.m[i] + __logf(st.l[i]) : -__builtin_inff();
    }
    CSA2_SPAN(a, 256, 1);
    return;
  }
  const int64_t pidx = (int64_t)lr * a.n_blocks + blk;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    float* dst = a.part_o + pidx * (16 * 512) + h * 512 + d0;
#pragma unroll
    for (int j4 = 0; j4 < NT / 4; ++j4)
      *(float4*)(dst + 4 * j4) = make_float4(st.o[4 * j4][i], st.o[4 * j4 + 1][i], st.o[4 * j4 + 2][i],
                                             st.o[4 * j4 + 3][i]);
    if (w == 0 && c == 0) {
      a.part_ml[pidx * 32 + h * 2 + 0] = st.m[i];
      a.part_ml[pidx * 32 + h * 2 + 1] = st.l[i];
    }
  }
  CSA2_MARK(a, 5);
  CSA2_SPAN(a, 256, 1);
}

// The merge (merge_row.h) as a launch of its own.
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) { merge_block(a, blockIdx.x, threadIdx.x); }

int attn_steps(int k) { return (k + kStepKeys - 1) / kStepKeys + 1; }

int attn_blocks(int k, int rows_x_layers, int* steps_per_block) {
  const int n_steps = attn_steps(k), n_main = n_steps - 1;
  // many row-layers: one block per row-layer writes its output directly
  if (rows_x_layers >= 512) {
    if (steps_per_block) *steps_per_block = n_steps;
    return 1;
  }
  // few (decode): partials + merge.  One main step per block and the window
  // step in four quarters, else in two halves, while the launch fits on the
  // CUs at one block each (else the window step whole, if that fits); past
  // that, two blocks per CU: the window step in halves, and two main steps
  // per block when one each would take the launch past one round of two
  // blocks per CU.
  const int64_t rl = rows_x_layers;
  int mpb = 1, nb = n_main + 2;
  if (rl * (n_main + 4) <= 256) nb = n_main + 4;
  if (rl * (n_main + 2) > 256) {
    if (rl * (n_main + 1) <= 256) {
      nb = n_main + 1;
    } else if (rl * (n_main + 2) > 512 && n_main > 1) {
      mpb = 2;
      nb = (n_main + 1) / 2 + 2;
    }
  }
  if (steps_per_block) *steps_per_block = mpb;
  return nb;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st, const TopkArgs* cand) {
  if (a.R == 0 || a.n_layers == 0) return cand ? launch_seg_final(*cand, st) : hipSuccess;
  const int64_t blocks = (int64_t)a.n_blocks * a.R * a.n_layers;
  const bool sel = a.sel.out != nullptr;    // the split Top-k's final selection is still to run
  if (blocks <= 256) {   // one block of eight waves per CU
    if (sel)
      hipLaunchKernelGGL((fp4_attn_kernel<1, 8, true>), dim3((unsigned)blocks), dim3(8 * 64), 0, st, a);
    else
      hipLaunchKernelGGL((fp4_attn_kernel<1, 8, false>), dim3((unsigned)blocks), dim3(8 * 64), 0, st, a);
  } else {               // two blocks of four waves per CU, after the selection's own launch
    if (sel) {
      const hipError_t e = launch_desc_final(a.sel, st);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((fp4_attn_kernel<2, 4, false>), dim3((unsigned)blocks), dim3(4 * 64), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.n_blocks == 1) return cand ? launch_seg_final(*cand, st) : hipSuccess;
  if (cand) return launch_merge_final(a, *cand, st);
  hipLaunchKernelGGL(attn_merge_kernel, dim3(4 * a.n_layers * a.R), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa2
