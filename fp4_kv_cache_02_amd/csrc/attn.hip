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
// (ceil(k/128) main steps, one window step).  A block of 4 waves processes
// steps of one (layer, row):
//   1. wave w computes the logits of keys 32w .. 32w+31 of the step for all 16
//      heads: S^T[32 keys x 16 heads] = K Q^T as two 16-key MFMA groups
//      (16x16x32, 16 steps over the 512 dims; lane (c, g) = (l % 16, l / 16)
//      loads key 16u + c, dims 128g .. 128g+127, and reads the query fragment
//      of head c from LDS);
//   2. the block's softmax statistics per head are combined through LDS and
//      P (split into hi + lo halves, so the product keeps ~22 (fp16) or 16
//      (bf16) bits) is written to LDS as [16 heads x 128 keys];
//   3. wave w computes O[16 heads x dims 128w .. 128w+127] = P V over all 128
//      keys: 4 K-steps of 32 keys, 8 output tiles, tile j covering dims
//      {128w + 8c + j : c = 0..15}, so lane (c, g) needs one 8-dim word of
//      each of its 8 keys -- V is read straight from the cache in that layout.
// A block that covers every step of its row (many rows) keeps an online
// softmax over the steps and writes the output; otherwise (few rows: decode)
// each block takes one step (the window step split over two blocks of 64
// keys, halving the window K/V one CU fetches) and writes a partial (O, max, sum), and
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

namespace csa2 {

constexpr int kAttnWaves = 4;
constexpr int kStepKeys = 128;                  // keys per step (32 per wave)
constexpr int kQRow = 65;                       // uint4 per head row of Q in LDS (64 + 1 pad)
constexpr int kPRow = kStepKeys + 8;            // halves per head row of P in LDS

constexpr int kCodeRow = 68;                   // dwords per staged key row (256 B of codes + 16 B pad)
constexpr int kSh2Row = 34;                    // dwords per staged scale row (32 fp16 pairs + 2 pad)

struct AttnSmem {
  uint4 q[16 * kQRow];         // query of the step kind: fp16 (main steps) or bf16 (window step)
  uint16_t p_hi[16 * kPRow];
  uint16_t p_lo[16 * kPRow];
  int32_t slot[kStepKeys];     // slot of each main key of the step (-1: absent)
  uint32_t code[kStepKeys * kCodeRow];   // FP4 codes of the step's main keys (zeros when absent)
  uint32_t sh2[kStepKeys * kSh2Row];     // their scales as fp16 pairs {s, s}, one per 16 channels (0: absent)
  float red_m[kAttnWaves][16];
  float red_l[kAttnWaves][16];
  float qscale[16];            // main steps: sm_scale * 2^t_h, the query of head h held as q * 2^-t_h
};

// Per-wave running state over the steps of one (layer, row).
struct RowState {
  f32x4 o[8];      // O[head 4g+i][dim 128w + 8c + j] in o[j][i]
  float m[4];      // running max of heads 4g+i (block-wide)
  float l[4];      // running sum of heads 4g+i
};

// ---- phase 1: logits of this wave's 32 keys (lane (c, g): head c, keys sigma(g, e)) ----
// sigma(g, e) = 4g + e (e < 4), 16 + 4g + e - 4 (e >= 4)
CSA2_DEV void qk_main(const AttnSmem& sm, int w, int c, int g, float (&s)[8]) {
  const uint4* qrow = sm.q + c * kQRow + 16 * g;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int key = 32 * w + 16 * u + c;
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

// Window keys of this wave's two 16-key groups: lane (c, g) holds key
// 32w + 16u + c of the step (window entry koff + that), dims 128g .. 128g+127
// (entry 0 of the buffer stands in for an absent key: its logits are replaced
// by -inf, whatever the entry holds).  Loaded at the head of the window step,
// with the query, so that one round trip brings both.
struct WinK {
  uint4 k[2][16];
};
CSA2_DEV void win_k_load(const AttnLayer& Ly, int b, int wst, int wl, int koff, int nkeys, int w, int c, int g,
                         WinK& wk) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = 32 * w + 16 * u + c, kk = koff + e;
    const bool ok = e < nkeys && kk < wl && wst >= 0 && (int64_t)wst + kk < Ly.S;
    const uint4* src = Ly.swa_k + ((int64_t)b * Ly.S + (ok ? wst + kk : 0)) * 64 + g * 16;
#pragma unroll
    for (int t = 0; t < 16; ++t) wk.k[u][t] = src[t];
  }
}

CSA2_DEV void qk_win(const AttnSmem& sm, const WinK& wk, int c, int g, float (&s)[8]) {
  const uint4* qrow = sm.q + c * kQRow + 16 * g;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 16; ++t)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(wk.k[u][t]), as_bf8(qrow[t]), acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) s[4 * u + i] = acc[i];
  }
}

// ---- phase 3: O[16 heads x dims 128w .. 128w+127] += P V over the step's 128 keys ----
CSA2_DEV void pv_main(const AttnSmem& sm, RowState& st, int w, int c, int g) {
#pragma unroll 1
  for (int ks = 0; ks < 4; ++ks) {
    const int key0 = 32 * ks + 8 * g;
    uint32_t dw[8];
    half2_t sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = key0 + i;
      dw[i] = sm.code[key * kCodeRow + 16 * w + c];
      sv[i] = u2h(sm.sh2[key * kSh2Row + 8 * w + (c >> 1)]);
    }
    const uint4 ph = *(const uint4*)&sm.p_hi[c * kPRow + key0];
    const uint4 pl = *(const uint4*)&sm.p_lo[c * kPRow + key0];
#pragma unroll
    for (int sel = 0; sel < 4; ++sel) {
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = h2u(fp4x2(dw[i], sel) * sv[i]);
      const uint4 b0 = make_uint4(pack_lo(h[0], h[1]), pack_lo(h[2], h[3]), pack_lo(h[4], h[5]), pack_lo(h[6], h[7]));
      const uint4 b1 = make_uint4(pack_hi(h[0], h[1]), pack_hi(h[2], h[3]), pack_hi(h[4], h[5]), pack_hi(h[6], h[7]));
      st.o[2 * sel] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(ph), as_h8(b0), st.o[2 * sel], 0, 0, 0);
      st.o[2 * sel] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(pl), as_h8(b0), st.o[2 * sel], 0, 0, 0);
      st.o[2 * sel + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(ph), as_h8(b1), st.o[2 * sel + 1], 0, 0, 0);
      st.o[2 * sel + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(pl), as_h8(b1), st.o[2 * sel + 1], 0, 0, 0);
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

// Window V words of keys 32 ks + 8g + i (i < 8) of the step (window entries
// koff + those), dims 128w + 8c .. 128w + 8c + 7; an absent key reads entry 0
// and is zeroed (P is 0 there, but the entry may hold any bits).
CSA2_DEV void win_v_load(const AttnLayer& Ly, const WinGeo& wg, int ks, int w, int c, int g, uint4 (&vr)[8]) {
  const int key0 = wg.koff + 32 * ks + 8 * g;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int kk = key0 + i;
    const bool ok = win_key_ok(Ly, wg, kk);
    vr[i] = Ly.swa_v[((int64_t)wg.b * Ly.S + (ok ? wg.wst + kk : 0)) * 64 + 16 * w + c];
    vr[i] = mask4(vr[i], ok ? 0xFFFFFFFFu : 0u);
  }
}

// O += P V over keys 32 ks .. 32 ks + 31 of the window step.
CSA2_DEV void pv_win_part(const AttnLayer& Ly, const WinGeo& wg, const AttnSmem& sm, RowState& st, int ks, int c,
                          int g, const uint4 (&v)[8]) {
  const int key0 = 32 * ks + 8 * g;
  const uint4 ph = *(const uint4*)&sm.p_hi[c * kPRow + key0];
  const uint4 pl = *(const uint4*)&sm.p_lo[c * kPRow + key0];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    uint32_t x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (m == 0) ? v[i].x : (m == 1) ? v[i].y : (m == 2) ? v[i].z : v[i].w;
    const uint4 b0 = make_uint4(pack_lo_w(x[0], x[1]), pack_lo_w(x[2], x[3]), pack_lo_w(x[4], x[5]), pack_lo_w(x[6], x[7]));
    const uint4 b1 = make_uint4(pack_hi_w(x[0], x[1]), pack_hi_w(x[2], x[3]), pack_hi_w(x[4], x[5]), pack_hi_w(x[6], x[7]));
    st.o[2 * m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(ph), as_bf8(b0), st.o[2 * m], 0, 0, 0);
    st.o[2 * m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(pl), as_bf8(b0), st.o[2 * m], 0, 0, 0);
    st.o[2 * m + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(ph), as_bf8(b1), st.o[2 * m + 1], 0, 0, 0);
    st.o[2 * m + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(pl), as_bf8(b1), st.o[2 * m + 1], 0, 0, 0);
  }
}

// The window step's P V over its 32-key parts (4, or 2 for half a window):
// the first two were loaded before the softmax statistics; the later ones are
// loaded ahead of the MFMAs that precede their use.
CSA2_DEV void pv_win(const AttnLayer& Ly, const WinGeo& wg, const AttnSmem& sm, RowState& st, int nparts, int w,
                     int c, int g, const uint4 (&v0)[8], const uint4 (&v1)[8]) {
  if (nparts <= 2) {
    pv_win_part(Ly, wg, sm, st, 0, c, g, v0);
    pv_win_part(Ly, wg, sm, st, 1, c, g, v1);
    return;
  }
  uint4 v2[8], v3[8];
  win_v_load(Ly, wg, 2, w, c, g, v2);
  pv_win_part(Ly, wg, sm, st, 0, c, g, v0);
  win_v_load(Ly, wg, 3, w, c, g, v3);
  pv_win_part(Ly, wg, sm, st, 1, c, g, v1);
  pv_win_part(Ly, wg, sm, st, 2, c, g, v2);
  pv_win_part(Ly, wg, sm, st, 3, c, g, v3);
}

// Window step with loads issued part by part (the variant with two blocks
// per CU, whose register budget does not hold the batched loads).
CSA2_DEV void qk_win_seq(const AttnLayer& Ly, const AttnSmem& sm, int b, int wst, int wl, int koff, int nkeys, int w,
                         int c, int g, float (&s)[8]) {
  const uint4* qrow = sm.q + c * kQRow + 16 * g;
#pragma unroll 1
  for (int u = 0; u < 2; ++u) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int e = 32 * w + 16 * u + c, kk = koff + e;
    const bool ok = e < nkeys && kk < wl && wst >= 0 && (int64_t)wst + kk < Ly.S;
    const uint4* src = Ly.swa_k + ((int64_t)b * Ly.S + (ok ? wst + kk : 0)) * 64 + g * 16;
    uint4 kr[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) kr[t] = src[t];
#pragma unroll
    for (int t = 0; t < 16; ++t)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(kr[t]), as_bf8(qrow[t]), acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) s[4 * u + i] = acc[i];
  }
}
CSA2_DEV void pv_win_seq(const AttnLayer& Ly, const WinGeo& wg, const AttnSmem& sm, RowState& st, int nparts, int w,
                         int c, int g) {
#pragma unroll 1
  for (int ks = 0; ks < nparts; ++ks) {
    uint4 vr[8];
    win_v_load(Ly, wg, ks, w, c, g, vr);
    pv_win_part(Ly, wg, sm, st, ks, c, g, vr);
  }
}

// ---- phase 2: softmax statistics of the step (head c), P into LDS, running
// statistics of this lane's output heads 4g+i (O rescaled) ----
template <bool MAIN>
CSA2_DEV void step_softmax(AttnSmem& sm, RowState& st, float (&s)[8], uint64_t vmask, float sm_scale, int w, int c,
                           int g) {
    float cmax = -__builtin_inff();
    // main steps: the logits of head c carry the power of two its fp16 query was scaled by
    const float f = MAIN ? sm.qscale[c] : sm_scale;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = (e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4);
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
    for (int v = 1; v < kAttnWaves; ++v) mstep = fmaxf(mstep, sm.red_m[v][c]);
    // running max of head c before this step: kept in st.m[c & 3] by the lanes
    // of group c >> 2 (lane 16 * (c >> 2) + c evaluates pick4 with its own c)
    const float mold_c = __shfl(pick4(st.m, c & 3), 16 * (c >> 2) + c, 64);
    const float mnew_c = fmaxf(mold_c, mstep);
    float p[8], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = (mnew_c == -__builtin_inff()) ? 0.f : __expf(s[e] - mnew_c);
      psum += p[e];
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    if (g == 0) sm.red_l[w][c] = psum;
    // P hi/lo -> LDS [head c][key 32w + sigma(g, e)]
    {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        uint32_t h0, h1, l0, l1;
        if (MAIN) {
          const _Float16 a0 = (_Float16)p[e], a1 = (_Float16)p[e + 1];
          h0 = __builtin_bit_cast(uint16_t, a0);
          h1 = __builtin_bit_cast(uint16_t, a1);
          l0 = __builtin_bit_cast(uint16_t, (_Float16)(p[e] - (float)a0));
          l1 = __builtin_bit_cast(uint16_t, (_Float16)(p[e + 1] - (float)a1));
        } else {
          h0 = f32_to_bf16_rne(p[e]);
          h1 = f32_to_bf16_rne(p[e + 1]);
          l0 = f32_to_bf16_rne(p[e] - __uint_as_float(h0 << 16));
          l1 = f32_to_bf16_rne(p[e + 1] - __uint_as_float(h1 << 16));
        }
        hw[e / 2] = h0 | (h1 << 16);
        lw[e / 2] = l0 | (l1 << 16);
      }
      uint16_t* ph = &sm.p_hi[c * kPRow + 32 * w];
      uint16_t* pl = &sm.p_lo[c * kPRow + 32 * w];
      *(uint2*)(ph + 4 * g) = make_uint2(hw[0], hw[1]);
      *(uint2*)(ph + 16 + 4 * g) = make_uint2(hw[2], hw[3]);
      *(uint2*)(pl + 4 * g) = make_uint2(lw[0], lw[1]);
      *(uint2*)(pl + 16 + 4 * g) = make_uint2(lw[2], lw[3]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      float mh = sm.red_m[0][h], lh = sm.red_l[0][h];
#pragma unroll
      for (int v = 1; v < kAttnWaves; ++v) {
        mh = fmaxf(mh, sm.red_m[v][h]);
        lh += sm.red_l[v][h];
      }
      const float mn = fmaxf(st.m[i], mh);
      const float alpha = (st.m[i] == -__builtin_inff()) ? 0.f : __expf(st.m[i] - mn);
      st.l[i] = st.l[i] * alpha + lh;
      st.m[i] = mn;
      if (alpha != 1.f) {
#pragma unroll
        for (int j = 0; j < 8; ++j) st.o[j][i] *= alpha;
      }
    }
}

// The query of the row into LDS from loads issued earlier: fp16 for main
// steps, bf16 for the window step (per-word selects: a select of whole uint4s
// becomes a branch per load, each waiting for its load).
//
// fp16 holds a narrower range than bf16, so for main steps each head's query
// is first scaled by a power of two 2^-t_h (exact) that puts its largest
// element in [2^14, 2^15); the logits of that head are multiplied by
// sm_scale * 2^t_h instead of sm_scale.  Elements more than 2^28 below the
// head's largest one become fp16 subnormals or zero (a relative change of the
// head's logits below 2^-28 of sum |q| |k|).  Wave w holds heads w + 4i.
CSA2_DEV void store_q(AttnSmem& sm, const uint4 (&qv)[4], bool to_f16, int tid, float sm_scale) {
  if (!to_f16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      sm.q[(e >> 6) * kQRow + (e & 63)] = qv[i];
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i;
    // bf16 exponent field of the head's largest |element|; t = exponent - 14,
    // kept >= -126 so that 2^-t and sm_scale * 2^t stay normal floats
    const uint32_t ex = wave_max_u32(bf16_abs_max8(qv[i])) >> 7;
    const int t = max((int)ex - 127 - 14, -126);
    const float down = __uint_as_float((uint32_t)(127 - t) << 23);
    sm.q[(e >> 6) * kQRow + (e & 63)] = bf16x8_to_f16x8_scaled(qv[i], down);
    if ((tid & 63) == 0) sm.qscale[e >> 6] = sm_scale * __uint_as_float((uint32_t)(127 + t) << 23);
  }
}

// WPE: waves per SIMD (blocks per CU).  WPE = 1 (a launch whose blocks all
// fit on the CUs at once, as in decode) doubles the registers of a wave: the
// window step then issues its keys with the query and its values ahead of
// use, and a main step its indices with the query.  WPE = 2 (many blocks,
// prefill) loads them part by part.
template <int WPE>
__global__ __launch_bounds__(kAttnWaves * 64) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void fp4_attn_kernel(AttnArgs a) {
  constexpr bool kEarly = WPE == 1;
  __shared__ AttnSmem sm;
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
  // window step in one block, or split over two blocks of 64 keys (whalf 0,
  // 1) when the row-layer has one block more.
  int st0, st1, whalf = -1;
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
      if (a.n_blocks == nmb + 2) whalf = blk - nmb;
    }
  }
  const int koff = whalf < 0 ? 0 : (kStepKeys / 2) * whalf;        // the step's first window entry
  const int nwk = whalf < 0 ? kStepKeys : kStepKeys / 2;           // its window keys
  const int nwp = nwk / 32;                                         // 32-key parts
  const int32_t* idx_row = a.idx + (int64_t)r * a.k;
  const int wst = Ly.swa_start[r];
  const int wl = min(Ly.swa_len[r], CSA2_MAX_WINDOW);
  CSA2_MARK(a, 0);
  CSA2_SPAN(a, 256, 0);

  RowState st;
#pragma unroll
  for (int j = 0; j < 8; ++j) st.o[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    st.m[i] = -__builtin_inff();
    st.l[i] = 0.f;
  }

  const uint4* qsrc = Ly.q + (int64_t)r * 16 * 64;
  const int wb = Ly.swa_shared ? 0 : b;
  // The two kinds of step are separate code paths (their registers do not
  // overlap).  In each, the loads that head its longest chain go first -- the
  // main keys' indices (their slots, then their rows), or the window keys --
  // with the query in flight beside them.
  // a block with several main steps loads the next step's index while the
  // current step runs (the index heads each step's chain of loads)
  int pos_next = -1;
  for (int step = st0; step < st1; ++step) {
    const bool is_main = step < n_main;
    const bool need_q = step == st0 || !is_main;
    if (is_main) {
      int pos = -1;
      if (tid < kStepKeys) {
        const int kk = step * kStepKeys + tid;
        pos = (step > st0) ? pos_next : (kk < a.k ? idx_row[kk] : -1);
      }
      uint4 qv[4];
      if (need_q) {
#pragma unroll
        for (int i = 0; i < 4; ++i) qv[i] = qsrc[tid + 256 * i];   // uint4 e: head e / 64, piece e % 64
        if (!kEarly) store_q(sm, qv, true, tid, Ly.sm_scale);
      }
      if (tid < kStepKeys) sm.slot[tid] = (pos >= 0 && pos < L) ? (int32_t)a.map(b, pos) : -1;
      __syncthreads();
      // the step's FP4 rows: thread t loads half (t & 1) of key t >> 1
      // (unconditional loads from slot 0 for absent keys, zeroed after)
      const int key = tid >> 1, half = tid & 1;
      const int32_t sl = sm.slot[key];
      const int64_t ss = sl >= 0 ? sl : 0;
      const uint4* src = (const uint4*)(a.kv + ss * 256 + 128 * half);
      uint4 rv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) rv[i] = src[i];
      const uint4 rsc = *(const uint4*)(a.kv_scale + ss * 32 + 16 * half);
      const uint32_t rmask = sl >= 0 ? 0xFFFFFFFFu : 0u;    // (a select of whole uint4s goes through scratch)
      if (tid < kStepKeys && step + 1 < min(st1, n_main)) {
        const int kk = (step + 1) * kStepKeys + tid;
        pos_next = kk < a.k ? idx_row[kk] : -1;
      }
      if (kEarly && need_q) store_q(sm, qv, true, tid, Ly.sm_scale);
      // codes as loaded; an absent key's scales are zero, so its values are
      // zero whatever slot 0 holds (its logits are masked as well)
      uint4* dst = (uint4*)&sm.code[key * kCodeRow + 32 * half];
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[i] = rv[i];
      {
        const uint4 scz = mask4(rsc, rmask);
        const uint32_t sw[4] = {scz.x, scz.y, scz.z, scz.w};
        uint2* sd = (uint2*)&sm.sh2[key * kSh2Row + 16 * half];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t o[4];
          scale_pairs4(sw[i], o);
          sd[2 * i] = make_uint2(o[0], o[1]);
          sd[2 * i + 1] = make_uint2(o[2], o[3]);
        }
      }
      const uint64_t vmask = __ballot(sm.slot[32 * w + (lane & 31)] >= 0);
      __syncthreads();    // query, codes and scales visible
      CSA2_MARK(a, 1);
      float s[8];
      qk_main(sm, w, c, g, s);
      CSA2_MARK(a, 2);
      step_softmax<true>(sm, st, s, vmask, Ly.sm_scale, w, c, g);
      CSA2_MARK(a, 3);
      pv_main(sm, st, w, c, g);
      CSA2_MARK(a, 4);
    } else if (!kEarly) {
      uint4 qv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) qv[i] = qsrc[tid + 256 * i];
      store_q(sm, qv, false, tid, Ly.sm_scale);
      const int e = 32 * w + (lane & 31);
      const uint64_t vmask = __ballot(e < nwk && koff + e < wl && wst >= 0 && (int64_t)wst + koff + e < Ly.S);
      __syncthreads();    // query visible
      float s[8];
      qk_win_seq(Ly, sm, wb, wst, wl, koff, nwk, w, c, g, s);
      step_softmax<false>(sm, st, s, vmask, Ly.sm_scale, w, c, g);
      const WinGeo wg{wb, wst, wl, koff};
      pv_win_seq(Ly, wg, sm, st, nwp, w, c, g);
    } else {
      WinK wk;
      win_k_load(Ly, wb, wst, wl, koff, nwk, w, c, g, wk);
      uint4 qv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) qv[i] = qsrc[tid + 256 * i];
      store_q(sm, qv, false, tid, Ly.sm_scale);
      const int e = 32 * w + (lane & 31);
      const uint64_t vmask = __ballot(e < nwk && koff + e < wl && wst >= 0 && (int64_t)wst + koff + e < Ly.S);
      __syncthreads();    // query visible
      float s[8];
      qk_win(sm, wk, c, g, s);
      // the first two 32-key parts of the values, in flight during the statistics
      const WinGeo wg{wb, wst, wl, koff};
      uint4 v0[8], v1[8];
      win_v_load(Ly, wg, 0, w, c, g, v0);
      win_v_load(Ly, wg, 1, w, c, g, v1);
      step_softmax<false>(sm, st, s, vmask, Ly.sm_scale, w, c, g);
      pv_win(Ly, wg, sm, st, nwp, w, c, g, v0, v1);
    }
    __syncthreads();    // P, slots and statistics may be overwritten by the next step
  }

  // ---- output (one block per row) or partial ----
  if (a.n_blocks == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      const float inv = (st.l[i] > 0.f) ? 1.0f / st.l[i] : 0.f;
      float* dst = Ly.out + ((int64_t)r * 16 + h) * 512 + 128 * w + 8 * c;
      *(float4*)dst = make_float4(st.o[0][i] * inv, st.o[1][i] * inv, st.o[2][i] * inv, st.o[3][i] * inv);
      *(float4*)(dst + 4) = make_float4(st.o[4][i] * inv, st.o[5][i] * inv, st.o[6][i] * inv, st.o[7][i] * inv);
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
    float* dst = a.part_o + pidx * (16 * 512) + h * 512 + 128 * w + 8 * c;
    *(float4*)dst = make_float4(st.o[0][i], st.o[1][i], st.o[2][i], st.o[3][i]);
    *(float4*)(dst + 4) = make_float4(st.o[4][i], st.o[5][i], st.o[6][i], st.o[7][i]);
    if (w == 0 && c == 0) {
      a.part_ml[pidx * 32 + h * 2 + 0] = st.m[i];
      a.part_ml[pidx * 32 + h * 2 + 1] = st.l[i];
    }
  }
  CSA2_MARK(a, 5);
  CSA2_SPAN(a, 256, 1);
}

// One block per (layer, row, quarter of the heads): out = sum_j w_j O_j /
// sum_j w_j l_j with w_j = exp(m_j - max_j m_j), the partials of the row's
// blocks merged as one softmax; lse = max + log(sum).  Block id = quarter *
// (layers x rows) + layer * R + row.
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const int nlr = a.n_layers * a.R;
  const int hq = blockIdx.x / nlr, lr = blockIdx.x - hq * nlr;   // lr = li * R + r
  const int li = lr / a.R, r = lr - li * a.R;
  const AttnLayer& Ly = a.layer[li];
  const int tid = threadIdx.x, th = 4 * hq + (tid >> 6), tc = tid & 63;   // head th, dims 8tc .. 8tc+7
  const int64_t prow = (int64_t)lr * a.n_blocks;
  CSA2_MARK(a, 16);
  CSA2_SPAN(a, 1280, 0);
  // every load is unconditional (blocks past n_blocks re-read the last one
  // and get weight 0), so all of them are in flight at once
  float mj[kMaxAttnBlocks], lj[kMaxAttnBlocks];
  float4 v[kMaxAttnBlocks][2];
#pragma unroll
  for (int j = 0; j < kMaxAttnBlocks; ++j) {
    const int64_t pj = prow + min(j, a.n_blocks - 1);
    mj[j] = a.part_ml[pj * 32 + th * 2 + 0];
    lj[j] = a.part_ml[pj * 32 + th * 2 + 1];
    const float* po = a.part_o + pj * (16 * 512) + th * 512 + tc * 8;
    v[j][0] = *(const float4*)po;
    v[j][1] = *(const float4*)(po + 4);
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < kMaxAttnBlocks; ++j) M = fmaxf(M, j < a.n_blocks ? mj[j] : -__builtin_inff());
  CSA2_MARK(a, 17);
  float Lsum = 0.f, wj[kMaxAttnBlocks];
#pragma unroll
  for (int j = 0; j < kMaxAttnBlocks; ++j) {
    wj[j] = (j >= a.n_blocks || mj[j] == -__builtin_inff()) ? 0.f : __expf(mj[j] - M);
    Lsum += wj[j] * lj[j];
  }
  float4 acc[2];
#pragma unroll
  for (int q4 = 0; q4 < 2; ++q4) acc[q4] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < kMaxAttnBlocks; ++j) {
#pragma unroll
    for (int q4 = 0; q4 < 2; ++q4) {
      acc[q4].x += wj[j] * v[j][q4].x;
      acc[q4].y += wj[j] * v[j][q4].y;
      acc[q4].z += wj[j] * v[j][q4].z;
      acc[q4].w += wj[j] * v[j][q4].w;
    }
  }
  const float inv = (Lsum > 0.f) ? 1.0f / Lsum : 0.f;
  float* out_row = Ly.out + ((int64_t)r * 16 + th) * 512 + tc * 8;
#pragma unroll
  for (int q4 = 0; q4 < 2; ++q4)
    *(float4*)(out_row + 4 * q4) = make_float4(acc[q4].x * inv, acc[q4].y * inv, acc[q4].z * inv, acc[q4].w * inv);
  if (Ly.lse && tc == 0) Ly.lse[(int64_t)r * 16 + th] = (Lsum > 0.f) ? M + __logf(Lsum) : -__builtin_inff();
  CSA2_MARK(a, 18);
  CSA2_SPAN(a, 1280, 1);
}

int attn_steps(int k) { return (k + kStepKeys - 1) / kStepKeys + 1; }

int attn_blocks(int k, int rows_x_layers, int* steps_per_block) {
  const int n_steps = attn_steps(k), n_main = n_steps - 1;
  // many row-layers: one block per row-layer writes its output directly
  if (rows_x_layers >= 512) {
    if (steps_per_block) *steps_per_block = n_steps;
    return 1;
  }
  // few (decode): partials + merge.  One main step per block and the window
  // step in two halves while the launch fits on the CUs at one block each
  // (else the window step whole, if that fits); past that, two blocks per CU:
  // the window step in halves, and two main steps per block when one each
  // would take the launch past one round of two blocks per CU.
  const int64_t rl = rows_x_layers;
  int mpb = 1, nb = n_main + 2;
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

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
  if (a.R == 0 || a.n_layers == 0) return hipSuccess;
  const int64_t blocks = (int64_t)a.n_blocks * a.R * a.n_layers;
  if (blocks <= 256)   // one block per CU
    hipLaunchKernelGGL(fp4_attn_kernel<1>, dim3((unsigned)blocks), dim3(kAttnWaves * 64), 0, st, a);
  else
    hipLaunchKernelGGL(fp4_attn_kernel<2>, dim3((unsigned)blocks), dim3(kAttnWaves * 64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_blocks == 1) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(4 * a.n_layers * a.R), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa2
