// Sparse FP4 attention + sliding window (decode / generic rows).
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
// Decomposition (flash-decoding): a block takes 16*NW keys of one row (main
// keys or window keys, never mixed) and all 16 heads.  Per wave, 16 keys:
//   S^T[16 keys x 16 heads] = K[16 x 512] * Q^T  with 16 MFMA 16x16x32 steps.
//   Lane l loads key l%16, dims 128*(l/16) .. +127 (64 contiguous FP4 bytes +
//   8 scale bytes, or 256 bytes of bf16); the K index of the MFMA walks those
//   dims, and the query fragment uses the same dim order.
// FP4 -> fp16 dequantisation is exact: the hardware E2M1 conversion (scale 1)
// followed by an fp16 multiply by the E4M3 scale (products have <= 6
// significant bits inside fp16's normal range).  Window keys stay bf16.
// Softmax statistics per head over the block; P (fp32) is split into hi + lo
// halves (fp16 for FP4 blocks, bf16 for window blocks) so that P*V keeps ~16+
// bits; V^T is staged in LDS (dim-major, key column swizzled by dim/128) for
// the P*V MFMA (O[16 heads x 512] = P[16 x keys] * V[keys x 512]).
// Each block writes its unnormalised partial (O, max, sum); the last block of
// a row (atomic ticket) merges all partials exactly as one softmax.
#include "kernels.h"

namespace csa2 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));


CSA2_DEV half8_t dequant8(uint32_t word, uint32_t scale_byte) {
  const _Float16 s = (_Float16)e4m3_to_float(scale_byte);
  const half2_t sv = {s, s};
  half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0) * sv;
  half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1) * sv;
  half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2) * sv;
  half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3) * sv;
  half8_t r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

CSA2_DEV half8_t bf16x8_to_half8(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  half8_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = (_Float16)bf16_lo(w[i]);
    r[2 * i + 1] = (_Float16)bf16_hi(w[i]);
  }
  return r;
}

CSA2_DEV bf8_t as_bf8(uint4 v) { return __builtin_bit_cast(bf8_t, v); }
CSA2_DEV uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void fp4_attn_kernel(AttnArgs a) {
  constexpr int KEYS = NW * 16;
  constexpr int VTS = KEYS + 8;       // halves per V^T row (padding keeps 16-B alignment)
  constexpr int PS = KEYS + 8;        // halves per P row
  constexpr int TILES_PER_WAVE = 32 / NW;
  __shared__ __attribute__((aligned(16))) uint16_t vt[512 * VTS];
  __shared__ __attribute__((aligned(16))) uint16_t p_hi[16 * PS];
  __shared__ __attribute__((aligned(16))) uint16_t p_lo[16 * PS];
  __shared__ float red_m[NW][16];
  __shared__ float red_l[NW][16];
  __shared__ float ml[2][16];
  __shared__ uint32_t s_last;

  const int split = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c = l & 15;
  const int b = a.row_seq ? a.row_seq[r] : r;
  const int L = a.seq_len[b];
  const bool is_main = split < a.n_main_splits;
  const int key_local = w * 16 + c;

  // query fragment: head c, dims 128g + 8t .. +7
  const uint4* qrow = a.q + ((int64_t)r * 16 + c) * 64 + g * 16;
  uint4 qf[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) qf[t] = qrow[t];

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  bool valid;
  const int vcol = ((w ^ g) << 4) + c;   // swizzled V^T column of this lane's key
  if (is_main) {
    const int kk = split * KEYS + key_local;
    const int pos = kk < a.k ? a.idx[(int64_t)r * a.k + kk] : -1;
    const int64_t slot = (pos >= 0 && pos < L) ? a.map(b, pos) : -1;
    valid = slot >= 0;
    uint4 raw[4];
    uint2 sc;
    if (valid) {
      const uint4* src = (const uint4*)(a.kv + slot * 256 + g * 64);
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[i] = src[i];
      sc = *(const uint2*)(a.kv_scale + slot * 32 + g * 8);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) raw[i] = make_uint4(0, 0, 0, 0);
      sc = make_uint2(0, 0);
    }
    const uint32_t rw[16] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y,
                             raw[1].z, raw[1].w, raw[2].x, raw[2].y, raw[2].z, raw[2].w,
                             raw[3].x, raw[3].y, raw[3].z, raw[3].w};
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint32_t sbyte = ((t < 8 ? sc.x : sc.y) >> (8 * ((t >> 1) & 3))) & 0xFFu;
      const half8_t kf = dequant8(rw[t], sbyte);
      const half8_t qh = bf16x8_to_half8(qf[t]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qh, acc, 0, 0, 0);
      // V^T: rows 128g + 8t + i, this key's column
      const uint4 kb = __builtin_bit_cast(uint4, kf);
      const uint32_t kw[4] = {kb.x, kb.y, kb.z, kb.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vt[(128 * g + 8 * t + 2 * i) * VTS + vcol] = (uint16_t)(kw[i] & 0xFFFFu);
        vt[(128 * g + 8 * t + 2 * i + 1) * VTS + vcol] = (uint16_t)(kw[i] >> 16);
      }
    }
  } else {
    const int wpos0 = a.swa_start[r];
    const int wl = a.swa_len[r];
    const int kk = (split - a.n_main_splits) * KEYS + key_local;
    valid = kk < wl && kk < CSA2_MAX_WINDOW && wpos0 >= 0 && (int64_t)wpos0 + kk < a.S;
    const int64_t rowoff = ((int64_t)b * a.S + wpos0 + (valid ? kk : 0)) * 64 + g * 16;
    uint4 kr[16], vr[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      kr[t] = valid ? a.swa_k[rowoff + t] : make_uint4(0, 0, 0, 0);
      vr[t] = valid ? a.swa_v[rowoff + t] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint32_t vw[4] = {vr[t].x, vr[t].y, vr[t].z, vr[t].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vt[(128 * g + 8 * t + 2 * i) * VTS + vcol] = (uint16_t)(vw[i] & 0xFFFFu);
        vt[(128 * g + 8 * t + 2 * i + 1) * VTS + vcol] = (uint16_t)(vw[i] >> 16);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(kr[t]), as_bf8(qf[t]), acc, 0, 0, 0);
    }
  }

  // ---- scores and softmax statistics (lane: keys 4g..4g+3 of this wave, head c) ----
  const uint64_t vm = __ballot(valid);
  float s[4];
  float mloc = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool kv_ok = (vm >> (4 * g + i)) & 1ull;
    s[i] = kv_ok ? acc[i] * a.sm_scale : -__builtin_inff();
    mloc = fmaxf(mloc, s[i]);
  }
  mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
  if (g == 0) red_m[w][c] = mloc;
  __syncthreads();
  float m = red_m[0][c];
#pragma unroll
  for (int i = 1; i < NW; ++i) m = fmaxf(m, red_m[i][c]);
  float p[4], lsum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = (m == -__builtin_inff()) ? 0.f : __expf(s[i] - m);
    lsum += p[i];
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (g == 0) red_l[w][c] = lsum;
  // P hi/lo into LDS: P[head c][key w*16 + 4g + i]
  {
    uint16_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (is_main) {
        const _Float16 h = (_Float16)p[i];
        const _Float16 e = (_Float16)(p[i] - (float)h);
        hi[i] = __builtin_bit_cast(uint16_t, h);
        lo[i] = __builtin_bit_cast(uint16_t, e);
      } else {
        const uint16_t h = f32_to_bf16_rne(p[i]);
        const float hf = __uint_as_float((uint32_t)h << 16);
        hi[i] = h;
        lo[i] = f32_to_bf16_rne(p[i] - hf);
      }
    }
    const int off = c * PS + w * 16 + 4 * g;
    *(uint2*)&p_hi[off] = make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
    *(uint2*)&p_lo[off] = make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
  }
  __syncthreads();
  float lt = red_l[0][c];
#pragma unroll
  for (int i = 1; i < NW; ++i) lt += red_l[i][c];

  // ---- O[16 heads x 512] = P[16 x KEYS] * V[KEYS x 512] ----
  f32x4 o[TILES_PER_WAVE];
#pragma unroll
  for (int n = 0; n < TILES_PER_WAVE; ++n) o[n] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KEYS / 32; ++ks) {
    const uint4 ah = *(const uint4*)&p_hi[c * PS + ks * 32 + 8 * g];
    const uint4 al = *(const uint4*)&p_lo[c * PS + ks * 32 + 8 * g];
#pragma unroll
    for (int n = 0; n < TILES_PER_WAVE; ++n) {
      const int dim = (w * TILES_PER_WAVE + n) * 16 + c;
      const int col = (ks * 32 + 8 * g) ^ (((dim >> 7) & 3) << 4);
      const uint4 bv = *(const uint4*)&vt[dim * VTS + col];
      if (is_main) {
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ah),
                                                      __builtin_bit_cast(half8_t, bv), o[n], 0, 0, 0);
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, al),
                                                      __builtin_bit_cast(half8_t, bv), o[n], 0, 0, 0);
      } else {
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(ah), as_bf8(bv), o[n], 0, 0, 0);
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(al), as_bf8(bv), o[n], 0, 0, 0);
      }
    }
  }

  // ---- partial results: O[head 4g+i][dim], max and sum per head ----
  const int64_t pbase = (int64_t)r * a.n_splits + split;
  float* po = a.part_o + pbase * (16 * 512);
#pragma unroll
  for (int n = 0; n < TILES_PER_WAVE; ++n) {
    const int dim = (w * TILES_PER_WAVE + n) * 16 + c;
#pragma unroll
    for (int i = 0; i < 4; ++i) po[(4 * g + i) * 512 + dim] = o[n][i];
  }
  if (tid < 16) {
    a.part_ml[pbase * 32 + tid * 2 + 0] = m;
    a.part_ml[pbase * 32 + tid * 2 + 1] = lt;
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = (atomicAdd(&a.ticket[r], 1u) == (uint32_t)(a.n_splits - 1)) ? 1u : 0u;
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- merge (last block of the row) ----
  if (tid < 16) {
    float M = -__builtin_inff();
    for (int j = 0; j < a.n_splits; ++j)
      M = fmaxf(M, a.part_ml[((int64_t)r * a.n_splits + j) * 32 + tid * 2]);
    float Lsum = 0.f;
    for (int j = 0; j < a.n_splits; ++j) {
      const float mj = a.part_ml[((int64_t)r * a.n_splits + j) * 32 + tid * 2];
      const float lj = a.part_ml[((int64_t)r * a.n_splits + j) * 32 + tid * 2 + 1];
      Lsum += (mj == -__builtin_inff()) ? 0.f : __expf(mj - M) * lj;
    }
    ml[0][tid] = M;
    ml[1][tid] = Lsum;
    if (a.lse) a.lse[(int64_t)r * 16 + tid] = (Lsum > 0.f) ? M + __logf(Lsum) : -__builtin_inff();
  }
  __syncthreads();
  // each thread: 4 consecutive dims of some heads
  for (int e4 = tid; e4 < 16 * 128; e4 += NW * 64) {
    const int h = e4 >> 7, d4 = (e4 & 127) * 4;
    const float M = ml[0][h], Lsum = ml[1][h];
    float4 accv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (Lsum > 0.f) {
      for (int j = 0; j < a.n_splits; ++j) {
        const int64_t pj = (int64_t)r * a.n_splits + j;
        const float mj = a.part_ml[pj * 32 + h * 2];
        if (mj == -__builtin_inff()) continue;
        const float wj = __expf(mj - M);
        const float4 v = *(const float4*)&a.part_o[pj * (16 * 512) + h * 512 + d4];
        accv.x += wj * v.x; accv.y += wj * v.y; accv.z += wj * v.z; accv.w += wj * v.w;
      }
      const float inv = 1.0f / Lsum;
      accv.x *= inv; accv.y *= inv; accv.z *= inv; accv.w *= inv;
    }
    *(float4*)&a.out[((int64_t)r * 16 + h) * 512 + d4] = accv;
  }
  if (tid == 0) a.ticket[r] = 0u;
}

constexpr int kAttnWaves = 4;
constexpr int kAttnKeys = kAttnWaves * 16;

int attn_splits(int k, int* n_main) {
  const int nm = (k + kAttnKeys - 1) / kAttnKeys;
  const int ns = (CSA2_MAX_WINDOW + kAttnKeys - 1) / kAttnKeys;
  if (n_main) *n_main = nm;
  return nm + ns;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
  if (a.R == 0) return hipSuccess;
  hipLaunchKernelGGL(fp4_attn_kernel<kAttnWaves>, dim3(a.n_splits, a.R), dim3(kAttnWaves * 64), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa2
