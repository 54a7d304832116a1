// FP4 quantisation of main-KV vectors: E2M1 codes with one E4M3 scale per 16
// channels and no global scale, the NVFP4 pattern without its global scale
// (conexaotc.com.br page "DeepSeek lança V4.1-Flash...", paragraph on the KV
// quantisation; 7minutos.es page, section "FP4 KV, repetición limitada y otras
// extensiones").
//
// Per block of 16 channels: amax = max|x|; scale = E4M3(amax / 6) with
// round-to-nearest-even and saturation at 448; code_i = E2M1(x_i / scale) with
// round-to-nearest-even, saturation at 6, sign kept; scale 0 -> all codes 0.
// Both divisions are float32.  One wave per vector: lane l owns channels
// 8l .. 8l+7 (half a scale block) and writes bytes 4l .. 4l+3.
#include "kernels.h"

namespace csa2 {

// E4M3FN code of a finite a >= 0, nearest-even, saturating at 448 (0x7E).
CSA2_DEV uint32_t e4m3_rne(float a) {
  if (!(a < 448.0f)) return 0x7Eu;
  if (a < 0x1p-6f) return (uint32_t)__builtin_rintf(a * 512.0f);   // subnormal grid m * 2^-9
  const uint32_t bits = __float_as_uint(a);
  const uint32_t e = (bits >> 23) - 127u + 7u;                       // biased E4M3 exponent, >= 1
  const uint32_t m23 = bits & 0x7FFFFFu;
  const uint32_t m3 = (m23 + 0x7FFFFu + ((m23 >> 20) & 1u)) >> 20;   // 0..8, ties to even
  const uint32_t code = (e << 3) + m3;                               // m3 == 8 carries
  return code > 0x7Eu ? 0x7Eu : code;
}

// E2M1 code of y: magnitude rounded to {0,.5,1,1.5,2,3,4,6} (ties to the even
// code, saturating at 6); the count of grid midpoints below |y| is the code.
CSA2_DEV uint32_t e2m1_rne(float y) {
  const float m = fabsf(y);
  uint32_t c = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) +
               (m >= 3.5f) + (m > 5.0f);
  return c | (__float_as_uint(y) >> 31 << 3);
}

__global__ __launch_bounds__(256) void fp4_quant_kernel(const float* __restrict__ x, int64_t n,
                                                        const int64_t* __restrict__ dst,
                                                        uint8_t* __restrict__ fp4,
                                                        uint8_t* __restrict__ scale,
                                                        int64_t n_slots) {
  const int lane = threadIdx.x & 63;
  const int64_t v = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (v >= n) return;
  const int64_t slot = dst ? dst[v] : v;
  const float4* src = (const float4*)(x + v * 512 + lane * 8);
  const float4 a0 = src[0], a1 = src[1];
  const float xs[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(xs[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  const uint32_t sc = e4m3_rne(amax / 6.0f);
  const float s = e4m3_to_float(sc);
  uint32_t packed = 0;
  if (s != 0.f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= e2m1_rne(xs[i] / s) << (4 * i);
  }
  if (slot < 0 || slot >= n_slots) return;
  *(uint32_t*)(fp4 + slot * 256 + lane * 4) = packed;
  if ((lane & 1) == 0) scale[slot * 32 + (lane >> 1)] = (uint8_t)sc;
}

// FP8 indexer keys (64 E4M3 codes and a float32 scale per position): one
// wave per key, lane l owns channel l.  s = amax / 448 (float32 division),
// code_l = E4M3(|k_l| / s) nearest-even with the sign of k_l; s == 0 gives
// all codes 0.
__global__ __launch_bounds__(256) void fp8_key_quant_kernel(const uint16_t* __restrict__ k, int64_t n,
                                                            const int64_t* __restrict__ dst,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ scale, int64_t n_slots) {
  const int lane = threadIdx.x & 63;
  const int64_t v = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (v >= n) return;
  const int64_t slot = dst ? dst[v] : v;
  const uint32_t bits = (uint32_t)k[v * 64 + lane] << 16;
  // |k| as float bits orders like |k| (non-negative floats)
  const float amax = __uint_as_float(wave_max_u32(bits & 0x7FFFFFFFu));
  const float s = amax / 448.0f;
  uint32_t code = 0u;
  if (s != 0.0f) code = e4m3_rne(__uint_as_float(bits & 0x7FFFFFFFu) / s) | ((bits >> 31) << 7);
  if (slot < 0 || slot >= n_slots) return;
  codes[slot * 64 + lane] = (uint8_t)code;
  if (lane == 0) scale[slot] = s;
}

hipError_t launch_fp8_key_quant(const uint16_t* k, int64_t n, const int64_t* dst, uint8_t* codes, float* scale,
                                int64_t n_slots, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 3) / 4;
  hipLaunchKernelGGL(fp8_key_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, st, k, n, dst, codes, scale,
                     n_slots);
  return hipGetLastError();
}

hipError_t launch_quant(const float* x, int64_t n, const int64_t* dst, uint8_t* fp4, uint8_t* scale,
                        int64_t n_slots, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 3) / 4;
  hipLaunchKernelGGL(fp4_quant_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, n, dst, fp4, scale,
                     n_slots);
  return hipGetLastError();
}

}  // namespace csa2

namespace csa2 {

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

}  // namespace csa2
