// Row-wise MXFP4 quantisation and exact dequantisation (gfx950).
//
// Format: two E2M1 codes per byte (element 2m in the low nibble), one UE8M0
// scale per 32 elements along K (OCP Microscaling Formats v1.0; the pages
// "Integrate finegrained kernels ..." note that the mxfp4 format pins UE8M0
// scales and that the row-wise quantizers run one launch per tensor).
// Both kernels are HBM-bound streaming kernels: 4 fp32 (16 B) in and 2 B of
// codes out per lane, eight lanes per 32-block.
#include "common.hpp"
#include "launch.hpp"

namespace mxmoe {

// Shared exponent of a block: the smallest e with 6 * 2^e >= amax, clamped
// to [-127, 127].  For a normal amax = 1.m * 2^(E-127): e = E - 129 when
// 1.m <= 1.5 and E - 128 otherwise; subnormal or zero amax clamps to -127.
__device__ __forceinline__ int block_exponent(float amax) {
  uint32_t bits = __float_as_uint(amax);
  int E = (int)(bits >> 23);
  uint32_t mant = bits & 0x7FFFFFu;
  int e = (E == 0) ? -127 : ((mant <= 0x400000u) ? E - 129 : E - 128);
  return max(-127, min(127, e));
}

// Nearest E2M1 code to y, ties to the even code, sign bit kept.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  float m = fabsf(y);
  uint32_t c = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) +
               (m >= 3.5f) + (m > 5.0f);
  return c | ((__float_as_uint(y) >> 31) << 3);
}

__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w, int64_t n4,
                                                       uint16_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // index of a group of 4 elements
  bool live = i < n4;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (live) v = *reinterpret_cast<const f32x4*>(w + i * 4);
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  // eight consecutive lanes hold one 32-block (blocks never straddle rows)
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  int e = block_exponent(amax);
  if (!live) return;
  uint32_t c0 = e2m1_code(ldexpf(v[0], -e));
  uint32_t c1 = e2m1_code(ldexpf(v[1], -e));
  uint32_t c2 = e2m1_code(ldexpf(v[2], -e));
  uint32_t c3 = e2m1_code(ldexpf(v[3], -e));
  codes[i] = (uint16_t)(c0 | (c1 << 4) | (c2 << 8) | (c3 << 12));
  if ((i & 7) == 0) scales[i >> 3] = (uint8_t)(e + 127);
}

// Each lane decodes one dword of codes (8 elements, inside one 32-block).
__global__ __launch_bounds__(256) void dequantize_kernel(const uint32_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         int64_t n8, int out_bf16,
                                                         void* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  uint32_t c = codes[i];
  uint32_t s = scales[i >> 2];
  if (out_bf16) {
    reinterpret_cast<u32x4*>(out)[i] = dequant8_bf16(c, scale_operand(s));
  } else {
    float sc = scale_operand(s);
    f32x4 lo, hi;
    auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, sc, 0);
    auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, sc, 1);
    auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, sc, 2);
    auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, sc, 3);
    lo[0] = p0[0]; lo[1] = p0[1]; lo[2] = p1[0]; lo[3] = p1[1];
    hi[0] = p2[0]; hi[1] = p2[1]; hi[2] = p3[0]; hi[3] = p3[1];
    f32x4* o = reinterpret_cast<f32x4*>(out) + i * 2;
    o[0] = lo;
    o[1] = hi;
  }
}

// MXFP8 activation quantization ("Integrate finegrained kernels", commit
// notes: MXFP8 through row-wise quantizers; activation_format None = the
// weights' block-scaled format).  One thread per 32-element block of a bf16
// row: scale exponent e = the smallest integer with amax <= 448 * 2^e
// (clamped to [-127, 127], 0 for an all-zero block gives -127), elements
// x * 2^-e rounded to the nearest OCP E4M3 value, ties to the even
// mantissa.  With lo: the residual x - deq(code) (exact in fp32) is
// quantized the same way into its own codes and scale.

// E4M3 code (sign in bit 7) of v, |v| <= 448, round to nearest even.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: multiples of 2^-9
    code = (uint32_t)rintf(a * 512.0f);      // 8 is the smallest normal
  } else {
    const uint32_t b = __float_as_uint(a);
    int ex = (int)(b >> 23) - 127;
    const uint32_t mant = b & 0x7FFFFFu;
    uint32_t m3 = mant >> 20;
    const uint32_t rem = mant & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
    if (m3 == 8u) {
      m3 = 0;
      ++ex;
    }
    code = ((uint32_t)(ex + 7) << 3) | m3;
  }
  return sign | code;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e == 0 ? (float)m * 0.001953125f : ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
  return (c & 0x80u) ? -mag : mag;
}

// e for a block with largest magnitude amax (finite, >= 0)
__device__ __forceinline__ int mx8_exponent(float amax) {
  if (amax == 0.0f) return -127;
  int ex;
  const float fr = frexpf(amax, &ex);        // amax = fr * 2^ex, fr in [0.5, 1)
  // amax <= 1.75 * 2^(e + 8)  <=>  e >= ex - 9 + (fr > 0.875)
  const int e = ex - 9 + (fr > 0.875f ? 1 : 0);
  return max(-127, min(127, e));
}

// 32 values -> 32 codes (as 8 words) and the scale byte; v becomes the
// residual v - deq.
__device__ __forceinline__ uint32_t mx8_block(float (&v)[32], uint32_t (&w)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx8_exponent(amax);
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t c = e4m3_encode(ldexpf(v[i], -e));
    w[i >> 2] |= c << (8 * (i & 3));
    v[i] -= ldexpf(e4m3_value(c), e);
  }
  return (uint32_t)(e + 127);
}

__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(
    const uint16_t* __restrict__ x, int64_t nblk, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, uint8_t* __restrict__ lo_codes, uint8_t* __restrict__ lo_scales) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblk) return;
  float v[32];
  const u32x4* src = reinterpret_cast<const u32x4*>(x + b * 32);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 r = src[q];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      v[8 * q + 2 * m] = bf16_to_f32((uint16_t)(r[m] & 0xFFFFu));
      v[8 * q + 2 * m + 1] = bf16_to_f32((uint16_t)(r[m] >> 16));
    }
  }
  uint32_t w[8];
  scales[b] = (uint8_t)mx8_block(v, w);
  u32x4* dst = reinterpret_cast<u32x4*>(codes + b * 32);
  dst[0] = u32x4{w[0], w[1], w[2], w[3]};
  dst[1] = u32x4{w[4], w[5], w[6], w[7]};
  if (lo_codes) {
    lo_scales[b] = (uint8_t)mx8_block(v, w);
    u32x4* ld = reinterpret_cast<u32x4*>(lo_codes + b * 32);
    ld[0] = u32x4{w[0], w[1], w[2], w[3]};
    ld[1] = u32x4{w[4], w[5], w[6], w[7]};
  }
}

hipError_t launch_mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes,
                                 uint8_t* scales, uint8_t* lo_codes, uint8_t* lo_scales,
                                 hipStream_t s) {
  if (K % 32) return hipErrorInvalidValue;
  const int64_t nblk = rows * (K / 32);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp8_quantize_kernel, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, s,
                     x, nblk, codes, scales, lo_codes, lo_scales);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* w, int64_t rows, int64_t K, uint8_t* codes,
                           uint8_t* scales, hipStream_t s) {
  int64_t n4 = rows * K / 4;
  int64_t blocks = (n4 + 255) / 256;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, n4,
                     reinterpret_cast<uint16_t*>(codes), scales);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                             int64_t K, int out_bf16, void* out, hipStream_t s) {
  int64_t n8 = rows * K / 8;
  int64_t blocks = (n8 + 255) / 256;
  hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(codes), scales, n8, out_bf16, out);
  return hipGetLastError();
}

}  // namespace mxmoe
