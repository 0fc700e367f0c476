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
