// Rank-16 LoRA on the down projection of every expert ("Add MXFP4 training
// support via a dequantize-on-the-fly fallback", "What this does": adapters
// train on top of the frozen MXFP4 base, whose backward only has to deliver
// input and adapter gradients).  Per expert e with A_e [r, I], B_e [H, r]:
//
//   forward   v = a A_e^T                     (this file, lora_proj)
//             y += s (v B_e^T)                (down GEMM epilogue, gemm_fwd.hip)
//   backward  dv_u = s dY_t B_e                (lora_proj over gathered dY rows)
//             da_u += dv_u A_e                 (bwd_down epilogue, gemm_bwd.hip)
//             dB_e = s sum_p w_p dY_t(p)^T v_p (lora_grad)
//             dA_e = sum_p (w_p dv_u,p)^T a_p  (lora_grad)
//
// v and dv_u are fp32 [R, 16] in sorted-row order.  The epilogues feed them
// to bf16 MFMAs as a hi/lo bf16 pair, so they keep about 17 bits.
#include "common.hpp"
#include "launch.hpp"

namespace mxmoe {

// out[p, j] = scale * sum_c src[row(p), c] * M[e][j][c] for the j < 16 rank
// columns and every sorted row p of a tile of expert e.  row(p) =
// sorted_rows[p] / k (GATHER: token rows of a [T, C] tensor) or p (rows
// already in sorted order).  One 32-row MFMA block per wave: the A-operand
// is 32 source rows, the B-operand the 16 rank rows of M (lanes 16..31 of
// each half repeat them; their columns are dropped).  C % 64 == 0.
template <bool GATHER>
__global__ __launch_bounds__(256) void lora_proj_kernel(
    const uint16_t* __restrict__ src, const int32_t* __restrict__ sorted_rows, int k,
    const uint16_t* __restrict__ M, int C, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, float scale, float* __restrict__ out) {
  if ((int)blockIdx.x >= *num_tiles) return;
  const Tile tl = tiles[blockIdx.x];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave * 32 >= tl.rows) return;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int64_t p = tl.row0 + min(wave * 32 + l32, tl.rows - 1);
  const int64_t srow = GATHER ? sorted_rows[p] / k : p;
  const uint16_t* ap = src + srow * C + 8 * hlf;
  const uint16_t* bp = M + ((int64_t)tl.expert * LORA_R + (l32 & 15)) * C + 8 * hlf;

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  // 64 columns per step, the next step's loads in flight during the MFMAs
  u32x4 a[2][4], b[2][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    a[0][s] = *reinterpret_cast<const u32x4*>(ap + 16 * s);
    b[0][s] = *reinterpret_cast<const u32x4*>(bp + 16 * s);
  }
  const int nsteps = C / 64;
  for (int c = 0; c < nsteps; c += 2) {
    const int c1 = min(c + 1, nsteps - 1), c2 = min(c + 2, nsteps - 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a[1][s] = *reinterpret_cast<const u32x4*>(ap + 64 * c1 + 16 * s);
      b[1][s] = *reinterpret_cast<const u32x4*>(bp + 64 * c1 + 16 * s);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[0][s]), as_bf16x8(b[0][s]), acc, 0, 0, 0);
    if (c + 1 >= nsteps) break;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a[0][s] = *reinterpret_cast<const u32x4*>(ap + 64 * c2 + 16 * s);
      b[0][s] = *reinterpret_cast<const u32x4*>(bp + 64 * c2 + 16 * s);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[1][s]), as_bf16x8(b[1][s]), acc, 0, 0, 0);
  }
  if (l32 >= LORA_R) return;
  // lane holds rank column l32 of rows 8*(r/4) + 4*hlf + r%4
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rt = wave * 32 + 8 * (r >> 2) + 4 * hlf + (r & 3);
    if (rt < tl.rows) out[(int64_t)(tl.row0 + rt) * LORA_R + l32] = scale * acc[r];
  }
}

// out[b][c][r] = in[b][r][c] for `batches` row-major [R1, R2] bf16 matrices.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in,
                                                             int64_t n, int R1, int R2,
                                                             uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // index into out
  if (i >= n) return;
  const int64_t per = (int64_t)R1 * R2;
  const int64_t b = i / per, rem = i % per;
  const int c = (int)(rem / R1), r = (int)(rem % R1);
  out[i] = in[b * per + (int64_t)r * R2 + c];
}

// G[e][c][j] = sum over the sorted rows p of expert e of
// (scale * topk_w[sorted_rows[p]] * P[p][j]) * Q[row(p)][c], written to
// out[e * e_stride + c * c_stride + j * j_stride]; row(p) as in lora_proj.
// A workgroup takes 128 columns of one expert: lane l of each wave owns
// columns 2l and 2l+1 (one 4-byte load of Q per row), and the expert's rows
// go in rounds of 64, wave w taking rounds w, w + 4, ..  For its round a
// wave stages the 64 scaled P rows in its own LDS slice (lane = row), then
// issues the 64 loads of its columns before the 2048 FMAs.  The four waves'
// partial sums are added in wave order at the end, so the result is
// deterministic; an expert with no rows gets zeros.  C % 64 == 0.
constexpr int LG_RB = 64;     // rows per round
constexpr int LG_COLS = 128;  // columns per workgroup
template <bool GATHER>
__global__ __launch_bounds__(256) void lora_grad_kernel(
    const uint16_t* __restrict__ Q, int C, const int32_t* __restrict__ sorted_rows, int k,
    const float* __restrict__ P, const float* __restrict__ topk_w, float scale,
    const int32_t* __restrict__ offsets, float* __restrict__ out, int64_t e_stride,
    int c_stride, int j_stride) {
  __shared__ __attribute__((aligned(16))) float ps[4][LG_RB][LORA_R];
  __shared__ int64_t qrow[4][LG_RB];
  __shared__ float red[4][LG_COLS][LORA_R + 1];
  const int e = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = blockIdx.x * LG_COLS;
  const int cc = min(c0 + 2 * lane, C - 2);
  const int p0 = offsets[e], p1 = offsets[e + 1];
  const int nrounds = (p1 - p0 + LG_RB - 1) / LG_RB;
  float acc[2][LORA_R];
#pragma unroll
  for (int j = 0; j < LORA_R; ++j) acc[0][j] = acc[1][j] = 0.0f;
  for (int r = wave; r < nrounds; r += 4) {
    const int pb = p0 + r * LG_RB;
    const int n = min(LG_RB, p1 - pb);
    {
      // lane = row: its scaled P row (zero past the expert) and source row
      const int64_t p = pb + min(lane, n - 1);
      const int32_t f = sorted_rows[p];
      const f32x4* pr = reinterpret_cast<const f32x4*>(P + p * LORA_R);
      f32x4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = pr[q];
      const float w = lane < n ? scale * topk_w[f] : 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 t;
#pragma unroll
        for (int m = 0; m < 4; ++m) t[m] = w * v[q][m];
        *reinterpret_cast<f32x4*>(&ps[wave][lane][4 * q]) = t;
      }
      qrow[wave][lane] = GATHER ? (int64_t)(f / k) : p;
    }
    wave_lds_sync();
    uint32_t qv[LG_RB];
#pragma unroll
    for (int i = 0; i < LG_RB; ++i) qv[i] = *reinterpret_cast<const uint32_t*>(Q + qrow[wave][i] * C + cc);
#pragma unroll
    for (int i = 0; i < LG_RB; ++i) {
      const float qa = bf16_to_f32((uint16_t)(qv[i] & 0xFFFFu));
      const float qb = bf16_to_f32((uint16_t)(qv[i] >> 16));
#pragma unroll
      for (int j4 = 0; j4 < LORA_R / 4; ++j4) {
        const f32x4 pv = *reinterpret_cast<const f32x4*>(&ps[wave][i][4 * j4]);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          acc[0][4 * j4 + m] += qa * pv[m];
          acc[1][4 * j4 + m] += qb * pv[m];
        }
      }
    }
    wave_lds_sync();   // this round's LDS reads are done before the next staging
  }
#pragma unroll
  for (int j = 0; j < LORA_R; ++j) {
    red[wave][2 * lane][j] = acc[0][j];
    red[wave][2 * lane + 1][j] = acc[1][j];
  }
  __syncthreads();
  for (int q = tid; q < LG_COLS * LORA_R; q += 256) {
    const int col = q / LORA_R, j = q % LORA_R;
    const int c = c0 + col;
    if (c < C) {
      const float s = ((red[0][col][j] + red[1][col][j]) + red[2][col][j]) + red[3][col][j];
      out[(int64_t)e * e_stride + (int64_t)c * c_stride + (int64_t)j * j_stride] = s;
    }
  }
}

hipError_t launch_lora_proj(const uint16_t* src, bool gather, const int32_t* sorted_rows, int k,
                            const uint16_t* M, int C, const Tile* tiles, const int32_t* num_tiles,
                            int max_tiles, float scale, float* out, hipStream_t s) {
  if (C % 64) return hipErrorInvalidValue;
  if (gather)
    hipLaunchKernelGGL(lora_proj_kernel<true>, dim3(max_tiles), dim3(256), 0, s, src, sorted_rows,
                       k, M, C, tiles, num_tiles, scale, out);
  else
    hipLaunchKernelGGL(lora_proj_kernel<false>, dim3(max_tiles), dim3(256), 0, s, src,
                       sorted_rows, k, M, C, tiles, num_tiles, scale, out);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t batches, int R1, int R2,
                                 uint16_t* out, hipStream_t s) {
  const int64_t n = batches * R1 * R2;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     in, n, R1, R2, out);
  return hipGetLastError();
}

hipError_t launch_lora_grad(const uint16_t* Q, bool gather, int C, const int32_t* sorted_rows,
                            int k, const float* P, const float* topk_w, float scale,
                            const int32_t* offsets, int E, float* out, int64_t e_stride,
                            int c_stride, int j_stride, hipStream_t s) {
  if (C % 64) return hipErrorInvalidValue;
  dim3 grid((C + LG_COLS - 1) / LG_COLS, E);
  if (gather)
    hipLaunchKernelGGL(lora_grad_kernel<true>, grid, dim3(256), 0, s, Q, C, sorted_rows, k, P,
                       topk_w, scale, offsets, out, e_stride, c_stride, j_stride);
  else
    hipLaunchKernelGGL(lora_grad_kernel<false>, grid, dim3(256), 0, s, Q, C, sorted_rows, k, P,
                       topk_w, scale, offsets, out, e_stride, c_stride, j_stride);
  return hipGetLastError();
}

}  // namespace mxmoe
