// Rank-r LoRA (r = 8, 16, 32 or 64) on the down and/or the gate_up
// projection of every expert ("Add MXFP4 training support via a
// dequantize-on-the-fly fallback", "What this does": adapters train on top
// of the frozen MXFP4 base, whose backward only has to deliver input and
// adapter gradients).  For the down projection, per expert e with
// A_e [r, I], B_e [H, r] (the gate_up adapter is the same with x for a, h
// for y, A_gu [r, H] and B_gu [2I, r], its delta added before the bias):
//
//   forward   v = a A_e^T                     (this file, lora_proj)
//             y += s (v B_e^T)                (down GEMM epilogue, gemm_fwd.hip)
//   backward  dv_u = s dY_t B_e                (lora_proj over gathered dY rows)
//             da_u += dv_u A_e                 (bwd_down epilogue, gemm_bwd.hip)
//             dB_e = s sum_p w_p dY_t(p)^T v_p (lora_grad)
//             dA_e = sum_p (w_p dv_u,p)^T a_p  (lora_grad)
//
// v and dv_u are fp32 [R, r] in sorted-row order.  The epilogues feed them
// to bf16 MFMAs as a hi/lo bf16 pair, so they keep about 17 bits.
#include "common.hpp"
#include "launch.hpp"

namespace mxmoe {

// out[p, j] = scale * sum_c src[row(p), c] * M[e][j][c] for the j < r rank
// columns and every sorted row p of a tile of expert e.  row(p) =
// sorted_rows[p] / k (GATHER: token rows of a [T, C] tensor) or p (rows
// already in sorted order).  One 32-row MFMA block per wave and NB = r / 32
// (at least 1) rank blocks: the A-operand is 32 source rows, the B-operand
// 32 rank rows of M (for r < 32 the lanes past r repeat them; their columns
// are dropped).  C % 32 == 0: with C an odd multiple of 32 the last 64-wide
// step reads zeros past C.
template <bool GATHER, int NB>
__global__ __launch_bounds__(256) void lora_proj_kernel(
    const uint16_t* __restrict__ src, const int32_t* __restrict__ sorted_rows, int k,
    const uint16_t* __restrict__ M, int C, int r, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, float scale, float* __restrict__ out) {
  if ((int)blockIdx.x >= *num_tiles) return;
  const Tile tl = tiles[blockIdx.x];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave * 32 >= tl.rows) return;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int64_t p = tl.row0 + min(wave * 32 + l32, tl.rows - 1);
  const int64_t srow = GATHER ? sorted_rows[p] / k : p;
  const uint16_t* ap = src + srow * C + 8 * hlf;
  const uint16_t* bp[NB];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb)
    bp[jb] = M + ((int64_t)tl.expert * r + 32 * jb + (l32 & (min(r, 32) - 1))) * C + 8 * hlf;

  f32x16 acc[NB];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[jb][q] = 0.0f;
  const int nsteps = (C + 63) / 64;
  // pieces 16 s + 8 hlf .. of step c, zeros past C
  auto ld = [&](const uint16_t* base, int c, int s) {
    const bool past = 64 * c + 16 * s >= C;
    return gload16(past ? reinterpret_cast<const uint16_t*>(g_zero64) : base + 64 * c + 16 * s);
  };
  // 64 columns per step, the next step's loads in flight during the MFMAs
  u32x4 a[2][4], b[2][NB][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    a[0][s] = ld(ap, 0, s);
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) b[0][jb][s] = ld(bp[jb], 0, s);
  }
  for (int c = 0; c < nsteps; c += 2) {
    const int c1 = min(c + 1, nsteps - 1), c2 = min(c + 2, nsteps - 1);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a[1][s] = ld(ap, c1, s);
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) b[1][jb][s] = ld(bp[jb], c1, s);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int jb = 0; jb < NB; ++jb)
        acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[0][s]), as_bf16x8(b[0][jb][s]),
                                                          acc[jb], 0, 0, 0);
    if (c + 1 >= nsteps) break;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a[0][s] = ld(ap, c2, s);
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) b[0][jb][s] = ld(bp[jb], c2, s);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int jb = 0; jb < NB; ++jb)
        acc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[1][s]), as_bf16x8(b[1][jb][s]),
                                                          acc[jb], 0, 0, 0);
  }
  // lane holds rank column 32 jb + l32 of rows 8*(q/4) + 4*hlf + q%4
#pragma unroll
  for (int jb = 0; jb < NB; ++jb) {
    const int j = 32 * jb + l32;
    if (j >= r) continue;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int rt = wave * 32 + 8 * (q >> 2) + 4 * hlf + (q & 3);
      if (rt < tl.rows) out[(int64_t)(tl.row0 + rt) * r + j] = scale * acc[jb][q];
    }
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
// (scale * topk_w[sorted_rows[p]] * P[p][j]) * Q[row(p)][c] (topk_w NULL:
// no routing weight), written to
// out[e * e_stride + c * c_stride + j * j_stride]; row(p) as in lora_proj,
// P [R, r].  A workgroup takes 128 columns of one expert and 16 rank
// columns 16 z .. (blockIdx.z; past r: zeros, not written): lane l of each
// wave owns columns 2l and 2l+1 (one 4-byte load of Q per row), and the
// expert's rows go in rounds of 64, wave w taking rounds w, w + 4, ..  For
// its round a wave stages the 64 scaled P rows in its own LDS slice (lane =
// row), then issues the 64 loads of its columns before the 2048 FMAs.  The
// four waves' partial sums are added in wave order at the end, so the
// result is deterministic; an expert with no rows gets zeros.  C % 32 == 0.
constexpr int LG_RB = 64;     // rows per round
constexpr int LG_COLS = 128;  // columns per workgroup
constexpr int LG_J = 16;      // rank columns per workgroup
template <bool GATHER>
__global__ __launch_bounds__(256) void lora_grad_kernel(
    const uint16_t* __restrict__ Q, int C, const int32_t* __restrict__ sorted_rows, int k,
    const float* __restrict__ P, int r, const float* __restrict__ topk_w, float scale,
    const int32_t* __restrict__ offsets, float* __restrict__ out, int64_t e_stride,
    int c_stride, int j_stride) {
  __shared__ __attribute__((aligned(16))) float ps[4][LG_RB][LG_J];
  __shared__ int64_t qrow[4][LG_RB];
  __shared__ float red[4][LG_COLS][LG_J + 1];
  const int e = blockIdx.y, j0 = LG_J * blockIdx.z;
  const int nj = min(LG_J, r - j0);   // rank columns of this workgroup (8 or 16)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = blockIdx.x * LG_COLS;
  const int cc = min(c0 + 2 * lane, C - 2);
  const int p0 = offsets[e], p1 = offsets[e + 1];
  const int nrounds = (p1 - p0 + LG_RB - 1) / LG_RB;
  float acc[2][LG_J];
#pragma unroll
  for (int j = 0; j < LG_J; ++j) acc[0][j] = acc[1][j] = 0.0f;
  for (int rd = wave; rd < nrounds; rd += 4) {
    const int pb = p0 + rd * LG_RB;
    const int n = min(LG_RB, p1 - pb);
    {
      // lane = row: its scaled P row (zero past the expert and past r) and
      // source row
      const int64_t p = pb + min(lane, n - 1);
      const int32_t f = sorted_rows[p];
      const float* pr = P + p * r + j0;
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      f32x4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = 4 * q < nj ? *reinterpret_cast<const f32x4*>(pr + 4 * q) : z;
      const float w = lane < n ? (topk_w ? scale * topk_w[f] : scale) : 0.0f;
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
      for (int j4 = 0; j4 < LG_J / 4; ++j4) {
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
  for (int j = 0; j < LG_J; ++j) {
    red[wave][2 * lane][j] = acc[0][j];
    red[wave][2 * lane + 1][j] = acc[1][j];
  }
  __syncthreads();
  for (int q = tid; q < LG_COLS * LG_J; q += 256) {
    const int col = q / LG_J, j = q % LG_J;
    const int c = c0 + col;
    if (c < C && j < nj) {
      const float s = ((red[0][col][j] + red[1][col][j]) + red[2][col][j]) + red[3][col][j];
      out[(int64_t)e * e_stride + (int64_t)c * c_stride + (int64_t)(j0 + j) * j_stride] = s;
    }
  }
}

hipError_t launch_lora_proj(const uint16_t* src, bool gather, const int32_t* sorted_rows, int k,
                            const uint16_t* M, int C, int r, const Tile* tiles,
                            const int32_t* num_tiles, int max_tiles, float scale, float* out,
                            hipStream_t s) {
  if (C % 32 || !lora_rank_ok(r)) return hipErrorInvalidValue;
#define LORA_PROJ(G, NB)                                                                      \
  hipLaunchKernelGGL((lora_proj_kernel<G, NB>), dim3(max_tiles), dim3(256), 0, s, src,        \
                     sorted_rows, k, M, C, r, tiles, num_tiles, scale, out)
  if (gather) {
    if (r > 32) LORA_PROJ(true, 2); else LORA_PROJ(true, 1);
  } else {
    if (r > 32) LORA_PROJ(false, 2); else LORA_PROJ(false, 1);
  }
#undef LORA_PROJ
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
                            int k, const float* P, int r, const float* topk_w, float scale,
                            const int32_t* offsets, int E, float* out, int64_t e_stride,
                            int c_stride, int j_stride, hipStream_t s) {
  if (C % 32 || !lora_rank_ok(r)) return hipErrorInvalidValue;
  dim3 grid((C + LG_COLS - 1) / LG_COLS, E, (r + LG_J - 1) / LG_J);
  if (gather)
    hipLaunchKernelGGL(lora_grad_kernel<true>, grid, dim3(256), 0, s, Q, C, sorted_rows, k, P, r,
                       topk_w, scale, offsets, out, e_stride, c_stride, j_stride);
  else
    hipLaunchKernelGGL(lora_grad_kernel<false>, grid, dim3(256), 0, s, Q, C, sorted_rows, k, P, r,
                       topk_w, scale, offsets, out, e_stride, c_stride, j_stride);
  return hipGetLastError();
}

}  // namespace mxmoe
