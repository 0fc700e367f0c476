// Base-weight gradients of the expert block (full MXFP4 fine-tuning: "Add
// MXFP4 training support via a dequantize-on-the-fly fallback", Relation to
// the backward triton kernels -- native MXFP4 training needs the gradients
// of the expert weights themselves, taken with respect to the dequantized
// weights and requantized by the optimizer step):
//
//   dW_gu[e] = sum_p dh[p]^T x[t(p)]          [2I, H]
//   dW_dn[e] = sum_p (w_p dY[t(p)])^T a[p]     [H, I]
//   db_gu[e] = sum_p dh[p],  db_dn[e] = sum_p w_p dY[t(p)]
//
// over the sorted routed rows p of expert e.  dw_kernel computes the
// generic grouped product out[e] = sum_p A[rowA(p)]^T B[rowB(p)] in fp32 on
// bf16 MFMAs.  Both operands are row-major with the contraction (the routed
// row) as the slow axis, while the MFMA wants 8 consecutive rows per lane:
// the tiles go global -> LDS unchanged (LDS-DMA, two stages) and gfx950's
// 16-bit transposing LDS read (ds_read_b64_tr_b16: a 16-lane group reads a
// 4-row x 16-column block, each lane receiving one column's 4 values) turns
// them into fragments, two reads per fragment.
//
// Tiling: a workgroup owns a 256 x 256 tile of one expert's out and loops
// over the expert's rows in steps of 64.  Eight waves, wave w = (wm, wn):
// rows 128 wm .. + 127 (four 32-row MFMA blocks) by columns 64 wn .. + 63
// (two), 8 accumulators of 32 x 32 fp32.  An LDS tile row (one routed row,
// 256 columns = 32 chunks of 16 bytes) keeps chunk c at c ^ 4 (p % 4), so a
// transposing read's 4 rows x 32 bytes hit 16 distinct bank groups.  Rows
// past the expert and columns past M or N are read from a block of zeros.
#include "common.hpp"
#include "launch.hpp"

namespace mxmoe {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int DW_T = 256;                      // output tile (rows and columns)
constexpr int DW_KC = 64;                      // routed rows per step
constexpr int DW_W = 8;                        // waves
constexpr int DW_TILE = DW_KC * DW_T * 2;      // one operand's tile (32 KB)
constexpr int DW_STAGE = 2 * DW_TILE;          // A and B (64 KB)
constexpr int DW_IDX = 2 * DW_KC * 4;          // two steps' sorted_rows (512 B)
constexpr int DW_LDS = 2 * DW_STAGE + DW_IDX;

__device__ __forceinline__ int dw_swz(int p) { return (p & 3) << 2; }

struct DwOp {
  const uint16_t* base;   // row-major bf16, ld elements per row
  int ld;
  bool gather;            // row(p) = sorted_rows[p] / k, else p
  int c0, C;              // the tile's first column and the column count
};

// This lane's 4 pieces of one operand's tile for the step starting at
// routed row pb: LDS slot q = (4 w + i) * 64 + lane is tile row q / 32,
// physical chunk q % 32 (logical chunk (q % 32) ^ dw_swz(row)).
__device__ __forceinline__ void dw_dma_op(const DwOp& op, uint8_t* __restrict__ tile,
                                          const int32_t* __restrict__ idx, int pb, int p1, int k,
                                          int wave, int lane) {
  int64_t off[4];
  bool ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = (4 * wave + i) * 64 + lane;
    const int pr = q >> 5, ls = (q & 31) ^ dw_swz(pr);
    const int col = op.c0 + 8 * ls;
    ok[i] = pb + pr < p1 && col < op.C;
    off[i] = (op.gather ? (int64_t)(idx[pr] / k) : (int64_t)(pb + pr)) * op.ld + col;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint16_t* src = ok[i] ? op.base + off[i] : reinterpret_cast<const uint16_t*>(g_zero64);
    __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)(tile + (4 * wave + i) * 1024), 16, 0, 0);
  }
}

// Fragment of MFMA block (32 columns at col_local) for sub-step s: rows
// 16 s + 8 (lane / 32) .. + 7, column col_local + lane % 32, from two
// transposing reads.
__device__ __forceinline__ bf16x8 dw_frag(const uint8_t* tile, int s, int col_local, int lane) {
  const int g = lane >> 4, j = lane & 15, q = j >> 2, t = j & 3;
  const int c = col_local + 16 * (g & 1) + 4 * t;             // first of this lane's 4 columns
  s16x4 h[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int p = 16 * s + 8 * (g >> 1) + 4 * half + q;
    const int off = p * (DW_T * 2) + 16 * ((c >> 3) ^ dw_swz(p)) + 2 * (c & 7);
    h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<uint8_t*>(tile) + off));
  }
  const s16x4 lo = h[0], hi = h[1];
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// One step s: start the copies of step s + 1's tiles (into nxt, addressed
// by the row numbers in idx_nxt) and of step s + 2's row numbers (into
// idx_dst), run step s's MFMAs from cur, then wait for this wave's copies
// and meet the others.  The four regions are distinct, which keeps the
// compiler from waiting for the copies before reading cur.
__device__ __forceinline__ void dw_step(const DwOp& A, const DwOp& B, const uint8_t* __restrict__ cur,
                                        uint8_t* __restrict__ nxt,
                                        const int32_t* __restrict__ idx_nxt,
                                        int32_t* __restrict__ idx_dst, int s, int ns, int p0, int p1,
                                        const int32_t* __restrict__ sorted_rows, int k, int wave,
                                        int lane, int wm, int wn, f32x16 (&acc)[4][2]) {
  if (s + 1 < ns) {
    dw_dma_op(A, nxt, idx_nxt, p0 + (s + 1) * DW_KC, p1, k, wave, lane);
    dw_dma_op(B, nxt + DW_TILE, idx_nxt, p0 + (s + 1) * DW_KC, p1, k, wave, lane);
  }
  if (s + 2 < ns && wave == 0)
    __builtin_amdgcn_global_load_lds((gptr_t)(sorted_rows + min(p0 + (s + 2) * DW_KC + lane, p1 - 1)),
                                     (lptr_t)idx_dst, 4, 0, 0);
  const uint8_t* sa = cur;
  const uint8_t* sb = cur + DW_TILE;
  bf16x8 a[2][4], bb[2][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[0][i] = dw_frag(sa, 0, 128 * wm + 32 * i, lane);
#pragma unroll
  for (int j = 0; j < 2; ++j) bb[0][j] = dw_frag(sb, 0, 64 * wn + 32 * j, lane);
#pragma unroll
  for (int ss = 0; ss < 4; ++ss) {
    const int cu = ss & 1, nx = cu ^ 1;
    if (ss < 3) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[nx][i] = dw_frag(sa, ss + 1, 128 * wm + 32 * i, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) bb[nx][j] = dw_frag(sb, ss + 1, 64 * wn + 32 * j, lane);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cu][i], bb[cu][j], acc[i][j], 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  __syncthreads();
}

__global__ __launch_bounds__(64 * DW_W) __attribute__((amdgpu_waves_per_eu(2, 2))) void dw_kernel(
    DwOp A, DwOp B, const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows,
    int k, int M, int N, int mtiles, int ntiles, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[DW_LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int b = blockIdx.x;
  const int e = b / (mtiles * ntiles), mt = (b / ntiles) % mtiles, nt = b % ntiles;
  const int m0 = mt * DW_T, n0 = nt * DW_T;
  A.c0 = m0;
  A.C = M;
  B.c0 = n0;
  B.C = N;
  const int p0 = offsets[e], p1 = offsets[e + 1];
  const int ns = (p1 - p0 + DW_KC - 1) / DW_KC;
  int32_t* idx = reinterpret_cast<int32_t*>(lds + 2 * DW_STAGE);   // [2][64]

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (ns > 0) {
    // step 0's row numbers, then step 0's tiles and step 1's row numbers
    if (wave == 0)
      __builtin_amdgcn_global_load_lds((gptr_t)(sorted_rows + min(p0 + lane, p1 - 1)),
                                       (lptr_t)idx, 4, 0, 0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __syncthreads();
    dw_dma_op(A, lds, idx, p0, p1, k, wave, lane);
    dw_dma_op(B, lds + DW_TILE, idx, p0, p1, k, wave, lane);
    if (ns > 1 && wave == 0)
      __builtin_amdgcn_global_load_lds((gptr_t)(sorted_rows + min(p0 + DW_KC + lane, p1 - 1)),
                                       (lptr_t)(idx + DW_KC), 4, 0, 0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __syncthreads();
  }
  for (int s = 0; s < ns; ++s) {
    const int c = s & 1;
    dw_step(A, B, lds + c * DW_STAGE, lds + (c ^ 1) * DW_STAGE, idx + (c ^ 1) * DW_KC,
            idx + c * DW_KC, s, ns, p0, p1, sorted_rows, k, wave, lane, wm, wn, acc);
  }
  // D lane layout: column n = lane % 32, rows 8 (r / 4) + 4 (lane / 32) + r % 4
  const int l32 = lane & 31, hlf = lane >> 5;
  float* oe = out + (int64_t)e * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 64 * wn + 32 * j + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 128 * wm + 32 * i + 8 * (r >> 2) + 4 * hlf + (r & 3);
        if (m < M && n < N) __builtin_nontemporal_store(acc[i][j][r], oe + (int64_t)m * N + n);
      }
    }
}

// db[e][c] = sum over expert e's sorted rows p of w_p * src[row(p)][c] in
// row order (w_p = topk_w[sorted_rows[p]] when weighted, else 1; row(p) as
// in dw_kernel).  A thread per column, 8 rows' loads in flight.
__global__ __launch_bounds__(256) void colsum_kernel(const uint16_t* __restrict__ src, int ld,
                                                     bool gather, const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ sorted_rows, int k,
                                                     const float* __restrict__ topk_w, int C,
                                                     float* __restrict__ db) {
  const int e = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  const int p0 = offsets[e], p1 = offsets[e + 1];
  float s = 0.0f;
  for (int pb = p0; pb < p1; pb += 8) {
    float v[8], w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = min(pb + u, p1 - 1);
      const int32_t f = sorted_rows[p];
      const int64_t row = gather ? (int64_t)(f / k) : (int64_t)p;
      v[u] = bf16_to_f32(src[row * ld + c]);
      w[u] = topk_w ? topk_w[f] : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (pb + u < p1) s += w[u] * v[u];
  }
  db[(int64_t)e * C + c] = s;
}

// out[p][c] = bf16(topk_w[sorted_rows[p]] * in[p][c]) for R sorted rows of C
// columns (8 columns a thread).
__global__ __launch_bounds__(256) void scale_rows_kernel(const uint16_t* __restrict__ in, int64_t R,
                                                         int C, const int32_t* __restrict__ sorted_rows,
                                                         const float* __restrict__ topk_w,
                                                         uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 8-column piece
  const int C8 = C / 8;
  if (i >= R * C8) return;
  const int64_t p = i / C8;
  const float w = topk_w[sorted_rows[p]];
  const u32x4 v = reinterpret_cast<const u32x4*>(in)[i];
  u32x4 o;
#pragma unroll
  for (int m = 0; m < 4; ++m)
    o[m] = pack_bf16x2(w * bf16_to_f32((uint16_t)(v[m] & 0xFFFFu)), w * bf16_to_f32((uint16_t)(v[m] >> 16)));
  reinterpret_cast<u32x4*>(out)[i] = o;
}

hipError_t launch_dw(const uint16_t* A, int lda, bool gatherA, const uint16_t* B, int ldb,
                     bool gatherB, const int32_t* offsets, const int32_t* sorted_rows, int k,
                     int E, int M, int N, float* out, hipStream_t s) {
  if (M % 32 || N % 32 || lda % 8 || ldb % 8) return hipErrorInvalidValue;
  const int mtiles = (M + DW_T - 1) / DW_T, ntiles = (N + DW_T - 1) / DW_T;
  DwOp a{A, lda, gatherA, 0, M}, b{B, ldb, gatherB, 0, N};
  hipLaunchKernelGGL(dw_kernel, dim3(E * mtiles * ntiles), dim3(64 * DW_W), 0, s, a, b, offsets,
                     sorted_rows, k, M, N, mtiles, ntiles, out);
  return hipGetLastError();
}

hipError_t launch_colsum(const uint16_t* src, int ld, bool gather, const int32_t* offsets,
                         const int32_t* sorted_rows, int k, const float* topk_w, int E, int C,
                         float* db, hipStream_t s) {
  hipLaunchKernelGGL(colsum_kernel, dim3((C + 255) / 256, E), dim3(256), 0, s, src, ld, gather,
                     offsets, sorted_rows, k, topk_w, C, db);
  return hipGetLastError();
}

hipError_t launch_scale_rows(const uint16_t* in, int64_t R, int C, const int32_t* sorted_rows,
                             const float* topk_w, uint16_t* out, hipStream_t s) {
  if (C % 8) return hipErrorInvalidValue;
  const int64_t n = R * (C / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(scale_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, in, R,
                     C, sorted_rows, topk_w, out);
  return hipGetLastError();
}

}  // namespace mxmoe
