// Forward grouped expert GEMMs on gfx950 MFMA (bf16 in, fp32 accumulate).
//
// gate_up: h[p, n] = sum_k x[t(p), k] * deq(Wgu[e, n, k]) + bgu[e, n], with the
//          SwiGLU epilogue on the stride-2 split (gate = row 2j, up = row
//          2j+1, "Integrate finegrained kernels ...": interleaved gate|up
//          rows and the fused GLU epilogue's split_gate_up), bias as an
//          operand indexed by the tile's expert (same pages, bias= note).
// down:    y[p, n] = sum_i a[p, i] * deq(Wd[e, n, i]) + bd[e, n], scaled by
//          the routing weight and written to the routed row's own slot, so
//          the combine can sum a token's k slots in a fixed order.
//
// Tiling (per workgroup): MT = 128 routed rows of one expert x 64*WN weight
// rows; WN waves, each owning 64 weight rows (two 32-row MFMA blocks) for
// all 128 rows (four 32-column blocks): 8 accumulators of 32x32 fp32.
// The product is computed transposed, D[n][p] = W[n][:] . X[p][:], so that
// the weights are the MFMA A-operand: each lane loads 16 bytes (32 codes)
// of one weight row straight from global memory and decodes them in
// registers with the scaled fp4->bf16 conversion (one UE8M0 scale per 32
// codes); nothing of the weights goes through LDS and no lane decodes a
// weight another lane also decodes.  The routed activation rows are the
// B-operand, staged through LDS (double buffered, one barrier per 64-wide
// K step) because every wave reads all 128 of them.
//
// K order inside a 64-wide step: lane half h (lanes 32h..32h+31) holds the
// codes of elements 32h..32h+31 and feeds elements 32h+8s..32h+8s+7 to MFMA
// step s; the B-operand reads the same elements, so each MFMA contracts
// matching K indices (the hardware pairs A and B by lane group and
// register slot).
//
// In the 32x32 accumulator a lane holds column p = lane % 32 and rows
// 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15: gate/up pairs (2j, 2j+1) sit in
// registers (r, r+1) of the same lane, so the GLU needs no data exchange.
#include "common.hpp"
#include "launch.hpp"

namespace mxmoe {

template <int WN>
struct FwdTile {
  static constexpr int NTHR = 64 * WN;
  static constexpr int NT = 64 * WN;             // weight rows per workgroup
  static constexpr int PPT = MT * 8 / NTHR;      // 16-byte B pieces per thread per step
};

// Main loop shared by both forward GEMMs.  brow[j] points at the start of
// the activation row for B piece j (already offset by its 8-element piece);
// rows past the tile point at the tile's first row, so every load is
// unconditional (their columns of the product are never stored).  Only the
// first NRB 32-row blocks of the tile hold rows: the MFMAs of the others
// are not issued.  wcode/wscale point at this lane's first weight row
// (row block 0) and are valid even for a wave past the last weight row,
// whose results are dropped.
//
// Pipeline: global loads run two K steps ahead.  In step c the lane decodes
// the weights of step c (loaded two steps earlier), issues the loads of step
// c+2 into the registers just freed, writes the activations of step c+1
// (loaded one step earlier) into the other LDS buffer, then runs the MFMAs
// of step c; one barrier per step.  Near the end the step index of a load
// is clamped to the last step instead of branching, so the compiler's wait
// counts stay exact (a branch around a load makes it wait for all loads).
// The loop is unrolled by two so every register set has a fixed name.
template <int WN>
struct FwdPipe {
  using FT = FwdTile<WN>;
  u32x4 xv[2][FT::PPT];  // activation pieces, by step parity
  u32x4 wv[2][2];        // raw codes, [parity][row block]
  uint32_t sv[2][2];     // raw scales
};

template <int WN, int PAR>
__device__ __forceinline__ void fwd_issue(FwdPipe<WN>& pp, const uint16_t* const (&brow)[FwdTile<WN>::PPT],
                                          const uint8_t* wp0, const uint8_t* wp1,
                                          const uint8_t* sp0, const uint8_t* sp1, int c) {
#pragma unroll
  for (int j = 0; j < FwdTile<WN>::PPT; ++j)
    pp.xv[PAR][j] = *reinterpret_cast<const u32x4*>(brow[j] + c * KC);
  pp.wv[PAR][0] = *reinterpret_cast<const u32x4*>(wp0 + c * 32);
  pp.wv[PAR][1] = *reinterpret_cast<const u32x4*>(wp1 + c * 32);
  pp.sv[PAR][0] = sp0[c * 2];
  pp.sv[PAR][1] = sp1[c * 2];
}

template <int WN, int PAR>
__device__ __forceinline__ void fwd_stage_x(const FwdPipe<WN>& pp, uint16_t (*xs)[MT][LDS_ROW]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < FwdTile<WN>::PPT; ++j) {
    int q = tid + j * FwdTile<WN>::NTHR;
    *reinterpret_cast<u32x4*>(&xs[PAR][q >> 3][(q & 7) * 8]) = pp.xv[PAR][j];
  }
}

template <int WN, int NRB, int PAR>
__device__ __forceinline__ void fwd_step(FwdPipe<WN>& pp, const uint16_t* const (&brow)[FwdTile<WN>::PPT],
                                         const uint8_t* wp0, const uint8_t* wp1,
                                         const uint8_t* sp0, const uint8_t* sp1, int c, int nsteps,
                                         uint16_t (*xs)[MT][LDS_ROW], f32x16 (&acc)[2][4]) {
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hlf = lane >> 5;
  bf16x8 a[2][4];
  const float sc0 = scale_operand(pp.sv[PAR][0]), sc1 = scale_operand(pp.sv[PAR][1]);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    a[0][st] = as_bf16x8(dequant8_bf16(pp.wv[PAR][0][st], sc0));
    a[1][st] = as_bf16x8(dequant8_bf16(pp.wv[PAR][1][st], sc1));
  }
  fwd_issue<WN, PAR>(pp, brow, wp0, wp1, sp0, sp1, min(c + 2, nsteps - 1));
  fwd_stage_x<WN, PAR ^ 1>(pp, xs);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
#pragma unroll
    for (int tb = 0; tb < NRB; ++tb) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(&xs[PAR][tb * 32 + l32][hlf * 32 + st * 8]);
      acc[0][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][st], b, acc[0][tb], 0, 0, 0);
      acc[1][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][st], b, acc[1][tb], 0, 0, 0);
    }
  }
  __syncthreads();
}

template <int WN, int NRB>
__device__ __forceinline__ void fwd_mainloop_n(const uint16_t* const (&brow)[FwdTile<WN>::PPT],
                                               const uint8_t* wp0, const uint8_t* wp1,
                                               const uint8_t* sp0, const uint8_t* sp1, int nsteps,
                                               uint16_t (*xs)[MT][LDS_ROW], f32x16 (&acc)[2][4]) {
  FwdPipe<WN> pp;
  fwd_issue<WN, 0>(pp, brow, wp0, wp1, sp0, sp1, 0);
  fwd_issue<WN, 1>(pp, brow, wp0, wp1, sp0, sp1, min(1, nsteps - 1));
  fwd_stage_x<WN, 0>(pp, xs);
  __syncthreads();
  int c = 0;
  for (; c + 1 < nsteps; c += 2) {
    fwd_step<WN, NRB, 0>(pp, brow, wp0, wp1, sp0, sp1, c, nsteps, xs, acc);
    fwd_step<WN, NRB, 1>(pp, brow, wp0, wp1, sp0, sp1, c + 1, nsteps, xs, acc);
  }
  if (c < nsteps) fwd_step<WN, NRB, 0>(pp, brow, wp0, wp1, sp0, sp1, c, nsteps, xs, acc);
}

template <int WN>
__device__ __forceinline__ void fwd_mainloop(const uint16_t* const (&brow)[FwdTile<WN>::PPT],
                                             const uint8_t* __restrict__ wcode,
                                             const uint8_t* __restrict__ wscale, int K, int nrb,
                                             uint16_t (*xs)[MT][LDS_ROW], f32x16 (&acc)[2][4]) {
  const int lane = threadIdx.x & 63;
  const int hlf = lane >> 5;
  const int64_t KB = K / 2, KS = K / 32;
  const int nsteps = K / KC;
  const uint8_t* wp0 = wcode + hlf * 16;
  const uint8_t* wp1 = wp0 + 32 * KB;
  const uint8_t* sp0 = wscale + hlf;
  const uint8_t* sp1 = sp0 + 32 * KS;

#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][tb][r] = 0.0f;

  switch (nrb) {
    case 1: fwd_mainloop_n<WN, 1>(brow, wp0, wp1, sp0, sp1, nsteps, xs, acc); break;
    case 2: fwd_mainloop_n<WN, 2>(brow, wp0, wp1, sp0, sp1, nsteps, xs, acc); break;
    case 3: fwd_mainloop_n<WN, 3>(brow, wp0, wp1, sp0, sp1, nsteps, xs, acc); break;
    default: fwd_mainloop_n<WN, 4>(brow, wp0, wp1, sp0, sp1, nsteps, xs, acc); break;
  }
}

template <int WN>
__global__ __launch_bounds__(64 * WN, 2) void gate_up_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const uint16_t* __restrict__ bias,
    const int32_t* __restrict__ sorted_rows, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int H, int I, int k, float alpha, float limit,
    uint16_t* __restrict__ h_out, uint16_t* __restrict__ a_out) {
  using FT = FwdTile<WN>;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MT][LDS_ROW];
  if ((int)blockIdx.y >= *num_tiles) return;
  const Tile tl = tiles[blockIdx.y];
  const int N = 2 * I;
  const int n0 = blockIdx.x * FT::NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int e = tl.expert;

  const uint16_t* brow[FT::PPT];
#pragma unroll
  for (int j = 0; j < FT::PPT; ++j) {
    int q = tid + j * FT::NTHR;
    int r = q >> 3;
    const int f = sorted_rows[tl.row0 + (r < tl.rows ? r : 0)];
    brow[j] = x + (int64_t)(f / k) * H + (q & 7) * 8;
  }
  const bool wave_live = n0 + wave * 64 < N;
  const int wrow = (wave_live ? n0 + wave * 64 : 0) + l32;
  const uint8_t* wcode = codes + ((int64_t)e * N + wrow) * (H / 2);
  const uint8_t* wscale = scales + ((int64_t)e * N + wrow) * (H / 32);
  f32x16 acc[2][4];
  fwd_mainloop<WN>(brow, wcode, wscale, H, (tl.rows + 31) / 32, xs, acc);
  if (!wave_live) return;

#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int nb = n0 + wave * 64 + rb * 32 + 4 * hlf;  // + 8q + (r % 4)
    float bv[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bv[q][i] = bias ? bf16_to_f32(bias[(int64_t)e * N + nb + 8 * q + i]) : 0.0f;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int rt = tb * 32 + l32;
      if (rt >= tl.rows) continue;
      const int64_t p = tl.row0 + rt;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float g0 = acc[rb][tb][4 * q + 0] + bv[q][0];
        const float u0 = acc[rb][tb][4 * q + 1] + bv[q][1];
        const float g1 = acc[rb][tb][4 * q + 2] + bv[q][2];
        const float u1 = acc[rb][tb][4 * q + 3] + bv[q][3];
        const int n = nb + 8 * q;
        if (h_out) {
          u32x2 hv = {saved_preact_bf16(g0, limit, false) | (saved_preact_bf16(u0, limit, true) << 16),
                      saved_preact_bf16(g1, limit, false) | (saved_preact_bf16(u1, limit, true) << 16)};
          *reinterpret_cast<u32x2*>(h_out + p * N + n) = hv;
        }
        *reinterpret_cast<uint32_t*>(a_out + p * I + n / 2) =
            pack_bf16x2(swiglu(g0, u0, alpha, limit), swiglu(g1, u1, alpha, limit));
      }
    }
  }
}

template <int WN>
__global__ __launch_bounds__(64 * WN, 2) void down_kernel(
    const uint16_t* __restrict__ a, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const uint16_t* __restrict__ bias,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_rows,
    const Tile* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int H, int I,
    float* __restrict__ y_w) {
  using FT = FwdTile<WN>;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MT][LDS_ROW];
  if ((int)blockIdx.y >= *num_tiles) return;
  const Tile tl = tiles[blockIdx.y];
  const int N = H;
  const int n0 = blockIdx.x * FT::NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int e = tl.expert;

  const uint16_t* brow[FT::PPT];
#pragma unroll
  for (int j = 0; j < FT::PPT; ++j) {
    int q = tid + j * FT::NTHR;
    int r = q >> 3;
    brow[j] = a + (int64_t)(tl.row0 + (r < tl.rows ? r : 0)) * I + (q & 7) * 8;
  }
  const bool wave_live = n0 + wave * 64 < N;
  const int wrow = (wave_live ? n0 + wave * 64 : 0) + l32;
  const uint8_t* wcode = codes + ((int64_t)e * N + wrow) * (I / 2);
  const uint8_t* wscale = scales + ((int64_t)e * N + wrow) * (I / 32);
  f32x16 acc[2][4];
  fwd_mainloop<WN>(brow, wcode, wscale, I, (tl.rows + 31) / 32, xs, acc);
  if (!wave_live) return;

#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int nb = n0 + wave * 64 + rb * 32 + 4 * hlf;
    float bv[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bv[q][i] = bias ? bf16_to_f32(bias[(int64_t)e * N + nb + 8 * q + i]) : 0.0f;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int rt = tb * 32 + l32;
      if (rt >= tl.rows) continue;
      const int64_t f = sorted_rows[tl.row0 + rt];
      const float wf = topk_w[f];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = wf * (acc[rb][tb][4 * q + i] + bv[q][i]);
        *reinterpret_cast<f32x4*>(y_w + f * N + nb + 8 * q) = y;
      }
    }
  }
}

// out[t, :] = sum_j y_w[t*k + j, :] in slot order, rounded once to bf16.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_w, int64_t n4,
                                                      int H4, int k, uint16_t* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  int64_t t = i / H4, c = i % H4;
  const f32x4* src = reinterpret_cast<const f32x4*>(y_w) + t * k * H4 + c;
  f32x4 s = src[0];
  for (int j = 1; j < k; ++j) {
    f32x4 v = src[(int64_t)j * H4];
    s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
  }
  u32x2 o = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  reinterpret_cast<u32x2*>(out)[i] = o;
}

constexpr int FWD_WN = 4;

hipError_t launch_gate_up(const uint16_t* x, const uint8_t* codes, const uint8_t* scales,
                          const uint16_t* bias, const int32_t* sorted_rows, const Tile* tiles,
                          const int32_t* num_tiles, int max_tiles, int H, int I, int k,
                          float alpha, float limit, uint16_t* h_out, uint16_t* a_out,
                          hipStream_t s) {
  constexpr int NT = FwdTile<FWD_WN>::NT;
  dim3 grid((2 * I + NT - 1) / NT, max_tiles);
  hipLaunchKernelGGL(gate_up_kernel<FWD_WN>, grid, dim3(64 * FWD_WN), 0, s, x, codes, scales,
                     bias, sorted_rows, tiles, num_tiles, H, I, k, alpha, limit, h_out, a_out);
  return hipGetLastError();
}

hipError_t launch_down(const uint16_t* a, const uint8_t* codes, const uint8_t* scales,
                       const uint16_t* bias, const float* topk_w, const int32_t* sorted_rows,
                       const Tile* tiles, const int32_t* num_tiles, int max_tiles, int H, int I,
                       float* y_w, hipStream_t s) {
  constexpr int NT = FwdTile<FWD_WN>::NT;
  dim3 grid((H + NT - 1) / NT, max_tiles);
  hipLaunchKernelGGL(down_kernel<FWD_WN>, grid, dim3(64 * FWD_WN), 0, s, a, codes, scales, bias,
                     topk_w, sorted_rows, tiles, num_tiles, H, I, y_w);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y_w, int64_t T, int H, int k, uint16_t* out,
                          hipStream_t s) {
  int64_t n4 = T * H / 4;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, y_w,
                     n4, H / 4, k, out);
  return hipGetLastError();
}

}  // namespace mxmoe
