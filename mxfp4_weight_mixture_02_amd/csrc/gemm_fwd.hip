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
// the activation row for B piece j (already offset by its 8-element piece),
// or is null for rows past the tile.  Weights: wrow = first weight row of
// this lane (row block 0), N rows per expert, K columns.
template <int WN>
__device__ __forceinline__ void fwd_mainloop(const uint16_t* const (&brow)[FwdTile<WN>::PPT],
                                             const uint8_t* __restrict__ wcode,
                                             const uint8_t* __restrict__ wscale, int K,
                                             bool wave_live, uint16_t (*xs)[MT][LDS_ROW],
                                             f32x16 (&acc)[2][4]) {
  using FT = FwdTile<WN>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int64_t KB = K / 2, KS = K / 32;
  const int nsteps = K / KC;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

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

  u32x4 xv[FT::PPT];
  u32x4 wv0 = zero4, wv1 = zero4;
  uint32_t s0 = 0, s1 = 0;
#pragma unroll
  for (int j = 0; j < FT::PPT; ++j)
    xv[j] = brow[j] ? *reinterpret_cast<const u32x4*>(brow[j]) : zero4;
  if (wave_live) {
    wv0 = *reinterpret_cast<const u32x4*>(wp0);
    wv1 = *reinterpret_cast<const u32x4*>(wp1);
    s0 = sp0[0];
    s1 = sp1[0];
  }
#pragma unroll
  for (int j = 0; j < FT::PPT; ++j) {
    int q = tid + j * FT::NTHR;
    *reinterpret_cast<u32x4*>(&xs[0][q >> 3][(q & 7) * 8]) = xv[j];
  }
  __syncthreads();

  for (int c = 0; c < nsteps; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nsteps;
    u32x4 nwv0 = zero4, nwv1 = zero4;
    uint32_t ns0 = 0, ns1 = 0;
    if (more) {
#pragma unroll
      for (int j = 0; j < FT::PPT; ++j)
        xv[j] = brow[j] ? *reinterpret_cast<const u32x4*>(brow[j] + (c + 1) * KC) : zero4;
      if (wave_live) {
        nwv0 = *reinterpret_cast<const u32x4*>(wp0 + (c + 1) * 32);
        nwv1 = *reinterpret_cast<const u32x4*>(wp1 + (c + 1) * 32);
        ns0 = sp0[(c + 1) * 2];
        ns1 = sp1[(c + 1) * 2];
      }
    }
    if (wave_live) {
      const float sc0 = scale_operand(s0), sc1 = scale_operand(s1);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 a0 = as_bf16x8(dequant8_bf16(wv0[s], sc0));
        const bf16x8 a1 = as_bf16x8(dequant8_bf16(wv1[s], sc1));
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const bf16x8 b =
              *reinterpret_cast<const bf16x8*>(&xs[buf][tb * 32 + l32][hlf * 32 + s * 8]);
          acc[0][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, acc[0][tb], 0, 0, 0);
          acc[1][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, acc[1][tb], 0, 0, 0);
        }
      }
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < FT::PPT; ++j) {
        int q = tid + j * FT::NTHR;
        *reinterpret_cast<u32x4*>(&xs[buf ^ 1][q >> 3][(q & 7) * 8]) = xv[j];
      }
      wv0 = nwv0;
      wv1 = nwv1;
      s0 = ns0;
      s1 = ns1;
    }
    __syncthreads();
  }
}

template <int WN>
__global__ __launch_bounds__(64 * WN) void gate_up_kernel(
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
    if (r < tl.rows) {
      int f = sorted_rows[tl.row0 + r];
      brow[j] = x + (int64_t)(f / k) * H + (q & 7) * 8;
    } else {
      brow[j] = nullptr;
    }
  }
  const int wrow = n0 + wave * 64 + l32;
  const bool wave_live = n0 + wave * 64 < N;
  const uint8_t* wcode = codes + ((int64_t)e * N + wrow) * (H / 2);
  const uint8_t* wscale = scales + ((int64_t)e * N + wrow) * (H / 32);
  f32x16 acc[2][4];
  fwd_mainloop<WN>(brow, wcode, wscale, H, wave_live, xs, acc);
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
__global__ __launch_bounds__(64 * WN) void down_kernel(
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
    brow[j] = (r < tl.rows) ? a + (int64_t)(tl.row0 + r) * I + (q & 7) * 8 : nullptr;
  }
  const int wrow = n0 + wave * 64 + l32;
  const bool wave_live = n0 + wave * 64 < N;
  const uint8_t* wcode = codes + ((int64_t)e * N + wrow) * (I / 2);
  const uint8_t* wscale = scales + ((int64_t)e * N + wrow) * (I / 32);
  f32x16 acc[2][4];
  fwd_mainloop<WN>(brow, wcode, wscale, I, wave_live, xs, acc);
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
