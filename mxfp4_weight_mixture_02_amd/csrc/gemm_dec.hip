// Decode-sized forward GEMMs (few routed rows per expert): the same math as
// gate_up_kernel / down_kernel in gemm_fwd.hip, reorganised so that the
// packed weights of the touched experts stream from HBM at full rate.
//
// With T*k <= 256 an expert owns a handful of rows, so the work is bound by
// reading its weights once (13.2 MB per gpt-oss-20b expert), not by MFMA.
// A workgroup takes one tile (one expert's rows, at most 128) and 32 weight
// rows; its 4 waves split the contraction K into 4 contiguous ranges.  Each
// wave issues every code and scale load of its range before computing, so a
// workgroup keeps 32 x K/2 bytes in flight at once, and the grid (tiles x
// N/32 workgroups) covers the chip even at one token.  The routed rows'
// activations are staged in LDS in groups of 8 and fed as the MFMA
// B-operand (columns 8..31 of the 32-wide block repeat them and are
// dropped); the codes stay in registers across groups.  The 4 partial
// accumulators are summed through LDS (over the staged rows, once every
// wave has finished reading them), and wave w finishes accumulator
// registers 4w..4w+3: gate/up pairs still sit in neighbouring registers of
// one lane, so the bias + clamped SwiGLU epilogue is the forward GEMM's.
#include "common.hpp"
#include "launch.hpp"

namespace mxmoe {

constexpr int DW = 4;                    // waves per workgroup (K split)
constexpr int DG = 8;                    // routed rows per activation group
constexpr int DSTEPS = 12;               // max 64-wide K steps per wave
constexpr int DEC_MAXK = DW * DSTEPS * 64;
constexpr int DEC_XPAD = 8;              // bf16 of padding per staged row

int dec_max_k() { return DEC_MAXK; }

template <bool GATE_UP, int RB>
__global__ __launch_bounds__(64 * DW) void dec_kernel(
    const uint16_t* __restrict__ src,      // gate_up: x [T, K]; down: a [R, K] (sorted)
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ bias, const float* __restrict__ topk_w,
    const int32_t* __restrict__ sorted_rows, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int K, int N, int k, float alpha, float limit,
    uint16_t* __restrict__ h_out, uint16_t* __restrict__ a_out, float* __restrict__ y_w) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int nrb = N / (32 * RB);
  const int tile = blockIdx.x / nrb, rb0 = (blockIdx.x % nrb) * RB;
  if (tile >= *num_tiles) return;
  const Tile tl = tiles[tile];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int e = tl.expert;
  const int xrow = K + DEC_XPAD;                       // staged row stride (bf16)
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds);      // [DG][xrow]
  float* red = reinterpret_cast<float*>(lds);          // [DW][RB][16][64], reuses xs

  // this wave's K steps; per row block its row of codes and scales
  const int nsteps = K / 64;
  const int per = (nsteps + DW - 1) / DW;
  const int c0 = min(wave * per, nsteps), cnt = min(per, nsteps - c0);
  u32x4 cv[RB][DSTEPS];
  uint32_t sv[RB][DSTEPS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int n = (rb0 + rb) * 32 + l32;
    const uint8_t* wrow = codes + ((int64_t)e * N + n) * (K / 2) + hlf * 16;
    const uint8_t* srow = scales + ((int64_t)e * N + n) * (K / 32) + hlf;
#pragma unroll
    for (int i = 0; i < DSTEPS; ++i) {
      const int c = c0 + min(i, cnt - 1);             // clamped: never past the row
      cv[rb][i] = *reinterpret_cast<const u32x4*>(wrow + c * 32);
      sv[rb][i] = srow[2 * c];
    }
  }

  for (int g0 = 0; g0 < tl.rows; g0 += DG) {
    // stage the group's activation rows (only the ones that exist)
    const int ng = min(DG, tl.rows - g0);
    for (int q = tid; q < ng * (K / 8); q += 64 * DW) {
      const int p = q / (K / 8), col = (q % (K / 8)) * 8;
      const int rt = tl.row0 + g0 + p;
      const int64_t srow_ = GATE_UP ? (int64_t)(sorted_rows[rt] / k) : (int64_t)rt;
      *reinterpret_cast<u32x4*>(xs + p * xrow + col) =
          *reinterpret_cast<const u32x4*>(src + srow_ * K + col);
    }
    __syncthreads();
    f32x16 acc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][r] = 0.0f;
    // B-operand column l32 reads row min(l32 % 8, ng - 1): columns past the
    // group repeat its last row and are dropped
    const uint16_t* xb = xs + min(l32 & (DG - 1), ng - 1) * xrow + 32 * hlf;
#pragma unroll
    for (int i = 0; i < DSTEPS; ++i) {
      if (i < cnt) {
        const int c = c0 + i;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(xb + 64 * c + 8 * s);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const bf16x8 a = as_bf16x8(dequant8_bf16(cv[rb][i][s], scale_operand(sv[rb][i])));
            acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[rb], 0, 0, 0);
          }
        }
      }
    }
    // sum the K-range partials: wave w finishes registers 4w..4w+3 of
    // every row block
    __syncthreads();   // every wave is done reading xs
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((wave * RB + rb) * 16 + r) * 64 + lane] = acc[rb][r];
    __syncthreads();
    const int p = g0 + l32;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < DW; ++w) sum += red[((w * RB + rb) * 16 + 4 * wave + i) * 64 + lane];
        v[i] = sum;
      }
      // lane: column p of the group, weight rows nb + i
      if (l32 < DG && p < tl.rows) {
        const int nb = (rb0 + rb) * 32 + 8 * wave + 4 * hlf;
        float bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) bv[i] = bias ? bf16_to_f32(bias[(int64_t)e * N + nb + i]) : 0.0f;
        const int64_t rho = tl.row0 + p;
        if (GATE_UP) {
          const int I = N / 2;
          const float g0v = v[0] + bv[0], u0 = v[1] + bv[1], g1v = v[2] + bv[2], u1 = v[3] + bv[3];
          if (h_out) {
            u32x2 hv = {saved_preact_bf16(g0v, limit, false) | (saved_preact_bf16(u0, limit, true) << 16),
                        saved_preact_bf16(g1v, limit, false) | (saved_preact_bf16(u1, limit, true) << 16)};
            *reinterpret_cast<u32x2*>(h_out + rho * N + nb) = hv;
          }
          *reinterpret_cast<uint32_t*>(a_out + rho * I + nb / 2) =
              pack_bf16x2(swiglu(g0v, u0, alpha, limit), swiglu(g1v, u1, alpha, limit));
        } else {
          const int64_t f = sorted_rows[rho];
          const float wf = topk_w[f];
          f32x4 y;
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = wf * (v[i] + bv[i]);
          *reinterpret_cast<f32x4*>(y_w + f * N + nb) = y;
        }
      }
    }
    __syncthreads();   // LDS is restaged for the next group
  }
}

static size_t dec_lds_bytes(int K, int rb) {
  const size_t xs = (size_t)DG * (K + DEC_XPAD) * 2, red = (size_t)DW * rb * 16 * 64 * 4;
  return xs > red ? xs : red;
}

// Weight rows per workgroup: 32 while few rows are routed (so the grid
// still covers the chip), 64 when more are, so that one staging of the
// activation rows serves more weight rows (128 drops to one wave per SIMD
// and measured slower).
static int dec_rb(int64_t R, int N) {
  int rb = R <= 16 ? 1 : 2;
  while (rb > 1 && N % (32 * rb)) rb >>= 1;
  return rb;
}

template <bool GATE_UP>
static hipError_t dec_launch(int rb, int max_tiles, int K, int N, hipStream_t s,
                             const uint16_t* src, const uint8_t* codes, const uint8_t* scales,
                             const uint16_t* bias, const float* topk_w,
                             const int32_t* sorted_rows, const Tile* tiles,
                             const int32_t* num_tiles, int k, float alpha, float limit,
                             uint16_t* h_out, uint16_t* a_out, float* y_w) {
  const dim3 grid(max_tiles * (N / (32 * rb))), block(64 * DW);
  const size_t lds = dec_lds_bytes(K, rb);
#define DEC_ARGS src, codes, scales, bias, topk_w, sorted_rows, tiles, num_tiles, K, N, k, alpha, \
                 limit, h_out, a_out, y_w
  switch (rb) {
    case 1: hipLaunchKernelGGL((dec_kernel<GATE_UP, 1>), grid, block, lds, s, DEC_ARGS); break;
    case 2: hipLaunchKernelGGL((dec_kernel<GATE_UP, 2>), grid, block, lds, s, DEC_ARGS); break;
    default: hipLaunchKernelGGL((dec_kernel<GATE_UP, 4>), grid, block, lds, s, DEC_ARGS); break;
  }
#undef DEC_ARGS
  return hipGetLastError();
}

hipError_t launch_dec_gate_up(const uint16_t* x, const uint8_t* codes, const uint8_t* scales,
                              const uint16_t* bias, const int32_t* sorted_rows, const Tile* tiles,
                              const int32_t* num_tiles, int max_tiles, int64_t R, int H, int I, int k,
                              float alpha, float limit, uint16_t* h_out, uint16_t* a_out,
                              hipStream_t s) {
  if (H % 64 || H > DEC_MAXK || I % 32) return hipErrorInvalidValue;
  const int N = 2 * I;
  return dec_launch<true>(dec_rb(R, N), max_tiles, H, N, s, x, codes, scales,
                          bias, nullptr, sorted_rows, tiles, num_tiles, k, alpha, limit, h_out,
                          a_out, nullptr);
}

hipError_t launch_dec_down(const uint16_t* a, const uint8_t* codes, const uint8_t* scales,
                           const uint16_t* bias, const float* topk_w, const int32_t* sorted_rows,
                           const Tile* tiles, const int32_t* num_tiles, int max_tiles, int64_t R,
                           int H, int I,
                           float* y_w, hipStream_t s) {
  if (I % 64 || I > DEC_MAXK || H % 32) return hipErrorInvalidValue;
  return dec_launch<false>(dec_rb(R, H), max_tiles, I, H, s, a, codes, scales,
                           bias, topk_w, sorted_rows, tiles, num_tiles, 1, 0.0f, 0.0f, nullptr,
                           nullptr, y_w);
}

}  // namespace mxmoe
