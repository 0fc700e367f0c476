// Backward (dX) grouped expert GEMMs on gfx950 MFMA, over the same packed
// MXFP4 weights the forward reads, now contracted over their stored row
// axis ("Add MXFP4 training support via a dequantize-on-the-fly fallback":
// the backward of the frozen base only needs input and adapter gradients;
// the fallback recomputes dequantisation, which here happens once per
// workgroup tile in LDS).
//
// bwd_down:    da_u[p, i] = sum_h dY[t(p), h] * deq(Wd[e, h, i])
//              epilogue: dw partial sum_i da_u * a, then the SwiGLU backward
//              with da = w * da_u on the saved h, writing dh interleaved
//              (dh[2i] = d/dgate, dh[2i+1] = d/dup).
// bwd_gate_up: dxr[p, h] = sum_n dh[p, n] * deq(Wgu[e, n, h]), written to the
//              routed row's own slot for an ordered combine.
// bwd_combine: dX[t] = sum_j dxr[(t,j)] + sum_j dl_j * Wr[idx_j], with the
//              softmax-over-selected gradient dl_j = w_j (dw_j - sum_i w_i dw_i).
//
// Transposed operand.  The MFMA wants 8 consecutive contraction elements
// per lane, but the packed rows run along the output axis and the UE8M0
// scales are blocked along it too.  Each thread therefore loads an 8x8
// block (8 stored rows x one dword of 8 codes), decodes each row with its
// own scale (one scaled conversion per code pair), transposes the 8x8 bf16
// block in registers with byte permutes, and writes 8 contraction-ordered
// 16-byte rows into LDS; the MFMA A-operand is then one 16-byte LDS read.
// Output tiling and accumulator layout are those of the forward GEMMs.
#include "common.hpp"
#include "launch.hpp"

namespace mxmoe {

template <int WN>
struct BwdTile {
  static constexpr int NTHR = 64 * WN;
  static constexpr int NT = 64 * WN;         // output columns per workgroup
  static constexpr int PPT = MT * 8 / NTHR;  // 16-byte B pieces per thread per step
  static constexpr int OB = NT / 8;          // 8-column blocks across the tile
};

// Raw codes and scales of one thread's 8x8 block for one K step.
struct RawBlock {
  uint32_t code[8];
  uint32_t scale[8];
};

__device__ __forceinline__ void load_block(RawBlock& rb, const uint8_t* __restrict__ code0,
                                           const uint8_t* __restrict__ scale0, int64_t crow,
                                           int64_t srow) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    rb.code[r] = *reinterpret_cast<const uint32_t*>(code0 + r * crow);
    rb.scale[r] = scale0[r * srow];
  }
}

// Decode the 8x8 block and store it transposed: dst row o (0..7) gets the
// 8 contraction-ordered bf16 of output column o.
__device__ __forceinline__ void store_block_t(const RawBlock& rb, uint16_t* dst_row0) {
  u32x4 R[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) R[r] = dequant8_bf16(rb.code[r], scale_operand(rb.scale[r]));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4 lo, hi;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      lo[m] = __builtin_amdgcn_perm(R[2 * m + 1][j], R[2 * m][j], 0x05040100u);
      hi[m] = __builtin_amdgcn_perm(R[2 * m + 1][j], R[2 * m][j], 0x07060302u);
    }
    *reinterpret_cast<u32x4*>(dst_row0 + (2 * j) * LDS_ROW) = lo;
    *reinterpret_cast<u32x4*>(dst_row0 + (2 * j + 1) * LDS_ROW) = hi;
  }
}

// Main loop shared by the two backward GEMMs.  W is stored [C rows][O
// cols] (packed along O); this workgroup produces output columns o0.. for
// routed rows whose contraction vectors are brow[j] (length C).  Rows past
// the tile point at its first row and weight blocks past the last output
// column at the first one, so every load is unconditional (the affected
// products are never stored); only the first NRB 32-row blocks hold rows.
//
// Pipeline: global loads run two K steps ahead.  In step c a thread issues
// the loads of step c+2 (activation pieces and its raw 8x8 weight block),
// stores the step c+1 data it loaded one step earlier into the other LDS
// buffers (the weight block decoded and transposed on the way), then the
// waves run the MFMAs of step c from LDS; one barrier per step.  Step
// indices are clamped at the end instead of branching around loads, so the
// compiler's wait counts stay exact.  The loop is unrolled by two so every
// register set has a fixed name.  The step's barrier waits for LDS stores
// only, so the loads of step c + 2 stay in flight across it.
template <int WN>
struct BwdPipe {
  u32x4 xv[2][BwdTile<WN>::PPT];
  RawBlock raw[2];
};

template <int WN, int PAR>
__device__ __forceinline__ void bwd_issue(BwdPipe<WN>& pp, const uint16_t* const (&brow)[BwdTile<WN>::PPT],
                                          const uint8_t* bcode, const uint8_t* bscale,
                                          int64_t crow, int64_t srow, int c) {
#pragma unroll
  for (int j = 0; j < BwdTile<WN>::PPT; ++j)
    pp.xv[PAR][j] = *reinterpret_cast<const u32x4*>(brow[j] + c * KC);
  load_block(pp.raw[PAR], bcode + (int64_t)c * KC * crow, bscale + (int64_t)c * KC * srow, crow,
             srow);
}

template <int WN, int PAR>
__device__ __forceinline__ void bwd_stage(const BwdPipe<WN>& pp, uint16_t* wdst,
                                          uint16_t (*xs)[MT][LDS_ROW]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < BwdTile<WN>::PPT; ++j) {
    int q = tid + j * BwdTile<WN>::NTHR;
    *reinterpret_cast<u32x4*>(&xs[PAR][q >> 3][(q & 7) * 8]) = pp.xv[PAR][j];
  }
  store_block_t(pp.raw[PAR], wdst);
}

template <int WN, int NRB, int PAR>
__device__ __forceinline__ void bwd_step(BwdPipe<WN>& pp, const uint16_t* const (&brow)[BwdTile<WN>::PPT],
                                         const uint8_t* bcode, const uint8_t* bscale,
                                         int64_t crow, int64_t srow, int c, int nsteps,
                                         uint16_t* wdst_next,
                                         uint16_t (*ws)[BwdTile<WN>::NT][LDS_ROW],
                                         uint16_t (*xs)[MT][LDS_ROW], f32x16 (&acc)[2][4]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  bwd_issue<WN, PAR>(pp, brow, bcode, bscale, crow, srow, min(c + 2, nsteps - 1));
  __builtin_amdgcn_sched_barrier(0);  // keep the loads at the top of the step
  bwd_stage<WN, PAR ^ 1>(pp, wdst_next, xs);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int r0 = wave * 64 + l32, r1 = r0 + 32;
    const int lcb = 4 * hlf + st;
    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&ws[PAR][r0][(lcb ^ ((r0 >> 4) & 7)) * 8]);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&ws[PAR][r1][(lcb ^ ((r1 >> 4) & 7)) * 8]);
#pragma unroll
    for (int tb = 0; tb < NRB; ++tb) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(&xs[PAR][tb * 32 + l32][hlf * 32 + st * 8]);
      acc[0][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b, acc[0][tb], 0, 0, 0);
      acc[1][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b, acc[1][tb], 0, 0, 0);
    }
  }
  // The next step reads what this one staged: wait for this wave's LDS
  // stores (lgkmcnt) only.  A fenced __syncthreads would also drain the
  // global loads of step c + 2 issued above; their registers get the
  // compiler's own counted waits where they are used.
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  barrier_only();
}

template <int WN, int NRB>
__device__ __forceinline__ void bwd_mainloop_n(const uint16_t* const (&brow)[BwdTile<WN>::PPT],
                                               const uint8_t* bcode, const uint8_t* bscale,
                                               int64_t crow, int64_t srow, int nsteps,
                                               uint16_t* wdst0, uint16_t* wdst1,
                                               uint16_t (*ws)[BwdTile<WN>::NT][LDS_ROW],
                                               uint16_t (*xs)[MT][LDS_ROW], f32x16 (&acc)[2][4]) {
  BwdPipe<WN> pp;
  bwd_issue<WN, 0>(pp, brow, bcode, bscale, crow, srow, 0);
  bwd_issue<WN, 1>(pp, brow, bcode, bscale, crow, srow, min(1, nsteps - 1));
  bwd_stage<WN, 0>(pp, wdst0, xs);
  __syncthreads();
  int c = 0;
  for (; c + 1 < nsteps; c += 2) {
    bwd_step<WN, NRB, 0>(pp, brow, bcode, bscale, crow, srow, c, nsteps, wdst1, ws, xs, acc);
    bwd_step<WN, NRB, 1>(pp, brow, bcode, bscale, crow, srow, c + 1, nsteps, wdst0, ws, xs, acc);
  }
  if (c < nsteps)
    bwd_step<WN, NRB, 0>(pp, brow, bcode, bscale, crow, srow, c, nsteps, wdst1, ws, xs, acc);
}

template <int WN>
__device__ __forceinline__ void bwd_mainloop(const uint16_t* const (&brow)[BwdTile<WN>::PPT],
                                             const uint8_t* __restrict__ wcode,
                                             const uint8_t* __restrict__ wscale, int C, int O,
                                             int o0, int nrb,
                                             uint16_t (*ws)[BwdTile<WN>::NT][LDS_ROW],
                                             uint16_t (*xs)[MT][LDS_ROW], f32x16 (&acc)[2][4]) {
  using BT = BwdTile<WN>;
  const int tid = threadIdx.x;
  const int nsteps = C / KC;
  const int64_t crow = O / 2, srow = O / 32;

  // this thread's 8x8 weight block: rows 8*cb.., output columns 8*ob..
  const int cb = tid / BT::OB, ob = tid % BT::OB;
  const int ocol = (o0 + 8 * ob < O) ? o0 + 8 * ob : 0;
  const uint8_t* bcode = wcode + (int64_t)(8 * cb) * crow + ocol / 2;
  const uint8_t* bscale = wscale + (int64_t)(8 * cb) * srow + ocol / 32;
  // column block swizzle: 16-byte block c of row r sits at c ^ ((r >> 4) & 7),
  // which spreads both these transposed writes and the MFMA reads over all
  // banks (all 8 rows of this thread's block share r >> 4 = ob >> 1)
  const int pcb = cb ^ ((ob >> 1) & 7);
  uint16_t* const wdst0 = &ws[0][8 * ob][8 * pcb];
  uint16_t* const wdst1 = &ws[1][8 * ob][8 * pcb];

#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][tb][r] = 0.0f;

  switch (nrb) {
    case 1: bwd_mainloop_n<WN, 1>(brow, bcode, bscale, crow, srow, nsteps, wdst0, wdst1, ws, xs, acc); break;
    case 2: bwd_mainloop_n<WN, 2>(brow, bcode, bscale, crow, srow, nsteps, wdst0, wdst1, ws, xs, acc); break;
    case 3: bwd_mainloop_n<WN, 3>(brow, bcode, bscale, crow, srow, nsteps, wdst0, wdst1, ws, xs, acc); break;
    default: bwd_mainloop_n<WN, 4>(brow, bcode, bscale, crow, srow, nsteps, wdst0, wdst1, ws, xs, acc); break;
  }
}

template <int WN>
__global__ __launch_bounds__(64 * WN) void bwd_down_kernel(
    const uint16_t* __restrict__ dy, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ topk_w,
    const int32_t* __restrict__ sorted_rows, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, const uint16_t* __restrict__ hsv,
    const uint16_t* __restrict__ asv, int H, int I, int k, float alpha, float limit,
    const uint16_t* __restrict__ lora_At, const float* __restrict__ lora_dvu,
    uint16_t* __restrict__ dh, float* __restrict__ dw_part) {
  using BT = BwdTile<WN>;
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][BT::NT][LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MT][LDS_ROW];
  __shared__ float red[WN][MT];
  int mt, ot;
  const int otiles = (I + BT::NT - 1) / BT::NT;
  if (!xcd_work_item(*num_tiles, otiles, &mt, &ot)) return;
  const Tile tl = tiles[mt];
  const int o0 = ot * BT::NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int e = tl.expert;

  const uint16_t* brow[BT::PPT];
#pragma unroll
  for (int j = 0; j < BT::PPT; ++j) {
    int q = tid + j * BT::NTHR;
    int r = q >> 3;
    const int f = sorted_rows[tl.row0 + (r < tl.rows ? r : 0)];
    brow[j] = dy + (int64_t)(f / k) * H + (q & 7) * 8;
  }
  // Wd is stored [H rows][I cols]: contraction over h (C = H), output i (O = I)
  const bool wave_live = o0 + wave * 64 < I;
  const uint8_t* wcode = codes + (int64_t)e * H * (I / 2);
  const uint8_t* wscale = scales + (int64_t)e * H * (I / 32);
  f32x16 acc[2][4];
  bwd_mainloop<WN>(brow, wcode, wscale, H, I, o0, (tl.rows + 31) / 32, ws, xs, acc);
  if (lora_At) {
    // + dv_u A_e (dv_u = s dY B_e, unweighted like the accumulators): a
    // 16-deep contraction, A-operand = rows of A_e^T, B-operand = dv_u as
    // hi + lo bf16.  Through the accumulators it also reaches the dw
    // partial: sum_i (dv_u A_e)_i a_i = dv_u . v, the adapter's share of dY . y.
    bf16x8 vh[4], vl[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const float* vp = lora_dvu + (int64_t)(tl.row0 + min(tb * 32 + l32, tl.rows - 1)) * LORA_R + 8 * hlf;
      split_bf16x8(*reinterpret_cast<const f32x4*>(vp), *reinterpret_cast<const f32x4*>(vp + 4),
                   1.0f, &vh[tb], &vl[tb]);
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int i = o0 + wave * 64 + rb * 32 + l32;
      const bf16x8 aw = as_bf16x8(*reinterpret_cast<const u32x4*>(lora_At + ((int64_t)e * I + (i < I ? i : 0)) * LORA_R + 8 * hlf));
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        acc[rb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, vh[tb], acc[rb][tb], 0, 0, 0);
        acc[rb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, vl[tb], acc[rb][tb], 0, 0, 0);
      }
    }
  }

  const int N2 = 2 * I;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int rt = tb * 32 + l32;
    float dwp = 0.0f;
    if (wave_live && rt < tl.rows) {
      const int64_t p = tl.row0 + rt;
      const float wf = topk_w[sorted_rows[p]];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i4 = o0 + wave * 64 + rb * 32 + 8 * q + 4 * hlf;
          const u32x2 av = *reinterpret_cast<const u32x2*>(asv + p * I + i4);
          const u32x4 hv = *reinterpret_cast<const u32x4*>(hsv + p * N2 + 2 * i4);
          u32x4 out;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float du_ = acc[rb][tb][4 * q + m];
            const uint32_t aw = av[m >> 1];
            const float a_m = bf16_to_f32((uint16_t)((m & 1) ? (aw >> 16) : (aw & 0xFFFFu)));
            dwp += du_ * a_m;
            const uint32_t hw = hv[m];
            const float g = bf16_to_f32((uint16_t)(hw & 0xFFFFu));
            const float u = bf16_to_f32((uint16_t)(hw >> 16));
            float dg, dup;
            swiglu_grad(g, u, wf * du_, alpha, limit, &dg, &dup);
            out[m] = pack_bf16x2(dg, dup);
          }
          *reinterpret_cast<u32x4*>(dh + p * N2 + 2 * i4) = out;
        }
      }
    }
    dwp += __shfl_xor(dwp, 32);
    if (hlf == 0) red[wave][rt] = dwp;
  }
  __syncthreads();
  if (tid < tl.rows) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < WN; ++w) s += red[w][tid];
    const int64_t f = sorted_rows[tl.row0 + tid];
    dw_part[f * otiles + ot] = s;
  }
}

template <int WN>
__global__ __launch_bounds__(64 * WN) void bwd_gate_up_kernel(
    const uint16_t* __restrict__ dh, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const int32_t* __restrict__ sorted_rows,
    const Tile* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int H, int I,
    float* __restrict__ dxr) {
  using BT = BwdTile<WN>;
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][BT::NT][LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MT][LDS_ROW];
  int mt, ot;
  const int otiles = (H + BT::NT - 1) / BT::NT;
  if (!xcd_work_item(*num_tiles, otiles, &mt, &ot)) return;
  const Tile tl = tiles[mt];
  const int o0 = ot * BT::NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int e = tl.expert;
  const int N2 = 2 * I;

  const uint16_t* brow[BT::PPT];
#pragma unroll
  for (int j = 0; j < BT::PPT; ++j) {
    int q = tid + j * BT::NTHR;
    int r = q >> 3;
    brow[j] = dh + (int64_t)(tl.row0 + (r < tl.rows ? r : 0)) * N2 + (q & 7) * 8;
  }
  // Wgu is stored [2I rows][H cols]: contraction over n (C = 2I), output h (O = H)
  const bool wave_live = o0 + wave * 64 < H;
  const uint8_t* wcode = codes + (int64_t)e * N2 * (H / 2);
  const uint8_t* wscale = scales + (int64_t)e * N2 * (H / 32);
  f32x16 acc[2][4];
  bwd_mainloop<WN>(brow, wcode, wscale, N2, H, o0, (tl.rows + 31) / 32, ws, xs, acc);
  if (!wave_live) return;

#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int rt = tb * 32 + l32;
    if (rt >= tl.rows) continue;
    const int64_t f = sorted_rows[tl.row0 + rt];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int h4 = o0 + wave * 64 + rb * 32 + 8 * q + 4 * hlf;
        f32x4 v;
#pragma unroll
        for (int m = 0; m < 4; ++m) v[m] = acc[rb][tb][4 * q + m];
        *reinterpret_cast<f32x4*>(dxr + f * H + h4) = v;
      }
  }
}

// One workgroup (256 threads) per token.
__global__ __launch_bounds__(256) void bwd_combine_kernel(
    const uint16_t* __restrict__ dy, const float* __restrict__ dxr,
    const float* __restrict__ dw_part, int n_dw_part, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, const uint16_t* __restrict__ dn_bias,
    const float* __restrict__ router_w, int H, int k, uint16_t* __restrict__ dx) {
  __shared__ float red[4][8];
  __shared__ float dl[8];
  __shared__ int32_t ex[8];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < k) ex[tid] = topk_idx[t * k + tid];
  __syncthreads();
  // dY . bd[e_j] for each slot (the bias part of dw_j = dY . y_j)
  float part[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) part[j] = 0.0f;
  if (dn_bias) {
    for (int h = tid; h < H; h += 256) {
      const float g = bf16_to_f32(dy[t * H + h]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < k) part[j] += g * bf16_to_f32(dn_bias[(int64_t)ex[j] * H + h]);
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float v = part[j];
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0 && j < k) red[wave][j] = v;
  }
  __syncthreads();
  if (tid == 0) {
    float dw[8], w[8], sw = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int64_t f = t * k + j;
      float s = red[0][j] + red[1][j] + red[2][j] + red[3][j];
      for (int q = 0; q < n_dw_part; ++q) s += dw_part[f * n_dw_part + q];
      dw[j] = s;
      w[j] = topk_w[f];
      sw += w[j] * s;
    }
    for (int j = 0; j < k; ++j) dl[j] = w[j] * (dw[j] - sw);
  }
  __syncthreads();
  const int H4 = H / 4;
  for (int c = tid; c < H4; c += 256) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const f32x4 v = reinterpret_cast<const f32x4*>(dxr + (t * k + j) * H)[c];
      const f32x4 r = reinterpret_cast<const f32x4*>(router_w + (int64_t)ex[j] * H)[c];
      const float d = dl[j];
#pragma unroll
      for (int m = 0; m < 4; ++m) s[m] += v[m] + d * r[m];
    }
    u32x2 o = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
    reinterpret_cast<u32x2*>(dx + t * H)[c] = o;
  }
}

constexpr int BWD_WN = 4;

int bwd_down_ntiles(int I) { return (I + BwdTile<BWD_WN>::NT - 1) / BwdTile<BWD_WN>::NT; }

hipError_t launch_bwd_down(const uint16_t* dy, const uint8_t* codes, const uint8_t* scales,
                           const float* topk_w, const int32_t* sorted_rows, const Tile* tiles,
                           const int32_t* num_tiles, int max_tiles, const uint16_t* h,
                           const uint16_t* a, int H, int I, int k, float alpha, float limit,
                           const uint16_t* lora_At, const float* lora_dvu, uint16_t* dh,
                           float* dw_part, hipStream_t s) {
  dim3 grid(bwd_down_ntiles(I) * max_tiles);
  hipLaunchKernelGGL(bwd_down_kernel<BWD_WN>, grid, dim3(64 * BWD_WN), 0, s, dy, codes, scales,
                     topk_w, sorted_rows, tiles, num_tiles, h, a, H, I, k, alpha, limit,
                     lora_At, lora_dvu, dh, dw_part);
  return hipGetLastError();
}

hipError_t launch_bwd_gate_up(const uint16_t* dh, const uint8_t* codes, const uint8_t* scales,
                              const int32_t* sorted_rows, const Tile* tiles,
                              const int32_t* num_tiles, int max_tiles, int H, int I,
                              float* dxr, hipStream_t s) {
  constexpr int NT = BwdTile<BWD_WN>::NT;
  dim3 grid(((H + NT - 1) / NT) * max_tiles);
  hipLaunchKernelGGL(bwd_gate_up_kernel<BWD_WN>, grid, dim3(64 * BWD_WN), 0, s, dh, codes,
                     scales, sorted_rows, tiles, num_tiles, H, I, dxr);
  return hipGetLastError();
}

hipError_t launch_bwd_combine(const uint16_t* dy, const float* dxr, const float* dw_part,
                              int n_dw_part, const int32_t* topk_idx, const float* topk_w,
                              const uint16_t* dn_bias, const float* router_w, int64_t T, int H,
                              int k, uint16_t* dx, hipStream_t s) {
  hipLaunchKernelGGL(bwd_combine_kernel, dim3((unsigned)T), dim3(256), 0, s, dy, dxr, dw_part,
                     n_dw_part, topk_idx, topk_w, dn_bias, router_w, H, k, dx);
  return hipGetLastError();
}

}  // namespace mxmoe
