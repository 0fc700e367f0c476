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
// scales are blocked along it too.  Each thread therefore loads 8x8 blocks
// (8 stored rows x one dword of 8 codes), decodes each row with its own
// scale (one scaled conversion per code pair), transposes the bf16 block in
// registers with byte permutes, and writes 8 contraction-ordered 16-byte
// rows into LDS; the MFMA A-operand is then one 16-byte LDS read.
//
// Tiling.  A workgroup computes 512 output columns x 128 routed rows with 8
// waves, two per SIMD; wave w owns output columns 64w..64w+63 (two
// 32-column MFMA blocks) for all 128 rows (four 32-row blocks): 8
// accumulators of 32x32 fp32.  Per K step of 64 a wave reads 2 A- and 4
// B-fragments per 8 MFMAs from LDS; the second wave per SIMD hides the
// other's LDS and load waits (measured faster than one wave with four
// column blocks, which reads less LDS per MFMA).
//
// LDS: the transposed weights [512][64] bf16 and the activations [128][64]
// bf16, both double-buffered, exactly 160 KB, no padding.  Row r's eight
// 16-byte blocks are permuted by XOR with f(r) = (r ^ (r >> 3)) & 7 for
// the weights and r & 7 for the activations; the MFMA reads (32
// consecutive rows, one logical block), the transposed writes (rows 8j+c
// for 64 consecutive j) and the activation writes (8 blocks of one row)
// then each touch 8 distinct 16-byte bank groups per 8 lanes.
#include "common.hpp"
#include "launch.hpp"

namespace mxmoe {

constexpr int BW = 8;                      // waves per workgroup, two per SIMD
constexpr int BTHR = 64 * BW;
constexpr int BRB = 2;                     // 32-column output blocks per wave
constexpr int BNT = 32 * BRB * BW;         // output columns per workgroup (512)
constexpr int BKC = 64;                    // contraction per step
constexpr int BBLK = (BKC / 8) * (BNT / 8) / BTHR;   // 8x8 weight blocks per thread per step (1)
constexpr int BPPT = MT * 8 / BTHR;        // 16-byte activation pieces per thread per step (2)
constexpr int WS_BYTES = BNT * BKC * 2;    // one weight buffer (64 KB)
constexpr int XS_BYTES = MT * BKC * 2;     // one activation buffer (16 KB)
constexpr int BLDS = 2 * WS_BYTES + 2 * XS_BYTES;    // 160 KB
static_assert(BNT == 512, "thread work assumed below");

__device__ __forceinline__ int ws_off(int row, int blk) {
  return row * 128 + ((blk ^ ((row ^ (row >> 3)) & 7)) << 4);
}
__device__ __forceinline__ int xs_off(int row, int blk) {
  return row * 128 + ((blk ^ (row & 7)) << 4);
}

// Raw codes and scales of one thread's 8x8 block for one K step.
struct RawBlock {
  uint32_t code[8];
  uint32_t scale[8];
};

// Addresses are the expert's (workgroup-uniform) bases plus 32-bit offsets:
// one register per address instead of a 64-bit pointer pair.
__device__ __forceinline__ void load_block(RawBlock& rb, const uint8_t* __restrict__ cbase,
                                           const uint8_t* __restrict__ sbase, uint32_t coff,
                                           uint32_t soff, uint32_t crow, uint32_t srow) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    rb.code[r] = *reinterpret_cast<const uint32_t*>(cbase + (coff + r * crow));
    rb.scale[r] = sbase[soff + r * srow];
  }
}

// Decode the 8x8 block (contraction rows 8cb.., output columns 8ob..) and
// store it transposed: weight row 8ob + j gets the 8 contraction-ordered
// bf16 of output column j, in logical block cb.
// Column pair (2J, 2J+1) of the block's 8 rows, decoded with each row's
// scale, split into two contraction-ordered weight rows with byte permutes.
template <int J>
__device__ __forceinline__ void store_block_col(const RawBlock& rb, uint8_t* ws, int ob, int cb) {
  uint32_t d[8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
    d[r] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(
                                            rb.code[r], scale_operand(rb.scale[r]), J));
  u32x4 lo, hi;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    lo[m] = __builtin_amdgcn_perm(d[2 * m + 1], d[2 * m], 0x05040100u);
    hi[m] = __builtin_amdgcn_perm(d[2 * m + 1], d[2 * m], 0x07060302u);
  }
  *reinterpret_cast<u32x4*>(ws + ws_off(8 * ob + 2 * J, cb)) = lo;
  *reinterpret_cast<u32x4*>(ws + ws_off(8 * ob + 2 * J + 1, cb)) = hi;
}

// Decode the 8x8 block (contraction rows 8cb.., output columns 8ob..) and
// store it transposed: weight row 8ob + j gets the 8 contraction-ordered
// bf16 of output column j, in logical block cb.  One column pair at a time
// keeps 8 decoded dwords live instead of 32.
__device__ __forceinline__ void store_block_t(const RawBlock& rb, uint8_t* ws, int ob, int cb) {
  store_block_col<0>(rb, ws, ob, cb);
  store_block_col<1>(rb, ws, ob, cb);
  store_block_col<2>(rb, ws, ob, cb);
  store_block_col<3>(rb, ws, ob, cb);
}

// Per-thread state of the two-deep pipeline: registers of steps c+1 and c+2.
struct BwdPipe {
  u32x4 xv[2][BPPT];
  RawBlock raw[2][BBLK];
};

struct BwdArgs {
  const uint16_t* brow[BPPT];   // activation rows this thread stages (+ its 8-element piece)
  const uint8_t* wcode;         // the expert's codes and scales (workgroup-uniform)
  const uint8_t* wscale;
  uint32_t bcode[BBLK];         // byte offset of its weight blocks' first code row, at step 0
  uint32_t bscale[BBLK];        // and of the first scale row (an expert is < 4 GiB)
  uint32_t crow, srow;          // bytes between stored rows (codes, scales)
  int nsteps;
};

template <int PAR>
__device__ __forceinline__ void bwd_issue(BwdPipe& pp, const BwdArgs& g, int c) {
#pragma unroll
  for (int j = 0; j < BPPT; ++j) pp.xv[PAR][j] = *reinterpret_cast<const u32x4*>(g.brow[j] + c * BKC);
#pragma unroll
  for (int i = 0; i < BBLK; ++i)
    load_block(pp.raw[PAR][i], g.wcode, g.wscale, g.bcode[i] + (uint32_t)c * BKC * g.crow,
               g.bscale[i] + (uint32_t)c * BKC * g.srow, g.crow, g.srow);
}

template <int PAR>
__device__ __forceinline__ void bwd_stage(const BwdPipe& pp, uint8_t* lds) {
  const int tid = threadIdx.x;
  uint8_t* ws = lds + PAR * WS_BYTES;
  uint8_t* xs = lds + 2 * WS_BYTES + PAR * XS_BYTES;
#pragma unroll
  for (int j = 0; j < BPPT; ++j) {
    const int q = tid + j * BTHR;
    *reinterpret_cast<u32x4*>(xs + xs_off(q >> 3, q & 7)) = pp.xv[PAR][j];
  }
#pragma unroll
  for (int i = 0; i < BBLK; ++i) {
    const int q = tid + i * BTHR;
    store_block_t(pp.raw[PAR][i], ws, q & (BNT / 8 - 1), q / (BNT / 8));
  }
}

template <int NRB, int PAR>
__device__ __forceinline__ void bwd_step(BwdPipe& pp, const BwdArgs& g, int c, uint8_t* lds,
                                         f32x16 (&acc)[BRB][4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  bwd_issue<PAR>(pp, g, min(c + 2, g.nsteps - 1));
  __builtin_amdgcn_sched_barrier(0);  // keep the loads at the top of the step
  bwd_stage<PAR ^ 1>(pp, lds);
  const uint8_t* ws = lds + PAR * WS_BYTES;
  const uint8_t* xs = lds + 2 * WS_BYTES + PAR * XS_BYTES;
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int lb = 4 * hlf + st;
    bf16x8 a[BRB], b[NRB];
#pragma unroll
    for (int rb = 0; rb < BRB; ++rb)
      a[rb] = *reinterpret_cast<const bf16x8*>(ws + ws_off(wave * 32 * BRB + rb * 32 + l32, lb));
#pragma unroll
    for (int tb = 0; tb < NRB; ++tb)
      b[tb] = *reinterpret_cast<const bf16x8*>(xs + xs_off(tb * 32 + l32, lb));
#pragma unroll
    for (int rb = 0; rb < BRB; ++rb)
#pragma unroll
      for (int tb = 0; tb < NRB; ++tb)
        acc[rb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rb], b[tb], acc[rb][tb], 0, 0, 0);
  }
  // The next step reads what this one staged: wait for this wave's LDS
  // stores (lgkmcnt) only.  A fenced __syncthreads would also drain the
  // global loads of step c + 2 issued above; their registers get the
  // compiler's own counted waits where they are used.
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  barrier_only();
}

// Pipeline: global loads run two K steps ahead.  In step c a thread issues
// the loads of step c+2, stores the step c+1 data it loaded one step
// earlier into the other LDS buffers (the weight blocks decoded and
// transposed on the way), then the waves run the MFMAs of step c from LDS;
// one barrier per step.  Step indices are clamped at the end instead of
// branching around loads, so the compiler's wait counts stay exact.  The
// loop is unrolled by two so every register set has a fixed name.
template <int NRB>
__device__ __forceinline__ void bwd_loop(const BwdArgs& g, uint8_t* lds, f32x16 (&acc)[BRB][4]) {
  BwdPipe pp;
  bwd_issue<0>(pp, g, 0);
  bwd_issue<1>(pp, g, min(1, g.nsteps - 1));
  bwd_stage<0>(pp, lds);
  __syncthreads();
  int c = 0;
  for (; c + 1 < g.nsteps; c += 2) {
    bwd_step<NRB, 0>(pp, g, c, lds, acc);
    bwd_step<NRB, 1>(pp, g, c + 1, lds, acc);
  }
  if (c < g.nsteps) bwd_step<NRB, 0>(pp, g, c, lds, acc);
  __syncthreads();   // LDS is free for the epilogue
}

// Main loop shared by the two backward GEMMs.  W is stored [C rows][O
// cols] (packed along O); this workgroup produces output columns o0..o0+511
// for routed rows whose contraction vectors are brow[j] (length C).  Rows
// past the tile point at its first row and weight blocks past the last
// output column at the first one, so every load is unconditional (the
// affected products are never stored); only the first NRB 32-row blocks
// hold rows.
__device__ __forceinline__ void bwd_mainloop(const uint16_t* const (&brow)[BPPT],
                                             const uint8_t* __restrict__ wcode,
                                             const uint8_t* __restrict__ wscale, int C, int O,
                                             int o0, int nrb, uint8_t* lds,
                                             f32x16 (&acc)[BRB][4]) {
  const int tid = threadIdx.x;
  BwdArgs g;
  g.nsteps = C / BKC;
  g.crow = O / 2;
  g.srow = O / 32;
  g.wcode = wcode;
  g.wscale = wscale;
#pragma unroll
  for (int j = 0; j < BPPT; ++j) g.brow[j] = brow[j];
#pragma unroll
  for (int i = 0; i < BBLK; ++i) {
    const int q = tid + i * BTHR;
    const int cb = q / (BNT / 8), ob = q & (BNT / 8 - 1);
    const int ocol = (o0 + 8 * ob < O) ? o0 + 8 * ob : 0;
    g.bcode[i] = (uint32_t)(8 * cb) * g.crow + ocol / 2;
    g.bscale[i] = (uint32_t)(8 * cb) * g.srow + ocol / 32;
  }
#pragma unroll
  for (int rb = 0; rb < BRB; ++rb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][tb][r] = 0.0f;
  switch (nrb) {
    case 1: bwd_loop<1>(g, lds, acc); break;
    case 2: bwd_loop<2>(g, lds, acc); break;
    case 3: bwd_loop<3>(g, lds, acc); break;
    default: bwd_loop<4>(g, lds, acc); break;
  }
}

// LORA: add dv_u A_e (a template parameter: a runtime branch around these
// MFMAs makes the compiler spill accumulators).
template <bool LORA>
__global__ __launch_bounds__(BTHR) void bwd_down_kernel(
    const uint16_t* __restrict__ dy, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ topk_w,
    const int32_t* __restrict__ sorted_rows, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, const uint16_t* __restrict__ hsv,
    const uint16_t* __restrict__ asv, int H, int I, int k, float alpha, float limit,
    const uint16_t* __restrict__ lora_At, const float* __restrict__ lora_dvu,
    uint16_t* __restrict__ dh, float* __restrict__ dw_part) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[BLDS];
  int mt, ot;
  const int otiles = (I + BNT - 1) / BNT;
  if (!xcd_work_item(*num_tiles, otiles, &mt, &ot)) return;
  const Tile tl = tiles[mt];
  const int o0 = ot * BNT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int e = tl.expert;

  const uint16_t* brow[BPPT];
#pragma unroll
  for (int j = 0; j < BPPT; ++j) {
    const int q = tid + j * BTHR;
    const int r = q >> 3;
    const int f = sorted_rows[tl.row0 + (r < tl.rows ? r : 0)];
    brow[j] = dy + (int64_t)(f / k) * H + (q & 7) * 8;
  }
  // Wd is stored [H rows][I cols]: contraction over h (C = H), output i (O = I)
  const uint8_t* wcode = codes + (int64_t)e * H * (I / 2);
  const uint8_t* wscale = scales + (int64_t)e * H * (I / 32);
  f32x16 acc[BRB][4];
  bwd_mainloop(brow, wcode, wscale, H, I, o0, (tl.rows + 31) / 32, lds, acc);
  if (LORA) {
    // + dv_u A_e (dv_u = s dY B_e, unweighted like the accumulators): a
    // 16-deep contraction, A-operand = rows of A_e^T, B-operand = dv_u as
    // hi + lo bf16.  Through the accumulators it also reaches the dw
    // partial: sum_i (dv_u A_e)_i a_i = dv_u . v, the adapter's share of dY . y.
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const float* vp = lora_dvu + (int64_t)(tl.row0 + min(tb * 32 + l32, tl.rows - 1)) * LORA_R + 8 * hlf;
      bf16x8 vh, vl;
      split_bf16x8(*reinterpret_cast<const f32x4*>(vp), *reinterpret_cast<const f32x4*>(vp + 4),
                   1.0f, &vh, &vl);
#pragma unroll
      for (int rb = 0; rb < BRB; ++rb) {
        const int i = o0 + wave * 32 * BRB + rb * 32 + l32;
        const bf16x8 aw = as_bf16x8(*reinterpret_cast<const u32x4*>(
            lora_At + ((int64_t)e * I + (i < I ? i : 0)) * LORA_R + 8 * hlf));
        acc[rb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, vh, acc[rb][tb], 0, 0, 0);
        acc[rb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, vl, acc[rb][tb], 0, 0, 0);
      }
    }
  }

  // Epilogue through LDS (the main loop ended with a barrier).  Per 32-row
  // block a wave stages its rows of a (64 bf16) and h (128 bf16) with
  // row-contiguous loads, reads them back in the accumulator layout, writes
  // dh over h in place and stores dh rows whole.
  const int N2 = 2 * I;
  const int ow = o0 + wave * 32 * BRB;        // this wave's first output column
  const bool active = ow < I;                 // I % 64 == 0: a wave's 64 columns are all in or out
  uint8_t* ast = lds + wave * 12288;          // a strip: 32 rows x 64 bf16 (128-byte rows)
  uint8_t* hst = ast + 4096;                  // h / dh strip: 32 rows x 128 bf16 (256-byte rows)
  float* red = reinterpret_cast<float*>(lds + BW * 12288);   // [BW][MT]
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    float dwp = 0.0f;
    if (active && tb * 32 < tl.rows) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = it * 8 + (lane >> 3), c = lane & 7;
        const int64_t p = tl.row0 + min(tb * 32 + r, tl.rows - 1);
        *reinterpret_cast<u32x4*>(ast + stg_off<128>(r, c)) =
            *reinterpret_cast<const u32x4*>(asv + p * I + ow + 8 * c);
      }
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = it * 4 + (lane >> 4), c = lane & 15;
        const int64_t p = tl.row0 + min(tb * 32 + r, tl.rows - 1);
        *reinterpret_cast<u32x4*>(hst + stg_off<256>(r, c)) =
            *reinterpret_cast<const u32x4*>(hsv + p * N2 + 2 * ow + 8 * c);
      }
      const float wf = topk_w[sorted_rows[tl.row0 + min(tb * 32 + l32, tl.rows - 1)]];
      wave_lds_sync();
#pragma unroll
      for (int rb = 0; rb < BRB; ++rb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c4 = 8 * rb + 2 * q + hlf;    // columns 4 c4 .. 4 c4 + 3 of the strip
          const u32x2 av = *reinterpret_cast<const u32x2*>(ast + stg_off<128>(l32, c4 >> 1) + 8 * (c4 & 1));
          uint8_t* hp = hst + stg_off<256>(l32, c4);
          const u32x4 hv = *reinterpret_cast<const u32x4*>(hp);
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
          *reinterpret_cast<u32x4*>(hp) = out;
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = it * 4 + (lane >> 4), c = lane & 15;
        const int rt = tb * 32 + r;
        const u32x4 v = *reinterpret_cast<const u32x4*>(hst + stg_off<256>(r, c));
        if (rt < tl.rows) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dh + (int64_t)(tl.row0 + rt) * N2 + 2 * ow + 8 * c));
      }
      wave_lds_sync();
      if (tb * 32 + l32 >= tl.rows) dwp = 0.0f;
    }
    dwp += __shfl_xor(dwp, 32);
    if (hlf == 0) red[wave * MT + tb * 32 + l32] = dwp;
  }
  __syncthreads();
  if (tid < tl.rows) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < BW; ++w) s += red[w * MT + tid];
    const int64_t f = sorted_rows[tl.row0 + tid];
    dw_part[f * otiles + ot] = s;
  }
}

__global__ __launch_bounds__(BTHR) void bwd_gate_up_kernel(
    const uint16_t* __restrict__ dh, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const int32_t* __restrict__ sorted_rows,
    const Tile* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int H, int I,
    uint16_t* __restrict__ dxr) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[BLDS];
  int mt, ot;
  const int otiles = (H + BNT - 1) / BNT;
  if (!xcd_work_item(*num_tiles, otiles, &mt, &ot)) return;
  const Tile tl = tiles[mt];
  const int o0 = ot * BNT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int e = tl.expert;
  const int N2 = 2 * I;

  const uint16_t* brow[BPPT];
#pragma unroll
  for (int j = 0; j < BPPT; ++j) {
    const int q = tid + j * BTHR;
    const int r = q >> 3;
    brow[j] = dh + (int64_t)(tl.row0 + (r < tl.rows ? r : 0)) * N2 + (q & 7) * 8;
  }
  // Wgu is stored [2I rows][H cols]: contraction over n (C = 2I), output h (O = H)
  const uint8_t* wcode = codes + (int64_t)e * N2 * (H / 2);
  const uint8_t* wscale = scales + (int64_t)e * N2 * (H / 32);
  f32x16 acc[BRB][4];
  bwd_mainloop(brow, wcode, wscale, N2, H, o0, (tl.rows + 31) / 32, lds, acc);

  // Epilogue through LDS (the main loop ended with a barrier).
  const int ow = o0 + wave * 32 * BRB;
  if (ow >= H) return;                        // H % 64 == 0: a wave's columns are all in or out
  uint8_t* yst = lds + wave * 4096;           // 32 rows x 64 bf16 (128-byte rows)
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    if (tb * 32 >= tl.rows) break;
    const int32_t f = sorted_rows[tl.row0 + min(tb * 32 + l32, tl.rows - 1)];
#pragma unroll
    for (int rb = 0; rb < BRB; ++rb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x16& a = acc[rb][tb];
        const u32x2 v = {pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
        *reinterpret_cast<u32x2*>(yst + stg_off<128>(l32, 4 * rb + q) + 8 * hlf) = v;
      }
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = it * 8 + (lane >> 3), c = lane & 7;
      const int rt = tb * 32 + r;
      const int64_t fr = __shfl(f, r);
      const u32x4 v = *reinterpret_cast<const u32x4*>(yst + stg_off<128>(r, c));
      if (rt < tl.rows) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dxr + fr * H + ow + 8 * c));
    }
    wave_lds_sync();
  }
}

// One workgroup (256 threads) per token.  Slot j's dw = the sum of its
// column-tile partials (in tile order) + dY . bd[e_j] (a fixed-order block
// reduction); then dX[t] = sum_j dxr[(t,j)] + dl_j Wr[e_j].  The bias dot
// reads dY and the slots' bias rows in 16-byte pieces, one batch of k + 1
// loads per piece (2-byte loads in a "load, use" loop paid a memory round
// trip per element group), and the dw partials go through LDS.
template <int K>
__global__ __launch_bounds__(256) void bwd_combine_kernel(
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ dxr,
    const float* __restrict__ dw_part, int n_dw_part, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, const uint16_t* __restrict__ dn_bias,
    const float* __restrict__ router_w, int H, uint16_t* __restrict__ dx) {
  __shared__ float red[4][K];
  __shared__ float dl[K];
  __shared__ int32_t ex[K];
  __shared__ float dwps[K * 20];   // k slots x ceil(I / 256) <= 20 column tiles
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H8 = H / 8;   // 16-byte pieces (8 bf16) per row
  // this thread's first piece of every slot's dxr, loaded before the bias
  // dot so its latency overlaps that phase (index clamped; used only when
  // the piece exists)
  u32x4 v0[K];
#pragma unroll
  for (int j = 0; j < K; ++j)
    v0[j] = reinterpret_cast<const u32x4*>(dxr + (t * K + j) * H)[min(tid, H8 - 1)];
  if (tid < K) ex[tid] = topk_idx[t * K + tid];
  for (int q = tid; q < K * n_dw_part; q += 256) dwps[q] = dw_part[t * K * n_dw_part + q];
  __syncthreads();
  float part[K];
#pragma unroll
  for (int j = 0; j < K; ++j) part[j] = 0.0f;
  if (dn_bias) {
    for (int c = tid; c < H / 8; c += 256) {
      const u32x4 g = reinterpret_cast<const u32x4*>(dy + t * H)[c];
      u32x4 b[K];
#pragma unroll
      for (int j = 0; j < K; ++j) b[j] = reinterpret_cast<const u32x4*>(dn_bias + (int64_t)ex[j] * H)[c];
#pragma unroll
      for (int j = 0; j < K; ++j) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          part[j] += bf16_to_f32((uint16_t)(g[m] & 0xFFFFu)) * bf16_to_f32((uint16_t)(b[j][m] & 0xFFFFu));
          part[j] += bf16_to_f32((uint16_t)(g[m] >> 16)) * bf16_to_f32((uint16_t)(b[j][m] >> 16));
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    float v = part[j];
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) red[wave][j] = v;
  }
  __syncthreads();
  if (tid == 0) {
    float dw[K], w[K], sw = 0.0f;
    for (int j = 0; j < K; ++j) {
      float s = red[0][j] + red[1][j] + red[2][j] + red[3][j];
      for (int q = 0; q < n_dw_part; ++q) s += dwps[j * n_dw_part + q];
      dw[j] = s;
      w[j] = topk_w[t * K + j];
      sw += w[j] * s;
    }
    for (int j = 0; j < K; ++j) dl[j] = w[j] * (dw[j] - sw);
  }
  __syncthreads();
  // dX piece c (8 columns) from the slots' dxr pieces v, in slot order
  auto emit = [&](int c, const u32x4 (&v)[K]) {
    f32x4 r[K][2];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const f32x4* rw = reinterpret_cast<const f32x4*>(router_w + (int64_t)ex[j] * H) + 2 * c;
      r[j][0] = rw[0];
      r[j][1] = rw[1];
    }
    float s[8] = {};
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float d = dl[j];
#pragma unroll
      for (int m = 0; m < 8; ++m)
        s[m] += bf16_to_f32((uint16_t)(v[j][m >> 1] >> (16 * (m & 1)))) + d * r[j][m >> 2][m & 3];
    }
    const u32x4 o = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]), pack_bf16x2(s[4], s[5]),
                     pack_bf16x2(s[6], s[7])};
    reinterpret_cast<u32x4*>(dx + t * H)[c] = o;
  };
  if (tid < H8) emit(tid, v0);
  for (int c = tid + 256; c < H8; c += 256) {
    u32x4 v[K];
#pragma unroll
    for (int j = 0; j < K; ++j) v[j] = reinterpret_cast<const u32x4*>(dxr + (t * K + j) * H)[c];
    emit(c, v);
  }
}

int bwd_down_ntiles(int I) { return (I + BNT - 1) / BNT; }

hipError_t launch_bwd_down(const uint16_t* dy, const uint8_t* codes, const uint8_t* scales,
                           const float* topk_w, const int32_t* sorted_rows, const Tile* tiles,
                           const int32_t* num_tiles, int max_tiles, const uint16_t* h,
                           const uint16_t* a, int H, int I, int k, float alpha, float limit,
                           const uint16_t* lora_At, const float* lora_dvu, uint16_t* dh,
                           float* dw_part, hipStream_t s) {
  if (H % BKC || I % 64) return hipErrorInvalidValue;
  dim3 grid(bwd_down_ntiles(I) * max_tiles);
  if (lora_At)
    hipLaunchKernelGGL(bwd_down_kernel<true>, grid, dim3(BTHR), 0, s, dy, codes, scales, topk_w,
                       sorted_rows, tiles, num_tiles, h, a, H, I, k, alpha, limit, lora_At,
                       lora_dvu, dh, dw_part);
  else
    hipLaunchKernelGGL(bwd_down_kernel<false>, grid, dim3(BTHR), 0, s, dy, codes, scales, topk_w,
                       sorted_rows, tiles, num_tiles, h, a, H, I, k, alpha, limit, lora_At,
                       lora_dvu, dh, dw_part);
  return hipGetLastError();
}

hipError_t launch_bwd_gate_up(const uint16_t* dh, const uint8_t* codes, const uint8_t* scales,
                              const int32_t* sorted_rows, const Tile* tiles,
                              const int32_t* num_tiles, int max_tiles, int H, int I,
                              uint16_t* dxr, hipStream_t s) {
  if ((2 * I) % BKC || H % 64) return hipErrorInvalidValue;
  dim3 grid(((H + BNT - 1) / BNT) * max_tiles);
  hipLaunchKernelGGL(bwd_gate_up_kernel, grid, dim3(BTHR), 0, s, dh, codes, scales, sorted_rows,
                     tiles, num_tiles, H, I, dxr);
  return hipGetLastError();
}

hipError_t launch_bwd_combine(const uint16_t* dy, const uint16_t* dxr, const float* dw_part,
                              int n_dw_part, const int32_t* topk_idx, const float* topk_w,
                              const uint16_t* dn_bias, const float* router_w, int64_t T, int H,
                              int k, uint16_t* dx, hipStream_t s) {
  if (n_dw_part > 20 || H % 8) return hipErrorInvalidValue;
#define BWD_COMBINE(KK)                                                                        \
  case KK:                                                                                     \
    hipLaunchKernelGGL(bwd_combine_kernel<KK>, dim3((unsigned)T), dim3(256), 0, s, dy, dxr,    \
                       dw_part, n_dw_part, topk_idx, topk_w, dn_bias, router_w, H, dx);        \
    break;
  switch (k) {
    BWD_COMBINE(1) BWD_COMBINE(2) BWD_COMBINE(3) BWD_COMBINE(4)
    BWD_COMBINE(5) BWD_COMBINE(6) BWD_COMBINE(7) BWD_COMBINE(8)
    default: return hipErrorInvalidValue;
  }
#undef BWD_COMBINE
  return hipGetLastError();
}

}  // namespace mxmoe
