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
// Tiling.  A workgroup computes MT = 128 routed rows of one expert against
// NT = 64 W weight rows with W waves (FwdShape: W = 8, one 160 KB workgroup
// per CU, for down; W = 4, two 80 KB workgroups per CU, for gate_up); two
// waves per SIMD either way.  Wave w owns weight rows 64w..64w+63 (two
// 32-row MFMA blocks) for all 128 routed rows (four 32-column blocks): 8
// accumulators of 32x32 fp32 (128 accumulation registers).  Each decoded
// weight fragment feeds four MFMAs and each activation fragment read from
// LDS two; the second wave per SIMD hides the other's load and LDS waits
// (measured faster than one wave with four weight blocks).  The product is
// computed transposed, D[n][p] = W[n][:] . X[p][:], so the weights are the
// MFMA A-operand: a lane reads its weight rows straight from global memory
// and decodes the codes in registers with the scaled fp4 -> bf16
// conversion; no weight passes through LDS and no weight is decoded twice.
// The routed activation rows are the B-operand, shared by the workgroup's
// waves through LDS.  The NT x (K/32) UE8M0 scale panel of the workgroup's
// weight rows is one contiguous span of memory; it is copied into LDS once.
//
// Pipeline.  K advances in steps of 64; loads run NST - 1 steps ahead: the
// activations of a step go straight from global memory into one of NST LDS
// stages (the gfx950 global-to-LDS load; no registers), the lane's codes
// into one of NST register slots.  In step c a wave issues the loads of
// step c + NST - 1, runs the MFMAs of step c, waits until its loads of step
// c + 1 have landed, and meets the others at the step's one barrier.  The
// loop is unrolled by NST so every stage and slot has a fixed name; loads
// are never under a branch (rows past the tile or past N are clamped to
// valid rows, their results dropped), so the compiler's own wait counts
// stay exact.
//
// K order inside a step: lane half h (lanes 32h..32h+31) holds the codes of
// elements 32h..32h+31 of its row and feeds elements 32h+8s..32h+8s+7 to MFMA
// sub-step s; the B-operand reads the same elements, so each MFMA contracts
// matching K indices (the hardware pairs A and B by lane group and register
// slot).  An activation row of a stage is 128 bytes = eight 16-byte slots;
// column block g of row r sits in slot g ^ ((r >> 1) & 7), which makes the
// 16 rows a half-wave reads land on 16 distinct bank groups.
//
// In the 32x32 accumulator a lane holds column p = lane % 32 and rows
// 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15: gate/up pairs (2j, 2j+1) sit in
// registers (r, r+1) of the same lane, so the GLU needs no data exchange.
#include "common.hpp"
#include "launch.hpp"

namespace mxmoe {

constexpr int FRB = 2;                 // 32-row weight blocks per wave
constexpr int FKS = 64;                // K per step
constexpr int XSTAGE = MT * FKS * 2;   // bytes of one activation stage (16 KB)

// Workgroup shapes.  W = 8: eight waves (two per SIMD), 512 weight rows,
// four stages, all 160 KB of LDS (one workgroup per CU).  W = 4: four waves,
// 256 weight rows, three stages, 80 KB (two workgroups per CU, so one's
// prologue and epilogue overlap the other's main loop; measured faster for
// gate_up, slower for down).
template <int W>
struct FwdShape {
  static constexpr int NTHR = 64 * W;
  static constexpr int NT = 32 * FRB * W;                 // weight rows per workgroup
  static constexpr int LDS = W == 8 ? 160 * 1024 : 80 * 1024;
  static constexpr int NST = W == 8 ? 4 : 3;              // pipeline stages
  static constexpr int XCH = XSTAGE / 1024 / W;           // 1 KB global-to-LDS chunks per wave per step
  static constexpr int LPS = XCH + FRB;                   // vector loads a lane issues per step
  static constexpr int MAXK = (LDS - NST * XSTAGE) / NT * 32;   // largest K whose scale panel fits
};

__device__ constexpr int vmcnt_imm(int n) { return waitcnt_imm(n, 15); }

// Per-lane pipeline state (the first FwdShape<W>::XCH activation entries
// are used).
constexpr int XCH_MAX = 4;
struct FwdPipe {
  const uint16_t* xbase;           // activations (workgroup-uniform)
  uint32_t xrow[XCH_MAX];          // element offsets of the rows this lane stages
  int xcol[XCH_MAX];               // element offset of its 16-byte slot within a step
  const uint8_t* wbase;            // the expert's codes (workgroup-uniform)
  uint32_t wp[FRB];                // byte offsets of this lane's codes per row block (+ lane half)
  const uint8_t* srow[FRB];        // its scale panel rows in LDS
  uint8_t* xs;                     // LDS stages
  int nsteps;                      // ceil(K / 64)
  int kb32;                        // K / 32: scale bytes per weight row
  int tail;                        // K % 64 == 32: the last step's upper 32 K lie past K
  uint32_t tmask;                  // pieces past K in that step: bit j activation chunk j, bit 8 codes
};

// Loads of step c into stage/slot SL: activations global -> LDS directly,
// codes into registers.
// (codes: u32x4 [NST][FRB], taken as a deduced type)
// In the half last step of a K that is an odd multiple of 32, the pieces
// past K are read from a block of zeros (both MFMA operands exactly 0).
template <int W, int SL, class Codes>
__device__ __forceinline__ void fwd_issue(const FwdPipe& p, Codes& codes, int c) {
  constexpr int XCH = FwdShape<W>::XCH;
  // uniform by construction; read into a scalar so the copies' LDS bases
  // (M0) are formed with scalar instructions
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint16_t* xp[XCH];
  const uint8_t* wp[FRB];
#pragma unroll
  for (int j = 0; j < XCH; ++j) xp[j] = p.xbase + (p.xrow[j] + (uint32_t)(c * FKS + p.xcol[j]));
#pragma unroll
  for (int rb = 0; rb < FRB; ++rb) wp[rb] = p.wbase + (p.wp[rb] + (uint32_t)c * 32);
  if (p.tail && c == p.nsteps - 1) {
#pragma unroll
    for (int j = 0; j < XCH; ++j)
      if (p.tmask & (1u << j)) xp[j] = reinterpret_cast<const uint16_t*>(g_zero64);
#pragma unroll
    for (int rb = 0; rb < FRB; ++rb)
      if (p.tmask & 256u) wp[rb] = g_zero64;
  }
#pragma unroll
  for (int j = 0; j < XCH; ++j)
    __builtin_amdgcn_global_load_lds((gptr_t)xp[j], (lptr_t)(p.xs + SL * XSTAGE + (XCH * wave + j) * 1024),
                                     16, 0, 0);
  // the counted waits below assume this issue order: activations, then codes
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int rb = 0; rb < FRB; ++rb) codes[SL][rb] = gload16(wp[rb]);
}

template <int W, int SL, int NRB, class Codes>
__device__ __forceinline__ void fwd_compute(const FwdPipe& p, Codes& codes, int c,
                                            float (&sc)[FRB], f32x16 (&acc)[FRB][4]) {
  constexpr int NST = FwdShape<W>::NST;
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hlf = lane >> 5;
  const uint8_t* st = p.xs + SL * XSTAGE;
  // Sub-step s's B-operand fragments and decoded weights are double
  // buffered: sub-step s + 1's LDS reads and decodes are issued while the
  // MFMAs of sub-step s run, so neither the LDS latency nor the conversions
  // sit between two MFMAs.  The loads of step c + NST - 1 go out after
  // sub-step 0's MFMAs, so their address arithmetic runs while those
  // MFMAs execute instead of ahead of the step's first one.
  bf16x8 b[2][NRB], a[2][FRB];
  auto read_b = [&](int s, bf16x8(&bb)[NRB]) {
    const int g = 4 * hlf + s;
#pragma unroll
    for (int tb = 0; tb < NRB; ++tb) {
      const int r = tb * 32 + l32;
      bb[tb] = *reinterpret_cast<const bf16x8*>(st + r * 128 + 16 * (g ^ ((r >> 1) & 7)));
    }
  };
  read_b(0, b[0]);
#pragma unroll
  for (int rb = 0; rb < FRB; ++rb) a[0][rb] = as_bf16x8(dequant8_bf16(codes[SL][rb][0], sc[rb]));
  __builtin_amdgcn_sched_barrier(0);
  uint32_t scn[FRB];   // the next step's scale bytes (the panel never changes)
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int cur = s & 1, nxt = cur ^ 1;
    if (s < 3) read_b(s + 1, b[nxt]);
    if (s == 1) {
      const int cn = min(c + 1, p.nsteps - 1);
#pragma unroll
      for (int rb = 0; rb < FRB; ++rb) scn[rb] = p.srow[rb][min(2 * cn + hlf, p.kb32 - 1)];
    }
#pragma unroll
    for (int rb = 0; rb < FRB; ++rb)
#pragma unroll
      for (int tb = 0; tb < NRB; ++tb)
        acc[rb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][rb], b[cur][tb], acc[rb][tb], 0, 0, 0);
    if (s < 3) {
#pragma unroll
      for (int rb = 0; rb < FRB; ++rb)
        a[nxt][rb] = as_bf16x8(dequant8_bf16(codes[SL][rb][s + 1], sc[rb]));
      // issue order: one MFMA, the next sub-step's LDS reads, then each
      // further MFMA followed by its share of the next sub-step's conversions
      constexpr int NM = FRB * NRB, NV = 4 * FRB;
      constexpr int PER = (NV + NM - 2) / (NM > 1 ? NM - 1 : 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (s == 1)
        __builtin_amdgcn_sched_group_barrier(0x100, NRB + FRB, 0);
      else
        __builtin_amdgcn_sched_group_barrier(0x100, NRB, 0);
#pragma unroll
      for (int i = 1; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if ((i - 1) * PER < NV) __builtin_amdgcn_sched_group_barrier(0x002, PER, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (s == 0) {
      // the loads of step c + NST - 1 into the slot step c - 1 used (every
      // wave passed the barrier after it)
      fwd_issue<W, (SL + NST - 1) % NST>(p, codes, min(c + NST - 1, p.nsteps - 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int rb = 0; rb < FRB; ++rb) sc[rb] = scale_operand(scn[rb]);
}

// One pipeline step: compute step c (which issues step c + NST - 1 after
// its first sub-step), wait for this wave's loads of step c + 1, barrier.
// A lane issues LPS vector loads per step (activations first, then codes),
// in step order, so after issuing step c + NST - 1 the loads newer than all
// of step c + 1's number LPS * (NST - 2).  Waiting for step c + 1's codes
// too (not only its activations) keeps the compiler's own wait for the
// code registers from falling back to a full drain at the top of the
// unrolled loop.
template <int W, int SL, int NRB, class Codes>
__device__ __forceinline__ void fwd_step(const FwdPipe& p, Codes& codes, int c, float (&sc)[FRB],
                                         f32x16 (&acc)[FRB][4]) {
  constexpr int NST = FwdShape<W>::NST;
  fwd_compute<W, SL, NRB>(p, codes, c, sc, acc);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(FwdShape<W>::LPS * (NST - 2)));
  barrier_only();
}

template <int W, int NRB>
__device__ __forceinline__ void fwd_loop(const FwdPipe& p, f32x16 (&acc)[FRB][4]) {
  constexpr int NST = FwdShape<W>::NST;
  static_assert(NST == 3 || NST == 4, "the main loop is unrolled for 3 or 4 stages");
  u32x4 codes[NST][FRB];
  const int last = p.nsteps - 1;
  // The prologue's loads must stay in issue order ahead of the wait: the
  // compiler may otherwise sink the register loads below it, and the count
  // would then release before stage 0 has landed.
  __builtin_amdgcn_sched_barrier(0);
  fwd_issue<W, 0>(p, codes, 0);
  __builtin_amdgcn_sched_barrier(0);
  fwd_issue<W, 1>(p, codes, min(1, last));
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NST == 4) {
    fwd_issue<W, 2>(p, codes, min(2, last));
    __builtin_amdgcn_sched_barrier(0);
  }
  // the scale panel was written with ordinary LDS stores
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(FwdShape<W>::LPS * (NST - 2), 0));
  barrier_only();
  const int hlf = (threadIdx.x & 63) >> 5;
  float sc[FRB];
#pragma unroll
  for (int rb = 0; rb < FRB; ++rb) sc[rb] = scale_operand(p.srow[rb][min(hlf, p.kb32 - 1)]);
  int c = 0;
  for (; c + NST <= p.nsteps; c += NST) {
    fwd_step<W, 0, NRB>(p, codes, c + 0, sc, acc);
    fwd_step<W, 1, NRB>(p, codes, c + 1, sc, acc);
    fwd_step<W, 2, NRB>(p, codes, c + 2, sc, acc);
    if constexpr (NST == 4) fwd_step<W, 3, NRB>(p, codes, c + 3, sc, acc);
  }
  const int rem = p.nsteps - c;
  if (rem > 0) fwd_step<W, 0, NRB>(p, codes, c + 0, sc, acc);
  if (rem > 1) fwd_step<W, 1, NRB>(p, codes, c + 1, sc, acc);
  if constexpr (NST == 4)
    if (rem > 2) fwd_step<W, 2, NRB>(p, codes, c + 2, sc, acc);
  // drain: nothing may still be writing LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

// Shared body of both forward GEMMs up to the accumulators.  xrow[j]: the
// activation row this lane stages for chunk j (clamped to the tile's first
// row past the tile).  wrow_local: first weight row of this lane within the
// workgroup's rows (row blocks follow 32 rows apart; clamped for waves past
// N).
template <int W>
__device__ __forceinline__ void fwd_body(const uint16_t* xbase, const uint32_t* xrow,
                                         const uint8_t* __restrict__ codes_e,
                                         const uint8_t* __restrict__ scales_e, int K, int n0,
                                         int nrows, int wrow_local, int nrb, uint8_t* lds,
                                         f32x16 (&acc)[FRB][4]) {
  constexpr int XCH = FwdShape<W>::XCH;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hlf = lane >> 5;
  uint8_t* panel = lds + FwdShape<W>::NST * XSTAGE;
  const int KB32 = K / 32;

  // scale panel: nrows * K/32 contiguous bytes, 16-byte aligned
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(scales_e + (int64_t)n0 * KB32);
    u32x4* dst = reinterpret_cast<u32x4*>(panel);
    stage_lds<6>(nrows * KB32 / 16, tid, FwdShape<W>::NTHR, [&](int q) { return src[q]; },
                 [&](int q, u32x4 v) { dst[q] = v; });
  }
#pragma unroll
  for (int rb = 0; rb < FRB; ++rb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][tb][r] = 0.0f;

  static_assert(XCH <= XCH_MAX, "activation chunks per wave");
  FwdPipe p;
  p.tmask = hlf ? 256u : 0u;
#pragma unroll
  for (int j = 0; j < XCH; ++j) {
    const int row = (XCH * wave + j) * 8 + lane / 8;   // row of the tile this lane stages
    const int blk = (lane & 7) ^ ((row >> 1) & 7);     // global column block of its slot
    p.xrow[j] = xrow[j];
    p.xcol[j] = 8 * blk;
    if (blk >= 4) p.tmask |= 1u << j;
  }
  const int64_t rowbytes = K / 2;
  // row blocks past the workgroup's rows (the last column tile can hold
  // fewer than 128 rows per wave) read its last row; their results are dropped
#pragma unroll
  for (int rb = 0; rb < FRB; ++rb) {
    const int r = min(wrow_local + 32 * rb, nrows - 1);
    p.wp[rb] = (uint32_t)(n0 + r) * (uint32_t)rowbytes + hlf * 16;
    p.srow[rb] = panel + r * KB32;
  }
  p.xbase = xbase;
  p.wbase = codes_e;
  p.xs = lds;
  p.nsteps = (K + FKS - 1) / FKS;
  p.kb32 = KB32;
  p.tail = (K % FKS) != 0;
  switch (nrb) {
    case 1: fwd_loop<W, 1>(p, acc); break;
    case 2: fwd_loop<W, 2>(p, acc); break;
    case 3: fwd_loop<W, 3>(p, acc); break;
    default: fwd_loop<W, 4>(p, acc); break;
  }
}

// The bias of a lane's accumulator rows, rb * 32 + 8 q + i (i < 4) from
// base: four consecutive bf16 per (rb, q), one 8-byte load each (base is a
// multiple of 4 elements and the bias 16-byte aligned); zeros without bias.
__device__ __forceinline__ void load_bias_rows(const uint16_t* __restrict__ bias, int64_t base,
                                               int nblk, float (&bv)[FRB][4][4]) {
  u32x2 raw[FRB][4];
#pragma unroll
  for (int rb = 0; rb < FRB; ++rb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      raw[rb][q] = (bias && rb < nblk) ? *reinterpret_cast<const u32x2*>(bias + base + rb * 32 + 8 * q)
                                       : u32x2{0u, 0u};
#pragma unroll
  for (int rb = 0; rb < FRB; ++rb)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bv[rb][q][i] = bf16_to_f32((uint16_t)(raw[rb][q][i >> 1] >> (16 * (i & 1))));
}

// + s v B_e^T, an adapter's rank-r delta, into the accumulators: 16-deep
// contractions over the rank, A-operand = B_e rows (this lane's weight
// rows, [N, r] per expert), B-operand = s v as hi + lo bf16 (v [R, r] in
// sorted order); one token block at a time to keep few registers live.
__device__ __forceinline__ void lora_delta(f32x16 (&acc)[FRB][4], const Tile& tl, int e, int N,
                                           int n0, int nrows, int wrow_local,
                                           const uint16_t* __restrict__ lora_B,
                                           const float* __restrict__ lora_v, float lora_scale,
                                           int lora_r) {
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hlf = lane >> 5;
  for (int j = 0; j < lora_chunks(lora_r); ++j) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      bf16x8 vh, vl;
      lora_frag_split(lora_v + (int64_t)(tl.row0 + min(tb * 32 + l32, tl.rows - 1)) * lora_r,
                      lora_r, j, hlf, lora_scale, &vh, &vl);
#pragma unroll
      for (int rb = 0; rb < FRB; ++rb) {
        const int r = min(wrow_local + 32 * rb, nrows - 1);
        const bf16x8 bw = lora_frag(lora_B + ((int64_t)e * N + n0 + r) * lora_r, lora_r, j, hlf);
        acc[rb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw, vh, acc[rb][tb], 0, 0, 0);
        acc[rb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw, vl, acc[rb][tb], 0, 0, 0);
      }
    }
  }
}

// The gate_up epilogue (after a barrier that frees LDS): bias, the saved
// pre-activation h (when h_out) and the clamped SwiGLU a, through a private
// LDS strip per wave, stored as whole row pieces.  acc: this wave's 64
// weight rows (wcol = 64 w) by the tile's routed rows.
__device__ __forceinline__ void gate_up_epilogue(const f32x16 (&acc)[FRB][4], const Tile& tl, int e,
                                                 int N, int n0, int I,
                                                 const uint16_t* __restrict__ bias, float alpha,
                                                 float limit, uint8_t* lds,
                                                 uint16_t* __restrict__ h_out,
                                                 uint16_t* __restrict__ a_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int wcol = wave * 32 * FRB;           // this wave's first weight row in the tile
  if (n0 + wcol >= N) return;                 // N % 64 == 0: a wave's 64 rows are all in or all out
  uint8_t* hst = lds + wave * 6144;           // h strip: 32 rows x 64 bf16 (128-byte rows)
  uint8_t* ast = hst + 4096;                  // a strip: 32 rows x 32 bf16 (64-byte rows)
  float bv[FRB][4][4];
  load_bias_rows(bias, (int64_t)e * N + n0 + wcol + 4 * hlf, FRB, bv);
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    if (tb * 32 >= tl.rows) break;
#pragma unroll
    for (int rb = 0; rb < FRB; ++rb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float g0 = acc[rb][tb][4 * q + 0] + bv[rb][q][0];
        const float u0 = acc[rb][tb][4 * q + 1] + bv[rb][q][1];
        const float g1 = acc[rb][tb][4 * q + 2] + bv[rb][q][2];
        const float u1 = acc[rb][tb][4 * q + 3] + bv[rb][q][3];
        if (h_out) {
          u32x2 hv = {saved_preact_bf16(g0, limit, false) | (saved_preact_bf16(u0, limit, true) << 16),
                      saved_preact_bf16(g1, limit, false) | (saved_preact_bf16(u1, limit, true) << 16)};
          *reinterpret_cast<u32x2*>(hst + stg_off<128>(l32, 4 * rb + q) + 8 * hlf) = hv;
        }
        // a columns 16 rb + 4 q + 2 hlf, +1
        *reinterpret_cast<uint32_t*>(ast + stg_off<64>(l32, 2 * rb + (q >> 1)) + 8 * (q & 1) + 4 * hlf) =
            pack_bf16x2(swiglu(g0, u0, alpha, limit), swiglu(g1, u1, alpha, limit));
      }
    wave_lds_sync();
    if (h_out) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = it * 8 + (lane >> 3), c = lane & 7;
        const int rt = tb * 32 + r;
        const u32x4 v = *reinterpret_cast<const u32x4*>(hst + stg_off<128>(r, c));
        if (rt < tl.rows)
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(h_out + (int64_t)(tl.row0 + rt) * N + n0 + wcol + 8 * c));
      }
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int r = it * 16 + (lane >> 2), c = lane & 3;
      const int rt = tb * 32 + r;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ast + stg_off<64>(r, c));
      if (rt < tl.rows)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(a_out + (int64_t)(tl.row0 + rt) * I + (n0 + wcol) / 2 + 8 * c));
    }
    wave_lds_sync();
  }
}

// Two waves per SIMD in either shape (amdgpu_waves_per_eu keeps the W = 4
// kernel within the registers of two waves, so two workgroups fit a CU).
// LORA: add the gate_up adapter's rank-r delta s (vg B_gu^T) before the
// bias, as the down GEMM adds its adapter's.
template <int W, bool LORA>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 2))) void gate_up_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const uint16_t* __restrict__ bias,
    const int32_t* __restrict__ sorted_rows, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int H, int I, int k, float alpha, float limit,
    const uint16_t* __restrict__ lora_B, const float* __restrict__ lora_v, float lora_scale,
    int lora_r, uint16_t* __restrict__ h_out, uint16_t* __restrict__ a_out) {
  using S = FwdShape<W>;
  constexpr int XCHUNKS = S::XCH, FNT = S::NT;
  __shared__ __attribute__((aligned(16))) uint8_t lds[S::LDS];
  const int N = 2 * I;
  Tile tl;
  int nt;
  if (!xcd_item_range(tiles, num_tiles, (N + FNT - 1) / FNT, &tl, &nt)) return;
  const int n0 = nt * FNT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int e = tl.expert;

  uint32_t xrow[XCHUNKS];   // element offsets into x (T * H < 2^31)
#pragma unroll
  for (int j = 0; j < XCHUNKS; ++j) {
    const int r = (XCHUNKS * wave + j) * 8 + lane / 8;
    const int f = sorted_rows[tl.row0 + (r < tl.rows ? r : 0)];
    xrow[j] = (uint32_t)(f / k) * (uint32_t)H;
  }
  const int nrows = min(FNT, N - n0);
  f32x16 acc[FRB][4];
  const int wrow_local = (wave * 32 * FRB < nrows ? wave * 32 * FRB : 0) + l32;
  fwd_body<W>(x, xrow, codes + (int64_t)e * N * (H / 2), scales + (int64_t)e * N * (H / 32), H, n0,
           nrows, wrow_local, (tl.rows + 31) / 32, lds, acc);
  if (LORA) lora_delta(acc, tl, e, N, n0, nrows, wrow_local, lora_B, lora_v, lora_scale, lora_r);
  // Epilogue through LDS: every wave's loads have landed (fwd_loop drained
  // them) and every wave is past its last stage read.
  barrier_only();
  gate_up_epilogue(acc, tl, e, N, n0, I, bias, alpha, limit, lds, h_out, a_out);
}

// Block-scaled variant of gate_up: the gfx950 scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4) takes the packed FP4 weight codes and
// their UE8M0 scales as they are stored, and the token rows quantized to
// MXFP8 (E4M3 codes, UE8M0 per 32; NH = 2: a hi and a lo pass, x ~ hi +
// lo) -- the pages' activation_format None (activations in the weights'
// block-scaled family) next to the weight-only bf16 path above.  No weight
// is decoded: an MFMA contracts 64 K; a lane of half h (lanes 32h..32h+31)
// holds its row's scale of K block h (K 32h..32h+31) and, for a weight
// row, that block's 32 FP4 codes (16 bytes straight from global memory).
// Paired with 4-bit elements, the FP8 operand of half h holds K 16h..16h+15
// and 32+16h..32+16h+15 of its routed row (two 16-byte LDS chunks): the
// layout found by one-hot probes of the instruction.
// Tile: 128 routed rows x 256 weight rows, four waves of 64 weight rows (two
// 32-row MFMA blocks) by the four 32-row blocks of routed rows; the same
// accumulator layout and epilogue as gate_up_kernel.  K % 64 == 0.
constexpr int MX_XB = MT * 64;                 // one pass's codes per stage (8 KB)
constexpr int MX_SB = MT * 2;                  // its scale bytes (2 blocks per row)

typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int NH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void mx_gate_up_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
    const uint8_t* __restrict__ xq_lo, const uint8_t* __restrict__ xs_lo,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ bias, const int32_t* __restrict__ sorted_rows,
    const Tile* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int H, int I, int k,
    float alpha, float limit, uint16_t* __restrict__ h_out, uint16_t* __restrict__ a_out) {
  constexpr int NT = 256;
  constexpr int MX_PD = NH == 1 ? 3 : 2;        // weight steps in flight per lane
  constexpr int STAGE = NH * (MX_XB + MX_SB);
  constexpr int LDSB = 2 * STAGE > 4 * 6144 ? 2 * STAGE : 4 * 6144;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDSB];
  const int N = 2 * I;
  Tile tl;
  int nt;
  if (!xcd_item_range(tiles, num_tiles, (N + NT - 1) / NT, &tl, &nt)) return;
  const int n0 = nt * NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int e = tl.expert;
  const int nsteps = H / 64, KB = H / 32;
  // weight rows of this lane's two MFMA blocks (rows past N read row N - 1)
  const uint8_t* wrow[FRB];
  const uint8_t* srow[FRB];
#pragma unroll
  for (int rb = 0; rb < FRB; ++rb) {
    const int n = min(n0 + wave * 64 + 32 * rb + l32, N - 1);
    wrow[rb] = codes + ((int64_t)e * N + n) * (H / 2) + 16 * hlf;
    srow[rb] = scales + ((int64_t)e * N + n) * KB + hlf;
  }
  // staging: thread = (tile row r, 32-byte half hh) of each pass's 64-byte step row
  const int r = tid >> 1, hh = tid & 1;
  const int64_t tok = sorted_rows[tl.row0 + min(r, tl.rows - 1)] / k;
  const uint8_t* xsrc[NH];
  const uint8_t* ssrc[NH];
  xsrc[0] = xq + tok * H + 32 * hh;
  ssrc[0] = xs + tok * KB;
  if constexpr (NH == 2) {
    xsrc[1] = xq_lo + tok * H + 32 * hh;
    ssrc[1] = xs_lo + tok * KB;
  }
  // LDS row r of a pass: four 16-byte chunks, chunk c at c ^ ((r / 4) % 4)
  auto chunk_off = [](int row, int c) { return row * 64 + 16 * (c ^ ((row >> 2) & 3)); };

  u32x4 xr[NH][2];
  uint32_t sr[NH];
  auto load_act = [&](int c) {
#pragma unroll
    for (int h2 = 0; h2 < NH; ++h2) {
      xr[h2][0] = *reinterpret_cast<const u32x4*>(xsrc[h2] + 64 * c);
      xr[h2][1] = *reinterpret_cast<const u32x4*>(xsrc[h2] + 64 * c + 16);
      sr[h2] = hh == 0 ? *reinterpret_cast<const uint16_t*>(ssrc[h2] + 2 * c) : 0u;
    }
  };
  auto stage_act = [&](uint8_t* st) {
#pragma unroll
    for (int h2 = 0; h2 < NH; ++h2) {
      uint8_t* base = st + h2 * (MX_XB + MX_SB);
      *reinterpret_cast<u32x4*>(base + chunk_off(r, 2 * hh)) = xr[h2][0];
      *reinterpret_cast<u32x4*>(base + chunk_off(r, 2 * hh + 1)) = xr[h2][1];
      if (hh == 0) *reinterpret_cast<uint16_t*>(base + MX_XB + 2 * r) = (uint16_t)sr[h2];
    }
  };
  // the lane's weight codes and scales MX_PD steps ahead: ring slot j
  // holds step c with c % MX_PD == j (the step loop is unrolled by MX_PD,
  // so slots are never moved while their loads are in flight)
  u32x4 wq[MX_PD][FRB];
  uint32_t wsq[MX_PD][FRB];
  auto load_w = [&](int c, u32x4 (&wa)[FRB], uint32_t (&wsc)[FRB]) {
#pragma unroll
    for (int rb = 0; rb < FRB; ++rb) {
      wa[rb] = *reinterpret_cast<const u32x4*>(wrow[rb] + 32 * c);
      wsc[rb] = srow[rb][2 * c];
    }
  };

  f32x16 acc[FRB][4];
#pragma unroll
  for (int rb = 0; rb < FRB; ++rb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[rb][tb][q] = 0.0f;

  auto step = [&](int c, const u32x4 (&wa)[FRB], const uint32_t (&wsc)[FRB]) {
    const uint8_t* st = lds + (c & 1) * STAGE;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      if (tb * 32 >= tl.rows) break;
      const int p = tb * 32 + l32;
#pragma unroll
      for (int h2 = 0; h2 < NH; ++h2) {
        const uint8_t* base = st + h2 * (MX_XB + MX_SB);
        const u32x4 b0 = *reinterpret_cast<const u32x4*>(base + chunk_off(p, hlf));
        const u32x4 b1 = *reinterpret_cast<const u32x4*>(base + chunk_off(p, hlf + 2));
        const i32x8 bop = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                           (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
        const int sb = base[MX_XB + 2 * p + hlf];
#pragma unroll
        for (int rb = 0; rb < FRB; ++rb) {
          const i32x8 aop = {(int)wa[rb][0], (int)wa[rb][1], (int)wa[rb][2], (int)wa[rb][3],
                             0, 0, 0, 0};
          // A = FP4 weights (format 4), B = FP8 E4M3 activations (format 0)
          acc[rb][tb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              aop, bop, acc[rb][tb], 4, 0, 0, (int)wsc[rb], 0, sb);
        }
        if (NH > 1) __builtin_amdgcn_sched_barrier(0);
      }
      // one routed-row block's operands live at a time
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  load_act(0);
#pragma unroll
  for (int j = 0; j < MX_PD; ++j) load_w(min(j, nsteps - 1), wq[j], wsq[j]);
  stage_act(lds);
  if (nsteps > 1) load_act(1);
  __syncthreads();
  // steps past nsteps (the last group's tail) compute nothing; their weight
  // loads re-read the last step, in bounds
  for (int c0 = 0; c0 < nsteps; c0 += MX_PD) {
#pragma unroll
    for (int j = 0; j < MX_PD; ++j) {
      const int c = c0 + j;
      if (c < nsteps) step(c, wq[j], wsq[j]);
      load_w(min(c + MX_PD, nsteps - 1), wq[j], wsq[j]);
      if (c + 1 < nsteps) {
        stage_act(lds + ((c + 1) & 1) * STAGE);
        if (c + 2 < nsteps) load_act(c + 2);
      }
      __syncthreads();
    }
  }
  gate_up_epilogue(acc, tl, e, N, n0, I, bias, alpha, limit, lds, h_out, a_out);
}

hipError_t launch_mx_gate_up(const uint8_t* xq, const uint8_t* xs, const uint8_t* xq_lo,
                             const uint8_t* xs_lo, const uint8_t* codes, const uint8_t* scales,
                             const uint16_t* bias, const int32_t* sorted_rows, const Tile* tiles,
                             const int32_t* num_tiles, int max_tiles, int H, int I, int k,
                             float alpha, float limit, uint16_t* h_out, uint16_t* a_out,
                             hipStream_t s) {
  if (H % 64 || I % 32) return hipErrorInvalidValue;
  const dim3 grid(((2 * I + 255) / 256) * max_tiles), block(256);
  if (xq_lo)
    hipLaunchKernelGGL(mx_gate_up_kernel<2>, grid, block, 0, s, xq, xs, xq_lo, xs_lo, codes, scales,
                       bias, sorted_rows, tiles, num_tiles, H, I, k, alpha, limit, h_out, a_out);
  else
    hipLaunchKernelGGL(mx_gate_up_kernel<1>, grid, block, 0, s, xq, xs, xq_lo, xs_lo, codes, scales,
                       bias, sorted_rows, tiles, num_tiles, H, I, k, alpha, limit, h_out, a_out);
  return hipGetLastError();
}

// LORA: add the rank-r delta s (v B_e^T) (a template parameter: a runtime
// branch around these MFMAs makes the compiler spill accumulators inside
// the main loop).
template <bool LORA>
__global__ __launch_bounds__(FwdShape<8>::NTHR) void down_kernel(
    const uint16_t* __restrict__ a, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const uint16_t* __restrict__ bias,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_rows,
    const Tile* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int H, int I,
    const uint16_t* __restrict__ lora_B, const float* __restrict__ lora_v, float lora_scale,
    int lora_r, uint16_t* __restrict__ y_w) {
  using S = FwdShape<8>;
  constexpr int XCHUNKS = S::XCH, FNT = S::NT;
  __shared__ __attribute__((aligned(16))) uint8_t lds[S::LDS];
  const int N = H;
  Tile tl;
  int nt;
  if (!xcd_item_range(tiles, num_tiles, (N + FNT - 1) / FNT, &tl, &nt)) return;
  const int n0 = nt * FNT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int e = tl.expert;

  uint32_t xrow[XCHUNKS];   // element offsets from the tile's first row of a
#pragma unroll
  for (int j = 0; j < XCHUNKS; ++j) {
    const int r = (XCHUNKS * wave + j) * 8 + lane / 8;
    xrow[j] = (uint32_t)(r < tl.rows ? r : 0) * (uint32_t)I;
  }
  const int nrows = min(FNT, N - n0);
  f32x16 acc[FRB][4];
  const int wrow_local = (wave * 32 * FRB < nrows ? wave * 32 * FRB : 0) + l32;
  fwd_body<8>(a + (int64_t)tl.row0 * I, xrow, codes + (int64_t)e * N * (I / 2), scales + (int64_t)e * N * (I / 32), I, n0,
           nrows, wrow_local, (tl.rows + 31) / 32, lds, acc);
  if (LORA) lora_delta(acc, tl, e, N, n0, nrows, wrow_local, lora_B, lora_v, lora_scale, lora_r);
  barrier_only();   // as in gate_up: LDS is free for the epilogue
  const int wcol = wave * 32 * FRB;
  if (n0 + wcol >= N) return;
  // N % 32 == 0: the wave's second 32-row block may lie past N
  const int nblk = min(FRB, (N - n0 - wcol) / 32);
  uint8_t* yst = lds + wave * 4096;           // y strip: 32 rows x 64 bf16 (128-byte rows)
  float bv[FRB][4][4];
  load_bias_rows(bias, (int64_t)e * N + n0 + wcol + 4 * hlf, nblk, bv);
  // the row blocks' flat rows and routing weights for this lane: one batch
  // of loads each (not a dependent pair per block)
  int32_t fv[4];
  float wfv[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) fv[tb] = sorted_rows[tl.row0 + min(tb * 32 + l32, tl.rows - 1)];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) wfv[tb] = topk_w[fv[tb]];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    if (tb * 32 >= tl.rows) break;
    const int32_t f = fv[tb];
    const float wf = wfv[tb];
#pragma unroll
    for (int rb = 0; rb < FRB; ++rb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = wf * (acc[rb][tb][4 * q + i] + bv[rb][q][i]);
        const u32x2 yv = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        *reinterpret_cast<u32x2*>(yst + stg_off<128>(l32, 4 * rb + q) + 8 * hlf) = yv;
      }
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = it * 8 + (lane >> 3), c = lane & 7;
      const int rt = tb * 32 + r;
      const int64_t fr = __shfl(f, r);
      const u32x4 v = *reinterpret_cast<const u32x4*>(yst + stg_off<128>(r, c));
      if (rt < tl.rows && 8 * c < 32 * nblk)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(y_w + fr * N + n0 + wcol + 8 * c));
    }
    wave_lds_sync();
  }
}

// out[t, :] = sum_j y_w[t*k + j, :] in slot order, summed in fp32 and
// rounded once to bf16 (K = k, a template parameter, so the slot loop
// unrolls without guards).  y_w holds each slot's weighted output in bf16.
// Each thread takes one 16-byte piece (8 columns) of a token's row.
template <int K>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y_w, int64_t n8,
                                                      int H8, uint16_t* __restrict__ out) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  int64_t t = i / H8, c = i % H8;
  const u32x4* src = reinterpret_cast<const u32x4*>(y_w) + t * K * H8 + c;
  u32x4 v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) v[j] = src[(int64_t)j * H8];
  float s[8] = {};
#pragma unroll
  for (int j = 0; j < K; ++j)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      s[2 * m] += bf16_to_f32((uint16_t)(v[j][m] & 0xFFFFu));
      s[2 * m + 1] += bf16_to_f32((uint16_t)(v[j][m] >> 16));
    }
  const u32x4 o = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]), pack_bf16x2(s[4], s[5]),
                   pack_bf16x2(s[6], s[7])};
  reinterpret_cast<u32x4*>(out)[i] = o;
}

// K step of the forward GEMMs for a contraction length K (0: unsupported).
int fwd_step_k(int K) { return (K % 32 == 0 && K <= FwdShape<8>::MAXK) ? FKS : 0; }

hipError_t launch_gate_up(const uint16_t* x, const uint8_t* codes, const uint8_t* scales,
                          const uint16_t* bias, const int32_t* sorted_rows, const Tile* tiles,
                          const int32_t* num_tiles, int max_tiles, int H, int I, int k,
                          float alpha, float limit, const uint16_t* lora_B, const float* lora_v,
                          float lora_scale, int lora_r, uint16_t* h_out, uint16_t* a_out,
                          hipStream_t s) {
  if (!fwd_step_k(H) || (lora_B && !lora_rank_ok(lora_r))) return hipErrorInvalidValue;
#define GATE_UP(W, LORA)                                                                         \
  hipLaunchKernelGGL((gate_up_kernel<W, LORA>),                                                  \
                     dim3(((2 * I + FwdShape<W>::NT - 1) / FwdShape<W>::NT) * max_tiles),         \
                     dim3(FwdShape<W>::NTHR), 0, s, x, codes, scales, bias, sorted_rows, tiles,   \
                     num_tiles, H, I, k, alpha, limit, lora_B, lora_v, lora_scale, lora_r, h_out, \
                     a_out)
  if (H <= FwdShape<4>::MAXK) {
    if (lora_B) GATE_UP(4, true); else GATE_UP(4, false);
  } else {
    if (lora_B) GATE_UP(8, true); else GATE_UP(8, false);
  }
#undef GATE_UP
  return hipGetLastError();
}

hipError_t launch_down(const uint16_t* a, const uint8_t* codes, const uint8_t* scales,
                       const uint16_t* bias, const float* topk_w, const int32_t* sorted_rows,
                       const Tile* tiles, const int32_t* num_tiles, int max_tiles, int H, int I,
                       const uint16_t* lora_B, const float* lora_v, float lora_scale, int lora_r,
                       uint16_t* y_w, hipStream_t s) {
  if (!fwd_step_k(I) || (lora_B && !lora_rank_ok(lora_r))) return hipErrorInvalidValue;
  using S = FwdShape<8>;
  dim3 grid(((H + S::NT - 1) / S::NT) * max_tiles), block(S::NTHR);
  if (lora_B)
    hipLaunchKernelGGL(down_kernel<true>, grid, block, 0, s, a, codes, scales, bias, topk_w,
                       sorted_rows, tiles, num_tiles, H, I, lora_B, lora_v, lora_scale, lora_r,
                       y_w);
  else
    hipLaunchKernelGGL(down_kernel<false>, grid, block, 0, s, a, codes, scales, bias, topk_w,
                       sorted_rows, tiles, num_tiles, H, I, lora_B, lora_v, lora_scale, 0, y_w);
  return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* y_w, int64_t T, int H, int k, uint16_t* out,
                          hipStream_t s) {
  if (H % 8) return hipErrorInvalidValue;
  int64_t n8 = T * H / 8;
  const dim3 grid((unsigned)((n8 + 255) / 256));
#define COMBINE(KK)                                                                      \
  case KK:                                                                               \
    hipLaunchKernelGGL(combine_kernel<KK>, grid, dim3(256), 0, s, y_w, n8, H / 8, out);  \
    break;
  switch (k) {
    COMBINE(1) COMBINE(2) COMBINE(3) COMBINE(4) COMBINE(5) COMBINE(6) COMBINE(7) COMBINE(8)
    default: return hipErrorInvalidValue;
  }
#undef COMBINE
  return hipGetLastError();
}

}  // namespace mxmoe
