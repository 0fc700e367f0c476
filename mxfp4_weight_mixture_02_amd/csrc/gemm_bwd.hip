// Backward (dX) grouped expert GEMMs on gfx950 MFMA, over the same packed
// MXFP4 weights the forward reads, contracted over their stored row axis
// ("Add MXFP4 training support via a dequantize-on-the-fly fallback": the
// backward of the frozen base only needs input and adapter gradients; the
// fallback recomputes dequantisation, which here happens in registers right
// before the matrix cores use it).
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
// Both GEMMs compute out[p][o] = sum_c act[p][c] * W[c][o] with W stored
// [C rows][O cols] (codes packed along o, one UE8M0 scale per 32 o): the
// contraction runs along the stored row axis, and the scales vary along the
// output axis.
//
// Weight path.  The workgroup's slice of each 64-row step (64 stored rows x
// 256 columns: 8 KB of packed codes) is copied into LDS as raw bytes, and
// its 64 x 8 scale bytes into a transposed LDS table of words (per scale
// block, a lane's four sub-steps' words side by side, so one 16-byte read
// per step gives a lane its row's scale for every sub-step; the 16 lanes
// that decode the same 8 rows then broadcast them with DPP row_newbcast).  The MFMA A-operand needs
// 8 consecutive c of one output column per lane.  gfx950's 8-bit
// transposing LDS read (ds_read_b64_tr_b8) gives each lane 8 rows x one
// code byte, i.e. 8 consecutive c for the column pair (2m, 2m+1); the lane
// decodes each byte with its own row's scale (one scaled fp4 -> bf16
// conversion per byte, exact) and splits the 8 packed pairs into the even
// and the odd column's fragment with byte permutes.  So the MFMA rows of one
// such fragment pair are the even and the odd columns of a 64-column
// double block, and LDS holds 4 bits per weight instead of 16: a quarter of
// the bytes written and read of a decoded bf16 tile (gfx950's LDS writes run
// at well under half its read rate).
//
// Activation path (the B-operand, contraction-contiguous in memory): each
// step's 128 rows x 64 bf16 (16 KB) are copied into an LDS stage by LDS-DMA
// loads, 16-byte chunks swizzled per row; the MFMA reads them with 16-byte
// LDS reads.
//
// Tiling.  A workgroup is 4 waves (one per SIMD) and computes 128 routed
// rows (one 128-row tile of an expert) x 256 output columns; two
// workgroups share a CU (78 KB of LDS each), so each SIMD interleaves
// waves of two independent workgroups, and a workgroup's barrier only
// meets waves on different SIMDs (with two waves of one workgroup per SIMD
// the one the SIMD favours reached every barrier early and the other
// finished each step alone).  Wave wo owns the 64-column double block wo
// (two MFMA row blocks: its even and its odd columns) and the four 32-row
// blocks of the tile: 8 accumulators of 32 x 32 fp32, 128 registers.
//
// Pipeline (one barrier per 64-deep step k): stage step k + 1's codes,
// scales and activations (loaded during step k - 1) into the other LDS
// stage and reload the registers with step k + 2's; then for each 16-deep
// sub-step the next sub-step's LDS reads, its decode, and this sub-step's
// 16 MFMAs, interleaved; the barrier sits before the last sub-step's MFMAs,
// after which the next step's first reads issue.  Step indices are clamped
// at the end instead of branching around loads; rows past the tile and
// columns past O read valid memory whose products are never stored.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mxmoe {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int GW = 4;                       // waves per workgroup, one per SIMD
constexpr int GTHR = 64 * GW;
constexpr int GO = 256;                     // output columns per workgroup
constexpr int GKC = 64;                     // contraction per step
constexpr int GCB = GKC * (GO / 2);         // code tile per step: 64 rows x 128 bytes (8 KB)
constexpr int GSB = (GO / 32) * GKC * 4;    // scale table per step: 8 blocks x 64 rows, a word each (2 KB)
constexpr int GRB = BMT / 32;               // 32-row blocks per tile (and per wave)
constexpr int GXB = BMT * GKC * 2;          // activation stage
constexpr int GXI = GXB / (1024 * GW);      // activation DMA loads per wave per step
constexpr int GSTAGE = GCB + GSB + GXB;     // one stage
constexpr int GNST = 3;                     // stages in flight
constexpr int GLDS_LOOP = GNST * GSTAGE;    // main loop
constexpr int GDMA = GXI + 4;               // LDS-DMA loads per wave per step
static_assert(BMT == 128 || BMT == 256, "tile rows assumed below");

// Chunk swizzle of activation row p (16-byte chunks; distinct banks for the
// 16-byte reads of 8 and of 16 consecutive rows).
__device__ __forceinline__ int x_swz(int p) { return (p & 7) ^ ((p >> 3) & 1); }

// Per-lane addressing, fixed for the whole main loop (LDS offsets are
// relative to a stage).  Every step's tile is copied global -> LDS by
// LDS-DMA loads: a lane names its source, and the data lands at the
// instruction's LDS base + 16 (or, for a byte, 4) x lane.
struct GArgs {
  const uint16_t* xbase;    // activations (workgroup-uniform)
  uint32_t xoff[GXI];       // element offsets of the activation pieces this lane copies (step 0)
  // buffer descriptors over the activations (xbytes from xbase), the
  // expert's codes and its scales: the copies of every step but a half
  // last one name a descriptor, the lane's fixed byte offset and the
  // step's uniform offset, so they need no per-step vector arithmetic
  __amdgpu_buffer_rsrc_t rx, rc, rs;
  const uint8_t* wcode;     // the expert's codes and scales (workgroup-uniform)
  const uint8_t* wscale;
  uint32_t coff[2];         // byte offsets of this lane's two 16-byte code pieces (step 0)
  uint32_t soff[2];         // byte offsets of its two scale bytes (step 0)
  uint32_t cstep, sstep;    // bytes per step of 64 stored rows
  uint32_t aoff;            // code-tile offset of the transposing read (sub-step 0)
  uint32_t sofs;            // scale-table offset of the lane's four scale words
  uint32_t boff[4];         // activation-stage offsets of the B-fragment reads per sub-step (row block 0)
  uint32_t tailmask;        // pieces past C in a half last step: 1 activations, 2 code, 4 scale
  int wave;                 // wave index (uniform)
  int nsteps;               // ceil(C / 64)
  int half_last;            // C % 64 == 32: the last step holds 32 stored rows
};

// MFMA operand registers carried between sub-steps (and from one step to
// the next): decoded A-fragments (even, odd) and B-fragments of two
// sub-steps, and the raw transposed code bytes and scale words of two
// sub-steps (read a region before their decode).
template <int NRB>
struct GFrags {
  bf16x8 a[2][2];
  bf16x8 b[2][NRB > 0 ? NRB : 1];
  i32x2 raw[2];
  u32x4 sq;          // this step's scale words of the lane's row, one per sub-step
};

// rowoff(p): element offset of activation row p (clamping rows past the
// tile to a valid row).  C, O: contraction and output lengths; o0: the
// workgroup's first output column.
// Buffer descriptor word 3 for raw (untyped) dword access on this target.
constexpr int BUF_RSRC_W3 = 0x00020000;

template <class RowOff>
__device__ __forceinline__ void g_setup(GArgs& g, const uint16_t* xbase, uint32_t xbytes,
                                        RowOff rowoff, const uint8_t* wcode,
                                        const uint8_t* wscale, int C, int O, int o0) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wo = wave & 3;
  g.wave = wave;
  g.xbase = xbase;
  // activations: instruction i of wave w fills rows 8 (GXI w + i) .. + 7,
  // slot lane % 8 of row p holding chunk (lane % 8) ^ x_swz(p)
#pragma unroll
  for (int i = 0; i < GXI; ++i) {
    const int p = 8 * GXI * wave + 8 * i + (lane >> 3);
    g.xoff[i] = rowoff(p) + 8 * (uint32_t)((lane & 7) ^ x_swz(p));
  }
  g.wcode = wcode;
  g.wscale = wscale;
  g.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xbase), (short)0, (int)xbytes, BUF_RSRC_W3);
  g.rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wcode), (short)0, C * (O / 2), BUF_RSRC_W3);
  g.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wscale), (short)0, C * (O / 32), BUF_RSRC_W3);
  // codes: LDS slot 256 m + tid of the tile (copy m = 0, 1) is row c0 =
  // 32 m + tid / 8, slot tid % 8, holding 16-byte chunk j = (tid % 8) ^
  // (c0 % 8) (32 columns)
  const int c0 = tid >> 3, j = (tid & 7) ^ (c0 & 7);
  const int col = (o0 + 32 * j < O) ? o0 + 32 * j : 0;   // past O: any valid column
  g.coff[0] = (uint32_t)c0 * (uint32_t)(O / 2) + col / 2;
  g.coff[1] = g.coff[0] + 32u * (uint32_t)(O / 2);
  // scales: table word 64 b + 32 h + 4 r + s holds row 16 s + 8 h + r
  // (sub-step s, half h, r < 8) of scale block b (copy m of wave w: b = 4 m
  // + w), so the four sub-steps' words of one row are consecutive
  {
    const int ss = lane & 3, r = (lane >> 2) & 7, h = lane >> 5;
    const int row = 16 * ss + 8 * h + r;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int b = 4 * m + wave;
      const int scol = (o0 + 32 * b < O) ? o0 + 32 * b : 0;
      g.soff[m] = (uint32_t)row * (uint32_t)(O / 32) + scol / 32;
    }
  }
  g.cstep = (uint32_t)GKC * (O / 2);
  g.sstep = (uint32_t)GKC * (O / 32);
  // transposing read: 16-lane group grp reads rows 8 (grp / 2) .. + 7 of
  // the sub-step, code chunk 2 wo + grp % 2 of double block wo; lane jj
  // names row jj / 2, bytes 8 (jj % 2) .. + 7
  const int grp = lane >> 4, jj = lane & 15;
  const int row = 8 * (grp >> 1) + (jj >> 1);
  const int chunk = 2 * wo + (grp & 1);
  g.aoff = row * (GO / 2) + 16 * (chunk ^ (row & 7)) + 8 * (jj & 1);
  // the words of row 8 (grp / 2) + jj % 8 of scale block 2 wo + grp % 2
  // (lanes jj and jj + 8 read the same ones)
  g.sofs = GCB + ((2 * wo + (grp & 1)) * GKC + 32 * (grp >> 1) + 4 * (jj & 7)) * 4;
  const int prel = lane & 31;
#pragma unroll
  for (int s = 0; s < 4; ++s) g.boff[s] = GCB + GSB + prel * 128 + 16 * ((2 * s + (lane >> 5)) ^ x_swz(prel));
  g.nsteps = (C + GKC - 1) / GKC;
  g.half_last = (C % GKC) != 0;
  // in a half last step the activation slots of k >= 32 (chunk >= 4), the
  // code rows >= 32 (all of copy 1) and the scale rows >= 32 lie past C
  {
    const int ch = (lane & 7) ^ ((lane >> 3) & 7);   // the chunk of all the lane's pieces
    g.tailmask = (ch >= 4 ? 1u : 0u) | 2u | ((lane & 3) >= 2 ? 4u : 0u);
  }
}

// Step k's tile into LDS stage st (GDMA loads of this wave).  In a half
// last step the pieces past C are read from a block of zeros.
__device__ __forceinline__ void g_dma(const GArgs& g, uint8_t* __restrict__ st, int k) {
  if (!(g.half_last && k == g.nsteps - 1)) {
#pragma unroll
    for (int i = 0; i < GXI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          g.rx, (lptr_t)(st + GCB + GSB + (g.wave * GXI + i) * 1024), 16, 2 * g.xoff[i],
          k * (2 * GKC), 0, 0);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(g.rc, (lptr_t)(st + (4 * m + g.wave) * 1024), 16,
                                               g.coff[m], k * g.cstep, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(g.rs, (lptr_t)(st + GCB + (4 * m + g.wave) * 256), 1,
                                               g.soff[m], k * g.sstep, 0, 0);
    }
    return;
  }
  const uint16_t* xp[GXI];
  const uint8_t* cp[2];
  const uint8_t* sp[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    cp[m] = g.wcode + (g.coff[m] + (uint32_t)k * g.cstep);
    sp[m] = g.wscale + (g.soff[m] + (uint32_t)k * g.sstep);
  }
#pragma unroll
  for (int i = 0; i < GXI; ++i) xp[i] = g.xbase + (g.xoff[i] + (uint32_t)(k * GKC));
  if (g.half_last && k == g.nsteps - 1) {
#pragma unroll
    for (int i = 0; i < GXI; ++i)
      if (g.tailmask & 1u) xp[i] = reinterpret_cast<const uint16_t*>(g_zero64);
    if (g.tailmask & 2u) cp[1] = g_zero64;
    if (g.tailmask & 4u) {
      sp[0] = g_zero64;
      sp[1] = g_zero64;
    }
  }
#pragma unroll
  for (int i = 0; i < GXI; ++i)
    __builtin_amdgcn_global_load_lds((gptr_t)xp[i], (lptr_t)(st + GCB + GSB + (g.wave * GXI + i) * 1024),
                                     16, 0, 0);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    __builtin_amdgcn_global_load_lds((gptr_t)cp[m], (lptr_t)(st + (4 * m + g.wave) * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((gptr_t)sp[m], (lptr_t)(st + GCB + (4 * m + g.wave) * 256), 1, 0, 0);
  }
}

// LDS reads from stage st: the transposed code bytes of sub-step s (the
// wave's double block) into slot s % 2; the lane's scale words of the
// step; and sub-step s's NRB B-fragments into slot bi.
template <int NRB>
__device__ __forceinline__ void g_read_a(const GArgs& g, const uint8_t* __restrict__ st, int s,
                                         GFrags<NRB>& F) {
  F.raw[s & 1] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (lds_i32x2*)(const_cast<uint8_t*>(st) + g.aoff + s * 16 * (GO / 2)));
}

template <int NRB>
__device__ __forceinline__ void g_read_s(const GArgs& g, const uint8_t* __restrict__ st,
                                         GFrags<NRB>& F) {
  F.sq = *reinterpret_cast<const u32x4*>(st + g.sofs);
}

template <int NRB>
__device__ __forceinline__ void g_read_b(const GArgs& g, const uint8_t* __restrict__ st, int s,
                                         GFrags<NRB>& F, int bi) {
#pragma unroll
  for (int j = 0; j < NRB; ++j)
    F.b[bi][j] = *reinterpret_cast<const bf16x8*>(st + g.boff[s] + j * 4096);
}

// row_newbcast:R -- lane R of each 16-lane row to the whole row.  Every
// lane has a valid source, so no "old" value is needed: the plain DPP move
// leaves it undefined, where a defined one costs a register copy per
// broadcast.
template <int R>
__device__ __forceinline__ uint32_t row_bcast(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x150 + R, 0xF, 0xF, false);
}

// Decode sub-step s's raw bytes into A-fragment slot ai: fragment 0 holds
// the even columns, 1 the odd ones.  Byte r of the 8 is row r of the lane's
// 8, whose scale word lane r of the 16-lane group holds (the UE8M0 byte
// moved to the exponent field: the scaled conversion reads only that field
// of its scale operand); its two nibbles are the column pair, so one scaled
// conversion gives (even, odd) as packed bf16, and byte permutes gather the
// evens and the odds.
template <int NRB>
__device__ __forceinline__ void g_decode(GFrags<NRB>& F, int ai, int s) {
  uint32_t pr[8];
  const uint32_t own = F.sq[s] << 23;
  const uint32_t scw[8] = {row_bcast<0>(own), row_bcast<1>(own), row_bcast<2>(own),
                           row_bcast<3>(own), row_bcast<4>(own), row_bcast<5>(own),
                           row_bcast<6>(own), row_bcast<7>(own)};
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint32_t w = (uint32_t)F.raw[s & 1][r >> 2];
    const float sc = __builtin_bit_cast(float, scw[r]);
    switch (r & 3) {
      case 0: pr[r] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0)); break;
      case 1: pr[r] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1)); break;
      case 2: pr[r] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2)); break;
      default: pr[r] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3)); break;
    }
  }
  u32x4 ev, od;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    ev[m] = __builtin_amdgcn_perm(pr[2 * m + 1], pr[2 * m], 0x05040100u);
    od[m] = __builtin_amdgcn_perm(pr[2 * m + 1], pr[2 * m], 0x07060302u);
  }
  F.a[ai][0] = as_bf16x8(ev);
  F.a[ai][1] = as_bf16x8(od);
}

// The 2 x NRB MFMAs of one sub-step (independent accumulators).
template <int NRB>
__device__ __forceinline__ void g_mfmas(const GFrags<NRB>& F, int ai, int bi,
                                        f32x16 (&acc)[2][GRB]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NRB; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.a[ai][i], F.b[bi][j], acc[i][j], 0, 0, 0);
}

// Issue order inside one region: its LDS reads first, then its MFMAs, each
// of the first NF followed by FPER VALU instructions (the decode), the rest
// back to back.
template <int NR, int NM, int NF, int FPER>
__device__ __forceinline__ void g_order() {
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (m < NF) __builtin_amdgcn_sched_group_barrier(0x002, FPER, 0);
  }
}

// The same with the first half of the MFMAs back to back after the reads
// and the VALU work spread over the second half (its inputs are this
// region's reads, which then have half the MFMAs' time to arrive).
template <int NR, int NM, int FPER>
__device__ __forceinline__ void g_order_late() {
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, NM / 2, 0);
#pragma unroll
  for (int m = NM / 2; m < NM; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 2 * FPER, 0);
  }
}

// The same with the region's first MFMA issued before its LDS reads (its
// operands come from the previous region, so waiting for them does not
// wait for this region's reads).
template <int NR, int NM, int NF, int FPER>
__device__ __forceinline__ void g_order_mfirst() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
  __builtin_amdgcn_sched_group_barrier(0x002, FPER, 0);
#pragma unroll
  for (int m = 1; m < NM; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (m < NF) __builtin_amdgcn_sched_group_barrier(0x002, FPER, 0);
  }
}

// One step k (stages: cur = k % 3 holds step k, nxt = (k + 1) % 3 step k +
// 1, dst = (k + 2) % 3 was last read in step k - 1), in scheduling regions
// fenced by sched_barrier.  On entry sub-step 0's operands are decoded (A,
// slot 0) and read (B, slot 0) and sub-step 1's code bytes and scales are
// read; step k + 1's copy is in flight.
//   (0) start step k + 2's copy into dst;
//   (1..3) sub-step s + 2's code bytes and scales and s + 1's B-fragments,
//       then sub-step s's MFMAs with the decode of s + 1 interleaved (its
//       operands were read a region earlier);
//   wait for this wave's copy of step k + 1 and its LDS reads, and meet the
//   other waves: nxt is complete and every wave is done reading cur, so
//   (4) step k + 1's sub-step 0 and 1 code bytes and scales and sub-step 0
//       B-fragments, then sub-step 3's MFMAs with the decode of step k + 1's
//       sub-step 0 interleaved.
template <int NRB>
__device__ __forceinline__ void g_step(GFrags<NRB>& F, const GArgs& g, int k,
                                       const uint8_t* __restrict__ cur,
                                       const uint8_t* __restrict__ nxt, uint8_t* __restrict__ dst,
                                       f32x16 (&acc)[2][GRB]) {
  // 25 decode instructions spread over the MFMAs
  constexpr int NM = 2 * NRB, FPER = (25 + NM - 1) / (NM > 0 ? NM : 1);
  __builtin_amdgcn_sched_barrier(0);
  g_dma(g, dst, min(k + 2, g.nsteps - 1));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    if constexpr (NRB > 0) {
      if (s < 2) g_read_a<NRB>(g, cur, s + 2, F);
      g_read_b<NRB>(g, cur, s + 1, F, (s + 1) & 1);
      g_mfmas<NRB>(F, s & 1, s & 1, acc);
      g_decode<NRB>(F, (s + 1) & 1, s + 1);
      if (s == 0)
        g_order<1 + NRB, NM, NM, FPER>();
      else if (s == 1)
        g_order_mfirst<1 + NRB, NM, NM, FPER>();
      else
        g_order_mfirst<NRB, NM, NM, FPER>();
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(GDMA, 0));
  barrier_only();
  if constexpr (NRB > 0) {
    g_read_s<NRB>(g, nxt, F);
    g_read_a<NRB>(g, nxt, 0, F);
    g_read_a<NRB>(g, nxt, 1, F);
    g_read_b<NRB>(g, nxt, 0, F, 0);
    g_mfmas<NRB>(F, 1, 1, acc);
    g_decode<NRB>(F, 0, 0);
    g_order_late<3 + NRB, NM, FPER>();
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Steps k .. k + n - 1 (n <= 3) with k % 3 == 0: stage i holds step k + i.
// The three stages are distinct, which lets the compiler see that a stage's
// reads do not depend on the copies into the others.
template <int NRB>
__device__ __forceinline__ void g_trip(GFrags<NRB>& F, const GArgs& g, int k, int n,
                                       uint8_t* __restrict__ st0, uint8_t* __restrict__ st1,
                                       uint8_t* __restrict__ st2, f32x16 (&acc)[2][GRB]) {
  g_step<NRB>(F, g, k, st0, st1, st2, acc);
  if (n > 1) g_step<NRB>(F, g, k + 1, st1, st2, st0, acc);
  if (n > 2) g_step<NRB>(F, g, k + 2, st2, st0, st1, acc);
}

template <int NRB>
__device__ __forceinline__ void g_loop(const GArgs& g, uint8_t* lds, f32x16 (&acc)[2][GRB]) {
  GFrags<NRB> F;
  uint8_t* st0 = lds;
  uint8_t* st1 = lds + GSTAGE;
  uint8_t* st2 = lds + 2 * GSTAGE;
  g_dma(g, st0, 0);
  g_dma(g, st1, min(1, g.nsteps - 1));
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(GDMA, 0));
  barrier_only();
  if constexpr (NRB > 0) {
    g_read_s<NRB>(g, st0, F);
    g_read_a<NRB>(g, st0, 0, F);
    g_read_a<NRB>(g, st0, 1, F);
    g_read_b<NRB>(g, st0, 0, F, 0);
    g_decode<NRB>(F, 0, 0);
  }
  // three steps per trip, so each step's stages are fixed pointers
  int k = 0;
  for (; k + 3 <= g.nsteps; k += 3) g_trip<NRB>(F, g, k, 3, st0, st1, st2, acc);
  if (k < g.nsteps) g_trip<NRB>(F, g, k, g.nsteps - k, st0, st1, st2, acc);
  // the last steps copied and read (unused) operands of other stages; every
  // wave must be past them before the epilogue reuses LDS
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  __syncthreads();
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[2][GRB]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < GRB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// Live 32-row blocks in a tile of `rows` rows.
__device__ __forceinline__ int live_blocks(int rows) { return min(GRB, (rows + 31) >> 5); }

// f(integral_constant<int, n>) for n = live (1 <= live <= N): the body
// instantiated for each live block count.
template <int N, class F>
__device__ __forceinline__ void with_blocks(int live, F&& f) {
  if constexpr (N >= 1) {
    if (live == N) {
      f(std::integral_constant<int, N>{});
      return;
    }
    with_blocks<N - 1>(live, f);
  }
}

// Accumulator layout.  Fragment par covers the columns 2 m + par of the
// wave's double block (m: MFMA row); lane l holds rows m = 8 (r / 4) + 4 (l /
// 32) + r % 4 of column l % 32 (a routed row).  So for q = r / 4 a lane
// holds 8 consecutive columns of its wave's 64, 16 q + 8 (l / 32) + 0..7:
// registers 4q..4q+3 of fragment 0 give the even ones and of fragment 1 the
// odd ones.  cols8 returns them as 8 fp32 in column order.
__device__ __forceinline__ void cols8(const f32x16 (&acc)[2][GRB], int q, int j, float (&v)[8]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    v[2 * m] = acc[0][j][4 * q + m];
    v[2 * m + 1] = acc[1][j][4 * q + m];
  }
}

// + dv A over an adapter's rank into the accumulators: 16-deep MFMA
// contractions, A-operand = rows of A^T (At, [O, r] per expert; fragment
// i's MFMA row l32 is output column ow + 2 l32 + i), B-operand = dv [R, r]
// (sorted order) as hi + lo bf16.
template <int NRB>
__device__ __forceinline__ void lora_term(f32x16 (&acc)[2][GRB], const Tile& tl, int ow,
                                          int O, const uint16_t* __restrict__ At,
                                          const float* __restrict__ dv, int r) {
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hlf = lane >> 5;
  for (int q = 0; q < lora_chunks(r); ++q) {
#pragma unroll
    for (int j = 0; j < NRB; ++j) {
      const int pb = j;
      bf16x8 vh, vl;
      lora_frag_split(dv + (int64_t)(tl.row0 + min(32 * pb + l32, tl.rows - 1)) * r, r, q, hlf,
                      1.0f, &vh, &vl);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int col = ow + 2 * l32 + i;
        const bf16x8 aw = lora_frag(At + ((int64_t)tl.expert * O + (col < O ? col : 0)) * r, r, q, hlf);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, vh, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, vl, acc[i][j], 0, 0, 0);
      }
    }
  }
}

// bwd_gate_up body for a wave with NRB live row blocks: main loop, then the
// epilogue through a private LDS strip per wave (32 rows x 128 columns of
// bf16 per row block), stored as whole 16-byte row pieces to the routed
// rows' own dxr slots.
template <bool LORA, int NRB>
__device__ __forceinline__ void bwd_gate_up_body(const GArgs& g, uint8_t* lds, const Tile& tl,
                                                 const int32_t* __restrict__ sorted_rows, int H,
                                                 int o0, const uint16_t* __restrict__ lora_At,
                                                 const float* __restrict__ lora_dv, int lora_r,
                                                 uint16_t* __restrict__ dxr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wo = wave;
  const int l32 = lane & 31, hlf = lane >> 5;
  // each row block's flat row for this lane, loaded before the main loop
  int32_t fv[NRB > 0 ? NRB : 1];
#pragma unroll
  for (int j = 0; j < NRB; ++j) fv[j] = sorted_rows[tl.row0 + min(32 * j + l32, tl.rows - 1)];
  f32x16 acc[2][GRB];
  zero_acc(acc);
  g_loop<NRB>(g, lds, acc);
  const int ow = o0 + 64 * wo;                // this wave's first output column
  if (LORA && NRB > 0) lora_term<NRB>(acc, tl, ow, H, lora_At, lora_dv, lora_r);
  if (NRB == 0 || ow >= H) return;
  uint8_t* st = lds + wave * 4096;            // 32 rows x 128 bytes
#pragma unroll
  for (int j = 0; j < NRB; ++j) {
    const int pb = j;
    const int32_t f = fv[j];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[8];
      cols8(acc, q, j, v);
      const u32x4 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7])};
      *reinterpret_cast<u32x4*>(st + stg_off<128>(l32, 2 * q + hlf)) = w;
    }
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = 8 * it + (lane >> 3), c = lane & 7;
      const int rt = 32 * pb + r;
      const int64_t fr = __shfl(f, r);
      const u32x4 v = *reinterpret_cast<const u32x4*>(st + stg_off<128>(r, c));
      if (rt < tl.rows && ow + 8 * c < H)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dxr + fr * H + ow + 8 * c));
    }
    wave_lds_sync();
  }
}

template <bool LORA>
__global__ __launch_bounds__(GTHR) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_gate_up_kernel(
    const uint16_t* __restrict__ dh, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const int32_t* __restrict__ sorted_rows,
    const Tile* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int H, int I,
    const uint16_t* __restrict__ lora_At, const float* __restrict__ lora_dv, int lora_r,
    uint16_t* __restrict__ dxr) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[GLDS_LOOP];
  Tile tl;
  int ot;
  if (!xcd_work_item(tiles, num_tiles, (H + GO - 1) / GO, &tl, &ot)) return;
  const int o0 = ot * GO, N2 = 2 * I;
  // Wgu is stored [2I rows][H cols]: contraction over n (C = 2I), output h (O = H);
  // the activations are dh's rows in sorted order
  GArgs g;
  // the tile's dh rows (a contiguous range in sorted order) from its first
  g_setup(g, dh + (int64_t)tl.row0 * N2, (uint32_t)tl.rows * (uint32_t)N2 * 2u,
          [&](int p) { return (uint32_t)min(p, tl.rows - 1) * (uint32_t)N2; },
          codes + (int64_t)tl.expert * N2 * (H / 2), scales + (int64_t)tl.expert * N2 * (H / 32),
          N2, H, o0);
  with_blocks<GRB>(live_blocks(tl.rows), [&](auto nrb) {
    bwd_gate_up_body<LORA, decltype(nrb)::value>(g, lds, tl, sorted_rows, H, o0, lora_At, lora_dv,
                                                 lora_r, dxr);
  });
}

// bwd_down body: main loop; with LORA the adapter term dv_u A_e (a 16-deep
// MFMA contraction per fragment, dv_u as hi + lo bf16); then per live row
// block the epilogue through a private LDS region: the block's saved a (32
// x 128) and h (32 x 256) rows staged with row-contiguous loads, read back
// as 8 consecutive columns per lane, the dw partial sum_i da_u * a (masked
// to i < I), the SwiGLU backward with da = w * da_u written over h, and dh
// stored as whole row pieces.  The two waves of a row group (wo = 0, 1) add
// their dw partials in wave order through LDS.
template <bool LORA, int NRB>
__device__ __forceinline__ void bwd_down_body(
    const GArgs& g, uint8_t* lds, const Tile& tl, int ot, int otiles, int o0,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_rows,
    const uint16_t* __restrict__ hsv, const uint16_t* __restrict__ asv, int I, float alpha,
    float limit, const uint16_t* __restrict__ lora_At, const float* __restrict__ lora_dvu,
    int lora_r, uint16_t* __restrict__ dh, float* __restrict__ dw_part) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wo = wave;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int e = tl.expert;
  // the routing weight of this lane's row in each block, loaded before the
  // main loop (two dependent loads, in flight under it)
  float wfv[NRB > 0 ? NRB : 1];
#pragma unroll
  for (int j = 0; j < NRB; ++j) wfv[j] = topk_w[sorted_rows[tl.row0 + min(32 * j + l32, tl.rows - 1)]];
  f32x16 acc[2][GRB];
  zero_acc(acc);
  g_loop<NRB>(g, lds, acc);
  const int ow = o0 + 64 * wo;                // this wave's first column of I
  if (LORA && NRB > 0) lora_term<NRB>(acc, tl, ow, I, lora_At, lora_dvu, lora_r);
  const int N2 = 2 * I;
  const bool active = ow < I;
  uint8_t* ast = lds + wave * 12288;          // a strip: 32 rows x 64 bf16 (128-byte rows)
  uint8_t* hst = ast + 4096;                  // h / dh strip: 32 rows x 128 bf16 (256-byte rows)
  float* red = reinterpret_cast<float*>(lds + GW * 12288);   // [GW][BMT]
#pragma unroll
  for (int j = 0; j < NRB; ++j) {
    const int pb = j;
    float dwp = 0.0f;
    if (active) {
      // a pieces past I are staged as zeros, so the dw partial needs no
      // per-column test (the accumulator columns there are finite copies)
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int r = 8 * it + (lane >> 3), c = lane & 7;
        const int64_t p = tl.row0 + min(32 * pb + r, tl.rows - 1);
        const int col = ow + 8 * c;
        const u32x4 av = *reinterpret_cast<const u32x4*>(asv + p * I + min(col, I - 8));
        *reinterpret_cast<u32x4*>(ast + stg_off<128>(r, c)) = col < I ? av : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = 4 * it + (lane >> 4), c = lane & 15;
        const int64_t p = tl.row0 + min(32 * pb + r, tl.rows - 1);
        const int col = min(2 * ow + 8 * c, N2 - 8);
        *reinterpret_cast<u32x4*>(hst + stg_off<256>(r, c)) =
            *reinterpret_cast<const u32x4*>(hsv + p * N2 + col);
      }
      const float wf = wfv[j];
      wave_lds_sync();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cb = 2 * q + hlf;                    // 8-column chunk of the wave's 64
        float v[8];
        cols8(acc, q, j, v);
        const u32x4 av = *reinterpret_cast<const u32x4*>(ast + stg_off<128>(l32, cb));
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          uint8_t* hp = hst + stg_off<256>(l32, 2 * cb + half);
          const u32x4 hv = *reinterpret_cast<const u32x4*>(hp);
          u32x4 out;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int c = 4 * half + m;                // column ow + 8 cb + c
            const float du_ = v[c];
            const uint32_t aw = av[c >> 1];
            const float a_c = bf16_to_f32((uint16_t)((c & 1) ? (aw >> 16) : (aw & 0xFFFFu)));
            dwp += du_ * a_c;
            const uint32_t hw = hv[m];
            float dg, dup;
            swiglu_grad(bf16_to_f32((uint16_t)(hw & 0xFFFFu)), bf16_to_f32((uint16_t)(hw >> 16)),
                        wf * du_, alpha, limit, &dg, &dup);
            out[m] = pack_bf16x2(dg, dup);
          }
          *reinterpret_cast<u32x4*>(hp) = out;
        }
      }
      wave_lds_sync();
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int r = 4 * it + (lane >> 4), c = lane & 15;
        const int rt = 32 * pb + r;
        const u32x4 v = *reinterpret_cast<const u32x4*>(hst + stg_off<256>(r, c));
        if (rt < tl.rows && 2 * ow + 8 * c < N2)
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dh + (int64_t)(tl.row0 + rt) * N2 + 2 * ow + 8 * c));
      }
      wave_lds_sync();
    }
    dwp += __shfl_xor(dwp, 32);
    if (hlf == 0) red[wave * BMT + 32 * j + l32] = dwp;
  }
  __syncthreads();
  // row p of the tile: the four waves' partials, wo = 0..3, added in order
  if (tid < tl.rows) {
    const int p = tid;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < GW; ++w) sum += red[w * BMT + p];
    const int64_t f = sorted_rows[tl.row0 + p];
    dw_part[f * otiles + ot] = sum;
  }
}

template <bool LORA>
__global__ __launch_bounds__(GTHR) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_down_kernel(
    const uint16_t* __restrict__ dy, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const float* __restrict__ topk_w,
    const int32_t* __restrict__ sorted_rows, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, const uint16_t* __restrict__ hsv,
    const uint16_t* __restrict__ asv, int H, int I, int k, float alpha, float limit,
    const uint16_t* __restrict__ lora_At, const float* __restrict__ lora_dvu, int lora_r,
    uint16_t* __restrict__ dh, float* __restrict__ dw_part) {
  // the epilogue's strips (8 x 12 KB) and dw reduction reuse the main loop's stages
  __shared__ __attribute__((aligned(16))) uint8_t lds[GLDS_LOOP];
  static_assert(GW * 12288 + GW * BMT * 4 <= GLDS_LOOP, "the epilogue fits the loop's LDS");
  Tile tl;
  int ot;
  const int otiles = (I + GO - 1) / GO;
  if (!xcd_work_item(tiles, num_tiles, otiles, &tl, &ot)) return;
  const int o0 = ot * GO;
  // Wd is stored [H rows][I cols]: contraction over h (C = H), output i (O =
  // I); the activations are the routed rows' tokens' dY rows
  GArgs g;
  // dy's token rows: T * H < 2^31, so every byte offset fits the descriptor
  g_setup(g, dy, 0xFFFFFFFFu,
          [&](int p) {
            return (uint32_t)(sorted_rows[tl.row0 + min(p, tl.rows - 1)] / k) * (uint32_t)H;
          },
          codes + (int64_t)tl.expert * H * (I / 2), scales + (int64_t)tl.expert * H * (I / 32), H,
          I, o0);
  with_blocks<GRB>(live_blocks(tl.rows), [&](auto nrb) {
    bwd_down_body<LORA, decltype(nrb)::value>(g, lds, tl, ot, otiles, o0, topk_w, sorted_rows, hsv,
                                              asv, I, alpha, limit, lora_At, lora_dvu, lora_r, dh,
                                              dw_part);
  });
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

int bwd_down_ntiles(int I) { return (I + GO - 1) / GO; }

hipError_t launch_bwd_down(const uint16_t* dy, const uint8_t* codes, const uint8_t* scales,
                           const float* topk_w, const int32_t* sorted_rows, const Tile* tiles,
                           const int32_t* num_tiles, int max_tiles, const uint16_t* h,
                           const uint16_t* a, int H, int I, int k, float alpha, float limit,
                           const uint16_t* lora_At, const float* lora_dvu, int lora_r,
                           uint16_t* dh, float* dw_part, hipStream_t s) {
  if (H % 32 || I % 32 || (lora_At && !lora_rank_ok(lora_r))) return hipErrorInvalidValue;
  dim3 grid(bwd_down_ntiles(I) * max_tiles);
  if (lora_At)
    hipLaunchKernelGGL(bwd_down_kernel<true>, grid, dim3(GTHR), 0, s, dy, codes, scales, topk_w,
                       sorted_rows, tiles, num_tiles, h, a, H, I, k, alpha, limit, lora_At,
                       lora_dvu, lora_r, dh, dw_part);
  else
    hipLaunchKernelGGL(bwd_down_kernel<false>, grid, dim3(GTHR), 0, s, dy, codes, scales, topk_w,
                       sorted_rows, tiles, num_tiles, h, a, H, I, k, alpha, limit, lora_At,
                       lora_dvu, 0, dh, dw_part);
  return hipGetLastError();
}

hipError_t launch_bwd_gate_up(const uint16_t* dh, const uint8_t* codes, const uint8_t* scales,
                              const int32_t* sorted_rows, const Tile* tiles,
                              const int32_t* num_tiles, int max_tiles, int H, int I,
                              const uint16_t* lora_At, const float* lora_dv, int lora_r,
                              uint16_t* dxr, hipStream_t s) {
  if (I % 32 || H % 32 || (lora_At && !lora_rank_ok(lora_r))) return hipErrorInvalidValue;
  dim3 grid(((H + GO - 1) / GO) * max_tiles);
  if (lora_At)
    hipLaunchKernelGGL(bwd_gate_up_kernel<true>, grid, dim3(GTHR), 0, s, dh, codes, scales,
                       sorted_rows, tiles, num_tiles, H, I, lora_At, lora_dv, lora_r, dxr);
  else
    hipLaunchKernelGGL(bwd_gate_up_kernel<false>, grid, dim3(GTHR), 0, s, dh, codes, scales,
                       sorted_rows, tiles, num_tiles, H, I, lora_At, lora_dv, 0, dxr);
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
