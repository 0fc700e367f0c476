// Decode-sized forward GEMMs (few routed rows per expert): the same math as
// gate_up_kernel / down_kernel in gemm_fwd.hip, reorganised so that the
// packed weights of the touched experts stream from HBM at full rate.
//
// With T*k <= 256 an expert owns a handful of rows, so the work is bound by
// reading its weights once (13.2 MB per gpt-oss-20b expert), not by MFMA.
// A workgroup takes one tile (one expert's rows, at most 128) and WPB x 32
// weight rows; each wave owns 32 rows over the whole contraction and
// streams their codes in chunks of DD K-steps, two chunks in registers (the
// next one in flight while the current one is computed), so no wave waits
// on another after the activation rows are staged.  The routed rows'
// activations are staged in LDS in groups of DG (8 or 16) and fed as the
// MFMA B-operand (columns past the group repeat its last row and are
// dropped); a larger group re-streams the codes.  The accumulator layout and
// the bias + clamped SwiGLU epilogue are those of the forward GEMMs: gate/up
// pairs sit in neighbouring registers of one lane.
#include "common.hpp"
#include "launch.hpp"

namespace mxmoe {

constexpr int DEC_MAXK = 3072;           // contraction lengths the kernels take
constexpr int DEC_XPAD = 8;              // bf16 of padding per staged row

int dec_max_k() { return DEC_MAXK; }

constexpr int DD = 9;                    // K steps (64 wide) per streamed chunk


struct DecChunk {
  u32x4 c[DD];
};

// Codes of chunk ch (steps DD*ch ..), clamped to the last step.  ztail: the
// lane's half of the last step lies past K (K an odd multiple of 32); its
// codes then come from a block of zeros.
__device__ __forceinline__ void dec_issue(DecChunk& b, const uint8_t* wrow, int ch, int nsteps,
                                          bool ztail) {
#pragma unroll
  for (int i = 0; i < DD; ++i) {
    const int c = min(ch * DD + i, nsteps - 1);
    const uint8_t* ptr = (ztail && c == nsteps - 1) ? g_zero64 : wrow + c * 32;
    b.c[i] = gload16(ptr);
  }
}

// srow: this lane's row of the scale panel in LDS (+ lane half); smax: the
// largest index it may read (K / 32 - 1 - lane half)
// cs: the first step staged in LDS (the activation segment's start)
__device__ __forceinline__ void dec_compute(const DecChunk& b, const uint16_t* xb,
                                            const uint8_t* srow, int smax, int ch, int nsteps,
                                            int cs, f32x16& acc) {
#pragma unroll
  for (int i = 0; i < DD; ++i) {
    const int c = ch * DD + i;
    if (c < nsteps) {
      const float sc = scale_operand(srow[min(2 * c, smax)]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 a = as_bf16x8(dequant8_bf16(b.c[i][s], sc));
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(xb + 64 * (c - cs) + 8 * s);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc, 0, 0, 0);
      }
    }
  }
}

template <bool GATE_UP>
__global__ __launch_bounds__(512) void dec_kernel(
    const uint16_t* __restrict__ src,      // gate_up: x [T, K]; down: a [R, K] (sorted)
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ bias, const float* __restrict__ topk_w,
    const int32_t* __restrict__ sorted_rows, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, int K, int N, int k, int DG, int seg_ch, float alpha,
    float limit, uint16_t* __restrict__ h_out, uint16_t* __restrict__ a_out,
    uint16_t* __restrict__ y_w, const uint16_t* __restrict__ lora_B,
    const float* __restrict__ lora_v, float lora_scale, int lora_r) {
  // LDS: the scale panel of the workgroup's weight rows [32 * wpb][K / 32]
  // (one contiguous span of the scale tensor, copied in 16-byte pieces), then
  // the activation group [DG][xcols + DEC_XPAD] bf16: one segment of seg_ch
  // chunks of K (xcols = seg_ch * DD * 64 columns, or K rounded up to 64 if
  // that is less; zeros past K), restaged as the codes stream past it
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int wpb = blockDim.x >> 6;
  const int nblk = (N + 32 * wpb - 1) / (32 * wpb);
  const int tile = blockIdx.x / nblk, rbk = blockIdx.x % nblk;
  if (tile >= *num_tiles) return;
  const Tile tl = tiles[tile];
  if (tl.rows <= 0) return;   // empty slot of the XCD deal
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int e = tl.expert;
  const int Kp = (K + 63) & ~63;               // K rounded up to whole 64-wide steps
  const int scols = seg_ch * DD * 64;          // columns per staged segment
  const int xrow = min(Kp, scols) + DEC_XPAD;
  const int n0 = (rbk * wpb + wave) * 32;      // this wave's first weight row
  const bool live = n0 < N;                    // N % 32 == 0: a block is all in or out
  const int n = live ? n0 + l32 : l32;
  const uint8_t* wrow = codes + ((int64_t)e * N + n) * (K / 2) + hlf * 16;
  const int nsteps = Kp / 64;
  const bool ztail = (K & 63) && hlf;          // this lane's half of the last step lies past K
  const int smax = K / 32 - 1 - hlf;
  const int nch = (nsteps + DD - 1) / DD;
  // staged pieces per row of segment sg; those past K are zeros
  auto spieces = [&](int sg) { return (min(Kp, (sg + 1) * scols) - sg * scols) / 8; };
  uint8_t* panel = lds;
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds + 32 * wpb * (K / 32));
  const int nthr = blockDim.x;
  // Load order: the row indices, the scale panel, the bias, a group's
  // activation pieces, then the group's first chunk of codes, and only then
  // the LDS stores of the staged pieces.  The wait counter retires loads in
  // issue order, so the stores wait for the staged loads alone while the
  // codes stay in flight.  Per thread at most PP panel pieces (wpb * K / 16
  // over 64 * wpb threads) and XP activation pieces (DG * xcols / 8 over
  // 64 * wpb threads): the launch keeps to these.  No
  // load of this staging sits under a branch: at a branch merge the wait
  // counter's bookkeeping takes the path with fewer loads in flight, so a
  // conditional code issue would make the stores wait for the codes.
  constexpr int PP = DEC_MAXK / 1024;
  constexpr int XP = 12;
  // gate_up: the token row of each group row, one per lane, shared by shuffle
  auto group_rows = [&](int g0) -> int {
    return GATE_UP ? sorted_rows[tl.row0 + g0 + min(lane, min(DG, tl.rows - g0) - 1)] / k : 0;
  };
  int grow = group_rows(0);
  int64_t f0 = 0;
  float wf0 = 0.0f;
  if (!GATE_UP) f0 = sorted_rows[tl.row0 + min(l32, tl.rows - 1)];
  const int r0 = rbk * wpb * 32;
  const int n16 = min(32 * wpb, N - r0) * (K / 32) / 16;
  const u32x4* ps = reinterpret_cast<const u32x4*>(scales + ((int64_t)e * N + r0) * (K / 32));
  u32x4 pv[PP];
#pragma unroll
  for (int u = 0; u < PP; ++u) pv[u] = gload16(ps + min(tid + u * nthr, n16 - 1));
  // the epilogue's bias pairs, fetched now so they arrive under the codes
  u32x2 bwv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const void* bp = (bias && live) ? static_cast<const void*>(bias + (int64_t)e * N + n0 + 8 * q + 4 * hlf)
                                    : static_cast<const void*>(g_zero64);
    bwv[q] = *(const __attribute__((address_space(1))) u32x2*)bp;
  }
  __builtin_amdgcn_sched_barrier(0);
  if (!GATE_UP) wf0 = topk_w[f0];
  // activation piece q of group g0, segment sg: group row q / np, 8 columns
  // from the segment's start (zeros past K); no branch around the load
  auto xsrc = [&](int g0, int sg, int np, int q) -> const uint16_t* {
    const int pr = q / np, col = sg * scols + (q % np) * 8;
    const int64_t sr = GATE_UP ? (int64_t)__shfl(grow, pr) : (int64_t)(tl.row0 + g0 + pr);
    return src + sr * K + min(col, K - 8);
  };
  u32x4 xv[XP];
  auto xload_all = [&](int g0, int sg, int ng) {
    const int np = spieces(sg), nx = ng * np;
#pragma unroll
    for (int u = 0; u < XP; ++u) xv[u] = gload16(xsrc(g0, sg, np, min(tid + u * nthr, nx - 1)));
  };
  // unconditional stores (a store under a branch lets the compiler sink its
  // load there, behind the codes); the clamped threads repeat the last piece
  auto xstore_all = [&](int sg, int ng) {
    const int np = spieces(sg), nx = ng * np;
#pragma unroll
    for (int u = 0; u < XP; ++u) {
      const int q = min(tid + u * nthr, nx - 1);
      const int col = (q % np) * 8;
      *reinterpret_cast<u32x4*>(xs + (q / np) * xrow + col) =
          sg * scols + col < K ? xv[u] : u32x4{0u, 0u, 0u, 0u};
    }
  };
  const uint8_t* srow = panel + (live ? wave * 32 + l32 : 0) * (K / 32) + hlf;

  DecChunk b0, b1;
  {
    const int ng = min(DG, tl.rows);
    xload_all(0, 0, ng);
    __builtin_amdgcn_sched_barrier(0);
    dec_issue(b0, wrow, 0, nsteps, ztail);     // a wave past N reads rows it then leaves unused
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < PP; ++u)
      reinterpret_cast<u32x4*>(panel)[min(tid + u * nthr, n16 - 1)] = pv[u];
    xstore_all(0, ng);
  }

  for (int g0 = 0; g0 < tl.rows; g0 += DG) {
    const int ng = min(DG, tl.rows - g0);
    if (g0 > 0) {
      // the group's staging as the first one's, its codes issued in between
      grow = group_rows(g0);
      xload_all(g0, 0, ng);
      __builtin_amdgcn_sched_barrier(0);
      dec_issue(b0, wrow, 0, nsteps, ztail);
      __builtin_amdgcn_sched_barrier(0);
      xstore_all(0, ng);
    }
    __syncthreads();
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    // every wave runs the stream (the segment restaging has workgroup
    // barriers); a wave past N computes on rows it leaves unused
    // B-operand column l32 reads row min(l32 % DG, ng - 1)
    const uint16_t* xb = xs + min(l32 % DG, ng - 1) * xrow + 32 * hlf;
    for (int ch = 0; ch < nch; ch += 2) {
      if (ch > 0 && ch % seg_ch == 0) {
        // next segment (seg_ch is even): every wave is past the last one
        __syncthreads();
        xload_all(g0, ch / seg_ch, ng);
        xstore_all(ch / seg_ch, ng);
        __syncthreads();
      }
      const int cs = (ch / seg_ch) * seg_ch * DD;
      dec_issue(b1, wrow, min(ch + 1, nch - 1), nsteps, ztail);
      dec_compute(b0, xb, srow, smax, ch, nsteps, cs, acc);
      if (ch + 1 >= nch) break;
      dec_issue(b0, wrow, min(ch + 2, nch - 1), nsteps, ztail);
      dec_compute(b1, xb, srow, smax, ch + 1, nsteps, cs, acc);
    }
    if (live) {
      if (lora_B) {
        // + s v B_e^T over the rank (as the GEMMs' adapter term): A-operand
        // = B_e row n, B-operand column l32 = the group row it repeats
        const float* vrow = lora_v + (int64_t)(tl.row0 + g0 + min(l32 % DG, ng - 1)) * lora_r;
        const uint16_t* brow = lora_B + ((int64_t)e * N + n) * lora_r;
        for (int j = 0; j < lora_chunks(lora_r); ++j) {
          bf16x8 vh, vl;
          lora_frag_split(vrow, lora_r, j, hlf, lora_scale, &vh, &vl);
          const bf16x8 bw = lora_frag(brow, lora_r, j, hlf);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw, vh, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw, vl, acc, 0, 0, 0);
        }
      }
      // lane: column p = l32 of the group, weight rows nb + i (registers 4q + i)
      const int p = g0 + l32;
      if (l32 < DG && p < tl.rows) {
        const int64_t rho = tl.row0 + p;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nb = n0 + 8 * q + 4 * hlf;
          float v[4];
          const u32x2 bw = bwv[q];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            v[i] = acc[4 * q + i] + bf16_to_f32((uint16_t)(bw[i >> 1] >> (16 * (i & 1))));
          if (GATE_UP) {
            const int I = N / 2;
            if (h_out) {
              u32x2 hv = {saved_preact_bf16(v[0], limit, false) | (saved_preact_bf16(v[1], limit, true) << 16),
                          saved_preact_bf16(v[2], limit, false) | (saved_preact_bf16(v[3], limit, true) << 16)};
              *reinterpret_cast<u32x2*>(h_out + rho * N + nb) = hv;
            }
            *reinterpret_cast<uint32_t*>(a_out + rho * I + nb / 2) =
                pack_bf16x2(swiglu(v[0], v[1], alpha, limit), swiglu(v[2], v[3], alpha, limit));
          } else {
            const int64_t f = g0 == 0 ? f0 : (int64_t)sorted_rows[rho];
            const float wf = g0 == 0 ? wf0 : topk_w[f];
            const u32x2 y = {pack_bf16x2(wf * v[0], wf * v[1]), pack_bf16x2(wf * v[2], wf * v[3])};
            *reinterpret_cast<u32x2*>(y_w + f * N + nb) = y;
          }
        }
      }
    }
    __syncthreads();   // LDS is restaged for the next group
  }
}

// Very few routed rows (T*k <= 16: a few experts, a row or two each): the
// streaming kernel's one-wave-per-32-rows grid is too small to keep enough
// bytes in flight, so here the 4 waves of a workgroup split one 32-row
// block's contraction and issue every code load of their K quarter up
// front.  The partial accumulators are summed through LDS in wave order
// (over the staged rows, once every wave has read them) and wave w finishes
// accumulator registers 4w..4w+3 (gate/up pairs stay in one lane).
constexpr int KW = 4;                        // waves per workgroup (K quarters)
constexpr int KSTEPS = DEC_MAXK / 64 / KW;   // K steps per wave at most (12)

template <bool GATE_UP>
__global__ __launch_bounds__(64 * KW) void dec_ksplit_kernel(
    const uint16_t* __restrict__ src, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const uint16_t* __restrict__ bias,
    const float* __restrict__ topk_w, const int32_t* __restrict__ sorted_rows,
    const Tile* __restrict__ tiles, const int32_t* __restrict__ num_tiles, int K, int N, int k,
    int DG, float alpha, float limit, uint16_t* __restrict__ h_out, uint16_t* __restrict__ a_out,
    uint16_t* __restrict__ y_w, const uint16_t* __restrict__ lora_B,
    const float* __restrict__ lora_v, float lora_scale, int lora_r) {
  // LDS: scale panel [32][K / 32], then the activation group [DG][Kp + DEC_XPAD]
  // bf16, which the partial sums [KW][16][64] fp32 reuse after the MFMAs
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int nrb = N / 32;
  const int tile = blockIdx.x / nrb, rb = blockIdx.x % nrb;
  if (tile >= *num_tiles) return;
  const Tile tl = tiles[tile];
  if (tl.rows <= 0) return;   // empty slot of the XCD deal
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hlf = lane >> 5;
  const int e = tl.expert;
  const int Kp = (K + 63) & ~63;               // K rounded up to whole 64-wide steps
  const int xrow = Kp + DEC_XPAD;
  uint8_t* panel = lds;
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds + K);   // the panel is 32 x K/32 = K bytes
  float* red = reinterpret_cast<float*>(xs);

  const int nsteps = Kp / 64;
  const bool ztail = (K & 63) && hlf;          // this lane's half of the last step lies past K
  const int smax = K / 32 - 1 - hlf;
  const int per = (nsteps + KW - 1) / KW;
  const int c0 = min(wave * per, nsteps), cnt = min(per, nsteps - c0);
  const int n = rb * 32 + l32;
  const uint8_t* wrow = codes + ((int64_t)e * N + n) * (K / 2) + hlf * 16;
  const int npieces = Kp / 8;                  // staged pieces per row; those past K are zeros
  // activation piece q of group g0: row q / npieces of the group, 8 columns;
  // no branch around the load, so no merge of loaded registers forces a
  // wait for every load in flight
  auto xload = [&](int g0, int q) -> u32x4 {
    const int pr = q / npieces, col = (q % npieces) * 8;
    const int rt = tl.row0 + g0 + pr;
    const int64_t sr = GATE_UP ? (int64_t)(sorted_rows[rt] / k) : (int64_t)rt;
    const u32x4 v = gload16(src + sr * K + min(col, K - 8));
    return col < K ? v : u32x4{0u, 0u, 0u, 0u};
  };
  // Loads in this order: the row indices, the scale-panel piece, the bias,
  // up to XP activation pieces of the first group, then the codes.  The
  // wait counter retires loads in issue order, so storing the staged pieces
  // waits for them alone while the codes stay in flight (issued first, the
  // codes would be waited for before the panel could be stored).
  constexpr int XP = 4;
  const int npanel = K / 16;                   // <= 192 pieces, one per thread
  const int nx0 = min(DG, tl.rows) * npieces;
  int xq[XP];
  int64_t xsr[XP];
#pragma unroll
  for (int u = 0; u < XP; ++u) xq[u] = min(tid + u * 64 * KW, nx0 - 1);
  int64_t f0 = 0;
  float wf0 = 0.0f;
  if (!GATE_UP) f0 = sorted_rows[tl.row0 + min(l32, tl.rows - 1)];
#pragma unroll
  for (int u = 0; u < XP; ++u) {
    const int rt = tl.row0 + xq[u] / npieces;
    xsr[u] = GATE_UP ? (int64_t)(sorted_rows[rt] / k) : (int64_t)rt;
  }
  const u32x4* ps = reinterpret_cast<const u32x4*>(scales + ((int64_t)e * N + rb * 32) * (K / 32));
  const u32x4 pv = gload16(ps + min(tid, npanel - 1));
  // the epilogue's bias pair, ahead of the codes so waiting for it does not
  // wait for them
  const int nbw = rb * 32 + 8 * wave + 4 * hlf;
  const void* bptr = bias ? static_cast<const void*>(bias + (int64_t)e * N + nbw) : static_cast<const void*>(g_zero64);
  const u32x2 bw0 = *(const __attribute__((address_space(1))) u32x2*)bptr;
  __builtin_amdgcn_sched_barrier(0);
  if (!GATE_UP) wf0 = topk_w[f0];
  u32x4 xv[XP];
#pragma unroll
  for (int u = 0; u < XP; ++u)
    xv[u] = gload16(src + xsr[u] * K + min((xq[u] % npieces) * 8, K - 8));
  __builtin_amdgcn_sched_barrier(0);
  u32x4 cv[KSTEPS];
#pragma unroll
  for (int i = 0; i < KSTEPS; ++i) {
    const int c = c0 + min(i, cnt - 1);               // clamped: never past the row
    const uint8_t* ptr = (ztail && c == nsteps - 1) ? g_zero64 : wrow + c * 32;
    cv[i] = gload16(ptr);
  }
  __builtin_amdgcn_sched_barrier(0);
  auto xstore = [&](int q, u32x4 v) {
    *reinterpret_cast<u32x4*>(xs + (q / npieces) * xrow + (q % npieces) * 8) = v;
  };
  reinterpret_cast<u32x4*>(panel)[min(tid, npanel - 1)] = pv;   // the clamped threads repeat the last piece
  // unconditional stores (a store under a branch lets the compiler sink its
  // load there, behind the codes); the clamped threads repeat the last piece
#pragma unroll
  for (int u = 0; u < XP; ++u)
    xstore(xq[u], (xq[u] % npieces) * 8 < K ? xv[u] : u32x4{0u, 0u, 0u, 0u});
  for (int q = tid + XP * 64 * KW; q < nx0; q += 64 * KW) xstore(q, xload(0, q));
  const uint8_t* srow = panel + l32 * (K / 32) + hlf;

  for (int g0 = 0; g0 < tl.rows; g0 += DG) {
    const int ng = min(DG, tl.rows - g0);
    if (g0 > 0)
      stage_lds<8>(ng * npieces, tid, 64 * KW, [&](int q) { return xload(g0, q); }, xstore);
    __syncthreads();
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const uint16_t* xb = xs + min(l32 % DG, ng - 1) * xrow + 32 * hlf;
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      if (i < cnt) {
        const int c = c0 + i;
        const float sc = scale_operand(srow[min(2 * c, smax)]);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const bf16x8 a = as_bf16x8(dequant8_bf16(cv[i][s4], sc));
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(xb + 64 * c + 8 * s4);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
      }
    }
    if (lora_B && wave == 0) {
      // + s v B_e^T over the rank, added to one wave's partial sum
      const float* vrow = lora_v + (int64_t)(tl.row0 + g0 + min(l32 % DG, ng - 1)) * lora_r;
      const uint16_t* brow = lora_B + ((int64_t)e * N + n) * lora_r;
      for (int j = 0; j < lora_chunks(lora_r); ++j) {
        bf16x8 vh, vl;
        lora_frag_split(vrow, lora_r, j, hlf, lora_scale, &vh, &vl);
        const bf16x8 bw = lora_frag(brow, lora_r, j, hlf);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw, vh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw, vl, acc, 0, 0, 0);
      }
    }
    __syncthreads();   // every wave is done reading xs
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[r];
    __syncthreads();
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < KW; ++w) sum += red[(w * 16 + 4 * wave + i) * 64 + lane];
      v[i] = sum;
    }
    // lane: column p = l32 of the group, weight rows nb + i
    const int p = g0 + l32;
    if (l32 < DG && p < tl.rows) {
      const int nb = nbw;
      {
        const u32x2 bw = bw0;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += bf16_to_f32((uint16_t)(bw[i >> 1] >> (16 * (i & 1))));
      }
      const int64_t rho = tl.row0 + p;
      if (GATE_UP) {
        const int I = N / 2;
        if (h_out) {
          u32x2 hv = {saved_preact_bf16(v[0], limit, false) | (saved_preact_bf16(v[1], limit, true) << 16),
                      saved_preact_bf16(v[2], limit, false) | (saved_preact_bf16(v[3], limit, true) << 16)};
          *reinterpret_cast<u32x2*>(h_out + rho * N + nb) = hv;
        }
        *reinterpret_cast<uint32_t*>(a_out + rho * I + nb / 2) =
            pack_bf16x2(swiglu(v[0], v[1], alpha, limit), swiglu(v[2], v[3], alpha, limit));
      } else {
        const int64_t f = g0 == 0 ? f0 : (int64_t)sorted_rows[rho];
        const float wf = g0 == 0 ? wf0 : topk_w[f];
        const u32x2 y = {pack_bf16x2(wf * v[0], wf * v[1]), pack_bf16x2(wf * v[2], wf * v[3])};
        *reinterpret_cast<u32x2*>(y_w + f * N + nb) = y;
      }
    }
    __syncthreads();   // LDS is restaged for the next group
  }
}

// Launch shape from the routed-row count: few rows -> 4 waves (128 weight
// rows) per workgroup; more rows -> 8 waves (256 weight rows, gate_up) or 4
// with the group staged in segments of K (down), sharing one staging of the
// activation group (at most R rows, 8 or 16 at a time).  Splitting K over
// waves measured slower.
template <bool GATE_UP>
static hipError_t dec_launch_stream(int64_t R, int max_tiles, int K, int N, hipStream_t s,
                             const uint16_t* src, const uint8_t* codes, const uint8_t* scales,
                             const uint16_t* bias, const float* topk_w,
                             const int32_t* sorted_rows, const Tile* tiles,
                             const int32_t* num_tiles, int k, float alpha, float limit,
                             uint16_t* h_out, uint16_t* a_out, uint16_t* y_w,
                             const uint16_t* lora_B, const float* lora_v, float lora_scale,
                             int lora_r) {
  if (K % 32 || K > DEC_MAXK || N % 32) return hipErrorInvalidValue;
  const int Kp = (K + 63) & ~63;
  const int nch = (Kp / 64 + DD - 1) / DD;
  // More rows: groups of 16.  gate_up: 8 waves share the whole-K staging
  // (one workgroup per CU).  down: 4 waves, the group staged two chunks of
  // K at a time, so that two workgroups fit a CU's LDS and one's staging and
  // epilogue overlap the other's stream (measured faster for down, slower
  // for gate_up, whose epilogue and grid are twice as large).
  const bool seg = R > 64 && !GATE_UP;
  const int wpb = R > 64 && GATE_UP ? 8 : 4;
  const int dg = R <= 64 ? (int)(R < 8 ? R : 8) : 16;   // an expert owns at most R rows
  const int seg_ch = seg ? 2 : nch;
  const int xcols = seg_ch * DD * 64 < Kp ? seg_ch * DD * 64 : Kp;
  // one staging pass of at most 12 pieces per thread, even segments
  if (dg * (xcols / 8) > 12 * 64 * wpb || (seg_ch < nch && seg_ch % 2)) return hipErrorInvalidValue;
  const int nblk = (N + 32 * wpb - 1) / (32 * wpb);
  const size_t lds = (size_t)32 * wpb * (K / 32) + (size_t)dg * (xcols + DEC_XPAD) * 2;
  // dynamic LDS above 64 KB (16 staged rows) must be allowed explicitly
  static bool lds_attr_set = false;
  if (!lds_attr_set) {
    const int most = 16 * (DEC_MAXK + DEC_XPAD) * 2 + 256 * (DEC_MAXK / 32);
    const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&dec_kernel<GATE_UP>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, most);
    if (err != hipSuccess) return err;
    lds_attr_set = true;
  }
  const dim3 grid(max_tiles * nblk), block(64 * wpb);
#define DEC_ARGS src, codes, scales, bias, topk_w, sorted_rows, tiles, num_tiles, K, N, k, dg, \
                 seg_ch, alpha, limit, h_out, a_out, y_w, lora_B, lora_v, lora_scale, lora_r
  hipLaunchKernelGGL((dec_kernel<GATE_UP>), grid, block, lds, s, DEC_ARGS);
#undef DEC_ARGS
  return hipGetLastError();
}

template <bool GATE_UP>
static hipError_t dec_launch(int64_t R, int max_tiles, int K, int N, hipStream_t s,
                             const uint16_t* src, const uint8_t* codes, const uint8_t* scales,
                             const uint16_t* bias, const float* topk_w,
                             const int32_t* sorted_rows, const Tile* tiles,
                             const int32_t* num_tiles, int k, float alpha, float limit,
                             uint16_t* h_out, uint16_t* a_out, uint16_t* y_w,
                             const uint16_t* lora_B, const float* lora_v, float lora_scale,
                             int lora_r) {
  if (K % 32 || K > DEC_MAXK || N % 32 || (lora_B && !lora_rank_ok(lora_r)))
    return hipErrorInvalidValue;
  if (R <= 16) {
    const int dg = (int)(R < 8 ? R : 8);
    const int Kp = (K + 63) & ~63;
    const size_t xb = (size_t)dg * (Kp + DEC_XPAD) * 2, rb = (size_t)KW * 16 * 64 * 4;
    hipLaunchKernelGGL(dec_ksplit_kernel<GATE_UP>, dim3(max_tiles * (N / 32)), dim3(64 * KW),
                       (size_t)K + (xb > rb ? xb : rb), s, src, codes, scales, bias, topk_w,
                       sorted_rows, tiles, num_tiles, K, N, k, dg, alpha, limit, h_out, a_out,
                       y_w, lora_B, lora_v, lora_scale, lora_r);
    return hipGetLastError();
  }
  return dec_launch_stream<GATE_UP>(R, max_tiles, K, N, s, src, codes, scales, bias, topk_w,
                                    sorted_rows, tiles, num_tiles, k, alpha, limit, h_out, a_out,
                                    y_w, lora_B, lora_v, lora_scale, lora_r);
}

hipError_t launch_dec_gate_up(const uint16_t* x, const uint8_t* codes, const uint8_t* scales,
                              const uint16_t* bias, const int32_t* sorted_rows, const Tile* tiles,
                              const int32_t* num_tiles, int max_tiles, int64_t R, int H, int I, int k,
                              float alpha, float limit, const uint16_t* lora_B,
                              const float* lora_v, float lora_scale, int lora_r, uint16_t* h_out,
                              uint16_t* a_out, hipStream_t s) {
  return dec_launch<true>(R, max_tiles, H, 2 * I, s, x, codes, scales, bias, nullptr, sorted_rows,
                          tiles, num_tiles, k, alpha, limit, h_out, a_out, nullptr, lora_B, lora_v,
                          lora_scale, lora_r);
}

hipError_t launch_dec_down(const uint16_t* a, const uint8_t* codes, const uint8_t* scales,
                           const uint16_t* bias, const float* topk_w, const int32_t* sorted_rows,
                           const Tile* tiles, const int32_t* num_tiles, int max_tiles, int64_t R,
                           int H, int I, const uint16_t* lora_B, const float* lora_v,
                           float lora_scale, int lora_r, uint16_t* y_w, hipStream_t s) {
  return dec_launch<false>(R, max_tiles, I, H, s, a, codes, scales, bias, topk_w, sorted_rows,
                           tiles, num_tiles, 1, 0.0f, 0.0f, nullptr, nullptr, y_w, lora_B, lora_v,
                           lora_scale, lora_r);
}

}  // namespace mxmoe
