// Router (logits, top-k, softmax over the selected k), expert histogram,
// exclusive scan and the stable token permutation (gfx950).
//
// The pages ("Add MXFP4 training support via a dequantize-on-the-fly
// fallback", "What this does") run a top-k router before the per-expert
// loop; the finegrained-kernels note on the bias operand describes the
// grouped path that orders routed rows by expert.  Here the logits come
// from the fp64 matrix cores (exact products, fp64 sums, one rounding to
// fp32), and the permutation is a deterministic counting sort: per-
// workgroup histograms, one scan over (expert, workgroup), then each
// workgroup scatters its rows in ascending flat-row order.  For few routed
// rows (decode sizes) the logits are split over many workgroups as fp64
// partial sums, and one workgroup then does the sums, top-k, counts, scan,
// permutation and the tile list.  No atomics on global memory, and every
// sum in a fixed order, so the result is identical run to run.
#include "common.hpp"
#include "launch.hpp"

namespace mxmoe {

constexpr int RT = ROUTER_TOKENS;

int router_blocks(int64_t T) { return (int)((T + RT - 1) / RT); }

// Router logits on the fp64 matrix cores.  l[t, e] = sum_h x[t, h] Wr[e, h]
// + b[e]: the bf16 x fp32 products are exact in fp64 and are summed in fp64,
// then the logit is rounded once to fp32 (the routing decision is taken on
// that value).  A workgroup of LG_W waves computes one 16-token x 16-expert
// tile with v_mfma_f64_16x16x4f64, wave w over the w-th of LG_W contiguous
// ranges of h: lane l feeds A[i = l%16][kk = l/16] (token i) and B[kk][j =
// l%16] (expert j) and holds D[4r + l/16][l%16] in register r.  The
// contraction index of MFMA step s is mapped to h = base + 8*kk + s, so
// over 8 steps a lane reads 8 consecutive h of its token row and of its
// expert row (one 16-byte and one 32-byte load per 32 h).  The LG_W partial
// tiles are summed through LDS in wave order.  Rows past T or E are clamped
// and dropped.
constexpr int LG_CH = 32;   // h per chunk (8 MFMA steps of 4)
constexpr int LG_W = 16;    // waves per workgroup (h ranges)
constexpr int LG_P = 6;     // chunks a logits_kernel wave has in flight (H <= 3072: all)
constexpr int LP_P = 8;     // chunks a logits_part_kernel wave has in flight

__device__ __forceinline__ void lg_load(const uint16_t* xp, const float* wp, int c, u32x4& xv,
                                        f32x4& w0, f32x4& w1) {
  xv = *reinterpret_cast<const u32x4*>(xp + c * LG_CH);
  w0 = *reinterpret_cast<const f32x4*>(wp + c * LG_CH);
  w1 = *reinterpret_cast<const f32x4*>(wp + c * LG_CH + 4);
}

__device__ __forceinline__ void lg_mfma(const u32x4& xv, const f32x4& w0, const f32x4& w1,
                                        f64x4& acc) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const uint32_t xw = xv[s >> 1];
    const float xf = __uint_as_float((s & 1) ? (xw & 0xFFFF0000u) : (xw << 16));
    const float wf = (s < 4) ? w0[s] : w1[s - 4];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xf, (double)wf, acc, 0, 0, 0);
  }
}

__global__ __launch_bounds__(64 * LG_W) void logits_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ wr,
                                                           const float* __restrict__ br, int T,
                                                           int H, int E,
                                                           float* __restrict__ logits) {
  __shared__ double red[LG_W][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntt = (T + 15) / 16;
  const int tt = blockIdx.x % ntt, et = blockIdx.x / ntt;
  const int nch = H / LG_CH;
  const int c0 = wave * nch / LG_W, c1 = (wave + 1) * nch / LG_W;
  const int i = lane & 15, kk = lane >> 4;
  const int t = min(tt * 16 + i, T - 1), e = min(et * 16 + i, E - 1);
  const uint16_t* xp = x + (int64_t)t * H + 8 * kk;
  const float* wp = wr + (int64_t)e * H + 8 * kk;
  // all of this wave's loads first (up to LG_P chunks at a time), then the
  // MFMAs: chunk c - c0 into accumulator (c - c0) mod 4 (four independent
  // chains), added in a fixed order at the end
  f64x4 acc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int cb = c0; cb < c1; cb += LG_P) {
    u32x4 xv[LG_P];
    f32x4 w0[LG_P], w1[LG_P];
#pragma unroll
    for (int q = 0; q < LG_P; ++q) lg_load(xp, wp, min(cb + q, c1 - 1), xv[q], w0[q], w1[q]);
#pragma unroll
    for (int q = 0; q < LG_P; ++q)
      if (cb + q < c1) lg_mfma(xv[q], w0[q], w1[q], acc[q % 4]);
  }
  const f64x4 sum4 = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][r][lane] = sum4[r];
  __syncthreads();
  if (wave == 0) {
    const int ex = et * 16 + i;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = tt * 16 + 4 * r + kk;
      double sum = 0.0;
#pragma unroll
      for (int w = 0; w < LG_W; ++w) sum += red[w][r][lane];
      if (tok < T && ex < E) logits[(int64_t)tok * E + ex] = (float)(sum + (br ? (double)br[ex] : 0.0));
    }
  }
}

// Router logits for few tokens (the planned path).  The same 16x16 fp64
// MFMA tiles as logits_kernel, but one wave per (tile, range of h) and
// many workgroups, so the router weights stream through many CUs at once:
// part[hs][t][e] is range hs's fp64 partial sum, and plan_kernel adds the
// ranges in order, adds the bias and rounds once to fp32.  Within a range,
// chunk c - c0 goes to accumulator (c - c0) mod 4 (four independent MFMA
// chains instead of one), and the four are added in a fixed order.  With
// few ranges (many logits: the plan's LDS bounds ranges x logits) the
// workgroup has LPW waves, each over a contiguous sub-range, whose sums
// are added in wave order through LDS.
constexpr int LPW = 4;
__global__ __launch_bounds__(64 * LPW) void logits_part_kernel(const uint16_t* __restrict__ x,
                                                               const float* __restrict__ wr, int T,
                                                               int H, int E, int hs_parts,
                                                               double* __restrict__ part) {
  __shared__ double red[LPW][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int ntt = (T + 15) / 16;
  const int hs = blockIdx.x % hs_parts, tile = blockIdx.x / hs_parts;
  const int tt = tile % ntt, et = tile / ntt;
  const int nch = H / LG_CH;
  const int r0 = hs * nch / hs_parts, r1 = (hs + 1) * nch / hs_parts;
  const int c0 = r0 + wave * (r1 - r0) / nw, c1 = r0 + (wave + 1) * (r1 - r0) / nw;
  const int i = lane & 15, kk = lane >> 4;
  const int t = min(tt * 16 + i, T - 1), e = min(et * 16 + i, E - 1);
  const uint16_t* xp = x + (int64_t)t * H + 8 * kk;
  const float* wp = wr + (int64_t)e * H + 8 * kk;
  f64x4 acc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) acc[a] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int cb = c0; cb < c1; cb += LP_P) {
    u32x4 xv[LP_P];
    f32x4 w0[LP_P], w1[LP_P];
    // only the chunks that exist are loaded (a range holds few chunks when
    // there are many ranges; the guard is uniform)
#pragma unroll
    for (int q = 0; q < LP_P; ++q)
      if (cb + q < c1) lg_load(xp, wp, cb + q, xv[q], w0[q], w1[q]);
#pragma unroll
    for (int q = 0; q < LP_P; ++q)
      if (cb + q < c1) lg_mfma(xv[q], w0[q], w1[q], acc[q % 4]);
  }
  f64x4 sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  if (nw > 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][r][lane] = sum[r];
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      double v = red[0][r][lane];
      for (int w = 1; w < nw; ++w) v += red[w][r][lane];
      sum[r] = v;
    }
  }
  const int ex = et * 16 + i;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tok = tt * 16 + 4 * r + kk;
    if (tok < T && ex < E) part[((int64_t)hs * T + tok) * E + ex] = sum[r];
  }
}

// Ranges of h per 16x16 logit tile in logits_part_kernel: about 128 waves
// in all, at most 64 ranges and at least one 32-element chunk of h per
// range, and at most PLAN_PARTS partial sums (plan_kernel stages them all
// in LDS).  The planned path requires T*E <= PLAN_LOGITS <= PLAN_PARTS.
constexpr int PLAN_PARTS = 16384;
constexpr int PLAN_LOGITS = 4096;
int plan_hs_parts(int T, int E, int H) {
  const int tiles = ((T + 15) / 16) * ((E + 15) / 16);
  int hs = min(128 / tiles, 64);
  hs = min(hs, PLAN_PARTS / (T * E));
  hs = min(hs, H / LG_CH);
  return max(hs, 1);
}

// Total-order key of a logit for the top-k: larger key = larger logit,
// -0.0 and +0.0 equal, and NaN below every number (-inf included), all NaNs
// equal.  Ties then go to the lower expert index, which is the order of a
// stable sort of the negated logits with NaN last.  On keys, "beats" is a
// strict total order, so the k selected experts are always distinct and
// every token adds exactly k rows to the histogram, whatever its values.
__device__ __forceinline__ int32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;   // -0.0 -> +0.0
  const int32_t b = (int32_t)u;
  return (f != f) ? INT32_MIN : (b ^ ((b >> 31) & 0x7FFFFFFF));
}

// The logit back from its key (exact for numbers; -0.0 comes back as +0.0,
// a NaN key as a NaN).
__device__ __forceinline__ float key_value(int32_t k) {
  return __uint_as_float((uint32_t)(k ^ ((k >> 31) & 0x7FFFFFFF)));
}

// Top-k and softmax of token t by one wave, from its row lt of E logit keys
// (order_key) in LDS, without a cross-lane reduction per selection round (a
// chain of wave shuffles per round measured several times slower): lane l
// owns experts l + 64q (q < NQ = ceil(E / 64), a template parameter, since
// this count loop is VALU-bound) and counts, for each, the experts that
// beat it (a larger key, or an equal one with a lower index).  The expert
// with count j < k is slot j: the k largest logits in descending order,
// ties to the lower index.  With E <= 32 the two wave halves split the row
// (16 compares per lane, one shuffle to add the halves).  Otherwise the row
// is read in chunks of 32 keys, all of a chunk's LDS reads issued before
// the first compare (one wait per chunk), and the counts use integer masks,
// not branches (8-logit chunks with guarded compares measured 1.8 us per
// token for E = 32).  The selected logits go through the wave's LDS slots
// zs[8]; lane j < k forms the softmax denominator over them in slot order
// (exponents relative to slot 0, the same sum in every lane) and writes
// slot j's weight.  With `ex` (LDS) slot (t, j)'s expert is also recorded
// there; with `hist` (LDS) each selected expert is counted.
template <int NQ>
__device__ __forceinline__ void topk_rank(const int32_t* lt, int E, int k, int t, int lane,
                                          int32_t* __restrict__ topk_idx,
                                          float* __restrict__ topk_w, int32_t* ex, int32_t* hist,
                                          float* zs) {
  int32_t v[NQ];
  int rank[NQ];
  if (NQ == 1 && E <= 32) {
    // both halves of the wave: lane l takes expert l mod 32 against half
    // l / 32 of the row (16 logits), and the two partial counts are added
    // (lanes 32..63 own no expert: l >= 32 >= E)
    const int e = lane & 31, h = lane >> 5;
    const int32_t ve = lt[min(e, E - 1)];
    int32_t o[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) o[j] = lt[min(16 * h + j, E - 1)];
    int r = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e2 = 16 * h + j;
      const int beats = (int)(o[j] > ve) | ((int)(o[j] == ve) & (int)(e2 < e));
      r += (int)(e2 < E) & beats;
    }
    r += __shfl_xor(r, 32);
    v[0] = ve;
    rank[0] = r;
  } else {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      v[q] = lt[min(lane + 64 * q, E - 1)];
      rank[q] = 0;
    }
  }
  for (int b0 = (NQ == 1 && E <= 32) ? E : 0; b0 < E; b0 += 32) {
    int32_t o[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) o[j] = lt[min(b0 + j, E - 1)];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int e2 = b0 + j;
      const int live = e2 < E;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int beats = (int)(o[j] > v[q]) | ((int)(o[j] == v[q]) & (int)(e2 < lane + 64 * q));
        rank[q] += live & beats;
      }
    }
  }
  wave_lds_sync();   // the previous token's zs reads are done
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = lane + 64 * q;
    if (e < E && rank[q] < k) {
      const int64_t f = (int64_t)t * k + rank[q];
      topk_idx[f] = e;
      if (ex) ex[f] = e;
      if (hist) atomicAdd(&hist[e], 1);   // counts only: order does not matter
      zs[rank[q]] = key_value(v[q]);
    }
  }
  wave_lds_sync();
  if (lane < k) {
    const float sel0 = zs[0];
    float zsum = 0.0f, zl = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        const float z = expf(zs[j] - sel0);
        zsum += z;
        if (j == lane) zl = z;
      }
    }
    topk_w[(int64_t)t * k + lane] = zl / zsum;
  }
}

// RT tokens per workgroup (rank-count selection on the tokens' logits
// staged in LDS; with E <= 64 all of the block's (token, expert) pairs at
// once); writes the workgroup's expert histogram for the scan.
template <int NQ>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_w,
                                                   int32_t* __restrict__ blk_hist) {
  __shared__ int32_t hist[256];
  __shared__ int32_t lgs[RT * 256];   // logit keys
  __shared__ float zr[RT * 8];        // the selected logits, [token][rank]
  __shared__ float zs[4][8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT;
  const int nt = min(RT, T - t0);
  hist[tid] = 0;
  {
    const int n = nt * E;   // the block's logits are contiguous
    float v[RT];
#pragma unroll
    for (int u = 0; u < RT; ++u) v[u] = logits[(int64_t)t0 * E + min(tid + u * 256, n - 1)];
#pragma unroll
    for (int u = 0; u < RT; ++u)
      if (tid + u * 256 < n) lgs[tid + u * 256] = order_key(v[u]);
  }
  __syncthreads();
  if (NQ > 1) {
    // many experts: two tokens per wave, each lane ranking NQ experts
    // against the row read 32 keys at a time
#pragma unroll
    for (int q = 0; q < RT / 4; ++q) {
      const int i = wave * (RT / 4) + q;
      if (i < nt) topk_rank<NQ>(lgs + i * E, E, k, t0 + i, lane, topk_idx, topk_w, nullptr, hist, zs[wave]);
    }
    __syncthreads();
    if (tid < E) blk_hist[(int64_t)blockIdx.x * E + tid] = hist[tid];
    return;
  }
  // E <= 64: every (token, expert) pair of the block at once: the pair's
  // rank among the token's row (a larger key, or an equal key and a lower
  // index beats it); ranked below k it fills slot rank of the token
  for (int q = tid; q < nt * E; q += 256) {
    const int i = q / E, e = q - i * E;
    const int32_t* row = lgs + i * E;
    const int32_t ve = row[e];
    int r = 0;
#pragma unroll 8
    for (int e2 = 0; e2 < E; ++e2) {
      const int32_t o = row[e2];
      r += (int)(o > ve) | ((int)(o == ve) & (int)(e2 < e));
    }
    if (r < k) {
      topk_idx[(int64_t)(t0 + i) * k + r] = e;
      zr[i * 8 + r] = key_value(ve);
      atomicAdd(&hist[e], 1);   // counts only: order does not matter
    }
  }
  __syncthreads();
  // the softmax over each token's k selected logits, added in rank order
  if (tid < nt * k) {
    const int i = tid / k, j = tid - i * k;
    const float* z = zr + i * 8;
    const float sel0 = z[0];
    float zsum = 0.0f, zl = 0.0f;
    for (int m = 0; m < k; ++m) {
      const float zm = expf(z[m] - sel0);
      zsum += zm;
      if (m == j) zl = zm;
    }
    topk_w[(int64_t)t0 * k + tid] = zl / zsum;
  }
  if (tid < E) blk_hist[(int64_t)blockIdx.x * E + tid] = hist[tid];
}

// Few routed rows (R = T*k <= PLAN_MAX_ROWS, so T <= 256): the logits from
// logits_part_kernel's partial sums, top-k (topk_rank), expert counts, offsets, the
// stable permutation and the tile list in one workgroup of 1024 threads
// (16 waves), with T*E <= PLAN_LOGITS so the logits stay in LDS.  Counts
// and ranks come
// from wave ballots over the flat rows in ascending order, so row f = (t,
// j) of expert e lands at offsets[e] + (number of earlier rows routed to
// e): ascending f within an expert.
__global__ __launch_bounds__(1024) void plan_kernel(
    const double* __restrict__ part, int hs_parts, const float* __restrict__ br, int T, int E,
    int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_rows, Tile* __restrict__ tiles,
    int32_t* __restrict__ num_tiles) {
  __shared__ int32_t lg[PLAN_LOGITS];   // logit keys
  __shared__ double pst[PLAN_PARTS];
  __shared__ float brs[256];             // the router bias (E <= 256)
  __shared__ float zr[PLAN_MAX_ROWS];    // the selected logits, slot t * k + rank
  __shared__ int32_t ex[PLAN_MAX_ROWS];
  __shared__ int32_t cnt[256];
  __shared__ int32_t off[257];
  __shared__ int32_t tstart[257];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int TE = T * E, R = T * k;
  // every partial sum into LDS (up to 16 independent loads per thread),
  // then each logit's ranges added in order (16 LDS reads in flight)
  const int P = hs_parts * TE;
  {
    double v[PLAN_PARTS / 1024];   // all loads issued before the first store
    const int nu = (P + 1023) / 1024;   // load rounds needed (uniform)
#pragma unroll
    for (int u = 0; u < PLAN_PARTS / 1024; ++u)
      if (u < nu) v[u] = part[min(tid + u * 1024, P - 1)];
    // the bias with the partials: one memory round trip for both
    if (tid < E) brs[tid] = br ? br[tid] : 0.0f;
#pragma unroll
    for (int u = 0; u < PLAN_PARTS / 1024; ++u)
      if (u < nu && tid + u * 1024 < P) pst[tid + u * 1024] = v[u];
  }
  __syncthreads();
  if (TE > 512) {
    for (int q = tid; q < TE; q += 1024) {
      double sum = 0.0;
      for (int h0 = 0; h0 < hs_parts; h0 += 16) {
        double v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = pst[min(h0 + j, hs_parts - 1) * TE + q];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (h0 + j < hs_parts) sum += v[j];
      }
      lg[q] = order_key((float)(sum + (double)brs[q % E]));
    }
  } else {
    // few logits: G consecutive lanes per logit (G = 2 .. 16, G * TE <=
    // 1024); lane g sums ranges g, g + G, ... in order, and an xor-shuffle
    // tree adds the group's sums (each step adds the same two values in
    // every lane of a pair, so all lanes hold the same, fixed-order total)
    const int G = TE > 256 ? 2 : TE > 128 ? 4 : TE > 64 ? 8 : 16;
    const int q = tid / G, g = tid % G;
    double sum = 0.0;
    if (q < TE) {
      for (int h0 = g; h0 < hs_parts; h0 += 16 * G) {
        double v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = pst[min(h0 + j * G, hs_parts - 1) * TE + q];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (h0 + j * G < hs_parts) sum += v[j];
      }
    }
    for (int m = 1; m < G; m <<= 1) sum += __shfl_xor(sum, m);
    if (q < TE && g == 0) lg[q] = order_key((float)(sum + (double)brs[q % E]));
  }
  __syncthreads();
  // Top-k of every token at once: thread (t, e) counts the experts that
  // beat e in token t's row (a larger key, or an equal key and a lower
  // index) and, ranked below k, fills slot t * k + rank.
  for (int q = tid; q < TE; q += 1024) {
    const int t = q / E, e = q - t * E;
    const int32_t* row = lg + t * E;
    const int32_t ve = row[e];
    int r = 0;
#pragma unroll 8
    for (int e2 = 0; e2 < E; ++e2) {
      const int32_t o = row[e2];
      r += (int)(o > ve) | ((int)(o == ve) & (int)(e2 < e));
    }
    if (r < k) {
      const int f = t * k + r;
      topk_idx[f] = e;
      ex[f] = e;
      zr[f] = key_value(ve);
    }
  }
  __syncthreads();
  // the softmax over each token's k selected logits (rank 0 is the largest),
  // terms added in rank order
  if (tid < R) {
    const int t = tid / k, j = tid - t * k;
    const float* z = zr + t * k;
    const float sel0 = z[0];
    float zsum = 0.0f, zl = 0.0f;
    for (int i = 0; i < k; ++i) {
      const float zi = expf(z[i] - sel0);
      zsum += zi;
      if (i == j) zl = zi;
    }
    topk_w[tid] = zl / zsum;
  }
  for (int e = wave; e < E; e += 16) {
    int c = 0;
    for (int f0 = 0; f0 < R; f0 += 64) {
      const int f = f0 + lane;
      c += __popcll(__ballot(f < R && ex[f] == e));
    }
    if (lane == 0) cnt[e] = c;
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scans of the counts and of the tiles per expert; lane l
    // owns experts 4l .. 4l+3
    int c[4], tc[4], sc = 0, st = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      c[q] = e < E ? cnt[e] : 0;
      tc[q] = (c[q] + MT - 1) / MT;
      sc += c[q];
      st += tc[q];
    }
    int ic = sc, it = st;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int oc = __shfl_up(ic, d), ot = __shfl_up(it, d);
      if (lane >= d) { ic += oc; it += ot; }
    }
    int rc = ic - sc, rt = it - st;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      if (e < E) { off[e] = rc; tstart[e] = rt; }
      rc += c[q];
      rt += tc[q];
    }
    if (lane == 63) {
      off[E] = ic;
      *num_tiles = it;
    }
  }
  __syncthreads();
  if (tid <= E) offsets[tid] = off[tid];
  if (tid < E) {
    const int32_t n = cnt[tid];
    for (int32_t q = 0; q * MT < n; ++q) {
      Tile tl;
      tl.expert = tid;
      tl.row0 = off[tid] + q * MT;
      tl.rows = min(MT, n - q * MT);
      tl.pos = tile_pos(q, (n + MT - 1) / MT);
      tiles[tstart[tid] + q] = tl;
    }
  }
  for (int e = wave; e < E; e += 16) {
    int base = off[e];
    for (int f0 = 0; f0 < R; f0 += 64) {
      const int f = f0 + lane;
      const bool m = f < R && ex[f] == e;
      const unsigned long long b = __ballot(m);
      if (m) sorted_rows[base + __popcll(b & ((1ull << lane) - 1ull))] = f;
      base += __popcll(b);
    }
  }
}

// Tile lists from the E + 1 offsets in LDS (offs); start is LDS scratch of
// E + 1 entries.  Called by every thread of one workgroup; ends with the
// list written.
//
// write_tiles: tiles of at most mt sorted rows, expert by expert (the
// forward's list: its GEMMs give each XCD a contiguous range of it).
// Exclusive scan of cnt(e) over e < E (E <= 256) by one wave: lane l owns
// e = 4l .. 4l + 3; out[e] = sum of cnt(e') over e' < e, out[E] = the total,
// which is also returned to every lane.
template <class Cnt>
__device__ __forceinline__ int32_t wave_scan_experts(int E, int lane, Cnt cnt, int32_t* out) {
  int32_t c[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * lane + q;
    c[q] = e < E ? cnt(e) : 0;
    sum += c[q];
  }
  int32_t inc = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t o = __shfl_up(inc, d);
    if (lane >= d) inc += o;
  }
  int32_t run = inc - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * lane + q;
    if (e < E) out[e] = run;
    run += c[q];
  }
  const int32_t total = __shfl(inc, 63);
  if (lane == 0) out[E] = total;
  return total;
}

__device__ __forceinline__ void write_tiles(const int32_t* offs, int E, int mt, int32_t* start,
                                            Tile* __restrict__ tiles,
                                            int32_t* __restrict__ num_tiles) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int32_t total = wave_scan_experts(
        E, tid, [&](int e) { return (offs[e + 1] - offs[e] + mt - 1) / mt; }, start);
    if (tid == 0) *num_tiles = total;
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    const int32_t o = offs[e], n = offs[e + 1] - o;
    const int32_t nt = (n + mt - 1) / mt;
    for (int32_t q = 0; q < nt; ++q)
      tiles[start[e] + q] = Tile{e, o + q * mt, min(mt, n - q * mt), tile_pos(q, nt)};
  }
  __syncthreads();
}

// write_dealt_tiles: the same tiles in the order the backward GEMMs deal
// them to the 8 XCDs.  XCD x's tiles sit at x, 8 + x, 16 + x, ... (a
// workgroup on XCD x reads only those).  The F full tiles (expert by
// expert) are split into 8 contiguous ranges, one per XCD, so the row tiles
// of an expert that run together share its weights in one L2.  Each
// expert's ragged last tile then follows, dealt longest first (rows
// descending, ties by expert) in snake order (round r runs over the XCDs
// downward when r is even, upward when odd, starting with the XCDs whose
// full range is one shorter), so the XCDs' totals balance and every XCD
// ends on its shortest tiles.  Slots past an XCD's share up to the longest
// share hold empty tiles (rows = 0); *num_tiles = 8 x the longest share.
struct TileDeal {
  int full_base, full_ext, ragged;   // F / 8, F % 8, number of ragged tiles
  __device__ int full_count(int x) const { return full_base + (x < full_ext); }
  __device__ int ragged_xcd(int j) const {
    const int r = j >> 3, pos = j & 7;
    return (r & 1) ? pos : 7 - pos;
  }
  __device__ int ragged_count(int x) const {
    int n = ragged >> 3;
    for (int pos = 0; pos < (ragged & 7); ++pos) n += ragged_xcd(8 * (ragged >> 3) + pos) == x;
    return n;
  }
  // XCD x's range of full tiles [full_lo(x), full_lo(x) + full_count(x))
  __device__ int full_lo(int x) const {
    return x < full_ext ? x * (full_base + 1) : full_ext * (full_base + 1) + (x - full_ext) * full_base;
  }
  __device__ int full_xcd(int i) const {
    const int boundary = full_ext * (full_base + 1);
    return i < boundary ? i / (full_base + 1) : full_ext + (i - boundary) / full_base;
  }
  // list index of full tile i (0 <= i < F)
  __device__ int full_slot(int i) const {
    const int boundary = full_ext * (full_base + 1);
    int x, q;
    if (i < boundary) {
      x = i / (full_base + 1);
      q = i % (full_base + 1);
    } else {
      x = full_ext + (i - boundary) / full_base;
      q = (i - boundary) % full_base;
    }
    return 8 * q + x;
  }
  // list index of the ragged tile of rank j
  __device__ int ragged_slot(int j) const {
    const int x = ragged_xcd(j);
    return 8 * (full_count(x) + (j >> 3)) + x;
  }
};

__device__ __forceinline__ void write_dealt_tiles(const int32_t* offs, int E, int mt,
                                                  int32_t* start, Tile* __restrict__ tiles,
                                                  int32_t* __restrict__ num_tiles) {
  const int tid = threadIdx.x;
  __shared__ TileDeal deal;
  __shared__ int32_t rems[256];   // each expert's ragged tile rows (0: none)
  for (int e = tid; e < E; e += blockDim.x) rems[e] = (offs[e + 1] - offs[e]) % mt;
  if (tid < 64) {
    const int lane = tid;
    const int32_t run = wave_scan_experts(
        E, lane, [&](int e) { return (offs[e + 1] - offs[e]) / mt; }, start);
    int32_t rg = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * lane + q;
      rg += e < E && (offs[e + 1] - offs[e]) % mt != 0;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) rg += __shfl_xor(rg, m);
    const TileDeal d{run >> 3, run & 7, rg};
    // lane x < 8: XCD x's tile count; the longest share over the 8 lanes
    const int cnt = lane < 8 ? d.full_count(lane) + d.ragged_count(lane) : 0;
    int longest = cnt;
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) longest = max(longest, __shfl_xor(longest, m));
    if (lane < 8)
      for (int q = cnt; q < longest; ++q) tiles[8 * q + lane] = Tile{0, 0, 0, 0};
    if (lane == 0) {
      *num_tiles = 8 * longest;
      deal = d;
    }
  }
  __syncthreads();
  const TileDeal d = deal;
  for (int e = tid; e < E; e += blockDim.x) {
    const int32_t o = offs[e], n = offs[e + 1] - o;
    const int32_t nfull = n / mt, rem = n % mt;
    // an expert's full tiles on one XCD form a run of consecutive slots; a
    // tile records its index in the run and the run's length (the GEMMs
    // order a run's items row tile fastest)
    for (int32_t q = 0; q < nfull; ++q) {
      const int i = start[e] + q, x = d.full_xcd(i);
      const int lo = max(start[e], d.full_lo(x));
      const int hi = min(start[e] + nfull, d.full_lo(x) + d.full_count(x));
      tiles[d.full_slot(i)] = Tile{e, o + q * mt, mt, tile_pos(i - lo, hi - lo)};
    }
    if (rem) {
      int32_t rank = 0;
      for (int e2 = 0; e2 < E; ++e2) {
        const int32_t r2 = rems[e2];
        rank += (r2 > rem) || (r2 == rem && e2 < e);
      }
      tiles[d.ragged_slot(rank)] = Tile{e, o + nfull * mt, rem, tile_pos(0, 1)};
    }
  }
  __syncthreads();
}

// One workgroup of 1024 threads.  In place, blk_hist[b][e] becomes the
// first sorted position of workgroup b's rows of expert e:
// offsets[e] + sum_{b' < b} count[b'][e].  offsets = exclusive scan of the
// expert totals (E + 1 entries).
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ blk_hist, int nblk,
                                                    int E, int32_t* __restrict__ offsets,
                                                    Tile* __restrict__ tiles,
                                                    int32_t* __restrict__ num_tiles) {
  __shared__ int32_t part[1024];
  __shared__ int32_t total[256];
  __shared__ int32_t off[257];
  __shared__ int32_t tstart[257];
  const int tid = threadIdx.x;
  const int C = 1024 / E;                    // chunks of workgroups
  const int per = (nblk + C - 1) / C;
  const int e = tid % E, c = tid / E;
  int32_t sum = 0;
  if (c < C) {
    const int b1 = min(nblk, (c + 1) * per);
    for (int b0 = c * per; b0 < b1; b0 += 16) {   // 16 loads in flight
      int32_t v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = blk_hist[(int64_t)min(b0 + u, b1 - 1) * E + e];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (b0 + u < b1) sum += v[u];
    }
  }
  part[tid] = sum;
  __syncthreads();
  if (tid < E) {
    int32_t run = 0;
    for (int cc = 0; cc < C; ++cc) {
      int32_t v = part[cc * E + tid];
      part[cc * E + tid] = run;
      run += v;
    }
    total[tid] = run;
  }
  __syncthreads();
  if (tid == 0) {
    int32_t run = 0;
    for (int ee = 0; ee < E; ++ee) { off[ee] = run; run += total[ee]; }
    off[E] = run;
  }
  __syncthreads();
  if (tid <= E) offsets[tid] = off[tid];
  // the GEMMs' tile list from the offsets (no separate launch)
  write_tiles(off, E, MT, tstart, tiles, num_tiles);
  if (c < C) {
    int32_t run = off[e] + part[tid];
    const int b1 = min(nblk, (c + 1) * per);
    for (int b0 = c * per; b0 < b1; b0 += 16) {
      int32_t v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = blk_hist[(int64_t)min(b0 + u, b1 - 1) * E + e];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (b0 + u < b1) {
          blk_hist[(int64_t)(b0 + u) * E + e] = run;
          run += v[u];
        }
      }
    }
  }
}

// One workgroup per router workgroup's rows (RT * k <= 64 flat rows).  Row
// f goes to blk_base[b][e] + (number of earlier rows of this workgroup
// routed to the same expert), which keeps ascending f within an expert.
__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                     const int32_t* __restrict__ blk_base,
                                                     int T, int k, int E,
                                                     int32_t* __restrict__ sorted_rows) {
  __shared__ int32_t ex[64];
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int64_t f0 = (int64_t)b * RT * k;
  const int nrows = (int)min((int64_t)RT * k, (int64_t)T * k - f0);
  int e = (i < nrows) ? topk_idx[f0 + i] : -1;
  ex[i] = e;
  __syncthreads();
  if (i < nrows) {
    int rank = 0;
    for (int q = 0; q < i; ++q) rank += (ex[q] == e);
    sorted_rows[blk_base[(int64_t)b * E + e] + rank] = (int32_t)(f0 + i);
  }
}

// Upper bound on the tile count: sum_e ceil(n_e / mt) <= R / mt + (number
// of non-empty experts), and at most min(E, R) experts are non-empty.
int max_tiles(int64_t R, int E, int mt) {
  // full tiles plus at most one ragged tile per expert; the XCD deal pads
  // each of the 8 shares to the longest, which is at most
  // ceil(F / 8) + ceil(ragged / 8)
  const int64_t f = R / mt, g = (R < E ? R : E);
  return (int)(8 * ((f + 7) / 8 + (g + 7) / 8));
}

// Tile lists from offsets in global memory (the backward rebuilds them):
// tiles of at most mt rows dealt to the XCDs, and with tiles2 != nullptr a
// second list of at most mt2 rows in expert order (one workgroup).
__global__ __launch_bounds__(256) void tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                    int mt, Tile* __restrict__ tiles,
                                                    int32_t* __restrict__ num_tiles, int mt2,
                                                    Tile* __restrict__ tiles2,
                                                    int32_t* __restrict__ num_tiles2) {
  __shared__ int32_t start[257];
  __shared__ int32_t offs[257];
  const int tid = threadIdx.x;
  // offsets into LDS in one parallel load (a serial loop over global
  // memory would pay a round trip per expert)
  for (int e = tid; e <= E; e += 256) offs[e] = offsets[e];
  __syncthreads();
  write_dealt_tiles(offs, E, mt, start, tiles, num_tiles);
  if (tiles2) write_tiles(offs, E, mt2, start, tiles2, num_tiles2);
}

hipError_t launch_logits(const uint16_t* x, const float* wr, const float* br, int T, int H,
                         int E, float* logits, hipStream_t s) {
  if (H % LG_CH) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)((T + 15) / 16) * ((E + 15) / 16);
  hipLaunchKernelGGL(logits_kernel, dim3((unsigned)blocks), dim3(64 * LG_W), 0, s, x, wr, br, T, H,
                     E, logits);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* topk_idx, float* topk_w,
                       int32_t* blk_hist, hipStream_t s) {
  if (E <= 64)
    hipLaunchKernelGGL(topk_kernel<1>, dim3(router_blocks(T)), dim3(256), 0, s, logits, T, E, k,
                       topk_idx, topk_w, blk_hist);
  else if (E <= 128)
    hipLaunchKernelGGL(topk_kernel<2>, dim3(router_blocks(T)), dim3(256), 0, s, logits, T, E, k,
                       topk_idx, topk_w, blk_hist);
  else
    hipLaunchKernelGGL(topk_kernel<4>, dim3(router_blocks(T)), dim3(256), 0, s, logits, T, E, k,
                       topk_idx, topk_w, blk_hist);
  return hipGetLastError();
}

hipError_t launch_plan_logits(const uint16_t* x, const float* wr, int T, int H, int E,
                              double* part, hipStream_t s) {
  if (H % LG_CH) return hipErrorInvalidValue;
  const int hs = plan_hs_parts(T, E, H);
  const int blocks = ((T + 15) / 16) * ((E + 15) / 16) * hs;
  // fewer than 32 ranges: 4 waves per range
  hipLaunchKernelGGL(logits_part_kernel, dim3(blocks), dim3(hs < 32 ? 64 * LPW : 64), 0, s, x, wr,
                     T, H, E, hs, part);
  return hipGetLastError();
}

bool plan_fits(int64_t T, int E, int k) { return T * k <= PLAN_MAX_ROWS && T * E <= PLAN_LOGITS; }

hipError_t launch_plan(const double* part, const float* br, int T, int H, int E, int k,
                       int32_t* topk_idx, float* topk_w, int32_t* offsets, int32_t* sorted_rows,
                       Tile* tiles, int32_t* num_tiles, hipStream_t s) {
  if (!plan_fits(T, E, k)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, part, plan_hs_parts(T, E, H), br, T,
                     E, k, topk_idx, topk_w, offsets, sorted_rows, tiles, num_tiles);
  return hipGetLastError();
}

hipError_t launch_scan(int32_t* blk_hist, int nblk, int E, int32_t* offsets, Tile* tiles,
                       int32_t* num_tiles, hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, blk_hist, nblk, E, offsets, tiles,
                     num_tiles);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* topk_idx, const int32_t* blk_base, int T, int k, int E,
                          int32_t* sorted_rows, hipStream_t s) {
  hipLaunchKernelGGL(scatter_kernel, dim3(router_blocks(T)), dim3(64), 0, s, topk_idx, blk_base,
                     T, k, E, sorted_rows);
  return hipGetLastError();
}

hipError_t launch_build_tiles(const int32_t* offsets, int E, int mt, Tile* tiles,
                              int32_t* num_tiles, int mt2, Tile* tiles2, int32_t* num_tiles2,
                              hipStream_t s) {
  hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(256), 0, s, offsets, E, mt, tiles, num_tiles,
                     mt2, tiles2, num_tiles2);
  return hipGetLastError();
}

}  // namespace mxmoe
