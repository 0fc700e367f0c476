// Router (logits, top-k, softmax over the selected k), expert histogram,
// exclusive scan and the stable token permutation (gfx950).
//
// The pages ("Add MXFP4 training support via a dequantize-on-the-fly
// fallback", "What this does") run a top-k router before the per-expert
// loop; the finegrained-kernels note on the bias operand describes the
// grouped path that orders routed rows by expert.  Here the permutation is
// a deterministic counting sort: per-workgroup histograms, one scan over
// (expert, workgroup), then each workgroup scatters its rows in ascending
// flat-row order.  No atomics on global memory, so the result is identical
// run to run.
#include "common.hpp"
#include "launch.hpp"

namespace mxmoe {

constexpr int RT = ROUTER_TOKENS;

int router_blocks(int64_t T) { return (int)((T + RT - 1) / RT); }

// One workgroup of 256 threads routes RT tokens.  Each of the four waves
// takes a quarter of the hidden dimension; lane l owns the (token, expert)
// pairs p = l + 64m (token p / E, expert p % E), so with E <= 64 a lane's
// router-weight row is loaded once per step and used for RT*E/64 tokens.
// The bf16 x fp32 products are exact in fp64 and are summed in fp64 (each
// lane in h order within its quarter, then the four quarters in order);
// the logit is rounded once to fp32 and the top-k decision is taken on it.
template <int NPL>  // pairs per lane: ceil(RT * E / 64), rounded up to a power of two
__global__ __launch_bounds__(256) void router_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ br,
    int T, int H, int E, int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ blk_hist) {
  __shared__ double part[4][RT * 256];
  __shared__ float lg[RT][257];
  __shared__ int32_t hist[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT;
  const int P = RT * E;                   // pairs in this block
  const int hq = H / 4;                   // this wave's share of h (H % 64 == 0)
  const int h0 = wave * hq;

  double acc[NPL];
  int wo[NPL], xo[NPL];                   // element offsets of the pair's rows; -1 = none
#pragma unroll
  for (int m = 0; m < NPL; ++m) {
    acc[m] = 0.0;
    const int p = lane + 64 * m;
    const int tt = p / E, e = p % E;
    const bool live = p < P && t0 + tt < T;
    wo[m] = live ? e * H + h0 : -1;
    xo[m] = live ? (t0 + tt) * H + h0 : -1;
  }
  for (int h = 0; h < hq; h += 4) {
#pragma unroll
    for (int m = 0; m < NPL; ++m) {
      if (wo[m] < 0) continue;
      const f32x4 wv = *reinterpret_cast<const f32x4*>(wr + wo[m] + h);
      const u32x2 xv = *reinterpret_cast<const u32x2*>(x + (int64_t)xo[m] + h);
      double a = acc[m];
      a = fma((double)__uint_as_float(xv[0] << 16), (double)wv[0], a);
      a = fma((double)__uint_as_float(xv[0] & 0xFFFF0000u), (double)wv[1], a);
      a = fma((double)__uint_as_float(xv[1] << 16), (double)wv[2], a);
      a = fma((double)__uint_as_float(xv[1] & 0xFFFF0000u), (double)wv[3], a);
      acc[m] = a;
    }
  }
#pragma unroll
  for (int m = 0; m < NPL; ++m) {
    const int p = lane + 64 * m;
    if (p < P) part[wave][p] = acc[m];
  }
  hist[tid] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += 256) {
    const int tt = p / E, e = p % E;
    double v = part[0][p] + part[1][p];
    v += part[2][p];
    v += part[3][p];
    if (br) v += (double)br[e];
    lg[tt][e] = (float)v;
  }
  __syncthreads();

  // top-k per token: k passes of an arg-max, ties to the lower index
  if (tid < RT && t0 + tid < T) {
    const int tt = tid;
    uint64_t taken[4] = {0, 0, 0, 0};
    float sel[8];
    int idx[8];
    for (int j = 0; j < k; ++j) {
      int best = -1;
      float bv = 0.0f;
      for (int e = 0; e < E; ++e) {
        if ((taken[e >> 6] >> (e & 63)) & 1) continue;
        float v = lg[tt][e];
        if (best < 0 || v > bv) { best = e; bv = v; }
      }
      taken[best >> 6] |= 1ull << (best & 63);
      idx[j] = best;
      sel[j] = bv;
    }
    float z[8], sum = 0.0f;
    for (int j = 0; j < k; ++j) { z[j] = expf(sel[j] - sel[0]); sum += z[j]; }
    const int64_t f0 = (int64_t)(t0 + tt) * k;
    for (int j = 0; j < k; ++j) {
      topk_idx[f0 + j] = idx[j];
      topk_w[f0 + j] = z[j] / sum;
      atomicAdd(&hist[idx[j]], 1);  // counts only: order does not matter
    }
  }
  __syncthreads();
  if (tid < E) blk_hist[(int64_t)blockIdx.x * E + tid] = hist[tid];
}

// One workgroup of 1024 threads.  In place, blk_hist[b][e] becomes the
// first sorted position of workgroup b's rows of expert e:
// offsets[e] + sum_{b' < b} count[b'][e].  offsets = exclusive scan of the
// expert totals (E + 1 entries).
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ blk_hist, int nblk,
                                                    int E, int32_t* __restrict__ offsets) {
  __shared__ int32_t part[1024];
  __shared__ int32_t total[256];
  __shared__ int32_t off[257];
  const int tid = threadIdx.x;
  const int C = 1024 / E;                    // chunks of workgroups
  const int per = (nblk + C - 1) / C;
  const int e = tid % E, c = tid / E;
  int32_t sum = 0;
  if (c < C) {
    int b1 = min(nblk, (c + 1) * per);
    for (int b = c * per; b < b1; ++b) sum += blk_hist[(int64_t)b * E + e];
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
  if (c < C) {
    int32_t run = off[e] + part[tid];
    int b1 = min(nblk, (c + 1) * per);
    for (int b = c * per; b < b1; ++b) {
      int32_t v = blk_hist[(int64_t)b * E + e];
      blk_hist[(int64_t)b * E + e] = run;
      run += v;
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

int max_tiles(int64_t R, int E) { return (int)((R + MT - 1) / MT) + E; }

// Tiles of at most MT sorted rows, expert by expert (one workgroup).
__global__ __launch_bounds__(256) void tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                    Tile* __restrict__ tiles,
                                                    int32_t* __restrict__ num_tiles) {
  __shared__ int32_t start[257];
  const int tid = threadIdx.x;
  if (tid == 0) {
    int32_t run = 0;
    for (int e = 0; e < E; ++e) {
      start[e] = run;
      int32_t n = offsets[e + 1] - offsets[e];
      run += (n + MT - 1) / MT;
    }
    start[E] = run;
    *num_tiles = run;
  }
  __syncthreads();
  if (tid < E) {
    int32_t o = offsets[tid], n = offsets[tid + 1] - o;
    for (int32_t q = 0; q * MT < n; ++q) {
      Tile tl;
      tl.expert = tid;
      tl.row0 = o + q * MT;
      tl.rows = min(MT, n - q * MT);
      tl.pad = 0;
      tiles[start[tid] + q] = tl;
    }
  }
}

hipError_t launch_router(const uint16_t* x, const float* wr, const float* br, int T, int H,
                         int E, int k, int32_t* topk_idx, float* topk_w, int32_t* blk_hist,
                         hipStream_t s) {
  const int npl = (RT * E + 63) / 64;
  dim3 g(router_blocks(T)), b(256);
#define ROUTER(N) hipLaunchKernelGGL(router_kernel<N>, g, b, 0, s, x, wr, br, T, H, E, k, \
                                     topk_idx, topk_w, blk_hist)
  if (npl <= 1) ROUTER(1);
  else if (npl <= 2) ROUTER(2);
  else if (npl <= 4) ROUTER(4);
  else if (npl <= 8) ROUTER(8);
  else if (npl <= 16) ROUTER(16);
  else ROUTER(32);
#undef ROUTER
  return hipGetLastError();
}

hipError_t launch_scan(int32_t* blk_hist, int nblk, int E, int32_t* offsets, hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, blk_hist, nblk, E, offsets);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* topk_idx, const int32_t* blk_base, int T, int k, int E,
                          int32_t* sorted_rows, hipStream_t s) {
  hipLaunchKernelGGL(scatter_kernel, dim3(router_blocks(T)), dim3(64), 0, s, topk_idx, blk_base,
                     T, k, E, sorted_rows);
  return hipGetLastError();
}

hipError_t launch_build_tiles(const int32_t* offsets, int E, Tile* tiles, int32_t* num_tiles,
                              hipStream_t s) {
  hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(256), 0, s, offsets, E, tiles, num_tiles);
  return hipGetLastError();
}

}  // namespace mxmoe
