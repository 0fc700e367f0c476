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
constexpr int RH = 32;  // hidden elements staged per router step

int router_blocks(int64_t T) { return (int)((T + RT - 1) / RT); }

// One workgroup of 256 threads routes RT tokens.  Thread i owns expert
// i % E for the tokens i / E, i / E + G, ... (G = 256 / E groups).  The
// bf16 x fp32 products are exact in fp64 and are summed in fp64; the logit
// is rounded once to fp32 and the top-k decision is taken on it.
__global__ __launch_bounds__(256) void router_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ br,
    int T, int H, int E, int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ blk_hist) {
  __shared__ float ws[RH][257];       // router weight chunk, [h][e]
  __shared__ float xs[RT][RH + 1];    // activations chunk
  __shared__ float lg[RT][257];       // logits
  __shared__ int32_t hist[256];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * RT;
  const int G = 256 / E;              // token groups
  const int e_own = tid % E;
  const int g_own = tid / E;          // >= G: idle lane
  constexpr int TPT = RT;             // upper bound of tokens per thread
  double acc[TPT];
#pragma unroll
  for (int j = 0; j < TPT; ++j) acc[j] = 0.0;

  for (int h0 = 0; h0 < H; h0 += RH) {
    for (int q = tid; q < E * RH; q += 256) {
      int e = q / RH, hh = q % RH;
      ws[hh][e] = wr[(int64_t)e * H + h0 + hh];
    }
    for (int q = tid; q < RT * RH; q += 256) {
      int tt = q / RH, hh = q % RH;
      int t = t0 + tt;
      xs[tt][hh] = (t < T) ? bf16_to_f32(x[(int64_t)t * H + h0 + hh]) : 0.0f;
    }
    __syncthreads();
    if (g_own < G) {
      for (int hh = 0; hh < RH; ++hh) {
        double wv = (double)ws[hh][e_own];
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
          int tt = g_own + j * G;
          if (tt < RT) acc[j] = fma((double)xs[tt][hh], wv, acc[j]);
        }
      }
    }
    __syncthreads();
  }
  if (g_own < G) {
    double b = br ? (double)br[e_own] : 0.0;
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      int tt = g_own + j * G;
      if (tt < RT) lg[tt][e_own] = (float)(acc[j] + b);
    }
  }
  hist[tid] = 0;
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
  hipLaunchKernelGGL(router_kernel, dim3(router_blocks(T)), dim3(256), 0, s, x, wr, br, T, H, E,
                     k, topk_idx, topk_w, blk_hist);
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
