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

// One workgroup of 256 threads routes RT tokens.  The tokens' activations
// are staged in LDS once; each wave then takes experts wave, wave + 4, ...
// and for each holds the expert's router-weight row in registers, spread
// over the lanes along h (lane l owns h = 4l + 256j .. +3), while the other
// expert's row is already in flight (two register sets, loop unrolled by
// two).  Every lane forms partial dot products with all RT tokens; a
// butterfly over the wave sums them.  The bf16 x fp32 products are exact in
// fp64 and every partial and total sum is fp64; the logit is rounded once
// to fp32 and the top-k decision is taken on it.
constexpr int RCH = 12;             // float4 chunks of a row per lane: h < 256 * RCH = 3072
constexpr int RH = 256 * RCH;

__device__ __forceinline__ void router_load_row(f32x4 (&w)[RCH], const float* __restrict__ row,
                                                int H, int h0, int lane) {
#pragma unroll
  for (int j = 0; j < RCH; ++j) {
    const int h = h0 + 4 * lane + 256 * j;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    w[j] = (h < H) ? *reinterpret_cast<const f32x4*>(row + h) : z;
  }
}

__device__ __forceinline__ void router_dot_row(const f32x4 (&w)[RCH], const uint16_t* xs, int H,
                                               int h0, int lane, double (&acc)[RT]) {
#pragma unroll
  for (int j = 0; j < RCH; ++j) {
    const int h = h0 + 4 * lane + 256 * j;
    if (h < H) {
#pragma unroll
      for (int tt = 0; tt < RT; ++tt) {
        const u32x2 xv = *reinterpret_cast<const u32x2*>(xs + tt * H + h);
        double a = acc[tt];
        a = fma((double)__uint_as_float(xv[0] << 16), (double)w[j][0], a);
        a = fma((double)__uint_as_float(xv[0] & 0xFFFF0000u), (double)w[j][1], a);
        a = fma((double)__uint_as_float(xv[1] << 16), (double)w[j][2], a);
        a = fma((double)__uint_as_float(xv[1] & 0xFFFF0000u), (double)w[j][3], a);
        acc[tt] = a;
      }
    }
  }
}

// Sum over the wave (fixed butterfly order) and store the RT logits of e.
__device__ __forceinline__ void router_finish(double (&acc)[RT], int e, const float* br,
                                              int lane, float (*lg)[257]) {
#pragma unroll
  for (int tt = 0; tt < RT; ++tt) {
    double v = acc[tt];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) lg[tt][e] = (float)(v + (br ? (double)br[e] : 0.0));
    acc[tt] = 0.0;
  }
}

__global__ __launch_bounds__(256) void router_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ br,
    int T, int H, int E, int k, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ blk_hist) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [RT][H]
  __shared__ float lg[RT][257];
  __shared__ int32_t hist[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT;
  const int nt = min(RT, T - t0);

  // stage the tokens (rows past T are zero)
  const int row8 = H / 8;  // 16-byte pieces per row
  for (int q = tid; q < RT * row8; q += 256) {
    const int tt = q / row8, c = q % row8;
    const u32x4 z = {0u, 0u, 0u, 0u};
    reinterpret_cast<u32x4*>(xs)[q] =
        tt < nt ? reinterpret_cast<const u32x4*>(x + (int64_t)(t0 + tt) * H)[c] : z;
  }
  hist[tid] = 0;
  __syncthreads();

  double acc[RT];
#pragma unroll
  for (int tt = 0; tt < RT; ++tt) acc[tt] = 0.0;
  f32x4 w0[RCH], w1[RCH];
  if (H <= RH) {
    // whole rows in registers; the next expert's row loads during this one
    int e = wave;
    if (e < E) router_load_row(w0, wr + (int64_t)e * H, H, 0, lane);
    for (; e < E; e += 8) {
      if (e + 4 < E) router_load_row(w1, wr + (int64_t)(e + 4) * H, H, 0, lane);
      router_dot_row(w0, xs, H, 0, lane, acc);
      router_finish(acc, e, br, lane, lg);
      if (e + 4 >= E) break;
      if (e + 8 < E) router_load_row(w0, wr + (int64_t)(e + 8) * H, H, 0, lane);
      router_dot_row(w1, xs, H, 0, lane, acc);
      router_finish(acc, e + 4, br, lane, lg);
    }
  } else {
    for (int e = wave; e < E; e += 4) {
      for (int h0 = 0; h0 < H; h0 += RH) {
        router_load_row(w0, wr + (int64_t)e * H, H, h0, lane);
        router_dot_row(w0, xs, H, h0, lane, acc);
      }
      router_finish(acc, e, br, lane, lg);
    }
  }
  __syncthreads();

  // top-k per token: k passes of an arg-max, ties to the lower index
  if (tid < nt) {
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
  const size_t lds = (size_t)RT * H * sizeof(uint16_t);
  hipLaunchKernelGGL(router_kernel, dim3(router_blocks(T)), dim3(256), lds, s, x, wr, br, T, H, E,
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
