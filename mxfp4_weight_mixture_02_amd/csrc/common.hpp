// Device-side helpers shared by the gfx950 kernels of the MXFP4 MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even: gfx950's conversion instruction
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 -> packed bf16 (lo in the low half), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// UE8M0 scale byte -> the fp32 operand of the scaled fp4 conversions.  The
// hardware takes the exponent field of that operand as the E8M0 scale, so
// the byte goes straight into the exponent bits (byte 0 means 2^-127).
__device__ __forceinline__ float scale_operand(uint32_t s) {
  return __uint_as_float(s << 23);
}

// Eight E2M1 codes (one dword, element 2m in the low nibble of byte m) times
// 2^(s-127) -> eight bf16, exactly.  The packed result of each conversion
// is moved as a whole dword: the two bf16 halves are never extracted one by
// one.
__device__ __forceinline__ u32x4 dequant8_bf16(uint32_t codes, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight fp32 values v (two f32x4), times s, as a pair of bf16 vectors with
// hi + lo = s*v to about 2^-17 relative: hi = bf16(s*v), lo = bf16(s*v - hi).
// Two bf16 MFMAs over (hi, lo) then carry an fp32 operand.
__device__ __forceinline__ void split_bf16x8(f32x4 v0, f32x4 v1, float s, bf16x8* hi, bf16x8* lo) {
  u32x4 h, l;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float x0 = s * (m < 2 ? v0[2 * m] : v1[2 * m - 4]);
    const float x1 = s * (m < 2 ? v0[2 * m + 1] : v1[2 * m - 3]);
    const uint32_t b0 = f32_to_bf16(x0), b1 = f32_to_bf16(x1);
    h[m] = b0 | (b1 << 16);
    l[m] = pack_bf16x2(x0 - bf16_to_f32((uint16_t)b0), x1 - bf16_to_f32((uint16_t)b1));
  }
  *hi = as_bf16x8(h);
  *lo = as_bf16x8(l);
}

// bf16 bits of a gate (is_up = false) or up pre-activation for the saved
// state.  Round to nearest even, except that a value the rounding would move
// across a clamp bound (gate: +limit; up: -limit and +limit) is moved one
// ulp back to the side its fp32 value is on, so the backward takes the
// same clamp decisions as the forward did.
__device__ __forceinline__ uint32_t saved_preact_bf16(float v, float limit, bool is_up) {
  uint32_t b = f32_to_bf16(v);
  const float r = bf16_to_f32((uint16_t)b);
  if ((v > limit) != (r > limit)) b = (v > limit) ? b + 1 : b - 1;         // positive side
  if (is_up && ((v < -limit) != (r < -limit))) b = (v < -limit) ? b + 1 : b - 1;  // negative
  return b;
}

// Logistic sigmoid from the hardware base-2 exponential and reciprocal
// (v_exp_f32, v_rcp_f32; about 1 ulp each).  Every caller rounds its result
// to bf16 (2^-9 relative), so the library expf and a correctly rounded
// division would only cost instructions.  z -> -inf gives 1/inf = 0.
__device__ __forceinline__ float sigmoid_hw(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// Clamped SwiGLU of GPT-OSS: gate clamped above, up clamped both sides.
__device__ __forceinline__ float swiglu(float g, float u, float alpha, float limit) {
  float gc = fminf(g, limit);
  float uc = fminf(fmaxf(u, -limit), limit);
  float sig = sigmoid_hw(alpha * gc);
  return gc * sig * (uc + 1.0f);
}

// d/dg and d/du of swiglu times da; no gradient beyond a clamp bound.  An
// input lies within its bounds exactly when the clamp leaves it unchanged
// (a NaN input never compares equal, so it gets no gradient either; the
// gate's lower bound is the most negative finite float, so g = -inf, whose
// sigmoid factor is 0 times an infinity, gets none too); the clamps are
// single median-of-three operations, alpha * gc is shared by the
// sigmoid and the gate derivative, and both (uc + 1) ds and
// 1 + alpha gc (1 - s) are fused multiply-adds.
__device__ __forceinline__ void swiglu_grad(float g, float u, float da, float alpha, float limit,
                                            float* dg, float* du) {
  const float gc = __builtin_amdgcn_fmed3f(g, -3.402823466e38f, limit);
  const float uc = __builtin_amdgcn_fmed3f(u, -limit, limit);
  const float ag = alpha * gc;
  const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(ag * -1.4426950408889634f));
  const float ds = da * sig;
  *dg = (gc == g) ? fmaf(ds, uc, ds) * fmaf(ag, 1.0f - sig, 1.0f) : 0.0f;
  *du = (uc == u) ? ds * gc : 0.0f;
}

// Global and LDS pointer types of the global -> LDS load builtin.
typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// 16 bytes from device memory through a global-address-space pointer.  A
// generic pointer that the compiler cannot prove global (one chosen between
// a tensor and g_zero64, say) becomes a flat load, which also counts as an
// LDS operation: every wait for an LDS read would then wait for it as well,
// draining the loads kept in flight for later steps.
__device__ __forceinline__ u32x4 gload16(const void* p) {
  return *(const __attribute__((address_space(1))) u32x4*)p;
}

// 64 zero bytes in device memory: the source of the loads that fall past
// the end of a contraction whose length is an odd multiple of 32 (the last
// 64-deep step's upper half), so that both MFMA operands are exact zeros
// there.  E2M1 code 0 is +0, and scale byte 0 is a finite 2^-127.
static __device__ __attribute__((aligned(16))) const uint8_t g_zero64[64] = {};

// s_waitcnt immediate: wait until at most vm vector-memory and lgkm LDS /
// scalar-memory operations of this wave are outstanding (expcnt untouched).
__device__ constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14);
}

// Workgroup barrier without the memory fence of __syncthreads(): that fence
// makes the compiler wait for every outstanding global load first, which
// would drain a software pipeline's prefetches at every step.  Callers wait
// for exactly the loads and LDS writes the other waves need before calling.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Epilogue staging.  With the weights as the MFMA A-operand, the 32x32
// accumulator of a block gives lane l the output row l % 32 and, for a
// wave's two blocks rb and q, m = 0..3, the columns 32 rb + 8 q + 4 (l/32)
// + m: 16-byte column chunk c4 = 8 rb + 2 q + l/32 of a 64-column strip.
// Stores straight from that layout write 8-16 bytes into each of 32 rows
// per instruction; whole-row stores measured faster (by 2-7% of the GEMM
// time).  So each wave passes its strip through a private LDS region, 32
// rows at a time, and writes back row-contiguous 16-byte pieces.  Rows of
// RB bytes are split into 16-byte chunks; chunk c of row r sits at slot
// c ^ (r mod (RB/16)), so both access patterns spread over the banks.
// The row stores are non-temporal: the outputs are consumed by a later
// kernel, and streaming them past the caches measured slightly faster than
// letting them displace the weights and activations still being read.
template <int RB>
__device__ __forceinline__ int stg_off(int r, int c) {
  return r * RB + ((c ^ (r & (RB / 16 - 1))) << 4);
}

// Orders this wave's LDS writes before its later LDS reads of other lanes'
// data (and those reads before the next writes): a compiler barrier for
// memory and a wait for the wave's outstanding LDS operations.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  asm volatile("" ::: "memory");
}

// Block-wide staging of n 16-byte pieces from global memory into LDS:
// piece q is load(q) -> store(q, v).  A loop of "load, store" pays one
// memory round trip per iteration, because the store waits for its load;
// here every thread issues up to MAXP loads (indices clamped to n - 1)
// before its first store, so a batch costs one round trip.
template <int MAXP, class Load, class Store>
__device__ __forceinline__ void stage_lds(int n, int tid, int nthr, Load load, Store store) {
  for (int b = 0; b < n; b += MAXP * nthr) {
    u32x4 v[MAXP];
#pragma unroll
    for (int u = 0; u < MAXP; ++u) v[u] = load(min(b + tid + u * nthr, n - 1));
#pragma unroll
    for (int u = 0; u < MAXP; ++u) {
      const int q = b + tid + u * nthr;
      if (q < n) store(q, v[u]);
    }
  }
}

// One tile of routed rows of one expert for the grouped GEMMs.
struct Tile {
  int32_t expert;
  int32_t row0;  // first sorted position
  int32_t rows;  // 1..MT
  // forward lists: this tile's index q among its expert's tiles (bits 0-15)
  // and that expert's tile count n (bits 16-31, 0xFFFF when n >= 0xFFFF);
  // the backward's dealt list: the same for the expert's run of tiles on
  // the tile's XCD; 0 for an empty slot
  int32_t pos;
};
__host__ __device__ constexpr int32_t tile_pos(int32_t q, int32_t n) {
  return (int32_t)(((uint32_t)(n < 0xFFFF ? n : 0xFFFF) << 16) | ((uint32_t)q & 0xFFFFu));
}

// Work items of the grouped GEMMs.  Workgroups are dealt to the 8 XCDs
// round-robin by block index, and each XCD has its own L2.
//
// Tile list in expert order (forward): with L live work items (row tiles x
// column tiles), XCD i gets the contiguous range of items [start_i,
// start_i + L/8 (+1)).  Within it each expert's items go row tile fastest
// (item t_e C + c n_e + q is row tile q of column tile c, for an expert
// with n_e tiles from list index t_e), so the row tiles of an expert load
// the same weight columns at the same time and the XCD's L2 serves them
// once, while the column tiles of a row tile (same activations) still run
// close together.  Experts with 0xFFFF or more tiles go column tile
// fastest.  Returns false for blocks past the live items.
__device__ __forceinline__ bool xcd_item_range(const Tile* __restrict__ tiles,
                                               const int32_t* __restrict__ num_tiles,
                                               int col_tiles, Tile* tl, int* col_tile) {
  const int L = *num_tiles * col_tiles;
  const int b = blockIdx.x;
  if (b >= L) return false;
  const int xcd = b & 7, idx = b >> 3;
  const int base = L >> 3, extra = L & 7;
  const int item = xcd * base + min(xcd, extra) + idx;
  const int j = item / col_tiles;
  const Tile t = tiles[j];
  const uint32_t n = (uint32_t)t.pos >> 16, q = (uint32_t)t.pos & 0xFFFFu;
  if (n == 0 || n == 0xFFFF) {
    *tl = t;
    *col_tile = item % col_tiles;
    return true;
  }
  const int te = j - (int)q;
  const int local = item - te * col_tiles;
  *tl = tiles[te + local % (int)n];
  *col_tile = local / (int)n;
  return true;
}

// Tile list dealt to the XCDs (backward): XCD x's row tiles sit at x, 8 +
// x, 16 + x, ... (the XCDs' shares balanced, each ending on its shortest
// tiles; empty tiles have rows = 0), so block b runs on XCD x = b % 8 and
// takes its XCD's (b / 8)-th item.  An expert's full tiles on one XCD are
// consecutive slots (a run, recorded in each tile's pos), and a run's items
// go row tile fastest, so the run's row tiles read the same weight columns
// at the same time from one L2; otherwise column tile fastest (the column
// tiles of a row tile share its activations).  Returns false for blocks
// past the XCD's items and for empty tiles.
__device__ __forceinline__ bool xcd_work_item(const Tile* __restrict__ tiles,
                                              const int32_t* __restrict__ num_tiles,
                                              int col_tiles, Tile* tl, int* col_tile) {
  const int b = blockIdx.x;
  const int x = b & 7, idx = b >> 3;
  const int q = idx / col_tiles;
  if (8 * q + x >= *num_tiles) return false;
  const Tile t = tiles[8 * q + x];
  const uint32_t n = (uint32_t)t.pos >> 16, qi = (uint32_t)t.pos & 0xFFFFu;
  if (n <= 1 || n == 0xFFFF) {
    *tl = t;
    *col_tile = idx % col_tiles;
    return t.rows > 0;
  }
  const int q0 = q - (int)qi;                 // the run's first slot
  const int local = idx - q0 * col_tiles;
  *tl = tiles[8 * (q0 + local % (int)n) + x];
  *col_tile = local / (int)n;
  return tl->rows > 0;
}

constexpr int MT = 128;      // routed rows per forward GEMM tile
constexpr int BMT = 128;     // routed rows per backward GEMM tile
// LoRA ranks: 8, 16, 32 or 64, contracted in 16-deep MFMA chunks (rank 8
// zero-padded to one chunk).
constexpr int LORA_RMAX = 64;
__host__ __device__ constexpr bool lora_rank_ok(int r) {
  return r == 8 || r == 16 || r == 32 || r == 64;
}
__host__ __device__ constexpr int lora_chunks(int r) { return (r + 15) / 16; }

// The 8 rank values 16 j + 8 h .. + 7 of a bf16 row of rank r as one MFMA
// operand fragment (zeros past r).
__device__ __forceinline__ bf16x8 lora_frag(const uint16_t* row, int r, int j, int h) {
  const int c = 16 * j + 8 * h;
  return as_bf16x8(c < r ? *reinterpret_cast<const u32x4*>(row + c) : u32x4{0u, 0u, 0u, 0u});
}

// The same 8 values of an fp32 row, times s, as a hi + lo bf16 pair.
__device__ __forceinline__ void lora_frag_split(const float* row, int r, int j, int h, float s,
                                                bf16x8* hi, bf16x8* lo) {
  const int c = 16 * j + 8 * h;
  const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  const f32x4 v0 = c < r ? *reinterpret_cast<const f32x4*>(row + c) : z;
  const f32x4 v1 = c < r ? *reinterpret_cast<const f32x4*>(row + c + 4) : z;
  split_bf16x8(v0, v1, s, hi, lo);
}

}  // namespace mxmoe
