// Host-side launchers of the library's kernels (internal; the public
// surface is include/mxfp4_moe.h).  Every launcher only enqueues work on
// `s`; shapes were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxmoe {

struct Tile;

// quant.hip
hipError_t launch_quantize(const float* w, int64_t rows, int64_t K, uint8_t* codes,
                           uint8_t* scales, hipStream_t s);
// MXFP8 (E4M3, UE8M0 per 32) of bf16 rows; with lo_codes also the residual
hipError_t launch_mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes,
                                 uint8_t* scales, uint8_t* lo_codes, uint8_t* lo_scales,
                                 hipStream_t s);
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                             int64_t K, int out_bf16, void* out, hipStream_t s);

// route.hip
constexpr int ROUTER_TOKENS = 8;    // tokens per top-k workgroup (one histogram row each)
constexpr int PLAN_MAX_ROWS = 256;  // routed rows up to which one workgroup plans the routing
int router_blocks(int64_t T);
hipError_t launch_logits(const uint16_t* x, const float* wr, const float* br, int T, int H,
                         int E, float* logits, hipStream_t s);
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* topk_idx, float* topk_w,
                       int32_t* blk_hist, hipStream_t s);
// Planned routing (plan_fits: R = T*k <= PLAN_MAX_ROWS and T*E <= 4096):
// partial fp64 logits over plan_hs_parts(T, E, H) ranges of h (part: that
// many x T x E doubles), then one workgroup for the logits, top-k, offsets,
// permutation and tiles.
bool plan_fits(int64_t T, int E, int k);
int plan_hs_parts(int T, int E, int H);
hipError_t launch_plan_logits(const uint16_t* x, const float* wr, int T, int H, int E,
                              double* part, hipStream_t s);
hipError_t launch_plan(const double* part, const float* br, int T, int H, int E, int k,
                       int32_t* topk_idx, float* topk_w, int32_t* offsets, int32_t* sorted_rows,
                       Tile* tiles, int32_t* num_tiles, hipStream_t s);
hipError_t launch_scan(int32_t* blk_hist, int nblk, int E, int32_t* offsets, Tile* tiles,
                       int32_t* num_tiles, hipStream_t s);   // also writes the tile list
hipError_t launch_scatter(const int32_t* topk_idx, const int32_t* blk_base, int T, int k, int E,
                          int32_t* sorted_rows, hipStream_t s);
int max_tiles(int64_t R, int E, int mt);
// tile lists from the offsets: at most mt rows per tile, dealt to the XCDs
// (the backward GEMMs' order), and with tiles2 at most mt2 rows in expert order
hipError_t launch_build_tiles(const int32_t* offsets, int E, int mt, Tile* tiles,
                              int32_t* num_tiles, int mt2, Tile* tiles2, int32_t* num_tiles2,
                              hipStream_t s);

// gemm_fwd.hip
int fwd_step_k(int K);   // K step of the forward GEMMs for contraction length K; 0 = unsupported
// with lora_B: + the gate_up adapter's rank-r delta s (v B_gu^T) before the
// bias (v [R, r] sorted, B_gu [E, 2I, r])
hipError_t launch_gate_up(const uint16_t* x, const uint8_t* codes, const uint8_t* scales,
                          const uint16_t* bias, const int32_t* sorted_rows, const Tile* tiles,
                          const int32_t* num_tiles, int max_tiles, int H, int I, int k,
                          float alpha, float limit, const uint16_t* lora_B, const float* lora_v,
                          float lora_scale, int lora_r, uint16_t* h_out, uint16_t* a_out,
                          hipStream_t s);
// lora_B/lora_v/lora_scale/lora_r: the rank-r delta s (v B_e^T) added
// before the bias (lora_B == nullptr: none).
hipError_t launch_down(const uint16_t* a, const uint8_t* codes, const uint8_t* scales,
                       const uint16_t* bias, const float* topk_w, const int32_t* sorted_rows,
                       const Tile* tiles, const int32_t* num_tiles, int max_tiles, int H, int I,
                       const uint16_t* lora_B, const float* lora_v, float lora_scale, int lora_r,
                       uint16_t* y_w, hipStream_t s);
hipError_t launch_combine(const uint16_t* y_w, int64_t T, int H, int k, uint16_t* out,
                          hipStream_t s);
// gate_up on the block-scaled MFMA: FP4 weights as stored, activations as
// MXFP8 codes [T, H] + scales [T, H/32] (with xq_lo: a second, residual pass)
hipError_t launch_mx_gate_up(const uint8_t* xq, const uint8_t* xs, const uint8_t* xq_lo,
                             const uint8_t* xs_lo, const uint8_t* codes, const uint8_t* scales,
                             const uint16_t* bias, const int32_t* sorted_rows, const Tile* tiles,
                             const int32_t* num_tiles, int max_tiles, int H, int I, int k,
                             float alpha, float limit, uint16_t* h_out, uint16_t* a_out,
                             hipStream_t s);

// gemm_dec.hip: forward GEMMs for few rows per expert (weight-streaming)
int dec_max_k();   // largest contraction length the decode kernels take
hipError_t launch_dec_gate_up(const uint16_t* x, const uint8_t* codes, const uint8_t* scales,
                              const uint16_t* bias, const int32_t* sorted_rows, const Tile* tiles,
                              const int32_t* num_tiles, int max_tiles, int64_t R, int H, int I, int k,
                              float alpha, float limit, const uint16_t* lora_B,
                              const float* lora_v, float lora_scale, int lora_r, uint16_t* h_out,
                              uint16_t* a_out, hipStream_t s);
// with lora_B: + the rank-r delta s (v B_e^T), as launch_down
hipError_t launch_dec_down(const uint16_t* a, const uint8_t* codes, const uint8_t* scales,
                           const uint16_t* bias, const float* topk_w, const int32_t* sorted_rows,
                           const Tile* tiles, const int32_t* num_tiles, int max_tiles, int64_t R,
                           int H, int I, const uint16_t* lora_B, const float* lora_v,
                           float lora_scale, int lora_r, uint16_t* y_w, hipStream_t s);

// gemm_bwd.hip
int bwd_down_ntiles(int I);
hipError_t launch_bwd_down(const uint16_t* dy, const uint8_t* codes, const uint8_t* scales,
                           const float* topk_w, const int32_t* sorted_rows, const Tile* tiles,
                           const int32_t* num_tiles, int max_tiles, const uint16_t* h,
                           const uint16_t* a, int H, int I, int k, float alpha, float limit,
                           const uint16_t* lora_At, const float* lora_dvu, int lora_r,
                           uint16_t* dh, float* dw_part, hipStream_t s);
// with lora_At: + the gate_up adapter's input-gradient term dv_g A_gu
// (lora_At = A_gu transposed, [E, H, r]; dv_g [R, r] sorted)
hipError_t launch_bwd_gate_up(const uint16_t* dh, const uint8_t* codes, const uint8_t* scales,
                              const int32_t* sorted_rows, const Tile* tiles,
                              const int32_t* num_tiles, int max_tiles, int H, int I,
                              const uint16_t* lora_At, const float* lora_dv, int lora_r,
                              uint16_t* dxr, hipStream_t s);
hipError_t launch_bwd_combine(const uint16_t* dy, const uint16_t* dxr, const float* dw_part,
                              int n_dw_part, const int32_t* topk_idx, const float* topk_w,
                              const uint16_t* dn_bias, const float* router_w, int64_t T, int H,
                              int k, uint16_t* dx, hipStream_t s);

// lora.hip
// out [R, r] fp32 = scale * src rows . M_e rows (M: [E, r, C] bf16)
hipError_t launch_lora_proj(const uint16_t* src, bool gather, const int32_t* sorted_rows, int k,
                            const uint16_t* M, int C, int r, const Tile* tiles,
                            const int32_t* num_tiles, int max_tiles, float scale, float* out,
                            hipStream_t s);
hipError_t launch_transpose_bf16(const uint16_t* in, int64_t batches, int R1, int R2,
                                 uint16_t* out, hipStream_t s);
// P: [R, r] fp32
hipError_t launch_lora_grad(const uint16_t* Q, bool gather, int C, const int32_t* sorted_rows,
                            int k, const float* P, int r, const float* topk_w, float scale,
                            const int32_t* offsets, int E, float* out, int64_t e_stride,
                            int c_stride, int j_stride, hipStream_t s);

// gemm_dw.hip: base-weight gradients.  out[e] (fp32 [M, N]) = sum over
// expert e's sorted rows p of A[rowA(p)]^T B[rowB(p)] (bf16 row-major, the
// gathered operand's row = sorted_rows[p] / k, else p).
hipError_t launch_dw(const uint16_t* A, int lda, bool gatherA, const uint16_t* B, int ldb,
                     bool gatherB, const int32_t* offsets, const int32_t* sorted_rows, int k,
                     int E, int M, int N, float* out, hipStream_t s);
// db[e][c] = sum_p w_p src[row(p)][c] (topk_w NULL: w = 1)
hipError_t launch_colsum(const uint16_t* src, int ld, bool gather, const int32_t* offsets,
                         const int32_t* sorted_rows, int k, const float* topk_w, int E, int C,
                         float* db, hipStream_t s);
// out[p] = bf16(topk_w[sorted_rows[p]] * in[p]) for R rows of C columns
hipError_t launch_scale_rows(const uint16_t* in, int64_t R, int C, const int32_t* sorted_rows,
                             const float* topk_w, uint16_t* out, hipStream_t s);

}  // namespace mxmoe
