/*
 * mxfp4_moe.h -- C ABI of the MI355X (gfx950) MXFP4 mixture-of-experts
 * expert block: forward and activation-gradient (dX) backward over frozen
 * expert weights that stay packed as MXFP4.
 *
 * Sources (cited by page title and section):
 *  [P1] "Add MXFP4 training support via a dequantize-on-the-fly fallback"
 *       (huggingface/transformers pull request 47464), "What this does",
 *       "Why (the silent-gradient trap)", "Relation to the backward triton
 *       kernels": the expert block (top-k router, GPT-OSS expert loop),
 *       packed weights never modified, gradients needed only for the inputs
 *       and the adapters of a frozen base.
 *  [P3] "Integrate finegrained kernels: SOTA performance and per-module
 *       quantization" (pull request 49658), commit notes: gate|up rows
 *       interleaved (gate j at row 2j, up j at 2j+1) and split stride-2 by
 *       the fused GLU epilogue; a per-expert bias operand in both GEMMs,
 *       passed as null when absent; the routing-weighted reduce; row-wise
 *       MXFP4 quantizers with UE8M0 scales, one launch per tensor; guards
 *       that refuse (rather than re-permute or fall back) before a launch.
 *  [OCP] OCP Microscaling Formats (MX) v1.0: E2M1 elements, E8M0 scales.
 *
 * Conventions for every entry point
 *  - All tensors are dense, row-major (last dimension contiguous), in
 *    device memory owned by the caller.  The library allocates no device
 *    memory; scratch comes in through `workspace` (mxfp4_moe_forward_noalloc
 *    uses a fixed static device array instead).
 *  - bf16 tensors are passed as uint16_t bit patterns.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *    enqueued on it asynchronously with no host synchronisation, so calls
 *    can be captured into a HIP graph.
 *  - All validation happens on the host before anything is enqueued; on a
 *    non-zero return nothing was enqueued (except MXFP4_EHIP, which reports
 *    a failed launch) and mxfp4_last_error() describes the problem.
 *  - Calls that share a workspace must be ordered on one stream.
 */
#ifndef MXFP4_MOE_H
#define MXFP4_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MXFP4_OK 0
#define MXFP4_EINVAL (-1)       /* null required pointer or a count < 1 */
#define MXFP4_EUNSUPPORTED (-2) /* a shape or option outside the contract */
#define MXFP4_EWORKSPACE (-3)   /* workspace smaller than the query says */
#define MXFP4_EHIP (-4)         /* a HIP call or launch failed */

/* Layer shape and activation constants.
 *  T tokens, H hidden, I intermediate, E experts, k experts per token.
 *  Requirements: T >= 1; H % 32 == 0 and I % 32 == 0 (whole 32-element
 *  scale blocks, [P3] group-32 guard; the kernels run 64-element K steps
 *  and read zeros past an odd multiple of 32); 1 <= k <= min(E, 8);
 *  E <= 256; T * k < 2^31; T * H < 2^31; H, I <= 5120;
 *  lora_rank in {0, 8, 16, 32, 64}.  Weight, scale, bias, activation and
 *  output pointers 16-byte aligned.
 *  swiglu_alpha, swiglu_limit: the clamped SwiGLU constants (GPT-OSS uses
 *  1.702 and 7).  lora_scale multiplies the LoRA deltas (1.0 when
 *  lora_alpha equals the rank).  lora_targets: which projections carry a
 *  rank-lora_rank adapter, MXFP4_LORA_DOWN | MXFP4_LORA_GATE_UP (0 means
 *  MXFP4_LORA_DOWN); ignored when lora_rank == 0.
 *  activation_format: what the gate_up product consumes ([P3] commit notes:
 *  activation_format "bf16" = weight-only, None = the weights' block-scaled
 *  format): MXFP4_ACT_BF16 (0, default) decodes the weights to bf16 for the
 *  matrix cores; MXFP4_ACT_MXFP8 quantizes each token row to MXFP8 (E4M3,
 *  UE8M0 per 32) and runs the block-scaled MFMA on the packed FP4 weights as
 *  stored; MXFP4_ACT_MXFP8X2 adds a second MXFP8 pass of the residual (x ~
 *  hi + lo).  The block-scaled formats need H % 64 == 0 and no gate_up
 *  adapter; the down product and the backward are unchanged (the backward
 *  treats the quantization as the identity). */
#define MXFP4_LORA_DOWN 1
#define MXFP4_LORA_GATE_UP 2
#define MXFP4_ACT_BF16 0
#define MXFP4_ACT_MXFP8 1
#define MXFP4_ACT_MXFP8X2 2
typedef struct mxfp4_moe_dims {
  int64_t T;
  int64_t H;
  int64_t I;
  int32_t E;
  int32_t k;
  float swiglu_alpha;
  float swiglu_limit;
  int32_t lora_rank;
  float lora_scale;
  int32_t lora_targets;
  int32_t activation_format;
} mxfp4_moe_dims;

/* Frozen layer parameters ([P3] MXFP4 layout; weights never written).
 *  router_w  fp32 [E, H];    router_b fp32 [E] or NULL (zero bias)
 *  gu_codes  uint8 [E, 2I, H/2]  two E2M1 codes per byte, element 2m in
 *            the low nibble; rows interleaved gate/up ([P3]): gate j at
 *            row 2j, up j at row 2j+1.  A stacked [gate; up] tensor is NOT
 *            detected (the bytes cannot tell) and gives wrong results.
 *  gu_scales uint8 [E, 2I, H/32] UE8M0, value 2^(s-127); s = 255 is NaN
 *  gu_bias   bf16 [E, 2I] (same interleaved row order) or NULL
 *  dn_codes  uint8 [E, H, I/2];  dn_scales uint8 [E, H, I/32]
 *  dn_bias   bf16 [E, H] or NULL
 *  lora_A    bf16 [E, r, I] and lora_B bf16 [E, H, r]: per-expert LoRA on
 *            the down projection ([P1] "What this does": adapters train on
 *            the frozen MXFP4 base), y += scale * (a A_e^T) B_e^T.  Both
 *            NULL when lora_rank == 0 (MXFP4_EINVAL otherwise), both
 *            required and 16-byte aligned when lora_rank > 0.  Inside the
 *            down GEMMs, scale * v and the rank-space gradient enter the
 *            bf16 matrix cores as a hi + lo bf16 pair (about 17 bits), in
 *            16-deep chunks of the rank (rank 8 zero-padded to one).
 *  lora_gu_A bf16 [E, r, H] and lora_gu_B bf16 [E, 2I, r] (rows in the
 *            interleaved gate/up order): the adapter on the gate_up
 *            projection, h += scale * (x A_gu_e^T) B_gu_e^T before the
 *            bias; both required (16-byte aligned) iff MXFP4_LORA_GATE_UP
 *            is a target, else NULL. */
typedef struct mxfp4_moe_weights {
  const float* router_w;
  const float* router_b;
  const uint8_t* gu_codes;
  const uint8_t* gu_scales;
  const uint16_t* gu_bias;
  const uint8_t* dn_codes;
  const uint8_t* dn_scales;
  const uint16_t* dn_bias;
  const uint16_t* lora_A;
  const uint16_t* lora_B;
  const uint16_t* lora_gu_A;
  const uint16_t* lora_gu_B;
} mxfp4_moe_weights;

/* State the forward saves for the backward (caller-owned device buffers,
 * R = T * k routed rows, flat row f = t * k + j for token t, slot j).
 *  topk_idx       int32 [T, k]   selected experts, logit descending, ties
 *                                to the lower index
 *  topk_w         fp32  [T, k]   softmax over the k selected logits
 *  expert_offsets int32 [E + 1]  exclusive prefix sum of the expert
 *                                histogram; offsets[E] = R
 *  sorted_rows    int32 [R]      flat rows grouped by expert, ascending f
 *                                within an expert (stable)
 *  h              bf16  [R, 2I]  gate_up output incl. bias, sorted order
 *  a              bf16  [R, I]   SwiGLU output, sorted order
 *  lora_v         fp32  [R, r]   v = a A_e^T (sorted order, before the
 *                                lora_scale); required iff the down
 *                                projection has an adapter, else ignored;
 *                                16-byte aligned
 *  lora_vg        fp32  [R, r]   vg = x A_gu_e^T likewise, for the gate_up
 *                                adapter */
typedef struct mxfp4_moe_saved {
  int32_t* topk_idx;
  float* topk_w;
  int32_t* expert_offsets;
  int32_t* sorted_rows;
  uint16_t* h;
  uint16_t* a;
  float* lora_v;
  float* lora_vg;
} mxfp4_moe_saved;

/* Byte sizes of the saved-state buffers for given dims (one field per
 * mxfp4_moe_saved buffer, same order; lora_v and lora_vg are 0 without
 * the matching adapter).
 * The caller allocates them (each 16-byte aligned) and passes their
 * addresses in mxfp4_moe_saved; the library never allocates them ([P1]
 * "What this does": the transients belong to the caller's framework). */
typedef struct mxfp4_moe_saved_sizes {
  size_t topk_idx;
  size_t topk_w;
  size_t expert_offsets;
  size_t sorted_rows;
  size_t h;
  size_t a;
  size_t lora_v;
  size_t lora_vg;
} mxfp4_moe_saved_sizes;

/* Fills *out for dims.  Returns MXFP4_OK, MXFP4_EINVAL (null out, or dims
 * with a count < 1) or MXFP4_EUNSUPPORTED (dims outside the contract); on
 * an error *out is left untouched. */
int mxfp4_moe_saved_bytes(const mxfp4_moe_dims* dims, mxfp4_moe_saved_sizes* out);

/* Workspace modes for mxfp4_moe_workspace_bytes. */
#define MXFP4_WS_FORWARD 0        /* mxfp4_moe_forward, saved == NULL */
#define MXFP4_WS_FORWARD_SAVED 1  /* mxfp4_moe_forward, saved != NULL */
#define MXFP4_WS_BACKWARD 2       /* mxfp4_moe_backward_dx */
#define MXFP4_WS_BACKWARD_FULL 3  /* mxfp4_moe_backward */

/* Bytes of device workspace an entry point needs for these dims (0 if
 * the dims are invalid; mxfp4_last_error() then says why).  The workspace
 * must be 256-byte aligned. */
size_t mxfp4_moe_workspace_bytes(const mxfp4_moe_dims* dims, int mode);

/* Expert-block forward ([P1] "What this does": top-k router, then the
 * GPT-OSS expert math; [P3] fused bias + stride-2 GLU epilogue and the
 * routing-weighted reduce):
 *   logits l[t,e] = sum_h x[t,h] Wr[e,h] + br[e]  (products summed in fp64,
 *                   rounded once to fp32 before the top-k decision)
 *   top-k experts, softmax over the k selected logits -> w[t,j]
 *   h = x Wgu_e^T + bgu_e (+ lora_scale (x A_gu_e^T) B_gu_e^T);
 *   a = min(g,L) sig(alpha min(g,L)) (clamp(u,-L,L)+1)
 *       with g = h[2i], u = h[2i+1]
 *   y = a Wd_e^T + bd_e (+ lora_scale (a A_e^T) B_e^T)
 *   out[t] = sum_j w[t,j] y_(t,j)   (each term w y rounded to bf16, then
 *                                    an fp32 sum in slot order, then bf16)
 * x bf16 [T, H] in; out bf16 [T, H] out.  saved may be NULL (inference);
 * otherwise every buffer it names is written. */
int mxfp4_moe_forward(const mxfp4_moe_dims* dims, const mxfp4_moe_weights* w,
                      const uint16_t* x, uint16_t* out, const mxfp4_moe_saved* saved,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Forward that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, checks,
 * kernels and results (bit for bit) as mxfp4_moe_forward, except that its
 * scratch is a static device array of MXFP4_NOALLOC_SCRATCH_BYTES inside
 * the library (one copy per GPU, held until the process ends; its address
 * is looked up once per device with hipGetSymbolAddress, on the first call
 * made with that device current).  Dims whose forward needs more scratch
 * than that -- mxfp4_moe_workspace_bytes() of MXFP4_WS_FORWARD or
 * MXFP4_WS_FORWARD_SAVED -- are refused with MXFP4_EUNSUPPORTED before
 * anything is enqueued (16 MiB covers every decode-size forward, T * k <=
 * 256, and the 20b layer up to about 350 tokens).  The stream must belong
 * to the current device.  Calls on one GPU share its array: calls that
 * overlap (several streams, or several threads) race; calls ordered on one
 * stream do not.  Nothing in the array needs to start zeroed (every byte a
 * call reads was written earlier in that call). */
#define MXFP4_NOALLOC_SCRATCH_BYTES (16u << 20)
int mxfp4_moe_forward_noalloc(const mxfp4_moe_dims* dims, const mxfp4_moe_weights* w,
                              const uint16_t* x, uint16_t* out, const mxfp4_moe_saved* saved,
                              void* stream);

/* Activation-gradient backward of the expert block for the loss
 * sum(dY * out), base weights and biases frozen ([P1]: LoRA training needs
 * gradients only for the inputs and the adapters):
 *   per routed row f = (t, j), expert e:
 *     dw_f = dY_t . y_f;   da = w_f dY_t Wd_e (+ LoRA: dv = s w_f dY_t B_e,
 *     da += dv A_e);  (dg, du) = SwiGLU'(h) * da (no gradient through a
 *     clamped input beyond its bound);  dx_f = dh Wgu_e (+ gate_up
 *     adapter: dvg = s dh B_gu_e, dx_f += dvg A_gu_e)
 *   router: dl_j = w_j (dw_j - sum_i w_i dw_i)
 *   dX[t] = sum_j dx_(t,j) + sum_j dl_j Wr[idx_j]          (bf16 out;
 *           each dx_(t,j) rounded to bf16, the sum taken in fp32)
 *   dA_e = sum_f dv_f^T a_f  [E, r, I];  dB_e = s sum_f (w_f dY_t)^T v_f
 *   [E, H, r]; both fp32, overwritten, required iff the down projection
 *   has an adapter (else ignored).
 *   dA_gu_e = sum_f dvg_f^T x_t [E, r, H];  dB_gu_e = s sum_f dh_f^T vg_f
 *   [E, 2I, r]; fp32, overwritten, required iff gate_up has an adapter.
 * saved: the buffers a forward with the same dims, weights and x filled.
 * x bf16 [T, H]: the forward's input, required only with the gate_up
 * adapter (else may be NULL).  dy bf16 [T, H] in; dx bf16 [T, H] out. */
int mxfp4_moe_backward_dx(const mxfp4_moe_dims* dims, const mxfp4_moe_weights* w,
                          const mxfp4_moe_saved* saved, const uint16_t* x, const uint16_t* dy,
                          uint16_t* dx, float* dA, float* dB, float* dA_gu, float* dB_gu,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Gradients the full backward writes (fp32 ones overwritten; a NULL
 * optional pointer skips that gradient):
 *  dx     bf16 [T, H], required
 *  dA, dB, dA_gu, dB_gu   the adapter gradients, as in mxfp4_moe_backward_dx
 *  dW_gu  fp32 [E, 2I, H]  sum over expert e's routed rows of dh^T x_t
 *  dW_dn  fp32 [E, H, I]   sum of (w dY_t)^T a
 *  db_gu  fp32 [E, 2I]     sum of dh;   db_dn fp32 [E, H]  sum of w dY_t
 * dW_* are the gradients with respect to the dequantized weights (the
 * optimizer updates a master copy and requantizes it, e.g. with
 * mxfp4_quantize); an expert with no rows gets zeros. */
typedef struct mxfp4_moe_grads {
  uint16_t* dx;
  float* dA;
  float* dB;
  float* dA_gu;
  float* dB_gu;
  float* dW_gu;
  float* dW_dn;
  float* db_gu;
  float* db_dn;
} mxfp4_moe_grads;

/* Full backward for fine-tuning the MXFP4 base itself ([P1] "Relation to
 * the backward triton kernels": native MXFP4 training is the end goal;
 * [P2] MxFp4MatMulFunction with forward and backward): everything
 * mxfp4_moe_backward_dx computes, plus the base-weight and bias gradients
 * grads names.  Same arguments and checks as mxfp4_moe_backward_dx; x is
 * also required for dW_gu.  The workspace is mxfp4_moe_workspace_bytes(
 * dims, MXFP4_WS_BACKWARD_FULL).  dW_gu and dW_dn are bf16 x bf16 matrix-
 * core products summed in fp32 in a fixed order (deterministic); w a is
 * rounded to bf16 before its product. */
int mxfp4_moe_backward(const mxfp4_moe_dims* dims, const mxfp4_moe_weights* w,
                       const mxfp4_moe_saved* saved, const uint16_t* x, const uint16_t* dy,
                       const mxfp4_moe_grads* grads, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Row-wise MXFP4 quantisation, one launch ([P3] note on the row-wise
 * quantizers).  w fp32 [rows, K] -> codes uint8 [rows, K/2] (low nibble =
 * even element), scales uint8 [rows, K/32].  Per 32-block: e = the smallest
 * integer with 6 * 2^e >= max|x| (= ceil(log2(amax/6))), clamped to
 * [-127, 127] (amax = 0 gives -127); scale byte e + 127; code = nearest
 * E2M1 value to x / 2^e, ties to the even code, sign kept (so -0.0 and
 * small negatives give code 8).  K % 32 == 0.  NaN/Inf inputs are outside
 * the contract. */
int mxfp4_quantize(const float* w, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                   void* stream);

/* Row-wise MXFP8 activation quantisation (the forward's pre-pass for the
 * block-scaled activation formats, exported for tests; [P3] note on the
 * row-wise quantizers): x bf16 [rows, K] -> codes uint8 [rows, K] (OCP
 * E4M3) and scales uint8 [rows, K/32] (UE8M0).  Per 32-block: e = the
 * smallest integer with amax <= 448 * 2^e, clamped to [-127, 127] (amax = 0
 * gives -127); scale byte e + 127; code = nearest E4M3 value to x / 2^e,
 * ties to the even mantissa.  With lo_codes and lo_scales (both or
 * neither) the residual x - deq(code) is quantized the same way.  K % 32
 * == 0; x, codes and lo_codes 16-byte aligned.  Non-finite x is outside the
 * contract. */
int mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                   uint8_t* lo_codes, uint8_t* lo_scales, void* stream);

/* Dequantisation (the decode used inside every GEMM, exported for tests):
 * out[n, k] = e2m1(code) * 2^(scale - 127), exactly (every such value is a
 * float32, and a bf16 when finite; [P3] note that dequantisation is
 * bit-reproducible).  out_dtype 0 = fp32, 1 = bf16.  K % 32 == 0.
 * Scale byte 255 gives a NaN. */
int mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
                     int out_dtype, void* out, void* stream);

/* Per-kernel timing, for measurement.  mxfp4_moe_kernel_timing(1) clears
 * the totals and makes every later forward/backward call record a HIP event
 * before and after each kernel it launches, on that call's stream;
 * mxfp4_moe_kernel_timing(0) stops recording.  mxfp4_moe_kernel_times
 * waits for the recorded events, adds their elapsed times to per-kernel
 * totals and copies up to max_kernels entries: the kernel's name (a static
 * string), total milliseconds and launch count.  Returns the number of
 * distinct kernels seen, or a negative error code.  Off by default;
 * process-wide, not for concurrent use from several threads. */
int mxfp4_moe_kernel_timing(int enable);
int mxfp4_moe_kernel_times(const char** names, double* total_ms, int* launches, int max_kernels);

/* Message for the last non-zero return on this thread ("" if none). */
const char* mxfp4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_MOE_H */
