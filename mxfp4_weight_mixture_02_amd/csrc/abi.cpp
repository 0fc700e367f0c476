// C ABI of the MXFP4 MoE expert block: host-side validation, workspace
// layout and launch sequencing.  Declarations and the contract live in
// include/mxfp4_moe.h.  Every check runs before the first enqueue, so an
// invalid call leaves the stream untouched ("Integrate finegrained kernels
// ...": guards refuse before the kernel is reached rather than fall back).
#include "mxfp4_moe.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.hpp"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MXFP4_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t ALIGN = 256;
// Routed-row count up to which the forward takes the decode kernels.
constexpr int64_t DECODE_MAX_ROWS = 256;
size_t up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

struct Layout {
  // offsets into the workspace; SIZE_MAX = not placed
  size_t topk_idx = SIZE_MAX, topk_w = SIZE_MAX, offsets = SIZE_MAX, sorted_rows = SIZE_MAX,
         a = SIZE_MAX, blk_hist = SIZE_MAX, tiles = SIZE_MAX, num_tiles = SIZE_MAX,
         tiles_l = SIZE_MAX, num_tiles_l = SIZE_MAX,
         y_w = SIZE_MAX, dh = SIZE_MAX, dw_part = SIZE_MAX, dxr = SIZE_MAX,
         lora_v = SIZE_MAX, lora_At = SIZE_MAX, lora_Bt = SIZE_MAX, lora_dvu = SIZE_MAX,
         lora_vg = SIZE_MAX, lora_guAt = SIZE_MAX, lora_guBt = SIZE_MAX, lora_dvg = SIZE_MAX,
         wa = SIZE_MAX, xq = SIZE_MAX, xs = SIZE_MAX, xq_lo = SIZE_MAX, xs_lo = SIZE_MAX,
         logits = SIZE_MAX, logit_part = SIZE_MAX;
  size_t total = 0;
  size_t put(size_t bytes) {
    size_t at = total;
    total += up(bytes);
    return at;
  }
};

// Which projections carry an adapter (lora_targets 0 means the down one).
bool lora_dn(const mxfp4_moe_dims& d) {
  return d.lora_rank && (d.lora_targets == 0 || (d.lora_targets & MXFP4_LORA_DOWN));
}
bool lora_gu(const mxfp4_moe_dims& d) {
  return d.lora_rank && (d.lora_targets & MXFP4_LORA_GATE_UP);
}

int check_dims(const mxfp4_moe_dims* d) {
  if (!d) return fail(MXFP4_EINVAL, "dims is NULL");
  if (d->T < 1 || d->H < 1 || d->I < 1 || d->E < 1 || d->k < 1)
    return fail(MXFP4_EINVAL, "T, H, I, E and k must be >= 1 (T=%lld H=%lld I=%lld E=%d k=%d)",
                (long long)d->T, (long long)d->H, (long long)d->I, d->E, d->k);
  if (d->H % 32 || d->I % 32)
    return fail(MXFP4_EUNSUPPORTED, "H and I must be multiples of 32 (H=%lld I=%lld)",
                (long long)d->H, (long long)d->I);
  if (d->E > 256) return fail(MXFP4_EUNSUPPORTED, "E=%d > 256", d->E);
  if (d->k > d->E || d->k > 8) return fail(MXFP4_EUNSUPPORTED, "k=%d must be <= min(E, 8)", d->k);
  if (d->T * d->k >= (int64_t(1) << 31))
    return fail(MXFP4_EUNSUPPORTED, "T*k = %lld routed rows exceed int32", (long long)(d->T * d->k));
  if (d->H > 5120 || d->I > 5120 || !mxmoe::fwd_step_k((int)d->H) || !mxmoe::fwd_step_k((int)d->I))
    return fail(MXFP4_EUNSUPPORTED, "H and I must be <= 5120 (H=%lld I=%lld)", (long long)d->H,
                (long long)d->I);
  if (d->T * d->H >= (int64_t(1) << 31))
    return fail(MXFP4_EUNSUPPORTED, "T*H = %lld elements exceed int32", (long long)(d->T * d->H));
  if (d->lora_rank != 0 && !mxmoe::lora_rank_ok(d->lora_rank))
    return fail(MXFP4_EUNSUPPORTED, "lora_rank=%d: supported ranks are 0, 8, 16, 32 and 64",
                d->lora_rank);
  if (d->lora_rank && !(d->lora_scale == d->lora_scale && d->lora_scale - d->lora_scale == 0.0f))
    return fail(MXFP4_EINVAL, "lora_scale must be finite");
  if (d->lora_targets & ~(MXFP4_LORA_DOWN | MXFP4_LORA_GATE_UP))
    return fail(MXFP4_EINVAL, "lora_targets=%d: only MXFP4_LORA_DOWN and MXFP4_LORA_GATE_UP",
                d->lora_targets);
  if (d->activation_format < MXFP4_ACT_BF16 || d->activation_format > MXFP4_ACT_MXFP8X2)
    return fail(MXFP4_EINVAL, "activation_format=%d unknown", d->activation_format);
  if (d->activation_format != MXFP4_ACT_BF16) {
    if (d->H % 64)
      return fail(MXFP4_EUNSUPPORTED, "block-scaled activations need H %% 64 == 0 (H=%lld)",
                  (long long)d->H);
    if (d->lora_rank && (d->lora_targets & MXFP4_LORA_GATE_UP))
      return fail(MXFP4_EUNSUPPORTED, "block-scaled activations with a gate_up adapter");
  }
  return MXFP4_OK;
}

Layout layout(const mxfp4_moe_dims& d, int mode) {
  Layout L;
  const size_t R = (size_t)(d.T * d.k);
  const int maxt = mxmoe::max_tiles((int64_t)R, d.E, mxmoe::MT);
  if (mode == MXFP4_WS_FORWARD || mode == MXFP4_WS_FORWARD_SAVED) {
    if (mode == MXFP4_WS_FORWARD) {
      L.topk_idx = L.put(R * 4);
      L.topk_w = L.put(R * 4);
      L.offsets = L.put((size_t)(d.E + 1) * 4);
      L.sorted_rows = L.put(R * 4);
      L.a = L.put(R * (size_t)d.I * 2);
      if (lora_dn(d)) L.lora_v = L.put(R * (size_t)d.lora_rank * 4);
      if (lora_gu(d)) L.lora_vg = L.put(R * (size_t)d.lora_rank * 4);
    }
    L.logits = L.put((size_t)d.T * d.E * 4);
    if (mxmoe::plan_fits(d.T, d.E, d.k))
      L.logit_part = L.put((size_t)mxmoe::plan_hs_parts((int)d.T, d.E, (int)d.H) * d.T * d.E * 8);
    L.blk_hist = L.put((size_t)mxmoe::router_blocks(d.T) * d.E * 4);
    L.tiles = L.put((size_t)maxt * sizeof(mxmoe::Tile));
    L.num_tiles = L.put(4);
    L.y_w = L.put(R * (size_t)d.H * 2);
    if (d.activation_format != MXFP4_ACT_BF16) {
      L.xq = L.put((size_t)d.T * d.H);
      L.xs = L.put((size_t)d.T * d.H / 32);
      if (d.activation_format == MXFP4_ACT_MXFP8X2) {
        L.xq_lo = L.put((size_t)d.T * d.H);
        L.xs_lo = L.put((size_t)d.T * d.H / 32);
      }
    }
  } else {
    // the backward GEMMs' tiles (BMT rows); with LoRA also the MT-row tiles
    // of the adapter projection
    L.tiles = L.put((size_t)mxmoe::max_tiles((int64_t)R, d.E, mxmoe::BMT) * sizeof(mxmoe::Tile));
    L.num_tiles = L.put(4);
    if (d.lora_rank) {
      L.tiles_l = L.put((size_t)maxt * sizeof(mxmoe::Tile));
      L.num_tiles_l = L.put(4);
    }
    L.dh = L.put(R * (size_t)d.I * 2 * 2);
    L.dw_part = L.put(R * (size_t)mxmoe::bwd_down_ntiles((int)d.I) * 4);
    L.dxr = L.put(R * (size_t)d.H * 2);
    if (lora_dn(d)) {
      L.lora_At = L.put((size_t)d.E * d.I * d.lora_rank * 2);
      L.lora_Bt = L.put((size_t)d.E * d.H * d.lora_rank * 2);
      L.lora_dvu = L.put(R * (size_t)d.lora_rank * 4);
    }
    if (lora_gu(d)) {
      L.lora_guAt = L.put((size_t)d.E * d.H * d.lora_rank * 2);
      L.lora_guBt = L.put((size_t)d.E * 2 * d.I * d.lora_rank * 2);
      L.lora_dvg = L.put(R * (size_t)d.lora_rank * 4);
    }
    // the full backward's base-weight gradients: w_p a_p rows for dW_dn
    if (mode == MXFP4_WS_BACKWARD_FULL) L.wa = L.put(R * (size_t)d.I * 2);
  }
  return L;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int check_weights(const mxfp4_moe_weights* w, const mxfp4_moe_dims& d) {
  if (!w) return fail(MXFP4_EINVAL, "weights is NULL");
  if (lora_dn(d)) {
    if (!w->lora_A || !w->lora_B)
      return fail(MXFP4_EINVAL, "lora_rank=%d on the down projection needs lora_A and lora_B",
                  d.lora_rank);
    if (!aligned(w->lora_A, 16) || !aligned(w->lora_B, 16))
      return fail(MXFP4_EINVAL, "lora_A and lora_B must be 16-byte aligned");
  } else if (w->lora_A || w->lora_B) {
    return fail(MXFP4_EINVAL, "lora_A/lora_B given but lora_rank is 0 or the down projection is "
                              "not a lora target");
  }
  if (lora_gu(d)) {
    if (!w->lora_gu_A || !w->lora_gu_B)
      return fail(MXFP4_EINVAL, "lora_rank=%d on gate_up needs lora_gu_A and lora_gu_B",
                  d.lora_rank);
    if (!aligned(w->lora_gu_A, 16) || !aligned(w->lora_gu_B, 16))
      return fail(MXFP4_EINVAL, "lora_gu_A and lora_gu_B must be 16-byte aligned");
  } else if (w->lora_gu_A || w->lora_gu_B) {
    return fail(MXFP4_EINVAL, "lora_gu_A/lora_gu_B given but gate_up is not a lora target");
  }
  if (!w->router_w || !w->gu_codes || !w->gu_scales || !w->dn_codes || !w->dn_scales)
    return fail(MXFP4_EINVAL, "router_w, gu_codes, gu_scales, dn_codes and dn_scales are required");
  if (!aligned(w->router_w, 16) || !aligned(w->gu_codes, 16) || !aligned(w->dn_codes, 16) ||
      !aligned(w->gu_scales, 16) || !aligned(w->dn_scales, 16))
    return fail(MXFP4_EINVAL, "router_w and the codes and scales must be 16-byte aligned");
  if ((w->gu_bias && !aligned(w->gu_bias, 16)) || (w->dn_bias && !aligned(w->dn_bias, 16)))
    return fail(MXFP4_EINVAL, "biases must be 16-byte aligned");
  return MXFP4_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MXFP4_EHIP, "%s: %s", what, hipGetErrorString(e));
  return MXFP4_OK;
}

// Optional per-kernel event timing (mxfp4_moe_kernel_timing).
struct KernelTimer {
  struct Pending {
    const char* name;
    hipEvent_t start, stop;
  };
  struct Total {
    const char* name;
    double ms;
    int launches;
  };
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<Pending> pending;
  std::vector<Total> totals;

  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void drain() {
    for (auto& p : pending) {
      float ms = 0.0f;
      if (hipEventSynchronize(p.stop) == hipSuccess &&
          hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
        bool found = false;
        for (auto& t : totals)
          if (strcmp(t.name, p.name) == 0) {
            t.ms += ms;
            t.launches += 1;
            found = true;
          }
        if (!found) totals.push_back({p.name, (double)ms, 1});
      }
      pool.push_back(p.start);
      pool.push_back(p.stop);
    }
    pending.clear();
  }
};
KernelTimer g_timer;

// Enqueue one kernel; with timing on, bracket it with events on stream s.
template <class F>
int launch_timed(F&& enqueue, const char* name, hipStream_t s) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const bool on = g_timer.on;
  if (on) {
    std::lock_guard<std::mutex> g(g_timer.mu);
    e0 = g_timer.take();
    e1 = g_timer.take();
    if (e0) (void)hipEventRecord(e0, s);
  }
  int rc = hip_status(enqueue(), name);
  if (on && e0 && e1) {
    (void)hipEventRecord(e1, s);
    std::lock_guard<std::mutex> g(g_timer.mu);
    g_timer.pending.push_back({name, e0, e1});
  }
  return rc;
}

#define LAUNCH(call, name)                                            \
  do {                                                                \
    int rc_ = launch_timed([&]() { return (call); }, name, s);        \
    if (rc_ != MXFP4_OK) return rc_;                                  \
  } while (0)

// Validation shared by the two forward entry points (everything but the
// scratch memory).
int check_forward(const mxfp4_moe_dims* dims, const mxfp4_moe_weights* w, const uint16_t* x,
                  const uint16_t* out, const mxfp4_moe_saved* saved) {
  int rc = check_dims(dims);
  if (rc) return rc;
  rc = check_weights(w, *dims);
  if (rc) return rc;
  const mxfp4_moe_dims& d = *dims;
  if (!x || !out) return fail(MXFP4_EINVAL, "x and out are required");
  if (!aligned(x, 16) || !aligned(out, 16)) return fail(MXFP4_EINVAL, "x and out must be 16-byte aligned");
  if (saved) {
    if (!saved->topk_idx || !saved->topk_w || !saved->expert_offsets || !saved->sorted_rows ||
        !saved->h || !saved->a)
      return fail(MXFP4_EINVAL, "saved: topk_idx, topk_w, expert_offsets, sorted_rows, h, a are required");
    if (!aligned(saved->h, 16) || !aligned(saved->a, 16))
      return fail(MXFP4_EINVAL, "saved h and a must be 16-byte aligned");
    if (lora_dn(d) && (!saved->lora_v || !aligned(saved->lora_v, 16)))
      return fail(MXFP4_EINVAL, "down adapter: saved lora_v is required, 16-byte aligned");
    if (lora_gu(d) && (!saved->lora_vg || !aligned(saved->lora_vg, 16)))
      return fail(MXFP4_EINVAL, "gate_up adapter: saved lora_vg is required, 16-byte aligned");
  }
  return MXFP4_OK;
}

// The forward's launches on stream s, with the workspace laid out by
// layout(d, mode) at `workspace` (validated by the caller).
int enqueue_forward(const mxfp4_moe_dims& d, const mxfp4_moe_weights* w, const uint16_t* x,
                    uint16_t* out, const mxfp4_moe_saved* saved, void* workspace,
                    hipStream_t s) {
  const int mode = saved ? MXFP4_WS_FORWARD_SAVED : MXFP4_WS_FORWARD;
  const Layout L = layout(d, mode);
  const int T = (int)d.T, H = (int)d.H, I = (int)d.I, E = d.E, k = d.k;
  const int64_t R = d.T * d.k;
  int32_t* topk_idx = saved ? saved->topk_idx : at<int32_t>(workspace, L.topk_idx);
  float* topk_w = saved ? saved->topk_w : at<float>(workspace, L.topk_w);
  int32_t* offsets = saved ? saved->expert_offsets : at<int32_t>(workspace, L.offsets);
  int32_t* sorted_rows = saved ? saved->sorted_rows : at<int32_t>(workspace, L.sorted_rows);
  uint16_t* a = saved ? saved->a : at<uint16_t>(workspace, L.a);
  uint16_t* h = saved ? saved->h : nullptr;
  int32_t* blk_hist = at<int32_t>(workspace, L.blk_hist);
  mxmoe::Tile* tiles = at<mxmoe::Tile>(workspace, L.tiles);
  int32_t* num_tiles = at<int32_t>(workspace, L.num_tiles);
  uint16_t* y_w = at<uint16_t>(workspace, L.y_w);
  float* lora_v = !lora_dn(d) ? nullptr : saved ? saved->lora_v : at<float>(workspace, L.lora_v);
  float* lora_vg = !lora_gu(d) ? nullptr : saved ? saved->lora_vg : at<float>(workspace, L.lora_vg);
  const int r = d.lora_rank;
  const int maxt = mxmoe::max_tiles(R, E, mxmoe::MT);

  float* logits = at<float>(workspace, L.logits);
  if (mxmoe::plan_fits(d.T, E, k)) {
    // partial logits over many CUs, then one workgroup for the logits,
    // top-k, offsets, permutation and tiles
    double* part = at<double>(workspace, L.logit_part);
    LAUNCH(mxmoe::launch_plan_logits(x, w->router_w, T, H, E, part, s), "router_logits");
    LAUNCH(mxmoe::launch_plan(part, w->router_b, T, H, E, k, topk_idx, topk_w, offsets,
                              sorted_rows, tiles, num_tiles, s),
           "route_plan");
  } else {
    LAUNCH(mxmoe::launch_logits(x, w->router_w, w->router_b, T, H, E, logits, s), "router_logits");
    LAUNCH(mxmoe::launch_topk(logits, T, E, k, topk_idx, topk_w, blk_hist, s), "router_topk");
    LAUNCH(mxmoe::launch_scan(blk_hist, mxmoe::router_blocks(T), E, offsets, tiles, num_tiles, s),
           "scan");
    LAUNCH(mxmoe::launch_scatter(topk_idx, blk_hist, T, k, E, sorted_rows, s), "scatter");
  }
  // the gate_up adapter's rank-space activations vg = x A_gu^T
  if (lora_vg)
    LAUNCH(mxmoe::launch_lora_proj(x, true, sorted_rows, k, w->lora_gu_A, H, r, tiles, num_tiles,
                                   maxt, 1.0f, lora_vg, s),
           "lora_vg");
  const uint16_t* gu_B = lora_vg ? w->lora_gu_B : nullptr;
  const uint16_t* dn_B = lora_v ? w->lora_B : nullptr;
  // few rows per expert: the weight-streaming decode kernels
  const bool decode = R <= DECODE_MAX_ROWS && H <= mxmoe::dec_max_k() && I <= mxmoe::dec_max_k();
  if (d.activation_format != MXFP4_ACT_BF16) {
    // block-scaled activations: quantize the token rows, then the scaled-MFMA gate_up
    uint8_t* xq = at<uint8_t>(workspace, L.xq);
    uint8_t* xs = at<uint8_t>(workspace, L.xs);
    const bool two = d.activation_format == MXFP4_ACT_MXFP8X2;
    uint8_t* xq_lo = two ? at<uint8_t>(workspace, L.xq_lo) : nullptr;
    uint8_t* xs_lo = two ? at<uint8_t>(workspace, L.xs_lo) : nullptr;
    LAUNCH(mxmoe::launch_mxfp8_quantize(x, T, H, xq, xs, xq_lo, xs_lo, s), "act_quantize");
    LAUNCH(mxmoe::launch_mx_gate_up(xq, xs, xq_lo, xs_lo, w->gu_codes, w->gu_scales, w->gu_bias,
                                    sorted_rows, tiles, num_tiles, maxt, H, I, k, d.swiglu_alpha,
                                    d.swiglu_limit, h, a, s),
           "mx_gate_up");
  } else if (decode) {
    LAUNCH(mxmoe::launch_dec_gate_up(x, w->gu_codes, w->gu_scales, w->gu_bias, sorted_rows, tiles,
                                     num_tiles, maxt, R, H, I, k, d.swiglu_alpha, d.swiglu_limit,
                                     gu_B, lora_vg, d.lora_scale, r, h, a, s),
           "dec_gate_up");
  } else {
    LAUNCH(mxmoe::launch_gate_up(x, w->gu_codes, w->gu_scales, w->gu_bias, sorted_rows, tiles,
                                 num_tiles, maxt, H, I, k, d.swiglu_alpha, d.swiglu_limit, gu_B,
                                 lora_vg, d.lora_scale, r, h, a, s),
           "gate_up");
  }
  if (lora_v)
    LAUNCH(mxmoe::launch_lora_proj(a, false, sorted_rows, k, w->lora_A, I, r, tiles, num_tiles,
                                   maxt, 1.0f, lora_v, s),
           "lora_v");
  if (decode) {
    LAUNCH(mxmoe::launch_dec_down(a, w->dn_codes, w->dn_scales, w->dn_bias, topk_w, sorted_rows,
                                  tiles, num_tiles, maxt, R, H, I, dn_B, lora_v, d.lora_scale, r,
                                  y_w, s),
           "dec_down");
    LAUNCH(mxmoe::launch_combine(y_w, d.T, H, k, out, s), "combine");
    return ok();
  }
  LAUNCH(mxmoe::launch_down(a, w->dn_codes, w->dn_scales, w->dn_bias, topk_w, sorted_rows, tiles,
                            num_tiles, maxt, H, I, dn_B, lora_v, d.lora_scale, r, y_w, s),
         "down");
  LAUNCH(mxmoe::launch_combine(y_w, d.T, H, k, out, s), "combine");
  return ok();
}

// Scratch of the no-allocation forward: one file-scope device array, of
// which every GPU the library runs on holds its own copy until the process
// ends.  Host code never uses the array's name as an address (on the host
// it is only a stand-in for the symbol): device_scratch() looks up this
// device's address once, with hipGetSymbolAddress, and kernels get that.
static __device__ __align__(256) uint8_t scratch[MXFP4_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES] = {};

int device_scratch(void** out) {
  int dev = 0;
  int rc = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (rc) return rc;
  if (dev < 0 || dev >= MAX_DEVICES) return fail(MXFP4_EUNSUPPORTED, "device %d >= %d", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    rc = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (rc) return rc;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MXFP4_OK;
}

}  // namespace

extern "C" {

const char* mxfp4_last_error(void) { return g_err; }

int mxfp4_moe_kernel_timing(int enable) {
  std::lock_guard<std::mutex> g(g_timer.mu);
  g_timer.drain();
  g_timer.totals.clear();
  g_timer.on = enable != 0;
  return ok();
}

int mxfp4_moe_kernel_times(const char** names, double* total_ms, int* launches, int max_kernels) {
  std::lock_guard<std::mutex> g(g_timer.mu);
  g_timer.drain();
  const int n = (int)g_timer.totals.size();
  for (int i = 0; i < n && i < max_kernels; ++i) {
    if (names) names[i] = g_timer.totals[i].name;
    if (total_ms) total_ms[i] = g_timer.totals[i].ms;
    if (launches) launches[i] = g_timer.totals[i].launches;
  }
  ok();
  return n;
}

size_t mxfp4_moe_workspace_bytes(const mxfp4_moe_dims* dims, int mode) {
  if (check_dims(dims) != MXFP4_OK) return 0;
  if (mode < MXFP4_WS_FORWARD || mode > MXFP4_WS_BACKWARD_FULL) {
    fail(MXFP4_EINVAL, "unknown workspace mode %d", mode);
    return 0;
  }
  ok();
  return layout(*dims, mode).total;
}

int mxfp4_moe_saved_bytes(const mxfp4_moe_dims* dims, mxfp4_moe_saved_sizes* out) {
  const int rc = check_dims(dims);
  if (rc) return rc;
  if (!out) return fail(MXFP4_EINVAL, "out is required");
  const mxfp4_moe_dims& d = *dims;
  const size_t T = (size_t)d.T, R = T * (size_t)d.k, I = (size_t)d.I;
  mxfp4_moe_saved_sizes z;
  z.topk_idx = T * d.k * sizeof(int32_t);
  z.topk_w = T * d.k * sizeof(float);
  z.expert_offsets = ((size_t)d.E + 1) * sizeof(int32_t);
  z.sorted_rows = R * sizeof(int32_t);
  z.h = R * 2 * I * sizeof(uint16_t);
  z.a = R * I * sizeof(uint16_t);
  z.lora_v = lora_dn(d) ? R * (size_t)d.lora_rank * sizeof(float) : 0;
  z.lora_vg = lora_gu(d) ? R * (size_t)d.lora_rank * sizeof(float) : 0;
  *out = z;
  return ok();
}

int mxfp4_moe_forward(const mxfp4_moe_dims* dims, const mxfp4_moe_weights* w, const uint16_t* x,
                      uint16_t* out, const mxfp4_moe_saved* saved, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int rc = check_forward(dims, w, x, out, saved);
  if (rc) return rc;
  const Layout L = layout(*dims, saved ? MXFP4_WS_FORWARD_SAVED : MXFP4_WS_FORWARD);
  if (!workspace || workspace_bytes < L.total)
    return fail(MXFP4_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, L.total);
  if (!aligned(workspace, ALIGN)) return fail(MXFP4_EINVAL, "workspace must be 256-byte aligned");
  return enqueue_forward(*dims, w, x, out, saved, workspace, static_cast<hipStream_t>(stream));
}

int mxfp4_moe_forward_noalloc(const mxfp4_moe_dims* dims, const mxfp4_moe_weights* w,
                              const uint16_t* x, uint16_t* out, const mxfp4_moe_saved* saved,
                              void* stream) {
  int rc = check_forward(dims, w, x, out, saved);
  if (rc) return rc;
  const Layout L = layout(*dims, saved ? MXFP4_WS_FORWARD_SAVED : MXFP4_WS_FORWARD);
  if (L.total > MXFP4_NOALLOC_SCRATCH_BYTES)
    return fail(MXFP4_EUNSUPPORTED,
                "these dims need %zu bytes of scratch; the static scratch holds %zu (use "
                "mxfp4_moe_forward with a workspace)", L.total, (size_t)MXFP4_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  rc = device_scratch(&ws);
  if (rc) return rc;
  return enqueue_forward(*dims, w, x, out, saved, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// The backward of both entry points: dX and the adapter gradients, and with
// mode MXFP4_WS_BACKWARD_FULL the base-weight and bias gradients g names.
int backward_impl(const mxfp4_moe_dims* dims, const mxfp4_moe_weights* w,
                  const mxfp4_moe_saved* saved, const uint16_t* x, const uint16_t* dy,
                  const mxfp4_moe_grads& g, int mode, void* workspace, size_t workspace_bytes,
                  void* stream) {
  uint16_t* dx = g.dx;
  float *dA = g.dA, *dB = g.dB, *dA_gu = g.dA_gu, *dB_gu = g.dB_gu;
  int rc = check_dims(dims);
  if (rc) return rc;
  rc = check_weights(w, *dims);
  if (rc) return rc;
  const mxfp4_moe_dims& d = *dims;
  if (!saved || !saved->topk_idx || !saved->topk_w || !saved->expert_offsets ||
      !saved->sorted_rows || !saved->h || !saved->a)
    return fail(MXFP4_EINVAL, "saved state with topk_idx, topk_w, expert_offsets, sorted_rows, h, a is required");
  if (!dy || !dx) return fail(MXFP4_EINVAL, "dy and dx are required");
  if (!aligned(dy, 16) || !aligned(dx, 16) || !aligned(saved->h, 16) || !aligned(saved->a, 16))
    return fail(MXFP4_EINVAL, "dy, dx, saved h and a must be 16-byte aligned");
  if (lora_dn(d)) {
    if (!saved->lora_v || !aligned(saved->lora_v, 16))
      return fail(MXFP4_EINVAL, "down adapter: saved lora_v is required, 16-byte aligned");
    if (!dA || !dB) return fail(MXFP4_EINVAL, "down adapter: dA and dB are required");
  }
  if (lora_gu(d)) {
    if (!saved->lora_vg || !aligned(saved->lora_vg, 16))
      return fail(MXFP4_EINVAL, "gate_up adapter: saved lora_vg is required, 16-byte aligned");
    if (!dA_gu || !dB_gu) return fail(MXFP4_EINVAL, "gate_up adapter: dA_gu and dB_gu are required");
    if (!x || !aligned(x, 16))
      return fail(MXFP4_EINVAL, "gate_up adapter: x (the forward's input) is required, 16-byte aligned");
  }
  const bool full = mode == MXFP4_WS_BACKWARD_FULL;
  if (full) {
    if (g.dW_gu && (!x || !aligned(x, 16)))
      return fail(MXFP4_EINVAL, "dW_gu needs x (the forward's input), 16-byte aligned");
  }
  const Layout L = layout(d, mode);
  if (!workspace || workspace_bytes < L.total)
    return fail(MXFP4_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, L.total);
  if (!aligned(workspace, ALIGN)) return fail(MXFP4_EINVAL, "workspace must be 256-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = (int)d.H, I = (int)d.I, E = d.E, k = d.k;
  const int64_t R = d.T * d.k;
  mxmoe::Tile* tiles = at<mxmoe::Tile>(workspace, L.tiles);
  int32_t* num_tiles = at<int32_t>(workspace, L.num_tiles);
  uint16_t* dh = at<uint16_t>(workspace, L.dh);
  float* dw_part = at<float>(workspace, L.dw_part);
  uint16_t* dxr = at<uint16_t>(workspace, L.dxr);
  const int maxt = mxmoe::max_tiles(R, E, mxmoe::BMT);
  const int r = d.lora_rank;
  const bool dn = lora_dn(d), gu = lora_gu(d);
  mxmoe::Tile* tiles_l = r ? at<mxmoe::Tile>(workspace, L.tiles_l) : nullptr;
  int32_t* num_tiles_l = r ? at<int32_t>(workspace, L.num_tiles_l) : nullptr;
  uint16_t* lora_At = dn ? at<uint16_t>(workspace, L.lora_At) : nullptr;
  uint16_t* lora_Bt = dn ? at<uint16_t>(workspace, L.lora_Bt) : nullptr;
  float* lora_dvu = dn ? at<float>(workspace, L.lora_dvu) : nullptr;
  uint16_t* lora_guAt = gu ? at<uint16_t>(workspace, L.lora_guAt) : nullptr;
  uint16_t* lora_guBt = gu ? at<uint16_t>(workspace, L.lora_guBt) : nullptr;
  float* lora_dvg = gu ? at<float>(workspace, L.lora_dvg) : nullptr;
  const int maxt_l = mxmoe::max_tiles(R, E, mxmoe::MT);

  LAUNCH(mxmoe::launch_build_tiles(saved->expert_offsets, E, mxmoe::BMT, tiles, num_tiles,
                                   mxmoe::MT, tiles_l, num_tiles_l, s),
         "bwd_tiles");
  if (dn) {
    LAUNCH(mxmoe::launch_transpose_bf16(w->lora_A, E, r, I, lora_At, s), "lora_transpose");
    LAUNCH(mxmoe::launch_transpose_bf16(w->lora_B, E, H, r, lora_Bt, s), "lora_transpose");
    // dv_u = s dY_t B_e over the token rows of dY
    LAUNCH(mxmoe::launch_lora_proj(dy, true, saved->sorted_rows, k, lora_Bt, H, r, tiles_l,
                                   num_tiles_l, maxt_l, d.lora_scale, lora_dvu, s),
           "lora_dvu");
  }
  if (gu) {
    LAUNCH(mxmoe::launch_transpose_bf16(w->lora_gu_A, E, r, H, lora_guAt, s), "lora_transpose");
    LAUNCH(mxmoe::launch_transpose_bf16(w->lora_gu_B, E, 2 * I, r, lora_guBt, s),
           "lora_transpose");
  }
  LAUNCH(mxmoe::launch_bwd_down(dy, w->dn_codes, w->dn_scales, saved->topk_w, saved->sorted_rows,
                                tiles, num_tiles, maxt, saved->h, saved->a, H, I, k,
                                d.swiglu_alpha, d.swiglu_limit, lora_At, lora_dvu, r, dh, dw_part,
                                s),
         "bwd_down");
  if (dn) {
    // dA_e[j, i] = sum_p w_p dv_u[p, j] a[p, i];  dB_e[h, j] = s sum_p w_p dY[t(p), h] v[p, j]
    LAUNCH(mxmoe::launch_lora_grad(saved->a, false, I, saved->sorted_rows, k, lora_dvu, r,
                                   saved->topk_w, 1.0f, saved->expert_offsets, E, dA,
                                   (int64_t)r * I, 1, I, s),
           "lora_grad");
    LAUNCH(mxmoe::launch_lora_grad(dy, true, H, saved->sorted_rows, k, saved->lora_v, r,
                                   saved->topk_w, d.lora_scale, saved->expert_offsets, E, dB,
                                   (int64_t)H * r, r, 1, s),
           "lora_grad");
  }
  if (gu) {
    // dv_g = s dh B_gu (dh holds the routing weight already), then
    // dA_gu_e[j, h] = sum_p dv_g[p, j] x[t(p), h];  dB_gu_e[n, j] = s sum_p dh[p, n] vg[p, j]
    LAUNCH(mxmoe::launch_lora_proj(dh, false, saved->sorted_rows, k, lora_guBt, 2 * I, r, tiles_l,
                                   num_tiles_l, maxt_l, d.lora_scale, lora_dvg, s),
           "lora_dvg");
    LAUNCH(mxmoe::launch_lora_grad(x, true, H, saved->sorted_rows, k, lora_dvg, r, nullptr, 1.0f,
                                   saved->expert_offsets, E, dA_gu, (int64_t)r * H, 1, H, s),
           "lora_grad");
    LAUNCH(mxmoe::launch_lora_grad(dh, false, 2 * I, saved->sorted_rows, k, saved->lora_vg, r,
                                   nullptr, d.lora_scale, saved->expert_offsets, E, dB_gu,
                                   (int64_t)2 * I * r, r, 1, s),
           "lora_grad");
  }
  LAUNCH(mxmoe::launch_bwd_gate_up(dh, w->gu_codes, w->gu_scales, saved->sorted_rows, tiles,
                                   num_tiles, maxt, H, I, lora_guAt, lora_dvg, r, dxr, s),
         "bwd_gate_up");
  LAUNCH(mxmoe::launch_bwd_combine(dy, dxr, dw_part, mxmoe::bwd_down_ntiles(I), saved->topk_idx,
                                   saved->topk_w, w->dn_bias, w->router_w, d.T, H, k, dx, s),
         "bwd_combine");
  if (full) {
    // base-weight and bias gradients (dh still in the workspace):
    // dW_gu = sum dh^T x, db_gu = sum dh, dW_dn = sum dY^T (w a), db_dn = sum w dY
    if (g.dW_gu)
      LAUNCH(mxmoe::launch_dw(dh, 2 * I, false, x, H, true, saved->expert_offsets,
                              saved->sorted_rows, k, E, 2 * I, H, g.dW_gu, s),
             "dw_gate_up");
    if (g.db_gu)
      LAUNCH(mxmoe::launch_colsum(dh, 2 * I, false, saved->expert_offsets, saved->sorted_rows, k,
                                  nullptr, E, 2 * I, g.db_gu, s),
             "db_gate_up");
    if (g.dW_dn) {
      uint16_t* wa = at<uint16_t>(workspace, L.wa);
      LAUNCH(mxmoe::launch_scale_rows(saved->a, R, I, saved->sorted_rows, saved->topk_w, wa, s),
             "scale_rows");
      LAUNCH(mxmoe::launch_dw(dy, H, true, wa, I, false, saved->expert_offsets, saved->sorted_rows,
                              k, E, H, I, g.dW_dn, s),
             "dw_down");
    }
    if (g.db_dn)
      LAUNCH(mxmoe::launch_colsum(dy, H, true, saved->expert_offsets, saved->sorted_rows, k,
                                  saved->topk_w, E, H, g.db_dn, s),
             "db_down");
  }
  return ok();
}

}  // namespace

extern "C" {

int mxfp4_moe_backward_dx(const mxfp4_moe_dims* dims, const mxfp4_moe_weights* w,
                          const mxfp4_moe_saved* saved, const uint16_t* x, const uint16_t* dy,
                          uint16_t* dx, float* dA, float* dB, float* dA_gu, float* dB_gu,
                          void* workspace, size_t workspace_bytes, void* stream) {
  mxfp4_moe_grads g{};
  g.dx = dx;
  g.dA = dA;
  g.dB = dB;
  g.dA_gu = dA_gu;
  g.dB_gu = dB_gu;
  return backward_impl(dims, w, saved, x, dy, g, MXFP4_WS_BACKWARD, workspace, workspace_bytes,
                       stream);
}

int mxfp4_moe_backward(const mxfp4_moe_dims* dims, const mxfp4_moe_weights* w,
                       const mxfp4_moe_saved* saved, const uint16_t* x, const uint16_t* dy,
                       const mxfp4_moe_grads* grads, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!grads) return fail(MXFP4_EINVAL, "grads is NULL");
  return backward_impl(dims, w, saved, x, dy, *grads, MXFP4_WS_BACKWARD_FULL, workspace,
                       workspace_bytes, stream);
}

int mxfp4_quantize(const float* w, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                   void* stream) {
  if (!w || !codes || !scales) return fail(MXFP4_EINVAL, "w, codes and scales are required");
  if (rows < 1 || K < 1) return fail(MXFP4_EINVAL, "rows and K must be >= 1");
  if (K % 32) return fail(MXFP4_EUNSUPPORTED, "K=%lld is not a multiple of 32", (long long)K);
  if (rows * K / 4 / 256 >= (int64_t(1) << 31)) return fail(MXFP4_EUNSUPPORTED, "tensor too large");
  if (!aligned(w, 16) || !aligned(codes, 2))
    return fail(MXFP4_EINVAL, "w must be 16-byte and codes 2-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  LAUNCH(mxmoe::launch_quantize(w, rows, K, codes, scales, s), "quantize");
  return ok();
}

int mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                   uint8_t* lo_codes, uint8_t* lo_scales, void* stream) {
  if (!x || !codes || !scales) return fail(MXFP4_EINVAL, "x, codes and scales are required");
  if (!lo_codes != !lo_scales) return fail(MXFP4_EINVAL, "lo_codes and lo_scales go together");
  if (rows < 1 || K < 1) return fail(MXFP4_EINVAL, "rows and K must be >= 1");
  if (K % 32) return fail(MXFP4_EUNSUPPORTED, "K=%lld is not a multiple of 32", (long long)K);
  if (rows * K / 32 / 256 >= (int64_t(1) << 31)) return fail(MXFP4_EUNSUPPORTED, "tensor too large");
  if (!aligned(x, 16) || !aligned(codes, 16) || (lo_codes && !aligned(lo_codes, 16)))
    return fail(MXFP4_EINVAL, "x, codes and lo_codes must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  LAUNCH(mxmoe::launch_mxfp8_quantize(x, rows, K, codes, scales, lo_codes, lo_scales, s),
         "mxfp8_quantize");
  return ok();
}

int mxfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
                     int out_dtype, void* out, void* stream) {
  if (!codes || !scales || !out) return fail(MXFP4_EINVAL, "codes, scales and out are required");
  if (rows < 1 || K < 1) return fail(MXFP4_EINVAL, "rows and K must be >= 1");
  if (K % 32) return fail(MXFP4_EUNSUPPORTED, "K=%lld is not a multiple of 32", (long long)K);
  if (out_dtype != 0 && out_dtype != 1) return fail(MXFP4_EINVAL, "out_dtype must be 0 or 1");
  if (rows * K / 8 / 256 >= (int64_t(1) << 31)) return fail(MXFP4_EUNSUPPORTED, "tensor too large");
  if (!aligned(codes, 4) || !aligned(out, 16))
    return fail(MXFP4_EINVAL, "codes must be 4-byte and out 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  LAUNCH(mxmoe::launch_dequantize(codes, scales, rows, K, out_dtype, out, s), "dequantize");
  return ok();
}

}  // extern "C"
