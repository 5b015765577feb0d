// C ABI of the MoE hot path: argument validation (pure host code, run before
// any HIP call), workspace carving, kernel launches, and the two-stream
// dual-microbatch forward.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <cstdint>

#include "moe.h"
#include "moe_internal.h"

using moe::align_up;

extern "C" int32_t moe_dbo_split_point(int32_t num_tokens);

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

moe_status_t check_config(const moe_config_t* c) {
  if (!c) return MOE_ERR_INVALID_ARGUMENT;
  if (c->num_tokens < 1 || c->hidden < 1 || c->intermediate < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (c->num_experts < 1 || c->num_experts > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARGUMENT;
  if (c->top_k < 1 || c->top_k > MOE_MAX_TOPK || c->top_k > c->num_experts)
    return MOE_ERR_INVALID_ARGUMENT;
  if (c->expert_begin < 0 || c->expert_end > c->num_experts || c->expert_begin >= c->expert_end)
    return MOE_ERR_INVALID_ARGUMENT;
  if (c->num_shared < 0 || c->num_shared > MOE_MAX_SHARED) return MOE_ERR_INVALID_ARGUMENT;
  if (c->score != MOE_SCORE_SOFTMAX && c->score != MOE_SCORE_SIGMOID)
    return MOE_ERR_INVALID_ARGUMENT;
  if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARGUMENT;
  if (c->weight_layout != MOE_WEIGHTS_ROW_MAJOR && c->weight_layout != MOE_WEIGHTS_PACKED)
    return MOE_ERR_INVALID_ARGUMENT;
  if (c->shared_placement != MOE_SHARED_FUSED && c->shared_placement != MOE_SHARED_BESIDE_COMBINE)
    return MOE_ERR_INVALID_ARGUMENT;
  if ((int64_t)c->num_tokens * c->top_k >= (int64_t(1) << 31)) return MOE_ERR_INVALID_ARGUMENT;
  const int q = c->dtype == MOE_BF16 ? 64 : 16;
  if (c->hidden % q != 0 || c->intermediate % q != 0) return MOE_ERR_UNSUPPORTED;
  if (c->weight_layout == MOE_WEIGHTS_PACKED &&
      (c->dtype != MOE_BF16 || c->hidden % 128 != 0 || c->intermediate % 128 != 0))
    return MOE_ERR_UNSUPPORTED;
  // A launch holds fewer than 2^32 work-items: one wave per token in the
  // router, scatter and combine; the grouped GEMMs' grids.
  if (c->num_tokens >= MOE_MAX_TOKENS) return MOE_ERR_UNSUPPORTED;
  if (moe::expert_mlp_max_workitems(*c) >= moe::kMaxWorkItems) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Intermediates of one whole-layer call, carved from a workspace.
struct LayerScratch {
  void* route_ws;
  int32_t* counts;
  int32_t* offsets;
  int32_t* src_index;
  int32_t* row_of;
  void* x_sorted;
  void* y_sorted;
  void* y_shared;
  void* dispatch_ws;
  void* mlp_ws;
  float* sums;  // [T, d] fp32: the routed combine's sums (shared experts beside the combine)
};

bool shared_beside_combine(const moe_config_t& c) {
  return c.num_shared > 0 && c.shared_placement == MOE_SHARED_BESIDE_COMBINE;
}

size_t layer_scratch(const moe_config_t& c, void* base, LayerScratch* out) {
  const size_t T = c.num_tokens, K = c.top_k, d = c.hidden;
  const size_t elem = c.dtype == MOE_BF16 ? 2 : 4;
  const size_t n_loc = c.expert_end - c.expert_begin;
  const size_t sizes[11] = {
      align_up(moe::route_workspace_bytes(c), 256),
      align_up(c.num_experts * 4, 256),
      align_up((n_loc + 1) * 4, 256),
      align_up(T * K * 4, 256),
      align_up(T * K * 4, 256),
      align_up(T * K * d * elem, 256),
      align_up(T * K * d * elem, 256),
      align_up((size_t)c.num_shared * T * d * elem, 256),
      align_up(moe::dispatch_workspace_bytes(c), 256),
      align_up(moe::mlp_workspace_bytes(c), 256),
      shared_beside_combine(c) ? align_up(T * d * 4, 256) : 0};
  size_t off[11];
  size_t total = 0;
  for (int i = 0; i < 11; ++i) {
    off[i] = total;
    total += sizes[i];
  }
  if (out) {
    char* b = static_cast<char*>(base);
    out->route_ws = b + off[0];
    out->counts = reinterpret_cast<int32_t*>(b + off[1]);
    out->offsets = reinterpret_cast<int32_t*>(b + off[2]);
    out->src_index = reinterpret_cast<int32_t*>(b + off[3]);
    out->row_of = reinterpret_cast<int32_t*>(b + off[4]);
    out->x_sorted = b + off[5];
    out->y_sorted = b + off[6];
    out->y_shared = c.num_shared > 0 ? b + off[7] : nullptr;
    out->dispatch_ws = b + off[8];
    out->mlp_ws = b + off[9];
    out->sums = shared_beside_combine(c) ? reinterpret_cast<float*>(b + off[10]) : nullptr;
  }
  return total;
}

moe_status_t check_layer_tensors(const moe_config_t& c, const moe_layer_tensors_t* t) {
  if (!t) return MOE_ERR_INVALID_ARGUMENT;
  if (!t->x || !t->w_router || !t->w_gate || !t->w_up || !t->w_down || !t->out ||
      !t->topk_ids || !t->topk_weights)
    return MOE_ERR_INVALID_ARGUMENT;
  const bool sh = c.num_shared > 0;
  if (sh != (t->ws_gate != nullptr) || sh != (t->ws_up != nullptr) ||
      sh != (t->ws_down != nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(t->x, 16) || !aligned(t->out, 16) || !aligned(t->w_router, 16) ||
      !aligned(t->w_gate, 16) || !aligned(t->w_up, 16) || !aligned(t->w_down, 16))
    return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

moe_config_t with_tokens(const moe_config_t& c, int32_t t) {
  moe_config_t r = c;
  r.num_tokens = t;
  return r;
}

// Launch the four steps of one layer call on the given streams, recording the
// events between steps when two streams are used.
moe_status_t enqueue_layer(const moe_config_t& c, const moe_layer_tensors_t& t, void* ws,
                           hipStream_t s) {
  LayerScratch sc;
  layer_scratch(c, ws, &sc);
  hipError_t e = moe::launch_route(c, t.x, t.w_router, t.bias, t.topk_ids, t.topk_weights,
                                   nullptr, sc.route_ws, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_dispatch(c, t.x, t.topk_ids, sc.counts, sc.offsets, sc.x_sorted, sc.src_index,
                           sc.row_of, sc.dispatch_ws, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (shared_beside_combine(c)) {
    // routed MLP, shared MLP, routed combine (its fp32 sums), shared rows added
    e = moe::launch_expert_mlp(c, sc.x_sorted, sc.offsets, t.w_gate, t.w_up, t.w_down,
                               sc.y_sorted, t.x, t.ws_gate, t.ws_up, t.ws_down, sc.y_shared,
                               sc.mlp_ws, s, moe::kMlpRouted);
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = moe::launch_expert_mlp(c, sc.x_sorted, sc.offsets, t.w_gate, t.w_up, t.w_down,
                               sc.y_sorted, t.x, t.ws_gate, t.ws_up, t.ws_down, sc.y_shared,
                               sc.mlp_ws, s, moe::kMlpShared);
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = moe::launch_combine_sums(c, sc.y_sorted, sc.row_of, t.topk_weights, sc.sums, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    return hip_status(moe::launch_combine_finish(c, sc.sums, sc.y_shared, t.out, s));
  }
  e = moe::launch_expert_mlp(c, sc.x_sorted, sc.offsets, t.w_gate, t.w_up, t.w_down, sc.y_sorted,
                             t.x, t.ws_gate, t.ws_up, t.ws_down, sc.y_shared, sc.mlp_ws, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_combine(c, sc.y_sorted, sc.row_of, t.topk_weights, sc.y_shared, t.out, s);
  return hip_status(e);
}

// Workspace of a layer call split at `split` (microbatch 1's scratch follows
// microbatch 0's), or of the unsplit call.
size_t dbo_workspace(const moe_config_t& c, int32_t split) {
  if (split <= 0 || split >= c.num_tokens) return layer_scratch(c, nullptr, nullptr);
  return layer_scratch(with_tokens(c, split), nullptr, nullptr) +
         layer_scratch(with_tokens(c, c.num_tokens - split), nullptr, nullptr);
}

// An upper bound of dbo_workspace over every split point: the token-linear
// parts of the two scratches add up to those of the whole call, the parts
// that do not depend on the token count (expert counts, offsets, histogram
// columns) appear twice -- once more than in a one-token call covers -- the
// chunk counts round up at most once more, and each of the eleven 256-byte
// alignments may add up to 255 bytes per scratch.
size_t dbo_workspace_bound(const moe_config_t& c) {
  const size_t whole = layer_scratch(c, nullptr, nullptr);
  const size_t one = layer_scratch(with_tokens(c, 1), nullptr, nullptr);
  return std::max(whole, dbo_workspace(c, moe_dbo_split_point(c.num_tokens))) + one + 22 * 256;
}

// The tensors of microbatch [t0, t0 + n) of a layer call.
moe_layer_tensors_t slice(const moe_config_t& c, const moe_layer_tensors_t& t, int32_t t0) {
  const size_t rb = (size_t)c.hidden * (c.dtype == MOE_BF16 ? 2 : 4);
  moe_layer_tensors_t r = t;
  r.x = static_cast<const char*>(t.x) + (size_t)t0 * rb;
  r.out = static_cast<char*>(t.out) + (size_t)t0 * rb;
  r.topk_ids = t.topk_ids + (size_t)t0 * c.top_k;
  r.topk_weights = t.topk_weights + (size_t)t0 * c.top_k;
  return r;
}

// Events of the dual-microbatch schedule.  An eager call takes them from a
// pool made once per host thread and device (a thread enqueues each call's
// records and waits in order, and a wait sees the latest record, so reusing
// them is safe and creates no runtime objects per call); they last until the
// process ends.  Under stream capture a call makes its own and destroys them
// once enqueued, as the captured graph keeps the dependencies.
enum { EV_START, EV_R0, EV_R1, EV_D0, EV_D1, EV_M0, EV_M1, EV_S0, EV_S1, EV_DONE, EV_N };
constexpr int kMaxEventDevices = 64;

hipError_t pooled_events(hipEvent_t** out) {
  struct Pool {
    hipEvent_t ev[EV_N];
    bool made;
  };
  thread_local Pool pools[kMaxEventDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxEventDevices) return hipErrorInvalidDevice;
  Pool& p = pools[dev];
  if (!p.made) {
    for (int i = 0; i < EV_N; ++i) {
      e = hipEventCreateWithFlags(&p.ev[i], hipEventDisableTiming);
      if (e != hipSuccess) {
        for (int j = 0; j < i; ++j) hipEventDestroy(p.ev[j]);
        return e;
      }
    }
    p.made = true;
  }
  *out = p.ev;
  return hipSuccess;
}

// The dual-microbatch schedule for a cut at `split` (0: the unsplit layer on
// `cs`): route on the compute stream, dispatch on the comm stream, the expert
// MLPs on compute, the combines on comm, with events between; `cs` then waits
// for both microbatches.  With the shared experts beside the combine, each
// microbatch's shared-expert MLP follows its routed MLP on compute, while its
// combine runs on comm; the shared rows are added on comm once both are done.
moe_status_t enqueue_dbo(const moe_config_t& cfg, const moe_layer_tensors_t& tensors,
                         void* workspace, int32_t split, hipStream_t cs, hipStream_t ms) {
  const int32_t T = cfg.num_tokens;
  if (split <= 0 || split >= T) return enqueue_layer(cfg, tensors, workspace, cs);

  const moe_config_t c0 = with_tokens(cfg, split), c1 = with_tokens(cfg, T - split);
  const moe_layer_tensors_t t0 = slice(cfg, tensors, 0), t1 = slice(cfg, tensors, split);
  const size_t first = layer_scratch(c0, nullptr, nullptr);

  if (cs == ms) {
    const moe_status_t st = enqueue_layer(c0, t0, workspace, cs);
    if (st != MOE_OK) return st;
    return enqueue_layer(c1, t1, static_cast<char*>(workspace) + first, cs);
  }
  LayerScratch s0, s1;
  layer_scratch(c0, workspace, &s0);
  layer_scratch(c1, static_cast<char*>(workspace) + first, &s1);

  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(cs, &cap) != hipSuccess) return MOE_ERR_HIP;
  const bool own = cap != hipStreamCaptureStatusNone;
  hipEvent_t made[EV_N] = {};
  hipEvent_t* ev = made;
  if (own) {
    for (int i = 0; i < EV_N; ++i)
      if (hipEventCreateWithFlags(&made[i], hipEventDisableTiming) != hipSuccess) {
        for (int j = 0; j < i; ++j) hipEventDestroy(made[j]);
        return MOE_ERR_HIP;
      }
  } else if (pooled_events(&ev) != hipSuccess) {
    return MOE_ERR_HIP;
  }
  moe_status_t result = MOE_OK;
  auto ok = [&](hipError_t e) {
    if (e != hipSuccess) result = MOE_ERR_HIP;
    return e == hipSuccess;
  };
  const bool beside = shared_beside_combine(cfg);
  const int parts = beside ? moe::kMlpRouted : moe::kMlpBoth;
  auto mlp = [&](const moe_config_t& c, const moe_layer_tensors_t& t, const LayerScratch& sc,
                 int which) {
    return moe::launch_expert_mlp(c, sc.x_sorted, sc.offsets, t.w_gate, t.w_up, t.w_down,
                                  sc.y_sorted, t.x, t.ws_gate, t.ws_up, t.ws_down, sc.y_shared,
                                  sc.mlp_ws, cs, which);
  };
  auto combine = [&](const moe_config_t& c, const moe_layer_tensors_t& t, const LayerScratch& sc,
                     int ev_shared) {
    if (!beside)
      return ok(moe::launch_combine(c, sc.y_sorted, sc.row_of, t.topk_weights, sc.y_shared,
                                    t.out, ms));
    return ok(moe::launch_combine_sums(c, sc.y_sorted, sc.row_of, t.topk_weights, sc.sums, ms)) &&
           ok(hipStreamWaitEvent(ms, ev[ev_shared], 0)) &&
           ok(moe::launch_combine_finish(c, sc.sums, sc.y_shared, t.out, ms));
  };
  // The comm stream must see the caller's earlier work on the compute stream.
  bool good = ok(hipEventRecord(ev[EV_START], cs)) && ok(hipStreamWaitEvent(ms, ev[EV_START], 0));
  // compute: route both microbatches.
  good = good && ok(moe::launch_route(c0, t0.x, t0.w_router, t0.bias, t0.topk_ids,
                                      t0.topk_weights, nullptr, s0.route_ws, cs)) &&
         ok(hipEventRecord(ev[EV_R0], cs)) &&
         ok(moe::launch_route(c1, t1.x, t1.w_router, t1.bias, t1.topk_ids, t1.topk_weights,
                              nullptr, s1.route_ws, cs)) &&
         ok(hipEventRecord(ev[EV_R1], cs));
  // comm: dispatch both as their routes finish.
  good = good && ok(hipStreamWaitEvent(ms, ev[EV_R0], 0)) &&
         ok(moe::launch_dispatch(c0, t0.x, t0.topk_ids, s0.counts, s0.offsets, s0.x_sorted,
                                 s0.src_index, s0.row_of, s0.dispatch_ws, ms)) &&
         ok(hipEventRecord(ev[EV_D0], ms)) && ok(hipStreamWaitEvent(ms, ev[EV_R1], 0)) &&
         ok(moe::launch_dispatch(c1, t1.x, t1.topk_ids, s1.counts, s1.offsets, s1.x_sorted,
                                 s1.src_index, s1.row_of, s1.dispatch_ws, ms)) &&
         ok(hipEventRecord(ev[EV_D1], ms));
  // compute: experts of microbatch 0 (overlapping dispatch 1), then of
  // microbatch 1; each microbatch's shared experts right after its routed
  // ones when they sit beside the combine.
  good = good && ok(hipStreamWaitEvent(cs, ev[EV_D0], 0)) && ok(mlp(c0, t0, s0, parts)) &&
         ok(hipEventRecord(ev[EV_M0], cs)) &&
         (!beside || (ok(mlp(c0, t0, s0, moe::kMlpShared)) && ok(hipEventRecord(ev[EV_S0], cs)))) &&
         ok(hipStreamWaitEvent(cs, ev[EV_D1], 0)) && ok(mlp(c1, t1, s1, parts)) &&
         ok(hipEventRecord(ev[EV_M1], cs)) &&
         (!beside || (ok(mlp(c1, t1, s1, moe::kMlpShared)) && ok(hipEventRecord(ev[EV_S1], cs))));
  // comm: combine 0 (overlapping the experts of microbatch 1), then combine 1.
  good = good && ok(hipStreamWaitEvent(ms, ev[EV_M0], 0)) && combine(c0, t0, s0, EV_S0) &&
         ok(hipStreamWaitEvent(ms, ev[EV_M1], 0)) && combine(c1, t1, s1, EV_S1) &&
         ok(hipEventRecord(ev[EV_DONE], ms)) && ok(hipStreamWaitEvent(cs, ev[EV_DONE], 0));
  (void)good;
  if (own)
    for (int i = 0; i < EV_N; ++i) hipEventDestroy(made[i]);
  return result;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t moe_dbo_split_point(int32_t num_tokens) {
  if (num_tokens < 0) return 0;
  const int64_t t_pad = ((int64_t)num_tokens + 255) / 256 * 256;
  return (int32_t)(t_pad / 2);
}

size_t moe_workspace_bytes(const moe_config_t* cfg, int32_t kind) {
  if (check_config(cfg) != MOE_OK) return 0;
  switch (kind) {
    case MOE_WS_ROUTE: return moe::route_workspace_bytes(*cfg);
    case MOE_WS_DISPATCH: return moe::dispatch_workspace_bytes(*cfg);
    case MOE_WS_EXPERT_MLP: return moe::mlp_workspace_bytes(*cfg);
    case MOE_WS_FORWARD: return layer_scratch(*cfg, nullptr, nullptr);
    case MOE_WS_FORWARD_DBO: return dbo_workspace_bound(*cfg);
    default: return 0;
  }
}

moe_status_t moe_route(const moe_config_t* cfg, const void* x, const void* w_router,
                       const float* bias, int32_t* topk_ids, float* topk_weights, float* logits,
                       void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !topk_ids || !topk_weights) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(w_router, 16)) return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = moe::route_workspace_bytes(*cfg);
  if (need > 0 && (!workspace || !aligned(workspace, 256))) return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(moe::launch_route(*cfg, x, w_router, bias, topk_ids, topk_weights, logits,
                                      workspace, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_dispatch(const moe_config_t* cfg, const void* x, const int32_t* topk_ids,
                          int32_t* expert_counts, int32_t* expert_offsets, void* x_sorted,
                          int32_t* src_index, int32_t* row_of, void* workspace,
                          size_t workspace_bytes, moe_stream_t stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!x || !topk_ids || !expert_counts || !expert_offsets || !x_sorted || !src_index ||
      !row_of || !workspace)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(x_sorted, 16) || !aligned(workspace, 256))
    return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < moe::dispatch_workspace_bytes(*cfg)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(moe::launch_dispatch(*cfg, x, topk_ids, expert_counts, expert_offsets,
                                         x_sorted, src_index, row_of, workspace,
                                         static_cast<hipStream_t>(stream)));
}

moe_status_t moe_dispatch_noalloc(const moe_config_t* cfg, const void* x, const int32_t* topk_ids,
                                  int32_t* expert_counts, int32_t* expert_offsets, void* x_sorted,
                                  int32_t* src_index, int32_t* row_of, int32_t* n_invalid,
                                  moe_stream_t stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!x || !topk_ids || !expert_counts || !expert_offsets || !x_sorted || !src_index || !row_of)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(x_sorted, 16) || (n_invalid && !aligned(n_invalid, 4)))
    return MOE_ERR_INVALID_ARGUMENT;
  // The workspace moe_dispatch would take, here carved from the library's own
  // array; its first 256 bytes (the count of invalid ids) are not used when
  // the caller asks for that count.
  if (moe::dispatch_workspace_bytes(*cfg) > moe::kNoallocScratchBytes) return MOE_ERR_UNSUPPORTED;
  void* scratch = nullptr;
  if (moe::noalloc_scratch(&scratch) != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_dispatch(*cfg, x, topk_ids, expert_counts, expert_offsets,
                                         x_sorted, src_index, row_of, scratch,
                                         static_cast<hipStream_t>(stream), nullptr, nullptr,
                                         n_invalid));
}

moe_status_t moe_dispatch_mxfp8(const moe_config_t* cfg, const void* x, const int32_t* topk_ids,
                                int32_t* expert_counts, int32_t* expert_offsets,
                                uint8_t* xq_sorted, uint8_t* xq_scales, int32_t* src_index,
                                int32_t* row_of, void* workspace, size_t workspace_bytes,
                                moe_stream_t stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_BF16 || cfg->hidden % 512 != 0) return MOE_ERR_UNSUPPORTED;
  if (!x || !topk_ids || !expert_counts || !expert_offsets || !xq_sorted || !xq_scales ||
      !src_index || !row_of || !workspace)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(xq_sorted, 16) || !aligned(xq_scales, 4) ||
      !aligned(workspace, 256))
    return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < moe::dispatch_workspace_bytes(*cfg)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(moe::launch_dispatch(*cfg, x, topk_ids, expert_counts, expert_offsets,
                                         nullptr, src_index, row_of, workspace,
                                         static_cast<hipStream_t>(stream), xq_sorted,
                                         reinterpret_cast<uint32_t*>(xq_scales)));
}

moe_status_t moe_expert_mlp(const moe_config_t* cfg, const void* x_sorted,
                            const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                            const void* w_down, void* y_sorted, const void* x,
                            const void* ws_gate, const void* ws_up, const void* ws_down,
                            void* y_shared, void* workspace, size_t workspace_bytes,
                            moe_stream_t stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!x_sorted || !expert_offsets || !w_gate || !w_up || !w_down || !y_sorted || !workspace)
    return MOE_ERR_INVALID_ARGUMENT;
  const bool sh = cfg->num_shared > 0;
  if (sh != (x != nullptr) || sh != (ws_gate != nullptr) || sh != (ws_up != nullptr) ||
      sh != (ws_down != nullptr) || sh != (y_shared != nullptr))
    return MOE_ERR_INVALID_ARGUMENT;
  for (const void* p : {x_sorted, w_gate, w_up, w_down, (const void*)y_sorted})
    if (!aligned(p, 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (sh)
    for (const void* p : {x, ws_gate, ws_up, ws_down, (const void*)y_shared})
      if (!aligned(p, 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < moe::mlp_workspace_bytes(*cfg)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(moe::launch_expert_mlp(*cfg, x_sorted, expert_offsets, w_gate, w_up, w_down,
                                           y_sorted, x, ws_gate, ws_up, ws_down, y_shared,
                                           workspace, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_combine(const moe_config_t* cfg, const void* y_sorted, const int32_t* row_of,
                         const float* topk_weights, const void* y_shared, void* out,
                         moe_stream_t stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!y_sorted || !row_of || !topk_weights || !out) return MOE_ERR_INVALID_ARGUMENT;
  if ((cfg->num_shared > 0) != (y_shared != nullptr)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(y_sorted, 16) || !aligned(out, 16) || (y_shared && !aligned(y_shared, 16)))
    return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(moe::launch_combine(*cfg, y_sorted, row_of, topk_weights, y_shared, out,
                                        static_cast<hipStream_t>(stream)));
}

moe_status_t moe_pack_weights(int32_t n, int32_t rows, int32_t cols, const void* in, void* packed,
                              moe_stream_t stream) {
  if (n < 0 || rows < 1 || cols < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (rows % 128 != 0 || cols % 64 != 0) return MOE_ERR_UNSUPPORTED;
  // one work-item per 16 bytes, 256 per workgroup, fewer than 2^32 in all
  if ((int64_t)n * rows * cols / 8 + 255 >= moe::kMaxWorkItems) return MOE_ERR_UNSUPPORTED;
  if (n == 0) return MOE_OK;
  if (!in || !packed || !aligned(in, 16) || !aligned(packed, 16)) return MOE_ERR_INVALID_ARGUMENT;
  const uintptr_t a = reinterpret_cast<uintptr_t>(in), b = reinterpret_cast<uintptr_t>(packed);
  const uintptr_t bytes = (uintptr_t)n * rows * cols * 2;
  if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARGUMENT;  // overlapping
  return hip_status(
      moe::launch_pack_weights(n, rows, cols, in, packed, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_quantize_mxfp8(int32_t rows, int32_t cols, int32_t dtype, const void* in,
                                int64_t ld, int32_t scale_layout, uint8_t* codes,
                                uint8_t* scales, moe_stream_t stream) {
  if (rows < 0 || cols <= 0 || cols % 32 != 0 || ld < cols) return MOE_ERR_INVALID_ARGUMENT;
  if (dtype != MOE_BF16 && dtype != MOE_F32) return MOE_ERR_INVALID_ARGUMENT;
  if (scale_layout != MOE_MX_ROWS && scale_layout != MOE_MX_MFMA) return MOE_ERR_INVALID_ARGUMENT;
  if (scale_layout == MOE_MX_MFMA && cols % 512 != 0) return MOE_ERR_INVALID_ARGUMENT;
  if (rows == 0) return MOE_OK;
  // One work-item per 8 elements, 256 per workgroup, fewer than 2^32 in all.
  if ((int64_t)rows * (cols / 8) + 255 >= moe::kMaxWorkItems) return MOE_ERR_UNSUPPORTED;
  if (!in || !codes || !scales) return MOE_ERR_INVALID_ARGUMENT;
  const int elem = dtype == MOE_BF16 ? 2 : 4;
  if (!aligned(in, 16) || (ld * elem) % 16 != 0 || !aligned(codes, 8) || !aligned(scales, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(moe::launch_mxfp8_quantize(rows, cols, dtype, in, ld, scale_layout, codes,
                                               scales, static_cast<hipStream_t>(stream)));
}

// Host checks shared by the block-scaled MLP and layer: configuration,
// down-projection weights (exactly one of bf16 w_down and MX-FP8 wq_down +
// scales) and the 32-bit scale indexing of the kernels.  Shared experts only
// where the caller handles them (the layer).
moe_status_t check_mxfp8_common(const moe_config_t* cfg, const void* w_down,
                                const uint8_t* wq_down, const uint8_t* wq_down_scales,
                                bool allow_shared) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_BF16 || (cfg->num_shared != 0 && !allow_shared) ||
      cfg->hidden % 512 != 0 || cfg->weight_layout != MOE_WEIGHTS_ROW_MAJOR)
    return MOE_ERR_UNSUPPORTED;
  const bool fp8_down = wq_down != nullptr || wq_down_scales != nullptr;
  if (fp8_down == (w_down != nullptr) || (fp8_down && (!wq_down || !wq_down_scales)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (w_down && !aligned(w_down, 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (fp8_down && (!aligned(wq_down, 16) || !aligned(wq_down_scales, 4)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (fp8_down && cfg->intermediate % 512 != 0) return MOE_ERR_UNSUPPORTED;
  // Each scale array is indexed in 32-bit dwords.
  const int64_t n_loc = cfg->expert_end - cfg->expert_begin;
  const int64_t rows = (int64_t)cfg->num_tokens * cfg->top_k;
  const int64_t lim = int64_t(1) << 31;
  if (rows * (cfg->hidden / 128) >= lim || n_loc * cfg->intermediate * (cfg->hidden / 128) >= lim)
    return MOE_ERR_UNSUPPORTED;
  if (fp8_down && (rows * (cfg->intermediate / 128) >= lim ||
                   n_loc * cfg->hidden * (cfg->intermediate / 128) >= lim))
    return MOE_ERR_UNSUPPORTED;
  const int64_t S = cfg->num_shared;
  if (S * cfg->intermediate * (cfg->hidden / 128) >= lim ||
      (fp8_down && S * cfg->hidden * (cfg->intermediate / 128) >= lim))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t moe_expert_mlp_mxfp8(const moe_config_t* cfg, const uint8_t* xq_sorted,
                                  const uint8_t* xq_scales, const int32_t* expert_offsets,
                                  const uint8_t* wq_gate, const uint8_t* wq_gate_scales,
                                  const uint8_t* wq_up, const uint8_t* wq_up_scales,
                                  const void* w_down, const uint8_t* wq_down,
                                  const uint8_t* wq_down_scales, void* y_sorted, void* workspace,
                                  size_t workspace_bytes, moe_stream_t stream) {
  moe_status_t st = check_mxfp8_common(cfg, w_down, wq_down, wq_down_scales, false);
  if (st != MOE_OK) return st;
  if (!xq_sorted || !xq_scales || !expert_offsets || !wq_gate || !wq_gate_scales || !wq_up ||
      !wq_up_scales || !y_sorted || !workspace)
    return MOE_ERR_INVALID_ARGUMENT;
  for (const void* p : {(const void*)xq_sorted, (const void*)wq_gate, (const void*)wq_up,
                        (const void*)y_sorted})
    if (!aligned(p, 16)) return MOE_ERR_INVALID_ARGUMENT;
  for (const void* p : {(const void*)xq_scales, (const void*)wq_gate_scales,
                        (const void*)wq_up_scales})
    if (!aligned(p, 4)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < moe::mlp_workspace_bytes(*cfg)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(moe::launch_expert_mlp_mxfp8(
      *cfg, xq_sorted, xq_scales, expert_offsets, wq_gate, wq_gate_scales, wq_up, wq_up_scales,
      w_down, wq_down, wq_down_scales, y_sorted, workspace, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_forward(const moe_config_t* cfg, const moe_layer_tensors_t* tensors,
                         void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  st = check_layer_tensors(*cfg, tensors);
  if (st != MOE_OK) return st;
  if (!workspace || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < layer_scratch(*cfg, nullptr, nullptr)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return enqueue_layer(*cfg, *tensors, workspace, static_cast<hipStream_t>(stream));
}

// Host checks of a block-scaled whole-layer call (MOE_OK when it may be
// enqueued).
moe_status_t check_forward_mxfp8(const moe_config_t* cfg, const moe_layer_tensors_mxfp8_t* t,
                                 const void* workspace, size_t workspace_bytes) {
  if (!t) return MOE_ERR_INVALID_ARGUMENT;
  moe_status_t st = check_mxfp8_common(cfg, t->w_down, t->wq_down, t->wq_down_scales, true);
  if (st != MOE_OK) return st;
  if (!t->x || !t->w_router || !t->wq_gate || !t->wq_gate_scales || !t->wq_up ||
      !t->wq_up_scales || !t->out || !t->topk_ids || !t->topk_weights)
    return MOE_ERR_INVALID_ARGUMENT;
  // Shared experts: encoded gate / up stacks, and down weights of the routed
  // experts' kind; all seven pointers NULL without shared experts.
  const bool sh = cfg->num_shared > 0;
  const bool fp8_down = t->wq_down != nullptr;
  const void* shp[7] = {t->wsq_gate, t->wsq_gate_scales, t->wsq_up, t->wsq_up_scales,
                        t->ws_down, t->wsq_down, t->wsq_down_scales};
  const bool want[7] = {sh, sh, sh, sh, sh && !fp8_down, sh && fp8_down, sh && fp8_down};
  for (int i = 0; i < 7; ++i)
    if ((shp[i] != nullptr) != want[i]) return MOE_ERR_INVALID_ARGUMENT;
  for (const void* p : {shp[0], shp[2], shp[4], shp[5]})
    if (!aligned(p, 16)) return MOE_ERR_INVALID_ARGUMENT;
  for (const void* p : {shp[1], shp[3], shp[6]})
    if (!aligned(p, 4)) return MOE_ERR_INVALID_ARGUMENT;
  for (const void* p : {t->x, t->w_router, (const void*)t->wq_gate, (const void*)t->wq_up,
                        (const void*)t->out})
    if (!aligned(p, 16)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(t->wq_gate_scales, 4) || !aligned(t->wq_up_scales, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!workspace || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < layer_scratch(*cfg, nullptr, nullptr)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

moe_status_t enqueue_forward_mxfp8(const moe_config_t& c, const moe_layer_tensors_mxfp8_t& t,
                                   void* workspace, hipStream_t s) {
  // The bf16 x_sorted region of the layer scratch (T*K*d*2 bytes) holds the
  // codes (T*K*d bytes) and, after them, the scales (T*K*d/32 bytes).
  LayerScratch sc;
  layer_scratch(c, workspace, &sc);
  const size_t n_codes = (size_t)c.num_tokens * c.top_k * c.hidden;
  uint8_t* xq = static_cast<uint8_t*>(sc.x_sorted);
  uint8_t* xs = xq + align_up(n_codes, 256);
  hipError_t e = moe::launch_route(c, t.x, t.w_router, t.bias, t.topk_ids, t.topk_weights,
                                   nullptr, sc.route_ws, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  e = moe::launch_dispatch(c, t.x, t.topk_ids, sc.counts, sc.offsets, nullptr, sc.src_index,
                           sc.row_of, sc.dispatch_ws, s, xq, reinterpret_cast<uint32_t*>(xs));
  if (e != hipSuccess) return MOE_ERR_HIP;
  // Shared experts read every token, encoded once more (T rows, MFMA layout)
  // into the y_sorted region: the gate/up kernel is its last reader and the
  // down kernel, after it on the stream, the first writer of y_sorted.
  moe::MxfpShared sh{};
  if (c.num_shared > 0) {
    // T*d + T*d/32 bytes; y_sorted holds T*K*d*2 (d is a multiple of 512)
    const size_t n_tok = (size_t)c.num_tokens * c.hidden;
    if (align_up(n_tok, 256) + n_tok / 32 > n_tok * c.top_k * 2) return MOE_ERR_UNSUPPORTED;
    uint8_t* tq = static_cast<uint8_t*>(sc.y_sorted);
    uint8_t* ts = tq + align_up(n_tok, 256);
    e = moe::launch_mxfp8_quantize(c.num_tokens, c.hidden, MOE_BF16, t.x, c.hidden, MOE_MX_MFMA,
                                   tq, ts, s);
    if (e != hipSuccess) return MOE_ERR_HIP;
    sh = moe::MxfpShared{tq,          ts,          t.wsq_gate, t.wsq_gate_scales,
                         t.wsq_up,    t.wsq_up_scales,         t.ws_down,
                         t.wsq_down,  t.wsq_down_scales,       sc.y_shared};
  }
  e = moe::launch_expert_mlp_mxfp8(c, xq, xs, sc.offsets, t.wq_gate, t.wq_gate_scales, t.wq_up,
                                   t.wq_up_scales, t.w_down, t.wq_down, t.wq_down_scales,
                                   sc.y_sorted, sc.mlp_ws, s, c.num_shared > 0 ? &sh : nullptr);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(
      moe::launch_combine(c, sc.y_sorted, sc.row_of, t.topk_weights, sc.y_shared, t.out, s));
}

moe_status_t moe_forward_mxfp8(const moe_config_t* cfg,
                               const moe_layer_tensors_mxfp8_t* tensors, void* workspace,
                               size_t workspace_bytes, moe_stream_t stream) {
  const moe_status_t st = check_forward_mxfp8(cfg, tensors, workspace, workspace_bytes);
  if (st != MOE_OK) return st;
  return enqueue_forward_mxfp8(*cfg, *tensors, workspace, static_cast<hipStream_t>(stream));
}

moe_status_t moe_forward_dbo(const moe_config_t* cfg, const moe_layer_tensors_t* tensors,
                             void* workspace, size_t workspace_bytes,
                             int32_t min_tokens_to_split, moe_stream_t compute,
                             moe_stream_t comm) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  st = check_layer_tensors(*cfg, tensors);
  if (st != MOE_OK) return st;
  if (!workspace || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < moe_workspace_bytes(cfg, MOE_WS_FORWARD_DBO))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  const int32_t T = cfg->num_tokens;
  const int32_t mid = moe_dbo_split_point(T);
  const int32_t split = (T < min_tokens_to_split || mid >= T) ? 0 : mid;
  return enqueue_dbo(*cfg, *tensors, workspace, split, static_cast<hipStream_t>(compute),
                     static_cast<hipStream_t>(comm));
}

moe_status_t moe_forward_dbo_at(const moe_config_t* cfg, const moe_layer_tensors_t* tensors,
                                void* workspace, size_t workspace_bytes, int32_t split,
                                moe_stream_t compute, moe_stream_t comm) {
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  st = check_layer_tensors(*cfg, tensors);
  if (st != MOE_OK) return st;
  if (!workspace || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  if (split <= 0 || split >= cfg->num_tokens) split = 0;
  if (workspace_bytes < dbo_workspace(*cfg, split)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return enqueue_dbo(*cfg, *tensors, workspace, split, static_cast<hipStream_t>(compute),
                     static_cast<hipStream_t>(comm));
}

int32_t moe_dbo_plan_split(int32_t num_tokens, int32_t has_prefill, int32_t decode_threshold,
                           int32_t prefill_threshold, int32_t uniform_query_len) {
  if (num_tokens < 1) return 0;
  if (num_tokens < (has_prefill ? prefill_threshold : decode_threshold)) return 0;
  int32_t cut = moe_dbo_split_point(num_tokens);
  const int32_t q = uniform_query_len;
  if (!has_prefill && q > 1 && num_tokens % q == 0) {
    // Nearest request boundary; the lower of two equally near ones.
    const int32_t r = cut % q;
    cut = (2 * r <= q) ? cut - r : cut - r + q;
  }
  return (cut > 0 && cut < num_tokens) ? cut : 0;
}

}  // extern "C"

struct moe_graph {
  hipGraphExec_t exec;
};

namespace {

// Runs `enqueue(capture_stream, second_stream)` under stream capture on two
// private streams and instantiates the result.  The second stream joins the
// capture through the events the enqueued call records.
template <typename F>
moe_status_t capture(F enqueue, moe_graph_t* out) {
  hipStream_t s0 = nullptr, s1 = nullptr;
  if (hipStreamCreateWithFlags(&s0, hipStreamNonBlocking) != hipSuccess) return MOE_ERR_HIP;
  if (hipStreamCreateWithFlags(&s1, hipStreamNonBlocking) != hipSuccess) {
    hipStreamDestroy(s0);
    return MOE_ERR_HIP;
  }
  moe_status_t st = MOE_OK;
  hipGraph_t g = nullptr;
  hipGraphExec_t exec = nullptr;
  if (hipStreamBeginCapture(s0, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    st = MOE_ERR_HIP;
  } else {
    st = enqueue(s0, s1);
    // End the capture in every case; a failed enqueue discards the graph.
    const hipError_t e = hipStreamEndCapture(s0, &g);
    if (st == MOE_OK && (e != hipSuccess || g == nullptr)) st = MOE_ERR_HIP;
  }
  if (st == MOE_OK && hipGraphInstantiate(&exec, g, nullptr, nullptr, 0) != hipSuccess)
    st = MOE_ERR_HIP;
  if (g) hipGraphDestroy(g);
  hipStreamDestroy(s1);
  hipStreamDestroy(s0);
  if (st != MOE_OK) return st;
  moe_graph_t h = new (std::nothrow) moe_graph{exec};
  if (!h) {
    hipGraphExecDestroy(exec);
    return MOE_ERR_HIP;
  }
  *out = h;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_graph_capture_forward(const moe_config_t* cfg,
                                       const moe_layer_tensors_t* tensors, void* workspace,
                                       size_t workspace_bytes, moe_graph_t* graph) {
  if (!graph) return MOE_ERR_INVALID_ARGUMENT;
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  st = check_layer_tensors(*cfg, tensors);
  if (st != MOE_OK) return st;
  if (!workspace || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < layer_scratch(*cfg, nullptr, nullptr)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return capture(
      [&](hipStream_t s0, hipStream_t) {
        return moe_forward(cfg, tensors, workspace, workspace_bytes, s0);
      },
      graph);
}

moe_status_t moe_graph_capture_forward_dbo(const moe_config_t* cfg,
                                           const moe_layer_tensors_t* tensors, void* workspace,
                                           size_t workspace_bytes, int32_t min_tokens_to_split,
                                           moe_graph_t* graph) {
  if (!graph) return MOE_ERR_INVALID_ARGUMENT;
  moe_status_t st = check_config(cfg);
  if (st != MOE_OK) return st;
  st = check_layer_tensors(*cfg, tensors);
  if (st != MOE_OK) return st;
  if (!workspace || !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < moe_workspace_bytes(cfg, MOE_WS_FORWARD_DBO))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  return capture(
      [&](hipStream_t s0, hipStream_t s1) {
        return moe_forward_dbo(cfg, tensors, workspace, workspace_bytes, min_tokens_to_split, s0,
                               s1);
      },
      graph);
}

moe_status_t moe_graph_capture_forward_mxfp8(const moe_config_t* cfg,
                                             const moe_layer_tensors_mxfp8_t* tensors,
                                             void* workspace, size_t workspace_bytes,
                                             moe_graph_t* graph) {
  if (!graph) return MOE_ERR_INVALID_ARGUMENT;
  const moe_status_t st = check_forward_mxfp8(cfg, tensors, workspace, workspace_bytes);
  if (st != MOE_OK) return st;
  return capture(
      [&](hipStream_t s0, hipStream_t) {
        return enqueue_forward_mxfp8(*cfg, *tensors, workspace, s0);
      },
      graph);
}

moe_status_t moe_graph_launch(moe_graph_t graph, moe_stream_t stream) {
  if (!graph) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_graph_destroy(moe_graph_t graph) {
  if (!graph) return MOE_ERR_INVALID_ARGUMENT;
  const hipError_t e = hipGraphExecDestroy(graph->exec);
  delete graph;
  return hip_status(e);
}

}  // extern "C"
