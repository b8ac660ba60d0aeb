// C ABI of libmoe: host-side argument checks, workspace sizing and launches.
// Every check runs before the first launch; no call reads device memory on
// the host or synchronises (shapes stay on the device, Megatron Core MoE
// summary, section 2.4, device-initiated kernels).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/moe.h"
#include "launch.hpp"

// The device array behind moe_dispatch_scratch (see scratch_ptr below).
static __device__ __align__(256) uint8_t scratch[MOE_DISPATCH_SCRATCH_BYTES];

namespace {

using moe::dispatch_chunks;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t act_bytes(int dt) { return dt == MOE_DTYPE_F32 ? 4 : 2; }

// FP8 E4M3 codes with either scale kind (fp32 block scales or MXFP8 E8M0)
bool is_fp8(const moe_config* c) {
  return c->weight_dtype == MOE_DTYPE_FP8_E4M3 || c->weight_dtype == MOE_DTYPE_MXFP8;
}
int weight_kind(const moe_config* c) {
  switch (c->weight_dtype) {
    case MOE_DTYPE_F32: return 0;
    case MOE_DTYPE_BF16: return 1;
    case MOE_DTYPE_FP8_E4M3: return 2;
    default: return 3;
  }
}

// Limits of the kernels' addressing, checked in 64-bit arithmetic:
//  - the grouped GEMMs address operands through buffer descriptors with
//    32-bit offsets from a per-K-step base; the largest such offset is a
//    row of one expert's weight matrix away from its start, so one expert's
//    W1 ([2f, d]) must stay below 4 GiB;
//  - tile counts (grid sizes) of every GEMM stay within 2^30 workgroups;
//  - no [A, max(d, 2f)] activation tensor exceeds 2^38 elements (more than
//    one GPU's memory holds), which keeps the element-wise grids in range.
int check_sizes(const moe_config* c) {
  const int64_t T = c->num_tokens, d = c->hidden, E = c->num_experts, k = c->top_k, f = c->ffn_hidden;
  const int64_t wb = c->weight_dtype == MOE_DTYPE_F32 ? 4 : (c->weight_dtype == MOE_DTYPE_BF16 ? 2 : 1);
  if (2 * f * d * wb > int64_t(0xffffffff)) return MOE_ERR_INVALID_ARG;
  const int64_t A = T * k, wide = d > 2 * f ? d : 2 * f;
  if (A * wide > (int64_t(1) << 38)) return MOE_ERR_INVALID_ARG;
  const int64_t row_tiles = (A + E * 127) / 128;  // the smallest row tile
  if (row_tiles * (wide / 128) > (int64_t(1) << 30)) return MOE_ERR_INVALID_ARG;
  if (E * (2 * f / 128) * (d / 128) > (int64_t(1) << 30)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Validates the configuration; returns MOE_OK or an error code.
int check_cfg(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->num_tokens < 0 || c->num_tokens > (int64_t(1) << 26)) return MOE_ERR_INVALID_ARG;
  if (c->hidden <= 0 || c->hidden % 128 != 0 || c->hidden > (1 << 20)) return MOE_ERR_INVALID_ARG;
  if (c->ffn_hidden <= 0 || c->ffn_hidden % 128 != 0 || c->ffn_hidden > (1 << 20))
    return MOE_ERR_INVALID_ARG;
  if (c->num_experts < 1 || c->num_experts > 1024) return MOE_ERR_INVALID_ARG;
  if (c->top_k < 1 || c->top_k > c->num_experts || c->top_k > 16) return MOE_ERR_INVALID_ARG;
  if (c->num_tokens * c->top_k > (int64_t(1) << 30)) return MOE_ERR_INVALID_ARG;
  if (c->score_fn != MOE_SCORE_SOFTMAX && c->score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (!(c->gate_scale == c->gate_scale)) return MOE_ERR_INVALID_ARG;
  if (c->num_groups < 1 || c->num_groups > 32 || c->num_experts % c->num_groups != 0)
    return MOE_ERR_INVALID_ARG;
  if (c->topk_groups < 1 || c->topk_groups > c->num_groups) return MOE_ERR_INVALID_ARG;
  if (c->group_score != MOE_GROUP_TOP2_SUM && c->group_score != MOE_GROUP_MAX) return MOE_ERR_INVALID_ARG;
  const bool grouped = c->num_groups > 1 && c->topk_groups < c->num_groups;
  if (grouped) {
    if (c->score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
    if (int64_t(c->topk_groups) * (c->num_experts / c->num_groups) < c->top_k) return MOE_ERR_INVALID_ARG;
  }
  if (c->ffn_mode != MOE_FFN_SWIGLU && c->ffn_mode != MOE_FFN_IDENTITY) return MOE_ERR_INVALID_ARG;
  if (c->gemm_tile < MOE_TILE_AUTO || c->gemm_tile > MOE_TILE_BIG) return MOE_ERR_INVALID_ARG;
  if (!(c->aux_coeff >= 0.0f && c->aux_coeff < __builtin_inff())) return MOE_ERR_INVALID_ARG;
  if (c->recompute < MOE_RECOMPUTE_NONE || c->recompute > MOE_RECOMPUTE_FULL) return MOE_ERR_INVALID_ARG;
  if (c->act_dtype != MOE_DTYPE_F32 && c->act_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED_DTYPE;
  if (c->weight_dtype == MOE_DTYPE_FP8_E4M3) {
    if (c->act_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED_DTYPE;
    if (c->quant_block != 128) return MOE_ERR_INVALID_ARG;
  } else if (c->weight_dtype == MOE_DTYPE_MXFP8) {
    if (c->act_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED_DTYPE;
    if (c->quant_block != 32) return MOE_ERR_INVALID_ARG;
    // the backward holds the column-quantised weights only: it cannot rerun GEMM1
    if (c->recompute == MOE_RECOMPUTE_FULL) return MOE_ERR_UNSUPPORTED_DTYPE;
  } else if (c->weight_dtype != c->act_dtype) {
    return MOE_ERR_UNSUPPORTED_DTYPE;
  }
  return check_sizes(c);
}

#define MOE_CHECK(expr)          \
  do {                           \
    const int _rc = (expr);      \
    if (_rc != MOE_OK) return _rc; \
  } while (0)

int need(const void* p) { return p ? MOE_OK : MOE_ERR_INVALID_ARG; }
int align(const void* p) { return (!p || aligned16(p)) ? MOE_OK : MOE_ERR_ALIGNMENT; }

template <typename... P>
int align_all(P... ps) {
  const void* arr[] = {static_cast<const void*>(ps)...};
  for (const void* p : arr)
    if (align(p) != MOE_OK) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

int launched() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

size_t round_up(size_t v) { return (v + 255) & ~size_t(255); }

// One [aux_blocks(T), E] array of 4-byte partials (counts or probability sums).
size_t aux_part_bytes(const moe_config* c) {
  return round_up(size_t(moe::aux_blocks(c->num_tokens)) * size_t(c->num_experts) * 4);
}

// Router backward's extra workspace for the auxiliary loss: counts + f [E].
size_t aux_bwd_bytes(const moe_config* c) {
  return c->aux_coeff != 0.0f ? aux_part_bytes(c) + round_up(size_t(c->num_experts) * 4) : 0;
}

// Workspace of moe_dispatch_scratch, for callers that cannot allocate: one
// array per device (each GPU the library runs on holds its own copy until
// the process ends), shared by every call on that device. Host code never
// passes its name to a kernel (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, once per
// device, with that device current, and is kept in g_scratch. The dispatch
// kernels overwrite every entry they read (per-chunk counts, then bases), so
// nothing needs clearing between calls.
constexpr size_t kDispatchScratchBytes = size_t(MOE_DISPATCH_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MOE_OK;
}

// An empty batch (T = 0): every expert has no rows.
int dispatch_empty(const moe_config* cfg, int32_t* counts, int32_t* offsets, void* stream) {
  MOE_CHECK(need(counts)); MOE_CHECK(need(offsets)); MOE_CHECK(align_all(counts, offsets));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  moe::launch_zero(counts, cfg->num_experts * 4, st);
  moe::launch_zero(offsets, (cfg->num_experts + 1) * 4, st);
  return launched();
}

// Checks moe_dispatch's arguments (T > 0) and fills its launch; touches no
// device state. topk_idx may be produced later on the stream (fused route).
// With from_scratch the workspace is the device array `scratch`.
int dispatch_args(const moe_config* cfg, const void* x, const int32_t* topk_idx, int32_t* counts,
                  int32_t* offsets, int32_t* row_id_map, int32_t* perm_token, void* x_perm,
                  void* x_scale, void* ws, size_t ws_bytes, bool from_scratch, moe::DispatchLaunch* out) {
  const bool fp8 = is_fp8(cfg);
  MOE_CHECK(need(x)); MOE_CHECK(need(topk_idx)); MOE_CHECK(need(counts)); MOE_CHECK(need(offsets));
  MOE_CHECK(need(row_id_map)); MOE_CHECK(need(perm_token)); MOE_CHECK(need(x_perm));
  if (fp8) MOE_CHECK(need(x_scale));
  MOE_CHECK(align(x)); MOE_CHECK(align(topk_idx)); MOE_CHECK(align(counts)); MOE_CHECK(align(offsets));
  MOE_CHECK(align(row_id_map)); MOE_CHECK(align(perm_token)); MOE_CHECK(align(x_perm));
  MOE_CHECK(align(x_scale)); MOE_CHECK(align(ws));
  const size_t need_ws = moe_workspace_size(cfg, MOE_OP_DISPATCH);
  if (from_scratch) {
    if (need_ws > kDispatchScratchBytes) return MOE_ERR_WORKSPACE;
    MOE_CHECK(scratch_ptr(&ws));
    ws_bytes = kDispatchScratchBytes;
  }
  if (!ws || ws_bytes < need_ws) return MOE_ERR_WORKSPACE;
  moe::DispatchLaunch a{};
  a.x = x; a.idx = topk_idx; a.counts = counts; a.offsets = offsets; a.row_id_map = row_id_map;
  a.perm_token = perm_token; a.x_perm = x_perm; a.x_scale = static_cast<float*>(x_scale);
  a.chunk_base = static_cast<int32_t*>(ws);
  a.counted = false;
  a.T = cfg->num_tokens; a.d = cfg->hidden; a.E = cfg->num_experts; a.k = cfg->top_k;
  a.act = cfg->act_dtype == MOE_DTYPE_BF16 ? 1 : 0;
  a.fp8 = fp8;
  a.mx = cfg->weight_dtype == MOE_DTYPE_MXFP8;
  a.qblock = cfg->quant_block;
  *out = a;
  return MOE_OK;
}

// moe_dispatch, with its workspace either the caller's (ws, ws_bytes) or,
// with from_scratch, the device array `scratch` (taken after every argument
// check, so that a refused call touches no device state).
int dispatch_call(const moe_config* cfg, const void* x, const int32_t* topk_idx, int32_t* counts,
                  int32_t* offsets, int32_t* row_id_map, int32_t* perm_token, void* x_perm,
                  void* x_scale, void* ws, size_t ws_bytes, void* stream, bool from_scratch) {
  MOE_CHECK(check_cfg(cfg));
  if (from_scratch && moe_workspace_size(cfg, MOE_OP_DISPATCH) > kDispatchScratchBytes)
    return MOE_ERR_WORKSPACE;
  if (cfg->num_tokens == 0) return dispatch_empty(cfg, counts, offsets, stream);
  moe::DispatchLaunch a{};
  MOE_CHECK(dispatch_args(cfg, x, topk_idx, counts, offsets, row_id_map, perm_token, x_perm, x_scale, ws,
                          ws_bytes, from_scratch, &a));
  moe::launch_dispatch(a, static_cast<hipStream_t>(stream));
  return launched();
}

// moe_route_dispatch counts the dispatch histogram in the top-k selection
// from this many experts up
constexpr int64_t kFuseHistMinExperts = 128;

// Checks moe_route's arguments (T > 0) and fills its launch; touches no
// device state.
int route_args(const moe_config* cfg, const void* x, const float* w_router, const float* expert_bias,
               float* logits, int32_t* topk_idx, float* topk_gate, uint8_t* routing_map,
               moe::RouteLaunch* out) {
  MOE_CHECK(need(x)); MOE_CHECK(need(w_router)); MOE_CHECK(need(logits));
  MOE_CHECK(need(topk_idx)); MOE_CHECK(need(topk_gate));
  MOE_CHECK(align(x)); MOE_CHECK(align(w_router)); MOE_CHECK(align(expert_bias));
  MOE_CHECK(align(logits)); MOE_CHECK(align(topk_idx)); MOE_CHECK(align(topk_gate));
  MOE_CHECK(align(routing_map));
  moe::RouteLaunch r{};
  r.x = x; r.w_router = w_router; r.bias = expert_bias; r.logits = logits;
  r.idx = topk_idx; r.gate = topk_gate; r.rmap = routing_map;
  r.T = cfg->num_tokens; r.d = cfg->hidden; r.E = cfg->num_experts; r.k = cfg->top_k;
  r.score_fn = cfg->score_fn; r.renorm = cfg->renormalize; r.gate_scale = cfg->gate_scale;
  r.num_groups = cfg->num_groups; r.topk_groups = cfg->topk_groups; r.group_score = cfg->group_score;
  r.act_bf16 = cfg->act_dtype == MOE_DTYPE_BF16;
  r.chunk_cnt = nullptr;
  *out = r;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype combination";
    case MOE_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t moe_workspace_size(const moe_config* cfg, int op) {
  if (check_cfg(cfg) != MOE_OK) return 0;
  const int64_t T = cfg->num_tokens, E = cfg->num_experts, k = cfg->top_k, f = cfg->ffn_hidden;
  switch (op) {
    case MOE_OP_DISPATCH: return T ? round_up(size_t(dispatch_chunks(T)) * size_t(E) * 4) : 0;
    case MOE_OP_GROUPED_FFN:
      return round_up(moe::ffn_ws_bytes(T * k, cfg->hidden, f, E, int(act_bytes(cfg->act_dtype)),
                                        weight_kind(cfg), false, cfg->recompute));
    case MOE_OP_GROUPED_FFN_BWD:
      return round_up(moe::ffn_ws_bytes(T * k, cfg->hidden, f, E, int(act_bytes(cfg->act_dtype)),
                                        weight_kind(cfg), true, cfg->recompute));
    case MOE_OP_ROUTE_BWD: {
      const int Z = moe::route_bwd_zsplit(T, cfg->hidden, E);
      const size_t parts = Z > 1 ? size_t(Z) * size_t(E) * size_t(cfg->hidden) * 4 : 0;
      return round_up(size_t(T) * size_t(E) * 4) + round_up(parts) + aux_bwd_bytes(cfg);
    }
    case MOE_OP_AUX_LOSS: return 2 * aux_part_bytes(cfg);
    default: return 0;
  }
}

int moe_route(const moe_config* cfg, const void* x, const float* w_router, const float* expert_bias,
              float* logits, int32_t* topk_idx, float* topk_gate, uint8_t* routing_map, void* ws,
              size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  MOE_CHECK(check_cfg(cfg));
  if (cfg->num_tokens == 0) return MOE_OK;  // every output is empty
  moe::RouteLaunch r{};
  MOE_CHECK(route_args(cfg, x, w_router, expert_bias, logits, topk_idx, topk_gate, routing_map, &r));
  moe::launch_route_fwd(r, static_cast<hipStream_t>(stream));
  return launched();
}

int moe_route_dispatch(const moe_config* cfg, const void* x, const float* w_router,
                       const float* expert_bias, float* logits, int32_t* topk_idx, float* topk_gate,
                       uint8_t* routing_map, int32_t* counts, int32_t* offsets, int32_t* row_id_map,
                       int32_t* perm_token, void* x_perm, void* x_scale, void* ws, size_t ws_bytes,
                       void* stream) {
  MOE_CHECK(check_cfg(cfg));
  if (cfg->num_tokens == 0) return dispatch_empty(cfg, counts, offsets, stream);
  moe::RouteLaunch r{};
  MOE_CHECK(route_args(cfg, x, w_router, expert_bias, logits, topk_idx, topk_gate, routing_map, &r));
  moe::DispatchLaunch a{};
  MOE_CHECK(dispatch_args(cfg, x, topk_idx, counts, offsets, row_id_map, perm_token, x_perm, x_scale, ws,
                          ws_bytes, false, &a));
  // from 128 experts up the selection kernel writes the per-chunk histogram
  // into the dispatch workspace and the dispatch skips its own counting
  // pass. With fewer experts the counters share a few cache lines and the
  // selection's global atomics queue on them (8 experts: route and dispatch
  // 84.7 -> 93.0 us on the Mixtral-style layer; 128: 290 -> 293 us; 256:
  // 674 us either way), so the LDS-histogram pass counts instead.
  if (cfg->num_experts >= kFuseHistMinExperts) {
    r.chunk_cnt = a.chunk_base;
    a.counted = true;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  moe::launch_route_fwd(r, st);
  moe::launch_dispatch(a, st);
  return launched();
}

int moe_dispatch(const moe_config* cfg, const void* x, const int32_t* topk_idx, int32_t* counts,
                 int32_t* offsets, int32_t* row_id_map, int32_t* perm_token, void* x_perm,
                 void* x_scale, void* ws, size_t ws_bytes, void* stream) {
  return dispatch_call(cfg, x, topk_idx, counts, offsets, row_id_map, perm_token, x_perm, x_scale, ws,
                       ws_bytes, stream, false);
}

int moe_dispatch_scratch(const moe_config* cfg, const void* x, const int32_t* topk_idx, int32_t* counts,
                         int32_t* offsets, int32_t* row_id_map, int32_t* perm_token, void* x_perm,
                         void* x_scale, void* stream) {
  return dispatch_call(cfg, x, topk_idx, counts, offsets, row_id_map, perm_token, x_perm, x_scale,
                       nullptr, 0, stream, true);
}

int moe_grouped_ffn(const moe_config* cfg, const void* x_perm, const void* x_scale,
                    const int32_t* offsets, const void* w1, const void* w1_scale, const void* w2,
                    const void* w2_scale, void* act_gu, void* act_h, void* h_scale, void* out_perm,
                    void* ws, size_t ws_bytes, void* stream) {
  MOE_CHECK(check_cfg(cfg));
  const bool identity = cfg->ffn_mode == MOE_FFN_IDENTITY;
  const bool fp8 = is_fp8(cfg);
  if (fp8 && identity) return MOE_ERR_UNSUPPORTED_DTYPE;
  if (cfg->num_tokens == 0) return MOE_OK;  // every output is empty
  MOE_CHECK(need(x_perm)); MOE_CHECK(need(offsets)); MOE_CHECK(need(out_perm));
  if (!identity) {
    MOE_CHECK(need(w1)); MOE_CHECK(need(w2));
    if (cfg->recompute < MOE_RECOMPUTE_FULL) MOE_CHECK(need(act_gu));
    if (cfg->recompute == MOE_RECOMPUTE_NONE) MOE_CHECK(need(act_h));
    if (fp8) {
      MOE_CHECK(need(x_scale)); MOE_CHECK(need(w1_scale)); MOE_CHECK(need(w2_scale));
      if (cfg->recompute == MOE_RECOMPUTE_NONE) MOE_CHECK(need(h_scale));
    }
  }
  MOE_CHECK(align_all(x_perm, x_scale, offsets, w1, w1_scale, w2, w2_scale, act_gu, act_h, h_scale, out_perm, ws));
  const size_t need_ws = moe_workspace_size(cfg, MOE_OP_GROUPED_FFN);
  if (need_ws && (!ws || ws_bytes < need_ws)) return MOE_ERR_WORKSPACE;
  moe::FfnLaunch a{};
  a.x_perm = x_perm; a.x_scale = static_cast<const float*>(x_scale); a.offsets = offsets; a.w1 = w1;
  a.w1_scale = static_cast<const float*>(w1_scale); a.w2 = w2; a.w2_scale = static_cast<const float*>(w2_scale);
  a.act_gu = act_gu; a.act_h = act_h; a.h_scale = static_cast<float*>(h_scale);
  a.out_perm = out_perm; a.ws = ws;
  a.A = cfg->num_tokens * cfg->top_k; a.d = cfg->hidden; a.f = cfg->ffn_hidden; a.E = cfg->num_experts;
  a.act = cfg->act_dtype == MOE_DTYPE_BF16 ? 1 : 0;
  a.wt = weight_kind(cfg);
  a.identity = identity;
  a.tile = cfg->gemm_tile;
  a.recompute = cfg->recompute;
  moe::launch_grouped_ffn(a, static_cast<hipStream_t>(stream));
  return launched();
}

int moe_combine(const moe_config* cfg, const void* out_perm, const int32_t* row_id_map,
                const float* topk_gate, const void* shared_out, void* y, void* stream) {
  MOE_CHECK(check_cfg(cfg));
  if (cfg->num_tokens == 0) return MOE_OK;
  MOE_CHECK(need(out_perm)); MOE_CHECK(need(row_id_map)); MOE_CHECK(need(topk_gate)); MOE_CHECK(need(y));
  MOE_CHECK(align_all(out_perm, row_id_map, topk_gate, shared_out, y));
  moe::CombineLaunch a{};
  a.src = out_perm; a.row_id_map = row_id_map; a.gate = topk_gate; a.add = shared_out; a.dst = y;
  a.T = cfg->num_tokens; a.d = cfg->hidden; a.k = cfg->top_k;
  a.act = cfg->act_dtype == MOE_DTYPE_BF16 ? 1 : 0;
  moe::launch_combine(a, static_cast<hipStream_t>(stream));
  return launched();
}

int moe_combine_bwd(const moe_config* cfg, const void* dy, const void* out_perm,
                    const int32_t* row_id_map, const float* topk_gate, void* d_out_perm, float* d_gate,
                    void* stream) {
  MOE_CHECK(check_cfg(cfg));
  if (cfg->num_tokens == 0) return MOE_OK;
  MOE_CHECK(need(dy)); MOE_CHECK(need(out_perm)); MOE_CHECK(need(row_id_map)); MOE_CHECK(need(topk_gate));
  MOE_CHECK(need(d_out_perm)); MOE_CHECK(need(d_gate));
  MOE_CHECK(align_all(dy, out_perm, row_id_map, topk_gate, d_out_perm, d_gate));
  moe::CombineBwdLaunch a{};
  a.dy = dy; a.out_perm = out_perm; a.row_id_map = row_id_map; a.gate = topk_gate;
  a.d_out_perm = d_out_perm; a.d_gate = d_gate;
  a.T = cfg->num_tokens; a.d = cfg->hidden; a.k = cfg->top_k;
  a.act = cfg->act_dtype == MOE_DTYPE_BF16 ? 1 : 0;
  moe::launch_combine_bwd(a, static_cast<hipStream_t>(stream));
  return launched();
}

int moe_grouped_ffn_bwd(const moe_config* cfg, const void* x_perm, const void* x_scale,
                        const int32_t* offsets, const void* w1, const void* w1_scale, const void* w2,
                        const void* w2_scale, const void* act_gu, const void* act_h,
                        const void* h_scale, const void* d_out_perm, void* dx_perm, void* dw1, void* dw2,
                        void* ws, size_t ws_bytes, void* stream) {
  MOE_CHECK(check_cfg(cfg));
  const bool identity = cfg->ffn_mode == MOE_FFN_IDENTITY;
  const bool fp8 = is_fp8(cfg);
  if (fp8 && identity) return MOE_ERR_UNSUPPORTED_DTYPE;
  if (cfg->num_tokens == 0) {  // no rows: the weight gradients are exact zeros
    MOE_CHECK(need(dw1)); MOE_CHECK(need(dw2)); MOE_CHECK(align_all(dw1, dw2));
    const int64_t pb = cfg->weight_dtype == MOE_DTYPE_F32 ? 4 : 2;
    const int64_t E = cfg->num_experts, d = cfg->hidden, f = cfg->ffn_hidden;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    moe::launch_zero(dw1, E * 2 * f * d * pb, st);
    moe::launch_zero(dw2, E * d * f * pb, st);
    return launched();
  }
  MOE_CHECK(need(d_out_perm)); MOE_CHECK(need(dx_perm)); MOE_CHECK(need(dw1)); MOE_CHECK(need(dw2));
  MOE_CHECK(need(offsets));
  if (!identity) {
    MOE_CHECK(need(x_perm)); MOE_CHECK(need(w1)); MOE_CHECK(need(w2));
    if (cfg->recompute < MOE_RECOMPUTE_FULL) MOE_CHECK(need(act_gu));
    if (cfg->recompute == MOE_RECOMPUTE_NONE) MOE_CHECK(need(act_h));
    if (fp8) {
      MOE_CHECK(need(x_scale)); MOE_CHECK(need(w1_scale)); MOE_CHECK(need(w2_scale));
      if (cfg->recompute == MOE_RECOMPUTE_NONE) MOE_CHECK(need(h_scale));
    }
  }
  MOE_CHECK(align_all(x_perm, x_scale, offsets, w1, w1_scale, w2, w2_scale, act_gu, act_h, h_scale, d_out_perm, dx_perm, dw1, dw2, ws));
  if (!identity && (!ws || ws_bytes < moe_workspace_size(cfg, MOE_OP_GROUPED_FFN_BWD)))
    return MOE_ERR_WORKSPACE;
  moe::FfnBwdLaunch a{};
  a.x_perm = x_perm; a.x_scale = static_cast<const float*>(x_scale); a.offsets = offsets; a.w1 = w1;
  a.w1_scale = static_cast<const float*>(w1_scale); a.w2 = w2; a.w2_scale = static_cast<const float*>(w2_scale);
  a.act_gu = act_gu; a.act_h = act_h; a.h_scale = static_cast<const float*>(h_scale);
  a.d_out = d_out_perm; a.dx_perm = dx_perm; a.dw1 = dw1; a.dw2 = dw2; a.ws = ws;
  a.A = cfg->num_tokens * cfg->top_k; a.d = cfg->hidden; a.f = cfg->ffn_hidden; a.E = cfg->num_experts;
  a.act = cfg->act_dtype == MOE_DTYPE_BF16 ? 1 : 0;
  a.wt = weight_kind(cfg);
  a.identity = identity;
  a.tile = cfg->gemm_tile;
  a.recompute = cfg->recompute;
  moe::launch_grouped_ffn_bwd(a, static_cast<hipStream_t>(stream));
  return launched();
}

int moe_dispatch_bwd(const moe_config* cfg, const void* dx_perm, const int32_t* row_id_map, const void* dx_add,
                     void* dx, void* stream) {
  MOE_CHECK(check_cfg(cfg));
  if (cfg->num_tokens == 0) return MOE_OK;
  MOE_CHECK(need(dx_perm)); MOE_CHECK(need(row_id_map)); MOE_CHECK(need(dx));
  MOE_CHECK(align_all(dx_perm, row_id_map, dx_add, dx));
  moe::CombineLaunch a{};
  a.src = dx_perm; a.row_id_map = row_id_map; a.gate = nullptr; a.add = dx_add; a.dst = dx;
  a.T = cfg->num_tokens; a.d = cfg->hidden; a.k = cfg->top_k;
  a.act = cfg->act_dtype == MOE_DTYPE_BF16 ? 1 : 0;
  moe::launch_combine(a, static_cast<hipStream_t>(stream));
  return launched();
}

int moe_route_aux_loss(const moe_config* cfg, const float* logits, const int32_t* topk_idx,
                       float* aux_loss, void* ws, size_t ws_bytes, void* stream) {
  MOE_CHECK(check_cfg(cfg));
  if (cfg->aux_coeff == 0.0f) return MOE_ERR_INVALID_ARG;
  MOE_CHECK(need(aux_loss));
  if (cfg->num_tokens == 0) {  // no tokens, no imbalance: the loss is 0
    moe::launch_zero(aux_loss, 4, static_cast<hipStream_t>(stream));
    return launched();
  }
  MOE_CHECK(need(logits)); MOE_CHECK(need(topk_idx));
  MOE_CHECK(align_all(logits, topk_idx, ws));
  if (!ws || ws_bytes < moe_workspace_size(cfg, MOE_OP_AUX_LOSS)) return MOE_ERR_WORKSPACE;
  moe::AuxLaunch a{};
  a.logits = logits; a.idx = topk_idx; a.loss = aux_loss;
  a.c_part = static_cast<int32_t*>(ws);
  a.p_part = reinterpret_cast<float*>(static_cast<char*>(ws) + aux_part_bytes(cfg));
  a.T = cfg->num_tokens; a.E = cfg->num_experts; a.k = cfg->top_k; a.coeff = cfg->aux_coeff;
  moe::launch_route_aux_loss(a, static_cast<hipStream_t>(stream));
  return launched();
}

int moe_route_bwd(const moe_config* cfg, const void* x, const float* w_router, const float* logits,
                  const int32_t* topk_idx, const float* topk_gate, const float* d_gate,
                  const float* d_aux, void* dx, float* dw_router, void* ws, size_t ws_bytes,
                  void* stream) {
  MOE_CHECK(check_cfg(cfg));
  if (cfg->num_tokens == 0) {  // a sum over no tokens: dw_router = 0
    MOE_CHECK(need(dw_router)); MOE_CHECK(align(dw_router));
    moe::launch_zero(dw_router, cfg->num_experts * cfg->hidden * 4, static_cast<hipStream_t>(stream));
    return launched();
  }
  MOE_CHECK(need(x)); MOE_CHECK(need(w_router)); MOE_CHECK(need(logits)); MOE_CHECK(need(topk_idx));
  MOE_CHECK(need(topk_gate)); MOE_CHECK(need(d_gate)); MOE_CHECK(need(dx)); MOE_CHECK(need(dw_router));
  MOE_CHECK(align_all(x, w_router, logits, topk_idx, topk_gate, d_gate, dx, dw_router, ws));
  if (!ws || ws_bytes < moe_workspace_size(cfg, MOE_OP_ROUTE_BWD)) return MOE_ERR_WORKSPACE;
  const int Z = moe::route_bwd_zsplit(cfg->num_tokens, cfg->hidden, cfg->num_experts);
  const size_t dl_bytes = round_up(size_t(cfg->num_tokens) * size_t(cfg->num_experts) * 4);
  const size_t part_bytes =
      round_up(Z > 1 ? size_t(Z) * size_t(cfg->num_experts) * size_t(cfg->hidden) * 4 : 0);
  char* w = static_cast<char*>(ws);
  moe::RouteBwdLaunch r{};
  r.x = x; r.w_router = w_router; r.logits = logits; r.idx = topk_idx; r.dgate = d_gate;
  r.dx = dx; r.dw_router = dw_router; r.dL = reinterpret_cast<float*>(w);
  r.dw_part = reinterpret_cast<float*>(w + dl_bytes);
  if (cfg->aux_coeff != 0.0f && d_aux) {
    r.d_aux = d_aux;
    r.aux_counts = reinterpret_cast<int32_t*>(w + dl_bytes + part_bytes);
    r.aux_f = reinterpret_cast<float*>(w + dl_bytes + part_bytes + aux_part_bytes(cfg));
    r.aux_coeff = cfg->aux_coeff;
  }
  r.T = cfg->num_tokens; r.d = cfg->hidden; r.E = cfg->num_experts; r.k = cfg->top_k;
  r.score_fn = cfg->score_fn; r.renorm = cfg->renormalize; r.gate_scale = cfg->gate_scale;
  r.act_bf16 = cfg->act_dtype == MOE_DTYPE_BF16;
  moe::launch_route_bwd(r, static_cast<hipStream_t>(stream));
  return launched();
}

int moe_quantize_fp8_blockwise(const void* src, int src_dtype, int64_t rows, int64_t cols, int64_t block_r,
                               int64_t block_c, uint8_t* dst, float* scale, void* stream) {
  if (src_dtype != MOE_DTYPE_F32 && src_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED_DTYPE;
  if (rows < 0 || cols < 0 || block_r < 1 || block_c < 1 || block_r * block_c > (1 << 20))
    return MOE_ERR_INVALID_ARG;
  if (rows == 0 || cols == 0) return MOE_OK;
  MOE_CHECK(need(src)); MOE_CHECK(need(dst)); MOE_CHECK(need(scale));
  if ((rows + block_r - 1) / block_r > 65535) return MOE_ERR_INVALID_ARG;
  if (block_r == 1 && block_c == 128 && cols % 128 == 0 && aligned16(src) && aligned16(dst)) {
    // activation rows: 16 lanes per block, same definition as below
    moe::launch_quant_rows(src, src_dtype == MOE_DTYPE_BF16, rows, cols, dst, scale,
                           static_cast<hipStream_t>(stream));
    return launched();
  }
  moe::QuantLaunch q{};
  q.src = src; q.src_bf16 = src_dtype == MOE_DTYPE_BF16; q.rows = rows; q.cols = cols;
  q.br = block_r; q.bc = block_c; q.dst = dst; q.scale = scale;
  moe::launch_quant_blocks(q, static_cast<hipStream_t>(stream));
  return launched();
}

int moe_quantize_mxfp8(const void* src, int src_dtype, int64_t rows, int64_t cols, int colwise, uint8_t* dst,
                       uint8_t* e8m0, void* stream) {
  if (src_dtype != MOE_DTYPE_F32 && src_dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED_DTYPE;
  if (rows < 0 || cols < 0 || (colwise != 0 && colwise != 1)) return MOE_ERR_INVALID_ARG;
  if (colwise ? rows % 32 != 0 : cols % 32 != 0) return MOE_ERR_INVALID_ARG;
  if (rows * cols > (int64_t(1) << 40)) return MOE_ERR_INVALID_ARG;
  if (rows == 0 || cols == 0) return MOE_OK;
  MOE_CHECK(need(src)); MOE_CHECK(need(dst)); MOE_CHECK(need(e8m0));
  if (!colwise && (!aligned16(src) || !aligned16(dst))) return MOE_ERR_ALIGNMENT;
  const bool bf16 = src_dtype == MOE_DTYPE_BF16;
  if (colwise) moe::launch_quant_mx_cols(src, bf16, rows, cols, dst, e8m0, static_cast<hipStream_t>(stream));
  else moe::launch_quant_mx_rows(src, bf16, rows, cols, dst, e8m0, static_cast<hipStream_t>(stream));
  return launched();
}

}  // extern "C"
