// Internal launch interface between the C ABI (moe_api.hip) and the kernel
// files. Arguments are validated by the caller; launchers only enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Tokens per dispatch chunk: the dispatch ranks tokens inside chunks of this
// many and keeps one expert histogram per chunk ([nchunks, E] i32).
constexpr int kChunkTok = 256;

struct RouteLaunch {
  const void* x;
  const float* w_router;
  const float* bias;
  float* logits;
  int32_t* idx;
  float* gate;
  uint8_t* rmap;
  int64_t T, d, E, k;
  int score_fn, renorm;
  float gate_scale;
  int num_groups, topk_groups, group_score;
  bool act_bf16;
  // fused route and dispatch: when set, the per-chunk expert histogram
  // [ceil(T / kChunkTok), E] i32 of the selection (cleared by the logits
  // kernel, counted by the selection kernel); nullptr otherwise
  int32_t* chunk_cnt;
};
void launch_route_fwd(const RouteLaunch& r, hipStream_t st);

struct RouteBwdLaunch {
  const void* x;
  const float* w_router;
  const float* logits;
  const int32_t* idx;
  const float* dgate;
  void* dx;
  float* dw_router;
  float* dL;       // workspace [T,E]
  float* dw_part;  // workspace [Z,E,d] (token-chunk partial sums), Z = route_bwd_zsplit
  // auxiliary-loss gradient, on when d_aux is set: counts [aux_blocks(T),E]
  // i32 and f [E] f32 in workspace
  const float* d_aux;
  int32_t* aux_counts;
  float* aux_f;
  float aux_coeff;
  int64_t T, d, E, k;
  int score_fn, renorm;
  float gate_scale;
  bool act_bf16;
};
void launch_route_bwd(const RouteBwdLaunch& r, hipStream_t st);
int route_bwd_zsplit(int64_t T, int64_t d, int64_t E);

// Load-balancing auxiliary loss: per-block partial probability sums and
// expert counts (workspace, [aux_blocks(T), E] each), then the loss.
struct AuxLaunch {
  const float* logits;
  const int32_t* idx;
  float* p_part;
  int32_t* c_part;
  float* loss;
  int64_t T, E, k;
  float coeff;
};
void launch_route_aux_loss(const AuxLaunch& a, hipStream_t st);
int aux_blocks(int64_t T);

// Dispatch: histogram -> scan -> positions -> gather.
struct DispatchLaunch {
  const void* x;
  const int32_t* idx;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_id_map;
  int32_t* perm_token;
  void* x_perm;
  float* x_scale;        // fp8 only (mx: E8M0 bytes [T*k, d/32])
  int32_t* chunk_base;   // workspace [nchunks, E]
  bool counted;          // chunk_base already holds the per-chunk expert counts (fused route)
  int64_t T, d, E, k;
  int act;               // 0 f32, 1 bf16
  bool fp8;
  bool mx;               // MXFP8: 1 x 32 blocks, E8M0 scales
  int qblock;
};
void launch_dispatch(const DispatchLaunch& a, hipStream_t st);
int64_t dispatch_chunks(int64_t T);

struct CombineLaunch {
  const void* src;       // out_perm (fwd) / dx_perm (dispatch bwd)
  const int32_t* row_id_map;
  const float* gate;     // null: unit gates (dispatch bwd)
  const void* add;       // shared_out / dx_add, may be null
  void* dst;
  int64_t T, d, k;
  int act;
};
void launch_combine(const CombineLaunch& a, hipStream_t st);

struct CombineBwdLaunch {
  const void* dy;
  const void* out_perm;
  const int32_t* row_id_map;
  const float* gate;
  void* d_out_perm;
  float* d_gate;
  int64_t T, d, k;
  int act;
};
void launch_combine_bwd(const CombineBwdLaunch& a, hipStream_t st);

// Grouped expert FFN.
struct FfnLaunch {
  const void* x_perm;
  const float* x_scale;
  const int32_t* offsets;
  const void* w1;
  const float* w1_scale;
  const void* w2;
  const float* w2_scale;
  void* act_gu;
  void* act_h;
  float* h_scale;
  void* out_perm;
  void* ws;  // ffn_ws_bytes(..., bwd = false)
  int64_t A, d, f, E;
  int act;   // 0 f32, 1 bf16
  int wt;    // 0 f32, 1 bf16, 2 fp8, 3 mxfp8 (scale pointers then hold E8M0 bytes)
  bool identity;
  int tile;       // MOE_TILE_*
  int recompute;  // 0 keep GU and H, 1 keep GU only, 2 keep neither
};
void launch_grouped_ffn(const FfnLaunch& a, hipStream_t st);
// Workspace bytes of the grouped FFN forward (bwd = false) or backward; wt as
// in FfnLaunch.
size_t ffn_ws_bytes(int64_t A, int64_t d, int64_t f, int64_t E, int act_bytes, int wt, bool bwd,
                    int recompute);
// FP8 E4M3 quantisation of rows in 1 x 128 blocks (cols a multiple of 128).
void launch_quant_rows(const void* src, bool src_bf16, int64_t rows, int64_t cols, uint8_t* q,
                       float* scale, hipStream_t st);
// MXFP8: rows in 1 x 32 blocks (cols % 32 == 0), E8M0 [rows, cols/32]; or
// columns in 32 x 1 blocks (rows % 32 == 0), E8M0 [rows/32, cols].
void launch_quant_mx_rows(const void* src, bool src_bf16, int64_t rows, int64_t cols, uint8_t* q,
                          uint8_t* e8m0, hipStream_t st);
void launch_quant_mx_cols(const void* src, bool src_bf16, int64_t rows, int64_t cols, uint8_t* q,
                          uint8_t* e8m0, hipStream_t st);

struct FfnBwdLaunch {
  const void* x_perm;
  const float* x_scale;
  const int32_t* offsets;
  const void* w1;
  const float* w1_scale;
  const void* w2;
  const float* w2_scale;
  const void* act_gu;
  const void* act_h;
  const float* h_scale;
  const void* d_out;
  void* dx_perm;
  void* dw1;
  void* dw2;
  void* ws;              // ffn_ws_bytes(..., bwd = true)
  int64_t A, d, f, E;
  int act;
  int wt;
  bool identity;
  int tile;       // MOE_TILE_*
  int recompute;  // as FfnLaunch: what the backward rebuilds in its workspace
};
void launch_grouped_ffn_bwd(const FfnBwdLaunch& a, hipStream_t st);

// Fills bytes (a multiple of 4) of device memory with zeros (a kernel, not
// a memset, so that the call can be captured into a graph).
void launch_zero(void* dst, int64_t bytes, hipStream_t st);

struct QuantLaunch {
  const void* src;
  int src_bf16;
  int64_t rows, cols, br, bc;
  uint8_t* dst;
  float* scale;
};
void launch_quant_blocks(const QuantLaunch& a, hipStream_t st);

}  // namespace moe
