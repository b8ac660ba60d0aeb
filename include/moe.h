/*
 * libmoe: the token path of a Mixture-of-Experts layer on one AMD Instinct
 * MI355X (gfx950), forward and backward, behind a plain C ABI.
 *
 * The path, stage by stage, with the passage of the pages that defines it:
 *   route        a router scores every expert for every token and keeps a
 *                few; only those experts run (Megatron Core MoE summary,
 *                "O essencial" and technical summary section 1; top-k flags
 *                of the Megatron-Core skill page, "Workflow 2: MoE").
 *   dispatch     tokens are sent to their experts following the routing map
 *                (Hybrid-EP article, dispatch operator and routing-map
 *                paragraphs); on one GPU this is the permutation into
 *                expert-contiguous rows. Dropless: exactly T*k rows
 *                (Megatron Core MoE summary, section 2.4).
 *   grouped_ffn  the experts' GEMMs grouped into one kernel launch
 *                (Megatron Core MoE summary, section 2.4 "Grouped GEMM").
 *   combine      tokens come back to their original order with
 *                high-precision accumulation (Hybrid-EP article, combine
 *                operator paragraph).
 * Shapes live in device memory and are never read on the host
 * (Megatron Core MoE summary, section 2.4, device-initiated kernels), and
 * every buffer has a size known from the configuration alone (Hybrid-EP
 * article, buffer pre-allocation paragraph).
 *
 * Conventions for every call below.
 *  - Pointers are device pointers owned by the caller; the library never
 *    allocates, frees or keeps device memory. Tensors are dense and
 *    row-major. Every pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every call only enqueues work on it: no device synchronisation, no
 *    device-to-host copy, no host read of counts or offsets.
 *  - All argument checks run on the host before any launch; on failure a
 *    negative MOE_ERR_* code is returned and nothing is enqueued.
 *  - Sizes (MOE_ERR_INVALID_ARG otherwise): d and f are multiples of 128,
 *    for every dtype: the expert GEMMs tile the hidden and expert dimensions
 *    in blocks of 128 and the contraction in whole K steps, with no partial
 *    block (a finer multiple, such as 8 for 16-byte rows, is not taken).
 *    One expert's W1 ([2f, d] in the weight dtype) stays below 4 GiB, since
 *    the GEMMs address operands with 32-bit offsets from a per-step base;
 *    an [A, max(d, 2f)] tensor holds at most 2^38 elements (more than one
 *    GPU's memory), which also keeps every grid below 2^28 workgroups.
 *  - num_tokens == 0 is valid. Buffers with T or A rows may then be NULL
 *    and are not touched; outputs whose size does not depend on T get their
 *    exact values, by a fill kernel: zero counts and offsets (moe_dispatch),
 *    zero weight gradients (moe_grouped_ffn_bwd, moe_route_bwd), a zero
 *    auxiliary loss. Every other call enqueues nothing.
 *  - Outputs are overwritten unless marked "+=". For the same inputs every
 *    output is bitwise identical from run to run (no floating-point atomics).
 *  - The library keeps no global state, except the per-device scratch array
 *    of moe_dispatch_scratch; calls are thread-safe (that one excepted for
 *    overlapping calls on one GPU).
 *
 * Notation: T tokens, d hidden, E experts, k top-k, f expert hidden size,
 * A = T*k dispatched rows. "act" is cfg->act_dtype (f32 or bf16),
 * "wt" is cfg->weight_dtype (f32, bf16 or fp8 e4m3).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,       /* bad size, null required pointer, bad enum */
    MOE_ERR_UNSUPPORTED_DTYPE = -2, /* dtype combination not provided */
    MOE_ERR_ALIGNMENT = -3,         /* a pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = -4,         /* workspace missing or too small */
    MOE_ERR_HIP = -5                /* a launch failed (hipGetLastError) */
};

enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1, MOE_DTYPE_FP8_E4M3 = 2, MOE_DTYPE_MXFP8 = 3 };
enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };
enum { MOE_GROUP_TOP2_SUM = 0, MOE_GROUP_MAX = 1 };
enum { MOE_FFN_SWIGLU = 0, MOE_FFN_IDENTITY = 1 };
enum { MOE_TILE_AUTO = 0, MOE_TILE_SMALL = 1, MOE_TILE_BIG = 2 };
enum { MOE_RECOMPUTE_NONE = 0, MOE_RECOMPUTE_ACT = 1, MOE_RECOMPUTE_FULL = 2 };
enum {
    MOE_OP_ROUTE = 0,
    MOE_OP_DISPATCH = 1,
    MOE_OP_GROUPED_FFN = 2,
    MOE_OP_GROUPED_FFN_BWD = 3,
    MOE_OP_ROUTE_BWD = 4,
    MOE_OP_AUX_LOSS = 5
};

/* Layer configuration, read on the host only.
 *  score_fn    MOE_SCORE_SOFTMAX: p = softmax over all experts of the logits;
 *              MOE_SCORE_SIGMOID: s = 1/(1+exp(-logit)).
 *  renormalize 1: gates are normalised over the k selected experts.
 *  gate_scale  multiplies every gate (2.5 for DeepSeek-V3-style routing).
 *  num_groups, topk_groups  group-limited routing (sigmoid only): experts
 *              form num_groups contiguous groups; a group's score is the sum
 *              of its two best sigmoid scores (MOE_GROUP_TOP2_SUM) or its
 *              best (MOE_GROUP_MAX); top-k is taken inside the topk_groups
 *              best groups. 1 and 1 turns it off.
 *  quant_block FP8 block edge (128): activations 1 x block, weights
 *              block x block, fp32 scales.
 *  ffn_mode    MOE_FFN_IDENTITY makes every expert the identity (a test mode
 *              of route, dispatch and combine).
 *  gemm_tile   output tile of the bf16 expert GEMMs: MOE_TILE_AUTO picks per
 *              GEMM from the shapes (see DESIGN notes in gemm.hip);
 *              MOE_TILE_SMALL forces 128 x 128; MOE_TILE_BIG forces
 *              256 x 256 wherever the dimensions are multiples of 256.
 *              Results do not depend on it beyond rounding order: it exists
 *              for tuning and to test every kernel variant.
 *  aux_coeff   weight of the load-balancing auxiliary loss (0.01 in the
 *              MoE workflow of the Megatron Core page); 0 turns the loss
 *              and its gradient off.
 *  recompute   what the grouped FFN keeps between its forward and backward
 *              calls: MOE_RECOMPUTE_NONE saves GU and H; MOE_RECOMPUTE_ACT
 *              saves GU only (act_h, h_scale may be NULL) and the backward
 *              rebuilds the SwiGLU output H from it; MOE_RECOMPUTE_FULL
 *              saves nothing (act_gu may be NULL too) and the backward
 *              reruns the first expert GEMM. Outputs are bitwise the same
 *              in all three modes. */
typedef struct moe_config {
    int64_t num_tokens;  /* T */
    int64_t hidden;      /* d, a multiple of 128 */
    int64_t num_experts; /* E, 1..1024 */
    int64_t top_k;       /* k, 1..min(E, 16) */
    int64_t ffn_hidden;  /* f, a multiple of 128 */
    int32_t score_fn;
    int32_t renormalize;
    float gate_scale;
    int32_t num_groups;
    int32_t topk_groups;
    int32_t group_score;
    int32_t act_dtype;    /* MOE_DTYPE_F32 or MOE_DTYPE_BF16 */
    int32_t weight_dtype; /* act_dtype, or MOE_DTYPE_FP8_E4M3 / MOE_DTYPE_MXFP8 with bf16 act */
    int32_t quant_block;  /* 128 (FP8_E4M3) or 32 (MXFP8) */
    int32_t ffn_mode;
    int32_t gemm_tile;   /* MOE_TILE_*, 0 by default */
    float aux_coeff;     /* finite, >= 0 */
    int32_t recompute;   /* MOE_RECOMPUTE_*, 0 by default */
} moe_config;

/* Bytes of workspace the call `op` (MOE_OP_*) needs for this configuration;
 * 0 if none. Returns 0 as well for an invalid configuration. */
size_t moe_workspace_size(const moe_config *cfg, int op);

/* Router forward.
 *   x          [T,d] act
 *   w_router   [E,d] f32
 *   expert_bias [E] f32 or NULL: added to every logit before scoring and
 *              selection (it receives no gradient)
 * out:
 *   logits     [T,E] f32. logits[t,e] is the fp32 fused multiply-add
 *              recurrence acc = fma(x[t,i], w[e,i], acc) over i = 0..d-1
 *              from +0, then + bias[e]: bit-exact by construction.
 *   topk_idx   [T,k] i32, slot j = the j-th ranked expert: larger logit
 *              first, equal logits to the lower index (-0 == +0, NaN last),
 *              within the group limit when it is on.
 *   topk_gate  [T,k] f32 gates (see moe_config).
 *   routing_map [T,E] u8 or NULL: 1 where the expert is selected.
 * Workspace: none (ws may be NULL). */
int moe_route(const moe_config *cfg, const void *x, const float *w_router,
              const float *expert_bias, float *logits, int32_t *topk_idx,
              float *topk_gate, uint8_t *routing_map, void *ws,
              size_t ws_bytes, void *stream);

/* Dispatch: histogram, exclusive scan, positions and the gather of tokens
 * into expert-contiguous rows (Hybrid-EP article, dispatch operator;
 * Megatron Core MoE summary, sections 2.2 and 2.3 on permutation without
 * redundant steps or intermediate tensors).
 *   x          [T,d] act
 *   topk_idx   [T,k] i32 from moe_route or from the caller (router replay);
 *              every entry in [0,E), distinct within a token
 * out (all bit-exact):
 *   counts     [E] i32 rows per expert
 *   offsets    [E+1] i32 exclusive prefix sum, offsets[E] = A
 *   row_id_map [T,k] i32 row of (t, j): offsets[e] + #{t' < t routed to e}
 *              (rows sorted by expert, then token)
 *   perm_token [A] i32 source token of each row
 *   x_perm     [A,d]: act copy of x, or for wt = fp8 / mxfp8 the E4M3 codes
 *              of x quantised per token and 1 x quant_block block
 *   x_scale    [A, d/quant_block]: f32 scales (fp8), E8M0 bytes (mxfp8,
 *              see moe_quantize_mxfp8); NULL otherwise
 * Workspace: moe_workspace_size(cfg, MOE_OP_DISPATCH). */
int moe_dispatch(const moe_config *cfg, const void *x, const int32_t *topk_idx,
                 int32_t *counts, int32_t *offsets, int32_t *row_id_map,
                 int32_t *perm_token, void *x_perm, void *x_scale, void *ws,
                 size_t ws_bytes, void *stream);

/* Route and dispatch in one call, with the dispatch histogram fused into the
 * top-k selection (Megatron Core MoE summary, section 2.4: routing and
 * permutation in fused kernels). Arguments, results and errors are those of
 * moe_route followed by moe_dispatch on the same x and topk_idx, and every
 * output is bit-identical to theirs. The difference is where the per-chunk
 * expert histogram comes from: with E >= 128 the selection kernel counts
 * each token's k experts into it as it picks them (integer atomics, whose
 * order does not change the counts; the logits kernel clears it first), so
 * the dispatch skips its own counting pass over topk_idx; with fewer
 * experts that pass runs, as it is faster there (the atomics of few
 * experts queue on a few cache lines). For routing replay (top-k indices
 * from elsewhere) call moe_dispatch.
 * Workspace: moe_workspace_size(cfg, MOE_OP_DISPATCH) bytes, as moe_dispatch;
 * its contents are overwritten. Every argument is checked before anything is
 * enqueued, so a refused call leaves every buffer untouched. T = 0: counts
 * and offsets are zeroed, nothing else is touched. */
int moe_route_dispatch(const moe_config *cfg, const void *x, const float *w_router,
                       const float *expert_bias, float *logits, int32_t *topk_idx,
                       float *topk_gate, uint8_t *routing_map, int32_t *counts,
                       int32_t *offsets, int32_t *row_id_map, int32_t *perm_token,
                       void *x_perm, void *x_scale, void *ws, size_t ws_bytes,
                       void *stream);

/* moe_dispatch for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as moe_dispatch, without ws/ws_bytes:
 * the workspace is a device array inside the library, one per GPU, of
 * MOE_DISPATCH_SCRATCH_BYTES (8 MiB), held until the process ends. The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * its first call on a device looks the array's address up there
 * (hipGetSymbolAddress; MOE_ERR_HIP if that fails), with the device of
 * `stream` current. Every call on a GPU shares that GPU's array: calls that
 * may overlap on one GPU (different streams, or host threads, without
 * ordering between them) race and must not be made; calls on one stream
 * are ordered and safe. Nothing in the array needs clearing (each call
 * overwrites every entry it reads).
 * Errors: as moe_dispatch; MOE_ERR_WORKSPACE when the configuration needs
 * more than MOE_DISPATCH_SCRATCH_BYTES (moe_workspace_size(cfg,
 * MOE_OP_DISPATCH) = ceil(T / 256) * E * 4 bytes, rounded up to 256: e.g.
 * T up to 524288 tokens with E = 1024, up to 2^22 with E = 128). */
#define MOE_DISPATCH_SCRATCH_BYTES (8u << 20)
int moe_dispatch_scratch(const moe_config *cfg, const void *x, const int32_t *topk_idx,
                         int32_t *counts, int32_t *offsets, int32_t *row_id_map,
                         int32_t *perm_token, void *x_perm, void *x_scale, void *stream);

/* Grouped SwiGLU expert FFN forward over expert-contiguous rows (Megatron
 * Core MoE summary, section 2.4: many expert GEMMs in one kernel). For each
 * expert e and its rows r in [offsets[e], offsets[e+1]):
 *   GU = X W1_e^T ([gate | up], 2f wide), H = silu(G) * U, O = H W2_e^T.
 *   x_perm     [A,d] act (wt = fp8: E4M3 codes, with x_scale [A,d/128] f32;
 *              mxfp8: with x_scale [A,d/32] E8M0 bytes)
 *   offsets    [E+1] i32 (device)
 *   w1         [E,2f,d] wt, rows 0..f-1 gate, f..2f-1 up (fp8: + w1_scale
 *              [E,2f/128,d/128] f32; mxfp8: quantised along d, + w1_scale
 *              [E,2f,d/32] E8M0)
 *   w2         [E,d,f] wt (fp8: + w2_scale [E,d/128,f/128] f32; mxfp8:
 *              quantised along f, + w2_scale [E,d,f/32] E8M0)
 * out:
 *   act_gu     [A,2f] act: G and U (saved for the backward)
 *   act_h      [A,f]: act, or for wt = fp8 / mxfp8 E4M3 codes with h_scale
 *              [A,f/128] f32 / [A,f/32] E8M0 (H is quantised before the
 *              second GEMM)
 *   out_perm   [A,d] act
 * With cfg->recompute = MOE_RECOMPUTE_ACT, act_h and h_scale may be NULL and
 * are not written (H lives in the workspace only); with MOE_RECOMPUTE_FULL,
 * act_gu is not written either.
 * H is computed from G and U as stored in act_gu (rounded to act), so that
 * the backward can rebuild it bit for bit.
 * The shared expert of DeepSeek-style layers is this call with E = 1, k = 1
 * over the (quantised) unpermuted x and offsets {0, T}.
 * Workspace: moe_workspace_size(cfg, MOE_OP_GROUPED_FFN). */
int moe_grouped_ffn(const moe_config *cfg, const void *x_perm,
                    const void *x_scale, const int32_t *offsets,
                    const void *w1, const void *w1_scale, const void *w2,
                    const void *w2_scale, void *act_gu, void *act_h,
                    void *h_scale, void *out_perm, void *ws, size_t ws_bytes,
                    void *stream);

/* Combine forward (Hybrid-EP article, combine operator with high-precision
 * accumulation): y[t] = sum_j gate[t,j] * out_perm[row_id_map[t,j]]
 * (+ shared_out[t]), accumulated in fp32 in slot order, shared output added
 * last, one rounding to act.
 *   out_perm [A,d] act, row_id_map [T,k], topk_gate [T,k] f32,
 *   shared_out [T,d] act or NULL  ->  y [T,d] act. */
int moe_combine(const moe_config *cfg, const void *out_perm,
                const int32_t *row_id_map, const float *topk_gate,
                const void *shared_out, void *y, void *stream);

/* Combine backward.
 *   d_out_perm[row_id_map[t,j]] = gate[t,j] * dy[t]   ([A,d] act)
 *   d_gate[t,j] = <dy[t], out_perm[row_id_map[t,j]]>  ([T,k] f32, fixed-order
 *                 fp32 reduction). */
int moe_combine_bwd(const moe_config *cfg, const void *dy, const void *out_perm,
                    const int32_t *row_id_map, const float *topk_gate,
                    void *d_out_perm, float *d_gate, void *stream);

/* Grouped SwiGLU expert FFN backward. Per expert e and its rows:
 *   dH = dO W2_e, dW2_e = dO^T H,
 *   dG = dH * U * s(G) * (1 + G (1 - s(G))), dU = dH * silu(G),
 *   dX = [dG dU] W1_e, dW1_e = [dG dU]^T X.
 * Inputs as in moe_grouped_ffn plus d_out_perm [A,d] act, except that for
 * mxfp8 w1 and w2 are the copies quantised along their other dimension
 * (32 x 1 blocks: w1_scale [E,2f/32,d], w2_scale [E,d/32,f] E8M0), the
 * contraction of the two data-gradient products; mxfp8 takes no
 * MOE_RECOMPUTE_FULL (it would need the forward's w1 as well).
 * out: dx_perm [A,d] act; dw1 [E,2f,d], dw2 [E,d,f] in the parameter dtype
 * (f32 when wt is f32, else bf16), overwritten; an expert with no rows gets
 * exact zeros.
 * Low precision (the Megatron Core MoE summary trains in FP8, Resumo tecnico
 * section 2.2; the block rules are the library's reading): with
 * MOE_DTYPE_FP8_E4M3 all four products take E4M3 operands with fp32 scales
 * amax/448. The data-gradient products quantise dO and [dG dU] in 1 x 128
 * blocks along d and 2f and use the forward's 128 x 128 weight blocks. The
 * weight-gradient products quantise dO, H, [dG dU] and X in 128-row x 1
 * blocks inside each expert's rows (the first block starts at the expert's
 * first row, the last holds the rest), one scale per block and column; H and
 * X enter as their dequantised forward values. With MOE_DTYPE_MXFP8 the
 * data-gradient operands take 1 x 32 E8M0 blocks, and the weight-gradient
 * operands 32-row x 1 E8M0 blocks inside each expert's rows (the same
 * blocking as the FP8 rule, 32 rows deep, scales applied by the matrix
 * core).
 * Recompute (Megatron Core MoE summary, section 2.2: activations that take
 * memory but are cheap to compute are recomputed in the backward instead of
 * stored):
 *   MOE_RECOMPUTE_ACT: act_h and h_scale are ignored (may be NULL); the dH
 *     GEMM's epilogue, which reads G and U anyway, also writes H =
 *     silu(G) * U into the workspace ([A,f] act; fp8: [A,f] bf16, then
 *     its E4M3 codes and scales as in the forward).
 *   MOE_RECOMPUTE_FULL: act_gu is ignored too; GU and H are recomputed from
 *     x_perm and w1 by the forward's first GEMM into the workspace, which
 *     grows by [A,3f] act (fp8: + the bf16 H, codes and scales).
 * The results are bitwise those of MOE_RECOMPUTE_NONE.
 * Workspace: moe_workspace_size(cfg, MOE_OP_GROUPED_FFN_BWD). */
int moe_grouped_ffn_bwd(const moe_config *cfg, const void *x_perm,
                        const void *x_scale, const int32_t *offsets,
                        const void *w1, const void *w1_scale, const void *w2,
                        const void *w2_scale, const void *act_gu,
                        const void *act_h, const void *h_scale,
                        const void *d_out_perm, void *dx_perm, void *dw1,
                        void *dw2, void *ws, size_t ws_bytes, void *stream);

/* Dispatch backward: dx[t] = sum_j dx_perm[row_id_map[t,j]] (+ dx_add[t]),
 * fp32 in slot order, one rounding to act.
 *   dx_perm [A,d] act, dx_add [T,d] act or NULL -> dx [T,d] act. */
int moe_dispatch_bwd(const moe_config *cfg, const void *dx_perm,
                     const int32_t *row_id_map, const void *dx_add, void *dx,
                     void *stream);

/* Load-balancing auxiliary loss of the routing ("Distributed Training
 * Megatron Core" page, MoE workflow "Fluxo 2": the aux_loss balancing type
 * with coefficient 0.01; Megatron Core MoE summary, section 2.4: fused with
 * routing). The pages name the loss
 * but not its formula; this is the Switch-Transformer form:
 *   f_e = #{(t,j): topk_idx[t,j] = e} / (T k)   share of the routing slots
 *   P_e = (1/T) sum_t softmax(logits[t,:])_e    mean router probability
 *   aux_loss = aux_coeff * E * sum_e f_e P_e
 * The probabilities are the softmax over all E experts whatever score_fn is
 * (the logits include the expert bias when moe_route added one); f is a
 * constant of the selection. fp32 throughout, fixed summation order
 * (deterministic). Entries of topk_idx outside [0,E) are not counted.
 *   logits [T,E] f32, topk_idx [T,k] i32 (from moe_route)
 * out: aux_loss [1] f32 (device). T = 0 writes 0 (no tokens, no imbalance).
 * Requires aux_coeff != 0 (else MOE_ERR_INVALID_ARG).
 * Workspace: moe_workspace_size(cfg, MOE_OP_AUX_LOSS). */
int moe_route_aux_loss(const moe_config *cfg, const float *logits,
                       const int32_t *topk_idx, float *aux_loss, void *ws,
                       size_t ws_bytes, void *stream);

/* Router backward; selection, group choice and the bias are constants.
 *   dL = d(gates)/d(logits)^T d_gate for the configured score function,
 *        plus, when aux_coeff != 0 and d_aux is not NULL, the gradient of
 *        the auxiliary loss times d_aux[0]:
 *        aux_coeff * E / T * d_aux * p[t,e] * (f_e - sum_j f_j p[t,j])
 *        (p the softmax over all experts, f as in moe_route_aux_loss),
 *   dw_router = dL^T x   ([E,d] f32, overwritten)
 *   dx += dL w_router    ([T,d] act, read-modify-write)
 * Both products accumulate in fp32; with bf16 activations their operands
 * (dL, x, w_router) are rounded to bf16 first, with fp32 activations they
 * stay fp32. Results are deterministic (fixed summation order).
 * Inputs are those of moe_route plus its outputs, d_gate [T,k] f32 and
 * d_aux [1] f32 (device) or NULL.
 * Workspace: moe_workspace_size(cfg, MOE_OP_ROUTE_BWD) (larger when
 * aux_coeff != 0). */
int moe_route_bwd(const moe_config *cfg, const void *x, const float *w_router,
                  const float *logits, const int32_t *topk_idx,
                  const float *topk_gate, const float *d_gate,
                  const float *d_aux, void *dx, float *dw_router, void *ws,
                  size_t ws_bytes, void *stream);

/* FP8 E4M3 block quantisation: src [rows, cols] (src_dtype f32 or bf16) in
 * blocks of block_r x block_c: amax = max |v|, scale = amax / 448 (1 if
 * amax is 0), dst = e4m3(v / scale) rounded to nearest even, saturating.
 * scale is [ceil(rows/block_r), ceil(cols/block_c)] f32. Used for weights
 * (128 x 128) and for the shared expert's input (1 x 128). */
int moe_quantize_fp8_blockwise(const void *src, int src_dtype, int64_t rows,
                               int64_t cols, int64_t block_r, int64_t block_c,
                               uint8_t *dst, float *scale, void *stream);

/* MXFP8 quantisation (OCP Microscaling v1.0 MXFP8 E4M3, the format of the
 * Hybrid-EP article's FP8 results): src [rows, cols] (src_dtype f32 or bf16)
 * in blocks of 32 consecutive elements, along rows (colwise = 0: blocks
 * 1 x 32, cols % 32 == 0, e8m0 [rows, cols/32]) or along columns
 * (colwise = 1: blocks 32 x 1, rows % 32 == 0, e8m0 [rows/32, cols]).
 * Per block: x = the smallest integer in [-127, 127] with amax * 2^-x <=
 * 448 (0 for an all-zero block), e8m0 = x + 127, dst = e4m3(v * 2^-x)
 * rounded to nearest even (no element saturates). Weights are quantised
 * both ways: rows for the forward products, columns for the data-gradient
 * products, whose contraction runs along the weights' other dimension.
 * Errors: MOE_ERR_INVALID_ARG (sizes, NULL), MOE_ERR_UNSUPPORTED_DTYPE,
 * MOE_ERR_ALIGNMENT (colwise = 0 needs 16-byte aligned src and dst). */
int moe_quantize_mxfp8(const void *src, int src_dtype, int64_t rows, int64_t cols,
                       int colwise, uint8_t *dst, uint8_t *e8m0, void *stream);

/* Static description of a status code. */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
