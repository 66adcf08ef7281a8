/*
 * moe_mxfp4.h — C ABI of the MI355X (gfx950) routed MXFP4 Mixture-of-Experts feed-forward for decode.
 *
 * The layer is the path the pages keep measuring as the decode bottleneck (b70-optimization-lab,
 * "MTP1 Post-Portfolio Eager-Cycle Profile", Post-Portfolio Device Attribution table; vllm.cpp PR #52;
 * "Chunk 8.0"): route each token to its top-k experts, group the (token, slot) pairs by expert, run
 * each active expert's MXFP4 gate/up GEMM with a SwiGLU epilogue and its MXFP4 down GEMM, then
 * combine each token's k expert outputs with its routing weights. Three calls cover it, in order:
 *
 *     moe_route_topk  ->  moe_group_tokens  ->  moe_mxfp4_ffn
 *
 * (moe_route_group runs the first two as one call, in a single launch for small batches.)
 *
 * Conventions shared by every call:
 *   - Pointers marked [dev] are device pointers (hipMalloc'd or equivalent) on the current device;
 *     [host] pointers are host memory. The caller owns and allocates every buffer; the library
 *     allocates nothing, never synchronises, and returns before the GPU work completes.
 *   - `stream` is a hipStream_t (NULL = the default stream). All work is enqueued on it in order, so
 *     the three calls can be captured together into one HIP graph.
 *   - Shapes and pointers are validated on the host BEFORE anything is launched: a call that
 *     returns an error has enqueued nothing. Device-resident contents (ids out of range, NaN
 *     logits) are not validated; they are preconditions. After launching, a launch failure reported
 *     by hipGetLastError() is returned as MOE_ERR_LAUNCH.
 *   - All arrays are row-major and contiguous. T tokens, H hidden size, I per-expert intermediate
 *     size, E experts, k experts per token; P = T*k routed pairs numbered p = t*k + j.
 *   - bfloat16 values are passed as their 16-bit patterns (uint16_t).
 *
 * MXFP4 weights (OCP Microscaling Formats v1.0): 32-element blocks of E2M1 codes sharing one E8M0
 * scale byte 2^(s-127). Codes are packed two per byte, the element with the even index in the low
 * nibble; blocks run along the reduction dimension (H for w13, I for w2):
 *   w13_q u8[E, 2I, H/2]  rows [0, I) are the gate projection, rows [I, 2I) the up projection
 *   w13_s u8[E, 2I, H/32]
 *   w2_q  u8[E, H, I/2]   down projection
 *   w2_s  u8[E, H, I/32]
 * The GPU decodes exactly for scale bytes 2..254 (every decoded value is then a normal binary32);
 * bytes 0, 1 and 255 (NaN) are outside the device contract.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

/* Status codes returned by every entry point. */
typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,       /* a size is out of range (see each call's limits) */
  MOE_ERR_UNSUPPORTED = -3, /* misaligned pointer or unsupported flag / score function */
  MOE_ERR_WORKSPACE = -4,   /* ws_bytes is smaller than the workspace-size query returns */
  MOE_ERR_LAUNCH = -5       /* the HIP runtime reported an error after launching */
} moe_status;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_fn;

/* Flags of moe_mxfp4_ffn. */
enum {
  /* Run the gate and up projections as two separate passes (the unfused structure the vllm.cpp
   * PR #52 node-trace diff measures against the fused one). The result is bitwise identical to the
   * fused pass; only the launch structure changes. */
  MOE_UNFUSED_GATE_UP = 1,
  /* Force every active expert onto the weight-streaming small-M kernels, whatever its row count. */
  MOE_FORCE_SMALL_M = 2,
  /* Force every active expert onto the MFMA kernels (row-tile, or dense from 256 rows). */
  MOE_FORCE_LARGE_M = 4
};

/* Limits checked on the host. */
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_TOPK 16
#define MOE_MAX_HIDDEN 16384
#define MOE_MAX_INTER 16384
#define MOE_MAX_PAIRS (1 << 20)

/*
 * moe_route_topk — router top-k and renormalise.
 * ("Native router select/normalize" row, Post-Portfolio Device Attribution table, "MTP1
 * Post-Portfolio Eager-Cycle Profile".)
 *
 * For each token t, ranks the E experts on logits[t, :] (largest first, the lower expert index first
 * on equal logits) and emits the k best:
 *   topk_ids[t, j]  expert of rank j (descending logit);
 *   topk_w[t, j]    score_fn = MOE_SCORE_SOFTMAX: softmax over all E logits, taken at the selected
 *                   expert; score_fn = MOE_SCORE_SIGMOID: 1/(1+exp(-logit));
 *                   renorm != 0 divides each selected score by the sum of the k selected scores.
 * Both score functions increase with the logit, so ranking on logits ranks on scores; the ids are
 * therefore exact (bit-for-bit reproducible) and the weights are fp32 with a few ulps of rounding.
 *
 *   logits    [dev] f32[T, E]
 *   topk_ids  [dev] i32[T, k]  (written)
 *   topk_w    [dev] f32[T, k]  (written)
 * Limits: T >= 0 (T == 0 enqueues nothing), 1 <= E <= MOE_MAX_EXPERTS, 1 <= k <= min(E, MOE_MAX_TOPK),
 * score_fn in {0, 1}. NaN logits are outside the contract.
 */
int moe_route_topk(const float* logits, int T, int E, int k, int score_fn, int renorm,
                   int32_t* topk_ids, float* topk_w, void* stream);

/*
 * moe_router_gemm_topk — the router's projection and its top-k in one call:
 *   logits[t, e] = sum over h of x[t, h] * w_router[e, h]   (bfloat16 operands, fp32 accumulation)
 * followed by exactly the selection and weights of moe_route_topk on those logits (the same device
 * code). The pages time only the router's select/normalize kernel ("Native router select/normalize"
 * row, Post-Portfolio Device Attribution table, "MTP1 Post-Portfolio Eager-Cycle Profile") and leave
 * the projection before it undefined; here it is a dense bfloat16 matrix.
 * The projection runs on the matrix cores with K split into up to 16 slices (chosen from T, H and E
 * only); the slices' partial logits go to the workspace and are summed in slice order, so results
 * are deterministic for given sizes. Two kernels are enqueued.
 *
 *   x_bf16         [dev] u16[T, H]  bfloat16 activations, 16-byte aligned
 *   w_router_bf16  [dev] u16[E, H]  bfloat16 router weights (one row per expert), 16-byte aligned
 *   logits         [dev] f32[T, E]  (written) or NULL
 *   topk_ids, topk_w               as moe_route_topk (written)
 *   workspace, ws_bytes            [dev] at least moe_router_gemm_topk_workspace_size(T, H, E) bytes,
 *                                  256-byte aligned; contents on entry do not matter
 * Limits: T >= 0 (T == 0 enqueues nothing), 32 <= H <= MOE_MAX_HIDDEN, H % 32 == 0,
 * 1 <= E <= MOE_MAX_EXPERTS, 1 <= k <= min(E, MOE_MAX_TOPK), T*k <= MOE_MAX_PAIRS, score_fn in {0, 1}.
 */
size_t moe_router_gemm_topk_workspace_size(int T, int H, int E);  /* host; 0 for invalid sizes */
int moe_router_gemm_topk(const uint16_t* x_bf16, const uint16_t* w_router_bf16, int T, int H, int E,
                         int k, int score_fn, int renorm, float* logits, int32_t* topk_ids,
                         float* topk_w, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_group_tokens — token-to-expert grouping (expert histogram, exclusive prefix scan and a stable
 * permutation of the pairs by expert).
 * ("Direct M=2 route remap" row, Post-Portfolio Device Attribution table, "MTP1 Post-Portfolio
 * Eager-Cycle Profile".)
 *
 *   topk_ids     [dev] i32[T, k]   every id must lie in [0, E) (precondition)
 *   counts       [dev] i32[E]      pairs routed to each expert (written)
 *   offsets      [dev] i32[E + 1]  exclusive prefix sum of counts; offsets[E] = P (written)
 *   sorted_pair  [dev] i32[P]      the pairs p ordered by (expert, p): rows offsets[e] ..
 *                                  offsets[e+1]-1 hold expert e's pairs in ascending p (written)
 *   pair_pos     [dev] i32[P]      inverse permutation: sorted_pair[pair_pos[p]] == p (written)
 *   active       [dev] i32[E]      experts with counts > 0, ascending, in entries [0, n_active);
 *                                  entries from n_active on are set to -1 (written)
 *   n_active     [dev] i32[1]      number of active experts (written)
 * Every output is an integer and is deterministic. Limits: T >= 0, 1 <= k <= MOE_MAX_TOPK,
 * 1 <= E <= MOE_MAX_EXPERTS, T*k <= MOE_MAX_PAIRS. With T == 0 the counts, offsets, active and
 * n_active outputs are still written (all zero / -1). sorted_pair and pair_pos may be NULL only when
 * T == 0.
 */
int moe_group_tokens(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                     int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, int32_t* active,
                     int32_t* n_active, void* stream);

/*
 * moe_route_group — moe_route_topk followed by moe_group_tokens, with the same arguments, limits and
 * outputs (bitwise identical: the same device code runs). For small batches (T <= 16 and
 * T*k <= 1024, the decode regime) both steps run in one single-workgroup launch that keeps the ids in
 * LDS between them (a wave per token); larger batches enqueue the two separate kernels. topk_ids and topk_w are still
 * written in full. The fusion follows the pages' accounting of launch and dispatch overhead at
 * decode (vllm.cpp PR #52 node-trace diff; "MTP1 Post-Portfolio Eager-Cycle Profile").
 */
int moe_route_group(const float* logits, int T, int E, int k, int score_fn, int renorm,
                    int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                    int32_t* sorted_pair, int32_t* pair_pos, int32_t* active, int32_t* n_active,
                    void* stream);

/*
 * moe_mxfp4_ffn_workspace_size — bytes of device workspace moe_mxfp4_ffn needs for these sizes and
 * flags: the SwiGLU activations h (two bf16 planes, 4 bytes per element of P x I), one scale byte
 * per pair row, the per-pair down-projection outputs y (fp32, P x H) and, with
 * MOE_UNFUSED_GATE_UP, the gate activations. The size covers the worst case over every routing of the P pairs, so a workspace
 * sized once for (T, H, I, E, k, flags) is valid for every call with those sizes (cf. the split-K
 * workspace contract of tokenspeed PR #661, "The workspace contract": partial rows must be reserved
 * for the worst case, not the current M). Returns 0 for invalid sizes.
 */
size_t moe_mxfp4_ffn_workspace_size(int T, int H, int I, int E, int k, int flags);

/*
 * moe_mxfp4_ffn — expert feed-forward and weighted combine for routed, grouped tokens.
 * ("Compact routed MXFP4 GEMM", "Routed MoE gather" and "Routed clamp-SwiGLU" rows of the
 * Post-Portfolio Device Attribution table, "MTP1 Post-Portfolio Eager-Cycle Profile"; gate_up
 * fusion as in vllm.cpp PR #52.)
 *
 * For every pair p = (t, j) routed to expert e (row r = pair_pos[p] of the grouping):
 *   g = x[t] . W13[e][i]ᵀ and u = x[t] . W13[e][I + i]ᵀ for i in [0, I)   (fp32 accumulation)
 *   if clamp_limit > 0: g, u clamped to [-clamp_limit, clamp_limit]
 *   h_i = g_i / (1 + exp(-g_i)) * u_i                                   (SwiGLU)
 *   y_p = h . W2[e]ᵀ                                                     (fp32 accumulation)
 * and out[t] = sum over j = 0..k-1, in that order, of topk_w[t, j] * y_(t,j), rounded once to
 * bfloat16 (nearest-even). Experts with no pairs read no weights. h is kept between the two GEMMs
 * as hi = bf16(h) and lo = bf16(h - hi) (hi + lo equals h to about 2^-17 relative). Small per-expert
 * row counts run on weight-streaming kernels (down: hi + lo rebuilt, then scaled fp16 per 32-value
 * block); larger ones on MFMA kernels: below 256 rows bf16 (down: one MFMA on each plane), from
 * 256 rows on the dense kernels (gate_up bf16; down on hi + lo rebuilt as fp16 scaled per row and
 * weights decoded to fp16 relative to each output column's largest scale, one fp16 MFMA). Results
 * are deterministic: repeated calls give bitwise-identical outputs.
 *
 *   x_bf16                       [dev] u16[T, H]  bfloat16 activations, 16-byte aligned
 *   w13_q, w13_s, w2_q, w2_s     [dev] MXFP4 weights (layout above); w13_q and w2_q 16-byte aligned
 *   topk_w                       [dev] f32[T, k]  routing weights (from moe_route_topk)
 *   counts, offsets, sorted_pair, pair_pos, active, n_active
 *                                [dev] the outputs of moe_group_tokens for the same ids
 *   clamp_limit                  <= 0 disables the clamp
 *   flags                        MOE_UNFUSED_GATE_UP | MOE_FORCE_SMALL_M | MOE_FORCE_LARGE_M
 *                                (the two FORCE flags are mutually exclusive)
 *   out_bf16                     [dev] u16[T, H]  (written), 16-byte aligned
 *   workspace, ws_bytes          [dev] at least moe_mxfp4_ffn_workspace_size(T, H, I, E, k, flags)
 *                                bytes, 256-byte aligned; its contents on entry do not matter
 * Limits: T >= 0 (T == 0 enqueues nothing), 32 <= H <= MOE_MAX_HIDDEN, 32 <= I <= MOE_MAX_INTER,
 * H % 32 == 0, I % 32 == 0, 1 <= E <= MOE_MAX_EXPERTS, 1 <= k <= min(E, MOE_MAX_TOPK),
 * T*k <= MOE_MAX_PAIRS.
 */
int moe_mxfp4_ffn(const uint16_t* x_bf16, int T, int H, int I, int E, int k, const uint8_t* w13_q,
                  const uint8_t* w13_s, const uint8_t* w2_q, const uint8_t* w2_s,
                  const float* topk_w, const int32_t* counts, const int32_t* offsets,
                  const int32_t* sorted_pair, const int32_t* pair_pos, const int32_t* active,
                  const int32_t* n_active, float clamp_limit, int flags, uint16_t* out_bf16,
                  void* workspace, size_t ws_bytes, void* stream);

/*
 * Launch plan of moe_mxfp4_ffn (host only, no GPU needed): which kernels one call enqueues, for
 * tests and for reading the launch table. Per-expert row counts live on the device, so the plan is
 * decided from host-known bounds: with T <= small_m_max every expert has at most T rows and only the
 * weight-streaming kernels run; otherwise both kernel families are launched and each expert is
 * handled by the family its row count selects (the launch table keyed by token count of tokenspeed
 * PR #661, "What the sweep found").
 */
typedef struct {
  int small_m_max;       /* experts with at most this many rows use the weight-streaming kernels */
  int launch_small;      /* 1 if the weight-streaming gate_up and down kernels are launched */
  int launch_large;      /* 1 if the MFMA gate_up and down kernels are launched */
  int small_gateup_grid; /* workgroups of the weight-streaming gate_up launch(es) */
  int small_down_grid;   /* workgroups of the weight-streaming down launch */
  int large_gateup_grid; /* workgroups of the MFMA gate_up launch */
  int large_down_grid;   /* workgroups of the MFMA down launch */
  int combine_grid;      /* workgroups of the combine launch */
  int n_launches;        /* kernels enqueued by one call */
} moe_ffn_plan;

int moe_mxfp4_ffn_plan(int T, int H, int I, int E, int k, int flags, moe_ffn_plan* plan /*[host]*/);

/*
 * Launch-table threshold (host only, process-wide): experts with at most `small_m_max` rows run on
 * the weight-streaming kernels, the rest on the MFMA kernels. By default (-1) the threshold follows
 * the token count: 8 for T <= 8 (every expert streams), 2 above. Returns the previous setting (-1
 * for the default table), or MOE_ERR_SHAPE for a value below -1. Not synchronised with calls in
 * flight on other host threads.
 */
int moe_set_small_m_max(int small_m_max);

/*
 * Column tile of the dense (M >= 256 per expert) down GEMM (host only, process-wide): 256 or 224
 * output columns per workgroup. By default (0) the library takes the width that finishes the
 * expected ceil(T*k/256) x ceil(H/width) tiles in fewer, fuller rounds over the compute units (one
 * workgroup per compute unit), the wider on a tie; a value set here forces that width (tests cover
 * both). Returns the previous setting (0 for automatic), or MOE_ERR_SHAPE for any other value. Not
 * synchronised with calls in flight on other host threads.
 */
int moe_set_dense_down_cols(int cols);

/*
 * Stage timing hook (host only), for measuring one stage of moe_mxfp4_ffn with HIP events on the
 * stream its kernels run on. While set, every moe_mxfp4_ffn call records `start` before the first
 * kernel of `stage` and `stop` after its last kernel, on the call's stream. Pass NULL events to
 * clear. The events are hipEvent_t handles created by the caller; the library does not own them.
 * Returns MOE_ERR_SHAPE for an unknown stage.
 */
enum { MOE_STAGE_GATE_UP = 0, MOE_STAGE_DOWN = 1, MOE_STAGE_COMBINE = 2, MOE_NUM_STAGES = 3 };
int moe_set_stage_events(int stage, void* start_event, void* stop_event);

/* Human-readable name of a status code (host, static storage). */
const char* moe_status_string(int status);

/* MOE_ABI_VERSION of the built library (host). */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
