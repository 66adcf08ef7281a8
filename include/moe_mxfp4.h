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
 * The GPU decodes every element exactly for scale bytes 2..252: each decoded value, at most
 * 6 * 2^(s-127), is then a normal binary32 (at 253 and 254 the largest codes overflow binary32).
 * Bytes 0, 1, 253, 254 and 255 (NaN) are outside the device contract. One kernel rounds weights on
 * purpose: the down GEMM of experts with at least 256 rows decodes each element to fp16 relative
 * to the largest scale byte c of its output row, exactly while the element's scale byte s is at
 * least c - 36; below that it is rounded to a multiple of 2^(c-164) (nearest-even), an absolute
 * error of at most 2^(c-165), below 2^-40 of the largest value the row can hold (6 * 2^(c-127)).
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

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
  MOE_FORCE_LARGE_M = 4,
  /* Run the weighted combine as a launch of its own. Without it, when only the weight-streaming
   * kernels run and there are at most 32 routed pairs (T * k) whose activations fit one
   * workgroup's LDS, the combine is folded into the down launch. The result is bitwise identical
   * either way; only the launch structure changes. */
  MOE_SEPARATE_COMBINE = 8
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
 * are deterministic for given sizes. For T <= 32 (decode) both steps run in ONE launch: the
 * workgroup that completes the last slice (found with a device-scope counter at the workspace start)
 * sums the partials and selects; above 32 tokens two kernels are enqueued. Both give the same bits.
 *
 *   x_bf16         [dev] u16[T, H]  bfloat16 activations, 16-byte aligned
 *   w_router_bf16  [dev] u16[E, H]  bfloat16 router weights (one row per expert), 16-byte aligned
 *   logits         [dev] f32[T, E]  (written) or NULL
 *   topk_ids, topk_w               as moe_route_topk (written)
 *   workspace, ws_bytes            [dev] at least moe_router_gemm_topk_workspace_size(T, H, E) bytes,
 *                                  256-byte aligned. Its first 256 bytes hold the one-launch
 *                                  router's counter: ZERO them before the first call on this
 *                                  workspace (e.g. hipMemset once after allocating it); every call
 *                                  leaves them zero. The rest may hold anything on entry. One
 *                                  workspace serves one call at a time.
 * Limits: T >= 0 (T == 0 enqueues nothing), 32 <= H <= MOE_MAX_HIDDEN, H % 32 == 0,
 * 1 <= E <= MOE_MAX_EXPERTS, 1 <= k <= min(E, MOE_MAX_TOPK), T*k <= MOE_MAX_PAIRS, score_fn in {0, 1}.
 * moe_router_gemm_topk_ex adds flags: MOE_ROUTER_SPLIT_LAUNCH enqueues the two kernels at every T
 * (the two-launch structure, bitwise the same results).
 */
enum { MOE_ROUTER_SPLIT_LAUNCH = 1 };
size_t moe_router_gemm_topk_workspace_size(int T, int H, int E);  /* host; 0 for invalid sizes */
int moe_router_gemm_topk(const uint16_t* x_bf16, const uint16_t* w_router_bf16, int T, int H, int E,
                         int k, int score_fn, int renorm, float* logits, int32_t* topk_ids,
                         float* topk_w, void* workspace, size_t ws_bytes, void* stream);
int moe_router_gemm_topk_ex(const uint16_t* x_bf16, const uint16_t* w_router_bf16, int T, int H, int E,
                            int k, int score_fn, int renorm, float* logits, int32_t* topk_ids,
                            float* topk_w, void* workspace, size_t ws_bytes, int flags, void* stream);

/*
 * moe_layer_forward — the whole layer from the activations and the router weights: the router
 * projection and top-k, the grouping, and moe_mxfp4_ffn (the routed layer of the pages' Post-Portfolio
 * Device Attribution table, "MTP1 Post-Portfolio Eager-Cycle Profile", from router to combine). For
 * T <= 32 the router, its selection and the grouping are one launch, so decode runs in four
 * (router+group, gate_up, down, combine). Results are bitwise those of moe_router_gemm_topk +
 * moe_group_tokens + moe_mxfp4_ffn.
 *   x_bf16, w_router_bf16, score_fn, renorm   as moe_router_gemm_topk
 *   w13_q .. w2_s, clamp_limit, flags, out   as moe_mxfp4_ffn (flags: the MOE_* ffn flags)
 *   logits, topk_ids, topk_w                  [dev] outputs of the router when not NULL
 *   workspace, ws_bytes                       [dev] at least moe_layer_forward_workspace_size(T, H, I, E,
 *                                             k, flags) bytes, 256-byte aligned; its first 256 bytes
 *                                             must be ZERO before the first call (the router's counter,
 *                                             left zero by every call)
 * Limits and errors: as moe_mxfp4_ffn (and score_fn in {0, 1}).
 */
size_t moe_layer_forward_workspace_size(int T, int H, int I, int E, int k, int flags);  /* host; 0 if invalid */
int moe_layer_forward(const uint16_t* x_bf16, const uint16_t* w_router_bf16, int T, int H, int I, int E,
                      int k, int score_fn, int renorm, const uint8_t* w13_q, const uint8_t* w13_s,
                      const uint8_t* w2_q, const uint8_t* w2_s, float clamp_limit, int flags, float* logits,
                      int32_t* topk_ids, float* topk_w, uint16_t* out_bf16, void* workspace,
                      size_t ws_bytes, void* stream);

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
 * T == 0. Ids need not be distinct within a token (an expert then holds several of its pairs).
 *
 * Workspace: moe_group_tokens_workspace_size(T, k, E) returns the device bytes a call needs for
 * these sizes, or (size_t)-1 for invalid sizes. The grouping runs in one workgroup up to 1024
 * pairs and over up to 64 workgroups beyond (each counts every expert over all the ids itself, so
 * they exchange nothing); histograms and scans live in LDS, so the size is 0 for every valid shape and `workspace` may be
 * NULL; a caller that passes a buffer keeps working if a later version needs one (the size is a
 * function of T, k and E only, the worst case over every routing, as tokenspeed PR #661 "The
 * workspace contract" requires). ws_bytes below the query's result returns MOE_ERR_WORKSPACE.
 */
size_t moe_group_tokens_workspace_size(int T, int k, int E);  /* host */
int moe_group_tokens(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                     int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, int32_t* active,
                     int32_t* n_active, void* workspace, size_t ws_bytes, void* stream);

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
 *                                [dev] the outputs of moe_group_tokens for the same ids (which
 *                                need not be distinct within a token); the ids themselves are not
 *                                an argument, since the grouping carries everything the kernels
 *                                read of them (rows per expert, pair of each row, row of each pair)
 *   clamp_limit                  <= 0 disables the clamp
 *   flags                        MOE_UNFUSED_GATE_UP | MOE_FORCE_SMALL_M | MOE_FORCE_LARGE_M |
 *                                MOE_SEPARATE_COMBINE
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
 * Per-call options of moe_mxfp4_ffn_ex and moe_mxfp4_ffn_plan (host struct, read during the call
 * only; the library keeps no copy and no process-wide setting, so concurrent callers never see
 * each other's choices). moe_ffn_options_init fills the defaults that moe_mxfp4_ffn uses.
 *   small_m_max       launch-table threshold: experts with at most this many rows run on the
 *                     weight-streaming kernels, the others on the MFMA kernels. -1 (default) follows
 *                     the table keyed by token count (tokenspeed PR #661, "What the sweep found"):
 *                     8 for T <= 8 (every expert streams), 2 for 8 < T < 256, 0 from 256 tokens on
 *                     (every expert on the MFMA kernels). 0 launches no weight-streaming kernel.
 *                     Values below -1 are rejected (MOE_ERR_SHAPE). The FORCE flags take precedence.
 *   dense_down_cols   column tile of the dense (>= 256 rows per expert) down GEMM: 0 (default)
 *                     picks 256 or 224 output columns per workgroup, whichever finishes the expected
 *                     ceil(T*k/256) x ceil(H/width) tiles in fewer, fuller rounds over the compute
 *                     units; 256 or 224 forces that width; anything else is MOE_ERR_SHAPE. The width
 *                     decides which workgroup computes an output column, not its arithmetic: results
 *                     are bitwise the same.
 *   stage_start/stop  hipEvent_t handles (caller-owned) or NULL: when set, the call records
 *                     stage_start[s] before the first kernel of stage s and stage_stop[s] after its
 *                     last kernel, on the call's stream (stages MOE_STAGE_*), so one stage can be
 *                     timed on the stream its kernels run on. When the combine is folded into the
 *                     down launch (moe_ffn_plan.fold_combine), the down stage holds it and the
 *                     combine stage's two events bracket no work.
 */
enum { MOE_STAGE_GATE_UP = 0, MOE_STAGE_DOWN = 1, MOE_STAGE_COMBINE = 2, MOE_NUM_STAGES = 3 };
typedef struct {
  int small_m_max;
  int dense_down_cols;
  void* stage_start[MOE_NUM_STAGES];
  void* stage_stop[MOE_NUM_STAGES];
} moe_ffn_options;

void moe_ffn_options_init(moe_ffn_options* opts /*[host]*/);

/*
 * moe_mxfp4_ffn_ex — moe_mxfp4_ffn with per-call options (NULL = the defaults of
 * moe_ffn_options_init); same arguments, limits, results and errors otherwise.
 */
int moe_mxfp4_ffn_ex(const uint16_t* x_bf16, int T, int H, int I, int E, int k, const uint8_t* w13_q,
                     const uint8_t* w13_s, const uint8_t* w2_q, const uint8_t* w2_s,
                     const float* topk_w, const int32_t* counts, const int32_t* offsets,
                     const int32_t* sorted_pair, const int32_t* pair_pos, const int32_t* active,
                     const int32_t* n_active, float clamp_limit, int flags, uint16_t* out_bf16,
                     void* workspace, size_t ws_bytes, const moe_ffn_options* opts /*[host]*/,
                     void* stream);

/*
 * Launch plan of moe_mxfp4_ffn_ex (host only, no GPU needed): which kernels one call with these
 * sizes, flags and options enqueues, for tests and for reading the launch table. Per-expert row
 * counts live on the device, so the plan is decided from host-known bounds: with T <= small_m_max
 * every expert has at most T rows and only the weight-streaming kernels run; otherwise both kernel
 * families are launched and each expert is handled by the family its row count selects.
 * opts may be NULL (defaults).
 */
typedef struct {
  int small_m_max;       /* experts with at most this many rows use the weight-streaming kernels */
  int launch_small;      /* 1 if the weight-streaming gate_up and down kernels are launched */
  int launch_large;      /* 1 if the MFMA gate_up and down kernels are launched */
  int small_gateup_grid; /* workgroups of the weight-streaming gate_up launch(es) */
  int small_down_grid;   /* workgroups of the weight-streaming down launch */
  int large_gateup_grid; /* workgroups of the MFMA gate_up launch */
  int large_down_grid;   /* workgroups of the MFMA down launch */
  int combine_grid;      /* workgroups of the combine launch (0 when folded into down) */
  int n_launches;        /* kernels enqueued by one call */
  int fold_combine;      /* 1 if the weighted combine runs inside the weight-streaming down launch
                            (small_down_grid is then that launch's grid); decided from the LDS a
                            workgroup can have on the current device (64 KB assumed when no device
                            can be queried), so a plan made without a GPU can differ here */
} moe_ffn_plan;

int moe_mxfp4_ffn_plan(int T, int H, int I, int E, int k, int flags,
                       const moe_ffn_options* opts /*[host]*/, moe_ffn_plan* plan /*[host]*/);

/*
 * moe_layer_from_logits — the whole layer from the router logits: top-k routing, grouping, expert
 * FFN and combine (the routed layer of the Post-Portfolio Device Attribution table, "MTP1
 * Post-Portfolio Eager-Cycle Profile", from the router's select/normalize step to the combine).
 * Results are bitwise those of moe_route_group + moe_mxfp4_ffn with the same flags. When
 * moe_layer_from_logits_routed(T, H, I, E, k, flags, opts) returns 1 (decode batches: only the
 * weight-streaming kernels run with the fused gate/up pass, T*k <= 64, E <= 256, the activations fit
 * the gate_up kernel's LDS staging and T is at most its waves), every gate_up workgroup routes and
 * groups the batch itself from the logits and the first one writes the routing and grouping for the
 * launches that follow: the routing launch and a memory round trip before the first weight load are
 * saved. Otherwise the routing and grouping launches run first.
 *   logits, score_fn, renorm                  as moe_route_topk (logits [dev] f32[T, E])
 *   x_bf16, w13_q .. w2_s, clamp_limit, flags, out   as moe_mxfp4_ffn
 *   topk_ids, topk_w                          [dev] outputs of the routing when not NULL
 *   workspace, ws_bytes                       [dev] at least moe_layer_from_logits_workspace_size(T, H,
 *                                             I, E, k, flags) bytes, 256-byte aligned (no contents
 *                                             required)
 *   opts                                      [host] as moe_mxfp4_ffn_ex (NULL = the defaults)
 * Limits and errors: as moe_mxfp4_ffn (and score_fn in {0, 1}).
 */
size_t moe_layer_from_logits_workspace_size(int T, int H, int I, int E, int k, int flags);  /* host; 0 if invalid */
int moe_layer_from_logits_routed(int T, int H, int I, int E, int k, int flags,
                                 const moe_ffn_options* opts /*[host]*/);  /* host: 1 if routed in gate_up */
int moe_layer_from_logits(const float* logits, const uint16_t* x_bf16, int T, int H, int I, int E, int k,
                          int score_fn, int renorm, const uint8_t* w13_q, const uint8_t* w13_s,
                          const uint8_t* w2_q, const uint8_t* w2_s, float clamp_limit, int flags,
                          int32_t* topk_ids, float* topk_w, uint16_t* out_bf16, void* workspace,
                          size_t ws_bytes, const moe_ffn_options* opts, void* stream);

/*
 * Activation-quantised expert feed-forward (W4A8 / W4A4).
 * (The FP4 activation-quantise step of the FP4 GEMM path named in "Chunk 8.0", its summary;
 * read as OCP Microscaling Formats (MX) v1.0 blocks: 32 values along the reduction axis sharing an
 * E8M0 scale, with MXFP8 E4M3 or MXFP4 E2M1 elements.)
 *
 * A block's scale byte is floor(log2 amax) - emax + 127 (emax = 8 for E4M3, 2 for E2M1; amax the
 * block's largest magnitude), clamped to [0, 254]; each element is v / 2^(byte - 127) rounded to the
 * nearest element value (ties to even), saturating at +-448 (E4M3) or +-6 (E2M1); a zero block gets
 * byte 0. A value that rounds to zero keeps its sign bit.
 */
enum { MOE_ACT_MXFP8 = 1, MOE_ACT_MXFP4 = 2 };

/*
 * moe_mx_quantize — quantise bfloat16 rows to MX blocks.
 *   x_bf16        [dev] u16[rows, cols], 16-byte aligned; cols % 32 == 0, rows * cols < 2^31
 *   act_format    MOE_ACT_MXFP8 or MOE_ACT_MXFP4
 *   codes         [dev] u8[rows, cols] (E4M3 bytes) or u8[rows, cols / 2] (two E2M1 codes per byte, the
 *                 even element in the low nibble), 16-byte aligned (written)
 *   scales        [dev] u8[rows, cols / 32] (written)
 * The codes and bytes are exact functions of x (no rounding but the element rounding defined above).
 */
int moe_mx_quantize(const uint16_t* x_bf16, int rows, int cols, int act_format, uint8_t* codes,
                    uint8_t* scales, void* stream);

size_t moe_mxfp4_ffn_mx_workspace_size(int T, int H, int I, int E, int k, int act_format);  /* 0 if invalid */

/*
 * moe_mxfp4_ffn_mx — moe_mxfp4_ffn with both GEMMs' activations quantised to MX blocks: x per 32
 * values along H before gate_up, h per 32 values along I before down (h is computed in fp32 and its
 * codes are decided from that value). The GEMMs run the gfx950 block-scaled MFMA directly on the
 * MXFP4 weights and the activation codes (fp32 accumulation); every active expert runs on 256-row
 * tiles, so this is the large-batch variant (decode batches waste most of each tile). The result is
 * that of the FFN on the quantised activations, not of moe_mxfp4_ffn: the quantisation error is part
 * of the method. Deterministic (repeated calls give bitwise-identical outputs).
 *   arguments as moe_mxfp4_ffn (no active list or flags), plus
 *   act_format                   MOE_ACT_MXFP8 (W4A8) or MOE_ACT_MXFP4 (W4A4)
 *   w13_s, w2_s                  4-byte aligned (in addition to moe_mxfp4_ffn's alignments)
 *   workspace, ws_bytes          [dev] at least moe_mxfp4_ffn_mx_workspace_size(...) bytes, 256-byte
 *                                aligned; contents on entry do not matter
 *   opts                         NULL, or per-call options of which only the stage events are used
 *                                (gate_up: the gate_up GEMM after the x quantisation; down; combine)
 * Limits: as moe_mxfp4_ffn, and H % 128 == 0, I % 128 == 0 (MOE_ERR_SHAPE otherwise); act_format
 * otherwise is MOE_ERR_UNSUPPORTED.
 */
int moe_mxfp4_ffn_mx(const uint16_t* x_bf16, int T, int H, int I, int E, int k, const uint8_t* w13_q,
                     const uint8_t* w13_s, const uint8_t* w2_q, const uint8_t* w2_s, const float* topk_w,
                     const int32_t* counts, const int32_t* offsets, const int32_t* sorted_pair,
                     const int32_t* pair_pos, float clamp_limit, int act_format, uint16_t* out_bf16,
                     void* workspace, size_t ws_bytes, const moe_ffn_options* opts, void* stream);

/*
 * moe_mxfp4_ffn_mx_h_offsets — where moe_mxfp4_ffn_mx leaves the quantised h in its workspace.
 * After a call completes (and until the workspace is reused), h's codes u8[T*k, I] (E4M3) or
 * u8[T*k, I/2] (E2M1, even element in the low nibble) start at byte *codes_offset of the workspace
 * and its scale bytes u8[T*k, I/32] at *scales_offset, rows in the grouping's sorted order (row
 * pair_pos[p] holds pair p). For inspecting the decisions the GPU took (e.g. against a reference
 * quantiser); the call itself does not need it. Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (the sizes
 * moe_mxfp4_ffn_mx rejects).
 */
int moe_mxfp4_ffn_mx_h_offsets(int T, int H, int I, int E, int k, int act_format, size_t* codes_offset,
                               size_t* scales_offset);


/*
 * moe_layer_decode — the whole layer for decode batches in ONE kernel launch: router top-k and
 * renormalisation (as moe_route_topk), grouping, gate_up + SwiGLU, down and the weighted combine
 * (as moe_mxfp4_ffn), from logits to out. The pages point at persistent kernels and at merging
 * producer/reduction/consumer launches as the lever at low concurrency ("Chunk 8.0", summary;
 * "MTP1 Post-Portfolio Eager-Cycle Profile", Decision; launch cost per kernel in vllm.cpp PR #52).
 *
 * Every workgroup routes and groups all tokens itself (ids and weights bitwise equal to
 * moe_route_topk's). The active experts' intermediate dimension is cut into 32-wide blocks shared
 * out in contiguous ranges, one per workgroup: a workgroup computes h for its blocks (fp32, in LDS)
 * and the down projection restricted to those blocks, a partial output per (range, expert, token),
 * written to the workspace. After one grid barrier the partials are summed, in a fixed order, into
 * out. The result is deterministic and within the same bar of the exact layer as moe_mxfp4_ffn, but
 * not bitwise equal to it: h is not rounded to its bf16 pair, and the down sums are split over the
 * ranges. On MI355X it is slower than moe_route_group + moe_mxfp4_ffn at every decode size measured
 * (the exchange between workgroups across the eight XCDs' L2 caches costs more than the launches
 * it saves), so the multi-launch path remains the default.
 *
 *   logits, score_fn, renorm, k      as moe_route_topk
 *   x_bf16, weights, clamp_limit     as moe_mxfp4_ffn
 *   topk_ids, topk_w                 [dev] i32[T, k], f32[T, k] (written), or NULL
 *   out_bf16                         [dev] u16[T, H] (written), 16-byte aligned
 *   workspace, ws_bytes              [dev] at least moe_layer_decode_workspace_size(T, H, I, E, k)
 *                                    bytes, 256-byte aligned. Its first 256 bytes hold the barrier's
 *                                    counter and must be ZERO before the first call on this workspace
 *                                    (e.g. hipMemset once after allocating it); every call leaves
 *                                    them in a valid state for the next. The rest is overwritten.
 *                                    One workspace serves one device and one call at a time.
 * Limits (MOE_ERR_UNSUPPORTED otherwise): 1 <= T <= 16, T*k <= 256, E <= 512, and each
 * workgroup's share at most 32 blocks of 32 (min(E, T*k) * I/32 <= 32 * compute units); sizes as
 * moe_mxfp4_ffn otherwise (MOE_ERR_SHAPE). The grid is one workgroup per compute unit and the
 * barrier needs all of them resident at once: do not run it next to work that holds compute units
 * for long. Should the barrier wait exceed about a second it gives up (results then undefined)
 * and adds one to the 32-bit word at workspace byte 8. The workspace size is
 * 256 + (T * CUs + 2 * T * k) * H * 4 bytes (CUs = compute units of the current device).
 */
size_t moe_layer_decode_workspace_size(int T, int H, int I, int E, int k);  /* host; 0 if unsupported */
int moe_layer_decode(const float* logits, const uint16_t* x_bf16, int T, int H, int I, int E, int k,
                     int score_fn, int renorm, const uint8_t* w13_q, const uint8_t* w13_s,
                     const uint8_t* w2_q, const uint8_t* w2_s, float clamp_limit, int32_t* topk_ids,
                     float* topk_w, uint16_t* out_bf16, void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_mxfp4_ffn_noalloc — moe_mxfp4_ffn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same arguments
 * without a workspace, the same kernels, limits and results (bitwise equal to moe_mxfp4_ffn). Its
 * workspace is a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES (16 MiB) that every GPU the
 * library runs on holds until the process ends; the call allocates and frees nothing. Shapes whose
 * workspace (moe_mxfp4_ffn_workspace_size) exceeds that return MOE_ERR_WORKSPACE and enqueue
 * nothing: at H = 4096, I = 2048, k = 8 that admits up to T = 85 tokens (63 with MOE_UNFUSED_GATE_UP),
 * at H = 7168 up to T = 56. Nothing in the
 * array needs to start at zero; each call overwrites what it reads. All calls on one GPU share that
 * GPU's array, so calls that can overlap on one GPU (different streams, or different host threads
 * without ordering) race: order them on one stream. moe_mxfp4_ffn_noalloc_max_bytes returns the
 * array's size (host).
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
size_t moe_mxfp4_ffn_noalloc_max_bytes(void);
int moe_mxfp4_ffn_noalloc(const uint16_t* x_bf16, int T, int H, int I, int E, int k,
                          const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                          const uint8_t* w2_s, const float* topk_w, const int32_t* counts,
                          const int32_t* offsets, const int32_t* sorted_pair, const int32_t* pair_pos,
                          const int32_t* active, const int32_t* n_active, float clamp_limit, int flags,
                          uint16_t* out_bf16, void* stream);

/* Human-readable name of a status code (host, static storage). */
const char* moe_status_string(int status);

/* MOE_ABI_VERSION of the built library (host). */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
