// Internal launchers of the gfx950 kernels (host side). Only api.hip calls them; shapes and pointers
// have been validated there.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Router GEMM (bf16 MFMA, K split into `splits` slices whose partial logits go to the workspace)
// followed by the router's select/normalize on the in-order sum of the partials.
struct RouterPlan {
  int nb;               // 16-token blocks per workgroup tile (1, 2 or 4)
  int tiles_t;          // token tiles of 16 * nb tokens
  int splits;           // K slices
  int steps_per_split;  // 32-wide K steps per slice
  int blocks;           // workgroups of the GEMM
};
RouterPlan plan_router(int T, int H, int E);
// Workspace: a 256-byte header (the one-launch router's completion counter, zero before the first
// call and left zero by every call), then the partial logits.
constexpr size_t kRouterHeaderBytes = 256;
constexpr int kRouterMaxTopk = 16;
size_t router_workspace_bytes(int T, int H, int E);
bool router_fusable(int T);  // projection and selection in one launch
// split_launch: the projection and the selection as two kernels even where one would do
hipError_t launch_router_gemm_topk(const uint16_t* x, const uint16_t* w, int T, int H, int E, int k,
                                   int score_fn, int renorm, void* workspace, float* logits, int32_t* ids,
                                   float* weights, bool split_launch, hipStream_t stream);
// Grouping outputs (moe_group_tokens's)
struct RouterGroupOut {
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pair;
  int32_t* pair_pos;
  int32_t* active;
  int32_t* n_active;
};
// The router and the grouping of its ids: one launch for T <= 32, else the two router kernels and
// the grouping kernel.
hipError_t launch_router_group(const uint16_t* x, const uint16_t* w, int T, int H, int E, int k, int score_fn,
                               int renorm, void* workspace, float* logits, int32_t* ids, float* weights,
                               const RouterGroupOut& grp, hipStream_t stream);

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int score_fn, int renorm,
                             int32_t* ids, float* weights, hipStream_t stream);

hipError_t launch_group_tokens(const int32_t* ids, int P, int E, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_pair, int32_t* pair_pos, int32_t* active,
                               int32_t* n_active, hipStream_t stream);

// Router and grouping in one single-workgroup launch (small batches: route_group_fusable).
bool route_group_fusable(int T, int k);
hipError_t launch_route_group(const float* logits, int T, int E, int k, int score_fn, int renorm,
                              int32_t* ids, float* weights, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_pair, int32_t* pair_pos, int32_t* active,
                              int32_t* n_active, hipStream_t stream);

// Grouping results and activations every FFN kernel reads.
// Outputs of the routed gate_up variant (written by its first workgroup): the router's ids and
// weights [P] and the grouping (counts [E], offsets [E + 1], sorted_pair [P], pair_pos [P], active [E],
// n_active [1]), from router logits f32 [T, E].
struct RouteOut {
  const float* logits;
  int E, score_fn, renorm;
  int32_t* ids;
  float* weights;
  int32_t *counts, *offsets, *sorted_pair, *pair_pos, *active, *n_active;
};
constexpr int kRoutePairs = 64;     // the routed variant groups at most 64 pairs (one wave)
constexpr int kRouteExperts = 256;  // and at most 256 experts (4 logits per lane)

struct Routed {
  const uint16_t* x;         // bf16 [T, H]
  const int32_t* counts;     // [E]
  const int32_t* offsets;    // [E + 1]
  const int32_t* sorted_pair;// [P]
  const int32_t* active;     // [E]
  const int32_t* n_active;   // [1]
  int k;
};

// How one K-long weight row is spread over a wave: `lpr` lanes share a row (a power of two dividing
// 64), each lane owning the 32-element blocks q, q + lpr, q + 2*lpr, ... (`bpl` of them at most).
struct RowSplit {
  int nb;   // 32-element blocks per row (K / 32)
  int lpr;  // lanes per row
  int bpl;  // blocks per lane, ceil(nb / lpr), at most 8
};

RowSplit choose_row_split(int K);

// h travels between the gate_up and down kernels as two bf16 planes [P, I] (rows in sorted order):
// hi = bf16(h), lo = bf16(h - hi); the MFMA down kernels use them directly as operands.
// Weight-streaming kernels for experts with at most `small_m_max` rows. They work through the
// experts of `list` (the first *list_count entries; the active list, or the schedule's small list).
enum SmallGateUpMode { kGateUpFused = 0, kGateOnly = 1, kUpWithGate = 2 };

struct SmallPlan {
  RowSplit gu, dn;
  int gu_tile, dn_tile;    // rows per item, one wave's share (gate rows for gate_up, output rows for down)
  int gu_tiles, dn_tiles;  // items per expert
  int gu_grid, dn_grid;    // persistent workgroups (one per CU)
  int fold_grid;           // workgroups of down with the combine folded in (whole output-row tiles each)
  int gu_block, dn_block;  // threads per workgroup
  int slots;               // bound on the number of experts in the list (min(E, P))
  int T, P;                // tokens, routed pairs
  int E;                   // experts (entries of the work list)
  int mt_gu, mt_dn;        // tokens per pass
  int weighted;            // workgroup ranges weighted by the experts' row counts
};

SmallPlan plan_small(int T, int H, int I, int E, int k, int num_cus);

hipError_t launch_small_gateup(const SmallPlan& sp, const Routed& r, const int32_t* list,
                               const int32_t* list_count, int H, int I, const uint8_t* w13_q,
                               const uint8_t* w13_s, float clamp, int mode, uint16_t* h_hi,
                               uint16_t* h_lo, float* g_ws,
                               hipStream_t stream);

hipError_t launch_small_down(const SmallPlan& sp, const Routed& r, const int32_t* list,
                             const int32_t* list_count, bool list_is_active, int H, int I, const uint8_t* w2_q,
                             const uint8_t* w2_s, const uint16_t* h_hi, const uint16_t* h_lo, float* y,
                             hipStream_t stream);

// gate_up with the routing and grouping done by every workgroup (see RouteOut): for decode batches
// whose activations fit the LDS staging, T <= the workgroup's waves, T*k <= kRoutePairs and
// E <= kRouteExperts, the fused gate/up pass only (gateup_routed_ok says whether a plan qualifies).
bool gateup_routed_ok(const SmallPlan& sp, int H, int E);
hipError_t launch_small_gateup_routed(const SmallPlan& sp, const Routed& r, const RouteOut& ro, int H, int I,
                                      const uint8_t* w13_q, const uint8_t* w13_s, float clamp,
                                      uint16_t* h_hi, uint16_t* h_lo, hipStream_t stream);

// Down with the weighted combine folded in (one launch instead of two; results identical to
// launch_small_down followed by launch_combine, bit for bit). Only for lists holding every active
// expert, at most kCombinePairsMax routed pairs, and when down_combine_fits.
constexpr int kCombinePairsMax = 32;
bool down_combine_fits(const SmallPlan& sp, int H, int I);
hipError_t launch_small_down_combine(const SmallPlan& sp, const Routed& r, const int32_t* list,
                                     const int32_t* list_count, const int32_t* pair_pos,
                                     const float* topk_w, int H, int I, const uint8_t* w2_q,
                                     const uint8_t* w2_s, const uint16_t* h_hi, const uint16_t* h_lo,
                                     uint16_t* out, hipStream_t stream);

// bf16-MFMA kernels for experts with more than `small_m_max` rows: tiles of up to 64 rows of one
// expert; the weight rows are decoded from MXFP4 to bf16 in registers, the activation tile is staged
// in LDS (x for gate_up; h as a bf16 hi/lo pair for down). h is fp32 [P, I] on both kernel families.
struct LargePlan {
  int tile_m;        // rows per tile
  int gu_tile_n;     // gate columns per gate_up workgroup (the matching up columns come with them)
  int dn_tile_n;     // output columns per down workgroup
  int gu_grid_x, dn_grid_x;  // column blocks per row tile
  int tile_slots;    // upper bound on the number of (expert, row-tile) pairs
  int gu_blocks, dn_blocks;  // one-dimensional grids (XCD-interleaved tile order)
};

int tile_slots_bound(int T, int E, int k, int small_m_max);
LargePlan plan_large(int T, int H, int I, int E, int k, int small_m_max);

// Splits the active experts by row count: small_list/n_small for the weight-streaming kernels,
// tile_e/tile_m0 (tile_slots entries, -1 past the last tile) for the row-tile MFMA kernels and
// dense_e/dense_m0 (dense_slots entries) for the dense kernels (experts with >= dense_m_min rows).
hipError_t launch_schedule(const Routed& r, int E, int small_m_max, int tile_slots, int dense_m_min,
                           int dense_slots, int32_t* small_list, int32_t* n_small, int32_t* tile_e,
                           int32_t* tile_m0, int32_t* dense_e, int32_t* dense_m0, hipStream_t stream);

hipError_t launch_large_gateup(const LargePlan& lp, const Routed& r, int H, int I,
                               const uint8_t* w13_q, const uint8_t* w13_s, const int32_t* tile_e,
                               const int32_t* tile_m0, float clamp, uint16_t* h_hi, uint16_t* h_lo,
                               hipStream_t stream);

hipError_t launch_large_down(const LargePlan& lp, const Routed& r, int H, int I, const uint8_t* w2_q,
                             const uint8_t* w2_s, const int32_t* tile_e, const int32_t* tile_m0,
                             const uint16_t* h_hi, const uint16_t* h_lo, float* y, hipStream_t stream);

// Dense MFMA kernels for experts with at least kDenseMinRows rows: 256-row tiles, both operands
// staged in LDS, weights decoded once per workgroup. Between the GEMMs, launch_dense_h16 rewrites
// the hi plane of those rows as row-scaled fp16 (scale 2^(f - 127), f in rowf[row]), which the
// down GEMM reads.
constexpr int kDenseMinRows = 256;

struct DensePlan {
  int tile_m;                // rows per tile
  int gu_grid_x, dn_grid_x;  // column tiles per row tile
  int dn_ncb;                // down: 16-column MFMA blocks per wave (8: 256-column tiles, 7: 224)
  int slots;                 // upper bound on the number of (expert, row-tile) pairs
  int gu_blocks, dn_blocks;  // one-dimensional grids (XCD-interleaved tile order)
};

int dense_slots_bound(int T, int E, int k, int dense_m_min);
// force_ncb: 7 or 8 forces the down column tile; 0 picks it from the shape
DensePlan plan_dense(int T, int H, int I, int E, int k, int dense_m_min, int num_cus, int force_ncb = 0);

hipError_t launch_dense_gateup(const DensePlan& dp, const Routed& r, int H, int I, const uint8_t* w13_q,
                               const uint8_t* w13_s, const int32_t* dense_e, const int32_t* dense_m0,
                               float clamp, uint16_t* h_hi, uint16_t* h_lo, hipStream_t stream);

hipError_t launch_dense_h16(const DensePlan& dp, const Routed& r, int I, const int32_t* dense_e,
                            const int32_t* dense_m0, uint16_t* h_hi, const uint16_t* h_lo, uint8_t* rowf,
                            hipStream_t stream);

hipError_t launch_dense_down(const DensePlan& dp, const Routed& r, int H, int I, const uint8_t* w2_q,
                             const uint8_t* w2_s, const int32_t* dense_e, const int32_t* dense_m0,
                             const uint16_t* h16, const uint8_t* rowf, float* y, hipStream_t stream);

// The whole layer for decode in one launch (route, group, gate_up, down, combine); see layer_decode.hip.
constexpr int kLayerMaxTokens = 16;
constexpr int kLayerMaxPairs = 256;
constexpr int kLayerMaxExperts = 512;
constexpr int kLayerMaxRanges = 1024;           // workgroups (one per compute unit)
constexpr size_t kLayerSyncBytes = 256;         // barrier counter and status word at the workspace start
constexpr size_t kLayerMaxHLds = 92 * 1024;     // LDS for one workgroup's h (static LDS ~65 KB: 160 KB in all)
bool layer_supported(int T, int H, int I, int E, int k, int num_cus);
size_t layer_workspace_bytes(int T, int H, int I, int E, int k, int num_cus);
size_t layer_h_lds_bytes(int T, int I, int E, int k, int num_cus);
hipError_t launch_layer_decode(const float* logits, const uint16_t* x, int T, int H, int I, int E, int k,
                               int score_fn, int renorm, const uint8_t* w13_q, const uint8_t* w13_s,
                               const uint8_t* w2_q, const uint8_t* w2_s, float clamp, int32_t* ids_out,
                               float* w_out, uint16_t* out, void* workspace, int num_cus, hipStream_t stream);

// Activation-quantised GEMMs (W4A8 / W4A4; see ffn_mx.hip): x and h as MX blocks, block-scaled MFMA on
// the packed weights, 256-row tiles of every active expert.
constexpr int kActFp8 = 1;  // MXFP8 (E4M3) activations
constexpr int kActFp4 = 2;  // MXFP4 (E2M1) activations
constexpr int kMxTileM = 256;
constexpr int kMxTileN = 256;
struct MxPlan {
  int slots;                 // bound on the number of (expert, 256-row tile) pairs
  int gu_grid_x, dn_grid_x;  // column tiles: 128 h columns (gate_up), 256 output columns (down)
  int gu_blocks, dn_blocks;  // one-dimensional grids (XCD-interleaved tile order)
};
int mx_slots_bound(int T, int E, int k);
MxPlan plan_mx(int T, int H, int I, int E, int k);
hipError_t launch_mx_schedule(const int32_t* counts, int E, const MxPlan& mp, int32_t* tile_e, int32_t* tile_m0,
                              hipStream_t stream);
// rows x cols bf16 (cols % 32 == 0) -> codes [rows, cols] (E4M3) or [rows, cols/2] (E2M1) and scale
// bytes [rows, cols/32]
hipError_t launch_mx_quant_x(const uint16_t* x, int rows, int cols, int act, uint8_t* xq, uint8_t* xs,
                             hipStream_t stream);
hipError_t launch_mx_gateup(const MxPlan& mp, int act, const uint8_t* xq, const uint8_t* xs, const int32_t* counts,
                            const int32_t* offsets, const int32_t* sorted_pair, int k, int H, int I,
                            const int32_t* tile_e, const int32_t* tile_m0, const uint8_t* w13_q,
                            const uint8_t* w13_s, float clamp, uint8_t* hq, uint8_t* hs, hipStream_t stream);
hipError_t launch_mx_down(const MxPlan& mp, int act, const uint8_t* hq, const uint8_t* hs, const int32_t* counts,
                          const int32_t* offsets, int k, int H, int I, const int32_t* tile_e,
                          const int32_t* tile_m0, const uint8_t* w2_q, const uint8_t* w2_s, float* y,
                          hipStream_t stream);

// out[t] = bf16(sum_j topk_w[t, j] * y[pair_pos[t*k + j]])
hipError_t launch_combine(const float* y, const float* topk_w, const int32_t* pair_pos, int T, int H,
                          int k, uint16_t* out, int* grid_out, hipStream_t stream);
int combine_grid(int T, int H);

}  // namespace moe
