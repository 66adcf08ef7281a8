// C ABI of the routed MXFP4 MoE layer: host-side validation, workspace layout, launch plan and
// stream-ordered launches. Nothing here allocates, synchronises or reads device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>

#include "kernels.hpp"
#include "moe_mxfp4.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace {

// Launch table keyed by token count (tokenspeed PR #661, "What the sweep found"): experts with at
// most small_m_max rows run on the weight-streaming kernels, the others on the MFMA kernels. With
// T <= 8 every expert stays on the streaming kernels (no schedule or MFMA launches at decode); above
// that, experts with more than 2 rows go to the MFMA kernels (the streaming kernels hold two
// tokens' activations in registers, and each further pair of tokens costs another decode pass and a
// reload). A value set through moe_set_small_m_max overrides the table; -1 restores it.
std::atomic<int> g_small_m_max{-1};
std::atomic<int> g_dense_down_cols{0};  // 0: chosen per shape; 256 or 224: forced

int table_small_m_max(int T) { return T <= 8 ? 8 : 2; }

std::atomic<void*> g_stage_start[MOE_NUM_STAGES];
std::atomic<void*> g_stage_stop[MOE_NUM_STAGES];

constexpr size_t kAlign = 256;

// Compute units of the current device (the persistent grids are sized from it); 256 (MI355X) if it
// cannot be queried, e.g. on a host without a GPU.
int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  return n;
}
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct WsLayout {
  size_t h, rowf, g_f32, y, sched, total;
  int tile_slots_max, dense_slots_max;
};

// Every region is sized for the worst case over routings and launch-table thresholds, so one
// workspace serves every call with the same sizes and flags.
WsLayout ws_layout(long P, int H, int I, int E, int k, int flags) {
  WsLayout w;
  size_t off = 0;
  w.tile_slots_max = moe::tile_slots_bound((int)(P / k), E, k, 0);
  w.dense_slots_max = moe::dense_slots_bound((int)(P / k), E, k, moe::kDenseMinRows);
  // small_list[E], n_small[1], tile_e[slots], tile_m0[slots], dense_e[dslots], dense_m0[dslots]
  w.sched = off;
  off = align_up(off + sizeof(int32_t) * ((size_t)E + 1 + 2 * (size_t)w.tile_slots_max +
                                          2 * (size_t)w.dense_slots_max));
  // h as two bf16 planes [P, I] (hi, then lo)
  w.h = off;
  off = align_up(off + (size_t)P * I * 2 * sizeof(uint16_t));
  // per h row of a dense expert, the exponent of its fp16 scale (one byte)
  w.rowf = off;
  off = align_up(off + (size_t)P);
  w.g_f32 = off;
  if (flags & MOE_UNFUSED_GATE_UP) off = align_up(off + (size_t)P * I * sizeof(float));
  w.y = off;
  off = align_up(off + (size_t)P * H * sizeof(float));
  w.total = off;
  return w;
}

bool ffn_sizes_ok(int T, int H, int I, int E, int k) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E) return false;
  if (H < 32 || H > MOE_MAX_HIDDEN || H % 32) return false;
  if (I < 32 || I > MOE_MAX_INTER || I % 32) return false;
  if ((long)T * k > MOE_MAX_PAIRS) return false;
  return true;
}

constexpr int kKnownFlags = MOE_UNFUSED_GATE_UP | MOE_FORCE_SMALL_M | MOE_FORCE_LARGE_M;

int effective_small_m_max(int T, int flags) {
  if (flags & MOE_FORCE_SMALL_M) return INT_MAX;
  if (flags & MOE_FORCE_LARGE_M) return 0;
  const int v = g_small_m_max.load();
  return v >= 0 ? v : table_small_m_max(T);
}

void fill_plan(int T, int H, int I, int E, int k, int flags, moe_ffn_plan* plan) {
  const int thr = effective_small_m_max(T, flags);
  const moe::SmallPlan sp = moe::plan_small(T, H, I, E, k, num_cus());
  const moe::LargePlan lp = moe::plan_large(T, H, I, E, k, thr == INT_MAX ? INT_MAX - 1 : thr);
  plan->small_m_max = thr;
  plan->launch_small = (flags & MOE_FORCE_LARGE_M) ? 0 : 1;
  plan->launch_large = (flags & MOE_FORCE_LARGE_M) ? 1 : ((flags & MOE_FORCE_SMALL_M) ? 0 : (T > thr));
  if (T == 0) plan->launch_small = plan->launch_large = 0;
  const int gu_launches = (flags & MOE_UNFUSED_GATE_UP) ? 2 : 1;
  plan->small_gateup_grid = plan->launch_small ? sp.gu_grid : 0;
  plan->small_down_grid = plan->launch_small ? sp.dn_grid : 0;
  plan->large_gateup_grid = plan->launch_large ? lp.gu_blocks : 0;
  plan->large_down_grid = plan->launch_large ? lp.dn_blocks : 0;
  plan->combine_grid = T > 0 ? moe::combine_grid(T, H) : 0;
  // the MFMA kernels need the schedule kernel's tile lists first; the dense kernels (gate_up, the
  // fp16 rewrite of their h rows, down) run only when an expert can have kDenseMinRows rows (an
  // expert has at most T)
  const bool dense = plan->launch_large && T >= moe::kDenseMinRows;
  plan->n_launches = (plan->launch_small ? gu_launches + 1 : 0) + (plan->launch_large ? 3 : 0) +
                     (dense ? 3 : 0) + (T > 0 ? 1 : 0);
}

void record(int stage, bool start, hipStream_t stream) {
  void* ev = start ? g_stage_start[stage].load() : g_stage_stop[stage].load();
  if (ev) (void)hipEventRecord((hipEvent_t)ev, stream);
}

}  // namespace

MOE_API int moe_abi_version(void) { return MOE_ABI_VERSION; }

MOE_API const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: a size is out of range";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: misaligned pointer or unsupported option";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH: the HIP runtime reported a launch error";
    default: return "unknown moe_status";
  }
}

MOE_API int moe_set_small_m_max(int v) {
  if (v < -1) return MOE_ERR_SHAPE;
  return g_small_m_max.exchange(v);
}

MOE_API int moe_set_dense_down_cols(int cols) {
  if (cols != 0 && cols != 256 && cols != 224) return MOE_ERR_SHAPE;
  return g_dense_down_cols.exchange(cols);
}

MOE_API int moe_set_stage_events(int stage, void* start_event, void* stop_event) {
  if (stage < 0 || stage >= MOE_NUM_STAGES) return MOE_ERR_SHAPE;
  g_stage_start[stage].store(start_event);
  g_stage_stop[stage].store(stop_event);
  return MOE_OK;
}

MOE_API int moe_route_topk(const float* logits, int T, int E, int k, int score_fn, int renorm,
                           int32_t* topk_ids, float* topk_w, void* stream) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E ||
      (long)T * k > MOE_MAX_PAIRS)
    return MOE_ERR_SHAPE;
  if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_NULL;
  if (moe::launch_route_topk(logits, T, E, k, score_fn, renorm, topk_ids, topk_w,
                             (hipStream_t)stream) != hipSuccess)
    return MOE_ERR_LAUNCH;
  return MOE_OK;
}

MOE_API size_t moe_router_gemm_topk_workspace_size(int T, int H, int E) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || H < 32 || H > MOE_MAX_HIDDEN || H % 32) return 0;
  const size_t b = moe::router_workspace_bytes(T, H, E);
  return b > 0 ? b : 256;
}

MOE_API int moe_router_gemm_topk(const uint16_t* x_bf16, const uint16_t* w_router_bf16, int T, int H, int E,
                                 int k, int score_fn, int renorm, float* logits, int32_t* topk_ids,
                                 float* topk_w, void* workspace, size_t ws_bytes, void* stream) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E ||
      (long)T * k > MOE_MAX_PAIRS || H < 32 || H > MOE_MAX_HIDDEN || H % 32)
    return MOE_ERR_SHAPE;
  if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !w_router_bf16 || !topk_ids || !topk_w || !workspace) return MOE_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(w_router_bf16, 16) || !aligned(workspace, 256))
    return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < moe_router_gemm_topk_workspace_size(T, H, E)) return MOE_ERR_WORKSPACE;
  if (moe::launch_router_gemm_topk(x_bf16, w_router_bf16, T, H, E, k, score_fn, renorm, (float*)workspace,
                                   logits, topk_ids, topk_w, (hipStream_t)stream) != hipSuccess)
    return MOE_ERR_LAUNCH;
  return MOE_OK;
}

MOE_API int moe_group_tokens(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                             int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                             int32_t* active, int32_t* n_active, void* stream) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK ||
      (long)T * k > MOE_MAX_PAIRS)
    return MOE_ERR_SHAPE;
  if (!counts || !offsets || !active || !n_active) return MOE_ERR_NULL;
  if (T > 0 && (!topk_ids || !sorted_pair || !pair_pos)) return MOE_ERR_NULL;
  if (moe::launch_group_tokens(topk_ids, T * k, E, counts, offsets, sorted_pair, pair_pos, active,
                               n_active, (hipStream_t)stream) != hipSuccess)
    return MOE_ERR_LAUNCH;
  return MOE_OK;
}

MOE_API int moe_route_group(const float* logits, int T, int E, int k, int score_fn, int renorm,
                            int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                            int32_t* sorted_pair, int32_t* pair_pos, int32_t* active,
                            int32_t* n_active, void* stream) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E ||
      (long)T * k > MOE_MAX_PAIRS)
    return MOE_ERR_SHAPE;
  if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets || !active || !n_active) return MOE_ERR_NULL;
  if (T > 0 && (!logits || !topk_ids || !topk_w || !sorted_pair || !pair_pos)) return MOE_ERR_NULL;
  hipStream_t s = (hipStream_t)stream;
  if (T > 0 && moe::route_group_fusable(T, k))
    return moe::launch_route_group(logits, T, E, k, score_fn, renorm, topk_ids, topk_w, counts, offsets,
                                   sorted_pair, pair_pos, active, n_active, s) == hipSuccess
               ? MOE_OK
               : MOE_ERR_LAUNCH;
  if (T > 0 && moe::launch_route_topk(logits, T, E, k, score_fn, renorm, topk_ids, topk_w, s) != hipSuccess)
    return MOE_ERR_LAUNCH;
  if (moe::launch_group_tokens(topk_ids, T * k, E, counts, offsets, sorted_pair, pair_pos, active,
                               n_active, s) != hipSuccess)
    return MOE_ERR_LAUNCH;
  return MOE_OK;
}

MOE_API size_t moe_mxfp4_ffn_workspace_size(int T, int H, int I, int E, int k, int flags) {
  if (!ffn_sizes_ok(T, H, I, E, k) || (flags & ~kKnownFlags)) return 0;
  return ws_layout((long)T * k, H, I, E, k, flags).total;
}

MOE_API int moe_mxfp4_ffn_plan(int T, int H, int I, int E, int k, int flags, moe_ffn_plan* plan) {
  if (!plan) return MOE_ERR_NULL;
  if (!ffn_sizes_ok(T, H, I, E, k)) return MOE_ERR_SHAPE;
  if ((flags & ~kKnownFlags) || ((flags & MOE_FORCE_SMALL_M) && (flags & MOE_FORCE_LARGE_M)))
    return MOE_ERR_UNSUPPORTED;
  fill_plan(T, H, I, E, k, flags, plan);
  return MOE_OK;
}

MOE_API int moe_mxfp4_ffn(const uint16_t* x_bf16, int T, int H, int I, int E, int k,
                          const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                          const uint8_t* w2_s, const float* topk_w, const int32_t* counts,
                          const int32_t* offsets, const int32_t* sorted_pair,
                          const int32_t* pair_pos, const int32_t* active, const int32_t* n_active,
                          float clamp_limit, int flags, uint16_t* out_bf16, void* workspace,
                          size_t ws_bytes, void* stream) {
  if (!ffn_sizes_ok(T, H, I, E, k)) return MOE_ERR_SHAPE;
  if ((flags & ~kKnownFlags) || ((flags & MOE_FORCE_SMALL_M) && (flags & MOE_FORCE_LARGE_M)))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !w13_q || !w13_s || !w2_q || !w2_s || !topk_w || !counts || !offsets ||
      !sorted_pair || !pair_pos || !active || !n_active || !out_bf16 || !workspace)
    return MOE_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(out_bf16, 16) || !aligned(w13_q, 16) || !aligned(w2_q, 16) ||
      !aligned(workspace, kAlign))
    return MOE_ERR_UNSUPPORTED;
  const long P = (long)T * k;
  const WsLayout wl = ws_layout(P, H, I, E, k, flags);
  if (ws_bytes < wl.total) return MOE_ERR_WORKSPACE;

  moe_ffn_plan plan;
  fill_plan(T, H, I, E, k, flags, &plan);
  const int thr = plan.small_m_max;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  uint16_t* h_hi = (uint16_t*)(ws + wl.h);
  uint16_t* h_lo = h_hi + (size_t)T * k * I;
  uint8_t* rowf = (uint8_t*)(ws + wl.rowf);
  float* g_f32 = (float*)(ws + wl.g_f32);
  float* y = (float*)(ws + wl.y);

  const moe::Routed r{x_bf16, counts, offsets, sorted_pair, active, n_active, k};
  const moe::SmallPlan sp = moe::plan_small(T, H, I, E, k, num_cus());
  const moe::LargePlan lp = moe::plan_large(T, H, I, E, k, thr == INT_MAX ? INT_MAX - 1 : thr);
  int32_t* small_list = (int32_t*)(ws + wl.sched);
  int32_t* n_small = small_list + E;
  int32_t* tile_e = n_small + 1;
  int32_t* tile_m0 = tile_e + wl.tile_slots_max;
  int32_t* dense_e = tile_m0 + wl.tile_slots_max;
  int32_t* dense_m0 = dense_e + wl.dense_slots_max;
  const bool dense = plan.launch_large && T >= moe::kDenseMinRows;
  const int dense_min = dense ? moe::kDenseMinRows : INT_MAX;
  const moe::DensePlan dp = moe::plan_dense(T, H, I, E, k, moe::kDenseMinRows, num_cus(), g_dense_down_cols.load() / 32);
  // without MFMA kernels every active expert is small: the grouping's active list is the work list
  const int32_t* list = plan.launch_large ? small_list : active;
  const int32_t* list_count = plan.launch_large ? n_small : n_active;
  bool ok = true;

  if (plan.launch_large)
    ok &= moe::launch_schedule(r, E, thr, wl.tile_slots_max, dense_min, dp.slots, small_list, n_small,
                               tile_e, tile_m0, dense_e, dense_m0, s) == hipSuccess;

  record(MOE_STAGE_GATE_UP, true, s);
  if (plan.launch_small) {
    if (flags & MOE_UNFUSED_GATE_UP) {
      ok &= moe::launch_small_gateup(sp, r, list, list_count, H, I, w13_q, w13_s, clamp_limit,
                                     moe::kGateOnly, h_hi, h_lo, g_f32, s) == hipSuccess;
      ok &= moe::launch_small_gateup(sp, r, list, list_count, H, I, w13_q, w13_s, clamp_limit,
                                     moe::kUpWithGate, h_hi, h_lo, g_f32, s) == hipSuccess;
    } else {
      ok &= moe::launch_small_gateup(sp, r, list, list_count, H, I, w13_q, w13_s, clamp_limit,
                                     moe::kGateUpFused, h_hi, h_lo, g_f32, s) == hipSuccess;
    }
  }
  if (plan.launch_large)
    ok &= moe::launch_large_gateup(lp, r, H, I, w13_q, w13_s, tile_e, tile_m0, clamp_limit, h_hi, h_lo, s) ==
          hipSuccess;
  if (dense)
    ok &= moe::launch_dense_gateup(dp, r, H, I, w13_q, w13_s, dense_e, dense_m0, clamp_limit, h_hi, h_lo, s) ==
          hipSuccess;
  record(MOE_STAGE_GATE_UP, false, s);

  record(MOE_STAGE_DOWN, true, s);
  if (dense)
    ok &= moe::launch_dense_h16(dp, r, I, dense_e, dense_m0, h_hi, h_lo, rowf, s) == hipSuccess;
  if (plan.launch_small)
    ok &= moe::launch_small_down(sp, r, list, list_count, !plan.launch_large, H, I, w2_q, w2_s, h_hi, h_lo, y,
                                 s) == hipSuccess;
  if (plan.launch_large)
    ok &= moe::launch_large_down(lp, r, H, I, w2_q, w2_s, tile_e, tile_m0, h_hi, h_lo, y, s) == hipSuccess;
  if (dense)
    ok &= moe::launch_dense_down(dp, r, H, I, w2_q, w2_s, dense_e, dense_m0, h_hi, rowf, y, s) == hipSuccess;
  record(MOE_STAGE_DOWN, false, s);

  record(MOE_STAGE_COMBINE, true, s);
  ok &= moe::launch_combine(y, topk_w, pair_pos, T, H, k, out_bf16, nullptr, s) == hipSuccess;
  record(MOE_STAGE_COMBINE, false, s);
  return ok ? MOE_OK : MOE_ERR_LAUNCH;
}
