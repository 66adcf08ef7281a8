// C ABI of the routed MXFP4 MoE layer: host-side validation, workspace layout, launch plan and
// stream-ordered launches. Nothing here allocates, synchronises or reads device memory.
#include <hip/hip_runtime.h>

#include <climits>
#include <mutex>

#include "kernels.hpp"
#include "moe_mxfp4.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

// Workspace of moe_mxfp4_ffn_noalloc: a file-scope device array, one copy on every GPU the library
// runs on, held until the process ends. On the host this name is only a stand-in for the symbol, not
// a device address: host code reaches the array through the per-device address that
// hipGetSymbolAddress returns (scratch_address below) and never passes `scratch` itself anywhere.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

// Launch table keyed by token count (tokenspeed PR #661, "What the sweep found"): experts with at
// most small_m_max rows run on the weight-streaming kernels, the others on the MFMA kernels. With
// T <= 8 every expert stays on the streaming kernels (no schedule or MFMA launches at decode); above
// that, experts with more than 2 rows go to the MFMA kernels (the streaming kernels hold two
// tokens' activations in registers, and each further pair of tokens costs another decode pass and a
// reload). A call's options may override the threshold.
// Launch table keyed by the token count (a launch structure chosen by M, as in tokenspeed PR #661,
// "What the sweep found"): up to 8 tokens every expert has at most 8 rows and streams; in between,
// experts of one or two rows stream and the rest run on the MFMA kernels; from 256 tokens on every
// active expert runs on the MFMA kernels and the weight-streaming launches are skipped (MI355X, same
// box, two alternations: medium_zipf, T = 256, 777-778 us per layer against 797-824 with experts of
// up to two rows streaming; high_c4, T = 1024, 1692-1702 against 1700-1719).
constexpr int kTableAllMfmaTokens = 256;
int table_small_m_max(int T) { return T <= 8 ? 8 : T < kTableAllMfmaTokens ? 2 : 0; }

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

constexpr int kKnownFlags = MOE_UNFUSED_GATE_UP | MOE_FORCE_SMALL_M | MOE_FORCE_LARGE_M | MOE_SEPARATE_COMBINE;

int effective_small_m_max(int T, int flags, const moe_ffn_options& o) {
  if (flags & MOE_FORCE_SMALL_M) return INT_MAX;
  if (flags & MOE_FORCE_LARGE_M) return 0;
  return o.small_m_max >= 0 ? o.small_m_max : table_small_m_max(T);
}

// The caller's options (validated), or the defaults.
int read_options(const moe_ffn_options* in, moe_ffn_options& o) {
  moe_ffn_options_init(&o);
  if (!in) return MOE_OK;
  if (in->small_m_max < -1) return MOE_ERR_SHAPE;
  if (in->dense_down_cols != 0 && in->dense_down_cols != 256 && in->dense_down_cols != 224)
    return MOE_ERR_SHAPE;
  o = *in;
  return MOE_OK;
}

void fill_plan(int T, int H, int I, int E, int k, int flags, const moe_ffn_options& o, moe_ffn_plan* plan) {
  const int thr = effective_small_m_max(T, flags, o);
  const moe::SmallPlan sp = moe::plan_small(T, H, I, E, k, num_cus());
  const moe::LargePlan lp = moe::plan_large(T, H, I, E, k, thr == INT_MAX ? INT_MAX - 1 : thr);
  plan->small_m_max = thr;
  // a threshold of 0 leaves no active expert (every one has a row) to the weight-streaming kernels
  plan->launch_small = thr > 0 ? 1 : 0;
  plan->launch_large = (flags & MOE_FORCE_LARGE_M) ? 1 : ((flags & MOE_FORCE_SMALL_M) ? 0 : (T > thr));
  if (T == 0) plan->launch_small = plan->launch_large = 0;
  const int gu_launches = (flags & MOE_UNFUSED_GATE_UP) ? 2 : 1;
  // the combine folds into the streaming down launch when that launch sees every pair
  const bool fold = plan->launch_small && !plan->launch_large && !(flags & MOE_SEPARATE_COMBINE) &&
                    moe::down_combine_fits(sp, H, I);
  plan->fold_combine = fold ? 1 : 0;
  plan->small_gateup_grid = plan->launch_small ? sp.gu_grid : 0;
  plan->small_down_grid = plan->launch_small ? (fold ? sp.fold_grid : sp.dn_grid) : 0;
  plan->large_gateup_grid = plan->launch_large ? lp.gu_blocks : 0;
  plan->large_down_grid = plan->launch_large ? lp.dn_blocks : 0;
  plan->combine_grid = (T > 0 && !fold) ? moe::combine_grid(T, H) : 0;
  // the MFMA kernels need the schedule kernel's tile lists first; the dense kernels (gate_up, the
  // fp16 rewrite of their h rows, down) run only when an expert can have kDenseMinRows rows (an
  // expert has at most T)
  const bool dense = plan->launch_large && T >= moe::kDenseMinRows;
  plan->n_launches = (plan->launch_small ? gu_launches + 1 : 0) + (plan->launch_large ? 3 : 0) +
                     (dense ? 3 : 0) + (T > 0 && !fold ? 1 : 0);
}

// Device address of `scratch` on the current device, looked up once per device with that device
// current (each GPU holds its own copy at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return MOE_ERR_LAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return MOE_ERR_LAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

void record(const moe_ffn_options& o, int stage, bool start, hipStream_t stream) {
  void* ev = start ? o.stage_start[stage] : o.stage_stop[stage];
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

MOE_API void moe_ffn_options_init(moe_ffn_options* o) {
  if (!o) return;
  o->small_m_max = -1;
  o->dense_down_cols = 0;
  for (int i = 0; i < MOE_NUM_STAGES; ++i) o->stage_start[i] = o->stage_stop[i] = nullptr;
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
  return moe::router_workspace_bytes(T, H, E);
}

namespace {

int router_check(const uint16_t* x_bf16, const uint16_t* w_router_bf16, int T, int H, int E, int k, int score_fn,
                 const void* workspace, size_t ws_bytes) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E ||
      (long)T * k > MOE_MAX_PAIRS || H < 32 || H > MOE_MAX_HIDDEN || H % 32)
    return MOE_ERR_SHAPE;
  if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !w_router_bf16 || !workspace) return MOE_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(w_router_bf16, 16) || !aligned(workspace, 256))
    return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < moe::router_workspace_bytes(T, H, E)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

}  // namespace

MOE_API int moe_router_gemm_topk_ex(const uint16_t* x_bf16, const uint16_t* w_router_bf16, int T, int H, int E,
                                    int k, int score_fn, int renorm, float* logits, int32_t* topk_ids,
                                    float* topk_w, void* workspace, size_t ws_bytes, int flags, void* stream) {
  if (flags & ~MOE_ROUTER_SPLIT_LAUNCH) return MOE_ERR_UNSUPPORTED;
  const int st = router_check(x_bf16, w_router_bf16, T, H, E, k, score_fn, workspace, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  if (!topk_ids || !topk_w) return MOE_ERR_NULL;
  if (moe::launch_router_gemm_topk(x_bf16, w_router_bf16, T, H, E, k, score_fn, renorm, workspace, logits,
                                   topk_ids, topk_w, (flags & MOE_ROUTER_SPLIT_LAUNCH) != 0,
                                   (hipStream_t)stream) != hipSuccess)
    return MOE_ERR_LAUNCH;
  return MOE_OK;
}

MOE_API int moe_router_gemm_topk(const uint16_t* x_bf16, const uint16_t* w_router_bf16, int T, int H, int E,
                                 int k, int score_fn, int renorm, float* logits, int32_t* topk_ids,
                                 float* topk_w, void* workspace, size_t ws_bytes, void* stream) {
  return moe_router_gemm_topk_ex(x_bf16, w_router_bf16, T, H, E, k, score_fn, renorm, logits, topk_ids, topk_w,
                                 workspace, ws_bytes, 0, stream);
}

// The grouping keeps its histograms and scans in LDS (each workgroup counts all the ids itself when
// there are several): no device workspace.
MOE_API size_t moe_group_tokens_workspace_size(int T, int k, int E) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || (long)T * k > MOE_MAX_PAIRS)
    return (size_t)-1;
  return 0;
}

MOE_API int moe_group_tokens(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                             int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                             int32_t* active, int32_t* n_active, void* workspace, size_t ws_bytes,
                             void* stream) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK ||
      (long)T * k > MOE_MAX_PAIRS)
    return MOE_ERR_SHAPE;
  (void)workspace;
  if (ws_bytes < moe_group_tokens_workspace_size(T, k, E)) return MOE_ERR_WORKSPACE;
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

MOE_API int moe_mxfp4_ffn_plan(int T, int H, int I, int E, int k, int flags, const moe_ffn_options* opts,
                               moe_ffn_plan* plan) {
  if (!plan) return MOE_ERR_NULL;
  if (!ffn_sizes_ok(T, H, I, E, k)) return MOE_ERR_SHAPE;
  if ((flags & ~kKnownFlags) || ((flags & MOE_FORCE_SMALL_M) && (flags & MOE_FORCE_LARGE_M)))
    return MOE_ERR_UNSUPPORTED;
  moe_ffn_options o;
  const int st = read_options(opts, o);
  if (st != MOE_OK) return st;
  fill_plan(T, H, I, E, k, flags, o, plan);
  return MOE_OK;
}

namespace {

// moe_mxfp4_ffn_ex; with `ro`, the gate_up launch is the routed variant, which also produces the
// routing and the grouping (ids, topk_w and the grouping arrays passed here are its outputs; the
// caller checks routed_ffn_ok first).
int ffn_impl(const uint16_t* x_bf16, int T, int H, int I, int E, int k, const uint8_t* w13_q,
             const uint8_t* w13_s, const uint8_t* w2_q, const uint8_t* w2_s, const float* topk_w,
             const int32_t* counts, const int32_t* offsets, const int32_t* sorted_pair, const int32_t* pair_pos,
             const int32_t* active, const int32_t* n_active, float clamp_limit, int flags, uint16_t* out_bf16,
             void* workspace, size_t ws_bytes, const moe_ffn_options* opts, void* stream,
             const moe::RouteOut* ro) {
  if (!ffn_sizes_ok(T, H, I, E, k)) return MOE_ERR_SHAPE;
  if ((flags & ~kKnownFlags) || ((flags & MOE_FORCE_SMALL_M) && (flags & MOE_FORCE_LARGE_M)))
    return MOE_ERR_UNSUPPORTED;
  moe_ffn_options o;
  {
    const int st = read_options(opts, o);
    if (st != MOE_OK) return st;
  }
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
  fill_plan(T, H, I, E, k, flags, o, &plan);
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
  const moe::DensePlan dp = moe::plan_dense(T, H, I, E, k, moe::kDenseMinRows, num_cus(), o.dense_down_cols / 32);
  // without MFMA kernels every active expert is small: the grouping's active list is the work list
  const int32_t* list = plan.launch_large ? small_list : active;
  const int32_t* list_count = plan.launch_large ? n_small : n_active;
  bool ok = true;

  if (plan.launch_large)
    ok &= moe::launch_schedule(r, E, thr, wl.tile_slots_max, dense_min, dp.slots, small_list, n_small,
                               tile_e, tile_m0, dense_e, dense_m0, s) == hipSuccess;

  record(o, MOE_STAGE_GATE_UP, true, s);
  if (plan.launch_small) {
    if (flags & MOE_UNFUSED_GATE_UP) {
      ok &= moe::launch_small_gateup(sp, r, list, list_count, H, I, w13_q, w13_s, clamp_limit,
                                     moe::kGateOnly, h_hi, h_lo, g_f32, s) == hipSuccess;
      ok &= moe::launch_small_gateup(sp, r, list, list_count, H, I, w13_q, w13_s, clamp_limit,
                                     moe::kUpWithGate, h_hi, h_lo, g_f32, s) == hipSuccess;
    } else if (ro) {
      ok &= moe::launch_small_gateup_routed(sp, r, *ro, H, I, w13_q, w13_s, clamp_limit, h_hi, h_lo, s) ==
            hipSuccess;
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
  record(o, MOE_STAGE_GATE_UP, false, s);

  record(o, MOE_STAGE_DOWN, true, s);
  if (dense)
    ok &= moe::launch_dense_h16(dp, r, I, dense_e, dense_m0, h_hi, h_lo, rowf, s) == hipSuccess;
  if (plan.launch_small && plan.fold_combine)
    ok &= moe::launch_small_down_combine(sp, r, list, list_count, pair_pos, topk_w, H, I, w2_q, w2_s, h_hi,
                                         h_lo, out_bf16, s) == hipSuccess;
  else if (plan.launch_small)
    ok &= moe::launch_small_down(sp, r, list, list_count, !plan.launch_large, H, I, w2_q, w2_s, h_hi, h_lo, y,
                                 s) == hipSuccess;
  if (plan.launch_large)
    ok &= moe::launch_large_down(lp, r, H, I, w2_q, w2_s, tile_e, tile_m0, h_hi, h_lo, y, s) == hipSuccess;
  if (dense)
    ok &= moe::launch_dense_down(dp, r, H, I, w2_q, w2_s, dense_e, dense_m0, h_hi, rowf, y, s) == hipSuccess;
  record(o, MOE_STAGE_DOWN, false, s);

  // (folded into the down launch: the combine stage's events bracket no work)
  record(o, MOE_STAGE_COMBINE, true, s);
  if (!plan.fold_combine)
    ok &= moe::launch_combine(y, topk_w, pair_pos, T, H, k, out_bf16, nullptr, s) == hipSuccess;
  record(o, MOE_STAGE_COMBINE, false, s);
  return ok ? MOE_OK : MOE_ERR_LAUNCH;
}

// Whether the routed gate_up variant serves a call: only the weight-streaming kernels run, the
// gate/up pass is fused, and the batch fits the variant (gateup_routed_ok).
bool routed_ffn_ok(int T, int H, int I, int E, int k, int flags, const moe_ffn_options& o) {
  if (T < 1 || (flags & MOE_UNFUSED_GATE_UP)) return false;
  moe_ffn_plan plan;
  fill_plan(T, H, I, E, k, flags, o, &plan);
  if (!plan.launch_small || plan.launch_large) return false;
  return moe::gateup_routed_ok(moe::plan_small(T, H, I, E, k, num_cus()), H, E);
}

}  // namespace

MOE_API int moe_mxfp4_ffn_ex(const uint16_t* x_bf16, int T, int H, int I, int E, int k,
                             const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                             const uint8_t* w2_s, const float* topk_w, const int32_t* counts,
                             const int32_t* offsets, const int32_t* sorted_pair,
                             const int32_t* pair_pos, const int32_t* active, const int32_t* n_active,
                             float clamp_limit, int flags, uint16_t* out_bf16, void* workspace,
                             size_t ws_bytes, const moe_ffn_options* opts, void* stream) {
  return ffn_impl(x_bf16, T, H, I, E, k, w13_q, w13_s, w2_q, w2_s, topk_w, counts, offsets, sorted_pair,
                  pair_pos, active, n_active, clamp_limit, flags, out_bf16, workspace, ws_bytes, opts, stream,
                  nullptr);
}

MOE_API int moe_mxfp4_ffn(const uint16_t* x_bf16, int T, int H, int I, int E, int k,
                          const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                          const uint8_t* w2_s, const float* topk_w, const int32_t* counts,
                          const int32_t* offsets, const int32_t* sorted_pair,
                          const int32_t* pair_pos, const int32_t* active, const int32_t* n_active,
                          float clamp_limit, int flags, uint16_t* out_bf16, void* workspace,
                          size_t ws_bytes, void* stream) {
  return moe_mxfp4_ffn_ex(x_bf16, T, H, I, E, k, w13_q, w13_s, w2_q, w2_s, topk_w, counts, offsets,
                          sorted_pair, pair_pos, active, n_active, clamp_limit, flags, out_bf16,
                          workspace, ws_bytes, nullptr, stream);
}

MOE_API size_t moe_mxfp4_ffn_noalloc_max_bytes(void) { return MOE_NOALLOC_SCRATCH_BYTES; }

// ---- activation-quantised FFN (W4A8 / W4A4) ---------------------------------------------------

namespace {

struct MxLayout {
  size_t sched, xq, xs, hq, hs, y, total;
  int slots;
};

bool mx_sizes_ok(int T, int H, int I, int E, int k, int act) {
  return ffn_sizes_ok(T, H, I, E, k) && H % 128 == 0 && I % 128 == 0 &&
         (act == MOE_ACT_MXFP8 || act == MOE_ACT_MXFP4);
}

// tile_e[slots], tile_m0[slots] | x codes | x scales | h codes | h scales | y f32[P, H]
MxLayout mx_layout(int T, int H, int I, int E, int k, int act) {
  MxLayout w;
  const size_t P = (size_t)T * k;
  const size_t ebits = act == MOE_ACT_MXFP8 ? 8 : 4;
  w.slots = moe::mx_slots_bound(T, E, k);
  size_t off = 0;
  w.sched = off;
  off = align_up(off + sizeof(int32_t) * 2 * (size_t)w.slots);
  w.xq = off;
  off = align_up(off + (size_t)T * H * ebits / 8);
  w.xs = off;
  off = align_up(off + (size_t)T * (H / 32));
  w.hq = off;
  off = align_up(off + P * I * ebits / 8);
  w.hs = off;
  off = align_up(off + P * (I / 32));
  w.y = off;
  off = align_up(off + P * H * sizeof(float));
  w.total = off;
  return w;
}

}  // namespace

MOE_API int moe_mx_quantize(const uint16_t* x_bf16, int rows, int cols, int act_format, uint8_t* codes,
                            uint8_t* scales, void* stream) {
  if (rows < 0 || cols < 32 || cols % 32 || (long)rows * cols > (1L << 31) - 1) return MOE_ERR_SHAPE;
  if (act_format != MOE_ACT_MXFP8 && act_format != MOE_ACT_MXFP4) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x_bf16 || !codes || !scales) return MOE_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(codes, 16)) return MOE_ERR_UNSUPPORTED;
  return moe::launch_mx_quant_x(x_bf16, rows, cols, act_format, codes, scales, (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

MOE_API size_t moe_mxfp4_ffn_mx_workspace_size(int T, int H, int I, int E, int k, int act_format) {
  if (!mx_sizes_ok(T, H, I, E, k, act_format)) return 0;
  return mx_layout(T, H, I, E, k, act_format).total;
}

MOE_API int moe_mxfp4_ffn_mx_h_offsets(int T, int H, int I, int E, int k, int act_format, size_t* codes_offset,
                                      size_t* scales_offset) {
  if (!codes_offset || !scales_offset) return MOE_ERR_NULL;
  if (!mx_sizes_ok(T, H, I, E, k, act_format)) return MOE_ERR_SHAPE;
  const MxLayout wl = mx_layout(T, H, I, E, k, act_format);
  *codes_offset = wl.hq;
  *scales_offset = wl.hs;
  return MOE_OK;
}

MOE_API int moe_mxfp4_ffn_mx(const uint16_t* x_bf16, int T, int H, int I, int E, int k, const uint8_t* w13_q,
                             const uint8_t* w13_s, const uint8_t* w2_q, const uint8_t* w2_s, const float* topk_w,
                             const int32_t* counts, const int32_t* offsets, const int32_t* sorted_pair,
                             const int32_t* pair_pos, float clamp_limit, int act_format, uint16_t* out_bf16,
                             void* workspace, size_t ws_bytes, const moe_ffn_options* opts, void* stream) {
  if (!ffn_sizes_ok(T, H, I, E, k) || H % 128 || I % 128) return MOE_ERR_SHAPE;
  if (act_format != MOE_ACT_MXFP8 && act_format != MOE_ACT_MXFP4) return MOE_ERR_UNSUPPORTED;
  moe_ffn_options o;
  {
    const int st = read_options(opts, o);
    if (st != MOE_OK) return st;
  }
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !w13_q || !w13_s || !w2_q || !w2_s || !topk_w || !counts || !offsets || !sorted_pair ||
      !pair_pos || !out_bf16 || !workspace)
    return MOE_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(out_bf16, 16) || !aligned(w13_q, 16) || !aligned(w2_q, 16) ||
      !aligned(w13_s, 4) || !aligned(w2_s, 4) || !aligned(workspace, kAlign))
    return MOE_ERR_UNSUPPORTED;
  const MxLayout wl = mx_layout(T, H, I, E, k, act_format);
  if (ws_bytes < wl.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  int32_t* tile_e = (int32_t*)(ws + wl.sched);
  int32_t* tile_m0 = tile_e + wl.slots;
  uint8_t* xq = (uint8_t*)(ws + wl.xq);
  uint8_t* xs = (uint8_t*)(ws + wl.xs);
  uint8_t* hq = (uint8_t*)(ws + wl.hq);
  uint8_t* hs = (uint8_t*)(ws + wl.hs);
  float* y = (float*)(ws + wl.y);
  const moe::MxPlan mp = moe::plan_mx(T, H, I, E, k);
  bool ok = moe::launch_mx_schedule(counts, E, mp, tile_e, tile_m0, s) == hipSuccess;
  ok &= moe::launch_mx_quant_x(x_bf16, T, H, act_format, xq, xs, s) == hipSuccess;
  record(o, MOE_STAGE_GATE_UP, true, s);
  ok &= moe::launch_mx_gateup(mp, act_format, xq, xs, counts, offsets, sorted_pair, k, H, I, tile_e, tile_m0, w13_q,
                              w13_s, clamp_limit, hq, hs, s) == hipSuccess;
  record(o, MOE_STAGE_GATE_UP, false, s);
  record(o, MOE_STAGE_DOWN, true, s);
  ok &= moe::launch_mx_down(mp, act_format, hq, hs, counts, offsets, k, H, I, tile_e, tile_m0, w2_q, w2_s, y, s) ==
        hipSuccess;
  record(o, MOE_STAGE_DOWN, false, s);
  record(o, MOE_STAGE_COMBINE, true, s);
  ok &= moe::launch_combine(y, topk_w, pair_pos, T, H, k, out_bf16, nullptr, s) == hipSuccess;
  record(o, MOE_STAGE_COMBINE, false, s);
  return ok ? MOE_OK : MOE_ERR_LAUNCH;
}

MOE_API int moe_mxfp4_ffn_noalloc(const uint16_t* x_bf16, int T, int H, int I, int E, int k,
                                  const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                                  const uint8_t* w2_s, const float* topk_w, const int32_t* counts,
                                  const int32_t* offsets, const int32_t* sorted_pair,
                                  const int32_t* pair_pos, const int32_t* active,
                                  const int32_t* n_active, float clamp_limit, int flags,
                                  uint16_t* out_bf16, void* stream) {
  if (!ffn_sizes_ok(T, H, I, E, k)) return MOE_ERR_SHAPE;
  if ((flags & ~kKnownFlags) || ((flags & MOE_FORCE_SMALL_M) && (flags & MOE_FORCE_LARGE_M)))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  // the same regions moe_mxfp4_ffn would take from a caller's workspace, here from `scratch`
  if (ws_layout((long)T * k, H, I, E, k, flags).total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != MOE_OK) return st;
  return moe_mxfp4_ffn_ex(x_bf16, T, H, I, E, k, w13_q, w13_s, w2_q, w2_s, topk_w, counts, offsets,
                          sorted_pair, pair_pos, active, n_active, clamp_limit, flags, out_bf16, ws,
                          MOE_NOALLOC_SCRATCH_BYTES, nullptr, stream);
}

MOE_API size_t moe_layer_decode_workspace_size(int T, int H, int I, int E, int k) {
  if (!ffn_sizes_ok(T, H, I, E, k) || T < 1) return 0;
  const int cus = num_cus();
  if (!moe::layer_supported(T, H, I, E, k, cus)) return 0;
  return moe::layer_workspace_bytes(T, H, I, E, k, cus);
}

MOE_API int moe_layer_decode(const float* logits, const uint16_t* x_bf16, int T, int H, int I, int E, int k,
                             int score_fn, int renorm, const uint8_t* w13_q, const uint8_t* w13_s,
                             const uint8_t* w2_q, const uint8_t* w2_s, float clamp_limit, int32_t* topk_ids,
                             float* topk_w, uint16_t* out_bf16, void* workspace, size_t ws_bytes,
                             void* stream) {
  if (!ffn_sizes_ok(T, H, I, E, k)) return MOE_ERR_SHAPE;
  if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  const int cus = num_cus();
  if (!moe::layer_supported(T, H, I, E, k, cus)) return MOE_ERR_UNSUPPORTED;
  if (!logits || !x_bf16 || !w13_q || !w13_s || !w2_q || !w2_s || !out_bf16 || !workspace) return MOE_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(out_bf16, 16) || !aligned(w13_q, 16) || !aligned(w2_q, 16) ||
      !aligned(workspace, kAlign))
    return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < moe::layer_workspace_bytes(T, H, I, E, k, cus)) return MOE_ERR_WORKSPACE;
  return moe::launch_layer_decode(logits, x_bf16, T, H, I, E, k, score_fn, renorm, w13_q, w13_s, w2_q, w2_s,
                                  clamp_limit, topk_ids, topk_w, out_bf16, workspace, cus,
                                  (hipStream_t)stream) == hipSuccess
             ? MOE_OK
             : MOE_ERR_LAUNCH;
}

namespace {

// Workspace of moe_layer_forward: the router's (header first), the routing and grouping arrays, then
// the FFN's.
struct LayerWs {
  size_t router, ids, w, counts, offsets, sorted_pair, pair_pos, active, n_active, ffn, total;
};

LayerWs layer_ws(int T, int H, int I, int E, int k, int flags) {
  LayerWs l;
  const size_t P = (size_t)T * k;
  size_t off = 0;
  l.router = off;
  off = align_up(off + moe::router_workspace_bytes(T, H, E));
  l.ids = off;
  off = align_up(off + P * 4);
  l.w = off;
  off = align_up(off + P * 4);
  l.counts = off;
  off = align_up(off + (size_t)E * 4);
  l.offsets = off;
  off = align_up(off + (size_t)(E + 1) * 4);
  l.sorted_pair = off;
  off = align_up(off + P * 4);
  l.pair_pos = off;
  off = align_up(off + P * 4);
  l.active = off;
  off = align_up(off + (size_t)E * 4);
  l.n_active = off;
  off = align_up(off + 4);
  l.ffn = off;
  off += ws_layout((long)P, H, I, E, k, flags).total;
  l.total = off;
  return l;
}

}  // namespace

namespace {

// Workspace of moe_layer_from_logits: the routing and grouping arrays, then the FFN's.
struct LogitsWs {
  size_t ids, w, counts, offsets, sorted_pair, pair_pos, active, n_active, ffn, total;
};

LogitsWs logits_ws(int T, int H, int I, int E, int k, int flags) {
  LogitsWs l;
  const size_t P = (size_t)T * k;
  size_t off = 0;
  l.ids = off;
  off = align_up(off + P * 4);
  l.w = off;
  off = align_up(off + P * 4);
  l.counts = off;
  off = align_up(off + (size_t)E * 4);
  l.offsets = off;
  off = align_up(off + (size_t)(E + 1) * 4);
  l.sorted_pair = off;
  off = align_up(off + P * 4);
  l.pair_pos = off;
  off = align_up(off + P * 4);
  l.active = off;
  off = align_up(off + (size_t)E * 4);
  l.n_active = off;
  off = align_up(off + 4);
  l.ffn = off;
  off += ws_layout((long)P, H, I, E, k, flags).total;
  l.total = off;
  return l;
}

}  // namespace

MOE_API size_t moe_layer_from_logits_workspace_size(int T, int H, int I, int E, int k, int flags) {
  if (!ffn_sizes_ok(T, H, I, E, k) || (flags & ~kKnownFlags)) return 0;
  return logits_ws(T, H, I, E, k, flags).total;
}

MOE_API int moe_layer_from_logits_routed(int T, int H, int I, int E, int k, int flags,
                                         const moe_ffn_options* opts) {
  moe_ffn_options o;
  if (!ffn_sizes_ok(T, H, I, E, k) || (flags & ~kKnownFlags) || read_options(opts, o) != MOE_OK) return 0;
  return routed_ffn_ok(T, H, I, E, k, flags, o) ? 1 : 0;
}

MOE_API int moe_layer_from_logits(const float* logits, const uint16_t* x_bf16, int T, int H, int I, int E, int k,
                                  int score_fn, int renorm, const uint8_t* w13_q, const uint8_t* w13_s,
                                  const uint8_t* w2_q, const uint8_t* w2_s, float clamp_limit, int flags,
                                  int32_t* topk_ids, float* topk_w, uint16_t* out_bf16, void* workspace,
                                  size_t ws_bytes, const moe_ffn_options* opts, void* stream) {
  if (!ffn_sizes_ok(T, H, I, E, k)) return MOE_ERR_SHAPE;
  if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_UNSUPPORTED;
  if ((flags & ~kKnownFlags) || ((flags & MOE_FORCE_SMALL_M) && (flags & MOE_FORCE_LARGE_M)))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!logits || !x_bf16 || !w13_q || !w13_s || !w2_q || !w2_s || !out_bf16 || !workspace) return MOE_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(out_bf16, 16) || !aligned(w13_q, 16) || !aligned(w2_q, 16) ||
      !aligned(workspace, kAlign))
    return MOE_ERR_UNSUPPORTED;
  const LogitsWs l = logits_ws(T, H, I, E, k, flags);
  if (ws_bytes < l.total) return MOE_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  int32_t* ids = topk_ids ? topk_ids : reinterpret_cast<int32_t*>(ws + l.ids);
  float* tw = topk_w ? topk_w : reinterpret_cast<float*>(ws + l.w);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + l.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + l.offsets);
  int32_t* sorted_pair = reinterpret_cast<int32_t*>(ws + l.sorted_pair);
  int32_t* pair_pos = reinterpret_cast<int32_t*>(ws + l.pair_pos);
  int32_t* active = reinterpret_cast<int32_t*>(ws + l.active);
  int32_t* n_active = reinterpret_cast<int32_t*>(ws + l.n_active);
  hipStream_t s = (hipStream_t)stream;
  moe_ffn_options o;
  {
    const int st = read_options(opts, o);
    if (st != MOE_OK) return st;
  }
  if (routed_ffn_ok(T, H, I, E, k, flags, o)) {
    const moe::RouteOut ro{logits, E, score_fn, renorm, ids, tw, counts, offsets, sorted_pair, pair_pos, active,
                           n_active};
    return ffn_impl(x_bf16, T, H, I, E, k, w13_q, w13_s, w2_q, w2_s, tw, counts, offsets, sorted_pair, pair_pos,
                    active, n_active, clamp_limit, flags, out_bf16, ws + l.ffn, ws_bytes - l.ffn, opts, stream,
                    &ro);
  }
  const int st = moe_route_group(logits, T, E, k, score_fn, renorm, ids, tw, counts, offsets, sorted_pair, pair_pos,
                                 active, n_active, s);
  if (st != MOE_OK) return st;
  return ffn_impl(x_bf16, T, H, I, E, k, w13_q, w13_s, w2_q, w2_s, tw, counts, offsets, sorted_pair, pair_pos,
                  active, n_active, clamp_limit, flags, out_bf16, ws + l.ffn, ws_bytes - l.ffn, opts, stream,
                  nullptr);
}

MOE_API size_t moe_layer_forward_workspace_size(int T, int H, int I, int E, int k, int flags) {
  if (!ffn_sizes_ok(T, H, I, E, k) || (flags & ~kKnownFlags)) return 0;
  return layer_ws(T, H, I, E, k, flags).total;
}

MOE_API int moe_layer_forward(const uint16_t* x_bf16, const uint16_t* w_router_bf16, int T, int H, int I, int E,
                              int k, int score_fn, int renorm, const uint8_t* w13_q, const uint8_t* w13_s,
                              const uint8_t* w2_q, const uint8_t* w2_s, float clamp_limit, int flags,
                              float* logits, int32_t* topk_ids, float* topk_w, uint16_t* out_bf16,
                              void* workspace, size_t ws_bytes, void* stream) {
  if (!ffn_sizes_ok(T, H, I, E, k)) return MOE_ERR_SHAPE;
  if (score_fn != MOE_SCORE_SOFTMAX && score_fn != MOE_SCORE_SIGMOID) return MOE_ERR_UNSUPPORTED;
  if ((flags & ~kKnownFlags) || ((flags & MOE_FORCE_SMALL_M) && (flags & MOE_FORCE_LARGE_M)))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !w_router_bf16 || !w13_q || !w13_s || !w2_q || !w2_s || !out_bf16 || !workspace)
    return MOE_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(w_router_bf16, 16) || !aligned(out_bf16, 16) || !aligned(w13_q, 16) ||
      !aligned(w2_q, 16) || !aligned(workspace, kAlign))
    return MOE_ERR_UNSUPPORTED;
  const LayerWs l = layer_ws(T, H, I, E, k, flags);
  if (ws_bytes < l.total) return MOE_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  int32_t* ids = topk_ids ? topk_ids : reinterpret_cast<int32_t*>(ws + l.ids);
  float* tw = topk_w ? topk_w : reinterpret_cast<float*>(ws + l.w);
  const moe::RouterGroupOut grp{reinterpret_cast<int32_t*>(ws + l.counts), reinterpret_cast<int32_t*>(ws + l.offsets),
                                reinterpret_cast<int32_t*>(ws + l.sorted_pair),
                                reinterpret_cast<int32_t*>(ws + l.pair_pos), reinterpret_cast<int32_t*>(ws + l.active),
                                reinterpret_cast<int32_t*>(ws + l.n_active)};
  if (moe::launch_router_group(x_bf16, w_router_bf16, T, H, E, k, score_fn, renorm, ws + l.router, logits, ids, tw,
                               grp, (hipStream_t)stream) != hipSuccess)
    return MOE_ERR_LAUNCH;
  return moe_mxfp4_ffn_ex(x_bf16, T, H, I, E, k, w13_q, w13_s, w2_q, w2_s, tw, grp.counts, grp.offsets,
                          grp.sorted_pair, grp.pair_pos, grp.active, grp.n_active, clamp_limit, flags, out_bf16,
                          ws + l.ffn, ws_bytes - l.ffn, nullptr, stream);
}
