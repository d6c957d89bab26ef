// The C ABI of libmoe (declared and documented in include/moe.h): argument
// checks on the host, workspace carving, launches.  No allocation, no
// synchronisation, no host reads of device data.
#include "../../include/moe.h"

#include <stdio.h>
#include <string.h>

#include "launch.hpp"

using namespace moe;

namespace {

thread_local hipError_t g_last_hip = hipSuccess;
thread_local char g_msg[256];
thread_local hipEvent_t g_events[K_COUNT][2];

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip = e;
  return MOE_ERR_HIP;
}

bool dims_ok(int64_t v) { return v > 0 && v % 64 == 0 && v <= (1 << 20); }

// Workspace layouts (byte offsets, each 256-aligned).
struct RouteWs { size_t w3, logits, part, total; };
RouteWs route_ws(int64_t T, int d, int E) {
  RouteWs w;
  w.w3 = 0;
  w.logits = align_up((size_t)3 * E * d * 2);
  w.part = w.logits + align_up((size_t)router_ksplit(T, E) * T * E * 4);
  w.total = w.part + align_up((size_t)topk_partial_floats(T, E) * 4);
  return w;
}
struct PermWs { size_t counts, base, total; };
PermWs perm_ws(int64_t T, int E) {
  const size_t nch = (size_t)ceil_div(T, PERM_CHUNK);
  PermWs w;
  w.counts = 0;
  w.base = align_up(nch * E * 4);
  w.total = w.base + align_up(nch * E * 4);
  return w;
}
struct FfnWs { size_t z, h, pre_a, pre_b, exp_a, exp_b, queues, total; };
FfnWs ffn_ws(int64_t T, int L, int E, int k, int F) {
  // tile tables sized for the smallest M tile any plan uses (128 rows)
  const size_t mt = (size_t)grouped_mtile_bound(T * k, E, 128);
  FfnWs w;
  w.z = 0;
  w.h = align_up((size_t)T * L * 2);
  w.pre_a = w.h + align_up((size_t)T * k * F * 2);
  w.pre_b = w.pre_a + align_up((size_t)(E + 1) * 4);
  w.exp_a = w.pre_b + align_up((size_t)(E + 1) * 4);
  w.exp_b = w.exp_a + align_up(mt * 4);
  w.queues = w.exp_b + align_up(mt * 4);
  w.total = w.queues + align_up(16 * 4);
  return w;
}
// FP8 experts: z and H as E4M3 bytes, then the same tile tables
FfnWs ffn8_ws(int64_t T, int L, int E, int k, int F) {
  const size_t mt = (size_t)grouped_mtile_bound(T * k, E, 128);
  FfnWs w;
  w.z = 0;
  w.h = align_up((size_t)T * L);
  w.pre_a = w.h + align_up((size_t)T * k * F);
  w.pre_b = w.pre_a + align_up((size_t)(E + 1) * 4);
  w.exp_a = w.pre_b + align_up((size_t)(E + 1) * 4);
  w.exp_b = w.exp_a + align_up(mt * 4);
  w.queues = w.exp_b + align_up(mt * 4);
  w.total = w.queues + align_up(16 * 4);
  return w;
}
size_t combine_ws(int64_t T, int L) { return align_up((size_t)T * L * 2); }

// multi-round dropless: z, the round buffer (E * C rows of H), the round's
// row tables, tile tables sized for a round's rows, queue counters
struct RoundsWs { size_t z, h, seg_start, seg_end, h_base, pre_a, pre_b, exp_a, exp_b, queues, total; };
int64_t round_rows_bound(int64_t T, int E, int k, int C) {
  const int64_t cap = (int64_t)E * C;
  return T * k < cap ? T * k : cap;
}
RoundsWs rounds_ws(int64_t T, int L, int E, int k, int F, int C) {
  const int64_t rb = round_rows_bound(T, E, k, C);
  const size_t mt = (size_t)grouped_mtile_bound(rb, E, 128);
  RoundsWs w;
  w.z = 0;
  w.h = align_up((size_t)T * L * 2);
  w.seg_start = w.h + align_up((size_t)E * C * F * 2);
  w.seg_end = w.seg_start + align_up((size_t)E * 4);
  w.h_base = w.seg_end + align_up((size_t)E * 4);
  w.pre_a = w.h_base + align_up((size_t)E * 4);
  w.pre_b = w.pre_a + align_up((size_t)(E + 1) * 4);
  w.exp_a = w.pre_b + align_up((size_t)(E + 1) * 4);
  w.exp_b = w.exp_a + align_up(mt * 4);
  w.queues = w.exp_b + align_up(mt * 4);
  w.total = w.queues + align_up(16 * 4);
  return w;
}
// Rounds any routing can need: a group of n experts holds at most
// T * min(k, n) rows and n * C slots per round.
int64_t max_rounds(int64_t T, int E, int k, int G, int C) {
  int64_t m = 0;
  const int sizes[2] = {G < E ? G : E, E % G ? E % G : (G < E ? G : E)};
  for (int n : sizes) {
    const int64_t load = T * (k < n ? k : n);
    const int64_t cap = (int64_t)n * C;
    const int64_t r = (load + cap - 1) / cap;
    if (r > m) m = r;
  }
  return m;
}

// backward: gradient casts and their transposes, recomputed expert
// activations, the padded K layout of the weight-gradient GEMMs
struct BwdWs {
  size_t go, goT, z, cb, cbT, dc, dyb, dtw, dh, h, dgb, dub, dzp, dzb, dzbT, xT, kpre, dybT, hT,
      dgbT, dubT, zpT, dl, dbp, dwp, pre_a, pre_b, exp_a, exp_b, queues, dy8, dg8, du8,
      rs_start, rs_end, rh_base, rh_end, total;
  int64_t Tp, Rp, RF;
};
// fp8: the E5M2 codes of dy, dg and du as well (FP8 data gradients)
// rounds > 0 (the multi-round backward, capacity C per expert and round):
// the expert rows' F-wide buffers and the weight gradients' transposes hold
// one round's rows, at most min(T k, E C), instead of all T k rows
BwdWs bwd_ws(int64_t T, int d, int L, int E, int k, int F, bool fp8 = false, int C = 0) {
  BwdWs w;
  const int64_t R = T * k;
  w.RF = C > 0 ? round_rows_bound(T, E, k, C) : R;  // rows of the per-round buffers
  w.Tp = ceil_div(T, 64) * 64;
  w.Rp = ceil_div(w.RF, 64) * 64 + (int64_t)64 * E;   // >= sum_e ceil64(rows_e)
  const size_t mt = (size_t)grouped_mtile_bound(w.RF, E, 128);
  const int64_t RF = w.RF;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align_up(bytes); return at; };
  w.go = take((size_t)T * d * 2);
  w.goT = take((size_t)d * w.Tp * 2);
  w.z = take((size_t)T * L * 2);
  w.cb = take((size_t)T * L * 2);
  w.cbT = take((size_t)L * w.Tp * 2);
  w.dc = take((size_t)T * L * 4);
  w.dyb = take((size_t)R * L * 2);
  w.dtw = take((size_t)R * 4);
  w.dh = take((size_t)RF * F * 4);
  w.h = take((size_t)RF * F * 2);
  w.dgb = take((size_t)RF * F * 2);
  w.dub = take((size_t)RF * F * 2);
  w.dzp = take((size_t)R * L * 4);
  w.dzb = take((size_t)T * L * 2);
  w.dzbT = take((size_t)L * w.Tp * 2);
  w.xT = take((size_t)d * w.Tp * 2);
  w.kpre = take((size_t)(E + 1) * 4);
  w.dybT = take((size_t)L * w.Rp * 2);
  w.hT = take((size_t)F * w.Rp * 2);
  w.dgbT = take((size_t)F * w.Rp * 2);
  w.dubT = take((size_t)F * w.Rp * 2);
  w.zpT = take((size_t)L * w.Rp * 2);
  w.dl = take((size_t)T * E * 4);
  w.dbp = take((size_t)router_db_partial_floats(T, E) * 4);
  w.dwp = take((size_t)router_dw_partial_floats(T, d, E) * 4);
  w.pre_a = take((size_t)(E + 1) * 4);
  w.pre_b = take((size_t)(E + 1) * 4);
  w.exp_a = take(mt * 4);
  w.exp_b = take(mt * 4);
  w.queues = take(24 * 4);
  w.dy8 = fp8 ? take((size_t)R * L) : 0;
  w.dg8 = fp8 ? take((size_t)R * F) : 0;
  w.du8 = fp8 ? take((size_t)R * F) : 0;
  w.rs_start = C > 0 ? take((size_t)E * 4) : 0;
  w.rs_end = C > 0 ? take((size_t)E * 4) : 0;
  w.rh_base = C > 0 ? take((size_t)E * 4) : 0;
  w.rh_end = C > 0 ? take((size_t)E * 4) : 0;
  w.total = o;
  return w;
}

// backward of the shared expert: g_out cast and its transpose, dhs, the
// recomputed hs and the cast gate/up gradients, their transposes and x^T
struct SharedBwdWs { size_t go, goT, dhs, hs, dgs, dus, hsT, dgsT, dusT, xT, total; int64_t Tp; };
SharedBwdWs shared_bwd_ws(int64_t T, int d, int Fs) {
  SharedBwdWs w;
  w.Tp = ceil_div(T, 64) * 64;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align_up(bytes); return at; };
  w.go = take((size_t)T * d * 2);
  w.goT = take((size_t)d * w.Tp * 2);
  w.dhs = take((size_t)T * Fs * 4);
  w.hs = take((size_t)T * Fs * 2);
  w.dgs = take((size_t)T * Fs * 2);
  w.dus = take((size_t)T * Fs * 2);
  w.hsT = take((size_t)Fs * w.Tp * 2);
  w.dgsT = take((size_t)Fs * w.Tp * 2);
  w.dusT = take((size_t)Fs * w.Tp * 2);
  w.xT = take((size_t)d * w.Tp * 2);
  w.total = o;
  return w;
}

int check_route_dims(int64_t T, int d, int E, int k) {
  if (T < 0 || d <= 0 || E <= 0 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (k > 16 || E > 1024 || !dims_ok(d)) return MOE_ERR_UNSUPPORTED;
  if (T * (int64_t)k >= (int64_t(1) << 31) || T * (int64_t)E >= (int64_t(1) << 40))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace

namespace moe {
EventScope::EventScope(int id_, hipStream_t s_) : s(s_), id(id_) {
  if (g_events[id][0]) hipEventRecord(g_events[id][0], s);
}
EventScope::~EventScope() {
  if (g_events[id][1]) hipEventRecord(g_events[id][1], s);
}
}  // namespace moe

extern "C" {

size_t moe_workspace_bytes(int op, int64_t T, int32_t d, int32_t L, int32_t E, int32_t k,
                           int32_t F, int32_t Fs) {
  if (op == MOE_OP_SHARED_BACKWARD)   // the shared expert: no experts or top-k involved
    return (T >= 0 && d > 0 && Fs > 0) ? shared_bwd_ws(T, d, Fs).total : 0;
  if (T < 0 || E <= 0 || k < 1) return 0;
  switch (op) {
    case MOE_OP_ROUTE: return d > 0 ? route_ws(T, d, E).total : 0;
    case MOE_OP_PERMUTE: return perm_ws(T, E).total;
    case MOE_OP_LATENT_FFN: return (L > 0 && F > 0) ? ffn_ws(T, L, E, k, F).total : 0;
    case MOE_OP_COMBINE: return L > 0 ? combine_ws(T, L) : 0;
    case MOE_OP_LATENT_FFN_FP8: return (L > 0 && F > 0) ? ffn8_ws(T, L, E, k, F).total : 0;
    case MOE_OP_BACKWARD:
      return (d > 0 && L > 0 && F > 0) ? bwd_ws(T, d, L, E, k, F).total : 0;
    case MOE_OP_BACKWARD_FP8:
      return (d > 0 && L > 0 && F > 0) ? bwd_ws(T, d, L, E, k, F, true).total : 0;
    case MOE_OP_SHARED_BACKWARD: return (d > 0 && Fs > 0) ? shared_bwd_ws(T, d, Fs).total : 0;
    default: return 0;
  }
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size, k < 1 or k > E)";
    case MOE_ERR_UNSUPPORTED:
      return "unsupported (k > 16, E > 1024, a width not a positive multiple of 64 (128 for "
             "the FP8 expert widths), T*k >= 2^31, or a pointer not 16-byte aligned)";
    case MOE_ERR_WORKSPACE: return "workspace too small (see moe_workspace_bytes)";
    case MOE_ERR_HIP:
      snprintf(g_msg, sizeof g_msg, "HIP error: %s", hipGetErrorString(g_last_hip));
      return g_msg;
    default: return "unknown status";
  }
}

int moe_set_kernel_events(int kernel, void* start_event, void* stop_event) {
  if (kernel < 0 || kernel >= K_COUNT) return MOE_ERR_INVALID_ARG;
  g_events[kernel][0] = (hipEvent_t)start_event;
  g_events[kernel][1] = (hipEvent_t)stop_event;
  return MOE_OK;
}

int moe_route_ex(const uint16_t* x, const float* w_router, const float* b_router,
                 int32_t bias_mode, int64_t T, int32_t d, int32_t E, int32_t k,
                 int32_t* topk_idx, float* topk_w, float* logits_out, float* prob_sum,
                 void* ws, size_t ws_bytes, void* stream) {
  int st = check_route_dims(T, d, E, k);
  if (st) return st;
  if (bias_mode != MOE_BIAS_LOGITS && bias_mode != MOE_BIAS_SELECTION) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_w || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(ws) ||
      (logits_out && !aligned16(logits_out)))
    return MOE_ERR_UNSUPPORTED;
  const RouteWs w = route_ws(T, d, E);
  if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  // one K chunk: the GEMM writes the final logits (into logits_out when
  // given); several: partial logits in the workspace, summed by the top-k
  // kernel, which then writes logits_out
  const int ks = router_ksplit(T, E);
  float* logits = (ks == 1 && logits_out) ? logits_out : (float*)(base + w.logits);
  // bias in the logits: added by the GEMM epilogue (one chunk) or the top-k
  // kernel (several); selection only: added by the top-k kernel to the
  // selection values
  const float* gemm_bias = bias_mode == MOE_BIAS_LOGITS ? b_router : nullptr;
  const float* sel_bias = bias_mode == MOE_BIAS_SELECTION ? b_router : nullptr;
  {
    EventScope ev(K_ROUTER_GEMM, s);
    st = hip_status(launch_router_gemm(x, w_router, gemm_bias, T, d, E, (uint16_t*)(base + w.w3),
                                       logits, s));
  }
  if (st) return st;
  EventScope ev(K_ROUTER_TOPK, s);
  return hip_status(launch_softmax_topk(logits, ks, ks > 1 ? gemm_bias : nullptr,
                                        ks > 1 ? logits_out : nullptr, sel_bias, T, E, k,
                                        topk_idx, topk_w,
                                        prob_sum ? (float*)(base + w.part) : nullptr, prob_sum,
                                        s));
}

int moe_route(const uint16_t* x, const float* w_router, const float* b_router, int64_t T,
              int32_t d, int32_t E, int32_t k, int32_t* topk_idx, float* topk_w,
              float* logits_out, void* ws, size_t ws_bytes, void* stream) {
  return moe_route_ex(x, w_router, b_router, MOE_BIAS_LOGITS, T, d, E, k, topk_idx, topk_w,
                      logits_out, nullptr, ws, ws_bytes, stream);
}

int moe_permute(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E, int32_t* expert_counts,
                int32_t* expert_offsets, int32_t* row_token, int32_t* assign_row, void* ws,
                size_t ws_bytes, void* stream) {
  if (T < 0 || E <= 0 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (k > 16 || E > 1024 || T * (int64_t)k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_idx || !row_token || !assign_row || !ws)) return MOE_ERR_INVALID_ARG;
  const PermWs w = perm_ws(T, E);
  if (T > 0 && ws_bytes < w.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  EventScope ev(K_PERMUTE, s);
  if (T == 0) {
    // an empty batch still defines the metadata: all counts and offsets zero
    // (a fill kernel, not hipMemsetAsync, so the call stays graph-capturable)
    return hip_status(launch_permute_empty(E, expert_counts, expert_offsets, s));
  }
  char* base = (char*)ws;
  return hip_status(launch_permute(topk_idx, T, k, E, expert_counts, expert_offsets, row_token,
                                   assign_row, (int32_t*)(base + w.counts),
                                   (int32_t*)(base + w.base), s));
}

int moe_permute_noalloc(const int32_t* topk_idx, int64_t T, int32_t k, int32_t E,
                        int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_token,
                        int32_t* assign_row, void* stream) {
  if (T < 0 || E <= 0 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (k > 16 || E > 1024 || T * (int64_t)k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_idx || !row_token || !assign_row)) return MOE_ERR_INVALID_ARG;
  if (permute_scratch_ints(T, E) > PERM_SCRATCH_INTS) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  EventScope ev(K_PERMUTE, s);
  if (T == 0) return hip_status(launch_permute_empty(E, expert_counts, expert_offsets, s));
  return hip_status(launch_permute_noalloc(topk_idx, T, k, E, expert_counts, expert_offsets,
                                           row_token, assign_row, s));
}

int moe_latent_ffn_forward(const uint16_t* x, const uint16_t* w_lat_down,
                           const int32_t* expert_offsets, const int32_t* row_token,
                           const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                           const uint16_t* ws_gate, const uint16_t* ws_up, int64_t T, int32_t d,
                           int32_t L, int32_t E, int32_t k, int32_t F, int32_t Fs,
                           float* y_rows, uint16_t* hs, void* ws, size_t ws_bytes,
                           void* stream) {
  if (T < 0 || E <= 0 || k < 1 || k > E || Fs < 0) return MOE_ERR_INVALID_ARG;
  if (k > 16 || E > 1024 || !dims_ok(d) || !dims_ok(L) || !dims_ok(F) ||
      (Fs > 0 && !dims_ok(Fs)) || T * (int64_t)k >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  // the gathered latent z[T, L] is addressed with 32-bit byte offsets
  if ((int64_t)T * L * 2 >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_lat_down || !expert_offsets || !row_token || !w_gate || !w_up || !w_down ||
      !y_rows || !ws)
    return MOE_ERR_INVALID_ARG;
  if (Fs > 0 && (!ws_gate || !ws_up || !hs)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {x, w_lat_down, w_gate, w_up, w_down, y_rows, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_UNSUPPORTED;
  if (Fs > 0 && (!aligned16(ws_gate) || !aligned16(ws_up) || !aligned16(hs)))
    return MOE_ERR_UNSUPPORTED;
  const FfnWs w = ffn_ws(T, L, E, k, F);
  if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  uint16_t* z = (uint16_t*)(base + w.z);
  uint16_t* H = (uint16_t*)(base + w.h);
  int32_t* pre_a = (int32_t*)(base + w.pre_a);
  int32_t* pre_b = (int32_t*)(base + w.pre_b);
  int32_t* exp_a = (int32_t*)(base + w.exp_a);
  int32_t* exp_b = (int32_t*)(base + w.exp_b);
  int32_t* queues = (int32_t*)(base + w.queues);
  const int64_t rows = T * k;
  const ExpertGemmPlan plan = plan_expert_gemms(rows, E);
  int st;
  {
    EventScope ev(K_LATENT_DOWN, s);
    st = hip_status(launch_latent_down(x, w_lat_down, T, d, L, z, s));
    if (!st && Fs > 0) st = hip_status(launch_shared_gate_up(x, ws_gate, ws_up, T, d, Fs, hs, s));
  }
  if (st) return st;
  st = hip_status(launch_tile_prefix(expert_offsets, E, plan.bm_gate_up, plan.bm_down, pre_a,
                                     pre_b, exp_a, exp_b, queues, s));
  if (st) return st;
  {
    EventScope ev(K_GATE_UP, s);
    st = hip_status(launch_gate_up(z, expert_offsets, row_token, pre_a, exp_a, queues, w_gate,
                                   w_up, T, rows, E, L, F, plan.bm_gate_up, H, s));
  }
  if (st) return st;
  EventScope ev(K_EXPERT_DOWN, s);
  return hip_status(launch_expert_down(H, expert_offsets, pre_b, exp_b, queues + 8, w_down, rows,
                                       E, L, F, plan.bm_down, y_rows, s));
}

int moe_combine(const float* y_rows, const float* topk_w, const int32_t* assign_row,
                const uint16_t* w_lat_up, const uint16_t* hs, const uint16_t* ws_down, int64_t T,
                int32_t d, int32_t L, int32_t k, int32_t Fs, float* out, void* ws,
                size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || Fs < 0) return MOE_ERR_INVALID_ARG;
  if (k > 16 || !dims_ok(d) || !dims_ok(L) || (Fs > 0 && !dims_ok(Fs)) ||
      T * (int64_t)k >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_rows || !topk_w || !assign_row || !w_lat_up || !out || !ws) return MOE_ERR_INVALID_ARG;
  if (Fs > 0 && (!hs || !ws_down)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_rows) || !aligned16(w_lat_up) || !aligned16(out) || !aligned16(ws) ||
      (Fs > 0 && (!aligned16(hs) || !aligned16(ws_down))))
    return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < combine_ws(T, L)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  uint16_t* c = (uint16_t*)ws;
  int st;
  {
    EventScope ev(K_COMBINE, s);
    st = hip_status(launch_combine(y_rows, topk_w, assign_row, T, L, k, c, s));
  }
  if (st) return st;
  EventScope ev(K_LATENT_UP, s);
  return hip_status(launch_latent_up(c, w_lat_up, hs, ws_down, T, d, L, Fs, out, s));
}

int moe_fp8_amax(const uint16_t* src, int64_t ntensor, int64_t numel, float* amax,
                 void* stream) {
  if (ntensor < 0 || numel < 0) return MOE_ERR_INVALID_ARG;
  if (ntensor == 0) return MOE_OK;
  if (!amax || (numel > 0 && !src)) return MOE_ERR_INVALID_ARG;
  if (numel % 8 != 0 || ntensor > 65535 || !aligned16(src)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_amax_bf16(src, ntensor, numel, (uint32_t*)amax, (hipStream_t)stream));
}

int moe_fp8_quantize(const uint16_t* src, int64_t ntensor, int64_t numel, const float* scale,
                     uint8_t* dst, void* stream) {
  if (ntensor < 0 || numel < 0) return MOE_ERR_INVALID_ARG;
  if (ntensor == 0 || numel == 0) return MOE_OK;
  if (!src || !scale || !dst) return MOE_ERR_INVALID_ARG;
  if (numel % 8 != 0 || ntensor > 65535 || !aligned16(src) || !aligned16(dst))
    return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_quantize_e4m3(src, ntensor, numel, scale, dst, (hipStream_t)stream));
}

int moe_fp8_scale_update(float* history, const float* amax, int64_t ntensor, int32_t hist_len,
                         int32_t slot, float* scale, void* stream) {
  if (ntensor < 0 || hist_len < 1 || slot < 0 || slot >= hist_len) return MOE_ERR_INVALID_ARG;
  if (ntensor == 0) return MOE_OK;
  if (!history || !amax || !scale) return MOE_ERR_INVALID_ARG;
  return hip_status(
      launch_scale_update(history, amax, ntensor, hist_len, slot, scale, (hipStream_t)stream));
}

int moe_latent_ffn_forward_fp8(const uint16_t* x, const uint16_t* w_lat_down,
                               const int32_t* expert_offsets, const int32_t* row_token,
                               const uint8_t* w_gate, const uint8_t* w_up, const uint8_t* w_down,
                               const float* w_scale, const float* act_scale,
                               const uint16_t* ws_gate, const uint16_t* ws_up, int64_t T,
                               int32_t d, int32_t L, int32_t E, int32_t k, int32_t F, int32_t Fs,
                               float* y_rows, uint16_t* hs, float* act_amax, void* ws,
                               size_t ws_bytes, void* stream) {
  if (T < 0 || E <= 0 || k < 1 || k > E || Fs < 0) return MOE_ERR_INVALID_ARG;
  if (k > 16 || E > 1024 || !dims_ok(d) || !dims_ok(L) || !dims_ok(F) ||
      (Fs > 0 && !dims_ok(Fs)) || T * (int64_t)k >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  // one K stage of an FP8 GEMM is 128 values
  if (L % 128 != 0 || F % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * L >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_lat_down || !expert_offsets || !row_token || !w_gate || !w_up || !w_down ||
      !w_scale || !act_scale || !y_rows || !act_amax || !ws)
    return MOE_ERR_INVALID_ARG;
  if (Fs > 0 && (!ws_gate || !ws_up || !hs)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {x, w_lat_down, w_gate, w_up, w_down, y_rows, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_UNSUPPORTED;
  if (Fs > 0 && (!aligned16(ws_gate) || !aligned16(ws_up) || !aligned16(hs)))
    return MOE_ERR_UNSUPPORTED;
  const FfnWs w = ffn8_ws(T, L, E, k, F);
  if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  uint8_t* z8 = (uint8_t*)(base + w.z);
  uint8_t* H8 = (uint8_t*)(base + w.h);
  int32_t* pre_a = (int32_t*)(base + w.pre_a);
  int32_t* pre_b = (int32_t*)(base + w.pre_b);
  int32_t* exp_a = (int32_t*)(base + w.exp_a);
  int32_t* exp_b = (int32_t*)(base + w.exp_b);
  int32_t* queues = (int32_t*)(base + w.queues);
  uint32_t* amax = (uint32_t*)act_amax;
  const int64_t rows = T * k;
  const ExpertGemmPlan plan = plan_expert_gemms(rows, E);
  int st = hip_status(launch_zero_u32(amax, 2, s));
  if (st) return st;
  {
    EventScope ev(K_LATENT_DOWN, s);
    st = hip_status(launch_latent_down_q8(x, w_lat_down, T, d, L, act_scale, amax, z8, s));
    if (!st && Fs > 0) st = hip_status(launch_shared_gate_up(x, ws_gate, ws_up, T, d, Fs, hs, s));
  }
  if (st) return st;
  st = hip_status(launch_tile_prefix(expert_offsets, E, plan.bm_gate_up, plan.bm_down, pre_a,
                                     pre_b, exp_a, exp_b, queues, s));
  if (st) return st;
  {
    EventScope ev(K_GATE_UP, s);
    st = hip_status(launch_gate_up_fp8(z8, expert_offsets, row_token, pre_a, exp_a, queues,
                                       w_gate, w_up, act_scale, w_scale, w_scale + E,
                                       act_scale + 1, amax + 1, T, rows, E, L, F,
                                       plan.bm_gate_up, H8, s));
  }
  if (st) return st;
  EventScope ev(K_EXPERT_DOWN, s);
  return hip_status(launch_expert_down_fp8(H8, expert_offsets, pre_b, exp_b, queues + 8, w_down,
                                           act_scale + 1, w_scale + 2 * E, rows, E, L, F,
                                           plan.bm_down, y_rows, s));
}

size_t moe_workspace_bytes_rounds(int64_t T, int32_t d, int32_t L, int32_t E, int32_t k,
                                  int32_t F, int32_t Fs, int32_t capacity, int32_t group_size) {
  (void)d;
  (void)Fs;
  if (T < 0 || E <= 0 || k < 1 || L <= 0 || F <= 0 || capacity < 1 || group_size < 1) return 0;
  return rounds_ws(T, L, E, k, F, capacity).total;
}

int moe_latent_ffn_forward_rounds(const uint16_t* x, const uint16_t* w_lat_down,
                                  const int32_t* expert_offsets, const int32_t* row_token,
                                  const uint16_t* w_gate, const uint16_t* w_up,
                                  const uint16_t* w_down, const uint16_t* ws_gate,
                                  const uint16_t* ws_up, int64_t T, int32_t d, int32_t L,
                                  int32_t E, int32_t k, int32_t F, int32_t Fs, int32_t capacity,
                                  int32_t group_size, float* y_rows, uint16_t* hs,
                                  int32_t* rounds_out, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || E <= 0 || k < 1 || k > E || Fs < 0 || capacity < 1 || group_size < 1)
    return MOE_ERR_INVALID_ARG;
  if (k > 16 || E > 1024 || !dims_ok(d) || !dims_ok(L) || !dims_ok(F) ||
      (Fs > 0 && !dims_ok(Fs)) || T * (int64_t)k >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * L * 2 >= (int64_t(1) << 31) ||
      (int64_t)E * capacity >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_lat_down || !expert_offsets || !row_token || !w_gate || !w_up || !w_down ||
      !y_rows || !ws)
    return MOE_ERR_INVALID_ARG;
  if (Fs > 0 && (!ws_gate || !ws_up || !hs)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {x, w_lat_down, w_gate, w_up, w_down, y_rows, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_UNSUPPORTED;
  if (Fs > 0 && (!aligned16(ws_gate) || !aligned16(ws_up) || !aligned16(hs)))
    return MOE_ERR_UNSUPPORTED;
  const RoundsWs w = rounds_ws(T, L, E, k, F, capacity);
  if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  uint16_t* z = (uint16_t*)(base + w.z);
  uint16_t* Hr = (uint16_t*)(base + w.h);
  int32_t* seg_start = (int32_t*)(base + w.seg_start);
  int32_t* seg_end = (int32_t*)(base + w.seg_end);
  int32_t* h_base = (int32_t*)(base + w.h_base);
  int32_t* pre_a = (int32_t*)(base + w.pre_a);
  int32_t* pre_b = (int32_t*)(base + w.pre_b);
  int32_t* exp_a = (int32_t*)(base + w.exp_a);
  int32_t* exp_b = (int32_t*)(base + w.exp_b);
  int32_t* queues = (int32_t*)(base + w.queues);
  const int64_t rb = round_rows_bound(T, E, k, capacity);
  const ExpertGemmPlan plan = plan_expert_gemms(rb, E);
  int st;
  {
    EventScope ev(K_LATENT_DOWN, s);
    st = hip_status(launch_latent_down(x, w_lat_down, T, d, L, z, s));
    if (!st && Fs > 0) st = hip_status(launch_shared_gate_up(x, ws_gate, ws_up, T, d, Fs, hs, s));
  }
  if (st) return st;
  // The host does not know the routing, so it enqueues the most rounds any
  // routing can need; rounds past the ones this routing needs find no rows
  // and their GEMMs exit at once.
  const int64_t R = max_rounds(T, E, k, group_size, capacity);
  EventScope ev(K_GATE_UP, s);   // brackets every round (gate/up and down)
  for (int64_t r = 0; r < R; ++r) {
    st = hip_status(launch_round_tables(expert_offsets, E, group_size, capacity, (int)r,
                                        plan.bm_gate_up, plan.bm_down, seg_start, seg_end, h_base,
                                        pre_a, pre_b, exp_a, exp_b, queues, rounds_out, s));
    if (st) return st;
    st = hip_status(launch_round_experts(z, seg_start, seg_end, h_base, row_token, pre_a, exp_a,
                                         pre_b, exp_b, queues, w_gate, w_up, w_down, T, rb, E, L,
                                         F, plan.bm_gate_up, plan.bm_down, Hr, y_rows, s));
    if (st) return st;
  }
  return MOE_OK;
}

}  // extern "C"

extern "C" {

int moe_grad_cast_bf16(const float* src, int64_t n, int32_t rounding, uint32_t seed,
                       int32_t stream_id, uint16_t* dst, void* stream) {
  if (n < 0 || (rounding != MOE_ROUND_NEAREST && rounding != MOE_ROUND_STOCHASTIC))
    return MOE_ERR_INVALID_ARG;
  if (n % 4 != 0) return MOE_ERR_UNSUPPORTED;
  if (n == 0) return MOE_OK;
  if (!src || !dst) return MOE_ERR_INVALID_ARG;
  if (!aligned16(src) || ((uintptr_t)dst & 7u)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_cvt_grad(src, n, rounding == MOE_ROUND_STOCHASTIC,
                                    sr_stream_key(seed, (uint32_t)stream_id), dst,
                                    (hipStream_t)stream));
}

int moe_backward_prepare(const uint16_t* w_lat_down, const uint16_t* w_gate,
                         const uint16_t* w_up, const uint16_t* w_down,
                         const uint16_t* w_lat_up, int32_t d, int32_t L, int32_t E, int32_t F,
                         uint16_t* w_lat_down_t, uint16_t* w_gate_t, uint16_t* w_up_t,
                         uint16_t* w_down_t, uint16_t* w_lat_up_t, void* stream) {
  if (E <= 0) return MOE_ERR_INVALID_ARG;
  if (E > 1024 || !dims_ok(d) || !dims_ok(L) || !dims_ok(F)) return MOE_ERR_UNSUPPORTED;
  const void* ptrs[] = {w_lat_down, w_gate, w_up, w_down, w_lat_up,
                        w_lat_down_t, w_gate_t, w_up_t, w_down_t, w_lat_up_t};
  for (const void* p : ptrs) {
    if (!p) return MOE_ERR_INVALID_ARG;
    if (!aligned16(p)) return MOE_ERR_UNSUPPORTED;
  }
  hipStream_t s = (hipStream_t)stream;
  const int64_t eFL = (int64_t)F * L;
  int st = hip_status(launch_transpose_dense(w_lat_down, L, d, w_lat_down_t, L, 1, 0, 0, s));
  if (!st) st = hip_status(launch_transpose_dense(w_gate, F, L, w_gate_t, F, E, eFL, eFL, s));
  if (!st) st = hip_status(launch_transpose_dense(w_up, F, L, w_up_t, F, E, eFL, eFL, s));
  if (!st) st = hip_status(launch_transpose_dense(w_down, L, F, w_down_t, L, E, eFL, eFL, s));
  if (!st) st = hip_status(launch_transpose_dense(w_lat_up, d, L, w_lat_up_t, d, 1, 0, 0, s));
  return st;
}

}  // extern "C"

namespace {

// FP8 data gradients of the backward: E4M3 transposed expert weights with
// their scales, the gradients' scales, and the maxima out
struct BwdFp8 {
  const uint8_t *w_gate_t8, *w_up_t8, *w_down_t8;
  const float* w_scale;      // [3E]: W_g, W_u, W_d
  const float* grad_scale;   // [3]: dy, dg, du
  float* grad_amax;          // [3]
};

int backward_impl(const uint16_t* x, const float* w_router, const float* router_logits,
                  int32_t bias_mode, const int32_t* topk_idx, const float* topk_w,
                  const int32_t* expert_offsets, const int32_t* row_token,
                  const int32_t* assign_row, const float* y_rows, const uint16_t* w_lat_down,
                  const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_lat_down_t,
                  const uint16_t* w_gate_t, const uint16_t* w_up_t, const uint16_t* w_down_t,
                  const uint16_t* w_lat_up_t, const float* g_out, int64_t T, int32_t d,
                  int32_t L, int32_t E, int32_t k, int32_t F, int32_t rounding, uint32_t seed,
                  float* dx, float* dw_router, float* db_router, float* dw_lat_down,
                  float* dw_gate, float* dw_up, float* dw_down, float* dw_lat_up, float* dtopk_w,
                  void* ws, size_t ws_bytes, void* stream, const BwdFp8* f8,
                  int32_t capacity = 0, int32_t group_size = 0) {
  if (T < 0 || E <= 0 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (bias_mode != MOE_BIAS_LOGITS && bias_mode != MOE_BIAS_SELECTION) return MOE_ERR_INVALID_ARG;
  if (rounding != MOE_ROUND_NEAREST && rounding != MOE_ROUND_STOCHASTIC)
    return MOE_ERR_INVALID_ARG;
  if (k > 16 || E > 1024 || !dims_ok(d) || !dims_ok(L) || !dims_ok(F) ||
      T * (int64_t)k >= (int64_t(1) << 31) || (int64_t)T * L * 2 >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (f8 && (L % 128 != 0 || F % 128 != 0)) return MOE_ERR_UNSUPPORTED;
  const bool rounds = capacity > 0;
  if (rounds && (f8 || (int64_t)E * capacity >= (int64_t(1) << 31))) return MOE_ERR_UNSUPPORTED;
  // the expert data-gradient GEMMs read the bf16 transposes, or (f8) the
  // E4M3 ones
  const void* wg_t = f8 ? (const void*)f8->w_gate_t8 : (const void*)w_gate_t;
  const void* wu_t = f8 ? (const void*)f8->w_up_t8 : (const void*)w_up_t;
  const void* wd_t = f8 ? (const void*)f8->w_down_t8 : (const void*)w_down_t;
  const void* req[] = {x, w_router, router_logits, topk_idx, topk_w, expert_offsets, row_token,
                       assign_row, y_rows, w_lat_down, w_gate, w_up, w_lat_down_t, wg_t,
                       wu_t, wd_t, w_lat_up_t, g_out, dx, dw_router, dw_lat_down,
                       dw_gate, dw_up, dw_down, dw_lat_up, ws};
  for (const void* p : req)
    if (!p) return MOE_ERR_INVALID_ARG;
  if (f8 && (!f8->w_scale || !f8->grad_scale || !f8->grad_amax)) return MOE_ERR_INVALID_ARG;
  const void* al[] = {x, w_router, router_logits, y_rows, w_lat_down, w_gate, w_up,
                      w_lat_down_t, wg_t, wu_t, wd_t, w_lat_up_t, g_out, dx,
                      dw_router, dw_lat_down, dw_gate, dw_up, dw_down, dw_lat_up, ws};
  for (const void* p : al)
    if (!aligned16(p)) return MOE_ERR_UNSUPPORTED;
  const BwdWs w = bwd_ws(T, d, L, E, k, F, f8 != nullptr, rounds ? capacity : 0);
  // the weight-gradient GEMMs read 256-row tiles of the transposed operands
  // (row length Tp or Rp) through 32-bit buffer offsets
  if ((int64_t)256 * 2 * (w.Tp > w.Rp ? w.Tp : w.Rp) >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  auto B16 = [&](size_t off) { return (uint16_t*)(base + off); };
  auto F32 = [&](size_t off) { return (float*)(base + off); };
  auto I32 = [&](size_t off) { return (int32_t*)(base + off); };
  const int sr = rounding == MOE_ROUND_STOCHASTIC;
  const int64_t R = T * k;
  const int64_t Tp = w.Tp, Rp = w.Rp;
  float* dtw = dtopk_w ? dtopk_w : F32(w.dtw);
  const ExpertGemmPlan plan = plan_expert_gemms(w.RF, E);
  int st;
  {
    // up-projection: g = bf16(g_out), dW_up = g^T c, dc = g W_up
    EventScope ev(K_BWD_UP, s);
    st = hip_status(launch_cvt_grad(g_out, T * d, sr, sr_stream_key(seed, 1), B16(w.go), s));
    if (!st) st = hip_status(launch_transpose_dense(B16(w.go), T, d, B16(w.goT), Tp, 1, 0, 0, s));
    if (!st) st = hip_status(launch_combine(y_rows, topk_w, assign_row, T, L, k, B16(w.cb), s));
    if (!st) st = hip_status(launch_transpose_dense(B16(w.cb), T, L, B16(w.cbT), Tp, 1, 0, 0, s));
    if (!st) st = hip_status(launch_dense_f32(B16(w.goT), Tp, B16(w.cbT), Tp, Tp, d, L, dw_lat_up,
                                              L, s));
    if (!st) st = hip_status(launch_dense_f32(B16(w.go), d, w_lat_up_t, d, d, T, L, F32(w.dc), L,
                                              s));
  }
  if (st) return st;
  uint32_t* gamax = f8 ? (uint32_t*)f8->grad_amax : nullptr;   // float bits, >= 0
  {
    EventScope ev(K_BWD_COMBINE, s);
    if (f8) {
      st = hip_status(launch_zero_u32(gamax, 3, s));
      if (!st) st = hip_status(launch_combine_bwd_q8(
          F32(w.dc), y_rows, topk_w, assign_row, T, L, k, sr, sr_stream_key(seed, 2), B16(w.dyb),
          dtw, (uint8_t*)(base + w.dy8), f8->grad_scale,
          sr_stream_key(seed, 6), gamax, s));
    } else {
      st = hip_status(launch_combine_bwd(F32(w.dc), y_rows, topk_w, assign_row, T, L, k, sr,
                                         sr_stream_key(seed, 2), B16(w.dyb), dtw, s));
    }
  }
  if (st) return st;
  if (rounds) {
    // the multi-round schedule: per round, the expert data gradients of the
    // round's rows (fixed-size buffers of round_rows_bound rows) and that
    // round's contribution to the expert weight gradients (round 0 writes,
    // later rounds add).  The host enqueues the most rounds any routing can
    // need; surplus rounds find no rows (their weight-gradient tiles are
    // skipped).  K_BWD_DGRAD brackets every round.
    EventScope ev(K_BWD_DGRAD, s);
    int32_t* kpre = I32(w.kpre);
    int32_t* r0 = I32(w.rs_start);
    int32_t* r1 = I32(w.rs_end);
    int32_t* hb = I32(w.rh_base);
    int32_t* he = I32(w.rh_end);
    st = hip_status(launch_latent_down(x, w_lat_down, T, d, L, B16(w.z), s));
    const int64_t NR = max_rounds(T, E, k, group_size, capacity);
    for (int64_t r = 0; r < NR && !st; ++r) {
      st = hip_status(launch_round_tables(expert_offsets, E, group_size, capacity, (int)r,
                                          plan.bm_gate_up, plan.bm_down, r0, r1, hb, I32(w.pre_a),
                                          I32(w.pre_b), I32(w.exp_a), I32(w.exp_b),
                                          I32(w.queues), nullptr, s, he));
      if (!st) st = hip_status(launch_round_expert_bwd(
          B16(w.dyb), B16(w.z), row_token, r0, r1, hb, I32(w.pre_a), I32(w.exp_a), I32(w.pre_b),
          I32(w.exp_b), I32(w.queues), w_gate, w_up, w_gate_t, w_up_t, w_down_t, T, w.RF, E, L, F,
          plan.bm_gate_up, plan.bm_down, sr, sr_stream_key(seed, 3), sr_stream_key(seed, 4),
          F32(w.dh), B16(w.dgb), B16(w.dub), B16(w.h), F32(w.dzp), s));
      // this round's weight gradients: dW_d += dy^T h, dW_g += dg^T z, dW_u += du^T z
      const bool acc = r > 0;
      if (!st) st = hip_status(launch_kpad_prefix(r0, E, kpre, s, r1));
      if (!st) st = hip_status(launch_transpose_grouped(B16(w.dyb), nullptr, 0, L, r0, kpre, E,
                                                        B16(w.dybT), Rp, s, r1));
      if (!st) st = hip_status(launch_transpose_grouped(B16(w.h), nullptr, 0, F, hb, kpre, E,
                                                        B16(w.hT), Rp, s, he));
      if (!st) st = hip_status(launch_kgrouped_f32(B16(w.dybT), Rp, B16(w.hT), Rp, kpre, E, L, F,
                                                   dw_down, (int64_t)L * F, s, acc));
      if (!st) st = hip_status(launch_transpose_grouped(B16(w.dgb), nullptr, 0, F, hb, kpre, E,
                                                        B16(w.dgbT), Rp, s, he));
      if (!st) st = hip_status(launch_transpose_grouped(B16(w.dub), nullptr, 0, F, hb, kpre, E,
                                                        B16(w.dubT), Rp, s, he));
      if (!st) st = hip_status(launch_transpose_grouped(B16(w.z), row_token, T, L, r0, kpre, E,
                                                        B16(w.zpT), Rp, s, r1));
      if (!st) st = hip_status(launch_kgrouped_f32(B16(w.dgbT), Rp, B16(w.zpT), Rp, kpre, E, F, L,
                                                   dw_gate, (int64_t)F * L, s, acc));
      if (!st) st = hip_status(launch_kgrouped_f32(B16(w.dubT), Rp, B16(w.zpT), Rp, kpre, E, F, L,
                                                   dw_up, (int64_t)F * L, s, acc));
    }
  } else {
  {
    // experts: dh = dy W_d; z and the gate/up GEMM recomputed with the SwiGLU
    // backward in its epilogue (dg, du, and h for dW_d); the rows' latent
    // gradient
    EventScope ev(K_BWD_DGRAD, s);
    st = hip_status(launch_latent_down(x, w_lat_down, T, d, L, B16(w.z), s));
    if (!st) st = hip_status(launch_tile_prefix(expert_offsets, E, plan.bm_gate_up, plan.bm_down,
                                                I32(w.pre_a), I32(w.pre_b), I32(w.exp_a),
                                                I32(w.exp_b), I32(w.queues), s));
    if (!st) st = hip_status(launch_zero_u32((uint32_t*)I32(w.queues) + 16, 8, s));
    if (f8) {
      uint8_t* dy8 = (uint8_t*)(base + w.dy8);
      uint8_t* dg8 = (uint8_t*)(base + w.dg8);
      uint8_t* du8 = (uint8_t*)(base + w.du8);
      const float* gs = f8->grad_scale;
      const float* wsc = f8->w_scale;
      if (!st) st = hip_status(launch_expert_dh_fp8(dy8, expert_offsets, I32(w.pre_b),
                                                    I32(w.exp_b), I32(w.queues), f8->w_down_t8,
                                                    gs, wsc + 2 * E, R, E, L, F, plan.bm_down,
                                                    F32(w.dh), s));
      if (!st) st = hip_status(launch_gate_up_bwd_q8(
          B16(w.z), expert_offsets, row_token, I32(w.pre_a), I32(w.exp_a), I32(w.queues) + 8,
          w_gate, w_up, F32(w.dh), T, R, E, L, F, plan.bm_gate_up, sr, sr_stream_key(seed, 3),
          sr_stream_key(seed, 4), sr_stream_key(seed, 7), sr_stream_key(seed, 8), gs, gamax,
          B16(w.dgb), B16(w.dub), B16(w.h), dg8, du8, s));
      if (!st) st = hip_status(launch_dzp_fp8(dg8, du8, expert_offsets, I32(w.pre_b),
                                              I32(w.exp_b), I32(w.queues) + 16, f8->w_gate_t8,
                                              f8->w_up_t8, gs + 1, gs + 2, wsc, wsc + E, R, E, L,
                                              F, plan.bm_down, F32(w.dzp), s));
    } else {
      if (!st) st = hip_status(launch_expert_dh(B16(w.dyb), expert_offsets, I32(w.pre_b),
                                                I32(w.exp_b), I32(w.queues), w_down_t, R, E, L, F,
                                                plan.bm_down, F32(w.dh), s));
      if (!st) st = hip_status(launch_gate_up_bwd(
          B16(w.z), expert_offsets, row_token, I32(w.pre_a), I32(w.exp_a), I32(w.queues) + 8,
          w_gate, w_up, F32(w.dh), T, R, E, L, F, plan.bm_gate_up, sr, sr_stream_key(seed, 3),
          sr_stream_key(seed, 4), B16(w.dgb), B16(w.dub), B16(w.h), s));
      if (!st) st = hip_status(launch_dzp(B16(w.dgb), B16(w.dub), expert_offsets, I32(w.pre_b),
                                          I32(w.exp_b), I32(w.queues) + 16, w_gate_t, w_up_t, R,
                                          E, L, F, plan.bm_down, F32(w.dzp), s));
    }
  }
  if (st) return st;
  {
    // expert weight gradients over each expert's rows (padded K layout)
    EventScope ev(K_BWD_WGRAD, s);
    int32_t* kpre = I32(w.kpre);
    st = hip_status(launch_kpad_prefix(expert_offsets, E, kpre, s));
    if (!st) st = hip_status(launch_transpose_grouped(B16(w.dyb), nullptr, 0, L, expert_offsets,
                                                      kpre, E, B16(w.dybT), Rp, s));
    if (!st) st = hip_status(launch_transpose_grouped(B16(w.h), nullptr, 0, F, expert_offsets,
                                                      kpre, E, B16(w.hT), Rp, s));
    if (!st) st = hip_status(launch_kgrouped_f32(B16(w.dybT), Rp, B16(w.hT), Rp, kpre, E, L, F,
                                                 dw_down, (int64_t)L * F, s));
    if (!st) st = hip_status(launch_transpose_grouped(B16(w.dgb), nullptr, 0, F, expert_offsets,
                                                      kpre, E, B16(w.dgbT), Rp, s));
    if (!st) st = hip_status(launch_transpose_grouped(B16(w.dub), nullptr, 0, F, expert_offsets,
                                                      kpre, E, B16(w.dubT), Rp, s));
    if (!st) st = hip_status(launch_transpose_grouped(B16(w.z), row_token, T, L, expert_offsets,
                                                      kpre, E, B16(w.zpT), Rp, s));
    if (!st) st = hip_status(launch_kgrouped_f32(B16(w.dgbT), Rp, B16(w.zpT), Rp, kpre, E, F, L,
                                                 dw_gate, (int64_t)F * L, s));
    if (!st) st = hip_status(launch_kgrouped_f32(B16(w.dubT), Rp, B16(w.zpT), Rp, kpre, E, F, L,
                                                 dw_up, (int64_t)F * L, s));
  }
  }
  if (st) return st;
  {
    // latent: dz per token (fixed slot order), dx = dz W_dn, dW_dn = dz^T x
    EventScope ev(K_BWD_LATENT, s);
    st = hip_status(launch_gather_sum(F32(w.dzp), assign_row, T, L, k, sr, sr_stream_key(seed, 5),
                                      B16(w.dzb), s));
    if (!st) st = hip_status(launch_dense_f32(B16(w.dzb), L, w_lat_down_t, L, L, T, d, dx, d, s));
    if (!st) st = hip_status(launch_transpose_dense(B16(w.dzb), T, L, B16(w.dzbT), Tp, 1, 0, 0,
                                                    s));
    if (!st) st = hip_status(launch_transpose_dense(x, T, d, B16(w.xT), Tp, 1, 0, 0, s));
    if (!st) st = hip_status(launch_dense_f32(B16(w.dzbT), Tp, B16(w.xT), Tp, Tp, L, d,
                                              dw_lat_down, d, s));
  }
  if (st) return st;
  // router (FP32): softmax backward, dx += dl W_r, dW_r = dl^T x, db
  EventScope ev(K_BWD_ROUTER, s);
  st = hip_status(launch_router_bwd(router_logits, topk_idx, dtw, T, E, k, F32(w.dl), s));
  if (!st) st = hip_status(launch_router_dx(F32(w.dl), w_router, T, d, E, dx, s));
  if (!st) st = hip_status(launch_router_dw(F32(w.dl), x, T, d, E, F32(w.dwp), dw_router, s));
  if (!st && db_router) {
    if (bias_mode == MOE_BIAS_LOGITS)
      st = hip_status(launch_router_db(F32(w.dl), T, E, F32(w.dbp), db_router, s));
    else
      st = hip_status(launch_zero_u32((uint32_t*)db_router, E, s));
  }
  return st;
}

}  // namespace

extern "C" {

int moe_backward(const uint16_t* x, const float* w_router, const float* router_logits,
                 int32_t bias_mode, const int32_t* topk_idx, const float* topk_w,
                 const int32_t* expert_offsets, const int32_t* row_token,
                 const int32_t* assign_row, const float* y_rows, const uint16_t* w_lat_down,
                 const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_lat_down_t,
                 const uint16_t* w_gate_t, const uint16_t* w_up_t, const uint16_t* w_down_t,
                 const uint16_t* w_lat_up_t, const float* g_out, int64_t T, int32_t d,
                 int32_t L, int32_t E, int32_t k, int32_t F, int32_t rounding, uint32_t seed,
                 float* dx, float* dw_router, float* db_router, float* dw_lat_down,
                 float* dw_gate, float* dw_up, float* dw_down, float* dw_lat_up, float* dtopk_w,
                 void* ws, size_t ws_bytes, void* stream) {
  return backward_impl(x, w_router, router_logits, bias_mode, topk_idx, topk_w, expert_offsets,
                       row_token, assign_row, y_rows, w_lat_down, w_gate, w_up, w_lat_down_t,
                       w_gate_t, w_up_t, w_down_t, w_lat_up_t, g_out, T, d, L, E, k, F, rounding,
                       seed, dx, dw_router, db_router, dw_lat_down, dw_gate, dw_up, dw_down,
                       dw_lat_up, dtopk_w, ws, ws_bytes, stream, nullptr);
}

int moe_backward_fp8(const uint16_t* x, const float* w_router, const float* router_logits,
                     int32_t bias_mode, const int32_t* topk_idx, const float* topk_w,
                     const int32_t* expert_offsets, const int32_t* row_token,
                     const int32_t* assign_row, const float* y_rows, const uint16_t* w_lat_down,
                     const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_lat_down_t,
                     const uint8_t* w_gate_t8, const uint8_t* w_up_t8, const uint8_t* w_down_t8,
                     const float* w_scale, const uint16_t* w_lat_up_t, const float* g_out,
                     const float* grad_scale, int64_t T, int32_t d, int32_t L, int32_t E,
                     int32_t k, int32_t F, int32_t rounding, uint32_t seed, float* dx,
                     float* dw_router, float* db_router, float* dw_lat_down, float* dw_gate,
                     float* dw_up, float* dw_down, float* dw_lat_up, float* dtopk_w,
                     float* grad_amax, void* ws, size_t ws_bytes, void* stream) {
  const BwdFp8 f8 = {w_gate_t8, w_up_t8, w_down_t8, w_scale, grad_scale, grad_amax};
  return backward_impl(x, w_router, router_logits, bias_mode, topk_idx, topk_w, expert_offsets,
                       row_token, assign_row, y_rows, w_lat_down, w_gate, w_up, w_lat_down_t,
                       nullptr, nullptr, nullptr, w_lat_up_t, g_out, T, d, L, E, k, F, rounding,
                       seed, dx, dw_router, db_router, dw_lat_down, dw_gate, dw_up, dw_down,
                       dw_lat_up, dtopk_w, ws, ws_bytes, stream, &f8);
}

int moe_grad_cast_e5m2(const float* src, int64_t n, const float* scale, int32_t rounding,
                       uint32_t seed, int32_t stream_id, uint8_t* dst, void* stream) {
  if (n < 0 || (rounding != MOE_ROUND_NEAREST && rounding != MOE_ROUND_STOCHASTIC))
    return MOE_ERR_INVALID_ARG;
  if (n % 4 != 0) return MOE_ERR_UNSUPPORTED;
  if (n == 0) return MOE_OK;
  if (!src || !dst || !scale) return MOE_ERR_INVALID_ARG;
  if (!aligned16(src) || ((uintptr_t)dst & 3u)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_cvt_e5m2(src, n, scale, rounding == MOE_ROUND_STOCHASTIC,
                                    sr_stream_key(seed, (uint32_t)stream_id), dst,
                                    (hipStream_t)stream));
}

}  // extern "C"

extern "C" {

int moe_backward_prepare_shared(const uint16_t* ws_gate, const uint16_t* ws_up,
                                const uint16_t* ws_down, int32_t d, int32_t Fs,
                                uint16_t* ws_gate_t, uint16_t* ws_up_t, uint16_t* ws_down_t,
                                void* stream) {
  if (d <= 0 || Fs <= 0) return MOE_ERR_INVALID_ARG;
  if (!dims_ok(d) || !dims_ok(Fs)) return MOE_ERR_UNSUPPORTED;
  const void* ptrs[] = {ws_gate, ws_up, ws_down, ws_gate_t, ws_up_t, ws_down_t};
  for (const void* p : ptrs) {
    if (!p) return MOE_ERR_INVALID_ARG;
    if (!aligned16(p)) return MOE_ERR_UNSUPPORTED;
  }
  hipStream_t s = (hipStream_t)stream;
  int st = hip_status(launch_transpose_dense(ws_gate, Fs, d, ws_gate_t, Fs, 1, 0, 0, s));
  if (!st) st = hip_status(launch_transpose_dense(ws_up, Fs, d, ws_up_t, Fs, 1, 0, 0, s));
  if (!st) st = hip_status(launch_transpose_dense(ws_down, d, Fs, ws_down_t, d, 1, 0, 0, s));
  return st;
}

int moe_shared_backward(const uint16_t* x, const float* g_out, const uint16_t* ws_gate,
                        const uint16_t* ws_up, const uint16_t* ws_gate_t,
                        const uint16_t* ws_up_t, const uint16_t* ws_down_t, int64_t T,
                        int32_t d, int32_t Fs, int32_t rounding, uint32_t seed, float* dx,
                        float* dws_gate, float* dws_up, float* dws_down, void* ws,
                        size_t ws_bytes, void* stream) {
  if (T < 0 || d <= 0 || Fs <= 0) return MOE_ERR_INVALID_ARG;
  if (rounding != MOE_ROUND_NEAREST && rounding != MOE_ROUND_STOCHASTIC)
    return MOE_ERR_INVALID_ARG;
  if (!dims_ok(d) || !dims_ok(Fs)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  const void* req[] = {x, g_out, ws_gate, ws_up, ws_gate_t, ws_up_t, ws_down_t, dx, dws_gate,
                       dws_up, dws_down, ws};
  for (const void* p : req) {
    if (!p) return MOE_ERR_INVALID_ARG;
    if (!aligned16(p)) return MOE_ERR_UNSUPPORTED;
  }
  const SharedBwdWs w = shared_bwd_ws(T, d, Fs);
  // the weight-gradient GEMMs read 256-row tiles of the transposed operands
  // (row length Tp) through 32-bit buffer offsets; rows of x, g and the
  // [T, Fs] gradients likewise within a tile
  if ((int64_t)256 * 2 * w.Tp >= (int64_t(1) << 31) || (int64_t)256 * 4 * Fs >= (int64_t(1) << 31) ||
      T * (int64_t)Fs >= (int64_t(1) << 40))
    return MOE_ERR_UNSUPPORTED;
  if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  auto B16 = [&](size_t off) { return (uint16_t*)(base + off); };
  auto F32 = [&](size_t off) { return (float*)(base + off); };
  const int sr = rounding == MOE_ROUND_STOCHASTIC;
  const int64_t Tp = w.Tp;
  EventScope ev(K_BWD_SHARED, s);
  // g = bf16(g_out) (the same cast as moe_backward's: stream 1), and g^T
  int st = hip_status(launch_cvt_grad(g_out, T * d, sr, sr_stream_key(seed, 1), B16(w.go), s));
  if (!st) st = hip_status(launch_transpose_dense(B16(w.go), T, d, B16(w.goT), Tp, 1, 0, 0, s));
  // dhs = g Ws_d  (B = Ws_d^T [Fs, d])
  if (!st) st = hip_status(launch_dense_f32(B16(w.go), d, ws_down_t, d, d, T, Fs, F32(w.dhs), Fs,
                                            s));
  // gs, us, hs recomputed; dgs, dus cast (streams 9, 10)
  if (!st) st = hip_status(launch_shared_gate_up_bwd(x, ws_gate, ws_up, F32(w.dhs), T, d, Fs, sr,
                                                     sr_stream_key(seed, 9),
                                                     sr_stream_key(seed, 10), B16(w.dgs),
                                                     B16(w.dus), B16(w.hs), s));
  // dx += dgs Ws_g + dus Ws_u  (B = Ws_g^T, Ws_u^T [d, Fs])
  if (!st) st = hip_status(launch_dense_f32_add2(B16(w.dgs), Fs, ws_gate_t, Fs, Fs, B16(w.dus), Fs,
                                                 ws_up_t, Fs, Fs, T, d, dx, d, s));
  // weight gradients over the tokens (K = Tp, zero-padded transposes):
  // dWs_d = g^T hs, dWs_g = dgs^T x, dWs_u = dus^T x
  if (!st) st = hip_status(launch_transpose_dense(B16(w.hs), T, Fs, B16(w.hsT), Tp, 1, 0, 0, s));
  if (!st) st = hip_status(launch_dense_f32(B16(w.goT), Tp, B16(w.hsT), Tp, Tp, d, Fs, dws_down,
                                            Fs, s));
  if (!st) st = hip_status(launch_transpose_dense(B16(w.dgs), T, Fs, B16(w.dgsT), Tp, 1, 0, 0, s));
  if (!st) st = hip_status(launch_transpose_dense(B16(w.dus), T, Fs, B16(w.dusT), Tp, 1, 0, 0, s));
  if (!st) st = hip_status(launch_transpose_dense(x, T, d, B16(w.xT), Tp, 1, 0, 0, s));
  if (!st) st = hip_status(launch_dense_f32(B16(w.dgsT), Tp, B16(w.xT), Tp, Tp, Fs, d, dws_gate, d,
                                            s));
  if (!st) st = hip_status(launch_dense_f32(B16(w.dusT), Tp, B16(w.xT), Tp, Tp, Fs, d, dws_up, d,
                                            s));
  return st;
}

}  // extern "C"

extern "C" {

size_t moe_workspace_bytes_backward_rounds(int64_t T, int32_t d, int32_t L, int32_t E, int32_t k,
                                           int32_t F, int32_t capacity, int32_t group_size) {
  if (T < 0 || E <= 0 || k < 1 || d <= 0 || L <= 0 || F <= 0 || capacity < 1 || group_size < 1)
    return 0;
  return bwd_ws(T, d, L, E, k, F, false, capacity).total;
}

int moe_backward_rounds(const uint16_t* x, const float* w_router, const float* router_logits,
                        int32_t bias_mode, const int32_t* topk_idx, const float* topk_w,
                        const int32_t* expert_offsets, const int32_t* row_token,
                        const int32_t* assign_row, const float* y_rows,
                        const uint16_t* w_lat_down, const uint16_t* w_gate, const uint16_t* w_up,
                        const uint16_t* w_lat_down_t, const uint16_t* w_gate_t,
                        const uint16_t* w_up_t, const uint16_t* w_down_t,
                        const uint16_t* w_lat_up_t, const float* g_out, int64_t T, int32_t d,
                        int32_t L, int32_t E, int32_t k, int32_t F, int32_t capacity,
                        int32_t group_size, int32_t rounding, uint32_t seed, float* dx,
                        float* dw_router, float* db_router, float* dw_lat_down, float* dw_gate,
                        float* dw_up, float* dw_down, float* dw_lat_up, float* dtopk_w, void* ws,
                        size_t ws_bytes, void* stream) {
  if (capacity < 1 || group_size < 1) return MOE_ERR_INVALID_ARG;
  return backward_impl(x, w_router, router_logits, bias_mode, topk_idx, topk_w, expert_offsets,
                       row_token, assign_row, y_rows, w_lat_down, w_gate, w_up, w_lat_down_t,
                       w_gate_t, w_up_t, w_down_t, w_lat_up_t, g_out, T, d, L, E, k, F, rounding,
                       seed, dx, dw_router, db_router, dw_lat_down, dw_gate, dw_up, dw_down,
                       dw_lat_up, dtopk_w, ws, ws_bytes, stream, nullptr, capacity, group_size);
}

}  // extern "C"
