// C-ABI entry points: host-side validation, workspace carving, launches.
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe_dispatch.h"
#include "layout.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// optional per-kernel timing
// ---------------------------------------------------------------------------
namespace {
struct TimingRec {
  const char* name;
  hipEvent_t b, e;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_pool;
// read by every call that launches an ordered fold, set by moe_set_spin_limit
// from any thread
std::atomic<int> g_spin_limit{1 << 20};

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

void timing_mark(hipStream_t st, const char* name, bool begin) {
  if (!g_timing) return;
  std::lock_guard<std::mutex> lk(g_tmu);
  if (begin) {
    TimingRec r{name, take_event(), nullptr};
    if (r.b) hipEventRecord(r.b, st);
    g_recs.push_back(r);
  } else {
    for (auto it = g_recs.rbegin(); it != g_recs.rend(); ++it) {
      if (it->e == nullptr && it->name == name) {
        it->e = take_event();
        if (it->e) hipEventRecord(it->e, st);
        break;
      }
    }
  }
}

}  // namespace moe

using namespace moe;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(const moe_shape* s, Shape* out) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->T < 1 || s->d < 1 || s->E < 1 || s->K < 1 || s->h < 1) return MOE_ERR_INVALID_ARG;
  if (s->K > s->E) return MOE_ERR_INVALID_ARG;
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if ((long long)s->T * s->K >= (1LL << 31)) return MOE_ERR_INVALID_ARG;
  if ((long long)s->T * s->d >= (1LL << 40)) return MOE_ERR_INVALID_ARG;
  if (s->E > 1024 || s->K > 32) return MOE_ERR_UNSUPPORTED;
  if (s->d % 128 != 0 || s->h % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if (s->act != MOE_ACT_SWIGLU && s->act != MOE_ACT_SILU && s->act != MOE_ACT_RELU) return MOE_ERR_INVALID_ARG;
  {
    // the kernels read whole tensors through buffer resources with 32-bit
    // byte offsets: x and dY [T,d] (gathered rows), one expert's weights
    // [h,d], and up to T rows of H or dH [*, 2h] (an expert's rows)
    const long long eb = s->dtype == MOE_BF16 ? 2 : 4, lim = 0x7ffffff0LL;
    const long long hw = s->act == MOE_ACT_SWIGLU ? 2LL * s->h : s->h;
    if ((long long)s->T * s->d * eb > lim || (long long)s->h * s->d * eb > lim || (long long)s->T * hw * eb > lim)
      return MOE_ERR_UNSUPPORTED;
  }
  out->T = s->T;
  out->act = s->act;
  out->d = s->d;
  out->E = s->E;
  out->K = s->K;
  out->h = s->h;
  out->bf16 = s->dtype == MOE_BF16;
  return MOE_OK;
}

#define REQ(p)                                           \
  do {                                                   \
    if (!(p) || !aligned16(p)) return MOE_ERR_INVALID_ARG; \
  } while (0)
#define OPT(p)                                 \
  do {                                         \
    if ((p) && !aligned16(p)) return MOE_ERR_INVALID_ARG; \
  } while (0)

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_shape* s, int which) {
  Shape sh;
  if (check_shape(s, &sh) != MOE_OK) return 0;
  switch (which) {
    case MOE_WS_INDEX: return index_ws(sh, nullptr).bytes;
    case MOE_WS_EXPERT_FWD: return expert_ws(sh, WS_EXPERT_FWD, nullptr).bytes;
    case MOE_WS_COMBINE: return expert_ws(sh, WS_COMBINE, nullptr).bytes;
    case MOE_WS_EXPERT_BWD: return expert_ws(sh, WS_EXPERT_BWD, nullptr).bytes;
    case MOE_WS_EXPERT_BWD_H: return expert_ws(sh, WS_EXPERT_BWD_H, nullptr).bytes;
    case MOE_WS_COMBINE_STAGED: return expert_ws(sh, WS_COMBINE_STAGED, nullptr).bytes;
    case MOE_WS_INDEX_DENSE: return dense_index_ws(sh, nullptr).bytes;
    case MOE_WS_EXPERT_BWD_LEAN: return expert_ws(sh, WS_EXPERT_BWD_LEAN, nullptr).bytes;
    default: return 0;
  }
}

const char* moe_status_string(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

int moe_set_spin_limit(int polls) {
  if (polls > 0) return g_spin_limit.exchange(polls, std::memory_order_relaxed);
  return g_spin_limit.load(std::memory_order_relaxed);
}

int moe_route_topk(const moe_shape* s, const void* x, const void* wg, const float* bias, float* logits,
                   int32_t* topk_ids, float* topk_w, void* stream) {
  Shape sh;
  int rc = check_shape(s, &sh);
  if (rc) return rc;
  REQ(logits);
  REQ(topk_ids);
  REQ(topk_w);
  hipStream_t st = (hipStream_t)stream;
  if (x) {
    REQ(wg);
    OPT(x);
    if (!aligned16(x)) return MOE_ERR_INVALID_ARG;
    OPT(bias);
    if (route_fused_applies(sh)) return hip_status(launch_route_fused(sh, x, wg, bias, logits, topk_ids, topk_w, st));
    rc = hip_status(launch_router_logits(sh, x, wg, bias, logits, topk_ids, topk_w, st));
    if (rc || router_logits_has_topk(sh)) return rc;
  }
  return hip_status(launch_topk(sh, logits, topk_ids, topk_w, st));
}

int moe_build_index(const moe_shape* s, const int32_t* topk_ids, int32_t* offsets, int32_t* expert_token_indices,
                    int32_t* token_index_map, void* ws, size_t ws_bytes, void* stream) {
  Shape sh;
  int rc = check_shape(s, &sh);
  if (rc) return rc;
  REQ(topk_ids);
  REQ(offsets);
  REQ(expert_token_indices);
  REQ(token_index_map);
  REQ(ws);
  const IndexWs w = index_ws(sh, ws);
  if (ws_bytes < w.bytes) return MOE_ERR_WORKSPACE;
  return hip_status(launch_build_index(sh, topk_ids, offsets, expert_token_indices, token_index_map, w,
                                       (hipStream_t)stream));
}

int moe_build_index_noalloc(const moe_shape* s, const int32_t* topk_ids, int32_t* offsets,
                            int32_t* expert_token_indices, int32_t* token_index_map, void* stream) {
  Shape sh;
  int rc = check_shape(s, &sh);
  if (rc) return rc;
  REQ(topk_ids);
  REQ(offsets);
  REQ(expert_token_indices);
  REQ(token_index_map);
  if (index_ws(sh, nullptr).bytes > index_scratch_bytes()) return MOE_ERR_WORKSPACE;
  void* p = nullptr;
  if (index_scratch_ptr(&p) != hipSuccess) return MOE_ERR_HIP;
  const IndexWs w = index_ws(sh, p);
  return hip_status(launch_build_index(sh, topk_ids, offsets, expert_token_indices, token_index_map, w,
                                       (hipStream_t)stream));
}

int moe_build_index_dense(const moe_shape* s, const int32_t* topk_ids, int32_t* offsets,
                          int32_t* expert_token_indices, int32_t* token_index_map, void* ws, size_t ws_bytes,
                          void* stream) {
  Shape sh;
  int rc = check_shape(s, &sh);
  if (rc) return rc;
  REQ(topk_ids);
  REQ(offsets);
  REQ(expert_token_indices);
  REQ(token_index_map);
  REQ(ws);
  const DenseIndexWs w = dense_index_ws(sh, ws);
  if (ws_bytes < w.bytes) return MOE_ERR_WORKSPACE;
  return hip_status(launch_build_index_dense(sh, topk_ids, offsets, expert_token_indices, token_index_map, w,
                                             (hipStream_t)stream));
}

int moe_expert_fwd(const moe_shape* s, const void* x, const int32_t* offsets, const int32_t* expert_token_indices,
                   const void* w_gate, const void* w_up, void* h_ab, void* y_swi, void* ws, size_t ws_bytes,
                   void* stream) {
  Shape sh;
  int rc = check_shape(s, &sh);
  if (rc) return rc;
  REQ(x);
  REQ(offsets);
  REQ(expert_token_indices);
  REQ(w_gate);
  if (sh.gated()) REQ(w_up);
  else OPT(w_up);  // plain two-layer expert: no up projection
  OPT(h_ab);  // NULL: nothing is saved for a backward
  REQ(y_swi);
  REQ(ws);
  const ExpertWs w = expert_ws(sh, WS_EXPERT_FWD, ws);
  if (ws_bytes < w.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  rc = hip_status(launch_prep(sh, w, offsets, nullptr, nullptr, nullptr, false, -1, st));
  if (rc) return rc;
  return hip_status(launch_gate_up(sh, x, offsets, expert_token_indices, w_gate, w_up, h_ab, y_swi, w, st));
}

int moe_combine(const moe_shape* s, const void* y_swi, const void* w_down, const int32_t* offsets,
                const int32_t* expert_token_indices, const int32_t* token_index_map, const int32_t* topk_ids,
                const float* topk_w, void* out, void* ws, size_t ws_bytes, void* stream) {
  Shape sh;
  int rc = check_shape(s, &sh);
  if (rc) return rc;
  REQ(y_swi);
  REQ(w_down);
  REQ(offsets);
  REQ(expert_token_indices);
  REQ(token_index_map);
  REQ(topk_ids);
  REQ(topk_w);
  REQ(out);
  REQ(ws);
  const ExpertWs w = expert_ws(sh, WS_COMBINE, ws);
  if (ws_bytes < w.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  rc = hip_status(launch_prep(sh, w, offsets, topk_ids, topk_w, token_index_map, true, ERR_COMBINE, st));
  if (rc) return rc;
  return hip_status(launch_down_combine(sh, y_swi, w_down, offsets, expert_token_indices, out, w,
                                        g_spin_limit.load(std::memory_order_relaxed), st));
}

int moe_combine_staged(const moe_shape* s, const void* y_swi, const void* w_down, const int32_t* offsets,
                       const int32_t* expert_token_indices, const int32_t* token_index_map, const int32_t* topk_ids,
                       const float* topk_w, void* out, void* ws, size_t ws_bytes, void* stream) {
  Shape sh;
  int rc = check_shape(s, &sh);
  if (rc) return rc;
  REQ(y_swi);
  REQ(w_down);
  REQ(offsets);
  REQ(expert_token_indices);
  REQ(token_index_map);
  REQ(topk_ids);
  REQ(topk_w);
  REQ(out);
  REQ(ws);
  const ExpertWs w = expert_ws(sh, WS_COMBINE_STAGED, ws);
  if (ws_bytes < w.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  rc = hip_status(launch_prep(sh, w, offsets, nullptr, nullptr, nullptr, false, -1, st));
  if (rc) return rc;
  return hip_status(launch_combine_staged(sh, y_swi, w_down, offsets, token_index_map, topk_w, out, w, st));
}

int moe_expert_bwd(const moe_shape* s, const void* dout, const void* x, const void* wg, const void* w_gate,
                   const void* w_up, const void* w_down, const int32_t* topk_ids, const float* topk_w,
                   const int32_t* offsets, const int32_t* expert_token_indices, const int32_t* token_index_map,
                   const void* h_ab, const void* y_swi, void* a_prime, void* dh, void* dx, float* dwg,
                   float* dw_gate, float* dw_up, float* dw_down, float* ds, void* ws, size_t ws_bytes,
                   void* stream) {
  Shape sh;
  int rc = check_shape(s, &sh);
  if (rc) return rc;
  REQ(dout);
  REQ(x);
  REQ(wg);
  REQ(w_gate);
  if (sh.gated()) REQ(w_up);
  else OPT(w_up);  // plain two-layer expert: no up projection
  REQ(w_down);
  REQ(topk_ids);
  REQ(topk_w);
  REQ(offsets);
  REQ(expert_token_indices);
  REQ(token_index_map);
  REQ(h_ab);
  OPT(y_swi);  // NULL: H-only saving, y recomputed from h_ab
  OPT(a_prime);  // H-only: where A' goes (else the workspace); must be NULL with a saved y_swi
  if (y_swi && a_prime) return MOE_ERR_INVALID_ARG;
  if (a_prime && a_prime == h_ab) return MOE_ERR_INVALID_ARG;
  OPT(dh);  // where dH goes (else the workspace); may be h_ab itself
  if (dh && !y_swi && !a_prime) return MOE_ERR_INVALID_ARG;  // a lean workspace has no room for A'
  if (dh && (dh == y_swi || dh == a_prime || dh == dout || dh == x || dh == dx)) return MOE_ERR_INVALID_ARG;
  REQ(dx);
  REQ(dwg);
  REQ(dw_gate);
  if (sh.gated()) REQ(dw_up);
  else OPT(dw_up);
  REQ(dw_down);
  OPT(ds);
  REQ(ws);
  const int kind = dh ? WS_EXPERT_BWD_LEAN : (y_swi || a_prime) ? WS_EXPERT_BWD : WS_EXPERT_BWD_H;
  const ExpertWs w = expert_ws(sh, kind, ws);
  if (ws_bytes < w.bytes) return MOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  rc = hip_status(launch_prep(sh, w, offsets, topk_ids, topk_w, token_index_map, true, ERR_BWD, st));
  if (rc) return rc;
  return hip_status(launch_backward(sh, dout, x, wg, w_gate, w_up, w_down, topk_ids, topk_w, offsets,
                                    expert_token_indices, token_index_map, h_ab, y_swi, a_prime, dh, dx, dwg,
                                    dw_gate, dw_up, dw_down, ds, w, g_spin_limit.load(std::memory_order_relaxed),
                                    st));
}

int moe_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  const int prev = g_timing ? 1 : 0;
  g_timing = on != 0;
  return prev;
}

int moe_timing_read(const char** names, float* ms, int cap) {
  std::lock_guard<std::mutex> lk(g_tmu);
  int n = 0;
  for (auto& r : g_recs) {
    if (r.b && r.e) {
      hipEventSynchronize(r.e);
      if (n < cap) {
        float t = 0.0f;
        hipEventElapsedTime(&t, r.b, r.e);
        if (names) names[n] = r.name;
        if (ms) ms[n] = t;
        ++n;
      }
    }
    if (r.b) g_pool.push_back(r.b);
    if (r.e) g_pool.push_back(r.e);
  }
  g_recs.clear();
  return n;
}

}  // extern "C"
