// Host-side checks of the C ABI's validation and workspace carving, built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code
// (tests/test_host_sanitized.py builds and runs it; no GPU is touched).
//
// The ABI translation unit (csrc/api.hip) is linked against stand-ins for
// the kernel launchers defined here.  A stand-in records that it was reached
// and checks the workspace carving it receives: every region lies inside the
// workspace the caller passed -- a real heap allocation of exactly
// moe_workspace_bytes -- and is written at its first and last byte, so a
// region past the end is a heap-buffer-overflow under the sanitizer; regions
// do not overlap.  Invalid arguments must come back with their status before
// any launcher is reached.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../dropless_moe_dispatch_amd/csrc/layout.hpp"
#include "../include/moe_dispatch.h"

namespace {
int g_fail = 0;
int g_launches = 0;
const char* g_case = "";
char* g_ws = nullptr;
size_t g_ws_bytes = 0;

#define CHECK(c)                                                            \
  do {                                                                      \
    if (!(c)) {                                                             \
      fprintf(stderr, "FAIL [%s] line %d: %s\n", g_case, __LINE__, #c);     \
      ++g_fail;                                                             \
    }                                                                       \
  } while (0)

struct Region {
  const void* p;
  size_t n;
};

// every region inside [g_ws, g_ws + g_ws_bytes), 16-byte aligned, disjoint;
// touch the first and last byte of each
void check_regions(std::vector<Region> rs) {
  for (size_t i = 0; i < rs.size(); ++i) {
    const char* p = (const char*)rs[i].p;
    if (rs[i].n == 0 || p == nullptr) continue;
    CHECK(p >= g_ws && p + rs[i].n <= g_ws + g_ws_bytes);
    CHECK(((uintptr_t)p & 15) == 0);
    char* q = const_cast<char*>(p);
    q[0] = 1;
    q[rs[i].n - 1] = 1;
    for (size_t j = 0; j < i; ++j) {
      const char* r = (const char*)rs[j].p;
      if (rs[j].n == 0 || r == nullptr) continue;
      CHECK(p + rs[i].n <= r || r + rs[j].n <= p);
    }
  }
}

long long row_blocks_bound(const moe::Shape& s, int bm) { return (s.A() + (long long)s.E * (bm - 1)) / bm; }

// the expert workspace's regions, from what each field holds
void check_expert_ws(const moe::Shape& s, const moe::ExpertWs& w) {
  const size_t A = (size_t)s.A(), eb = s.bf16 ? 2 : 4;
  std::vector<Region> rs = {{w.counters, 64 * 4}, {w.mb_off, 2 * (size_t)(s.E + 1) * 4}};
  if (w.w_pos) {
    rs.push_back({w.w_pos, A * 4});
    rs.push_back({w.rank_pos, A * 4});
    rs.push_back({w.turn, (size_t)s.T * ((s.d + 127) / 128) * 4});
    rs.push_back({w.acc, (size_t)s.T * s.d * 4});
  }
  if (w.ds_part) {  // a backward kind (the lean one has no dH buffer)
    rs.push_back({w.ds_part, A * ((s.h + 127) / 128) * 4});
    rs.push_back({w.dz_pos, A * 4});
    rs.push_back({w.dz_tok, A * 4});
    rs.push_back({w.dwg_part, s.bf16 ? (size_t)moe::dwg_chunks(s) * s.E * s.d * 4
                                     : (size_t)row_blocks_bound(s, 128) * s.d * 4});
    const size_t pd = moe::dw_down_split(s) > 1 ? (size_t)moe::dw_down_split(s) * s.E * s.d * s.h : 0;
    const size_t pg = moe::dw_gate_up_split(s) > 1 ? (size_t)moe::dw_gate_up_split(s) * s.E * s.hw() * s.d : 0;
    rs.push_back({w.dw_part, (pd > pg ? pd : pg) * 4});
    rs.push_back({w.dh, w.dh ? A * s.hw() * eb : 0});
  }
  rs.push_back({w.a_prime, w.a_prime ? A * s.h * eb : 0});
  rs.push_back({w.ystage, w.ystage ? A * s.d * eb : 0});
  check_regions(rs);
}
}  // namespace

// ---- stand-ins for the kernel launchers -----------------------------------
namespace moe {
hipError_t launch_router_logits(const Shape&, const void*, const void*, const float*, float*, int32_t*, float*,
                                hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
bool router_logits_has_topk(const Shape& s) { return s.E <= 128; }
hipError_t launch_topk(const Shape&, const float*, int32_t*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
bool route_fused_applies(const Shape&) { return false; }
hipError_t launch_route_fused(const Shape&, const void*, const void*, const float*, float*, int32_t*, float*,
                              hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_build_index(const Shape& s, const int32_t*, int32_t*, int32_t*, int32_t*, const IndexWs& w,
                              hipStream_t) {
  ++g_launches;
  check_regions({{w.masks, (size_t)w.nchunks * 4 * s.E * 8}, {w.base, (size_t)s.E * w.nchunks * 4},
                 {w.tot, (size_t)s.E * 4}});
  CHECK(w.nchunks == (s.T + 255) / 256);
  return hipSuccess;
}
// the no-alloc index's static scratch: a heap block of the same size here
size_t index_scratch_bytes() { return MOE_NOALLOC_INDEX_MAX_BYTES; }
hipError_t index_scratch_ptr(void** out) {
  static char* block = nullptr;
  if (!block) block = (char*)malloc(MOE_NOALLOC_INDEX_MAX_BYTES);
  g_ws = block;
  g_ws_bytes = MOE_NOALLOC_INDEX_MAX_BYTES;
  *out = block;
  return hipSuccess;
}
hipError_t launch_build_index_dense(const Shape& s, const int32_t*, int32_t*, int32_t*, int32_t*,
                                    const DenseIndexWs& w, hipStream_t) {
  ++g_launches;
  check_regions({{w.d5, (size_t)s.E * s.T * 4}, {w.loc, (size_t)s.E * s.T * 4}, {w.lengths, (size_t)s.E * 4}});
  return hipSuccess;
}
hipError_t launch_prep(const Shape& s, const ExpertWs& w, const int32_t*, const int32_t*, const float*,
                       const int32_t*, bool, int own_err, hipStream_t) {
  ++g_launches;
  CHECK(own_err >= -1 && own_err < N_ERR_WORDS);
  check_expert_ws(s, w);
  return hipSuccess;
}
hipError_t launch_gate_up(const Shape& s, const void*, const int32_t*, const int32_t*, const void*, const void*,
                          void*, void*, const ExpertWs& w, hipStream_t) {
  ++g_launches;
  check_expert_ws(s, w);
  return hipSuccess;
}
hipError_t launch_down_combine(const Shape& s, const void*, const void*, const int32_t*, const int32_t*, void*,
                               const ExpertWs& w, int spin, hipStream_t) {
  ++g_launches;
  CHECK(spin > 0);
  check_expert_ws(s, w);
  return hipSuccess;
}
hipError_t launch_combine_staged(const Shape& s, const void*, const void*, const int32_t*, const int32_t*,
                                 const float*, void*, const ExpertWs& w, hipStream_t) {
  ++g_launches;
  CHECK(w.ystage != nullptr);
  check_expert_ws(s, w);
  return hipSuccess;
}
hipError_t launch_backward(const Shape& s, const void*, const void*, const void*, const void*, const void*,
                           const void*, const int32_t*, const float*, const int32_t*, const int32_t*,
                           const int32_t*, const void*, const void* y_swi, void* a_prime, void* dh, void*, float*,
                           float*, float*, float*, float*, const ExpertWs& w, int spin, hipStream_t) {
  ++g_launches;
  CHECK(spin > 0);
  CHECK(!(y_swi && a_prime));
  CHECK(y_swi || a_prime || w.a_prime);  // H-only: A' has somewhere to go
  CHECK(dh || w.dh);                     // and so has dH
  check_expert_ws(s, w);
  return hipSuccess;
}
}  // namespace moe

// ---- the cases --------------------------------------------------------------
namespace {
void* const F = (void*)0x10000;  // aligned stand-in for a device pointer (never dereferenced)

moe_shape shape(int T, int d, int E, int K, int h, int dtype = MOE_BF16, int act = MOE_ACT_SWIGLU) {
  moe_shape s;
  s.T = T; s.d = d; s.E = E; s.K = K; s.h = h; s.dtype = dtype; s.act = act;
  return s;
}

// one call of every entry point with a workspace of exactly the reported size
void valid_calls(const moe_shape& s) {
  const int kinds[] = {MOE_WS_INDEX,          MOE_WS_EXPERT_FWD,  MOE_WS_COMBINE,        MOE_WS_EXPERT_BWD,
                       MOE_WS_EXPERT_BWD_H,   MOE_WS_COMBINE_STAGED, MOE_WS_INDEX_DENSE, MOE_WS_EXPERT_BWD_LEAN};
  const bool gated = s.act == MOE_ACT_SWIGLU;
  for (int kind : kinds) {
    const size_t n = moe_workspace_bytes(&s, kind);
    CHECK(n > 0);
    g_ws_bytes = n;
    g_ws = (char*)malloc(n);  // exactly n bytes: the sanitizer guards what lies past them
    CHECK(((uintptr_t)g_ws & 15) == 0);
    const int before = g_launches;
    int rc = 0;
    void* up = gated ? F : nullptr;
    switch (kind) {
      case MOE_WS_INDEX:
        rc = moe_build_index(&s, (int32_t*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, g_ws, n, nullptr);
        break;
      case MOE_WS_INDEX_DENSE:
        rc = moe_build_index_dense(&s, (int32_t*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, g_ws, n, nullptr);
        break;
      case MOE_WS_EXPERT_FWD:
        rc = moe_expert_fwd(&s, F, (int32_t*)F, (int32_t*)F, F, up, F, F, g_ws, n, nullptr);
        break;
      case MOE_WS_COMBINE:
        rc = moe_combine(&s, F, F, (int32_t*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, (float*)F, F, g_ws, n,
                         nullptr);
        break;
      case MOE_WS_COMBINE_STAGED:
        rc = moe_combine_staged(&s, F, F, (int32_t*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, (float*)F, F, g_ws, n,
                                nullptr);
        break;
      case MOE_WS_EXPERT_BWD:
      case MOE_WS_EXPERT_BWD_H: {
        const bool honly = kind == MOE_WS_EXPERT_BWD_H;
        rc = moe_expert_bwd(&s, F, F, F, F, up, F, (int32_t*)F, (float*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F,
                            (char*)F + 0x100, honly ? nullptr : F, nullptr, nullptr, F, (float*)F, (float*)F,
                            gated ? (float*)F : nullptr, (float*)F, nullptr, g_ws, n, nullptr);
        if (!honly) {  // H-only with a buffer of its own for A' fits the smaller workspace
          rc |= moe_expert_bwd(&s, F, F, F, F, up, F, (int32_t*)F, (float*)F, (int32_t*)F, (int32_t*)F,
                               (int32_t*)F, (char*)F + 0x100, nullptr, (char*)F + 0x200, nullptr, F, (float*)F,
                               (float*)F, gated ? (float*)F : nullptr, (float*)F, nullptr, g_ws, n, nullptr);
        }
        break;
      }
      case MOE_WS_EXPERT_BWD_LEAN: {
        // dH over the saved H, with a saved y and (H-only) with A' in a buffer of its own
        rc = moe_expert_bwd(&s, F, F, F, F, up, F, (int32_t*)F, (float*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F,
                            (char*)F + 0x100, F, nullptr, (char*)F + 0x100, F, (float*)F, (float*)F,
                            gated ? (float*)F : nullptr, (float*)F, nullptr, g_ws, n, nullptr);
        rc |= moe_expert_bwd(&s, F, F, F, F, up, F, (int32_t*)F, (float*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F,
                             (char*)F + 0x100, nullptr, (char*)F + 0x200, (char*)F + 0x100, F, (float*)F,
                             (float*)F, gated ? (float*)F : nullptr, (float*)F, nullptr, g_ws, n, nullptr);
        break;
      }
    }
    CHECK(rc == MOE_OK);
    CHECK(g_launches > before);
    // one byte short is refused before any launch
    const int mid = g_launches;
    if (kind == MOE_WS_INDEX)
      CHECK(moe_build_index(&s, (int32_t*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, g_ws, n - 1, nullptr) ==
            MOE_ERR_WORKSPACE);
    if (kind == MOE_WS_COMBINE)
      CHECK(moe_combine(&s, F, F, (int32_t*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, (float*)F, F, g_ws, n - 1,
                        nullptr) == MOE_ERR_WORKSPACE);
    CHECK(g_launches == mid);
    free(g_ws);
    g_ws = nullptr;
  }
  // the no-alloc index: within the static scratch, or refused before any launch
  {
    const int before = g_launches;
    const int rc = moe_build_index_noalloc(&s, (int32_t*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, nullptr);
    if (moe_workspace_bytes(&s, MOE_WS_INDEX) <= MOE_NOALLOC_INDEX_MAX_BYTES) {
      CHECK(rc == MOE_OK);
      CHECK(g_launches == before + 1);
    } else {
      CHECK(rc == MOE_ERR_WORKSPACE);
      CHECK(g_launches == before);
    }
    g_ws = nullptr;
  }
  // the shared-workspace rule: the backward's kind is the largest of the expert calls
  CHECK(moe_workspace_bytes(&s, MOE_WS_EXPERT_BWD) >= moe_workspace_bytes(&s, MOE_WS_COMBINE));
  CHECK(moe_workspace_bytes(&s, MOE_WS_EXPERT_BWD_LEAN) >= moe_workspace_bytes(&s, MOE_WS_COMBINE));
  CHECK(moe_workspace_bytes(&s, MOE_WS_EXPERT_BWD_LEAN) < moe_workspace_bytes(&s, MOE_WS_EXPERT_BWD));
  CHECK(moe_workspace_bytes(&s, MOE_WS_COMBINE) >= moe_workspace_bytes(&s, MOE_WS_EXPERT_FWD));
}

void invalid(const moe_shape& s, int code) {
  const int before = g_launches;
  static char ws[64];
  CHECK(moe_workspace_bytes(&s, MOE_WS_INDEX) == 0);
  CHECK(moe_route_topk(&s, F, F, nullptr, (float*)F, (int32_t*)F, (float*)F, nullptr) == code);
  CHECK(moe_build_index(&s, (int32_t*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, ws, (size_t)1 << 40, nullptr) ==
        code);
  CHECK(g_launches == before);
}
}  // namespace

int main() {
  // validation of shapes (the cases of tests/test_abi.py)
  struct { int T, d, E, K, h, dt, code; } bad[] = {
      {0, 128, 8, 2, 128, MOE_BF16, MOE_ERR_INVALID_ARG},
      {16, 128, 4, 5, 128, MOE_BF16, MOE_ERR_INVALID_ARG},
      {16, 128, 2000, 2, 128, MOE_BF16, MOE_ERR_UNSUPPORTED},
      {16, 128, 64, 40, 128, MOE_BF16, MOE_ERR_UNSUPPORTED},
      {16, 96, 8, 2, 128, MOE_BF16, MOE_ERR_UNSUPPORTED},
      {16, 128, 8, 2, 200, MOE_F32, MOE_ERR_UNSUPPORTED},
      {1 << 29, 128, 8, 8, 128, MOE_BF16, MOE_ERR_INVALID_ARG},
      {1 << 20, 1024, 8, 2, 128, MOE_BF16, MOE_ERR_UNSUPPORTED},
      {1 << 19, 1024, 8, 2, 128, MOE_F32, MOE_ERR_UNSUPPORTED},
      {64, 8192, 8, 2, 131072, MOE_BF16, MOE_ERR_UNSUPPORTED},
      {1 << 18, 128, 8, 2, 2048, MOE_BF16, MOE_ERR_UNSUPPORTED},
      {0x7fffffff, 0x7fffff80, 1024, 32, 0x7fffff80, MOE_BF16, MOE_ERR_INVALID_ARG},  // products past 64 bits
      {16, -128, 8, 2, 128, MOE_BF16, MOE_ERR_INVALID_ARG},
      {16, 128, 8, 2, 128, 7, MOE_ERR_INVALID_ARG},  // dtype
  };
  for (auto& b : bad) {
    g_case = "invalid shape";
    invalid(shape(b.T, b.d, b.E, b.K, b.h, b.dt), b.code);
  }
  {
    g_case = "bad act";
    moe_shape s = shape(64, 128, 8, 2, 128);
    s.act = 7;
    invalid(s, MOE_ERR_INVALID_ARG);
    CHECK(moe_workspace_bytes(nullptr, MOE_WS_INDEX) == 0);
    CHECK(moe_build_index(nullptr, (int32_t*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, F, 1, nullptr) ==
          MOE_ERR_INVALID_ARG);
  }
  {
    // pointer validation: null, misaligned, ambiguous H-only arguments
    g_case = "pointers";
    moe_shape s = shape(64, 128, 8, 2, 128);
    const int before = g_launches;
    CHECK(moe_route_topk(&s, F, F, nullptr, nullptr, (int32_t*)F, (float*)F, nullptr) == MOE_ERR_INVALID_ARG);
    CHECK(moe_build_index(&s, (int32_t*)((char*)F + 4), (int32_t*)F, (int32_t*)F, (int32_t*)F, F, 1 << 30,
                          nullptr) == MOE_ERR_INVALID_ARG);
    const size_t n = moe_workspace_bytes(&s, MOE_WS_EXPERT_BWD);
    CHECK(moe_expert_bwd(&s, F, F, F, F, F, F, (int32_t*)F, (float*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, F,
                         F, F, nullptr, F, (float*)F, (float*)F, (float*)F, (float*)F, nullptr, F, n,
                         nullptr) == MOE_ERR_INVALID_ARG);  // y_swi and a_prime both given
    CHECK(moe_expert_bwd(&s, F, F, F, F, F, F, (int32_t*)F, (float*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, F,
                         nullptr, F, nullptr, F, (float*)F, (float*)F, (float*)F, (float*)F, nullptr, F, n,
                         nullptr) == MOE_ERR_INVALID_ARG);  // A' over h_ab
    CHECK(moe_expert_bwd(&s, F, F, F, F, F, F, (int32_t*)F, (float*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, F,
                         nullptr, nullptr, (char*)F + 0x100, F, (float*)F, (float*)F, (float*)F, (float*)F, nullptr,
                         F, n, nullptr) == MOE_ERR_INVALID_ARG);  // dH given, H-only, no A' buffer
    CHECK(moe_expert_bwd(&s, F, F, F, F, F, F, (int32_t*)F, (float*)F, (int32_t*)F, (int32_t*)F, (int32_t*)F, F,
                         (char*)F + 0x100, nullptr, (char*)F + 0x100, F, (float*)F, (float*)F, (float*)F, (float*)F,
                         nullptr, F, n, nullptr) == MOE_ERR_INVALID_ARG);  // dH over y_swi
    CHECK(g_launches == before);
    CHECK(moe_set_spin_limit(0) > 0);
  }
  // carving over a grid of shapes (every kind, both dtypes and expert kinds)
  const int Ts[] = {1, 255, 300, 1000};
  const int ds[] = {128, 256, 1024};
  const int Es[] = {1, 8, 130, 1024};
  const int Ks[] = {1, 2, 8, 32};
  const int hs[] = {128, 384};
  for (int T : Ts)
    for (int d : ds)
      for (int E : Es)
        for (int K : Ks)
          for (int h : hs)
            for (int dt = 0; dt < 2; ++dt)
              for (int act = 0; act < 2; ++act) {
                if (K > E) continue;
                g_case = "carving";
                valid_calls(shape(T, d, E, K, h, dt, act));
              }
  {
    g_case = "no-alloc index limit";  // 0.14 * T * E bytes against the static scratch
    valid_calls(shape(32768, 128, 1024, 8, 128));
    valid_calls(shape(65536, 128, 1024, 8, 128));
  }
  {
    g_case = "dW row split";  // few experts, many rows: the dW GEMMs split their rows
    valid_calls(shape(8192, 256, 2, 2, 256));
    valid_calls(shape(8192, 128, 2, 2, 128, MOE_F32));
  }
  if (g_fail) {
    fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  printf("abi host checks ok (%d launcher calls)\n", g_launches);
  return 0;
}
