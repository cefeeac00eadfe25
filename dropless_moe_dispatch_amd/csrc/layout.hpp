// Workspace layouts and launch-side declarations shared by the C-ABI and the
// kernel translation units.  Every size depends on the shape only, never on
// the routing, so a workspace sized once serves any routing of that shape.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Expert GEMM tiles are 128 or 256 rows/columns (chosen per kernel and shape
// on the host); per-call state is sized for the finer 128 blocking.
constexpr int TILE_S = 128;
constexpr int TILE_L = 256;
constexpr int IDX_CHUNK = 256;      // tokens per index-build workgroup
constexpr int IDX_WAVES = IDX_CHUNK / 64;
constexpr int N_COUNTERS = 64;      // [0], [1] error words, [8..16) fold queue heads, others reserved
// Error words of the two calls with an ordered fold, so that one workspace
// may serve both: moe_combine sets counters[ERR_COMBINE], moe_expert_bwd
// counters[ERR_BWD] when a bounded wait runs out; each call clears only its own.
constexpr int ERR_COMBINE = 0, ERR_BWD = 1, N_ERR_WORDS = 2;

enum { ACT_SWIGLU = 0, ACT_SILU = 1, ACT_RELU = 2 };

struct Shape {
  int T, d, E, K, h, bf16;
  int act;  // ACT_*: SwiGLU (gated) or a plain two-layer expert
  long long A() const { return (long long)T * K; }
  int elem() const { return bf16 ? 2 : 4; }
  bool gated() const { return act == ACT_SWIGLU; }
  int hw() const { return gated() ? 2 * h : h; }  // columns of the saved pre-activations and of dH
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
// Address `off` bytes into a workspace based at p, in integer arithmetic:
// sizing a workspace carves it from a null base, where pointer arithmetic
// would be undefined.
inline void* ws_at(void* p, size_t off) { return (void*)((uintptr_t)p + off); }
// column blocks of width bn covering n columns (the last may be partial)
__host__ __device__ inline int col_blocks(int n, int bn) { return (n + bn - 1) / bn; }

// Upper bound on the number of bm-row blocks over all experts.
inline long long max_row_blocks(const Shape& s, int bm) {
  return (s.A() + (long long)s.E * (bm - 1)) / bm;
}

// ---- index workspace ------------------------------------------------------
struct IndexWs {
  uint64_t* masks;     // [nchunks][IDX_WAVES][E] token bitmaps per (chunk, wave, expert)
  int32_t* base;       // [E][nchunks] counts, scanned in place to bases inside each expert
  int32_t* tot;        // [E] tokens per expert
  size_t bytes;
  int nchunks;
};
inline IndexWs index_ws(const Shape& s, void* p) {
  IndexWs w{};
  w.nchunks = (s.T + IDX_CHUNK - 1) / IDX_CHUNK;
  size_t off = 0;
  w.masks = (uint64_t*)ws_at(p, off);
  off = align_up(off + (size_t)w.nchunks * IDX_WAVES * s.E * 8, 256);
  w.base = (int32_t*)ws_at(p, off);
  off = align_up(off + (size_t)s.E * w.nchunks * 4, 256);
  w.tot = (int32_t*)ws_at(p, off);
  off = align_up(off + (size_t)s.E * 4, 256);
  w.bytes = off;
  return w;
}

// ---- dense-map index workspace (the literal three-step backend) -----------
struct DenseIndexWs {
  int32_t* d5;         // [E][T] token id or -1
  int32_t* loc;        // [E][T] position in expert_token_indices (where d5 >= 0)
  int32_t* lengths;    // [E]
  size_t bytes;
};
inline DenseIndexWs dense_index_ws(const Shape& s, void* p) {
  DenseIndexWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { void* q = ws_at(p, off); off = align_up(off + bytes, 256); return q; };
  w.d5 = (int32_t*)take((size_t)s.E * s.T * 4);
  w.loc = (int32_t*)take((size_t)s.E * s.T * 4);
  w.lengths = (int32_t*)take((size_t)s.E * 4);
  w.bytes = off;
  return w;
}

// Split of a dW GEMM's K (an expert's rows) into chunks when its 256 x 256
// tiles alone cannot fill the chip: each chunk writes an fp32 partial and a
// second pass sums the partials in chunk order.  m x n is the per-expert
// output; the split depends on the shape only (average rows per expert), so
// the workspace does too, and every chunk keeps 512 rows on average.
inline int dw_split(const Shape& s, int m, int n) {
  const long long tiles = (long long)s.E * col_blocks(m, TILE_L) * col_blocks(n, TILE_L);
  const long long rows = s.A() / s.E;
  int k = 1;
  while (k < 8 && tiles * (2 * k) <= 512 && rows >= 512LL * (2 * k)) k *= 2;
  return k;
}
inline int dw_down_split(const Shape& s) { return dw_split(s, s.d, s.h); }
inline int dw_gate_up_split(const Shape& s) { return dw_split(s, s.hw(), s.d); }

// ---- per-call expert workspace (tile map, per-position data, fold state) --
// dWg on MFMA (bf16): the tokens are cut into dwg_chunks(s) chunks of
// dwg_chunk_tokens(s) (a multiple of 64) so that the grid of (128-column
// block, expert block of dwg_expert_tile(s), chunk) workgroups has about 512 of them, and a
// chunk's rows of x stay under 1 GiB (32-bit buffer offsets).  Shape only:
// the partial buffer never depends on the routing.
inline int dwg_expert_tile(const Shape& s) { return s.E <= 32 ? 32 : s.E <= 64 ? 64 : 128; }
inline int dwg_chunk_tokens(const Shape& s) {
  const int bm = dwg_expert_tile(s);
  const long long tiles = (long long)col_blocks(s.d, 128) * ((s.E + bm - 1) / bm);
  const long long ktiles = (s.T + 63) / 64;
  long long want = (512 + tiles - 1) / tiles;
  if (want > ktiles) want = ktiles;
  if (want < 1) want = 1;
  long long per = (ktiles + want - 1) / want;  // k-tiles per chunk
  const long long cap = (1LL << 23) / s.d;     // 64 tokens * d * 2 bytes * cap <= 2^30
  if (per > cap) per = cap > 0 ? cap : 1;
  return (int)(per * 64);
}
inline int dwg_chunks(const Shape& s) { return (s.T + dwg_chunk_tokens(s) - 1) / dwg_chunk_tokens(s); }

struct ExpertWs {
  int32_t* counters;   // [N_COUNTERS]
  int32_t* mb_off;     // [2][E+1] exclusive prefix of ceil(count_e / bm), bm = 128 then 256
  float* w_pos;        // [A] combine weight of the assignment at each position
  int32_t* rank_pos;   // [A] rank of the position's expert among its token's experts
  int32_t* turn;       // [T][d/128] ordered-fold turn counters
  float* acc;          // [T][d] fp32 fold accumulator
  float* ds_part;      // [A][h/128] router-score partial sums (backward)
  float* dz_pos;       // [A] router logit gradient per position (backward)
  float* dz_tok;       // [A] the same per (token, slot), token-major (backward)
  float* dwg_part;     // dWg partial sums (backward): bf16 [token chunks][E][d], fp32 [row blocks of 128][d]
  float* dw_part;      // [split][E][m][n] dW chunk partials when a dW GEMM splits its rows (backward)
  void* dh;            // [A][hw] activation-dtype gradient of the pre-activations (backward,
                       // unless the caller passes a buffer for it)
  void* a_prime;       // [A][h] activation-dtype A' = w * y recomputed from a, b (H-only backward,
                       // unless the caller passes a buffer for it)
  void* ystage;        // [A][d] activation-dtype staged expert outputs (staged-Y combine ablation)
  size_t bytes;
  int E;
  const int32_t* tile_map(int bm) const { return mb_off + (bm == TILE_L ? E + 1 : 0); }
};
enum { WS_EXPERT_FWD = 1, WS_COMBINE = 2, WS_EXPERT_BWD = 3, WS_EXPERT_BWD_H = 4, WS_COMBINE_STAGED = 5,
       WS_EXPERT_BWD_LEAN = 7 };

inline ExpertWs expert_ws(const Shape& s, int which, void* p) {
  ExpertWs w{};
  w.E = s.E;
  const size_t A = (size_t)s.A();
  size_t off = 0;
  auto take = [&](size_t bytes) { void* q = ws_at(p, off); off = align_up(off + bytes, 256); return q; };
  w.counters = (int32_t*)take(N_COUNTERS * 4);
  w.mb_off = (int32_t*)take((size_t)2 * (s.E + 1) * 4);
  const bool bwd = which == WS_EXPERT_BWD || which == WS_EXPERT_BWD_H || which == WS_EXPERT_BWD_LEAN;
  if (which == WS_COMBINE || bwd) {
    w.w_pos = (float*)take(A * 4);
    w.rank_pos = (int32_t*)take(A * 4);
    w.turn = (int32_t*)take((size_t)s.T * col_blocks(s.d, TILE_S) * 4);
    w.acc = (float*)take((size_t)s.T * s.d * 4);
  }
  if (bwd) {
    w.ds_part = (float*)take(A * col_blocks(s.h, TILE_S) * 4);
    w.dz_pos = (float*)take(A * 4);
    w.dz_tok = (float*)take(A * 4);
    w.dwg_part = (float*)take(s.bf16 ? (size_t)dwg_chunks(s) * s.E * s.d * 4
                                     : (size_t)max_row_blocks(s, TILE_S) * s.d * 4);
    const int sd = dw_down_split(s), sg = dw_gate_up_split(s);
    const size_t pd = sd > 1 ? (size_t)sd * s.E * s.d * s.h : 0;
    const size_t pg = sg > 1 ? (size_t)sg * s.E * s.hw() * s.d : 0;
    if (pd || pg) w.dw_part = (float*)take((pd > pg ? pd : pg) * 4);
    if (which != WS_EXPERT_BWD_LEAN) w.dh = take(A * (size_t)s.hw() * s.elem());  // the last item: LEAN is a prefix
  }
  if (which == WS_EXPERT_BWD_H) w.a_prime = take(A * (size_t)s.h * s.elem());
  if (which == WS_COMBINE_STAGED) w.ystage = take(A * (size_t)s.d * s.elem());
  w.bytes = off;
  return w;
}

// ---- kernel launchers (defined in the kernel translation units) -----------
hipError_t launch_router_logits(const Shape& s, const void* x, const void* wg, const float* bias, float* logits,
                                int32_t* ids, float* w, hipStream_t st);
bool router_logits_has_topk(const Shape& s);  // the logits kernel also writes ids and w
hipError_t launch_topk(const Shape& s, const float* logits, int32_t* ids, float* w, hipStream_t st);
bool route_fused_applies(const Shape& s);
hipError_t launch_route_fused(const Shape& s, const void* x, const void* wg, const float* bias, float* logits,
                              int32_t* ids, float* w, hipStream_t st);
hipError_t launch_build_index(const Shape& s, const int32_t* ids, int32_t* offsets, int32_t* eti, int32_t* tim,
                              const IndexWs& ws, hipStream_t st);
hipError_t launch_build_index_dense(const Shape& s, const int32_t* ids, int32_t* offsets, int32_t* eti, int32_t* tim,
                                    const DenseIndexWs& ws, hipStream_t st);
hipError_t launch_prep(const Shape& s, const ExpertWs& ws, const int32_t* offsets, const int32_t* ids,
                       const float* topk_w, const int32_t* tim, bool per_position, int own_err, hipStream_t st);
hipError_t launch_gate_up(const Shape& s, const void* x, const int32_t* offsets, const int32_t* eti,
                          const void* w_gate, const void* w_up, void* h_ab, void* y_swi, const ExpertWs& ws,
                          hipStream_t st);
hipError_t launch_down_combine(const Shape& s, const void* y_swi, const void* w_down, const int32_t* offsets,
                               const int32_t* eti, void* out, const ExpertWs& ws, int spin_limit, hipStream_t st);
hipError_t launch_combine_staged(const Shape& s, const void* y_swi, const void* w_down, const int32_t* offsets,
                                 const int32_t* tim, const float* topk_w, void* out, const ExpertWs& ws,
                                 hipStream_t st);
hipError_t launch_backward(const Shape& s, const void* dout, const void* x, const void* wg, const void* w_gate,
                           const void* w_up, const void* w_down, const int32_t* ids, const float* topk_w,
                           const int32_t* offsets, const int32_t* eti, const int32_t* tim, const void* h_ab,
                           const void* y_swi, void* a_prime, void* dh, void* dx, float* dwg, float* dw_gate,
                           float* dw_up, float* dw_down, float* ds, const ExpertWs& ws, int spin_limit,
                           hipStream_t st);

// Static index scratch of moe_build_index_noalloc (index.hip): its size, and
// the device address of the current device's copy (looked up once per device).
size_t index_scratch_bytes();
hipError_t index_scratch_ptr(void** out);

// Optional per-kernel timing hooks (set by the C-ABI timing calls).
void timing_mark(hipStream_t st, const char* name, bool begin);

}  // namespace moe
