// Expert GEMMs of the dropless MoE layer: forward gate/up with the SwiGLU
// epilogue, the down projection with the ordered weighted combine, and the
// backward kernels.  All are grouped GEMMs over the expert-sorted position
// space p in [0, T*K) defined by expert_token_offsets; token rows are read in
// place through expert_token_indices (no permuted copy of x or dY).
//
//  forward (MoEBlaze analysis page, "Memory-Efficient Token Routing: Forward
//  Pass" and "Fused SwiGLU Kernel with Activation Checkpoint"; MoEBlaze
//  reading notes sec. 5.2 Algorithm 1):
//    a = x W_gate^T, b = x W_up^T        (one kernel, x loaded once)
//    y = SiLU(a) * b                     (epilogue, from the fp32 a, b)
//    store a, b, y  (Algorithm 1 keeps A, B and Y_swi for the backward)
//    out[t] = sum_k w_{t,k} y_{p(t,k)} W_down^T    (owner-ordered combine)
//  backward (same pages, "Backward Pass" and Algorithm 1 backward; SonicMoE
//  analysis page sec. 3.4.1 for dS = <dA', y>, dA = s * dA', dW2 = A'^T dO):
//    dA' = dO W_down;  dS = <dA', y>;  dy = w dA'
//    sigma, SiLU recomputed from the stored a:  da = dy b SiLU'(a), db = dy SiLU(a)
//    dW_down[e] = sum_p dO_p^T (w_p y_p);  dW_gate/up[e] = sum_p da/db_p^T x_p
//    dX[t] = sum_k (da W_gate + db W_up)_{p(t,k)} + router term
#include <stdlib.h>

#include <type_traits>

#include "gemm.hpp"
#include "layout.hpp"

namespace moe {

// A 128 x 128 fp32 tile parked in LDS for an epilogue uses rows of FOLD_LD floats
// (128 + 8: the rows written by the two half-waves land on disjoint banks).
constexpr int FOLD_LD = 136;  // floats per parked row (128 + 8: the two half-waves' rows land on disjoint banks)

// Park rows [r0, r0 + PR) of an accumulator tile in LDS, rows of PITCH floats
// holding tile columns 0 .. BN-1: the waves whose fragments fall in the range
// write them (fragments are 32-row aligned, so the test is per wave and
// fragment).  PITCH = BN + 8 puts the two half-waves' rows on disjoint banks.
template <class C, int PR, int PITCH>
MOE_DEV void park_rows(const f32x16_t (&acc)[C::FM][C::FN], float* s_c, int r0, int wm, int wn) {
  const int l = lane_id();
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int row0 = C::a_row0(wm, fm) - r0;
    if (row0 < 0 || row0 >= PR) continue;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) s_c[(row0 + frag_row(r, l)) * PITCH + C::b_row0(wn, fn) + frag_col(l)] = acc[fm][fn][r];
  }
}

template <typename T> MOE_DEV float ld_f(const T* p) { return ElemT<T>::load(p); }
template <typename T> MOE_DEV void st_f(T* p, float v) { ElemT<T>::store(p, v); }

// The host picks a tile per kernel and shape (see XCfg below).
template <typename TIN, int B> using GCfg = Cfg<TIN, B, B, 2, 2>;
// Operands whose source is k-major (weights read as [k][n], activations
// reduced over rows) are staged k-major and read with the LDS transpose in
// bf16; fp32 operands are transposed in registers (KRowLoader).
template <typename TIN> constexpr bool kTr = sizeof(TIN) == 2;
// Tile configurations (BM rows x BN columns).  128 x 128: four waves of
// 64 x 64, two workgroups per CU.  128 x 256 (bf16): eight waves of 64 x 64,
// one workgroup per CU and two waves per SIMD, a quarter less operand traffic
// per MFMA than 128 x 128 with the same row padding.  256 x 256 in bf16:
// eight waves of 64 x 128, one workgroup per CU and two waves per SIMD (half
// the operand traffic per MFMA of the small tile, with a second wave per SIMD
// to cover latencies); in fp32 four waves of 128 x 128.  AK / BK: operand
// staged k-major (bf16 only).
template <typename TIN, int BM, int BN, bool PAIRED, bool AK, bool BK>
using XCfg = Cfg<TIN, BM, BN, (BM == TILE_L && kTr<TIN>) ? 4 : 2, (BM == TILE_S && BN == TILE_L) ? 4 : 2, PAIRED,
                 AK && kTr<TIN>, BK && kTr<TIN>>;
template <typename TIN, int BM, int BN, bool AK, bool BK> using KCfg = XCfg<TIN, BM, BN, false, AK, BK>;
// LDS of an expert kernel: its two operand stages, or its parked epilogue
// rows where those take more (the 128 x 256 tile parks two 128 x 128 fp32
// halves plus the fold's per-row token, weight and rank).
template <class C> constexpr int smem_bytes() {
  constexpr int park = C::BN > 128 && C::BM == 128 ? 2 * 128 * FOLD_LD * 4 + 3 * 128 * 4 : 0;
  return C::LDS_BYTES > park ? C::LDS_BYTES : park;
}
template <class C, bool KM, int ROWS, class Src, bool SCALED>
struct KSrcSel {
  static_assert(KM || C::NT == NTHREADS, "the register transpose assumes four waves");
  using type = std::conditional_t<KM, KLoader<ROWS, Src, SCALED, C::NT>, KRowLoader<typename C::T, ROWS, Src, SCALED>>;
};
template <class C, bool KM, int ROWS, class Src, bool SCALED>
using KSrcLoader = typename KSrcSel<C, KM, ROWS, Src, SCALED>::type;

// MOE_DISPATCH_TILE=128|256 forces one tile for every expert GEMM (tuning aid).
static int forced_tile() {
  static int v = [] {
    const char* e = getenv("MOE_DISPATCH_TILE");
    if (!e) return 0;
    const int t = atoi(e);
    return (t == TILE_S || t == TILE_L) ? t : 0;
  }();
  return v;
}
// Tile order of the varlen-M kernels (gate/up, plain-expert forward, dH,
// staged down projection): groups of R = 8 row blocks (grouped_tile), and
// over each group an XCD grid (tile_of): workgroups go to the eight XCDs in
// turn, so in launch order all XCDs work on the same group -- one expert's
// weights and rows, which the memory-side cache then serves to all of them --
// and each XCD takes a 2-D part of it (xg row residues x 8/xg column residues)
// for reuse in its own L2.  The host takes xg = 2, else 4, else 8, the first
// that divides the group.  Measured on MI355X at T=32768, d=6144, E=64, K=4,
// h=2048: gate/up 7.47 -> 6.81 ms and dH 4.12 -> 3.78 ms against the earlier
// order (each XCD a contiguous range of groups, one expert per XCD at a
// time); xg = 4 and 8 land within 1% of xg = 2.
// Tuning switches, read once per process:
//   MOE_DISPATCH_GROUP_ROWS=R (1..64), MOE_DISPATCH_GROUP_XCD=1|2|4|8 forces
//   xg, MOE_DISPATCH_GROUP_XCD=0 turns the grid off and runs the earlier
//   orders: contiguous XCD ranges (MOE_DISPATCH_XCD_SWIZZLE=1, default) or
//   launch order (=0), with groups inside each expert
//   (MOE_DISPATCH_EXPERT_GROUPS=1, default) or over the global row blocks (=0).
static int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  return e ? atoi(e) : dflt;
}
struct TileOrder {
  int nblk;  // block count for the XCD swizzle (0: launch order)
  int grp;   // group rows: > 0 global groups, < 0 groups inside each expert
  int xg;    // XCD grid rows over a group (0: none)
};
static TileOrder tile_order(long long nblk, int nbn) {
  static const int R = [] {
    const int r = env_int("MOE_DISPATCH_GROUP_ROWS", 8);
    return r >= 1 && r <= 64 ? r : 8;
  }();
  static const int force_xg = env_int("MOE_DISPATCH_GROUP_XCD", -1);
  static const bool swizzle = env_int("MOE_DISPATCH_XCD_SWIZZLE", 1) != 0;
  static const bool expert_groups = env_int("MOE_DISPATCH_EXPERT_GROUPS", 1) != 0;
  int xg = 0;
  if (force_xg == 1 || force_xg == 2 || force_xg == 4 || force_xg == 8) {
    xg = force_xg;
  } else if (force_xg != 0) {
    for (int c : {2, 4, 8})
      if (R % c == 0 && nbn % (8 / c) == 0) {
        xg = c;
        break;
      }
  }
  if (xg) return {0, R, xg};
  return {swizzle ? (int)nblk : 0, expert_groups ? -R : R, 0};
}
static bool pick_large(bool auto_choice) {
  const int f = forced_tile();
  return f ? f == TILE_L : auto_choice;
}
// 128 x 256 (bf16) where the 256 x 256 tile is not taken.  MOE_DISPATCH_MID=0|1
// forces it off or on (tuning aid; MOE_DISPATCH_TILE takes precedence).
static bool pick_mid(const Shape& s, bool auto_choice) {
  static int v = [] {
    const char* e = getenv("MOE_DISPATCH_MID");
    return e ? (atoi(e) ? 1 : 0) : -1;
  }();
  if (!s.bf16 || forced_tile()) return false;
  return v >= 0 ? v == 1 : auto_choice;
}
// The folds can run the 256 x 256 tile in bf16 when d is a multiple of 256:
// its eight waves park their accumulators in LDS and four of them fold the two
// 128-column halves side by side.  It pays where each tile's reduction (kdim)
// is long next to the fold.  Measured on MI355X against the 128 x 256 tile:
// dX fold 7.4% faster at d = 6144, kdim = 4096, 3% at d = 4096, kdim = 3072,
// and faster at d = 1024-2048 with kdim = 4096-8192 too (MoEBlaze's conf3
// and conf4), but 15% slower at d = 2048, kdim = 1536.  Down-combine (its
// main loop loading a whole iteration ahead): 4.32 -> 4.22 ms at d = 6144,
// kdim = 2048, 2-4% faster at d = 1024-2048, kdim = 4096-8192 with 4096 or
// more tiles and at d = 4096, kdim = 14336 (512 tiles), but 4-8% slower with
// 512-1024 tiles at kdim = 2048-8192 and level at d = 4096, kdim = 1536.
// dx: the dX fold (else down-combine).
static bool wide_fold(const Shape& s, int kdim, bool dx) {
  static const int force = env_int("MOE_DISPATCH_WIDE_FOLD", -1);  // tuning aid: 1 on, 0 off
  const long long tiles = s.A() / TILE_L * (s.d / TILE_L);
  const bool auto_choice = force >= 0 ? force == 1
                           : dx      ? kdim >= 3072
                                     : (kdim >= 3072 && s.d >= 4096) || (kdim >= 2048 && tiles >= 4096);
  return s.bf16 && s.d % TILE_L == 0 && pick_large(auto_choice);
}
// Otherwise the folds take the 128 x 256 tile where d is a multiple of 256
// (it folds its two 128-column halves against their own turn columns).
// Measured on MI355X against 128 x 128: down-combine 3-6% faster on the
// fine-grained and large-d workloads and MoEBlaze's conf3 and conf4 (level on
// the skewed one); dX fold 1.5-3% faster on fine-grained, large-d and conf4,
// 0.5-1.7% slower on skewed and conf3.  The gate/up and dH kernels measured
// 2-14% slower on it and keep 128 x 128 (dH except for a long reduction,
// see the backward).
static bool mid_fold(const Shape& s, int kdim, bool dx) {
  return !wide_fold(s, kdim, dx) && s.d % TILE_L == 0 && pick_mid(s, true);
}

// ===========================================================================
// Forward gate/up: M = rows of expert e, N = 128 gate + 128 up columns, K = d.
// ===========================================================================
template <class C>
__global__ __launch_bounds__(C::NT, C::WAVES_PER_EU) void gate_up_kernel(
    const typename C::T* __restrict__ x, const int32_t* __restrict__ offsets, const int32_t* __restrict__ eti,
    const int32_t* __restrict__ mb_off, const typename C::T* __restrict__ w_gate,
    const typename C::T* __restrict__ w_up, typename C::T* __restrict__ h_ab, typename C::T* __restrict__ y_swi,
    int T, int d, int E, int h, int nbn, int nblk, int grp, int xg) {
  __shared__ __attribute__((aligned(16))) char smem[smem_bytes<C>()];
  using TIN = typename C::T;
  constexpr int HB = C::BN / 2;     // gate (= up) columns per tile
  constexpr int HF = C::FN / 2;     // gate fragments per wave
  int g, nb;
  if (!tile_of(xcd_swizzle(blockIdx.x, nblk), mb_off, E, nbn, grp, xg, g, nb)) return;
  const RowTile rt = decode_row_tile<C::BM>(mb_off, offsets, E, g);
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  const uint32_t ldx = (uint32_t)d * sizeof(TIN);
  const int j0 = nb * HB;  // first gate/up column of this tile
  using LA = RowLoader<C::BM, false, C::NT>;
  using LB = RowLoader<C::BN, true, C::NT>;  // rows [0,HB) gate, [HB,BN) up
  LA la;
  LB lb;
  la.rs[0] = make_rsrc(x, (size_t)T * ldx);
#pragma unroll
  for (int i = 0; i < LA::CPT; ++i) {
    const int p = rt.r0 + LA::my_row(i);
    la.roff[i] = p < rt.r1 ? (uint32_t)eti[p] * ldx : OOB_OFF;
  }
  lb.rs[0] = make_rsrc(w_gate + (size_t)rt.e * h * d, (size_t)h * ldx);
  lb.rs[1] = make_rsrc(w_up + (size_t)rt.e * h * d, (size_t)h * ldx);
#pragma unroll
  for (int i = 0; i < LB::CPT; ++i) {
    const int j = j0 + (LB::my_row(i) % HB);
    lb.roff[i] = j < h ? (uint32_t)j * ldx : OOB_OFF;
  }
  f32x16_t acc[C::FM][C::FN];
  gemm_mainloop<C>(la, lb, d / C::BK, smem, acc, wm, wn);
  {
    // park the tile (gate columns in [0, HB), up columns in [HB, BN)) in LDS,
    // 128 rows at a time, then write a, b and y as whole 16-byte row chunks
    constexpr int PR = 128, PITCH = C::BN + 8;
    static_assert(PR * PITCH * 4 <= smem_bytes<C>(), "the parked rows fit the LDS");
    float* s_c = (float*)smem;
    constexpr int VPC = 16 / sizeof(TIN);
    constexpr int CPR = HB / VPC;           // output chunks per row (per half)
#pragma unroll 1
    for (int r0 = 0; r0 < C::BM; r0 += PR) {
      __syncthreads();  // the LDS stages (first pass) or the previous rows are reused
      park_rows<C, PR, PITCH>(acc, s_c, r0, wm, wn);
      __syncthreads();
      const int left = rt.r1 - rt.r0 - r0;
      const int rows = left < PR ? left : PR;
      for (int c = threadIdx.x; c < PR * CPR; c += C::NT) {
        const int row = c / CPR, cc = c % CPR;
        if (row >= rows) break;
        const int p = rt.r0 + r0 + row;
        const float* ar = s_c + row * PITCH + cc * VPC;
        float a[VPC], b[VPC], y[VPC];
#pragma unroll
        for (int v = 0; v < VPC; ++v) {
          a[v] = ar[v];
          b[v] = ar[HB + v];
          y[v] = a[v] * sigmoidf_(a[v]) * b[v];
        }
        const int j = j0 + cc * VPC;         // h is a multiple of the half tile: in range
        if (h_ab) {  // NULL: a forward that saves nothing for a backward
          st16(h_ab + (size_t)p * 2 * h + j, a);
          st16(h_ab + (size_t)p * 2 * h + h + j, b);
        }
        st16(y_swi + (size_t)p * h + j, y);
      }
    }
  }
}

template <typename TIN, int BM, int BN>
static hipError_t gate_up_t(const Shape& s, const void* x, const int32_t* offsets, const int32_t* eti,
                            const void* w_gate, const void* w_up, void* h_ab, void* y_swi, const ExpertWs& ws,
                            hipStream_t st) {
  using C = XCfg<TIN, BM, BN, true, false, false>;
  const int nbn = col_blocks(s.h, C::BN / 2);
  long long nblk = max_row_blocks(s, BM) * nbn;
  nblk = (nblk + 7) / 8 * 8;
  const TileOrder to = tile_order(nblk, nbn);
  gate_up_kernel<C><<<dim3((unsigned)nblk), dim3(C::NT), 0, st>>>(
      (const TIN*)x, offsets, eti, ws.tile_map(BM), (const TIN*)w_gate, (const TIN*)w_up, (TIN*)h_ab, (TIN*)y_swi,
      s.T, s.d, s.E, s.h, nbn, to.nblk, to.grp, to.xg);
  return hipGetLastError();
}

// Forward first layer of a plain two-layer expert: a = x W_1^T (W_1 in the
// w_gate slot), y = sigma(a) (SiLU or ReLU) from the fp32 a; stores a (the
// saved pre-activation, [A][h]) and y.
template <class C>
__global__ __launch_bounds__(C::NT, C::WAVES_PER_EU) void up_act_kernel(
    const typename C::T* __restrict__ x, const int32_t* __restrict__ offsets, const int32_t* __restrict__ eti,
    const int32_t* __restrict__ mb_off, const typename C::T* __restrict__ w1, typename C::T* __restrict__ h_a,
    typename C::T* __restrict__ y_swi, int T, int d, int E, int h, int act, int nbn, int nblk, int grp, int xg) {
  __shared__ __attribute__((aligned(16))) char smem[smem_bytes<C>()];
  using TIN = typename C::T;
  int g, nb;
  if (!tile_of(xcd_swizzle(blockIdx.x, nblk), mb_off, E, nbn, grp, xg, g, nb)) return;
  const RowTile rt = decode_row_tile<C::BM>(mb_off, offsets, E, g);
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  const uint32_t ldx = (uint32_t)d * sizeof(TIN);
  using LA = RowLoader<C::BM, false, C::NT>;
  using LB = RowLoader<C::BN, false, C::NT>;
  LA la;
  LB lb;
  la.rs[0] = make_rsrc(x, (size_t)T * ldx);
#pragma unroll
  for (int i = 0; i < LA::CPT; ++i) {
    const int p = rt.r0 + LA::my_row(i);
    la.roff[i] = p < rt.r1 ? (uint32_t)eti[p] * ldx : OOB_OFF;
  }
  lb.rs[0] = make_rsrc(w1 + (size_t)rt.e * h * d, (size_t)h * ldx);
#pragma unroll
  for (int i = 0; i < LB::CPT; ++i) {
    const int j = nb * C::BN + LB::my_row(i);
    lb.roff[i] = j < h ? (uint32_t)j * ldx : OOB_OFF;
  }
  f32x16_t acc[C::FM][C::FN];
  gemm_mainloop<C>(la, lb, d / C::BK, smem, acc, wm, wn);
  {
    // parked in LDS 128 rows at a time, written as 16-byte row chunks (as in the gated kernel)
    constexpr int PR = 128, PITCH = C::BN + 8;
    static_assert(PR * PITCH * 4 <= smem_bytes<C>(), "the parked rows fit the LDS");
    float* s_c = (float*)smem;
    constexpr int VPC = 16 / sizeof(TIN);
    constexpr int CPR = C::BN / VPC;
#pragma unroll 1
    for (int r0 = 0; r0 < C::BM; r0 += PR) {
      __syncthreads();
      park_rows<C, PR, PITCH>(acc, s_c, r0, wm, wn);
      __syncthreads();
      const int left = rt.r1 - rt.r0 - r0;
      const int rows = left < PR ? left : PR;
      for (int c = threadIdx.x; c < PR * CPR; c += C::NT) {
        const int row = c / CPR, cc = c % CPR;
        if (row >= rows) break;
        const int j = nb * C::BN + cc * VPC;
        if (j >= h) continue;  // a 256-column tile can pass h (a multiple of 128): whole chunks out
        const int p = rt.r0 + r0 + row;
        const float* ar = s_c + row * PITCH + cc * VPC;
        float a[VPC], y[VPC];
#pragma unroll
        for (int v = 0; v < VPC; ++v) {
          a[v] = ar[v];
          y[v] = act_fwd(a[v], act);
        }
        if (h_a) st16(h_a + (size_t)p * h + j, a);  // NULL: nothing saved
        st16(y_swi + (size_t)p * h + j, y);
      }
    }
  }
}

template <typename TIN, int BM, int BN>
static hipError_t up_act_t(const Shape& s, const void* x, const int32_t* offsets, const int32_t* eti,
                           const void* w1, void* h_a, void* y_swi, const ExpertWs& ws, hipStream_t st) {
  using C = XCfg<TIN, BM, BN, false, false, false>;
  const int nbn = col_blocks(s.h, C::BN);
  long long nblk = max_row_blocks(s, BM) * nbn;
  nblk = (nblk + 7) / 8 * 8;
  const TileOrder to = tile_order(nblk, nbn);
  up_act_kernel<C><<<dim3((unsigned)nblk), dim3(C::NT), 0, st>>>(
      (const TIN*)x, offsets, eti, ws.tile_map(BM), (const TIN*)w1, (TIN*)h_a, (TIN*)y_swi, s.T, s.d, s.E, s.h,
      s.act, nbn, to.nblk, to.grp, to.xg);
  return hipGetLastError();
}

hipError_t launch_gate_up(const Shape& s, const void* x, const int32_t* offsets, const int32_t* eti,
                          const void* w_gate, const void* w_up, void* h_ab, void* y_swi, const ExpertWs& ws,
                          hipStream_t st) {
  timing_mark(st, "gate_up", true);
  // measured on MI355X: the large tile wins from d = 4096 on (the small one
  // wastes less on partial row tiles for short reductions); a plain expert's
  // first layer (one projection, N = h) takes it at every d in bf16: 4-8.5%
  // faster at d = 512-2048, h = 4d (MoEBlaze's conf1, conf3, conf4)
  const bool big = pick_large(s.d >= 4096 || (!s.gated() && s.bf16));
  const bool mid = !big && pick_mid(s, false);
  hipError_t e;
  if (!s.gated()) {
    if (s.bf16)
      e = big   ? up_act_t<bf16_t, TILE_L, TILE_L>(s, x, offsets, eti, w_gate, h_ab, y_swi, ws, st)
          : mid ? up_act_t<bf16_t, TILE_S, TILE_L>(s, x, offsets, eti, w_gate, h_ab, y_swi, ws, st)
                : up_act_t<bf16_t, TILE_S, TILE_S>(s, x, offsets, eti, w_gate, h_ab, y_swi, ws, st);
    else
      e = big ? up_act_t<float, TILE_L, TILE_L>(s, x, offsets, eti, w_gate, h_ab, y_swi, ws, st)
              : up_act_t<float, TILE_S, TILE_S>(s, x, offsets, eti, w_gate, h_ab, y_swi, ws, st);
  } else if (s.bf16)
    e = big   ? gate_up_t<bf16_t, TILE_L, TILE_L>(s, x, offsets, eti, w_gate, w_up, h_ab, y_swi, ws, st)
        : mid ? gate_up_t<bf16_t, TILE_S, TILE_L>(s, x, offsets, eti, w_gate, w_up, h_ab, y_swi, ws, st)
              : gate_up_t<bf16_t, TILE_S, TILE_S>(s, x, offsets, eti, w_gate, w_up, h_ab, y_swi, ws, st);
  else
    e = big ? gate_up_t<float, TILE_L, TILE_L>(s, x, offsets, eti, w_gate, w_up, h_ab, y_swi, ws, st)
            : gate_up_t<float, TILE_S, TILE_S>(s, x, offsets, eti, w_gate, w_up, h_ab, y_swi, ws, st);
  timing_mark(st, "gate_up", false);
  return e;
}

// ===========================================================================
// Ordered fold: the owner-computes weighted combine through the reverse index.
//
// Every output row out[t] (per 128-column block) receives K contributions
// from K different expert tiles.  Tiles are claimed through a ticket counter
// in ascending (expert, row-block, column-block) order, and a contribution of
// rank r (the position of its expert among the token's experts, ascending)
// is applied only after turn[t][block] == r; it then bumps the turn.  The
// fp32 accumulator sees the K contributions in ascending expert order:
// deterministic, with integer flags only (no float atomics).  The last rank
// writes the output row.
//
// Row-granular waits.  The tile's result is parked in LDS and each wave
// folds its 32 rows in whatever order their turns arrive, publishing each
// row's turn as soon as that row is stored.  A row therefore waits only on
// its own token's lower-ranked contributions (at most K - 1 of them), never
// on the other rows of the tile; a tile-wide wait would chain every expert's
// tiles behind the previous expert's slowest row.  Every predecessor of a
// contribution lives in a tile with a smaller ticket, held by a running
// workgroup, so the waits drain (bounded by the spin limit all the same).
//
// Visibility across XCDs without cache-wide fences: every accumulator load
// and store is a device-coherent access (the cache policy the compiler gives
// a relaxed device-scope atomic), so no XCD's L2 holds a stale or dirty
// accumulator line.  A wave waits for its accumulator stores to complete
// before it publishes their turns, and issues accumulator loads only for rows
// whose turns it has seen.  A device-scope release/acquire fence pair would
// instead write back and invalidate the whole L2 of the XCD on every tile,
// evicting the weight tiles the other workgroups are reusing.
//
// INIT_FIRST: rank 0 writes the accumulator (forward); otherwise the
// accumulator is pre-initialised and every rank adds (backward dX, where the
// router term is the initial value).
// ===========================================================================
MOE_DEV u32x2_t coherent_load2(const float* p) {
  const uint64_t v = __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_bit_cast(u32x2_t, v);
}
MOE_DEV void coherent_store2(float* p, float a, float b) {
  const uint64_t v = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MOE_DEV void store2(float* p, float a, float b) { *(float2*)p = make_float2(a, b); }
MOE_DEV void store2(bf16_t* p, float a, float b) { *(uint32_t*)p = pack_bf16x2(a, b); }

constexpr int FOLD_ROWS_PER_WAVE = 32;
// Rows per batch of a wave's fold: 16 in the forward, all 32 in the dX fold.
// Measured on MI355X at large d against 16 everywhere: the dX fold 0.9%
// faster with 32, down-combine 1.1% slower.
template <bool INIT_FIRST>
constexpr int fold_batch() { return INIT_FIRST ? 16 : 32; }

// Fold of one parked 128 x 128 block (rows of 136 floats in s_c, per-row
// token, weight and rank in s_t, s_w, s_rank) into the 128 accumulator
// columns of column block nb (of NB), by four waves: wave w (0..3) folds block
// rows w, w + 4, ..., w + 124.
template <bool INIT_FIRST, typename TOUT>
MOE_DEV void fold_rows(const float* s_c, const int* s_t, const float* s_w, const int* s_rank, int rows, int wave,
                       int nb, int NB, int K, int d, int32_t* turn, float* __restrict__ accws, TOUT* __restrict__ out,
                       int32_t* err, int spin_limit) {
  constexpr int BATCH = fold_batch<INIT_FIRST>();
  const int l = lane_id();
  // wave w folds tile rows w, w + 4, ..., w + 124; lane j < 32 watches row w + 4j
  const int j = l & 31;
  const int my_row = wave + 4 * j;
  const bool mine = l < 32 && my_row < rows;
  const int my_t = mine ? s_t[my_row] : 0;
  const int my_rank = mine ? s_rank[my_row] : 0;
  const float my_w = mine ? s_w[my_row] : 1.0f;
  int32_t* my_turn = turn + (size_t)my_t * NB + nb;
  const int col = 2 * l;  // each lane folds two adjacent columns of a row
  // byte offsets of the lane's two columns in an accumulator row and in an
  // output row: 32-bit lane offsets on scalar row addresses
  const uint32_t cbyte = (uint32_t)(nb * 128 + col) * (uint32_t)sizeof(float);
  const uint32_t obyte = (uint32_t)(nb * 128 + col) * (uint32_t)sizeof(TOUT);
  uint64_t pending = __builtin_amdgcn_ballot_w64(mine);
  int spins = 0;
  while (pending) {
    const bool ready = ((pending >> j) & 1) && l < 32 &&
                       __hip_atomic_load(my_turn, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= my_rank;
    const uint64_t m = __builtin_amdgcn_ballot_w64(ready) & pending;
    if (m == 0) {
      if (++spins > spin_limit) {
        __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
      continue;
    }
    spins = 0;
    // In batches of BATCH rows: read the accumulator of every row of the batch
    // without branches (a row that is not ready yet, or past the tile, reads
    // a value that is never stored), combine, then store the ready rows, so
    // that no store waits on a load.  A row's token, rank and weight come
    // from the lane that watches it (readlane: scalars, with no LDS read and
    // no wait per row); the row's two parked values are read from LDS for the
    // whole batch at once.
#pragma unroll
    for (int b0 = 0; b0 < FOLD_ROWS_PER_WAVE; b0 += BATCH) {
      if (((m >> b0) & ((1ull << BATCH) - 1)) == 0) continue;
      int t_r[BATCH], rank_r[BATCH];
      float w_r[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        t_r[i] = __builtin_amdgcn_readlane(my_t, b0 + i);
        rank_r[i] = __builtin_amdgcn_readlane(my_rank, b0 + i);
        w_r[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), b0 + i));
      }
      u32x2_t prev[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i)
        prev[i] = coherent_load2((const float*)((const char*)(accws + (size_t)t_r[i] * d) + cbyte));
      float2 c[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i) c[i] = *(const float2*)(s_c + (wave + 4 * (b0 + i)) * FOLD_LD + col);
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const bool fresh = INIT_FIRST && rank_r[i] == 0;  // rank 0 starts the sum (forward)
        const float a = (fresh ? 0.0f : __uint_as_float(prev[i][0])) + w_r[i] * c[i].x;
        const float b = (fresh ? 0.0f : __uint_as_float(prev[i][1])) + w_r[i] * c[i].y;
        if ((m >> (b0 + i)) & 1) {
          const size_t row = (size_t)t_r[i] * d;
          if (rank_r[i] == K - 1) store2((TOUT*)((char*)(out + row) + obyte), a, b);
          else coherent_store2((float*)((char*)(accws + row) + cbyte), a, b);
        }
      }
    }
    // this wave's stores have completed before the turns of its rows move on
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if ((m >> j) & 1 && l < 32)
      __hip_atomic_store(my_turn, my_rank + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    pending &= ~m;
  }
}

// Token, weight and rank of tile row threadIdx.x (< 128) for the fold of a
// 128-row tile (down-combine fetches them before its main loop, so that their
// latency hides behind it); rows past the tile get token 0, weight 1 and rank
// 0 and are never stored.
struct FoldRowMeta {
  int t = 0;
  float w = 1.0f;
  int rank = 0;
};
MOE_DEV FoldRowMeta fold_row_meta(const RowTile& rt, const int32_t* __restrict__ eti, const float* __restrict__ w_pos,
                                  const int32_t* __restrict__ rank_pos) {
  FoldRowMeta m;
  const int p = rt.r0 + (int)threadIdx.x;
  if (threadIdx.x < 128 && p < rt.r1) {
    m.t = eti[p];
    if (w_pos) m.w = w_pos[p];
    m.rank = rank_pos[p];
  }
  return m;
}

template <class C, bool INIT_FIRST>
MOE_DEV void fold_epilogue(const f32x16_t (&acc)[C::FM][C::FN], const RowTile& rt, int nb, int NB, int wm, int wn,
                           const FoldRowMeta& meta, const int32_t* __restrict__ eti,
                           const float* __restrict__ w_pos, const int32_t* __restrict__ rank_pos, int K, int d,
                           int32_t* turn, float* __restrict__ accws, typename C::T* __restrict__ out,
                           int32_t* counters, int spin_limit, char* smem) {
  const int tid = threadIdx.x;
  const int l = lane_id();
  if constexpr (C::BM == 128 && C::BN == 128) {
    static_assert(C::NT == NTHREADS, "the fold parks a 128 x 128 tile, four waves");
    static_assert(C::BM * FOLD_LD * 4 + 3 * C::BM * 4 <= C::LDS_BYTES, "parked tile fits the LDS stages");
    float* s_c = (float*)smem;
    int* s_t = (int*)(smem + C::BM * FOLD_LD * 4);
    float* s_w = (float*)(s_t + C::BM);
    int* s_rank = (int*)(s_w + C::BM);
    const int rows = rt.r1 - rt.r0;
    __syncthreads();  // the LDS stages are reused below
    if (tid < 128) {
      s_t[tid] = meta.t;
      s_w[tid] = meta.w;
      s_rank[tid] = meta.rank;
    }
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s_c[(C::a_row0(wm, fm) + frag_row(r, l)) * FOLD_LD + C::b_row0(wn, fn) + frag_col(l)] = acc[fm][fn][r];
    __syncthreads();
    fold_rows<INIT_FIRST>(s_c, s_t, s_w, s_rank, rows, tid >> 6, nb, NB, K, d, turn, accws, out, counters,
                          spin_limit);
  } else if constexpr (C::BM == 128) {
    // 128 x 256 tile, eight waves of 64 x 64: both 128-column halves are
    // parked at once; waves 0-3 then fold half 0 (column block 2 nb of the
    // 128-wide turn grid) and waves 4-7 half 1 (column block 2 nb + 1).
    static_assert(C::BN == 256 && C::NT == 512 && C::WM == 2 && C::WN == 4, "eight-wave 128 x 256 tile");
    static_assert(2 * 128 * FOLD_LD * 4 + 3 * 128 * 4 <= smem_bytes<C>(), "two parked halves fit the LDS");
    float* s_c0 = (float*)smem;
    float* s_c1 = s_c0 + 128 * FOLD_LD;
    int* s_t = (int*)(s_c1 + 128 * FOLD_LD);
    float* s_w = (float*)(s_t + 128);
    int* s_rank = (int*)(s_w + 128);
    const int wave = tid >> 6, group = wave >> 2;
    const int rows = rt.r1 - rt.r0;
    __syncthreads();  // the LDS stages are reused below
    if (tid < 128) {
      s_t[tid] = meta.t;
      s_w[tid] = meta.w;
      s_rank[tid] = meta.rank;
    }
    float* s_c = (wn >> 1) ? s_c1 : s_c0;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s_c[(C::a_row0(wm, fm) + frag_row(r, l)) * FOLD_LD + (wn & 1) * 64 + fn * 32 + frag_col(l)] =
              acc[fm][fn][r];
    __syncthreads();
    fold_rows<INIT_FIRST>(group ? s_c1 : s_c0, s_t, s_w, s_rank, rows, wave & 3, 2 * nb + group, 2 * NB, K, d, turn,
                          accws, out, counters, spin_limit);
  } else {
    // 256 x 256 tile, eight waves of 64 x 128: two passes of 128 rows.  The
    // waves holding rows 0..127 (wm < 2) park both 128-column halves and fold
    // them (column blocks 2 nb and 2 nb + 1 of the 128-wide turn grid), four
    // waves for both halves; then the waves holding rows 128..255 park theirs
    // and all eight fold (waves 0-3 half 0, 4-7 half 1).  The two kinds of
    // wave take separate branches, each through the same four workgroup
    // barriers, so no fold code runs while a wave still holds accumulators:
    // in one shared pass sequence the second half's accumulators would stay
    // live through the first pass's fold and spill.
    static_assert(C::BM == 256 && C::BN == 256 && C::NT == 512 && C::WM == 4 && C::WN == 2, "eight-wave 256 tile");
    static_assert(2 * 128 * FOLD_LD * 4 + 3 * 128 * 4 <= C::LDS_BYTES, "two parked halves fit the LDS stages");
    float* s_c0 = (float*)smem;
    float* s_c1 = s_c0 + 128 * FOLD_LD;
    int* s_t = (int*)(s_c1 + 128 * FOLD_LD);
    float* s_w = (float*)(s_t + 128);
    int* s_rank = (int*)(s_w + 128);
    const int wave = tid >> 6, group = wave >> 2;
    const int all = rt.r1 - rt.r0;
    const int rows0 = all > 128 ? 128 : all, rows1 = all > 128 ? all - 128 : 0;
    // per-row token, weight and rank of rows hp*128 .. +127 (threads 0..127,
    // which are waves 0 and 1: the first kind)
    auto meta = [&](int hp, int rows) {
      if (tid < 128) {
        const int p = rt.r0 + hp * 128 + tid;
        const bool in = tid < rows;
        s_t[tid] = in ? eti[p] : 0;
        s_w[tid] = in && w_pos ? w_pos[p] : 1.0f;
        s_rank[tid] = in ? rank_pos[p] : 0;
      }
    };
    auto park = [&]() {
      float* s_c = wn ? s_c1 : s_c0;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s_c[((wm & 1) * 64 + fm * 32 + frag_row(r, l)) * FOLD_LD + fn * 32 + frag_col(l)] = acc[fm][fn][r];
    };
    if ((wm >> 1) == 0) {
      __syncthreads();  // 1: the LDS stages are free
      meta(0, rows0);
      park();
      __syncthreads();  // 2: rows 0..127 parked
      if (rows0 > 0) {
        fold_rows<INIT_FIRST>(s_c0, s_t, s_w, s_rank, rows0, wave, 2 * nb, 2 * NB, K, d, turn, accws, out, counters,
                              spin_limit);
        fold_rows<INIT_FIRST>(s_c1, s_t, s_w, s_rank, rows0, wave, 2 * nb + 1, 2 * NB, K, d, turn, accws, out,
                              counters, spin_limit);
      }
      __syncthreads();  // 3: the first pass has read its rows
      meta(1, rows1);
      __syncthreads();  // 4: rows 128..255 parked
    } else {
      __syncthreads();  // 1
      __syncthreads();  // 2
      __syncthreads();  // 3
      park();
      __syncthreads();  // 4
    }
    if (rows1 > 0)
      fold_rows<INIT_FIRST>(group ? s_c1 : s_c0, s_t, s_w, s_rank, rows1, wave & 3, 2 * nb + group, 2 * NB, K, d,
                            turn, accws, out, counters, spin_limit);
  }
}

// Fold tiles come from eight queues, one per XCD: queue q holds the column
// blocks nb = q, q + 8, ... of every row block, in ascending (row block,
// column block) order.  A tile waits only on the same column block of a
// token's lower experts, i.e. on earlier tiles of its own queue, so the claim
// order per queue is all the fold needs.  A workgroup claims from its own
// XCD's queue first (an expert's weight column block then stays in one L2,
// and a row block's rows serve the XCD's two column blocks back to back),
// then from the next queues when its own is empty, so every tile is taken
// however the workgroups spread over the XCDs.  Counters [8, 16) of the
// counters block (zeroed per call) are the queue heads.
constexpr int FOLD_QUEUES = 8;
MOE_DEV bool claim_fold_tile(int32_t* counters, char* smem, int ng, int nbn, int& g, int& nb) {
  int* s = (int*)smem;
  if (threadIdx.x == 0) {
    const int x = (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & (FOLD_QUEUES - 1));  // HW_REG_XCC_ID
    int qt = -1, tt = 0;
    for (int j = 0; j < FOLD_QUEUES; ++j) {
      const int q = (x + j) & (FOLD_QUEUES - 1);
      const int per = (nbn - q + FOLD_QUEUES - 1) / FOLD_QUEUES;  // column blocks of queue q
      if (per <= 0) continue;
      const int t = atomicAdd(counters + 8 + q, 1);
      if (t < ng * per) {
        qt = q;
        tt = t;
        break;
      }
    }
    s[0] = qt;
    s[1] = tt;
  }
  __syncthreads();
  const int q = s[0], t = s[1];
  __syncthreads();
  if (q < 0) return false;
  const int per = (nbn - q + FOLD_QUEUES - 1) / FOLD_QUEUES;
  g = t / per;
  nb = q + FOLD_QUEUES * (t - g * per);
  return true;
}

// ===========================================================================
// Down projection + combine: M = rows of expert e, N = TILE output columns, K = h.
// ===========================================================================
template <class C>
__global__ __launch_bounds__(C::NT, C::WAVES_PER_EU) void down_combine_kernel(
    const typename C::T* __restrict__ y_swi, const typename C::T* __restrict__ w_down,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ eti, const int32_t* __restrict__ mb_off,
    const float* __restrict__ w_pos, const int32_t* __restrict__ rank_pos, int32_t* turn, float* accws,
    typename C::T* __restrict__ out, int32_t* counters, int d, int E, int K, int h, int spin_limit) {
  __shared__ __attribute__((aligned(16))) char smem[smem_bytes<C>()];
  using TIN = typename C::T;
  const int NB = col_blocks(d, C::BN);
  int g, nb;
  if (!claim_fold_tile(counters, smem, mb_off[E], NB, g, nb)) return;
  const RowTile rt = decode_row_tile<C::BM>(mb_off, offsets, E, g);
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  const uint32_t ldy = (uint32_t)h * sizeof(TIN);
  using LA = RowLoader<C::BM, false, C::NT>;
  using LB = RowLoader<C::BN, false, C::NT>;
  LA la;
  LB lb;
  la.rs[0] = make_rsrc(y_swi + (size_t)rt.r0 * h, (size_t)(rt.r1 - rt.r0) * ldy);
#pragma unroll
  for (int i = 0; i < LA::CPT; ++i) {
    const int r = LA::my_row(i);
    la.roff[i] = rt.r0 + r < rt.r1 ? (uint32_t)r * ldy : OOB_OFF;
  }
  lb.rs[0] = make_rsrc(w_down + (size_t)rt.e * d * h, (size_t)d * ldy);
#pragma unroll
  for (int i = 0; i < LB::CPT; ++i) {
    const int n = nb * C::BN + LB::my_row(i);
    lb.roff[i] = n < d ? (uint32_t)n * ldy : OOB_OFF;
  }
  const FoldRowMeta meta = C::BM == 128 ? fold_row_meta(rt, eti, w_pos, rank_pos) : FoldRowMeta{};
  f32x16_t acc[C::FM][C::FN];
  gemm_mainloop<C>(la, lb, h / C::BK, smem, acc, wm, wn);
  fold_epilogue<C, true>(acc, rt, nb, NB, wm, wn, meta, eti, w_pos, rank_pos, K, d, turn, accws, out,
                         counters + ERR_COMBINE, spin_limit, smem);
}

template <typename TIN, int BM, int BN>
static hipError_t down_combine_t(const Shape& s, const void* y_swi, const void* w_down, const int32_t* offsets,
                                 const int32_t* eti, void* out, const ExpertWs& ws, int spin_limit, hipStream_t st) {
  using C = XCfg<TIN, BM, BN, false, false, false>;
  const long long nblk = max_row_blocks(s, BM) * col_blocks(s.d, BN);
  down_combine_kernel<C><<<dim3((unsigned)nblk), dim3(C::NT), 0, st>>>(
      (const TIN*)y_swi, (const TIN*)w_down, offsets, eti, ws.tile_map(BM), ws.w_pos, ws.rank_pos, ws.turn, ws.acc,
      (TIN*)out, ws.counters, s.d, s.E, s.K, s.h, spin_limit);
  return hipGetLastError();
}

hipError_t launch_down_combine(const Shape& s, const void* y_swi, const void* w_down, const int32_t* offsets,
                               const int32_t* eti, void* out, const ExpertWs& ws, int spin_limit, hipStream_t st) {
  timing_mark(st, "down_combine", true);
  const hipError_t e =
      !s.bf16               ? down_combine_t<float, TILE_S, TILE_S>(s, y_swi, w_down, offsets, eti, out, ws, spin_limit, st)
      : wide_fold(s, s.h, false) ? down_combine_t<bf16_t, TILE_L, TILE_L>(s, y_swi, w_down, offsets, eti, out, ws, spin_limit, st)
      : mid_fold(s, s.h, false)  ? down_combine_t<bf16_t, TILE_S, TILE_L>(s, y_swi, w_down, offsets, eti, out, ws, spin_limit, st)
                          : down_combine_t<bf16_t, TILE_S, TILE_S>(s, y_swi, w_down, offsets, eti, out, ws, spin_limit, st);
  timing_mark(st, "down_combine", false);
  return e;
}

// ===========================================================================
// Staged-Y combine (ablation of the ordered fold, never the product path):
// the down projection writes Y[p] = y_swi[p] W_down[e]^T for every position
// (a T*K x d buffer, in the activation dtype), then a gather-and-sum kernel
// forms out[t] = sum_k w[t,k] Y[token_index_map[t*K+k]] in slot order --
// the SonicMoE analysis page's temporary Y (sec. 3.4.1) and gather-and-sum
// aggregation ("O") kernel (sec. 3.4.2, Figure 17 left).
// ===========================================================================
template <class C>
__global__ __launch_bounds__(C::NT, C::WAVES_PER_EU) void down_staged_kernel(
    const typename C::T* __restrict__ y_swi, const typename C::T* __restrict__ w_down,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ mb_off, typename C::T* __restrict__ ystage,
    int d, int E, int h, int nbn, int nblk, int grp, int xg) {
  static_assert(C::BM == 128 && C::BN == 128 && C::NT == NTHREADS, "128 x 128 tile, four waves");
  __shared__ __attribute__((aligned(16))) char smem[smem_bytes<C>()];
  using TIN = typename C::T;
  int g, nb;
  if (!tile_of(xcd_swizzle(blockIdx.x, nblk), mb_off, E, nbn, grp, xg, g, nb)) return;
  const RowTile rt = decode_row_tile<C::BM>(mb_off, offsets, E, g);
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  const uint32_t ldy = (uint32_t)h * sizeof(TIN);
  using LA = RowLoader<C::BM, false, C::NT>;
  using LB = RowLoader<C::BN, false, C::NT>;
  LA la;
  LB lb;
  la.rs[0] = make_rsrc(y_swi + (size_t)rt.r0 * h, (size_t)(rt.r1 - rt.r0) * ldy);
#pragma unroll
  for (int i = 0; i < LA::CPT; ++i) {
    const int r = LA::my_row(i);
    la.roff[i] = rt.r0 + r < rt.r1 ? (uint32_t)r * ldy : OOB_OFF;
  }
  lb.rs[0] = make_rsrc(w_down + (size_t)rt.e * d * h, (size_t)d * ldy);
#pragma unroll
  for (int i = 0; i < LB::CPT; ++i) {
    const int n = nb * C::BN + LB::my_row(i);
    lb.roff[i] = n < d ? (uint32_t)n * ldy : OOB_OFF;
  }
  f32x16_t acc[C::FM][C::FN];
  gemm_mainloop<C>(la, lb, h / C::BK, smem, acc, wm, wn);
  // park the tile in LDS, then write whole 16-byte row chunks
  float* s_c = (float*)smem;
  const int l = lane_id();
  __syncthreads();
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s_c[(C::a_row0(wm, fm) + frag_row(r, l)) * FOLD_LD + C::b_row0(wn, fn) + frag_col(l)] = acc[fm][fn][r];
  __syncthreads();
  constexpr int VPC = 16 / sizeof(TIN);          // values per 16-byte chunk
  constexpr int CPR = C::BN / VPC;               // chunks per tile row
  const int rows = rt.r1 - rt.r0;
  for (int c = threadIdx.x; c < C::BM * CPR; c += C::NT) {
    const int row = c / CPR, cc = c % CPR;
    if (row >= rows) break;
    const float* src = s_c + row * FOLD_LD + cc * VPC;
    TIN* dst = ystage + (size_t)(rt.r0 + row) * d + nb * C::BN + cc * VPC;
    if constexpr (sizeof(TIN) == 2) {
      u32x4_t v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = pack_bf16x2(src[2 * q], src[2 * q + 1]);
      *(u32x4_t*)dst = v;
    } else {
      *(f32x4_t*)dst = *(const f32x4_t*)src;
    }
  }
}

// out[t] = sum_k w[t,k] Y[tim[t*K+k]] (slot order, fp32), 8 columns per thread
template <typename TIN>
__global__ __launch_bounds__(256) void gather_sum_kernel(const TIN* __restrict__ ystage,
                                                         const int32_t* __restrict__ tim,
                                                         const float* __restrict__ topk_w, TIN* __restrict__ out,
                                                         int d, int K) {
  const int t = blockIdx.x;
  __shared__ int s_p[32];
  __shared__ float s_w[32];
  if (threadIdx.x < K) {
    s_p[threadIdx.x] = tim[(size_t)t * K + threadIdx.x];
    s_w[threadIdx.x] = topk_w[(size_t)t * K + threadIdx.x];
  }
  __syncthreads();
  for (int c0 = threadIdx.x * 8; c0 < d; c0 += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[v] = 0.0f;
    for (int k = 0; k < K; ++k) {
      const TIN* row = ystage + (size_t)s_p[k] * d + c0;
      const float w = s_w[k];
      if constexpr (sizeof(TIN) == 2) {
        const u32x4_t q = *(const u32x4_t*)row;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          acc[2 * v] += w * bf16_to_f32(q[v] & 0xffffu);
          acc[2 * v + 1] += w * bf16_to_f32(q[v] >> 16);
        }
      } else {
        const f32x4_t q0 = *(const f32x4_t*)row, q1 = *(const f32x4_t*)(row + 4);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          acc[v] += w * q0[v];
          acc[4 + v] += w * q1[v];
        }
      }
    }
    TIN* o = out + (size_t)t * d + c0;
    if constexpr (sizeof(TIN) == 2) {
      u32x4_t q;
#pragma unroll
      for (int v = 0; v < 4; ++v) q[v] = pack_bf16x2(acc[2 * v], acc[2 * v + 1]);
      *(u32x4_t*)o = q;
    } else {
      *(f32x4_t*)o = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
      *(f32x4_t*)(o + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
    }
  }
}

template <typename TIN>
static hipError_t combine_staged_t(const Shape& s, const void* y_swi, const void* w_down, const int32_t* offsets,
                                   const int32_t* tim, const float* topk_w, void* out, const ExpertWs& ws,
                                   hipStream_t st) {
  using C = GCfg<TIN, TILE_S>;
  const int nbn = col_blocks(s.d, TILE_S);
  const long long nblk = (max_row_blocks(s, TILE_S) * nbn + 7) / 8 * 8;
  const TileOrder to = tile_order(nblk, nbn);
  timing_mark(st, "down_staged", true);
  down_staged_kernel<C><<<dim3((unsigned)nblk), dim3(C::NT), 0, st>>>(
      (const TIN*)y_swi, (const TIN*)w_down, offsets, ws.tile_map(TILE_S), (TIN*)ws.ystage, s.d, s.E, s.h, nbn,
      to.nblk, to.grp, to.xg);
  timing_mark(st, "down_staged", false);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  timing_mark(st, "gather_sum", true);
  gather_sum_kernel<TIN><<<dim3(s.T), dim3(256), 0, st>>>((const TIN*)ws.ystage, tim, topk_w, (TIN*)out, s.d, s.K);
  timing_mark(st, "gather_sum", false);
  return hipGetLastError();
}

hipError_t launch_combine_staged(const Shape& s, const void* y_swi, const void* w_down, const int32_t* offsets,
                                 const int32_t* tim, const float* topk_w, void* out, const ExpertWs& ws,
                                 hipStream_t st) {
  return s.bf16 ? combine_staged_t<bf16_t>(s, y_swi, w_down, offsets, tim, topk_w, out, ws, st)
                : combine_staged_t<float>(s, y_swi, w_down, offsets, tim, topk_w, out, ws, st);
}

// ===========================================================================
// Backward
// ===========================================================================

// Each source gives the buffer resource of a k-tile (rsrc), the value that
// locates k-row k and has to be read from memory (key: the gathered row index,
// or 0), the byte offset of k-row k at the tile's first column from it
// (row_off, OOB_OFF outside the problem) and optionally a per-k-row scale.
template <typename T>
struct SrcWeightKN {   // B[k][n] = W[k][n0 + n], W one expert's [K, ld] matrix
  rsrc_t rs;
  uint32_t ld_bytes, col0;
  MOE_DEV rsrc_t rsrc(int) const { return rs; }
  MOE_DEV uint32_t key(int) const { return 0; }
  MOE_DEV uint32_t row_off(int k, uint32_t) const { return (uint32_t)k * ld_bytes + col0; }
  MOE_DEV float scale(int) const { return 1.0f; }
};
template <typename T>
struct SrcWeightKN2 {  // k < h: W1[k][n0+n], else W2[k-h][n0+n]; a k-tile never straddles h
  rsrc_t rs1, rs2;
  uint32_t ld_bytes, col0;
  int h, kpt;
  MOE_DEV rsrc_t rsrc(int kt) const { return kt * kpt < h ? rs1 : rs2; }
  MOE_DEV uint32_t key(int) const { return 0; }
  MOE_DEV uint32_t row_off(int k, uint32_t) const { return (uint32_t)(k < h ? k : k - h) * ld_bytes + col0; }
  MOE_DEV float scale(int) const { return 1.0f; }
};
template <typename T>
struct SrcRowsContig {  // rows p0 + k < p1 of a [rows, ld] array (resource based at row p0)
  rsrc_t rs;
  uint32_t ld_bytes, col0;
  int n;                // p1 - p0
  rsrc_t rscl;          // optional per-row scale: n floats from position p0 (reads 0 past them)
  MOE_DEV rsrc_t rsrc(int) const { return rs; }
  MOE_DEV uint32_t key(int) const { return 0; }
  MOE_DEV uint32_t row_off(int k, uint32_t) const { return k < n ? (uint32_t)k * ld_bytes + col0 : OOB_OFF; }
  MOE_DEV float scale(int k) const { return __builtin_bit_cast(float, buf_load4(rscl, (uint32_t)k * 4u)); }
};
template <typename T>
struct SrcRowsGather {  // rows eti[p0 + k], k < n
  rsrc_t rs;
  uint32_t ld_bytes, col0;
  int n;                // p1 - p0
  rsrc_t reti;          // n row indices from position p0 (read 0 past them)
  MOE_DEV rsrc_t rsrc(int) const { return rs; }
  // a buffer load, not a guarded one: no branch, so the compiler's wait
  // counts stay exact and the index load is not waited for early
  MOE_DEV uint32_t key(int k) const { return buf_load4(reti, (uint32_t)k * 4u); }
  MOE_DEV uint32_t row_off(int k, uint32_t row) const { return k < n ? row * ld_bytes + col0 : OOB_OFF; }
  MOE_DEV float scale(int) const { return 1.0f; }
};

MOE_DEV int min_i(int a, int b) { return a < b ? a : b; }

// dH kernel: dA' = dO W_down (M rows of e, N = TILE of h, K = d) + SwiGLU backward
// (or, for a plain two-layer expert, dA = w dA' * sigma'(a), dH = [dA]).
// HONLY (H-only saving, SonicMoE analysis page sec. 3.4.1): y is recomputed
// as SiLU(a) * b from the saved a, b instead of read from y_swi, and the
// kernel also writes A' = w * y for the dW_down GEMM.
template <class C, bool HONLY>
__global__ __launch_bounds__(C::NT, C::WAVES_PER_EU) void dh_kernel(
    const typename C::T* __restrict__ dout, const typename C::T* __restrict__ w_down,
    const typename C::T* h_ab, const typename C::T* __restrict__ y_swi,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ eti, const int32_t* __restrict__ mb_off,
    const float* __restrict__ w_pos, typename C::T* dh, float* __restrict__ ds_part,
    typename C::T* __restrict__ a_prime, int T, int d, int E, int h, int act, int nbn, int nblk, int grp, int xg) {
  __shared__ __attribute__((aligned(16))) char smem[smem_bytes<C>()];
  using TIN = typename C::T;
  int g, nb;
  if (!tile_of(xcd_swizzle(blockIdx.x, nblk), mb_off, E, nbn, grp, xg, g, nb)) return;
  const RowTile rt = decode_row_tile<C::BM>(mb_off, offsets, E, g);
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  const uint32_t ldd = (uint32_t)d * sizeof(TIN);
  using LA = RowLoader<C::BM, false, C::NT>;
  LA la;
  la.rs[0] = make_rsrc(dout, (size_t)T * ldd);
#pragma unroll
  for (int i = 0; i < LA::CPT; ++i) {
    const int p = rt.r0 + LA::my_row(i);
    la.roff[i] = p < rt.r1 ? (uint32_t)eti[p] * ldd : OOB_OFF;
  }
  KSrcLoader<C, C::BKM, C::BN, SrcWeightKN<TIN>, false> lb;
  lb.src.rs = make_rsrc(w_down + (size_t)rt.e * d * h, (size_t)d * h * sizeof(TIN));
  lb.src.ld_bytes = (uint32_t)h * sizeof(TIN);
  lb.src.col0 = (uint32_t)(nb * C::BN) * sizeof(TIN);
  lb.ncols = min_i(C::BN, h - nb * C::BN);
  f32x16_t acc[C::FM][C::FN];
  gemm_mainloop<C>(la, lb, d / C::BK, smem, acc, wm, wn);

  {
    // Park dA' (fp32) in LDS, 128 rows at a time; then each thread takes
    // 16-byte row chunks, so a, b, y are read and dA, dB (and A') written as
    // whole chunks.  dh may be h_ab itself (no __restrict__ on either): each
    // chunk of a and b is loaded by the thread that later stores da and db at
    // the same place, from those very values, and no other chunk is touched (a, b and the outputs with the non-temporal policy: each
    // is touched once here; measured 1-3% faster).  dS of a row is reduced over the row's chunk-owning lanes
    // in a fixed order.
    constexpr int PR = 128, PITCH = C::BN + 8;
    static_assert(PR * PITCH * 4 <= smem_bytes<C>(), "the parked rows fit the LDS");
    float* s_c = (float*)smem;
    constexpr int VPC = 16 / sizeof(TIN);   // values per chunk
    constexpr int CPR = C::BN / VPC;        // chunks per row
    constexpr int RPI = C::NT / CPR;        // rows per pass of the workgroup
    static_assert(CPR <= 64 && C::NT % CPR == 0, "a row's chunks within one wave");
    const int cc = (int)threadIdx.x % CPR;
    const int j0 = nb * C::BN + cc * VPC;
    const bool jin = j0 < h;                // a 256-column tile can pass h (a multiple of 128)
    const int hw = act == ACT_SWIGLU ? 2 * h : h;
#pragma unroll 1
    for (int r0 = 0; r0 < C::BM; r0 += PR) {
      __syncthreads();  // the LDS stages (first pass) or the previous rows are reused
      park_rows<C, PR, PITCH>(acc, s_c, r0, wm, wn);
      __syncthreads();
      const int left = rt.r1 - rt.r0 - r0;
      const int rows = left < PR ? left : PR;
      // RB rows per thread at a time: their loads of a, b (and y) are issued
      // together, so that the thread waits once per batch rather than per row
      // (one row on the 256 x 256 tile, whose other half's accumulators are
      // still live here: more would spill)
      constexpr int RB = C::BM == 256 ? 1 : 4;
      static_assert(PR % (RB * RPI) == 0, "whole batches of rows");
      const bool gated = act == ACT_SWIGLU;
      for (int rb = (int)threadIdx.x / CPR; rb < PR; rb += RB * RPI) {
        u32x4_t qa[RB] = {}, qb[RB] = {}, qy[RB] = {};
        float w[RB] = {};
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          const int rr = rb + i * RPI;
          if (rr < rows && jin) {
            const int p = rt.r0 + r0 + rr;
            w[i] = w_pos[p];
            qa[i] = raw16nt(h_ab + (size_t)p * hw + j0);
            if (gated) qb[i] = raw16nt(h_ab + (size_t)p * hw + h + j0);
            if constexpr (!HONLY) qy[i] = raw16(y_swi + (size_t)p * h + j0);
          }
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          const int rr = rb + i * RPI;
          float dsum = 0.0f;
          if (rr < rows && jin) {
            const int p = rt.r0 + r0 + rr;
            const float* dapr = s_c + rr * PITCH + cc * VPC;
            float a[VPC], y[VPC], da[VPC];
            unpack16(qa[i], a);
            if constexpr (!HONLY) unpack16(qy[i], y);
            if (gated) {
              float b[VPC], db[VPC];
              unpack16(qb[i], b);
#pragma unroll
              for (int v = 0; v < VPC; ++v) {
                const float sg = sigmoidf_(a[v]);
                if constexpr (HONLY) y[v] = a[v] * sg * b[v];
                const float dy = w[i] * dapr[v];
                da[v] = dy * b[v] * sg * (1.0f + a[v] * (1.0f - sg));
                db[v] = dy * a[v] * sg;
                dsum += dapr[v] * y[v];
              }
              st16nt(dh + (size_t)p * hw + h + j0, db);
            } else {  // plain expert: dA = dy * sigma'(a), from the saved pre-activation
#pragma unroll
              for (int v = 0; v < VPC; ++v) {
                float yv, gv;
                act_fwd_grad(a[v], act, yv, gv);
                if constexpr (HONLY) y[v] = yv;
                da[v] = w[i] * dapr[v] * gv;
                dsum += dapr[v] * y[v];
              }
            }
            st16nt(dh + (size_t)p * hw + j0, da);
            if constexpr (HONLY) {
              float ap[VPC];
#pragma unroll
              for (int v = 0; v < VPC; ++v) ap[v] = w[i] * y[v];
              st16nt(a_prime + (size_t)p * h + j0, ap);
            }
          }
#pragma unroll
          for (int off = CPR / 2; off > 0; off >>= 1) dsum += __shfl_xor(dsum, off, CPR);
          if (cc == 0 && rr < rows) ds_part[(size_t)(rt.r0 + r0 + rr) * nbn + nb] = dsum;
        }
      }
    }
  }
}

// router backward per token: dS, dz (closed form), and the router term of dX
//   dz[t,S_k] = w_k (dS_k - sum_j w_j dS_j)          (renormalised softmax)
//   dX_router[t] = sum_k dz[t,S_k] Wg[S_k]          -> fold accumulator init
// One wave per token: lane k < K finishes dS_k from its h-block partials; the
// weighted sum over k is a butterfly (every lane gets the same bits, since each
// step adds the same two values); the router term is written 16 bytes of Wg
// per lane per step, k in ascending order.
constexpr int RB_TOKENS = 4;  // tokens (waves) per workgroup
template <typename TIN>
__global__ __launch_bounds__(64 * RB_TOKENS) void router_bwd_kernel(const int32_t* __restrict__ ids,
                                                                    const float* __restrict__ topk_w,
                                                                    const int32_t* __restrict__ tim,
                                                                    const float* __restrict__ ds_part, int nbh,
                                                                    const TIN* __restrict__ wg,
                                                                    float* __restrict__ dz_pos,
                                                                    float* __restrict__ dz_tok,
                                                                    float* __restrict__ ds_out,
                                                                    float* __restrict__ accws, int T, int d, int K) {
  const int t = blockIdx.x * RB_TOKENS + (int)(threadIdx.x >> 6);
  if (t >= T) return;  // whole waves
  const int l = lane_id();
  float dsv = 0.0f, wv = 0.0f;
  int e = 0, p = 0;
  if (l < K) {
    p = tim[(size_t)t * K + l];
    for (int nb = 0; nb < nbh; ++nb) dsv += ds_part[(size_t)p * nbh + nb];
    wv = topk_w[(size_t)t * K + l];
    e = ids[(size_t)t * K + l];
  }
  float c = wv * dsv;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, 64);
  const float dz = wv * (dsv - c);
  if (l < K) {
    dz_pos[p] = dz;
    dz_tok[(size_t)t * K + l] = dz;
    if (ds_out) ds_out[(size_t)t * K + l] = dsv;
  }
  constexpr int VPL = 16 / sizeof(TIN);  // values per 16-byte load
  float* orow = accws + (size_t)t * d;
  // every lane runs every pass, so that the shuffles below read slot k's dz
  // and expert from lane k even where d has fewer columns than the wave
  for (int c0 = 0; c0 < d; c0 += 64 * VPL) {
    const int col = c0 + l * VPL;
    const bool in = col < d;
    float acc[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) acc[v] = 0.0f;
    for (int k = 0; k < K; ++k) {
      const float z = __shfl(dz, k, 64);
      const int ek = __shfl(e, k, 64);
      if (!in) continue;
      const TIN* wr = wg + (size_t)ek * d + col;
      if constexpr (sizeof(TIN) == 2) {
        const u32x4_t q = *(const u32x4_t*)wr;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          acc[2 * v] += z * bf16_to_f32(q[v] & 0xffffu);
          acc[2 * v + 1] += z * bf16_to_f32(q[v] >> 16);
        }
      } else {
        const f32x4_t q = *(const f32x4_t*)wr;
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] += z * q[v];
      }
    }
    if (in) {
#pragma unroll
      for (int v = 0; v < VPL; v += 4)
        *(f32x4_t*)(orow + col + v) = f32x4_t{acc[v], acc[v + 1], acc[v + 2], acc[v + 3]};
    }
  }
}

// dWg[e] = sum_{p in e} dz_p x[eti[p]], in two deterministic passes so that
// the work spreads over the expert's rows, not over E workgroups:
//   pass 1: one workgroup per (128-row block g of the GEMM tile map, column
//           block): part[g][c] = sum over the block's rows in ascending order;
//   pass 2: dWg[e][c] = sum of part[g][c] over the expert's blocks, ascending.
template <typename TIN>
__global__ __launch_bounds__(256) void dwg_part_kernel(const TIN* __restrict__ x, const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ eti,
                                                       const int32_t* __restrict__ mb_off,
                                                       const float* __restrict__ dz_pos, float* __restrict__ part,
                                                       int d, int E) {
  constexpr int VPL = 16 / sizeof(TIN);  // values per thread (one 16-byte chunk per row)
  const int g = blockIdx.x;
  if (g >= mb_off[E]) return;
  const RowTile rt = decode_row_tile<TILE_S>(mb_off, offsets, E, g);
  const int col = (blockIdx.y * 256 + (int)threadIdx.x) * VPL;
  if (col >= d) return;
  float acc[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) acc[v] = 0.0f;
  for (int p = rt.r0; p < rt.r1; ++p) {
    const float z = dz_pos[p];
    const TIN* row = x + (size_t)eti[p] * d + col;
    if constexpr (sizeof(TIN) == 2) {
      const u32x4_t q = *(const u32x4_t*)row;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        acc[2 * v] += z * bf16_to_f32(q[v] & 0xffffu);
        acc[2 * v + 1] += z * bf16_to_f32(q[v] >> 16);
      }
    } else {
      const f32x4_t q = *(const f32x4_t*)row;
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] += z * q[v];
    }
  }
  float* o = part + (size_t)g * d + col;
#pragma unroll
  for (int v = 0; v < VPL; v += 4) *(f32x4_t*)(o + v) = f32x4_t{acc[v], acc[v + 1], acc[v + 2], acc[v + 3]};
}

__global__ __launch_bounds__(256) void dwg_reduce_kernel(const float* __restrict__ part,
                                                         const int32_t* __restrict__ mb_off, float* __restrict__ dwg,
                                                         int d) {
  const int e = blockIdx.x;
  const int c = (blockIdx.y * 256 + (int)threadIdx.x) * 4;
  if (c >= d) return;
  f32x4_t acc{0.0f, 0.0f, 0.0f, 0.0f};
  for (int g = mb_off[e]; g < mb_off[e + 1]; ++g) acc += *(const f32x4_t*)(part + (size_t)g * d + c);
  *(f32x4_t*)(dwg + (size_t)e * d + c) = acc;
}

// dWg on MFMA (bf16): dWg = dZ^T X, with dZ [T][E] the router-logit
// gradients, dense: token t's K entries dz[t,k] at columns ids[t,k] and zeros
// elsewhere.  X is read once (as rows of tokens), where the per-position form
// above reads a gathered row for each of the K assignments of a token.
//
// Workgroup (column block nb, expert block eb, token chunk z): the 128 x 128
// tile dWg[eb*128 .., nb*128 ..] summed over the chunk's tokens, 64 at a
// time.  For each 64-token k-tile the A operand (experts x tokens) is built in
// LDS: cleared, then each (token, slot) entry of the tile's experts written
// at [expert][token].  dz enters as two bf16 operands, hi = bf16(dz) and
// lo = bf16(dz - hi), whose products with the bf16 x are exact in the fp32
// accumulation; hi + lo carries dz to about 2^-18.  The B operand (tokens x
// columns of x) is staged k-major and read with the LDS transpose read.  The
// x rows and the ids and dz are loaded two k-tiles ahead, in two register
// sets.  Each chunk's tile goes to part[z]; dwg_mfma_reduce
// sums the chunks in ascending order.
// BM experts per tile (32, 64 or 128: the smallest that holds E, else 128).
template <int BM, int EPT>  // EPT: (token, slot) entries per thread per k-tile, 64 K / 256 rounded up
__global__ __launch_bounds__(256, 2) void dwg_mfma_kernel(const bf16_t* __restrict__ x,
                                                          const int32_t* __restrict__ ids,
                                                          const float* __restrict__ dz_tok, float* __restrict__ part,
                                                          int T, int d, int E, int K, int chunk_tokens) {
  using M = Mfma<bf16_t>;
  using G = KmGeom<128>;
  constexpr int WM = BM >= 64 ? 2 : 1, WN = 4 / WM;  // wave grid
  constexpr int FM = BM / WM / 32, FN = 128 / WN / 32;
  constexpr int A_BYTES = BM * LDS_ROW;
  __shared__ __attribute__((aligned(16))) char smem[2 * A_BYTES + G::BYTES];
  char* s_hi = smem;
  char* s_lo = smem + A_BYTES;
  char* s_b = smem + 2 * A_BYTES;
  const int nb = blockIdx.x, e0 = blockIdx.y * BM, z = blockIdx.z;
  const int t0 = z * chunk_tokens;
  const int t1 = min_i(T, t0 + chunk_tokens);
  const int nkt = (t1 - t0 + 63) / 64;
  const int tid = threadIdx.x, l = lane_id(), wave = tid >> 6, wm = wave / WN, wn = wave % WN;
  // B: k-row r of k-tile kt is token t0 + 64 kt + r, columns nb*128 + 8 cc ..
  const rsrc_t rx = make_rsrc(x + (size_t)t0 * d, (size_t)(t1 - t0) * d * 2);
  const int cc = tid % G::CPR, kr0 = tid / G::CPR;
  const uint32_t col_off = (uint32_t)(nb * 128 + cc * 8) * 2u;
  // entries (token, slot) i = tid + 256 j of the k-tile: ids / dz_tok index t0*K + 64 kt K + i
  const rsrc_t rid = make_rsrc(ids + (size_t)t0 * K, (size_t)(t1 - t0) * K * 4);
  const rsrc_t rdz = make_rsrc(dz_tok + (size_t)t0 * K, (size_t)(t1 - t0) * K * 4);
  // two register sets: k-tile kt's loads go to set kt % 2, two k-tiles ahead
  u32x4_t xb[2][G::NPASS];
  int ide[2][EPT];
  float dze[2][EPT];
  auto load = [&](auto setc, int kt) {
    constexpr int SET = decltype(setc)::value;
#pragma unroll
    for (int i = 0; i < G::NPASS; ++i) {
      const int r = kt * 64 + kr0 + G::RPP * i;
      xb[SET][i] = buf_load16(rx, (uint32_t)r * (uint32_t)d * 2u + col_off);  // past t1: out of range, zeros
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const uint32_t o = (uint32_t)(kt * 64 * K + tid + 256 * j) * 4u;
      ide[SET][j] = (int)buf_load4(rid, o);  // past the chunk: 0, never used
      dze[SET][j] = __builtin_bit_cast(float, buf_load4(rdz, o));
    }
  };
  f32x16_t acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x16_t{};
  const int a_lane = (l & 31) * LDS_ROW + (l >> 5) * 16;  // row l % 32, k-group l / 32
  const int b_lane = km_lane_off(G::PITCH);
  auto tile = [&](auto setc, int kt) {
    constexpr int SET = decltype(setc)::value;
    __syncthreads();  // the previous k-tile's operands have been read
    // clear A (hi and lo): 2 * BM rows of LDS_ROW bytes
    for (int o = tid * 16; o < 2 * A_BYTES; o += 256 * 16) *(u32x4_t*)(smem + o) = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < G::NPASS; ++i) *(u32x4_t*)(s_b + (kr0 + G::RPP * i) * G::PITCH + cc * 16) = xb[SET][i];
    int my_e[EPT];
    float my_z[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      my_e[j] = ide[SET][j];
      my_z[j] = dze[SET][j];
    }
    if (kt + 2 < nkt) load(setc, kt + 2);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int i = tid + 256 * j;
      const int tk = i / K;  // token within the k-tile
      const int e = my_e[j] - e0;
      if (i < 64 * K && t0 + kt * 64 + tk < t1 && e >= 0 && e < BM) {
        const uint32_t hi = f32_to_bf16(my_z[j]);
        const uint32_t lo = f32_to_bf16(my_z[j] - bf16_to_f32(hi));
        *(bf16_t*)(s_hi + e * LDS_ROW + tk * 2) = (bf16_t)hi;
        *(bf16_t*)(s_lo + e * LDS_ROW + tk * 2) = (bf16_t)lo;
      }
    }
    __syncthreads();
#pragma unroll
    for (int st = 0; st < 4; ++st) {  // k-steps of 16 tokens
      typename M::Frag ah[FM], al[FM], b[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int off = a_lane + (wm * (BM / WM) + fm * 32) * LDS_ROW + st * 32;
        ah[fm] = M::lds_read(s_hi + off);
        al[fm] = M::lds_read(s_lo + off);
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        b[fn].v = km_read(s_b + b_lane + st * 16 * G::PITCH + (wn * (128 / WN) + fn * 32) * 2, G::PITCH);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          M::mma(acc[fm][fn], ah[fm], b[fn]);
          M::mma(acc[fm][fn], al[fm], b[fn]);
        }
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  if (nkt > 0) load(S0{}, 0);
  if (nkt > 1) load(S1{}, 1);
  for (int kt = 0; kt < nkt; kt += 2) {
    tile(S0{}, kt);
    if (kt + 1 < nkt) tile(S1{}, kt + 1);
  }
  float* o = part + (size_t)z * E * d;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int c = nb * 128 + wn * (128 / WN) + fn * 32 + frag_col(l);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = e0 + wm * (BM / WM) + fm * 32 + frag_row(r, l);
        if (e < E && c < d) o[(size_t)e * d + c] = acc[fm][fn][r];
      }
    }
}

// dWg[e][c] = sum over the token chunks z of part[z][e][c], in a fixed order:
// a workgroup takes 64 consecutive floats (16 quads) of the n = E*d; its 16
// z-lanes g sum the chunks z = g, g + 16, ... in ascending order, and the 16
// lane sums are added in ascending g.  Many loads in flight per output even
// where n is small and the chunks many.
constexpr int DWG_ZL = 16;
__global__ __launch_bounds__(256) void dwg_mfma_reduce_kernel(const float* __restrict__ part, float* __restrict__ dwg,
                                                              long long n, int nz) {
  __shared__ f32x4_t s_p[DWG_ZL][16];
  const int q = (int)threadIdx.x & 15, g = (int)threadIdx.x >> 4;
  const long long i = (long long)blockIdx.x * 64 + q * 4;
  f32x4_t a{0.0f, 0.0f, 0.0f, 0.0f};
  if (i < n)
    for (int zz = g; zz < nz; zz += DWG_ZL) a += *(const f32x4_t*)(part + (size_t)zz * n + i);
  s_p[g][q] = a;
  __syncthreads();
  if (g == 0 && i < n) {
    f32x4_t r = s_p[0][q];
#pragma unroll
    for (int j = 1; j < DWG_ZL; ++j) r += s_p[j][q];
    *(f32x4_t*)(dwg + i) = r;
  }
}

// dW_down[e] (d x h) = sum_p dO[eti[p]]^T (w_p y[p]): M = d, N = h, K = rows of e.
// Rows [p0, p1) of expert rows [q0, q1) that chunk blockIdx.z of gridDim.z
// reduces: equal chunks, rounded up to whole k-tiles (the last may be short or
// empty; an empty chunk writes a zero partial).
template <int BK>
MOE_DEV void split_rows(int q0, int q1, int& p0, int& p1) {
  const int ns = (int)gridDim.z;
  const int len = ((q1 - q0 + ns - 1) / ns + BK - 1) / BK * BK;
  p0 = min_i(q1, q0 + (int)blockIdx.z * len);
  p1 = min_i(q1, p0 + len);
}

// Tile of a dW GEMM's workgroup.  Workgroups go to the eight XCDs in turn
// (linear block id mod 8), and a dW grid has E (and split) planes of nmb x nnb
// tiles.  With gr x gc = 8 (host-chosen; 0 keeps launch order), XCD x takes the
// row blocks = x / gc (mod gr) and column blocks = x % gc (mod gc) of every
// plane, in row-major order: an XCD's L2 then serves nmb / gr row blocks and
// nnb / gc column blocks of an expert, and each operand block is fetched by gc
// (A) or gr (B) XCDs, not by all eight.  Needs nmb % gr == nnb % gc == 0,
// which also makes the plane size a multiple of 8.
MOE_DEV void dw_tile(int bx, int nmb, int nnb, int gr, int gc, int& mb, int& nb) {
  if (gr == 0) {
    mb = bx / nnb;
    nb = bx % nnb;
    return;
  }
  const int x = bx & 7, j = bx >> 3;  // the XCD of the block and its turn there
  const int cols = nnb / gc;          // column blocks of one XCD
  mb = x / gc + gr * (j / cols);
  nb = x % gc + gc * (j % cols);
}

// dW from its chunk partials [ns][E][M][N]: the sum over chunks in chunk
// order; rows m < M0 of expert e go to out0 ([E][M0][N]), the others to out1
// ([E][M - M0][N]).  Four floats per thread (N is a multiple of 128).
__global__ __launch_bounds__(256) void dw_split_reduce_kernel(const float* __restrict__ part, int ns, long long stride,
                                                              int M, int M0, int N, float* __restrict__ out0,
                                                              float* __restrict__ out1) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= stride) return;
  f32x4_t acc = *(const f32x4_t*)(part + i);
  for (int c = 1; c < ns; ++c) acc += *(const f32x4_t*)(part + (size_t)c * stride + i);
  const long long row = i / N;
  const int n = (int)(i - row * N);
  const long long e = row / M;
  const int m = (int)(row - e * M);
  float* o = m < M0 ? out0 + ((size_t)e * M0 + m) * N + n : out1 + ((size_t)e * (M - M0) + (m - M0)) * N + n;
  *(f32x4_t*)o = acc;
}
static void launch_dw_split_reduce(const float* part, int ns, int E, int M, int M0, int N, float* out0, float* out1,
                                   hipStream_t st) {
  const long long stride = (long long)E * M * N;
  dw_split_reduce_kernel<<<dim3((unsigned)((stride / 4 + 255) / 256)), dim3(256), 0, st>>>(part, ns, stride, M, M0,
                                                                                         N, out0, out1);
}

// The score-scaled activation A' = w_p y[p] is formed while staging the B
// operand and held in the activation dtype, as the SonicMoE analysis page
// (sec. 3.4.1) defines A' = Broadcast(s) A for the dW2 grouped GEMM.
// SCALE: the right-hand rows are y_swi and get the score here; otherwise
// they are A' written by the H-only dH kernel.
template <class C, bool SCALE>
__global__ __launch_bounds__(C::NT, C::WAVES_PER_EU) void dw_down_kernel(
    const typename C::T* __restrict__ dout, const typename C::T* __restrict__ y_swi,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ eti, const float* __restrict__ w_pos,
    float* __restrict__ dw_down, float* __restrict__ part, int T, int d, int h, int gr, int gc) {
  __shared__ __attribute__((aligned(16))) char smem[smem_bytes<C>()];
  using TIN = typename C::T;
  const int nnb = col_blocks(h, C::BN);
  const int e = blockIdx.y;
  int mb, nb;
  dw_tile(blockIdx.x, col_blocks(d, C::BM), nnb, gr, gc, mb, nb);
  int p0, p1;
  split_rows<C::BK>(offsets[e], offsets[e + 1], p0, p1);
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  KSrcLoader<C, C::AKM, C::BM, SrcRowsGather<TIN>, false> la;
  la.src.rs = make_rsrc(dout, (size_t)T * d * sizeof(TIN));
  la.src.ld_bytes = (uint32_t)d * sizeof(TIN);
  la.src.col0 = (uint32_t)(mb * C::BM) * sizeof(TIN);
  la.src.n = p1 - p0;
  la.src.reti = make_rsrc(eti + p0, (size_t)(p1 - p0) * 4);
  la.ncols = min_i(C::BM, d - mb * C::BM);
  KSrcLoader<C, C::BKM, C::BN, SrcRowsContig<TIN>, SCALE> lb;
  lb.src.rs = make_rsrc(y_swi + (size_t)p0 * h, (size_t)(p1 - p0) * h * sizeof(TIN));
  lb.src.ld_bytes = (uint32_t)h * sizeof(TIN);
  lb.src.col0 = (uint32_t)(nb * C::BN) * sizeof(TIN);
  lb.src.n = p1 - p0;
  lb.src.rscl = make_rsrc(w_pos + p0, (size_t)(p1 - p0) * 4);
  lb.ncols = min_i(C::BN, h - nb * C::BN);
  f32x16_t acc[C::FM][C::FN];
  gemm_mainloop<C>(la, lb, (p1 - p0 + C::BK - 1) / C::BK, smem, acc, wm, wn);
  const int l = lane_id();
  // one chunk of a split writes its partial, laid out like dW_down
  float* o = (gridDim.z > 1 ? part + (size_t)blockIdx.z * gridDim.y * d * h : dw_down) + (size_t)e * d * h;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int n = nb * C::BN + C::b_row0(wn, fn) + frag_col(l);
      if (n >= h) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb * C::BM + C::a_row0(wm, fm) + frag_row(r, l);
        if (m < d) __builtin_nontemporal_store(acc[fm][fn][r], &o[(size_t)m * h + n]);  // written once, read later
      }
    }
}

// dW_gate / dW_up [e] (h x d) = sum_p dH[p]^T x[eti[p]]: M = hw (2h gated, h for a
// plain expert, whose W_1 gradient goes to dw_gate), N = d, K = rows of e
template <class C>
__global__ __launch_bounds__(C::NT, C::WAVES_PER_EU) void dw_gate_up_kernel(
    const typename C::T* __restrict__ dh, const typename C::T* __restrict__ x, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ eti, float* __restrict__ dw_gate, float* __restrict__ dw_up, float* __restrict__ part,
    int T, int d, int h, int hw, int gr, int gc) {
  __shared__ __attribute__((aligned(16))) char smem[smem_bytes<C>()];
  using TIN = typename C::T;
  const int nnb = col_blocks(d, C::BN);
  const int e = blockIdx.y;
  int mb, nb;
  dw_tile(blockIdx.x, col_blocks(hw, C::BM), nnb, gr, gc, mb, nb);
  int p0, p1;
  split_rows<C::BK>(offsets[e], offsets[e + 1], p0, p1);
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  KSrcLoader<C, C::AKM, C::BM, SrcRowsContig<TIN>, false> la;
  la.src.rs = make_rsrc(dh + (size_t)p0 * hw, (size_t)(p1 - p0) * hw * sizeof(TIN));
  la.src.ld_bytes = (uint32_t)hw * sizeof(TIN);
  la.src.col0 = (uint32_t)(mb * C::BM) * sizeof(TIN);
  la.src.n = p1 - p0;
  la.ncols = min_i(C::BM, hw - mb * C::BM);
  KSrcLoader<C, C::BKM, C::BN, SrcRowsGather<TIN>, false> lb;
  lb.src.rs = make_rsrc(x, (size_t)T * d * sizeof(TIN));
  lb.src.ld_bytes = (uint32_t)d * sizeof(TIN);
  lb.src.col0 = (uint32_t)(nb * C::BN) * sizeof(TIN);
  lb.src.n = p1 - p0;
  lb.src.reti = make_rsrc(eti + p0, (size_t)(p1 - p0) * 4);
  lb.ncols = min_i(C::BN, d - nb * C::BN);
  f32x16_t acc[C::FM][C::FN];
  gemm_mainloop<C>(la, lb, (p1 - p0 + C::BK - 1) / C::BK, smem, acc, wm, wn);
  const int l = lane_id();
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mb * C::BM + C::a_row0(wm, fm) + frag_row(r, l);
      if (m >= hw) continue;
      // one chunk of a split writes its partial as [E][hw][d]
      float* o = gridDim.z > 1 ? part + (((size_t)blockIdx.z * gridDim.y + e) * hw + m) * d
                 : m < h       ? dw_gate + ((size_t)e * h + m) * d
                               : dw_up + ((size_t)e * h + (m - h)) * d;
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int n = nb * C::BN + C::b_row0(wn, fn) + frag_col(l);
        if (n < d) __builtin_nontemporal_store(acc[fm][fn][r], &o[n]);  // written once: keep it out of L2
      }
    }
}

// dX~ = dH [W_gate; W_up] (M rows of e, N = TILE of d, K = hw: 2h, or h with W_1
// only for a plain expert) + ordered fold into dX
template <class C>
__global__ __launch_bounds__(C::NT, C::WAVES_PER_EU) void dx_fold_kernel(
    const typename C::T* __restrict__ dh, const typename C::T* __restrict__ w_gate,
    const typename C::T* __restrict__ w_up, const int32_t* __restrict__ offsets, const int32_t* __restrict__ eti,
    const int32_t* __restrict__ mb_off, const int32_t* __restrict__ rank_pos, int32_t* turn, float* accws,
    typename C::T* __restrict__ dx, int32_t* counters, int d, int E, int K, int h, int hw, int spin_limit) {
  __shared__ __attribute__((aligned(16))) char smem[smem_bytes<C>()];
  using TIN = typename C::T;
  const int NB = col_blocks(d, C::BN);
  int g, nb;
  if (!claim_fold_tile(counters, smem, mb_off[E], NB, g, nb)) return;
  const RowTile rt = decode_row_tile<C::BM>(mb_off, offsets, E, g);
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  const uint32_t ldh = (uint32_t)hw * sizeof(TIN);
  using LA = RowLoader<C::BM, false, C::NT>;
  LA la;
  la.rs[0] = make_rsrc(dh + (size_t)rt.r0 * hw, (size_t)(rt.r1 - rt.r0) * ldh);
#pragma unroll
  for (int i = 0; i < LA::CPT; ++i) {
    const int r = LA::my_row(i);
    la.roff[i] = rt.r0 + r < rt.r1 ? (uint32_t)r * ldh : OOB_OFF;
  }
  KSrcLoader<C, C::BKM, C::BN, SrcWeightKN2<TIN>, false> lb;
  lb.src.rs1 = make_rsrc(w_gate + (size_t)rt.e * h * d, (size_t)h * d * sizeof(TIN));
  lb.src.rs2 = make_rsrc(w_up + (size_t)rt.e * h * d, (size_t)h * d * sizeof(TIN));
  lb.src.ld_bytes = (uint32_t)d * sizeof(TIN);
  lb.src.col0 = (uint32_t)(nb * C::BN) * sizeof(TIN);
  lb.src.h = h;
  lb.src.kpt = C::BK;
  lb.ncols = min_i(C::BN, d - nb * C::BN);
  f32x16_t acc[C::FM][C::FN];
  gemm_mainloop<C, false>(la, lb, hw / C::BK, smem, acc, wm, wn);
  // fetched after the main loop here: before it, down-combine gained 1% and
  // this kernel lost 0.2-0.5% (MI355X, three workloads)
  const FoldRowMeta meta = C::BM == 128 ? fold_row_meta(rt, eti, nullptr, rank_pos) : FoldRowMeta{};
  fold_epilogue<C, false>(acc, rt, nb, NB, wm, wn, meta, eti, nullptr, rank_pos, K, d, turn, accws, dx,
                          counters + ERR_BWD, spin_limit, smem);
}

// MOE_DISPATCH_DW_XCD=0 keeps the dW GEMMs' tiles in launch order (tuning aid).
static bool dw_xcd_map_on() {
  static int v = [] {
    const char* e = getenv("MOE_DISPATCH_DW_XCD");
    return e ? (atoi(e) ? 1 : 0) : 1;
  }();
  return v == 1;
}
// XCD grid gr x gc = 8 for a dW GEMM of nmb x nnb tiles per expert: the one
// that fetches the fewest operand bytes into the eight L2s, gc * a_bytes +
// gr * b_bytes (a_bytes, b_bytes: an expert's A and B operands), among those
// dividing the tile grid; {0, 0} (launch order) if none does.
static void dw_xcd_grid(int nmb, int nnb, double a_bytes, double b_bytes, int& gr, int& gc) {
  gr = gc = 0;
  if (!dw_xcd_map_on()) return;
  double best = 0.0;
  for (int r = 1; r <= 8; r *= 2) {
    const int c = 8 / r;
    if (nmb % r || nnb % c) continue;
    const double cost = c * a_bytes + r * b_bytes;
    if (gr == 0 || cost < best) {
      best = cost;
      gr = r;
      gc = c;
    }
  }
}

template <typename TIN, int BM, int BN, bool HONLY>
static void launch_dh(const Shape& s, const void* dout, const void* w_down, const void* h_ab, const void* y_swi,
                      void* a_prime, const int32_t* offsets, const int32_t* eti, const ExpertWs& ws, hipStream_t st) {
  using C = KCfg<TIN, BM, BN, false, true>;
  const int nbn = col_blocks(s.h, BN);
  const long long nblk = (max_row_blocks(s, BM) * nbn + 7) / 8 * 8;
  const TileOrder to = tile_order(nblk, nbn);
  dh_kernel<C, HONLY><<<dim3((unsigned)nblk), dim3(C::NT), 0, st>>>(
      (const TIN*)dout, (const TIN*)w_down, (const TIN*)h_ab, (const TIN*)y_swi, offsets, eti, ws.tile_map(BM),
      ws.w_pos, (TIN*)ws.dh, ws.ds_part, (TIN*)a_prime, s.T, s.d, s.E, s.h, s.act, nbn, to.nblk,
      to.grp, to.xg);
}

template <typename TIN, int BM, int BN>
static void launch_dx_fold(const Shape& s, const void* w_gate, const void* w_up, const int32_t* offsets,
                           const int32_t* eti, void* dx, const ExpertWs& ws, int spin_limit, hipStream_t st) {
  using C = KCfg<TIN, BM, BN, false, true>;
  const long long nblk = max_row_blocks(s, BM) * col_blocks(s.d, BN);
  dx_fold_kernel<C><<<dim3((unsigned)nblk), dim3(C::NT), 0, st>>>(
      (const TIN*)ws.dh, (const TIN*)w_gate, (const TIN*)w_up, offsets, eti, ws.tile_map(BM), ws.rank_pos, ws.turn,
      ws.acc, (TIN*)dx, ws.counters, s.d, s.E, s.K, s.h, s.hw(), spin_limit);
}

template <typename TIN>
static hipError_t backward_t(const Shape& s, const void* dout, const void* x, const void* wg, const void* w_gate,
                             const void* w_up, const void* w_down, const int32_t* ids, const float* topk_w,
                             const int32_t* offsets, const int32_t* eti, const int32_t* tim, const void* h_ab,
                             const void* y_swi, void* a_prime, void* dx, float* dwg, float* dw_gate, float* dw_up,
                             float* dw_down, float* ds, const ExpertWs& ws, int spin_limit, hipStream_t st) {
  // H-only: A' goes to the caller's buffer when one is passed, else to the workspace
  void* ap = a_prime ? a_prime : ws.a_prime;
  using CL = KCfg<TIN, TILE_L, TILE_L, true, true>;
  // dH on the 256 x 256 tile measured no faster on MI355X (4.23 vs 4.21 ms at
  // d = 4096, h = 14336; 0.88 vs 0.75 ms at d = 2048, h = 1536): the small
  // tile is used unless the large one is forced.  The 128 x 256 tile pays
  // only for a long reduction (d): 4.28 -> 4.05 ms at d = 6144, h = 2048, but
  // 3-9% slower at d = 2048-4096.
  const bool dh_big = forced_tile() == TILE_L;
  const bool dh_mid = pick_mid(s, s.d >= 6144);
  const int nbh = col_blocks(s.h, dh_big || dh_mid ? TILE_L : TILE_S);
  hipError_t err;
  timing_mark(st, "dh", true);
  const bool honly = y_swi == nullptr;
  if (dh_big) {
    if (honly) launch_dh<TIN, TILE_L, TILE_L, true>(s, dout, w_down, h_ab, y_swi, ap, offsets, eti, ws, st);
    else launch_dh<TIN, TILE_L, TILE_L, false>(s, dout, w_down, h_ab, y_swi, ap, offsets, eti, ws, st);
  } else if (dh_mid) {
    if constexpr (sizeof(TIN) == 2) {
      if (honly) launch_dh<TIN, TILE_S, TILE_L, true>(s, dout, w_down, h_ab, y_swi, ap, offsets, eti, ws, st);
      else launch_dh<TIN, TILE_S, TILE_L, false>(s, dout, w_down, h_ab, y_swi, ap, offsets, eti, ws, st);
    }
  } else {
    if (honly) launch_dh<TIN, TILE_S, TILE_S, true>(s, dout, w_down, h_ab, y_swi, ap, offsets, eti, ws, st);
    else launch_dh<TIN, TILE_S, TILE_S, false>(s, dout, w_down, h_ab, y_swi, ap, offsets, eti, ws, st);
  }
  timing_mark(st, "dh", false);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  timing_mark(st, "router_bwd", true);
  router_bwd_kernel<TIN><<<dim3((s.T + RB_TOKENS - 1) / RB_TOKENS), dim3(64 * RB_TOKENS), 0, st>>>(
      ids, topk_w, tim, ws.ds_part, nbh, (const TIN*)wg, ws.dz_pos, ws.dz_tok, ds, ws.acc, s.T, s.d, s.K);
  timing_mark(st, "router_bwd", false);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  timing_mark(st, "dwg", true);
  if constexpr (sizeof(TIN) == 2) {
    const int ct = dwg_chunk_tokens(s), nz = dwg_chunks(s);
    const int bm = dwg_expert_tile(s);
    const dim3 grid(col_blocks(s.d, 128), (s.E + bm - 1) / bm, nz);
    const int ept = (64 * s.K + 255) / 256;
    auto go = [&](auto bmc) {
      constexpr int BM = decltype(bmc)::value;
      auto run = [&](auto kern) {
        kern<<<grid, dim3(256), 0, st>>>((const bf16_t*)x, ids, ws.dz_tok, ws.dwg_part, s.T, s.d, s.E, s.K, ct);
      };
      if (ept <= 1) run(dwg_mfma_kernel<BM, 1>);
      else if (ept <= 2) run(dwg_mfma_kernel<BM, 2>);
      else if (ept <= 4) run(dwg_mfma_kernel<BM, 4>);
      else run(dwg_mfma_kernel<BM, 8>);
    };
    if (bm == 32) go(std::integral_constant<int, 32>{});
    else if (bm == 64) go(std::integral_constant<int, 64>{});
    else go(std::integral_constant<int, 128>{});
    const long long n = (long long)s.E * s.d;
    dwg_mfma_reduce_kernel<<<dim3((unsigned)((n + 63) / 64)), dim3(256), 0, st>>>(ws.dwg_part, dwg, n, nz);
  } else {
    constexpr int VPL = 16 / sizeof(TIN);
    const int ncb = (s.d + 256 * VPL - 1) / (256 * VPL);
    dwg_part_kernel<TIN><<<dim3((unsigned)max_row_blocks(s, TILE_S), ncb), dim3(256), 0, st>>>(
        (const TIN*)x, offsets, eti, ws.tile_map(TILE_S), ws.dz_pos, ws.dwg_part, s.d, s.E);
    dwg_reduce_kernel<<<dim3(s.E, (s.d + 1023) / 1024), dim3(256), 0, st>>>(ws.dwg_part, ws.tile_map(TILE_S), dwg,
                                                                           s.d);
  }
  timing_mark(st, "dwg", false);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  timing_mark(st, "dw_down", true);
  {
    const int ns = dw_down_split(s);
    const int nmb = col_blocks(s.d, CL::BM), nnb = col_blocks(s.h, CL::BN);
    int gr, gc;  // A: dO rows (d columns), B: A' rows (h columns)
    dw_xcd_grid(nmb, nnb, (double)s.d, (double)s.h, gr, gc);
    const dim3 grid(nmb * nnb, s.E, ns);
    if (honly)
      dw_down_kernel<CL, false><<<grid, dim3(CL::NT), 0, st>>>((const TIN*)dout, (const TIN*)ap, offsets, eti,
                                                               ws.w_pos, dw_down, ws.dw_part, s.T, s.d, s.h, gr, gc);
    else
      dw_down_kernel<CL, true><<<grid, dim3(CL::NT), 0, st>>>((const TIN*)dout, (const TIN*)y_swi, offsets, eti,
                                                              ws.w_pos, dw_down, ws.dw_part, s.T, s.d, s.h, gr, gc);
    if (ns > 1) launch_dw_split_reduce(ws.dw_part, ns, s.E, s.d, s.d, s.h, dw_down, nullptr, st);
  }
  timing_mark(st, "dw_down", false);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  timing_mark(st, "dw_gate_up", true);
  {
    const int ns = dw_gate_up_split(s);
    const int nmb = col_blocks(s.hw(), CL::BM), nnb = col_blocks(s.d, CL::BN);
    int gr, gc;  // A: dH rows (hw columns), B: gathered x rows (d columns)
    dw_xcd_grid(nmb, nnb, (double)s.hw(), (double)s.d, gr, gc);
    dw_gate_up_kernel<CL><<<dim3(nmb * nnb, s.E, ns), dim3(CL::NT), 0, st>>>(
        (const TIN*)ws.dh, (const TIN*)x, offsets, eti, dw_gate, dw_up, ws.dw_part, s.T, s.d, s.h, s.hw(), gr, gc);
    if (ns > 1) launch_dw_split_reduce(ws.dw_part, ns, s.E, s.hw(), s.h, s.d, dw_gate, dw_up, st);
  }
  timing_mark(st, "dw_gate_up", false);
  if ((err = hipGetLastError()) != hipSuccess) return err;

  timing_mark(st, "dx_fold", true);
  // a plain expert has no up projection: its k never reaches h, so the second
  // weight slot is never read
  const void* w2 = s.gated() ? w_up : w_gate;
  if constexpr (sizeof(TIN) == 2) {
    if (wide_fold(s, s.hw(), true)) launch_dx_fold<TIN, TILE_L, TILE_L>(s, w_gate, w2, offsets, eti, dx, ws, spin_limit, st);
    else if (mid_fold(s, s.hw(), true)) launch_dx_fold<TIN, TILE_S, TILE_L>(s, w_gate, w2, offsets, eti, dx, ws, spin_limit, st);
    else launch_dx_fold<TIN, TILE_S, TILE_S>(s, w_gate, w2, offsets, eti, dx, ws, spin_limit, st);
  } else {
    launch_dx_fold<TIN, TILE_S, TILE_S>(s, w_gate, w2, offsets, eti, dx, ws, spin_limit, st);
  }
  timing_mark(st, "dx_fold", false);
  return hipGetLastError();
}

hipError_t launch_backward(const Shape& s, const void* dout, const void* x, const void* wg, const void* w_gate,
                           const void* w_up, const void* w_down, const int32_t* ids, const float* topk_w,
                           const int32_t* offsets, const int32_t* eti, const int32_t* tim, const void* h_ab,
                           const void* y_swi, void* a_prime, void* dh, void* dx, float* dwg, float* dw_gate,
                           float* dw_up, float* dw_down, float* ds, const ExpertWs& ws, int spin_limit,
                           hipStream_t st) {
  // dH goes to the caller's buffer when one is passed (possibly h_ab itself:
  // the dH kernel reads each element of H before it writes the gradient
  // element at the same place, and nothing after it reads H), else to the
  // workspace
  ExpertWs w = ws;
  if (dh) w.dh = dh;
  if (s.bf16)
    return backward_t<bf16_t>(s, dout, x, wg, w_gate, w_up, w_down, ids, topk_w, offsets, eti, tim, h_ab, y_swi,
                              a_prime, dx, dwg, dw_gate, dw_up, dw_down, ds, w, spin_limit, st);
  return backward_t<float>(s, dout, x, wg, w_gate, w_up, w_down, ids, topk_w, offsets, eti, tim, h_ab, y_swi,
                           a_prime, dx, dwg, dw_gate, dw_up, dw_down, ds, w, spin_limit, st);
}

}  // namespace moe
