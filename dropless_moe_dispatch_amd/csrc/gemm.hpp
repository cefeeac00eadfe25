// Generic grouped-GEMM core for the expert projections (gfx950 MFMA).
//
// One workgroup = 256 threads = 4 wave64s, computing a BM x BN fp32 tile of
// C = A * B^T where both operands are staged in LDS as [row][k] (k
// contiguous), 128 bytes of k per row per stage (64 bf16 or 32 fp32), rows
// padded to 144 bytes so that the 16-byte MFMA operand reads of 8 lanes hit
// distinct banks.  Two LDS stages: the global loads of k-tile t+1 are issued
// before the MFMAs of tile t and written to the other stage afterwards, one
// barrier per k-tile.
//
// Operand sources:
//   RowLoader  - rows that are contiguous in k in global memory (activations
//                [rows, k] gathered through an index, weights [out, in]).
//                8 consecutive threads fetch one row's 128-byte slice.
//   KRowLoader - sources whose rows are k (activations [rows, m] reduced over
//                rows, or weights [k, n]).  Each thread fetches four k-rows of
//                one 16-byte column chunk and transposes them in registers so
//                that LDS still holds [m][k].
#pragma once
#include "common.hpp"

namespace moe {

constexpr int NTHREADS = 256;
constexpr int LDS_ROW = 144;
constexpr int KBYTES = 128;

template <typename TIN, int BM_, int BN_, int WM_, int WN_, bool PAIRED_ = false>
struct Cfg {
  using T = TIN;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr bool PAIRED = PAIRED_;   // B rows [0,BN/2) and [BN/2,BN) pair up column-wise
  static constexpr int EB = (int)sizeof(TIN);
  static constexpr int BK = KBYTES / EB;
  static constexpr int FM = BM / WM / 32;
  static constexpr int FN = BN / WN / 32;
  static constexpr int A_BYTES = BM * LDS_ROW;
  static constexpr int B_BYTES = BN * LDS_ROW;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static_assert(WM * WN == 4, "four waves per workgroup");
  static_assert(FM >= 1 && FN >= 1 && FM * WM * 32 == BM && FN * WN * 32 == BN, "tile shape");
  static_assert(!PAIRED || (FN == 2 && WN * 32 * 2 == BN), "paired layout");

  // tile-local row of A fragment fm for this wave
  static MOE_DEV int a_row0(int wm, int fm) { return wm * (BM / WM) + fm * 32; }
  // tile-local column (B row) of fragment fn for this wave
  static MOE_DEV int b_row0(int wn, int fn) {
    if constexpr (PAIRED) return fn * (BN / 2) + wn * 32;
    else return wn * (BN / WN) + fn * 32;
  }
};

// ---------------------------------------------------------------------------
// RowLoader<ROWS>: ROWS tile rows, each a 128-byte k-slice per stage.
// The caller sets row_ptr[i] (byte pointer to the row's first element, or
// nullptr for a row outside the problem -> zeros) for the rows this thread
// owns: row = (tid >> 3) + 32*i, i < ROWS/32.
// ---------------------------------------------------------------------------
template <int ROWS>
struct RowLoader {
  static constexpr int CPT = ROWS / 32;
  const char* row_ptr[CPT];
  u32x4_t reg[CPT];

  static MOE_DEV int my_row(int i) { return (int)(threadIdx.x >> 3) + 32 * i; }

  MOE_DEV void load(int kt) {
    const int off = kt * KBYTES + (int)(threadIdx.x & 7) * 16;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      if (row_ptr[i]) reg[i] = *(const u32x4_t*)(row_ptr[i] + off);
      else reg[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  MOE_DEV void store(char* lds) const {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      *(u32x4_t*)(lds + my_row(i) * LDS_ROW + (threadIdx.x & 7) * 16) = reg[i];
  }
};

// ---------------------------------------------------------------------------
// KRowLoader<T, Src>: 128 tile rows (m), k-rows from a source functor.
//   Src::ptr(krow, scale&) -> byte pointer to element (krow, col0) or nullptr,
//   with an optional per-k-row scale (1.0f when unused).
// bf16: thread owns k-rows 4*(tid&15)+0..3, columns 8*(tid>>4)+0..7.
// fp32: thread owns k-rows 4*(tid&7)+0..3,  columns 4*(tid>>3)+0..3.
// ---------------------------------------------------------------------------
template <typename T, class Src, bool SCALED>
struct KRowLoader;

template <class Src, bool SCALED>
struct KRowLoader<bf16_t, Src, SCALED> {
  Src src;
  u32x4_t reg[4];
  float scl[4];
  MOE_DEV int kg() const { return (int)(threadIdx.x & 15); }
  MOE_DEV int mc() const { return (int)(threadIdx.x >> 4); }

  MOE_DEV void load(int kt) {
    const int kbase = kt * 64 + 4 * kg();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = 1.0f;
      const char* p = src.ptr(kbase + j, s);
      scl[j] = s;
      if (p) reg[j] = *(const u32x4_t*)(p + mc() * 16);
      else reg[j] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  MOE_DEV void store(char* lds) const {
    u32x4_t r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] = reg[j];
      if constexpr (SCALED) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t v = r[j][q];
          const uint32_t lo = f32_to_bf16(bf16_to_f32(v & 0xffffu) * scl[j]);
          const uint32_t hi = f32_to_bf16(bf16_to_f32(v >> 16) * scl[j]);
          r[j][q] = lo | (hi << 16);
        }
      }
    }
    char* base = lds + (mc() * 8) * LDS_ROW + kg() * 8;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // columns 2q (low halves) and 2q+1 (high halves)
      u32x2_t e, o;
      e[0] = (r[0][q] & 0xffffu) | (r[1][q] << 16);
      e[1] = (r[2][q] & 0xffffu) | (r[3][q] << 16);
      o[0] = (r[0][q] >> 16) | (r[1][q] & 0xffff0000u);
      o[1] = (r[2][q] >> 16) | (r[3][q] & 0xffff0000u);
      *(u32x2_t*)(base + (2 * q) * LDS_ROW) = e;
      *(u32x2_t*)(base + (2 * q + 1) * LDS_ROW) = o;
    }
  }
};

template <class Src, bool SCALED>
struct KRowLoader<float, Src, SCALED> {
  Src src;
  f32x4_t reg[4];
  MOE_DEV int kg() const { return (int)(threadIdx.x & 7); }
  MOE_DEV int mc() const { return (int)(threadIdx.x >> 3); }

  MOE_DEV void load(int kt) {
    const int kbase = kt * 32 + 4 * kg();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = 1.0f;
      const char* p = src.ptr(kbase + j, s);
      if (p) {
        reg[j] = *(const f32x4_t*)(p + mc() * 16);
        if constexpr (SCALED) reg[j] *= s;
      } else {
        reg[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  MOE_DEV void store(char* lds) const {
    char* base = lds + (mc() * 4) * LDS_ROW + kg() * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4_t v{reg[0][q], reg[1][q], reg[2][q], reg[3][q]};
      *(f32x4_t*)(base + q * LDS_ROW) = v;
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA over one LDS stage.
// ---------------------------------------------------------------------------
template <class C>
MOE_DEV void mma_stage(const char* stage, f32x16_t (&acc)[C::FM][C::FN], int wm, int wn) {
  using M = Mfma<typename C::T>;
  const int l = lane_id();
  constexpr int STEP = 16 * C::EB;            // bytes of k per MFMA step
  constexpr int NSTEP = KBYTES / STEP;
  const char* a_base = stage + (l & 31) * LDS_ROW + (l >> 5) * (8 * C::EB);
  const char* b_base = stage + C::A_BYTES + (l & 31) * LDS_ROW + (l >> 5) * (8 * C::EB);
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    typename M::Frag a[C::FM], b[C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) a[fm] = M::lds_read(a_base + C::a_row0(wm, fm) * LDS_ROW + s * STEP);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) b[fn] = M::lds_read(b_base + C::b_row0(wn, fn) * LDS_ROW + s * STEP);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) M::mma(acc[fm][fn], a[fm], b[fn]);
  }
}

template <class C, class LA, class LB>
MOE_DEV void gemm_mainloop(LA& la, LB& lb, int nk, char* smem, f32x16_t (&acc)[C::FM][C::FN], int wm, int wn) {
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;
  if (nk <= 0) return;
  la.load(0);
  lb.load(0);
  la.store(smem);
  lb.store(smem + C::A_BYTES);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * C::STAGE;
    char* nxt = smem + ((kt + 1) & 1) * C::STAGE;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(kt + 1);
      lb.load(kt + 1);
    }
    mma_stage<C>(cur, acc, wm, wn);
    if (more) {
      la.store(nxt);
      lb.store(nxt + C::A_BYTES);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Varlen-M tile decode: global row-block g -> expert e and its row range,
// from the per-expert exclusive prefix of row-block counts mb_off[0..E].
// ---------------------------------------------------------------------------
MOE_DEV int find_expert(const int32_t* __restrict__ mb_off, int E, int g) {
  int lo = 0, hi = E;        // invariant: mb_off[lo] <= g, answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mb_off[mid] <= g) lo = mid; else hi = mid;
  }
  return lo;
}

struct RowTile {
  int e;       // expert
  int r0, r1;  // rows [r0, r1) in expert-sorted position space
};

template <int BM>
MOE_DEV RowTile decode_row_tile(const int32_t* __restrict__ mb_off, const int32_t* __restrict__ offsets, int E, int g) {
  RowTile t;
  t.e = find_expert(mb_off, E, g);
  t.r0 = offsets[t.e] + (g - mb_off[t.e]) * BM;
  const int end = offsets[t.e + 1];
  t.r1 = (t.r0 + BM < end) ? t.r0 + BM : end;
  return t;
}

// Map a linear tile id to an id such that consecutive ids land on the same
// XCD (the dispatcher hands consecutive workgroup ids to the 8 XCDs in turn).
MOE_DEV int xcd_swizzle(int bid, int nblk) {
  const int per = nblk >> 3;  // nblk is padded to a multiple of 8 by the launcher
  return (bid & 7) * per + (bid >> 3);
}

}  // namespace moe
