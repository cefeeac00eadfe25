// Generic grouped-GEMM core for the expert projections (gfx950 MFMA).
//
// One workgroup computes a BM x BN fp32 tile of C = A * B^T with
// v_mfma_f32_32x32x16_bf16 (32x32x2 in fp32).  Tiles:
//   128 x 128: four waves of 64 x 64, two workgroups per CU;
//   128 x 256 (bf16): eight waves of 64 x 64, one workgroup per CU, two waves
//     per SIMD;
//   256 x 256 (bf16): eight waves of 64 x 128, one workgroup per CU, two waves
//     per SIMD; in fp32 four waves of 128 x 128.
// Operands are staged in LDS two k-tiles deep, 128 bytes of k per row per
// stage, either [row][k] (k contiguous, rows padded to 144 bytes so that the
// 16-byte operand reads of eight lanes hit distinct banks) or k-major (rows
// padded by 64 bytes, MFMA operands formed by the LDS transpose read).
//
// Pipeline: two LDS stages, one barrier per k-tile.  Global loads go through
// registers (two sets on the 128-row tiles, one on the 256 tile) and are written to
// the free stage between the MFMA k-steps (on the 256 tile after the last one,
// with the next load issued right after, except in the dX fold).  Loaders whose rows come through an
// index (gathered k-rows of the weight-gradient GEMMs) fetch the indices one
// stage ahead and form the byte offsets only when they load.
//
// Operand sources:
//   RowLoader  - rows that are contiguous in k in global memory (activations
//                [rows, k] gathered through an index, weights [out, in]).
//                8 consecutive threads fetch one row's 128-byte slice.
//   KLoader    - sources whose rows are k (weights read as [k][n], activations
//                reduced over rows), staged k-major as they are (bf16).
//   KRowLoader - the same sources in fp32, transposed in registers so that
//                LDS holds [m][k].
#pragma once
#include <type_traits>

#include "common.hpp"

namespace moe {

constexpr int NTHREADS = 256;
constexpr int LDS_ROW = 144;
constexpr int KBYTES = 128;

// k-major LDS layout (bf16 only): the stage holds 64 k-rows of ROWS
// elements, each k-row padded to PITCH bytes; MFMA operands are read from it
// with the LDS transpose read (ds_read_b64_tr_b16).
constexpr int KM_PAD = 64;  // 64 banks: the four k-rows of a transpose read land on disjoint banks
template <int ROWS, int NT = NTHREADS>
struct KmGeom {
  static constexpr int PITCH = ROWS * 2 + KM_PAD;
  static constexpr int BYTES = 64 * PITCH;
  static constexpr int CPR = ROWS / 8;          // 16-byte chunks per k-row
  static constexpr int RPP = NT / CPR;          // k-rows per pass of the workgroup
  static constexpr int NPASS = 64 / RPP;        // chunks per thread per stage
};

template <typename TIN, int BM_, int BN_, int WM_, int WN_, bool PAIRED_ = false, bool AKM_ = false,
          bool BKM_ = false, int NSETS_ = 0>
struct Cfg {
  using T = TIN;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  // PAIRED: B rows [0,BN/2) and [BN/2,BN) pair up column by column, and each
  // wave holds both halves of its columns (fragments fn and fn + FN/2).
  static constexpr bool PAIRED = PAIRED_;
  // AKM / BKM: the operand is staged k-major (see KmGeom) instead of [row][k]
  static constexpr bool AKM = AKM_, BKM = BKM_;
  static constexpr int EB = (int)sizeof(TIN);
  static_assert(!(AKM || BKM) || EB == 2, "k-major staging is bf16 only");
  static constexpr int BK = KBYTES / EB;
  static constexpr int FM = BM / WM / 32;
  static constexpr int FN = BN / WN / 32;
  static constexpr int A_BYTES = AKM ? KmGeom<BM>::BYTES : BM * LDS_ROW;
  static constexpr int B_BYTES = BKM ? KmGeom<BN>::BYTES : BN * LDS_ROW;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGE;
  // workgroup size follows the wave grid: 4 waves, or 8 with two waves per
  // SIMD (a 256 x 256 tile with 64 x 128 per wave, or 128 x 256 with 64 x 64)
  static constexpr int NT = WM * WN * 64;
  static constexpr int WAVES_PER_EU = (BM * BN >= 256 * 256) ? NT / 256 : 2;
  // register sets for staging global loads (the 256 x 256 tile has no room for two)
  static constexpr int NSETS = NSETS_ ? NSETS_ : (BM * BN >= 256 * 256) ? 1 : 2;
  static_assert(WM * WN == 4 || (WM * WN == 8 && BM * BN >= 128 * 256), "four or eight waves per workgroup");
  static_assert(FM >= 1 && FN >= 1 && FM * WM * 32 == BM && FN * WN * 32 == BN, "tile shape");
  static_assert(!PAIRED || (FN % 2 == 0), "paired layout");

  // tile-local row of A fragment fm for this wave
  static MOE_DEV int a_row0(int wm, int fm) { return wm * (BM / WM) + fm * 32; }
  // tile-local column (B row) of fragment fn for this wave
  static MOE_DEV int b_row0(int wn, int fn) {
    if constexpr (PAIRED) {
      constexpr int H = FN / 2;
      return (fn >= H ? BN / 2 : 0) + wn * (BN / 2 / WN) + (fn % H) * 32;
    } else {
      return wn * (BN / WN) + fn * 32;
    }
  }
};

// ---------------------------------------------------------------------------
// Buffer-resource loads.  Every operand fetch is a 16-byte buffer load from a
// resource descriptor held in SGPRs with a 32-bit byte offset; an offset at or
// beyond the descriptor's size returns zeros, which is how rows and columns
// outside the problem are masked (OOB_OFF), without branches around loads.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t OOB_OFF = 0x80000000u;

MOE_DEV rsrc_t make_rsrc(const void* base, size_t bytes) {
  const int n = bytes > 0x7ffffff0ull ? 0x7ffffff0 : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
MOE_DEV u32x4_t buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
MOE_DEV uint32_t buf_load4(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// ---------------------------------------------------------------------------
// RowLoader<ROWS, SPLIT>: ROWS tile rows, each a 128-byte k-slice per stage.
// The caller sets rs[0] (and rs[1] for the second half of the rows when
// SPLIT) and roff[i], the byte offset of the row's first element, or OOB_OFF
// for a row outside the problem, for the rows this thread owns:
// row = (tid >> 3) + (NT/8)*i, i < CPT.
// ---------------------------------------------------------------------------
template <int ROWS, bool SPLIT = false, int NT = NTHREADS>
struct RowLoader {
  static constexpr int RPP = NT / 8;     // rows per pass of the workgroup
  static constexpr int CPT = ROWS / RPP;
  rsrc_t rs[2];
  uint32_t roff[CPT];
  u32x4_t reg[2][CPT];  // two register sets: k-tile j lives in set j % 2

  static MOE_DEV int my_row(int i) { return (int)(threadIdx.x >> 3) + RPP * i; }

  MOE_DEV void prefetch(int) {}
  template <int SET>
  MOE_DEV void load(int kt) {
    const uint32_t off = (uint32_t)(kt * KBYTES) + (threadIdx.x & 7) * 16;
#pragma unroll
    for (int i = 0; i < CPT; ++i) reg[SET][i] = buf_load16(rs[(SPLIT && i >= CPT / 2) ? 1 : 0], roff[i] + off);
  }
  // chunks i with i % NPART == PART
  template <int SET, int PART, int NPART>
  MOE_DEV void store(char* lds) const {
#pragma unroll
    for (int i = PART; i < CPT; i += NPART)
      *(u32x4_t*)(lds + my_row(i) * LDS_ROW + (threadIdx.x & 7) * 16) = reg[SET][i];
  }
};

// ---------------------------------------------------------------------------
// KRowLoader<T, ROWS, Src, SCALED>: ROWS tile rows (m), k-rows from a source:
//   Src::rsrc(kt)        -> buffer resource of k-tile kt (uniform);
//   Src::key(k)          -> what locates k-row k and must come from memory
//                           (a gathered row index), 0 if nothing does;
//   Src::row_off(k, key) -> byte offset of element (k-row k, tile column 0),
//                           or OOB_OFF outside the problem;
//   Src::scale(k)        -> per-k-row scale, 0 outside the problem (SCALED only).
// ncols: valid tile columns (multiple of the chunk width); others read 0.
// prefetch(kt) fetches the keys (and scales) of k-tile kt and load(kt)
// issues the data loads.  The byte offsets are formed only in load(): a
// prefetch that already multiplied its freshly loaded index would make the
// compiler wait for that load, and for the data loads queued before it,
// right where it is issued.
// bf16: thread owns k-rows 4*(tid&15)+0..3, columns c*128 + 8*(tid>>4)+0..7.
// fp32: thread owns k-rows 4*(tid&7)+0..3,  columns c*128 + 4*(tid>>3)+0..3.
// ---------------------------------------------------------------------------
template <typename T> struct KRowGeom;
template <> struct KRowGeom<bf16_t> {
  static MOE_DEV int kg() { return (int)(threadIdx.x & 15); }
  static MOE_DEV int mc() { return (int)(threadIdx.x >> 4); }
  static constexpr int KPT = 64;  // k-rows per stage
  static constexpr int CW = 8;    // columns per chunk
};
template <> struct KRowGeom<float> {
  static MOE_DEV int kg() { return (int)(threadIdx.x & 7); }
  static MOE_DEV int mc() { return (int)(threadIdx.x >> 3); }
  static constexpr int KPT = 32;
  static constexpr int CW = 4;
};

template <typename T, int ROWS, class Src, bool SCALED>
struct KRowLoader {
  using G = KRowGeom<T>;
  static constexpr int NC = ROWS / 128;  // column chunks per thread
  Src src;
  int ncols;
  uint32_t keys[4];
  float spre[4];         // scales fetched with the keys
  float sdat[2][4];      // scales of the loaded data, per register set
  u32x4_t reg[2][NC][4];

  MOE_DEV int col(int c) const { return c * 128 + G::mc() * G::CW; }

  MOE_DEV void prefetch(int kt) {
    const int kbase = kt * G::KPT + 4 * G::kg();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      keys[j] = src.key(kbase + j);
      if constexpr (SCALED) spre[j] = src.scale(kbase + j);
    }
  }
  template <int SET>
  MOE_DEV void load(int kt) {
    const rsrc_t r = src.rsrc(kt);
    const int kbase = kt * G::KPT + 4 * G::kg();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (SCALED) sdat[SET][j] = spre[j];
      const uint32_t off = src.row_off(kbase + j, keys[j]);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint32_t o = col(c) < ncols ? off + (uint32_t)(col(c) * (int)sizeof(T)) : OOB_OFF;
        reg[SET][c][j] = buf_load16(r, o);
      }
    }
  }
  // the register transpose writes a whole chunk column at once: all in part 0
  template <int SET, int PART, int NPART>
  MOE_DEV void store(char* lds) const {
    if constexpr (PART != 0) return;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if constexpr (sizeof(T) == 2) {
        u32x4_t r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          r[j] = reg[SET][c][j];
          if constexpr (SCALED) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t v = r[j][q];
              r[j][q] = pack_bf16x2(bf16_to_f32(v & 0xffffu) * sdat[SET][j], bf16_to_f32(v >> 16) * sdat[SET][j]);
            }
          }
        }
        char* base = lds + col(c) * LDS_ROW + G::kg() * 8;
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
      } else {
        f32x4_t r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          r[j] = __builtin_bit_cast(f32x4_t, reg[SET][c][j]);
          if constexpr (SCALED) r[j] *= sdat[SET][j];
        }
        char* base = lds + col(c) * LDS_ROW + G::kg() * 16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4_t v{r[0][q], r[1][q], r[2][q], r[3][q]};
          *(f32x4_t*)(base + q * LDS_ROW) = v;
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// KLoader<ROWS, Src, SCALED> (bf16): the same sources as KRowLoader, staged
// k-major without any transpose: thread t copies the 16-byte chunk
// (t % CPR) of k-rows t / CPR + RPP * i into LDS as is.  The transpose
// happens in the LDS read that forms the MFMA operand.
// ---------------------------------------------------------------------------
template <int ROWS, class Src, bool SCALED, int NT = NTHREADS>
struct KLoader {
  using G = KmGeom<ROWS, NT>;
  Src src;
  int ncols;
  uint32_t keys[G::NPASS];
  float spre[G::NPASS];
  float sdat[2][G::NPASS];
  u32x4_t reg[2][G::NPASS];

  static MOE_DEV int cc() { return (int)threadIdx.x % G::CPR; }
  static MOE_DEV int kr(int i) { return (int)threadIdx.x / G::CPR + G::RPP * i; }

  MOE_DEV void prefetch(int kt) {
#pragma unroll
    for (int i = 0; i < G::NPASS; ++i) {
      keys[i] = src.key(kt * 64 + kr(i));
      if constexpr (SCALED) spre[i] = src.scale(kt * 64 + kr(i));
    }
  }
  template <int SET>
  MOE_DEV void load(int kt) {
    const rsrc_t r = src.rsrc(kt);
    const uint32_t co = cc() * 8 < ncols ? (uint32_t)cc() * 16 : OOB_OFF;
#pragma unroll
    for (int i = 0; i < G::NPASS; ++i) {
      if constexpr (SCALED) sdat[SET][i] = spre[i];
      const uint32_t off = src.row_off(kt * 64 + kr(i), keys[i]);
      reg[SET][i] = buf_load16(r, off + co);  // OOB_OFF plus a chunk offset stays out of range
    }
  }
  template <int SET, int PART, int NPART>
  MOE_DEV void store(char* lds) const {
#pragma unroll
    for (int i = PART; i < G::NPASS; i += NPART) {
      u32x4_t v = reg[SET][i];
      if constexpr (SCALED) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = pack_bf16x2(bf16_to_f32(v[q] & 0xffffu) * sdat[SET][i], bf16_to_f32(v[q] >> 16) * sdat[SET][i]);
        }
      }
      *(u32x4_t*)(lds + kr(i) * G::PITCH + cc() * 16) = v;
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA over one LDS stage.
//
// k-major operands: ds_read_b64_tr_b16 works on groups of 16 lanes; lane
// 4q + s of a group receives element s of the 8-byte chunks addressed by
// lanes q, q + 4, q + 8 and q + 12 of the group.  Lane j therefore points at
// k-row kb + j / 4, columns mb + 4 (j % 4) .. + 3, and every lane ends up with
// four consecutive k of one row: lanes 0-15 rows 0-15 and lanes 16-31 rows
// 16-31 (k 0-3 of the step, then k 4-7 from the next four k-rows), lanes
// 32-63 the same rows for k 8-15 -- the 32x32x16 operand layout.
// ---------------------------------------------------------------------------
typedef short s16x4_t __attribute__((ext_vector_type(4)));

MOE_DEV int km_lane_off(int pitch) {
  const int l = lane_id(), g = l >> 4, j = l & 15;
  return (8 * (g >> 1) + (j >> 2)) * pitch + (16 * (g & 1) + 4 * (j & 3)) * 2;
}
MOE_DEV u32x4_t km_read(const char* p, int pitch) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s4;
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)p);
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p + 4 * pitch));
  const u32x2_t a = __builtin_bit_cast(u32x2_t, lo), b = __builtin_bit_cast(u32x2_t, hi);
  return u32x4_t{a[0], a[1], b[0], b[1]};
}

template <bool KM, int ROWS, class M>
struct OperandReader {
  // lane base for [row][k] staging: row l % 32, k-group l / 32
  static MOE_DEV const char* base(const char* op, int eb) {
    if constexpr (KM) return op + km_lane_off(KmGeom<ROWS>::PITCH);
    else return op + (lane_id() & 31) * LDS_ROW + (lane_id() >> 5) * (8 * eb);
  }
  // fragment of tile rows row0 .. row0+31, k-step s (16 k)
  static MOE_DEV typename M::Frag read(const char* b, int row0, int s, int step_bytes) {
    if constexpr (KM) {
      typename M::Frag f;
      f.v = km_read(b + s * 16 * KmGeom<ROWS>::PITCH + row0 * 2, KmGeom<ROWS>::PITCH);
      return f;
    } else {
      return M::lds_read(b + row0 * LDS_ROW + s * step_bytes);
    }
  }
};
// compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1
template <int N, int I = 0, class F>
MOE_DEV void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(static_cast<F&&>(f));
  }
}

// MFMAs of one LDS stage; after the MFMAs of k-step s >= FIRST, share
// s - FIRST of the next k-tile (register set SET of the loaders) is written
// to the other stage.
template <class C, int SET, int FIRST, class LA, class LB>
MOE_DEV void mma_stage(const char* stage, f32x16_t (&acc)[C::FM][C::FN], int wm, int wn, const LA& la,
                       const LB& lb, char* next) {
  using M = Mfma<typename C::T>;
  using RA = OperandReader<C::AKM, C::BM, M>;
  using RB = OperandReader<C::BKM, C::BN, M>;
  constexpr int STEP = 16 * C::EB;            // bytes of k per MFMA step ([row][k] staging)
  constexpr int NSTEP = KBYTES / STEP;
  const char* a_base = RA::base(stage, C::EB);
  const char* b_base = RB::base(stage + C::A_BYTES, C::EB);
  // operand fragments are read one k-step ahead of the MFMAs that use them;
  // the scheduling barrier keeps the compiler from hoisting every step's
  // reads (and their registers) to the top of the stage
  typename M::Frag a[2][C::FM], b[2][C::FN];
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) a[0][fm] = RA::read(a_base, C::a_row0(wm, fm), 0, STEP);
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) b[0][fn] = RB::read(b_base, C::b_row0(wn, fn), 0, STEP);
  static_for<NSTEP>([&](auto sc) {
    constexpr int s = decltype(sc)::value;
    constexpr int cur = s & 1;
    if constexpr (s + 1 < NSTEP) {
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) a[cur ^ 1][fm] = RA::read(a_base, C::a_row0(wm, fm), s + 1, STEP);
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) b[cur ^ 1][fn] = RB::read(b_base, C::b_row0(wn, fn), s + 1, STEP);
    }
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) M::mma(acc[fm][fn], a[cur][fm], b[cur][fn]);
    if constexpr (s >= FIRST) {
      la.template store<SET, s - FIRST, NSTEP - FIRST>(next);
      lb.template store<SET, s - FIRST, NSTEP - FIRST>(next + C::A_BYTES);
    }
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Main loop.  LDS holds two stages, one barrier per k-tile.
//
// Two register sets (NSETS = 2): at the top of iteration kt, k-tile kt sits
// in stage kt % 2 and k-tile kt + 1 in register set (kt + 1) % 2; k-tile
// kt + 2 is loaded into the free set, and k-tile kt + 1 goes to the other
// stage piecewise between the MFMAs of kt.  The global loads have a whole
// iteration to land.
//
// One register set (NSETS = 1), AHEAD: k-tile kt + 1 goes to the other stage
// after the MFMAs of kt's last k-step, and k-tile kt + 2 is loaded right
// after that, before the barrier, so each load has a whole iteration to land.
// The last two k-tiles are peeled off the loop: they load nothing, so no
// load is in flight when the epilogue starts.  Measured against the placement
// below (MI355X, large-d workload): gate/up -5%, dW_gate/up -1.5%,
// dW_down -3%, down-combine on this tile -6%; the dX fold was 1.6% slower
// with it and keeps the placement below.
// One register set, !AHEAD: k-tile kt + 1 is loaded at the top of iteration
// kt and written to the other stage between the MFMAs of the second half of
// kt's k-steps.
//
// Loads and index fetches run past the last k-tile unconditionally
// (out-of-range rows, columns and k read zeros or unused in-range data, never
// consumed), so every iteration has the same loads in flight and the
// compiler's waits stay exact.
template <class C, bool AHEAD = true, class LA, class LB>
MOE_DEV void gemm_mainloop(LA& la, LB& lb, int nk, char* smem, f32x16_t (&acc)[C::FM][C::FN], int wm, int wn) {
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;
  if (nk <= 0) return;
  constexpr int NSTEP = KBYTES / (16 * C::EB);
  la.prefetch(0);
  lb.prefetch(0);
  la.template load<0>(0);
  lb.template load<0>(0);
  la.prefetch(1);
  lb.prefetch(1);
  if constexpr (C::NSETS == 2) {
    la.template load<1>(1);
    lb.template load<1>(1);
    la.prefetch(2);
    lb.prefetch(2);
  }
  la.template store<0, 0, 1>(smem);
  lb.template store<0, 0, 1>(smem + C::A_BYTES);
  if constexpr (C::NSETS == 1 && AHEAD) {
    la.template load<0>(1);
    lb.template load<0>(1);
    la.prefetch(2);
    lb.prefetch(2);
  }
  __syncthreads();
  if constexpr (C::NSETS == 2) {
    // two k-tiles per iteration, the odd last one after the loop: a loop
    // without an exit in the middle keeps the accumulators in place
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      la.template load<0>(kt + 2);
      lb.template load<0>(kt + 2);
      la.prefetch(kt + 3);
      lb.prefetch(kt + 3);
      mma_stage<C, 1, 0>(smem, acc, wm, wn, la, lb, smem + C::STAGE);
      __syncthreads();
      la.template load<1>(kt + 3);
      lb.template load<1>(kt + 3);
      la.prefetch(kt + 4);
      lb.prefetch(kt + 4);
      mma_stage<C, 0, 0>(smem + C::STAGE, acc, wm, wn, la, lb, smem);
      __syncthreads();
    }
    if (kt < nk) {
      mma_stage<C, 1, 0>(smem, acc, wm, wn, la, lb, smem + C::STAGE);
      __syncthreads();
    }
  } else if constexpr (AHEAD) {
    int kt = 0;
    for (; kt + 2 < nk; ++kt) {
      const int cur = kt & 1;
      mma_stage<C, 0, NSTEP - 1>(smem + cur * C::STAGE, acc, wm, wn, la, lb, smem + (cur ^ 1) * C::STAGE);
      la.template load<0>(kt + 2);
      lb.template load<0>(kt + 2);
      la.prefetch(kt + 3);
      lb.prefetch(kt + 3);
      __syncthreads();
    }
    if (kt + 1 < nk) {  // next to last: stores the last k-tile, loads nothing
      const int cur = kt & 1;
      mma_stage<C, 0, NSTEP - 1>(smem + cur * C::STAGE, acc, wm, wn, la, lb, smem + (cur ^ 1) * C::STAGE);
      __syncthreads();
      ++kt;
    }
    mma_stage<C, 0, NSTEP>(smem + (kt & 1) * C::STAGE, acc, wm, wn, la, lb, nullptr);  // stores nothing
    __syncthreads();
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      la.template load<0>(kt + 1);
      lb.template load<0>(kt + 1);
      la.prefetch(kt + 2);
      lb.prefetch(kt + 2);
      mma_stage<C, 0, NSTEP / 2>(smem + cur * C::STAGE, acc, wm, wn, la, lb, smem + (cur ^ 1) * C::STAGE);
      __syncthreads();
    }
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
// Tile order of the varlen-M kernels: groups of R consecutive row blocks;
// inside a group the column block is major and the row block minor, so
// consecutive tiles share the B column block (weights) and a row block's A
// rows come back every R tiles, both within the span of tiles one XCD runs
// at a time.  Ids at or past ng * nbn (launch padding) return false.
MOE_DEV bool grouped_tile(int id, int ng, int nbn, int R, int& g, int& nb) {
  if (id >= ng * nbn) return false;
  const int g0 = id / (R * nbn) * R;
  const int rows = ng - g0 < R ? ng - g0 : R;
  const int rem = id - g0 * nbn;
  nb = rem / rows;
  g = g0 + rem % rows;
  return true;
}

// The same order inside each expert's own tiles (the ids of expert e are
// [mb_off[e], mb_off[e+1]) * nbn), so that a group of R row blocks never
// spans two experts and the tiles an XCD runs together share one expert's
// weights.  grp > 0: groups over the global row blocks (R = grp); grp < 0:
// groups inside each expert (R = -grp).
//
// xg (1, 2, 4 or 8; 0 = off, global groups only): the tiles of a group are
// handed out so that the eight XCDs (workgroups go to them in turn) form an
// xg x (8 / xg) grid over the group's R row blocks x nbn column blocks: XCD
// (xr, xc) takes the row blocks = xr (mod xg) and the column blocks = xc
// (mod 8 / xg) of the group, row-major.  All XCDs then work on the same
// group -- one expert's weights and rows, shared through the memory-side
// cache -- each on a 2-D part of it.  Groups that do not divide (the last,
// short one) keep the plain order.
MOE_DEV bool tile_of(int id, const int32_t* __restrict__ mb_off, int E, int nbn, int grp, int xg, int& g, int& nb) {
  if (grp > 0 && xg > 0) {
    const int ng = mb_off[E];
    if (id >= ng * nbn) return false;
    const int g0 = id / (grp * nbn) * grp;
    const int rows = ng - g0 < grp ? ng - g0 : grp;
    const int rem = id - g0 * nbn;
    const int xc = 8 / xg;
    if (rows == grp && grp % xg == 0 && nbn % xc == 0) {
      const int x = rem & 7, j = rem >> 3, cols = nbn / xc;
      g = g0 + x / xc + xg * (j / cols);
      nb = x % xc + xc * (j % cols);
    } else {
      nb = rem / rows;
      g = g0 + rem % rows;
    }
    return true;
  }
  if (grp > 0) return grouped_tile(id, mb_off[E], nbn, grp, g, nb);
  if (id >= mb_off[E] * nbn) return false;
  const int e = find_expert(mb_off, E, id / nbn);
  const int base = mb_off[e];
  int gl;
  grouped_tile(id - base * nbn, mb_off[e + 1] - base, nbn, -grp, gl, nb);
  g = base + gl;
  return true;
}

MOE_DEV int xcd_swizzle(int bid, int nblk) {
  if (nblk <= 0) return bid;  // launch order (the launcher's tuning switch)
  const int per = nblk >> 3;  // nblk is padded to a multiple of 8 by the launcher
  return (bid & 7) * per + (bid >> 3);
}

}  // namespace moe
