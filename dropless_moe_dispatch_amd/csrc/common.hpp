// Shared device helpers for the dropless MoE kernels (gfx950 / CDNA4).
//
// Element storage: bf16 as raw uint16_t bits, fp32 as float.  Accumulation is
// always fp32 (MFMA accumulators).  Conversions to bf16 round to nearest even.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

MOE_DEV float bf16_to_f32(uint32_t v) { return __uint_as_float(v << 16); }

// fp32 -> bf16, rounded to nearest even: gfx950 converts two values in one
// v_cvt_pk_bf16_f32 (low half a, high half b).  A NaN stays a NaN.
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
MOE_DEV uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_v){a, b}, bf16x2_v));
}
MOE_DEV uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

template <typename T> struct ElemT;
template <> struct ElemT<float> {
  static MOE_DEV float to_f32(float v) { return v; }
  static MOE_DEV float from_f32(float v) { return v; }
  static MOE_DEV float load(const float* p) { return *p; }
  static MOE_DEV void store(float* p, float v) { *p = v; }
};
template <> struct ElemT<bf16_t> {
  static MOE_DEV float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static MOE_DEV void store(bf16_t* p, float v) { *p = (bf16_t)f32_to_bf16(v); }
};

// One 16-byte chunk of a row: 8 bf16 or 4 fp32 values, converted to/from fp32.
MOE_DEV void ld16(const bf16_t* p, float (&v)[8]) {
  const u32x4_t q = *(const u32x4_t*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(q[i] & 0xffffu);
    v[2 * i + 1] = bf16_to_f32(q[i] >> 16);
  }
}
MOE_DEV void ld16(const float* p, float (&v)[4]) {
  const f32x4_t q = *(const f32x4_t*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = q[i];
}
MOE_DEV void st16(bf16_t* p, const float (&v)[8]) {
  u32x4_t q;
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  *(u32x4_t*)p = q;
}
MOE_DEV void st16(float* p, const float (&v)[4]) { *(f32x4_t*)p = f32x4_t{v[0], v[1], v[2], v[3]}; }
// The same with the non-temporal cache policy, for data a kernel streams
// through once (read once here, or written here and read by a later kernel).
MOE_DEV void ld16nt(const bf16_t* p, float (&v)[8]) {
  const u32x4_t q = __builtin_nontemporal_load((const u32x4_t*)p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(q[i] & 0xffffu);
    v[2 * i + 1] = bf16_to_f32(q[i] >> 16);
  }
}
MOE_DEV void ld16nt(const float* p, float (&v)[4]) {
  const f32x4_t q = __builtin_nontemporal_load((const f32x4_t*)p);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = q[i];
}
// 16 bytes as they are (plain or non-temporal), unpacked to floats where
// they are used: a batch of such loads is not split by the waits that each
// unpacking needs.
MOE_DEV u32x4_t raw16(const void* p) { return *(const u32x4_t*)p; }
MOE_DEV u32x4_t raw16nt(const void* p) { return __builtin_nontemporal_load((const u32x4_t*)p); }
MOE_DEV void unpack16(const u32x4_t& q, float (&v)[8]) {  // 8 bf16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(q[i] & 0xffffu);
    v[2 * i + 1] = bf16_to_f32(q[i] >> 16);
  }
}
MOE_DEV void unpack16(const u32x4_t& q, float (&v)[4]) {  // 4 fp32
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(q[i]);
}
MOE_DEV void st16nt(bf16_t* p, const float (&v)[8]) {
  u32x4_t q;
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  __builtin_nontemporal_store(q, (u32x4_t*)p);
}
MOE_DEV void st16nt(float* p, const float (&v)[4]) {
  __builtin_nontemporal_store(f32x4_t{v[0], v[1], v[2], v[3]}, (f32x4_t*)p);
}

// Logistic function from the hardware exp2 and reciprocal (v_exp_f32 of
// -u log2(e), then v_rcp_f32): four instructions where expf and an IEEE
// division take about thirty, with an error of a few ulp in fp32 for the
// pre-activations met here, far below the bf16 rounding of everything it
// feeds (y, dA, dB and A').
MOE_DEV float sigmoidf_(float u) { return __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }

// Activation of a plain two-layer expert (act: 1 = SiLU, 2 = ReLU).
MOE_DEV float act_fwd(float a, int act) { return act == 2 ? (a > 0.0f ? a : 0.0f) : a * sigmoidf_(a); }
// The activation and its derivative (ReLU: 0 at the kink), from one logistic.
MOE_DEV void act_fwd_grad(float a, int act, float& y, float& g) {
  if (act == 2) {
    y = a > 0.0f ? a : 0.0f;
    g = a > 0.0f ? 1.0f : 0.0f;
    return;
  }
  const float s = sigmoidf_(a);
  y = a * s;
  g = s * (1.0f + a * (1.0f - s));
}

MOE_DEV int lane_id() { return (int)(threadIdx.x & 63); }

// ---------------------------------------------------------------------------
// MFMA: one 32x32 output fragment per instruction, K consumed 16 at a time.
//
// Operand layout (both operands are staged in LDS as [row][k] with k
// contiguous): lane l supplies row (l % 32), k = 8*(l/32) .. 8*(l/32)+7.
// The accumulator of lane l holds column (l % 32), rows
// 8*(r/4) + 4*(l/32) + (r%4) for r = 0..15.
// ---------------------------------------------------------------------------
template <typename TIN> struct Mfma;

template <> struct Mfma<bf16_t> {
  // 16 B per lane per k-step: 8 bf16 values.
  struct Frag { u32x4_t v; };
  static MOE_DEV Frag lds_read(const char* p) { Frag f; f.v = *(const u32x4_t*)p; return f; }
  static MOE_DEV void mma(f32x16_t& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                  __builtin_bit_cast(bf16x8_t, b.v), acc, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  // 32 B per lane per 16-k step: 8 fp32 values, consumed by 8 K=2 MFMAs.
  struct Frag { f32x4_t lo, hi; };
  static MOE_DEV Frag lds_read(const char* p) {
    Frag f; f.lo = *(const f32x4_t*)p; f.hi = *(const f32x4_t*)(p + 16); return f;
  }
  static MOE_DEV void mma(f32x16_t& acc, const Frag& a, const Frag& b) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[s], b.lo[s], acc, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[s], b.hi[s], acc, 0, 0, 0);
  }
};

// Row of accumulator register r for lane l inside a 32x32 fragment.
MOE_DEV int frag_row(int r, int l) { return 8 * (r >> 2) + 4 * (l >> 5) + (r & 3); }
MOE_DEV int frag_col(int l) { return l & 31; }
