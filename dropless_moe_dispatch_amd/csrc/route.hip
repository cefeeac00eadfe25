// Router: logits z = x Wg^T (+ b) on MFMA, then a wavefront-level top-K over
// each token's logits with renormalised weights.
//
// Gating: topk experts = TopK(softmax(W_g x)), W_g in R^{E x d}
//   (MoEBlaze reading notes, sec. 2.1 "gating network").
// Renormalisation over the chosen K (Dropless MoE in depth, "A reference
//   implementation"): w_k = p_{S_k} / sum_j p_{S_j}, which equals the softmax
//   of the K chosen logits; it is computed that way here.
// Selection is on the fp32 logits (softmax is monotone): ties go to the lower
// expert id, slots are ordered by descending logit.
#include "gemm.hpp"
#include "layout.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// top-K of one token's logits, by a group of G lanes (a power of two, 1..64,
// aligned inside a wave); lane gl holds the V logits of experts gl*V ..
// gl*V+V-1 in z.  K rounds of a group arg-max (larger value wins, ties to the
// lower id).  Every lane of the group ends each round with the same winner,
// so the softmax denominator over the chosen logits, sum_k exp(z_k - z_0) in
// k order, is the same in all of them; lane gl keeps the winners of rounds
// gl, gl + G, ... and writes their ids and weights at the end.
// ---------------------------------------------------------------------------
template <int G, int V>
MOE_DEV void topk_group(const float (&z)[V], int e0, int E, int K, int gl, bool valid, int32_t* __restrict__ ids,
                        float* __restrict__ wts) {
  constexpr int Q = (32 + G - 1) / G;  // rounds kept per lane (K <= 32)
  uint32_t live = 0;  // experts of this lane still selectable
#pragma unroll
  for (int v = 0; v < V; ++v) live |= (e0 + v < E ? 1u : 0u) << v;
  float kz[Q];
  int kid[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    kz[q] = 0.0f;
    kid[q] = 0;
  }
  float m0 = 0.0f, ssum = 0.0f;
  for (int k = 0; k < K; ++k) {
    float bz = -INFINITY;
    int bid = 0x7fffffff;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      // ascending ids inside the lane: a strict > keeps the lowest id of a tie
      if (((live >> v) & 1u) && (z[v] > bz || bid == 0x7fffffff)) {
        bz = z[v];
        bid = e0 + v;
      }
    }
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) {
      const float oz = __shfl_xor(bz, off, G);
      const int oid = __shfl_xor(bid, off, G);
      if (oz > bz || (oz == bz && oid < bid)) {
        bz = oz;
        bid = oid;
      }
    }
    if (bid - e0 >= 0 && bid - e0 < V) live &= ~(1u << (bid - e0));
    if (k == 0) m0 = bz;
    ssum += expf(bz - m0);
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (k == q * G + gl) {
        kz[q] = bz;
        kid[q] = bid;
      }
  }
  if (valid) {
    const float inv = 1.0f / ssum;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int j = q * G + gl;
      if (j < K) {
        ids[j] = kid[q];
        wts[j] = expf(kz[q] - m0) * inv;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// logits GEMM: M = T tokens, N = E experts, K = d.  With TOPK the tile holds
// every expert (E <= BN): the logits are parked in LDS after they are
// written, and the NTHREADS / BM lanes of each token run topk_group on them.
// ---------------------------------------------------------------------------
template <class C, bool TOPK>
__global__ __launch_bounds__(NTHREADS, 2) void router_logits_kernel(const typename C::T* __restrict__ x,
                                                                    const typename C::T* __restrict__ wg,
                                                                    const float* __restrict__ bias,
                                                                    float* __restrict__ logits,
                                                                    int32_t* __restrict__ ids,
                                                                    float* __restrict__ wts, int T, int d, int E,
                                                                    int K) {
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  using TIN = typename C::T;
  const int m0 = blockIdx.x * C::BM;
  const int n0 = blockIdx.y * C::BN;
  const int wave = threadIdx.x >> 6, wm = wave / C::WN, wn = wave % C::WN;
  const uint32_t ld = (uint32_t)d * sizeof(TIN);
  RowLoader<C::BM> la;
  RowLoader<C::BN> lb;
  la.rs[0] = make_rsrc(x + (size_t)m0 * d, (size_t)(T - m0) * ld);
#pragma unroll
  for (int i = 0; i < RowLoader<C::BM>::CPT; ++i) {
    const int r = RowLoader<C::BM>::my_row(i);
    la.roff[i] = m0 + r < T ? (uint32_t)r * ld : OOB_OFF;
  }
  lb.rs[0] = make_rsrc(wg, (size_t)E * ld);
#pragma unroll
  for (int i = 0; i < RowLoader<C::BN>::CPT; ++i) {
    const int e = n0 + RowLoader<C::BN>::my_row(i);
    lb.roff[i] = e < E ? (uint32_t)e * ld : OOB_OFF;
  }
  f32x16_t acc[C::FM][C::FN];
  gemm_mainloop<C>(la, lb, d / C::BK, smem, acc, wm, wn);
  const int l = lane_id();
  constexpr int PITCH = C::BN + 4;  // floats per parked row
  float* s_z = (float*)smem;
  if constexpr (TOPK) {
    static_assert(C::BM * PITCH * 4 <= C::LDS_BYTES, "parked logits fit the LDS stages");
    __syncthreads();  // the LDS stages are reused below
  }
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) {
    const int e = n0 + C::b_row0(wn, fn) + frag_col(l);
    const float b = e < E && bias ? bias[e] : 0.0f;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tr = C::a_row0(wm, fm) + frag_row(r, l);
        const int t = m0 + tr;
        const float z = acc[fm][fn][r] + b;
        if (t < T && e < E) logits[(size_t)t * E + e] = z;
        if constexpr (TOPK) s_z[tr * PITCH + e] = z;
      }
  }
  if constexpr (TOPK) {
    constexpr int G = NTHREADS / C::BM;  // lanes per token
    constexpr int V = C::BN / G;         // logits per lane
    __syncthreads();
    const int g = (int)threadIdx.x / G, gl = (int)threadIdx.x % G;
    const int t = m0 + g;
    const int e0 = gl * V;
    float z[V];
#pragma unroll
    for (int v = 0; v < V; ++v) z[v] = e0 + v < E ? s_z[g * PITCH + e0 + v] : -INFINITY;
    const bool valid = t < T;
    const size_t o = (size_t)(valid ? t : 0) * K;
    topk_group<G, V>(z, e0, E, K, gl, valid, ids + o, wts + o);
  }
}

// E <= 128 takes one column block, so the top-K runs in the epilogue (TOPK)
// and ids, wts are written too; beyond, the logits only.
template <typename TIN>
static hipError_t router_logits_t(const Shape& s, const void* x, const void* wg, const float* bias, float* logits,
                                  int32_t* ids, float* w, hipStream_t st) {
  const dim3 blk(NTHREADS);
  auto go = [&](auto kern, int bm, int bn) {
    const dim3 grd((s.T + bm - 1) / bm, (s.E + bn - 1) / bn);
    kern<<<grd, blk, 0, st>>>((const TIN*)x, (const TIN*)wg, bias, logits, ids, w, s.T, s.d, s.E, s.K);
  };
  if (s.E <= 32) {
    go(router_logits_kernel<Cfg<TIN, 128, 32, 4, 1>, true>, 128, 32);
  } else if (s.E <= 64) {
    // 64-token tiles: a grid of T/64 workgroups fills the chip from a few thousand tokens
    go(router_logits_kernel<Cfg<TIN, 64, 64, 2, 2>, true>, 64, 64);
  } else if (s.E <= 128) {
    // one 128-expert column block: 32-token tiles keep enough workgroups in flight
    go(router_logits_kernel<Cfg<TIN, 32, 128, 1, 4>, true>, 32, 128);
  } else {
    go(router_logits_kernel<Cfg<TIN, 128, 128, 2, 2>, false>, 128, 128);
  }
  return hipGetLastError();
}

bool router_logits_has_topk(const Shape& s) { return s.E <= 128; }

hipError_t launch_router_logits(const Shape& s, const void* x, const void* wg, const float* bias, float* logits,
                                int32_t* ids, float* w, hipStream_t st) {
  timing_mark(st, "router_logits", true);
  hipError_t e = s.bf16 ? router_logits_t<bf16_t>(s, x, wg, bias, logits, ids, w, st)
                        : router_logits_t<float>(s, x, wg, bias, logits, ids, w, st);
  timing_mark(st, "router_logits", false);
  return e;
}

template <int G, int V>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int32_t* __restrict__ ids,
                                                   float* __restrict__ wts, int T, int E, int K) {
  constexpr int GPB = 256 / G;  // tokens per workgroup
  const int g = (int)(threadIdx.x / G), gl = (int)(threadIdx.x % G);
  const int t = blockIdx.x * GPB + g;
  const bool valid = t < T;
  const int e0 = gl * V;
  float z[V];
  const float* zr = logits + (size_t)(valid ? t : 0) * E + e0;
  if (valid && e0 + V <= E && (E & 3) == 0 && (V & 3) == 0) {
#pragma unroll
    for (int v = 0; v < V; v += 4) {
      const f32x4_t q = *(const f32x4_t*)(zr + v);
      z[v] = q[0];
      z[v + 1] = q[1];
      z[v + 2] = q[2];
      z[v + 3] = q[3];
    }
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) z[v] = valid && e0 + v < E ? zr[v] : -INFINITY;
  }
  const size_t o = (size_t)(valid ? t : 0) * K;
  topk_group<G, V>(z, e0, E, K, gl, valid, ids + o, wts + o);
}

hipError_t launch_topk(const Shape& s, const float* logits, int32_t* ids, float* w, hipStream_t st) {
  timing_mark(st, "topk", true);
  const int E = s.E;
  auto go = [&](auto kern, int G) {
    const int gpb = 256 / G;
    kern<<<dim3((s.T + gpb - 1) / gpb), dim3(256), 0, st>>>(logits, ids, w, s.T, s.E, s.K);
  };
  // about eight logits per lane
  if (E <= 8) go(topk_kernel<1, 8>, 1);
  else if (E <= 16) go(topk_kernel<2, 8>, 2);
  else if (E <= 32) go(topk_kernel<4, 8>, 4);
  else if (E <= 64) go(topk_kernel<8, 8>, 8);
  else if (E <= 128) go(topk_kernel<16, 8>, 16);
  else if (E <= 256) go(topk_kernel<32, 8>, 32);
  else if (E <= 512) go(topk_kernel<64, 8>, 64);
  else go(topk_kernel<64, 16>, 64);
  hipError_t e = hipGetLastError();
  timing_mark(st, "topk", false);
  return e;
}

// ---------------------------------------------------------------------------
// Fused router for bf16 and E <= 128: logits and top-K in one pass over x.
//
// A workgroup takes 32 tokens.  Its NWV waves split d into NWV slices; each
// wave computes the 32 x 32FN partial logits of its slice on MFMA with both
// operands loaded from global memory straight into registers.  For a 32-wide
// k-chunk, lane l reads 16 consecutive values of row (l % 32) at k offset
// 16 (l / 32), of x and of Wg alike, and feeds them to two 32x32x16 MFMA
// steps.  A dot product does not depend on which lane and step carry which
// k, as long as both operands agree, so this assignment gives every lane
// 32-byte contiguous reads and needs no LDS staging.  A ring of D chunks in
// registers keeps D x 2 KB of x per wave in flight: x streams from HBM once,
// while Wg (at most 128 x d) is re-read from L2 by every workgroup.  Chunks
// past the slice (the ring rounds the slice up to D chunks) read zeros.
//
// The partials meet in LDS and are summed in wave order (plus the bias);
// each token's G = NWV*64/32 lanes then write its logits and run topk_group
// on the same values, so the ids and weights are those the stand-alone top-K
// gives for the logits written.
// ---------------------------------------------------------------------------
template <int FN, int NWV, int D>
__global__ __launch_bounds__(NWV * 64, 2) void route_fused_kernel(const bf16_t* __restrict__ x,
                                                               const bf16_t* __restrict__ wg,
                                                               const float* __restrict__ bias,
                                                               float* __restrict__ logits, int32_t* __restrict__ ids,
                                                               float* __restrict__ wts, int T, int d, int E, int K) {
  constexpr int NE = 32 * FN;    // expert columns computed (E <= NE)
  constexpr int G = NWV * 2;     // lanes per token in the top-K: NWV*64 threads over 32 tokens
  constexpr int V = NE / G;      // logits per lane
  constexpr int PITCH = NE + 4;  // floats per LDS row
  static_assert(NE % G == 0, "whole logits per lane");
  __shared__ __attribute__((aligned(16))) float s_part[NWV][32][PITCH];
  const int t0 = blockIdx.x * 32;
  const int rows = T - t0 < 32 ? T - t0 : 32;
  const int wave = (int)threadIdx.x >> 6, l = lane_id();
  const int r = l & 31, hf = l >> 5;
  const int dq = d / NWV;  // this wave's slice of d (d is a multiple of 32 NWV)
  const int nch = dq / 32;
  // rows past T or E repeat the last valid row; their results are never used
  const uint32_t kofs = (uint32_t)(wave * dq + 16 * hf) * 2u;
  const rsrc_t rx = make_rsrc(x + (size_t)t0 * d, (size_t)rows * d * 2);
  const rsrc_t rw = make_rsrc(wg, (size_t)E * d * 2);
  const uint32_t xo = (uint32_t)(r < rows ? r : rows - 1) * (uint32_t)d * 2u + kofs;
  uint32_t wo[FN];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int e = fn * 32 + r;
    wo[fn] = (uint32_t)(e < E ? e : E - 1) * (uint32_t)d * 2u + kofs;
  }
  u32x4_t xa[D][2], wb[D][FN][2];
  f32x16_t acc[FN];
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) acc[fn] = f32x16_t{};
  // chunk c of the slice into ring slot j; past the slice the offset is out of
  // range and the load returns zeros
#define ROUTE_LOAD(j, c)                                                        \
  {                                                                             \
    const uint32_t co = (c) < nch ? (uint32_t)(c) * 64u : OOB_OFF;              \
    _Pragma("unroll") for (int s = 0; s < 2; ++s) {                             \
      xa[j][s] = buf_load16(rx, xo + co + 16u * s);                             \
      _Pragma("unroll") for (int fn = 0; fn < FN; ++fn) wb[j][fn][s] =          \
          buf_load16(rw, wo[fn] + co + 16u * s);                                \
    }                                                                           \
  }
#pragma unroll
  for (int j = 0; j < D; ++j) {
    ROUTE_LOAD(j, j)
    __builtin_amdgcn_sched_barrier(0);  // issue in slot order, as the loop refills them
  }
  for (int c0 = 0; c0 < nch; c0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, xa[j][s]),
                                                            __builtin_bit_cast(bf16x8_t, wb[j][fn][s]), acc[fn], 0, 0,
                                                            0);
      ROUTE_LOAD(j, c0 + D + j)
      // keep slot order: the MFMAs of slot j + 1 must not be hoisted above
      // this refill, which would make every slot wait for the whole ring
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#undef ROUTE_LOAD
#pragma unroll
  for (int fn = 0; fn < FN; ++fn)
#pragma unroll
    for (int i = 0; i < 16; ++i) s_part[wave][frag_row(i, l)][fn * 32 + frag_col(l)] = acc[fn][i];
  __syncthreads();

  const int g = (int)threadIdx.x / G, gl = (int)threadIdx.x % G;
  const int t = t0 + g;
  const bool valid = g < rows;
  const int e0 = gl * V;
  float z[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float a = s_part[0][g][e0 + v];
#pragma unroll
    for (int w = 1; w < NWV; ++w) a += s_part[w][g][e0 + v];
    const int e = e0 + v;
    z[v] = e < E ? a + (bias ? bias[e] : 0.0f) : -INFINITY;
  }
  if (valid) {
    float* zr = logits + (size_t)t * E + e0;
    if constexpr (V % 4 == 0) {
      if ((E & 3) == 0 && e0 + V <= E) {
#pragma unroll
        for (int v = 0; v < V; v += 4) *(f32x4_t*)(zr + v) = f32x4_t{z[v], z[v + 1], z[v + 2], z[v + 3]};
      } else {
#pragma unroll
        for (int v = 0; v < V; ++v)
          if (e0 + v < E) zr[v] = z[v];
      }
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (e0 + v < E) zr[v] = z[v];
    }
  }
  const size_t o = (size_t)(valid ? t : t0) * K;
  topk_group<G, V>(z, e0, E, K, gl, valid, ids + o, wts + o);
}

// The fused router is used for bf16, E <= 128, fewer than 16384 tokens (a
// grid under 512 workgroups of eight waves) and d a multiple of 256.  Measured
// on MI355X it takes 21 us where logits + top-K took 43 us (T = 4096,
// d = 4096, E = 8) and 19 us for 31 us (T = 8192, d = 2048, E = 8).  With
// more tokens the LDS-staged logits GEMM and the separate top-K are faster
// (45 vs 68 us at T = 16384, d = 2048, E = 128; 110 vs 250 us at T = 32768,
// d = 6144, E = 64): reading 32 rows per load instruction at 32 bytes each
// costs more than the wider grid gains once the grid fills the chip.
bool route_fused_applies(const Shape& s) {
  return s.bf16 && s.E <= 128 && (s.T + 31) / 32 < 512 && s.d % 256 == 0;
}

hipError_t launch_route_fused(const Shape& s, const void* x, const void* wg, const float* bias, float* logits,
                              int32_t* ids, float* w, hipStream_t st) {
  timing_mark(st, "route", true);
  const dim3 grd((s.T + 31) / 32);
  auto go = [&](auto kern) {
    kern<<<grd, dim3(8 * 64), 0, st>>>((const bf16_t*)x, (const bf16_t*)wg, bias, logits, ids, w, s.T, s.d, s.E, s.K);
  };
  const int fn = (s.E + 31) / 32;
  if (fn == 1) go(route_fused_kernel<1, 8, 8>);
  else if (fn == 2) go(route_fused_kernel<2, 8, 6>);
  else go(route_fused_kernel<4, 8, 4>);
  hipError_t e = hipGetLastError();
  timing_mark(st, "route", false);
  return e;
}

}  // namespace moe
