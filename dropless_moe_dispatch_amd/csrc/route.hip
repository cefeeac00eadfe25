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
// logits GEMM: M = T tokens, N = E experts, K = d.
// ---------------------------------------------------------------------------
template <class C>
__global__ __launch_bounds__(NTHREADS, 2) void router_logits_kernel(const typename C::T* __restrict__ x,
                                                                    const typename C::T* __restrict__ wg,
                                                                    const float* __restrict__ bias,
                                                                    float* __restrict__ logits, int T, int d, int E) {
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
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) {
    const int e = n0 + C::b_row0(wn, fn) + frag_col(l);
    if (e >= E) continue;
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = m0 + C::a_row0(wm, fm) + frag_row(r, l);
        if (t < T) logits[(size_t)t * E + e] = acc[fm][fn][r] + b;
      }
  }
}

template <typename TIN>
static hipError_t router_logits_t(const Shape& s, const void* x, const void* wg, const float* bias, float* logits,
                                  hipStream_t st) {
  const dim3 blk(NTHREADS);
  if (s.E <= 32) {
    using C = Cfg<TIN, 128, 32, 4, 1>;
    const dim3 grd((s.T + C::BM - 1) / C::BM, (s.E + C::BN - 1) / C::BN);
    router_logits_kernel<C><<<grd, blk, 0, st>>>((const TIN*)x, (const TIN*)wg, bias, logits, s.T, s.d, s.E);
  } else if (s.E <= 64) {
    // 64-token tiles: a grid of T/64 workgroups fills the chip from a few thousand tokens
    using C = Cfg<TIN, 64, 64, 2, 2>;
    const dim3 grd((s.T + C::BM - 1) / C::BM, (s.E + C::BN - 1) / C::BN);
    router_logits_kernel<C><<<grd, blk, 0, st>>>((const TIN*)x, (const TIN*)wg, bias, logits, s.T, s.d, s.E);
  } else if (s.E <= 128) {
    // one 128-expert column block: 32-token tiles keep enough workgroups in flight
    using C = Cfg<TIN, 32, 128, 1, 4>;
    const dim3 grd((s.T + C::BM - 1) / C::BM, 1);
    router_logits_kernel<C><<<grd, blk, 0, st>>>((const TIN*)x, (const TIN*)wg, bias, logits, s.T, s.d, s.E);
  } else {
    using C = Cfg<TIN, 128, 128, 2, 2>;
    const dim3 grd((s.T + C::BM - 1) / C::BM, (s.E + C::BN - 1) / C::BN);
    router_logits_kernel<C><<<grd, blk, 0, st>>>((const TIN*)x, (const TIN*)wg, bias, logits, s.T, s.d, s.E);
  }
  return hipGetLastError();
}

hipError_t launch_router_logits(const Shape& s, const void* x, const void* wg, const float* bias, float* logits,
                                hipStream_t st) {
  timing_mark(st, "router_logits", true);
  hipError_t e = s.bf16 ? router_logits_t<bf16_t>(s, x, wg, bias, logits, st)
                        : router_logits_t<float>(s, x, wg, bias, logits, st);
  timing_mark(st, "router_logits", false);
  return e;
}

// ---------------------------------------------------------------------------
// top-K: a group of G lanes (a power of two, 1..64) per token; lane gl holds
// the V logits of experts gl*V .. gl*V+V-1 (contiguous, 16-byte loads when the
// rows allow).  K rounds of a group arg-max (larger value wins, ties to the
// lower id); the group's lane 0 writes each round's id at once and parks its
// logit in LDS.  Every lane of a group sees the same arg-max bits, so the
// softmax denominator over the chosen logits, sum_k exp(z_k - z_0) in k
// order, is the same in all of them; the weights are then written in
// parallel.
// ---------------------------------------------------------------------------
template <int G, int V>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int32_t* __restrict__ ids,
                                                   float* __restrict__ wts, int T, int E, int K) {
  constexpr int GPB = 256 / G;  // tokens per workgroup
  __shared__ float s_z[GPB][32];
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
  uint32_t live = 0;  // experts of this lane still selectable
#pragma unroll
  for (int v = 0; v < V; ++v) live |= (e0 + v < E ? 1u : 0u) << v;
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
    if (gl == 0 && valid) {
      ids[(size_t)t * K + k] = bid;
      s_z[g][k] = bz;
    }
  }
  __syncthreads();
  if (valid) {
    const float inv = 1.0f / ssum;
    for (int j = gl; j < K; j += G) wts[(size_t)t * K + j] = expf(s_z[g][j] - m0) * inv;
  }
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

}  // namespace moe
