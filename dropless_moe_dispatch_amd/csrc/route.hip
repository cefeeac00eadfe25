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
    using C = Cfg<TIN, 128, 64, 2, 2>;
    const dim3 grd((s.T + C::BM - 1) / C::BM, (s.E + C::BN - 1) / C::BN);
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
// top-K: a group of G lanes (G = power of two, 8..64) per token, each lane
// holding up to V logits (experts lane, lane+G, ...).  K rounds of a group
// arg-max (larger value wins, ties to the lower id), then the weights.
// ---------------------------------------------------------------------------
template <int G, int V>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int32_t* __restrict__ ids,
                                                   float* __restrict__ wts, int T, int E, int K) {
  const int gpb = 256 / G;
  const int t = blockIdx.x * gpb + (int)(threadIdx.x / G);
  const int gl = (int)(threadIdx.x % G);
  if (t >= T) return;  // the whole group exits together
  float z[V];
  const float* zr = logits + (size_t)t * E;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int e = gl + v * G;
    z[v] = e < E ? zr[e] : -INFINITY;
  }
  uint32_t taken = 0;
  float sel_z[32];
  int sel_id[32];
  for (int k = 0; k < K; ++k) {
    float bz = -INFINITY;
    int bid = 0x7fffffff;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e = gl + v * G;
      if (e < E && !((taken >> v) & 1u) && (z[v] > bz || (z[v] == bz && e < bid))) {
        bz = z[v];
        bid = e;
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
    if (bid % G == gl) taken |= 1u << (bid / G);
    sel_z[k & 31] = bz;
    sel_id[k & 31] = bid;
  }
  if (gl == 0) {
    const float m = sel_z[0];
    float ssum = 0.0f;
    float ex[32];
    for (int k = 0; k < K; ++k) {
      ex[k] = expf(sel_z[k] - m);
      ssum += ex[k];
    }
    const float inv = 1.0f / ssum;
    for (int k = 0; k < K; ++k) {
      ids[(size_t)t * K + k] = sel_id[k];
      wts[(size_t)t * K + k] = ex[k] * inv;
    }
  }
}

hipError_t launch_topk(const Shape& s, const float* logits, int32_t* ids, float* w, hipStream_t st) {
  timing_mark(st, "topk", true);
  const int E = s.E;
  auto go = [&](auto kern, int G) {
    const int gpb = 256 / G;
    kern<<<dim3((s.T + gpb - 1) / gpb), dim3(256), 0, st>>>(logits, ids, w, s.T, s.E, s.K);
  };
  if (E <= 8) go(topk_kernel<8, 1>, 8);
  else if (E <= 16) go(topk_kernel<16, 1>, 16);
  else if (E <= 32) go(topk_kernel<32, 1>, 32);
  else if (E <= 64) go(topk_kernel<64, 1>, 64);
  else if (E <= 128) go(topk_kernel<64, 2>, 64);
  else if (E <= 256) go(topk_kernel<64, 4>, 64);
  else if (E <= 512) go(topk_kernel<64, 8>, 64);
  else go(topk_kernel<64, 16>, 64);
  hipError_t e = hipGetLastError();
  timing_mark(st, "topk", false);
  return e;
}

}  // namespace moe
