// Routing index by counting sort: no global sort, no atomics.
//
// The four structures (MoEBlaze analysis page, "Dispatch Data Structures:
// Specification and Roles"; MoEBlaze reading notes sec. 4.1, Figure 2):
//   expert_token_indices [T*K]: token ids grouped by expert, ascending token
//                               id inside each expert;
//   expert_token_offsets [E+1]: exclusive prefix sum of per-expert counts;
//   token_expert_indices [T*K]: the router's top-K ids (the caller's array);
//   token_index_map      [T*K]: position of (t, ids[t,k]) in the first array.
//
// Construction follows the atomic-free three steps of the MoEBlaze analysis
// page ("Dispatch Data Structure Construction"), recast for wave64:
//   1. dense token-expert map: per chunk of 256 tokens, one 64-bit ballot
//      mask per (wave, expert) -- bit i set iff token i of the wave chose the
//      expert.  Each mask has a single writer.
//   2. expert lengths: popcounts of the masks give the per-(expert, chunk)
//      counts; one workgroup scans the [E][chunks] count matrix (expert-major)
//      into absolute bases, which also yields expert_token_offsets.
//   3. conflict-free scatter: a token's position is its (expert, chunk) base
//      plus the popcount of the lower tokens' bits in the same masks; every
//      destination is written exactly once.
#include "common.hpp"
#include "layout.hpp"

namespace moe {

// Step 1 + counts.  Each lane first turns its token's K expert ids into an
// E-bit set (NW words of 64 experts); the mask of expert e is then the ballot
// of bit e over the wave, which is how a compare result is produced anyway.
// Lane b keeps expert 64 w + b's mask, so the masks of 64 experts leave in one
// coalesced store.
template <int NW>
__global__ __launch_bounds__(256) void index_hist_kernel(const int32_t* __restrict__ ids, uint64_t* __restrict__ masks,
                                                         int32_t* __restrict__ base, int T, int E, int K,
                                                         int nchunks) {
  const int chunk = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int l = lane_id();
  const int t = chunk * IDX_CHUNK + (int)threadIdx.x;
  uint32_t bits[2 * NW];  // 32-bit halves of the expert set
#pragma unroll
  for (int w = 0; w < 2 * NW; ++w) bits[w] = 0;
  if (t < T) {
    for (int k = 0; k < K; ++k) {
      const int e = ids[(size_t)t * K + k];
#pragma unroll
      for (int w = 0; w < 2 * NW; ++w) bits[w] |= (e >> 5) == w ? 1u << (e & 31) : 0u;
    }
  }
  __shared__ uint32_t s_cnt[IDX_WAVES][NW * 64];
  uint64_t* mrow = masks + ((size_t)chunk * IDX_WAVES + wave) * E;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w * 64 >= E) break;
    uint32_t lo = 0, hi = 0;  // lane b: mask of expert 64 w + b
#pragma unroll
    for (int b = 0; b < 64; ++b) {
      const uint64_t m = __ballot((bits[2 * w + (b >> 5)] >> (b & 31)) & 1u);
      lo = l == b ? (uint32_t)m : lo;
      hi = l == b ? (uint32_t)(m >> 32) : hi;
    }
    const int e = w * 64 + l;
    if (e < E) {
      const uint64_t m = ((uint64_t)hi << 32) | lo;
      mrow[e] = m;
      s_cnt[wave][e] = (uint32_t)__popcll(m);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < IDX_WAVES; ++w) c += s_cnt[w][e];
    base[(size_t)e * nchunks + chunk] = (int32_t)c;
  }
}

// Exclusive scan of the [E][nchunks] count matrix in expert-major order by
// one 1024-thread workgroup: each thread sums a contiguous segment, the
// segment sums are scanned with wave shuffles (then across the 16 waves), and
// each thread writes its segment's bases.  All sums are below T*K < 2^31.
__global__ __launch_bounds__(1024) void index_scan_kernel(int32_t* __restrict__ base, int32_t* __restrict__ offsets,
                                                          int E, int nchunks) {
  const long long n = (long long)E * nchunks;
  const int tid = threadIdx.x, l = lane_id(), wave = tid >> 6;
  const long long per = (n + 1023) / 1024;
  const long long s0 = tid * per < n ? tid * per : n;
  const long long s1 = s0 + per < n ? s0 + per : n;
  int sum = 0;
  for (long long i = s0; i < s1; ++i) sum += base[i];
  int incl = sum;  // inclusive scan inside the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (l >= off) incl += v;
  }
  __shared__ int wsum[16];
  if (l == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int run = before + incl - sum;  // exclusive prefix of this segment
  if (s0 < s1) {
    int e = (int)(s0 / nchunks), c = (int)(s0 % nchunks);
    for (long long i = s0; i < s1; ++i) {
      const int v = base[i];
      base[i] = run;
      if (c == 0) offsets[e] = run;
      run += v;
      if (++c == nchunks) { c = 0; ++e; }
    }
  }
  if (tid == 1023) offsets[E] = run;
}

__global__ __launch_bounds__(256) void index_scatter_kernel(const int32_t* __restrict__ ids,
                                                            const uint64_t* __restrict__ masks,
                                                            const int32_t* __restrict__ base,
                                                            int32_t* __restrict__ eti, int32_t* __restrict__ tim,
                                                            int T, int E, int K, int nchunks) {
  const int chunk = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int l = lane_id();
  const int t = chunk * IDX_CHUNK + (int)threadIdx.x;
  if (t >= T) return;
  const uint64_t lower = (l == 0) ? 0ull : (~0ull >> (64 - l));
  const uint64_t* mchunk = masks + (size_t)chunk * IDX_WAVES * E;
  for (int k = 0; k < K; ++k) {
    const int e = ids[(size_t)t * K + k];
    int r = __popcll(mchunk[(size_t)wave * E + e] & lower);
    for (int w = 0; w < wave; ++w) r += __popcll(mchunk[(size_t)w * E + e]);
    const int pos = base[(size_t)e * nchunks + chunk] + r;
    eti[pos] = t;
    tim[(size_t)t * K + k] = pos;
  }
}

hipError_t launch_build_index(const Shape& s, const int32_t* ids, int32_t* offsets, int32_t* eti, int32_t* tim,
                              const IndexWs& ws, hipStream_t st) {
  timing_mark(st, "index", true);
  {
    const dim3 g(ws.nchunks), b(256);
    if (s.E <= 64) index_hist_kernel<1><<<g, b, 0, st>>>(ids, ws.masks, ws.base, s.T, s.E, s.K, ws.nchunks);
    else if (s.E <= 128) index_hist_kernel<2><<<g, b, 0, st>>>(ids, ws.masks, ws.base, s.T, s.E, s.K, ws.nchunks);
    else if (s.E <= 256) index_hist_kernel<4><<<g, b, 0, st>>>(ids, ws.masks, ws.base, s.T, s.E, s.K, ws.nchunks);
    else if (s.E <= 512) index_hist_kernel<8><<<g, b, 0, st>>>(ids, ws.masks, ws.base, s.T, s.E, s.K, ws.nchunks);
    else index_hist_kernel<16><<<g, b, 0, st>>>(ids, ws.masks, ws.base, s.T, s.E, s.K, ws.nchunks);
  }
  index_scan_kernel<<<dim3(1), dim3(1024), 0, st>>>(ws.base, offsets, s.E, ws.nchunks);
  index_scatter_kernel<<<dim3(ws.nchunks), dim3(256), 0, st>>>(ids, ws.masks, ws.base, eti, tim, s.T, s.E, s.K,
                                                               ws.nchunks);
  hipError_t e = hipGetLastError();
  timing_mark(st, "index", false);
  return e;
}

// ---------------------------------------------------------------------------
// Per-call preparation for the expert GEMMs:
//   block 0: mb_off[b][e] = sum_{e' < e} ceil(count_e' / bm_b), bm = 128, 256
//            (tile maps of the two row blockings);
//   all blocks: per position p = token_index_map[t*K+k]:
//     w_pos[p] = topk_w[t,k], rank_pos[p] = #{j : ids[t,j] < ids[t,k]};
//   zero the fold turn counters and the counters block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prep_kernel(int T, int E, int K, const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ ids, const float* __restrict__ topk_w,
                                                   const int32_t* __restrict__ tim, int32_t* __restrict__ mb_off,
                                                   float* __restrict__ w_pos, int32_t* __restrict__ rank_pos,
                                                   int32_t* __restrict__ turn, long long n_turn,
                                                   int32_t* __restrict__ counters) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    __shared__ int sh[256];
    const int per = (E + 255) / 256;
    for (int b = 0; b < 2; ++b) {
      const int bm = b ? TILE_L : TILE_S;
      int32_t* mo = mb_off + b * (E + 1);
      int loc[4];
      int sum = 0;
      for (int i = 0; i < per; ++i) {
        const int e = tid * per + i;
        const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
        loc[i] = (c + bm - 1) / bm;
        sum += loc[i];
      }
      __syncthreads();
      sh[tid] = sum;
      __syncthreads();
      for (int off = 1; off < 256; off <<= 1) {
        const int v = tid >= off ? sh[tid - off] : 0;
        __syncthreads();
        sh[tid] += v;
        __syncthreads();
      }
      int run = sh[tid] - sum;
      for (int i = 0; i < per; ++i) {
        const int e = tid * per + i;
        if (e < E) mo[e] = run;
        run += loc[i];
      }
      if (tid == 255) mo[E] = sh[255];
    }
    if (tid < N_COUNTERS) counters[tid] = 0;
  }
  const long long gsz = (long long)gridDim.x * 256;
  const long long gid = (long long)blockIdx.x * 256 + tid;
  if (w_pos) {
    // one thread per assignment a = t*K + k (T*K < 2^31)
    const int A = T * K;
    for (long long a = gid; a < A; a += gsz) {
      const int ai = (int)a, t0 = ai - ai % K;
      const int ek = ids[ai];
      int r = 0;
      for (int j = 0; j < K; ++j) r += ids[t0 + j] < ek;
      const int p = tim[ai];
      w_pos[p] = topk_w[ai];
      rank_pos[p] = r;
    }
  }
  if (turn)
    for (long long i = gid; i < n_turn; i += gsz) turn[i] = 0;
}

hipError_t launch_prep(const Shape& s, const ExpertWs& ws, const int32_t* offsets, const int32_t* ids,
                       const float* topk_w, const int32_t* tim, bool per_position, hipStream_t st) {
  timing_mark(st, "prep", true);
  const long long n_turn = per_position ? (long long)s.T * col_blocks(s.d, TILE_S) : 0;
  long long work = per_position ? (n_turn > s.A() ? n_turn : s.A()) : 1;
  int blocks = (int)((work + 255) / 256);
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  prep_kernel<<<dim3(blocks), dim3(256), 0, st>>>(s.T, s.E, s.K, offsets, ids, topk_w, tim, ws.mb_off,
                                                  per_position ? ws.w_pos : nullptr,
                                                  per_position ? ws.rank_pos : nullptr,
                                                  per_position ? ws.turn : nullptr, n_turn, ws.counters);
  hipError_t e = hipGetLastError();
  timing_mark(st, "prep", false);
  return e;
}

}  // namespace moe
