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
//      counts; one wave per expert scans its row of the [E][chunks] count
//      matrix into bases inside the expert and leaves the expert's length.
//   3. conflict-free scatter: every workgroup scans the E lengths in LDS
//      (the expert offsets, which workgroup 0 also writes out as
//      expert_token_offsets); a token's position is its expert's offset plus
//      its (expert, chunk) base plus the popcount of the lower tokens' bits in
//      the same masks; every destination is written exactly once.
#include <mutex>

#include "../../include/moe_dispatch.h"
#include "common.hpp"
#include "layout.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Static scratch of moe_build_index_noalloc: the index workspace of callers
// that cannot allocate.  Each GPU the library runs on holds its own copy
// until the process ends.  Host code never uses the array's name as an
// address: the device address of this device's copy comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// on the entry point's first call there.  The index kernels write every byte
// of the workspace they read (masks, counts, totals), so nothing is cleared
// between calls; calls that overlap in time on one GPU share the array and
// race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[MOE_NOALLOC_INDEX_MAX_BYTES];

size_t index_scratch_bytes() { return sizeof(scratch); }

hipError_t index_scratch_ptr(void** out) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* ptrs[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

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

// Step 2: one wave per expert e scans row e of the [E][nchunks] count matrix,
// 64 chunks at a time (coalesced), replacing each count by the number of the
// expert's tokens in lower chunks; tot[e] gets the row's total.
__global__ __launch_bounds__(256) void index_rowscan_kernel(int32_t* __restrict__ base, int32_t* __restrict__ tot,
                                                            int E, int nchunks) {
  const int e = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (e >= E) return;  // whole waves
  const int l = lane_id();
  int32_t* row = base + (size_t)e * nchunks;
  int carry = 0;
  for (int c0 = 0; c0 < nchunks; c0 += 64) {
    const int c = c0 + l;
    const int v = c < nchunks ? row[c] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(incl, off, 64);
      if (l >= off) incl += u;
    }
    if (c < nchunks) row[c] = carry + incl - v;
    carry += __shfl(incl, 63, 64);
  }
  if (l == 0) tot[e] = carry;
}

// Step 3.  The expert offsets (exclusive scan of tot, E <= 1024) are formed
// in LDS by every workgroup: each thread sums IDX_SCAN_PER consecutive
// experts, the 256 sums are scanned (wave shuffles, then the four wave
// totals), and each thread writes its experts' offsets.  All sums are below
// T*K < 2^31.
constexpr int IDX_SCAN_PER = 4;  // experts per thread: 256 * 4 = 1024 = the largest E
__global__ __launch_bounds__(256) void index_scatter_kernel(const int32_t* __restrict__ ids,
                                                            const uint64_t* __restrict__ masks,
                                                            const int32_t* __restrict__ base,
                                                            const int32_t* __restrict__ tot,
                                                            int32_t* __restrict__ eti, int32_t* __restrict__ tim,
                                                            int32_t* __restrict__ offsets, int T, int E, int K,
                                                            int nchunks) {
  __shared__ int32_t s_off[256 * IDX_SCAN_PER + 1];
  __shared__ int32_t s_wsum[IDX_WAVES];
  const int chunk = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int l = lane_id();
  {
    const int e0 = (int)threadIdx.x * IDX_SCAN_PER;
    int v[IDX_SCAN_PER];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < IDX_SCAN_PER; ++i) {
      v[i] = e0 + i < E ? tot[e0 + i] : 0;
      sum += v[i];
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(incl, off, 64);
      if (l >= off) incl += u;
    }
    if (l == 63) s_wsum[wave] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < wave; ++w) run += s_wsum[w];
#pragma unroll
    for (int i = 0; i < IDX_SCAN_PER; ++i) {
      s_off[e0 + i] = run;
      run += v[i];
    }
    if (threadIdx.x == 255) s_off[256 * IDX_SCAN_PER] = run;
    __syncthreads();
    if (chunk == 0) {
      for (int e = threadIdx.x; e < E; e += 256) offsets[e] = s_off[e];
      if (threadIdx.x == 0) offsets[E] = s_off[256 * IDX_SCAN_PER];  // = T*K: experts past E add nothing
    }
  }
  const int t = chunk * IDX_CHUNK + (int)threadIdx.x;
  if (t >= T) return;
  const uint64_t lower = (l == 0) ? 0ull : (~0ull >> (64 - l));
  const uint64_t* mchunk = masks + (size_t)chunk * IDX_WAVES * E;
  for (int k = 0; k < K; ++k) {
    const int e = ids[(size_t)t * K + k];
    int r = __popcll(mchunk[(size_t)wave * E + e] & lower);
    for (int w = 0; w < wave; ++w) r += __popcll(mchunk[(size_t)w * E + e]);
    const int pos = s_off[e] + base[(size_t)e * nchunks + chunk] + r;
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
  index_rowscan_kernel<<<dim3((s.E + 3) / 4), dim3(256), 0, st>>>(ws.base, ws.tot, s.E, ws.nchunks);
  index_scatter_kernel<<<dim3(ws.nchunks), dim3(256), 0, st>>>(ids, ws.masks, ws.base, ws.tot, eti, tim, offsets,
                                                               s.T, s.E, s.K, ws.nchunks);
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
//   zero the fold turn counters and the counters block, except the error
//   word of the other call that may share the workspace (counters[0] is
//   moe_combine's, counters[1] moe_expert_bwd's; own_err names the calling
//   entry's word, which is cleared, or -1 for neither).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prep_kernel(int T, int E, int K, const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ ids, const float* __restrict__ topk_w,
                                                   const int32_t* __restrict__ tim, int32_t* __restrict__ mb_off,
                                                   float* __restrict__ w_pos, int32_t* __restrict__ rank_pos,
                                                   int32_t* __restrict__ turn, long long n_turn,
                                                   int32_t* __restrict__ counters, int own_err) {
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
    if (tid < N_COUNTERS && (tid >= N_ERR_WORDS || tid == own_err)) counters[tid] = 0;
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
                       const float* topk_w, const int32_t* tim, bool per_position, int own_err, hipStream_t st) {
  timing_mark(st, "prep", true);
  const long long n_turn = per_position ? (long long)s.T * col_blocks(s.d, TILE_S) : 0;
  long long work = per_position ? (n_turn > s.A() ? n_turn : s.A()) : 1;
  int blocks = (int)((work + 255) / 256);
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  prep_kernel<<<dim3(blocks), dim3(256), 0, st>>>(s.T, s.E, s.K, offsets, ids, topk_w, tim, ws.mb_off,
                                                  per_position ? ws.w_pos : nullptr,
                                                  per_position ? ws.rank_pos : nullptr,
                                                  per_position ? ws.turn : nullptr, n_turn, ws.counters,
                                                  own_err);
  hipError_t e = hipGetLastError();
  timing_mark(st, "prep", false);
  return e;
}

}  // namespace moe
