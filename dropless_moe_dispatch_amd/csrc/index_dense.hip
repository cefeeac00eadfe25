// Alternate index backend: MoEBlaze's three steps taken literally, with a
// dense token-expert map (MoEBlaze analysis page, "Dispatch Data Structure
// Construction: The Atomic-Free Three-Step Algorithm").  Same outputs as the
// ballot-mask backend in index.hip (moe_build_index), bit for bit.
//
//   step 1  dense map D5[e][t] = t if token t chose expert e, else -1 (the
//           unset value is -1 rather than 0, which is a valid token id).
//           Stored expert-major ([E][T]) so that the per-expert passes of
//           steps 2 and 3 read contiguous memory.  Two kernels: fill with
//           the sentinel, then one writer per (t, k) -- a token's K experts
//           are distinct, so no cell is written twice.
//   step 2  expert lengths: one workgroup per expert counts its column with
//           wave ballots; one workgroup scans the lengths into offsets.
//   step 3  location map: one workgroup per expert walks its column in
//           tiles of 256 tokens; per tile, wave counts in LDS give each
//           wave's exclusive offset, the running tile offset is carried
//           across tiles, and the expert's global offset is added:
//           loc[e][t] = offsets[e] + (entries of column e before token t).
//           A final kernel over (t, k) writes expert_token_indices[loc] = t
//           and token_index_map[t*K + k] = loc; every destination has a
//           single writer.
// Workspace: two [E][T] int32 maps and the lengths -- O(T*E), which is the
// page's own trade (the dense map is what makes the column passes simple).
#include "common.hpp"
#include "layout.hpp"

namespace moe {

__global__ __launch_bounds__(256) void dense_fill_kernel(int32_t* __restrict__ d5, long long n) {
  const long long n4 = n >> 2;
  const long long gsz = (long long)gridDim.x * 256;
  int32_t* p = d5;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += gsz)
    *(int4*)(p + 4 * i) = make_int4(-1, -1, -1, -1);
  for (long long i = 4 * n4 + (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += gsz) p[i] = -1;
}

// ids outside [0, E) are skipped (their token_index_map entries become -1)
__global__ __launch_bounds__(256) void dense_mark_kernel(const int32_t* __restrict__ ids, int32_t* __restrict__ d5,
                                                         int T, int E, int K) {
  const long long A = (long long)T * K;
  const long long gsz = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < A; i += gsz) {
    const int t = (int)(i / K);
    const int e = ids[i];
    if ((unsigned)e < (unsigned)E) d5[(size_t)e * T + t] = t;
  }
}

__global__ __launch_bounds__(256) void dense_count_kernel(const int32_t* __restrict__ d5, int32_t* __restrict__ lengths,
                                                          int T) {
  const int e = blockIdx.x;
  const int32_t* col = d5 + (size_t)e * T;
  int c = 0;
  for (int t = threadIdx.x; t < T; t += 256) c += col[t] >= 0;
  // wave sum, then the four waves in a fixed order
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
  __shared__ int s[4];
  if (lane_id() == 0) s[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) lengths[e] = ((s[0] + s[1]) + s[2]) + s[3];
}

// exclusive scan of E <= 1024 lengths by one workgroup; offsets[E] = T*K
__global__ __launch_bounds__(1024) void lengths_scan_kernel(const int32_t* __restrict__ lengths,
                                                            int32_t* __restrict__ offsets, int E) {
  __shared__ int s[1024];
  const int i = threadIdx.x;
  const int v = i < E ? lengths[i] : 0;
  s[i] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int a = i >= off ? s[i - off] : 0;
    __syncthreads();
    s[i] += a;
    __syncthreads();
  }
  if (i < E) offsets[i] = s[i] - v;
  if (i == 1023) offsets[E] = s[1023];
}

__global__ __launch_bounds__(256) void dense_locate_kernel(const int32_t* __restrict__ d5,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ loc, int T) {
  const int e = blockIdx.x;
  const int32_t* col = d5 + (size_t)e * T;
  int32_t* lcol = loc + (size_t)e * T;
  const int wave = threadIdx.x >> 6, l = lane_id();
  const uint64_t below = (l == 0) ? 0ull : (~0ull >> (64 - l));   // lanes lower than this one
  __shared__ int s_cnt[4];
  int running = offsets[e];
  for (int t0 = 0; t0 < T; t0 += 256) {
    const int t = t0 + (int)threadIdx.x;
    const bool has = t < T && col[t] >= 0;
    const uint64_t m = __ballot(has);
    if (l == 0) s_cnt[wave] = __popcll(m);
    __syncthreads();
    int wave_off = 0, tile = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wave_off += w < wave ? s_cnt[w] : 0;
      tile += s_cnt[w];
    }
    if (has) lcol[t] = running + wave_off + __popcll(m & below);
    running += tile;
    __syncthreads();  // s_cnt is rewritten by the next tile
  }
}

__global__ __launch_bounds__(256) void dense_scatter_kernel(const int32_t* __restrict__ ids,
                                                            const int32_t* __restrict__ loc,
                                                            int32_t* __restrict__ eti, int32_t* __restrict__ tim,
                                                            int T, int E, int K) {
  const long long A = (long long)T * K;
  const long long gsz = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < A; i += gsz) {
    const int t = (int)(i / K);
    const int e = ids[i];
    if ((unsigned)e >= (unsigned)E) {
      tim[i] = -1;
      continue;
    }
    const int p = loc[(size_t)e * T + t];
    eti[p] = t;
    tim[i] = p;
  }
}

static unsigned grid_for(long long n) {
  const long long b = (n + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 4096 ? 4096 : b));
}

hipError_t launch_build_index_dense(const Shape& s, const int32_t* ids, int32_t* offsets, int32_t* eti, int32_t* tim,
                                    const DenseIndexWs& ws, hipStream_t st) {
  const long long n = (long long)s.E * s.T;
  timing_mark(st, "index_dense", true);
  dense_fill_kernel<<<dim3(grid_for(n / 4)), dim3(256), 0, st>>>(ws.d5, n);
  dense_mark_kernel<<<dim3(grid_for(s.A())), dim3(256), 0, st>>>(ids, ws.d5, s.T, s.E, s.K);
  dense_count_kernel<<<dim3(s.E), dim3(256), 0, st>>>(ws.d5, ws.lengths, s.T);
  lengths_scan_kernel<<<dim3(1), dim3(1024), 0, st>>>(ws.lengths, offsets, s.E);
  dense_locate_kernel<<<dim3(s.E), dim3(256), 0, st>>>(ws.d5, offsets, ws.loc, s.T);
  dense_scatter_kernel<<<dim3(grid_for(s.A())), dim3(256), 0, st>>>(ids, ws.loc, eti, tim, s.T, s.E, s.K);
  const hipError_t e = hipGetLastError();
  timing_mark(st, "index_dense", false);
  return e;
}

}  // namespace moe
