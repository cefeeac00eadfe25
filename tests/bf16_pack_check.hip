// The library's fp32 -> bf16 packing (pack_bf16x2 in csrc/common.hpp, one
// v_cvt_pk_bf16_f32 on gfx950) against round-to-nearest-even written out on
// the host, the rounding the oracle's storage mirror applies.  Inputs: 2^24
// values of pseudo-random bits, every exact tie (a half-ulp pattern under each
// of the 65536 upper halves), and special values (zeros, infinities, NaNs,
// denormals, the largest finite values).  Prints the mismatches of normal,
// NaN and denormal inputs; exit status 0 only when there are none.
#include "../dropless_moe_dispatch_amd/csrc/common.hpp"

#include <cstdio>
#include <vector>

static uint32_t rne_host(uint32_t u) {
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // a NaN stays a (quiet) NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__global__ void pack_kernel(const uint32_t* in, uint32_t* out, int pairs) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < pairs) out[i] = pack_bf16x2(__uint_as_float(in[2 * i]), __uint_as_float(in[2 * i + 1]));
}

int main() {
  const int n = 1 << 24, pairs = n / 2;
  std::vector<uint32_t> h(n);
  uint64_t s = 0x9E3779B97F4A7C15ull;  // xorshift64
  for (int i = 0; i < n; ++i) {
    s ^= s << 13;
    s ^= s >> 7;
    s ^= s << 17;
    h[i] = (uint32_t)s;
  }
  const uint32_t special[] = {0x00000000u, 0x80000000u, 0x7f800000u, 0xff800000u, 0x7fc00000u, 0x7f800001u,
                              0xffc00001u, 0x00000001u, 0x007fffffu, 0x00008000u, 0x00018000u, 0x3f808000u,
                              0x3f818000u, 0x3f807fffu, 0x3f808001u, 0x7f7fffffu, 0x7f7f8000u, 0xff7fffffu};
  const int ns = (int)(sizeof(special) / sizeof(special[0]));
  for (int i = 0; i < ns; ++i) h[i] = special[i];
  for (int i = 0; i < 65536; ++i) h[64 + i] = ((uint32_t)i << 16) | 0x8000u;
  uint32_t *din = nullptr, *dout = nullptr;
  if (hipMalloc((void**)&din, (size_t)n * 4) != hipSuccess || hipMalloc((void**)&dout, (size_t)pairs * 4) != hipSuccess)
    return 2;
  if (hipMemcpy(din, h.data(), (size_t)n * 4, hipMemcpyHostToDevice) != hipSuccess) return 2;
  pack_kernel<<<(pairs + 255) / 256, 256>>>(din, dout, pairs);
  if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) return 3;
  std::vector<uint32_t> r(pairs);
  if (hipMemcpy(r.data(), dout, (size_t)pairs * 4, hipMemcpyDeviceToHost) != hipSuccess) return 2;
  (void)hipFree(din);
  (void)hipFree(dout);
  long normal = 0, nan = 0, denormal = 0;
  for (int i = 0; i < pairs; ++i) {
    for (int j = 0; j < 2; ++j) {
      const uint32_t u = h[2 * i + j], got = (r[i] >> (16 * j)) & 0xffffu, want = rne_host(u) & 0xffffu;
      if (got == want) continue;
      if ((u & 0x7fffffffu) > 0x7f800000u) ++nan;
      else if ((u & 0x7f800000u) == 0) ++denormal;
      else if (normal++ < 8) printf("mismatch %08x -> %04x, round-to-nearest-even gives %04x\n", u, got, want);
    }
  }
  printf("values %d mismatches: normal %ld nan %ld denormal %ld\n", n, normal, nan, denormal);
  return (normal || nan || denormal) ? 1 : 0;
}
