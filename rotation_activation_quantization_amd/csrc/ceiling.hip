// The memory-traffic ceiling of the online path: a kernel that moves exactly
// the bytes the rotate + quantize kernels move per token -- reads the bf16
// row (2n bytes), writes n/2 code bytes and the two 4-byte per-token values
// -- with none of their arithmetic.  Each 16-byte input chunk becomes one
// 4-byte output word (the XOR of its four words, so no load can be dropped).
// Of the layouts timed for it (rows per work-group, persistent grids, 2 to 8
// chunks per thread, cached or nontemporal accesses) this one-shot grid of
// four nontemporal chunks per thread moved the bytes fastest.
// It exists to measure what the HBM system sustains for this read/write mix
// at these shapes; it computes nothing of the method.
#include "internal.h"

namespace signrot {
namespace {

constexpr int kCeilThreads = 256;
constexpr int kCeilUnroll = 4;  // 16-byte chunks per thread, all loads issued before the stores

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_c;

// One-shot grid over the 16-byte chunks of the batch, chunk e = (row e / cpr,
// chunk e % cpr); loads and stores bypass the caches' retention
// (nontemporal), since no byte is touched twice.
__global__ __launch_bounds__(kCeilThreads) void stream_ceiling_kernel(const uint16_t* __restrict__ x, uint32_t total,
                                                                      uint32_t cpr, int64_t ld,
                                                                      uint32_t* __restrict__ out, float* s0,
                                                                      float* s1) {
  const uint32_t base = blockIdx.x * (kCeilThreads * kCeilUnroll) + threadIdx.x;
  u32x4_c v[kCeilUnroll];
#pragma unroll
  for (int u = 0; u < kCeilUnroll; ++u) {
    const uint32_t e = base + u * kCeilThreads;
    if (e < total) {
      const uint32_t row = e / cpr;
      const uint32_t j = e - row * cpr;
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_c*>(x + row * ld) + j);
    }
  }
#pragma unroll
  for (int u = 0; u < kCeilUnroll; ++u) {
    const uint32_t e = base + u * kCeilThreads;
    if (e < total) {
      __builtin_nontemporal_store(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3], out + e);
      const uint32_t row = e / cpr;
      if (e == row * cpr) {
        s0[row] = __uint_as_float(v[u][0]);
        s1[row] = __uint_as_float(v[u][1]);
      }
    }
  }
}

}  // namespace

hipError_t launch_stream_ceiling(const uint16_t* x, int64_t tokens, int n, int64_t ld, uint8_t* out, float* s0,
                                 float* s1, hipStream_t s) {
  const uint32_t cpr = static_cast<uint32_t>(n / 8);
  const uint32_t total = static_cast<uint32_t>(tokens) * cpr;  // < 2^32, checked by the caller
  const uint32_t per = kCeilThreads * kCeilUnroll;
  hipLaunchKernelGGL(stream_ceiling_kernel, dim3((total + per - 1) / per), dim3(kCeilThreads), 0, s, x, total, cpr, ld,
                     reinterpret_cast<uint32_t*>(out), s0, s1);
  return hipGetLastError();
}

}  // namespace signrot
