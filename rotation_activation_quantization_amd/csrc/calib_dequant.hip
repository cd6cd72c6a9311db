// Calibration (outlier channel and sign vector) and dequantization kernels.
//
// Calibration follows the SignRot abstract (one calibration pass that finds
// the massive-outlier channel and builds a sign vector) and the explainer's
// paragraph on the sign adjustment (the channel with the largest absolute
// activation; each column j of H is multiplied by the sign of that row's
// entry).  The global argmax is one 64-bit key per element,
//   key = |x| bits (15) << 48 | (2^20 - 1 - j) << 28 | (2^28 - 1 - t),
// so the unsigned maximum is the largest |x|, then the smallest channel j,
// then the smallest token t.  bf16 magnitudes order like their bit patterns.
#include <mutex>
#include <vector>

#include "device_common.h"

namespace signrot {

// The argmax record of signrot_calibrate_noalloc: key (word 0) and the bf16
// bits of M_c (word 1), in a file-scope device array instead of a per-call
// allocation.  Every call on a device reuses that device's copy (cleared by
// cal_init_kernel at the start of each call); calls that overlap on one
// device race on it.  Host code never passes the array's name to a kernel:
// it passes the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned long long scratch[kCalScratchWords];

namespace {

constexpr int kCalThreads = 256;

__device__ __forceinline__ unsigned long long cal_key(uint32_t bits, int64_t t, int64_t j) {
  return (static_cast<unsigned long long>(bits & 0x7fffu) << 48) |
         (static_cast<unsigned long long>(0xfffffu - static_cast<uint32_t>(j)) << 28) |
         static_cast<unsigned long long>(0x0fffffffu - static_cast<uint32_t>(t));
}

__global__ void cal_init_kernel(unsigned long long* scratch) {
  if (threadIdx.x == 0) {
    scratch[0] = 0ull;
    scratch[1] = 0ull;
  }
}

__global__ __launch_bounds__(kCalThreads) void cal_argmax_kernel(const uint16_t* x, int64_t tokens,
                                                                 int64_t n, int64_t ld,
                                                                 unsigned long long* scratch) {
  __shared__ unsigned long long red[kCalThreads / 64];
  unsigned long long best = 0ull;
  const int64_t total = tokens * n;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t t = e / n, j = e - t * n;
    const unsigned long long key = cal_key(x[t * ld + j], t, j);
    best = key > best ? key : best;
  }
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long other = __shfl_xor(best, o);
    best = other > best ? other : best;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kCalThreads / 64; ++i) best = red[i] > best ? red[i] : best;
    atomicMax(&scratch[0], best);
  }
}

// Sign bit (1 = negative) of entry j of row c of H = H_m (x) H_{2^k}: the
// Sylvester part from the parity of c & j over the low k bits, the outer part
// from the order-28 row masks passed by value (m = 28) or from the device mask
// table of H_m (other m > 1).
__device__ __forceinline__ uint32_t row_negbit(int c, int j, int k, int m, int hw, const uint32_t* hm,
                                               const H28Masks& h28) {
  const int bmask = (1 << k) - 1;
  uint32_t bit = __popc(static_cast<uint32_t>(c & j & bmask)) & 1u;
  if (m == 28) bit ^= (h28.m[c >> k] >> (j >> k)) & 1u;
  else if (m > 1) bit ^= (hm[(c >> k) * hw + ((j >> k) >> 5)] >> ((j >> k) & 31)) & 1u;
  return bit;
}

// Fills d[j] = sigma * H[c][j]; also records the bf16 bits of M_c in scratch[1].
__global__ void cal_fill_kernel(const uint16_t* x, int64_t ld, int n, int k, int m, int hw,
                                const uint32_t* hm, H28Masks h28, unsigned long long* scratch, int8_t* d) {
  const unsigned long long key = scratch[0];
  const int c = static_cast<int>(0xfffffu - static_cast<uint32_t>((key >> 28) & 0xfffffu));
  const int64_t t = static_cast<int64_t>(0x0fffffffu - static_cast<uint32_t>(key & 0x0fffffffu));
  const uint32_t mbits = x[t * ld + c];
  // sigma = sign(M_c), with sign(+-0) = +1
  const uint32_t neg = ((mbits & 0x7fffu) != 0u) && ((mbits & 0x8000u) != 0u);
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n; j += gridDim.x * blockDim.x)
    d[j] = (row_negbit(c, j, k, m, hw, hm, h28) ^ neg) ? static_cast<int8_t>(-1) : static_cast<int8_t>(1);
  if (blockIdx.x == 0 && threadIdx.x == 0) scratch[1] = mbits;
}

// d[j] = sigma * H[c][j] for a given (c, sigma): the same entries as the
// calibration fill.
__global__ void sign_fill_kernel(int n, int k, int m, int hw, const uint32_t* hm, H28Masks h28, int c, int neg,
                                 int8_t* d) {
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n; j += gridDim.x * blockDim.x)
    d[j] = (row_negbit(c, j, k, m, hw, hm, h28) ^ static_cast<uint32_t>(neg)) ? static_cast<int8_t>(-1)
                                                                             : static_cast<int8_t>(1);
}

// y[t][j] = scale[t] * (q - zero[t]); one thread per code byte.
__global__ void dequant_kernel(const uint8_t* codes, const float* scale, const float* zero,
                               int64_t tokens, int n, float* y) {
  const int64_t half = n / 2;
  const int64_t total = tokens * half;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t t = e / half;
    const uint32_t b = codes[e];
    const float s = scale[t], z = zero[t];
    float2 v;
    v.x = s * (static_cast<float>(b & 15u) - z);
    v.y = s * (static_cast<float>(b >> 4) - z);
    *reinterpret_cast<float2*>(y + 2 * e) = v;
  }
}

}  // namespace

hipError_t launch_calibrate(const uint16_t* x, int64_t tokens, int64_t ld, const Shape& sh,
                            int8_t* d_out, unsigned long long* scratch, hipStream_t s) {
  hipLaunchKernelGGL(cal_init_kernel, dim3(1), dim3(64), 0, s, scratch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t total = tokens * sh.n;
  int64_t blocks = (total + kCalThreads - 1) / kCalThreads;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(cal_argmax_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kCalThreads), 0, s,
                     x, tokens, static_cast<int64_t>(sh.n), ld, scratch);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t* hm = nullptr;
  if (sh.m > 1 && sh.m != 28 && !(hm = outer_mask_device(sh.m, &e, s))) return e;
  const int fill_blocks = (sh.n + 255) / 256;
  hipLaunchKernelGGL(cal_fill_kernel, dim3(fill_blocks), dim3(256), 0, s, x, ld, sh.n, sh.k, sh.m,
                     (sh.m + 31) / 32, hm, h28_masks(), scratch, d_out);
  return hipGetLastError();
}

unsigned long long* calib_scratch_device(hipError_t* err) {
  static std::mutex mu;
  static std::vector<unsigned long long*> per_dev;
  int dev = 0;
  if ((*err = hipGetDevice(&dev)) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= static_cast<int>(per_dev.size())) per_dev.resize(dev + 1, nullptr);
  if (!per_dev[dev]) {
    unsigned long long* ptr = nullptr;
    if ((*err = hipGetSymbolAddress(reinterpret_cast<void**>(&ptr), HIP_SYMBOL(scratch))) != hipSuccess)
      return nullptr;
    per_dev[dev] = ptr;
  }
  *err = hipSuccess;
  return per_dev[dev];
}

hipError_t launch_dequant(const uint8_t* codes, const float* scale, const float* zero, int64_t tokens,
                          int n, float* y, hipStream_t s) {
  const int64_t total = tokens * (n / 2);
  int64_t blocks = (total + 255) / 256;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 16;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(dequant_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, codes, scale,
                     zero, tokens, n, y);
  return hipGetLastError();
}

hipError_t launch_sign_fill(const Shape& sh, int c, int neg, int8_t* d, hipStream_t s) {
  hipError_t e = hipSuccess;
  const uint32_t* hm = nullptr;
  if (sh.m > 1 && sh.m != 28 && !(hm = outer_mask_device(sh.m, &e, s))) return e;
  const int blocks = (sh.n + 255) / 256;
  hipLaunchKernelGGL(sign_fill_kernel, dim3(blocks), dim3(256), 0, s, sh.n, sh.k, sh.m, (sh.m + 31) / 32, hm,
                     h28_masks(), c, neg, d);
  return hipGetLastError();
}

}  // namespace signrot
