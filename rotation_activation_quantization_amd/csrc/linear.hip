// The consumer of the INT4 activations: the down-projection on the folded
// weights, with the asymmetric zero-point handled by one precomputed sum per
// weight row (explainer "SignRot for 4-bit LLM quantization", paragraph on
// the symmetric versus the asymmetric quantizer):
//
//   out[t][k] = scale[t] * (sum_j q[t][j] W'[k][j] - zero[t] * rowsum[k]),
//   rowsum[k] = sum_j W'[k][j],
//
// which is sum_j yhat[t][j] W'[k][j] with yhat = scale * (q - zero).
//
// int4_linear_kernel is a bf16 MFMA GEMM (v_mfma_f32_16x16x32_bf16) whose A
// operand is read from the packed codes and widened to bf16 in registers (the
// integers 0..15 are exact in bf16), so the codes cross HBM and LDS at 4 bits
// a value.  B is W' in bf16.  Accumulation is binary32; the epilogue applies
// scale and zero.  Work-group tile 128 tokens x 256 weight rows x 64 k, four
// waves of 64 x 128, LDS double-buffered; one barrier per k step.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "wave_ops.h"

namespace signrot {
namespace {

using wave::bf16x8_t;
using wave::f32x4_t;
using wave::u32x4_t;

constexpr int kBM = 128;  // tokens per work-group tile
constexpr int kBN = 256;  // weight rows per work-group tile
constexpr int kBK = 64;   // k per LDS stage
constexpr int kThreads = 256;
constexpr int kAStage = kBM * kBK / 2;  // packed codes, 4 KiB
constexpr int kBStage = kBN * kBK * 2;  // bf16 weights, 32 KiB
constexpr int kStage = kAStage + kBStage;

// Eight codes (one dword; code 2i in the low nibble of byte i) -> the eight
// bf16 values of an MFMA operand, element e = code e.
__device__ __forceinline__ bf16x8_t widen8(uint32_t c) {
  const uint32_t lo = c & 0x0F0F0F0Fu;         // codes 0, 2, 4, 6
  const uint32_t hi = (c >> 4) & 0x0F0F0F0Fu;  // codes 1, 3, 5, 7
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float e0 = static_cast<float>((lo >> (8 * i)) & 0xffu);
    const float e1 = static_cast<float>((hi >> (8 * i)) & 0xffu);
    // top halves of the two binary32 values: (bf16(e0), bf16(e1)), exact
    r[i] = __builtin_amdgcn_perm(__float_as_uint(e1), __float_as_uint(e0), 0x07060302u);
  }
  return __builtin_bit_cast(bf16x8_t, r);
}

// Block id -> (token tile, row tile).  Consecutive block ids go to different
// XCDs (round-robin dispatch), so ids are first regrouped into one contiguous
// range per XCD; inside a range, tiles run token-tile fastest over groups of
// eight token tiles, so the work-groups resident on one XCD share a few
// panels of codes and weights in its L2.
__device__ __forceinline__ void tile_of(int bid, int nblocks, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int q = nblocks >> 3, rem = nblocks & 7;
  const int x = bid & 7, j = bid >> 3;
  const int p = (x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q) + j;
  constexpr int kGroup = 8;
  const int per_group = kGroup * tiles_n;
  const int group = p / per_group;
  const int first = group * kGroup;
  const int gm = min(tiles_m - first, kGroup);
  const int r = p - group * per_group;
  tm = first + r % gm;
  tn = r / gm;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void int4_linear_kernel(LinearArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int wm = wid & 1, wn = wid >> 1;  // wave tile: tokens 64*wm.., rows 128*wn..
  const int g = lane >> 4, nl = lane & 15;

  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, a.tiles_m, a.tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int64_t row_bytes = a.n >> 1;

  // Global -> LDS staging.  Codes: thread -> token row ra, 32 codes (16 B) at
  // k = 32*ha of the stage.  Weights: thread -> 16-B chunk cb of rows
  // rb0 + 32 i.  Rows past the end are clamped (their results are not stored).
  const int ra = tid >> 1, ha = tid & 1;
  const uint8_t* gA = a.codes + static_cast<int64_t>(min(m0 + ra, a.T - 1)) * row_bytes + 16 * ha;
  const int cb = tid & 7, rb0 = tid >> 3;
  int offB[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) offB[i] = min(n0 + rb0 + 32 * i, a.R - 1) * a.ldw + 8 * cb;

  // LDS layouts.  Codes, per wave-row half wm, in read order: the dword of
  // (token frag mf, k half kk, lane) at word 512 wm + 256 (mf>>1) + 4 lane +
  // 2 (mf&1) + kk, so each lane reads its eight dwords with two b128 reads.
  // Weights: row r (0..255) holds 8 chunks of 16 B, chunk c at c ^ (r & 7).
  const int rowA_w = ra >> 6, mfA = (ra >> 4) & 3, nlA = ra & 15;
  const int a_store = 4 * (512 * rowA_w + 256 * (mfA >> 1) + 4 * nlA + 2 * (mfA & 1) + ha);  // + 256 g bytes
  const int b_store = kAStage + 128 * rb0 + 16 * (cb ^ (rb0 & 7));                         // + 4096 i
  const int a_load = 2048 * wm + 16 * lane;                                                  // + 1024
  const int b_load = kAStage + 128 * (128 * wn + nl);                                        // + 2048 nf
  const int b_chunk = g ^ (nl & 7);                                                          // ^ 4 kk

  f32x4_t acc[4][8];
#pragma unroll
  for (int mf = 0; mf < 4; ++mf)
#pragma unroll
    for (int nf = 0; nf < 8; ++nf) acc[mf][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 ra_reg;
  uint4 rb_reg[8];
  auto gload = [&](int kt) {
    ra_reg = *reinterpret_cast<const uint4*>(gA + static_cast<int64_t>(kt) * (kBK / 2));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rb_reg[i] = *reinterpret_cast<const uint4*>(a.w + static_cast<int64_t>(offB[i]) + kt * kBK);
  };
  auto lstore = [&](int stage) {
    uint8_t* base = lds + stage * kStage;
    *reinterpret_cast<uint32_t*>(base + a_store) = ra_reg.x;
    *reinterpret_cast<uint32_t*>(base + a_store + 256) = ra_reg.y;
    *reinterpret_cast<uint32_t*>(base + a_store + 512) = ra_reg.z;
    *reinterpret_cast<uint32_t*>(base + a_store + 768) = ra_reg.w;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(base + b_store + 4096 * i) = rb_reg[i];
  };

  const int ktiles = a.n / kBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < ktiles; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < ktiles) gload(kt + 1);
    const uint8_t* base = lds + stage * kStage;
    const u32x4_t c01 = *reinterpret_cast<const u32x4_t*>(base + a_load);
    const u32x4_t c23 = *reinterpret_cast<const u32x4_t*>(base + a_load + 1024);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t af[4];
      af[0] = widen8(c01[kk]);
      af[1] = widen8(c01[2 + kk]);
      af[2] = widen8(c23[kk]);
      af[3] = widen8(c23[2 + kk]);
      const uint8_t* bb = base + b_load + 16 * (b_chunk ^ (4 * kk));
#pragma unroll
      for (int nf = 0; nf < 8; ++nf) {
        const bf16x8_t bf = *reinterpret_cast<const bf16x8_t*>(bb + 2048 * nf);
#pragma unroll
        for (int mf = 0; mf < 4; ++mf)
          acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mf], bf, acc[mf][nf], 0, 0, 0);
      }
    }
    if (kt + 1 < ktiles) {
      lstore(stage ^ 1);
      __syncthreads();
    }
  }

  // Epilogue: lane (g, nl) holds tokens 4g + r of each 16-token frag, for
  // weight row nl of each 16-row frag.
#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = m0 + 64 * wm + 16 * mf + 4 * g + r;
      if (t >= a.T) continue;
      const float s = a.scale[t], z = a.zero[t];
      float* orow = a.out + static_cast<int64_t>(t) * a.R;
#pragma unroll
      for (int nf = 0; nf < 8; ++nf) {
        const int k = n0 + 128 * wn + 16 * nf + nl;
        if (k < a.R) orow[k] = s * fmaf(-z, a.rowsum[k], acc[mf][nf][r]);
      }
    }
  }
}

// Any shape: one thread per output, binary32 accumulation over j in order.
__global__ void int4_linear_simple_kernel(LinearArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(a.T) * a.R) return;
  const int t = static_cast<int>(i / a.R);
  const int k = static_cast<int>(i - static_cast<int64_t>(t) * a.R);
  const uint8_t* c = a.codes + static_cast<int64_t>(t) * (a.n >> 1);
  const uint16_t* w = a.w + static_cast<int64_t>(k) * a.ldw;
  float acc = 0.f;
  for (int j = 0; j < a.n; j += 2) {
    const uint32_t b = c[j >> 1];
    acc = fmaf(static_cast<float>(b & 0xfu), __uint_as_float(static_cast<uint32_t>(w[j]) << 16), acc);
    acc = fmaf(static_cast<float>(b >> 4), __uint_as_float(static_cast<uint32_t>(w[j + 1]) << 16), acc);
  }
  a.out[i] = a.scale[t] * fmaf(-a.zero[t], a.rowsum[k], acc);
}

// rowsum[k] = sum_j w[k][j] over bf16 rows, accumulated in binary64 by one
// work-group per row and rounded once to binary32.
__global__ void weight_rowsum_kernel(const uint16_t* __restrict__ w, int64_t n, int64_t ld,
                                     float* __restrict__ rowsum) {
  const int64_t k = blockIdx.x;
  const uint16_t* row = w + k * ld;
  double acc = 0.0;
  for (int64_t j = threadIdx.x; j < n; j += blockDim.x)
    acc += static_cast<double>(__uint_as_float(static_cast<uint32_t>(row[j]) << 16));
  __shared__ double part[256];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int s = blockDim.x / 2; s > 0; s >>= 1) {
    if (static_cast<int>(threadIdx.x) < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) rowsum[k] = static_cast<float>(part[0]);
}

}  // namespace

bool int4_linear_fast_ok(const LinearArgs& a) {
  return a.n % kBK == 0 && a.ldw % 8 == 0 && static_cast<int64_t>(a.R) * a.ldw < (int64_t{1} << 31) &&
         (reinterpret_cast<uintptr_t>(a.codes) & 15u) == 0 && (reinterpret_cast<uintptr_t>(a.w) & 15u) == 0;
}

const char* int4_linear_name(const LinearArgs& a) {
  return int4_linear_fast_ok(a) ? "int4_linear_mfma" : "int4_linear_simple";
}

hipError_t launch_int4_linear(LinearArgs a, hipStream_t s) {
  if (int4_linear_fast_ok(a)) {
    a.tiles_m = (a.T + kBM - 1) / kBM;
    a.tiles_n = (a.R + kBN - 1) / kBN;
    const int64_t blocks = static_cast<int64_t>(a.tiles_m) * a.tiles_n;
    int4_linear_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s>>>(a);
  } else {
    const int64_t m = static_cast<int64_t>(a.T) * a.R;
    int4_linear_simple_kernel<<<dim3(static_cast<unsigned>((m + 255) / 256)), dim3(256), 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_weight_rowsum(const uint16_t* w, int64_t rows, int64_t n, int64_t ld, float* rowsum,
                                hipStream_t s) {
  weight_rowsum_kernel<<<dim3(static_cast<unsigned>(rows)), dim3(256), 0, s>>>(w, n, ld, rowsum);
  return hipGetLastError();
}

}  // namespace signrot
