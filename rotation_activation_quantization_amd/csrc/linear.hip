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
// scale and zero.  Work-group tile 256 tokens x 256 weight rows, k steps of
// 64, eight waves of 64 x 128; both operands stream global -> LDS through
// four-deep rings; one barrier per k step.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "wave_ops.h"

namespace signrot {
namespace {

using wave::bf16x8_t;
using wave::f32x4_t;
using wave::u32x4_t;

constexpr int kBM = 256;  // tokens per work-group tile
constexpr int kBN = 256;  // weight rows per work-group tile
constexpr int kBK = 64;   // k per step
constexpr int kThreads = 512;
constexpr int kStages = 4;
constexpr int kBStage = kBN * kBK * 2;  // one LDS buffer of bf16 weights, 32 KiB
constexpr int kAStage = kBM * kBK / 2;  // one LDS buffer of packed codes, 8 KiB

typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

// Eight codes (one dword; code 2i in the low nibble of byte i) -> the eight
// bf16 values of an MFMA operand, element e = code e, in two halves so that
// the conversion can be spread between MFMAs.  Nibbles: codes 0, 2, 4, 6 in
// the bytes of lo, codes 1, 3, 5, 7 in the bytes of hi.
struct Nibbles {
  uint32_t lo, hi;
};
__device__ __forceinline__ Nibbles split_nibbles(uint32_t c) {
  Nibbles v{c & 0x0F0F0F0Fu, (c >> 4) & 0x0F0F0F0Fu};
  // hide the known-zero high nibbles, so that each byte goes through one
  // v_cvt_f32_ubyte{0..3} instead of an extract and a convert
  asm("" : "+v"(v.lo), "+v"(v.hi));
  return v;
}
// Words 2h and 2h + 1 of the operand: elements 4h .. 4h + 3.
template <int H>
__device__ __forceinline__ void widen_half(const Nibbles& v, u32x4_t& r) {
#pragma unroll
  for (int i = 2 * H; i < 2 * H + 2; ++i) {
    const float e0 = static_cast<float>((v.lo >> (8 * i)) & 0xffu);
    const float e1 = static_cast<float>((v.hi >> (8 * i)) & 0xffu);
    // top halves of the two binary32 values: (bf16(e0), bf16(e1)), exact
    r[i] = __builtin_amdgcn_perm(__float_as_uint(e1), __float_as_uint(e0), 0x07060302u);
  }
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

// The MFMA's 32 k positions are a free relabelling of channels, as long as
// both operands use the same one: in k step kt, lane group g (lanes 16 g ..
// 16 g + 15) takes channels 64 kt + 16 g + 8 kk + (0..7) for MFMA half kk.
// A lane's codes for both halves are then 8 consecutive bytes, and its
// weights chunk 2 g + kk of the row's 128-byte k slice.
//
// Both operands go global -> LDS by global_load_lds_dwordx4 (lane L of an
// instruction writes LDS bytes 16 L .. 16 L + 15 above the wave-uniform base),
// into rings of four buffers; no global load targets registers, so every
// memory wait in the loop is the explicit one before the barrier.
//
// Weights, 32 KiB a step, [256 rows][8 chunks of 16 bytes]: instruction i of
// wave w fills rows 32 w + 8 i .. + 7, lane L at row (L >> 3), physical chunk
// L & 7.  Logical chunk c of row r sits at physical chunk c ^ h(r),
// h(r) = (r & 7) ^ ((r >> 3) & 1).  An operand read has 16 lanes on 16
// consecutive rows at one logical chunk; with this h the rocprofv3 counter
// SQ_LDS_BANK_CONFLICT reads zero for them on gfx950, where no swizzle, or
// c ^ (r & 7), cost 12 and 4 conflict cycles per read.
//
// Codes, 8 KiB a step (256 tokens x 32 bytes): wave w fills token rows
// 32 w .. + 31; in each 16-row group the first 16 bytes of every row come
// first (256 bytes), then the second 16 bytes.  Each lane reads its 8 bytes
// of a step with one conflict-free 8-byte LDS read.
//
// Eight waves: wave (wm, wn) owns tokens 64 wm .. + 63 and rows
// 128 wn .. + 127 of the tile.  Step kt: read the next step's codes from LDS;
// half 0 (32 MFMAs on the codes widened last step, while half 1's are
// widened); half 1 (32 MFMAs, while the next step's half 0 is widened, and
// step kt + 3's codes and weights are issued into the buffers step kt - 1
// used); then wait for step kt + 2's codes (and so for everything older) and
// pass one barrier.  Weights have two steps to arrive, codes one and a half.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void int4_linear_kernel(LinearArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * (kBStage + kAStage)];
  uint8_t* const lds_b = lds;
  uint8_t* const lds_a = lds + kStages * kBStage;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid & 3, wn = wid >> 2;
  const int g = lane >> 4, nl = lane & 15;

  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, a.tiles_m, a.tiles_n, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int ktiles = a.n / kBK;
  const int last = ktiles - 1;

  // Code source of lane L (rows clamped; their results are not stored):
  // token row 32 wid + 16 (L >> 5) + (L & 15), bytes 16 ((L >> 4) & 1) of the step
  const uint32_t row_bytes = static_cast<uint32_t>(a.n) >> 1;
  const uint32_t offA =
      static_cast<uint32_t>(min(m0 + 32 * wid + 16 * (lane >> 5) + (lane & 15), a.T - 1)) * row_bytes +
      16 * ((lane >> 4) & 1);
  // Weight source of lane L in instruction i (rows clamped): tile row r =
  // 32 wid + 8 i + (L >> 3), logical chunk (L & 7) ^ h(r)
  auto h = [](int r) { return (r & 7) ^ ((r >> 3) & 1); };
  uint32_t offB[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wid + 8 * i + (lane >> 3);
    offB[i] = static_cast<uint32_t>(min(n0 + r, a.R - 1)) * a.ldw + 8 * ((lane & 7) ^ h(r));
  }
  // operand rows 128 wn + 16 nf + nl: h depends on nl only
  const int b_load = 128 * (128 * wn + nl);  // + 2048 nf
  const int b_kk[2] = {16 * ((2 * g) ^ h(nl)), 16 * ((2 * g + 1) ^ h(nl))};
  // codes of frag mf for this lane: 8 bytes at a_load + 512 mf
  const int a_load = 2048 * wm + 256 * (g >> 1) + 16 * nl + 8 * (g & 1);

  // Every step issues exactly one code and four weight loads per wave
  // (clamped to the last step at the end), so the vmcnt thresholds are exact.
  // Load j of step kt: j = 0 the codes, j = 1..4 the weights.
  auto issue_one = [&](int kt, int j) {
    const int ks = min(kt, last);
    const int buf = kt & (kStages - 1);
    if (j == 0) {
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(a.codes + offA + 32u * ks),
                                       (__attribute__((address_space(3))) void*)(lds_a + buf * kAStage + 1024 * wid),
                                       16, 0, 0);
    } else {
      __builtin_amdgcn_global_load_lds(
          static_cast<const void*>(a.w + ks * kBK + offB[j - 1]),
          (__attribute__((address_space(3))) void*)(lds_b + buf * kBStage + 4096 * wid + 1024 * (j - 1)), 16, 0, 0);
    }
  };
  auto read_codes = [&](int kt, u32x2_t (&dst)[4]) {
    const uint8_t* src = lds_a + (kt & (kStages - 1)) * kAStage + a_load;
#pragma unroll
    for (int mf = 0; mf < 4; ++mf) {
      dst[mf] = *reinterpret_cast<const u32x2_t*>(src + 512 * mf);
      // both dwords are used (one now, one a step later): keep the read 8 bytes wide
      asm("" : "+v"(dst[mf]));
    }
  };

  f32x4_t acc[4][8];
#pragma unroll
  for (int mf = 0; mf < 4; ++mf)
#pragma unroll
    for (int nf = 0; nf < 8; ++nf) acc[mf][nf] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t af[2][4];  // widened codes of half 0 and half 1

#pragma unroll
  for (int j = 0; j < 15; ++j) issue_one(j / 5, j % 5);
  wave::wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  u32x2_t c0[4];  // codes of the current step
  read_codes(0, c0);
#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
    const Nibbles v = split_nibbles(c0[mf][0]);
    widen_half<0>(v, af[0][mf]);
    widen_half<1>(v, af[0][mf]);
  }

  for (int kt = 0; kt <= last; ++kt) {
    const uint8_t* const sbase = lds_b + (kt & (kStages - 1)) * kBStage;
    u32x2_t c1[4];  // codes of the next step
    read_codes(kt + 1, c1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      Nibbles v[4];
      const uint8_t* const bsrc = sbase + b_load + b_kk[kk];
      u32x4_t bf[8];
      bf[0] = *reinterpret_cast<const u32x4_t*>(bsrc);
      bf[1] = *reinterpret_cast<const u32x4_t*>(bsrc + 2048);
#pragma unroll
      for (int nf = 0; nf < 8; ++nf) {
        if (nf + 2 < 8) bf[nf + 2] = *reinterpret_cast<const u32x4_t*>(bsrc + 2048 * (nf + 2));
        // step kt + 3's loads, spread over the second half
        if (kk == 1 && nf < 5) issue_one(kt + 3, nf);
#pragma unroll
        for (int mf = 0; mf < 4; ++mf)
          acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[kk][mf]),
                                                                __builtin_bit_cast(bf16x8_t, bf[nf]), acc[mf][nf],
                                                                0, 0, 0);
        // one half of one dword per frag column: four dwords over eight columns
        const int mfw = nf >> 1;
        const uint32_t src = kk == 0 ? c0[mfw][1] : c1[mfw][0];
        if ((nf & 1) == 0) {
          v[mfw] = split_nibbles(src);
          widen_half<0>(v[mfw], af[kk ^ 1][mfw]);
        } else {
          widen_half<1>(v[mfw], af[kk ^ 1][mfw]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int mf = 0; mf < 4; ++mf) c0[mf] = c1[mf];
    // after step kt + 2's code load (second half of step kt - 1) came nine
    // loads: weights kt + 2, codes kt + 3, weights kt + 3
    wave::wait_vmcnt<9>();
    __builtin_amdgcn_s_barrier();
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
         static_cast<int64_t>(a.T) * (a.n / 2) < (int64_t{1} << 31) &&
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
