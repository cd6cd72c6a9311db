// Shared by the fast rotate+INT4 kernels for gfx950 (rq_fast.hip: n = 28 * 2^k,
// k = 7..9, and n = 2^12..2^14; rq_halves.hip: n = 28 * 2^10): the row shape
// and LDS slot of a quad, the fused SwiGLU producer of the input, and guarded
// 16-byte stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "wave_ops.h"

namespace signrot {

// n = 28672 (rq_halves.hip)
hipError_t launch_rq_halves(const RqArgs& a, hipStream_t stream);

namespace {

using namespace wave;

template <int KA, int KB>
struct FastShape {
  static_assert(KA == 28 || KA == 32, "order-28 or Sylvester outer factor");
  static_assert(KB >= 7 && KB <= 9, "2 to 8 register tiles");
  static constexpr int kWaves = KA / 4;
  static constexpr int NKC = (KA + 7) / 8;       // K chunks of eight a-rows
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int NQ = 1 << (KB - 2);       // quads per a-row
  static constexpr int NT = NQ / 16;             // register tiles
  static constexpr int LG = (NT == 8) ? 3 : (NT == 4) ? 2 : 1;
  static constexpr int NV = 4 * NT;              // values per lane
  static constexpr int PB = 16 * NQ;             // bytes per pair-row
  static constexpr int kRowBytes = (KA / 2) * PB;
  // KA = 28: the fourth K chunk reads "pairs" 14 and 15 for lanes whose
  // weights are zero; two zero pair-rows behind the second buffer keep those
  // reads finite (for the first buffer they land in the second).
  static constexpr int kLdsBytes = 2 * kRowBytes + (KA == 28 ? 2 * PB : 0);
  static constexpr int CR = NQ / 2;              // 16-byte chunks per a-row
  static constexpr int CPT = CR / 16;            // chunks per thread per row
  static constexpr uint32_t KMUL = 256u + 128u / NT;
  static constexpr uint32_t SWZ = 8u / NT;
  static constexpr int N = KA << KB;
};

template <int KA, int KB>
__device__ __forceinline__ uint32_t quad_slot(uint32_t q) {
  using S = FastShape<KA, KB>;
  const uint32_t u = q & (S::NT - 1);
  return 16u * u + ((q >> S::LG) ^ (u * S::SWZ));
}

// x = bf16(SiLU(gate) * up) for the eight bf16 pairs of two 16-byte chunks:
// SiLU(z) = z / (1 + e^-z) with e^-z = 2^(-z log2 e) (v_exp_f32) and the
// reciprocal v_rcp_f32, in binary32, rounded once to bf16 by the hardware
// conversion (nearest, ties to even).  Relative error before that rounding
// stays below about 2e-6 for |gate| <= 16.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.44269504088896341f));
}
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
__device__ __forceinline__ u32x4_t swiglu_chunk(const u32x4_t& g, const u32x4_t& u) {
  u32x4_t x;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float lo = silu_f32(bf16_lo(g[k])) * bf16_lo(u[k]);
    const float hi = silu_f32(bf16_hi(g[k])) * bf16_hi(u[k]);
    x[k] = __builtin_bit_cast(uint32_t, bf16x2_t{static_cast<__bf16>(lo), static_cast<__bf16>(hi)});
  }
  return x;
}

// 16-byte stores that hold their data registers for two wait states.  On
// gfx950 a VALU write to a data register of a store wider than 8 bytes issued
// directly after the store changed the stored value (the compiler emitted such
// writes with no wait state between, reusing the registers of one y chunk for
// the next); the asm reads the data registers after an s_nop, so no write to
// them can come earlier.
template <int AUX>
__device__ __forceinline__ void store_b128_held(const u32x4_t& v, __amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, voff, soff, AUX);
  asm volatile("s_nop 1" : : "v"(v) : "memory");
}
__device__ __forceinline__ void store_f32x4_held(float* p, const f32x4_t& v) {
  *reinterpret_cast<f32x4_t*>(p) = v;
  asm volatile("s_nop 1" : : "v"(v) : "memory");
}

}  // namespace
}  // namespace signrot
