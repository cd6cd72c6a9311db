// Wave-level building blocks shared by the MFMA rotate+quant kernels (gfx950):
// operand vector types, the DPP butterfly stages of the 16-point lane
// transform, in-register butterflies, min/max helpers and wave reductions,
// buffer resources, and the LDS-only barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace signrot {
namespace wave {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// The four DPP stages below (masks 1, 2, 7, 8 with the sign selectors
// gdpp0..3 of the kernels) compute the 16-point Walsh-Hadamard transform of
// the values held by the lanes of a 16-lane row when lane nl starts with the
// input of index nl ^ kXLane; the output of index lane_perm(nl) ends in lane nl.
constexpr int kXLane = 12;

// Output pair-lane index of lane n after the four DPP stages (a linear map on
// the 4 lane bits): bit 0 -> 5, bit 1 -> 6, bit 2 -> 7, bit 3 -> 8.
__device__ __forceinline__ int lane_perm(int nl) {
  int r = (nl & 8);
  if (nl & 1) r ^= 5;
  if (nl & 2) r ^= 6;
  if (nl & 4) r ^= 7;
  return r;
}

__device__ __forceinline__ uint16_t bf16_of_sign(int s) {
  return s > 0 ? 0x3f80u : (s < 0 ? 0xbf80u : 0u);
}

// Entry (row, col) of the outer Hadamard factor: Paley's H28 (row masks in
// h28, bit set = -1) or the Sylvester matrix.
template <int KA>
__device__ __forceinline__ int hka_sign(const uint32_t* h28, int row, int col) {
  if (KA == 28) return ((h28[row] >> col) & 1u) ? -1 : 1;
  return (__popc(static_cast<uint32_t>(row & col)) & 1) ? -1 : 1;
}

// One DPP butterfly stage on 16 registers: v += g * v[lane ^ m] (m given by
// the DPP control).  The leading s_nop covers the VALU-write -> DPP-read hazard
// for whatever instruction preceded the block; inside the block every
// instruction reads and writes its own register.
#define SR_DPP16(CTRL, R, G)                                                              \
  asm volatile("s_nop 1\n"                                                               \
               "v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"        \
               "v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"        \
               "v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"        \
               "v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"        \
               "v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"        \
               "v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"        \
               "v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"        \
               "v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"        \
               "v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"        \
               "v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"        \
               "v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"      \
               "v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"      \
               "v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"      \
               "v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"      \
               "v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"      \
               "v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf\n"      \
               : "+v"(R[0]), "+v"(R[1]), "+v"(R[2]), "+v"(R[3]), "+v"(R[4]), "+v"(R[5]),   \
                 "+v"(R[6]), "+v"(R[7]), "+v"(R[8]), "+v"(R[9]), "+v"(R[10]), "+v"(R[11]), \
                 "+v"(R[12]), "+v"(R[13]), "+v"(R[14]), "+v"(R[15])                        \
               : "v"(G))

// The same on 8 registers.
#define SR_DPP8(CTRL, R, G)                                                              \
  asm volatile("s_nop 1\n"                                                              \
               "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
               "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
               "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
               "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
               "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
               "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
               "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
               "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf\n"         \
               : "+v"(R[0]), "+v"(R[1]), "+v"(R[2]), "+v"(R[3]), "+v"(R[4]), "+v"(R[5]),  \
                 "+v"(R[6]), "+v"(R[7])                                                   \
               : "v"(G))

template <int NV>
__device__ __forceinline__ void dpp_stage(float (&v)[NV], float g, int which) {
  static_assert(NV % 8 == 0, "registers in blocks of 8");
#pragma unroll
  for (int b = 0; b + 16 <= NV; b += 16) {
    float* R = v + b;
    if (which == 0) SR_DPP16("quad_perm:[1,0,3,2]", R, g);
    else if (which == 1) SR_DPP16("quad_perm:[2,3,0,1]", R, g);
    else if (which == 2) SR_DPP16("row_half_mirror", R, g);
    else SR_DPP16("row_ror:8", R, g);
  }
  if (NV % 16 != 0) {
    float* R = v + (NV - 8);
    if (which == 0) SR_DPP8("quad_perm:[1,0,3,2]", R, g);
    else if (which == 1) SR_DPP8("quad_perm:[2,3,0,1]", R, g);
    else if (which == 2) SR_DPP8("row_half_mirror", R, g);
    else SR_DPP8("row_ror:8", R, g);
  }
}

// In-register butterflies (p, q) -> (p + q, p - q) over tile bit U of the
// value array v[t * 4 + r].
template <int NT, int U>
__device__ __forceinline__ void reg_stage(float (&v)[NT * 4]) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t & (1 << U)) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float& p = v[t * 4 + r];
      float& q = v[(t | (1 << U)) * 4 + r];
      const float s = p + q;
      const float dd = p - q;
      p = s;
      q = dd;
    }
  }
}

// acc = min(acc, x, y) and acc = max(acc, x, y) as single v_min3/v_max3 ops
__device__ __forceinline__ void min3_acc(float& acc, float x, float y) {
  asm("v_min3_f32 %0, %0, %1, %2" : "+v"(acc) : "v"(x), "v"(y));
}
__device__ __forceinline__ void max3_acc(float& acc, float x, float y) {
  asm("v_max3_f32 %0, %0, %1, %2" : "+v"(acc) : "v"(x), "v"(y));
}

// Plain v_min_f32 / v_max_f32.  fminf / fmaxf make the compiler quiet NaN
// inputs with an extra v_max_f32 x, x, x on every operand it cannot prove
// canonical (DPP results, LDS loads); the inputs here are finite.
__device__ __forceinline__ float fmin_raw(float x, float y) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(y));
  return r;
}
__device__ __forceinline__ float fmax_raw(float x, float y) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(y));
  return r;
}

// Wave-wide min and max, the result guaranteed in lane 63 (other lanes end
// with the min / max of a subset of the wave, never below / above the true
// one): DPP inside 16-lane rows (lane ^ 1, lane ^ 2, mirror in 8, mirror in
// 16), then the gfx9 row broadcasts (rows 1 and 3 take the last lane of rows
// 0 and 2; rows 2 and 3 take the last lane of row 1).  Each step is one
// v_min / v_max with a DPP source; the s_nop cover the VALU-write ->
// DPP-read hazard of the chained registers.
__device__ __forceinline__ void wave_minmax(float& mn, float& mx) {
  asm volatile(
      "s_nop 1\n"
      "v_min_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_min_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_min_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n"
      "v_max_f32_dpp %1, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_min_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n"
      "v_max_f32_dpp %1, %1, %1 row_mirror row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_min_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n"
      "v_max_f32_dpp %1, %1, %1 row_bcast:15 row_mask:0xa bank_mask:0xf\n"
      "s_nop 1\n"
      "v_min_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n"
      "v_max_f32_dpp %1, %1, %1 row_bcast:31 row_mask:0xc bank_mask:0xf\n"
      : "+v"(mn), "+v"(mx));
}

// Quantizer constants of a token from the min and max of its rotated values
// (any common scale): inv = 15 / range through v_rcp_f32 (within 1 ulp, so a
// code can move only for a value within ~1e-6 of a rounding boundary), the
// offset cq = -mn * inv, and the zero-point in code units -(mn + shift) * inv
// when the values exclude a constant shift.  A zero range gives inv = 0, all
// codes 0.
struct QuantParams {
  float inv, cq, range;
  bool degenerate;
};
__device__ __forceinline__ QuantParams quant_params(float mn, float mx) {
  QuantParams q;
  q.range = mx - mn;
  q.degenerate = !(q.range > 0.0f);
  q.inv = q.degenerate ? 0.0f : 15.0f * __builtin_amdgcn_rcpf(q.range);
  q.cq = -mn * q.inv;
  return q;
}

// Workgroup barrier that orders LDS only: this wave's LDS operations complete,
// then s_barrier.  Unlike __syncthreads() it does not wait for outstanding
// global loads and stores (the next row's DMA and this row's code stores stay
// in flight); the memory clobber keeps the compiler from moving memory
// accesses across it.  Global data that other waves read from LDS (the DMA'd
// row) is covered by an explicit vmcnt wait before the barrier that needs it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// vmcnt(N) with expcnt and lgkmcnt left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

// Cache policy of the buffer accesses that touch each byte once (the row
// loads and the code stores): the gfx940+ nontemporal bit.  Timed on the
// n = 14336 x 8192 workload it saves about 2% (from the stores).
constexpr int kNontemporal = 2;

// Buffer resource over `bytes` bytes from a wave-uniform base (raw access,
// no stride).  Loads and stores through it take the base from scalar
// registers and a 32-bit per-lane offset, so no per-lane 64-bit address is
// kept or recomputed per row; accesses beyond `bytes` read 0 and write nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

}  // namespace wave
}  // namespace signrot
