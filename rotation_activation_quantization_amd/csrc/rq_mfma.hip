// Fused rotate + sign flip + per-token asymmetric INT4 for gfx950, built
// around one bf16 MFMA stage.
//
// Index split.  A token row of n = KA * 2^kb values (KA = 28 for the Paley
// widths, 32 for pure powers of two) is viewed as X[a][b] with i = a*2^kb + b.
// The transform is Y = H_KA^T-mix over a, then a Walsh-Hadamard transform over
// b (explainer "SignRot for 4-bit LLM quantization", paragraphs on rotation
// and on the down-projection: a Hadamard matrix applied with a fast
// Walsh-Hadamard transform).  Adjacent b come in pairs p = b >> 1.
//
// Stage 1 (MFMA, exact): v_mfma_f32_16x16x32_bf16 on the raw bf16 input
// contracts over k = (a, b&1) and produces m = (a', b'&1): the KA-point mix
// fused with the first butterfly stage.  Products are +-1 * bf16, so they are
// exact; only the fp32 accumulation rounds.  The data operand is gathered from
// LDS one dword (a pair of bf16) at a time.
//
// Stage 2 (VALU): the Walsh-Hadamard transform over the pair index, four lane
// bits with v_fmac_f32_dpp butterflies inside 16-lane rows and the remaining
// bits across registers.
//
// Stage 3 (VALU): min/max, scale and zero-point, rounding by v_cvt_pk_u8_f32
// (round half to even, clamped), nibble packing, stores.
//
// Sign vector.  When d = sigma * (row c of H) -- the form calibration
// produces (explainer, paragraph on the sign adjustment) -- the flip costs no
// arithmetic: sigma * H_KA[c_a][a'] is folded into the MFMA weights, the
// Sylvester part (-1)^popcount(c_b & b') becomes the input permutation
// b -> b xor c_b (gather addresses, MFMA weights and the signs of the
// register butterflies), and the outlier x_c itself is taken out of the
// transform and added back as the constant sigma * x_c.  Any other d is
// applied element by element after the transform (GENERAL instance).
//
// Work split: one workgroup of four waves per token row; wave w computes the
// output rows a' in [8w, 8w+8) for every b.  Each row is staged in LDS by the
// global->LDS DMA (global_load_lds_dwordx4), one a-row per instruction.
#include <math.h>

#include "device_common.h"

namespace signrot {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kLanePerm[16] = {0, 5, 6, 3, 7, 2, 1, 4, 8, 13, 14, 11, 15, 10, 9, 12};
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

template <int NV>
__device__ __forceinline__ void dpp_stage(float (&v)[NV], float g, int which) {
  static_assert(NV % 16 == 0, "registers in blocks of 16");
#pragma unroll
  for (int b = 0; b < NV; b += 16) {
    float* R = v + b;
    if (which == 0) SR_DPP16("quad_perm:[1,0,3,2]", R, g);
    else if (which == 1) SR_DPP16("quad_perm:[2,3,0,1]", R, g);
    else if (which == 2) SR_DPP16("row_half_mirror", R, g);
    else SR_DPP16("row_ror:8", R, g);
  }
}

// In-register butterflies over tile bit U of the value array laid out as
// v[(c0 * NT + t) * 4 + r].  FLIP negates the difference outputs.
// In-register butterflies over tile bit U of v[t * 4 + r].
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

// Wave-wide min and max, every lane gets the result: DPP inside 16-lane rows,
// then the gfx950 row swaps across rows and halves.
__device__ __forceinline__ float dpp_f(float x, int ctrl_sel) {
  int xi = __float_as_int(x);
  switch (ctrl_sel) {
    case 0: xi = __builtin_amdgcn_mov_dpp(xi, 0xB1, 0xF, 0xF, true); break;   // lane ^ 1
    case 1: xi = __builtin_amdgcn_mov_dpp(xi, 0x4E, 0xF, 0xF, true); break;   // lane ^ 2
    case 2: xi = __builtin_amdgcn_mov_dpp(xi, 0x141, 0xF, 0xF, true); break;  // lane ^ 7
    default: xi = __builtin_amdgcn_mov_dpp(xi, 0x140, 0xF, 0xF, true); break; // lane ^ 15
  }
  return __int_as_float(xi);
}

__device__ __forceinline__ void wave_minmax(float& mn, float& mx) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    mn = fminf(mn, dpp_f(mn, c));
    mx = fmaxf(mx, dpp_f(mx, c));
  }
  {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mn = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    mx = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  }
  {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(mn), __float_as_uint(mn), false, false);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mn = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    mx = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  }
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

// Work split: four waves per token row.  Wave w owns the output rows
// a' = 8 w .. 8 w + 7; its MFMA tile row m is a' = 8 w + (m >> 1) with the
// first-butterfly parity c0 = m & 1, so a lane holds both parities of its a'
// and packs nibbles in registers.  Lane (g, nl) of wave w ends up with
// v[t * 4 + r] = y'[a' = 8 w + 2 g + (r >> 1)][pair = NT * perm(nl) + t][c0 = r & 1].
template <int KA, int LOGNT, bool GENERAL, bool YOUT>
__device__ void rq_mfma_body(const RqArgs& a, uint8_t* lds, const uint32_t* dbits_lds, const uint32_t* h28,
                             const DForm& form, uint32_t* red_lds, float* xc_lds) {
  constexpr int NT = 1 << LOGNT;          // tiles of pairs held in registers
  constexpr int NV = NT * 4;              // values per lane
  constexpr int ROWB = 64 * NT;           // bytes of one a-row (= 32 NT bf16)
  constexpr int PITCH = ROWB + 4;         // LDS pitch: rows start 1 dword apart mod 4
  static_assert(NT == 16, "one DMA instruction (64 x 16 B) per a-row");
  constexpr int KB = LOGNT + 5;           // log2 of the b range
  constexpr int NPAIR = 1 << (KB - 1);    // pairs per a-row
  constexpr int kDmaPerWave = (KA + kWaves - 1) / kWaves;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int nl = lane & 15;

  // sign-vector form (uniform across the block)
  const int c = GENERAL ? 0 : __builtin_amdgcn_readfirstlane(form.c);
  const int ca = c >> KB;
  const int cb = c & ((1 << KB) - 1);
  const int cb0 = cb & 1;
  const int cbp = cb >> 1;                                           // pair part of c_b
  const int cbp_lo = cbp & (NT - 1);                                 // register (tile) bits
  const int cbp_hi = cbp >> LOGNT;                                   // lane bits
  const int sig = (!GENERAL && form.neg) ? -1 : 1;

  // MFMA weights (A operand): lane holds A[m = nl][k = 8 g + i] with
  // m -> (a' = 8 w + (nl >> 1), c0 = nl & 1) and k -> (a = 16 s + 4 (i >> 1) + g, b0 = i & 1).
  bf16x8_t wA[2];
  {
    const int ap = 8 * w + (nl >> 1);
    const int c0 = nl & 1;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ar = 16 * s + 4 * (i >> 1) + g;
        const int b0 = i & 1;
        int wv = 0;
        if (ap < KA && ar < KA) {
          wv = sig * hka_sign<KA>(h28, ca, ap) * hka_sign<KA>(h28, ar, ap);
          if (((b0 ^ cb0) & c0) != 0) wv = -wv;
        }
        wA[s][i] = static_cast<short>(bf16_of_sign(wv));
      }
  }

  // DPP butterfly multipliers (dual-basis selectors of the masks 1, 2, 7, 8)
  const float gdpp0 = (((nl >> 0) ^ (nl >> 2)) & 1) ? -1.0f : 1.0f;
  const float gdpp1 = (((nl >> 1) ^ (nl >> 2)) & 1) ? -1.0f : 1.0f;
  const float gdpp2 = ((nl >> 2) & 1) ? -1.0f : 1.0f;
  const float gdpp3 = ((nl >> 3) & 1) ? -1.0f : 1.0f;

  // LDS layout of an a-row: 16-byte slot 16 j + m holds the global chunk
  // 4 m + j (pairs 16 m + 4 j .. +3).  Lane (g, nl) gathers, for register tile
  // t, the pair 16 m + (t ^ cbp_lo) with m = nl ^ kXLane ^ cbp_hi from the
  // a-rows 16 s + 4 j + g: the input permutation b -> b xor c_b and the sign
  // pattern left by the DPP stages both become addresses.
  const int mlane = nl ^ kXLane ^ cbp_hi;
  const uint32_t gbase = static_cast<uint32_t>(g * PITCH + 16 * mlane);
  uint32_t gaddr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tt = t ^ cbp_lo;
    gaddr[t] = gbase + static_cast<uint32_t>(256 * (tt >> 2) + 4 * (tt & 3));
  }
  const int outm = lane_perm(nl);                 // lane bits of the output pair
  const int ap0 = 8 * w + 2 * g;                   // first of this lane's two a'
  const bool pad_lane = ap0 >= KA;                 // both a' are padding

  // General d: the 2 NT values of output row a' held by a lane are the 32
  // consecutive channels a' 2^KB + 2 NT outm + (0 .. 2NT-1), i.e. one word of
  // the d bitmask kept in LDS; the two words are re-read every row (keeping
  // 64 hoisted sign masks alive would cost registers on every path).
  const uint32_t dword_off0 = static_cast<uint32_t>(((ap0 + 0) << (KB - 5)) + outm);
  const uint32_t dword_off1 = static_cast<uint32_t>(((ap0 + 1) << (KB - 5)) + outm);

  const int64_t tokens = a.tokens;
  const int n = a.n;
  const int dma_row0 = w * kDmaPerWave;
  const int dma_rows = (KA - dma_row0) < kDmaPerWave ? (KA - dma_row0) : kDmaPerWave;
  // DMA lane L fills slot L of an a-row from global chunk 4 (L & 15) + (L >> 4)
  const uint32_t dma_src = static_cast<uint32_t>(16 * (4 * (lane & 15) + (lane >> 4)));

  auto issue_dma = [&](int64_t row) {
    const uint8_t* rowp = reinterpret_cast<const uint8_t*>(a.x + row * a.ld);
#pragma unroll
    for (int q = 0; q < kDmaPerWave; ++q) {
      if (q < dma_rows) {
        const int ar = dma_row0 + q;
        const uint8_t* src = rowp + ar * ROWB;
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(src + dma_src),
            (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) uint8_t*)lds + ar * PITCH),
            16, 0, 0);
      }
    }
  };

  int64_t row = blockIdx.x;
  if (row < tokens) issue_dma(row);
  bool first = true;

  for (; row < tokens; row += gridDim.x) {
    // (1) this row's a-rows are in LDS.  After the DMA this wave issued at
    // least the 2 code stores of the previous row (more with scale/zero or
    // y_out), so vmcnt(2) covers the DMA; the first row has nothing after it.
    if (first) wait_vmcnt<0>();
    else wait_vmcnt<2>();
    first = false;
    if (!GENERAL) {
      const int owner = ca / kDmaPerWave;
      if (w == owner && lane == 0) {
        const int pc = cb >> 1;
        const int slot = 16 * ((pc >> 2) & 3) + (pc >> 4);
        uint16_t* px = reinterpret_cast<uint16_t*>(lds + ca * PITCH + 16 * slot + 4 * (pc & 3) + 2 * (cb & 1));
        xc_lds[0] = __uint_as_float(static_cast<uint32_t>(*px) << 16);
        *px = 0;
      }
    }
    lds_barrier();
    const float xc = GENERAL ? 0.0f : xc_lds[0];

    // (2) MFMA stage: gather the data operand (dwords = bf16 pairs) and
    // multiply; the gathers of tile t+1 are issued before the MFMAs of tile t.
    float v[NV];
    auto gather = [&](int t, u32x4_t& w0, u32x4_t& w1) {
      const uint8_t* base = lds + gaddr[t];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w0[j] = *reinterpret_cast<const uint32_t*>(base + (4 * j) * PITCH);
        w1[j] = (16 + 4 * j < KA) ? *reinterpret_cast<const uint32_t*>(base + (16 + 4 * j) * PITCH) : 0u;
      }
    };
    u32x4_t cw0, cw1;
    gather(0, cw0, cw1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      u32x4_t nw0, nw1;
      if (t + 1 < NT) gather(t + 1, nw0, nw1);
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wA[0], __builtin_bit_cast(bf16x8_t, cw0), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wA[1], __builtin_bit_cast(bf16x8_t, cw1), acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) v[t * 4 + r] = acc[r];
      if (t + 1 < NT) {
        cw0 = nw0;
        cw1 = nw1;
      }
    }
    // (3) every wave has read the row buffer: start the next row's DMA
    lds_barrier();
    const int64_t next = row + gridDim.x;
    if (next < tokens) issue_dma(next);

    // (4) Walsh-Hadamard transform over the pair index
    reg_stage<NT, 0>(v);
    reg_stage<NT, 1>(v);
    reg_stage<NT, 2>(v);
    reg_stage<NT, 3>(v);
    dpp_stage<NV>(v, gdpp0, 0);
    dpp_stage<NV>(v, gdpp1, 1);
    dpp_stage<NV>(v, gdpp2, 2);
    dpp_stage<NV>(v, gdpp3, 3);

    if (GENERAL) {
      uint32_t dword[2] = {0u, 0u};
      if (ap0 < KA) dword[0] = dbits_lds[dword_off0];
      if (ap0 + 1 < KA) dword[1] = dbits_lds[dword_off1];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int bitpos = 2 * t + (r & 1);
          const uint32_t sbit = (dword[r >> 1] << (31 - bitpos)) & 0x80000000u;
          float& x = v[t * 4 + r];
          x = __uint_as_float(__float_as_uint(x) ^ sbit);
        }
    }

    // (5) min / max over the row
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int e = 1; e + 1 < NV; e += 2) {
      min3_acc(mn, v[e], v[e + 1]);
      max3_acc(mx, v[e], v[e + 1]);
    }
    mn = fminf(mn, v[NV - 1]);
    mx = fmaxf(mx, v[NV - 1]);
    if (pad_lane) {
      mn = INFINITY;
      mx = -INFINITY;
    }
    wave_minmax(mn, mx);
    if (lane == 0) {
      red_lds[2 * w] = __float_as_uint(mn);
      red_lds[2 * w + 1] = __float_as_uint(mx);
    }
    lds_barrier();
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
      mn = fminf(mn, __uint_as_float(red_lds[2 * q]));
      mx = fmaxf(mx, __uint_as_float(red_lds[2 * q + 1]));
    }

    const float range = mx - mn;
    const bool degenerate = !(range > 0.0f);
    const float inv = degenerate ? 0.0f : 15.0f / range;
    const float cq = -mn * inv;
    const float shift = sig > 0 ? xc : -xc;

    // (6) quantize, pack, store: per a' a lane has 2 NT consecutive codes
    uint8_t* crow = a.codes + row * static_cast<int64_t>(n / 2);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x4_t q4;
#pragma unroll
      for (int tq = 0; tq < NT / 4; ++tq) {
        uint32_t ev = 0u, od = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int t = 4 * tq + k;
          ev = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(v[t * 4 + 2 * u], inv, cq), k, ev);
          od = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(v[t * 4 + 2 * u + 1], inv, cq), k, od);
        }
        q4[tq] = ev | (od << 4);
      }
      if (ap0 + u < KA)
        *reinterpret_cast<u32x4_t*>(crow + (ap0 + u) * NPAIR + NT * outm) = q4;
    }
    if (tid == 0) {
      const float s = degenerate ? 1.0f : range * a.inv_15sqrt_n;
      a.scale[row] = s;
      a.zero[row] = -((mn + shift) * a.inv_sqrt_n) / s;
    }
    if (YOUT) {
      float* yrow = a.yout + row * static_cast<int64_t>(n);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if (ap0 + u >= KA) continue;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int c0 = 0; c0 < 2; ++c0)
            yrow[(ap0 + u) * (1 << KB) + 2 * (NT * outm + t) + c0] =
                (v[t * 4 + 2 * u + c0] + shift) * a.inv_sqrt_n;
      }
    }
  }
  wait_vmcnt<0>();
}

template <int KA, int LOGNT, bool YOUT>
__global__ __launch_bounds__(kThreads) void rq_mfma_kernel(RqArgs a) {
  constexpr int NT = 1 << LOGNT;
  constexpr int PITCH = 64 * NT + 4;
  constexpr int NMAX = KA << (LOGNT + 5);
  __shared__ __attribute__((aligned(16))) uint8_t lds[KA * PITCH];
  __shared__ uint32_t dbits[NMAX / 32];
  __shared__ uint32_t red_lds[2 * kWaves];
  __shared__ float xc_lds[1];
  __shared__ int scratch[4];
  __shared__ uint32_t h28_lds[28];
  if (threadIdx.x < 28) h28_lds[threadIdx.x] = a.h28mask[threadIdx.x];
  build_dbits(a.d, a.n, dbits);  // bit j set when d_j = -1
  __syncthreads();
  const DForm form = decode_d_form_fast(a, dbits, h28_lds, scratch);
  if (form.structured) rq_mfma_body<KA, LOGNT, false, YOUT>(a, lds, dbits, h28_lds, form, red_lds, xc_lds);
  else rq_mfma_body<KA, LOGNT, true, YOUT>(a, lds, dbits, h28_lds, form, red_lds, xc_lds);
}

}  // namespace

bool rq_mfma_supports(int n, int k, bool m28) { return m28 && k == 9 && n == 14336; }

hipError_t launch_rq_mfma(const RqArgs& a, hipStream_t s) {
  int per_cu = 4;
  int64_t grid = static_cast<int64_t>(device_cu_count()) * per_cu;
  if (grid > a.tokens) grid = a.tokens;
  if (a.yout)
    hipLaunchKernelGGL((rq_mfma_kernel<28, 4, true>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((rq_mfma_kernel<28, 4, false>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

const char* rq_mfma_name() { return "rq_mfma28_w4"; }

}  // namespace signrot
