// Fused rotate + sign flip + per-token asymmetric INT4 for n = 28 * 2^9
// (14336, the LLaMA3-8B down-projection input), seven waves per token row.
//
// Index split.  A row x[i], i = a * 512 + b (a < 28, b < 512), is read as
// quads: b = 4 q + bb (q < 128, bb < 4).  The transform H = H28 (x) H512
// (explainer "SignRot for 4-bit LLM quantization", paragraphs on rotation and
// on the down-projection: a Hadamard matrix applied as a fast Walsh-Hadamard
// transform) is evaluated as
//   stage 1 (MFMA): the 28-point mix over a together with the 4-point
//     transform over bb, as v_mfma_f32_16x16x32_bf16 on the raw bf16 input.
//     Rows m = (a' & 3, c) with c the output bb; k = (a, bb) in 4 chunks of
//     eight a-rows; columns = 16 quads.  The weights are +-1, so every product
//     is exact and only the fp32 sums round.  Wave w owns a' = 4 w .. 4 w + 3,
//     which splits the 28 output rows over 7 waves with no padding.
//   stage 2 (VALU): the 128-point transform over q: three butterfly stages
//     across the 8 register tiles (quad bits 0..2) and four DPP stages across
//     the 16 lanes of a row (quad bits 3..6).
//   stage 3: per-token min / max, scale and zero-point, rounding by
//     v_cvt_pk_u8_f32 (round half to even), nibble packing, one 16-byte code
//     store per lane: after stage 2 lane (g, nl) of wave w holds the 32
//     consecutive channels (4 w + g) * 512 + 32 * lane_perm(nl) + 0..31.
//
// Sign vector.  For d = sigma * (row c of H) (explainer, paragraph on the sign
// adjustment) the flip is folded in for free: sigma * H28[c_a][a'] into the
// weights, the Sylvester part as the input permutation b -> b ^ c_b (its low
// two bits in the weights, the quad part in the LDS read addresses), and the
// outlier x_c is zeroed while staging and added back as the constant
// sigma * x_c.  Any other d is applied as a sign-bit XOR after stage 2.
//
// Data movement.  Each row goes HBM -> VGPRs (16-byte loads issued one row
// ahead) -> LDS (double buffered) -> MFMA operands (16-byte LDS reads).  An
// LDS slot of 16 bytes holds quad q of the a-row pair (2p, 2p+1); inside a
// pair-row the slot of quad q is 16 (q & 7) + ((q >> 3) ^ (q & 7)), so both
// the staging writes and the operand reads are free of bank conflicts.  One
// LDS barrier per row: it publishes the next row's buffer and the per-wave
// min / max.
#include <math.h>

#include "device_common.h"
#include "wave_ops.h"

namespace signrot {
namespace {

using namespace wave;

constexpr int kW7Waves = 7;
constexpr int kW7Threads = 64 * kW7Waves;
constexpr int kPairBytes = 2048;                 // 128 slots of 16 B
constexpr int kRowBytes = 14 * kPairBytes;       // one token row, a-pairs 0..13
// Two row buffers plus two zero pair-rows behind the second: the fourth K
// chunk reads "pairs" 14 and 15 for lanes whose weights are zero, which land
// on finite data (the other buffer or the zero rows).
constexpr int kLdsBytes = 2 * kRowBytes + 2 * kPairBytes;
constexpr int kChunksPerThread = 4;              // 1792 chunks of 16 B per row

// Slot (16-byte unit) of quad q inside a pair-row.
__device__ __forceinline__ uint32_t quad_slot(uint32_t q) { return 16u * (q & 7u) + ((q >> 3) ^ (q & 7u)); }

template <bool GENERAL, bool YOUT>
__device__ void rq_w7_body(const RqArgs& a, uint8_t* lds, const uint32_t* dbits, const uint32_t* h28,
                           const DForm& form, float* red, float* xcl) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int nl = lane & 15;

  const int c = GENERAL ? 0 : __builtin_amdgcn_readfirstlane(form.c);
  const int ca = c >> 9;
  const int cb = c & 511;
  const int cbb = cb & 3;
  const int cbq_lo = (cb >> 2) & 7;
  const int cbq_hi = cb >> 5;
  const int sig = (!GENERAL && form.neg) ? -1 : 1;

  // MFMA weights, A operand: lane (g, nl) holds A[m = nl][k = 8 g + i] with
  // m -> (a' = 4 w + (nl >> 2), c = nl & 3), k -> (a = 8 kc + 2 g + (i >> 2), bb = i & 3).
  bf16x8_t wA[4];
  {
    const int ap = 4 * w + (nl >> 2);
    const int cc = nl & 3;
    const int hrow = hka_sign<28>(h28, ca, ap) * sig;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ar = 8 * kc + 2 * g + (i >> 2);
        const int bb = i & 3;
        int wv = 0;
        if (ar < 28) {
          wv = hrow * hka_sign<28>(h28, ar, ap);
          if (__popc(static_cast<uint32_t>((bb ^ cbb) & cc)) & 1) wv = -wv;
        }
        wA[kc][i] = static_cast<short>(bf16_of_sign(wv));
      }
  }

  const float gdpp0 = (((nl >> 0) ^ (nl >> 2)) & 1) ? -1.0f : 1.0f;
  const float gdpp1 = (((nl >> 1) ^ (nl >> 2)) & 1) ? -1.0f : 1.0f;
  const float gdpp2 = ((nl >> 2) & 1) ? -1.0f : 1.0f;
  const float gdpp3 = ((nl >> 3) & 1) ? -1.0f : 1.0f;

  // Operand reads: lane (g, nl) of tile t reads pair 4 kc + g, logical quad
  // 8 (nl ^ kXLane) + t, i.e. stored quad q = 8 (nl ^ kXLane ^ cbq_hi) + (t ^ cbq_lo).
  // Its slot offset 256 u + 16 (v ^ u) (u = q & 7, v = q >> 3) equals
  // (16 v) ^ (272 u), so the address of tile t is rbase ^ (272 t).
  const uint32_t rbase = 2048u * static_cast<uint32_t>(g) +
                         ((16u * static_cast<uint32_t>(nl ^ kXLane ^ cbq_hi)) ^ (272u * static_cast<uint32_t>(cbq_lo)));

  // Staging: chunk unit s = w + 7 i (i < 4) covers pair p = s >> 1, half jh = s & 1;
  // lane L takes a-row 2 p + (L & 1), 16-byte chunk j = 32 jh + (L >> 1)
  // (quads 2 j and 2 j + 1).  Byte offsets split into a wave-uniform part
  // (per i) and a lane part: global 16 (64 arow + j) = 2048 p + 512 jh + gl,
  // LDS (slot of quad 2 j + h) = 2048 p + 128 jh + wl[h].
  const uint32_t ul = static_cast<uint32_t>(lane);
  const uint32_t gl = 16u * (64u * (ul & 1u) + (ul >> 1));
  uint32_t wl[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t q = 2u * (ul >> 1) + h;  // quad with jh = 0; jh adds 64 to q, i.e. 8 to q >> 3
    wl[h] = 16u * quad_slot(q) + 8u * (ul & 1u);
  }
  auto unit_g = [&](int i) -> uint32_t {
    const uint32_t s = static_cast<uint32_t>(w + kW7Waves * i);
    return 2048u * (s >> 1) + 512u * (s & 1u);
  };
  auto unit_l = [&](int i) -> uint32_t {
    const uint32_t s = static_cast<uint32_t>(w + kW7Waves * i);
    return 2048u * (s >> 1) + 128u * (s & 1u);
  };
  // The thread and chunk that hold x_c (structured d only).
  int xc_wave = -1, xc_lane = 0, xc_i = 0, xc_e = 0;
  if (!GENERAL) {
    const int chunk = c >> 3;
    const int arow = chunk >> 6, j = chunk & 63;
    const int s = 2 * (arow >> 1) + (j >> 5);
    xc_i = s / kW7Waves;
    xc_wave = s % kW7Waves;
    xc_lane = 2 * (j & 31) + (arow & 1);
    xc_e = c & 7;
  }
  const bool xc_thread = !GENERAL && w == xc_wave && lane == xc_lane;

  const int ap = 4 * w + g;                      // this lane's output row a'
  const int outm = lane_perm(nl);
  const uint32_t dword = GENERAL ? dbits[ap * 16 + outm] : 0u;

  const int64_t tokens = a.tokens;
  const int64_t grid = gridDim.x;
  const int n = a.n;

  u32x4_t st[kChunksPerThread];
  auto load_row = [&](int64_t r) {
    const uint8_t* rowp = reinterpret_cast<const uint8_t*>(a.x + r * a.ld);
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i)
      st[i] = *reinterpret_cast<const u32x4_t*>(rowp + unit_g(i) + gl);
  };
  auto write_row = [&](uint32_t bo, int xslot) {
    if (xc_thread) {
#pragma unroll
      for (int i = 0; i < kChunksPerThread; ++i) {
        if (i != xc_i) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q != (xc_e >> 1)) continue;
          const uint32_t word = st[i][q];
          const int hi = xc_e & 1;
          xcl[xslot] = __uint_as_float(hi ? (word & 0xffff0000u) : (word << 16));
          st[i][q] = hi ? (word & 0x0000ffffu) : (word & 0xffff0000u);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      uint8_t* base = lds + (bo + unit_l(i));
      *reinterpret_cast<uint2*>(base + wl[0]) = make_uint2(st[i][0], st[i][1]);
      *reinterpret_cast<uint2*>(base + wl[1]) = make_uint2(st[i][2], st[i][3]);
    }
  };

  // Rows by grid stride: cur (in the LDS buffer), nxt (loads in flight),
  // nn (loaded while cur is processed).
  int64_t cur = blockIdx.x;
  int64_t nxt = cur + grid;
  int64_t nn = nxt + grid;
  if (cur >= tokens) return;
  load_row(cur);
  wait_vmcnt<0>();
  write_row(0u, 0);
  if (nxt < tokens) load_row(nxt);
  lds_barrier();

  for (int it = 0; cur < tokens; ++it) {
    const int64_t row = cur;
    const int par = it & 1;
    const uint32_t bo = par ? static_cast<uint32_t>(kRowBytes) : 0u;

    // (1) MFMA stage from this row's buffer
    float v[32];
    {
      const uint32_t base = rbase + bo;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint8_t* tp = lds + (base ^ (272u * t));
        u32x4_t b[4];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) b[kc] = *reinterpret_cast<const u32x4_t*>(tp + 4 * kPairBytes * kc);
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wA[kc], __builtin_bit_cast(bf16x8_t, b[kc]), acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) v[4 * t + r] = acc[r];
      }
    }

    // (2) stage the next row into the other buffer; start loading the one after
    if (nxt < tokens) {
      // The loads were issued a row ago; after them every wave issued the
      // previous row's code store (plus eight y stores with y_out); wave 0
      // also scale and zero, so the same count only makes it wait longer.
      if (it == 0) wait_vmcnt<0>();
      else if (YOUT) wait_vmcnt<9>();
      else wait_vmcnt<1>();
      write_row(bo ^ static_cast<uint32_t>(kRowBytes), par ^ 1);
      if (nn < tokens) load_row(nn);
    }

    // (3) 128-point transform over the quad index
    reg_stage<8, 0>(v);
    reg_stage<8, 1>(v);
    reg_stage<8, 2>(v);
    dpp_stage<32>(v, gdpp0, 0);
    dpp_stage<32>(v, gdpp1, 1);
    dpp_stage<32>(v, gdpp2, 2);
    dpp_stage<32>(v, gdpp3, 3);
    if (GENERAL) {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const uint32_t sbit = (dword << (31 - e)) & 0x80000000u;
        v[e] = __uint_as_float(__float_as_uint(v[e]) ^ sbit);
      }
    }

    // (4) min / max over the row: lanes, then waves through LDS
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int e = 1; e + 1 < 32; e += 2) {
      min3_acc(mn, v[e], v[e + 1]);
      max3_acc(mx, v[e], v[e + 1]);
    }
    mn = fmin_raw(mn, v[31]);
    mx = fmax_raw(mx, v[31]);
    wave_minmax(mn, mx);
    float* rd = red + 16 * par;
    if (lane == 0) {
      rd[w] = mn;
      rd[8 + w] = mx;
    }
    lds_barrier();
    {
      const f32x4_t m0 = *reinterpret_cast<const f32x4_t*>(rd);
      const f32x4_t m1 = *reinterpret_cast<const f32x4_t*>(rd + 4);
      const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(rd + 8);
      const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(rd + 12);
      mn = m0[0];
      min3_acc(mn, m0[1], m0[2]);
      min3_acc(mn, m0[3], m1[0]);
      min3_acc(mn, m1[1], m1[2]);
      mx = x0[0];
      max3_acc(mx, x0[1], x0[2]);
      max3_acc(mx, x0[3], x1[0]);
      max3_acc(mx, x1[1], x1[2]);
    }

    // (5) quantize, pack, store
    const QuantParams qp = quant_params(mn, mx);
    const float range = qp.range;
    const bool degenerate = qp.degenerate;
    const float inv = qp.inv;
    const float cq = qp.cq;
    const float shift = GENERAL ? 0.0f : (sig > 0 ? xcl[par] : -xcl[par]);
    if (tid == 0) {
      const float s = degenerate ? 1.0f : range * a.inv_15sqrt_n;
      a.scale[row] = s;
      // zero = -(mn / sqrt(n)) / s with s = range / (15 sqrt(n)) = -(mn + shift) * inv
      a.zero[row] = degenerate ? -((mn + shift) * a.inv_sqrt_n) : -(mn + shift) * inv;
    }
    u32x4_t q4;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t ev = 0u, od = 0u;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ev = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(v[8 * u + 2 * k], inv, cq), k, ev);
        od = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(v[8 * u + 2 * k + 1], inv, cq), k, od);
      }
      q4[u] = ev | (od << 4);
    }
    const int64_t chan0 = static_cast<int64_t>(ap) * 512 + 32 * outm;
    *reinterpret_cast<u32x4_t*>(a.codes + row * static_cast<int64_t>(n / 2) + chan0 / 2) = q4;
    if (YOUT) {
      float* yp = a.yout + row * static_cast<int64_t>(n) + chan0;
#pragma unroll
      for (int e4 = 0; e4 < 8; ++e4) {
        f32x4_t o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = (v[4 * e4 + k] + shift) * a.inv_sqrt_n;
        *reinterpret_cast<f32x4_t*>(yp + 4 * e4) = o;
      }
    }

    // (6) advance the row queue
    cur = nxt;
    nxt = nn;
    nn += grid;
  }
  wait_vmcnt<0>();
}

template <bool YOUT>
__global__ __launch_bounds__(kW7Threads) __attribute__((amdgpu_waves_per_eu(4))) void rq_w7_kernel(RqArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  __shared__ uint32_t dbits[14336 / 32];
  __shared__ __attribute__((aligned(16))) float red[32];
  __shared__ float xcl[2];
  __shared__ int scratch[4];
  __shared__ uint32_t h28_lds[28];
  const int tid = threadIdx.x;
  if (tid < 28) h28_lds[tid] = a.h28mask[tid];
  // zero the second buffer's first two pair-rows and the two rows behind it
  // (read with zero weights before any row has been staged there)
  for (int o = 16 * tid; o < 2 * kPairBytes; o += 16 * kW7Threads) {
    *reinterpret_cast<u32x4_t*>(lds + kRowBytes + o) = u32x4_t{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4_t*>(lds + 2 * kRowBytes + o) = u32x4_t{0u, 0u, 0u, 0u};
  }
  build_dbits(a.d, a.n, dbits);  // bit j set when d_j = -1
  __syncthreads();
  const DForm form = decode_d_form_fast(a, dbits, h28_lds, scratch);
  if (form.structured) rq_w7_body<false, YOUT>(a, lds, dbits, h28_lds, form, red, xcl);
  else rq_w7_body<true, YOUT>(a, lds, dbits, h28_lds, form, red, xcl);
}

}  // namespace

bool rq_w7_supports(int n, int k, bool m28) { return m28 && k == 9 && n == 14336; }

hipError_t launch_rq_w7(const RqArgs& a, hipStream_t s) {
  int64_t grid = static_cast<int64_t>(device_cu_count()) * 2;
  if (grid > a.tokens) grid = a.tokens;
  if (a.yout)
    hipLaunchKernelGGL((rq_w7_kernel<true>), dim3(static_cast<unsigned>(grid)), dim3(kW7Threads), 0, s, a);
  else
    hipLaunchKernelGGL((rq_w7_kernel<false>), dim3(static_cast<unsigned>(grid)), dim3(kW7Threads), 0, s, a);
  return hipGetLastError();
}

const char* rq_w7_name() { return "rq_mfma28_w7"; }

}  // namespace signrot
