// Fused rotate + sign flip + per-token asymmetric INT4 for gfx950: the fast
// kernels for n = 28 * 2^k, k = 7..9 (3584, 7168, 14336 -- the LLaMA3-8B
// down-projection input; seven waves per token row) and n = 2^12, 2^13, 2^14
// (eight waves).  n = 28 * 2^10 (28672, the LLaMA3-70B one) runs as two halves
// of the n = 14336 transform (rq_halves.hip).
//
// Index split.  A row x[i], i = a * 2^KB + b (a < KA, b < 2^KB), is read as
// quads: b = 4 q + bb (q < NQ = 2^(KB-2), bb < 4).  The transform
// H = H_KA (x) H_{2^KB} (KA = 28: Paley's order-28 matrix; KA = 32: the
// Sylvester matrix, so H is the Sylvester matrix of order n)
// -- explainer
// "SignRot for 4-bit LLM quantization", paragraphs on rotation and on the
// down-projection: a Hadamard matrix applied as a fast Walsh-Hadamard
// transform -- is evaluated as
//   stage 1 (MFMA): the KA-point mix over a together with the 4-point
//     transform over bb, as v_mfma_f32_16x16x32_bf16 on the raw bf16 input.
//     Rows m = (a' & 3, c) with c the output bb; k = (a, bb) in KA / 8
//     chunks of eight a-rows (the fourth of four half empty for KA = 28);
//     columns = 16 quads.  The weights are +-1, so every product
//     is exact and only the fp32 sums round.  Wave w owns a' = 4 w .. 4 w + 3,
//     which splits the output rows over KA / 4 waves with no padding.
//   stage 2 (VALU): the NQ-point transform over q: butterfly stages across
//     the NT = NQ / 16 register tiles (quad bits below log2 NT) and four DPP
//     stages across the 16 lanes of a row (the four quad bits above).
//   stage 3: per-token min / max, scale and zero-point, rounding by
//     v_cvt_pk_u8_f32 (round half to even), nibble packing, one code store
//     per lane: after stage 2 lane (g, nl) of wave w holds the 4 NT
//     consecutive channels (4 w + g) * 2^KB + 4 NT * lane_perm(nl) + (0 .. 4 NT - 1).
//
// Sign vector.  For d = sigma * (row c of H) (explainer, paragraph on the sign
// adjustment) the flip is folded in for free: sigma * H_KA[c_a][a'] into the
// weights, the order-2^KB part as the input permutation b -> b ^ c_b (its low
// two bits in the weights, the quad part in the LDS read addresses), and the
// outlier x_c is zeroed while staging and added back as the constant
// sigma * x_c.  Any other d is applied as a sign-bit XOR after stage 2.
//
// Data movement.  Each row goes HBM -> VGPRs (16-byte loads issued one row
// ahead) -> LDS (double buffered) -> MFMA operands (16-byte LDS reads).  An
// LDS slot of 16 bytes holds quad q of the a-row pair (2p, 2p+1); inside a
// pair-row the slot of quad q is 16 u + (v ^ u * 8 / NT) with u = q % NT,
// v = q / NT, and adjacent lanes stage the two rows of a pair, so both the
// staging writes and the operand reads are free of bank conflicts.  One LDS
// barrier per row: it publishes the next row's buffer and the per-wave
// min / max.
#include <math.h>

#include <atomic>
#include <type_traits>

#include "rq_fast_common.h"


namespace signrot {
namespace {

// min(x, y, z) and max(x, y, z) as single v_min3 / v_max3 ops
__device__ __forceinline__ float min3_of(float x, float y, float z) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}
__device__ __forceinline__ float max3_of(float x, float y, float z) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}

// MAYBE_GENERAL: d arrived as a vector and may lack the calibrated form; the
// body then takes `general` (a wave-uniform flag) at run time, so that both
// cases share one register allocation.  Without it d is given as (c, sigma).
// get_form() yields the form of d; every thread calls it once, after the
// first row's loads have been issued.
template <int KA, int KB, bool MAYBE_GENERAL, bool YOUT, bool ZINT = false, bool SWIGLU = false, class GetForm>
__device__ void rq_fast_body(const RqArgs& a, uint8_t* lds, const uint32_t* dbits, const uint32_t* h28,
                             GetForm get_form, float* red, float* xcl) {
  using S = FastShape<KA, KB>;
  constexpr int NT = S::NT;
  constexpr int NV = S::NV;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int nl = lane & 15;

  // Staging: chunk unit s = w + W i (i < CPT) of 64 chunks; lane L takes the
  // a-row of parity L & 1 and chunk index e = L >> 1 inside the unit.  With
  // CR >= 32 chunks per a-row a pair-row spans CR / 32 units; otherwise a
  // unit spans 32 / CR pair-rows.  Byte offsets split into a wave-uniform
  // part (per i) and a lane part.
  const uint32_t ul = static_cast<uint32_t>(lane);
  const uint32_t ue = ul >> 1;
  uint32_t gl;
  uint32_t wl[2];
  if constexpr (S::CR >= 32) {
    gl = 16u * S::CR * (ul & 1u) + 16u * ue;
#pragma unroll
    for (int h = 0; h < 2; ++h) wl[h] = 16u * quad_slot<KA, KB>(2u * ue + h) + 8u * (ul & 1u);
  } else {
    gl = 32u * S::CR * (ue / S::CR) + 16u * S::CR * (ul & 1u) + 16u * (ue % S::CR);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      wl[h] = (ue / S::CR) * S::PB + 16u * quad_slot<KA, KB>(2u * (ue % S::CR) + h) + 8u * (ul & 1u);
  }
  auto unit_g = [&](int i) -> uint32_t {
    const uint32_t s = static_cast<uint32_t>(w + S::kWaves * i);
    if constexpr (S::CR >= 32) {
      constexpr uint32_t per = S::CR / 32;
      return 32u * S::CR * (s / per) + 512u * (s % per);
    } else {
      return 1024u * s;
    }
  };
  auto unit_l = [&](int i) -> uint32_t {
    const uint32_t s = static_cast<uint32_t>(w + S::kWaves * i);
    if constexpr (S::CR >= 32) {
      constexpr uint32_t per = S::CR / 32;
      return S::PB * (s / per) + 128u * (s % per);
    } else {
      return S::PB * s * (32u / S::CR);
    }
  };
  u32x4_t st[S::CPT];
  u32x4_t stu[SWIGLU ? S::CPT : 1];  // SwiGLU: the up chunks beside the gate chunks in st
  // Row loads through a buffer resource on the row (scalar base, the
  // wave-uniform unit offset as the scalar offset, the lane offset gl), so no
  // per-lane 64-bit address is kept across the loop.
  // (bytes < 2 n: a row past the batch, read as zeros without a memory access)
  auto load_row = [&](int64_t r, uint32_t bytes = 2u * S::N) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.x + r * a.ld, bytes);
#pragma unroll
    for (int i = 0; i < S::CPT; ++i)
      st[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, gl, unit_g(i), kNontemporal));
    if constexpr (SWIGLU) {
      const __amdgpu_buffer_rsrc_t ru = buffer_rsrc(a.x2 + r * a.ld, bytes);
#pragma unroll
      for (int i = 0; i < S::CPT; ++i)
        stu[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ru, gl, unit_g(i), kNontemporal));
    }
  };
  // The first row's loads go out before the sign vector's form is known and
  // before the weights are built, so their latency overlaps the set-up
  // (reading and decoding d included: a workgroup barrier does not wait for
  // global loads); that matters most for a few tokens per call.  The launch
  // has at most one work-group per row.  When d is decoded here, the loads are
  // issued on every path, so that the compiler's memory-counter wait for d's
  // earlier loads can count them as outstanding.
  if constexpr (MAYBE_GENERAL)
    load_row(blockIdx.x, static_cast<int64_t>(blockIdx.x) < a.tokens ? 2u * S::N : 0u);
  else if (static_cast<int64_t>(blockIdx.x) < a.tokens)
    load_row(blockIdx.x);

  const DForm form = get_form();
  const bool general = MAYBE_GENERAL && __builtin_amdgcn_readfirstlane(form.structured) == 0;
  const int c = general ? 0 : __builtin_amdgcn_readfirstlane(form.c);
  const int ca = c >> KB;
  const int cb = c & ((1 << KB) - 1);
  const int cbb = cb & 3;
  const int cbq_lo = (cb >> 2) & (NT - 1);
  const int cbq_hi = cb >> (2 + S::LG);
  const int sig = (!general && __builtin_amdgcn_readfirstlane(form.neg)) ? -1 : 1;

  // MFMA weights, A operand: lane (g, nl) holds A[m = nl][k = 8 g + i] with
  // m -> (a' = 4 w + (nl >> 2), c = nl & 3), k -> (a = 8 kc + 2 g + (i >> 2), bb = i & 3).
  bf16x8_t wA[S::NKC];
  {
    const int ap = 4 * w + (nl >> 2);
    const int cc = nl & 3;
    const int hrow = hka_sign<KA>(h28, ca, ap) * sig;
#pragma unroll
    for (int kc = 0; kc < S::NKC; ++kc)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ar = 8 * kc + 2 * g + (i >> 2);
        const int bb = i & 3;
        int wv = 0;
        if (ar < KA) {
          wv = hrow * hka_sign<KA>(h28, ar, ap);
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
  // NT (nl ^ kXLane) + t, i.e. stored quad q = NT (nl ^ kXLane ^ cbq_hi) + (t ^ cbq_lo).
  // Its slot offset 256 u + 16 (v ^ u SWZ) (u = q % NT, v = q / NT) equals
  // (16 v) ^ (KMUL u), so the address of tile t is rbase ^ (KMUL t).
  const uint32_t rbase = static_cast<uint32_t>(S::PB) * static_cast<uint32_t>(g) +
                         ((16u * static_cast<uint32_t>(nl ^ kXLane ^ cbq_hi)) ^ (S::KMUL * static_cast<uint32_t>(cbq_lo)));

  // The thread and chunk that hold x_c (structured d only).
  int xc_wave = -1, xc_lane = 0, xc_i = 0, xc_e = 0;
  if (!general) {
    const int chunk = c >> 3;
    const int arow = chunk / S::CR, j = chunk % S::CR;
    const int p = arow >> 1;
    int s, e;
    if constexpr (S::CR >= 32) {
      s = p * (S::CR / 32) + (j >> 5);
      e = j & 31;
    } else {
      s = p / (32 / S::CR);
      e = (p % (32 / S::CR)) * S::CR + j;
    }
    xc_i = s / S::kWaves;
    xc_wave = s % S::kWaves;
    xc_lane = 2 * e + (arow & 1);
    xc_e = c & 7;
  }
  const bool xc_thread = !general && w == xc_wave && lane == xc_lane;

  const int ap = 4 * w + g;                      // this lane's output row a'
  const int outm = lane_perm(nl);
  const int chan0 = (ap << KB) + 4 * NT * outm;  // first of this lane's channels
  const uint32_t dword = general ? (dbits[chan0 >> 5] >> (chan0 & 31)) : 0u;

  // Row indices fit in 32 bits: the launcher splits larger calls.
  const int tokens = static_cast<int>(a.tokens);
  const int grid = static_cast<int>(gridDim.x);

  // LDS byte offsets kept for the whole loop, so that the buffer and the K
  // chunk enter the LDS instructions as immediate offsets: the operand read
  // of tile t at taddr[t], the staging write of chunk unit i, half h at
  // waddr[i][h] (both in buffer 0).
  uint32_t taddr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) taddr[t] = rbase ^ (S::KMUL * static_cast<uint32_t>(t));
  uint32_t waddr[S::CPT][2];
#pragma unroll
  for (int i = 0; i < S::CPT; ++i) {
    waddr[i][0] = unit_l(i) + wl[0];
    waddr[i][1] = unit_l(i) + wl[1];
  }

  // Stage the row held in st into buffer BO (0 or kRowBytes).
  auto write_row = [&](auto boc) {
    constexpr uint32_t BO = decltype(boc)::value;
    constexpr int XSLOT = BO ? 1 : 0;
    if constexpr (SWIGLU) {
#pragma unroll
      for (int i = 0; i < S::CPT; ++i) st[i] = swiglu_chunk(st[i], stu[i]);
    }
    if (xc_thread) {
#pragma unroll
      for (int i = 0; i < S::CPT; ++i) {
        if (i != xc_i) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (q != (xc_e >> 1)) continue;
          const uint32_t word = st[i][q];
          const int hi = xc_e & 1;
          xcl[XSLOT] = __uint_as_float(hi ? (word & 0xffff0000u) : (word << 16));
          st[i][q] = hi ? (word & 0x0000ffffu) : (word & 0xffff0000u);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < S::CPT; ++i) {
      *reinterpret_cast<uint2*>(lds + waddr[i][0] + BO) = make_uint2(st[i][0], st[i][1]);
      *reinterpret_cast<uint2*>(lds + waddr[i][1] + BO) = make_uint2(st[i][2], st[i][3]);
    }
  };
  using Buf0 = std::integral_constant<uint32_t, 0u>;
  using Buf1 = std::integral_constant<uint32_t, static_cast<uint32_t>(S::kRowBytes)>;

  // Rows by grid stride: cur (in the LDS buffer), nxt (loads in flight),
  // nn (loaded while cur is processed).
  int cur = blockIdx.x;
  int nxt = cur + grid;
  int nn = nxt + grid;
  if (cur >= tokens) return;
  wait_vmcnt<0>();
  write_row(Buf0{});
  if (nxt < tokens) load_row(nxt);
  lds_barrier();
  bool first = true;

  // One row from buffer PAR (a compile-time constant: the loop below runs the
  // two buffers in turn).
  auto row_step = [&](auto parc) {
    constexpr int PAR = decltype(parc)::value;
    constexpr uint32_t BO = PAR ? static_cast<uint32_t>(S::kRowBytes) : 0u;
    const int row = cur;
    const uint64_t urow = static_cast<uint32_t>(row);  // (64-bit offsets from a uniform row)

    // (1) MFMA stage from this row's buffer
    float v[NV];
    // Operands of tile t + 1 are read while tile t's MFMAs run (pinned by the
    // scheduling groups below), so the LDS latency overlaps the MFMAs.  The
    // SwiGLU instances other than the order-28 one without y_out read tile by
    // tile instead: they have no registers to spare.
    constexpr bool kPipe = !SWIGLU || (KA == 28 && !YOUT);
    u32x4_t bq[2][S::NKC];
#pragma unroll
    for (int kc = 0; kc < S::NKC; ++kc)
      bq[0][kc] = *reinterpret_cast<const u32x4_t*>(lds + taddr[0] + BO + 4 * S::PB * kc);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int cb_ = kPipe ? (t & 1) : 0;
      if (t + 1 < NT && kPipe) {
#pragma unroll
        for (int kc = 0; kc < S::NKC; ++kc)
          bq[cb_ ^ 1][kc] = *reinterpret_cast<const u32x4_t*>(lds + taddr[t + 1] + BO + 4 * S::PB * kc);
      } else if (t > 0 && !kPipe) {
#pragma unroll
        for (int kc = 0; kc < S::NKC; ++kc)
          bq[0][kc] = *reinterpret_cast<const u32x4_t*>(lds + taddr[t] + BO + 4 * S::PB * kc);
      }
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kc = 0; kc < S::NKC; ++kc)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wA[kc], __builtin_bit_cast(bf16x8_t, bq[cb_][kc]), acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * t + r] = acc[r];
    }
    if constexpr (kPipe) {
      // tile 0's reads, then (tile t + 1's reads, tile t's MFMAs), then the
      // last tile's MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, S::NKC, 0);
#pragma unroll
      for (int t = 0; t + 1 < NT; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x100, S::NKC, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, S::NKC, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, S::NKC, 0);
    }

    // (2) stage the next row into the other buffer; start loading the one after
    if (nxt < tokens) {
      // The loads were issued a row ago; after them every wave issued the
      // previous row's code store (plus NT y stores with y_out); wave 0 also
      // scale and zero, so the same count only makes it wait longer.
      if (first) wait_vmcnt<0>();
      else if (YOUT) wait_vmcnt<1 + NT>();
      else wait_vmcnt<1>();
      if constexpr (PAR) write_row(Buf0{});
      else write_row(Buf1{});
      if (nn < tokens) load_row(nn);
    }
    first = false;

    // (3) NQ-point transform over the quad index
    reg_stage<NT, 0>(v);
    if constexpr (NT >= 4) reg_stage<NT, 1>(v);
    if constexpr (NT >= 8) reg_stage<NT, 2>(v);
    dpp_stage<NV>(v, gdpp0, 0);
    dpp_stage<NV>(v, gdpp1, 1);
    dpp_stage<NV>(v, gdpp2, 2);
    dpp_stage<NV>(v, gdpp3, 3);
    if (general) {
      // re-derived every row (an opaque copy), so the compiler does not keep
      // NV shifted masks live across the loop
      uint32_t dw = dword;
      asm volatile("" : "+v"(dw));
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        const uint32_t sbit = (dw << (31 - e)) & 0x80000000u;
        v[e] = __uint_as_float(__float_as_uint(v[e]) ^ sbit);
      }
    }

    // (4) min / max over the row: lanes, then waves through LDS
    float mn = min3_of(v[0], v[1], v[2]);
    float mx = max3_of(v[0], v[1], v[2]);
#pragma unroll
    for (int e = 3; e + 1 < NV; e += 2) {
      min3_acc(mn, v[e], v[e + 1]);
      max3_acc(mx, v[e], v[e + 1]);
    }
    if constexpr (NV % 2 == 0) {
      mn = fmin_raw(mn, v[NV - 1]);
      mx = fmax_raw(mx, v[NV - 1]);
    }
    wave_minmax(mn, mx);
    float* rd = red + 32 * PAR;  // per-wave min at rd[w], max at rd[16 + w]
    if (lane == 63) {
      rd[w] = mn;
      rd[16 + w] = mx;
    }
    // x_c of this row, read before the barrier: the previous barrier published
    // it, and its slot is next written (for the row after next) after this one
    const float xc = general ? 0.0f : xcl[PAR];
    lds_barrier();
#pragma unroll
    for (int q = 0; q < S::kWaves; q += 4) {
      const f32x4_t m4 = *reinterpret_cast<const f32x4_t*>(rd + q);
      const f32x4_t x4 = *reinterpret_cast<const f32x4_t*>(rd + 16 + q);
#pragma unroll
      for (int k = 0; k < 4; k += 2) {
        if (q + k + 1 < S::kWaves) {
          min3_acc(mn, m4[k], m4[k + 1]);
          max3_acc(mx, x4[k], x4[k + 1]);
        } else if (q + k < S::kWaves) {
          mn = fmin_raw(mn, m4[k]);
          mx = fmax_raw(mx, x4[k]);
        }
      }
    }

    // (5) quantize, pack, store
    const QuantParams qp = quant_params(mn, mx);
    const float shift = sig > 0 ? xc : -xc;
    // code of value v: rne(v * inv + cq); with the integer zero-point z the
    // code is rne((v + shift) * inv + z), so cq = shift * inv + z
    float cq = qp.cq;
    float zq = 0.0f;
    if constexpr (ZINT) {
      zq = qp.degenerate ? rintf(-((mn + shift) * a.inv_sqrt_n)) : rintf(-(mn + shift) * qp.inv);
      cq = qp.degenerate ? 0.0f : fmaf(shift, qp.inv, zq);
    }
    if (tid == 0) {
      a.scale[row] = qp.degenerate ? 1.0f : qp.range * a.inv_15sqrt_n;
      // zero = -(mn / sqrt(n)) / s with s = range / (15 sqrt(n)) = -(mn + shift) * inv
      a.zero[row] = ZINT ? zq : (qp.degenerate ? -((mn + shift) * a.inv_sqrt_n) : -(mn + shift) * qp.inv);
    }
    uint32_t q[NT / 2];
#pragma unroll
    for (int u = 0; u < NT / 2; ++u) {
      uint32_t ev = 0u, od = 0u;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float fe = fmaf(v[8 * u + 2 * k], qp.inv, cq);
        float fo = fmaf(v[8 * u + 2 * k + 1], qp.inv, cq);
        if constexpr (ZINT) {
          // the rounded zero-point can put the top of the range at 15.5
          fe = fminf(fe, 15.0f);
          fo = fminf(fo, 15.0f);
        }
        ev = __builtin_amdgcn_cvt_pk_u8_f32(fe, k, ev);
        od = __builtin_amdgcn_cvt_pk_u8_f32(fo, k, od);
      }
      q[u] = ev | (od << 4);
    }
    const __amdgpu_buffer_rsrc_t cs = buffer_rsrc(a.codes + urow * (S::N / 2), S::N / 2);
    const uint32_t coff = static_cast<uint32_t>(chan0 / 2);
    if constexpr (NT == 8) {
      store_b128_held<kNontemporal>(u32x4_t{q[0], q[1], q[2], q[3]}, cs, coff, 0);
    } else if constexpr (NT == 4) {
      __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{q[0], q[1]}, cs, coff, 0, kNontemporal);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(q[0], cs, coff, 0, kNontemporal);
    }
    if (YOUT) {
      float* yp = a.yout + urow * S::N + chan0;
#pragma unroll
      for (int e4 = 0; e4 < NT; ++e4) {
        f32x4_t o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = (v[4 * e4 + k] + shift) * a.inv_sqrt_n;
        store_f32x4_held(yp + 4 * e4, o);
      }
    }

    // (6) advance the row queue
    cur = nxt;
    nxt = nn;
    nn += grid;
  };
  for (;;) {
    row_step(std::integral_constant<int, 0>{});
    if (cur >= tokens) break;
    row_step(std::integral_constant<int, 1>{});
    if (cur >= tokens) break;
  }
  wait_vmcnt<0>();
}

// DVEC: d is a vector (its form is decided here); otherwise (c, sigma) given.
template <int KA, int KB, bool DVEC, bool YOUT, bool ZINT = false, bool SWIGLU = false>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4)))
void rq_fast_kernel(RqArgs a) {
  using S = FastShape<KA, KB>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[S::kLdsBytes];
  __shared__ uint32_t dbits[S::N / 32];
  __shared__ __attribute__((aligned(16))) float red[64];
  __shared__ float xcl[2];
  __shared__ int scratch[4];
  __shared__ __attribute__((aligned(16))) uint32_t h28_lds[28];
  const int tid = threadIdx.x;
  if constexpr (KA == 28) {
    // The H28 row masks are kernel arguments: read with constant offsets they
    // are scalar loads, so no wait on the vector memory counter (which would
    // also wait for the first row's loads) comes before the row is requested.
    if (tid == 0) {
#pragma unroll
      for (int q = 0; q < 7; ++q)
        *reinterpret_cast<u32x4_t*>(h28_lds + 4 * q) =
            u32x4_t{a.h28mask[4 * q], a.h28mask[4 * q + 1], a.h28mask[4 * q + 2], a.h28mask[4 * q + 3]};
    }
    // zero the second buffer's first two pair-rows and the two rows behind it
    // (read with zero weights before any row has been staged there)
    for (int o = 16 * tid; o < 2 * S::PB; o += 16 * S::kThreads) {
      *reinterpret_cast<u32x4_t*>(lds + S::kRowBytes + o) = u32x4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(lds + 2 * S::kRowBytes + o) = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  if constexpr (!DVEC) {
    // d = sigma * (row c of H) by construction: nothing to read or decode;
    // the barrier publishes h28_lds and the zeroed rows
    rq_fast_body<KA, KB, false, YOUT, ZINT, SWIGLU>(
        a, lds, dbits, h28_lds,
        [&] {
          __syncthreads();
          return DForm{1, a.form_c, a.form_neg};
        },
        red, xcl);
  } else {
    // This thread's first 32 entries of d are read before the body issues the
    // first row's loads, so that the decode waits for them alone.
    constexpr int kWords = S::N / 32;
    const int8_t* d32 = a.d + 32 * (tid < kWords ? tid : 0);
    const uint4 dlo = *reinterpret_cast<const uint4*>(d32);
    const uint4 dhi = *reinterpret_cast<const uint4*>(d32 + 16);
    __builtin_amdgcn_sched_barrier(0);  // keep them ahead of the row's loads
    rq_fast_body<KA, KB, true, YOUT, ZINT, SWIGLU>(
        a, lds, dbits, h28_lds,
        [&] {
          // the bitmask of d in LDS, bit j set when d_j = -1
          if (tid < kWords) dbits[tid] = sign_word_of(dlo, dhi);
          if (tid == 0) scratch[3] = 0;  // the form check's flag
          for (int wd = tid + S::kThreads; wd < kWords; wd += S::kThreads) dbits[wd] = sign_word(a.d + 32 * wd);
          __syncthreads();
          return decode_d_form_fast<S::kThreads>(a, dbits, h28_lds, scratch);
        },
        red, xcl);
  }
}

template <int KA, int KB>
hipError_t launch_shape_rows(const RqArgs& a, hipStream_t stream);

// The kernel keeps row indices in 32 bits: calls of more than 2^30 rows run
// as consecutive launches over slices of the batch.
template <int KA, int KB>
hipError_t launch_shape(const RqArgs& a, hipStream_t stream) {
  constexpr int64_t kMaxRows = int64_t{1} << 30;
  if (a.tokens <= kMaxRows) return launch_shape_rows<KA, KB>(a, stream);
  for (int64_t r0 = 0; r0 < a.tokens; r0 += kMaxRows) {
    RqArgs s = a;
    s.tokens = (a.tokens - r0 < kMaxRows) ? a.tokens - r0 : kMaxRows;
    s.x = a.x + r0 * a.ld;
    if (a.x2) s.x2 = a.x2 + r0 * a.ld;
    s.codes = a.codes + r0 * (a.n / 2);
    s.scale = a.scale + r0;
    s.zero = a.zero + r0;
    if (a.yout) s.yout = a.yout + r0 * a.n;
    const hipError_t e = launch_shape_rows<KA, KB>(s, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int KA, int KB>
hipError_t launch_shape_rows(const RqArgs& a, hipStream_t stream) {
  using S = FastShape<KA, KB>;
  // resident workgroups per CU (registers and LDS), asked once per shape
  // (computed by any thread that finds 0; all compute the same value)
  static std::atomic<int> per_cu_cache{0};
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, rq_fast_kernel<KA, KB, true, false>, S::kThreads, 0) !=
            hipSuccess ||
        blocks < 1)
      blocks = 1;
    per_cu = blocks;
    per_cu_cache.store(per_cu, std::memory_order_relaxed);
  }
  // Short launches (fewer than 4 rows per work-group at full occupancy) run
  // at most two work-groups per CU: 8192 x 2048 tokens took 12.7-12.9 us
  // against 13.2-13.9 us with three, 4096 x 2048 8.9 against 9.5 us; from
  // 4096 tokens up three were as fast or faster.
  const int64_t cus = device_cu_count();
  if (per_cu > 2 && a.tokens < 4 * cus * per_cu) per_cu = 2;
  int64_t grid = cus * per_cu;
  if (grid > a.tokens) grid = a.tokens;
  const dim3 blocks(static_cast<unsigned>(grid));
  const dim3 threads(static_cast<unsigned>(S::kThreads));
  if (a.x2)  // SwiGLU producer fused in: d given as (c, sigma)
    (a.yout ? rq_fast_kernel<KA, KB, false, true, false, true> : rq_fast_kernel<KA, KB, false, false, false, true>)
        <<<blocks, threads, 0, stream>>>(a);
  else if (a.zint)  // only with d given as (c, sigma), and no y_out
    rq_fast_kernel<KA, KB, false, false, true><<<blocks, threads, 0, stream>>>(a);
  else if (a.form_given)
    (a.yout ? rq_fast_kernel<KA, KB, false, true> : rq_fast_kernel<KA, KB, false, false>)<<<blocks, threads, 0, stream>>>(a);
  else
    (a.yout ? rq_fast_kernel<KA, KB, true, true> : rq_fast_kernel<KA, KB, true, false>)<<<blocks, threads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

bool rq_fast_supports(int n, int k, bool m28) {
  if (m28) return k >= 7 && k <= 10 && n == (28 << k);  // 3584, 7168, 14336, 28672
  return n == 4096 || n == 8192 || n == 16384;
}

hipError_t launch_rq_fast(const RqArgs& a, hipStream_t s) {
  if (a.m28) {
    switch (a.k) {
      case 7: return launch_shape<28, 7>(a, s);
      case 8: return launch_shape<28, 8>(a, s);
      case 9: return launch_shape<28, 9>(a, s);
      default: return launch_rq_halves(a, s);  // 28 * 2^10 as two halves of 28 * 2^9
    }
  }
  if (a.n == 4096) return launch_shape<32, 7>(a, s);
  if (a.n == 8192) return launch_shape<32, 8>(a, s);
  return launch_shape<32, 9>(a, s);
}

const char* rq_fast_name(int n) {
  if (n == 28672) return "rq_mfma28x2_w7";
  if (n % 28 == 0) return "rq_mfma28_w7";
  return "rq_mfma32_w8";
}

}  // namespace signrot
