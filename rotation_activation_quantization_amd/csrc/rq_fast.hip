// Fused rotate + sign flip + per-token asymmetric INT4 for gfx950: the fast
// kernels for n = 28 * 2^k, k = 7..9 (3584, 7168, 14336 -- the LLaMA3-8B
// down-projection input; seven waves per token row), n = 56 * 2^9 (28672, the
// LLaMA3-70B one; fourteen waves) and n = 2^12, 2^13, 2^14 (eight waves).
//
// Index split.  A row x[i], i = a * 2^KB + b (a < KA, b < 2^KB), is read as
// quads: b = 4 q + bb (q < NQ = 2^(KB-2), bb < 4).  The transform
// H = H_KA (x) H_{2^KB} (KA = 28: Paley's order-28 matrix; KA = 56: H28 (x) H2,
// so that H28 (x) H_1024 reads as H56 (x) H_512 with a = 2 a28 + (top bit of
// b); KA = 32: the Sylvester matrix, so H is the Sylvester matrix of order n)
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

#include "device_common.h"
#include "wave_ops.h"

namespace signrot {
namespace {

using namespace wave;

template <int KA, int KB>
struct FastShape {
  static_assert(KA == 28 || KA == 32 || KA == 56, "order-28, order-56 or Sylvester outer factor");
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

template <int KA, int KB, bool GENERAL, bool YOUT, bool ZINT = false>
__device__ void rq_fast_body(const RqArgs& a, uint8_t* lds, const uint32_t* dbits, const uint32_t* h28,
                             const DForm& form, float* red, float* xcl) {
  using S = FastShape<KA, KB>;
  constexpr int NT = S::NT;
  constexpr int NV = S::NV;
  constexpr bool kLateStage = (KA == 56);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int nl = lane & 15;

  const int c = GENERAL ? 0 : __builtin_amdgcn_readfirstlane(form.c);
  const int ca = c >> KB;
  const int cb = c & ((1 << KB) - 1);
  const int cbb = cb & 3;
  const int cbq_lo = (cb >> 2) & (NT - 1);
  const int cbq_hi = cb >> (2 + S::LG);
  const int sig = (!GENERAL && form.neg) ? -1 : 1;

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
  auto load_row = [&](int64_t r) {
    const uint8_t* rowp = reinterpret_cast<const uint8_t*>(a.x + r * a.ld);
#pragma unroll
    for (int i = 0; i < S::CPT; ++i) st[i] = *reinterpret_cast<const u32x4_t*>(rowp + unit_g(i) + gl);
  };
  // The first row's loads go out before the weights are built (all but the
  // 56-row shape, whose registers are short), so their latency overlaps the
  // set-up; that matters most for a few tokens per call.
  constexpr bool kEarlyLoad = (KA != 56);
  if (kEarlyLoad && static_cast<int64_t>(blockIdx.x) < a.tokens) load_row(blockIdx.x);

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
  if (!GENERAL) {
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
  const bool xc_thread = !GENERAL && w == xc_wave && lane == xc_lane;

  const int ap = 4 * w + g;                      // this lane's output row a'
  const int outm = lane_perm(nl);
  const int chan0 = (ap << KB) + 4 * NT * outm;  // first of this lane's channels
  const uint32_t dword = GENERAL ? (dbits[chan0 >> 5] >> (chan0 & 31)) : 0u;

  const int64_t tokens = a.tokens;
  const int64_t grid = gridDim.x;

  auto write_row = [&](uint32_t bo, int xslot) {
    if (xc_thread) {
#pragma unroll
      for (int i = 0; i < S::CPT; ++i) {
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
    for (int i = 0; i < S::CPT; ++i) {
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
  if (!kEarlyLoad) load_row(cur);
  wait_vmcnt<0>();
  write_row(0u, 0);
  if (nxt < tokens) load_row(nxt);
  lds_barrier();

  for (int it = 0; cur < tokens; ++it) {
    const int64_t row = cur;
    const int par = it & 1;
    const uint32_t bo = par ? static_cast<uint32_t>(S::kRowBytes) : 0u;

    // (0) KA = 56 stages the next row here, before the MFMA stage, so that
    // its registers are not live while the operands and the 28 weight
    // registers are (the other shapes do it in (2), a longer lead time).
    if (kLateStage && nxt < tokens) {
      if (it == 0) wait_vmcnt<0>();
      else if (YOUT) wait_vmcnt<1 + NT>();
      else wait_vmcnt<1>();
      write_row(bo ^ static_cast<uint32_t>(S::kRowBytes), par ^ 1);
    }

    // (1) MFMA stage from this row's buffer
    float v[NV];
    {
      const uint32_t base = rbase + bo;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint8_t* tp = lds + (base ^ (S::KMUL * t));
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        // operands in groups of four chunks, or two for the seven chunks of
        // KA = 56 (whose 28 weight registers leave less room)
        constexpr int kGroup = S::NKC > 4 ? 2 : 4;
#pragma unroll
        for (int k0 = 0; k0 < S::NKC; k0 += kGroup) {
          u32x4_t b[kGroup];
#pragma unroll
          for (int kc = 0; kc < kGroup; ++kc)
            if (k0 + kc < S::NKC) b[kc] = *reinterpret_cast<const u32x4_t*>(tp + 4 * S::PB * (k0 + kc));
#pragma unroll
          for (int kc = 0; kc < kGroup; ++kc)
            if (k0 + kc < S::NKC)
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wA[k0 + kc], __builtin_bit_cast(bf16x8_t, b[kc]), acc, 0,
                                                            0, 0);
          if (S::NKC > 4) __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) v[4 * t + r] = acc[r];
      }
    }

    // (2) stage the next row into the other buffer; start loading the one after
    if (kLateStage) {
      if (nn < tokens) load_row(nn);
    } else if (nxt < tokens) {
      // The loads were issued a row ago; after them every wave issued the
      // previous row's code store (plus NT y stores with y_out); wave 0 also
      // scale and zero, so the same count only makes it wait longer.
      if (it == 0) wait_vmcnt<0>();
      else if (YOUT) wait_vmcnt<1 + NT>();
      else wait_vmcnt<1>();
      write_row(bo ^ static_cast<uint32_t>(S::kRowBytes), par ^ 1);
      if (nn < tokens) load_row(nn);
    }

    // (3) NQ-point transform over the quad index
    reg_stage<NT, 0>(v);
    if constexpr (NT >= 4) reg_stage<NT, 1>(v);
    if constexpr (NT >= 8) reg_stage<NT, 2>(v);
    dpp_stage<NV>(v, gdpp0, 0);
    dpp_stage<NV>(v, gdpp1, 1);
    dpp_stage<NV>(v, gdpp2, 2);
    dpp_stage<NV>(v, gdpp3, 3);
    if (GENERAL) {
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        const uint32_t sbit = (dword << (31 - e)) & 0x80000000u;
        v[e] = __uint_as_float(__float_as_uint(v[e]) ^ sbit);
      }
    }

    // (4) min / max over the row: lanes, then waves through LDS
    float mn = v[0], mx = v[0];
#pragma unroll
    for (int e = 1; e + 1 < NV; e += 2) {
      min3_acc(mn, v[e], v[e + 1]);
      max3_acc(mx, v[e], v[e + 1]);
    }
    mn = fmin_raw(mn, v[NV - 1]);
    mx = fmax_raw(mx, v[NV - 1]);
    wave_minmax(mn, mx);
    float* rd = red + 32 * par;  // per-wave min at rd[w], max at rd[16 + w]
    if (lane == 0) {
      rd[w] = mn;
      rd[16 + w] = mx;
    }
    // x_c of this row, read before the barrier: the previous barrier published
    // it, and its slot is next written (for the row after next) after this one
    const float xc = GENERAL ? 0.0f : xcl[par];
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
    uint8_t* cp = a.codes + row * static_cast<int64_t>(S::N / 2) + chan0 / 2;
    if constexpr (NT == 8) {
      *reinterpret_cast<u32x4_t*>(cp) = u32x4_t{q[0], q[1], q[2], q[3]};
    } else if constexpr (NT == 4) {
      *reinterpret_cast<uint2*>(cp) = make_uint2(q[0], q[1]);
    } else {
      *reinterpret_cast<uint32_t*>(cp) = q[0];
    }
    if (YOUT) {
      float* yp = a.yout + row * static_cast<int64_t>(S::N) + chan0;
#pragma unroll
      for (int e4 = 0; e4 < NT; ++e4) {
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

template <int KA, int KB, bool YOUT, bool ZINT = false>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4)))
void rq_fast_kernel(RqArgs a) {
  using S = FastShape<KA, KB>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[S::kLdsBytes];
  __shared__ uint32_t dbits[S::N / 32];
  __shared__ __attribute__((aligned(16))) float red[64];
  __shared__ float xcl[2];
  __shared__ int scratch[4];
  __shared__ uint32_t h28_lds[28];
  const int tid = threadIdx.x;
  if (tid < 28) h28_lds[tid] = a.h28mask[tid];
  if constexpr (KA == 28) {
    // zero the second buffer's first two pair-rows and the two rows behind it
    // (read with zero weights before any row has been staged there)
    for (int o = 16 * tid; o < 2 * S::PB; o += 16 * S::kThreads) {
      *reinterpret_cast<u32x4_t*>(lds + S::kRowBytes + o) = u32x4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4_t*>(lds + 2 * S::kRowBytes + o) = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  DForm form;
  if (a.form_given) {
    // d = sigma * (row c of H) by construction: nothing to read or decode
    __syncthreads();
    form = DForm{1, a.form_c, a.form_neg};
  } else {
    build_dbits(a.d, a.n, dbits);  // bit j set when d_j = -1
    __syncthreads();
    form = decode_d_form_fast(a, dbits, h28_lds, scratch);
  }
  if constexpr (ZINT) {
    // only with d given as (c, sigma): always the structured form
    rq_fast_body<KA, KB, false, YOUT, true>(a, lds, dbits, h28_lds, form, red, xcl);
  } else {
    if (form.structured) rq_fast_body<KA, KB, false, YOUT>(a, lds, dbits, h28_lds, form, red, xcl);
    else rq_fast_body<KA, KB, true, YOUT>(a, lds, dbits, h28_lds, form, red, xcl);
  }
}

template <int KA, int KB>
hipError_t launch_shape(const RqArgs& a, hipStream_t stream) {
  using S = FastShape<KA, KB>;
  // resident workgroups per CU (registers and LDS), asked once per shape
  // (computed by any thread that finds 0; all compute the same value)
  static std::atomic<int> per_cu_cache{0};
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, rq_fast_kernel<KA, KB, false>, S::kThreads, 0) !=
            hipSuccess ||
        blocks < 1)
      blocks = 1;
    per_cu = blocks;
    per_cu_cache.store(per_cu, std::memory_order_relaxed);
  }
  int64_t grid = static_cast<int64_t>(device_cu_count()) * per_cu;
  if (grid > a.tokens) grid = a.tokens;
  const dim3 blocks(static_cast<unsigned>(grid));
  const dim3 threads(static_cast<unsigned>(S::kThreads));
  if (a.zint)
    rq_fast_kernel<KA, KB, false, true><<<blocks, threads, 0, stream>>>(a);  // no y_out with zint
  else if (a.yout)
    rq_fast_kernel<KA, KB, true><<<blocks, threads, 0, stream>>>(a);
  else
    rq_fast_kernel<KA, KB, false><<<blocks, threads, 0, stream>>>(a);
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
      default: return launch_shape<56, 9>(a, s);  // 28 * 2^10 read as 56 * 2^9
    }
  }
  if (a.n == 4096) return launch_shape<32, 7>(a, s);
  if (a.n == 8192) return launch_shape<32, 8>(a, s);
  return launch_shape<32, 9>(a, s);
}

const char* rq_fast_name(int n) {
  if (n == 28672) return "rq_mfma56_w14";
  if (n % 28 == 0) return "rq_mfma28_w7";
  return "rq_mfma32_w8";
}

}  // namespace signrot
