// Fused rotate + sign flip + per-token asymmetric INT4 for gfx950 when
// n = m * 2^k with an outer factor H_m given by its sign tables (m a
// multiple of 4 up to 512: a Paley matrix, possibly times a Sylvester factor)
// and 16 <= 2^k <= 256: 11008 = 344 * 2^5, 13824 = 108 * 2^7,
// 18944 = 148 * 2^7, 8960 = 140 * 2^6, 27648 = 108 * 2^8, 5120 = 20 * 2^8,
// 5504 = 344 * 2^4 and the other shapes of the table at the end of this file.
//
// Method: explainer "SignRot for 4-bit LLM quantization -- Sign-adjusted
// Hadamard rotation", paragraphs on rotation (every output a signed sum of all
// inputs, scaled by 1/sqrt(n)), on the sign adjustment and on the quantizer.
//
// With x[a * B + b] (a < m, b < B = 2^k = 16 NTL) the transform
// H = H_m (x) H_B is evaluated per token row as
//   staging: HBM -> VGPRs (16-byte loads issued one row ahead) -> LDS,
//     transposed: b-row b holds x[0..m-1][b] in bf16 with a contiguous,
//     zero-padded to 32 KC entries, at LDS row rho(b) (the four lane bits of b
//     low, its tile bits high) with a pitch of 64 KC + 32 bytes (64 KC + 16
//     where the wider rows would cost a resident work-group, and with 16
//     column tiles; see OuterShape::RS).  Two a-rows are staged together so
//     that every LDS write is a whole dword.
//   stage 1 (MFMA): Z[a'][b] = sum_a W[a'][a] x[a][b], W = H_m^T (each row
//     a' times sigma * H_m[c_a][a'] for the calibrated sign vector), as
//     v_mfma_f32_16x16x32_bf16 with M = a' (16 per tile), K = a (32 per
//     chunk), N = b (16 per tile).  The weights are +-1 and the input is
//     bf16, so every product is exact and only the binary32 sums round.  Wave
//     w owns M-tiles w MTW .. w MTW + MTW - 1 and holds their weights in VGPRs
//     for the whole launch.  Lane column nl of N-tile nt reads the b-row
//     ((nl ^ kXLane) NTL + nt) ^ c_b.
//   stage 2 (VALU): the B-point Walsh-Hadamard transform over b: butterflies
//     across the NTL tiles in registers, then the four DPP stages across the
//     16 lanes of a row.  Lane (g, nl) then holds, for its rows
//     a' = 16 mt + 4 g + r, the NTL consecutive channels
//     a' B + NTL lane_perm(nl) + (0 .. NTL - 1).
//   stage 3: min / max over the token (lanes, then waves through LDS), scale
//     and zero-point, rounding by v_cvt_pk_u8_f32, nibble packing, NTL / 2
//     bytes of codes per row and lane.
//
// Sign vector.  For d = sigma * (row c of H) the flip is free: the factor
// sigma * H_m[c_a][a'] goes into the weights, the Sylvester factor
// (-1)^popcount(c_b & b') becomes the read of b-row b ^ c_b, and x_c is staged
// as zero and added back as the constant sigma * x_c.  Any other d is applied
// as a sign-bit XOR after stage 2.
#pragma once

#include <math.h>

#include <atomic>

#include "device_common.h"
#include "wave_ops.h"

namespace signrot {
namespace {

using namespace wave;

template <int KC, int NTL, int MTW>
struct OuterShape {
  static constexpr int LGN = NTL == 1 ? 0 : NTL == 2 ? 1 : NTL == 4 ? 2 : NTL == 8 ? 3 : 4;
  static_assert(NTL == (1 << LGN) && NTL >= 1 && NTL <= 16, "1 to 16 column tiles");
  static_assert(NTL > 1 || MTW % 2 == 0, "one column tile: an even number of M-tiles per wave");
  static_assert(KC >= 1 && KC <= 16, "outer order up to 512");
  static constexpr int KB = 4 + LGN;          // log2 B
  static constexpr int B = 16 * NTL;
  // LDS bytes per b-row.  An operand read serves 32 lanes (16 b-rows, two
  // 16-byte chunks) per pass in 8-byte halves.  On gfx950 that was 2-way bank
  // conflicted with a 64 KC + 16 pitch (rocprofv3 SQ_LDS_BANK_CONFLICT: 4
  // cycles per read, 8.0e6 per launch at n = 11008 x 8192) and is conflict-free
  // with 64 KC + 32 (1.4e5, what is left coming from other accesses); the
  // counts fit 64 banks of 8 bytes.  The staging writes then conflict more
  // (1.4e6 -> 4.2e6 there); the launch is 1-8 % faster at most widths with
  // 2^k <= 128 (384 and 8832 ran 1-3 % slower).
  // The wider pitch is not used where it would leave room for fewer
  // work-groups per CU (n = 9216 ran 81 -> 135 us, 5632 34 -> 38 us) nor with
  // 16 column tiles, where it measured slower (n = 27648, 17408, 5120).
  static constexpr int kMaxN = 32 * KC * B;
  // waves per work-group for m <= 32 KC: ceil(ceil(m / 16) / MTW)
  static constexpr int kMaxWaves = (2 * KC + MTW - 1) / MTW;
  // work-groups per CU that the LDS (160 KiB) leaves room for at pitch rs,
  // capped by 32 waves per CU
  static constexpr int lds_bytes(int rs) { return 2 * B * rs + 4 * (kMaxN / 32) + 280; }  // + d bits, reductions
  static constexpr int wgs_per_cu(int rs) {
    const int by_lds = 163840 / ((lds_bytes(rs) + 511) / 512 * 512);
    return by_lds < 32 / kMaxWaves ? by_lds : 32 / kMaxWaves;
  }
  static constexpr bool kWidePitch = NTL <= 8 && wgs_per_cu(64 * KC + 32) == wgs_per_cu(64 * KC + 16);
  static constexpr int RS = 64 * KC + (kWidePitch ? 32 : 16);
  static constexpr int kBufBytes = B * RS;
  static constexpr int NV = MTW * NTL * 4;    // values per lane
  // staging units (two 16-byte loads: 8 channels of a-rows 2p and 2p + 1)
  // per thread: m NTL units over 64 ceil(m / (16 MTW)) threads
  static constexpr int UPT = (NTL * MTW + 3) / 4;
  static_assert(kMaxWaves <= 16, "at most 16 waves per work-group");
};

// LDS row of b-row b: lane bits (b >> LGN) low, tile bits (b mod NTL) high.
template <int LGN>
__device__ __forceinline__ uint32_t lds_row(uint32_t b) {
  return (b >> LGN) | ((b & ((1u << LGN) - 1u)) << 4);
}

// One column tile (2^k = 16): lane nl reads input index one_tile_in(nl);
// after the four DPP stages it holds output one_tile_out(nl), and lanes nl
// and nl ^ 1 hold adjacent outputs (one_tile_out(nl ^ 1) = one_tile_out(nl) ^ 1),
// so a code byte pairs the two lanes of a quad half.  (With the usual input
// nl ^ kXLane the pairs would sit six lanes apart.)
__device__ __forceinline__ int one_tile_in(int nl) {
  const int v = nl ^ kXLane;
  return v ^ ((v >> 2) & 1);
}
__device__ __forceinline__ int one_tile_out(int nl) {
  return (nl & 9) ^ ((nl & 2) ? 6 : 0) ^ ((nl & 4) ? 3 : 0);
}

template <int KC, int NTL, int MTW, bool GENERAL, bool YOUT, bool ZINT = false>
__device__ void rq_outer_body(const RqArgs& a, uint8_t* lds, const uint32_t* dbits, const DForm& form, float* red,
                              float* xcl) {
  using S = OuterShape<KC, NTL, MTW>;
  constexpr int NV = S::NV;
  constexpr int LGN = S::LGN;
  constexpr int B = S::B;
  constexpr int RS = S::RS;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = static_cast<int>(blockDim.x >> 6);
  const int nthr = static_cast<int>(blockDim.x);
  const int g4 = lane >> 4;
  const int nl = lane & 15;
  const int m = a.m;
  const int mtiles = (m + 15) >> 4;
  const int n = a.n;

  const int c = GENERAL ? 0 : __builtin_amdgcn_readfirstlane(form.c);
  const int ca = c >> S::KB;
  const int cb = c & (B - 1);
  const int cbl = cb & (NTL - 1);
  const int cbh = cb >> LGN;
  const int sig = (!GENERAL && form.neg) ? -1 : 1;

  // Weights: A operand of M-tile mt = w MTW + i, K chunk kc.  Lane (g4, nl)
  // holds row a' = 16 mt + nl, k = a = 32 kc + 8 g4 + j (j < 8): H_m[a][a']
  // from bit a of row a' of the transposed table, times the row's flip.
  // Rows beyond m get zero weights (their outputs are never used); columns
  // beyond m meet the zero padding of the staged row.
  bf16x8_t wA[MTW][KC];
#pragma unroll
  for (int i = 0; i < MTW; ++i) {
    const int mt = w * MTW + i;
    const int ap = 16 * mt + nl;
    const bool ok = mt < mtiles && ap < m;
    uint32_t flip = 0u;
    if (!GENERAL && ok) flip = args_outer_negbit(a, ca, ap) ^ static_cast<uint32_t>(form.neg);
    // order 28 (KC = 1): the column a' of H28 gathered from the row masks
    uint32_t col28 = 0u;
    if (m == 28 && ok)
      for (int r = 0; r < 28; ++r) col28 |= ((a.h28mask[r] >> ap) & 1u) << r;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const uint32_t word = !ok ? 0u : (m == 28 ? col28 : a.hmt[ap * a.hw + kc]);
      const uint32_t bits = (word >> (8 * g4)) & 0xffu;
      bf16x8_t v;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = ok ? static_cast<short>((((bits >> j) ^ flip) & 1u) ? 0xbf80 : 0x3f80) : static_cast<short>(0);
      wA[i][kc] = v;
    }
  }

  // Staging: unit u = tid + nthr i; a-rows 2p, 2p + 1 with p = u / UPR,
  // channels b0 .. b0 + 7 with b0 = 8 (u mod UPR).
  constexpr int UPR = B / 8;
  const int units = n >> 4;
  uint4 st[S::UPT][2];
  auto load_row = [&](int64_t row) {
    const uint16_t* xr = a.x + row * a.ld;
#pragma unroll
    for (int i = 0; i < S::UPT; ++i) {
      const int u = tid + nthr * i;
      if (u < units) {
        const uint16_t* src = xr + (2 * (u / UPR)) * B + 8 * (u & (UPR - 1));
        st[i][0] = *reinterpret_cast<const uint4*>(src);
        st[i][1] = *reinterpret_cast<const uint4*>(src + B);
      }
    }
  };
  auto write_row = [&](uint32_t bo, int par) {
#pragma unroll
    for (int i = 0; i < S::UPT; ++i) {
      const int u = tid + nthr * i;
      if (u < units) {
        const int p = u / UPR;
        const int b0 = 8 * (u & (UPR - 1));
        uint32_t lo[4] = {st[i][0].x, st[i][0].y, st[i][0].z, st[i][0].w};
        uint32_t hi[4] = {st[i][1].x, st[i][1].y, st[i][1].z, st[i][1].w};
        if (!GENERAL && 2 * p == (ca & ~1) && b0 == (cb & ~7)) {
          // this unit holds x_c: keep its value for the shift, stage a zero
          const int e = cb & 7;
          const bool in_hi = (ca & 1) != 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (q == (e >> 1)) {
              const uint32_t wd = in_hi ? hi[q] : lo[q];
              const uint32_t bits = (e & 1) ? (wd >> 16) : (wd & 0xffffu);
              xcl[par] = __uint_as_float(bits << 16);
              const uint32_t z = (e & 1) ? (wd & 0xffffu) : (wd & 0xffff0000u);
              if (in_hi) hi[q] = z;
              else lo[q] = z;
            }
          }
        }
        uint8_t* dst = lds + bo + 4 * p;  // byte offset of a = 2p in a b-row
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t even = __builtin_amdgcn_perm(hi[q], lo[q], 0x05040100u);
          const uint32_t odd = __builtin_amdgcn_perm(hi[q], lo[q], 0x07060302u);
          *reinterpret_cast<uint32_t*>(dst + lds_row<LGN>(b0 + 2 * q) * RS) = even;
          *reinterpret_cast<uint32_t*>(dst + lds_row<LGN>(b0 + 2 * q + 1) * RS) = odd;
        }
      }
    }
  };

  // operand read offset of this lane inside a buffer (N-tile part added per nt)
  const int lane_in = NTL == 1 ? one_tile_in(nl) : (nl ^ kXLane);
  const uint32_t lane_off = static_cast<uint32_t>(lane_in ^ cbh) * RS + 16u * g4;
  const float gdpp0 = (((nl >> 0) ^ (nl >> 2)) & 1) ? -1.0f : 1.0f;
  const float gdpp1 = (((nl >> 1) ^ (nl >> 2)) & 1) ? -1.0f : 1.0f;
  const float gdpp2 = ((nl >> 2) & 1) ? -1.0f : 1.0f;
  const float gdpp3 = ((nl >> 3) & 1) ? -1.0f : 1.0f;
  const int outm = NTL == 1 ? one_tile_out(nl) : lane_perm(nl);

  // rows a' of this lane: 16 (w MTW + i) + 4 g4 + r
  bool rv[MTW][4];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mt = w * MTW + i;
      rv[i][r] = mt < mtiles && 16 * mt + 4 * g4 + r < m;
    }

  const int64_t tokens = a.tokens;
  const int64_t grid = gridDim.x;
  int64_t cur = blockIdx.x;
  int64_t nxt = cur + grid;
  int64_t nn = nxt + grid;
  if (cur >= tokens) return;
  load_row(cur);
  // K padding (a >= m) must read as zero: clear both buffers once
  for (int o = 16 * tid; o < 2 * S::kBufBytes; o += 16 * nthr)
    *reinterpret_cast<u32x4_t*>(lds + o) = u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();
  write_row(0u, 0);
  if (nxt < tokens) load_row(nxt);
  lds_barrier();

  for (int it = 0; cur < tokens; ++it) {
    const int64_t row = cur;
    const int par = it & 1;
    const uint32_t bo = par ? static_cast<uint32_t>(S::kBufBytes) : 0u;

    // (0) stage the next row (loaded a row ago) into the other buffer, whose
    // last reader was the previous row's MFMA stage, before the previous
    // barrier; done here so that the staging registers are dead during (1)
    if (nxt < tokens) write_row(bo ^ static_cast<uint32_t>(S::kBufBytes), par ^ 1);

    // (1) MFMA stage from this row's buffer
    f32x4_t acc[MTW][NTL];
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int t = 0; t < NTL; ++t) acc[i][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
      for (int t = 0; t < NTL; ++t) {
        const bf16x8_t op = *reinterpret_cast<const bf16x8_t*>(
            lds + bo + lane_off + static_cast<uint32_t>(((t ^ cbl) << 4) * RS + 64 * kc));
#pragma unroll
        for (int i = 0; i < MTW; ++i)
          acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wA[i][kc], op, acc[i][t], 0, 0, 0);
      }
    }
    // x_c of this row: published by the previous barrier; its slot is next
    // written after this row's barrier
    const float xc = GENERAL ? 0.0f : xcl[par];

    // (2) start loading the row after next
    if (nn < tokens) load_row(nn);

    // (3) B-point transform over b
    float v[NV];
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[(i * NTL + t) * 4 + r] = acc[i][t][r];
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      float(&vi)[NTL * 4] = *reinterpret_cast<float(*)[NTL * 4]>(v + i * NTL * 4);
      if constexpr (NTL >= 2) reg_stage<NTL, 0>(vi);
      if constexpr (NTL >= 4) reg_stage<NTL, 1>(vi);
      if constexpr (NTL >= 8) reg_stage<NTL, 2>(vi);
      if constexpr (NTL >= 16) reg_stage<NTL, 3>(vi);
    }
    dpp_stage<NV>(v, gdpp0, 0);
    dpp_stage<NV>(v, gdpp1, 1);
    dpp_stage<NV>(v, gdpp2, 2);
    dpp_stage<NV>(v, gdpp3, 3);
    if (GENERAL) {
#pragma unroll
      for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (!rv[i][r]) continue;
          const int j0 = (16 * (w * MTW + i) + 4 * g4 + r) * B + NTL * outm;
          const uint32_t bits = dbits[j0 >> 5] >> (j0 & 31);
#pragma unroll
          for (int t = 0; t < NTL; ++t) {
            float& e = v[(i * NTL + t) * 4 + r];
            e = __uint_as_float(__float_as_uint(e) ^ (((bits >> t) & 1u) << 31));
          }
        }
    }

    // (4) min / max over the row's valid outputs: lanes, then waves via LDS
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!rv[i][r]) continue;
        if constexpr (NTL == 1) {
          mn = fmin_raw(mn, v[i * 4 + r]);
          mx = fmax_raw(mx, v[i * 4 + r]);
        } else {
#pragma unroll
          for (int t = 0; t < NTL; t += 2) {
            min3_acc(mn, v[(i * NTL + t) * 4 + r], v[(i * NTL + t + 1) * 4 + r]);
            max3_acc(mx, v[(i * NTL + t) * 4 + r], v[(i * NTL + t + 1) * 4 + r]);
          }
        }
      }
    wave_minmax(mn, mx);
    float* rd = red + 32 * par;  // per-wave min at rd[w], max at rd[16 + w]
    if (lane == 63) {
      rd[w] = mn;
      rd[16 + w] = mx;
    }
    lds_barrier();
    // the other waves' min / max, four per 16-byte read
    for (int q = 0; q < nw; q += 4) {
      const f32x4_t m4 = *reinterpret_cast<const f32x4_t*>(rd + q);
      const f32x4_t x4 = *reinterpret_cast<const f32x4_t*>(rd + 16 + q);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (q + k < nw) {
          mn = fmin_raw(mn, m4[k]);
          mx = fmax_raw(mx, x4[k]);
        }
      }
    }

    // (5) quantize, pack, store
    const QuantParams qp = quant_params(mn, mx);
    const float shift = sig > 0 ? xc : -xc;
    float cq = qp.cq;
    float zq = 0.0f;
    if constexpr (ZINT) {
      zq = qp.degenerate ? rintf(-((mn + shift) * a.inv_sqrt_n)) : rintf(-(mn + shift) * qp.inv);
      cq = qp.degenerate ? 0.0f : fmaf(shift, qp.inv, zq);
    }
    if (tid == 0) {
      a.scale[row] = qp.degenerate ? 1.0f : qp.range * a.inv_15sqrt_n;
      a.zero[row] = ZINT ? zq : (qp.degenerate ? -((mn + shift) * a.inv_sqrt_n) : -(mn + shift) * qp.inv);
    }
    uint8_t* crow = a.codes + row * static_cast<int64_t>(n / 2);
    if constexpr (NTL == 1) {
      // one code per lane and row: every lane rounds its value and takes its
      // partner's code from lane nl ^ 1; the lane holding the even channel
      // stores the byte
#pragma unroll
      for (int i = 0; i < MTW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float f = fmaf(v[i * 4 + r], qp.inv, cq);
          if constexpr (ZINT) f = fminf(f, 15.0f);
          const int q = static_cast<int>(__builtin_amdgcn_cvt_pk_u8_f32(f, 0, 0u));
          const int qp1 = __builtin_amdgcn_mov_dpp(q, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
          if (!rv[i][r]) continue;
          const int j0 = (16 * (w * MTW + i) + 4 * g4 + r) * B + outm;
          if ((outm & 1) == 0) crow[j0 / 2] = static_cast<uint8_t>(q | (qp1 << 4));
          if (YOUT) a.yout[row * static_cast<int64_t>(n) + j0] = (v[i * 4 + r] + shift) * a.inv_sqrt_n;
        }
    }
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (NTL == 1 || !rv[i][r]) continue;
        const int j0 = (16 * (w * MTW + i) + 4 * g4 + r) * B + NTL * outm;
        uint32_t q[(NTL + 7) / 8] = {};
#pragma unroll
        for (int u = 0; u < (NTL + 7) / 8; ++u) {
          uint32_t ev = 0u, od = 0u;
#pragma unroll
          for (int k = 0; k < 4 && 8 * u + 2 * k < NTL; ++k) {
            float fe = fmaf(v[(i * NTL + 8 * u + 2 * k) * 4 + r], qp.inv, cq);
            float fo = fmaf(v[(i * NTL + 8 * u + 2 * k + 1) * 4 + r], qp.inv, cq);
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
        uint8_t* cp = crow + j0 / 2;
        if constexpr (NTL <= 2) *cp = static_cast<uint8_t>(q[0]);
        else if constexpr (NTL == 4) *reinterpret_cast<uint16_t*>(cp) = static_cast<uint16_t>(q[0]);
        else if constexpr (NTL == 8) *reinterpret_cast<uint32_t*>(cp) = q[0];
        else *reinterpret_cast<uint2*>(cp) = make_uint2(q[0], q[1]);
        if (YOUT) {
          float* yp = a.yout + row * static_cast<int64_t>(n) + j0;
#pragma unroll
          for (int t = 0; t + 1 < NTL; t += 2) {
            const float y0 = (v[(i * NTL + t) * 4 + r] + shift) * a.inv_sqrt_n;
            const float y1 = (v[(i * NTL + t + 1) * 4 + r] + shift) * a.inv_sqrt_n;
            *reinterpret_cast<float2*>(yp + t) = make_float2(y0, y1);
          }
        }
      }

    // (6) advance the row queue
    cur = nxt;
    nxt = nn;
    nn += grid;
  }
}

template <int KC, int NTL, int MTW, bool YOUT, bool ZINT = false>
__global__ __launch_bounds__((64 * OuterShape<KC, NTL, MTW>::kMaxWaves)) void rq_outer_kernel(RqArgs a) {
  using S = OuterShape<KC, NTL, MTW>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * S::kBufBytes];
  __shared__ uint32_t dbits[S::kMaxN / 32];
  __shared__ __attribute__((aligned(16))) float red[64];
  __shared__ float xcl[2];
  __shared__ int scratch[4];
  DForm form;
  if (a.form_given) {
    // d = sigma * (row c of H) by construction: nothing to read or decode
    form = DForm{1, a.form_c, a.form_neg};
  } else {
    build_dbits(a.d, a.n, dbits);  // bit j set when d_j = -1
    __syncthreads();
    form = decode_d_form(a, dbits, scratch);
  }
  if constexpr (ZINT) {
    // only with d given as (c, sigma): always the structured form
    rq_outer_body<KC, NTL, MTW, false, YOUT, true>(a, lds, dbits, form, red, xcl);
  } else {
    if (form.structured) rq_outer_body<KC, NTL, MTW, false, YOUT>(a, lds, dbits, form, red, xcl);
    else rq_outer_body<KC, NTL, MTW, true, YOUT>(a, lds, dbits, form, red, xcl);
  }
}

template <int KC, int NTL, int MTW>
hipError_t launch_outer_shape(const RqArgs& a, hipStream_t stream) {
  const int waves = ((a.m + 15) / 16 + MTW - 1) / MTW;
  const int threads = 64 * waves;
  // resident work-groups per CU at this block size, asked once per size
  // (computed by any thread that finds 0; all compute the same value)
  static std::atomic<int> per_cu_cache[17];
  int per_cu = per_cu_cache[waves].load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &blocks, reinterpret_cast<const void*>(&rq_outer_kernel<KC, NTL, MTW, false, false>), threads, 0) !=
            hipSuccess ||
        blocks < 1)
      blocks = 1;
    per_cu = blocks;
    per_cu_cache[waves].store(per_cu, std::memory_order_relaxed);
  }
  int64_t grid = static_cast<int64_t>(device_cu_count()) * per_cu;
  if (grid > a.tokens) grid = a.tokens;
  const dim3 blocks(static_cast<unsigned>(grid));
  const dim3 thr(static_cast<unsigned>(threads));
  if (a.zint)
    rq_outer_kernel<KC, NTL, MTW, false, true><<<blocks, thr, 0, stream>>>(a);  // no y_out with zint
  else if (a.yout)
    rq_outer_kernel<KC, NTL, MTW, true><<<blocks, thr, 0, stream>>>(a);
  else
    rq_outer_kernel<KC, NTL, MTW, false><<<blocks, thr, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

// The built shapes: (K chunks, column tiles, M-tiles per wave).  MTW keeps
// the weights of a wave (4 MTW KC VGPRs for the whole launch), its
// accumulators and its staging registers near the register share that its
// launch bound (ceil(2 KC / MTW) waves per work-group) leaves, and the
// work-group within 16 waves.  The shapes with KC >= 9 and MTW = 2 reach 168
// VGPRs and still spill 8-56 bytes per lane, as does KC = 4 with 16 column
// tiles and y_out (python -m rotation_activation_quantization_amd.build
// --resources lists every instance); separate instances for the two forms of
// d remove those spills but ran slower at n = 11008.  One translation unit
// per column-tile count instantiates them.
#define SR_OUTER_SHAPES_T1(X)                                                                                   \
  X(1, 1, 2) X(2, 1, 2) X(3, 1, 2) X(4, 1, 2) X(5, 1, 2) X(6, 1, 2) X(7, 1, 2) X(8, 1, 2) X(9, 1, 2) X(10, 1, 2) \
  X(11, 1, 2) X(12, 1, 2)
#define SR_OUTER_SHAPES_T2(X) \
  X(1, 2, 1) X(2, 2, 1) X(3, 2, 1) X(4, 2, 1) X(5, 2, 1) X(6, 2, 1) X(7, 2, 1) X(8, 2, 1) X(9, 2, 2) X(10, 2, 2) \
  X(11, 2, 2) X(12, 2, 2)
#define SR_OUTER_SHAPES_T4(X) X(1, 4, 1) X(2, 4, 1) X(3, 4, 1) X(4, 4, 1) X(5, 4, 1) X(6, 4, 1) X(7, 4, 1) X(8, 4, 1)
#define SR_OUTER_SHAPES_T8(X) X(1, 8, 1) X(2, 8, 1) X(3, 8, 1) X(4, 8, 1) X(5, 8, 1) X(6, 8, 1)
// (1 and 3 K chunks with 16 column tiles are not built: those widths run
// faster read with 8 column tiles, as (2m) x 2^(k - 1).)
#define SR_OUTER_SHAPES_T16(X) X(2, 16, 1) X(4, 16, 1)

// Per column-tile count: M-tiles per wave for kc (0: not built), and the launch.
#define SR_OUTER_DECLARE(NTL)                                \
  int rq_outer_mtw_t##NTL(int kc);                           \
  hipError_t rq_outer_launch_t##NTL(const RqArgs& a, hipStream_t s);
SR_OUTER_DECLARE(1)
SR_OUTER_DECLARE(2)
SR_OUTER_DECLARE(4)
SR_OUTER_DECLARE(8)
SR_OUTER_DECLARE(16)
#undef SR_OUTER_DECLARE

// Body of one instantiation unit: the table lookup and the launch switch.
#define SR_OUTER_DEFINE(NTL, SHAPES)                                             \
  int rq_outer_mtw_t##NTL(int kc) {                                            \
    SHAPES(SR_OUTER_MTW_CASE)                                                  \
    return 0;                                                                  \
  }                                                                            \
  hipError_t rq_outer_launch_t##NTL(const RqArgs& a, hipStream_t s) {          \
    const int kc = (a.m + 31) / 32;                                            \
    SHAPES(SR_OUTER_LAUNCH_CASE)                                               \
    return hipErrorInvalidValue;                                               \
  }
#define SR_OUTER_MTW_CASE(K, N, W) \
  if (kc == K) return W;
#define SR_OUTER_LAUNCH_CASE(K, N, W) \
  if (kc == K) return launch_outer_shape<K, N, W>(a, s);

}  // namespace signrot
