// Fused rotate + sign flip + per-token asymmetric INT4 for gfx950 at
// n = 28 * 2^10 = 28672 (the LLaMA3-70B down-projection input), as two halves
// of the n = 14336 kernel's transform (rq_fast.hip; the explainer "SignRot for
// 4-bit LLM quantization", paragraphs on rotation and on the down-projection:
// a Hadamard matrix applied as a fast Walsh-Hadamard transform).  Staging,
// the MFMA stage, the lane transform and the quantizer follow rq_fast.hip.
#include <math.h>

#include <atomic>

#include "rq_fast_common.h"

namespace signrot {
namespace {

// n = 28672 = 28 * 2^10 in two halves.  With i = a * 1024 + h * 512 + b
// (a < 28, h < 2, b < 512), H = H28 (x) H2 (x) H512, so
//   (x H)[a', h', b'] = Z_0[a', b'] + (-1)^h' Z_1[a', b'],
// where Z_h is half h of x (read as a 28 x 512 row: a-rows 2048 bytes apart,
// starting at byte 1024 h) times H28 (x) H512, the n = 14336 transform of
// rq_fast.hip.  For d = sigma * H[c][.] with c = (c_a, c_h, c_b), d[a', h', b']
// is sigma * H28[c_a][a'] * H512[c_b][b'] (folded into both Z_h as there)
// times (-1)^(c_h h').  A work-group of seven waves takes a row in two phases,
// one half each, through two 28 KB half-row buffers, so that each lane holds
// the same 32 positions of Z_0 and Z_1 and forms both outputs with one add or
// subtract each.  Against reading the row as H56 (x) H512 (fourteen waves,
// K = 224 per output) this halves the MFMA work per value, and with 61 KB of
// LDS and at most 128 VGPRs two work-groups fit on a CU.  Two LDS barriers
// per row: the first publishes the second half's buffer, the second the next
// row's first half and the per-wave min / max.
//
// GENERAL: d is any sign vector (applied as a sign-bit XOR after the
// transform; the weights then carry no fold); otherwise d = sigma * H[c][.].
// The d-vector kernel branches between the two bodies once per work-group,
// so each is register-allocated on its own.
template <bool GENERAL, bool YOUT, bool ZINT, bool SWIGLU>
__device__ void rq_halves_body(const RqArgs& a, uint8_t* lds, const uint32_t* dbits, const uint32_t* h28,
                               const DForm& form, float* red, float* xcl) {
  using S = FastShape<28, 9>;  // one half
  constexpr int NT = S::NT;
  constexpr int NV = S::NV;
  constexpr uint32_t kFull = 2u * S::N;  // 28672
  static_assert(NT == 8 && NV == 32 && S::CR == 64 && S::CPT == 4, "half-row shape");
  constexpr bool general = GENERAL;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int nl = lane & 15;

  const int c = general ? 0 : __builtin_amdgcn_readfirstlane(form.c);
  const int ca = c >> 10;
  const int ch = (c >> 9) & 1;
  const int cb = c & 511;
  const int cbb = cb & 3;
  const int cbq_lo = (cb >> 2) & (NT - 1);
  const int cbq_hi = cb >> (2 + S::LG);
  const int sig = (!general && __builtin_amdgcn_readfirstlane(form.neg)) ? -1 : 1;

  // Staging as in rq_fast.hip (units of 64 chunks, lane L on a-row parity
  // L & 1 and chunk L >> 1 of the unit), with the half's a-row stride, and
  // with wave w taking the four consecutive units s = 4 w + i (pair-rows 2 w
  // and 2 w + 1): the LDS offset of unit i is then the wave's base plus a
  // constant, so that the staging addresses are two registers plus
  // immediate offsets (both buffers).
  const uint32_t ul = static_cast<uint32_t>(lane);
  const uint32_t ue = ul >> 1;
  const uint32_t gl = 2048u * (ul & 1u) + 16u * ue;
  uint32_t wl[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    wl[h] = 2u * S::PB * static_cast<uint32_t>(w) + 16u * quad_slot<28, 9>(2u * ue + h) + 8u * (ul & 1u);
  auto unit_g = [&](int i, int half) -> uint32_t {
    const uint32_t s = static_cast<uint32_t>(S::CPT * w + i);
    return 4096u * (s >> 1) + 512u * (s & 1u) + 1024u * static_cast<uint32_t>(half);
  };
  auto unit_l = [&](int i) -> uint32_t {  // beyond the wave's base in wl
    return S::PB * static_cast<uint32_t>(i >> 1) + 128u * static_cast<uint32_t>(i & 1);
  };
  u32x4_t st[S::CPT];
  u32x4_t stu[SWIGLU ? S::CPT : 1];
  auto load_half = [&](int64_t r, int half) {
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.x + r * a.ld, 2u * kFull);
#pragma unroll
    for (int i = 0; i < S::CPT; ++i)
      st[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, gl, unit_g(i, half), kNontemporal));
    if constexpr (SWIGLU) {
      const __amdgpu_buffer_rsrc_t ru = buffer_rsrc(a.x2 + r * a.ld, 2u * kFull);
#pragma unroll
      for (int i = 0; i < S::CPT; ++i)
        stu[i] =
            __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ru, gl, unit_g(i, half), kNontemporal));
    }
  };
  // Past the last row the staging registers are given opaque new values
  // instead of a load, so that on every path they are redefined where the
  // loads would be: otherwise the compiler keeps the old ones live around the
  // loop, across the MFMA and transform stages.
  auto next_half = [&](int64_t r, int half) {
    if (r < a.tokens) {
      load_half(r, half);
    } else {
#pragma unroll
      for (int i = 0; i < S::CPT; ++i) {
        asm volatile("" : "=v"(st[i]));
        if constexpr (SWIGLU) asm volatile("" : "=v"(stu[i]));
      }
    }
  };
  if (static_cast<int64_t>(blockIdx.x) < a.tokens) load_half(blockIdx.x, 0);

  // MFMA weights (H28 (x) H4 with the (c_a, c_b) fold), as in rq_fast.hip.
  bf16x8_t wA[S::NKC];
  {
    const int ap = 4 * w + (nl >> 2);
    const int cc = nl & 3;
    const int hrow = hka_sign<28>(h28, ca, ap) * sig;
#pragma unroll
    for (int kc = 0; kc < S::NKC; ++kc)
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
  const uint32_t rbase = static_cast<uint32_t>(S::PB) * static_cast<uint32_t>(g) +
                         ((16u * static_cast<uint32_t>(nl ^ kXLane ^ cbq_hi)) ^ (S::KMUL * static_cast<uint32_t>(cbq_lo)));

  // x_c sits in half c_h at index c_a * 512 + c_b of that half.
  int xc_wave = -1, xc_lane = 0, xc_i = 0, xc_e = 0;
  if (!general) {
    const int chunk = (ca * 512 + cb) >> 3;
    const int arow = chunk / S::CR, j = chunk % S::CR;
    const int s = (arow >> 1) * 2 + (j >> 5);
    xc_i = s % S::CPT;
    xc_wave = s / S::CPT;
    xc_lane = 2 * (j & 31) + (arow & 1);
    xc_e = c & 7;
  }
  const bool xc_thread = !general && w == xc_wave && lane == xc_lane;

  const int ap = 4 * w + g;
  const int chan0 = ap * 1024 + 4 * NT * lane_perm(nl);  // output half 0; half 1 at + 512

  auto write_half = [&](uint32_t bo, int xslot, int half) {
    if constexpr (SWIGLU) {
#pragma unroll
      for (int i = 0; i < S::CPT; ++i) st[i] = swiglu_chunk(st[i], stu[i]);
    }
    if (xc_thread && half == ch) {
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
      *reinterpret_cast<uint2*>(lds + wl[0] + (bo + unit_l(i))) = make_uint2(st[i][0], st[i][1]);
      *reinterpret_cast<uint2*>(lds + wl[1] + (bo + unit_l(i))) = make_uint2(st[i][2], st[i][3]);
    }
  };
  auto mfma_half = [&](float (&v)[NV], uint32_t bo) {
    // an opaque copy, so that the NT - 1 other tile addresses are formed here
    // (one XOR each) rather than hoisted out of the loop as live registers;
    // the buffer offset rides in the instruction's offset field
    uint32_t rb = rbase;
    asm volatile("" : "+v"(rb));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint8_t* tp = lds + (rb ^ (S::KMUL * t)) + bo;
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
      // operands two chunks at a time (registers are short here)
#pragma unroll
      for (int k0 = 0; k0 < S::NKC; k0 += 2) {
        u32x4_t b[2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) b[kc] = *reinterpret_cast<const u32x4_t*>(tp + 4 * S::PB * (k0 + kc));
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wA[k0 + kc], __builtin_bit_cast(bf16x8_t, b[kc]), acc, 0, 0,
                                                        0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * t + r] = acc[r];
    }
  };
  auto fwht_half = [&](float (&v)[NV]) {
    reg_stage<NT, 0>(v);
    reg_stage<NT, 1>(v);
    reg_stage<NT, 2>(v);
    dpp_stage<NV>(v, gdpp0, 0);
    dpp_stage<NV>(v, gdpp1, 1);
    dpp_stage<NV>(v, gdpp2, 2);
    dpp_stage<NV>(v, gdpp3, 3);
  };

  const int64_t tokens = a.tokens;
  const int64_t grid = gridDim.x;
  int64_t cur = blockIdx.x;
  if (cur >= tokens) return;
  wait_vmcnt<0>();
  write_half(0u, 0, 0);
  load_half(cur, 1);
  lds_barrier();

  for (int it = 0; cur < tokens; ++it) {
    const int64_t row = cur;
    const int64_t nxt = cur + grid;
    const int par = it & 1;
    constexpr uint32_t kB1 = static_cast<uint32_t>(S::kRowBytes);

    // Phase 1: half 0 from buffer 0; stage half 1 (its loads were issued
    // between the previous row's two code stores; after them came the second
    // code store and, with y_out, NT y stores).
    float v0[NV];
    mfma_half(v0, 0u);
    if (it == 0) wait_vmcnt<0>();
    else if (YOUT) wait_vmcnt<1 + NT>();
    else wait_vmcnt<1>();
    write_half(kB1, par, 1);
    next_half(nxt, 0);
    fwht_half(v0);
    lds_barrier();

    // Phase 2: stage the next row's half 0 into buffer 0 (free since the
    // barrier), then half 1 from buffer 1.
    if (nxt < tokens) {
      wait_vmcnt<0>();
      write_half(0u, par ^ 1, 0);
    }
    float v1[NV];
    mfma_half(v1, kB1);
    fwht_half(v1);

    // Combine: output half 0 = Z_0 + Z_1, output half 1 = (-1)^(c_h) (Z_0 - Z_1).
    if (ch) {
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        const float p = v0[e], q = v1[e];
        v0[e] = p + q;
        v1[e] = q - p;
      }
    } else {
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        const float p = v0[e], q = v1[e];
        v0[e] = p + q;
        v1[e] = p - q;
      }
    }
    if (general) {
      // this lane's 32 bits of d for each output half, read from LDS every
      // row rather than held in registers
      const uint32_t* dp = dbits + (chan0 >> 5);
      const uint32_t d0 = dp[0];
      const uint32_t d1 = dp[16];
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        v0[e] = __uint_as_float(__float_as_uint(v0[e]) ^ ((d0 << (31 - e)) & 0x80000000u));
        v1[e] = __uint_as_float(__float_as_uint(v1[e]) ^ ((d1 << (31 - e)) & 0x80000000u));
      }
    }

    // min / max over the 64 values, the lanes, then the waves through LDS
    float mn = v0[0], mx = v0[0];
#pragma unroll
    for (int e = 1; e + 1 < NV; e += 2) {
      min3_acc(mn, v0[e], v0[e + 1]);
      max3_acc(mx, v0[e], v0[e + 1]);
    }
    mn = fmin_raw(mn, v0[NV - 1]);
    mx = fmax_raw(mx, v0[NV - 1]);
#pragma unroll
    for (int e = 0; e < NV; e += 2) {
      min3_acc(mn, v1[e], v1[e + 1]);
      max3_acc(mx, v1[e], v1[e + 1]);
    }
    wave_minmax(mn, mx);
    if (lane == 63) {
      red[w] = mn;
      red[16 + w] = mx;
    }
    const float xc = general ? 0.0f : xcl[par];
    lds_barrier();
    {
      const f32x4_t m4 = *reinterpret_cast<const f32x4_t*>(red);
      const f32x4_t x4 = *reinterpret_cast<const f32x4_t*>(red + 16);
      const f32x4_t m4b = *reinterpret_cast<const f32x4_t*>(red + 4);
      const f32x4_t x4b = *reinterpret_cast<const f32x4_t*>(red + 20);
      min3_acc(mn, m4[0], m4[1]);
      max3_acc(mx, x4[0], x4[1]);
      min3_acc(mn, m4[2], m4[3]);
      max3_acc(mx, x4[2], x4[3]);
      min3_acc(mn, m4b[0], m4b[1]);
      max3_acc(mx, x4b[0], x4b[1]);
      mn = fmin_raw(mn, m4b[2]);
      mx = fmax_raw(mx, x4b[2]);
    }

    // quantize, pack, store (output halves 0 and 1)
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
    auto pack = [&](const float (&v)[NV], uint32_t (&q)[NT / 2]) {
#pragma unroll
      for (int u = 0; u < NT / 2; ++u) {
        uint32_t ev = 0u, od = 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float fe = fmaf(v[8 * u + 2 * k], qp.inv, cq);
          float fo = fmaf(v[8 * u + 2 * k + 1], qp.inv, cq);
          if constexpr (ZINT) {
            fe = fminf(fe, 15.0f);
            fo = fminf(fo, 15.0f);
          }
          ev = __builtin_amdgcn_cvt_pk_u8_f32(fe, k, ev);
          od = __builtin_amdgcn_cvt_pk_u8_f32(fo, k, od);
        }
        q[u] = ev | (od << 4);
      }
    };
    const __amdgpu_buffer_rsrc_t cs = buffer_rsrc(a.codes + row * static_cast<int64_t>(kFull / 2), kFull / 2);
    const uint32_t coff = static_cast<uint32_t>(chan0 / 2);
    auto store_y = [&](const float (&v)[NV], int half) {
      const __amdgpu_buffer_rsrc_t ys = buffer_rsrc(a.yout + row * static_cast<int64_t>(kFull), 4u * kFull);
#pragma unroll
      for (int e4 = 0; e4 < NT; ++e4) {
        f32x4_t o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = (v[4 * e4 + k] + shift) * a.inv_sqrt_n;
        store_b128_held<0>(__builtin_bit_cast(u32x4_t, o), ys, 8u * coff, 2048 * half + 16 * e4);
      }
    };
    // Output half 0 first; the next row's half-1 loads go out once its values
    // are dead (they are then live beside half 1's values only).
    {
      uint32_t q[NT / 2];
      pack(v0, q);
      store_b128_held<kNontemporal>(u32x4_t{q[0], q[1], q[2], q[3]}, cs, coff, 0);
      if (YOUT) store_y(v0, 0);
    }
    next_half(nxt, 1);
    {
      uint32_t q[NT / 2];
      pack(v1, q);
      store_b128_held<kNontemporal>(u32x4_t{q[0], q[1], q[2], q[3]}, cs, coff, 256);
      if (YOUT) store_y(v1, 1);
    }
    cur = nxt;
  }
  wait_vmcnt<0>();
}

// n = 28672 in two halves of 28 x 512 (seven waves).
template <bool DVEC, bool YOUT, bool ZINT = false, bool SWIGLU = false>
__global__ __launch_bounds__(448) __attribute__((amdgpu_waves_per_eu(4)))
void rq_halves_kernel(RqArgs a) {
  using S = FastShape<28, 9>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[S::kLdsBytes];
  __shared__ uint32_t dbits[2 * S::N / 32];
  __shared__ __attribute__((aligned(16))) float red[32];
  __shared__ float xcl[2];
  __shared__ int scratch[4];
  __shared__ uint32_t h28_lds[28];
  const int tid = threadIdx.x;
  if (tid < 28) h28_lds[tid] = a.h28mask[tid];
  // zero the second buffer's first two pair-rows and the two rows behind it
  // (read with zero weights before any half has been staged there)
  for (int o = 16 * tid; o < 2 * S::PB; o += 16 * S::kThreads) {
    *reinterpret_cast<u32x4_t*>(lds + S::kRowBytes + o) = u32x4_t{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4_t*>(lds + 2 * S::kRowBytes + o) = u32x4_t{0u, 0u, 0u, 0u};
  }
  DForm form;
  if constexpr (!DVEC) {
    __syncthreads();
    form = DForm{1, a.form_c, a.form_neg};
  } else {
    build_dbits(a.d, a.n, dbits);
    if (tid == 0) scratch[3] = 0;  // the form check's flag
    __syncthreads();
    form = decode_d_form_fast(a, dbits, h28_lds, scratch);
  }
  if (DVEC && __builtin_amdgcn_readfirstlane(form.structured) == 0)
    rq_halves_body<true, YOUT, ZINT, SWIGLU>(a, lds, dbits, h28_lds, form, red, xcl);
  else
    rq_halves_body<false, YOUT, ZINT, SWIGLU>(a, lds, dbits, h28_lds, form, red, xcl);
}

}  // namespace

hipError_t launch_rq_halves(const RqArgs& a, hipStream_t stream) {
  using S = FastShape<28, 9>;
  static std::atomic<int> per_cu_cache{0};
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, rq_halves_kernel<true, false>, S::kThreads, 0) !=
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
  if (a.x2)
    (a.yout ? rq_halves_kernel<false, true, false, true> : rq_halves_kernel<false, false, false, true>)
        <<<blocks, threads, 0, stream>>>(a);
  else if (a.zint)
    rq_halves_kernel<false, false, true><<<blocks, threads, 0, stream>>>(a);
  else if (a.form_given)
    (a.yout ? rq_halves_kernel<false, true> : rq_halves_kernel<false, false>)<<<blocks, threads, 0, stream>>>(a);
  else
    (a.yout ? rq_halves_kernel<true, true> : rq_halves_kernel<true, false>)<<<blocks, threads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace signrot
