// Generic rotate + sign flip + per-token asymmetric INT4 kernel.
//
// One workgroup per token row (persistent: a workgroup walks rows with a grid
// stride).  The row is widened to binary32 in LDS; the order-28 mix (when
// n = 28 * 2^k) runs column by column, one thread per column b, in LDS; a
// mix of another outer order m (n = m * 2^k, H_m a Paley matrix) reads the
// bf16 row from global memory and writes the mixed row to LDS, 16 outputs per
// work item; the 2^k Walsh-Hadamard transform runs as radix-2 butterfly
// passes over LDS with a barrier between passes; the flip, the min/max
// reduction, the quantizer and the nibble packing follow.  It handles every
// supported n and is the HIP path for the shapes that have no specialised
// kernel.
//
// Method: explainer "SignRot for 4-bit LLM quantization -- Sign-adjusted
// Hadamard rotation", paragraphs on rotation (entries +-1/sqrt(n), fast
// Walsh-Hadamard transform), on the sign adjustment (the flip of the columns
// of H) and on the quantizer (16 levels from min to max, nearest level).
#include <math.h>

#include "device_common.h"

namespace signrot {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxN = 32768;

__device__ inline float block_reduce_min(float v, float* sh) {
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fminf(r, sh[i]);
  __syncthreads();
  return r;
}

__device__ inline float block_reduce_max(float v, float* sh) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fmaxf(r, sh[i]);
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void rq_generic_kernel(RqArgs a) {
  extern __shared__ float row[];  // n floats
  __shared__ uint32_t dbits[kMaxN / 32];
  __shared__ float red[16];
  __shared__ int scratch[4];
  __shared__ float s_xc;

  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int n = a.n;
  const int B = 1 << a.k;

  // d as a bitmask (bit set = -1)
  for (int w = tid; w < (n + 31) / 32; w += nt) {
    uint32_t bits = 0;
    for (int i = 0; i < 32 && w * 32 + i < n; ++i)
      bits |= static_cast<uint32_t>(a.d[w * 32 + i] < 0) << i;
    dbits[w] = bits;
  }
  __syncthreads();
  const DForm form = decode_d_form(a, dbits, scratch);

  // Outer orders other than 28 mix straight from the bf16 row in global
  // memory (the mix writes every entry of the LDS row, so no copy is needed).
  const bool outer_general = a.m > 1 && !a.m28;

  for (int64_t t = blockIdx.x; t < a.tokens; t += gridDim.x) {
    const uint16_t* xr = a.x + t * a.ld;
    if (outer_general) {
      // nothing to widen
    } else if ((n & 7) == 0) {
      for (int i = tid * 8; i < n; i += nt * 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(xr + i);
        row[i + 0] = bf16_lo(v.x); row[i + 1] = bf16_hi(v.x);
        row[i + 2] = bf16_lo(v.y); row[i + 3] = bf16_hi(v.y);
        row[i + 4] = bf16_lo(v.z); row[i + 5] = bf16_hi(v.z);
        row[i + 6] = bf16_lo(v.w); row[i + 7] = bf16_hi(v.w);
      }
    } else {
      for (int i = tid; i < n; i += nt) row[i] = __uint_as_float(static_cast<uint32_t>(xr[i]) << 16);
    }
    __syncthreads();
    // SignRot form: take the outlier channel out of the transform; its
    // contribution after the flip is the constant sigma * x_c.
    if (form.structured && tid == 0) {
      if (outer_general) {
        s_xc = __uint_as_float(static_cast<uint32_t>(xr[form.c]) << 16);
      } else {
        s_xc = row[form.c];
        row[form.c] = 0.0f;
      }
    }
    __syncthreads();
    const float xc = form.structured ? s_xc : 0.0f;

    if (a.m28) {
      // Z[a'][b] = sum_a H28[a][a'] X[a][b]
      for (int b = tid; b < B; b += nt) {
        float v[28];
#pragma unroll
        for (int r = 0; r < 28; ++r) v[r] = row[r * B + b];
        float out[28];
#pragma unroll
        for (int ap = 0; ap < 28; ++ap) out[ap] = 0.0f;
#pragma unroll
        for (int r = 0; r < 28; ++r) {
          const uint32_t m = a.h28mask[r];
#pragma unroll
          for (int ap = 0; ap < 28; ++ap) out[ap] += ((m >> ap) & 1u) ? -v[r] : v[r];
        }
#pragma unroll
        for (int ap = 0; ap < 28; ++ap) row[ap * B + b] = out[ap];
      }
      __syncthreads();
    } else if (outer_general) {
      // Z[a'][b] = sum_a H_m[a][a'] X[a][b], 16 consecutive a' per work item;
      // the outlier entry (when d has the SignRot form) counts as zero.
      const int groups = (a.m + 15) >> 4;
      const int skip = form.structured ? form.c : -1;
      for (int it = tid; it < groups * B; it += nt) {
        const int ap0 = (it / B) << 4;
        const int b = it - (it / B) * B;
        float acc[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = 0.0f;
        for (int r = 0; r < a.m; ++r) {
          const int idx = r * B + b;
          const float v = idx == skip ? 0.0f : __uint_as_float(static_cast<uint32_t>(xr[idx]) << 16);
          const uint32_t sg = a.hm[r * a.hw + (ap0 >> 5)] >> (ap0 & 31);
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[j] += ((sg >> j) & 1u) ? -v : v;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (ap0 + j < a.m) row[(ap0 + j) * B + b] = acc[j];
      }
      __syncthreads();
    }

    // Walsh-Hadamard transform over b inside each block of 2^k
    for (int h = 1; h < B; h <<= 1) {
      for (int p = tid; p < n / 2; p += nt) {
        const int i0 = ((p & ~(h - 1)) << 1) | (p & (h - 1));
        const float u = row[i0], w = row[i0 + h];
        row[i0] = u + w;
        row[i0 + h] = u - w;
      }
      __syncthreads();
    }

    // flip, min, max (unnormalised domain)
    float lmin = INFINITY, lmax = -INFINITY;
    for (int j = tid; j < n; j += nt) {
      float u = row[j];
      if ((dbits[j >> 5] >> (j & 31)) & 1u) u = -u;
      row[j] = u;
      lmin = fminf(lmin, u);
      lmax = fmaxf(lmax, u);
    }
    const float mn = block_reduce_min(lmin, red);
    const float mx = block_reduce_max(lmax, red);
    const float range = mx - mn;
    const bool degenerate = !(range > 0.0f);
    const float inv = degenerate ? 0.0f : 15.0f / range;

    const float shift = form.neg ? -xc : xc;
    const float s = degenerate ? 1.0f : range * a.inv_15sqrt_n;
    const float mn_y = (mn + shift) * a.inv_sqrt_n;
    // integer zero-point: z = rint(-mn_y / s), code = clamp(rint((u + shift) * inv + z), 0, 15)
    const float zq = rintf(-mn_y / s);
    uint8_t* crow = a.codes + t * (n / 2);
    if (a.zint) {
      const float off = degenerate ? 0.0f : fmaf(shift, inv, zq);
      for (int m = tid; m < n / 2; m += nt) {
        const float q0 = fminf(fmaxf(rintf(fmaf(row[2 * m], inv, off)), 0.0f), 15.0f);
        const float q1 = fminf(fmaxf(rintf(fmaf(row[2 * m + 1], inv, off)), 0.0f), 15.0f);
        crow[m] = static_cast<uint8_t>(static_cast<uint32_t>(q0) | (static_cast<uint32_t>(q1) << 4));
      }
    } else {
      for (int m = tid; m < n / 2; m += nt) {
        const float q0 = fminf(fmaxf(rintf((row[2 * m] - mn) * inv), 0.0f), 15.0f);
        const float q1 = fminf(fmaxf(rintf((row[2 * m + 1] - mn) * inv), 0.0f), 15.0f);
        crow[m] = static_cast<uint8_t>(static_cast<uint32_t>(q0) | (static_cast<uint32_t>(q1) << 4));
      }
    }
    if (a.yout) {
      float* yr = a.yout + t * n;
      for (int j = tid; j < n; j += nt) yr[j] = (row[j] + shift) * a.inv_sqrt_n;
    }
    if (tid == 0) {
      a.scale[t] = s;
      a.zero[t] = a.zint ? zq : -mn_y / s;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_rq_generic(const RqArgs& a, hipStream_t s) {
  const size_t lds = static_cast<size_t>(a.n) * sizeof(float);
  static thread_local bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&rq_generic_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
    attr_set = true;
  }
  // LDS per block ~ 4n + 4 KiB; at most 160 KiB per CU.
  const size_t per_block = lds + kMaxN / 8 + 256;
  int per_cu = static_cast<int>((160 * 1024) / per_block);
  if (per_cu < 1) per_cu = 1;
  if (per_cu > 8) per_cu = 8;
  int64_t grid = static_cast<int64_t>(device_cu_count()) * per_cu;
  if (grid > a.tokens) grid = a.tokens;
  hipLaunchKernelGGL(rq_generic_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

const char* rq_generic_name() { return "rq_generic"; }

}  // namespace signrot
