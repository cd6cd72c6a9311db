// Device helpers shared by the rotate+quant kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace signrot {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Sign bit (1 = negative) of entry j of sigma * (row c of H), H = H28 (x) H_{2^k}
// or the Sylvester matrix alone.
__device__ __forceinline__ uint32_t hrow_negbit(const RqArgs& a, int c, int j) {
  const int bmask = (1 << a.k) - 1;
  uint32_t bit = __popc(static_cast<uint32_t>(c & j & bmask)) & 1u;
  if (a.m28) bit ^= (a.h28mask[c >> a.k] >> (j >> a.k)) & 1u;
  return bit;
}

// Decide whether the sign vector d (as a bitmask in LDS, bit j set when
// d_j = -1) equals sigma * (row c of H) for some channel c and sign sigma --
// the form calibration produces.  Every thread of the block must call this;
// it returns the same answer in every thread.  Cost: one pass over n bits.
//
// Decoding: over b (the Sylvester index) the row of a Sylvester matrix is the
// character (-1)^popcount(c_b & b), so bit t of c_b is read off the sign
// change between b = 0 and b = 2^t.  Over a (the order-28 index) the row of
// H28 normalised by its first entry is unique, so c_a is found by matching
// the 28 entries d[a' 2^k], again normalised by d[0].  Then every entry is
// checked.
struct DForm {
  int structured;  // 1 if d = sigma * H[c][.]
  int c;           // outlier channel
  int neg;         // 1 if sigma = -1
};

__device__ inline DForm decode_d_form(const RqArgs& a, const uint32_t* dbits, int* sh_scratch) {
  const int tid = threadIdx.x;
  auto dbit = [&](int j) -> uint32_t { return (dbits[j >> 5] >> (j & 31)) & 1u; };
  if (tid == 0) {
    const uint32_t d0 = dbit(0);
    int cb = 0;
    for (int t = 0; t < a.k; ++t)
      if (dbit(1 << t) != d0) cb |= 1 << t;
    int ca = 0;
    int found = 1;
    if (a.m28) {
      found = 0;
      for (int r = 0; r < 28 && !found; ++r) {
        const uint32_t r0 = a.h28mask[r] & 1u;
        int ok = 1;
        for (int ap = 0; ap < 28; ++ap) {
          const uint32_t want = dbit(ap << a.k) ^ d0;
          const uint32_t have = ((a.h28mask[r] >> ap) & 1u) ^ r0;
          if (want != have) { ok = 0; break; }
        }
        if (ok) { ca = r; found = 1; }
      }
    }
    const int c = (ca << a.k) | cb;
    // sigma: d_0 = sigma * H[c][0]
    const uint32_t neg = d0 ^ (a.m28 ? (a.h28mask[ca] & 1u) : 0u);
    sh_scratch[0] = found;
    sh_scratch[1] = c;
    sh_scratch[2] = static_cast<int>(neg);
  }
  __syncthreads();
  DForm f{sh_scratch[0], sh_scratch[1], sh_scratch[2]};
  int bad = 0;
  if (f.structured) {
    for (int j = tid; j < a.n; j += blockDim.x)
      bad |= static_cast<int>(dbit(j) != (hrow_negbit(a, f.c, j) ^ static_cast<uint32_t>(f.neg)));
  }
  bad = __syncthreads_or(bad);
  if (bad) f.structured = 0;
  if (!f.structured) { f.c = -1; f.neg = 0; }
  return f;
}

}  // namespace signrot
