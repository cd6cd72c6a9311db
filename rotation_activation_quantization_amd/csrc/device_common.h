// Device helpers shared by the rotate+quant kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace signrot {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Sign bit (1 = negative) of H_m[r][col] from the mask table (words per row).
__device__ __forceinline__ uint32_t outer_negbit(const uint32_t* hm, int words, int r, int col) {
  return (hm[r * words + (col >> 5)] >> (col & 31)) & 1u;
}

// Sign bit of H_m[r][col] for the outer factor of a: the order-28 row masks
// passed by value (m = 28), else the device mask table.
__device__ __forceinline__ uint32_t args_outer_negbit(const RqArgs& a, int r, int col) {
  if (a.m == 28) return (a.h28mask[r] >> col) & 1u;
  return outer_negbit(a.hm, a.hw, r, col);
}

// Sign bit (1 = negative) of entry j of row c of H, H = H_m (x) H_{2^k} or
// the Sylvester matrix alone (m = 1).
__device__ __forceinline__ uint32_t hrow_negbit(const RqArgs& a, int c, int j) {
  const int bmask = (1 << a.k) - 1;
  uint32_t bit = __popc(static_cast<uint32_t>(c & j & bmask)) & 1u;
  if (a.m > 1) bit ^= args_outer_negbit(a, c >> a.k, j >> a.k);
  return bit;
}

// Decide whether the sign vector d (as a bitmask in LDS, bit j set when
// d_j = -1) equals sigma * (row c of H) for some channel c and sign sigma --
// the form calibration produces.  Every thread of the block must call this;
// it returns the same answer in every thread.  Cost: one pass over n bits.
//
// Decoding: over b (the Sylvester index) the row of a Sylvester matrix is the
// character (-1)^popcount(c_b & b), so bit t of c_b is read off the sign
// change between b = 0 and b = 2^t.  Over a (the outer index) the row of H_m
// normalised by its first entry is unique (the rows are orthogonal), so c_a is
// found by matching the m entries d[a' 2^k], again normalised by d[0]; the
// threads share the candidate rows.  Then every entry is checked.
struct DForm {
  int structured;  // 1 if d = sigma * H[c][.]
  int c;           // outlier channel
  int neg;         // 1 if sigma = -1
};

__device__ inline DForm decode_d_form(const RqArgs& a, const uint32_t* dbits, int* sh_scratch) {
  const int tid = threadIdx.x;
  auto dbit = [&](int j) -> uint32_t { return (dbits[j >> 5] >> (j & 31)) & 1u; };
  // the normalised first column of every block, d[a' 2^k] ^ d[0], as words
  __shared__ uint32_t sh_e[kMaxOuter / 32];
  if (tid == 0) sh_scratch[3] = a.m > 1 ? -1 : 0;
  const uint32_t d0 = dbit(0);
  if (a.m > 1) {
    for (int wd = tid; wd < a.hw; wd += blockDim.x) {
      uint32_t word = 0u;
      for (int b = 0; b < 32; ++b) {
        const int ap = 32 * wd + b;
        if (ap < a.m) word |= (dbit(ap << a.k) ^ d0) << b;
      }
      sh_e[wd] = word;
    }
  }
  __syncthreads();
  if (a.m > 1) {
    // one candidate row per thread, compared a word at a time; the row's
    // words are read without an early exit, so the loads overlap
    for (int r = tid; r < a.m; r += blockDim.x) {
      const uint32_t r0 = args_outer_negbit(a, r, 0) ? 0xffffffffu : 0u;
      uint32_t diff = 0u;
      for (int wd = 0; wd < a.hw; ++wd) {
        const uint32_t valid = (32 * wd + 32 <= a.m) ? 0xffffffffu : ((1u << (a.m - 32 * wd)) - 1u);
        const uint32_t row = (a.m == 28) ? a.h28mask[r] : a.hm[r * a.hw + wd];
        diff |= ((row ^ r0) ^ sh_e[wd]) & valid;
      }
      if (diff == 0u) sh_scratch[3] = r;  // at most one row matches
    }
  }
  __syncthreads();
  if (tid == 0) {
    int cb = 0;
    for (int t = 0; t < a.k; ++t)
      if (dbit(1 << t) != d0) cb |= 1 << t;
    const int found = sh_scratch[3] >= 0;
    const int ca = found ? sh_scratch[3] : 0;
    const int c = (ca << a.k) | cb;
    // sigma: d_0 = sigma * H[c][0]
    const uint32_t neg = d0 ^ (a.m > 1 ? args_outer_negbit(a, ca, 0) : 0u);
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

// Sign bits (bit set when the byte is negative) of 32 consecutive int8
// entries, given as their two 16-byte halves.
__device__ __forceinline__ uint32_t sign_word_of(const uint4& lo, const uint4& hi) {
  const uint32_t q[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t word = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t s = (q[i] >> 7) & 0x01010101u;  // one sign per byte at bits 0, 8, 16, 24
    const uint32_t nib = (s | (s >> 7) | (s >> 14) | (s >> 21)) & 0xfu;
    word |= nib << (4 * i);
  }
  return word;
}

// The same for d[32 w .. 32 w + 31], read as two 16-byte loads.
__device__ __forceinline__ uint32_t sign_word(const int8_t* d32) {
  return sign_word_of(*reinterpret_cast<const uint4*>(d32), *reinterpret_cast<const uint4*>(d32 + 16));
}

// Builds the d bitmask in LDS (n / 32 words; needs n % 32 == 0 and d 16-byte
// aligned) with every thread of the block.
__device__ inline void build_dbits(const int8_t* d, int n, uint32_t* dbits) {
  for (int w = threadIdx.x; w < n / 32; w += blockDim.x) dbits[w] = sign_word(d + 32 * w);
}

// Same decision as decode_d_form, in parallel, for k >= 5 (a 32-bit word of
// the mask then lies inside one block of 2^k channels).  h28 holds the row
// masks of H28 in LDS.  Every thread of the block must call it, after a
// barrier that published the whole bitmask; before that barrier the caller
// sets sh_scratch[3] = 0 (the flag a thread raises when an entry is off the
// form).  Each wave decides the candidate form itself from the bitmask, so
// only one more barrier follows.  THREADS: the block size when the caller
// knows it at compile time (else 0: blockDim.x).
template <int THREADS = 0>
__device__ inline DForm decode_d_form_fast(const RqArgs& a, const uint32_t* dbits, const uint32_t* h28,
                                           int* sh_scratch) {
  const int nthreads = THREADS > 0 ? THREADS : static_cast<int>(blockDim.x);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  auto dbit = [&](int j) -> uint32_t { return (dbits[j >> 5] >> (j & 31)) & 1u; };
  const uint32_t d0 = dbit(0);
  // bit t of c_b: sign change between b = 0 and b = 2^t (first block)
  const unsigned long long cbm = __ballot(lane < a.k && dbit(1 << lane) != d0);
  const int cb = static_cast<int>(cbm & ((1ull << a.k) - 1ull));
  int ca = 0, found = 1;
  if (a.m28) {
    // normalised first column of each block against each normalised H28 row
    const unsigned long long em = __ballot(lane < 28 && (dbit(lane << a.k) ^ d0) != 0u);
    const uint32_t e = static_cast<uint32_t>(em);
    uint32_t norm = 0xffffffffu;
    if (lane < 28) {
      const uint32_t m = h28[lane];
      norm = (m & 1u) ? (~m & 0x0fffffffu) : m;
    }
    const unsigned long long hit = __ballot(lane < 28 && norm == e);
    found = hit != 0ull;
    ca = found ? __builtin_ctzll(hit) : 0;
  }
  DForm f{found, (ca << a.k) | cb, static_cast<int>(d0 ^ (a.m28 ? (h28[ca] & 1u) : 0u))};
  if (f.structured) {
    const int bmask = (1 << a.k) - 1;
    // parity(cb & i) for i = 0..31, as a word: the XOR of the index-bit
    // patterns of the set bits of cb & 31
    uint32_t pw = 0u;
    if (cb & 1) pw ^= 0xAAAAAAAAu;
    if (cb & 2) pw ^= 0xCCCCCCCCu;
    if (cb & 4) pw ^= 0xF0F0F0F0u;
    if (cb & 8) pw ^= 0xFF00FF00u;
    if (cb & 16) pw ^= 0xFFFF0000u;
    for (int w = tid; w < a.n / 32; w += nthreads) {
      const int j0 = 32 * w;
      uint32_t flip = static_cast<uint32_t>(f.neg) ^ (__popc(static_cast<uint32_t>(cb & j0 & bmask)) & 1u);
      if (a.m28) flip ^= (h28[ca] >> (j0 >> a.k)) & 1u;
      const uint32_t want = flip ? ~pw : pw;
      if (dbits[w] != want) sh_scratch[3] = 1;  // every writer stores the same value
    }
  }
  // (a plain flag in LDS rather than __syncthreads_or, whose group-size
  // lookup waits for every outstanding global load)
  __syncthreads();
  if (sh_scratch[3]) f.structured = 0;
  if (!f.structured) {
    f.c = -1;
    f.neg = 0;
  }
  return f;
}

}  // namespace signrot
