// Internal declarations of libsignrot (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

namespace signrot {

// Factorisation n = m * 2^k (n <= 32768): m = 1 for n = 2^k (k >= 1);
// otherwise n = o * 2^v with o odd and m = o * 2^j, the smallest j >= 2 for
// which a Paley matrix of order m <= kMaxOuter exists (m = 28 for o = 7).
constexpr int kMaxOuter = 512;
struct Shape {
  int n = 0;
  int k = 0;
  int m = 1;
  bool m28 = false;  // m == 28: the order-28 kernels and h28()
  bool ok = false;
};
Shape factor_n(int64_t n);

// Outer factors other than order 28's hand-built table: Paley's
// constructions I and II (outer.cpp).  outer_order_for returns m or 0;
// outer_table returns the cached host table (nullptr when no construction);
// mask[r * words + w] has bit b set iff H_m[r][32 w + b] == -1; mask_t is
// the same for the transpose (mask_t[r * words + w] bit b: H_m[32 w + b][r]).
struct OuterTable {
  int m = 0;
  int words = 0;
  std::vector<int8_t> h;  // m x m, row-major
  std::vector<uint32_t> mask;
  std::vector<uint32_t> mask_t;
};
int outer_order_for(int odd, int v);
const OuterTable* outer_table(int m);
// H_m (x) Syl_{2^j} as one outer factor of order m 2^j <= kMaxOuter (m = 1:
// the Sylvester matrix; m = 28: the order-28 table; else Paley): the same H
// read with j Sylvester index bits moved into the outer index.
const OuterTable* outer_table_folded(int m, int j);
// The mask table of H_m on the current device: copied there on first use
// (hipMalloc + hipMemcpy) and kept until the process ends, at most 32 KiB per
// table.  The first use cannot be captured into a graph: when `stream` is
// capturing and the table is not there yet, this returns nullptr with
// *err = hipErrorStreamCaptureUnsupported and leaves the capture intact.
// nullptr (with *err set) on any failure.  transposed: the table of H_m^T;
// fold: of H_m (x) Syl_{2^fold} (outer_table_folded).
const uint32_t* outer_mask_device(int m, hipError_t* err, hipStream_t stream, bool transposed = false,
                                  int fold = 0);

// The library's order-28 Hadamard matrix (Paley construction I over GF(27)),
// built once on the host.  rowmask[a] has bit a' set iff H28[a][a'] == -1.
struct H28Table {
  int8_t h[28][28];
  uint32_t rowmask[28];
};
const H28Table& h28();

// H28 row masks by value (a kernel argument).
struct H28Masks {
  uint32_t m[28];
};
H28Masks h28_masks();

// Everything a rotate+quant kernel needs, passed by value as the kernel
// argument block.
struct RqArgs {
  const uint16_t* x;   // bf16 bits, [tokens][ld] (SwiGLU entry point: the gate)
  const uint16_t* x2;  // SwiGLU entry point: up, bf16 bits [tokens][ld] (x = bf16(SiLU(gate) * up)); else null
  const int8_t* d;     // [n], +-1
  uint8_t* codes;      // [tokens][n/2]
  float* scale;        // [tokens]
  float* zero;         // [tokens]
  float* yout;         // [tokens][n] or nullptr
  int64_t tokens;
  int64_t ld;
  int n;
  int k;
  int m28;
  float inv_sqrt_n;    // binary32(1 / sqrt(n))
  float inv_15sqrt_n;  // binary32(1 / (15 sqrt(n)))
  int form_given;      // 1: d = sigma * (row form_c of H) is given by (form_c, form_neg); d unused
  int form_c;
  int form_neg;        // 1 when sigma = -1
  int zint;            // 1: integer zero-point z = rint(-mn / s), q = clamp(rint(y / s) + z, 0, 15)
  uint32_t h28mask[28];
  int m;                 // outer order (1: none)
  int hw;                // 32-bit words per mask row of H_m
  const uint32_t* hm;    // device mask table of H_m (m > 1), see OuterTable
  const uint32_t* hmt;   // device mask table of H_m^T (set for the outer-order MFMA kernel)
};

// Launchers; each returns the hipError_t of the launch.
hipError_t launch_rq_generic(const RqArgs& a, hipStream_t s);
const char* rq_generic_name();
bool rq_fast_supports(int n, int k, bool m28);
hipError_t launch_rq_fast(const RqArgs& a, hipStream_t s);
const char* rq_fast_name(int n);
// MFMA kernel for outer orders m (multiples of 4 up to 512) with
// 16 <= 2^k <= 256 (shapes in its table); rq_outer_supports is host-only.
bool rq_outer_supports(int m, int k);
hipError_t launch_rq_outer(const RqArgs& a, hipStream_t s);
const char* rq_outer_name();

// The calibration argmax record in static device memory (two 64-bit words:
// key, M_c bits): its address on the current device, looked up once per
// device with hipGetSymbolAddress.  nullptr (with *err set) on failure.
constexpr int kCalScratchWords = 2;
unsigned long long* calib_scratch_device(hipError_t* err);

hipError_t launch_calibrate(const uint16_t* x, int64_t tokens, int64_t ld, const Shape& sh,
                            int8_t* d_out, unsigned long long* scratch, hipStream_t s);
// d[j] = sigma * H[c][j] as int8 +-1 (the calibrated form from (c, sigma)).
hipError_t launch_sign_fill(const Shape& sh, int c, int neg, int8_t* d, hipStream_t s);
hipError_t launch_dequant(const uint8_t* codes, const float* scale, const float* zero,
                          int64_t tokens, int n, float* y, hipStream_t s);

// The memory-traffic ceiling kernel (same bytes per token as the rotate
// kernels, no arithmetic): x [tokens][ld] bf16, n % 8 == 0.
hipError_t launch_stream_ceiling(const uint16_t* x, int64_t tokens, int n, int64_t ld, uint8_t* out, float* s0,
                                 float* s1, hipStream_t s);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// The consumer GEMM: out[t][k] = scale[t] * (sum_j q[t][j] w[k][j] - zero[t] * rowsum[k]).
struct LinearArgs {
  const uint8_t* codes;  // [T][n/2], packed as signrot_rotate_quant_int4 writes them
  const float* scale;    // [T]
  const float* zero;     // [T]
  const uint16_t* w;     // bf16 bits, [R][ldw]
  const float* rowsum;   // [R]
  float* out;            // [T][R]
  int64_t ldw;
  int T;
  int R;
  int n;
  int tiles_m;  // set by the launcher
  int tiles_n;
};
bool int4_linear_fast_ok(const LinearArgs& a);
const char* int4_linear_name(const LinearArgs& a);
hipError_t launch_int4_linear(LinearArgs a, hipStream_t s);
hipError_t launch_weight_rowsum(const uint16_t* w, int64_t rows, int64_t n, int64_t ld, float* rowsum,
                                hipStream_t s);

}  // namespace signrot
