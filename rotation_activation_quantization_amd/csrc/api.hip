// C ABI of libsignrot: argument validation, dispatch and error reporting.
// Every check happens on the host before any HIP call; a failing HIP call is
// reported as SIGNROT_EHIP with its message kept per thread.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/signrot.h"
#include "internal.h"

namespace signrot {

namespace {

thread_local char g_last_error[512] = "";

void set_error(const char* fmt, const char* detail) {
  snprintf(g_last_error, sizeof(g_last_error), fmt, detail);
}

int fail_einval(const char* what) {
  set_error("invalid argument: %s", what);
  return SIGNROT_EINVAL;
}

int fail_hip(hipError_t e, const char* where) {
  char buf[400];
  snprintf(buf, sizeof(buf), "%s: %s (%d)", where, hipGetErrorString(e), static_cast<int>(e));
  set_error("%s", buf);
  return SIGNROT_EHIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

Shape factor_n(int64_t n) {
  Shape s;
  if (n < 2 || n > 32768) return s;
  int64_t o = n;
  int v = 0;
  while ((o & 1) == 0) {
    o >>= 1;
    ++v;
  }
  int m = 1;
  if (o > 1) {
    m = outer_order_for(static_cast<int>(o), v);
    if (m == 0) return s;
  }
  const int64_t p = n / m;
  int k = 0;
  while ((int64_t{1} << k) < p) ++k;
  if (m == 1 && k < 1) return s;
  s.n = static_cast<int>(n);
  s.k = k;
  s.m = m;
  s.m28 = (m == 28);
  s.ok = true;
  return s;
}

const uint32_t* outer_mask_device(int m, hipError_t* err, hipStream_t stream, bool transposed, int fold) {
  *err = hipSuccess;
  static std::mutex mu;
  static std::vector<std::vector<std::pair<int, uint32_t*>>> per_dev;
  int dev = 0;
  if ((*err = hipGetDevice(&dev)) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= static_cast<int>(per_dev.size())) per_dev.resize(dev + 1);
  const int key = ((m * 16 + fold) * 2) + (transposed ? 1 : 0);
  for (auto& e : per_dev[dev])
    if (e.first == key) return e.second;
  // the copy below would break a stream capture: refuse instead
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if ((*err = hipStreamIsCapturing(stream, &cap)) != hipSuccess) return nullptr;
  if (cap != hipStreamCaptureStatusNone) {
    *err = hipErrorStreamCaptureUnsupported;
    return nullptr;
  }
  std::vector<uint32_t> mask;
  if (fold > 0) {
    const OuterTable* t = outer_table_folded(m, fold);
    if (!t) {
      *err = hipErrorInvalidValue;
      return nullptr;
    }
    mask = transposed ? t->mask_t : t->mask;
  } else if (m == 28) {  // h28(): one word per row
    if (transposed) {
      mask.assign(28, 0u);
      for (int r = 0; r < 28; ++r)
        for (int c = 0; c < 28; ++c)
          if (h28().h[r][c] < 0) mask[c] |= 1u << r;
    } else {
      mask.assign(h28().rowmask, h28().rowmask + 28);
    }
  } else {
    const OuterTable* t = outer_table(m);
    if (!t) {
      *err = hipErrorInvalidValue;
      return nullptr;
    }
    mask = transposed ? t->mask_t : t->mask;
  }
  uint32_t* ptr = nullptr;
  if ((*err = hipMalloc(&ptr, mask.size() * sizeof(uint32_t))) != hipSuccess) return nullptr;
  if ((*err = hipMemcpy(ptr, mask.data(), mask.size() * sizeof(uint32_t), hipMemcpyHostToDevice)) != hipSuccess) {
    (void)hipFree(ptr);
    return nullptr;
  }
  per_dev[dev].push_back({key, ptr});
  return ptr;
}

// The rotate kernel for a shape: the 28 * 2^k / 2^k MFMA kernels, the
// outer-order MFMA kernel, or the generic one.  The outer-order kernel also
// takes n = m 2^k read as (m 2^fold) 2^(k - fold): the same H with fold
// Sylvester index bits moved into its outer factor, for 2^k >= 256 or a
// Sylvester width without a fast kernel.  2^(k - fold) = 128 comes first,
// then 256 (fold 0 when 2^k = 256), 32, 64, 16.  Measured at 8192 tokens, a
// 2^k = 256 width read with 128 columns ran 1.1-1.9x faster (3072, 5120,
// 13312-21504), except where that reading has 3 K chunks (65 <= 2m <= 96):
// 9216 and 11264 ran 11 % slower.  Such a plan is therefore taken only when
// no later one fits.
enum class RqKernel { kFast, kOuter, kGeneric };
struct RqPlan {
  RqKernel kind;
  int fold;
};

RqPlan rq_plan_for(const Shape& sh) {
  if (rq_fast_supports(sh.n, sh.k, sh.m28)) return {RqKernel::kFast, 0};
  if (sh.k != 8 && rq_outer_supports(sh.m, sh.k)) return {RqKernel::kOuter, 0};
  if (sh.m == 1 || (sh.m != 28 && sh.k >= 8)) {
    RqPlan kept{RqKernel::kGeneric, 0};
    for (const int kk : {7, 8, 5, 6, 4}) {
      const int fold = sh.k - kk;
      if (fold < (sh.m == 1 ? 2 : 0)) continue;
      const int64_t mm = static_cast<int64_t>(sh.m) << fold;
      if (mm > kMaxOuter || !rq_outer_supports(static_cast<int>(mm), kk)) continue;
      const RqPlan p{RqKernel::kOuter, fold};
      if (kk == 7 && (mm + 31) / 32 == 3) {
        if (kept.kind == RqKernel::kGeneric) kept = p;
        continue;
      }
      return p;
    }
    return kept;
  }
  return {RqKernel::kGeneric, 0};
}

RqKernel rq_kernel_for(const Shape& sh) { return rq_plan_for(sh).kind; }

// Fills the outer-factor fields of a (the device sign tables it needs); with
// a fold, also the outer order and Sylvester exponent the kernel sees.  Every
// kernel takes H28 by value (h28mask) and reads no table for m = 28, so those
// widths never allocate one; other outer orders read a per-device table that
// is copied there on a device's first call and kept.
hipError_t set_outer_tables(RqArgs& a, const Shape& sh, hipStream_t s) {
  hipError_t he = hipSuccess;
  const RqPlan p = rq_plan_for(sh);
  a.m = sh.m << p.fold;
  a.k = sh.k - p.fold;
  a.hw = (a.m + 31) / 32;
  a.hm = nullptr;
  a.hmt = nullptr;
  if (a.m > 1 && a.m != 28 && p.kind != RqKernel::kFast) {
    if (!(a.hm = outer_mask_device(sh.m, &he, s, false, p.fold))) return he;
    if (p.kind == RqKernel::kOuter && !(a.hmt = outer_mask_device(sh.m, &he, s, true, p.fold))) return he;
  }
  return hipSuccess;
}

hipError_t launch_rq(const RqArgs& a, const Shape& sh, hipStream_t s) {
  switch (rq_kernel_for(sh)) {
    case RqKernel::kFast: return launch_rq_fast(a, s);
    case RqKernel::kOuter: return launch_rq_outer(a, s);
    default: return launch_rq_generic(a, s);
  }
}

int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= static_cast<int>(cache.size())) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

}  // namespace signrot

using namespace signrot;

extern "C" {

int signrot_supported_n(int64_t n) { return factor_n(n).ok ? 1 : 0; }

const char* signrot_strerror(int status) {
  switch (status) {
    case SIGNROT_OK: return "ok";
    case SIGNROT_EINVAL: return "invalid argument";
    case SIGNROT_EUNSUPPORTED_N:
      return "unsupported n (need n <= 32768, n = 2^k with k >= 1, or n = m * 2^k with m = o * 2^j the smallest "
             "Paley order <= 512 for the odd part o of n)";
    case SIGNROT_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* signrot_last_error(void) { return g_last_error; }

int signrot_debug_h28(int8_t* out) {
  if (!out) return fail_einval("out is NULL");
  memcpy(out, h28().h, 28 * 28);
  return SIGNROT_OK;
}

int signrot_outer_order(int64_t n) {
  const Shape sh = factor_n(n);
  return sh.ok ? sh.m : 0;
}

int signrot_debug_outer(int m, int8_t* out) {
  g_last_error[0] = '\0';
  if (!out) return fail_einval("out is NULL");
  if (m == 28) {
    memcpy(out, h28().h, 28 * 28);
    return SIGNROT_OK;
  }
  if (m < 2 || m > kMaxOuter) return fail_einval("m out of range");
  const OuterTable* t = outer_table(m);
  if (!t) return fail_einval("no Paley construction of order m");
  memcpy(out, t->h.data(), static_cast<size_t>(m) * m);
  return SIGNROT_OK;
}

int signrot_debug_outer_folded(int m, int fold, int8_t* out) {
  g_last_error[0] = '\0';
  if (!out) return fail_einval("out is NULL");
  if (m < 1 || fold < 0 || fold > 9 || (static_cast<int64_t>(m) << fold) > kMaxOuter)
    return fail_einval("m * 2^fold out of range");
  const OuterTable* t = outer_table_folded(m, fold);
  if (!t) return fail_einval("no construction of H_m (x) Syl_{2^fold}");
  memcpy(out, t->h.data(), static_cast<size_t>(t->m) * t->m);
  return SIGNROT_OK;
}

int signrot_outer_fold(int64_t n) {
  const Shape sh = factor_n(n);
  return sh.ok ? rq_plan_for(sh).fold : -1;
}

const char* signrot_kernel_name(int64_t n) {
  const Shape sh = factor_n(n);
  if (!sh.ok) return nullptr;
  switch (rq_kernel_for(sh)) {
    case RqKernel::kFast: return rq_fast_name(sh.n);
    case RqKernel::kOuter: return rq_outer_name();
    default: return rq_generic_name();
  }
}

}  // extern "C"

namespace {
int calibrate_check(const Shape& sh, const void* x_bf16, int64_t tokens, int64_t n, int64_t ld, const int8_t* d_out) {
  if (!sh.ok) {
    set_error("unsupported n=%s", std::to_string(n).c_str());
    return SIGNROT_EUNSUPPORTED_N;
  }
  if (tokens <= 0) return fail_einval("calibration needs tokens >= 1");
  if (tokens >= (int64_t{1} << 28)) return fail_einval("tokens must be < 2^28");
  if (!x_bf16 || !d_out) return fail_einval("null device pointer");
  if (ld < n) return fail_einval("ld < n");
  if (!aligned16(x_bf16) || (ld & 7)) return fail_einval("x must be 16-byte aligned and ld a multiple of 8");
  return SIGNROT_OK;
}

// Decodes the argmax record (already on the host) into the outputs.
void calibrate_outputs(const unsigned long long host[2], int32_t* c_out, int64_t* t_out, float* mc_out) {
  const unsigned long long key = host[0];
  const int c = static_cast<int>(0xfffffu - static_cast<uint32_t>((key >> 28) & 0xfffffu));
  const int64_t t = static_cast<int64_t>(0x0fffffffu - static_cast<uint32_t>(key & 0x0fffffffu));
  const uint32_t mbits = static_cast<uint32_t>(host[1]) << 16;
  float m;
  memcpy(&m, &mbits, sizeof(m));
  if (c_out) *c_out = c;
  if (t_out) *t_out = t;
  if (mc_out) *mc_out = m;
}
}  // namespace

extern "C" {

int signrot_calibrate(const void* x_bf16, int64_t tokens, int64_t n, int64_t ld, int8_t* d_out,
                      int32_t* c_out, int64_t* t_out, float* mc_out, void* stream) {
  g_last_error[0] = '\0';
  const Shape sh = factor_n(n);
  const int st = calibrate_check(sh, x_bf16, tokens, n, ld, d_out);
  if (st != SIGNROT_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned long long* scratch = nullptr;
  hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&scratch), 16, s);
  if (e != hipSuccess) return fail_hip(e, "hipMallocAsync");
  e = launch_calibrate(static_cast<const uint16_t*>(x_bf16), tokens, ld, sh, d_out, scratch, s);
  unsigned long long host[2] = {0ull, 0ull};
  if (e == hipSuccess) e = hipMemcpyAsync(host, scratch, sizeof(host), hipMemcpyDeviceToHost, s);
  hipError_t ef = hipFreeAsync(scratch, s);
  if (e == hipSuccess) e = ef;
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail_hip(e, "calibrate");
  calibrate_outputs(host, c_out, t_out, mc_out);
  return SIGNROT_OK;
}

int signrot_calibrate_noalloc(const void* x_bf16, int64_t tokens, int64_t n, int64_t ld, int8_t* d_out,
                              int32_t* c_out, int64_t* t_out, float* mc_out, void* stream) {
  g_last_error[0] = '\0';
  const Shape sh = factor_n(n);
  const int st = calibrate_check(sh, x_bf16, tokens, n, ld, d_out);
  if (st != SIGNROT_OK) return st;
  if (sh.m != 1 && sh.m != 28) {
    set_error("n=%s needs the device table of its outer Hadamard factor, which only signrot_calibrate may "
              "allocate (the allocation-free call takes n = 2^k and n = 28 * 2^k)",
              std::to_string(n).c_str());
    return SIGNROT_EUNSUPPORTED_N;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  unsigned long long* rec = calib_scratch_device(&e);
  if (!rec) return fail_hip(e, "hipGetSymbolAddress(scratch)");
  e = launch_calibrate(static_cast<const uint16_t*>(x_bf16), tokens, ld, sh, d_out, rec, s);
  unsigned long long host[2] = {0ull, 0ull};
  if (e == hipSuccess) e = hipMemcpyAsync(host, rec, sizeof(host), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail_hip(e, "calibrate_noalloc");
  calibrate_outputs(host, c_out, t_out, mc_out);
  return SIGNROT_OK;
}

int signrot_rotate_quant_int4(const void* x_bf16, int64_t tokens, int64_t n, int64_t ld, const int8_t* d,
                              uint8_t* codes, float* scale, float* zero, float* y_out, void* stream) {
  g_last_error[0] = '\0';
  const Shape sh = factor_n(n);
  if (!sh.ok) {
    set_error("unsupported n=%s", std::to_string(n).c_str());
    return SIGNROT_EUNSUPPORTED_N;
  }
  if (tokens < 0) return fail_einval("tokens < 0");
  if (ld < n) return fail_einval("ld < n");
  if (ld & 7) return fail_einval("ld must be a multiple of 8");
  if (tokens == 0) return SIGNROT_OK;
  if (tokens > (int64_t{1} << 40)) return fail_einval("tokens too large");
  if (!x_bf16 || !d || !codes || !scale || !zero) return fail_einval("null device pointer");
  if (!aligned16(x_bf16)) return fail_einval("x must be 16-byte aligned");
  if (!aligned16(d)) return fail_einval("d must be 16-byte aligned");
  if (!aligned16(codes)) return fail_einval("codes must be 16-byte aligned");
  if (y_out && !aligned16(y_out)) return fail_einval("y_out must be 16-byte aligned");
  RqArgs a;
  memset(&a, 0, sizeof(a));
  a.x = static_cast<const uint16_t*>(x_bf16);
  a.d = d;
  a.codes = codes;
  a.scale = scale;
  a.zero = zero;
  a.yout = y_out;
  a.tokens = tokens;
  a.ld = ld;
  a.n = sh.n;
  a.k = sh.k;
  a.m28 = sh.m28 ? 1 : 0;
  a.inv_sqrt_n = static_cast<float>(1.0 / sqrt(static_cast<double>(n)));
  a.inv_15sqrt_n = static_cast<float>(1.0 / (15.0 * sqrt(static_cast<double>(n))));
  for (int i = 0; i < 28; ++i) a.h28mask[i] = h28().rowmask[i];
  {
    const hipError_t he = set_outer_tables(a, sh, static_cast<hipStream_t>(stream));
    if (he != hipSuccess) return fail_hip(he, "outer Hadamard factor table");
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_rq(a, sh, st);
  if (e != hipSuccess) return fail_hip(e, "rotate_quant_int4 launch");
  return SIGNROT_OK;
}

}  // extern "C"

namespace {
int rotate_quant_outlier_impl(const void* x_bf16, int64_t tokens, int64_t n, int64_t ld, int64_t c, int sigma,
                              uint8_t* codes, float* scale, float* zero, float* y_out, int zint, void* stream,
                              const void* up_bf16 = nullptr) {
  g_last_error[0] = '\0';
  const Shape sh = factor_n(n);
  if (!sh.ok) {
    set_error("unsupported n=%s", std::to_string(n).c_str());
    return SIGNROT_EUNSUPPORTED_N;
  }
  if (up_bf16 && rq_kernel_for(sh) != RqKernel::kFast) {
    set_error("n=%s: the fused SwiGLU producer runs on the fast widths only (3584, 7168, 14336, 28672, 4096, 8192, "
              "16384)", std::to_string(n).c_str());
    return SIGNROT_EUNSUPPORTED_N;
  }
  if (c < 0 || c >= n) return fail_einval("c must be a channel in [0, n)");
  if (sigma != 1 && sigma != -1) return fail_einval("sigma must be +1 or -1");
  if (tokens < 0) return fail_einval("tokens < 0");
  if (ld < n) return fail_einval("ld < n");
  if (ld & 7) return fail_einval("ld must be a multiple of 8");
  if (tokens == 0) return SIGNROT_OK;
  if (tokens > (int64_t{1} << 40)) return fail_einval("tokens too large");
  if (!x_bf16 || !codes || !scale || !zero) return fail_einval("null device pointer");
  if (!aligned16(x_bf16)) return fail_einval("x must be 16-byte aligned");
  if (!aligned16(codes)) return fail_einval("codes must be 16-byte aligned");
  if (y_out && !aligned16(y_out)) return fail_einval("y_out must be 16-byte aligned");
  if (up_bf16 && !aligned16(up_bf16)) return fail_einval("up must be 16-byte aligned");
  RqArgs a;
  memset(&a, 0, sizeof(a));
  a.x = static_cast<const uint16_t*>(x_bf16);
  a.x2 = static_cast<const uint16_t*>(up_bf16);
  a.codes = codes;
  a.scale = scale;
  a.zero = zero;
  a.yout = y_out;
  a.tokens = tokens;
  a.ld = ld;
  a.n = sh.n;
  a.k = sh.k;
  a.m28 = sh.m28 ? 1 : 0;
  a.inv_sqrt_n = static_cast<float>(1.0 / sqrt(static_cast<double>(n)));
  a.inv_15sqrt_n = static_cast<float>(1.0 / (15.0 * sqrt(static_cast<double>(n))));
  a.form_given = 1;
  a.form_c = static_cast<int>(c);
  a.form_neg = sigma < 0 ? 1 : 0;
  a.zint = zint;
  for (int i = 0; i < 28; ++i) a.h28mask[i] = h28().rowmask[i];
  {
    const hipError_t he = set_outer_tables(a, sh, static_cast<hipStream_t>(stream));
    if (he != hipSuccess) return fail_hip(he, "outer Hadamard factor table");
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (rq_kernel_for(sh) != RqKernel::kGeneric) {
    const hipError_t e = launch_rq(a, sh, st);
    if (e != hipSuccess) return fail_hip(e, "rotate_quant_int4_outlier launch");
    return SIGNROT_OK;
  }
  // the general kernel reads d: build it in a stream-ordered scratch
  int8_t* d = nullptr;
  hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&d), (static_cast<size_t>(n) + 15) & ~size_t{15}, st);
  if (e != hipSuccess) return fail_hip(e, "hipMallocAsync");
  e = launch_sign_fill(sh, a.form_c, a.form_neg, d, st);
  if (e == hipSuccess) {
    a.d = d;
    a.form_given = 0;
    e = launch_rq_generic(a, st);
  }
  const hipError_t ef = hipFreeAsync(d, st);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) return fail_hip(e, "rotate_quant_int4_outlier launch");
  return SIGNROT_OK;
}
}  // namespace

extern "C" {

int signrot_rotate_quant_int4_outlier(const void* x_bf16, int64_t tokens, int64_t n, int64_t ld, int64_t c,
                                      int sigma, uint8_t* codes, float* scale, float* zero, float* y_out,
                                      void* stream) {
  return rotate_quant_outlier_impl(x_bf16, tokens, n, ld, c, sigma, codes, scale, zero, y_out, 0, stream);
}

int signrot_rotate_quant_int4_zint(const void* x_bf16, int64_t tokens, int64_t n, int64_t ld, int64_t c, int sigma,
                                   uint8_t* codes, float* scale, float* zero, void* stream) {
  return rotate_quant_outlier_impl(x_bf16, tokens, n, ld, c, sigma, codes, scale, zero, nullptr, 1, stream);
}

int signrot_swiglu_rotate_quant_int4(const void* gate_bf16, const void* up_bf16, int64_t tokens, int64_t n, int64_t ld,
                                     int64_t c, int sigma, uint8_t* codes, float* scale, float* zero, float* y_out,
                                     void* stream) {
  if (tokens > 0 && !up_bf16) {
    g_last_error[0] = '\0';
    return fail_einval("null device pointer");
  }
  return rotate_quant_outlier_impl(gate_bf16, tokens, n, ld, c, sigma, codes, scale, zero, y_out, 0, stream,
                                   tokens > 0 ? up_bf16 : nullptr);
}

int signrot_fold_weights(const void* w_bf16, int64_t rows, int64_t n, int64_t ld, const int8_t* d, float* w_out,
                         void* stream) {
  g_last_error[0] = '\0';
  const Shape sh = factor_n(n);
  if (!sh.ok) {
    set_error("unsupported n=%s", std::to_string(n).c_str());
    return SIGNROT_EUNSUPPORTED_N;
  }
  if (rows < 0) return fail_einval("rows < 0");
  if (ld < n) return fail_einval("ld < n");
  if (ld & 7) return fail_einval("ld must be a multiple of 8");
  if (rows == 0) return SIGNROT_OK;
  if (rows > (int64_t{1} << 40)) return fail_einval("rows too large");
  if (!w_bf16 || !d || !w_out) return fail_einval("null device pointer");
  if (!aligned16(w_bf16) || !aligned16(d) || !aligned16(w_out)) return fail_einval("w, d and w_out must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  // scratch: codes [rows][n/2], then (16-byte aligned) scale [rows] and zero [rows]
  const size_t code_bytes = (static_cast<size_t>(rows) * static_cast<size_t>(n / 2) + 15) & ~size_t{15};
  uint8_t* scratch = nullptr;
  hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&scratch), code_bytes + 8 * static_cast<size_t>(rows), s);
  if (e != hipSuccess) return fail_hip(e, "hipMallocAsync");
  float* scale = reinterpret_cast<float*>(scratch + code_bytes);
  RqArgs a;
  memset(&a, 0, sizeof(a));
  a.x = static_cast<const uint16_t*>(w_bf16);
  a.d = d;
  a.codes = scratch;
  a.scale = scale;
  a.zero = scale + rows;
  a.yout = w_out;
  a.tokens = rows;
  a.ld = ld;
  a.n = sh.n;
  a.k = sh.k;
  a.m28 = sh.m28 ? 1 : 0;
  a.inv_sqrt_n = static_cast<float>(1.0 / sqrt(static_cast<double>(n)));
  a.inv_15sqrt_n = static_cast<float>(1.0 / (15.0 * sqrt(static_cast<double>(n))));
  for (int i = 0; i < 28; ++i) a.h28mask[i] = h28().rowmask[i];
  {
    const hipError_t he = set_outer_tables(a, sh, static_cast<hipStream_t>(stream));
    if (he != hipSuccess) {
      (void)hipFreeAsync(scratch, s);
      return fail_hip(he, "outer Hadamard factor table");
    }
  }
  e = launch_rq(a, sh, s);
  const hipError_t ef = hipFreeAsync(scratch, s);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) return fail_hip(e, "fold_weights launch");
  return SIGNROT_OK;
}

int signrot_dequant(const uint8_t* codes, const float* scale, const float* zero, int64_t tokens, int64_t n,
                    float* y_hat, void* stream) {
  g_last_error[0] = '\0';
  const Shape sh = factor_n(n);
  if (!sh.ok) {
    set_error("unsupported n=%s", std::to_string(n).c_str());
    return SIGNROT_EUNSUPPORTED_N;
  }
  if (tokens < 0) return fail_einval("tokens < 0");
  if (tokens == 0) return SIGNROT_OK;
  if (!codes || !scale || !zero || !y_hat) return fail_einval("null device pointer");
  if (reinterpret_cast<uintptr_t>(y_hat) & 7u) return fail_einval("y_hat must be 8-byte aligned");
  hipError_t e = launch_dequant(codes, scale, zero, tokens, sh.n, y_hat, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "dequant launch");
  return SIGNROT_OK;
}

int signrot_weight_rowsum(const void* w_bf16, int64_t rows, int64_t n, int64_t ld, float* rowsum, void* stream) {
  g_last_error[0] = '\0';
  if (rows < 0 || n < 0) return fail_einval("rows and n must be >= 0");
  if (ld < n) return fail_einval("ld < n");
  if (rows == 0) return SIGNROT_OK;
  if (rows > (int64_t{1} << 31) - 1) return fail_einval("rows too large");
  if (!w_bf16 || !rowsum) return fail_einval("null device pointer");
  hipError_t e = launch_weight_rowsum(static_cast<const uint16_t*>(w_bf16), rows, n, ld, rowsum,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "weight_rowsum launch");
  return SIGNROT_OK;
}

namespace {
int fill_linear(LinearArgs& a, const uint8_t* codes, const float* scale, const float* zero, int64_t tokens,
                int64_t n, const void* w_bf16, int64_t ldw, const float* rowsum, int64_t rows, float* out) {
  if (tokens < 0 || rows < 0) return fail_einval("tokens and rows must be >= 0");
  if (n < 2 || (n & 1)) return fail_einval("n must be even and >= 2");
  if (n > (int64_t{1} << 30)) return fail_einval("n too large");
  if (ldw < n) return fail_einval("ldw < n");
  if (tokens > (int64_t{1} << 31) - 1 || rows > (int64_t{1} << 31) - 1) return fail_einval("tokens or rows too large");
  memset(&a, 0, sizeof(a));
  a.codes = codes;
  a.scale = scale;
  a.zero = zero;
  a.w = static_cast<const uint16_t*>(w_bf16);
  a.rowsum = rowsum;
  a.out = out;
  a.ldw = ldw;
  a.T = static_cast<int>(tokens);
  a.R = static_cast<int>(rows);
  a.n = static_cast<int>(n);
  return SIGNROT_OK;
}
}  // namespace

int signrot_int4_linear(const uint8_t* codes, const float* scale, const float* zero, int64_t tokens, int64_t n,
                        const void* w_bf16, int64_t ldw, const float* rowsum, int64_t rows, float* out,
                        void* stream) {
  g_last_error[0] = '\0';
  LinearArgs a;
  const int st = fill_linear(a, codes, scale, zero, tokens, n, w_bf16, ldw, rowsum, rows, out);
  if (st != SIGNROT_OK) return st;
  if (tokens == 0 || rows == 0) return SIGNROT_OK;
  if (!codes || !scale || !zero || !w_bf16 || !rowsum || !out) return fail_einval("null device pointer");
  hipError_t e = launch_int4_linear(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "int4_linear launch");
  return SIGNROT_OK;
}

const char* signrot_int4_linear_kernel_name(const uint8_t* codes, int64_t tokens, int64_t n, const void* w_bf16,
                                            int64_t ldw, int64_t rows) {
  LinearArgs a;
  if (fill_linear(a, codes, nullptr, nullptr, tokens, n, w_bf16, ldw, nullptr, rows, nullptr) != SIGNROT_OK)
    return nullptr;
  return int4_linear_name(a);
}

int signrot_stream_ceiling(const void* x_bf16, int64_t tokens, int64_t n, int64_t ld, uint8_t* out, float* s0,
                           float* s1, void* stream) {
  g_last_error[0] = '\0';
  if (tokens < 0) return fail_einval("tokens < 0");
  if (n < 8 || n > 32768 || (n & 7)) return fail_einval("n must be a multiple of 8 in [8, 32768]");
  if (ld < n || (ld & 7)) return fail_einval("ld must be >= n and a multiple of 8");
  if (tokens == 0) return SIGNROT_OK;
  if (tokens * (n / 8) >= (int64_t{1} << 32)) return fail_einval("tokens * n / 8 must be < 2^32");
  if (!x_bf16 || !out || !s0 || !s1) return fail_einval("null device pointer");
  if (!aligned16(x_bf16) || (reinterpret_cast<uintptr_t>(out) & 3u)) return fail_einval("x must be 16-byte and out 4-byte aligned");
  hipError_t e = launch_stream_ceiling(static_cast<const uint16_t*>(x_bf16), tokens, static_cast<int>(n), ld, out, s0,
                                       s1, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail_hip(e, "stream_ceiling launch");
  return SIGNROT_OK;
}

}  // extern "C"
