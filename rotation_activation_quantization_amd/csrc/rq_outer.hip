// Outer-order MFMA kernel: which shapes are built, and the launch dispatch.
// The kernel itself is rq_outer_impl.h; rq_outer_t{1,2,4,8,16}.hip
// instantiate it per column-tile count.
#include "rq_outer_impl.h"

namespace signrot {

namespace {
int outer_mtw(int kc, int ntl) {
  switch (ntl) {
    case 1: return rq_outer_mtw_t1(kc);
    case 2: return rq_outer_mtw_t2(kc);
    case 4: return rq_outer_mtw_t4(kc);
    case 8: return rq_outer_mtw_t8(kc);
    case 16: return rq_outer_mtw_t16(kc);
    default: return 0;
  }
}
}  // namespace

bool rq_outer_supports(int m, int k) {
  // (m = 28 with 2^k = 128 .. 512 never gets here: the fast kernels take it)
  if (m <= 1 || m % 4 != 0 || m > kMaxOuter || k < 4 || k > 8) return false;
  const int kc = (m + 31) / 32;
  const int ntl = 1 << (k - 4);
  const int mtw = outer_mtw(kc, ntl);
  if (mtw == 0) return false;
  const int waves = ((m + 15) / 16 + mtw - 1) / mtw;
  if (waves > 16) return false;
  // every staging unit has a thread: m NTL units, (NTL MTW + 3) / 4 per thread
  return static_cast<int64_t>(m) * ntl <= static_cast<int64_t>(64) * waves * ((ntl * mtw + 3) / 4);
}

hipError_t launch_rq_outer(const RqArgs& a, hipStream_t s) {
  switch (1 << (a.k - 4)) {
    case 1: return rq_outer_launch_t1(a, s);
    case 2: return rq_outer_launch_t2(a, s);
    case 4: return rq_outer_launch_t4(a, s);
    case 8: return rq_outer_launch_t8(a, s);
    case 16: return rq_outer_launch_t16(a, s);
    default: return hipErrorInvalidValue;
  }
}

const char* rq_outer_name() { return "rq_outer_mfma"; }

}  // namespace signrot
