// Instantiations of the outer-order MFMA kernel with 1 column tile
// (2^k = 16); the shapes are SR_OUTER_SHAPES_T1 in rq_outer_impl.h.
#include "rq_outer_impl.h"

namespace signrot {
SR_OUTER_DEFINE(1, SR_OUTER_SHAPES_T1)
}  // namespace signrot
