// Instantiations of the outer-order MFMA kernel with 2 column tiles
// (2^k = 32); the shapes are SR_OUTER_SHAPES_T2 in rq_outer_impl.h.
#include "rq_outer_impl.h"

namespace signrot {
SR_OUTER_DEFINE(2, SR_OUTER_SHAPES_T2)
}  // namespace signrot
