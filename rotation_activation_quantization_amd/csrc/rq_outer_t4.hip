// Instantiations of the outer-order MFMA kernel with 4 column tiles
// (2^k = 64); the shapes are SR_OUTER_SHAPES_T4 in rq_outer_impl.h.
#include "rq_outer_impl.h"

namespace signrot {
SR_OUTER_DEFINE(4, SR_OUTER_SHAPES_T4)
}  // namespace signrot
