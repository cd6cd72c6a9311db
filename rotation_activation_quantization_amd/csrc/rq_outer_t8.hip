// Instantiations of the outer-order MFMA kernel with 8 column tiles
// (2^k = 128); the shapes are SR_OUTER_SHAPES_T8 in rq_outer_impl.h.
#include "rq_outer_impl.h"

namespace signrot {
SR_OUTER_DEFINE(8, SR_OUTER_SHAPES_T8)
}  // namespace signrot
