// Instantiations of the outer-order MFMA kernel with 16 column tiles
// (2^k = 256); the shapes are SR_OUTER_SHAPES_T16 in rq_outer_impl.h.
#include "rq_outer_impl.h"

namespace signrot {
SR_OUTER_DEFINE(16, SR_OUTER_SHAPES_T16)
}  // namespace signrot
