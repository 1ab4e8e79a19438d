// layout.hpp -- the row strides the kernels and the host share.
#pragma once

#include <stdint.h>

namespace mi355norm {

// Row strides, in elements of each matrix's own type (bytes for FP8 output):
// row r of x starts at x + r * x, and so on.  Contiguous matrices have N.
struct Strides {
    int64_t x, r, y, h;     // input, residual, output, residual sum
};

}  // namespace mi355norm
