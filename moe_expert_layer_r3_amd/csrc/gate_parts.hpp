// Column groups of the gate-gradient partials written by
// moe_combine_backward_rows and summed by moe_gate_backward_parts: groups of
// at least 4 chunks of 128 columns, at most MOE_GATE_PARTS groups.
#pragma once

#include <hip/hip_runtime.h>

#include "moe_mi355x.h"

namespace moe {
__host__ __device__ inline int gate_chunks_per_group(int d) {
    const int nchunk = d / 128;
    const int c = (nchunk + MOE_GATE_PARTS - 1) / MOE_GATE_PARTS;
    return c < 4 ? 4 : c;
}
__host__ __device__ inline int gate_groups(int d) {
    const int c = gate_chunks_per_group(d);
    return (d / 128 + c - 1) / c;
}

}  // namespace moe
