// Small helper kernels shared by the prefill and MoE paths.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace zinc {

// Zero n floats (n % 4 == 0, 16-byte aligned).  A kernel, not hipMemsetAsync,
// so the call stays valid inside a captured HIP graph.
void launch_fill_zero(float* p, size_t n, hipStream_t stream);

}  // namespace zinc
