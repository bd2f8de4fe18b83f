// Small helper kernels shared by the prefill and MoE paths.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace zinc {

// Zero n floats (n % 4 == 0, 16-byte aligned).  A kernel, not hipMemsetAsync,
// so the call stays valid inside a captured HIP graph.
void launch_fill_zero(float* p, size_t n, hipStream_t stream);

// The pre-MLP RMS norm: xn[t][k] = fp16(x[t][k] * r_t * gamma[k]) with
// r_t = 1 / sqrt(mean_k x[t][k]^2 + eps), in fp32; one workgroup per token.
// K % 8 == 0, K <= 16384; x, gamma, xn 16-byte aligned; xn must not overlap x.
void launch_rms_norm(const _Float16* x, const _Float16* gamma, float eps, int K, int M, _Float16* xn,
                     hipStream_t stream);

}  // namespace zinc
