// gates_math.h -- the gate activations of the scan's inputs.
// "Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
// Sec. 3.1 step 2 (a per-head forget gate with a learnable decay A and an
// input gate) and Sec. 4 (time-step bias and decay as in Gated DeltaNet):
//     a = exp(-A[h] softplus(a_raw + dt_bias[h])),   b = sigmoid(b_raw).
// Shared by the standalone gates kernel and the gated prefill scan's
// preparation pass, so both produce the same bits.
#pragma once

#include <hip/hip_runtime.h>

namespace sdm {

// 1 / (1 + e^-x) in the form whose exponential cannot overflow (so that
// very negative x give their subnormal values rather than 0)
__device__ __forceinline__ float gate_sigmoid(float x)
{
    const float e = expf(-fabsf(x));
    return x >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

// the forget gate from its pre-activation, the head's time-step bias and decay
__device__ __forceinline__ float gate_decay(float a_raw, float dt_bias, float A)
{
    const float z = a_raw + dt_bias;
    // ln(1 + e^z) in the form whose exponential cannot overflow
    const float sp = z > 0.f ? z + log1pf(expf(-z)) : log1pf(expf(z));
    return expf(-A * sp);
}

}  // namespace sdm
