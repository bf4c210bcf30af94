// gdr_gate_rows.hpp -- the row arithmetic of the output-gate epilogue (KDA
// blog, section 4.1) that its own kernel and the output kernel share, so that
// both normalise a row in the same order.
#pragma once
#include "gdr_gate.hpp"

namespace gdr {

// epsilon of the gate's RMS norm
constexpr float GATE_EPS = 1e-6f;

// sum over the TPR consecutive lanes of a row (TPR a power of two <= 16); both
// kernels reduce a row's squares in this order
template <int TPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) x += __shfl_xor(x, off);
    return x;
}

}  // namespace gdr
