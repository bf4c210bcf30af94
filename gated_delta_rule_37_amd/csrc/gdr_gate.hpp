// gdr_gate.hpp -- host interface of the output-gate epilogue fused into the
// output kernel (KDA blog, section 4.1: y = sigmoid(g) * w * o /
// sqrt(mean_j o_j^2 + eps) per token and head).
#pragma once
#include "gdr_launch.hpp"

namespace gdr {

// The gate's operands: g bf16 [B,T,H,D] (the inputs' dtype), w fp32 [H*D] or
// NULL = ones.
struct OutGate {
    const void* g;
    const float* w;
};

// launch_output with the gate applied to the assembled rows: o receives y
// instead of the operator's output (fp16 operands only).
hipError_t launch_output_gated(int D, bool out_f32, int64_t B, int64_t T, int H, int64_t NC, float scale,
                               const ChunkWs& ws, void* o, const float* beta, const float* lam, void* h_cler,
                               const OutGate& og, ChunkRange cr, hipStream_t stream);

}  // namespace gdr
