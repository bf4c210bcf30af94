// gdr_launch.hpp -- host launchers of the device kernels (private to libgdr).
// Arguments are validated by the ABI layer (gdr_abi.cpp) before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

// Per chunk-head intermediates written by the intra-chunk kernel and consumed by
// the state pass.  `op` is the element size of the matrix-core operands
// (2 for fp16, 4 for fp32).  Each array is [B*H*NC] chunk-heads of:
//   W   [64][D]   Ut  [64][D]   Qt  [64][D]   KbT [D][64]   A [64][64]
//   gam [D] fp32 (per-channel decay over the whole chunk)
// and, for the backward only,
//   AT  [64][64]  Kb [64][D]  QtT [D][64]  WT [D][64]  Nw [64][64] fp32
//   Ssnap [D][D] chunk-start state, Usave [64][D] (op elements)
//   dSsnap [D][D] chunk-end state gradient, dUsave [64][D]
struct ChunkWs {
    void *W, *Ut, *Qt, *KbT, *A;
    float* gam;
    void *AT, *Kb, *QtT, *WT;
    float* Nw;  // N = (I + L)^-1, [64][64] fp32 (backward)
    void *Ssnap, *Usave, *dSsnap, *dUsave;
};

// Per-launch event timing (gdr_profile_begin/end); no-ops unless enabled.
void prof_before(hipStream_t stream);
void prof_after(const char* name, hipStream_t stream);

size_t chunk_ws_bytes(int64_t nch, int D, int op_bytes, bool backward, ChunkWs* out, void* base);

hipError_t launch_decode(int D, int gate, bool in_f32, bool out_f32, int64_t nslab, int H,
                         float scale, const void* q, const void* k, const void* v,
                         const float* beta, const float* alpha, float* S, void* o,
                         hipStream_t stream);

hipError_t launch_intra(int D, int gate, bool in_f32, bool backward, int64_t B, int64_t T, int H,
                        int64_t NC, const void* q, const void* k, const void* v,
                        const float* beta, const float* alpha, void* h_clvr, const float* lam,
                        const ChunkWs& ws, hipStream_t stream);

hipError_t launch_state_fwd(int D, bool in_f32, bool out_f32, int64_t B, int64_t T, int H,
                            int64_t NC, float scale, const ChunkWs& ws, const float* S0,
                            float* ST, void* o, bool save_for_backward, hipStream_t stream);

}  // namespace gdr
