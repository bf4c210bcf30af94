// gdr_launch.hpp -- host launchers of the device kernels (private to libgdr).
// Arguments are validated by the ABI layer (gdr_abi.cpp) before these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

// Per chunk-head intermediates, [B*H*NC] chunk-heads each; "op" elements are
// fp16 for bf16 inputs and fp32 for fp32 inputs.  Operands read by matrix
// cores are stored in fragment order (frag_off / cfrag_off in gdr_common.hpp).
//   forward (written by the intra-chunk kernel, read by the state pass):
//     W [64][D], Ut [64][D] (accumulator order), Qt [64][D], KbT [D][64],
//     A [64][64] (op); gam [D] fp32
//   backward, additionally:
//     AT [64][64], Kb [64][D], QtT [D][64], WT [D][64]        reverse pass
//       (fp32 operands only: with fp16 operands the reverse pass reads these
//       transposes from Qt, A, KbT and W, which every mode then writes)
//     Nw, Pw [64][64] fp32: N = (I + L)^-1 and P = Kt Kh^T     gradient kernels
//     Ssnap [D][D] chunk-start state, Usave [64][D] (op)        state pass (save)
//     dSsnap [D][D] chunk-end state gradient, dUsave [64][D],
//     dUsaveT [D][64] (op; fp32 operands only)                  reverse pass
//     gQt, gKt, gKb [64][D], gA, gP [64][64], gGam [D] (fp32)  gradients w.r.t.
//       Qt, Kt, Kb, A, P and gamma, passed to the gate-gradient kernel
// A range of chunks [lo, lo + n) of every (batch, head): the per-chunk kernels
// run one workgroup per chunk-head of the range.
struct ChunkRange {
    int64_t lo, n;
};

#ifdef __HIPCC__
// Workgroup -> (batch * heads + head, chunk) of a launch over a range.  Grids
// have fewer than 2^31 workgroups, so 32-bit division suffices.
__device__ __forceinline__ void range_block(const ChunkRange& cr, int64_t& bh, int64_t& c) {
    const uint32_t n = static_cast<uint32_t>(cr.n), bid = blockIdx.x;
    bh = bid / n;
    c = cr.lo + bid % n;
}
#endif

// The gradient stages hand their partials (dQt, dKb, dKt, dA, dP, dgamma) on
// chip on the value route; on the error route, whose terms edit dKt and dP
// between the stages, all go through the workspace.  At d = 128 dQt and dKb
// still do on the value route (holding them on chip too would spill).
constexpr bool grad_qkb_on_chip(int D) { return D == 64; }
// fp32 operands at d = 128 run the two stages as two kernels, every partial in
// the workspace.
constexpr bool grad_split(int D, bool in_f32) { return in_f32 && D == 128; }

struct ChunkWs {
    void *W, *Ut, *Qt, *KbT, *A;
    float* gam;
    void *AT, *Kb, *QtT, *WT;
    float *Nw, *Pw;
    void *Ssnap, *Usave, *dSsnap, *dUsave, *dUsaveT;
    // per-chunk gradient partials, in operand precision (fp16 for bf16 inputs)
    void *gQt, *gKt, *gKb, *gA, *gP;
    float* gGam;
    void* Mt;  // error-routing backward: M^T dE [64][D] per chunk-head
    // prologue: activated beta ([B,T,H] layout) and the reciprocal row norms of
    // q and k (negative where the norm was clamped), written by the intra kernel
    float *Bact, *rq, *rk;
    // separate erase and write gates (Gated DeltaNet-2), fp32 accumulator order:
    // X [D][D] added to the state after each chunk, Y [64][D] added to its output
    float *X, *Y;
};

// Per-launch event timing (gdr_profile_begin/end); no-ops unless enabled.
void prof_before(hipStream_t stream);
void prof_after(const char* name, hipStream_t stream);

size_t chunk_ws_bytes(int64_t nch, int D, int op_bytes, bool backward, bool cler, bool pro, ChunkWs* out,
                      void* base);

hipError_t launch_decode(int D, int gate, bool in_f32, bool out_f32, int64_t nslab, int H,
                         float scale, const void* q, const void* k, const void* v,
                         const float* beta, const float* alpha, float* S, void* o,
                         hipStream_t stream);

// O = scale (Qt S + A U) for every chunk from the saved chunk-start states and U
// (fp16 operands only).
// h_cler (bf16 hidden stream, NULL = none): the error-routing epilogue, applied
// from the same read of U (fp16 operands only).
hipError_t launch_output(int D, bool out_f32, int64_t B, int64_t T, int H, int64_t NC, float scale,
                         const ChunkWs& ws, void* o, const float* beta, const float* lam, void* h_cler,
                         ChunkRange cr, hipStream_t stream);

// pro: the prologue (0 none; 1 / 2 the two alpha activations, gdr_prologue):
// q, k arrive unnormalised and beta, alpha as logits.  cr: the chunks of every
// (batch, head) this launch transforms.
hipError_t launch_intra(int D, int gate, bool in_f32, int mode, int64_t B, int64_t T, int H,
                        int64_t NC, const void* q, const void* k, const void* v,
                        const float* beta, const float* alpha, void* h_clvr, const float* lam,
                        const ChunkWs& ws, int pro, ChunkRange cr, hipStream_t stream);

// cr: the chunks this launch carries the state through (fp16 operands only; the
// fp32-operand pass always runs the whole sequence and ignores it).  wide: two
// state slices per workgroup (fp16 operands only), for a pass that shares the
// chip with other kernels or has more slices than there are CUs.
hipError_t launch_state_fwd(int D, bool in_f32, bool out_f32, int64_t B, int64_t T, int H,
                            int64_t NC, float scale, const ChunkWs& ws, const float* S0,
                            float* ST, void* o, bool save_for_backward, bool wide, ChunkRange cr,
                            hipStream_t stream);

// The pass of the separate-gate variant (Gated DeltaNet-2) over the chunks cr
// of every sequence (the state enters from S0, leaves into ST), o computed in
// the pass: operands W, Ut, Qt, KbT, A of ws in operand precision
// (fp16 for bf16 inputs, fp32 for fp32 inputs), gam, X, Y fp32.
hipError_t launch_state_fwd_xy(int D, bool in_f32, bool out_f32, int64_t B, int64_t T, int H, int64_t NC,
                               float scale, const ChunkWs& ws, const float* S0, float* ST, void* o, ChunkRange cr,
                               hipStream_t stream);

// Gated DeltaNet-2 (separate erase and write gates e, w [B,T,H,D] fp32): the
// intra-chunk kernel writes the pass's operands of the chunks cr into ws: W = N Kt,
// Ut = -N M_w V, Qt, KbT = (e*K*2^(G_last - G))^T, A = tril(Qt (e*Kh)^T), gam,
// X = ((w*K)*2^(G_last - G))^T V and Y = tril(Qt (w*Kh)^T) V, with
// N = (I + strict_tril(Kt (e*Kh)^T))^-1.
hipError_t launch_gdn2_intra(int D, int gate, bool in_f32, int64_t B, int64_t T, int H, int64_t NC, const void* q,
                             const void* k, const void* v, const float* erase, const float* write,
                             const float* alpha, const ChunkWs& ws, ChunkRange cr, hipStream_t stream);
hipError_t launch_gdn2_decode(int D, int gate, bool in_f32, bool out_f32, int64_t nslab, float scale, const void* q,
                              const void* k, const void* v, const float* erase, const float* write,
                              const float* alpha, float* S, void* o, hipStream_t stream);

// dh_cler (NULL = none): gradient at the hidden stream of the error-routing
// epilogue, which adds lam * dh / beta to dU.
// cr: the chunks this launch carries dS through, from lo + n - 1 down to lo; dST
// is the gradient arriving at the end of the range, dS0 the one leaving its start.
// wide: two 16-column state slices per workgroup (half the workgroups, a longer
// step) for fp16 operands.
hipError_t launch_state_bwd(int D, bool in_f32, int64_t B, int64_t T, int H, int64_t NC, float scale,
                            const ChunkWs& ws, const void* dO, const float* dST, float* dS0,
                            const void* dh_cler, const float* lam, const float* beta, bool wide, ChunkRange cr,
                            hipStream_t stream);

// The per-chunk gradients of a chunk range, both stages in one launch (one
// workgroup per chunk-head).  cler: the error-routing epilogue's terms run
// between the stages (dh, lam and beta as for the epilogue; partial, if not
// NULL, receives one scale-gradient row per chunk, [B*NC][H*D] floats, for
// launch_dlam_final).  ahead (a multiple of 8, 0 = none): each workgroup pulls
// into the L2 the first operands of the workgroup `ahead` places after it in
// the launch (bf16 inputs), which starts on the same XCD about when they are
// needed if `ahead` is somewhat less than the number of CUs the launch gets.
hipError_t launch_grads(int D, int gate, bool in_f32, bool out_f32, int64_t B, int64_t T, int H, int64_t NC,
                        float scale, const void* q, const void* k, const void* v, const float* beta,
                        const float* alpha, const void* dO, const void* dh, const float* lam, void* dq, void* dk,
                        void* dv, float* dbeta, float* dalpha, const ChunkWs& ws, int pro, ChunkRange cr,
                        bool cler, float* partial, int ahead, hipStream_t stream);

hipError_t launch_clvr_dlam(bool in_f32, int64_t BT, int H, int D, const void* dh, const void* v,
                            float* dlam, float* partial, int64_t nseg, hipStream_t stream);
// dlam[c] = sum over nseg rows of partial[seg][c], fixed order
hipError_t launch_dlam_final(int HD, int64_t nseg, const float* partial, float* dlam, hipStream_t stream);

// Error-routing epilogue (CLER-H).  Forward from the saved U: h += lam * U / beta.
// Backward: launch_cler_mt forms M^T dE (dE = lam dh) before the reverse state
// pass; the write errors' Kt and P terms and the scale-gradient rows are added
// inside launch_grads (cler).
hipError_t launch_cler_fwd(int D, bool in_f32, int64_t B, int64_t T, int H, int64_t NC, const ChunkWs& ws,
                           const float* beta, const float* lam, void* h, hipStream_t stream);
hipError_t launch_cler_mt(int D, bool in_f32, int64_t B, int64_t T, int H, int64_t NC, const ChunkWs& ws,
                          const float* lam, const void* dh, hipStream_t stream);

// Input checks of the debug mode (GDR_VALIDATE=1).  Rules, OR-ed:
enum CheckRule : uint32_t {
    CHECK_FINITE = 1u,        // no NaN or Inf
    CHECK_FP16_RANGE = 2u,    // |x| < 65504 (becomes an fp16 operand or snapshot)
    CHECK_ALPHA_OPEN = 4u,    // 0 < x <= 1 (the chunked kernels take log2 x)
    CHECK_ALPHA_CLOSED = 8u,  // 0 <= x <= 1 (the decode step)
    CHECK_NONZERO = 16u       // x != 0 (beta of the error route, e = u / beta)
};
// Clears res (two words), then ORs into res[0] the rules element i of p ([n],
// bf16 or fp32) breaks and lowers res[1] to the smallest such i.
hipError_t launch_check(const void* p, int64_t n, bool bf16, uint32_t rules, unsigned long long* res,
                        hipStream_t stream);
// Device address of the check result on the current device.
hipError_t check_result_address(unsigned long long** out);

// Output-gate epilogue y = sigmoid(g) * w * RMSNorm(o) per head (and its
// backward, with dw reduced from one partial row per token range).
int64_t gate_segments(int64_t BT);
hipError_t launch_gate(bool bwd, int D, bool in_f32, bool out_f32, int64_t BT, int H, const void* o, const void* g,
                       const float* w, void* y, const void* dy, void* dO, void* dg, float* dw, float* partial,
                       hipStream_t stream);

}  // namespace gdr
