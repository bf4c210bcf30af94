// gdr_gate.hip -- the output-gate epilogue, per head:
//   y = sigmoid(g) * w * o / sqrt(mean_j o_j^2 + eps)
// (KDA blog, section 4.1: the gated output o_t = W_o(Sigmoid(W_up W_down x_t) *
// RMSNorm(KDA(...))); the two projections are GEMMs outside the operator and g
// is the low-rank projection's output, supplied by the caller).  The norm runs
// over the dv channels of one token and head; w is [H*dv].
//
// Backward, with n = o * rstd, s = sigmoid(g), dn = dy * s * w:
//   do = rstd * (dn - n * mean_j(dn_j n_j)),   dg = dy * w * n * s * (1 - s),
//   dw = sum over tokens of dy * s * n.
//
// Both are streaming kernels (one read of every input, one write of every
// output).  A workgroup owns one head and a contiguous range of tokens: D / 8
// threads per row, eight channels each (16-byte accesses for bf16), so each
// thread keeps the same eight channels of w and of the dw sums for the whole
// range; the per-range dw rows are reduced afterwards in a fixed order.
#include "gdr_common.hpp"
#include "gdr_gate_rows.hpp"
#include "gdr_launch.hpp"

namespace gdr {

template <int D, bool IN_F32, bool OUT_F32>
__global__ __launch_bounds__(256) void gate_fwd_kernel(int64_t BT, int H, int64_t per, const void* __restrict__ o_,
                                                       const void* __restrict__ g_, const float* __restrict__ w,
                                                       void* y_) {
    using InT = typename InType<IN_F32>::T;
    using OutT = typename InType<OUT_F32>::T;
    constexpr int TPR = D / 8, RPI = 256 / TPR;
    const int h = blockIdx.x;
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * per;
    const int64_t r1 = r0 + per < BT ? r0 + per : BT;
    const int tid = threadIdx.x, rs = tid / TPR, c0 = (tid % TPR) * 8;
    const OutT* o = reinterpret_cast<const OutT*>(o_);
    const InT* g = reinterpret_cast<const InT*>(g_);
    OutT* y = reinterpret_cast<OutT*>(y_);
    float wv[8];
    load_lam8(w, static_cast<int64_t>(h) * D + c0, wv);
    // NB rows per round: all their loads are issued before the first reduction
    constexpr int NB = 4;
    for (int64_t rb = r0 + rs; rb < r1; rb += NB * RPI) {
        float ov[NB][8], gv[NB][8];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int64_t r = rb + k * RPI < r1 ? rb + k * RPI : r1 - 1;  // clamped; not stored
            const int64_t e = (r * H + h) * D + c0;
            load8f(o + e, ov[k]);
            load8f(g + e, gv[k]);
        }
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(ov[k][i], ov[k][i], ss);
            ss = row_sum<TPR>(ss);
            const float rstd = __builtin_amdgcn_rsqf(ss * (1.f / D) + GATE_EPS);
            float yv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) yv[i] = sigmoid_fast(gv[k][i]) * wv[i] * (ov[k][i] * rstd);
            const int64_t r = rb + k * RPI;
            if (r < r1) store8f(y + (r * H + h) * D + c0, yv);
        }
    }
}

template <int D, bool IN_F32, bool OUT_F32>
__global__ __launch_bounds__(256) void gate_bwd_kernel(int64_t BT, int H, int64_t per, const void* __restrict__ o_,
                                                       const void* __restrict__ g_, const float* __restrict__ w,
                                                       const void* __restrict__ dy_, void* __restrict__ do_,
                                                       void* __restrict__ dg_, float* __restrict__ partial) {
    using InT = typename InType<IN_F32>::T;
    using OutT = typename InType<OUT_F32>::T;
    constexpr int TPR = D / 8, RPI = 256 / TPR;
    __shared__ float red[RPI][D];
    const int h = blockIdx.x;
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * per;
    const int64_t r1 = r0 + per < BT ? r0 + per : BT;
    const int tid = threadIdx.x, rs = tid / TPR, c0 = (tid % TPR) * 8;
    const OutT* o = reinterpret_cast<const OutT*>(o_);
    const OutT* dy = reinterpret_cast<const OutT*>(dy_);
    const InT* g = reinterpret_cast<const InT*>(g_);
    InT* dO = reinterpret_cast<InT*>(do_);
    InT* dg = reinterpret_cast<InT*>(dg_);
    float wv[8], acc[8];
    load_lam8(w, static_cast<int64_t>(h) * D + c0, wv);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    constexpr int NB = 4;  // rows per round, loads first
    for (int64_t rb = r0 + rs; rb < r1; rb += NB * RPI) {
      float ovb[NB][8], gvb[NB][8], dyb[NB][8];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
          const int64_t r = rb + k * RPI < r1 ? rb + k * RPI : r1 - 1;  // clamped; not stored or summed
          const int64_t e = (r * H + h) * D + c0;
          load8f(o + e, ovb[k]);
          load8f(g + e, gvb[k]);
          load8f(dy + e, dyb[k]);
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int64_t r = rb + k * RPI;
        const bool live = r < r1;
        const int64_t e = (r * H + h) * D + c0;
        float (&ov)[8] = ovb[k];
        float (&gv)[8] = gvb[k];
        float (&dyv)[8] = dyb[k];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(ov[i], ov[i], ss);
        ss = row_sum<TPR>(ss);
        const float rstd = __builtin_amdgcn_rsqf(ss * (1.f / D) + GATE_EPS);
        float nv[8], sv[8], dn[8], dot = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            nv[i] = ov[i] * rstd;
            sv[i] = sigmoid_fast(gv[i]);
            dn[i] = dyv[i] * sv[i] * wv[i];
            dot = __builtin_fmaf(dn[i], nv[i], dot);
            if (live) acc[i] = __builtin_fmaf(dyv[i] * sv[i], nv[i], acc[i]);
        }
        dot = row_sum<TPR>(dot) * (1.f / D);
        float dov[8], dgv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            dov[i] = rstd * (dn[i] - nv[i] * dot);
            // s (1 - s) = sigmoid(g) sigmoid(-g), without the subtraction
            dgv[i] = dyv[i] * wv[i] * nv[i] * sv[i] * sigmoid_fast(-gv[i]);
        }
        if (live) {
            store8f(dO + e, dov);
            store8f(dg + e, dgv);
        }
      }
    }
    if (!partial) return;
    // dw partial of this token range: the RPI row slots in a fixed order
#pragma unroll
    for (int i = 0; i < 8; ++i) red[rs][c0 + i] = acc[i];
    __syncthreads();
    if (tid < D) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < RPI; ++k) s += red[k][tid];
        partial[static_cast<int64_t>(blockIdx.y) * H * D + static_cast<int64_t>(h) * D + tid] = s;
    }
}

// token ranges per head: at most 256, each a whole number of row slots
int64_t gate_segments(int64_t BT) { return BT < 1 ? 1 : (BT < 256 ? BT : 256); }

template <int D, bool IN_F32, bool OUT_F32>
static hipError_t launch_gate_t(bool bwd, int64_t BT, int H, const void* o, const void* g, const float* w,
                                void* y, const void* dy, void* dO, void* dg, float* dw, float* partial,
                                hipStream_t stream) {
    if (!bwd) {
        // the forward has no partial rows: finer token segments (shorter
        // workgroups, a shorter tail) measured 84 against 87 us at 1024 against
        // 256 segments on 32K tokens x 16 heads
        const int64_t fseg = BT < 1024 ? (BT < 1 ? 1 : BT) : 1024;
        const int64_t fper = (BT + fseg - 1) / fseg;
        hipLaunchKernelGGL((gate_fwd_kernel<D, IN_F32, OUT_F32>), dim3((unsigned)H, (unsigned)fseg), dim3(256), 0,
                           stream, BT, H, fper, o, g, w, y);
        return hipGetLastError();
    }
    const int64_t nseg = gate_segments(BT);
    const int64_t per = (BT + nseg - 1) / nseg;
    const dim3 grid((unsigned)H, (unsigned)nseg);
    hipLaunchKernelGGL((gate_bwd_kernel<D, IN_F32, OUT_F32>), grid, dim3(256), 0, stream, BT, H, per, o, g, w, dy,
                       dO, dg, dw ? partial : nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !dw) return e;
    return launch_dlam_final(H * D, nseg, partial, dw, stream);
}

hipError_t launch_gate(bool bwd, int D, bool in_f32, bool out_f32, int64_t BT, int H, const void* o, const void* g,
                       const float* w, void* y, const void* dy, void* dO, void* dg, float* dw, float* partial,
                       hipStream_t stream) {
    if (BT == 0 || H == 0) return hipSuccess;
#define GDR_GATE_ARGS bwd, BT, H, o, g, w, y, dy, dO, dg, dw, partial, stream
    if (D == 64) {
        if (in_f32) return out_f32 ? launch_gate_t<64, true, true>(GDR_GATE_ARGS) : launch_gate_t<64, true, false>(GDR_GATE_ARGS);
        return out_f32 ? launch_gate_t<64, false, true>(GDR_GATE_ARGS) : launch_gate_t<64, false, false>(GDR_GATE_ARGS);
    }
    if (in_f32) return out_f32 ? launch_gate_t<128, true, true>(GDR_GATE_ARGS) : launch_gate_t<128, true, false>(GDR_GATE_ARGS);
    return out_f32 ? launch_gate_t<128, false, true>(GDR_GATE_ARGS) : launch_gate_t<128, false, false>(GDR_GATE_ARGS);
#undef GDR_GATE_ARGS
}

}  // namespace gdr
