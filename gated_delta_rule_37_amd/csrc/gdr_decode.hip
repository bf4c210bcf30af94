// gdr_decode.hip -- single-token state update and read-out (decode step).
//
// One recurrence step per (sequence, head) slab, the inference case with a
// fixed-size state that the KDA blog discusses in section 6.1:
//     p = S^T (alpha*k),  r = S^T (alpha*q),  u = beta (v - p),
//     o = scale (r + u (k.q)),  S <- Diag(alpha) S + k u^T.
// Expanding S_new^T q = (Diag(alpha) S + k u^T)^T q shows o equals the read-out
// after the write, so the fp32 state is read once and written once.
//
// The step is a pair of GEMVs: pure HBM streaming, no matrix cores.  One
// workgroup of 256 threads owns one slab (64 KiB of fp32 state at d = 128).
// Thread (row group rg, column group cg) holds float4 columns 4cg..4cg+3 of rows
// rg, rg + RG, ...; a wave covers whole rows, so every load and store is a
// fully coalesced 16-byte access.  The two dk-reductions are partial sums in
// registers followed by one LDS exchange across the row groups.
#include "gdr_common.hpp"

namespace gdr {

template <int D, int GATE, bool IN_F32, bool OUT_F32>
__global__ __launch_bounds__(256) void decode_kernel(int64_t nslab, int H, float scale,
                                                     const void* __restrict__ q_,
                                                     const void* __restrict__ k_,
                                                     const void* __restrict__ v_,
                                                     const float* __restrict__ beta,
                                                     const float* __restrict__ alpha,
                                                     float* __restrict__ S, void* __restrict__ o_) {
    using InT = typename InType<IN_F32>::T;
    using OutT = typename InType<OUT_F32>::T;
    constexpr int TPR = D / 4;     // threads per state row (float4 each)
    constexpr int RG = 256 / TPR;  // row groups
    constexpr int RPT = D / RG;    // rows per thread

    const int64_t slab = blockIdx.x;
    if (slab >= nslab) return;
    (void)H;
    const int tid = threadIdx.x;
    const int rg = tid / TPR, cg = tid % TPR;

    const InT* q = reinterpret_cast<const InT*>(q_) + slab * D;
    const InT* k = reinterpret_cast<const InT*>(k_) + slab * D;
    const InT* v = reinterpret_cast<const InT*>(v_) + slab * D;
    OutT* o = reinterpret_cast<OutT*>(o_) + slab * D;
    float4v* Sv = reinterpret_cast<float4v*>(S + slab * (int64_t)D * D);

    __shared__ float s_ak[D], s_aq[D], s_k[D], s_a[D];
    __shared__ float s_p[RG][D], s_r[RG][D];
    __shared__ float s_kq;

    // issue the state loads first: they are the long-latency stream
    float4v st[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) st[m] = __builtin_nontemporal_load(&Sv[(rg + m * RG) * TPR + cg]);

    if (tid < D) {
        float a = 1.f;
        if constexpr (GATE == GATE_SCALAR) a = alpha[slab];
        if constexpr (GATE == GATE_CHANNEL) a = alpha[slab * D + tid];
        const float kk = to_f32(k[tid]), qq = to_f32(q[tid]);
        s_k[tid] = kk;
        s_a[tid] = a;
        s_ak[tid] = a * kk;
        s_aq[tid] = a * qq;
        // k.q by a wave reduction (D is 64 or 128: one or two waves)
        float kq = kk * qq;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) kq += __shfl_xor(kq, off);
        if (D == 64 && tid == 0) s_kq = kq;
        if (D == 128 && (tid & 63) == 0) s_p[0][tid] = kq;  // staged, summed below
    }
    __syncthreads();
    if (D == 128 && tid == 0) s_kq = s_p[0][0] + s_p[0][64];

    float4v p = zero4(), r = zero4();
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + m * RG;
        const float ak = s_ak[i], aq = s_aq[i];
        p += st[m] * ak;
        r += st[m] * aq;
    }
    __syncthreads();  // s_p[0] reuse above is finished
    *reinterpret_cast<float4v*>(&s_p[rg][4 * cg]) = p;
    *reinterpret_cast<float4v*>(&s_r[rg][4 * cg]) = r;
    __syncthreads();

    float4v pt = zero4(), rt = zero4();
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        pt += *reinterpret_cast<const float4v*>(&s_p[g][4 * cg]);
        rt += *reinterpret_cast<const float4v*>(&s_r[g][4 * cg]);
    }
    const float b = beta[slab];
    const float kq = s_kq;
    float4v u;
#pragma unroll
    for (int c = 0; c < 4; ++c) u[c] = b * (to_f32(v[4 * cg + c]) - pt[c]);
    if (rg == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) o[4 * cg + c] = from_f32<OutT>(scale * (rt[c] + u[c] * kq));
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + m * RG;
        const float a = s_a[i], kk = s_k[i];
        float4v sn;
#pragma unroll
        for (int c = 0; c < 4; ++c) sn[c] = __builtin_fmaf(a, st[m][c], kk * u[c]);
        __builtin_nontemporal_store(sn, &Sv[i * TPR + cg]);
    }
}

template <int D, int GATE, bool IN_F32, bool OUT_F32>
static hipError_t launch_decode_t(int64_t nslab, int H, float scale, const void* q, const void* k,
                                  const void* v, const float* beta, const float* alpha, float* S,
                                  void* o, hipStream_t stream) {
    hipLaunchKernelGGL((decode_kernel<D, GATE, IN_F32, OUT_F32>), dim3((unsigned)nslab), dim3(256),
                       0, stream, nslab, H, scale, q, k, v, beta, alpha, S, o);
    return hipGetLastError();
}

template <int D, int GATE>
static hipError_t launch_decode_g(bool in_f32, bool out_f32, int64_t nslab, int H, float scale,
                                  const void* q, const void* k, const void* v, const float* beta,
                                  const float* alpha, float* S, void* o, hipStream_t stream) {
    if (in_f32) {
        if (out_f32) return launch_decode_t<D, GATE, true, true>(nslab, H, scale, q, k, v, beta, alpha, S, o, stream);
        return launch_decode_t<D, GATE, true, false>(nslab, H, scale, q, k, v, beta, alpha, S, o, stream);
    }
    if (out_f32) return launch_decode_t<D, GATE, false, true>(nslab, H, scale, q, k, v, beta, alpha, S, o, stream);
    return launch_decode_t<D, GATE, false, false>(nslab, H, scale, q, k, v, beta, alpha, S, o, stream);
}

template <int D>
static hipError_t launch_decode_d(int gate, bool in_f32, bool out_f32, int64_t nslab, int H,
                                  float scale, const void* q, const void* k, const void* v,
                                  const float* beta, const float* alpha, float* S, void* o,
                                  hipStream_t stream) {
    switch (gate) {
        case GATE_NONE: return launch_decode_g<D, GATE_NONE>(in_f32, out_f32, nslab, H, scale, q, k, v, beta, alpha, S, o, stream);
        case GATE_SCALAR: return launch_decode_g<D, GATE_SCALAR>(in_f32, out_f32, nslab, H, scale, q, k, v, beta, alpha, S, o, stream);
        default: return launch_decode_g<D, GATE_CHANNEL>(in_f32, out_f32, nslab, H, scale, q, k, v, beta, alpha, S, o, stream);
    }
}

// Host launcher; arguments were validated by the ABI layer.
hipError_t launch_decode(int D, int gate, bool in_f32, bool out_f32, int64_t nslab, int H,
                         float scale, const void* q, const void* k, const void* v,
                         const float* beta, const float* alpha, float* S, void* o,
                         hipStream_t stream) {
    if (D == 64) return launch_decode_d<64>(gate, in_f32, out_f32, nslab, H, scale, q, k, v, beta, alpha, S, o, stream);
    return launch_decode_d<128>(gate, in_f32, out_f32, nslab, H, scale, q, k, v, beta, alpha, S, o, stream);
}

}  // namespace gdr
