// gdr_cler.hip -- the error-routing epilogue CLER-H outside the state passes.
//
// Forward (fp32 operands; for fp16 operands the output kernel applies it):
//   h[t, h*dv + j] += lam[h*dv + j] * u_t[j] / beta_t
// from the saved U of every chunk.
//
// Backward.  Inside a chunk the write errors are, without any beta,
//   E = (V - Kt S) - M U,   M = strict_tril(P)
// (the read-out of the decayed state at k_t before the token's own write), so
// the gradient dE = lam * dh arriving at them adds
//   dV += dE,  dKt -= dE S^T,  dS -= Kt^T dE,  dU -= M^T dE,  dP -= strict_tril(dE U^T).
// Taking beta out of the picture matters: through e = u / beta the same
// gradient would reach dbeta as a difference of two terms of size |dE| / beta,
// which fp16 operands cannot resolve.  cler_mt_kernel forms M^T dE before the
// reverse state pass (which needs it for dU), the first gradient stage adds
// dE to dV, and cler_post_body (run between the two gradient stages) adds the
// Kt and P terms and the partial sums of the scale gradient dlam = sum_t dh_t e_t.
#include "gdr_cler.hpp"
#include "gdr_launch.hpp"

#include <type_traits>

namespace gdr {

template <int D, bool IN_F32>
__global__ __launch_bounds__(256) void cler_fwd_kernel(int64_t T, int H, int64_t NC, ChunkWs ws,
                                                       const float* __restrict__ beta, const float* __restrict__ lam,
                                                       void* __restrict__ h_) {
    using OpT = typename std::conditional<IN_F32, float, _Float16>::type;
    using InT = typename InType<IN_F32>::T;
    const int64_t ch = blockIdx.x;
    const int64_t bh = ch / NC, c = ch % NC;
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh % H);
    const int64_t nvalid64 = T - c * CHUNK;
    const int nvalid = nvalid64 < CHUNK ? static_cast<int>(nvalid64) : CHUNK;
    const OpT* U = reinterpret_cast<const OpT*>(ws.Usave) + ch * CHUNK * D;
    InT* hs = reinterpret_cast<InT*>(h_);
#pragma unroll
    for (int i = 0; i < CHUNK * D / 8 / 256; ++i) {
        const int p = i * 256 + static_cast<int>(threadIdx.x);
        int pos, j;
        frag_piece<D>(p, pos, j);
        if (pos >= nvalid) continue;
        const int64_t t = c * CHUNK + pos;
        float u[8], lm[8];
        load8f(U + p * 8, u);
        load_lam8(lam, static_cast<int64_t>(h) * D + j, lm);
        cler_add8(hs + ((b * T + t) * H + h) * D + j, u, lm, beta[(b * T + t) * H + h]);
    }
}

// Shared layout of the two backward kernels: dE = lam * dh of the chunk in
// operand precision, rows = position (A operand rows, k = value column).

// Mt = M^T dE per chunk-head, M = strict_tril(P) the in-chunk key products
// (P[t][s] = k_t . decayed k_s, kept by the intra-chunk kernel), dE = lam dh.
// Output [64][D] row-major in operand precision (rows past the end are zero:
// M^T only reaches later positions, where dE is zero).
template <int D, bool IN_F32>
__global__ __launch_bounds__(256) void cler_mt_kernel(int64_t T, int H, int64_t NC, ChunkWs ws,
                                                      const float* __restrict__ lam, const void* __restrict__ dh_) {
    using Lc = ClerLayout<D, IN_F32>;
    using OpT = typename Lc::OpT;
    using InT = typename InType<IN_F32>::T;
    constexpr int LDT = Lc::LDT;
    __shared__ __attribute__((aligned(16))) OpT sMT[CHUNK * LDT];  // M^T [s][t]
    __shared__ __attribute__((aligned(16))) OpT sET[D * LDT];      // dE^T [j][t], later the output rows

    const int64_t ch = blockIdx.x;
    const int64_t bh = ch / NC, c = ch % NC;
    const int64_t b = bh / H;
    const int h = static_cast<int>(bh % H);
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int64_t nvalid64 = T - c * CHUNK;
    const int nvalid = nvalid64 < CHUNK ? static_cast<int>(nvalid64) : CHUNK;
    const InT* dh = reinterpret_cast<const InT*>(dh_);

    {
        const float* P = ws.Pw + ch * CHUNK * CHUNK;
        constexpr int NE = CHUNK * CHUNK / 256;
        float pv[NE];
#pragma unroll
        for (int i = 0; i < NE; ++i) pv[i] = P[i * 256 + tid];
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int e = i * 256 + tid, t = e / CHUNK, s2 = e % CHUNK;
            sMT[s2 * LDT + t] = static_cast<OpT>(pv[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < CHUNK * D / 8 / 256; ++i) {
        const int p = i * 256 + tid, t = p / (D / 8), j = (p % (D / 8)) * 8;
        float g[8], lm[8];
        if (t < nvalid) {
            load8f(dh + ((b * T + c * CHUNK + t) * H + h) * D + j, g);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) g[e] = 0.f;
        }
        load_lam8(lam, static_cast<int64_t>(h) * D + j, lm);
#pragma unroll
        for (int e = 0; e < 8; ++e) sET[(j + e) * LDT + t] = static_cast<OpT>(lm[e] * g[e]);
    }
    __syncthreads();

    // 4 x D/16 output tiles, k = position (two 32-steps)
    constexpr int NTI = 4 * (D / 16) / 4;
    float4v acc[NTI];
#pragma unroll
    for (int k = 0; k < NTI; ++k) {
        const int tile = wid + 4 * k, rs = tile & 3, ct = tile >> 2;
        acc[k] = zero4();
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
            Frag<OpT> fa, fb;
            fa.load(sMT + (16 * rs + l16) * LDT + 32 * kq + 8 * g4);
            fb.load(sET + (16 * ct + l16) * LDT + 32 * kq + 8 * g4);
            mma(fa, fb, acc[k]);
        }
    }
    __syncthreads();
    OpT* so = sET;  // [64][D] rows, dense
#pragma unroll
    for (int k = 0; k < NTI; ++k) {
        const int tile = wid + 4 * k, rs = tile & 3, ct = tile >> 2;
#pragma unroll
        for (int e = 0; e < 4; ++e) so[(16 * rs + 4 * g4 + e) * D + 16 * ct + l16] = static_cast<OpT>(acc[k][e]);
    }
    __syncthreads();
    OpT* Mt = reinterpret_cast<OpT*>(ws.Mt) + ch * CHUNK * D;
    constexpr int EPP = 16 / sizeof(OpT);
#pragma unroll
    for (int i = 0; i < CHUNK * D / EPP / 256; ++i) {
        const int p = i * 256 + tid;
        *reinterpret_cast<uint4*>(Mt + p * EPP) = *reinterpret_cast<const uint4*>(so + p * EPP);
    }
}

template <int D, bool IN_F32>
static hipError_t launch_cler_t(int which, int64_t B, int64_t T, int H, int64_t NC, const ChunkWs& ws,
                                const float* beta, const float* lam, void* h, const void* dh, float* partial,
                                ChunkRange cr, hipStream_t stream) {
    const int64_t nch = B * H * NC;
    if (nch == 0) return hipSuccess;
    if (which == 0)
        hipLaunchKernelGGL((cler_fwd_kernel<D, IN_F32>), dim3((unsigned)nch), dim3(256), 0, stream, T, H, NC, ws,
                           beta, lam, h);
    else
        hipLaunchKernelGGL((cler_mt_kernel<D, IN_F32>), dim3((unsigned)nch), dim3(256), 0, stream, T, H, NC, ws, lam,
                           dh);
    return hipGetLastError();
}

static hipError_t launch_cler(int which, int D, bool in_f32, int64_t B, int64_t T, int H, int64_t NC,
                              const ChunkWs& ws, const float* beta, const float* lam, void* h, const void* dh,
                              float* partial, ChunkRange cr, hipStream_t stream) {
    if (D == 64)
        return in_f32 ? launch_cler_t<64, true>(which, B, T, H, NC, ws, beta, lam, h, dh, partial, cr, stream)
                      : launch_cler_t<64, false>(which, B, T, H, NC, ws, beta, lam, h, dh, partial, cr, stream);
    return in_f32 ? launch_cler_t<128, true>(which, B, T, H, NC, ws, beta, lam, h, dh, partial, cr, stream)
                  : launch_cler_t<128, false>(which, B, T, H, NC, ws, beta, lam, h, dh, partial, cr, stream);
}

hipError_t launch_cler_fwd(int D, bool in_f32, int64_t B, int64_t T, int H, int64_t NC, const ChunkWs& ws,
                           const float* beta, const float* lam, void* h, hipStream_t stream) {
    return launch_cler(0, D, in_f32, B, T, H, NC, ws, beta, lam, h, nullptr, nullptr, ChunkRange{0, NC}, stream);
}

hipError_t launch_cler_mt(int D, bool in_f32, int64_t B, int64_t T, int H, int64_t NC, const ChunkWs& ws,
                          const float* lam, const void* dh, hipStream_t stream) {
    return launch_cler(1, D, in_f32, B, T, H, NC, ws, nullptr, lam, nullptr, dh, nullptr, ChunkRange{0, NC}, stream);
}

}  // namespace gdr
